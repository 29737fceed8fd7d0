/*
 * Paged-KV decode oracle -- TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Plain fp64 statement of the teaching version on the pages: for each sequence
 * gather the history through the block table into contiguous rows, then run
 * ordinary softmax attention.  No blocking, fusion, online softmax or split:
 * those belong to the GPU path and must reach this same result.
 *
 * Pages cited:
 *   [P1] "从正确到更快：PagedAttention 的优化路线"
 *   [P2] "实现教学版 PagedAttention：从 block table 读取历史 KV cache"
 *   [P3] "算子与编译器：推理 Attention 与 KV Kernel"
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24); /* subnormal: frac * 2^-14 / 2^10 */
    } else if (expo == 0x1f) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp(1.0 + (double)frac / 1024.0, expo - 15);
    }
    return sign ? -mag : mag;
}

/* bfloat16 is the upper 16 bits of a binary32. */
double oracle_decode_bf16(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int64_t index, int dtype) {
    if (dtype == 0) {
        float f;
        memcpy(&f, (const char *)base + index * 4, 4);
        return (double)f;
    }
    uint16_t b;
    memcpy(&b, (const char *)base + index * 2, 2);
    return dtype == 1 ? oracle_decode_f16(b) : oracle_decode_bf16(b);
}

/* [P2] "从逻辑 token 到物理 block": logical_block_id = token_index //
 * block_size, block_offset = token_index % block_size, physical_block_id =
 * block_table[logical_block_id]. */
int oracle_block_address(const int32_t *block_table, int32_t num_table_entries,
                         int64_t token_index, int32_t block_size,
                         int64_t *logical_block_id, int64_t *block_offset,
                         int64_t *physical_block_id) {
    if (!block_table || block_size <= 0 || token_index < 0)
        return ORACLE_ERR_ARG;
    int64_t lb = token_index / block_size;
    int64_t off = token_index % block_size;
    if (lb >= num_table_entries) return ORACLE_ERR_RANGE;
    *logical_block_id = lb;
    *block_offset = off;
    *physical_block_id = block_table[lb];
    return ORACLE_OK;
}

/* [P2] "单个 Sequence 的 paged gather" and "先定义一个简单的 KV cache 布局":
 * the pool is [num_blocks, block_size, num_kv_heads, head_dim]; the row of
 * (physical block pb, offset off, head h) starts at element
 * ((pb * block_size + off) * num_kv_heads + h) * head_dim. */
int oracle_paged_gather(double *keys, double *values,
                        const void *key_cache, const void *value_cache,
                        const int32_t *block_table, int32_t num_table_entries,
                        int32_t context_len, int32_t block_size,
                        int64_t num_blocks, int32_t num_kv_heads,
                        int32_t kv_head, int32_t head_dim, int dtype) {
    if (context_len < 0 || head_dim <= 0 || num_kv_heads <= 0 ||
        kv_head < 0 || kv_head >= num_kv_heads || dtype < 0 || dtype > 2)
        return ORACLE_ERR_ARG;
    for (int64_t t = 0; t < context_len; ++t) {
        int64_t lb, off, pb;
        int rc = oracle_block_address(block_table, num_table_entries, t,
                                      block_size, &lb, &off, &pb);
        if (rc) return rc;
        if (pb < 0 || pb >= num_blocks) return ORACLE_ERR_RANGE;
        int64_t row = ((pb * block_size + off) * num_kv_heads + kv_head) *
                      (int64_t)head_dim;
        for (int32_t d = 0; d < head_dim; ++d) {
            keys[t * head_dim + d] = load_elem(key_cache, row + d, dtype);
            values[t * head_dim + d] = load_elem(value_cache, row + d, dtype);
        }
    }
    return ORACLE_OK;
}

/* [P2] "从 gather 后的 K/V 做 attention": scores = q . K^T, weights =
 * softmax(scores), out = weights . V; [P1] "attention kernel 真正在做什么"
 * divides each score by sqrt(head_dim), carried here by `scale`.  The
 * softmax subtracts the largest score before exponentiating, which leaves
 * the exact result unchanged. */
int oracle_attention(double *out, const double *q, const double *keys,
                     const double *values, int32_t context_len,
                     int32_t head_dim, double scale) {
    if (context_len < 0 || head_dim <= 0) return ORACLE_ERR_ARG;
    for (int32_t d = 0; d < head_dim; ++d) out[d] = 0.0;
    if (context_len == 0) return ORACLE_OK;
    double *scores = (double *)malloc(sizeof(double) * (size_t)context_len);
    if (!scores) return ORACLE_ERR_NOMEM;
    double smax = -INFINITY;
    for (int64_t t = 0; t < context_len; ++t) {
        double dot = 0.0;
        for (int32_t d = 0; d < head_dim; ++d)
            dot += q[d] * keys[t * head_dim + d];
        scores[t] = scale * dot;
        if (scores[t] > smax) smax = scores[t];
    }
    double denom = 0.0;
    for (int64_t t = 0; t < context_len; ++t) {
        scores[t] = exp(scores[t] - smax);
        denom += scores[t];
    }
    for (int64_t t = 0; t < context_len; ++t) {
        double w = scores[t] / denom;
        for (int32_t d = 0; d < head_dim; ++d)
            out[d] += w * values[t * head_dim + d];
    }
    free(scores);
    return ORACLE_OK;
}

/* [P2] "扩展到 batch：每个 Sequence 都有自己的 block table": loop over the
 * sequences; each gathers its own history and attends with its own query.
 * The gather is done once per (sequence, KV head) and shared by the query
 * heads of that group (grouped-query attention maps query head h to KV head
 * h / group). */
int oracle_paged_decode(double *out, const void *query,
                        const void *key_cache, const void *value_cache,
                        const int32_t *block_tables,
                        const int32_t *context_lens, int32_t num_seqs,
                        int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int64_t num_blocks,
                        double scale, int dtype, int num_threads) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        num_heads % num_kv_heads != 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq < 0 || dtype < 0 || dtype > 2)
        return ORACLE_ERR_ARG;
    const int32_t group = num_heads / num_kv_heads;
    const int64_t units = (int64_t)num_seqs * num_kv_heads;
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel num_threads(num_threads)
#endif
    {
        double *keys = NULL, *values = NULL, *qd = NULL;
        int64_t cap = 0;
        qd = (double *)malloc(sizeof(double) * (size_t)head_dim);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t u = 0; u < units; ++u) {
            int32_t s = (int32_t)(u / num_kv_heads);
            int32_t kvh = (int32_t)(u % num_kv_heads);
            int32_t ctx = context_lens[s];
            int rc = ORACLE_OK;
            if (ctx < 0 || !qd) rc = ORACLE_ERR_ARG;
            if (!rc && ctx > cap) {
                free(keys);
                free(values);
                cap = ctx;
                keys = (double *)malloc(sizeof(double) * (size_t)cap * head_dim);
                values = (double *)malloc(sizeof(double) * (size_t)cap * head_dim);
                if (!keys || !values) {
                    rc = ORACLE_ERR_NOMEM;
                    cap = 0;
                }
            }
            if (!rc)
                rc = oracle_paged_gather(
                    keys, values, key_cache, value_cache,
                    block_tables + (int64_t)s * max_blocks_per_seq,
                    max_blocks_per_seq, ctx, block_size, num_blocks,
                    num_kv_heads, kvh, head_dim, dtype);
            for (int32_t g = 0; g < group && !rc; ++g) {
                int32_t h = kvh * group + g;
                int64_t qrow = ((int64_t)s * num_heads + h) * head_dim;
                for (int32_t d = 0; d < head_dim; ++d)
                    qd[d] = load_elem(query, qrow + d, dtype);
                rc = oracle_attention(out + qrow, qd, keys, values, ctx,
                                      head_dim, scale);
            }
            if (rc) {
#ifdef _OPENMP
#pragma omp critical
#endif
                status = rc;
            }
        }
        free(keys);
        free(values);
        free(qd);
    }
    return status;
}

/* [P3] "4.1 为什么页面化会改变 kernel 设计" and "6. Prefix Cache 与 Attention
 * Kernel 的关系": the shared prefix occupies read-only pages common to every
 * sequence, followed by each sequence's own pages.  Compose each sequence's
 * block table from the two and run the plain paged decode on it. */
int oracle_paged_prefix_decode(double *out, const void *query,
                               const void *key_cache, const void *value_cache,
                               const int32_t *prefix_table, int32_t prefix_len,
                               const int32_t *block_tables,
                               const int32_t *context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int64_t num_blocks,
                               double scale, int dtype, int num_threads) {
    if (num_seqs < 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
        prefix_len < 0 || prefix_len % block_size != 0 ||
        prefix_len / block_size > max_blocks_per_seq ||
        (prefix_len > 0 && !prefix_table))
        return ORACLE_ERR_ARG;
    const int32_t prefix_blocks = prefix_len / block_size;
    const size_t entries = (size_t)num_seqs * (size_t)max_blocks_per_seq;
    int32_t *tables = (int32_t *)malloc(sizeof(int32_t) * (entries ? entries : 1));
    if (!tables) return ORACLE_ERR_NOMEM;
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int32_t *own = block_tables + (int64_t)s * max_blocks_per_seq;
        int32_t *row = tables + (int64_t)s * max_blocks_per_seq;
        for (int32_t lb = 0; lb < max_blocks_per_seq; ++lb)
            row[lb] = lb < prefix_blocks ? prefix_table[lb] : own[lb];
    }
    int rc = oracle_paged_decode(out, query, key_cache, value_cache, tables,
                                 context_lens, num_seqs, num_heads,
                                 num_kv_heads, head_dim, block_size,
                                 max_blocks_per_seq, num_blocks, scale, dtype,
                                 num_threads);
    free(tables);
    return rc;
}

/* [P2] "写入 slot 和读取 block table 必须一致": the current token's K/V goes
 * to its slot (physical_block_id, block_offset), encoded as one integer
 * physical_block_id * block_size + block_offset. */
int oracle_paged_kv_write(const void *key, const void *value, void *key_cache,
                          void *value_cache, const int64_t *slot_mapping,
                          int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size,
                          int64_t num_blocks, int elem_bytes) {
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || (elem_bytes != 2 && elem_bytes != 4))
        return ORACLE_ERR_ARG;
    const size_t token_bytes = (size_t)num_kv_heads * head_dim * elem_bytes;
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
        int64_t pb = slot / block_size;
        int64_t off = slot % block_size;
        if (pb >= num_blocks) return ORACLE_ERR_RANGE;
        size_t dst = (size_t)(pb * block_size + off) * token_bytes;
        memcpy((char *)key_cache + dst, (const char *)key + i * token_bytes,
               token_bytes);
        memcpy((char *)value_cache + dst, (const char *)value + i * token_bytes,
               token_bytes);
    }
    return ORACLE_OK;
}

/* [P2] "attention mask 在哪里": each prompt token attends to itself and the
 * tokens before it.  The history of (sequence, KV head) is gathered once;
 * query i of the sequence attends to its first p + 1 rows (p = its
 * position), which is the causal mask applied to the gathered history. */
int oracle_paged_prefill(double *out, const void *query,
                         const void *key_cache, const void *value_cache,
                         const int32_t *block_tables, const int32_t *context_lens,
                         const int32_t *query_start_loc, int32_t num_seqs,
                         int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, int64_t num_blocks,
                         double scale, int dtype, int num_threads) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        num_heads % num_kv_heads != 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq < 0 || dtype < 0 || dtype > 2 ||
        (num_seqs > 0 && query_start_loc[0] != 0))
        return ORACLE_ERR_ARG;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t q_len = query_start_loc[s + 1] - query_start_loc[s];
        if (q_len < 0 || q_len > context_lens[s]) return ORACLE_ERR_ARG;
    }
    const int32_t group = num_heads / num_kv_heads;
    const int64_t units = (int64_t)num_seqs * num_kv_heads;
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel num_threads(num_threads)
#endif
    {
        double *keys = NULL, *values = NULL, *qd = NULL;
        int64_t cap = 0;
        qd = (double *)malloc(sizeof(double) * (size_t)head_dim);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t u = 0; u < units; ++u) {
            int32_t s = (int32_t)(u / num_kv_heads);
            int32_t kvh = (int32_t)(u % num_kv_heads);
            int32_t ctx = context_lens[s];
            int32_t q0 = query_start_loc[s];
            int32_t q_len = query_start_loc[s + 1] - q0;
            int rc = qd ? ORACLE_OK : ORACLE_ERR_NOMEM;
            if (!rc && ctx > cap) {
                free(keys);
                free(values);
                cap = ctx;
                keys = (double *)malloc(sizeof(double) * (size_t)cap * head_dim);
                values = (double *)malloc(sizeof(double) * (size_t)cap * head_dim);
                if (!keys || !values) {
                    rc = ORACLE_ERR_NOMEM;
                    cap = 0;
                }
            }
            if (!rc && q_len > 0)
                rc = oracle_paged_gather(
                    keys, values, key_cache, value_cache,
                    block_tables + (int64_t)s * max_blocks_per_seq,
                    max_blocks_per_seq, ctx, block_size, num_blocks,
                    num_kv_heads, kvh, head_dim, dtype);
            for (int32_t i = 0; i < q_len && !rc; ++i) {
                int32_t pos = ctx - q_len + i; /* this query's position */
                for (int32_t g = 0; g < group && !rc; ++g) {
                    int32_t head = kvh * group + g;
                    int64_t qrow = ((int64_t)(q0 + i) * num_heads + head) * head_dim;
                    for (int32_t d = 0; d < head_dim; ++d)
                        qd[d] = load_elem(query, qrow + d, dtype);
                    rc = oracle_attention(out + qrow, qd, keys, values, pos + 1,
                                          head_dim, scale);
                }
            }
            if (rc) {
#ifdef _OPENMP
#pragma omp critical
#endif
                status = rc;
            }
        }
        free(keys);
        free(values);
        free(qd);
    }
    return status;
}

/* OCP E4M3: sign, 4-bit exponent with bias 7, 3-bit fraction. */
double oracle_decode_e4m3(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int expo = (bits >> 3) & 0xf;
    int frac = bits & 0x7;
    double mag;
    if (expo == 0xf && frac == 0x7) {
        mag = NAN;
    } else if (expo == 0) {
        mag = ldexp((double)frac, -9); /* subnormal: frac/8 * 2^(1-7) */
    } else {
        mag = ldexp(1.0 + (double)frac / 8.0, expo - 7);
    }
    return sign ? -mag : mag;
}

/* Round |v| to the E4M3 grid: in the binade [2^e, 2^(e+1)) the step is
 * 2^(e-3); below 2^-6 (subnormals) the step is 2^-9.  rint() rounds to
 * nearest with ties to even in the default rounding mode. */
uint8_t oracle_encode_e4m3(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7f);
    double a = fabs((double)v);
    if (a > 448.0) a = 448.0;
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid m * 2^-9, m = 0..8 (8 is the smallest normal) */
        double m = rint(ldexp(a, 9));
        return (uint8_t)(sign | (uint8_t)m);
    }
    int e;
    frexp(a, &e);        /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;              /* a in [2^e, 2^(e+1)) */
    double m = rint(ldexp(a, -e) * 8.0) - 8.0; /* fraction steps, 0..8 */
    if (m >= 8.0) {      /* rounded up into the next binade */
        m = 0.0;
        e += 1;
    }
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | (int)m));
}

static float load_f32(const void *base, int64_t index, int dtype) {
    return (float)load_elem(base, index, dtype); /* every source type is exact in binary32 */
}

int oracle_paged_kv_write_e4m3(const void *key, const void *value,
                               uint8_t *key_cache, uint8_t *value_cache,
                               const int64_t *slot_mapping,
                               const float *k_scale, const float *v_scale,
                               int64_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int src_dtype) {
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || src_dtype < 0 || src_dtype > 2)
        return ORACLE_ERR_ARG;
    const int64_t token_elems = (int64_t)num_kv_heads * head_dim;
    for (int64_t i = 0; i < num_tokens; ++i) {
        int64_t slot = slot_mapping[i];
        if (slot < 0) continue;
        int64_t block = slot / block_size;
        int64_t offset = slot % block_size;
        if (block >= num_blocks) return ORACLE_ERR_RANGE;
        int64_t dst = (block * block_size + offset) * token_elems;
        for (int32_t h = 0; h < num_kv_heads; ++h) {
            const float kinv = 1.0f / k_scale[h];
            const float vinv = 1.0f / v_scale[h];
            for (int32_t d = 0; d < head_dim; ++d) {
                int64_t e = (int64_t)h * head_dim + d;
                float kx = load_f32(key, i * token_elems + e, src_dtype) * kinv;
                float vx = load_f32(value, i * token_elems + e, src_dtype) * vinv;
                key_cache[dst + e] = oracle_encode_e4m3(kx);
                value_cache[dst + e] = oracle_encode_e4m3(vx);
            }
        }
    }
    return ORACLE_OK;
}

/* The same batch loop as oracle_paged_decode, gathering E4M3 codes and
 * scaling them by the KV head's scale. */
int oracle_paged_decode_e4m3(double *out, const void *query,
                             const uint8_t *key_cache,
                             const uint8_t *value_cache,
                             const float *k_scale, const float *v_scale,
                             const int32_t *block_tables,
                             const int32_t *context_lens, int32_t num_seqs,
                             int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks,
                             double scale, int dtype, int num_threads) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        num_heads % num_kv_heads != 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq < 0 || dtype < 0 || dtype > 2)
        return ORACLE_ERR_ARG;
    const int32_t group = num_heads / num_kv_heads;
    const int64_t units = (int64_t)num_seqs * num_kv_heads;
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (num_threads <= 0) num_threads = omp_get_max_threads();
#pragma omp parallel num_threads(num_threads)
#endif
    {
        double *keys = NULL, *values = NULL, *qd = NULL;
        int64_t cap = 0;
        qd = (double *)malloc(sizeof(double) * (size_t)head_dim);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t u = 0; u < units; ++u) {
            int32_t s = (int32_t)(u / num_kv_heads);
            int32_t kvh = (int32_t)(u % num_kv_heads);
            int32_t ctx = context_lens[s];
            int rc = ORACLE_OK;
            if (ctx < 0 || !qd) rc = ORACLE_ERR_ARG;
            if (!rc && ctx > cap) {
                free(keys);
                free(values);
                cap = ctx;
                keys = (double *)malloc(sizeof(double) * (size_t)cap * head_dim);
                values = (double *)malloc(sizeof(double) * (size_t)cap * head_dim);
                if (!keys || !values) {
                    rc = ORACLE_ERR_NOMEM;
                    cap = 0;
                }
            }
            const int32_t *table = block_tables + (int64_t)s * max_blocks_per_seq;
            for (int64_t t = 0; t < ctx && !rc; ++t) {
                int64_t lb, off, pb;
                rc = oracle_block_address(table, max_blocks_per_seq, t, block_size, &lb, &off, &pb);
                if (!rc && (pb < 0 || pb >= num_blocks)) rc = ORACLE_ERR_RANGE;
                if (rc) break;
                int64_t row = ((pb * block_size + off) * num_kv_heads + kvh) * (int64_t)head_dim;
                for (int32_t d = 0; d < head_dim; ++d) {
                    keys[t * head_dim + d] = oracle_decode_e4m3(key_cache[row + d]) * (double)k_scale[kvh];
                    values[t * head_dim + d] = oracle_decode_e4m3(value_cache[row + d]) * (double)v_scale[kvh];
                }
            }
            for (int32_t g = 0; g < group && !rc; ++g) {
                int32_t qh = kvh * group + g; /* query head of the group */
                int64_t qrow = ((int64_t)s * num_heads + qh) * head_dim;
                for (int32_t d = 0; d < head_dim; ++d)
                    qd[d] = load_elem(query, qrow + d, dtype);
                rc = oracle_attention(out + qrow, qd, keys, values, ctx, head_dim, scale);
            }
            if (rc) {
#ifdef _OPENMP
#pragma omp critical
#endif
                status = rc;
            }
        }
        free(keys);
        free(values);
        free(qd);
    }
    return status;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
