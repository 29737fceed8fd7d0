/*
 * Paged-KV decode oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU statement of what single-query decode attention over
 * a paged KV cache computes.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code, header or constant with the GPU library.
 *
 * Sources (three web pages on PagedAttention):
 *   [P1] "从正确到更快：PagedAttention 的优化路线"
 *        (From correct to fast: the PagedAttention optimisation route)
 *   [P2] "实现教学版 PagedAttention：从 block table 读取历史 KV cache"
 *        (Implementing a teaching PagedAttention: reading the KV cache through
 *        the block table)
 *   [P3] "算子与编译器：推理 Attention 与 KV Kernel"
 *        (Operators and compilers: inference attention and KV kernels)
 *
 * Element encodings (dtype argument): 0 = IEEE binary32, 1 = IEEE binary16,
 * 2 = bfloat16 (upper half of a binary32).  16-bit elements are passed as their
 * raw bit patterns; 8-bit E4M3 codes (quantised caches) as bytes.
 *
 * Return codes: 0 on success, a negative value when an argument or a table
 * entry is out of range (the oracle checks device-side contents too, since it
 * is a checker).
 */
#ifndef PKV_ORACLE_H
#define PKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_RANGE (-2)
#define ORACLE_ERR_NOMEM (-3)

/* Decode one stored element to double (exact for all three encodings). */
double oracle_decode_f16(uint16_t bits);
double oracle_decode_bf16(uint16_t bits);

/* [P2] section "从逻辑 token 到物理 block": logical token index -> logical
 * block id -> physical block id, plus the offset inside the block.
 * block_table has num_table_entries valid entries. */
int oracle_block_address(const int32_t *block_table, int32_t num_table_entries,
                         int64_t token_index, int32_t block_size,
                         int64_t *logical_block_id, int64_t *block_offset,
                         int64_t *physical_block_id);

/* [P2] section "单个 Sequence 的 paged gather": copy the context_len history
 * rows of one KV head, in logical token order, out of the paged pool
 * [num_blocks, block_size, num_kv_heads, head_dim] into contiguous fp64
 * arrays keys/values [context_len, head_dim]. */
int oracle_paged_gather(double *keys, double *values,
                        const void *key_cache, const void *value_cache,
                        const int32_t *block_table, int32_t num_table_entries,
                        int32_t context_len, int32_t block_size,
                        int64_t num_blocks, int32_t num_kv_heads,
                        int32_t kv_head, int32_t head_dim, int dtype);

/* [P2] section "从 gather 后的 K/V 做 attention" with the score scale of
 * [P1] section "attention kernel 真正在做什么": one query head against
 * contiguous fp64 keys/values [context_len, head_dim]:
 *   scores[t] = scale * dot(q, keys[t]); weights = softmax(scores);
 *   out = sum_t weights[t] * values[t].
 * context_len == 0 yields zeros. */
int oracle_attention(double *out, const double *q, const double *keys,
                     const double *values, int32_t context_len,
                     int32_t head_dim, double scale);

/* [P2] section "扩展到 batch：每个 Sequence 都有自己的 block table":
 * for every sequence, gather its history through its block table and run
 * standard attention for each query head.  Query head h reads KV head
 * h / (num_heads / num_kv_heads).
 *   query  [num_seqs, num_heads, head_dim]            (dtype)
 *   out    [num_seqs, num_heads, head_dim]            (fp64)
 *   block_tables [num_seqs, max_blocks_per_seq] int32, context_lens [num_seqs].
 * num_threads <= 0 uses the OpenMP default. */
int oracle_paged_decode(double *out, const void *query,
                        const void *key_cache, const void *value_cache,
                        const int32_t *block_tables,
                        const int32_t *context_lens, int32_t num_seqs,
                        int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int64_t num_blocks,
                        double scale, int dtype, int num_threads);

/* [P3] sections "4.1 为什么页面化会改变 kernel 设计" and "6. Prefix Cache 与
 * Attention Kernel 的关系": sequences that share a prompt prefix read the same
 * read-only pages for it and append pages of their own.  Token t of sequence
 * s lives at prefix_table[t / block_size] when t < prefix_len and at
 * block_tables[s][t / block_size] otherwise; the attention is the ordinary
 * paged decode above over that composed table.  prefix_len is a multiple of
 * block_size and at most max_blocks_per_seq * block_size; the first
 * prefix_len / block_size entries of each block_tables row are ignored.  A
 * sequence shorter than the prefix sees the first context_lens[s] tokens of
 * it. */
int oracle_paged_prefix_decode(double *out, const void *query,
                               const void *key_cache, const void *value_cache,
                               const int32_t *prefix_table, int32_t prefix_len,
                               const int32_t *block_tables,
                               const int32_t *context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int64_t num_blocks,
                               double scale, int dtype, int num_threads);

/* [P2] section "写入 slot 和读取 block table 必须一致": store token i's K/V
 * rows [num_kv_heads, head_dim] at slot_mapping[i] = physical_block_id *
 * block_size + block_offset, a byte copy.  Negative slots are skipped; tokens
 * are applied in index order. */
int oracle_paged_kv_write(const void *key, const void *value, void *key_cache,
                          void *value_cache, const int64_t *slot_mapping,
                          int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size,
                          int64_t num_blocks, int elem_bytes);

/* [P2] section "attention mask 在哪里" and [P1] section "decode attention 和
 * prefill attention 不一样": a prefill processes a whole prompt at once, and
 * each prompt token may only see itself and the tokens before it (causal
 * mask).  Multi-token paged attention: sequence s has
 * q_len = query_start_loc[s+1] - query_start_loc[s] new query tokens, the
 * last q_len positions of its context_lens[s]-token history (already in the
 * pool); query i sits at position p = context_lens[s] - q_len + i and
 * attends to tokens 0..p through the sequence's block table.  q_len ==
 * context_lens[s] is a whole-prompt prefill; q_len == 1 is a decode step.
 *   query, out  [total_queries, num_heads, head_dim], rows packed in sequence
 *               order (query_start_loc[0] == 0, non-decreasing, q_len <= ctx). */
int oracle_paged_prefill(double *out, const void *query,
                         const void *key_cache, const void *value_cache,
                         const int32_t *block_tables, const int32_t *context_lens,
                         const int32_t *query_start_loc, int32_t num_seqs,
                         int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, int64_t num_blocks,
                         double scale, int dtype, int num_threads);

/* 8-bit floating point for a quantised KV cache ([P1] section "Triton 适合做
 *什么": the first kernel leaves quantisation out, a later one adds it).  The
 * format is OCP E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3
 * fraction bits; exponent field 0 is subnormal (fraction * 2^-9); no
 * infinities; 0x7F and 0xFF are NaN; the largest finite magnitude is 448. */
double oracle_decode_e4m3(uint8_t bits);

/* binary32 value -> E4M3 code: magnitudes above 448 saturate to 448, NaN
 * stays NaN (0x7F with the input's sign), everything else rounds to the
 * nearest representable value, ties to even fraction. */
uint8_t oracle_encode_e4m3(float v);

/* Quantised slot write: like oracle_paged_kv_write, but element e of KV head
 * h is stored as oracle_encode_e4m3(x * (1 / scale[h])), the reciprocal and
 * the product in binary32.  key/value hold src_dtype elements (0 f32, 1 f16,
 * 2 bf16); the caches hold E4M3 codes [num_blocks, block_size, num_kv_heads,
 * head_dim]; k_scale/v_scale have num_kv_heads entries. */
int oracle_paged_kv_write_e4m3(const void *key, const void *value,
                               uint8_t *key_cache, uint8_t *value_cache,
                               const int64_t *slot_mapping,
                               const float *k_scale, const float *v_scale,
                               int64_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int src_dtype);

/* oracle_paged_decode over E4M3 caches: the cached element of KV head h is
 * oracle_decode_e4m3(code) * k_scale[h] (keys) or * v_scale[h] (values),
 * formed in fp64; query is dtype (0 f32, 1 f16, 2 bf16). */
int oracle_paged_decode_e4m3(double *out, const void *query,
                             const uint8_t *key_cache,
                             const uint8_t *value_cache,
                             const float *k_scale, const float *v_scale,
                             const int32_t *block_tables,
                             const int32_t *context_lens, int32_t num_seqs,
                             int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size,
                             int32_t max_blocks_per_seq, int64_t num_blocks,
                             double scale, int dtype, int num_threads);

/* Number of OpenMP threads a parallel region of this library would use. */
int oracle_max_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_ORACLE_H */
