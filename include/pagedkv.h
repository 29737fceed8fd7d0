/*
 * pagedkv -- single-query decode attention over a paged KV cache on gfx950.
 *
 * The operation (three web pages on PagedAttention):
 *   [P1] "从正确到更快：PagedAttention 的优化路线"
 *   [P2] "实现教学版 PagedAttention：从 block table 读取历史 KV cache"
 *   [P3] "算子与编译器：推理 Attention 与 KV Kernel"
 *
 * Conventions shared by every entry point:
 *  - All tensor arguments are DEVICE pointers to contiguous row-major arrays
 *    owned by the caller.  The library allocates nothing, frees nothing and
 *    keeps no global state; calls are reentrant.
 *  - KV pool layout ([P2] section "先定义一个简单的 KV cache 布局", with the
 *    head axis holding the KV heads as grouped-query attention requires,
 *    [P3] section "7. MQA / GQA 为什么会改变服务性能"):
 *        key_cache, value_cache : [num_blocks, block_size, num_kv_heads, head_dim]
 *  - Every call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *    default stream) and returns.  Results are valid once the caller has
 *    synchronised with that stream.  A write followed by a decode on the same
 *    stream is ordered by the stream.
 *  - Arguments are checked on the host before anything is launched; a
 *    non-PKV_OK status means nothing was enqueued, except PKV_ERR_HIP, which
 *    reports a launch failure.  No exception crosses this interface.
 *  - Device-resident contents (table entries, slots, lengths) are range
 *    checked inside the kernels so that no access leaves the buffers the
 *    sizes describe: an out-of-range slot is skipped by the write, and a
 *    sequence whose length or table entries are out of range gets NaN
 *    outputs from the decode.
 *  - Pointers to tensors must be 16-byte aligned.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of queries, caches and outputs. */
typedef enum pkv_dtype {
    PKV_F32 = 0,  /* IEEE binary32 */
    PKV_F16 = 1,  /* IEEE binary16 */
    PKV_BF16 = 2  /* bfloat16 */
} pkv_dtype;

/* Largest batch one paged_decode_attention call accepts (every workgroup keeps
 * the batch's partition prefix sum in LDS). */
#define PKV_MAX_SEQS 4096

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_NULL = 1,        /* a required pointer is NULL */
    PKV_ERR_SHAPE = 2,       /* sizes negative or inconsistent */
    PKV_ERR_DTYPE = 3,       /* unknown dtype or out_dtype combination */
    PKV_ERR_UNSUPPORTED = 4, /* head_dim, block_size, group or partition not supported */
    PKV_ERR_ALIGN = 5,       /* a tensor pointer is not 16-byte aligned */
    PKV_ERR_WORKSPACE = 6,   /* workspace missing or too small */
    PKV_ERR_HIP = 7          /* the HIP runtime reported an error at launch */
} pkv_status;

/*
 * paged_kv_write -- store each new token's K and V rows in its slot.
 *
 * [P2] section "写入 slot 和读取 block table 必须一致": the slot handed out
 * for the current token is a (physical_block_id, block_offset) pair, and the
 * place a token is written to must be exactly the place the attention later
 * reads it from; [P2] section "PagedAttention 如何接入 mini vLLM": the
 * attention writes the current K/V through the slot mapping.
 *
 *   key, value    [num_tokens, num_kv_heads, head_dim]   dtype    (read)
 *   key_cache,
 *   value_cache   [num_blocks, block_size, num_kv_heads, head_dim] dtype (written)
 *   slot_mapping  [num_tokens] int64: slot = physical_block_id * block_size
 *                 + block_offset.  A negative slot skips the token; a slot
 *                 >= num_blocks * block_size is skipped too.
 *
 * A bit copy: no conversion.  Tokens with equal slots race (the result is
 * one of them).  num_tokens == 0 is a no-op.
 * Supported: head_dim in {64, 128}; block_size in {4, 8, 16, 32, 64}.
 */
pkv_status paged_kv_write(const void *key, const void *value, void *key_cache,
                          void *value_cache, const int64_t *slot_mapping,
                          int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size,
                          int64_t num_blocks, pkv_dtype dtype, void *stream);

/*
 * paged_decode_workspace_size -- bytes of device scratch paged_decode_attention
 * takes (0 only for an empty batch); required when the context is split,
 * optional otherwise.  partition_size == 0 means one partition per sequence.
 * Layout: a 256-byte work-counter area, then, when the context is split
 * (P = ceil(max_context_len / partition_size) > 1), fp32 partial outputs
 * [num_seqs, num_heads, P, head_dim] and per-partition (running max,
 * normaliser) pairs [num_seqs, num_heads, P, 2].
 */
size_t paged_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                   int32_t head_dim, int32_t max_context_len,
                                   int32_t partition_size);

/*
 * paged_decode_attention -- one query token per sequence attends to its
 * cached history, read from the paged pool through its block table.
 *
 * Computes, for sequence s and query head h with KV head kvh = h / G
 * (G = num_heads / num_kv_heads, contiguous head groups):
 *   token t of the history lives at physical block block_tables[s][t /
 *   block_size], offset t % block_size ([P2] section "从逻辑 token 到物理
 *   block");
 *   score_t = scale * dot(query[s][h], key_t)   ([P1] section "attention
 *   kernel 真正在做什么" scales by 1/sqrt(head_dim); the caller passes it);
 *   out[s][h] = sum_t softmax(score)_t * value_t   ([P2] section "从 gather
 *   后的 K/V 做 attention"),
 * over t < context_lens[s].  Decode needs no causal mask ([P2] section
 * "attention mask 在哪里").  The result equals attention over a contiguous
 * cache holding the same rows ([P2] section "和连续 KV cache 对齐验证").
 * It is computed without gathering the history and without storing the
 * scores ([P1] sections "高性能 PagedAttention 的核心思想" and "attention
 * kernel 真正在做什么"): the kernel resolves every page itself and keeps a
 * running softmax.  A sequence with context_lens[s] == 0 gets zeros.
 *
 *   out           [num_seqs, num_heads, head_dim]  out_dtype (written)
 *   query         [num_seqs, num_heads, head_dim]  dtype
 *   key_cache,
 *   value_cache   [num_blocks, block_size, num_kv_heads, head_dim] dtype
 *   block_tables  [num_seqs, max_blocks_per_seq] int32; entries at or past
 *                 ceil(context_lens[s] / block_size) are never read
 *   context_lens  [num_seqs] int32, each in [0, max_context_len] and
 *                 <= max_blocks_per_seq * block_size
 *   max_context_len  host-side upper bound of context_lens; sizes the grid
 *   scale         score multiplier (normally 1/sqrt(head_dim))
 *   partition_size   0: each (sequence, KV head) is one work unit; else the
 *                 context is cut into partitions of this many tokens (a
 *                 multiple of 16 and of block_size) whose partial results a
 *                 second kernel merges by log-sum-exp
 *   dtype         PKV_F32, PKV_F16 or PKV_BF16; out_dtype is dtype or PKV_F32
 *   workspace     device scratch of at least paged_decode_workspace_size()
 *                 bytes, 16-byte aligned, owned by the caller; any initial
 *                 contents (the decode kernel clears its work counter when
 *                 it starts, in a way no earlier contents can defeat, so no
 *                 call depends on what an earlier call left there).  May be
 *                 NULL (workspace_bytes ignored) when the context is not
 *                 split (partition_size == 0 or >= max_context_len): the
 *                 decode then runs one workgroup per (sequence, KV head)
 *                 instead of a persistent grid drawing work from a counter.
 *                 A split call without one returns PKV_ERR_WORKSPACE.  Calls
 *                 that can run at the same time (different streams) must
 *                 use different workspaces: sharing one is a race.
 *
 * Accumulation is fp32 throughout.  Supported: head_dim in {64, 128};
 * block_size in {4, 8, 16, 32, 64}; G in {1, 2, 4, 8}; num_seqs <=
 * PKV_MAX_SEQS.
 */
pkv_status paged_decode_attention(
    void *out, const void *query, const void *key_cache,
    const void *value_cache, const int32_t *block_tables,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
    float scale, int32_t partition_size, pkv_dtype dtype,
    pkv_dtype out_dtype, void *workspace, size_t workspace_bytes,
    void *stream);

/*
 * paged_decode_step -- one decode step in one launch: the slot write of
 * each sequence's new token and the decode attention over the history that
 * ends with it.
 *
 * [P2] section "PagedAttention 如何接入 mini vLLM": a decode step writes the
 * current token's K/V through its slot, then attends over the sequence's
 * history through the block table; section "写入 slot 和读取 block table 必须
 * 一致": the slot written is the place the attention reads that token from.
 * The result is paged_kv_write(new_key, new_value, ..., slot_mapping,
 * num_seqs) followed by paged_decode_attention, under one condition: a
 * non-negative slot_mapping[s] must be the slot of position
 * context_lens[s] - 1 of sequence s (block_tables[s][(ctx - 1) /
 * block_size] * block_size + (ctx - 1) % block_size), the position the
 * step appends.  The kernel then reads that token from new_key/new_value
 * while it stores them, so the launch needs no ordering between the store
 * and the reads.  A sequence whose slot is another one (or out of range)
 * stores nothing and gets NaN outputs; one whose context is empty stores
 * nothing and gets zeros, as in paged_decode_attention; a negative slot
 * stores nothing and attends over the history as it is.
 *
 *   new_key,
 *   new_value     [num_seqs, num_kv_heads, head_dim]  dtype  (read)
 *   slot_mapping  [num_seqs] int64 (device)
 *   key_cache,
 *   value_cache   written at the valid slots
 *   other arguments as paged_decode_attention.
 * Supported: what paged_decode_attention supports (every dtype, head_dim
 * 64 or 128); errors as there, and PKV_ERR_NULL / PKV_ERR_ALIGN for the
 * new rows and slots.  Slots of different sequences must differ.
 */
pkv_status paged_decode_step(
    void *out, const void *query, void *key_cache, void *value_cache,
    const void *new_key, const void *new_value, const int64_t *slot_mapping,
    const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
    float scale, int32_t partition_size, pkv_dtype dtype, pkv_dtype out_dtype,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_decode_attention_noalloc -- paged_decode_attention for callers that
 * cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  It calls
 * no allocating routine; the work counter and split partials live in a
 * library-owned static device array of PKV_NOALLOC_SCRATCH_BYTES bytes per
 * GPU (taken when the library's code is loaded on that GPU, held until the
 * process ends; its address is looked up on the first call per GPU).
 *
 * Arguments, result and errors are those of paged_decode_attention without
 * the workspace.  A call whose paged_decode_workspace_size() exceeds
 * PKV_NOALLOC_SCRATCH_BYTES returns PKV_ERR_WORKSPACE before anything is
 * enqueued (a smaller partition count fits: raise partition_size or split
 * the batch).  Every call on one GPU shares that GPU's array: no call
 * depends on what an earlier one left there, but calls whose kernels can
 * overlap on one GPU (different streams, or threads without ordering) race
 * on it and must be serialised by the caller.  `stream` must belong to the
 * GPU whose array is used (the current device when `stream` is NULL).
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

pkv_status paged_decode_attention_noalloc(
    void *out, const void *query, const void *key_cache,
    const void *value_cache, const int32_t *block_tables,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
    float scale, int32_t partition_size, pkv_dtype dtype,
    pkv_dtype out_dtype, void *stream);

/*
 * paged_prefix_decode_workspace_size -- bytes of device scratch
 * paged_prefix_decode_attention needs (0 for an empty batch or invalid
 * sizes).  Layout: the 256-byte work-counter area, then fp32 partial outputs
 * [num_seqs, num_heads, S, head_dim] and (running max, normaliser) pairs
 * [num_seqs, num_heads, S, 2], where S counts the prefix splits the library
 * plans for these sizes plus the suffix partitions
 * (ceil((max_context_len - prefix_len) / partition_size), at least 1; 1 when
 * partition_size == 0).
 */
size_t paged_prefix_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_context_len,
                                          int32_t prefix_len,
                                          int32_t partition_size);

/*
 * paged_prefix_decode_attention -- decode attention for a batch whose
 * sequences share a prompt prefix held in shared, read-only pages.
 *
 * [P3] section "4.1 为什么页面化会改变 kernel 设计": the pages decode reads
 * include prefix pages that several requests share; [P3] section "6. Prefix
 * Cache 与 Attention Kernel 的关系": shared prefix pages are read-only and the
 * access pattern becomes reuse of old pages plus appended new ones.
 *
 * Computes exactly what paged_decode_attention computes when token t of
 * sequence s lives at prefix_table[t / block_size] for t < prefix_len and at
 * block_tables[s][t / block_size] otherwise.  A sequence with
 * context_lens[s] < prefix_len attends to the first context_lens[s] tokens of
 * the prefix.  The prefix is read once per KV head for the whole batch: its
 * score and value products for all num_seqs * G query rows are dense
 * matrix products; the rest of each history goes through the paged decode,
 * and a log-sum-exp merge joins the partial results.
 *
 *   prefix_table  [prefix_len / block_size] int32 physical block ids
 *                 (device); may be NULL when prefix_len == 0
 *   prefix_len    tokens of the shared prefix, a multiple of block_size and
 *                 at most max_blocks_per_seq * block_size
 *   block_tables  [num_seqs, max_blocks_per_seq] int32; entries below
 *                 prefix_len / block_size and at or past
 *                 ceil(context_lens[s] / block_size) are never read
 *   workspace     at least paged_prefix_decode_workspace_size() bytes, any
 *                 contents (as for paged_decode_attention); always required;
 *                 one workspace per concurrently running call
 * Every other argument, the output and the error behaviour are those of
 * paged_decode_attention; an out-of-range prefix table entry makes the
 * outputs of the sequences that reach that page NaN.
 * Supported: dtype PKV_F16 or PKV_BF16, head_dim 128, block_size in
 * {4, 8, 16, 32, 64}, G in {1, 2, 4, 8}, num_seqs <= PKV_MAX_SEQS.
 */
pkv_status paged_prefix_decode_attention(
    void *out, const void *query, const void *key_cache,
    const void *value_cache, const int32_t *prefix_table, int32_t prefix_len,
    const int32_t *block_tables, const int32_t *context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int64_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, pkv_dtype dtype, pkv_dtype out_dtype,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_prefill_attention -- multi-token paged attention with a causal mask
 * (prefill and chunked prefill) over the same pool.
 *
 * [P2] section "attention mask 在哪里": a prefill processes the whole prompt
 * at once and each prompt token may only see itself and the tokens before
 * it; [P1] section "decode attention 和 prefill attention 不一样": prefill is
 * causal attention over the prompt.  Sequence s has q_len =
 * query_start_loc[s+1] - query_start_loc[s] new query tokens, the last q_len
 * positions of its context_lens[s]-token history, whose K/V are already in
 * the pool (paged_kv_write first).  Query i sits at position p =
 * context_lens[s] - q_len + i and attends to tokens 0..p through
 * block_tables[s].  q_len == context_lens[s] is a whole-prompt prefill;
 * q_len == 1 is one decode step.
 *
 *   out             [total_queries, num_heads, head_dim]  out_dtype (written)
 *   query           [total_queries, num_heads, head_dim]  dtype, rows packed
 *                   in sequence order
 *   query_start_loc [num_seqs + 1] int32 (device): 0 = query_start_loc[0] <=
 *                   ... <= query_start_loc[num_seqs] = total_queries.  A
 *                   sequence whose range leaves [0, total_queries] is skipped
 *                   (its rows are not written); one with q_len >
 *                   context_lens[s] or an out-of-range length or page id gets
 *                   NaN rows (only the rows that reach a bad page).
 *   other arguments as paged_decode_attention; no workspace is needed.
 * Supported: dtype PKV_F16 or PKV_BF16 (out_dtype dtype or PKV_F32),
 * head_dim 128, block_size in {4, 8, 16, 32, 64}, G in {1, 2, 4, 8},
 * num_seqs <= PKV_MAX_SEQS.
 */
pkv_status paged_prefill_attention(
    void *out, const void *query, const void *key_cache,
    const void *value_cache, const int32_t *block_tables,
    const int32_t *context_lens, const int32_t *query_start_loc,
    int32_t num_seqs, int32_t total_queries, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
    float scale, pkv_dtype dtype, pkv_dtype out_dtype, void *stream);

/*
 * 8-bit quantised KV cache.  [P1] section "Triton 适合做什么": the first
 * kernel leaves quantisation out; this is the later version that adds it.
 * Element format: OCP E4M3 ("e4m3fn": 1 sign, 4 exponent bits with bias 7, 3
 * fraction bits, no infinities, 0x7F/0xFF NaN, largest finite 448).  One
 * binary32 scale per KV head for K and one for V: the cached element of KV
 * head h stands for code * k_scale[h] (keys) or code * v_scale[h] (values).
 */

/*
 * paged_kv_write_fp8 -- paged_kv_write into E4M3 caches: element e of KV head
 * h of each token is stored as E4M3(x * (1 / scale[h])), the reciprocal and
 * the product in binary32 (correctly rounded), saturated to +-448 (NaN stays
 * NaN), rounded to nearest with ties to even.
 *
 *   key, value    [num_tokens, num_kv_heads, head_dim]  src_dtype (F32/F16/BF16)
 *   key_cache,
 *   value_cache   [num_blocks, block_size, num_kv_heads, head_dim] E4M3 bytes
 *   k_scale,
 *   v_scale       [num_kv_heads] binary32 (device), nonzero
 * Slots, errors and supported sizes as paged_kv_write.
 */
pkv_status paged_kv_write_fp8(const void *key, const void *value, void *key_cache,
                              void *value_cache, const int64_t *slot_mapping,
                              const float *k_scale, const float *v_scale,
                              int64_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, pkv_dtype src_dtype, void *stream);

/*
 * paged_decode_attention_fp8 -- paged_decode_attention over E4M3 caches with
 * per-KV-head scales: the same result as over caches holding code * scale.
 * The codes are widened exactly to the query's type (keys, for the score
 * product on the matrix cores) and to binary32 (values); k_scale joins the
 * score scale, v_scale multiplies the output.  Half the bytes of a 16-bit
 * cache are read.
 *
 *   query, out    as paged_decode_attention; dtype is PKV_F16 or PKV_BF16
 *                 (the query's type), out_dtype is dtype or PKV_F32
 *   key_cache,
 *   value_cache   [num_blocks, block_size, num_kv_heads, head_dim] E4M3 bytes
 *   k_scale,
 *   v_scale       [num_kv_heads] binary32 (device)
 *   workspace     paged_decode_workspace_size() bytes, same rules (NULL
 *                 allowed when the context is not split)
 * Supported: head_dim 128, block_size in {4, 8, 16, 32, 64}, G in {1, 2, 4,
 * 8}, num_seqs <= PKV_MAX_SEQS.
 */
pkv_status paged_decode_attention_fp8(
    void *out, const void *query, const void *key_cache,
    const void *value_cache, const float *k_scale, const float *v_scale,
    const int32_t *block_tables, const int32_t *context_lens,
    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int64_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, pkv_dtype dtype, pkv_dtype out_dtype,
    void *workspace, size_t workspace_bytes, void *stream);

/* Static, NUL-terminated description of a status code (host memory). */
const char *pkv_status_string(pkv_status status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
