// Internal launch interface between the C-ABI layer (pkv_api.hip) and the
// kernel translation units.  Not part of the public boundary.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

struct WriteArgs {
    const void *key;
    const void *value;
    void *key_cache;
    void *value_cache;
    const int64_t *slot_mapping;
    int64_t num_tokens;
    int64_t num_blocks;
    int32_t block_size;
    int32_t vecs_per_token;  // (num_kv_heads * head_dim * elem_bytes) / 16
};

// Quantising slot write: 16-bit or binary32 K/V rows -> E4M3 cache rows,
// element e of KV head h stored as encode(x * (1 / scale[h])).
struct WriteE4M3Args {
    const void *key;
    const void *value;
    void *key_cache;               // E4M3 bytes [NB, bs, KVH, D]
    void *value_cache;
    const int64_t *slot_mapping;
    const float *k_scale;          // [KVH]
    const float *v_scale;
    int64_t num_tokens;
    int64_t num_blocks;
    int32_t block_size;
    int32_t groups_per_token;      // KVH * D / 8 (eight elements per group)
    int32_t groups_per_head;       // D / 8
};

struct DecodeArgs {
    void *out;                  // [B, H, D] (out dtype)
    unsigned *work_counter;     // unit dispenser of the persistent kernel (any initial
                                // contents: the launch clears it first); nullptr: one
                                // workgroup per unit, no counter (unsplit calls only)
    float *part_out;            // [B, H, P, D] when split
    float *part_ml;             // [B, H, P, 2] when split
    const void *query;          // [B, H, D]
    const void *key_cache;      // [NB, bs, KVH, D]
    const void *value_cache;
    const int32_t *block_tables;  // [B, MB]
    const int32_t *context_lens;  // [B]
    int64_t num_blocks;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t log2_block_size;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t partition_size;     // tokens per partition (whole context when not split)
    int32_t num_partitions;     // P: partial slots per (sequence, head)
    int32_t unit_parts;         // partitions per work unit of the persistent kernels (>= 1)
    float scale_log2e;          // scale * log2(e): scores live in the exp2 domain
    int32_t out_f32;            // 1: out is binary32; 0: out has the cache dtype
    int32_t token_begin;        // first token read (a page boundary; 0 = whole history)
    int32_t part_stride;        // partial slots per (sequence, head) in the workspace
    int32_t part_base;          // slot of this launch's partition 0
    int32_t direct_out;         // 1: no shared prefix and one partition per suffix:
                                // the suffix epilogue stores out (no merge)
    const float *k_scale;       // [KVH] E4M3 caches only: cached K = code * k_scale
    const float *v_scale;       // [KVH]
    // The decode step's slot write fused into the decode (16-bit caches):
    // sequence s's new row new_key/new_value[s] ([KVH, D]) goes to slot
    // slot_mapping[s] (negative: none), which must be the slot of position
    // ctx - 1; key_cache / value_cache are then written.  nullptr: no write.
    const void *new_key;
    const void *new_value;
    const int64_t *slot_mapping;
};

// Waves per workgroup of the decode kernels, and page ids staged in LDS at a
// time (the host plans work units against both).
constexpr int kDecodeWaves = 4;
constexpr int kDecodeSegPages = 256;

// MFMA column blocks of 16 query rows per wave in the multi-query kernels
// (four waves per workgroup).  More blocks let every K/V operand a wave reads
// from LDS feed more rows (the prefill: one block 11.2 ms, two 9.5 ms on the
// 32-prompt workload; three, once its chunks load straight into LDS and need
// no staging registers, 6.27 against 6.75 ms for two); the shared-prefix
// kernel has few rows per KV head and keeps one, for more workgroups.  The
// host plans the prefix row blocks with kPrefixRowsPerBlock.
#ifndef PKV_PREFILL_BLOCKS
#define PKV_PREFILL_BLOCKS 3
#endif
#ifndef PKV_PREFIX_BLOCKS
#define PKV_PREFIX_BLOCKS 1
#endif
constexpr int kPrefillBlocks = PKV_PREFILL_BLOCKS;
constexpr int kPrefixBlocks = PKV_PREFIX_BLOCKS;
constexpr int kPrefixRowsPerBlock = 4 * 16 * kPrefixBlocks;

// Shared-prefix score/value kernel: every query row of every sequence
// against the prefix pages of one KV head, split along the prefix.
struct PrefixArgs {
    float *part_out;            // [B, H, part_stride, D]: slots 0..num_splits-1
    float *part_ml;             // [B, H, part_stride, 2]
    const void *query;          // [B, H, D]
    const void *key_cache;      // [NB, bs, KVH, D]
    const void *value_cache;
    const int32_t *prefix_table;  // [prefix_len / bs]
    const int32_t *context_lens;  // [B]
    int64_t num_blocks;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t log2_group;         // log2(H / KVH)
    int32_t block_size;
    int32_t log2_block_size;
    int32_t prefix_len;         // tokens, a multiple of block_size
    int32_t split_tokens;       // prefix tokens per unit (a multiple of 64)
    int32_t num_splits;
    int32_t row_blocks;         // ceil(B * G / kPrefixRowsPerBlock)
    int32_t part_stride;
    float scale_log2e;
};

// Multi-token paged attention with a causal mask (prefill, chunked prefill).
struct PrefillArgs {
    void *out;                      // [total_queries, H, D] (out dtype)
    const void *query;              // [total_queries, H, D]
    const void *key_cache;          // [NB, bs, KVH, D]
    const void *value_cache;
    const int32_t *block_tables;    // [B, MB]
    const int32_t *context_lens;    // [B]
    const int32_t *query_start_loc; // [B + 1]
    int64_t num_blocks;
    int32_t num_seqs;
    int32_t total_queries;
    int32_t num_heads;
    int32_t num_kv_heads;
    int32_t log2_group;
    int32_t block_size;
    int32_t log2_block_size;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    float scale_log2e;
    int32_t out_f32;
};

hipError_t launch_kv_write(const WriteArgs &a, hipStream_t stream);

// dtype: f16 or bf16 (queries, caches and, unless out_f32, the output).
hipError_t launch_paged_prefill(const PrefillArgs &a, int dtype, hipStream_t stream);
// src_dtype: 0 f32, 1 f16, 2 bf16.
hipError_t launch_kv_write_e4m3(const WriteE4M3Args &a, int src_dtype, hipStream_t stream);

// dtype: 0 f32, 1 f16, 2 bf16.  Launches the decode kernel and, when
// num_partitions > 1, the log-sum-exp merge.
hipError_t launch_paged_decode(const DecodeArgs &a, int dtype, int head_dim, hipStream_t stream);
// The decode step with its slot write in the decode launch (a.new_key,
// a.new_value, a.slot_mapping set), then the merge; the kernels of
// launch_paged_decode.
hipError_t launch_paged_decode_step(const DecodeArgs &a, int dtype, int head_dim, hipStream_t stream);

// Decode over E4M3 caches (head_dim 128; dtype of query and output: f16 or
// bf16), then the merge when the context is split.
hipError_t launch_paged_decode_e4m3(const DecodeArgs &a, int dtype, hipStream_t stream);

// Shared-prefix decode (16-bit caches, head_dim 128): with a prefix
// (num_splits > 0), the prefix units and the suffix decode over tokens
// [token_begin, ctx) in one launch, writing partial slots, then a merge
// kernel; with none, the suffix decode alone (direct_out: it stores the
// output; else partials and the merge).
hipError_t launch_paged_prefix_decode(const PrefixArgs &p, const DecodeArgs &a, int dtype,
                                      hipStream_t stream);

}  // namespace pkv
