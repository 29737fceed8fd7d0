// C-ABI layer of libpagedkv: host-side argument checks, work decomposition
// and kernel selection.  Declarations and the contract live in pagedkv.h.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "pagedkv.h"
#include "pkv_launch.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pkv_dtype d) { return d == PKV_F32 ? 4 : 2; }

bool valid_dtype(int d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }

bool pow2_block(int32_t bs) { return bs == 4 || bs == 8 || bs == 16 || bs == 32 || bs == 64; }

int log2i(int32_t v) {
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

// Tokens per decode work unit: every partition starts on a page boundary and
// on a 16-token boundary.
int32_t partition_granule(int32_t block_size) { return block_size > 16 ? block_size : 16; }

// Workspace layout: the unit counter in the first kCounterBytes, then the
// split partials (fp32 outputs, then (max, normaliser) pairs).
constexpr size_t kCounterBytes = 256;

int32_t num_partitions(int32_t max_context_len, int32_t partition_size) {
    if (partition_size <= 0 || max_context_len <= 0) return 1;
    return (int32_t)(((int64_t)max_context_len + partition_size - 1) / partition_size);
}

// Partitions per work unit of the persistent kernels: 4 when a span can hold
// four partitions (parts >= 4), they are short (at most
// PKV_WAVE_PARTITION_MAX tokens) and a run of four fits one page-id staging
// window (256 pages), else 1.  A sequence's span then
// starts with runs of four whole partitions, one unit each, in which each
// wave streams one partition alone and writes its partial directly: no
// cross-wave merge and no barrier at every partition end.  The rest of the
// span is one unit per partition.
#ifndef PKV_WAVE_PARTITION_MAX
#define PKV_WAVE_PARTITION_MAX 1024
#endif
int32_t unit_parts(int32_t parts, int32_t partition_size, int32_t block_size) {
    if (parts < pkv::kDecodeWaves || partition_size > PKV_WAVE_PARTITION_MAX) return 1;
    if ((int64_t)pkv::kDecodeWaves * partition_size > (int64_t)pkv::kDecodeSegPages * block_size) return 1;
    return pkv::kDecodeWaves;
}

// A decode call needs its workspace when the context is split (partials);
// an unsplit call may pass NULL (then one workgroup per unit, no counter).
// A workspace that is passed must be large enough and 16-byte aligned.
pkv_status check_workspace(const void *workspace, size_t workspace_bytes, int32_t parts, size_t need) {
    if (!workspace) return parts > 1 ? PKV_ERR_WORKSPACE : PKV_OK;
    if (workspace_bytes < need) return PKV_ERR_WORKSPACE;
    return aligned16(workspace) ? PKV_OK : PKV_ERR_ALIGN;
}

// Shared-prefix plan: blocks of kPrefixRowsPerBlock query rows per KV head, and
// the prefix cut into splits of whole 64-token chunks (at most 2048 tokens
// each) so that about kPrefixTargetUnits workgroups share the prefix work.
// The prefix units run beside the persistent suffix grid, so they should be
// few yet short enough to end within the suffix decode: on the 128-sequence,
// 2048-token-prefix batch (64 units per split) the call took 70.9-71.1 us
// at 64 units, 66.1-67.5 at 128, 69.6-70.2 at 192, 72.4-72.6 at 256 and
// 77.5-78.0 at 512.
constexpr int32_t kPrefixChunk = 64;
constexpr int32_t kPrefixMaxSplitChunks = 32;
#ifndef PKV_PFX_TARGET_UNITS
#define PKV_PFX_TARGET_UNITS 128
#endif
constexpr int64_t kPrefixTargetUnits = PKV_PFX_TARGET_UNITS;

struct PrefixPlan {
    int32_t row_blocks, num_splits, split_tokens;
    int32_t suffix_parts, suffix_partition;
};

PrefixPlan prefix_plan(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                       int32_t max_context_len, int32_t prefix_len, int32_t partition_size) {
    PrefixPlan p;
    const int64_t rows = (int64_t)num_seqs * (num_heads / num_kv_heads);
    p.row_blocks = (int32_t)((rows + pkv::kPrefixRowsPerBlock - 1) / pkv::kPrefixRowsPerBlock);
    p.num_splits = 0;
    p.split_tokens = kPrefixChunk;
    if (prefix_len > 0) {
        const int64_t chunks = (prefix_len + kPrefixChunk - 1) / kPrefixChunk;
        const int64_t base = (int64_t)num_kv_heads * p.row_blocks;
        int64_t want = (kPrefixTargetUnits + base - 1) / base;
        const int64_t most = (chunks + 3) / 4;  // keep >= 4 chunks per split
        if (want > most) want = most;
        const int64_t least = (chunks + kPrefixMaxSplitChunks - 1) / kPrefixMaxSplitChunks;
        if (want < least) want = least;
        const int64_t per = (chunks + want - 1) / want;
        p.split_tokens = (int32_t)(per * kPrefixChunk);
        p.num_splits = (int32_t)((chunks + per - 1) / per);
    }
    const int32_t span = max_context_len - prefix_len;
    if (partition_size > 0) {
        p.suffix_parts = span > 0 ? (int32_t)(((int64_t)span + partition_size - 1) / partition_size) : 1;
        p.suffix_partition = partition_size;
    } else {
        p.suffix_parts = 1;
        p.suffix_partition = span > 0 ? span : 1;
    }
    return p;
}


// Checks shared by the decode entry points, and the launch arguments they
// imply (all but the workspace).  kv8: E4M3 caches (16-bit queries,
// head_dim 128, per-KV-head scales).  `empty` is set for a batch with
// nothing to launch (the status is then PKV_OK).
pkv_status decode_setup(pkv::DecodeArgs &a, bool &empty, bool kv8, void *out, const void *query,
                        const void *key_cache, const void *value_cache, const float *k_scale,
                        const float *v_scale, const int32_t *block_tables,
                        const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int64_t num_blocks, int32_t max_context_len,
                        float scale, int32_t partition_size, pkv_dtype dtype, pkv_dtype out_dtype) {
    empty = false;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0 ||
        num_blocks < 0 || max_context_len < 0 || partition_size < 0)
        return PKV_ERR_SHAPE;
    if (num_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return PKV_ERR_DTYPE;
    if (out_dtype != dtype && out_dtype != PKV_F32) return PKV_ERR_DTYPE;
    if (kv8 ? (dtype == PKV_F32 || head_dim != 128) : (head_dim != 64 && head_dim != 128))
        return PKV_ERR_UNSUPPORTED;
    if (!pow2_block(block_size)) return PKV_ERR_UNSUPPORTED;
    const int32_t group = num_heads / num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8) return PKV_ERR_UNSUPPORTED;
    if (partition_size != 0 && partition_size % partition_granule(block_size) != 0)
        return PKV_ERR_UNSUPPORTED;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
    if (num_blocks == 0 && max_context_len > 0) return PKV_ERR_SHAPE;  // no page to read
    if (!isfinite(scale)) return PKV_ERR_SHAPE;
    if (num_seqs > PKV_MAX_SEQS) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) {
        empty = true;
        return PKV_OK;
    }
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
        (kv8 && (!k_scale || !v_scale)))
        return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
        return PKV_ERR_ALIGN;
    const int32_t parts = num_partitions(max_context_len, partition_size);
    if ((int64_t)num_seqs * num_kv_heads * parts > INT_MAX || (int64_t)num_seqs * num_heads > INT_MAX)
        return PKV_ERR_SHAPE;
    a = pkv::DecodeArgs{};
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_blocks = num_blocks;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.log2_block_size = log2i(block_size);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    // Unsplit: one unit covers any admissible context.
    a.partition_size = parts > 1 ? partition_size : (max_context_len > 0 ? max_context_len : 1);
    a.num_partitions = parts;
    a.unit_parts = unit_parts(parts, partition_size, block_size);
    a.scale_log2e = scale * 1.4426950408889634f;
    a.out_f32 = out_dtype == PKV_F32 ? 1 : 0;
    a.token_begin = 0;
    a.part_stride = parts;
    a.part_base = 0;
    a.direct_out = 0;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    return PKV_OK;
}

// Point the launch arguments at a workspace laid out as
// paged_decode_workspace_size describes (NULL: no counter, no partials).
void bind_workspace(pkv::DecodeArgs &a, void *workspace, int32_t head_dim) {
    a.work_counter = reinterpret_cast<unsigned *>(workspace);
    a.part_out = nullptr;
    a.part_ml = nullptr;
    if (workspace && a.num_partitions > 1) {
        a.part_out = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + kCounterBytes);
        a.part_ml = a.part_out + (size_t)a.num_seqs * a.num_heads * a.num_partitions * head_dim;
    }
}

// Scratch of the entry point that allocates nothing: one array per GPU the
// library runs on, held until the process ends.  In host code `scratch`
// only names the variable; its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the scratch array on the device `stream` runs on.
hipError_t scratch_address(hipStream_t stream, void **ptr) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (back != hipSuccess) return back;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

extern "C" {

const char *pkv_status_string(pkv_status status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL: return "a required pointer is NULL";
        case PKV_ERR_SHAPE: return "sizes are negative or inconsistent";
        case PKV_ERR_DTYPE: return "unsupported dtype or out_dtype";
        case PKV_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, head group or partition size";
        case PKV_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case PKV_ERR_WORKSPACE: return "workspace missing or too small";
        case PKV_ERR_HIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

pkv_status paged_kv_write(const void *key, const void *value, void *key_cache, void *value_cache,
                          const int64_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int64_t num_blocks, pkv_dtype dtype,
                          void *stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return PKV_ERR_SHAPE;
    if (!valid_dtype(dtype)) return PKV_ERR_DTYPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (!pow2_block(block_size)) return PKV_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PKV_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
        return PKV_ERR_ALIGN;
    pkv::WriteArgs a;
    a.key = key;
    a.value = value;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    a.vecs_per_token = (int32_t)(((int64_t)num_kv_heads * head_dim * elem_bytes(dtype)) / 16);
    hipError_t e = pkv::launch_kv_write(a, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t paged_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t partition_size) {
    if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0) return 0;
    const int32_t p = num_partitions(max_context_len, partition_size);
    if (p <= 1) return kCounterBytes;
    return kCounterBytes + (size_t)num_seqs * num_heads * p * (size_t)(head_dim + 2) * sizeof(float);
}

pkv_status paged_decode_attention(void *out, const void *query, const void *key_cache,
                                  const void *value_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  int32_t max_context_len, float scale, int32_t partition_size,
                                  pkv_dtype dtype, pkv_dtype out_dtype, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    pkv::DecodeArgs a;
    bool empty = false;
    pkv_status st = decode_setup(a, empty, false, out, query, key_cache, value_cache, nullptr, nullptr,
                                 block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                                 head_dim, block_size, max_blocks_per_seq, num_blocks,
                                 max_context_len, scale, partition_size, dtype, out_dtype);
    if (st != PKV_OK || empty) return st;
    st = check_workspace(workspace, workspace_bytes, a.num_partitions,
                         paged_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len,
                                                     partition_size));
    if (st != PKV_OK) return st;
    bind_workspace(a, workspace, head_dim);
    hipError_t e = pkv::launch_paged_decode(a, (int)dtype, head_dim,
                                            reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status paged_decode_step(void *out, const void *query, void *key_cache, void *value_cache,
                             const void *new_key, const void *new_value, const int64_t *slot_mapping,
                             const int32_t *block_tables, const int32_t *context_lens, int32_t num_seqs,
                             int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, float scale, int32_t partition_size,
                             pkv_dtype dtype, pkv_dtype out_dtype, void *workspace,
                             size_t workspace_bytes, void *stream) {
    pkv::DecodeArgs a;
    bool empty = false;
    pkv_status st = decode_setup(a, empty, false, out, query, key_cache, value_cache, nullptr, nullptr,
                                 block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                                 head_dim, block_size, max_blocks_per_seq, num_blocks,
                                 max_context_len, scale, partition_size, dtype, out_dtype);
    if (st != PKV_OK || empty) return st;
    if (!new_key || !new_value || !slot_mapping) return PKV_ERR_NULL;
    if (!aligned16(new_key) || !aligned16(new_value)) return PKV_ERR_ALIGN;
    st = check_workspace(workspace, workspace_bytes, a.num_partitions,
                         paged_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len,
                                                     partition_size));
    if (st != PKV_OK) return st;
    bind_workspace(a, workspace, head_dim);
    a.new_key = new_key;
    a.new_value = new_value;
    a.slot_mapping = slot_mapping;
    hipError_t e =
        pkv::launch_paged_decode_step(a, (int)dtype, head_dim, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status paged_decode_attention_noalloc(void *out, const void *query, const void *key_cache,
                                          const void *value_cache, const int32_t *block_tables,
                                          const int32_t *context_lens, int32_t num_seqs,
                                          int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_blocks_per_seq,
                                          int64_t num_blocks, int32_t max_context_len, float scale,
                                          int32_t partition_size, pkv_dtype dtype,
                                          pkv_dtype out_dtype, void *stream) {
    pkv::DecodeArgs a;
    bool empty = false;
    pkv_status st = decode_setup(a, empty, false, out, query, key_cache, value_cache, nullptr, nullptr,
                                 block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                                 head_dim, block_size, max_blocks_per_seq, num_blocks,
                                 max_context_len, scale, partition_size, dtype, out_dtype);
    if (st != PKV_OK || empty) return st;
    if (paged_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len, partition_size) >
        PKV_NOALLOC_SCRATCH_BYTES)
        return PKV_ERR_WORKSPACE;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (scratch_address(s, &ws) != hipSuccess) return PKV_ERR_HIP;
    bind_workspace(a, ws, head_dim);
    hipError_t e = pkv::launch_paged_decode(a, (int)dtype, head_dim, s);
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"

extern "C" {

size_t paged_prefix_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t max_context_len,
                                          int32_t prefix_len, int32_t partition_size) {
    if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        num_heads % num_kv_heads != 0 || prefix_len < 0 || max_context_len < 0 || partition_size < 0)
        return 0;
    const PrefixPlan p = prefix_plan(num_seqs, num_heads, num_kv_heads, max_context_len, prefix_len,
                                     partition_size);
    const int64_t slots = (int64_t)p.num_splits + p.suffix_parts;
    return kCounterBytes + (size_t)num_seqs * num_heads * (size_t)slots * (size_t)(head_dim + 2) * sizeof(float);
}

pkv_status paged_prefix_decode_attention(
    void *out, const void *query, const void *key_cache, const void *value_cache,
    const int32_t *prefix_table, int32_t prefix_len, const int32_t *block_tables,
    const int32_t *context_lens, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, pkv_dtype dtype,
    pkv_dtype out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq < 0 ||
        num_blocks < 0 || max_context_len < 0 || partition_size < 0 || prefix_len < 0)
        return PKV_ERR_SHAPE;
    if (num_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return PKV_ERR_DTYPE;
    if (out_dtype != dtype && out_dtype != PKV_F32) return PKV_ERR_DTYPE;
    if (dtype == PKV_F32 || head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (!pow2_block(block_size)) return PKV_ERR_UNSUPPORTED;
    const int32_t group = num_heads / num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8) return PKV_ERR_UNSUPPORTED;
    if (partition_size != 0 && partition_size % partition_granule(block_size) != 0)
        return PKV_ERR_UNSUPPORTED;
    if (prefix_len % block_size != 0) return PKV_ERR_SHAPE;  // whole pages are shared
    if ((int64_t)prefix_len > (int64_t)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
    if (num_blocks == 0 && (max_context_len > 0 || prefix_len > 0)) return PKV_ERR_SHAPE;
    if (!isfinite(scale)) return PKV_ERR_SHAPE;
    if (num_seqs > PKV_MAX_SEQS) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
        return PKV_ERR_NULL;
    if (prefix_len > 0 && !prefix_table) return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
        return PKV_ERR_ALIGN;

    const PrefixPlan plan = prefix_plan(num_seqs, num_heads, num_kv_heads, max_context_len,
                                        prefix_len, partition_size);
    const int64_t slots = (int64_t)plan.num_splits + plan.suffix_parts;
    if ((int64_t)num_seqs * num_kv_heads * plan.suffix_parts > INT_MAX ||
        (int64_t)num_seqs * num_heads > INT_MAX ||
        (int64_t)plan.row_blocks * plan.num_splits * num_kv_heads > INT_MAX || slots > INT_MAX)
        return PKV_ERR_SHAPE;
    const size_t need = paged_prefix_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                           max_context_len, prefix_len, partition_size);
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    float *part_out = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + kCounterBytes);
    float *part_ml = part_out + (size_t)num_seqs * num_heads * (size_t)slots * head_dim;
    const float sl2 = scale * 1.4426950408889634f;

    pkv::PrefixArgs p = {};
    p.part_out = part_out;
    p.part_ml = part_ml;
    p.query = query;
    p.key_cache = key_cache;
    p.value_cache = value_cache;
    p.prefix_table = prefix_table;
    p.context_lens = context_lens;
    p.num_blocks = num_blocks;
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.log2_group = log2i(group);
    p.block_size = block_size;
    p.log2_block_size = log2i(block_size);
    p.prefix_len = prefix_len;
    p.split_tokens = plan.split_tokens;
    p.num_splits = plan.num_splits;
    p.row_blocks = plan.row_blocks;
    p.part_stride = (int32_t)slots;
    p.scale_log2e = sl2;

    pkv::DecodeArgs a = {};
    a.out = out;
    a.work_counter = reinterpret_cast<unsigned *>(workspace);
    a.part_out = part_out;
    a.part_ml = part_ml;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_blocks = num_blocks;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.log2_block_size = log2i(block_size);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.partition_size = plan.suffix_partition;
    a.num_partitions = plan.suffix_parts;
    a.unit_parts = unit_parts(plan.suffix_parts, plan.suffix_partition, block_size);
    a.scale_log2e = sl2;
    a.out_f32 = out_dtype == PKV_F32 ? 1 : 0;
    a.token_begin = prefix_len;
    a.part_stride = (int32_t)slots;
    a.part_base = plan.num_splits;
    // With a prefix, the prefix units and the suffix decode share one launch
    // and a merge joins every partial; with none, a one-partition suffix
    // stores its output directly.
    a.direct_out = plan.suffix_parts == 1 && plan.num_splits == 0 ? 1 : 0;
    hipError_t e = pkv::launch_paged_prefix_decode(p, a, (int)dtype, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"

extern "C" {

pkv_status paged_kv_write_fp8(const void *key, const void *value, void *key_cache, void *value_cache,
                              const int64_t *slot_mapping, const float *k_scale, const float *v_scale,
                              int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks, pkv_dtype src_dtype,
                              void *stream) {
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0) return PKV_ERR_SHAPE;
    if (!valid_dtype(src_dtype)) return PKV_ERR_DTYPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (!pow2_block(block_size)) return PKV_ERR_UNSUPPORTED;
    if (num_tokens == 0) return PKV_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping || !k_scale || !v_scale)
        return PKV_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
        return PKV_ERR_ALIGN;
    pkv::WriteE4M3Args a;
    a.key = key;
    a.value = value;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.slot_mapping = slot_mapping;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.num_tokens = num_tokens;
    a.num_blocks = num_blocks;
    a.block_size = block_size;
    a.groups_per_token = (int32_t)(((int64_t)num_kv_heads * head_dim) / 8);
    a.groups_per_head = head_dim / 8;
    hipError_t e = pkv::launch_kv_write_e4m3(a, (int)src_dtype, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status paged_decode_attention_fp8(void *out, const void *query, const void *key_cache,
                                      const void *value_cache, const float *k_scale,
                                      const float *v_scale, const int32_t *block_tables,
                                      const int32_t *context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int32_t max_context_len, float scale,
                                      int32_t partition_size, pkv_dtype dtype, pkv_dtype out_dtype,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    pkv::DecodeArgs a;
    bool empty = false;
    pkv_status st = decode_setup(a, empty, true, out, query, key_cache, value_cache, k_scale, v_scale,
                                 block_tables, context_lens, num_seqs, num_heads, num_kv_heads,
                                 head_dim, block_size, max_blocks_per_seq, num_blocks,
                                 max_context_len, scale, partition_size, dtype, out_dtype);
    if (st != PKV_OK || empty) return st;
    st = check_workspace(workspace, workspace_bytes, a.num_partitions,
                         paged_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len,
                                                     partition_size));
    if (st != PKV_OK) return st;
    bind_workspace(a, workspace, head_dim);
    hipError_t e = pkv::launch_paged_decode_e4m3(a, (int)dtype, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"

extern "C" {

pkv_status paged_prefill_attention(void *out, const void *query, const void *key_cache,
                                   const void *value_cache, const int32_t *block_tables,
                                   const int32_t *context_lens, const int32_t *query_start_loc,
                                   int32_t num_seqs, int32_t total_queries, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t max_blocks_per_seq, int64_t num_blocks,
                                   int32_t max_context_len, float scale, pkv_dtype dtype,
                                   pkv_dtype out_dtype, void *stream) {
    if (num_seqs < 0 || total_queries < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
        max_blocks_per_seq < 0 || num_blocks < 0 || max_context_len < 0)
        return PKV_ERR_SHAPE;
    if (num_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return PKV_ERR_DTYPE;
    if (out_dtype != dtype && out_dtype != PKV_F32) return PKV_ERR_DTYPE;
    if (dtype == PKV_F32 || head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (!pow2_block(block_size)) return PKV_ERR_UNSUPPORTED;
    const int32_t group = num_heads / num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8) return PKV_ERR_UNSUPPORTED;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
    if (num_blocks == 0 && max_context_len > 0) return PKV_ERR_SHAPE;
    if (!isfinite(scale)) return PKV_ERR_SHAPE;
    if (num_seqs > PKV_MAX_SEQS) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0 || total_queries == 0) return PKV_OK;
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
        !query_start_loc)
        return PKV_ERR_NULL;
    if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
        return PKV_ERR_ALIGN;
    const int64_t rows = (int64_t)total_queries * group;
    if (((rows + 63) / 64 + num_seqs) * num_kv_heads > INT_MAX || rows * num_kv_heads > INT_MAX)
        return PKV_ERR_SHAPE;
    pkv::PrefillArgs a = {};
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.query_start_loc = query_start_loc;
    a.num_blocks = num_blocks;
    a.num_seqs = num_seqs;
    a.total_queries = total_queries;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.log2_group = log2i(group);
    a.block_size = block_size;
    a.log2_block_size = log2i(block_size);
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.scale_log2e = scale * 1.4426950408889634f;
    a.out_f32 = out_dtype == PKV_F32 ? 1 : 0;
    hipError_t e = pkv::launch_paged_prefill(a, (int)dtype, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
