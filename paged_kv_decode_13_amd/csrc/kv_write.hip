// paged_kv_write kernel: each new token's K/V rows are stored at the slot the
// block allocator handed out for them.
//
// Page "实现教学版 PagedAttention：从 block table 读取历史 KV cache", section
// "写入 slot 和读取 block table 必须一致": the slot is (physical_block_id,
// block_offset); the write position must be exactly the read position.  The
// same page, section "attention mask 在哪里": prefill stores the prompt's K/V
// in the blocks, decode stores one token per sequence per step.
//
// A pure copy, bound by HBM: every byte is read once and written once.  One
// slot lookup serves a whole token: a workgroup of 256 threads copies
// 256 / TPT tokens at a time, TPT (a power of two) threads per token
// striding over the token's 16-byte vectors of K then V, so consecutive
// lanes touch consecutive 16 bytes of a row.  Large writes (a prompt's
// thousands of tokens) loop grid-stride over token groups.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

template <int TPT>
__global__ __launch_bounds__(256) void kv_write_kernel(WriteArgs a) {
    constexpr int TOKENS_PER_GROUP = 256 / TPT;
    const int sub = threadIdx.x % TPT;      // lane inside the token's team
    const int team = threadIdx.x / TPT;     // token inside the group
    const int vpt = a.vecs_per_token;       // 16-byte vectors per K (or V) row set
    const u32x4 *key = reinterpret_cast<const u32x4 *>(a.key);
    const u32x4 *value = reinterpret_cast<const u32x4 *>(a.value);
    u32x4 *kc = reinterpret_cast<u32x4 *>(a.key_cache);
    u32x4 *vc = reinterpret_cast<u32x4 *>(a.value_cache);
    for (int64_t token = (int64_t)blockIdx.x * TOKENS_PER_GROUP + team; token < a.num_tokens;
         token += (int64_t)gridDim.x * TOKENS_PER_GROUP) {
        const int64_t slot = a.slot_mapping[token];
        if (slot < 0) continue;
        // slot -> (physical block, offset inside the block)
        const int64_t pb = slot / a.block_size;
        const int64_t off = slot - pb * a.block_size;
        if (pb >= a.num_blocks) continue;
        const int64_t dst = (pb * a.block_size + off) * vpt;
        const int64_t src = token * vpt;
        for (int j = sub; j < vpt; j += TPT) {
            const u32x4 kv = key[src + j];
            const u32x4 vv = value[src + j];
            kc[dst + j] = kv;
            vc[dst + j] = vv;
        }
    }
}

// Quantising variant for E4M3 caches (the pages' first kernel leaves
// quantisation out -- "从正确到更快：PagedAttention 的优化路线", section
// "Triton 适合做什么" -- this is the later version that adds it).  Each
// thread of a token's team converts groups of eight elements: load (16 bytes
// of 16-bit data or 32 bytes of binary32), multiply by the KV head's
// reciprocal scale (correctly rounded 1/scale), saturate to +-448, round to
// nearest even, store 8 bytes.
template <int SDT, int TPT>
__global__ __launch_bounds__(256) void kv_write_e4m3_kernel(WriteE4M3Args a) {
    constexpr int TOKENS_PER_GROUP = 256 / TPT;
    constexpr int SRC_BYTES = SDT == kF32 ? 32 : 16;  // one group of eight source elements
    const int sub = threadIdx.x % TPT;
    const int team = threadIdx.x / TPT;
    const int gpt = a.groups_per_token;
    const char *key = reinterpret_cast<const char *>(a.key);
    const char *value = reinterpret_cast<const char *>(a.value);
    u32x2 *kc = reinterpret_cast<u32x2 *>(a.key_cache);
    u32x2 *vc = reinterpret_cast<u32x2 *>(a.value_cache);
    for (int64_t token = (int64_t)blockIdx.x * TOKENS_PER_GROUP + team; token < a.num_tokens;
         token += (int64_t)gridDim.x * TOKENS_PER_GROUP) {
        const int64_t slot = a.slot_mapping[token];
        if (slot < 0) continue;
        const int64_t pb = slot / a.block_size;
        const int64_t off = slot - pb * a.block_size;
        if (pb >= a.num_blocks) continue;
        const int64_t dst = (pb * a.block_size + off) * gpt;
        const int64_t src = token * gpt;
        for (int j = sub; j < gpt; j += TPT) {
            const int h = j / a.groups_per_head;
            const float kinv = 1.0f / a.k_scale[h];
            const float vinv = 1.0f / a.v_scale[h];
            float kf[8], vf[8];
            if constexpr (SDT == kF32) {
                unpack16<kF32>(load16(key + (src + j) * SRC_BYTES), kf);
                unpack16<kF32>(load16(key + (src + j) * SRC_BYTES + 16), kf + 4);
                unpack16<kF32>(load16(value + (src + j) * SRC_BYTES), vf);
                unpack16<kF32>(load16(value + (src + j) * SRC_BYTES + 16), vf + 4);
            } else {
                unpack16<SDT>(load16(key + (src + j) * SRC_BYTES), kf);
                unpack16<SDT>(load16(value + (src + j) * SRC_BYTES), vf);
            }
            u32x2 kq, vq;
            kq.x = f32x4_to_e4m3(kf[0] * kinv, kf[1] * kinv, kf[2] * kinv, kf[3] * kinv);
            kq.y = f32x4_to_e4m3(kf[4] * kinv, kf[5] * kinv, kf[6] * kinv, kf[7] * kinv);
            vq.x = f32x4_to_e4m3(vf[0] * vinv, vf[1] * vinv, vf[2] * vinv, vf[3] * vinv);
            vq.y = f32x4_to_e4m3(vf[4] * vinv, vf[5] * vinv, vf[6] * vinv, vf[7] * vinv);
            kc[dst + j] = kq;
            vc[dst + j] = vq;
        }
    }
}

template <int SDT>
static hipError_t launch_e4m3(const WriteE4M3Args &a, hipStream_t stream) {
    int tpt = 1;
    while (tpt * 2 <= a.groups_per_token && tpt < 256) tpt *= 2;
    const int64_t per_group = 256 / tpt;
    int64_t groups = (a.num_tokens + per_group - 1) / per_group;
    if (groups > 16384) groups = 16384;
    const dim3 grid((unsigned)groups), block(256);
    switch (tpt) {
        case 1: hipLaunchKernelGGL((kv_write_e4m3_kernel<SDT, 1>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((kv_write_e4m3_kernel<SDT, 2>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((kv_write_e4m3_kernel<SDT, 4>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((kv_write_e4m3_kernel<SDT, 8>), grid, block, 0, stream, a); break;
        case 16: hipLaunchKernelGGL((kv_write_e4m3_kernel<SDT, 16>), grid, block, 0, stream, a); break;
        case 32: hipLaunchKernelGGL((kv_write_e4m3_kernel<SDT, 32>), grid, block, 0, stream, a); break;
        case 64: hipLaunchKernelGGL((kv_write_e4m3_kernel<SDT, 64>), grid, block, 0, stream, a); break;
        case 128: hipLaunchKernelGGL((kv_write_e4m3_kernel<SDT, 128>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((kv_write_e4m3_kernel<SDT, 256>), grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_kv_write_e4m3(const WriteE4M3Args &a, int src_dtype, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    switch (src_dtype) {
        case kF32: return launch_e4m3<kF32>(a, stream);
        case kF16: return launch_e4m3<kF16>(a, stream);
        case kBF16: return launch_e4m3<kBF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_kv_write(const WriteArgs &a, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    // threads per token: the token's vector count rounded down to a power of
    // two, at most 256 (head_dim 64..128, 1+ KV heads: 8..4096 vectors)
    int tpt = 1;
    while (tpt * 2 <= a.vecs_per_token && tpt < 256) tpt *= 2;
    const int64_t per_group = 256 / tpt;
    int64_t groups = (a.num_tokens + per_group - 1) / per_group;
    if (groups > 16384) groups = 16384;  // grid-stride beyond
    const dim3 grid((unsigned)groups), block(256);
    switch (tpt) {
        case 1: hipLaunchKernelGGL(kv_write_kernel<1>, grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(kv_write_kernel<2>, grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL(kv_write_kernel<4>, grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL(kv_write_kernel<8>, grid, block, 0, stream, a); break;
        case 16: hipLaunchKernelGGL(kv_write_kernel<16>, grid, block, 0, stream, a); break;
        case 32: hipLaunchKernelGGL(kv_write_kernel<32>, grid, block, 0, stream, a); break;
        case 64: hipLaunchKernelGGL(kv_write_kernel<64>, grid, block, 0, stream, a); break;
        case 128: hipLaunchKernelGGL(kv_write_kernel<128>, grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL(kv_write_kernel<256>, grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace pkv
