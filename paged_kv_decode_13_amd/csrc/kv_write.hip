// paged_kv_write kernel: each step's new K/V rows are stored at the slot the
// block allocator handed out for them.
//
// Page "实现教学版 PagedAttention：从 block table 读取历史 KV cache", section
// "写入 slot 和读取 block table 必须一致": the slot is (physical_block_id,
// block_offset); the write position must be exactly the read position.
//
// The copy is HBM-bound and tiny for decode (one token per sequence), large
// for a prompt's bulk write.  Work is flattened over 16-byte vectors of all
// tokens' K and V rows so that one grid shape serves both: consecutive lanes
// copy consecutive 16-byte vectors of one token row.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_write_kernel(WriteArgs a) {
    const int64_t per_token = 2 * (int64_t)a.vecs_per_token;  // K then V
    const int64_t total = a.num_tokens * per_token;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total; v += stride) {
        const int64_t token = v / per_token;
        int64_t j = v - token * per_token;
        const int64_t slot = a.slot_mapping[token];
        if (slot < 0) continue;
        // slot -> (physical block, offset inside the block)
        const int64_t pb = slot / a.block_size;
        const int64_t off = slot - pb * a.block_size;
        if (pb >= a.num_blocks) continue;
        const bool is_v = j >= a.vecs_per_token;
        if (is_v) j -= a.vecs_per_token;
        const int64_t dst = (pb * a.block_size + off) * a.vecs_per_token + j;
        const int64_t src = token * a.vecs_per_token + j;
        const u32x4 *s = reinterpret_cast<const u32x4 *>(is_v ? a.value : a.key);
        u32x4 *d = reinterpret_cast<u32x4 *>(is_v ? a.value_cache : a.key_cache);
        d[dst] = s[src];
    }
}

hipError_t launch_kv_write(const WriteArgs &a, hipStream_t stream) {
    if (a.num_tokens == 0) return hipSuccess;
    const int64_t total = a.num_tokens * 2 * (int64_t)a.vecs_per_token;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 8192) blocks = 8192;  // grid-stride beyond ~32 waves per CU
    hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
