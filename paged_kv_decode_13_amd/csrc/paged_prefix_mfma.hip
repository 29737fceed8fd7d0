// Shared-prefix decode: a prompt prefix whose pages every sequence of the
// batch shares is read once per KV head for all the batch's query rows, and
// the score and value products over it become dense matrix products on the
// matrix cores.  The rest of each history runs through the paged decode
// loop in the same launch (paged_prefix_fused_kernel, beside the prefix
// units), and a merge kernel joins the partial results by log-sum-exp.
//
// Pages on PagedAttention: "算子与编译器：推理 Attention 与 KV Kernel",
// section "4.1 为什么页面化会改变 kernel 设计" (decode reads page tables,
// in-page offsets and prefix pages that several requests share) and section
// "6. Prefix Cache 与 Attention Kernel 的关系" (shared pages are read-only;
// the access pattern becomes reuse of old pages plus appended new ones).  The
// result is the ordinary paged decode ("实现教学版 PagedAttention：从 block
// table 读取历史 KV cache", section "从 gather 后的 K/V 做 attention") over
// tables whose first prefix_len / block_size entries are the shared pages.
//
// Work unit = (KV head, prefix split, block of kPrefixRowsPerBlock query
// rows); a query row is one (sequence, head of the group) pair, rows ordered
// sequence-major, so the 16 rows of one wave span several sequences.  The
// 64-token chunks of the split go through the LDS machinery of pkv_mqa.h (K
// and V rows in LDS, V read back transposed, scores and values as MFMA
// products, a shared reference max per row); the next chunk's loads are in
// flight while the current one is computed.
//
// Workgroups of one (KV head, split) read the same chunks; the launch order
// places them on the same XCD so the chunk is fetched from HBM once per L2.
#include "pkv_prefix_unit.h"

namespace pkv {

// Log-sum-exp merge of every partial slot of one (sequence, query head):
// the prefix splits, then the suffix partitions.  Writes every output.
template <int DT, int NW, bool EARLY>
__global__ __launch_bounds__(NW * kWave) void prefix_merge_kernel(DecodeArgs a) {
    constexpr int D = 128;
    const int s = blockIdx.x / a.num_heads;
    const int h = blockIdx.x % a.num_heads;
    const int64_t row = (int64_t)s * a.num_heads + h;
    const int ctx = a.context_lens[s];
    EarlyPartials<D> e;
    if constexpr (EARLY) {
        const int k0 = (threadIdx.x / kWave) * kMergeEarly;
        load_early<D>(a, row * a.part_stride + k0, a.part_stride - k0, e);
    }
    if (bad_context(a, ctx) || ctx == 0) {
        const float v = ctx == 0 ? 0.f : __builtin_nanf("");
        for (int d = threadIdx.x; d < D; d += NW * kWave) store_out<DT>(a, row * D + d, v);
        return;
    }
    const int n = a.part_base + seq_units<true>(a, ctx);  // one slot per suffix unit
    if constexpr (EARLY)
        merge_early<DT, D, NW>(a, e, row * a.part_stride, n, row * D);
    else
        merge_partials<DT, D, NW>(a, row * a.part_stride, n, row * D);
}

// The same for rows of at most kMergeEarly slots, one wave per row and
// RW rows (consecutive heads of a sequence) per workgroup (the 128-sequence
// batch: 4096 rows of three slots; call 58.3 -> 57.9 us at block 16).
template <int DT, int RW>
__global__ __launch_bounds__(RW * kWave) void prefix_merge_rows_kernel(DecodeArgs a) {
    constexpr int D = 128;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * RW + threadIdx.x / kWave;
    if (row >= (int64_t)a.num_seqs * a.num_heads) return;  // a whole wave
    const int s = (int)(row / a.num_heads);
    const int ctx = a.context_lens[s];
    EarlyPartials<D> e;
    load_early<D>(a, row * a.part_stride, a.part_stride, e);
    if (bad_context(a, ctx) || ctx == 0) {
        const float v = ctx == 0 ? 0.f : __builtin_nanf("");
        for (int d = lane; d < D; d += kWave) store_out<DT>(a, row * D + d, v);
        return;
    }
    merge_early<DT, D, 1>(a, e, row * a.part_stride, a.part_base + seq_units<true>(a, ctx), row * D);
}

// With a shared prefix, its units and the suffix decode share one launch
// (they overlap: the prefix work is latency-bound, the suffix streams) and
// the merge joins every partial; without one, the suffix decode alone,
// storing the output itself when each suffix is one partition.
template <int DT>
static hipError_t launch_all(const PrefixArgs &p, const DecodeArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)p.row_blocks * p.num_splits * p.num_kv_heads;
    hipError_t e = units > 0 ? launch_paged_prefix_fused(p, a, DT, stream)
                             : launch_paged_decode_mfma_suffix(a, DT, stream);
    if (e != hipSuccess || a.direct_out) return e;
    const unsigned rows = (unsigned)((int64_t)a.num_seqs * a.num_heads);
    constexpr int kRows = 4;
    switch (merge_waves(a.part_stride)) {  // the row's slot capacity
        case 1:
            hipLaunchKernelGGL((prefix_merge_rows_kernel<DT, kRows>), dim3((rows + kRows - 1) / kRows),
                               dim3(kRows * kWave), 0, stream, a);
            break;
        case 2: hipLaunchKernelGGL((prefix_merge_kernel<DT, 2, true>), dim3(rows), dim3(2 * kWave), 0, stream, a); break;
        case kNumWaves:
            hipLaunchKernelGGL((prefix_merge_kernel<DT, kNumWaves, true>), dim3(rows), dim3(kThreads), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL((prefix_merge_kernel<DT, kNumWaves, false>), dim3(rows), dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_paged_prefix_decode(const PrefixArgs &p, const DecodeArgs &a, int dtype,
                                      hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (dtype == kBF16) return launch_all<kBF16>(p, a, stream);
    if (dtype == kF16) return launch_all<kF16>(p, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
