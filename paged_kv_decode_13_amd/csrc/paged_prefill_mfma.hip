// Multi-token paged attention with a causal mask: prefill and chunked
// prefill over the paged pool.
//
// Pages on PagedAttention: "实现教学版 PagedAttention：从 block table 读取历史
// KV cache", section "attention mask 在哪里" (a prefill handles the whole
// prompt at once, and each prompt token may only see itself and the tokens
// before it), and "从正确到更快：PagedAttention 的优化路线", section "decode
// attention 和 prefill attention 不一样" (prefill is causal attention over
// the prompt, a large dense product).  Each sequence's q_len new queries are
// the last q_len positions of its context (already written to the pool);
// query i at position p = ctx - q_len + i attends to tokens 0..p through the
// sequence's block table.
//
// Work unit = (sequence, KV head, tile of kPflRows = 128 query rows, 32 per
// wave); a query row is one (query token, head of the group) pair, so a tile
// holds 128 / G consecutive query tokens.  Each unit streams the visible
// history [0, last position of the tile] through the chunk machinery of
// pkv_mqa.h (64 tokens at a time, K and V rows in LDS, scores and values as
// MFMA products); each row masks the tokens past its own position, so only
// the chunks on the tile's diagonal carry masking work.  Page ids are staged
// in LDS 512 at a time.  The output is written directly (no partials): a
// unit sees all of its rows' history.
//
// Precision of the value product: a binary32 output keeps the two-term
// probability split (about 16 / 21 bits of each probability reach the fp32
// accumulators); a 16-bit output, which keeps 8 (bf16) or 11 (fp16)
// significant bits itself, takes each probability rounded once to the
// 16-bit type (relative error u = 2^-8 or 2^-11) and the normaliser summed
// from the same rounded values, so the error it adds to an output element
// is at most u / (1 - u) times (the softmax-weighted mean of |v| over the
// row's history plus |out|), and the value product needs half the MFMAs.
//
// Unit order: a sequence's tiles of one KV head are consecutive and share an
// XCD (they read the same history through one L2), the tiles with the
// longest history first.
#include <limits.h>
#include <math.h>

#include "pkv_mqa.h"

namespace pkv {

constexpr int kPflSegPages = 512;  // page ids staged in LDS at a time
constexpr int kPflRows = kNumWaves * 16 * kPrefillBlocks;  // query rows per tile



// Row tiles of a sequence; 0 when its query range lies outside
// [0, total_queries] (such rows are never read or written).
__device__ __forceinline__ int prefill_tiles(const PrefillArgs &a, int s, int &q0, int &q_len) {
    q0 = a.query_start_loc[s];
    const int q1 = a.query_start_loc[s + 1];
    q_len = q1 - q0;
    if (q0 < 0 || q1 > a.total_queries || q_len <= 0) return 0;
    return ((q_len << a.log2_group) + kPflRows - 1) / kPflRows;
}

// One 37 KiB LDS chunk buffer per workgroup.  With one 16-row block per
// wave three workgroups fit per CU (<= 168 VGPRs) and hid the chunk loads'
// latency better than two with double-buffered LDS (10.9 against 12.8 ms on
// the 32-prompt workload); two blocks per wave at two workgroups per CU
// took it to 9.5 ms, and a second LDS buffer there (one barrier per chunk)
// measured 1.5% slower.  A software pipeline (the next chunk's score MFMAs
// issued before this chunk's softmax, K and V in two-slot LDS rings, one
// barrier per chunk) reached 256 VGPRs, and without registers to prefetch
// LDS operands every MFMA waited on its read: 10.1 against 9.0 ms.
template <int DT, bool SPLIT>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(mqa_waves_per_simd(kPrefillBlocks), 8)))
void paged_prefill_mfma_kernel(PrefillArgs a) {
    constexpr int D = 128;
    constexpr int ROW = kMqaRowBytes;
    extern __shared__ int s_tpre[];  // [B + 1]: exclusive prefix sum of tiles
    __shared__ __attribute__((aligned(16))) char s_k[kMqaChunk * kMqaRowBytes];  // K rows of a chunk
    __shared__ __attribute__((aligned(16))) char s_v[kMqaChunk * kMqaVRow];        // V rows of a chunk
    __shared__ int s_pages[kPflSegPages];
    __shared__ int s_scan[kNumWaves];  // block_scan: one total per wave
    __shared__ int s_badtok;

    const int tid = threadIdx.x;
    const int B = a.num_seqs;
    {
        const int per = (B + kThreads - 1) / kThreads;
        const int lo = min(B, tid * per), hi = min(B, lo + per);
        int n = 0, q0, ql;
        for (int s = lo; s < hi; ++s) n += prefill_tiles(a, s, q0, ql);
        const int inc = block_scan(n, s_scan);
        int run = inc - n;
        for (int s = lo; s < hi; ++s) {
            s_tpre[s] = run;
            run += prefill_tiles(a, s, q0, ql);
        }
        if (tid == kThreads - 1) s_tpre[B] = inc;
        if (tid == 0) s_badtok = INT_MAX;
        __syncthreads();
    }
    const int total_tiles = s_tpre[B];
    const int total_units = total_tiles * a.num_kv_heads;
    if ((int)blockIdx.x >= total_units) return;  // the grid is an upper bound

    const int unit = xcd_unit(blockIdx.x, total_units);
    const int kvh = unit / total_tiles;
    const int T = unit - kvh * total_tiles;
    const int s = search_le(s_tpre, B, T);
    int q0, q_len;
    const int ntiles = prefill_tiles(a, s, q0, q_len);
    const int tile = ntiles - 1 - (T - s_tpre[s]);  // longest history first
    const int ctx = a.context_lens[s];
    const int bs = a.block_size;
    const int lbs = a.log2_block_size;
    const bool bad = ctx < 0 || ctx > a.max_context_len ||
                     (int64_t)ctx > (int64_t)a.max_blocks_per_seq * bs || q_len > ctx;

    // this lane's rows, one per column block b: query token i of the
    // sequence, head g of the group
    constexpr int NB = kPrefillBlocks;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int j = lane & 15;
    const int q = lane >> 4;
    const int G = 1 << a.log2_group;
    const int nrows = q_len << a.log2_group;
    // the tile's last query sees the most: the unit's token range
    const int i_last = min(q_len - 1, (tile * kPflRows + kPflRows - 1) >> a.log2_group);
    const int tok_end = bad ? 0 : ctx - q_len + i_last + 1;
    bool row_ok[NB];
    int lim[NB];
    int64_t qrow[NB];
    u32x4 qop[NB][4];
    int wlim = INT_MAX;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int r = tile * kPflRows + wave * 16 * NB + b * 16 + j;
        row_ok[b] = r < nrows;
        const int i = row_ok[b] ? (r >> a.log2_group) : 0;
        const int h = kvh * G + (r & (G - 1));
        lim[b] = row_ok[b] ? ctx - q_len + i + 1 : tok_end;  // padding rows compute, never store
        wlim = min(wlim, lim[b]);
        qrow[b] = ((int64_t)(q0 + i) * a.num_heads + h) * D;
        const char *row = reinterpret_cast<const char *>(a.query) + qrow[b] * 2;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qop[b][kk] = row_ok[b] ? load16(row + (4 * kk + q) * 16) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) wlim = min(wlim, __shfl_xor(wlim, off));
    wlim = __builtin_amdgcn_readfirstlane(wlim);
    const float sl2 = mqa_positive_scale<NB>(a.scale_log2e, qop);

    // staging roles as in the shared-prefix kernel
    const int lc = tid & 15;
    const int lg = tid >> 4;
    const char *kbase = reinterpret_cast<const char *>(a.key_cache);
    const char *vbase = reinterpret_cast<const char *>(a.value_cache);
    const int64_t tok_stride = (int64_t)a.num_kv_heads * ROW;
    const int64_t lane_off = (int64_t)kvh * ROW + lc * 16;
    const int32_t *table = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

    MqaRowState st[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) mqa_init(st[b]);

    for (int seg = 0; seg < tok_end; seg += kPflSegPages << lbs) {
        const int seg_end = min(tok_end, seg + (kPflSegPages << lbs));
        const int npages = (seg_end - seg + bs - 1) >> lbs;
        __syncthreads();  // the previous segment's chunks are done with s_pages
        for (int k = tid; k < npages; k += kThreads) {
            int pb = table[(seg >> lbs) + k];
            if (pb < 0 || (int64_t)pb >= a.num_blocks) {
                atomicMin(&s_badtok, seg + (k << lbs));
                pb = -1;
            }
            s_pages[k] = pb;
        }
        __syncthreads();

        // tokens past the segment or on a bad page read page-0 rows (always
        // in the pool): V staged as zeros, scores masked.  The range ends at
        // any token, so validity is per token (bit k: token 4 lg + k).
        auto load_chunk = [&](int t0, u32x4 (&kr)[4], u32x4 (&vr)[4]) -> uint32_t {
            const int t = t0 + 4 * lg;
            const int pb = s_pages[min((t - seg) >> lbs, npages - 1)];
            const bool page_ok = (t < seg_end) & (pb >= 0);
            const int64_t base = ((int64_t)(page_ok ? pb : 0) * bs + (t & (bs - 1))) * tok_stride + lane_off;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                kr[k] = load16(kbase + base + k * tok_stride);
                vr[k] = load16(vbase + base + k * tok_stride);
            }
            const int n_ok = page_ok ? min(4, seg_end - t) : 0;
            return (1u << n_ok) - 1u;
        };
        const int nch = (seg_end - seg + kMqaChunk - 1) / kMqaChunk;
        // chunk n is computed from the LDS buffer while chunk n + 1 is in
        // flight in registers (one buffer, two barriers per chunk)
        u32x4 kr[4], vr[4];
        uint32_t ok = load_chunk(seg, kr, vr);
        for (int n = 0; n < nch; ++n) {
            const int t0 = seg + n * kMqaChunk;
            mqa_store_chunk(s_k, s_v, lc, lg, kr, vr, ok);
            __syncthreads();
            ok = load_chunk(t0 + kMqaChunk, kr, vr);
            __builtin_amdgcn_sched_barrier(0);
            mqa_chunk<DT, NB, SPLIT>(s_k, s_v, qop, j, q, t0, lim, t0 + kMqaChunk > wlim, sl2, st);
            __syncthreads();
        }
    }

#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float L = mqa_row_sum<SPLIT>(st[b]);
        if (!row_ok[b]) continue;
        const bool nan = bad || s_badtok < lim[b];
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const int64_t o = qrow[b] + 16 * dt + 4 * q;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const float v = nan ? __builtin_nanf("") : st[b].acc[dt][rr] * inv;
                if (a.out_f32)
                    reinterpret_cast<float *>(a.out)[o + rr] = v;
                else
                    reinterpret_cast<uint16_t *>(a.out)[o + rr] = f32_to_bits16<DT>(v);
            }
        }
    }
}

template <int DT>
static hipError_t launch_dt(const PrefillArgs &a, hipStream_t stream) {
    // upper bound of the units: each sequence's last tile may be partial
    const int64_t rows = ((int64_t)a.total_queries << a.log2_group);
    const int64_t units = ((rows + kPflRows - 1) / kPflRows + a.num_seqs) * a.num_kv_heads;
    if (units == 0) return hipSuccess;
    const size_t dyn = (size_t)(a.num_seqs + 1) * sizeof(int);
    if (a.out_f32)
        hipLaunchKernelGGL((paged_prefill_mfma_kernel<DT, true>), dim3((unsigned)units), dim3(kThreads), dyn,
                           stream, a);
    else
        hipLaunchKernelGGL((paged_prefill_mfma_kernel<DT, false>), dim3((unsigned)units), dim3(kThreads), dyn,
                           stream, a);
    return hipGetLastError();
}

hipError_t launch_paged_prefill(const PrefillArgs &a, int dtype, hipStream_t stream) {
    if (a.num_seqs == 0 || a.total_queries == 0) return hipSuccess;
    if (dtype == kBF16) return launch_dt<kBF16>(a, stream);
    if (dtype == kF16) return launch_dt<kF16>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
