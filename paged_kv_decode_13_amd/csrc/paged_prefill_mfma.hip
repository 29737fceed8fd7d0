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
// Work unit = (sequence, KV head, tile of kPflRows = 192 query rows, 48 per
// wave); a query row is one (query token, head of the group) pair, so a tile
// holds 192 / G consecutive query tokens.  Each unit streams the visible
// history [0, last position of the tile] through the chunk machinery of
// pkv_mqa.h (64 tokens at a time, K and V rows loaded straight into LDS,
// scores and values as MFMA products); each row masks the tokens past its
// own position, so only the chunks on the tile's diagonal carry masking
// work.  Page ids are staged in LDS 512 at a time.  The output is written directly (no partials): a
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

// Chunks arrive through direct-to-LDS loads into two buffers (70 KiB of
// LDS per workgroup, two workgroups per CU): the loads of chunk n + 1 need
// no registers, so each wave holds three 16-row column blocks (one operand
// read from LDS feeds three MFMAs) within the budget of two waves per SIMD.
// Measured on the 32-prompt workload against the earlier design (one LDS
// buffer, the next chunk in registers, two blocks per wave): 6.93-7.00 ->
// 6.26-6.28 ms.  Earlier steps: one block per wave at three workgroups per
// CU 10.9 ms, two blocks 9.5 ms; a software pipeline (the next chunk's score
// MFMAs before this chunk's softmax) reached 256 VGPRs and was slower.
template <int DT, bool SPLIT, bool NARROW>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(mqa_waves_per_simd(kPrefillBlocks), 8)))
void paged_prefill_mfma_kernel(PrefillArgs a) {
    constexpr int D = 128;
    constexpr int ROW = kMqaRowBytes;
    extern __shared__ int s_tpre[];  // [B + 1]: exclusive prefix sum of tiles
    // two chunk buffers, each K rows then V rows in the kMqaDirect layout;
    // separate arrays, so the compiler can tell the reads of one from the
    // loads in flight into the other
    __shared__ __attribute__((aligned(16))) char s_kv0[2 * kMqaDirectBytes];
    __shared__ __attribute__((aligned(16))) char s_kv1[2 * kMqaDirectBytes];
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

    // staging roles: thread lg = tid / 16 loads tokens 4 lg .. 4 lg + 3 of
    // a chunk (one page), 16 bytes of each
    const int lc = tid & 15;
    const int lg = tid >> 4;
    const char *kbase = reinterpret_cast<const char *>(a.key_cache);
    const char *vbase = reinterpret_cast<const char *>(a.value_cache);
    const int64_t tok_stride = (int64_t)a.num_kv_heads * ROW;
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

        const int nch = (seg_end - seg + kMqaChunk - 1) / kMqaChunk;
        // Thread (wave w, lane group qq, lane lc of the group) loads tokens
        // 4 lg + i (lg = 4 w + qq, i = 0..3) straight into LDS in the
        // kMqaDirect layout: load i of wave w fills group i of block w, and
        // the thread's 16 bytes are K chunk lc ^ qq and V chunk lc ^ 2 qq.
        const int qq = lg & 3;
        const int koff = (lc ^ qq) * 16;
        const int voff = (lc ^ (2 * qq)) * 16;
        // Tokens past the segment or on a bad page read page-0 rows (always
        // in the pool): V zeroed after the loads land, scores masked.  The
        // range ends at any token, so validity is per token (bit i: token
        // 4 lg + i).
        auto issue = [&](int t0, char *buf) -> uint32_t {
            const int t = t0 + 4 * lg;
            const int pb = s_pages[min((t - seg) >> lbs, npages - 1)];
            const bool page_ok = (t < seg_end) & (pb >= 0);
            const int page = page_ok ? pb : 0;
            if constexpr (NARROW) {
                // pools under 4 GiB: 32-bit offsets from the pools' bases
                const uint32_t base = ((uint32_t)page * (uint32_t)bs + (uint32_t)(t & (bs - 1))) *
                                          (uint32_t)tok_stride + (uint32_t)(kvh * ROW);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    char *kd = buf + wave * kMqaBlockBytes + i * kMqaGroupBytes;
                    const uint32_t o = base + (uint32_t)i * (uint32_t)tok_stride;
                    __builtin_amdgcn_global_load_lds(kbase + (o + (uint32_t)koff),
                                                     (__attribute__((address_space(3))) void *)kd, 16, 0, 0);
                    __builtin_amdgcn_global_load_lds(vbase + (o + (uint32_t)voff),
                                                     (__attribute__((address_space(3))) void *)(kd + kMqaDirectBytes),
                                                     16, 0, 0);
                }
            } else {
                const int64_t base = ((int64_t)page * bs + (t & (bs - 1))) * tok_stride + (int64_t)kvh * ROW;
                const char *ks = kbase + base + koff;
                const char *vs = vbase + base + voff;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    char *kd = buf + wave * kMqaBlockBytes + i * kMqaGroupBytes;
                    __builtin_amdgcn_global_load_lds(ks + i * tok_stride, (__attribute__((address_space(3))) void *)kd,
                                                     16, 0, 0);
                    __builtin_amdgcn_global_load_lds(vs + i * tok_stride,
                                                     (__attribute__((address_space(3))) void *)(kd + kMqaDirectBytes),
                                                     16, 0, 0);
                }
            }
            const int n_ok = page_ok ? min(4, seg_end - t) : 0;
            return (1u << n_ok) - 1u;
        };
        // chunk n is computed from one buffer while chunk n + 1 loads into
        // the other (one barrier per chunk); unrolled by two so that every
        // step names its two buffers
        uint32_t ok = issue(seg, s_kv0);
        auto step = [&](int n, char *cur, char *nxt) {
            const int t0 = seg + n * kMqaChunk;
            // this thread's loads of chunk n have landed; V rows of tokens
            // that are not valid become zeros (a zero probability times a
            // NaN row would still be NaN), their scores are masked
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (ok != 0xFu) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!((ok >> i) & 1u))
                        *reinterpret_cast<u32x4 *>(cur + kMqaDirectBytes + wave * kMqaBlockBytes +
                                                   i * kMqaGroupBytes + lane * 16) = u32x4{0, 0, 0, 0};
            }
            __syncthreads();  // chunk n is staged; every wave is done with chunk n - 1
            if (n + 1 < nch) ok = issue(t0 + kMqaChunk, nxt);
            mqa_chunk<DT, NB, SPLIT, kMqaDirect>(cur, cur + kMqaDirectBytes, qop, j, q, t0, lim,
                                                  t0 + kMqaChunk > wlim, sl2, st);
        };
        for (int n = 0; n < nch; n += 2) {
            step(n, s_kv0, s_kv1);
            if (n + 1 < nch) step(n + 1, s_kv1, s_kv0);
        }
    }

    if (a.out_f32) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float L = mqa_row_sum<SPLIT>(st[b]);
            if (!row_ok[b]) continue;
            const bool nan = bad || s_badtok < lim[b];
            const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                // four consecutive head dims in one 16-byte store
                f32x4_t v;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = nan ? __builtin_nanf("") : st[b].acc[dt][rr] * inv;
                *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(a.out) + qrow[b] + 16 * dt + 4 * q) = v;
            }
        }
        return;
    }
    // 16-bit outputs: each wave's 16 NB rows go through LDS (the chunk
    // buffers, free once every wave has left the chunk loop), rounded to
    // nearest even by the pair conversion, so that the stores cover whole
    // 256-byte rows.  Rows sit kOutRow bytes apart in LDS (padding spreads
    // the eight-byte writes of one dim group over the banks).
    constexpr int kOutRow = 2 * D + 16;
    static_assert(2 * 16 * NB * kOutRow <= kMqaDirectBytes * 2, "two waves' rows fit one chunk buffer");
    __syncthreads();
    char *ob = (wave < 2 ? s_kv0 : s_kv1) + (wave & 1) * (16 * NB * kOutRow);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float L = mqa_row_sum<SPLIT>(st[b]);
        const bool nan = bad || s_badtok < lim[b];
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            f32x4_t v;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) v[rr] = nan ? __builtin_nanf("") : st[b].acc[dt][rr] * inv;
            *reinterpret_cast<u32x2 *>(ob + (b * 16 + j) * kOutRow + (16 * dt + 4 * q) * 2) =
                u32x2{pack_rne<DT>(v[0], v[1]), pack_rne<DT>(v[2], v[3])};
        }
    }
    // each wave reads back only its own rows (LDS accesses of a wave are
    // in order): lane (row group rg, chunk c) takes 16 bytes of row 4 it + rg
    const int rg = lane >> 4, c = lane & 15;
#pragma unroll
    for (int it = 0; it < 4 * NB; ++it) {
        const int rw = 4 * it + rg;  // row of this wave: block rw / 16, row rw % 16 of it
        const int r = tile * kPflRows + wave * 16 * NB + rw;
        if (r < nrows) {
            const int i = r >> a.log2_group;
            const int h = kvh * G + (r & (G - 1));
            const int64_t orow = ((int64_t)(q0 + i) * a.num_heads + h) * D;
            *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(a.out) + orow + 8 * c) =
                *reinterpret_cast<const u32x4 *>(ob + rw * kOutRow + 16 * c);
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
    // every K or V byte of a pool under 4 GiB is a 32-bit offset from its base
    const bool narrow = (uint64_t)a.num_blocks * (uint64_t)a.block_size * (uint64_t)a.num_kv_heads *
                            (uint64_t)kMqaRowBytes <= 0xFFFFFFFFull;
    const dim3 grid((unsigned)units), block(kThreads);
    if (a.out_f32) {
        if (narrow) hipLaunchKernelGGL((paged_prefill_mfma_kernel<DT, true, true>), grid, block, dyn, stream, a);
        else hipLaunchKernelGGL((paged_prefill_mfma_kernel<DT, true, false>), grid, block, dyn, stream, a);
    } else {
        if (narrow) hipLaunchKernelGGL((paged_prefill_mfma_kernel<DT, false, true>), grid, block, dyn, stream, a);
        else hipLaunchKernelGGL((paged_prefill_mfma_kernel<DT, false, false>), grid, block, dyn, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_paged_prefill(const PrefillArgs &a, int dtype, hipStream_t stream) {
    if (a.num_seqs == 0 || a.total_queries == 0) return hipSuccess;
    if (dtype == kBF16) return launch_dt<kBF16>(a, stream);
    if (dtype == kF16) return launch_dt<kF16>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
