// Shared-prefix decode: a prompt prefix whose pages every sequence of the
// batch shares is read once per KV head for all the batch's query rows, and
// the score and value products over it become dense matrix products on the
// matrix cores.  The rest of each history runs through the paged decode
// kernel, whose epilogue joins the prefix's partial results by log-sum-exp
// when each suffix is one partition; otherwise a merge kernel joins them.
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
// Work unit = (KV head, prefix split, block of 64 query rows); a query row
// is one (sequence, head of the group) pair, rows ordered sequence-major, so
// the 16 rows of one wave span several sequences.  Per 64-token chunk of the
// split the workgroup stages K and V in LDS once for its four waves:
//  - K keeps its row layout (16-byte chunks XOR-swizzled by token); the
//    score MFMA reads lane (i, q) = token i, head-dim chunk 4kk + q, and the
//    query operand (registers, loaded once) uses the same chunk order:
//        S^T[16 tokens x 16 rows] = K[16 x 128] . Q^T[128 x 16].
//  - V is transposed while it is staged (V^T[d][token], tokens of a
//    32-token block interleaved so that one 16-byte read gives a lane the
//    eight tokens whose probabilities it already holds), and the value
//    product is
//        O^T[16 d x 16 rows] += V^T[16 x 32 tokens] . P^T[32 x 16].
//    The probabilities in (0, 1] enter the 16-bit MFMA as a two-term split
//    p = hi + lo (hi = p rounded to the cache type, lo = the remainder
//    rounded), so the product keeps about 16 (bf16) or 22 (fp16) bits of p
//    and the accumulation is fp32, as in the decode kernel.
//  - The reference max is shared by the four lane groups of a row (two lane
//    shuffles per chunk), so every probability of a chunk is relative to the
//    same max and the value product can sum across lane groups.  It moves
//    only when passed by more than 2^8, so the fp32 accumulators are rarely
//    rescaled; the merge weights partials by their own (max, normaliser)
//    pair, so any reference max gives the same result.
// Loads of the next chunk are in flight while the current one is computed
// (register staging, two LDS buffers, one barrier per chunk).
//
// Workgroups of one (KV head, split) read the same 64-token chunks; the
// launch order places them on the same XCD (consecutive workgroup ids go to
// different XCDs) so the chunk is fetched from HBM once per L2.
#include <limits.h>
#include <math.h>

#include "pkv_decode_common.h"
#include "pkv_mfma.h"

namespace pkv {

constexpr int kPfxWaveRows = 16;                    // query rows per wave
constexpr int kPfxRows = kNumWaves * kPfxWaveRows;  // query rows per workgroup
constexpr int kPfxChunk = 64;                       // prefix tokens per LDS chunk
constexpr int kPfxMaxSplitTokens = 2048;            // matches the host-side plan
constexpr int kPfxMaxSplitPages = kPfxMaxSplitTokens / 4;
constexpr int kXcds = 8;

// 16-byte column of transposed-V row d that holds column `col`: XOR swizzle
// so that the transposing writes (rows 8c + e) and the operand reads (rows
// 16 dt + i) both spread over the LDS banks.
__device__ __forceinline__ int vt_swz(int d, int col) { return col ^ ((d ^ (d >> 3)) & 7); }

// Two probabilities -> packed 16-bit pairs (hi, lo) with hi + lo = p to
// about 16 (bf16: hardware round-to-nearest-even both times) or 21 (fp16:
// hardware pack with round toward zero; the remainder carries the rest)
// significant bits.
template <int DT>
__device__ __forceinline__ void split_pack(float p0, float p1, uint32_t &hi, uint32_t &lo) {
    if constexpr (DT == kBF16) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t h = {(__bf16)p0, (__bf16)p1};
        hi = __builtin_bit_cast(uint32_t, h);
        const float r0 = p0 - __uint_as_float(hi << 16);
        const float r1 = p1 - __uint_as_float(hi & 0xffff0000u);
        const bf16x2_t l = {(__bf16)r0, (__bf16)r1};
        lo = __builtin_bit_cast(uint32_t, l);
    } else {
        const auto h = __builtin_amdgcn_cvt_pkrtz(p0, p1);
        hi = __builtin_bit_cast(uint32_t, h);
        const float r0 = p0 - (float)h[0];
        const float r1 = p1 - (float)h[1];
        lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
    }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void paged_prefix_mfma_kernel(PrefixArgs a) {
    constexpr int D = 128;
    constexpr int ROW = D * 2;              // bytes of one K or V row
    constexpr int VT_ROW = kPfxChunk * 2;   // bytes of one transposed-V row
    __shared__ __attribute__((aligned(16))) char s_k[2][kPfxChunk * ROW];
    __shared__ __attribute__((aligned(16))) char s_vt[2][D * VT_ROW];
    __shared__ int s_pages[kPfxMaxSplitPages];
    __shared__ int s_badtok;

    // workgroup id -> unit, units of one (KV head, split) on one XCD
    const int nwg = gridDim.x;
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int per = nwg / kXcds, rem = nwg % kXcds;
    const int unit = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
    const int rb = unit % a.row_blocks;
    const int rest = unit / a.row_blocks;
    const int split = rest % a.num_splits;
    const int kvh = rest / a.num_splits;

    const int bs = a.block_size;
    const int lbs = a.log2_block_size;
    const int tok_begin = split * a.split_tokens;
    const int tok_end = min(a.prefix_len, tok_begin + a.split_tokens);
    const int npages = (tok_end - tok_begin) >> lbs;  // split bounds are page aligned

    const int tid = threadIdx.x;

    // this lane's query row (MFMA column j) and how far into the prefix it
    // sees; its loads are issued before the page-id staging so that the two
    // round trips overlap
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int j = lane & 15;
    const int q = lane >> 4;
    const int G = 1 << a.log2_group;
    const int nrows = a.num_seqs << a.log2_group;
    const int r = rb * kPfxRows + wave * kPfxWaveRows + j;
    const bool row_ok = r < nrows;
    const int s = row_ok ? (r >> a.log2_group) : 0;
    const int h = kvh * G + (r & (G - 1));
    const int ctx = row_ok ? a.context_lens[s] : tok_end;  // padding rows compute, never store
    u32x4 qop[4];
    {
        const char *row = reinterpret_cast<const char *>(a.query) + ((int64_t)s * a.num_heads + h) * ROW;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qop[kk] = row_ok ? load16(row + (4 * kk + q) * 16) : u32x4{0, 0, 0, 0};
    }

    if (tid == 0) s_badtok = INT_MAX;
    __syncthreads();
    for (int i = tid; i < npages; i += kThreads) {
        int pb = a.prefix_table[(tok_begin >> lbs) + i];
        if (pb < 0 || (int64_t)pb >= a.num_blocks) {
            atomicMin(&s_badtok, tok_begin + (i << lbs));
            pb = -1;
        }
        s_pages[i] = pb;
    }
    __syncthreads();

    const int lim = min(max(ctx, 0), tok_end);  // tokens t < lim are this row's
    int wlim = lim;  // smallest limit over the wave's rows
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) wlim = min(wlim, __shfl_xor(wlim, off));
    wlim = __builtin_amdgcn_readfirstlane(wlim);

    // staging roles: thread (lg, lc) moves 16-byte chunk lc of tokens
    // 4 lg .. 4 lg + 3 of a chunk (one page: pages hold >= 4 tokens)
    const int lc = tid & 15;
    const int lg = tid >> 4;
    const char *kbase = reinterpret_cast<const char *>(a.key_cache);
    const char *vbase = reinterpret_cast<const char *>(a.value_cache);
    const int64_t tok_stride = (int64_t)a.num_kv_heads * ROW;
    const int64_t lane_off = (int64_t)kvh * ROW + lc * 16;

    // Tokens past the split or on a bad page id read a row of page 0 (always
    // in the pool); their V is zeroed when staged and their scores masked.
    auto load_chunk = [&](int t0, u32x4 (&kr)[4], u32x4 (&vr)[4]) -> bool {
        const int t = t0 + 4 * lg;
        const int pb = s_pages[min((t - tok_begin) >> lbs, npages - 1)];
        const bool ok = (t < tok_end) & (pb >= 0);
        const int64_t base = ((int64_t)(ok ? pb : 0) * bs + (t & (bs - 1))) * tok_stride + lane_off;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kr[i] = load16(kbase + base + i * tok_stride);
            vr[i] = load16(vbase + base + i * tok_stride);
        }
        return ok;
    };
    auto store_chunk = [&](int buf, const u32x4 (&kr)[4], const u32x4 (&vin)[4], bool ok) {
        char *kt = s_k[buf];
        char *vt = s_vt[buf];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tt = 4 * lg + i;
            *reinterpret_cast<u32x4 *>(kt + tt * ROW + ((lc ^ tt) & 15) * 16) = kr[i];
        }
        u32x4 vr[4] = {vin[0], vin[1], vin[2], vin[3]};
        if (__builtin_amdgcn_ballot_w64(!ok)) {  // only the last chunk of a split
#pragma unroll
            for (int i = 0; i < 4; ++i) vr[i] = ok ? vr[i] : u32x4{0, 0, 0, 0};
        }
        // tokens 4 lg .. +3 sit in block lg / 8 (32 tokens), tile (lg / 4) & 1
        // of the block, row group lg & 3 of the tile
        const int col = ((lg >> 3) << 2) | (lg & 3);
        const int half = (lg >> 2) & 1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // word w of a row holds head dims 8 lc + 2w (low half) and + 1 (high
            // half); gather each across the four tokens: v_perm picks 16-bit
            // halves of two registers
            uint2 ev, od;
            ev.x = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x05040100u);
            ev.y = __builtin_amdgcn_perm(vr[3][w], vr[2][w], 0x05040100u);
            od.x = __builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x07060302u);
            od.y = __builtin_amdgcn_perm(vr[3][w], vr[2][w], 0x07060302u);
            const int d0 = 8 * lc + 2 * w;
            *reinterpret_cast<uint2 *>(vt + d0 * VT_ROW + vt_swz(d0, col) * 16 + half * 8) = ev;
            *reinterpret_cast<uint2 *>(vt + (d0 + 1) * VT_ROW + vt_swz(d0 + 1, col) * 16 + half * 8) = od;
        }
    };

    const float sl2 = a.scale_log2e;
    float m = -INFINITY;  // running max of row j (equal in the four lane groups)
    float lsum = 0.f;     // this lane's share of the normaliser
    f32x4_t acc[8];       // O^T: head dims 16 dt + 4q + r of row j
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf, int t0) {
        const char *kt = s_k[buf];
        const char *vt = s_vt[buf];
        float sc[4][4];  // [16-token tile][r]: token tile*16 + 4q + r, row j
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const u32x4 kop = *reinterpret_cast<const u32x4 *>(
                    kt + (tt * 16 + j) * ROW + (((4 * kk + q) ^ j) & 15) * 16);
                sacc = mfma_16x16x32<DT>(kop, qop[kk], sacc);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sc[tt][rr] = sacc[rr] * sl2;
        }
        if (t0 + kPfxChunk > wlim) {
            // some token of the chunk lies past some row's limit (the empty
            // asm keeps this a branch: full chunks skip the masking)
            asm volatile("" ::: "memory");
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    sc[tt][rr] = (t0 + tt * 16 + 4 * q + rr < lim) ? sc[tt][rr] : -INFINITY;
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, sc[tt][rr]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // The reference max moves only when a row's max passes it by more
        // than kMaxSlack, so most chunks skip the rescale of the accumulators
        // (probabilities then stay below 2^kMaxSlack).  m = -inf until the
        // row has seen a valid token.
        const bool bump = mx > m + kMaxSlack;
        if (__builtin_amdgcn_ballot_w64(bump)) {
            const float alpha = !bump ? 1.f : (m == -INFINITY ? 0.f : fast_exp2(m - mx));
            m = bump ? mx : m;
            lsum *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
        }
        // a row with m = -inf has only masked scores here: 2^(-inf - 0) = 0
        const float mref = m == -INFINITY ? 0.f : m;
        float ps = 0.f;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                sc[tt][rr] = fast_exp2(sc[tt][rr] - mref);
                ps += sc[tt][rr];
            }
        lsum += ps;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            // B operand: tokens (tile 2bb, 4q + e) for e < 4, (tile 2bb+1, 4q + e - 4) after
            uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
            split_pack<DT>(sc[2 * bb][0], sc[2 * bb][1], h0, l0);
            split_pack<DT>(sc[2 * bb][2], sc[2 * bb][3], h1, l1);
            split_pack<DT>(sc[2 * bb + 1][0], sc[2 * bb + 1][1], h2, l2);
            split_pack<DT>(sc[2 * bb + 1][2], sc[2 * bb + 1][3], h3, l3);
            const u32x4 ph = {h0, h1, h2, h3};
            const u32x4 pl = {l0, l1, l2, l3};
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const int d = 16 * dt + j;
                const u32x4 vop = *reinterpret_cast<const u32x4 *>(vt + d * VT_ROW + vt_swz(d, bb * 4 + q) * 16);
                acc[dt] = mfma_16x16x32<DT>(vop, ph, acc[dt]);
                acc[dt] = mfma_16x16x32<DT>(vop, pl, acc[dt]);
            }
        }
    };

    // Chunk n is computed from LDS buffer n % 2 while chunk n + 1 is in
    // flight in registers; loads are unconditional (a chunk past the split
    // reads page-0 rows and stages zeros) so that the compiler counts
    // outstanding loads exactly.
    const int nch = (tok_end - tok_begin + kPfxChunk - 1) / kPfxChunk;
    u32x4 kr[4], vr[4];
    bool ok = load_chunk(tok_begin, kr, vr);
    store_chunk(0, kr, vr, ok);
    __syncthreads();
    for (int n = 0; n < nch; ++n) {
        const int t0 = tok_begin + n * kPfxChunk;
        ok = load_chunk(t0 + kPfxChunk, kr, vr);
        // keep the next chunk's loads ahead of this chunk's compute
        __builtin_amdgcn_sched_barrier(0);
        compute(n & 1, t0);
        store_chunk((n + 1) & 1, kr, vr, ok);
        __syncthreads();
    }

    float L = lsum + __shfl_xor(lsum, 16);
    L += __shfl_xor(L, 32);
    if (row_ok) {
        const int64_t slot = ((int64_t)s * a.num_heads + h) * a.part_stride + split;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        float *po = a.part_out + slot * D + 4 * q;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4_t *>(po + 16 * dt) = acc[dt] * inv;
        if (q == 0) {
            a.part_ml[slot * 2] = s_badtok < lim ? __builtin_nanf("") : m;
            a.part_ml[slot * 2 + 1] = L;
        }
    }
}

// Log-sum-exp merge of every partial slot of one (sequence, query head):
// the prefix splits, then the suffix partitions.  Writes every output.
template <int DT>
__global__ __launch_bounds__(kWave) void prefix_merge_kernel(DecodeArgs a) {
    constexpr int D = 128;
    constexpr int PER_LANE = D / kWave;
    const int s = blockIdx.x / a.num_heads;
    const int h = blockIdx.x % a.num_heads;
    const int lane = threadIdx.x;
    const int ctx = a.context_lens[s];
    const int64_t obase = ((int64_t)s * a.num_heads + h) * D;
    if (bad_context(a, ctx) || ctx == 0) {
        const float v = ctx == 0 ? 0.f : __builtin_nanf("");
#pragma unroll
        for (int jj = 0; jj < PER_LANE; ++jj) store_out<DT>(a, obase + lane + jj * kWave, v);
        return;
    }
    const int n = a.part_base + seq_parts<true>(a, ctx);
    const int64_t base = ((int64_t)s * a.num_heads + h) * a.part_stride;
    float M = -INFINITY;
    for (int p = 0; p < n; ++p) M = fmaxf(M, a.part_ml[(base + p) * 2]);
    float L = 0.f, O[PER_LANE];
#pragma unroll
    for (int jj = 0; jj < PER_LANE; ++jj) O[jj] = 0.f;
    for (int p = 0; p < n; ++p) {
        const float w = a.part_ml[(base + p) * 2 + 1] * fast_exp2(a.part_ml[(base + p) * 2] - M);
        L += w;
#pragma unroll
        for (int jj = 0; jj < PER_LANE; ++jj) O[jj] = fmaf(w, a.part_out[(base + p) * D + lane + jj * kWave], O[jj]);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int jj = 0; jj < PER_LANE; ++jj) store_out<DT>(a, obase + lane + jj * kWave, O[jj] * inv);
}

template <int DT>
static hipError_t launch_all(const PrefixArgs &p, const DecodeArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)p.row_blocks * p.num_splits * p.num_kv_heads;
    if (units > 0) {
        hipLaunchKernelGGL(paged_prefix_mfma_kernel<DT>, dim3((unsigned)units), dim3(kThreads), 0,
                           stream, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipError_t e = launch_paged_decode_mfma_suffix(a, DT, stream);
    if (e != hipSuccess || a.fold_prefix) return e;
    const int64_t rows = (int64_t)a.num_seqs * a.num_heads;
    hipLaunchKernelGGL(prefix_merge_kernel<DT>, dim3((unsigned)rows), dim3(kWave), 0, stream, a);
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
