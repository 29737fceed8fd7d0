// One unit of the shared-prefix score/value work (KV head, prefix split,
// block of kPrefixRowsPerBlock query rows), written as a device function
// over an LDS struct the kernel provides: the shared-prefix launch runs
// these units on its first workgroups, beside the suffix decode, and the
// two share their LDS as a union.
//
// Pages on PagedAttention: "算子与编译器：推理 Attention 与 KV Kernel",
// sections "4.1 为什么页面化会改变 kernel 设计" and "6. Prefix Cache 与
// Attention Kernel 的关系".  Rows, chunks and the partial results are as
// described in paged_prefix_mfma.hip.
#pragma once

#include <limits.h>
#include <math.h>

#include "pkv_mqa.h"

namespace pkv {

constexpr int kPfxMaxSplitTokens = 2048;  // matches the host-side plan
constexpr int kPfxMaxSplitPages = kPfxMaxSplitTokens / 4;

// LDS of one prefix unit: the K and V rows of a 64-token chunk, the split's
// page ids and the first token on a bad page id.
struct PrefixLds {
    __attribute__((aligned(16))) char k[kMqaChunk * kMqaRowBytes];
    __attribute__((aligned(16))) char v[kMqaChunk * kMqaVRow];
    int pages[kPfxMaxSplitPages];
    int badtok;
};

template <int DT>
__device__ __forceinline__ void prefix_unit(const PrefixArgs &a, const int unit, PrefixLds &L) {
    constexpr int D = 128;
    constexpr int ROW = kMqaRowBytes;
    char *s_k = L.k;
    char *s_v = L.v;
    int *s_pages = L.pages;
    int &s_badtok = L.badtok;

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

    // this lane's query rows (MFMA column j of each column block b) and how
    // far into the prefix they see; their loads are issued before the
    // page-id staging so that the two round trips overlap
    constexpr int NB = kPrefixBlocks;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int j = lane & 15;
    const int q = lane >> 4;
    const int G = 1 << a.log2_group;
    const int nrows = a.num_seqs << a.log2_group;
    bool row_ok[NB];
    int64_t hrow[NB];  // (sequence, query head) row of the output and partials
    int ctx[NB];
    u32x4 qop[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int r = rb * kPrefixRowsPerBlock + wave * 16 * NB + b * 16 + j;
        row_ok[b] = r < nrows;
        const int s = row_ok[b] ? (r >> a.log2_group) : 0;
        const int h = kvh * G + (r & (G - 1));
        hrow[b] = (int64_t)s * a.num_heads + h;
        ctx[b] = row_ok[b] ? a.context_lens[s] : tok_end;  // padding rows compute, never store
        const char *row = reinterpret_cast<const char *>(a.query) + hrow[b] * ROW;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qop[b][kk] = row_ok[b] ? load16(row + (4 * kk + q) * 16) : u32x4{0, 0, 0, 0};
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

    int lim[NB];  // tokens t < lim are the row's
    int wlim = INT_MAX;  // smallest limit over the wave's rows
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        lim[b] = min(max(ctx[b], 0), tok_end);
        wlim = min(wlim, lim[b]);
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) wlim = min(wlim, __shfl_xor(wlim, off));
    wlim = __builtin_amdgcn_readfirstlane(wlim);
    const float sl2 = mqa_positive_scale<NB>(a.scale_log2e, qop);

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
    // (split bounds are page aligned and pages hold >= 4 tokens: a thread's
    // four tokens are all valid or all not)
    auto load_chunk = [&](int t0, u32x4 (&kr)[4], u32x4 (&vr)[4]) -> uint32_t {
        const int t = t0 + 4 * lg;
        const int pb = s_pages[min((t - tok_begin) >> lbs, npages - 1)];
        const bool ok = (t < tok_end) & (pb >= 0);
        const int64_t base = ((int64_t)(ok ? pb : 0) * bs + (t & (bs - 1))) * tok_stride + lane_off;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kr[i] = load16(kbase + base + i * tok_stride);
            vr[i] = load16(vbase + base + i * tok_stride);
        }
        return ok ? 0xFu : 0u;
    };

    MqaRowState st[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) mqa_init(st[b]);

    // Chunk n is computed from the LDS buffer while chunk n + 1 is in flight
    // in registers (two barriers per chunk); loads are unconditional (a
    // chunk past the split reads page-0 rows and stages zeros) so that the
    // compiler counts outstanding loads exactly.
    const int nch = (tok_end - tok_begin + kMqaChunk - 1) / kMqaChunk;
    u32x4 kr[4], vr[4];
    uint32_t ok = load_chunk(tok_begin, kr, vr);
    for (int n = 0; n < nch; ++n) {
        const int t0 = tok_begin + n * kMqaChunk;
        mqa_store_chunk(s_k, s_v, lc, lg, kr, vr, ok);
        __syncthreads();
        ok = load_chunk(t0 + kMqaChunk, kr, vr);
        // keep the next chunk's loads ahead of this chunk's compute
        __builtin_amdgcn_sched_barrier(0);
        mqa_chunk<DT, NB>(s_k, s_v, qop, j, q, t0, lim, t0 + kMqaChunk > wlim, sl2, st);
        __syncthreads();
    }

#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float L = mqa_row_sum(st[b]);
        if (!row_ok[b]) continue;
        const int64_t slot = hrow[b] * a.part_stride + split;
        const float inv = L > 0.f ? 1.f / L : 0.f;
        float *po = a.part_out + slot * D + 4 * q;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4_t *>(po + 16 * dt) = st[b].acc[dt] * inv;
        if (q == 0) {
            a.part_ml[slot * 2] = s_badtok < lim[b] ? __builtin_nanf("") : st[b].m;
            a.part_ml[slot * 2 + 1] = L;
        }
    }
}

}  // namespace pkv
