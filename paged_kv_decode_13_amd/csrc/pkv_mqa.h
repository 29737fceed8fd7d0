// Chunk machinery shared by the multi-query MFMA kernels (the shared-prefix
// kernel and the prefill kernel): a workgroup of four waves holds
// 4 x 16 x NB query rows (NB MFMA column blocks of 16 rows per wave) and
// streams the K/V rows of one KV head through LDS 64 tokens at
// a time, 16-bit caches, head_dim 128.  Every K or V operand a wave reads
// from LDS feeds the MFMAs of all its column blocks.  A chunk is staged from
// registers (the shared-prefix kernel) or placed by direct-to-LDS loads (the
// prefill kernel); the two LDS layouts are described below, the arithmetic
// is the same.
//
//  - K keeps its row layout in LDS (16-byte chunks XOR-swizzled by token);
//    the score MFMA reads lane (i, q) = token i, head-dim chunk 4kk + q, and
//    the query operand uses the same chunk order:
//        S^T[16 tokens x 16 rows] = K[16 x 128] . Q^T[128 x 16].
//  - V also keeps its row layout in LDS (rows padded to 288 bytes when
//    staged from registers), and the value MFMA reads it transposed with the gfx950 LDS transpose load
//    (ds_read_b64_tr_b16: within each 16-lane group, output lane 4a + b
//    receives element b of the 8-byte pieces that lanes a, a + 4, a + 8,
//    a + 12 point at), so a lane gathers the eight tokens whose
//    probabilities it already holds from two such loads:
//        O^T[16 d x 16 rows] += V^T[16 x 32 tokens] . P^T[32 x 16].
//    The padding puts rows 32 bytes apart in the banks: both the 16-byte
//    row stores and the transposed loads are free of bank conflicts (the
//    direct layout gets the same from padding per load and a per-row XOR).
//    With SPLIT the probabilities enter the 16-bit MFMA as a two-term split
//    p = hi + lo, so the product keeps about 16 (bf16) or 21 (fp16) bits of p;
//    without it p is rounded once to the 16-bit type (nearest even: relative
//    error at most 2^-8 for bf16, 2^-11 for fp16), which halves the value
//    product's MFMAs, and the row's normaliser is summed by the matrix cores
//    from the same rounded values.  The accumulation is fp32 either way.
//  - One reference max per row, shared by the row's four lane groups (two
//    lane swaps per chunk), so every probability of a chunk is relative to
//    the same max and the value product can sum across lane groups.  It
//    moves only when passed by more than 2^kMaxSlack, so the accumulators
//    are rarely rescaled.
#pragma once

#include <math.h>

#include "pkv_decode_common.h"
#include "pkv_mfma.h"

namespace pkv {

// Register budget of a kernel with NB column blocks per wave: three waves
// per SIMD with one block, two with more.
constexpr int mqa_waves_per_simd(int nb) { return nb == 1 ? 3 : 2; }
constexpr int kMqaChunk = 64;                       // tokens per LDS chunk
constexpr int kMqaRowBytes = 256;                   // one 16-bit K or V row (D = 128)
constexpr int kMqaVRow = kMqaRowBytes + 32;        // padded V row in LDS

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// LDS layouts of a staged 64-token chunk.
//  kMqaRegStaged: written from registers (mqa_store_chunk): K row t at
//    t * 256 with 16-byte chunk c at (c ^ t) & 15; V row t at t * 288
//    (padded rows, natural chunk order).
//  kMqaDirect: written by direct-to-LDS loads, each of which puts lane l's
//    16 bytes at byte 16 l of one contiguous KiB: four 256-byte rows.  The
//    thread with lane group g (lanes 16 g .. 16 g + 15) of wave w loads the
//    four tokens 16 w + 4 g + i (i = 0..3, one page), token i by load i, so
//    token t sits in block t >> 4, group t & 3 (one load), row g = (t >> 2) & 3
//    of the group.  Groups are kMqaGroupBytes apart (64 bytes of padding
//    after each KiB): rows of different groups start in different banks.
//    Within a row, K chunk c sits at c ^ g and V's 32-byte piece d at d ^ g,
//    which spreads the four rows of a group over the banks too.  A score
//    read (16 tokens, one chunk each) then covers 16 distinct chunk
//    positions of the banks, and a transposed V read 8 distinct 32-byte
//    bank groups per 32 lanes.  Every lane reads the same K and V chunk of
//    its four tokens, so one source offset per lane serves all four loads.
enum { kMqaRegStaged = 0, kMqaDirect = 1 };
constexpr int kMqaGroupBytes = 4 * kMqaRowBytes + 64;  // four rows of one load, then padding
constexpr int kMqaBlockBytes = 4 * kMqaGroupBytes;     // 16 tokens
constexpr int kMqaDirectBytes = 4 * kMqaBlockBytes;    // K (or V) rows of a chunk

// Byte offset of 16-byte chunk c of K row t (0 <= t < 64) in the K rows.
template <int L>
__device__ __forceinline__ int mqa_k_off(int t, int c) {
    if constexpr (L == kMqaRegStaged) {
        return t * kMqaRowBytes + ((c ^ t) & 15) * 16;
    } else {
        const int g = (t >> 2) & 3;
        return (t >> 4) * kMqaBlockBytes + (t & 3) * kMqaGroupBytes + g * kMqaRowBytes + ((c ^ g) & 15) * 16;
    }
}

// Byte offset of byte `byte` (a multiple of 8) of V row t in the V rows.
template <int L>
__device__ __forceinline__ int mqa_v_off(int t, int byte) {
    if constexpr (L == kMqaRegStaged) {
        return t * kMqaVRow + byte;
    } else {
        const int g = (t >> 2) & 3;
        return (t >> 4) * kMqaBlockBytes + (t & 3) * kMqaGroupBytes + g * kMqaRowBytes + (byte ^ (g << 5));
    }
}

// Transposed 8-byte LDS load (see the header comment) of the piece at `p`.
__device__ __forceinline__ u32x2 lds_read_tr16(const char *p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t *)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Stage the four tokens 4 lg .. 4 lg + 3 of a chunk that this thread loaded
// (16-byte chunk lc of each row): K rows into kt (chunks XOR-swizzled by
// token), V rows into vt (padded rows).  V of tokens that are not valid
// (bit k of `okmask` clear: past the range or on a bad page) is staged as
// zeros -- a zero probability times a NaN row would still be NaN -- and
// their scores are masked by the caller.
__device__ __forceinline__ void mqa_store_chunk(char *kt, char *vt, int lc, int lg,
                                                const u32x4 (&kr)[4], const u32x4 (&vin)[4],
                                                uint32_t okmask) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int tt = 4 * lg + i;
        *reinterpret_cast<u32x4 *>(kt + tt * kMqaRowBytes + ((lc ^ tt) & 15) * 16) = kr[i];
    }
    u32x4 vr[4] = {vin[0], vin[1], vin[2], vin[3]};
    if (__builtin_amdgcn_ballot_w64(okmask != 0xFu)) {  // only at the end of a range
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = (okmask >> i) & 1u ? vr[i] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4 *>(vt + (4 * lg + i) * kMqaVRow + lc * 16) = vr[i];
}

// The score scale as the softmax wants it: positive.  A negative scale has
// its sign moved into the query operand (the sign bit of every 16-bit
// element flipped), and a zero scale becomes the smallest normal float, for
// which 2^(x * scale) rounds to exactly 1 as 2^0 does (and -inf * scale
// stays -inf for masked tokens).
template <int NB>
__device__ __forceinline__ float mqa_positive_scale(float sl2, u32x4 (&qop)[NB][4]) {
    if (sl2 < 0.f) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qop[b][kk] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }
    return fmaxf(fabsf(sl2), 1.17549435e-38f);
}

// Running state of one query row (lane j of each lane group q).  The
// normaliser is kept either on the VALU (lsum: this lane's share, with the
// two-term split) or by the matrix cores (lacc: an MFMA of the rounded
// probabilities against a block of ones, every element the row's sum of
// exactly the probabilities the value product used).
struct MqaRowState {
    float m;          // reference max (equal in the row's four lane groups)
    float lsum;       // this lane's share of the normaliser (SPLIT)
    f32x4_t lacc;     // the row's normaliser in each element (not SPLIT)
    f32x4_t acc[8];   // O^T: head dims 16 dt + 4q + r of row j
};

__device__ __forceinline__ void mqa_init(MqaRowState &st) {
    st.m = -INFINITY;
    st.lsum = 0.f;
    st.lacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// Raw scores q.k of one 64-token chunk whose K rows are staged in kt, for
// this wave's NB column blocks of 16 rows: sc[b][tile][r] is token
// tile * 16 + 4q + r of row j of block b.  The score scale is applied in the
// softmax (mqa_softmax_values), folded into the exponent's fused
// multiply-add.
template <int DT, int NB, int L = kMqaRegStaged>
__device__ __forceinline__ void mqa_scores(const char *kt, const u32x4 (&qop)[NB][4], int j, int q,
                                           float (&sc)[NB][4][4]) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        f32x4_t sacc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) sacc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const u32x4 kop = *reinterpret_cast<const u32x4 *>(kt + mqa_k_off<L>(tt * 16 + j, 4 * kk + q));
#pragma unroll
            for (int b = 0; b < NB; ++b) sacc[b] = mfma_16x16x32<DT>(kop, qop[b][kk], sacc[b]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sc[b][tt][rr] = sacc[b][rr];
    }
}

// Value product of one 64-token chunk with single-rounded probabilities,
// given each row's reference max mref: the probabilities of tokens 0..31
// first, then the value MFMAs of those tokens (and their normaliser MFMA)
// in one region with the exponentials of tokens 32..63, which the compiler
// interleaves, so that the wave keeps the matrix pipe busy while it computes
// the second half's probabilities; then the second half's MFMAs.  Runs at
// raised wave priority (see mqa_softmax_values).  (A fixed pattern of three
// VALU instructions after each MFMA, by sched_group_barrier, measured 0.8%
// slower on the prefill and no different on the shared-prefix call.)
template <int DT, int NB, int L>
__device__ __forceinline__ void mqa_values_single(const char *vt, int j, int q, float sl2,
                                                  const float (&mref)[NB], float (&sc)[NB][4][4],
                                                  MqaRowState (&st)[NB]) {
    auto probs = [&](int bb) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int tt = 2 * bb; tt < 2 * bb + 2; ++tt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sc[b][tt][rr] = fast_exp2(fmaf(sc[b][tt][rr], sl2, -mref[b]));
    };
    auto values = [&](int bb) {
        u32x4 ph[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            ph[b] = u32x4{pack_rne<DT>(sc[b][2 * bb][0], sc[b][2 * bb][1]),
                          pack_rne<DT>(sc[b][2 * bb][2], sc[b][2 * bb][3]),
                          pack_rne<DT>(sc[b][2 * bb + 1][0], sc[b][2 * bb + 1][1]),
                          pack_rne<DT>(sc[b][2 * bb + 1][2], sc[b][2 * bb + 1][3])};
        const int vt0 = 32 * bb + 4 * q + (j >> 2);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const u32x2 v0 = lds_read_tr16(vt + mqa_v_off<L>(vt0, 32 * dt + 8 * (j & 3)));
            const u32x2 v1 = lds_read_tr16(vt + mqa_v_off<L>(vt0 + 16, 32 * dt + 8 * (j & 3)));
            const u32x4 vop = u32x4{v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
            for (int b = 0; b < NB; ++b) st[b].acc[dt] = mfma_16x16x32<DT>(vop, ph[b], st[b].acc[dt]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) st[b].lacc = mfma_16x16x32<DT>(ones16<DT>(), ph[b], st[b].lacc);
    };
    probs(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    values(0);
    probs(1);
    __builtin_amdgcn_sched_barrier(0);
    values(1);
    __builtin_amdgcn_s_setprio(0);
}

// The rest of one 64-token chunk (tokens t0 .. t0 + 63, V rows staged in
// vt) given its raw scores: masking, the online softmax with the score
// scale sl2 (> 0, exp2 domain; see mqa_positive_scale), the value product.
// Row j of block b sees tokens t < lim[b]; `masked` (wave-uniform) says some
// token of the chunk lies past some row's limit.
template <int DT, int NB, bool SPLIT, int L = kMqaRegStaged>
__device__ __forceinline__ void mqa_softmax_values(const char *vt, int j, int q, int t0,
                                                   const int (&lim)[NB], bool masked, float sl2,
                                                   float (&sc)[NB][4][4], MqaRowState (&st)[NB]) {
    if (masked) {
        // tokens left of this lane's row limits: the counts pass through an
        // empty asm inside the branch, so the compares cannot be hoisted out
        // of it and full chunks skip the masking
        int nv[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            nv[b] = lim[b] - (t0 + 4 * q);
            asm volatile("" : "+v"(nv[b]));
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    sc[b][tt][rr] = (tt * 16 + rr < nv[b]) ? sc[b][tt][rr] : -INFINITY;
    }
    float mref[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float mx = max3f(sc[b][0][0], sc[b][0][1], sc[b][0][2]);
#pragma unroll
        for (int i = 3; i < 15; i += 2) mx = max3f(mx, sc[b][i >> 2][i & 3], sc[b][(i + 1) >> 2][(i + 1) & 3]);
        mx = max2f(mx, sc[b][3][3]);
        // the scale is positive, so the scaled max is the raw max scaled
        mx = rowgroup_max_nn(mx) * sl2;
        // m = -inf until the row has seen a valid token
        const bool bump = mx > st[b].m + kMaxSlack;
        if (__builtin_amdgcn_ballot_w64(bump)) {
            const float alpha = !bump ? 1.f : (st[b].m == -INFINITY ? 0.f : fast_exp2(st[b].m - mx));
            st[b].m = bump ? mx : st[b].m;
            if constexpr (SPLIT) st[b].lsum *= alpha;
            else st[b].lacc *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) st[b].acc[dt] *= alpha;
        }
        // a row with m = -inf has only masked scores here: 2^(-inf - 0) = 0
        mref[b] = st[b].m == -INFINITY ? 0.f : st[b].m;
        if constexpr (SPLIT) {
            float ps = 0.f;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    sc[b][tt][rr] = fast_exp2(fmaf(sc[b][tt][rr], sl2, -mref[b]));
                    ps += sc[b][tt][rr];
                }
            st[b].lsum += ps;
        }
    }
    if constexpr (!SPLIT) {
        mqa_values_single<DT, NB, L>(vt, j, q, sl2, mref, sc, st);
        return;
    }
    // The value MFMAs run at raised wave priority: the SIMD then issues them
    // as soon as they are ready and fills the matrix pipe's busy cycles with
    // the other resident wave's softmax (prefill 9.35 -> 8.99 ms on the
    // 32-prompt workload; priority over the score MFMAs as well: no gain).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        // B operand: tokens (tile 2bb, 4q + e) for e < 4, (tile 2bb+1, 4q + e - 4) after
        u32x4 ph[NB], pl[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if constexpr (SPLIT) {
                uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
                split_pack<DT>(sc[b][2 * bb][0], sc[b][2 * bb][1], h0, l0);
                split_pack<DT>(sc[b][2 * bb][2], sc[b][2 * bb][3], h1, l1);
                split_pack<DT>(sc[b][2 * bb + 1][0], sc[b][2 * bb + 1][1], h2, l2);
                split_pack<DT>(sc[b][2 * bb + 1][2], sc[b][2 * bb + 1][3], h3, l3);
                ph[b] = u32x4{h0, h1, h2, h3};
                pl[b] = u32x4{l0, l1, l2, l3};
            } else {
                ph[b] = u32x4{pack_rne<DT>(sc[b][2 * bb][0], sc[b][2 * bb][1]),
                              pack_rne<DT>(sc[b][2 * bb][2], sc[b][2 * bb][3]),
                              pack_rne<DT>(sc[b][2 * bb + 1][0], sc[b][2 * bb + 1][1]),
                              pack_rne<DT>(sc[b][2 * bb + 1][2], sc[b][2 * bb + 1][3])};
            }
        }
        // A operand V^T[16 dt + j][token]: source lane j of row group q
        // points at head dims 16 dt + 4 (j & 3) .. + 3 of token
        // 32 bb + 16 h + 4 q + (j >> 2); the load for h = 0 gives the
        // lane's tokens of tile 2 bb, h = 1 those of tile 2 bb + 1
        const int vt0 = 32 * bb + 4 * q + (j >> 2);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const u32x2 v0 = lds_read_tr16(vt + mqa_v_off<L>(vt0, 32 * dt + 8 * (j & 3)));
            const u32x2 v1 = lds_read_tr16(vt + mqa_v_off<L>(vt0 + 16, 32 * dt + 8 * (j & 3)));
            const u32x4 vop = u32x4{v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                st[b].acc[dt] = mfma_16x16x32<DT>(vop, ph[b], st[b].acc[dt]);
                if constexpr (SPLIT) st[b].acc[dt] = mfma_16x16x32<DT>(vop, pl[b], st[b].acc[dt]);
            }
        }
        if constexpr (!SPLIT) {
#pragma unroll
            for (int b = 0; b < NB; ++b) st[b].lacc = mfma_16x16x32<DT>(ones16<DT>(), ph[b], st[b].lacc);
        }
    }
    __builtin_amdgcn_s_setprio(0);
}

// One 64-token chunk (tokens t0 .. t0 + 63 staged in kt / vt) for this
// wave's NB column blocks of 16 rows: scores, then softmax and values; sl2
// as for mqa_softmax_values.
template <int DT, int NB, bool SPLIT = true, int L = kMqaRegStaged>
__device__ __forceinline__ void mqa_chunk(const char *kt, const char *vt, const u32x4 (&qop)[NB][4],
                                          int j, int q, int t0, const int (&lim)[NB], bool masked,
                                          float sl2, MqaRowState (&st)[NB]) {
    float sc[NB][4][4];  // [block][16-token tile][r]: token tile*16 + 4q + r, row j
    mqa_scores<DT, NB, L>(kt, qop, j, q, sc);
    mqa_softmax_values<DT, NB, SPLIT, L>(vt, j, q, t0, lim, masked, sl2, sc, st);
}

// The row's normaliser: the sum of the four lane groups' shares.
template <bool SPLIT = true>
__device__ __forceinline__ float mqa_row_sum(const MqaRowState &st) {
    if constexpr (SPLIT) return rowgroup_sum(st.lsum);
    else return st.lacc[0];
}

// Workgroup id -> unit so that consecutive units share an XCD (consecutive
// workgroup ids are dealt to the 8 XCDs in turn); a bijection on [0, n).
__device__ __forceinline__ int xcd_unit(int id, int n) {
    constexpr int kXcds = 8;
    const int xcd = id % kXcds, slot = id / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
}

}  // namespace pkv
