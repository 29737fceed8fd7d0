// Fused paged decode attention with the score product on the matrix cores
// (gfx950 v_mfma_f32_16x16x32_{bf16,f16}), for 16-bit caches and head_dim 128.
//
// Same computation as the VALU kernel (pages on PagedAttention:
// "实现教学版 PagedAttention：从 block table 读取历史 KV cache", sections
// "从逻辑 token 到物理 block" and "从 gather 后的 K/V 做 attention";
// "从正确到更快：PagedAttention 的优化路线", sections "高性能 PagedAttention 的核心
// 思想" and "attention kernel 真正在做什么").  With a query-head group the
// score step of a 16-token tile is a small dense product
//     S[16 tokens x 16] = K_tile[16 x 128] . Q^T[128 x 16]
// whose 16 columns carry the group's heads (replicated when G < 4; two
// products of 4 heads each when G = 8).  Four MFMAs (k = 32 each) per tile
// replace the dot-product and lane-reduction work of the VALU kernel.
//
// Work distribution: a persistent grid (as many workgroups as fit on the
// chip) draws work units (sequence, KV partition, KV head) one at a time from
// a counter, KV head fastest so that the units reading the same pages run
// side by side, all full partitions before the shorter last ones.  Each
// workgroup first builds, in LDS, the prefix sums of partitions over the
// sequences of the batch, which map a unit index to its sequence and
// partition; no workgroup is spent on a partition past the end of its
// sequence, and no workgroup idles while units remain.
//
// Lane roles inside a wave (lane = 16 q + c):
//  - K and V rows are loaded whole: load instruction i gives lane (q, c)
//    16-byte chunk c of token 4q + i, so each instruction reads four complete
//    256-byte rows.  (Reading the MFMA operand layout straight from HBM --
//    64 bytes of 16 different rows per instruction -- measured 24% slower.)
//  - K operand: the tile's K rows are transposed through a wave-private LDS
//    tile so that lane (q, c) holds token c, chunks 4j + q (j = 0..3).  The
//    query operand uses the same chunk order, so the contraction pairs
//    equal head-dim indices.
//  - Scores come back as rows 4q + r (r = 0..3) of the tile for head c % 4
//    (+4 for the second product): lane (q, c) owns tokens 4q..4q+3.
//  - V stays in the loaded row order: lane (q, c) holds chunk c of tokens
//    4q + r, the same tokens whose scores it holds; the
//    other heads' probabilities come from the lanes of its quad (DPP quad
//    broadcast).  The running softmax is kept per lane and per row group q
//    and merged at the end, so the tile loop needs no cross-lane max.
//  - The loads of a wave's next tile are issued before the current tile is
//    computed (two register sets), so HBM requests stay in flight while the
//    wave computes.
#include <math.h>

#include "pkv_decode_common.h"
#include "pkv_mfma.h"

#ifndef PKV_TILES_PER_STEP
#define PKV_TILES_PER_STEP 2
#endif
// E4M3 caches: a tile is half the bytes, so twice the tiles per step keep
// the same bytes in flight
#ifndef PKV_TILES_PER_STEP_E4M3
#define PKV_TILES_PER_STEP_E4M3 4
#endif

namespace pkv {

// Value of head slot `hl` (0 <= hl < HS) held by the lanes of this lane's quad:
// lane c of a quad carries head slot c % HS.
template <int HS>
__device__ __forceinline__ float head_bcast(float x, int hl) {
    if constexpr (HS == 1) {
        return x;
    } else if constexpr (HS == 2) {
        return hl == 0 ? dpp<0xA0>(x) : dpp<0xF5>(x);  // quad_perm [0,0,2,2] / [1,1,3,3]
    } else {
        switch (hl) {
            case 0: return dpp<0x00>(x);  // quad_perm [0,0,0,0]
            case 1: return dpp<0x55>(x);  // [1,1,1,1]
            case 2: return dpp<0xAA>(x);  // [2,2,2,2]
            default: return dpp<0xFF>(x); // [3,3,3,3]
        }
    }
}

// Loaded rows of one 16-token tile: 16-byte chunks of 16-bit rows, or
// 8-byte chunks (eight E4M3 codes, the same head dims) of quantised rows.
template <bool KV8>
struct TileRegsT {
    u32x4 k[4];      // tokens 4q + i, chunk c (whole rows per load instruction)
    u32x4 v[4];      // tokens 4q + i, chunk c
    uint32_t vmask;  // bit i: row i holds a valid token
};
template <>
struct TileRegsT<true> {
    u32x2 k[4];
    u32x2 v[4];
    uint32_t vmask;
};

// Eight E4M3 codes -> the same eight values in the 16-bit compute type
// (exact: E4M3 values are representable in binary16 and bfloat16).
template <int DT>
__device__ __forceinline__ u32x4 widen_e4m3(const u32x2 w) {
    // one instruction per pair (scale 1: the plain value)
    u32x4 r;
    if constexpr (DT == kBF16) {
        r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, false));
        r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, true));
        r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, false));
        r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, true));
    } else {
        r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.f, false));
        r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.f, true));
        r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.f, false));
        r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.f, true));
    }
    return r;
}

// Unit order: all full partitions of the batch first, then the partial last
// partitions.  Units of one size drain the grid evenly and the variable-size
// units come at the end, where they fill the gaps.  Builds the exclusive
// prefix sums s_pf[0..B] (full partitions) and s_pp[0..B] (partial ones)
// and caches the lengths in s_ctx.
template <bool PFX>
__device__ __forceinline__ void build_unit_order(const DecodeArgs &a, int *s_pf, int *s_pp,
                                                 int *s_ctx, int *s_scan) {
    const int B = a.num_seqs;
    const int tid = threadIdx.x;
    const int chunk = (B + kThreads - 1) / kThreads;
    const int lo = min(B, tid * chunk), hi = min(B, lo + chunk);
    int nf = 0, np = 0;
    for (int s = lo; s < hi; ++s) {
        const int ctx = a.context_lens[s];
        s_ctx[s] = ctx;
        const int f = seq_full<PFX>(a, ctx);
        nf += f;
        np += seq_parts<PFX>(a, ctx) - f;
    }
    const int incf = block_scan(nf, s_scan);
    const int incp = block_scan(np, s_scan);
    int rf = incf - nf, rp = incp - np;
    for (int s = lo; s < hi; ++s) {
        s_pf[s] = rf;
        s_pp[s] = rp;
        const int f = seq_full<PFX>(a, s_ctx[s]);
        rf += f;
        rp += seq_parts<PFX>(a, s_ctx[s]) - f;
    }
    if (tid == kThreads - 1) {
        s_pf[B] = incf;
        s_pp[B] = incp;
    }
    __syncthreads();
}

// Three waves per SIMD (<= 168 VGPRs) keep enough loads in flight; the
// allocator is held to that budget.
//
// PFX: the launch covers tokens [token_begin, ctx) of each sequence and
// always writes partials (slots part_base.. of part_stride), for the
// shared-prefix path; the plain instantiation never reads those fields.
// KV8: the caches hold E4M3 codes (128-byte rows) with per-KV-head scales;
// DT is then the type of the query and the output.  K is widened to DT
// before the score MFMA, V to fp32 before the value product; k_scale joins
// the score scale and v_scale multiplies the result.
template <int DT, int G, bool PFX, bool KV8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
void paged_decode_mfma_kernel(DecodeArgs a) {
    constexpr int D = 128;
    constexpr int ROW_BYTES = D * 2;
    constexpr int TILE = 16;
    constexpr int HS = G < 4 ? G : 4;  // heads per score product
    constexpr int NSET = G / HS;       // score products per tile
    constexpr bool kQopInLds = NSET > 1;
    constexpr int KV_ROW = KV8 ? D : D * 2;     // bytes of one cached row
    constexpr int KV_CHUNK = KV8 ? 8 : 16;      // bytes of one lane's chunk
    using TileRegs = TileRegsT<KV8>;

    extern __shared__ int s_dyn[];     // full-unit prefix [B + 1], partial-unit prefix [B + 1], lengths [B]
    __shared__ int s_pages[kSegPages];
    __shared__ int s_bad;
    __shared__ float s_m[kNumWaves][G];
    __shared__ float s_l[kNumWaves][G];
    __shared__ float s_acc[kNumWaves][G][D];
    __shared__ __attribute__((aligned(16))) char s_ktile[kNumWaves][TILE * ROW_BYTES];
    __shared__ u32x4 s_qop[kQopInLds ? NSET : 1][4][kWave];

    int *s_pf = s_dyn;
    int *s_pp = s_dyn + a.num_seqs + 1;
    int *s_ctx = s_dyn + 2 * (a.num_seqs + 1);
    build_unit_order<PFX>(a, s_pf, s_pp, s_ctx, s_pages);
    const int total_full = s_pf[a.num_seqs];
    const int total_units = (total_full + s_pp[a.num_seqs]) * a.num_kv_heads;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // wave-uniform (scalar) so that the tile loop is a scalar loop
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int q = lane >> 4;  // row group: tokens 4q..4q+3 of a tile
    const int c = lane & 15;  // column: head slot c % HS; V chunk c

    const char *kbase = reinterpret_cast<const char *>(a.key_cache);
    const char *vbase = reinterpret_cast<const char *>(a.value_cache);
    const int bs = a.block_size;
    const int lbs = a.log2_block_size;
    const int64_t tok_stride = (int64_t)a.num_kv_heads * KV_ROW;  // bytes between slots
    const float sl2_q = a.scale_log2e;
    char *ktile = s_ktile[wave];

    // Units are handed out one at a time from a counter in the workspace, so
    // a workgroup that drew short units simply takes more: with a static
    // assignment the chip idles while the unluckiest workgroups finish.
    // Every workgroup ends with exactly one failed draw; the draw that sees
    // the last ticket of the launch (total + grid - 1) resets the counter to
    // zero for the next call on this workspace.
    __shared__ int s_unit;
    for (;;) {
        __syncthreads();  // previous unit's epilogue is done with LDS
        if (threadIdx.x == 0) {
            const unsigned got = atomicAdd(a.work_counter, 1u);
            if (got == (unsigned)total_units + gridDim.x - 1u) atomicExch(a.work_counter, 0u);
            s_unit = (int)got;
        }
        __syncthreads();
        const int unit = s_unit;
        if (unit >= total_units) break;
        // unit -> (sequence, partition, KV head)
        Unit u;
        u.kvh = unit % a.num_kv_heads;
        const int sp = unit / a.num_kv_heads;
        if (sp < total_full) {
            u.s = search_le(s_pf, a.num_seqs, sp);
            u.p = sp - s_pf[u.s];
        } else {
            u.s = search_le(s_pp, a.num_seqs, sp - total_full);
            u.p = seq_full<PFX>(a, s_ctx[u.s]);
        }
        u.ctx = s_ctx[u.s];
        u.bad_len = bad_context(a, u.ctx);
        u.tok_begin = first_token<PFX>(a) + u.p * a.partition_size;
        u.tok_end = u.bad_len ? 0 : min(u.ctx, u.tok_begin + a.partition_size);
        u.nparts = seq_parts<PFX>(a, u.ctx);
        u.empty = false;

        if (tid == 0) s_bad = 0;

        // query operand: head (set*HS + c%HS), chunks 4j + q.  It is the
        // same for every wave; with two score products (G = 8) it is parked
        // in LDS (wave 0 writes it before the first barrier below) to keep
        // the register count at three waves per SIMD.
        const int h0 = u.kvh * G;
        u32x4 qop[NSET][4];
        if (!kQopInLds || wave == 0) {
            const char *qb = reinterpret_cast<const char *>(a.query);
#pragma unroll
            for (int set = 0; set < NSET; ++set) {
                const int h = h0 + set * HS + (c % HS);
                const char *row = qb + ((int64_t)u.s * a.num_heads + h) * ROW_BYTES;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    qop[set][j] = load16(row + (4 * j + q) * 16);
                    if constexpr (kQopInLds) s_qop[set][j][lane] = qop[set][j];
                }
            }
        }

        float m[NSET], l[NSET], acc[G][8];
#pragma unroll
        for (int set = 0; set < NSET; ++set) {
            m[set] = -INFINITY;
            l[set] = 0.f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;

        const int64_t kvh_off = (int64_t)u.kvh * KV_ROW;
        float sl2 = sl2_q;
        if constexpr (KV8) sl2 *= a.k_scale[u.kvh];

        for (int seg = u.tok_begin; seg < u.tok_end; seg += kSegPages << lbs) {
            const int seg_end = min(u.tok_end, seg + (kSegPages << lbs));
            const int npages = (seg_end - seg + bs - 1) >> lbs;
            __syncthreads();  // previous segment's readers are done with s_pages
            stage_pages(a, u, seg >> lbs, npages, s_pages, &s_bad);
            __syncthreads();

            // token -> byte offset of its row in the pool.  Loads are issued
            // unconditionally so the compiler can count outstanding loads
            // exactly and keep the next tile's loads in flight: a token past
            // the segment or on a bad page id reads a row of page 0 (always
            // in the pool) and is flagged invalid; invalid V rows are zeroed
            // where they are consumed and invalid scores are masked.
            auto row_of = [&](int t, bool &valid) -> int64_t {
                const int pb = s_pages[min((t - seg) >> lbs, npages - 1)];
                valid = (t < seg_end) & (pb >= 0);
                const int64_t page = valid ? pb : 0;
                return (page * bs + (t & (bs - 1))) * tok_stride + kvh_off;
            };
            auto load_tile = [&](TileRegs &r, int t0) {
                r.vmask = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bool ok;
                    const int64_t row = row_of(t0 + 4 * q + i, ok) + c * KV_CHUNK;
                    if constexpr (KV8) {
                        r.k[i] = load8_stream(kbase + row);
                        r.v[i] = load8_stream(vbase + row);
                    } else {
                        r.k[i] = load16_stream(kbase + row);
                        r.v[i] = load16_stream(vbase + row);
                    }
                    r.vmask |= ok ? (1u << i) : 0u;
                }
            };
            auto compute_tile = [&](const TileRegs &r, int t0) {
                // K rows arrive whole (16 lanes per 256-byte row); the score
                // MFMA wants lane (q, c) to hold token c, chunks 4j + q.
                // Transpose through this wave's LDS tile, 16-byte chunks
                // XOR-swizzled by token so that writes and reads are free of
                // bank conflicts.  Rows are private to the wave and LDS
                // operations of one wave complete in order: no barrier.
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tt = 4 * q + i;
                    u32x4 krow;
                    if constexpr (KV8) krow = widen_e4m3<DT>(r.k[i]); else krow = r.k[i];
                    *reinterpret_cast<u32x4 *>(ktile + tt * ROW_BYTES + ((c ^ tt) & 15) * 16) = krow;
                }
                u32x4 kop[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    kop[j] = *reinterpret_cast<const u32x4 *>(ktile + c * ROW_BYTES + (((4 * j + q) ^ c) & 15) * 16);
                // The reference max of a lane's row group moves only when a
                // score passes it by more than kMaxSlack, so the accumulator
                // rescale (a multiply per accumulator) is skipped in nearly
                // every tile; the merges weight each state by its own
                // (max, normaliser), so any reference gives the same result.
                float p[NSET][4], alpha[NSET];
                bool bump_any = false;
#pragma unroll
                for (int set = 0; set < NSET; ++set) {
                    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        sacc = mfma_16x16x32<DT>(kop[j], kQopInLds ? s_qop[set][j][lane] : qop[set][j], sacc);
                    float sv[4];
                    float mt = -INFINITY;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sv[i] = (t0 + 4 * q + i < seg_end) ? sacc[i] * sl2 : -INFINITY;
                        mt = fmaxf(mt, sv[i]);
                    }
                    const bool bump = mt > m[set] + kMaxSlack;  // m = -inf: any valid score
                    alpha[set] = !bump ? 1.f : (m[set] == -INFINITY ? 0.f : fast_exp2(m[set] - mt));
                    m[set] = bump ? mt : m[set];
                    bump_any |= bump;
                    // m = -inf only while the row group has seen no valid
                    // score: then every score here is masked and 2^(-inf) = 0
                    const float mref = m[set] == -INFINITY ? 0.f : m[set];
                    float ps = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p[set][i] = fast_exp2(sv[i] - mref);
                        ps += p[set][i];
                    }
                    l[set] = l[set] * alpha[set] + ps;
                }
                if (__builtin_amdgcn_ballot_w64(bump_any)) {
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const float ag = head_bcast<HS>(alpha[g / HS], g % HS);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[g][e] *= ag;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float vf[8];
                    if constexpr (KV8) {
                        const u32x2 vw = (r.vmask >> i) & 1u ? r.v[i] : u32x2{0, 0};
                        e4m3x4_to_f32(vw.x, vf);
                        e4m3x4_to_f32(vw.y, vf + 4);
                    } else {
                        unpack16<DT>((r.vmask >> i) & 1u ? r.v[i] : u32x4{0, 0, 0, 0}, vf);
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const float pg = head_bcast<HS>(p[g / HS][i], g % HS);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pg, vf[e], acc[g][e]);
                    }
                }
            };

            // Each wave step issues the loads of TPS consecutive tiles at
            // once and then computes them in order, so up to TPS * 8 KiB of
            // HBM requests per wave are in flight while earlier tiles are
            // computed.  Straight-line code: the compiler waits for exactly
            // the loads a tile needs.  A tile past the segment is all
            // invalid and computes to no change.
            constexpr int TPS = KV8 ? (G == 8 ? 2 : PKV_TILES_PER_STEP_E4M3)
                                    : (G == 8 ? 1 : PKV_TILES_PER_STEP);  // register budget
            constexpr int STEP = kNumWaves * TILE * TPS;
            for (int t = seg + wave * TILE * TPS; t < seg_end; t += STEP) {
                TileRegs r[TPS];
#pragma unroll
                for (int i = 0; i < TPS; ++i) load_tile(r[i], t + i * TILE);
                // keep every load of the step ahead of the compute: left
                // alone, the scheduler sinks each load next to its use and
                // the wave then waits on one load at a time
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TPS; ++i) compute_tile(r[i], t + i * TILE);
            }
        }

        // merge the four row groups q of this wave (lanes c, c+16, c+32, c+48)
        float f[NSET];
#pragma unroll
        for (int set = 0; set < NSET; ++set) {
            float M = fmaxf(m[set], __shfl_xor(m[set], 16));
            M = fmaxf(M, __shfl_xor(M, 32));
            f[set] = (M == -INFINITY) ? 0.f : fast_exp2(m[set] - M);
            float L = l[set] * f[set];
            L += __shfl_xor(L, 16);
            L += __shfl_xor(L, 32);
            m[set] = M;
            l[set] = L;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float fg = head_bcast<HS>(f[g / HS], g % HS);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = acc[g][e] * fg;
                x += __shfl_xor(x, 16);
                x += __shfl_xor(x, 32);
                acc[g][e] = x;
            }
        }
        if (q == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_acc[wave][g][c * 8 + e] = acc[g][e];
            if (c < HS) {
#pragma unroll
                for (int set = 0; set < NSET; ++set) {
                    s_m[wave][set * HS + c] = m[set];
                    s_l[wave][set * HS + c] = l[set];
                }
            }
        }
        __syncthreads();
        unit_epilogue<DT, D, G, PFX>(a, u, u.bad_len || s_bad != 0, s_m, s_l, s_acc,
                                     KV8 ? a.v_scale[u.kvh] : 1.f);
    }
}

// Persistent grid: as many workgroups as are resident at once (queried once
// per kernel and LDS size), capped by the number of units.
template <typename K>
static hipError_t launch_persistent(K kernel, const DecodeArgs &a, hipStream_t stream) {
    const size_t dyn = (size_t)(3 * a.num_seqs + 2) * sizeof(int);
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kernel),
                                                         kThreads, dyn);
    if (e != hipSuccess) return e;
    int64_t grid = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions;  // upper bound
    if (grid > units) grid = units;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), dyn, stream, a);
    return hipGetLastError();
}

template <int DT, bool PFX, bool KV8 = false>
static hipError_t launch_group(const DecodeArgs &a, hipStream_t stream) {
    switch (a.num_heads / a.num_kv_heads) {
        case 1: return launch_persistent(paged_decode_mfma_kernel<DT, 1, PFX, KV8>, a, stream);
        case 2: return launch_persistent(paged_decode_mfma_kernel<DT, 2, PFX, KV8>, a, stream);
        case 4: return launch_persistent(paged_decode_mfma_kernel<DT, 4, PFX, KV8>, a, stream);
        case 8: return launch_persistent(paged_decode_mfma_kernel<DT, 8, PFX, KV8>, a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_paged_decode_mfma(const DecodeArgs &a, int dtype, hipStream_t stream) {
    if (dtype == kBF16) return launch_group<kBF16, false>(a, stream);
    if (dtype == kF16) return launch_group<kF16, false>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_paged_decode_mfma_e4m3(const DecodeArgs &a, int dtype, hipStream_t stream) {
    if (dtype == kBF16) return launch_group<kBF16, false, true>(a, stream);
    if (dtype == kF16) return launch_group<kF16, false, true>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_paged_decode_mfma_suffix(const DecodeArgs &a, int dtype, hipStream_t stream) {
    if (dtype == kBF16) return launch_group<kBF16, true>(a, stream);
    if (dtype == kF16) return launch_group<kF16, true>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
