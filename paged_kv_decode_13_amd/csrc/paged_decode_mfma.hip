// Fused paged decode attention with both products on the matrix cores
// (gfx950 v_mfma_f32_16x16x32_{bf16,f16}), head_dim 128, over 16-bit or
// E4M3 caches.
//
// Same computation as the VALU kernel (pages on PagedAttention:
// "实现教学版 PagedAttention：从 block table 读取历史 KV cache", sections
// "从逻辑 token 到物理 block" and "从 gather 后的 K/V 做 attention";
// "从正确到更快：PagedAttention 的优化路线", sections "高性能 PagedAttention 的核心
// 思想" and "attention kernel 真正在做什么").  With a query-head group both
// steps of a 16-token tile are small dense products whose 16 columns carry
// the group's heads (column c: head c % G):
//     S^T[16 tokens x 16] = K_tile[16 x 128] . Q^T[128 x 16]
//     O^T[128 x 16]      += V^T[128 x 32 tokens] . P^T[32 tokens x 16]
// (the second over a pair of tiles, k = 32).
//
// Work distribution: a persistent grid (as many workgroups as fit on the
// chip) takes work units (sequence, KV partition, KV head) one at a time --
// the first by workgroup index, the rest from a counter -- KV head fastest
// so that the units reading the same pages run side by side, all full
// partitions before the shorter last ones.  Each
// workgroup first builds, in LDS, the prefix sums of partitions over the
// sequences of the batch, which map a unit index to its sequence and
// partition; no workgroup is spent on a partition past the end of its
// sequence, and no workgroup idles while units remain.
//
// Lane roles inside a wave (lane = 16 q + c):
//  - K and V rows are loaded whole: load instruction i gives lane (q, c)
//    chunk c (head dims 8c..8c+7) of token 4q + i, so each instruction reads
//    four complete rows.  (Reading the MFMA operand layout straight from
//    HBM -- 64 bytes of 16 different rows per instruction -- measured 24%
//    slower.)
//  - K operand: the tile's K rows are transposed through a wave-private LDS
//    tile so that lane (q, c) holds token c, chunks 4j + q (j = 0..3).  The
//    query operand uses the same chunk order, so the contraction pairs
//    equal head-dim indices.
//  - Scores come back as rows 4q + r (r = 0..3) of the tile for column c:
//    lane (q, c) owns tokens 4q..4q+3, which is the B-operand layout of the
//    value product, and V^T is formed from the lane's own V registers (see
//    the kernel).
//  - A wave issues the loads of two tiles, then computes them; the other
//    resident waves keep HBM requests in flight meanwhile.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "pkv_decode_common.h"
#include "pkv_mfma.h"
#include "pkv_prefix_unit.h"

// Tiles whose loads a wave issues at once (even: tiles are computed in
// pairs); the register budget of three waves per SIMD allows two
#ifndef PKV_TILES_PER_STEP
#define PKV_TILES_PER_STEP 2
#endif
#ifndef PKV_TILES_PER_STEP_E4M3
#define PKV_TILES_PER_STEP_E4M3 2
#endif
// Resident workgroups per CU of the persistent grids.  Past a point more
// requests in flight only queue at HBM: two workgroups per CU (up to 128
// KiB of loads in flight per CU with 16-bit caches) already reach what the
// access pattern allows.  A third measured 1-4% slower on every 16-bit
// workload and 1.5% slower over E4M3 caches.
#ifndef PKV_WG_PER_CU
#define PKV_WG_PER_CU 2
#endif
// Register budget of the decode kernels: the allocator is held to this many
// resident waves per SIMD (3: at most 168 VGPRs)
#ifndef PKV_DECODE_MIN_WAVES
#define PKV_DECODE_MIN_WAVES 3
#endif

namespace pkv {

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

// Two E4M3 codes (bytes 0, 1 of `w`, or bytes 2, 3 with HIGH) -> the packed
// 16-bit pair of the same values (exact: E4M3 values are representable in
// binary16 and bfloat16); one instruction (scale 1: the plain value).
template <int DT, bool HIGH>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w) {
    if constexpr (DT == kBF16)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HIGH));
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, HIGH));
}

// Eight E4M3 codes -> the same eight values in the 16-bit compute type.
template <int DT>
__device__ __forceinline__ u32x4 widen_e4m3(const u32x2 w) {
    return u32x4{e4m3_pair<DT, false>(w.x), e4m3_pair<DT, true>(w.x), e4m3_pair<DT, false>(w.y),
                 e4m3_pair<DT, true>(w.y)};
}

// Unit order.  All whole runs of unit_parts partitions of the batch come
// first: units of one size drain the grid evenly.  Then:
//  - unit_parts == 1 (every whole partition is a run): the tail units, each
//    sequence's partial last partition, longest first, so the last units
//    drawn are the shortest and the grid ends together (longest-processing-
//    time order; 256-sequence batch at 2560-token partitions 559 -> 541 us);
//  - unit_parts > 1: each sequence's remaining partitions, its tail last,
//    sequence by sequence.  (The 32-sequence MHA batch ran 176 us so and
//    180 us with the whole partitions of every sequence before all tails.)
//
// Builds the exclusive prefix sums s_pf[0..B] (runs) and s_pp[0..B] (the
// partitions after the runs that are not sorted tails), caches the lengths
// in s_ctx, lists the sequences with a sorted tail unit in s_tail (by tail
// length in kTailBuckets classes, longest class first, sequence order within
// a class: a stable counting sort, so every workgroup builds the same list)
// and stores their number in *s_ntail.  s_tmp: 192 ints of scratch.
constexpr int kTailBuckets = 16;

__device__ __forceinline__ bool sorted_tails(const DecodeArgs &a) { return a.unit_parts == 1; }

// Partitions after a sequence's runs that sit in its s_pp range.
template <bool PFX>
__device__ __forceinline__ int seq_singles(const DecodeArgs &a, int ctx) {
    return sorted_tails(a) ? seq_whole_singles<PFX>(a, ctx) : seq_units<PFX>(a, ctx) - seq_full_units<PFX>(a, ctx);
}

// Class of a sequence's sorted tail unit (0: longest), -1 if it has none.
template <bool PFX>
__device__ __forceinline__ int tail_bucket(const DecodeArgs &a, int ctx) {
    const int t = seq_tail_tokens<PFX>(a, ctx);
    if (t < 0) return -1;
    // floor((ps - 1 - t) * kTailBuckets / ps) in binary32 (an ordering key
    // only; every workgroup computes the same one), clamped to the classes
    const float f = (float)(a.partition_size - 1 - t) * (float)kTailBuckets / (float)a.partition_size;
    return min(kTailBuckets - 1, (int)f);
}

template <bool PFX>
__device__ __forceinline__ void build_unit_order(const DecodeArgs &a, int *s_pf, int *s_pp, int *s_ctx,
                                                 uint16_t *s_tail, int *s_ntail, int *s_tmp) {
    const int B = a.num_seqs;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const bool sort = sorted_tails(a);
    int *s_scan = s_tmp;                      // [2][kNumWaves]: wave totals of runs, singles
    int *s_run = s_tmp + 8;                   // [kTailBuckets]: first free slot of each class
    int *s_whist = s_tmp + 8 + kTailBuckets;  // [kNumWaves][kTailBuckets]: class sizes per wave
    int *s_cnt = s_tmp + 64;                  // [2][kNumWaves][kTailBuckets]
    // Each thread takes `chunk` consecutive sequences: their lengths, their
    // unit counts (kept in s_pf / s_pp until they become prefix sums) and,
    // by wave ballots, the sizes of their tail classes (lane k of a wave
    // counts class k).
    const int chunk = (B + kThreads - 1) / kThreads;
    const int lo = min(B, tid * chunk), hi = min(B, lo + chunk);
    int nf = 0, np = 0, hist = 0;
    // one sequence per thread (B <= kThreads): its class and its rank among
    // the members of that class in its wave, from the same ballots
    int key1 = -1, rank1 = 0;
    for (int i = 0; i < chunk; ++i) {
        const int s = lo + i;
        int key = -1;
        if (s < hi) {
            const int ctx = a.context_lens[s];
            s_ctx[s] = ctx;
            const int f = seq_full_units<PFX>(a, ctx), p = seq_singles<PFX>(a, ctx);
            s_pf[s] = f;
            s_pp[s] = p;
            nf += f;
            np += p;
            if (sort) key = tail_bucket<PFX>(a, ctx);
        }
        if (sort) {
#pragma unroll
            for (int k = 0; k < kTailBuckets; ++k) {
                const uint64_t m = __ballot(key == k);
                if (lane == k) hist += __popcll(m);
                if (key == k) rank1 = __popcll(m & ((1ull << lane) - 1ull));
            }
        }
        key1 = key;
    }
    const int xf = wave_scan(nf), xp = wave_scan(np);
    if (lane == kWave - 1) {
        s_scan[wave] = xf;
        s_scan[kNumWaves + wave] = xp;
    }
    if (sort && lane < kTailBuckets) s_whist[wave * kTailBuckets + lane] = hist;
    __syncthreads();
    int rf = xf - nf, rp = xp - np;  // exclusive prefix within the wave
    for (int w = 0; w < wave; ++w) {
        rf += s_scan[w];
        rp += s_scan[kNumWaves + w];
    }
    for (int s = lo; s < hi; ++s) {
        const int f = s_pf[s], p = s_pp[s];
        s_pf[s] = rf;
        s_pp[s] = rp;
        rf += f;
        rp += p;
    }
    if (tid == kThreads - 1) {
        s_pf[B] = rf;
        s_pp[B] = rp;
    }
    if (tid < kWave) {  // exclusive scan of the class sizes in wave 0
        int n = 0;
        if (sort && tid < kTailBuckets)
            for (int w = 0; w < kNumWaves; ++w) n += s_whist[w * kTailBuckets + tid];
        const int x = wave_scan(n);
        if (tid < kTailBuckets) s_run[tid] = x - n;  // first slot of class tid
        if (tid == kTailBuckets - 1) *s_ntail = x;
    }
    __syncthreads();
    if (*s_ntail == 0) return;
    if (chunk == 1) {
        // a sequence's slot is its class's start, plus the class members of
        // earlier waves and lower lanes (s_whist is intact: no round ran)
        if (key1 >= 0) {
            int pos = s_run[key1] + rank1;
            for (int w = 0; w < wave; ++w) pos += s_whist[w * kTailBuckets + key1];
            s_tail[pos] = (uint16_t)lo;
        }
        __syncthreads();
        return;
    }
    // 256 sequences per round: a sequence's slot is its class's start, plus
    // the class members of earlier rounds, earlier waves and lower lanes
    for (int r0 = 0, par = 0; r0 < B; r0 += kThreads, par ^= 1) {
        const int s = r0 + tid;
        const int key = s < B ? tail_bucket<PFX>(a, s_ctx[s]) : -1;
        int *cnt = s_cnt + par * kNumWaves * kTailBuckets;
        int rank = 0;
#pragma unroll
        for (int k = 0; k < kTailBuckets; ++k) {
            const uint64_t m = __ballot(key == k);
            if (lane == 0) cnt[wave * kTailBuckets + k] = __popcll(m);
            if (key == k) rank = __popcll(m & ((1ull << lane) - 1ull));
        }
        __syncthreads();
        if (key >= 0) {
            int pos = s_run[key] + rank;
            for (int w = 0; w < wave; ++w) pos += cnt[w * kTailBuckets + key];
            s_tail[pos] = (uint16_t)s;
        }
        __syncthreads();
        if (tid < kTailBuckets) {
            int n = 0;
            for (int w = 0; w < kNumWaves; ++w) n += cnt[w * kTailBuckets + tid];
            s_run[tid] += n;
        }
    }
    __syncthreads();
}

// Unit index -> (sequence, partition, KV head) and its token range, in the
// order of build_unit_order (KV head fastest).  The fields are
// wave-uniform; readfirstlane keeps them in scalar registers.
template <bool PFX>
__device__ __forceinline__ void decode_unit(const DecodeArgs &a, const int *s_pf, const int *s_pp,
                                            const int *s_ctx, const uint16_t *s_tail, int unit, Unit &u) {
    const int total_full = s_pf[a.num_seqs];
    const int total_single = s_pp[a.num_seqs];
    u.kvh = unit % a.num_kv_heads;
    const int sp = unit / a.num_kv_heads;
    int span;
    if (sp < total_full) {  // a whole run of unit_parts partitions
        u.s = wave_search_le(s_pf, a.num_seqs, sp);
        u.p = sp - s_pf[u.s];
        u.part0 = u.p * a.unit_parts;
        span = run_tokens(a);
    } else if (sp < total_full + total_single) {  // a partition after the runs
        const int r = sp - total_full;
        u.s = wave_search_le(s_pp, a.num_seqs, r);
        const int runs = seq_full_units<PFX>(a, s_ctx[u.s]);
        u.p = runs + r - s_pp[u.s];
        u.part0 = runs * a.unit_parts + r - s_pp[u.s];
        span = a.partition_size;
    } else {                // a tail unit
        u.s = s_tail[sp - total_full - total_single];
        const int runs = seq_full_units<PFX>(a, s_ctx[u.s]);
        const int singles = seq_whole_singles<PFX>(a, s_ctx[u.s]);
        u.p = runs + singles;
        u.part0 = runs * a.unit_parts + singles;
        span = a.partition_size;
    }
    u.s = __builtin_amdgcn_readfirstlane(u.s);
    u.p = __builtin_amdgcn_readfirstlane(u.p);
    u.part0 = __builtin_amdgcn_readfirstlane(u.part0);
    u.ctx = __builtin_amdgcn_readfirstlane(s_ctx[u.s]);
    u.bad_len = bad_context(a, u.ctx);
    u.tok_begin = first_token<PFX>(a) + u.part0 * a.partition_size;
    u.tok_end = u.bad_len ? 0 : min(u.ctx, u.tok_begin + span);
    u.nparts = seq_parts<PFX>(a, u.ctx);
    u.empty = false;
}

// Units are handed out from a counter in the workspace, so a workgroup that
// drew short units simply takes more: with a static assignment the chip
// idles while the unluckiest workgroups finish.  The first unit of each
// workgroup is its own index among the `drawers` workgroups that draw
// (`first` is cleared on that call): all of them start at once, and one
// atomic per workgroup on a single address at launch delayed the last
// starts (long-context batch 105 -> 101 us, MHA 183 -> 180 us).  Later
// draws take ticket t from the counter and run unit drawers + t.
//
// No launch depends on what the counter held before it: drawer 0 clears it
// (an atomic exchange) before anything else, and a ticket outside the valid
// range ends the drawing workgroup's work.  A draw made before the clear
// (only possible if drawer 0 starts a whole unit late) either returns a
// valid ticket -- that unit then also goes to whoever draws the same ticket
// after the clear, and both write identical results -- or ends that
// workgroup early.  Drawer 0 draws only after its clear, and stops only on
// a ticket past the last unit, which it can only receive once every valid
// ticket has been handed out after the clear; so every unit runs.  Decodes
// the unit into (sequence, partition, KV head); false once the units are
// exhausted.  Starts with a barrier, so the previous unit's epilogue is done
// with LDS.
template <bool PFX>
__device__ __forceinline__ bool draw_unit(const DecodeArgs &a, const int *s_pf, const int *s_pp,
                                          const int *s_ctx, const uint16_t *s_tail, int n_tail,
                                          int *s_unit, Unit &u, int drawers, int drawer, bool &first) {
    const int total_units = (s_pf[a.num_seqs] + s_pp[a.num_seqs] + n_tail) * a.num_kv_heads;
    __syncthreads();
    if (first) {
        first = false;
        if (drawer == 0 && threadIdx.x == 0) atomicExch(a.work_counter, 0u);
        if (drawer >= total_units) return false;  // so are all counter tickets
        decode_unit<PFX>(a, s_pf, s_pp, s_ctx, s_tail, drawer, u);
        return true;
    }
    if (threadIdx.x == 0) {
        const unsigned got = atomicAdd(a.work_counter, 1u);
        const unsigned tickets = total_units > drawers ? (unsigned)(total_units - drawers) : 0u;
        *s_unit = got < tickets ? (int)got + drawers : -1;
    }
    __syncthreads();
    const int unit = *s_unit;
    if (unit < 0) return false;
    decode_unit<PFX>(a, s_pf, s_pp, s_ctx, s_tail, unit, u);
    return true;
}

// Without a workspace (one partition per sequence, no counter) the grid
// holds one workgroup per (sequence, KV head) and the hardware dispatcher
// balances them: unit = workgroup index, KV head fastest.
__device__ __forceinline__ bool direct_unit(const DecodeArgs &a, Unit &u, bool &first) {
    if (!first) return false;
    first = false;
    const int unit = blockIdx.x;
    u.kvh = unit % a.num_kv_heads;
    u.s = unit / a.num_kv_heads;
    u.p = 0;
    u.ctx = __builtin_amdgcn_readfirstlane(a.context_lens[u.s]);
    u.bad_len = bad_context(a, u.ctx);
    u.tok_begin = 0;
    u.tok_end = u.bad_len ? 0 : u.ctx;
    u.part0 = 0;
    u.nparts = 1;
    u.empty = false;
    return true;
}

// The value product.  Two consecutive 16-token tiles form a 32-token pair,
// and for each of eight head-dim blocks dt
//     O^T[16 x 16] += V^T[16 x 32 tokens] . P^T[32 tokens x 16]
// is one k = 32 MFMA (twice: the probabilities enter as a two-term split
// hi + lo, so about 16 (bf16) or 21 (fp16) bits of each p reach the fp32
// accumulators).  The 16 columns carry the group's heads (column c: head
// c % G), so one score product per tile covers every group size up to 8,
// and the accumulators are 32 floats per lane whatever G is.
//  - The score MFMA leaves lane (q, c) the probabilities of tokens 4q..4q+3
//    of each tile for column c, which is already the layout of the B
//    operand (k = 8q + e: tile A's token 4q + e for e < 4, tile B's 4q + e - 4
//    after): P^T needs no data movement.
//  - Row i of block dt's A operand is head dim 8i + dt.  Lane (q, c) then
//    needs dim 8c + dt of tokens 4q..4q+3 of both tiles -- values it loaded
//    itself (its V chunk c is dims 8c..8c+7 of exactly those tokens) -- so
//    V^T is formed in registers with one v_perm per operand register and
//    never touches LDS.  The accumulator of block dt holds dims
//    8 (4q + r) + dt: lane (q, c) ends with dims 32q..32q+31 of column c.
//  - One reference max per column, shared by the four row groups q (two
//    lane swaps per pair), so every probability of a column is relative
//    to the same max and the value product can sum over all 32 tokens; the
//    lazy rule (move only when passed by more than 2^kMaxSlack) keeps
//    rescales rare.
//
// The allocator is held to a three-waves-per-SIMD budget (<= 168 VGPRs);
// the launch keeps two workgroups per CU (PKV_WG_PER_CU).
//
// PFX: the launch covers tokens [token_begin, ctx) of each sequence and
// writes partials (slots part_base.. of part_stride), for the shared-prefix
// path, unless direct_out (no prefix, one partition per suffix); the plain
// instantiation never reads those fields.
// KV8: the caches hold E4M3 codes (128-byte rows) with per-KV-head scales;
// DT is then the type of the query and the output.  K and V are widened to
// DT (exact) for the MFMAs; k_scale joins the score scale and v_scale
// multiplies the result.
// Tiles whose loads a wave issues at once, and whether the query operand
// then moves to LDS (more tiles per step) to free its 16 registers for
// loads in flight.
template <bool KV8>
constexpr int tiles_per_step() { return KV8 ? PKV_TILES_PER_STEP_E4M3 : PKV_TILES_PER_STEP; }
#ifndef PKV_QOP_LDS
#define PKV_QOP_LDS (PKV_DECODE_MIN_WAVES >= 3)
#endif
template <bool KV8>
constexpr bool qop_in_lds() { return PKV_QOP_LDS && tiles_per_step<KV8>() > 2; }

// One wave's LDS region: the K rows of the 16-token tile being scored (the
// score operand transpose), then the wave's accumulators for the epilogue.
constexpr int kDecodeRegion = 16 * 128 * 2;

// LDS of the decode work loop (besides the dynamic unit-order tables).
template <int G, bool QOP_LDS>
struct DecodeLds {
    int pages[kSegPages];
    int bad;
    int unit;
    int ntail;  // tail units of the batch (build_unit_order)
    float m[kNumWaves][G];
    float l[kNumWaves][G];
    __attribute__((aligned(16))) char region[kNumWaves][kDecodeRegion];
    u32x4 qop[QOP_LDS ? 4 : 1][kWave];
};

// The decode work loop of one workgroup, as a device function over LDS the
// kernel provides (s_dyn: ints run prefix [B + 1], whole-partition prefix
// [B + 1], lengths [B], then the tail list, B 16-bit sequence indices);
// drawers = the launch's workgroups that draw units.
// W: the decode step's slot write is part of the launch (see the new-token
// block in the unit loop).
template <int DT, int G, bool PFX, bool KV8, bool RUNS, bool W = false>
__device__ __forceinline__ void decode_body(const DecodeArgs &a, int *s_dyn,
                                            DecodeLds<G, qop_in_lds<KV8>()> &L, int drawers) {
    static_assert(!W || (!PFX && !KV8), "the fused slot write serves the plain 16-bit decode");
    constexpr int D = 128;
    constexpr int ROW_BYTES = D * 2;
    constexpr int TILE = 16;
    constexpr int KV_ROW = KV8 ? D : D * 2;     // bytes of one cached row
    constexpr int KV_CHUNK = KV8 ? 8 : 16;      // bytes of one lane's chunk
    using TileRegs = TileRegsT<KV8>;
    constexpr int TPS = tiles_per_step<KV8>();
    static_assert(TPS % 2 == 0, "tiles go in pairs");
    constexpr int kRegion = kDecodeRegion;
    static_assert(TILE * ROW_BYTES == kRegion, "a region holds one tile of K rows");
    static_assert(G * D * 4 <= kRegion, "accumulators fit the wave's region");
    constexpr bool kQopLds = qop_in_lds<KV8>();

    int *s_pages = L.pages;
    int &s_bad = L.bad;
    float (*s_m)[G] = L.m;
    float (*s_l)[G] = L.l;
    char (*s_region)[kRegion] = L.region;
    u32x4 (*s_qop)[kWave] = L.qop;

    int *s_pf = s_dyn;
    int *s_pp = s_dyn + a.num_seqs + 1;
    int *s_ctx = s_dyn + 2 * (a.num_seqs + 1);
    uint16_t *s_tail = reinterpret_cast<uint16_t *>(s_ctx + a.num_seqs);
    // no counter: one unit per workgroup by index (unsplit calls without a
    // workspace; the plain instantiations only)
    const bool direct = !PFX && a.work_counter == nullptr;
    if (!direct) build_unit_order<PFX>(a, s_pf, s_pp, s_ctx, s_tail, &L.ntail, s_pages);
    const int n_tail = direct ? 0 : L.ntail;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int q = lane >> 4;  // row group: tokens 4q..4q+3 of a tile
    const int c = lane & 15;  // column (head c % G); K and V chunk c

    const char *kbase = reinterpret_cast<const char *>(a.key_cache);
    const char *vbase = reinterpret_cast<const char *>(a.value_cache);
    const int bs = a.block_size;
    const int lbs = a.log2_block_size;
    const int64_t tok_stride = (int64_t)a.num_kv_heads * KV_ROW;  // bytes between slots
    char *kt = s_region[wave];

    Unit u;
    bool first = true;
    // this workgroup's index among the drawers (the last `drawers` of the grid)
    const int drawer = (int)blockIdx.x - ((int)gridDim.x - drawers);
    while (direct ? direct_unit(a, u, first)
                  : draw_unit<PFX>(a, s_pf, s_pp, s_ctx, s_tail, n_tail, &L.unit, u, drawers, drawer,
                                   first)) {
        if (tid == 0) s_bad = 0;

        // query operand: head h0 + c % G, chunks 4j + q
        const int h0 = u.kvh * G;
        u32x4 qop[4];  // in registers, or parked in LDS (kQopLds) and read per tile
        {
            const char *row = reinterpret_cast<const char *>(a.query) +
                              ((int64_t)u.s * a.num_heads + h0 + c % G) * ROW_BYTES;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qop[j] = load16(row + (4 * j + q) * 16);
                // every wave of the unit holds the same operand: wave 0 parks
                // it before the segment loop's first barrier
                if (kQopLds && wave == 0) s_qop[j][lane] = qop[j];
            }
        }

        // The decode step's new token (W): the unit whose range holds its
        // sequence's position ctx - 1 stores the new K and V rows of its KV
        // head at the slot, and reads that token from the new rows instead
        // of the pool (no other unit reads those bytes, so the launch needs
        // no ordering between the store and the reads).  A slot that is not
        // the table's slot of ctx - 1 makes the sequence NaN and is not
        // written.
        int nt = -1;  // position of the new token this unit holds, or -1
        if constexpr (W) {
            const int pos = u.ctx - 1;
            if (!u.bad_len && pos >= u.tok_begin && pos < u.tok_end) {
                const int64_t slot = a.slot_mapping[u.s];
                if (slot >= 0) {
                    const int32_t pb = a.block_tables[(int64_t)u.s * a.max_blocks_per_seq + (pos >> lbs)];
                    const bool ok = pb >= 0 && (int64_t)pb < a.num_blocks &&
                                    slot == (int64_t)pb * bs + (pos & (bs - 1));
                    if (ok) {
                        nt = pos;
                        if (wave == 0 && q == 0) {  // 16 lanes: 16-byte chunk c of each row
                            const int64_t src = ((int64_t)u.s * a.num_kv_heads + u.kvh) * KV_ROW + c * KV_CHUNK;
                            const int64_t dst = slot * tok_stride + (int64_t)u.kvh * KV_ROW + c * KV_CHUNK;
                            store16(const_cast<char *>(kbase) + dst,
                                    load16(reinterpret_cast<const char *>(a.new_key) + src));
                            store16(const_cast<char *>(vbase) + dst,
                                    load16(reinterpret_cast<const char *>(a.new_value) + src));
                        }
                    } else if (tid == 0) {
                        s_bad = 1;
                    }
                }
            }
        }

        const int64_t kvh_off = (int64_t)u.kvh * KV_ROW;
        float sl2 = a.scale_log2e;
        if constexpr (KV8) sl2 *= a.k_scale[u.kvh];

        // page ids staged in LDS for tokens [stg_lo, stg_hi) (npages pages);
        // the running state of the partition being streamed; tokens at or
        // past seg_end are masked.  All wave-uniform.
        int stg_lo = u.tok_begin, stg_hi = u.tok_begin, npages = 0, seg_end = 0;
        float m = -INFINITY;  // reference max of column c (equal in the four row groups)
        float lsum = 0.f;     // this lane's share of column c's normaliser
        f32x4_t acc[8];       // block dt: dims 8 (4q + r) + dt of column c
        auto reset = [&]() {
            m = -INFINITY;
            lsum = 0.f;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        };
        auto stage = [&](int lo, int hi) {
            stg_lo = lo;  // a page boundary: partitions and staged windows start on one
            stg_hi = hi;
            npages = (hi - lo + bs - 1) >> lbs;
            __syncthreads();  // the previous window's readers are done with s_pages
            stage_pages(a, u, lo >> lbs, npages, s_pages, &s_bad);
            __syncthreads();
        };

        // Byte offset of this lane's chunk of token t0 + 4q, the first of
        // its four consecutive tokens (t0 is a multiple of 4 and pages
        // hold >= 4 tokens, so the four share a page and lie one
        // tok_stride apart).  A token at or past seg_end (the end of the
        // partition or of the staged window) or on a bad page id
        // reads a row of page 0 (always in the pool) and is flagged
        // invalid in `vmask` (its V zeroed; its score masked, or the
        // output made NaN by the bad-page flag).
        auto tile_base = [&](int t0, uint32_t &vmask) -> int64_t {
            const int t = t0 + 4 * q;
            const int pb = s_pages[min((t - stg_lo) >> lbs, npages - 1)];
            const int n_ok = pb >= 0 ? min(max(seg_end - t, 0), 4) : 0;
            vmask = (1u << n_ok) - 1u;
            const int64_t page = pb >= 0 ? pb : 0;
            return (page * bs + (t & (bs - 1))) * tok_stride + kvh_off + c * KV_CHUNK;
        };
        // Row `alt_row` of the lane's four (if 0..3) is read from `alt`
        // instead of the pool: the decode step's new token.
        auto load_k = [&](TileRegs &r, int t0, int alt_row = -1, const char *alt = nullptr) {
            uint32_t unused;
            const char *p = kbase + tile_base(t0, unused);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const char *pi = p + i * tok_stride;
                if constexpr (W) pi = i == alt_row ? alt : pi;
                if constexpr (KV8) r.k[i] = load8_stream(pi);
                else r.k[i] = load16_stream(pi);
            }
        };
        auto load_v = [&](TileRegs &r, int t0, int alt_row = -1, const char *alt = nullptr) {
            const char *p = vbase + tile_base(t0, r.vmask);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const char *pi = p + i * tok_stride;
                if constexpr (W) pi = i == alt_row ? alt : pi;
                if constexpr (KV8) r.v[i] = load8_stream(pi);
                else r.v[i] = load16_stream(pi);
            }
        };
        // S^T of one tile: K rows -> LDS (16-byte chunks XOR-swizzled by
        // token), read back so that lane (q, c) holds token c, chunks
        // 4j + q; four MFMAs against the query operand.  Rows are private
        // to the wave and its LDS operations complete in order.
        auto tile_scores = [&](const TileRegs &r) -> f32x4_t {
            // E4M3 rows stay 8-bit in LDS (8-byte chunks, 128-byte rows)
            // and are widened after the read, one operand at a time
            constexpr int LROW = KV8 ? D : ROW_BYTES;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = 4 * q + i;
                char *dst = kt + tt * LROW + ((c ^ tt) & 15) * KV_CHUNK;
                if constexpr (KV8) *reinterpret_cast<u32x2 *>(dst) = r.k[i];
                else *reinterpret_cast<u32x4 *>(dst) = r.k[i];
            }
            asm volatile("" ::: "memory");
            f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const char *src = kt + c * LROW + (((4 * j + q) ^ c) & 15) * KV_CHUNK;
                u32x4 kop;
                if constexpr (KV8) kop = widen_e4m3<DT>(*reinterpret_cast<const u32x2 *>(src));
                else kop = *reinterpret_cast<const u32x4 *>(src);
                sacc = mfma_16x16x32<DT>(kop, kQopLds ? s_qop[j][lane] : qop[j], sacc);
            }
            asm volatile("" ::: "memory");
            return sacc;
        };
        // softmax and value product of the pair (tiles A, B at t0, t0 + 16)
        // whose scores are sa, sb
        auto pair_values = [&](const f32x4_t sa, const f32x4_t sb, const TileRegs &ra,
                               const TileRegs &rb, int t0) {
            float sc[8];  // tokens t0 + 4q + i (i < 4), t0 + 16 + 4q + i - 4 (i >= 4)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[i] = sa[i] * sl2;
                sc[4 + i] = sb[i] * sl2;
            }
            if (t0 + 2 * TILE > seg_end) {  // wave-uniform: only at the end of a segment
                // tokens of this lane before the end; the count passes
                // through an empty asm inside the branch, so the compares
                // cannot be hoisted out of it
                int nv = seg_end - (t0 + 4 * q);
                asm volatile("" : "+v"(nv));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sc[i] = (i < nv) ? sc[i] : -INFINITY;
                    sc[4 + i] = (TILE + i < nv) ? sc[4 + i] : -INFINITY;
                }
            }
            float mx = sc[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
            mx = rowgroup_max(mx);
            const bool bump = mx > m + kMaxSlack;  // m = -inf: any valid score
            if (__builtin_amdgcn_ballot_w64(bump)) {
                const float alpha = !bump ? 1.f : (m == -INFINITY ? 0.f : fast_exp2(m - mx));
                m = bump ? mx : m;
                lsum *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acc[dt] *= alpha;
            }
            // m = -inf only while the column has seen no valid score:
            // every score here is then masked and 2^(-inf - 0) = 0
            const float mref = m == -INFINITY ? 0.f : m;
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sc[i] = fast_exp2(sc[i] - mref);
                ps += sc[i];
            }
            lsum += ps;
            u32x4 ph, pl;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t hi, lo;
                split_pack<DT>(sc[2 * w], sc[2 * w + 1], hi, lo);
                ph[w] = hi;
                pl[w] = lo;
            }

            // value operands: this lane's V rows (tokens 4q + i of tiles A
            // and B, dims 8c..8c+7); invalid rows (past the segment, bad
            // page) become zeros, since a zero probability times a NaN
            // row would still be NaN
            using VRow = std::conditional_t<KV8, u32x2, u32x4>;
            VRow va[4], vb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                va[i] = ra.v[i];
                vb[i] = rb.v[i];
            }
            if (__builtin_amdgcn_ballot_w64((ra.vmask & rb.vmask) != 0xFu)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    va[i] = (ra.vmask >> i) & 1u ? va[i] : VRow{};
                    vb[i] = (rb.vmask >> i) & 1u ? vb[i] : VRow{};
                }
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // word w of each row (dims 8c + 2w, + 1) in 16-bit form
                uint32_t xa[4], xb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (KV8) {
                        xa[i] = (w & 1) ? e4m3_pair<DT, true>(w < 2 ? va[i].x : va[i].y)
                                        : e4m3_pair<DT, false>(w < 2 ? va[i].x : va[i].y);
                        xb[i] = (w & 1) ? e4m3_pair<DT, true>(w < 2 ? vb[i].x : vb[i].y)
                                        : e4m3_pair<DT, false>(w < 2 ? vb[i].x : vb[i].y);
                    } else {
                        xa[i] = va[i][w];
                        xb[i] = vb[i][w];
                    }
                }
#pragma unroll
                for (int odd = 0; odd < 2; ++odd) {
                    // dim 8c + 2w + odd: v_perm pairs the 16-bit halves
                    // of two tokens
                    const int dt = 2 * w + odd;
                    const uint32_t sel = odd ? 0x07060302u : 0x05040100u;
                    u32x4 vop;
                    vop[0] = __builtin_amdgcn_perm(xa[1], xa[0], sel);
                    vop[1] = __builtin_amdgcn_perm(xa[3], xa[2], sel);
                    vop[2] = __builtin_amdgcn_perm(xb[1], xb[0], sel);
                    vop[3] = __builtin_amdgcn_perm(xb[3], xb[2], sel);
                    acc[dt] = mfma_16x16x32<DT>(vop, ph, acc[dt]);
                    acc[dt] = mfma_16x16x32<DT>(vop, pl, acc[dt]);
                }
            }
        };

        // Each wave step issues the loads of TPS consecutive tiles at once,
        // then computes them pair by pair; steps start at t_first and move
        // by t_stride while below seg_end.  A tile past seg_end is all
        // invalid and computes to no change.
        auto stream = [&](int t_first, int t_stride) {
            for (int t = t_first; t < seg_end; t += t_stride) {
                TileRegs r[TPS];
                if (W && nt >= t && nt < t + TPS * TILE) {
                    // the step holding the new token: the lanes that hold
                    // its row read it from new_key/new_value (offsets
                    // recomputed here, so no pointer stays live across the
                    // stream)
                    const int d = nt - t;
                    const int ti = d >> 4, rn = q == ((d >> 2) & 3) ? d & 3 : -1;
                    const int64_t src = ((int64_t)u.s * a.num_kv_heads + u.kvh) * KV_ROW + c * KV_CHUNK;
                    const char *nk = reinterpret_cast<const char *>(a.new_key) + src;
                    const char *nv = reinterpret_cast<const char *>(a.new_value) + src;
#pragma unroll
                    for (int i = 0; i < TPS; ++i) {
                        load_k(r[i], t + i * TILE, i == ti ? rn : -1, nk);
                        load_v(r[i], t + i * TILE, i == ti ? rn : -1, nv);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < TPS; ++i) {
                        load_k(r[i], t + i * TILE);
                        load_v(r[i], t + i * TILE);
                    }
                }
                // keep every load of the step ahead of the compute
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TPS; i += 2) {
                    const f32x4_t sa = tile_scores(r[i]);
                    const f32x4_t sb = tile_scores(r[i + 1]);
                    pair_values(sa, sb, r[i], r[i + 1], t + i * TILE);
                }
            }
        };

        reset();
        if (RUNS && u.tok_end - u.tok_begin == kNumWaves * a.partition_size) {
            // A whole run: wave w streams partition part0 + w alone, so the
            // waves meet only at the epilogue, which joins their four states
            // into the run's one partial (a quarter of the partials for the
            // merge to read).
            stage(u.tok_begin, u.tok_end);
            const int pt = u.tok_begin + wave * a.partition_size;
            seg_end = pt + a.partition_size;
            stream(pt, TILE * TPS);
        } else {
            // One partition, the four waves interleaved (32-token pairs);
            // page ids staged for up to kSegPages pages of it at a time.
            for (int seg = u.tok_begin; seg < u.tok_end; seg = seg_end) {
                if (seg >= stg_hi) stage(seg, min(u.tok_end, seg + (kSegPages << lbs)));
                seg_end = min(u.tok_end, stg_hi);
                stream(seg + wave * TILE * TPS, kNumWaves * TILE * TPS);
            }
        }

        // Epilogue: the column's normaliser is the sum over the four row
        // groups; lanes (q, c < G) hold head c's dims 32q + 8r + dt in
        // acc[dt][r].  The waves' states meet in LDS, and the unit stores
        // the output (an unsplit sequence) or its partial, in slot u.p of
        // the row (one slot per unit).
        const float Lc = rowgroup_sum(lsum);
        float *wacc = reinterpret_cast<float *>(kt);
        if (c < G) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *dst = wacc + c * D + 32 * q + 8 * r;
                *reinterpret_cast<f32x4_t *>(dst) = f32x4_t{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
                *reinterpret_cast<f32x4_t *>(dst + 4) = f32x4_t{acc[4][r], acc[5][r], acc[6][r], acc[7][r]};
            }
            if (q == 0) {
                s_m[wave][c] = m;
                s_l[wave][c] = Lc;
            }
        }
        __syncthreads();
        unit_epilogue<DT, D, G, PFX, kRegion / 4>(a, u, u.p, u.bad_len || s_bad != 0, s_m, s_l,
                                                         reinterpret_cast<const float *>(&s_region[0][0]),
                                                         KV8 ? a.v_scale[u.kvh] : 1.f);
        // the next draw starts with a barrier: every wave's region has been
        // read before the next unit's K tiles land there
    }
}

template <int DT, int G, bool PFX, bool KV8, bool RUNS, bool W = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PKV_DECODE_MIN_WAVES, 8)))
void paged_decode_mfma_kernel(DecodeArgs a) {
    extern __shared__ int s_dyn[];
    __shared__ DecodeLds<G, qop_in_lds<KV8>()> lds;
    decode_body<DT, G, PFX, KV8, RUNS, W>(a, s_dyn, lds, gridDim.x);
}

// Shared-prefix decode in one launch: workgroups [0, prefix_wgs) each run one
// prefix unit (units of one (KV head, split) on one XCD), the others are the
// persistent suffix grid.  The prefix units are latency-bound and the suffix
// streams from HBM, so the two overlap; their LDS is one union.  Every suffix
// partition writes a partial; a merge kernel joins them with the prefix's.
template <int DT, int G, bool RUNS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PKV_DECODE_MIN_WAVES, 8)))
void paged_prefix_fused_kernel(DecodeArgs a, PrefixArgs p, int prefix_wgs) {
    extern __shared__ int s_dyn[];
    __shared__ union {
        DecodeLds<G, qop_in_lds<false>()> d;
        PrefixLds x;
    } lds;
    if ((int)blockIdx.x < prefix_wgs) {
        prefix_unit<DT>(p, xcd_unit(blockIdx.x, prefix_wgs), lds.x);
        return;
    }
    decode_body<DT, G, true, false, RUNS>(a, s_dyn, lds.d, (int)gridDim.x - prefix_wgs);
}

// Resident workgroups per CU of a kernel and the CU count, per (kernel,
// device, dynamic LDS rounded up to 4 KiB): the HIP queries run once per
// entry, not on every call.  Rounding the LDS up can only lower the count.
namespace {
struct OccEntry {
    const void *fn;
    int dev;
    int dyn_kb4;
    int cus;
    int per_cu;
};
constexpr int kOccEntries = 256;
std::mutex g_occ_mu;
OccEntry g_occ[kOccEntries];
int g_occ_n = 0;

hipError_t occupancy(const void *fn, size_t dyn, int &cus, int &per_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int kb4 = (int)((dyn + 4095) / 4096);
    {
        std::lock_guard<std::mutex> lock(g_occ_mu);
        for (int i = 0; i < g_occ_n; ++i)
            if (g_occ[i].fn == fn && g_occ[i].dev == dev && g_occ[i].dyn_kb4 == kb4) {
                cus = g_occ[i].cus;
                per_cu = g_occ[i].per_cu;
                return hipSuccess;
            }
    }
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, (size_t)kb4 * 4096);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_occ_mu);
    if (g_occ_n < kOccEntries) g_occ[g_occ_n++] = OccEntry{fn, dev, kb4, cus, per_cu};
    return hipSuccess;
}
}  // namespace

// Workgroups of a persistent grid: as many as are resident at once
// (occupancy with `dyn` bytes of dynamic LDS), at most PKV_WG_PER_CU per CU,
// capped by `units`.  0 on a HIP error (returned in `e`).
// Dynamic LDS of the unit-order tables: three int arrays of B (+ 1) and the
// 16-bit tail list, rounded up to whole ints.
static size_t unit_order_bytes(int num_seqs) {
    return (size_t)(3 * num_seqs + 2) * sizeof(int) + ((size_t)num_seqs * 2 + 3) / 4 * 4;
}

template <typename K>
static int64_t resident_grid(K kernel, size_t dyn, int64_t units, hipError_t &e) {
    int cus = 0, per_cu = 0;
    e = occupancy(reinterpret_cast<const void *>(kernel), dyn, cus, per_cu);
    if (e != hipSuccess) return 0;
    if (per_cu > PKV_WG_PER_CU) per_cu = PKV_WG_PER_CU;
    const int64_t grid = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    return grid < units ? grid : units;
}

// Persistent grid: as many workgroups as are resident at once, capped by
// the number of units, drawing from the workspace counter.
// Without a workspace (one partition per sequence only) one workgroup per
// (sequence, KV head), no counter.
template <typename K>
static hipError_t launch_persistent(K kernel, const DecodeArgs &a, hipStream_t stream) {
    if (a.work_counter == nullptr) {
        const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads;
        hipLaunchKernelGGL(kernel, dim3((unsigned)units), dim3(kThreads), 0, stream, a);
        return hipGetLastError();
    }
    const size_t dyn = unit_order_bytes(a.num_seqs);
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions;  // upper bound
    hipError_t e;
    const int64_t grid = resident_grid(kernel, dyn, units, e);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), dyn, stream, a);
    return hipGetLastError();
}

// The kernels with the whole-run path (RUNS) are a second instantiation:
// compiled into the ordinary one it cost the GQA E4M3 and shared-prefix
// calls 0.7-2 us through register pressure.
template <int DT, int G, bool PFX, bool KV8, bool W = false>
static hipError_t launch_runs(const DecodeArgs &a, hipStream_t stream) {
    if (a.unit_parts == kNumWaves)
        return launch_persistent(paged_decode_mfma_kernel<DT, G, PFX, KV8, true, W>, a, stream);
    return launch_persistent(paged_decode_mfma_kernel<DT, G, PFX, KV8, false, W>, a, stream);
}

template <int DT, bool PFX, bool KV8 = false, bool W = false>
static hipError_t launch_group(const DecodeArgs &a, hipStream_t stream) {
    switch (a.num_heads / a.num_kv_heads) {
        case 1: return launch_runs<DT, 1, PFX, KV8, W>(a, stream);
        case 2: return launch_runs<DT, 2, PFX, KV8, W>(a, stream);
        case 4: return launch_runs<DT, 4, PFX, KV8, W>(a, stream);
        case 8: return launch_runs<DT, 8, PFX, KV8, W>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_paged_decode_mfma(const DecodeArgs &a, int dtype, hipStream_t stream) {
    if (dtype == kBF16) return launch_group<kBF16, false>(a, stream);
    if (dtype == kF16) return launch_group<kF16, false>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_paged_decode_mfma_write(const DecodeArgs &a, int dtype, hipStream_t stream) {
    if (dtype == kBF16) return launch_group<kBF16, false, false, true>(a, stream);
    if (dtype == kF16) return launch_group<kF16, false, false, true>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_paged_decode_mfma_e4m3(const DecodeArgs &a, int dtype, hipStream_t stream) {
    if (dtype == kBF16) return launch_group<kBF16, false, true>(a, stream);
    if (dtype == kF16) return launch_group<kF16, false, true>(a, stream);
    return hipErrorInvalidValue;
}

// The fused shared-prefix launch: prefix_units workgroups for the prefix,
// then the persistent suffix grid (resident_grid over the suffix units).
template <int DT, int G, bool RUNS>
static hipError_t launch_fused(const PrefixArgs &p, const DecodeArgs &a, int64_t prefix_units,
                               hipStream_t stream) {
    auto kernel = paged_prefix_fused_kernel<DT, G, RUNS>;
    const size_t dyn = unit_order_bytes(a.num_seqs);
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions;  // upper bound
    hipError_t e;
    const int64_t grid = resident_grid(kernel, dyn, units, e);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3((unsigned)(prefix_units + grid)), dim3(kThreads), dyn, stream, a, p,
                       (int)prefix_units);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_fused_group(const PrefixArgs &p, const DecodeArgs &a, hipStream_t stream) {
    const int64_t prefix_units = (int64_t)p.row_blocks * p.num_splits * p.num_kv_heads;
    const bool runs = a.unit_parts == kNumWaves;
    switch (a.num_heads / a.num_kv_heads) {
        case 1: return runs ? launch_fused<DT, 1, true>(p, a, prefix_units, stream)
                            : launch_fused<DT, 1, false>(p, a, prefix_units, stream);
        case 2: return runs ? launch_fused<DT, 2, true>(p, a, prefix_units, stream)
                            : launch_fused<DT, 2, false>(p, a, prefix_units, stream);
        case 4: return runs ? launch_fused<DT, 4, true>(p, a, prefix_units, stream)
                            : launch_fused<DT, 4, false>(p, a, prefix_units, stream);
        case 8: return runs ? launch_fused<DT, 8, true>(p, a, prefix_units, stream)
                            : launch_fused<DT, 8, false>(p, a, prefix_units, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_paged_prefix_fused(const PrefixArgs &p, const DecodeArgs &a, int dtype,
                                     hipStream_t stream) {
    if (dtype == kBF16) return launch_fused_group<kBF16>(p, a, stream);
    if (dtype == kF16) return launch_fused_group<kF16>(p, a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_paged_decode_mfma_suffix(const DecodeArgs &a, int dtype, hipStream_t stream) {
    if (a.work_counter == nullptr) return hipErrorInvalidValue;  // the suffix grid always draws
    if (dtype == kBF16) return launch_group<kBF16, true>(a, stream);
    if (dtype == kF16) return launch_group<kF16, true>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
