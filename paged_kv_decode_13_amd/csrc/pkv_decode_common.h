// Pieces shared by the two fused decode kernels: work-unit bookkeeping,
// staging of page ids in LDS, and the cross-wave epilogue (merge of the
// waves' running softmax states, then the output or the partition partial).
#pragma once

#include <math.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kNumWaves = kDecodeWaves;
constexpr int kThreads = kNumWaves * kWave;
constexpr int kSegPages = kDecodeSegPages;  // page ids staged in LDS at a time
// Lazy running max: a reference max moves only when passed by more than this
// (exp2 domain), so probabilities stay <= 256 and rescales are rare.
constexpr float kMaxSlack = 8.f;

struct Unit {
    int s, kvh, p;           // p: the unit's index among its sequence's units
    int ctx;
    int tok_begin, tok_end;  // token range of this unit
    int part0;               // partition index of the unit's first partition
    int nparts;              // partitions of this sequence (1: write out directly)
    bool bad_len;            // length outside what the table / grid can cover
    bool empty;              // unit past the end of its sequence: exit
};

// A context length the grid or the table cannot cover makes the sequence's
// output NaN instead of reading outside the table.
__device__ __forceinline__ bool bad_context(const DecodeArgs &a, int ctx) {
    return ctx < 0 || ctx > a.max_context_len ||
           (int64_t)ctx > (int64_t)a.max_blocks_per_seq * a.block_size;
}

// First token a launch reads: 0, or the end of a shared prefix when the
// launch covers only the rest of each history (PFX instantiations; the
// plain ones never read the extra fields, which keeps their registers).
template <bool PFX>
__device__ __forceinline__ int first_token(const DecodeArgs &a) {
    if constexpr (PFX) return a.token_begin; else return 0;
}

// Partitions of a sequence in the work list: its tokens [first_token, ctx)
// cut into partition_size pieces.  A sequence with nothing to read, or an
// out-of-range length, still gets one unit, which writes its zeros, empty
// partial or NaNs.
template <bool PFX = false>
__device__ __forceinline__ int seq_parts(const DecodeArgs &a, int ctx) {
    const int span = ctx - first_token<PFX>(a);
    if (bad_context(a, ctx) || span <= 0) return 1;
    return (span + a.partition_size - 1) / a.partition_size;
}

// Full partitions of a sequence (its last partition is partial when the
// span is not a multiple of the partition size; an empty or out-of-range
// context has one partial unit).
template <bool PFX = false>
__device__ __forceinline__ int seq_full(const DecodeArgs &a, int ctx) {
    const int span = ctx - first_token<PFX>(a);
    if (bad_context(a, ctx) || span <= 0) return 0;
    return span / a.partition_size;
}

// Work units of the persistent kernels.  With unit_parts == 1 a unit is one
// partition.  With unit_parts == kNumWaves a sequence's span starts with
// runs of kNumWaves whole partitions, one unit each, in which every wave
// streams one partition alone (the waves meet only at the unit's epilogue,
// which joins their four partition states); the rest of the span is one
// unit per partition.  Either way every unit of a split sequence writes one
// partial slot, so a row has seq_units slots for the merge to join.
__device__ __forceinline__ int run_tokens(const DecodeArgs &a) { return a.partition_size * a.unit_parts; }

// Units of a sequence that are whole runs of unit_parts partitions.
template <bool PFX = false>
__device__ __forceinline__ int seq_full_units(const DecodeArgs &a, int ctx) {
    const int span = ctx - first_token<PFX>(a);
    if (bad_context(a, ctx) || span <= 0) return 0;
    return span / run_tokens(a);
}

// All units of a sequence: its whole runs, then one per remaining partition
// (at least one unit, which writes the zeros, empty partial or NaNs of a
// sequence with nothing to read).
template <bool PFX = false>
__device__ __forceinline__ int seq_units(const DecodeArgs &a, int ctx) {
    const int span = ctx - first_token<PFX>(a);
    if (bad_context(a, ctx) || span <= 0) return 1;
    const int runs = span / run_tokens(a);
    const int rest = span - runs * run_tokens(a);
    return runs + (rest + a.partition_size - 1) / a.partition_size;
}

// Whole single partitions after a sequence's runs (not its last partition
// when that one is partial).
template <bool PFX = false>
__device__ __forceinline__ int seq_whole_singles(const DecodeArgs &a, int ctx) {
    const int span = ctx - first_token<PFX>(a);
    if (bad_context(a, ctx) || span <= 0) return 0;
    return (span % run_tokens(a)) / a.partition_size;
}

// Tokens of a sequence's tail unit -- its last partition when that one is
// partial -- or -1 when it has none.  A sequence with nothing to read or an
// out-of-range length has a tail unit of 0 tokens (it writes the zeros,
// empty partial or NaNs).
template <bool PFX = false>
__device__ __forceinline__ int seq_tail_tokens(const DecodeArgs &a, int ctx) {
    const int span = ctx - first_token<PFX>(a);
    if (bad_context(a, ctx) || span <= 0) return 0;
    const int rest = span % a.partition_size;
    return rest > 0 ? rest : -1;
}

__device__ __forceinline__ Unit make_unit(const DecodeArgs &a) {
    // KV head fastest: the units that read the same pages run side by side.
    int u = blockIdx.x;
    Unit r;
    r.kvh = u % a.num_kv_heads;
    u /= a.num_kv_heads;
    r.p = u % a.num_partitions;
    r.s = u / a.num_partitions;
    r.ctx = a.context_lens[r.s];
    r.bad_len = bad_context(a, r.ctx);
    r.tok_begin = r.p * a.partition_size;
    r.empty = r.p > 0 && (r.bad_len || r.tok_begin >= r.ctx);
    r.tok_end = r.bad_len ? 0 : min(r.ctx, r.tok_begin + a.partition_size);
    r.nparts = (r.bad_len || r.ctx == 0) ? 1 : (r.ctx + a.partition_size - 1) / a.partition_size;
    r.part0 = r.p;
    return r;
}

// Inclusive prefix sum across the 64 lanes of a wave by DPP lane moves (no
// LDS round trips): shifts by 1, 2, 4 and 8 lanes within each row of 16,
// then the last lane of rows 0 and 2 added to rows 1 and 3, then lane 31 to
// rows 2 and 3.  Lanes a shift reads from outside the row add 0; rows
// outside a row mask keep their value.
__device__ __forceinline__ int wave_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Inclusive prefix sum over the workgroup's NT threads: a scan in each wave,
// then each wave adds the totals of the waves before it (s_scan: NT / 64
// ints).  Ends with a barrier, so s_scan can be reused.
template <int NT = kThreads>
__device__ __forceinline__ int block_scan(int v, int *s_scan) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int x = wave_scan(v);
    if (lane == kWave - 1) s_scan[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_scan[w];
    __syncthreads();
    return x + base;
}

// Largest s in [0, n) with pre[s] <= x (pre non-decreasing, pre[0] = 0 <= x).
__device__ __forceinline__ int search_le(const int *pre, int n, int x) {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

// The same by a whole wave (every lane active; pre in LDS, x wave-uniform):
// a 64-way search, each round one LDS read per lane and a ballot.  Lane l
// probes entry lo + l * stride; the probes <= x form a prefix of the lanes,
// whose length narrows the range 64-fold.  Up to 4096 entries take two
// rounds where a binary search takes up to 12 dependent reads.
__device__ __forceinline__ int wave_search_le(const int *pre, int n, int x) {
    const int lane = threadIdx.x & (kWave - 1);
    int lo = 0, len = n;  // the answer lies in [lo, lo + len)
    while (len > 1) {
        const int stride = (len + kWave - 1) / kWave;
        const int i = lo + lane * stride;
        const bool le = lane * stride < len && pre[i] <= x;
        const int c = __popcll(__ballot(le));  // >= 1: pre[lo] <= x
        lo += (c - 1) * stride;
        len = min(stride, len - (c - 1) * stride);
    }
    return lo;
}

// Stage the physical block ids of logical blocks [lb0, lb0 + npages) of the
// sequence in LDS (-1 and a flag for ids outside the pool).  Caller brackets
// with __syncthreads().
__device__ __forceinline__ void stage_pages(const DecodeArgs &a, const Unit &u, int lb0, int npages,
                                            int *s_pages, int *s_bad) {
    const int32_t *table = a.block_tables + (int64_t)u.s * a.max_blocks_per_seq;
    for (int i = threadIdx.x; i < npages; i += kThreads) {
        int pb = table[lb0 + i];
        if (pb < 0 || (int64_t)pb >= a.num_blocks) {
            *s_bad = 1;
            pb = -1;
        }
        s_pages[i] = pb;
    }
}

template <int DT>
__device__ __forceinline__ void store_out(const DecodeArgs &a, int64_t idx, float v) {
    if (a.out_f32) {
        reinterpret_cast<float *>(a.out)[idx] = v;
    } else if constexpr (DT == kF32) {
        reinterpret_cast<float *>(a.out)[idx] = v;
    } else {
        reinterpret_cast<uint16_t *>(a.out)[idx] = f32_to_bits16<DT>(v);
    }
}

// Merge the per-wave states (running max m, normaliser l, unnormalised
// accumulator) of partition pi of a unit's sequence and store either the
// final output (one partition) or the partition's normalised partial with
// its (m, l).  Wave w's accumulator of head g is s_acc[w * WS + g * D + 0 ..
// D - 1].
template <int DT, int D, int G, bool PFX = false, int WS = G * D>
__device__ __forceinline__ void unit_epilogue(const DecodeArgs &a, const Unit &u, int pi, bool bad,
                                              const float (*s_m)[G], const float (*s_l)[G],
                                              const float *s_acc, float vscale = 1.f) {
    const int h0 = u.kvh * G;
    for (int i = threadIdx.x; i < G * D; i += kThreads) {
        const int g = i / D;
        const int d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kNumWaves; ++w) M = fmaxf(M, s_m[w][g]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kNumWaves; ++w) {
            const float f = (M == -INFINITY) ? 0.f : fast_exp2(s_m[w][g] - M);
            L += s_l[w][g] * f;
            O += s_acc[w * WS + g * D + d] * f;
        }
        const int h = h0 + g;
        float res = L > 0.f ? O / L * vscale : 0.f;  // empty context -> zeros
        if (bad) res = __builtin_nanf("");
        // a suffix launch stores the output only with no prefix to join
        if ((!PFX || a.direct_out) && u.nparts == 1) {
            store_out<DT>(a, ((int64_t)u.s * a.num_heads + h) * D + d, res);
        } else {
            // a suffix launch writes its partials after the prefix's slots
            const int64_t slot = PFX ? ((int64_t)u.s * a.num_heads + h) * a.part_stride + a.part_base + pi
                                     : ((int64_t)u.s * a.num_heads + h) * a.num_partitions + pi;
            a.part_out[slot * D + d] = res;
            if (d == 0) {
                a.part_ml[slot * 2] = bad ? __builtin_nanf("") : M;
                a.part_ml[slot * 2 + 1] = L;
            }
        }
    }
}

// Log-sum-exp join of the n partial results in slots base .. base + n - 1
// (normalised output o_p, max m_p and normaliser l_p in the exp2 domain):
// out = sum_p w_p o_p / sum_p w_p with w_p = l_p 2^(m_p - max_q m_q), stored at
// out[out_idx .. + D).  A workgroup of NW waves: all threads find the max,
// then wave w joins partials w, w + NW, ... (lane: dims lane + 64 j) with
// several partials' loads in flight, and with NW > 1 the waves' sums are
// added in LDS.  A NaN max (bad page) makes its weight and so the output
// NaN.
template <int DT, int D, int NW>
__device__ __forceinline__ void merge_partials(const DecodeArgs &a, int64_t base, int n, int64_t out_idx) {
    constexpr int PL = D / kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    float M = -INFINITY;
    for (int p = tid; p < n; p += NW * kWave) M = fmaxf(M, a.part_ml[(base + p) * 2]);
    M = group_max<kWave>(M);
    if constexpr (NW > 1) {
        __shared__ float s_red[NW];
        if (lane == 0) s_red[wave] = M;
        __syncthreads();
        M = s_red[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, s_red[w]);
    }
    float L = 0.f, O[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) O[j] = 0.f;
#pragma unroll 8
    for (int p = wave; p < n; p += NW) {
        const float w = a.part_ml[(base + p) * 2 + 1] * fast_exp2(a.part_ml[(base + p) * 2] - M);
        L += w;
#pragma unroll
        for (int j = 0; j < PL; ++j) O[j] = fmaf(w, a.part_out[(base + p) * D + lane + j * kWave], O[j]);
    }
    if constexpr (NW == 1) {
#pragma unroll
        for (int j = 0; j < PL; ++j) store_out<DT>(a, out_idx + lane + j * kWave, O[j] / L);
    } else {
        __shared__ float s_lw[NW];
        __shared__ float s_ow[NW][D];
#pragma unroll
        for (int j = 0; j < PL; ++j) s_ow[wave][lane + j * kWave] = O[j];
        if (lane == 0) s_lw[wave] = L;
        __syncthreads();
        for (int d = tid; d < D; d += NW * kWave) {
            float o = 0.f, l = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                o += s_ow[w][d];
                l += s_lw[w];
            }
            store_out<DT>(a, out_idx + d, o / l);
        }
    }
}
// Merges of rows with up to kNumWaves * kMergeEarly partials: each of NW
// waves issues the loads of its kMergeEarly slots (wave w: slots
// w * kMergeEarly ..) together with the row's length lookup, before the
// number of partials n is known (slots below `cap`, the row's slot count,
// always lie in the workspace; values past n are never used), so such a row
// costs one memory round trip instead of three (length, maxima, partials).
// Rows with more slots use merge_partials.
constexpr int kMergeEarly = 8;

// Waves of an early-load merge for rows of up to `slots` partials (slots
// past kMergeEarly per wave are loaded after the length lookup), or 0: the
// loop merge (merge_partials, four waves) for longer rows.
inline int merge_waves(int64_t slots) {
    if (slots <= kMergeEarly) return 1;
    if (slots <= 2 * kMergeEarly) return 2;
    if (slots <= kNumWaves * kMergeEarly) return kNumWaves;
    return 0;
}

template <int D>
struct EarlyPartials {
    float m[kMergeEarly], l[kMergeEarly];
    float o[kMergeEarly][D / kWave];
};

template <int D>
__device__ __forceinline__ void load_early(const DecodeArgs &a, int64_t base, int cap, EarlyPartials<D> &e) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int k = 0; k < kMergeEarly; ++k) {
        if (k < cap) {
            const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + (base + k) * 2);
            e.m[k] = ml.x;
            e.l[k] = ml.y;
#pragma unroll
            for (int j = 0; j < D / kWave; ++j) e.o[k][j] = a.part_out[(base + k) * D + lane + j * kWave];
        }
    }
}

// out = sum_p w_p o_p / sum_p w_p, w_p = l_p 2^(m_p - max_q m_q), over the n
// slots from base.  Wave w holds slots w * kMergeEarly .. + kMergeEarly - 1
// in `e` (see load_early) and loads slots NW * kMergeEarly + w, + NW, ...
// itself; with NW > 1 the waves' maxima and sums meet in LDS.  A NaN max
// makes the output NaN.
template <int DT, int D, int NW>
__device__ __forceinline__ void merge_early(const DecodeArgs &a, const EarlyPartials<D> &e, int64_t base,
                                            int n, int64_t out_idx) {
    constexpr int PL = D / kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = NW == 1 ? 0 : tid / kWave;  // a one-wave merge may share its workgroup
    const int k0 = wave * kMergeEarly;           // this wave's first early slot
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeEarly; ++k)
        if (k0 + k < n) M = fmaxf(M, e.m[k]);
    for (int p = NW * kMergeEarly + wave; p < n; p += NW) M = fmaxf(M, a.part_ml[(base + p) * 2]);
    if constexpr (NW > 1) {
        __shared__ float s_m[NW];
        if (lane == 0) s_m[wave] = M;
        __syncthreads();
        M = s_m[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w]);
    }
    float L = 0.f, O[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) O[j] = 0.f;
#pragma unroll
    for (int k = 0; k < kMergeEarly; ++k) {
        if (k0 + k < n) {
            const float w = e.l[k] * fast_exp2(e.m[k] - M);
            L += w;
#pragma unroll
            for (int j = 0; j < PL; ++j) O[j] = fmaf(w, e.o[k][j], O[j]);
        }
    }
    for (int p = NW * kMergeEarly + wave; p < n; p += NW) {
        const float w = a.part_ml[(base + p) * 2 + 1] * fast_exp2(a.part_ml[(base + p) * 2] - M);
        L += w;
#pragma unroll
        for (int j = 0; j < PL; ++j) O[j] = fmaf(w, a.part_out[(base + p) * D + lane + j * kWave], O[j]);
    }
    if constexpr (NW == 1) {
#pragma unroll
        for (int j = 0; j < PL; ++j) store_out<DT>(a, out_idx + lane + j * kWave, O[j] / L);
    } else {
        __shared__ float s_lw[NW];
        __shared__ float s_ow[NW][D];
#pragma unroll
        for (int j = 0; j < PL; ++j) s_ow[wave][lane + j * kWave] = O[j];
        if (lane == 0) s_lw[wave] = L;
        __syncthreads();
        for (int d = tid; d < D; d += NW * kWave) {
            float o = 0.f, l = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                o += s_ow[w][d];
                l += s_lw[w];
            }
            store_out<DT>(a, out_idx + d, o / l);
        }
    }
}

// MFMA decode kernel launcher (16-bit caches, head_dim 128); the merge
// kernel is launched by the caller.  Without a workspace counter
// (a.work_counter == nullptr; one partition per sequence only) the grid is
// one workgroup per (sequence, KV head).
hipError_t launch_paged_decode_mfma(const DecodeArgs &a, int dtype, hipStream_t stream);
// The same with the decode step's slot write in the launch (a.new_key,
// a.new_value, a.slot_mapping set; see DecodeArgs).
hipError_t launch_paged_decode_mfma_write(const DecodeArgs &a, int dtype, hipStream_t stream);
// The same over E4M3 caches with per-KV-head scales (DT: query and output).
hipError_t launch_paged_decode_mfma_e4m3(const DecodeArgs &a, int dtype, hipStream_t stream);
// The same over tokens [token_begin, ctx), partials only (shared-prefix path).
hipError_t launch_paged_decode_mfma_suffix(const DecodeArgs &a, int dtype, hipStream_t stream);
// The shared-prefix units and that suffix decode in one launch (partials
// only; the caller merges).
hipError_t launch_paged_prefix_fused(const PrefixArgs &p, const DecodeArgs &a, int dtype,
                                     hipStream_t stream);

}  // namespace pkv
