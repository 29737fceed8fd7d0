// Fused paged decode attention for gfx950, and the log-sum-exp merge of its
// split-KV partials.
//
// What is computed (pages on PagedAttention):
//  - "实现教学版 PagedAttention：从 block table 读取历史 KV cache", section
//    "从逻辑 token 到物理 block": token t of a sequence lives at physical block
//    block_table[t / block_size], offset t % block_size;
//  - same page, section "从 gather 后的 K/V 做 attention": scores = q.K^T,
//    softmax, weighted sum of V, per query head;
//  - "从正确到更快：PagedAttention 的优化路线", section "高性能 PagedAttention
//    的核心思想": the kernel resolves each page itself while computing the
//    scores (no gathered copy), and section "attention kernel 真正在做什么":
//    scores are scaled by 1/sqrt(head_dim) and folded chunk by chunk into a
//    running max and normaliser instead of being stored;
//  - same page, section "Triton 适合做什么": one program per head group and a
//    segment of the history per program, with tail masking where the context
//    is not a multiple of the block size.
//
// Work unit = (sequence, KV head, KV partition); one 256-thread workgroup
// (4 waves) per unit.  The whole query-head group of the KV head is handled
// by the unit, so each K/V row is loaded once for all G query heads.
//
// Data path inside a unit:
//  1. the page ids of the partition are staged in LDS once (coalesced), so
//     the per-token page lookup is an LDS read, never a dependent global load;
//  2. every lane loads 16-byte vectors: a K/V row of D elements is read by
//     LPR = D*bytes/16 adjacent lanes (one 128-bit load each), so a wave
//     instruction reads RPW = 64/LPR whole rows;
//  3. the partial dot products are summed over the LPR lanes of a row with
//     DPP row exchanges;
//  4. each row group keeps its own running (max, normaliser, accumulator) in
//     registers; U rows per lane are folded in per step;
//  5. row groups are merged with lane shuffles, waves through LDS.
// Scores are kept in the exp2 domain (scale * log2 e folded into q).
#include <math.h>

#include "pkv_decode_common.h"

namespace pkv {

// W: the decode step's slot write is part of the launch, as in the matrix-core
// kernel: the unit holding position ctx - 1 stores the new rows of its KV
// head at a slot that must be that position's, and reads that token from
// the new rows instead of the pool.
template <int DT, int D, int G, bool W = false>
__global__ __launch_bounds__(kThreads) void paged_decode_valu_kernel(DecodeArgs a) {
    using TR = ElemTraits<DT>;
    constexpr int EPL = TR::per16;  // elements per lane per row
    constexpr int LPR = D / EPL;    // lanes per row
    constexpr int RPW = kWave / LPR;  // rows per wave instruction
    constexpr int U = 4;            // rows per lane per step
    constexpr int CHUNK = RPW * U;  // tokens per wave per step
    constexpr int ROW_BYTES = D * TR::bytes;
    static_assert(LPR >= 4 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row layout");

    __shared__ int s_pages[kSegPages];
    __shared__ int s_bad;
    __shared__ float s_m[kNumWaves][G];
    __shared__ float s_l[kNumWaves][G];
    __shared__ float s_acc[kNumWaves][G][D];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int rg = lane / LPR;  // row group inside the wave
    const int li = lane % LPR;  // 16-byte column inside the row

    const Unit up = make_unit(a);
    if (up.empty) return;
    const int tok_begin = up.tok_begin;
    const int tok_end = up.tok_end;
    if (tid == 0) s_bad = 0;

    int nt = -1;  // W: position of the new token this unit holds, or -1
    const char *nk_row = nullptr, *nv_row = nullptr;
    if constexpr (W) {
        const int pos = up.ctx - 1;
        if (!up.bad_len && pos >= tok_begin && pos < tok_end) {
            const int64_t slot = a.slot_mapping[up.s];
            if (slot >= 0) {
                const int32_t pb =
                    a.block_tables[(int64_t)up.s * a.max_blocks_per_seq + (pos >> a.log2_block_size)];
                const bool ok = pb >= 0 && (int64_t)pb < a.num_blocks &&
                                slot == (int64_t)pb * a.block_size + (pos & (a.block_size - 1));
                if (ok) {
                    nt = pos;
                    const int64_t row = ((int64_t)up.s * a.num_kv_heads + up.kvh) * ROW_BYTES;
                    nk_row = reinterpret_cast<const char *>(a.new_key) + row;
                    nv_row = reinterpret_cast<const char *>(a.new_value) + row;
                    if (wave == 0 && rg == 0) {  // LPR lanes: 16-byte column li of each row
                        const int64_t dst = (slot * a.num_kv_heads + up.kvh) * ROW_BYTES + li * 16;
                        store16(reinterpret_cast<char *>(const_cast<void *>(a.key_cache)) + dst,
                                load16(nk_row + li * 16));
                        store16(reinterpret_cast<char *>(const_cast<void *>(a.value_cache)) + dst,
                                load16(nv_row + li * 16));
                    }
                } else if (tid == 0) {
                    s_bad = 1;
                }
            }
        }
    }

    // query rows of the head group, pre-scaled into the exp2 domain
    const int h0 = up.kvh * G;
    float qf[G][EPL];
    {
        const char *qb = reinterpret_cast<const char *>(a.query);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t off = (((int64_t)up.s * a.num_heads + h0 + g) * D) * TR::bytes + li * 16;
            unpack16<DT>(load16(qb + off), qf[g]);
#pragma unroll
            for (int e = 0; e < EPL; ++e) qf[g][e] *= a.scale_log2e;
        }
    }

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    const char *kbase = reinterpret_cast<const char *>(a.key_cache);
    const char *vbase = reinterpret_cast<const char *>(a.value_cache);
    const int bs = a.block_size;
    const int lbs = a.log2_block_size;

    for (int seg = tok_begin; seg < tok_end; seg += kSegPages << lbs) {
        const int seg_end = min(tok_end, seg + (kSegPages << lbs));
        const int lb0 = seg >> lbs;
        const int npages = (seg_end - seg + bs - 1) >> lbs;
        __syncthreads();  // previous segment's readers are done with s_pages
        stage_pages(a, up, lb0, npages, s_pages, &s_bad);
        __syncthreads();

        for (int c = seg + wave * CHUNK; c < seg_end; c += kNumWaves * CHUNK) {
            u32x4 kr[U], vr[U];
            bool ok[U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int t = c + i * RPW + rg;
                ok[i] = t < seg_end;
                kr[i] = u32x4{0, 0, 0, 0};
                vr[i] = u32x4{0, 0, 0, 0};
                if (ok[i]) {
                    // token -> logical block -> physical block, block offset
                    const int pb = s_pages[(t - seg) >> lbs];
                    ok[i] = pb >= 0;
                    if (ok[i]) {
                        const int64_t row = ((int64_t)pb * bs + (t & (bs - 1))) * a.num_kv_heads + up.kvh;
                        const int64_t byte = row * ROW_BYTES + li * 16;
                        if (W && t == nt) {  // the new token: from the new rows
                            kr[i] = load16(nk_row + li * 16);
                            vr[i] = load16(nv_row + li * 16);
                        } else {
                            kr[i] = load16_stream(kbase + byte);
                            vr[i] = load16_stream(vbase + byte);
                        }
                    }
                }
            }

            float sc[G][U];
#pragma unroll
            for (int i = 0; i < U; ++i) {
                float kf[EPL];
                unpack16<DT>(kr[i], kf);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) d = fmaf(qf[g][e], kf[e], d);
                    d = group_sum<LPR>(d);
                    sc[g][i] = ok[i] ? d : -INFINITY;
                }
            }

#pragma unroll
            for (int g = 0; g < G; ++g) {
                float mc = sc[g][0];
#pragma unroll
                for (int i = 1; i < U; ++i) mc = fmaxf(mc, sc[g][i]);
                const float mn = fmaxf(m[g], mc);
                const bool none = mn == -INFINITY;  // nothing seen yet by this row group
                const float alpha = none ? 1.f : fast_exp2(m[g] - mn);
                m[g] = mn;
                l[g] *= alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
                for (int i = 0; i < U; ++i) sc[g][i] = none ? 0.f : fast_exp2(sc[g][i] - mn);
            }

#pragma unroll
            for (int i = 0; i < U; ++i) {
                float vf[EPL];
                unpack16<DT>(vr[i], vf);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    l[g] += sc[g][i];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(sc[g][i], vf[e], acc[g][e]);
                }
            }
        }
    }

    // merge the row groups of this wave (lanes li, li+LPR, ... hold one column)
#pragma unroll
    for (int msk = LPR; msk < kWave; msk <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mo = __shfl_xor(m[g], msk);
            const float lo = __shfl_xor(l[g], msk);
            const float mn = fmaxf(m[g], mo);
            const bool none = mn == -INFINITY;
            const float a1 = none ? 0.f : fast_exp2(m[g] - mn);
            const float a2 = none ? 0.f : fast_exp2(mo - mn);
            l[g] = l[g] * a1 + lo * a2;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float ao = __shfl_xor(acc[g][e], msk);
                acc[g][e] = acc[g][e] * a1 + ao * a2;
            }
            m[g] = mn;
        }
    }
    if (lane < LPR) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) s_acc[wave][g][li * EPL + e] = acc[g][e];
            if (li == 0) {
                s_m[wave][g] = m[g];
                s_l[wave][g] = l[g];
            }
        }
    }
    __syncthreads();

    unit_epilogue<DT, D, G>(a, up, up.p, up.bad_len || s_bad != 0, s_m, s_l, &s_acc[0][0][0]);
}

// Log-sum-exp merge of the partitions of one (sequence, query head), one
// workgroup of NW waves each (sequences with one partition were written
// directly).
template <int DT, int D, int NW, bool EARLY>
__global__ __launch_bounds__(NW * kWave) void lse_merge_kernel(DecodeArgs a) {
    const int s = blockIdx.x / a.num_heads;
    const int h = blockIdx.x % a.num_heads;
    const int64_t row = (int64_t)s * a.num_heads + h;
    const int ctx = a.context_lens[s];
    // one slot per work unit of the sequence (seq_units), one partition each
    // unless runs of unit_parts partitions were joined in the decode kernel
    if constexpr (EARLY) {
        EarlyPartials<D> e;
        const int k0 = (threadIdx.x / kWave) * kMergeEarly;
        load_early<D>(a, row * a.num_partitions + k0, a.num_partitions - k0, e);
        if (bad_context(a, ctx) || ctx == 0) return;  // written by partition 0
        if (seq_parts(a, ctx) <= 1) return;            // written directly
        merge_early<DT, D, NW>(a, e, row * a.num_partitions, seq_units(a, ctx), row * D);
    } else {
        if (bad_context(a, ctx) || ctx == 0) return;
        if (seq_parts(a, ctx) <= 1) return;
        merge_partials<DT, D, NW>(a, row * a.num_partitions, seq_units(a, ctx), row * D);
    }
}

// The same for rows of at most kMergeEarly slots, one wave per row and RW
// rows (consecutive heads of a sequence) per workgroup, for calls with many
// rows (the 256-sequence, 32-head batches: 8192 rows; the E4M3 call 279.8
// -> 279.0 us, the 16-bit one unchanged).
template <int DT, int D, int RW>
__global__ __launch_bounds__(RW * kWave) void lse_merge_rows_kernel(DecodeArgs a) {
    const int64_t row = (int64_t)blockIdx.x * RW + threadIdx.x / kWave;
    if (row >= (int64_t)a.num_seqs * a.num_heads) return;  // a whole wave
    const int s = (int)(row / a.num_heads);
    const int ctx = a.context_lens[s];
    EarlyPartials<D> e;
    load_early<D>(a, row * a.num_partitions, a.num_partitions, e);
    if (bad_context(a, ctx) || ctx == 0) return;  // written by partition 0
    if (seq_parts(a, ctx) <= 1) return;            // written directly
    merge_early<DT, D, 1>(a, e, row * a.num_partitions, seq_units(a, ctx), row * D);
}

template <int DT, int D, int G, bool W>
static hipError_t launch_valu(const DecodeArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions;
    hipLaunchKernelGGL((paged_decode_valu_kernel<DT, D, G, W>), dim3((unsigned)units), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <int DT, int D, bool W = false>
static hipError_t launch_valu_group(const DecodeArgs &a, hipStream_t stream) {
    switch (a.num_heads / a.num_kv_heads) {
        case 1: return launch_valu<DT, D, 1, W>(a, stream);
        case 2: return launch_valu<DT, D, 2, W>(a, stream);
        case 4: return launch_valu<DT, D, 4, W>(a, stream);
        case 8: return launch_valu<DT, D, 8, W>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

// Slots of a row whose context is the call's longest (the merge's
// typical row size: every unit of a split sequence writes one slot).
static int64_t slots_at_longest(const DecodeArgs &a) {
    const int64_t span = a.max_context_len;
    if (span <= 0) return 1;
    const int64_t run = (int64_t)a.partition_size * a.unit_parts;
    const int64_t runs = span / run, rest = span - runs * run;
    return runs + (rest + a.partition_size - 1) / a.partition_size;
}

template <int DT, int D>
static hipError_t launch_merge(const DecodeArgs &a, hipStream_t stream) {
    if (a.num_partitions <= 1) return hipSuccess;
    const unsigned rows = (unsigned)((int64_t)a.num_seqs * a.num_heads);
    constexpr int kRows = 4;
    switch (merge_waves(slots_at_longest(a))) {
        case 1:
            if (rows >= 4096)
                hipLaunchKernelGGL((lse_merge_rows_kernel<DT, D, kRows>), dim3((rows + kRows - 1) / kRows),
                                   dim3(kRows * kWave), 0, stream, a);
            else
                hipLaunchKernelGGL((lse_merge_kernel<DT, D, 1, true>), dim3(rows), dim3(kWave), 0, stream, a);
            break;
        case 2: hipLaunchKernelGGL((lse_merge_kernel<DT, D, 2, true>), dim3(rows), dim3(2 * kWave), 0, stream, a); break;
        case kNumWaves:
            hipLaunchKernelGGL((lse_merge_kernel<DT, D, kNumWaves, true>), dim3(rows), dim3(kThreads), 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL((lse_merge_kernel<DT, D, kNumWaves, false>), dim3(rows), dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

// W: the decode step with its slot write (a.new_key, a.new_value,
// a.slot_mapping set).
template <int DT, bool W = false>
static hipError_t launch_dtype(const DecodeArgs &a, int head_dim, hipStream_t stream) {
    hipError_t e;
    if (head_dim == 128 && DT != kF32) {  // 16-bit caches: the matrix-core kernel
        e = W ? launch_paged_decode_mfma_write(a, DT, stream) : launch_paged_decode_mfma(a, DT, stream);
        return e != hipSuccess ? e : launch_merge<DT, 128>(a, stream);
    }
    // binary32 caches or head_dim 64: the VALU kernel, one slot per partition
    DecodeArgs v = a;
    v.unit_parts = 1;
    if (head_dim == 128) {
        e = launch_valu_group<DT, 128, W>(v, stream);
        return e != hipSuccess ? e : launch_merge<DT, 128>(v, stream);
    }
    if (head_dim == 64) {
        e = launch_valu_group<DT, 64, W>(v, stream);
        return e != hipSuccess ? e : launch_merge<DT, 64>(v, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_paged_decode_e4m3(const DecodeArgs &a, int dtype, hipStream_t stream) {
    if ((int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions == 0) return hipSuccess;
    hipError_t e = launch_paged_decode_mfma_e4m3(a, dtype, stream);
    if (e != hipSuccess) return e;
    if (dtype == kBF16) return launch_merge<kBF16, 128>(a, stream);
    if (dtype == kF16) return launch_merge<kF16, 128>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_paged_decode_step(const DecodeArgs &a, int dtype, int head_dim, hipStream_t stream) {
    if ((int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions == 0) return hipSuccess;
    switch (dtype) {
        case kF32: return launch_dtype<kF32, true>(a, head_dim, stream);
        case kF16: return launch_dtype<kF16, true>(a, head_dim, stream);
        case kBF16: return launch_dtype<kBF16, true>(a, head_dim, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_paged_decode(const DecodeArgs &a, int dtype, int head_dim, hipStream_t stream) {
    if ((int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions == 0) return hipSuccess;
    switch (dtype) {
        case kF32: return launch_dtype<kF32>(a, head_dim, stream);
        case kF16: return launch_dtype<kF16>(a, head_dim, stream);
        case kBF16: return launch_dtype<kBF16>(a, head_dim, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
