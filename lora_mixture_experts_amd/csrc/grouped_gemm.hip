// Grouped expert projections on bf16 MFMA (gfx950, v_mfma_f32_16x16x32_bf16)
// with the LoRA expand fused in, plus SwiGLU for gate_up.
//
// One launch covers every expert: a workgroup takes one block of the base
// alignment view (rows of a single expert, gathered through sorted_b) and one
// tile of output columns. After the base K loop the LoRA expand runs as extra
// MFMA K steps on the same accumulators, once per adapter present among the
// block's rows: acc += S . B^T with S (the shrink output) split into a bf16
// high part and a bf16 low part so that the rank-r product keeps ~16 bits of
// S. This is the fusion of the LoRA addition into the expand from the AWS ML Blog post
// "Efficiently serve dozens of fine-tuned models with vLLM on Amazon SageMaker
// AI and Amazon Bedrock" (section "Kernel optimizations"), taken one step
// further: the expand writes straight into the base accumulator in registers.
//
// gate_up: the tile's 16-column fragments alternate gate / up for the same
// activation columns, so every lane holds matching gate and up values and the
// SwiGLU epilogue h = silu(gate) * up runs in registers; h is stored in bf16.
// down: the fp32 result is either stored per base slot for the weighted
// combine launch, or weighted by the routing weight and added atomically into
// the layer output (the combine folded into this epilogue).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "local_route.h"

namespace moelora {

// W row of fragment f (16 rows each) of a tile whose first output column is c0.
template <bool GATEUP>
__device__ __forceinline__ int w_row_of_frag(int f, int c0, int I) {
    if (GATEUP) return ((f & 1) ? I : 0) + c0 + 16 * (f >> 1);
    return c0 + 16 * f;
}

__device__ __forceinline__ int row_adapter(const GemmArgs& a, int slot) { return a.slot_adapter[slot]; }

// Down epilogue with the weighted combine folded in: rows 4 i .. 4 i + 3 of a
// 16 x 16 fragment (base slots slot0 + i, this lane's column col) add
// w_p * value into out[t] (p = the slot's pair, t = p / top_k); padding slots
// add nothing. fp32 atomic adds at the L2, with no return value.
__device__ __forceinline__ void combine_rows(const GemmArgs& a, int slot0, int col, const f32x4& v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = a.sorted_b[slot0 + i];
        if (p < a.P)
            unsafeAtomicAdd(a.out_acc + static_cast<size_t>(p / a.top_k) * a.N_out + col, a.topk_w[p] * v[i]);
    }
}

// S row chunk (8 values starting at j0) as hi/lo bf16 operands; zero when the
// row is not in the current adapter run or j is past r. COHERENT: S was
// written during this launch by producer waves (possibly on another XCD, whose
// L2 this one does not see), so it is read with agent-coherent loads, which
// fetch from the coherence point instead of a possibly stale local L2 line.
template <bool COHERENT = false>
__device__ __forceinline__ void load_s_hilo(const GemmArgs& a, int slot, bool in_run, int j0,
                                            u32x4& hi, u32x4& lo) {
    float v[8], rest[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = 0.f;
    if (COHERENT && in_run && j0 < a.r) {
        for (int sp = 0; sp < a.s_split; ++sp) {
            const float* src = a.S + (static_cast<size_t>(sp) * a.C_b + slot) * a.r + j0;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                v[q] += __hip_atomic_load(src + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else if (in_run && j0 < a.r) {
        // the shrink's K-range partials, added in order (a loop, not an
        // unrolled batch of loads: holding every partial at once costs the
        // direct-load kernel enough registers to halve its occupancy)
        for (int sp = 0; sp < a.s_split; ++sp) {
            const float* src = a.S + (static_cast<size_t>(sp) * a.C_b + slot) * a.r + j0;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[q] += x0[q];
                v[4 + q] += x1[q];
            }
        }
    }
    hi = pack_bf16x8(v);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t word = hi[q >> 1];
        const uint16_t bits = (q & 1) ? static_cast<uint16_t>(word >> 16) : static_cast<uint16_t>(word);
        rest[q] = v[q] - bf16_to_f32(bits);
    }
    lo = pack_bf16x8(rest);
}

// LoRA B operand chunk: rows of Bl[ad][e] (each r wide), 8 values at j0.
__device__ __forceinline__ u32x4 load_lora_b(const GemmArgs& a, int Nw, int ad, int e, int wrow,
                                             int j0) {
    if (j0 >= a.r) return u32x4{0, 0, 0, 0};
    const uint16_t* src = a.Bl + ((static_cast<size_t>(ad) * a.E + e) * Nw + wrow) * a.r + j0;
    return ld16(src);
}

// ===========================================================================
// Skinny variant: 16-row blocks (few rows per expert: the weights are
// streamed from HBM once and each byte feeds at most 16 rows).

// 16-column fragments per block of the packed weight copies (both
// projections). A wave with more fragments (the 8-fragment gate_up form)
// reads that many adjacent blocks per K chunk.
constexpr int kPackFrags = 4;
//
// One wave is one workgroup and owns a 16-row x (16 FN)-column output tile
// over the whole K range, so there is no cross-wave reduction, no LDS and no
// barrier; thousands of independent waves fill the chip in a single round.
// In each 64-wide K chunk lane (n, g) reads 32 contiguous bytes of weight row
// n (elements 16 g .. 16 g + 15), so a wave-wide pair of loads consumes whole
// 128-byte lines of 16 rows; the two 16-byte halves feed two MFMA K steps and
// the activation operand uses the same K assignment. Loads of chunk q+1 are in
// flight while chunk q is multiplied.
//
// LoRA shrink inside the launch. When a.prod_units > 0 the first prod_units
// workgroups are producer waves that compute S = X . A^T (the shrink of the
// same post's section "Kernel optimizations") while the other waves stream the
// base weights, so the LoRA A bytes share the projection's HBM stream instead
// of a launch of their own. A projection wave multiplies its base K range
// first and waits for the producers only before its expand.

// Projection waves wait for the producers by polling a counter, at most
// GemmArgs::max_polls times (the library passes kMaxProducerPolls, about a
// second). The producers have the lowest workgroup indices and never wait, so
// in practice they are done long before (the dispatcher starts a grid's
// workgroups in index order). Nothing depends on that: a wave whose wait runs
// out computes the shrink of its own rows and flags the slow path in the
// call's status word, so every wave ends and the output is valid whatever the
// dispatch order.

// 16 x 16 block of X . A^T over 64-wide K chunks [q0, q1): xrow / arow are
// this lane's X row and A row at element 16 (lane / 16); two chunks in flight.
__device__ __forceinline__ f32x4 producer_dot(const uint16_t* xrow, const uint16_t* arow, int q0, int q1) {
    const int n = q1 - q0;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 xb[2][2], wb[2][2];
    auto load = [&](int buf, int q) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            xb[buf][h] = ld16(xrow + q * 64 + 8 * h);
            wb[buf][h] = ld16(arow + q * 64 + 8 * h);
        }
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) acc = mfma16x16x32(xb[buf][h], wb[buf][h], acc);
    };
    if (n > 0) {
        load(0, q0);
        int q = q0;
        for (int i = 0; i + 1 < n; i += 2, q += 2) {
            load(1, q + 1);
            __builtin_amdgcn_sched_barrier(0);
            compute(0);
            __builtin_amdgcn_sched_barrier(0);
            load(0, min(q + 2, q1 - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (n & 1) compute(0);
    }
    return acc;
}

// One producer unit: the 16 S columns cf of LoRA-view block bl over K range ks,
// for every real row of the block. Once all of its stores have completed, the
// unit counts itself in a.done.
__device__ __forceinline__ void shrink_producer(const GemmArgs& a, int unit) {
    const int lane = threadIdx.x & 63;
    const int kc = lane >> 4, lrow = lane & 15;
    const int cf = unit % a.prod_ncf, rest = unit / a.prod_ncf;
    const int ks = rest % a.s_split, bl = rest / a.s_split;
    const int e = a.blk_e_l[bl];
    if (e < 0) return;  // block past the live LoRA view: not counted
    const int ad = a.blk_a_l[bl];
    const int K = a.K;
    // LoRA A row j of this lane's column; with r = 8 the upper 8 columns
    // re-read rows j - 8 and are never stored
    const int j = cf * 16 + lrow;
    const uint16_t* arow =
        a.Al + ((static_cast<size_t>(ad) * a.E + e) * a.r + (j < a.r ? j : j - 8)) * K + kc * 16;
    const int nqa = K / 64;
    const int q0 = ks * nqa / a.s_split, q1 = (ks + 1) * nqa / a.s_split;
    const int base = bl * a.bm_l;
    const int p_first = a.sorted_l[base];
    for (int fm = 0; fm < a.bm_l / 16; ++fm) {
        if (a.sorted_l[base + fm * 16] >= a.P) break;  // the rest of the block is padding
        // X row of block row fm*16 + lrow (padding rows re-read the first row)
        int p = a.sorted_l[base + fm * 16 + lrow];
        if (p >= a.P) p = p_first;
        const size_t xr = a.gather_token ? static_cast<size_t>(p / a.top_k)
                                         : static_cast<size_t>(a.slot_of_pair[p]);
        const uint16_t* xrow = a.X + xr * K + kc * 16;
        const f32x4 acc = producer_dot(xrow, arow, q0, q1);
        if (j < a.r) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = a.sorted_l[base + fm * 16 + 4 * kc + i];
                if (q < a.P)
                    __hip_atomic_store(&a.S_out[(static_cast<size_t>(ks) * a.C_b + a.slot_of_pair[q]) * a.r + j],
                                       acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    // The S stores above are agent-coherent (they write through to the
    // coherence point that every XCD reads from), so waiting for this wave's
    // stores to complete orders them before the count. An agent-scope release
    // fence would also write back this XCD's whole L2; with 128 producer waves
    // that measured about 10 us more per decode-shaped layer call.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(a.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The same unit on a decode-sized gate_up launch that routes the batch itself
// (GemmArgs::logits): the block's expert, adapter and rows come from the
// wave's own routing and alignment of the batch (16-row LoRA blocks, one per
// (expert, adapter) segment).
__device__ __forceinline__ void shrink_producer_local(const GemmArgs& a, int unit, float* ls) {
    const int lane = threadIdx.x & 63;
    const int kc = lane >> 4;
    const int cf = unit % a.prod_ncf, rest = unit / a.prod_ncf;
    const int ks = rest % a.s_split, bl = rest / a.s_split;
    int e = 0, ad = 0, row_p, row_slot;
    if (!local_lora_rows(a.logits, a.adapter_ids, a.T, a.E, a.top_k, a.L, bl, ls, a.local_ids, e, ad, row_p,
                         row_slot)) {
        // past the used blocks: counted all the same (the projection waves of
        // such a launch wait for every unit, so that they need not know how
        // many blocks are used)
        if (lane == 0) __hip_atomic_fetch_add(a.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int K = a.K;
    const int j = cf * 16 + (lane & 15);
    const uint16_t* arow =
        a.Al + ((static_cast<size_t>(ad) * a.E + e) * a.r + (j < a.r ? j : j - 8)) * K + kc * 16;
    const int nqa = K / 64;
    const int q0 = ks * nqa / a.s_split, q1 = (ks + 1) * nqa / a.s_split;
    // padding rows re-read the block's first row (lane 0 holds row 0)
    const int p = row_p >= 0 ? row_p : __builtin_amdgcn_readlane(row_p, 0);
    const uint16_t* xrow = a.X + static_cast<size_t>(p / a.top_k) * K + kc * 16;
    const f32x4 acc = producer_dot(xrow, arow, q0, q1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rp = __shfl(row_p, 4 * kc + i), rs = __shfl(row_slot, 4 * kc + i);
        if (j < a.r && rp >= 0)
            __hip_atomic_store(&a.S_out[(static_cast<size_t>(ks) * a.C_b + rs) * a.r + j], acc[i], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(a.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whether every live producer unit has counted itself (live LoRA blocks x
// column fragments x K ranges); one poll, wave-uniform result. S is read only
// after a true result, with agent-coherent loads (load_s_hilo<true>), so no
// agent-scope acquire is needed: that acquire would invalidate this XCD's
// whole L2 once per projection wave, thousands of times per launch.
__device__ __forceinline__ bool producers_done(const GemmArgs& a, int target) {
    const int v = __hip_atomic_load(a.done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool ok = __builtin_amdgcn_readfirstlane(v) >= target;
    // keeps the compiler from moving the S loads above the poll (no cache
    // maintenance; the hardware issues them after the poll has returned)
    asm volatile("" ::: "memory");
    return ok;
}

__device__ __forceinline__ int producer_target(const GemmArgs& a) {
    return (*a.n_l / a.bm_l) * a.prod_ncf * a.s_split;
}

// Poll until producers_done, at most a.max_polls times. A wait that runs out
// returns false and sets the call's status word: the wave then computes the
// shrink of its own rows (expand_own_shrink), so the output stays valid and
// the word only tells the host that the slow path ran.
__device__ __forceinline__ bool wait_producers(const GemmArgs& a, int target) {
    for (int polls = 0; polls < a.max_polls; ++polls) {
        if (producers_done(a, target)) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_or(a.status, kStatusShrinkFallback, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
}

// The expand of a projection wave that computes the shrink of its own 16 rows
// (its wait for the shrink waves of the launch ran out). For each adapter run
// among the rows and each 32-wide chunk c of the rank, S^T = A . X^T by MFMA
// over the whole K, the LoRA A rows 32 c .. 32 c + 15 and 32 c + 16 .. 32 c + 31
// against the wave's 16 X rows (xrow0: this lane's X row at element 16 g).
// Lane (row, g) then holds S[row][32 c + 4 g + i] and S[row][32 c + 16 + 4 g + i],
// i < 4: the expand of chunk c takes its K slots in that order and reads the
// LoRA B operand as two 4-element halves to match. S is split into bf16 hi
// and lo parts as in load_s_hilo.
template <bool GATEUP, int FN>
__device__ __forceinline__ void expand_own_shrink(const GemmArgs& a, int e, int c0, int I, int Nw, int my_a,
                                                  const uint16_t* xrow0, f32x4 (&dst)[FN]) {
    const int lane = threadIdx.x & 63, g = lane >> 4, lrow = lane & 15;
    const int K = a.K, r = a.r;
    bool pending = my_a >= 0;
    while (true) {
        const uint64_t m = ballot64(pending);
        if (m == 0) break;
        const int acur = __shfl(my_a, __ffsll(static_cast<long long>(m)) - 1);
        const bool in_run = pending && my_a == acur;
        pending = pending && !in_run;
        const uint16_t* ablk = a.Al + static_cast<size_t>(acur * a.E + e) * r * K;
        // one 32-wide chunk c of the rank at a time: fragments 2 c and 2 c + 1
        for (int c = 0; 32 * c < r; ++c) {
            f32x4 st0 = f32x4{0.f, 0.f, 0.f, 0.f}, st1 = st0;
            // A rows 32 c + lrow and 32 c + 16 + lrow; rows past r re-read
            // row lrow % r and their outputs are never used
            const int ja = 32 * c + lrow, jb = ja + 16;
            const uint16_t* arow0 = ablk + static_cast<size_t>(ja < r ? ja : lrow % r) * K + 16 * g;
            const uint16_t* arow1 = ablk + static_cast<size_t>(jb < r ? jb : lrow % r) * K + 16 * g;
            for (int q = 0; q < K / 64; ++q) {
                const u32x4 x0 = ld16(xrow0 + q * 64), x1 = ld16(xrow0 + q * 64 + 8);
                const u32x4 a0 = ld16(arow0 + q * 64), a1 = ld16(arow0 + q * 64 + 8);
                const u32x4 b0 = ld16(arow1 + q * 64), b1 = ld16(arow1 + q * 64 + 8);
                st0 = mfma16x16x32(a0, x0, st0);
                st0 = mfma16x16x32(a1, x1, st0);
                st1 = mfma16x16x32(b0, x0, st1);
                st1 = mfma16x16x32(b1, x1, st1);
            }
            const int j1 = 32 * c + 4 * g, j2 = j1 + 16;
            float v[8], rest[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = (in_run && j1 + i < r) ? st0[i] : 0.f;
                v[4 + i] = (in_run && j2 + i < r) ? st1[i] : 0.f;
            }
            const u32x4 hi = pack_bf16x8(v);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t word = hi[q >> 1];
                const uint16_t bits = (q & 1) ? static_cast<uint16_t>(word >> 16) : static_cast<uint16_t>(word);
                rest[q] = v[q] - bf16_to_f32(bits);
            }
            const u32x4 lo = pack_bf16x8(rest);
#pragma unroll
            for (int f = 0; f < FN; ++f) {
                const uint16_t* brow =
                    a.Bl + (static_cast<size_t>(acur * a.E + e) * Nw + w_row_of_frag<GATEUP>(f, c0, I) + lrow) * r;
                const uint2 h1 = j1 < r ? *reinterpret_cast<const uint2*>(brow + j1) : make_uint2(0, 0);
                const uint2 h2 = j2 < r ? *reinterpret_cast<const uint2*>(brow + j2) : make_uint2(0, 0);
                const u32x4 bb = u32x4{h1.x, h1.y, h2.x, h2.y};
                dst[f] = mfma16x16x32(hi, bb, dst[f]);
                dst[f] = mfma16x16x32(lo, bb, dst[f]);
            }
        }
    }
}

template <bool GATEUP, int FN, int NS, int KSW, bool PAIR>
__global__ __launch_bounds__(64 * KSW) void k_gemm_skinny(GemmArgs a) {
    const int w = KSW > 1 ? wave_id() : 0;
    // 1-D grid: [the routing workgroup,] producer workgroups (one producer
    // unit per wave), then (column tile, block, K range) with the tile fastest.
    // Local routing (one-wave workgroups only): every wave routes the batch
    // itself, with the logits staged in LDS.
    __shared__ float local_ls[GATEUP && KSW == 1 ? kLocalMaxT * kLocalMaxE : 1];
    int wg = blockIdx.x;
    const bool local = GATEUP && KSW == 1 && a.local;
    if (local) {
        if (wg == 0) {
            // routing and alignment for the launches after this one
            local_publish(a.logits, a.adapter_ids, a.T, a.E, a.top_k, a.L, local_ls, a.local_ids, a.pub);
            return;
        }
        --wg;
    }
    const int prod_wgs = (a.prod_units + KSW - 1) / KSW;
    if (wg < prod_wgs) {
        const int unit = wg * KSW + w;
        if (unit < a.prod_units) {
            if (local) shrink_producer_local(a, unit, local_ls);
            else shrink_producer(a, unit);
        }
        return;
    }
    wg -= prod_wgs;
    constexpr int kCols = GATEUP ? FN * 8 : FN * 16;  // output columns per wave
    const int n_tiles = a.N_out / kCols;
    const int tile = wg % n_tiles, bidx = (wg / n_tiles) % a.n_blocks;
    const int z = wg / n_tiles / a.n_blocks;  // K range (down only)
    // with local routing, block index = expert (its slots are found below)
    const int e = local ? bidx : a.blk_e_b[bidx];
    if (e < 0) return;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, lrow = lane & 15;
    const int I = GATEUP ? a.N_out : 0;
    const int Nw = GATEUP ? 2 * a.N_out : a.N_out;
    const int c0 = tile * kCols;
    const int K = a.K;
    const int Kp = K / a.ksplit;  // this workgroup's K range starts at z Kp
    // this wave's part of it: 64-wide chunks [q0, q1) (the launcher gives
    // every wave at least one)
    const int q0 = w * (Kp / 64) / KSW, q1 = (w + 1) * (Kp / 64) / KSW;
    const int kbeg = z * Kp + q0 * 64;

    // The block's first slot and this lane's activation row. Padding rows
    // (sentinel P) re-read the block's first row, which is always a real row:
    // the duplicate addresses merge into the same memory request, MFMA output
    // rows depend only on their own A row, and padding rows are never
    // consumed, so no masking is needed and every load is issued
    // unconditionally (exact wait counts). With local routing both are known
    // only after the routing below.
    int b16 = bidx * 16, row_ad = 0, local_target = 0;
    const uint16_t* xrow = nullptr;
    if (!local) {
        if (GATEUP) {
            int p = a.sorted_b[b16 + lrow];
            if (p >= a.P) p = a.sorted_b[b16];
            xrow = a.X + static_cast<size_t>(p / a.top_k) * K + kbeg + g * 16;
        } else {
            xrow = a.X + static_cast<size_t>(b16 + lrow) * K + kbeg + g * 16;
        }
    }
    // Weight operand: the 64 rows of the tile at the matrix pitch, or the
    // packed copy, where a kPackFrags-fragment column tile's 64-wide K chunk q
    // is one 8 KiB block [fragment][half][lane][8] (lane = 16 g + lrow) and
    // the blocks of consecutive chunks follow each other; a wave of FN
    // fragments reads FN / kPackFrags such tiles. wq, wh: elements per K
    // chunk and per 16-byte half.
    static_assert(FN % kPackFrags == 0, "whole packed tiles per wave");
    const uint16_t* wrow[FN];
    int wq, wh;
    if (a.Wp) {
        constexpr int kTiles = FN / kPackFrags;
        const uint16_t* wt = a.Wp +
                             (static_cast<size_t>((e * n_tiles + tile) * kTiles) * (K / 64) + kbeg / 64) *
                                 (kPackFrags * 1024) +
                             lane * 8;
#pragma unroll
        for (int f = 0; f < FN; ++f)
            wrow[f] = wt + static_cast<size_t>(f / kPackFrags) * (K / 64) * (kPackFrags * 1024) +
                      (f % kPackFrags) * 1024;
        wq = kPackFrags * 1024;
        wh = 512;
    } else {
#pragma unroll
        for (int f = 0; f < FN; ++f)
            wrow[f] = a.W + (static_cast<size_t>(e) * Nw + w_row_of_frag<GATEUP>(f, c0, I) + lrow) * K +
                      kbeg + g * 16;
        wq = 64;
        wh = 8;
    }

    f32x4 acc[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 xb[NS][2], wb[NS][FN][2];
    auto loadx = [&](int buf, int q) {
#pragma unroll
        for (int h = 0; h < 2; ++h) xb[buf][h] = ld16(xrow + q * 64 + 8 * h);
    };
    // Every weight byte is read by exactly one wave of the launch: the loads
    // carry the non-temporal hint (decode-shaped layer 291 -> 261 us, its
    // gate_up projection 187 -> 165 us). The activation rows, which every
    // tile of the expert reads again, keep the default policy; so do the
    // LoRA operands (the hint measured 1-2 us slower on them).
    auto loadw = [&](int buf, int q) {
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int h = 0; h < 2; ++h) wb[buf][f][h] = ld16_nt(wrow[f] + static_cast<size_t>(q) * wq + h * wh);
    };
    auto load = [&](int buf, int q) {
        loadx(buf, q);
        loadw(buf, q);
    };
    const int nq = q1 - q0;
    // With local routing the wave's 16 rows are the batch's tokens (row r =
    // token r; rows past T re-read token 0): the loads start at once, and the
    // routing, worked out while the first chunks stream, only decides which
    // rows are stored and where (row_slot, -1 for a token that did not choose
    // this expert).
    int row_slot = -1;
    if (local) {
        xrow = a.X + static_cast<size_t>(min(lrow, a.T - 1)) * K + kbeg + g * 16;
#pragma unroll
        for (int st = 0; st + 1 < NS; ++st) load(st, min(st, nq - 1));
        bool in_row;
        int s;
        const bool any = local_token_rows(a.logits, a.adapter_ids, a.T, a.E, a.top_k, a.L, e, local_ls,
                                          a.local_ids, in_row, s, row_ad);
        local_target = a.prod_units;  // every unit counts itself in this mode
        if (!any) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no pair chose this expert
            return;
        }
        if (in_row) row_slot = s;
        else row_ad = a.L;
    }
    const int slot = local ? max(row_slot, 0) : b16 + lrow;
    auto compute = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int f = 0; f < FN; ++f) acc[f] = mfma16x16x32(xb[buf][h], wb[buf][f][h], acc[f]);
    };

    if (!local) {
#pragma unroll
        for (int st = 0; st + 1 < NS; ++st) load(st, min(st, nq - 1));
    }
    __builtin_amdgcn_sched_barrier(0);

    // LoRA expand: acc += S . B^T for every adapter present among the 16 rows
    // (added once: by the first K range, in its wave 0). With S from a
    // separate launch it runs first, so its latency overlaps the first weight
    // loads; with the producers in this launch it runs after the base K loop.
    const bool lora = a.L > 0 && z == 0 && w == 0;
    const int my_a = !lora ? -1 : local ? (row_ad < a.L ? row_ad : -1) : row_adapter(a, slot);
    // With the producers in this launch the expand runs part-way through or
    // after the base K loop, depending on when the producers finish; it then
    // accumulates into its own registers, added to the base result after the
    // loop, so the result does not depend on that timing.
    const bool late = lora && a.prod_units > 0;
    f32x4 acc_l[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) acc_l[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    // With PAIR, the rows' S chunk is read once per 32 of r (rows without an
    // adapter read zeros) and each adapter run masks it to its own rows; runs
    // are taken two at a time, so that the LoRA B loads of both are in flight
    // together (8 adapters among 16 rows would otherwise be 8 dependent
    // load-then-multiply rounds). It holds more registers (two waves per
    // SIMD instead of three), so the launcher picks it only for grids that
    // do not fill three waves per SIMD anyway.
    auto expand = [&](auto coherent, f32x4 (&dst)[FN]) {
        if constexpr (PAIR) {
            for (int kk = 0; kk < a.r; kk += 32) {
                const int j0 = kk + g * 8;
                u32x4 hi, lo;
                load_s_hilo<decltype(coherent)::value>(a, slot, my_a >= 0, j0, hi, lo);
                bool pending = my_a >= 0;
                while (true) {
                    uint64_t m = ballot64(pending);
                    if (m == 0) break;
                    const int a0 = __shfl(my_a, __ffsll(static_cast<long long>(m)) - 1);
                    const bool in0 = pending && my_a == a0;
                    pending = pending && !in0;
                    m = ballot64(pending);
                    const int a1 = m ? __shfl(my_a, __ffsll(static_cast<long long>(m)) - 1) : -1;
                    const bool in1 = m != 0 && pending && my_a == a1;
                    pending = pending && !in1;
                    u32x4 b0[FN], b1[FN];
#pragma unroll
                    for (int f = 0; f < FN; ++f)
                        b0[f] = load_lora_b(a, Nw, a0, e, w_row_of_frag<GATEUP>(f, c0, I) + lrow, j0);
                    if (a1 >= 0) {
#pragma unroll
                        for (int f = 0; f < FN; ++f)
                            b1[f] = load_lora_b(a, Nw, a1, e, w_row_of_frag<GATEUP>(f, c0, I) + lrow, j0);
                    }
                    const u32x4 z{0, 0, 0, 0};
                    const u32x4 h0 = in0 ? hi : z, l0 = in0 ? lo : z;
#pragma unroll
                    for (int f = 0; f < FN; ++f) {
                        dst[f] = mfma16x16x32(h0, b0[f], dst[f]);
                        dst[f] = mfma16x16x32(l0, b0[f], dst[f]);
                    }
                    if (a1 >= 0) {
                        const u32x4 h1 = in1 ? hi : z, l1 = in1 ? lo : z;
#pragma unroll
                        for (int f = 0; f < FN; ++f) {
                            dst[f] = mfma16x16x32(h1, b1[f], dst[f]);
                            dst[f] = mfma16x16x32(l1, b1[f], dst[f]);
                        }
                    }
                }
            }
        } else {
            bool pending = my_a >= 0;
            while (true) {
                const uint64_t m = ballot64(pending);
                if (m == 0) break;
                const int leader = __ffsll(static_cast<long long>(m)) - 1;
                const int acur = __shfl(my_a, leader);
                const bool in_run = pending && my_a == acur;
                pending = pending && !in_run;
                for (int kk = 0; kk < a.r; kk += 32) {
                    const int j0 = kk + g * 8;
                    u32x4 hi, lo, bb[FN];
#pragma unroll
                    for (int f = 0; f < FN; ++f)
                        bb[f] = load_lora_b(a, Nw, acur, e, w_row_of_frag<GATEUP>(f, c0, I) + lrow, j0);
                    load_s_hilo<decltype(coherent)::value>(a, slot, in_run, j0, hi, lo);
#pragma unroll
                    for (int f = 0; f < FN; ++f) {
                        dst[f] = mfma16x16x32(hi, bb[f], dst[f]);
                        dst[f] = mfma16x16x32(lo, bb[f], dst[f]);
                    }
                }
            }
        }
    };
    if (lora && !late) expand(std::false_type{}, acc);

    // With the producers in this launch, the expand runs a third of the way
    // through the K loop if they are done by then (one poll), so that its
    // load latency is hidden while the other waves keep HBM busy; otherwise
    // after the loop. The waves that finish last, which set the launch's
    // length, then expand mid-stream. Measured on the decode-shaped layer
    // with the non-temporal weight loads (µs per call): poll after the loop
    // in the down projection and half-way in gate_up 262.5, half-way in both
    // 260.8, a third 258.6, a quarter 259.4, a sixth 261.8 (dense layer
    // 143.5 -> 150.1 there), three quarters in the down projection 271.
    const int target = !late ? 0 : local ? local_target : producer_target(a);
    const int q_mid = nq / 3 / NS * NS;
    bool expanded = !late;

    // NS-stage register pipeline: chunk c sits in buffer c % NS and is
    // requested NS - 1 chunks ahead of its use. The main loop has one back
    // edge and no early exit, so the requests stay in flight across
    // iterations; scheduling barriers stop the compiler from sinking loads
    // next to their use. A request past the end re-reads the last chunk (in
    // bounds) and is discarded.
    int q = 0;
    for (; q + NS <= nq; q += NS) {
        if (!expanded && q == q_mid && a.max_polls > 0) {
            if (producers_done(a, target)) {
                expand(std::true_type{}, acc_l);
                expanded = true;
            }
        }
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            load((st + NS - 1) % NS, min(q + st + NS - 1, nq - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(st);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the last nq - q (< NS) chunks are already in buffers 0 .. nq - q - 1
#pragma unroll
    for (int st = 0; st + 1 < NS; ++st)
        if (st < nq - q) compute(st);

    if (!expanded) {
        if (wait_producers(a, target))
            expand(std::true_type{}, acc_l);
        else
            expand_own_shrink<GATEUP, FN>(a, e, c0, I, Nw, my_a, xrow, acc_l);  // xrow: K offset 0 here
    }
    if (late) {
#pragma unroll
        for (int f = 0; f < FN; ++f) acc[f] += acc_l[f];
    }
    if constexpr (KSW > 1) {
        __shared__ f32x4 red[KSW - 1][FN][64];
        if (w > 0) {
#pragma unroll
            for (int f = 0; f < FN; ++f) red[w - 1][f][lane] = acc[f];
        }
        __syncthreads();
        if (w > 0) return;
#pragma unroll
        for (int v = 0; v < KSW - 1; ++v)
#pragma unroll
            for (int f = 0; f < FN; ++f) acc[f] += red[v][f][lane];
    }

    const int orow0 = b16 + 4 * g;
    if (GATEUP) {
        // output rows 4 g .. 4 g + 3 of this lane: their slots (local routing:
        // the slots of those tokens' pairs, -1 for tokens that did not choose
        // this expert; their rows are not stored)
        int orow[4];
        if (local) {
#pragma unroll
            for (int i = 0; i < 4; ++i) orow[i] = __shfl(row_slot, 4 * g + i);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) orow[i] = orow0 + i;
        }
#pragma unroll
        for (int u = 0; u < FN / 2; ++u) {
            const int col = c0 + 16 * u + lrow;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (orow[i] >= 0)
                    a.h_out[static_cast<size_t>(orow[i]) * a.N_out + col] =
                        f32_to_bf16_rne(silu(acc[2 * u][i]) * acc[2 * u + 1][i]);
        }
    } else if (a.out_acc) {
#pragma unroll
        for (int f = 0; f < FN; ++f) combine_rows(a, orow0, c0 + 16 * f + lrow, acc[f]);
    } else {
        float* dpart = a.d_out + static_cast<size_t>(z) * a.C_b * a.N_out;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            const int col = c0 + 16 * f + lrow;
#pragma unroll
            for (int i = 0; i < 4; ++i) dpart[static_cast<size_t>(orow0 + i) * a.N_out + col] = acc[f][i];
        }
    }
}

// ===========================================================================
// Tiled variant: BM x BNT tile (BNT = GEMM columns), BK = 64, 2 x 2 waves,
// LDS double buffer with an XOR swizzle of the 16-byte chunks, and global
// loads issued two K steps ahead through two register sets, so a load has two
// steps of MFMA work to arrive.
//
// Tile order (the MI355X form of CTA swizzling, AWS ML Blog post "Efficiently
// serve dozens of fine-tuned models with vLLM on Amazon SageMaker AI and
// Amazon Bedrock", Korean summary, section "Kernel-level optimization"): the
// 1-D grid is dealt round-robin to the 8 XCDs, each with its own L2, so
// workgroup i is mapped to logical tile (i % 8) * chunk + i / 8: every XCD
// walks its own contiguous range of logical tiles. Logically, N tiles are
// taken in groups of kGroupN; inside a group, M blocks (consecutive blocks
// belong to one expert) run major and N tiles minor. The workgroups resident
// on one XCD then share the same expert's weight tiles and the same
// activation rows, and reread them from L2 instead of HBM.
template <int BM, int BNT, int WM, int WN>
struct TileCfg {
    static constexpr int NT = 64 * WM * WN;      // threads
    static constexpr int FM = BM / (16 * WM);    // 16-row fragments per wave
    static constexpr int FN = BNT / (16 * WN);   // 16-col fragments per wave
    static constexpr int A_LD = BM * 8 / NT;     // 16-byte chunks per thread per stage
    static constexpr int B_LD = BNT * 8 / NT;
    static constexpr int ROWS_PER_PASS = NT / 8;
    static constexpr int A_ELEMS = BM * 64;
    static constexpr int B_ELEMS = BNT * 64;
    static_assert(FM >= 1 && FN >= 1 && A_LD >= 1 && B_LD >= 1, "tile too small");
};
constexpr int kGroupN = 8;
constexpr int kXcds = 8;
constexpr int kCus = 256;  // compute units of the MI355X

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

// output columns of a tile and the number of tiles (the last may be partial)
template <int BNT, bool GATEUP>
__host__ __device__ constexpr int tile_cols() { return GATEUP ? BNT / 2 : BNT; }


// Tile epilogue shared by the LDS kernels: the LoRA expand for every adapter
// present among the wave's rows (extra MFMA K steps on the accumulators), then
// SwiGLU + bf16 store (gate_up) or the fp32 store (down). wrow_of maps a tile
// row (GEMM column) to its weight row.
template <int FM, int FN, bool GATEUP, typename WRowOf>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& a, f32x4 (&acc)[FM][FN], bool wlive,
                                              int wrow_base, int wn, int c0, int e, int kc,
                                              int lrow, WRowOf wrow_of, int z = 0,
                                              bool expand = true) {
    if (!wlive) return;
    const int Nw = GATEUP ? 2 * a.N_out : a.N_out;
    // the LoRA term is added once, by the first K range, unless the pipeline
    // already added it
    if (a.L > 0 && z == 0 && expand) {
        int my_a[FM];
        bool pending[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            my_a[i] = row_adapter(a, wrow_base + i * 16 + lrow);
            pending[i] = my_a[i] >= 0;
        }
        while (true) {
            int cand = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                if (pending[i] && my_a[i] < cand) cand = my_a[i];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) cand = min(cand, __shfl_xor(cand, off));
            if (cand == 0x7fffffff) break;
            for (int kk = 0; kk < a.r; kk += 32) {
                const int j0 = kk + kc * 8;
                u32x4 bb[FN];
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bb[j] = load_lora_b(a, Nw, cand, e, wrow_of((wn * FN + j) * 16 + lrow), j0);
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const bool in_run = pending[i] && my_a[i] == cand;
                    if (!__any(in_run)) continue;
                    u32x4 hi, lo;
                    load_s_hilo(a, wrow_base + i * 16 + lrow, in_run, j0, hi, lo);
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        acc[i][j] = mfma16x16x32(hi, bb[j], acc[i][j]);
                        acc[i][j] = mfma16x16x32(lo, bb[j], acc[i][j]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
                if (pending[i] && my_a[i] == cand) pending[i] = false;
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int orow0 = wrow_base + i * 16 + 4 * kc;
        if (GATEUP) {
#pragma unroll
            for (int j = 0; j < FN; j += 2) {
                const int col = c0 + 16 * ((wn * FN + j) >> 1) + lrow;
                if (col >= a.N_out) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a.h_out[static_cast<size_t>(orow0 + q) * a.N_out + col] =
                        f32_to_bf16_rne(silu(acc[i][j][q]) * acc[i][j + 1][q]);
            }
        } else if (a.out_acc) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = c0 + 16 * (wn * FN + j) + lrow;
                if (col < a.N_out) combine_rows(a, orow0, col, acc[i][j]);
            }
        } else {
            float* dpart = a.d_out + static_cast<size_t>(z) * a.C_b * a.N_out;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = c0 + 16 * (wn * FN + j) + lrow;
                if (col >= a.N_out) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dpart[static_cast<size_t>(orow0 + q) * a.N_out + col] = acc[i][j][q];
            }
        }
    }
}

// Tile order of the LDS-tiled and direct-load kernels. The live tiles (blocks
// 0 .. n_b / BM - 1 of the base view: the alignment packs every non-empty
// block first, so no workgroup is spent on an empty block) are numbered
// without holes: N tiles in groups of kGroupN, and inside a group block-major,
// so consecutive numbers are the group's N tiles of one block, then of the
// next block (which is usually the same expert). The hardware deals the 1-D
// grid's workgroups round-robin to the 8 XCDs, each with its own L2, so
// workgroup i is the (i / 8)-th of XCD i mod 8. With S workgroups resident per
// XCD (32 CUs x workgroups per CU), the XCD's k-th workgroup takes tile
// (8 (k / S) + x) S + k mod S: each XCD works through whole patches of S
// consecutive tiles (about S / kGroupN blocks x kGroupN N tiles: one expert's
// weight tiles and the same activation rows), patch x, x + 8, ..., so the
// workgroups resident on an XCD at a time share their operand slabs in its L2
// and every XCD gets an equal share of the tiles.
struct TileOrder {
    int n_tiles, n_live, per_group;
    __device__ TileOrder(const GemmArgs& a, int cols, int bm) {
        n_tiles = (a.N_out + cols - 1) / cols;
        // uniform: keeps the tile's block, expert and addresses scalar
        n_live = __builtin_amdgcn_readfirstlane(*a.n_b_live) / bm;
        per_group = n_live * kGroupN;
    }
    __device__ int total() const { return n_live * n_tiles; }
    // tile number of workgroup i of the 1-D grid (>= total(): nothing to do).
    // slots: workgroups resident per XCD. Every full round hands each XCD a
    // patch of `slots` consecutive tiles; the last, partial round hands each
    // XCD ceil(rest / 8) of the remaining tiles instead, so that no XCD sits
    // idle while others work through whole patches. The grid holds whole
    // rounds of 8 x slots workgroups (at least the tile capacity), so the map
    // covers every tile below total().
    __device__ int of_workgroup(int i, int slots) const {
        const int tot = total();
        const int k = i / kXcds, x = i % kXcds;
        const int q = k / slots, m = k % slots;
        const int full = tot / (kXcds * slots);  // full rounds
        if (q < full) return (q * kXcds + x) * slots + m;
        if (q > full) return tot;
        const int base = full * kXcds * slots;
        const int S = (tot - base + kXcds - 1) / kXcds;
        return m < S ? base + x * S + m : tot;
    }
    // tile number -> (block, N tile)
    __device__ void at(int t, int& b, int& tile) const {
        const int g = t / per_group, rem = t - g * per_group;
        const int w = min(kGroupN, n_tiles - g * kGroupN);  // N tiles in this group
        b = rem / w;
        tile = g * kGroupN + (rem - b * w);
    }
};

template <int BM, int BNT, int WM, int WN, bool GATEUP>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_tiled(GemmArgs a) {
    using C = TileCfg<BM, BNT, WM, WN>;
    constexpr int FM = C::FM, FN = C::FN;
    static_assert(!GATEUP || FN % 2 == 0, "gate/up fragments come in pairs");
    constexpr int kCols = tile_cols<BNT, GATEUP>();
    // the XCD's k-th workgroup of this K range takes the k-th tile of that
    // XCD's sequence (see TileOrder)
    const TileOrder order(a, kCols, BM);
    const int t = order.of_workgroup(blockIdx.x, a.xcd_slots);
    if (t >= order.total()) return;
    int b, tile;
    order.at(t, b, tile);
    const int e = a.blk_e_b[b];
    if (e < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int wm = wave / WN, wn = wave % WN;
    const int kc = lane >> 4, lrow = lane & 15;
    const int I = GATEUP ? a.N_out : 0;
    const int Nw = GATEUP ? 2 * a.N_out : a.N_out;
    const int c0 = tile * kCols;
    const int K = a.K;
    const int z = blockIdx.y, Kp = K / a.ksplit, kbeg = z * Kp;  // K range (down only)
    const int row0 = b * BM;
    // weight row of tile row r (columns past N_out, in a partial last tile,
    // re-read the last valid row; their results are not stored)
    auto wrow_of = [&](int r) {
        const int f = r >> 4;
        int col = c0 + 16 * (GATEUP ? (f >> 1) : f) + (r & 15);
        col = min(col, a.N_out - 1);
        return (GATEUP && (f & 1)) ? I + col : col;
    };

    __shared__ __attribute__((aligned(16))) uint16_t As[2][C::A_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][C::B_ELEMS];

    // global -> LDS assignment: thread owns rows tid/8 + (NT/8)*i, chunk tid%8
    const int ld_row = tid >> 3, ld_chunk = tid & 7;
    // padding rows re-read the block's first (real) row; their outputs are
    // never consumed
    const uint16_t* asrc[C::A_LD];
    const int p_first = a.sorted_b[row0];
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
        const int r = ld_row + C::ROWS_PER_PASS * i;
        const int slot = row0 + r;
        if (GATEUP) {
            const int p = a.sorted_b[slot];
            asrc[i] = a.X + static_cast<size_t>((p < a.P ? p : p_first) / a.top_k) * K + kbeg + ld_chunk * 8;
        } else {
            asrc[i] = a.X + static_cast<size_t>(slot) * K + kbeg + ld_chunk * 8;
        }
    }
    const uint16_t* bsrc[C::B_LD];
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
        const int r = ld_row + C::ROWS_PER_PASS * i;
        bsrc[i] = a.W + (static_cast<size_t>(e) * Nw + wrow_of(r)) * K + kbeg + ld_chunk * 8;
    }

    // A wave whose first row is padding holds no real row (rows are real
    // first, then padding): it skips its MFMAs and stores. The test is uniform
    // per wave and sits outside the K loop's inner loops, which stay
    // branch-free so that LDS reads overlap the MFMAs.
    const int wrow_base = row0 + wm * (BM / WM);
    const bool wlive = a.sorted_b[wrow_base] < a.P;
    u32x4 ra[2][C::A_LD], rb[2][C::B_LD];
    const int nk = Kp / 64;

    // LoRA expand as extra stages of the same pipeline, for every adapter run
    // of the tile (rows are ordered by adapter, so each adapter's rows form one
    // run; no cap on the number of runs): per run, s_hl_stride / 64 stages
    // whose A rows are the run's rows of S as bf16 [hi | lo | zeros] (rows of
    // other adapters load zeros) and whose B rows are the run's LoRA B rows,
    // each read twice (column j of both the hi and the lo part). The loads of
    // a run are then in flight while earlier stages multiply, instead of each
    // run waiting for its own loads in the epilogue. Only the first K range
    // adds the LoRA term.
    static_assert(BM <= 64, "one lane per tile row");
    int nruns = 0;
    int row_ad[C::A_LD];
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) row_ad[i] = -1;
    const bool pipe_expand = a.L > 0 && a.S_hl != nullptr && z == 0;
    // lane l: the adapter of tile row l; starts: the first row of each run
    // (wave-uniform)
    const int adr = pipe_expand && lane < BM ? a.slot_adapter[row0 + lane] : -1;
    uint64_t starts = 0;
    if (pipe_expand) {
        int prev = __shfl(adr, (lane + 63) & 63);
        if (lane == 0) prev = -2;
        starts = ballot64(adr >= 0 && adr != prev);
        nruns = __popcll(starts);
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i) row_ad[i] = __shfl(adr, ld_row + C::ROWS_PER_PASS * i);
    }
    // adapter of run q: the lane of the q-th set bit of starts
    auto run_adapter = [&](int q) {
        uint64_t m = starts;
        for (int i = 0; i < q; ++i) m &= m - 1;
        return __builtin_amdgcn_readlane(adr, __ffsll(static_cast<long long>(m)) - 1);
    };
    const int spr = pipe_expand ? a.s_hl_stride / 64 : 0;  // stages per run
    const int nk_all = nk + nruns * spr;
    auto gload = [&](int set, int kt) {
        if (kt < nk) {
            const int k0 = kt * 64;
#pragma unroll
            for (int i = 0; i < C::A_LD; ++i) ra[set][i] = ld16(asrc[i] + k0);
#pragma unroll
            for (int i = 0; i < C::B_LD; ++i) rb[set][i] = ld16(bsrc[i] + k0);
            return;
        }
        const int t = kt - nk, q = t / spr, sub = t - q * spr;
        const int ad = run_adapter(q);
        const int col = sub * 64 + ld_chunk * 8;
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i)
            ra[set][i] = row_ad[i] == ad
                             ? ld16(a.S_hl + static_cast<size_t>(row0 + ld_row + C::ROWS_PER_PASS * i) * a.s_hl_stride + col)
                             : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i)
            rb[set][i] = ld16(a.Bl + (static_cast<size_t>(ad * a.E + e) * Nw + wrow_of(ld_row + C::ROWS_PER_PASS * i)) * a.r +
                              (col & (a.r - 1)));
    };
    auto lstore = [&](int buf, int set) {
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i)
            *reinterpret_cast<u32x4*>(&As[buf][swz(ld_row + C::ROWS_PER_PASS * i, ld_chunk)]) = ra[set][i];
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i)
            *reinterpret_cast<u32x4*>(&Bs[buf][swz(ld_row + C::ROWS_PER_PASS * i, ld_chunk)]) = rb[set][i];
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf) {
        if (!wlive) return;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int chunk = kk * 4 + kc;
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = *reinterpret_cast<const u32x4*>(
                    &Bs[buf][swz(wn * (BNT / WN) + j * 16 + lrow, chunk)]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const u32x4*>(
                    &As[buf][swz(wm * (BM / WM) + i * 16 + lrow, chunk)]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
        }
    };

    // Stage s sits in LDS buffer s & 1. Loads past the last stage re-read it
    // (in bounds) so that every load and LDS store is unconditional and the
    // compiler keeps exact wait counts across the unrolled loop.
    gload(0, 0);
    lstore(0, 0);
    gload(1, min(1, nk_all - 1));
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk_all; kt += 2) {
        gload(0, min(kt + 2, nk_all - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(0);
        __builtin_amdgcn_sched_barrier(0);
        lstore(1, 1);
        __syncthreads();
        gload(1, min(kt + 3, nk_all - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        __builtin_amdgcn_sched_barrier(0);
        lstore(0, 0);
        __syncthreads();
    }
    if (nk_all & 1) compute(0);

    tile_epilogue<FM, FN, GATEUP>(a, acc, wlive, wrow_base, wn, c0, e, kc, lrow, wrow_of, z, !pipe_expand);
}

// ===========================================================================
// DMA variant for large blocks: the same tile order, fragment layout and
// epilogue as the tiled variant, but the global -> LDS copy uses gfx950's
// direct loads (global_load_lds_dwordx4): each wave-wide load deposits 64 x
// 16 bytes into a contiguous 1 KiB of LDS in lane order, so no registers hold
// staged tiles and no LDS store instructions are issued. A lane picks the
// global chunk that its LDS slot must hold under the XOR swizzle. NS LDS
// stages form a ring: stage k+NS-1 is requested while stage k is multiplied.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt with vmcnt = N (gfx9 encoding: bits 3:0 and 15:14); expcnt and
    // lgkmcnt at their maximum, i.e. not waited on
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// where the wave's fragments sit in a stage's LDS tiles
struct DmaCtx {
    int arow0, brow0, kc, lrow;
    bool wlive;
};

// One direct global -> LDS load of 16 bytes per lane: lane l's data lands at
// LDS byte offset lds + 16 l. Written as inline assembly so that the compiler
// does not see an LDS write it cannot disambiguate from the reads of the
// other pipeline stages (it would otherwise drain every load in flight before
// each LDS read); the kernel orders these loads itself with explicit vmcnt
// waits and barriers.
__device__ __forceinline__ void dma16(const void* g, const uint16_t* lds) {
    const uint32_t l = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(lds)));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(l), "v"(g) : "m0", "memory");
}

// The same with the non-temporal cache policy (data the launch reads once).
__device__ __forceinline__ void dma16_nt(const void* g, const uint16_t* lds) {
    const uint32_t l = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(lds)));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(l), "v"(g) : "m0", "memory");
}

// workgroup barrier without the memory fence of __syncthreads (that fence
// would wait for the stages requested ahead); the memory clobber keeps the
// compiler from moving LDS accesses across it
__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One stage's activation (A) and weight (B) tiles. w_once: each weight tile
// is read by about one block of rows (GemmArgs::w_stream), so its loads
// carry the non-temporal policy; the activation rows, which every column
// tile reads again, keep the default one.
template <int A_PW, int B_PW>
__device__ __forceinline__ void dma_issue(const uint16_t* const* asrc, const uint16_t* const* bsrc,
                                          uint16_t* ab, uint16_t* bb, int wave, int k0, bool w_once) {
#pragma unroll
    for (int i = 0; i < A_PW; ++i) dma16(asrc[i] + k0, ab + (wave * A_PW + i) * 512);
    if (w_once) {
#pragma unroll
        for (int i = 0; i < B_PW; ++i) dma16_nt(bsrc[i] + k0, bb + (wave * B_PW + i) * 512);
    } else {
#pragma unroll
        for (int i = 0; i < B_PW; ++i) dma16(bsrc[i] + k0, bb + (wave * B_PW + i) * 512);
    }
}

// Multiply the stage held in (ca, cb) into the accumulators: per 32-wide K
// half, the wave's B and A fragments from LDS, then its FM x FN MFMAs.
template <int FM, int FN>
__device__ __forceinline__ void dma_step(const DmaCtx& c, f32x4 (&acc)[FM][FN],
                                         const uint16_t* __restrict__ ca,
                                         const uint16_t* __restrict__ cb) {
    __builtin_amdgcn_sched_barrier(0);
    if (!c.wlive) return;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int ch = kk * 4 + c.kc;
        u32x4 fa[FM], fb[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            fb[j] = *reinterpret_cast<const u32x4*>(&cb[swz(c.brow0 + j * 16 + c.lrow, ch)]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            fa[i] = *reinterpret_cast<const u32x4*>(&ca[swz(c.arow0 + i * 16 + c.lrow, ch)]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
    }
}

// the zero row that the direct-load kernel's LoRA stages read for rows
// outside the run being expanded
__device__ __attribute__((aligned(128))) uint16_t g_zero_row[64] = {};

template <int BM, int BNT, int WM, int WN, int NS, bool GATEUP>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_dma(GemmArgs a) {
    constexpr int NW = WM * WN;
    constexpr int FM = BM / (16 * WM), FN = BNT / (16 * WN);
    constexpr int A_PW = BM / 8 / NW, B_PW = BNT / 8 / NW;  // 1 KiB blocks per wave per stage
    constexpr int LPS = A_PW + B_PW;                          // loads per wave per stage
    static_assert(A_PW * NW * 8 == BM && B_PW * NW * 8 == BNT, "tile rows must split over waves");
    static_assert(!GATEUP || FN % 2 == 0, "gate/up fragments come in pairs");
    static_assert(NS == 2 || NS == 3, "two or three LDS stages");
    constexpr int kCols = tile_cols<BNT, GATEUP>();
    const TileOrder order(a, kCols, BM);
    const int t = order.of_workgroup(blockIdx.x, a.xcd_slots);
    if (t >= order.total()) return;
    int b, tile;
    order.at(t, b, tile);
    const int e = a.blk_e_b[b];
    if (e < 0) return;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int wm = wave / WN, wn = wave % WN;
    const int kc = lane >> 4, lrow = lane & 15;
    const int I = GATEUP ? a.N_out : 0;
    const int Nw = GATEUP ? 2 * a.N_out : a.N_out;
    const int c0 = tile * kCols;
    const int K = a.K;
    const int row0 = b * BM;
    auto wrow_of = [&](int r) {
        const int f = r >> 4;
        int col = c0 + 16 * (GATEUP ? (f >> 1) : f) + (r & 15);
        col = min(col, a.N_out - 1);
        return (GATEUP && (f & 1)) ? I + col : col;
    };

    __shared__ __attribute__((aligned(1024))) uint16_t As0[BM * 64], As1[BM * 64], As2[NS > 2 ? BM * 64 : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t Bs0[BNT * 64], Bs1[BNT * 64], Bs2[NS > 2 ? BNT * 64 : 8];

    // lane l of a 1 KiB block fills row 8*blk + l/8, physical chunk l%8, which
    // holds logical chunk (l%8) ^ (row & 7) under the swizzle used by swz()
    const int lr = lane >> 3, pc = lane & 7;
    const uint16_t* asrc[A_PW];
    const int p_first = a.sorted_b[row0];
#pragma unroll
    for (int i = 0; i < A_PW; ++i) {
        const int r = 8 * (wave * A_PW + i) + lr;
        const int c = pc ^ (r & 7);
        size_t xr;
        if (GATEUP) {
            const int p = a.sorted_b[row0 + r];
            xr = static_cast<size_t>((p < a.P ? p : p_first) / a.top_k);
        } else {
            xr = static_cast<size_t>(row0 + r);
        }
        asrc[i] = a.X + xr * K + c * 8;
    }
    const uint16_t* bsrc[B_PW];
#pragma unroll
    for (int i = 0; i < B_PW; ++i) {
        const int r = 8 * (wave * B_PW + i) + lr;
        const int c = pc ^ (r & 7);
        bsrc[i] = a.W + (static_cast<size_t>(e) * Nw + wrow_of(r)) * K + c * 8;
    }

    const int wrow_base = row0 + wm * (BM / WM);
    const bool wlive = a.sorted_b[wrow_base] < a.P;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / 64;

    // LoRA expand as extra pipeline stages. The tile's rows hold one expert
    // and are ordered by adapter, so the adapters form runs. For each run the
    // pipeline appends s_hl_stride / 64 stages whose A rows are the run's
    // rows of S as bf16 [hi | lo | zeros] (other rows read a zero row) and
    // whose B rows are the run's LoRA B rows, each read twice (once against
    // hi, once against lo): the same MFMAs as the epilogue expand, now fed
    // through LDS with their loads in flight while earlier stages multiply.
    constexpr int RPL = BM / 64;  // tile rows per lane
    int nruns = 0;
    bool pipe_expand = false;
    int row_ad[A_PW];
#pragma unroll
    for (int i = 0; i < A_PW; ++i) row_ad[i] = -1;
    int adq[RPL];            // lane l: adapter of tile row 64 q + l
    uint64_t starts[RPL];    // first rows of the runs (wave-uniform)
#pragma unroll
    for (int q = 0; q < RPL; ++q) {
        adq[q] = -1;
        starts[q] = 0;
    }
    if (a.L > 0 && a.S_hl != nullptr) {
        pipe_expand = true;
#pragma unroll
        for (int q = 0; q < RPL; ++q) adq[q] = a.slot_adapter[row0 + 64 * q + lane];
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
            int prev = __shfl(adq[q], (lane + 63) & 63);
            const int carry = q > 0 ? __shfl(adq[q > 0 ? q - 1 : 0], 63) : -2;
            if (lane == 0) prev = carry;
            starts[q] = ballot64(adq[q] >= 0 && adq[q] != prev);
            nruns += __popcll(starts[q]);
        }
#pragma unroll
        for (int i = 0; i < A_PW; ++i) {
            const int r = 8 * (wave * A_PW + i) + lr;  // 8 rows of one 64-row group
            const int qi = (8 * (wave * A_PW + i)) / 64;
            int v = adq[0];
#pragma unroll
            for (int q = 1; q < RPL; ++q)
                if (q == qi) v = adq[q];
            row_ad[i] = __shfl(v, r & 63);
        }
    }
    // adapter of run n: the row of the n-th run start, counted over the
    // 64-row groups in order
    auto run_adapter = [&](int n) {
        int ad = -1;
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
            const int c = __popcll(starts[q]);
            if (ad < 0 && n < c) {
                uint64_t m = starts[q];
                for (int i = 0; i < n; ++i) m &= m - 1;
                ad = __builtin_amdgcn_readlane(adq[q], __ffsll(static_cast<long long>(m)) - 1);
            }
            n -= c;
        }
        return ad;
    };
    const int spr = pipe_expand ? a.s_hl_stride / 64 : 0;  // stages per run
    const int nk_all = nk + nruns * spr;
    auto issue = [&](int stage, uint16_t* ab, uint16_t* bb) {
        if (stage < nk) {
            dma_issue<A_PW, B_PW>(asrc, bsrc, ab, bb, wave, stage * 64, a.w_stream != 0);
            return;
        }
        const int t = stage - nk, q = t / spr, sub = t - q * spr;
        const int ad = run_adapter(q);
#pragma unroll
        for (int i = 0; i < A_PW; ++i) {
            const int r = 8 * (wave * A_PW + i) + lr;
            const int c = pc ^ (r & 7);
            const uint16_t* src = row_ad[i] == ad
                                      ? a.S_hl + static_cast<size_t>(row0 + r) * a.s_hl_stride + sub * 64 + c * 8
                                      : g_zero_row + c * 8;
            dma16(src, ab + (wave * A_PW + i) * 512);
        }
#pragma unroll
        for (int i = 0; i < B_PW; ++i) {
            const int r = 8 * (wave * B_PW + i) + lr;
            const int c = pc ^ (r & 7);
            const int j0 = (sub * 64 + c * 8) & (a.r - 1);
            dma16(a.Bl + (static_cast<size_t>(ad * a.E + e) * Nw + wrow_of(r)) * a.r + j0,
                  bb + (wave * B_PW + i) * 512);
        }
    };

    const DmaCtx ctx{wm * (BM / WM), wn * (BNT / WN), kc, lrow, wlive};
    uint16_t* const abufs[3] = {As0, As1, As2};
    uint16_t* const bbufs[3] = {Bs0, Bs1, Bs2};
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nk_all) issue(s, abufs[s], bbufs[s]);
    // one pipeline step: stage k (buffer k % NS) is complete for this wave once
    // at most the loads of the stage requested after it are in flight; the
    // barrier then makes every wave's part visible and frees the buffer that
    // the next request overwrites (it was multiplied one step earlier)
    for (int k = 0; k < nk_all; k += NS) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (k + s >= nk_all) break;
            if (k + s + 1 < nk_all)
                wait_vmcnt<(NS - 2) * LPS>();
            else
                wait_vmcnt<0>();
            bare_barrier();
            if (k + s + NS - 1 < nk_all) issue(k + s + NS - 1, abufs[(s + NS - 1) % NS], bbufs[(s + NS - 1) % NS]);
            dma_step(ctx, acc, abufs[s], bbufs[s]);
        }
    }

    tile_epilogue<FM, FN, GATEUP>(a, acc, wlive, wrow_base, wn, c0, e, kc, lrow, wrow_of, 0, !pipe_expand);
}

// ---------------------------------------------------------------------------
// Launch shapes by block height (rows per block of the base view):
//   16        skinny: one wave per 16 x 64 tile (gate_up: 32 h columns)
//   32, 64    tiled:  32 x 128 (1 x 4 waves) and 64 x 128 (2 x 2 waves)
//   128       direct-load: 128 x 192 (2 x 2 waves, 2 stages, 2 workgroups per CU)
//   256       direct-load: 256 x 256 (2 x 4 waves of 128 x 64, 2 stages, one
//             workgroup per CU)
// These shapes were the fastest of those measured on MI355X for the
// decode-, many-adapter- and prefill-shaped layers. The column count may
// leave a partial last tile.
// 16-column weight fragments per skinny wave and register pipeline stages,
// per projection (gate_up: fragments pair gate and up rows, so a wave writes
// FN * 8 h columns; down: FN * 16 D columns). The gate_up projection also has
// an 8-fragment form (GemmArgs::frags, one wave per tile): half the waves,
// each with twice the bytes per K chunk in flight.
constexpr int kSkinnyFNGateUp = 4;
constexpr int kSkinnyFNGateUpWide = 8;
constexpr int kSkinnyNSGateUp = 2;
constexpr int kSkinnyFNDown = 4;
constexpr int kSkinnyNSDown = 2;

template <int BM, int BNT, int WM, int WN, int NS>
static hipError_t launch_dma(const GemmArgs& a, hipStream_t s) {
    if (!a.n_b_live) return hipErrorInvalidValue;
    const int cols = a.gate_up ? BNT / 2 : BNT;
    const int n_tiles = (a.N_out + cols - 1) / cols;
    constexpr int lds = 2 * NS * (BM + BNT) * 64;        // bytes (NS stages of bf16 A and B)
    // by LDS (160 KiB per CU) and by registers (these kernels hold 2 waves per SIMD)
    constexpr int per_cu = (160 * 1024 / lds) < (8 / (WM * WN)) ? (160 * 1024 / lds) : (8 / (WM * WN));
    static_assert(per_cu >= 1, "tile does not fit one CU");
    GemmArgs b = a;
    b.xcd_slots = kCus / kXcds * per_cu;
    // every tile of the capacity, in whole rounds of 8 S workgroups
    const long round = static_cast<long>(kXcds) * b.xcd_slots;
    const long tiles = static_cast<long>(n_tiles) * a.n_blocks;
    const long g = (tiles + round - 1) / round * round;
    if (g > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(g)), block(64 * WM * WN);
    if (a.gate_up)
        hipLaunchKernelGGL((k_gemm_dma<BM, BNT, WM, WN, NS, true>), grid, block, 0, s, b);
    else
        hipLaunchKernelGGL((k_gemm_dma<BM, BNT, WM, WN, NS, false>), grid, block, 0, s, b);
    return hipGetLastError();
}

// PER_CU: workgroups per CU (by LDS and registers: 4 for 32-row tiles, 3 for
// 64-row tiles)
template <int BM, int BNT, int WM, int WN, int PER_CU>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t s) {
    if (!a.n_b_live) return hipErrorInvalidValue;
    const int cols = a.gate_up ? BNT / 2 : BNT;
    const int n_tiles = (a.N_out + cols - 1) / cols;
    GemmArgs b = a;
    b.xcd_slots = kCus / kXcds * PER_CU;
    const long round = static_cast<long>(kXcds) * b.xcd_slots;
    const long tiles = static_cast<long>(n_tiles) * a.n_blocks;
    const long g = (tiles + round - 1) / round * round;
    if (g > 0x7fffffffL) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(g), a.ksplit), block(64 * WM * WN);
    if (a.gate_up)
        hipLaunchKernelGGL((k_gemm_tiled<BM, BNT, WM, WN, true>), grid, block, 0, s, b);
    else
        hipLaunchKernelGGL((k_gemm_tiled<BM, BNT, WM, WN, false>), grid, block, 0, s, b);
    return hipGetLastError();
}

// The packed copy of W for the 16-row kernel: for expert e, column tile t and
// 64-wide K chunk q, one block of FN x 1 KiB, [fragment f][half h][lane][8]:
// lane (16 g + n) of (f, h) holds W[row of fragment f + n][64 q + 16 g + 8 h
// ... + 8], the 16 bytes that lane loads for that fragment and half. One
// thread copies one 16-byte piece.
template <bool GATEUP>
__global__ __launch_bounds__(256) void k_pack_skinny(const uint16_t* __restrict__ W, uint16_t* __restrict__ Wp,
                                                     int E, int N_out, int K) {
    constexpr int FN = kPackFrags;
    constexpr int kCols = GATEUP ? FN * 8 : FN * 16;
    const int n_tiles = N_out / kCols, nq = K / 64;
    const int I = GATEUP ? N_out : 0;
    const int Nw = GATEUP ? 2 * N_out : N_out;
    const long total = static_cast<long>(E) * n_tiles * nq * FN * 128;
    for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
         i += static_cast<long>(gridDim.x) * blockDim.x) {
        const int lane = static_cast<int>(i & 63);
        long r = i >> 6;
        const int h = static_cast<int>(r & 1);
        r >>= 1;
        const int f = static_cast<int>(r % FN);
        r /= FN;
        const int q = static_cast<int>(r % nq);
        r /= nq;
        const int t = static_cast<int>(r % n_tiles);
        const int e = static_cast<int>(r / n_tiles);
        const int row = w_row_of_frag<GATEUP>(f, t * kCols, I) + (lane & 15);
        const int col = q * 64 + 16 * (lane >> 4) + 8 * h;
        *reinterpret_cast<u32x4*>(Wp + i * 8) =
            *reinterpret_cast<const u32x4*>(W + (static_cast<size_t>(e) * Nw + row) * K + col);
    }
}

bool pack_skinny_supported(int N_out, int K, int gate_up) {
    const int cols = gate_up ? kPackFrags * 8 : kPackFrags * 16;
    return N_out > 0 && K > 0 && N_out % cols == 0 && K % 64 == 0;
}

hipError_t launch_pack_skinny(const uint16_t* W, uint16_t* Wp, int E, int N_out, int K, int gate_up,
                              hipStream_t s) {
    if (!pack_skinny_supported(N_out, K, gate_up) || E <= 0) return hipErrorInvalidValue;
    const long pieces = static_cast<long>(E) * (gate_up ? 2 : 1) * N_out * (K / 8);
    const long blocks = std::min<long>((pieces + 255) / 256, 65536);
    if (gate_up)
        hipLaunchKernelGGL(k_pack_skinny<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, W, Wp, E,
                           N_out, K);
    else
        hipLaunchKernelGGL(k_pack_skinny<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, W, Wp, E,
                           N_out, K);
    return hipGetLastError();
}

bool gemm_supported(int N_out, int K, int gate_up, int bm_b) {
    if (K % 64 != 0 || N_out % 32 != 0) return false;
    if (bm_b == 16) return N_out % (gate_up ? kSkinnyFNGateUp * 8 : kSkinnyFNDown * 16) == 0;
    return bm_b == 32 || bm_b == 64 || bm_b == 128 || bm_b == 256;
}

bool skinny_waves_ok(int K, int ksplit, int ksw) {
    // one wave per tile takes any K range; with more, every wave keeps at
    // least 4 chunks of 64 of its workgroup's K range
    if (ksplit < 1 || K % (64 * ksplit)) return false;
    if (ksw == 1) return true;
    return (ksw == 2 || ksw == 4) && K / ksplit / 64 >= 4 * ksw;
}

int gemm_down_ksplit(int N_out, int K, int bm_b, int n_blocks) {
    if (bm_b >= 128 || n_blocks <= 0) return 1;
    const long cols = bm_b == 16 ? 16 * kSkinnyFNDown : 128;
    const long waves = (N_out + cols - 1) / cols * n_blocks * (bm_b == 16 ? 1 : 4);
    // about one wave per SIMD: the dense layer's down projection (K = 25600,
    // 160 waves unsplit) measured 229 us with 5 ranges against 241 us with 25
    constexpr long kTargetWaves = 1024;
    constexpr int kMinChunks = 8;        // at least 512 of K per split
    constexpr int kLongK = 96;           // only long K ranges (>= 6144) are split
    const int chunks = K / 64;
    if (chunks < kLongK) return 1;
    int ks = static_cast<int>(std::min<long>((kTargetWaves + waves - 1) / waves, chunks / kMinChunks));
    for (; ks > 1; --ks)
        if (chunks % ks == 0) break;
    return std::max(ks, 1);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
    if (a.n_blocks == 0) return hipSuccess;
    if (!gemm_supported(a.N_out, a.K, a.gate_up, a.bm_b)) return hipErrorInvalidValue;
    if (a.ksplit < 1 || (a.K / 64) % a.ksplit || (a.ksplit > 1 && (a.gate_up || a.bm_b >= 128)))
        return hipErrorInvalidValue;
    if (a.L > 0 && (a.s_split < 1 || a.s_split > (a.prod_units > 0 ? kMaxProducerSplit : kMaxShrinkSplit)))
        return hipErrorInvalidValue;
    if (a.prod_units < 0 || (a.prod_units > 0 && (a.L <= 0 || a.bm_b != 16 || a.S_hl || !a.done || !a.status ||
                                                  !a.n_l || !a.S_out || a.S_out != a.S ||
                                                  a.prod_ncf != (a.r + 15) / 16 || a.bm_l < 16 ||
                                                  a.bm_l > 256 || (a.bm_l & (a.bm_l - 1)))))
        return hipErrorInvalidValue;
    if (a.L > 0 && a.S_hl && (a.s_split != 1 || a.s_hl_stride != s_hl_stride_of(a.r)))
        return hipErrorInvalidValue;
    if (a.bm_b == 16) {
        const bool wide = a.gate_up && a.frags == kSkinnyFNGateUpWide;
        const int cols = a.gate_up ? a.frags * 8 : kSkinnyFNDown * 16;
        const int ksw = a.ksw;
        if (!(ksw == 1 || ksw == 2 || ksw == 4) || (a.K / a.ksplit) / 64 < ksw) return hipErrorInvalidValue;
        if ((a.gate_up && a.frags != kSkinnyFNGateUp && !(wide && ksw == 1)) || a.N_out % cols)
            return hipErrorInvalidValue;
        if (a.local && (!a.gate_up || ksw != 1 || (a.L > 0 && a.bm_l != 16) || !local_route_fits(a.T, a.E, a.top_k) ||
                        a.n_blocks != a.E || !a.adapter_ids || (!a.logits && !a.local_ids)))
            return hipErrorInvalidValue;
        const long total = static_cast<long>(a.N_out / cols) * a.n_blocks * a.ksplit +
                           (a.prod_units + ksw - 1) / ksw + (a.local ? 1 : 0);
        if (total > 0x7fffffffL) return hipErrorInvalidValue;
        const dim3 grid(static_cast<unsigned>(total)), block(64 * ksw);
        // paired adapter runs where the grid holds at most two waves per SIMD
        const bool pair = total * ksw <= 2L * kCus * 4;
#define MOELORA_SKINNY(G, FN, NS, W)                                                                  \
    do {                                                                                              \
        if (pair) hipLaunchKernelGGL((k_gemm_skinny<G, FN, NS, W, true>), grid, block, 0, s, a);     \
        else hipLaunchKernelGGL((k_gemm_skinny<G, FN, NS, W, false>), grid, block, 0, s, a);         \
    } while (0)
        if (wide) {
            MOELORA_SKINNY(true, kSkinnyFNGateUpWide, kSkinnyNSGateUp, 1);
        } else if (a.gate_up) {
            if (ksw == 1) MOELORA_SKINNY(true, kSkinnyFNGateUp, kSkinnyNSGateUp, 1);
            if (ksw == 2) MOELORA_SKINNY(true, kSkinnyFNGateUp, kSkinnyNSGateUp, 2);
            if (ksw == 4) MOELORA_SKINNY(true, kSkinnyFNGateUp, kSkinnyNSGateUp, 4);
        } else {
            if (ksw == 1) MOELORA_SKINNY(false, kSkinnyFNDown, kSkinnyNSDown, 1);
            if (ksw == 2) MOELORA_SKINNY(false, kSkinnyFNDown, kSkinnyNSDown, 2);
            if (ksw == 4) MOELORA_SKINNY(false, kSkinnyFNDown, kSkinnyNSDown, 4);
        }
#undef MOELORA_SKINNY
        return hipGetLastError();
    }
    switch (a.bm_b) {
        case 32: return launch_tiled<32, 128, 1, 4, 4>(a, s);
        case 64: return launch_tiled<64, 128, 2, 2, 3>(a, s);
        case 128: return launch_dma<128, 192, 2, 2, 2>(a, s);
        case 256: return launch_dma<256, 256, 2, 4, 2>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moelora
