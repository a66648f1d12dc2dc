// Routing (top-k + renormalised softmax) and the deterministic expert x adapter
// alignment, for gfx950.
//
// Routing follows the AWS ML Blog post "Efficiently serve dozens of fine-tuned
// models with vLLM on Amazon SageMaker AI and Amazon Bedrock", section
// "Implementing multi-LoRA inference for MoE models in vLLM" (a router sends
// each token to its most relevant experts). The alignment realises the
// "additional grid dimension corresponding to the LoRA index" and the compound
// sparsity of several adapters on top of expert routing (same post, section
// "Tuning kernel configurations for Amazon SageMaker AI and Amazon Bedrock").
#include <climits>

#include "common.h"
#include "kernels.h"

namespace moelora {

// ---------------------------------------------------------------------------
// Route: one wave per token. Lane l holds the logits of experts l, l+64, ...
// k rounds of a wave-wide arg-max (larger value first, lower id on ties); lane
// j keeps the j-th pick. Weights are the softmax over the k picks.
constexpr int kRouteMaxPerLane = 16;  // E <= 1024

__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E,
                                               int k, int32_t* __restrict__ ids,
                                               float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* row = logits + static_cast<size_t>(t) * E;
    const int nper = (E + 63) >> 6;
    float v[kRouteMaxPerLane];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        const bool ok = i < nper && e < E;
        v[i] = ok ? row[e] : 0.0f;
        if (!ok) taken |= 1u << i;
    }
    float my_v = 0.0f;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = INT_MAX;  // INT_MAX = nothing left in this lane
#pragma unroll
        for (int i = 0; i < kRouteMaxPerLane; ++i) {
            if (!((taken >> i) & 1u) && (bi == INT_MAX || v[i] > bv)) {
                bv = v[i];
                bi = lane + 64 * i;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            const bool better = oi != INT_MAX &&
                                (bi == INT_MAX || ov > bv || (ov == bv && oi < bi));
            if (better) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (lane == j) {
            my_v = bv;
            my_id = bi;
        }
    }
    const float m = __shfl(my_v, 0);
    const float ex = lane < k ? expf(my_v - m) : 0.0f;
    float s = ex;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane < k) {
        ids[static_cast<size_t>(t) * k + lane] = my_id;
        w[static_cast<size_t>(t) * k + lane] = ex / s;
    }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(k_route, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, w);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Align: one 1024-thread workgroup.
//   key(p) = e * (L+1) + a',  a' = adapter if in [0,L) else L.
// Wave w < nw owns the contiguous pair range [w*R, (w+1)*R). Lanes with equal
// keys inside a 64-pair step are found with one ballot per key bit, so ranks
// inside a step come from popcounts; per-wave, per-key histograms in LDS give
// each wave its exclusive offset. The result is a stable counting sort whose
// output does not depend on scheduling.
constexpr int kAlignThreads = 1024;
constexpr int kAlignLdsInts = 38912;  // 152 KiB of the 160 KiB LDS

static int align_fixed_ints(int E, int L) {
    const int nkeys = E * (L + 1);
    return 2 * nkeys + E * L + E + 64;
}

int align_hist_waves(int E, int L) {
    const long nkeys = static_cast<long>(E) * (L + 1);
    const long avail = kAlignLdsInts - static_cast<long>(align_fixed_ints(E, L));
    if (nkeys <= 0 || avail < nkeys) return 0;
    const long nw = avail / nkeys;
    return static_cast<int>(nw > 16 ? 16 : nw);
}

__device__ __forceinline__ uint64_t match_key(int key, bool valid, int nbits) {
    uint64_t m = ballot64(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bb = ballot64(bit);
        m &= bit ? bb : ~bb;
    }
    return valid ? m : 0ull;
}

// Exclusive prefix sum of a[0..n) in LDS by all 1024 threads; returns the total.
__device__ int block_excl_scan(int* a, int n, int* red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n + kAlignThreads - 1) / kAlignThreads;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += a[i];
    int incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int w = 0; w < kAlignThreads / 64; ++w) {
            const int c = red[w];
            red[w] = run;
            run += c;
        }
        red[kAlignThreads / 64] = run;
    }
    __syncthreads();
    int prefix = red[wave] + incl - s;
    for (int i = lo; i < hi; ++i) {
        const int v = a[i];
        a[i] = prefix;
        prefix += v;
    }
    const int total = red[kAlignThreads / 64];
    __syncthreads();
    return total;
}

__device__ __forceinline__ int roundup_i(int v, int m) { return (v + m - 1) / m * m; }

__global__ __launch_bounds__(kAlignThreads) void k_align(
    const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ adapter_ids, int T, int k,
    int E, int L, int bm_b, int bm_l, int C_b, int C_l, int nw, int R,
    int32_t* __restrict__ sorted_b, int32_t* __restrict__ blk_e_b, int32_t* __restrict__ n_b_out,
    int32_t* __restrict__ sorted_l, int32_t* __restrict__ blk_e_l, int32_t* __restrict__ blk_a_l,
    int32_t* __restrict__ n_l_out, int32_t* __restrict__ slot_of_pair,
    int32_t* __restrict__ lslot_of_pair, int32_t* __restrict__ slot_adapter,
    int32_t* __restrict__ zero_buf, int zero_n) {
    __shared__ int lds[kAlignLdsInts];
    const int L1 = L + 1;
    const int nkeys = E * L1, nseg = E * L, P = T * k;
    int* hist = lds;                 // [nw][nkeys]
    int* cnt = hist + nw * nkeys;    // [nkeys]
    int* bpos = cnt + nkeys;         // [nkeys]  base-view start of each key
    int* lpos = bpos + nkeys;        // [nseg]   LoRA-view start of each segment
    int* ne = lpos + nseg;           // [E]      pairs per expert
    int* red = ne + E;               // [64]
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;

    auto pair_key = [&](int p) {
        const int e = min(max(topk_ids[p], 0), E - 1);  // memory safety for foreign ids
        int a = adapter_ids[p / k];
        if (a < 0 || a >= L) a = L;
        return e * L1 + a;
    };

    for (int i = tid; i < nw * nkeys; i += kAlignThreads) hist[i] = 0;
    for (int i = tid; i < E; i += kAlignThreads) ne[i] = 0;
    for (int i = tid; i < zero_n; i += kAlignThreads) zero_buf[i] = 0;
    __syncthreads();

    // 1. per-wave key histograms
    if (wave < nw) {
        const int lo = wave * R, hi = min(P, lo + R);
        int* h = hist + wave * nkeys;
        for (int base = lo; base < hi; base += 64) {
            const int p = base + lane;
            const bool valid = p < hi;
            const int key = valid ? pair_key(p) : 0;
            const uint64_t m = match_key(key, valid, nbits);
            if (valid && lane == __ffsll(static_cast<long long>(m)) - 1) h[key] += popc64(m);
        }
    }
    __syncthreads();

    // 2. column scan over waves -> exclusive per-wave offsets, totals per key
    for (int key = tid; key < nkeys; key += kAlignThreads) {
        int run = 0;
        for (int w = 0; w < nw; ++w) {
            const int c = hist[w * nkeys + key];
            hist[w * nkeys + key] = run;
            run += c;
        }
        cnt[key] = run;
        if (run) atomicAdd(&ne[key / L1], run);
    }
    __syncthreads();
    for (int key = tid; key < nkeys; key += kAlignThreads) {
        const int e = key / L1;
        int v = cnt[key];
        if (key % L1 == L) v += roundup_i(ne[e], bm_b) - ne[e];  // expert's padding
        bpos[key] = v;
    }
    for (int s = tid; s < nseg; s += kAlignThreads)
        lpos[s] = roundup_i(cnt[(s / L) * L1 + s % L], bm_l);
    __syncthreads();
    const int n_b = block_excl_scan(bpos, nkeys, red);
    const int n_l = block_excl_scan(lpos, nseg, red);

    // 3. sentinels, tails and block maps
    for (int idx = tid; idx < E * bm_b; idx += kAlignThreads) {
        const int e = idx / bm_b, i = idx % bm_b;
        const int last = e * L1 + L;
        if (i < roundup_i(ne[e], bm_b) - ne[e]) {
            sorted_b[bpos[last] + cnt[last] + i] = P;
            if (slot_adapter) slot_adapter[bpos[last] + cnt[last] + i] = -1;
        }
    }
    for (int i = n_b + tid; i < C_b; i += kAlignThreads) {
        sorted_b[i] = P;
        if (slot_adapter) slot_adapter[i] = -1;
    }
    for (int idx = tid; idx < nseg * bm_l; idx += kAlignThreads) {
        const int s = idx / bm_l, i = idx % bm_l;
        const int c = cnt[(s / L) * L1 + s % L];
        if (i < roundup_i(c, bm_l) - c) sorted_l[lpos[s] + c + i] = P;
    }
    for (int i = n_l + tid; i < C_l; i += kAlignThreads) sorted_l[i] = P;
    for (int b = tid; b < C_b / bm_b; b += kAlignThreads) {
        const int pos = b * bm_b;
        int e = -1;
        if (pos < n_b) {
            int lo = 0, hi = E - 1;  // largest e with start(e) <= pos
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (bpos[mid * L1] <= pos) lo = mid; else hi = mid - 1;
            }
            e = lo;
        }
        blk_e_b[b] = e;
    }
    for (int b = tid; b < C_l / bm_l; b += kAlignThreads) {
        const int pos = b * bm_l;
        int e = -1, a = -1;
        if (pos < n_l) {
            int lo = 0, hi = nseg - 1;  // largest segment with start <= pos
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (lpos[mid] <= pos) lo = mid; else hi = mid - 1;
            }
            e = lo / L;
            a = lo % L;
        }
        blk_e_l[b] = e;
        blk_a_l[b] = a;
    }
    if (tid == 0) {
        *n_b_out = n_b;
        *n_l_out = n_l;
    }

    // 4. stable scatter
    if (wave < nw) {
        const int lo = wave * R, hi = min(P, lo + R);
        int* h = hist + wave * nkeys;
        const uint64_t below = lanemask_lt();
        for (int base = lo; base < hi; base += 64) {
            const int p = base + lane;
            const bool valid = p < hi;
            const int key = valid ? pair_key(p) : 0;
            const uint64_t m = match_key(key, valid, nbits);
            const int off = valid ? h[key] : 0;
            if (valid && lane == __ffsll(static_cast<long long>(m)) - 1) h[key] = off + popc64(m);
            if (valid) {
                const int pos = off + popc64(m & below);
                const int slot = bpos[key] + pos;
                sorted_b[slot] = p;
                if (slot_of_pair) slot_of_pair[p] = slot;
                const int ap = key % L1;
                int lslot = -1;
                if (ap < L) {
                    lslot = lpos[(key / L1) * L + ap] + pos;
                    sorted_l[lslot] = p;
                }
                if (lslot_of_pair) lslot_of_pair[p] = lslot;
                if (slot_adapter) slot_adapter[slot] = ap < L ? ap : -1;
            }
        }
    }
}

hipError_t launch_align(const int32_t* topk_ids, const int32_t* adapter_ids, int T, int k,
                        int E, int L, int bm_b, int bm_l, int C_b, int C_l,
                        int32_t* sorted_b, int32_t* blk_e_b, int32_t* n_b,
                        int32_t* sorted_l, int32_t* blk_e_l, int32_t* blk_a_l, int32_t* n_l,
                        int32_t* slot_of_pair, int32_t* lslot_of_pair, int32_t* slot_adapter,
                        int32_t* zero_buf, int zero_n, hipStream_t s) {
    const int nw = align_hist_waves(E, L);
    if (nw <= 0) return hipErrorInvalidValue;
    const int P = T * k;
    const int per = (P + nw - 1) / nw;
    const int R = ((per + 63) / 64) * 64;
    hipLaunchKernelGGL(k_align, dim3(1), dim3(kAlignThreads), 0, s, topk_ids, adapter_ids, T, k,
                       E, L, bm_b, bm_l, C_b, C_l, nw, R > 0 ? R : 64, sorted_b, blk_e_b, n_b,
                       sorted_l, blk_e_l, blk_a_l, n_l, slot_of_pair, lslot_of_pair, slot_adapter,
                       zero_buf, zero_n);
    return hipGetLastError();
}

}  // namespace moelora
