// Routing (top-k + renormalised softmax) and the deterministic expert x adapter
// alignment, for gfx950.
//
// Routing follows the AWS ML Blog post "Efficiently serve dozens of fine-tuned
// models with vLLM on Amazon SageMaker AI and Amazon Bedrock", section
// "Implementing multi-LoRA inference for MoE models in vLLM" (a router sends
// each token to its most relevant experts). The alignment groups the pairs by
// expert and adapter slot at once, which gives the LoRA kernels their extra
// launch axis over adapters and captures how adapter choice thins out the rows
// of each expert further (same post, section "Tuning kernel configurations for
// Amazon SageMaker AI and Amazon Bedrock").
#include <algorithm>
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
                                               float* __restrict__ w,
                                               int32_t* __restrict__ zero_words, int n_zero,
                                               float* __restrict__ zero_out, int H) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    // counters that later kernels of the same call count up from zero
    if (blockIdx.x == 0 && threadIdx.x < n_zero) zero_words[threadIdx.x] = 0;
    // the output rows of this workgroup's tokens, when the down projection
    // adds its weighted rows into them
    if (zero_out) {
        const int t0 = blockIdx.x * 4, nt = min(4, T - t0);
        f32x4* o = reinterpret_cast<f32x4*>(zero_out + static_cast<size_t>(t0) * H);
        for (int i = threadIdx.x; i < nt * H / 4; i += 256) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
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
                        hipStream_t s, int32_t* zero_words, int n_zero, float* zero_out, int H) {
    if (T == 0) return hipSuccess;
    if (n_zero < 0 || n_zero > 256 || (n_zero > 0 && !zero_words)) return hipErrorInvalidValue;
    if (zero_out && (H <= 0 || H % 4)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_route, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, w,
                       zero_words, n_zero, zero_out, H);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Align. key(p) = e * (L+1) + a',  a' = adapter if in [0,L) else L.
// The P pairs are cut into nr contiguous ranges of R pairs (R a multiple of
// 64). One 1024-thread workgroup counts every range's keys into its own LDS
// histogram row (order-free LDS atomics), turns the rows into exclusive
// per-range offsets and the key totals into segment starts, and writes the
// padding, the tails and the block maps. The stable scatter then walks each
// range in 64-pair steps: lanes with equal keys in a step are found with one
// ballot per key bit, so ranks inside a step come from popcounts, and the
// range's running per-key offsets come from its LDS row. Small batches scatter
// in the same workgroup (wave w takes ranges w, w+16, ...); large ones hand
// the offsets to k_align_scatter, one workgroup per range, so the scattered
// stores are spread over many CUs. Nothing depends on scheduling order.
constexpr int kAlignThreads = 1024;
constexpr int kAlignLdsInts = 38912;  // 152 KiB of the 160 KiB LDS
constexpr int kAlignStepsPerRange = 4;

static int align_fixed_ints(int E, int L) {
    const int nkeys = E * (L + 1);
    return 2 * nkeys + E * L + E + 64;
}

// most ranges whose histograms fit the align kernel's LDS (0 = none fits)
static int align_max_ranges(int E, int L) {
    const long nkeys = static_cast<long>(E) * (L + 1);
    const long avail = kAlignLdsInts - static_cast<long>(align_fixed_ints(E, L));
    if (nkeys <= 0 || avail < nkeys) return 0;
    return static_cast<int>(std::min<long>(avail / nkeys, 4096));
}

// range count and range length for P pairs
static void align_ranges(int P, int E, int L, int* nr, int* R) {
    const int maxr = align_max_ranges(E, L);
    const int per = 64 * kAlignStepsPerRange;
    int n = std::max(1, (P + per - 1) / per);
    n = std::min(n, std::max(maxr, 1));
    int r = (P + n - 1) / n;
    r = std::max(64, (r + 63) / 64 * 64);
    *nr = std::max(1, (P + r - 1) / r);
    *R = r;
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

struct AlignKeys {
    const int32_t* topk_ids;
    const int32_t* adapter_ids;
    int k, E, L;
    __device__ __forceinline__ int operator()(int p) const {
        const int e = min(max(topk_ids[p], 0), E - 1);  // memory safety for foreign ids
        int a = adapter_ids[p / k];
        if (a < 0 || a >= L) a = L;
        return e * (L + 1) + a;
    }
};

struct AlignOut {
    int32_t* sorted_b;
    int32_t* sorted_l;
    int32_t* slot_of_pair;   // may be null
    int32_t* lslot_of_pair;  // may be null
    int32_t* slot_adapter;   // may be null
};

// Stable scatter of pairs [lo, hi) by one wave; h = the range's running
// per-key offsets (LDS), bpos / lpos = segment starts.
__device__ __forceinline__ void scatter_range(const AlignKeys& keyf, const AlignOut& o, int lo, int hi,
                                              int* h, const int* bpos, const int* lpos, int L,
                                              int nbits) {
    const int lane = lane_id();
    const int L1 = L + 1;
    const uint64_t below = lanemask_lt();
    int keys[kAlignStepsPerRange];
#pragma unroll
    for (int c = 0; c < kAlignStepsPerRange; ++c) {
        // clamped, unconditional loads, all in flight together
        const int p = lo + 64 * c + lane;
        const int key = keyf(min(p, hi - 1));
        keys[c] = p < hi ? key : -1;
    }
    for (int base = lo, c = 0; base < hi; base += 64, ++c) {
        const int p = base + lane;
        int key = -1;
        if (c < kAlignStepsPerRange) {
#pragma unroll
            for (int u = 0; u < kAlignStepsPerRange; ++u)
                if (u == c) key = keys[u];
        } else {
            key = p < hi ? keyf(p) : -1;  // ranges longer than the prefetch
        }
        const bool valid = key >= 0;
        if (!valid) key = 0;
        const uint64_t m = match_key(key, valid, nbits);
        const int off = valid ? h[key] : 0;
        if (valid && lane == __ffsll(static_cast<long long>(m)) - 1) h[key] = off + popc64(m);
        if (valid) {
            const int pos = off + popc64(m & below);
            const int slot = bpos[key] + pos;
            o.sorted_b[slot] = p;
            if (o.slot_of_pair) o.slot_of_pair[p] = slot;
            const int ap = key % L1;
            int lslot = -1;
            if (ap < L) {
                lslot = lpos[(key / L1) * L + ap] + pos;
                o.sorted_l[lslot] = p;
            }
            if (o.lslot_of_pair) o.lslot_of_pair[p] = lslot;
            if (o.slot_adapter) o.slot_adapter[slot] = ap < L ? ap : -1;
        }
    }
}

// a[from .. to) = v by the whole workgroup; 16-byte stores where a is
// 16-byte aligned and from, to are multiples of 4 (the view capacities and
// lengths are multiples of the block heights, so the library's own buffers
// always take that path)
__device__ __forceinline__ void fill_tail(int32_t* a, int from, int to, int v) {
    if ((reinterpret_cast<uintptr_t>(a) & 15) == 0 && (from & 3) == 0 && (to & 3) == 0) {
        const int4 q{v, v, v, v};
        for (int i = (from >> 2) + static_cast<int>(threadIdx.x); i < (to >> 2); i += blockDim.x)
            reinterpret_cast<int4*>(a)[i] = q;
    } else {
        for (int i = from + static_cast<int>(threadIdx.x); i < to; i += blockDim.x) a[i] = v;
    }
}

__global__ __launch_bounds__(kAlignThreads) void k_align(
    AlignKeys keyf, AlignOut o, int T, int bm_b_log2, int bm_l_log2, int C_b, int C_l, int nr,
    int R, int32_t* __restrict__ blk_e_b, int32_t* __restrict__ n_b_out,
    int32_t* __restrict__ blk_e_l, int32_t* __restrict__ blk_a_l, int32_t* __restrict__ n_l_out,
    int32_t* __restrict__ defer) {
    __shared__ int lds[kAlignLdsInts];
    const int E = keyf.E, L = keyf.L, L1 = L + 1;
    const int nkeys = E * L1, nseg = E * L, P = T * keyf.k;
    const int bm_b = 1 << bm_b_log2, bm_l = 1 << bm_l_log2;
    int* hist = lds;                 // [nr][nkeys]
    int* cnt = hist + nr * nkeys;    // [nkeys]
    int* bpos = cnt + nkeys;         // [nkeys]  base-view start of each key
    int* lpos = bpos + nkeys;        // [nseg]   LoRA-view start of each segment
    int* ne = lpos + nseg;           // [E]      pairs per expert
    int* red = ne + E;               // [64]
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;

    for (int i = tid; i < nr * nkeys; i += kAlignThreads) hist[i] = 0;
    for (int i = tid; i < E; i += kAlignThreads) ne[i] = 0;
    __syncthreads();

    // 1. per-range key counts (the order of the LDS atomics does not matter);
    // 8 keys per thread are loaded before their atomics, so the loads of a
    // round are in flight together (clamped indices, counted only if valid)
    for (int base = tid; base < P; base += 8 * kAlignThreads) {
        int key[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) key[u] = keyf(min(base + u * kAlignThreads, P - 1));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = base + u * kAlignThreads;
            if (p < P) atomicAdd(&hist[(p / R) * nkeys + key[u]], 1);
        }
    }
    __syncthreads();

    // 2. column scan over ranges -> exclusive per-range offsets, totals per key
    for (int key = tid; key < nkeys; key += kAlignThreads) {
        int run = 0;
        for (int r = 0; r < nr; ++r) {
            const int c = hist[r * nkeys + key];
            hist[r * nkeys + key] = run;
            run += c;
        }
        cnt[key] = run;
        if (run) atomicAdd(&ne[key / L1], run);
    }
    __syncthreads();
    for (int key = tid; key < nkeys; key += kAlignThreads) {
        const int e = key / L1;
        int v = cnt[key];
        if (key % L1 == L) v += ((ne[e] + bm_b - 1) & ~(bm_b - 1)) - ne[e];  // expert's padding
        bpos[key] = v;
    }
    for (int s = tid; s < nseg; s += kAlignThreads)
        lpos[s] = (cnt[(s / L) * L1 + s % L] + bm_l - 1) & ~(bm_l - 1);
    __syncthreads();
    const int n_b = block_excl_scan(bpos, nkeys, red);
    const int n_l = block_excl_scan(lpos, nseg, red);

    // 3. sentinels, tails and block maps
    for (int idx = tid; idx < (E << bm_b_log2); idx += kAlignThreads) {
        const int e = idx >> bm_b_log2, i = idx & (bm_b - 1);
        const int last = e * L1 + L;
        if (i < ((ne[e] + bm_b - 1) & ~(bm_b - 1)) - ne[e]) {
            const int slot = bpos[last] + cnt[last] + i;
            o.sorted_b[slot] = P;
            if (o.slot_adapter) o.slot_adapter[slot] = -1;
        }
    }
    // the tails past n_b and n_l
    fill_tail(o.sorted_b, n_b, C_b, P);
    if (o.slot_adapter) fill_tail(o.slot_adapter, n_b, C_b, -1);
    // each (expert, adapter) segment writes its own padding slots
    for (int s = tid; s < nseg; s += kAlignThreads) {
        const int e = s / L;
        const int c = cnt[e * L1 + (s - e * L)];
        const int base = lpos[s] + c, pad = ((c + bm_l - 1) & ~(bm_l - 1)) - c;
        for (int i = 0; i < pad; ++i) o.sorted_l[base + i] = P;
    }
    fill_tail(o.sorted_l, n_l, C_l, P);
    // block maps: each expert (base view) and each (expert, adapter) segment
    // (LoRA view) writes the entries of its own blocks; blocks past n_b / n_l
    // get -1
    for (int e = tid; e < E; e += kAlignThreads) {
        const int b0 = bpos[e * L1] >> bm_b_log2, nb = (ne[e] + bm_b - 1) >> bm_b_log2;
        for (int j = 0; j < nb; ++j) blk_e_b[b0 + j] = e;
    }
    fill_tail(blk_e_b, n_b >> bm_b_log2, C_b >> bm_b_log2, -1);
    for (int s = tid; s < nseg; s += kAlignThreads) {
        const int e = s / L, a = s - e * L;
        const int b0 = lpos[s] >> bm_l_log2, nb = (cnt[e * L1 + a] + bm_l - 1) >> bm_l_log2;
        for (int j = 0; j < nb; ++j) {
            blk_e_l[b0 + j] = e;
            blk_a_l[b0 + j] = a;
        }
    }
    fill_tail(blk_e_l, n_l >> bm_l_log2, C_l >> bm_l_log2, -1);
    fill_tail(blk_a_l, n_l >> bm_l_log2, C_l >> bm_l_log2, -1);
    if (tid == 0) {
        *n_b_out = n_b;
        *n_l_out = n_l;
    }

    // 4. stable scatter, here or in k_align_scatter
    if (defer) {
        for (int i = tid; i < nr * nkeys; i += kAlignThreads) defer[i] = hist[i];
        for (int i = tid; i < nkeys; i += kAlignThreads) defer[nr * nkeys + i] = bpos[i];
        for (int i = tid; i < nseg; i += kAlignThreads) defer[(nr + 1) * nkeys + i] = lpos[i];
        return;
    }
    for (int r = wave; r < nr; r += kAlignThreads / 64)
        scatter_range(keyf, o, r * R, min(P, (r + 1) * R), hist + r * nkeys, bpos, lpos, L, nbits);
}

// Step 4 for large batches: workgroup r (one wave) scatters range r with the
// offsets computed by k_align, kept in LDS.
__global__ __launch_bounds__(64) void k_align_scatter(AlignKeys keyf, AlignOut o, int T, int nr,
                                                      int R, const int32_t* __restrict__ defer) {
    extern __shared__ int h[];  // [nkeys] running offsets, [nkeys] bpos, [E*L] lpos
    const int E = keyf.E, L = keyf.L, L1 = L + 1, nkeys = E * L1, P = T * keyf.k;
    const int r = blockIdx.x, lane = threadIdx.x;
    int* bpos = h + nkeys;
    int* lpos = bpos + nkeys;
    for (int i = lane; i < nkeys; i += 64) h[i] = defer[r * nkeys + i];
    for (int i = lane; i < nkeys + E * L; i += 64) bpos[i] = defer[nr * nkeys + i];
    __syncthreads();
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;
    scatter_range(keyf, o, r * R, min(P, (r + 1) * R), h, bpos, lpos, L, nbits);
}

// ---------------------------------------------------------------------------
// Alignment for key counts beyond one workgroup's histogram rows (E (L+1) up
// to kAlignMaxKeys, e.g. 256 experts x 128 adapters): the same counting sort,
// spread over four launches so that no single workgroup holds more than one
// int per key in LDS.
//   1. k_align_hist: workgroup r counts the keys of pair range r in LDS and
//      writes its row H[r][key] to the workspace.
//   2. k_align_colscan: one thread per key turns its column of H into
//      exclusive per-range offsets (in place) and the key's total cnt[key].
//   3. k_align_offsets: one workgroup derives the expert totals, both views'
//      segment starts (bpos, lpos: block scans in LDS, one array at a time),
//      the padding sentinels, the tails and the block maps (each expert /
//      segment writes its own blocks, so no search is needed).
//   4. k_align_scatter_g: workgroup r (one wave) scatters range r as in the
//      one-workgroup path, with its running offsets in LDS and the segment
//      starts read from the workspace.
// The result is the same as the one-workgroup path's, bit for bit.
constexpr int kAlignMaxKeys = 36864;   // an int per key in a workgroup's LDS (+ E ints)
constexpr int kAlignMultiMaxRanges = 64;

bool align_fits(int E, int L) {
    return align_max_ranges(E, L) > 0 || static_cast<long>(E) * (L + 1) <= kAlignMaxKeys;
}

// batches of at least this many pairs take the multi-launch path too
constexpr int kAlignMultiMinPairs = 1 << 30;

static bool align_multi(int P, int E, int L) { return align_max_ranges(E, L) <= 0 || P >= kAlignMultiMinPairs; }
bool align_single_workgroup(int P, int E, int L) { return !align_multi(P, E, L); }

// ranges of the multi-workgroup path: at least 256 pairs each, at most 64
static void align_multi_ranges(int P, int* nr, int* R) {
    int n = std::min(kAlignMultiMaxRanges, std::max(1, (P + 255) / 256));
    int r = (P + n - 1) / n;
    r = std::max(64, (r + 63) / 64 * 64);
    *nr = std::max(1, (P + r - 1) / r);
    *R = r;
}

__global__ __launch_bounds__(256) void k_align_hist(AlignKeys keyf, int P, int R, int nkeys,
                                                    int32_t* __restrict__ H) {
    extern __shared__ int hl[];
    const int r = blockIdx.x, tid = threadIdx.x;
    for (int i = tid; i < nkeys; i += 256) hl[i] = 0;
    __syncthreads();
    const int lo = r * R, hi = min(P, lo + R);
    for (int p = lo + tid; p < hi; p += 256) atomicAdd(&hl[keyf(p)], 1);  // order-free: counts only
    __syncthreads();
    int32_t* row = H + static_cast<size_t>(r) * nkeys;
    for (int i = tid; i < nkeys; i += 256) row[i] = hl[i];
}

__global__ __launch_bounds__(256) void k_align_colscan(int32_t* __restrict__ H, int nr, int nkeys,
                                                       int32_t* __restrict__ cnt) {
    const int key = blockIdx.x * 256 + threadIdx.x;
    if (key >= nkeys) return;
    int run = 0;
    for (int r0 = 0; r0 < nr; r0 += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = r0 + u < nr ? H[static_cast<size_t>(r0 + u) * nkeys + key] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (r0 + u < nr) H[static_cast<size_t>(r0 + u) * nkeys + key] = run;
            run += c[u];
        }
    }
    cnt[key] = run;
}

__global__ __launch_bounds__(kAlignThreads) void k_align_offsets(
    int E, int L, int P, int bm_b_log2, int bm_l_log2, int C_b, int C_l, const int32_t* __restrict__ cnt,
    int32_t* __restrict__ bpos, int32_t* __restrict__ lpos, AlignOut o, int32_t* __restrict__ blk_e_b,
    int32_t* __restrict__ n_b_out, int32_t* __restrict__ blk_e_l, int32_t* __restrict__ blk_a_l,
    int32_t* __restrict__ n_l_out) {
    extern __shared__ int lds[];
    const int L1 = L + 1, nkeys = E * L1, nseg = E * L;
    const int bm_b = 1 << bm_b_log2, bm_l = 1 << bm_l_log2;
    int* buf = lds;           // [nkeys] scan buffer: base view, then LoRA view
    int* ne = buf + nkeys;    // [E] pairs per expert
    int* red = ne + E;        // [65]
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kAlignThreads) ne[e] = 0;
    __syncthreads();
    for (int key = tid; key < nkeys; key += kAlignThreads) {
        const int c = cnt[key];
        if (c) atomicAdd(&ne[key / L1], c);
    }
    __syncthreads();

    // base view: keys in (expert, adapter') order, each expert padded after
    // its last key; expert e's blocks start at its first key
    for (int key = tid; key < nkeys; key += kAlignThreads) {
        const int e = key / L1;
        buf[key] = cnt[key] + (key % L1 == L ? ((ne[e] + bm_b - 1) & ~(bm_b - 1)) - ne[e] : 0);
    }
    __syncthreads();
    const int n_b = block_excl_scan(buf, nkeys, red);
    for (int key = tid; key < nkeys; key += kAlignThreads) bpos[key] = buf[key];
    for (int e = tid; e < E; e += kAlignThreads) {
        const int last = e * L1 + L;
        const int base = buf[last] + cnt[last];
        const int np = ((ne[e] + bm_b - 1) & ~(bm_b - 1)) - ne[e];
        for (int i = 0; i < np; ++i) {
            o.sorted_b[base + i] = P;
            if (o.slot_adapter) o.slot_adapter[base + i] = -1;
        }
        const int b0 = buf[e * L1] >> bm_b_log2, nb = (ne[e] + bm_b - 1) >> bm_b_log2;
        for (int i = 0; i < nb; ++i) blk_e_b[b0 + i] = e;
    }
    for (int i = n_b + tid; i < C_b; i += kAlignThreads) {
        o.sorted_b[i] = P;
        if (o.slot_adapter) o.slot_adapter[i] = -1;
    }
    for (int i = (n_b >> bm_b_log2) + tid; i < (C_b >> bm_b_log2); i += kAlignThreads) blk_e_b[i] = -1;
    __syncthreads();  // buf is reused

    // LoRA view: segments (expert, adapter < L), each padded to bm_l
    for (int sg = tid; sg < nseg; sg += kAlignThreads)
        buf[sg] = (cnt[(sg / L) * L1 + sg % L] + bm_l - 1) & ~(bm_l - 1);
    __syncthreads();
    const int n_l = block_excl_scan(buf, nseg, red);
    for (int sg = tid; sg < nseg; sg += kAlignThreads) {
        lpos[sg] = buf[sg];
        const int c = cnt[(sg / L) * L1 + sg % L];
        const int np = ((c + bm_l - 1) & ~(bm_l - 1)) - c;
        for (int i = 0; i < np; ++i) o.sorted_l[buf[sg] + c + i] = P;
        const int b0 = buf[sg] >> bm_l_log2, nb = (c + bm_l - 1) >> bm_l_log2;
        for (int i = 0; i < nb; ++i) {
            blk_e_l[b0 + i] = sg / L;
            blk_a_l[b0 + i] = sg % L;
        }
    }
    for (int i = n_l + tid; i < C_l; i += kAlignThreads) o.sorted_l[i] = P;
    for (int i = (n_l >> bm_l_log2) + tid; i < (C_l >> bm_l_log2); i += kAlignThreads) {
        blk_e_l[i] = -1;
        blk_a_l[i] = -1;
    }
    if (tid == 0) {
        *n_b_out = n_b;
        *n_l_out = n_l;
    }
}

__global__ __launch_bounds__(64) void k_align_scatter_g(AlignKeys keyf, AlignOut o, int P, int R,
                                                        const int32_t* __restrict__ H,
                                                        const int32_t* __restrict__ bpos,
                                                        const int32_t* __restrict__ lpos) {
    extern __shared__ int hr[];  // [nkeys] running offsets of this range
    const int nkeys = keyf.E * (keyf.L + 1);
    const int r = blockIdx.x, lane = threadIdx.x;
    for (int i = lane; i < nkeys; i += 64) hr[i] = H[static_cast<size_t>(r) * nkeys + i];
    __syncthreads();
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;
    scatter_range(keyf, o, r * R, min(P, (r + 1) * R), hr, bpos, lpos, keyf.L, nbits);
}

int align_defer_ints(int P, int E, int L) {
    const int nkeys = E * (L + 1);
    if (!align_multi(P, E, L)) {
        const int maxr = align_max_ranges(E, L);
        return (maxr + 1) * nkeys + E * L;
    }
    int nr, R;
    align_multi_ranges(std::max(P, 1), &nr, &R);
    // H [nr][nkeys], cnt [nkeys], bpos [nkeys], lpos [E L]
    return nr * nkeys + 2 * nkeys + E * L;
}

hipError_t launch_align(const int32_t* topk_ids, const int32_t* adapter_ids, int T, int k,
                        int E, int L, int bm_b, int bm_l, int C_b, int C_l,
                        int32_t* sorted_b, int32_t* blk_e_b, int32_t* n_b,
                        int32_t* sorted_l, int32_t* blk_e_l, int32_t* blk_a_l, int32_t* n_l,
                        int32_t* slot_of_pair, int32_t* lslot_of_pair, int32_t* slot_adapter,
                        int32_t* defer, hipStream_t s) {
    if (!align_fits(E, L)) return hipErrorInvalidValue;
    if ((bm_b & (bm_b - 1)) || (bm_l & (bm_l - 1))) return hipErrorInvalidValue;
    const int P = T * k;
    if (P == 0) return hipSuccess;
    const AlignKeys keyf{topk_ids, adapter_ids, k, E, L};
    const AlignOut o{sorted_b, sorted_l, slot_of_pair, lslot_of_pair, slot_adapter};
    if (align_multi(P, E, L)) {
        if (!defer) return hipErrorInvalidValue;  // the multi-workgroup path needs its workspace
        int nr, R;
        align_multi_ranges(P, &nr, &R);
        const int nkeys = E * (L + 1);
        int32_t* H = defer;
        int32_t* cnt = H + static_cast<size_t>(nr) * nkeys;
        int32_t* bpos = cnt + nkeys;
        int32_t* lpos = bpos + nkeys;
        const size_t lds_keys = sizeof(int) * nkeys;
        const size_t lds_off = sizeof(int) * (nkeys + E + 65);
        // dynamic LDS beyond 64 KiB is opted into per kernel (once)
        static bool lds_raised = false;
        if (!lds_raised) {
            constexpr int kMaxDyn = 160 * 1024;
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_align_hist),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDyn) != hipSuccess ||
                hipFuncSetAttribute(reinterpret_cast<const void*>(k_align_offsets),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDyn) != hipSuccess ||
                hipFuncSetAttribute(reinterpret_cast<const void*>(k_align_scatter_g),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDyn) != hipSuccess)
                return hipErrorInvalidValue;
            lds_raised = true;
        }
        hipLaunchKernelGGL(k_align_hist, dim3(nr), dim3(256), lds_keys, s, keyf, P, R, nkeys, H);
        hipLaunchKernelGGL(k_align_colscan, dim3((nkeys + 255) / 256), dim3(256), 0, s, H, nr, nkeys, cnt);
        hipLaunchKernelGGL(k_align_offsets, dim3(1), dim3(kAlignThreads), lds_off, s, E,
                           L, P, __builtin_ctz(bm_b), __builtin_ctz(bm_l), C_b, C_l, cnt, bpos, lpos, o, blk_e_b,
                           n_b, blk_e_l, blk_a_l, n_l);
        hipLaunchKernelGGL(k_align_scatter_g, dim3(nr), dim3(64), lds_keys, s, keyf, o, P, R, H, bpos, lpos);
        return hipGetLastError();
    }
    int nr, R;
    align_ranges(P, E, L, &nr, &R);
    // one workgroup does everything for small batches; large ones hand the
    // scattered stores to one workgroup per range
    const size_t scatter_lds = sizeof(int) * (2 * E * (L + 1) + E * L);
    if (nr <= kAlignThreads / 64 || scatter_lds > 64 * 1024) defer = nullptr;
    hipLaunchKernelGGL(k_align, dim3(1), dim3(kAlignThreads), 0, s, keyf, o, T, __builtin_ctz(bm_b),
                       __builtin_ctz(bm_l), C_b, C_l, nr, R, blk_e_b, n_b, blk_e_l, blk_a_l, n_l,
                       defer);
    if (defer)
        hipLaunchKernelGGL(k_align_scatter, dim3(nr), dim3(64), scatter_lds, s, keyf, o, T, nr, R,
                           defer);
    return hipGetLastError();
}

}  // namespace moelora
