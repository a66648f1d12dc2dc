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

__global__ __launch_bounds__(256) void k_zero(int32_t* __restrict__ zero_words, int n_zero,
                                              float* __restrict__ zero_out, int T, int H) {
    if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < n_zero) zero_words[threadIdx.x] = 0;
    if (zero_out) {
        const int t0 = blockIdx.x * 4, nt = min(4, T - t0);
        f32x4* o = reinterpret_cast<f32x4*>(zero_out + static_cast<size_t>(t0) * H);
        for (int i = threadIdx.x; i < nt * H / 4; i += 256) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

hipError_t launch_zero(int32_t* zero_words, int n_zero, float* zero_out, int T, int H, hipStream_t s) {
    if (n_zero < 0 || n_zero > 256 || (n_zero > 0 && !zero_words)) return hipErrorInvalidValue;
    if (zero_out && (T <= 0 || H <= 0 || H % 4)) return hipErrorInvalidValue;
    const int blocks = zero_out ? (T + 3) / 4 : 1;
    hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(256), 0, s, zero_words, n_zero, zero_out, T, H);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Align. key(p) = e * (L+1) + a',  a' = adapter if in [0,L) else L.
// The result is a stable counting sort of the pairs by key: within a key the
// pairs keep ascending p. Pairs are cut into contiguous ranges; inside a range
// they are taken in 64-pair steps, and lanes with equal keys in a step are
// found with one ballot per key bit, so a pair's rank among the range's pairs
// of its key is a running per-key count plus a popcount. No result depends on
// the order in which workgroups or atomics run.
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

// range count and range length for P pairs (the one-workgroup kernel)
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

// The alignment without a workspace: one 1024-thread workgroup counts every
// range's keys into its own LDS histogram row (order-free LDS atomics), turns
// the rows into exclusive per-range offsets and the key totals into segment
// starts, writes the padding, the tails and the block maps, and then scatters
// (wave w takes ranges w, w+16, ...).
__global__ __launch_bounds__(kAlignThreads) void k_align(
    AlignKeys keyf, AlignOut o, int T, int bm_b_log2, int bm_l_log2, int C_b, int C_l, int nr,
    int R, int32_t* __restrict__ blk_e_b, int32_t* __restrict__ n_b_out,
    int32_t* __restrict__ blk_e_l, int32_t* __restrict__ blk_a_l, int32_t* __restrict__ n_l_out) {
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
    const int tid = threadIdx.x, wave = wave_id();
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

    // 4. stable scatter
    for (int r = wave; r < nr; r += kAlignThreads / 64)
        scatter_range(keyf, o, r * R, min(P, (r + 1) * R), hist + r * nkeys, bpos, lpos, L, nbits);
}

// ---------------------------------------------------------------------------
// The alignment with a workspace, in two launches (count, then place), or in
// one workgroup for small batches.
//   count: workgroup r (one wave) takes the pairs of range r in 64-pair steps
//     and writes each pair's key and its rank among the range's pairs of that
//     key, and the range's per-key counts as row r of H.
//   place: every workgroup reads all rows of H. The column sums are the key
//     totals, the sums over the rows before r the offsets of range r. From
//     the totals each workgroup derives the same expert totals, base-view
//     expert starts (each expert padded to the block height) and LoRA-view
//     segment starts (each segment padded) in its LDS, scatters the pairs of
//     range r, and writes its share of the padding, block maps and tails.
// Every store of the views lands on a slot that no other store writes, so the
// workgroups need no order among themselves.
constexpr int kPlaceThreads = 1024;
constexpr int kOneThreads = 256;
constexpr int kOneMaxPairs = 64 * (kOneThreads / 64);  // one 64-pair range per wave
constexpr int kPlaceMaxRowInts = 65536;  // ints of H one place workgroup reads

// The derived starts of both views, in LDS.
struct PlaceCtx {
    int E, L, L1, nkeys, nseg, P, bm_b_log2, bm_l_log2, C_b, C_l;
    int* scan1;  // [nkeys + 1] exclusive prefix of the key totals
    int* lscan;  // [nseg + 1]  exclusive prefix of the padded segment sizes
    int* ebase;  // [E + 1]     exclusive prefix of the padded expert sizes
    __device__ __forceinline__ int count_of(int key) const { return scan1[key + 1] - scan1[key]; }
    __device__ __forceinline__ int expert_total(int e) const { return scan1[(e + 1) * L1] - scan1[e * L1]; }
};

struct AlignMaps {
    int32_t* blk_e_b;
    int32_t* n_b;
    int32_t* blk_e_l;
    int32_t* blk_a_l;
    int32_t* n_l;
};

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4 and 8 lanes inside each row of 16, then the last lane of row 0 is
// added into row 1 and that of row 2 into row 3, then lane 31 into rows 2
// and 3. Lanes a move does not reach add 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
    return x;
}

// Exclusive prefix sum of a[0..n) in LDS by one wave (lane l takes a
// contiguous chunk); a[n] receives the total. The wave's own LDS accesses
// stay in program order, so no barrier is needed inside.
__device__ void wave_scan_lds(int* a, int n) {
    const int lane = threadIdx.x & 63;
    const int per = (n + 63) >> 6;
    const int lo = min(n, lane * per), hi = min(n, lo + per);
    int s = 0;
    for (int i = lo; i < hi; ++i) s += a[i];
    const int incl = wave_incl_scan(s);
    int run = incl - s;
    for (int i = lo; i < hi; ++i) {
        const int v = a[i];
        a[i] = run;
        run += v;
    }
    if (lane == 63) a[n] = incl;
}

// Exclusive prefix sums of a[0..na) and b[0..nb) in LDS by all waves of the
// workgroup: each thread sums a contiguous chunk of both, the waves scan the
// chunk sums (DPP), the wave totals are combined through red[2 NW], and each
// thread rewrites its chunks; a[na] and b[nb] receive the totals.
__device__ void block_scan2(int* a, int na, int* b, int nb, int* red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, NT = blockDim.x, NW = NT >> 6;
    const int pa = (na + NT - 1) / NT, pb = (nb + NT - 1) / NT;
    const int a0 = min(na, tid * pa), a1 = min(na, a0 + pa);
    const int b0 = min(nb, tid * pb), b1 = min(nb, b0 + pb);
    int sa = 0, sb = 0;
    for (int i = a0; i < a1; ++i) sa += a[i];
    for (int i = b0; i < b1; ++i) sb += b[i];
    const int ia = wave_incl_scan(sa), ib = wave_incl_scan(sb);
    if (lane == 63) {
        red[wave] = ia;
        red[NW + wave] = ib;
    }
    __syncthreads();
    int xa = 0, xb = 0, ta = 0, tb = 0;
    for (int w = 0; w < NW; ++w) {
        const int ra = red[w], rb = red[NW + w];
        if (w < wave) {
            xa += ra;
            xb += rb;
        }
        ta += ra;
        tb += rb;
    }
    int run = xa + ia - sa;
    for (int i = a0; i < a1; ++i) {
        const int v = a[i];
        a[i] = run;
        run += v;
    }
    run = xb + ib - sb;
    for (int i = b0; i < b1; ++i) {
        const int v = b[i];
        b[i] = run;
        run += v;
    }
    if (tid == 0) {
        a[na] = ta;
        b[nb] = tb;
    }
    __syncthreads();
}

// One wave scans at most this many entries of an array; longer arrays are
// scanned by the whole workgroup.
constexpr int kWaveScanMax = 512;

// scan1[0..nkeys) holds the key totals and lscan[0..nseg) the padded segment
// sizes: both become exclusive prefixes, then ebase the expert starts. Short
// arrays: wave 0 scans scan1 and then derives ebase while wave 1 scans lscan
// (one barrier); long ones: the whole workgroup scans both, then ebase.
// red: 2 (blockDim.x / 64) ints.
__device__ void place_scans(const PlaceCtx& c, int* red) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int bm_b = 1 << c.bm_b_log2;
    if (c.nkeys <= kWaveScanMax && c.nseg <= kWaveScanMax) {
        if (wave == 0) {
            wave_scan_lds(c.scan1, c.nkeys);
            for (int e = lane; e < c.E; e += 64) c.ebase[e] = (c.expert_total(e) + bm_b - 1) & ~(bm_b - 1);
            wave_scan_lds(c.ebase, c.E);
        } else if (wave == 1) {
            wave_scan_lds(c.lscan, c.nseg);
        }
        __syncthreads();
        return;
    }
    block_scan2(c.scan1, c.nkeys, c.lscan, c.nseg, red);
    for (int e = threadIdx.x; e < c.E; e += blockDim.x)
        c.ebase[e] = (c.expert_total(e) + bm_b - 1) & ~(bm_b - 1);
    __syncthreads();
    if (wave == 0) wave_scan_lds(c.ebase, c.E);
    __syncthreads();
}

// Slot of pair p in both views; `within` = its rank among all pairs of its key.
__device__ __forceinline__ void place_pair(const PlaceCtx& c, const AlignOut& o, int p, int key, int within) {
    const int e = key / c.L1, a = key - e * c.L1;
    const int slot = c.ebase[e] + c.scan1[key] - c.scan1[e * c.L1] + within;
    o.sorted_b[slot] = p;
    if (o.slot_of_pair) o.slot_of_pair[p] = slot;
    if (o.slot_adapter) o.slot_adapter[slot] = a < c.L ? a : -1;
    int lslot = -1;
    if (a < c.L) {
        lslot = c.lscan[e * c.L + a] + within;
        o.sorted_l[lslot] = p;
    }
    if (o.lslot_of_pair) o.lslot_of_pair[p] = lslot;
}

// Padding slots and block-map entries of a share of the experts and segments:
// wave gw of GW takes a contiguous run of each. A lane looks up one expert or
// segment; the wave then writes the entries of each non-empty one in turn,
// consecutive lanes on consecutive slots. Segments of short blocks (at most
// 2^kLanePadLog2 rows) instead write their few entries lane by lane, which
// takes fewer store instructions.
constexpr int kLanePadLog2 = 4;
__device__ void place_pads(const PlaceCtx& c, const AlignOut& o, const AlignMaps& mp, int gw, int GW) {
    const int lane = threadIdx.x & 63;
    const int lb = c.bm_b_log2, ll = c.bm_l_log2;
    const int per_e = (c.E + GW - 1) / GW;
    const int e_end = min(c.E, (gw + 1) * per_e);
    for (int base = gw * per_e; base < e_end; base += 64) {
        const int e = base + lane;
        int lo = 0, hi = 0, n = 0;
        if (e < e_end) {
            lo = c.ebase[e];
            hi = c.ebase[e + 1];
            n = c.expert_total(e);
        }
        uint64_t act = ballot64(n > 0);
        while (act) {
            const int j = __ffsll(static_cast<long long>(act)) - 1;
            act &= act - 1;
            const int ej = base + j;
            const int loj = __builtin_amdgcn_readlane(lo, j), hij = __builtin_amdgcn_readlane(hi, j);
            const int nj = __builtin_amdgcn_readlane(n, j);
            for (int i = loj + nj + lane; i < hij; i += 64) {
                o.sorted_b[i] = c.P;
                if (o.slot_adapter) o.slot_adapter[i] = -1;
            }
            for (int b = (loj >> lb) + lane; b < (hij >> lb); b += 64) mp.blk_e_b[b] = ej;
        }
    }
    const int per_s = (c.nseg + GW - 1) / GW;
    const int s_end = min(c.nseg, (gw + 1) * per_s);
    if (ll <= kLanePadLog2) {
        // short blocks: each lane writes its own segment's few entries
        for (int s = gw * per_s + lane; s < s_end; s += 64) {
            const int e = s / c.L, a = s - e * c.L;
            const int lo = c.lscan[s], hi = c.lscan[s + 1], n = c.count_of(e * c.L1 + a);
            for (int i = lo + n; i < hi; ++i) o.sorted_l[i] = c.P;
            for (int b = lo >> ll; b < (hi >> ll); ++b) {
                mp.blk_e_l[b] = e;
                mp.blk_a_l[b] = a;
            }
        }
        return;
    }
    for (int base = gw * per_s; base < s_end; base += 64) {
        const int s = base + lane;
        int lo = 0, hi = 0, n = 0;
        if (s < s_end) {
            const int e = s / c.L;
            lo = c.lscan[s];
            hi = c.lscan[s + 1];
            n = c.count_of(e * c.L1 + (s - e * c.L));
        }
        uint64_t act = ballot64(n > 0);
        while (act) {
            const int j = __ffsll(static_cast<long long>(act)) - 1;
            act &= act - 1;
            const int sj = base + j, ej = sj / c.L, aj = sj - ej * c.L;
            const int loj = __builtin_amdgcn_readlane(lo, j), hij = __builtin_amdgcn_readlane(hi, j);
            const int nj = __builtin_amdgcn_readlane(n, j);
            for (int i = loj + nj + lane; i < hij; i += 64) o.sorted_l[i] = c.P;
            for (int b = (loj >> ll) + lane; b < (hij >> ll); b += 64) {
                mp.blk_e_l[b] = ej;
                mp.blk_a_l[b] = aj;
            }
        }
    }
}

// piece r of nr of a[from .. to) = v (pieces of a multiple of 4 entries)
__device__ __forceinline__ void fill_piece(int32_t* a, int from, int to, int v, int r, int nr) {
    const int len = to - from;
    if (len <= 0) return;
    const int chunk = ((len + nr - 1) / nr + 3) & ~3;
    const int f = from + r * chunk, t = min(to, f + chunk);
    if (f < t) fill_tail(a, f, t, v);
}

// piece r of nr of the tails past n_b and n_l (views and block maps)
__device__ void place_tails(const PlaceCtx& c, const AlignOut& o, const AlignMaps& mp, int r, int nr) {
    const int n_b = c.ebase[c.E], n_l = c.lscan[c.nseg];
    fill_piece(o.sorted_b, n_b, c.C_b, c.P, r, nr);
    if (o.slot_adapter) fill_piece(o.slot_adapter, n_b, c.C_b, -1, r, nr);
    fill_piece(o.sorted_l, n_l, c.C_l, c.P, r, nr);
    fill_piece(mp.blk_e_b, n_b >> c.bm_b_log2, c.C_b >> c.bm_b_log2, -1, r, nr);
    fill_piece(mp.blk_e_l, n_l >> c.bm_l_log2, c.C_l >> c.bm_l_log2, -1, r, nr);
    fill_piece(mp.blk_a_l, n_l >> c.bm_l_log2, c.C_l >> c.bm_l_log2, -1, r, nr);
}

__device__ __forceinline__ PlaceCtx place_ctx(int* lds, int E, int L, int P, int bm_b_log2, int bm_l_log2,
                                              int C_b, int C_l) {
    PlaceCtx c;
    c.E = E;
    c.L = L;
    c.L1 = L + 1;
    c.nkeys = E * c.L1;
    c.nseg = E * L;
    c.P = P;
    c.bm_b_log2 = bm_b_log2;
    c.bm_l_log2 = bm_l_log2;
    c.C_b = C_b;
    c.C_l = C_l;
    c.scan1 = lds;
    c.lscan = c.scan1 + c.nkeys + 1;
    c.ebase = c.lscan + c.nseg + 1;
    return c;
}
__host__ __device__ __forceinline__ int place_ctx_ints(int E, int L) { return E * (L + 1) + 1 + E * L + 1 + E + 1; }

// Count: workgroup r (one wave), pairs [r R, min(P, (r+1) R)); h = the
// range's running per-key counts (LDS, hp ints: the key count rounded up to
// a multiple of 4, the row pitch of H).
constexpr int kCountBatch = 8;  // 64-pair steps whose key loads are in flight together

__global__ __launch_bounds__(64) void k_align_count(AlignKeys keyf, int P, int R, int hp, int32_t* __restrict__ H,
                                                    int32_t* __restrict__ kk, int32_t* __restrict__ kpos) {
    extern __shared__ __align__(16) int h[];
    const int nkeys = keyf.E * (keyf.L + 1);
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;
    const int r = blockIdx.x, lane = threadIdx.x;
    const int lo = r * R, hi = min(P, lo + R);
    const uint64_t below = lanemask_lt();
    for (int i = lane; i < (hp >> 2); i += 64) reinterpret_cast<int4*>(h)[i] = int4{0, 0, 0, 0};
    __syncthreads();
    for (int base = lo; base < hi; base += 64 * kCountBatch) {
        int keys[kCountBatch];
#pragma unroll
        for (int c = 0; c < kCountBatch; ++c) keys[c] = keyf(min(base + 64 * c + lane, hi - 1));
#pragma unroll
        for (int c = 0; c < kCountBatch; ++c) {
            if (base + 64 * c >= hi) break;
            const int p = base + 64 * c + lane;
            const bool valid = p < hi;
            const int key = valid ? keys[c] : 0;
            const uint64_t m = match_key(key, valid, nbits);
            // all lanes read the running count before the lowest lane of each
            // key advances it (one wave: LDS accesses stay in program order)
            const int off = valid ? h[key] : 0;
            if (valid && lane == __ffsll(static_cast<long long>(m)) - 1) h[key] = off + popc64(m);
            if (valid) {
                kk[p] = key;
                kpos[p] = off + popc64(m & below);
            }
        }
    }
    __syncthreads();
    int4* row = reinterpret_cast<int4*>(H + static_cast<size_t>(r) * hp);
    for (int i = lane; i < (hp >> 2); i += 64) row[i] = reinterpret_cast<const int4*>(h)[i];
}

// Place: workgroup r of nr (see above). LDS: the PlaceCtx arrays, ex[hp]
// (offsets of range r per key), red[2 NW].
__global__ __launch_bounds__(kPlaceThreads) void k_align_place(
    int E, int L, int P, int bm_b_log2, int bm_l_log2, int C_b, int C_l, int nr, int R, int hp,
    const int32_t* __restrict__ H, const int32_t* __restrict__ kk, const int32_t* __restrict__ kpos,
    AlignOut o, AlignMaps mp) {
    extern __shared__ int lds[];
    constexpr int NT = kPlaceThreads, NW = NT / 64;
    const PlaceCtx c = place_ctx(lds, E, L, P, bm_b_log2, bm_l_log2, C_b, C_l);
    int* ex = c.ebase + E + 1;
    int* red = ex + hp;
    const int r = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
    const int lo = r * R, hi = min(P, lo + R);
    // the first pair of each thread, in flight during the column pass
    int key0 = 0, pos0 = 0;
    if (lo + tid < hi) {
        key0 = kk[lo + tid];
        pos0 = kpos[lo + tid];
    }
    for (int i = tid; i < c.nkeys; i += NT) {
        c.scan1[i] = 0;
        ex[i] = 0;
    }
    __syncthreads();

    // column sums of H: thread (quad q, group g) adds rows g, g+G, ... of
    // keys 4q..4q+3 (16 rows in flight), then adds into LDS
    const int nq = hp >> 2;
    const int G = nq >= NT ? 1 : NT / nq;
    for (int it = tid; it < nq * G; it += NT) {
        const int q = it % nq, g = it / nq;
        int tot[4] = {0, 0, 0, 0}, exs[4] = {0, 0, 0, 0};
        for (int r0 = g; r0 < nr; r0 += 16 * G) {
            int4 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int rr = r0 + u * G;
                v[u] = rr < nr ? *reinterpret_cast<const int4*>(H + static_cast<size_t>(rr) * hp + 4 * q)
                               : int4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int rr = r0 + u * G;
                const int w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    tot[i] += w[i];
                    if (rr < r) exs[i] += w[i];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 4 * q + i;
            if (key < c.nkeys) {
                if (tot[i]) atomicAdd(&c.scan1[key], tot[i]);
                if (exs[i]) atomicAdd(&ex[key], exs[i]);
            }
        }
    }
    __syncthreads();
    const int bm_l = 1 << bm_l_log2;
    for (int s = tid; s < c.nseg; s += NT) {
        const int e = s / L;
        c.lscan[s] = (c.scan1[e * c.L1 + (s - e * L)] + bm_l - 1) & ~(bm_l - 1);
    }
    __syncthreads();
    place_scans(c, red);

    for (int p = lo + tid; p < hi; p += NT) {
        const int key = p == lo + tid ? key0 : kk[p];
        const int pos = p == lo + tid ? pos0 : kpos[p];
        place_pair(c, o, p, key, ex[key] + pos);
    }
    place_pads(c, o, mp, r * NW + wave, nr * NW);
    place_tails(c, o, mp, r, nr);
    if (r == 0 && tid == 0) {
        *mp.n_b = c.ebase[E];
        *mp.n_l = c.lscan[c.nseg];
    }
}

// The views of k_align_one in LDS, each at a 16-byte aligned offset.
struct OneViews {
    int *vb, *va, *vl, *mb, *mel, *mal, *end;
};
__host__ __device__ __forceinline__ int round4(int n) { return (n + 3) & ~3; }
__device__ __forceinline__ OneViews one_views(int* base, int C_b, int C_l, int nbb, int nbl) {
    OneViews v;
    v.vb = base;
    v.va = v.vb + round4(C_b);
    v.vl = v.va + round4(C_b);
    v.mb = v.vl + round4(C_l);
    v.mel = v.mb + round4(nbb);
    v.mal = v.mel + round4(nbl);
    v.end = v.mal + round4(nbl);
    return v;
}
static int one_lds_ints(int E, int L, int P, int C_b, int C_l, int lb, int ll) {
    const int nbb = C_b >> lb, nbl = C_l >> ll;
    return round4(place_ctx_ints(E, L)) + 2 * round4(C_b) + round4(C_l) + round4(nbb) + 2 * round4(nbl) +
           ((P + 63) / 64) * E * (L + 1) + 2 * (kOneThreads / 64);
}

// a[0..n) = v in LDS (a 16-byte aligned), by the whole workgroup
__device__ __forceinline__ void fill_lds(int* a, int n, int v) {
    const int4 q{v, v, v, v};
    for (int i = threadIdx.x; i < (n >> 2); i += blockDim.x) reinterpret_cast<int4*>(a)[i] = q;
    for (int i = (n & ~3) + threadIdx.x; i < n; i += blockDim.x) a[i] = v;
}

// dst[0..n) = src[0..n) from LDS (16-byte aligned) to global memory; 16-byte
// stores where dst is 16-byte aligned
__device__ __forceinline__ void copy_out(int32_t* dst, const int* src, int n) {
    int from = 0;
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        for (int i = threadIdx.x; i < (n >> 2); i += blockDim.x)
            reinterpret_cast<int4*>(dst)[i] = reinterpret_cast<const int4*>(src)[i];
        from = n & ~3;
    }
    for (int i = from + threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
}

// Both halves in one workgroup for P <= kOneMaxPairs: wave w counts range w
// (64 pairs) with its row of H in LDS. The views and block maps are built in
// LDS (filled with their padding values, then the pairs and block entries
// written in), then copied out with contiguous stores, so that the few
// global stores carry whole lines.
__global__ __launch_bounds__(kOneThreads) void k_align_one(AlignKeys keyf, int P, int bm_b_log2, int bm_l_log2,
                                                           int C_b, int C_l, AlignOut o, AlignMaps mp) {
    extern __shared__ __align__(16) int lds[];
    constexpr int NT = kOneThreads;
    const int E = keyf.E, L = keyf.L;
    const PlaceCtx c = place_ctx(lds, E, L, P, bm_b_log2, bm_l_log2, C_b, C_l);
    const int nkeys = c.nkeys, nr = (P + 63) >> 6;
    const int nbb = C_b >> bm_b_log2, nbl = C_l >> bm_l_log2;
    const OneViews v = one_views(lds + round4(place_ctx_ints(E, L)), C_b, C_l, nbb, nbl);
    int* Hl = v.end;  // [nr][nkeys]
    int* red = Hl + nr * nkeys;  // [2 NW]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nbits = nkeys > 1 ? 32 - __clz(nkeys - 1) : 0;

    // 1. wave w counts range w: the rank of each pair among the range's
    // pairs of its key, and the range's count per key (row w, written by the
    // lowest lane of each key after the wave has zeroed the row); meanwhile
    // every thread fills the views with their padding values
    const int p = wave * 64 + lane;
    int key = 0, pos = 0;
    const bool mine = wave < nr;
    const bool valid = mine && p < P;
    if (mine) {
        const int kv = keyf(min(p, P - 1));
        int* h = Hl + wave * nkeys;
        for (int i = lane; i < nkeys; i += 64) h[i] = 0;
        key = valid ? kv : 0;
        const uint64_t m = match_key(key, valid, nbits);
        if (valid && lane == __ffsll(static_cast<long long>(m)) - 1) h[key] = popc64(m);
        pos = popc64(m & lanemask_lt());
    }
    fill_lds(v.vb, C_b, P);
    if (o.slot_adapter) fill_lds(v.va, C_b, -1);
    fill_lds(v.vl, C_l, P);
    fill_lds(v.mb, nbb, -1);
    fill_lds(v.mel, nbl, -1);
    fill_lds(v.mal, nbl, -1);
    __syncthreads();

    // 2. rows -> exclusive per-range offsets; key totals; padded segment sizes
    const int bm_l = 1 << bm_l_log2;
    for (int k2 = tid; k2 < nkeys; k2 += NT) {
        int run = 0;
        for (int rr = 0; rr < nr; ++rr) {
            const int x = Hl[rr * nkeys + k2];
            Hl[rr * nkeys + k2] = run;
            run += x;
        }
        c.scan1[k2] = run;
        const int e = k2 / c.L1, a = k2 - e * c.L1;
        if (a < L) c.lscan[e * L + a] = (run + bm_l - 1) & ~(bm_l - 1);
    }
    __syncthreads();
    place_scans(c, red);

    // 3. pairs and block entries into the LDS views
    if (valid) {
        const int within = Hl[wave * nkeys + key] + pos;
        const int e = key / c.L1, a = key - e * c.L1;
        const int slot = c.ebase[e] + c.scan1[key] - c.scan1[e * c.L1] + within;
        v.vb[slot] = p;
        if (o.slot_adapter) v.va[slot] = a < L ? a : -1;
        if (o.slot_of_pair) o.slot_of_pair[p] = slot;
        int lslot = -1;
        if (a < L) {
            lslot = c.lscan[e * L + a] + within;
            v.vl[lslot] = p;
        }
        if (o.lslot_of_pair) o.lslot_of_pair[p] = lslot;
    }
    for (int e = tid; e < E; e += NT)
        for (int b = c.ebase[e] >> bm_b_log2; b < (c.ebase[e + 1] >> bm_b_log2); ++b) v.mb[b] = e;
    for (int s = tid; s < c.nseg; s += NT) {
        const int e = s / L, a = s - e * L;
        for (int b = c.lscan[s] >> bm_l_log2; b < (c.lscan[s + 1] >> bm_l_log2); ++b) {
            v.mel[b] = e;
            v.mal[b] = a;
        }
    }
    __syncthreads();

    // 4. copy out
    copy_out(o.sorted_b, v.vb, C_b);
    if (o.slot_adapter) copy_out(o.slot_adapter, v.va, C_b);
    copy_out(o.sorted_l, v.vl, C_l);
    copy_out(mp.blk_e_b, v.mb, nbb);
    copy_out(mp.blk_e_l, v.mel, nbl);
    copy_out(mp.blk_a_l, v.mal, nbl);
    if (tid == 0) {
        *mp.n_b = c.ebase[E];
        *mp.n_l = c.lscan[c.nseg];
    }
}

// ranges of the two-launch path: 64 S pairs each (S a power of two, at least
// 4), few enough that the rows of H a place workgroup reads stay within
// kPlaceMaxRowInts
static void align2_ranges(int P, int hp, int* nr, int* R) {
    long S = 4;
    for (;;) {
        const long n = (P + 64 * S - 1) / (64 * S);
        if (n * hp <= kPlaceMaxRowInts || n == 1) {
            *nr = static_cast<int>(n);
            *R = static_cast<int>(64 * S);
            return;
        }
        S *= 2;
    }
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
        // H [nr][hp], then each pair's key and rank
        const int hp = (nkeys + 3) & ~3;
        int nr, R;
        align2_ranges(std::max(P, 1), hp, &nr, &R);
        return nr * hp + 2 * std::max(P, 1);
    }
    int nr, R;
    align_multi_ranges(std::max(P, 1), &nr, &R);
    // H [nr][nkeys], cnt [nkeys], bpos [nkeys], lpos [E L]
    return nr * nkeys + 2 * nkeys + E * L;
}

// dynamic LDS beyond 64 KiB is opted into per kernel (once)
static bool raise_align_lds() {
    static bool raised = false;
    if (raised) return true;
    constexpr int kMaxDyn = 160 * 1024;
    const void* fns[] = {reinterpret_cast<const void*>(k_align_hist), reinterpret_cast<const void*>(k_align_offsets),
                         reinterpret_cast<const void*>(k_align_scatter_g),
                         reinterpret_cast<const void*>(k_align_count), reinterpret_cast<const void*>(k_align_place),
                         reinterpret_cast<const void*>(k_align_one)};
    for (const void* f : fns)
        if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDyn) != hipSuccess) return false;
    raised = true;
    return true;
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
    if (!raise_align_lds()) return hipErrorInvalidValue;
    const AlignKeys keyf{topk_ids, adapter_ids, k, E, L};
    const AlignOut o{sorted_b, sorted_l, slot_of_pair, lslot_of_pair, slot_adapter};
    const int lb = __builtin_ctz(bm_b), ll = __builtin_ctz(bm_l);
    const int nkeys = E * (L + 1);
    if (align_multi(P, E, L)) {
        if (!defer) return hipErrorInvalidValue;  // the multi-workgroup path needs its workspace
        int nr, R;
        align_multi_ranges(P, &nr, &R);
        int32_t* H = defer;
        int32_t* cnt = H + static_cast<size_t>(nr) * nkeys;
        int32_t* bpos = cnt + nkeys;
        int32_t* lpos = bpos + nkeys;
        const size_t lds_keys = sizeof(int) * nkeys;
        const size_t lds_off = sizeof(int) * (nkeys + E + 65);
        hipLaunchKernelGGL(k_align_hist, dim3(nr), dim3(256), lds_keys, s, keyf, P, R, nkeys, H);
        hipLaunchKernelGGL(k_align_colscan, dim3((nkeys + 255) / 256), dim3(256), 0, s, H, nr, nkeys, cnt);
        hipLaunchKernelGGL(k_align_offsets, dim3(1), dim3(kAlignThreads), lds_off, s, E,
                           L, P, lb, ll, C_b, C_l, cnt, bpos, lpos, o, blk_e_b,
                           n_b, blk_e_l, blk_a_l, n_l);
        hipLaunchKernelGGL(k_align_scatter_g, dim3(nr), dim3(64), lds_keys, s, keyf, o, P, R, H, bpos, lpos);
        return hipGetLastError();
    }
    if (!defer) {
        // no workspace: the one-workgroup kernel with its LDS histograms
        int nr, R;
        align_ranges(P, E, L, &nr, &R);
        hipLaunchKernelGGL(k_align, dim3(1), dim3(kAlignThreads), 0, s, keyf, o, T, lb, ll, C_b, C_l, nr, R,
                           blk_e_b, n_b, blk_e_l, blk_a_l, n_l);
        return hipGetLastError();
    }
    const AlignMaps mp{blk_e_b, n_b, blk_e_l, blk_a_l, n_l};
    const int hp = (nkeys + 3) & ~3;
    const size_t ctx_bytes = sizeof(int) * place_ctx_ints(E, L);
    const size_t one_bytes = sizeof(int) * static_cast<size_t>(one_lds_ints(E, L, P, C_b, C_l, lb, ll));
    if (P <= kOneMaxPairs && one_bytes <= sizeof(int) * kAlignLdsInts) {
        hipLaunchKernelGGL(k_align_one, dim3(1), dim3(kOneThreads), one_bytes, s, keyf, P, lb, ll, C_b, C_l, o, mp);
        return hipGetLastError();
    }
    int nr, R;
    align2_ranges(P, hp, &nr, &R);
    int32_t* H = defer;
    int32_t* kk = H + static_cast<size_t>(nr) * hp;
    int32_t* kpos = kk + P;
    const size_t place_bytes = ctx_bytes + sizeof(int) * (hp + 2 * (kPlaceThreads / 64));
    if (place_bytes > 160 * 1024) return hipErrorInvalidValue;  // not reached: the key limit above is lower
    hipLaunchKernelGGL(k_align_count, dim3(nr), dim3(64), sizeof(int) * hp, s, keyf, P, R, hp, H, kk, kpos);
    hipLaunchKernelGGL(k_align_place, dim3(nr), dim3(kPlaceThreads), place_bytes, s, E, L, P, lb, ll, C_b, C_l,
                       nr, R, hp, H, kk, kpos, o, mp);
    return hipGetLastError();
}

}  // namespace moelora
