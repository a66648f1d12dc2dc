// Routing and alignment of a decode-sized batch, computed by one wave from
// the logits and adapter ids. The waves of the gate_up launch derive the rows
// they work on this way, so that the launch streams weights from its first
// cycle instead of waiting behind separate routing and alignment launches;
// one wave of the same launch writes the routing and both alignment views
// for the launches that follow.
//
// Everything follows the routing and alignment kernels bit for bit:
//   - top-k of each token's logits, larger value first, lower expert id on
//     ties; weights = softmax over the picks, summed in the routing kernel's
//     butterfly order (AWS ML Blog post "Efficiently serve dozens of
//     fine-tuned models with vLLM on Amazon SageMaker AI and Amazon Bedrock",
//     section "Implementing multi-LoRA inference for MoE models in vLLM");
//   - pairs p = t k + j ordered by (expert, adapter', p), adapter' = L for no
//     adapter; base view padded per expert to 16 rows, LoRA view per
//     (expert, adapter) segment to 16 rows (same post, section "Tuning kernel
//     configurations for Amazon SageMaker AI and Amazon Bedrock").
// Limits: T <= 16 tokens, E <= 32 experts, k <= 8 and P = T k <= 64, so that
// one lane holds one token or one pair, an expert is picked at most once per
// token (at most 16 pairs: one 16-row base block) and a segment has at most
// 16 pairs (one 16-row LoRA block).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moelora {

constexpr int kLocalMaxT = 16;
constexpr int kLocalMaxE = 32;
constexpr int kLocalMaxK = 8;
constexpr int kLocalMaxP = 64;

// Whether a batch fits the wave-local routing (host check as well).
__host__ __device__ __forceinline__ bool local_route_fits(int T, int E, int k) {
    return T >= 1 && T <= kLocalMaxT && E >= 1 && E <= kLocalMaxE && k >= 1 && k <= kLocalMaxK && k <= E &&
           T * k <= kLocalMaxP;
}

// Lanes among `live` whose key x (nbits bits) is below this lane's, and those
// equal to it: one ballot per key bit, from the top bit down.
__device__ __forceinline__ void rank_by_bits(int x, uint64_t live, int nbits, int& below, uint64_t& equal) {
    uint64_t same = live;  // lanes whose bits above b equal this lane's
    int lt = 0;
#pragma unroll 1
    for (int b = nbits - 1; b >= 0; --b) {
        const uint64_t set = ballot64((x >> b) & 1);
        if ((x >> b) & 1) {
            lt += popc64(same & ~set);
            same &= set;
        } else {
            same &= ~set;
        }
    }
    below = lt;
    equal = same & live;
}

__device__ __forceinline__ int bits_for(int n) { return n > 1 ? 32 - __clz(n - 1) : 0; }

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4 and 8 lanes inside each row of 16, then the last lane of row 0 is
// added into row 1 and that of row 2 into row 3, then lane 31 into rows 2
// and 3. Lanes a move does not reach add 0.
__device__ __forceinline__ int wave_prefix(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
    return x;
}

// Token lane t < T: the picks of token t, in order (pid[j], value pv[j]),
// as a bit mask over experts, and the token's adapter' (L = none). The logits
// [T][E] go through ls (LDS, T E floats): each lane loads a few, then token
// lanes read their row. The selection scans the experts in id order: the
// first candidate is taken, then only strictly larger values replace it.
struct TokenPicks {
    int pid[kLocalMaxK];
    float pv[kLocalMaxK];
    uint32_t mask;
    int ad;
};
__device__ __forceinline__ TokenPicks local_picks(const float* __restrict__ logits,
                                                  const int32_t* __restrict__ adapter_ids, int T, int E, int k,
                                                  int L, float* ls, const int32_t* __restrict__ ids) {
    const int lane = threadIdx.x & 63;
    if (ids) {
        // the routing launch already picked: read them (no values needed)
        const int t = min(lane, T - 1);
        TokenPicks tp;
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < kLocalMaxK; ++j) {
            tp.pid[j] = j < k ? min(max(ids[t * k + j], 0), E - 1) : -1;
            tp.pv[j] = 0.0f;
            if (j < k) m |= 1u << tp.pid[j];
        }
        tp.mask = lane < T ? m : 0u;
        const int ad = adapter_ids[t];
        tp.ad = (ad < 0 || ad >= L) ? L : ad;
        return tp;
    }
    const int n = T * E;
    for (int i = lane; i < n; i += 64) ls[i] = logits[i];
    __syncthreads();
    const int t = min(lane, T - 1);
    const float* lrow = ls + t * E;
    TokenPicks tp;
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < kLocalMaxK; ++j) {
        int bi = -1;
        float bv = 0.0f;
        if (j < k) {
#pragma unroll 4
            for (int i = 0; i < E; ++i) {
                const float x = lrow[i];
                if (!((taken >> i) & 1u) && (bi < 0 || x > bv)) {
                    bv = x;
                    bi = i;
                }
            }
            taken |= 1u << bi;
        }
        tp.pid[j] = bi;
        tp.pv[j] = bv;
    }
    tp.mask = lane < T ? taken : 0u;
    const int ad = adapter_ids[t];
    tp.ad = (ad < 0 || ad >= L) ? L : ad;
    return tp;
}

// Expert lane e' < E: its pair count over the tokens' masks; returns the
// exclusive prefix of the padded (to 16) counts, their total in n_b.
__device__ __forceinline__ int local_expert_starts(uint32_t mask, int T, int E, int& count, int& n_b) {
    const int lane = threadIdx.x & 63;
    int c = 0;
#pragma unroll 1
    for (int q = 0; q < T; ++q) c += (__builtin_amdgcn_readlane(static_cast<int>(mask), q) >> (lane & 31)) & 1;
    count = lane < E ? c : 0;
    const int pad = (count + 15) & ~15;
    const int incl = wave_prefix(pad);
    n_b = __builtin_amdgcn_readlane(incl, 63);
    return incl - pad;
}

// Token lane t: the experts for which t is the first token (in t order) of
// its (expert, adapter) segment (none without an adapter).
__device__ __forceinline__ uint32_t local_segment_firsts(const TokenPicks& tp, int T, int L) {
    const int lane = threadIdx.x & 63;
    uint32_t prev = 0;
#pragma unroll 1
    for (int q = 0; q < T; ++q) {
        const uint32_t mq = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(tp.mask), q));
        const int aq = __builtin_amdgcn_readlane(tp.ad, q);
        if (q < lane && aq == tp.ad) prev |= mq;
    }
    return (lane < T && tp.ad < L) ? (tp.mask & ~prev) : 0u;
}

// Token lane t and expert e (wave-uniform): whether t chose e, the pick
// position of e, and t's row in e's base block (order (adapter', t)).
__device__ __forceinline__ int local_row_in_expert(const TokenPicks& tp, int e, int L, bool& in_e, int& j_of_e) {
    const int lane = threadIdx.x & 63;
    in_e = (tp.mask >> e) & 1u;
    j_of_e = 0;
#pragma unroll
    for (int j = 0; j < kLocalMaxK; ++j)
        if (tp.pid[j] == e) j_of_e = j;
    int below;
    uint64_t eq;
    rank_by_bits(tp.ad * kLocalMaxT + (lane & (kLocalMaxT - 1)), ballot64(in_e), bits_for((L + 1) * kLocalMaxT),
                 below, eq);
    return below;
}

// OR of x over the 64 lanes of a wave (DPP moves as in wave_prefix).
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
    int v = static_cast<int>(x);
    v |= __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v |= __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v |= __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v |= __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v |= __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v |= __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 63));
}

// A gate_up projection wave on expert e (wave-uniform) whose 16 MFMA rows
// are the batch's tokens (row r = token r): lane l learns whether token l & 15
// chose e, that pair's slot in e's base block and the token's adapter'.
// Returns false when no token chose e. The activation loads do not wait for
// this: the routing only decides which rows are stored, and where.
__device__ __forceinline__ bool local_token_rows(const float* logits, const int32_t* adapter_ids, int T, int E,
                                                 int k, int L, int e, float* ls, const int32_t* ids, bool& in_row,
                                                 int& slot, int& ad) {
    const TokenPicks tp = local_picks(logits, adapter_ids, T, E, k, L, ls, ids);
    const uint32_t used = wave_or(tp.mask);
    in_row = false;
    slot = 0;
    ad = L;
    if (!((used >> e) & 1u)) return false;
    const int ebase = 16 * __popc(used & ((1u << e) - 1u));
    bool in_e;
    int j_of_e;
    const int row = local_row_in_expert(tp, e, L, in_e, j_of_e);
    const int src = threadIdx.x & 15;
    in_row = __shfl(in_e ? 1 : 0, src) != 0;  // tokens >= T have an empty mask
    slot = ebase + __shfl(row, src);
    ad = __shfl(tp.ad, src);
    return true;
}

// LoRA-view block bl (wave-uniform): false past the used blocks; else its
// expert and adapter, and lane l gets the pair in row l & 15 (-1: padding)
// and that pair's base-view slot.
__device__ __forceinline__ bool local_lora_rows(const float* logits, const int32_t* adapter_ids, int T, int E,
                                                int k, int L, int bl, float* ls, const int32_t* ids, int& e, int& ad,
                                                int& row_p, int& row_slot) {
    const int lane = threadIdx.x & 63;
    const TokenPicks tp = local_picks(logits, adapter_ids, T, E, k, L, ls, ids);
    int cnt, n_b;
    const int ebase_lane = local_expert_starts(tp.mask, T, E, cnt, n_b);
    const uint32_t firsts = local_segment_firsts(tp, T, L);
    // segments per expert lane e' and their prefix: block bl lies in expert e
    int segs = 0;
#pragma unroll 1
    for (int q = 0; q < T; ++q)
        segs += (__builtin_amdgcn_readlane(static_cast<int>(firsts), q) >> (lane & 31)) & 1;
    if (lane >= E) segs = 0;
    const int incl = wave_prefix(segs);
    const uint64_t hit = ballot64(lane < E && incl - segs <= bl && bl < incl);
    row_p = -1;
    row_slot = 0;
    if (hit == 0) return false;
    e = __ffsll(static_cast<long long>(hit)) - 1;
    const int r_in = bl - __builtin_amdgcn_readlane(incl - segs, e);
    // its adapter: the r_in-th smallest among e's segment-first tokens
    const bool first_e = (firsts >> e) & 1u;
    int below;
    uint64_t eq;
    rank_by_bits(tp.ad, ballot64(first_e), bits_for(L + 1), below, eq);
    const uint64_t who = ballot64(first_e && below == r_in);
    ad = __builtin_amdgcn_readlane(tp.ad, __ffsll(static_cast<long long>(who)) - 1);
    // rows: the tokens that chose e with adapter ad, in t order; their slots
    // from their rows in e's base block
    bool in_e;
    int j_of_e;
    const int row = local_row_in_expert(tp, e, L, in_e, j_of_e);
    const int ebase = __builtin_amdgcn_readlane(ebase_lane, e);
    const uint64_t m = ballot64(in_e && tp.ad == ad);
    const int lrow = lane & 15;
    int i = 0;
#pragma unroll 1
    for (uint64_t mm = m; mm; mm &= mm - 1, ++i) {
        const int q = __ffsll(static_cast<long long>(mm)) - 1;
        const int rq = __builtin_amdgcn_readlane(row, q), jq = __builtin_amdgcn_readlane(j_of_e, q);
        if (i == lrow) {
            row_p = q * k + jq;
            row_slot = ebase + rq;
        }
    }
    return true;
}

// One wave writes the routing and both alignment views: the pair lanes
// their entries, then the padding and block-map entries of each expert and
// segment, then the tails. Lane p < P holds pair p here.
__device__ __forceinline__ void local_publish(const float* logits, const int32_t* adapter_ids, int T, int E,
                                              int k, int L, float* ls, const int32_t* ids, const LocalOut& o) {
    const int lane = threadIdx.x & 63;
    const int P = T * k;
    const TokenPicks tp = local_picks(logits, adapter_ids, T, E, k, L, ls, ids);
    // token lanes: weights e^(v_j - v_0) over their sum, the sum in the order
    // of the routing kernel's xor butterfly over lanes j < k (zeros elsewhere)
    float wt[kLocalMaxK];
    {
        float ex[kLocalMaxK], s[kLocalMaxK];
#pragma unroll
        for (int j = 0; j < kLocalMaxK; ++j) {
            ex[j] = j < k ? expf(tp.pv[j] - tp.pv[0]) : 0.0f;
            s[j] = ex[j];
        }
#pragma unroll
        for (int off = kLocalMaxK / 2; off > 0; off >>= 1)
#pragma unroll
            for (int i = 0; i < off; ++i) s[i] = s[i] + s[i + off];
#pragma unroll
        for (int j = 0; j < kLocalMaxK; ++j) wt[j] = ex[j] / s[0];
    }
    // pair lanes: p = t k + j takes pick j of token t
    const bool valid = lane < P;
    const int t = valid ? lane / k : 0, jj = valid ? lane - t * k : 0;
    int e = 0;
    float w = 0.0f;
#pragma unroll
    for (int j = 0; j < kLocalMaxK; ++j) {
        const int ej = __shfl(tp.pid[j], t);
        const float wj = __shfl(wt[j], t);
        if (j == jj) {
            e = ej;
            w = wj;
        }
    }
    const int ad = __shfl(tp.ad, t);
    const uint64_t live = ballot64(valid);
    const uint64_t below = lanemask_lt();
    // base view: position in (expert, adapter', p) order within the expert
    int lt_key, lt_e;
    uint64_t eq_key, eq_e;
    rank_by_bits(e * (L + 1) + ad, live, bits_for(E * (L + 1)), lt_key, eq_key);
    rank_by_bits(e, live, bits_for(E), lt_e, eq_e);
    int cnt, n_b;
    const int ebase_lane = local_expert_starts(tp.mask, T, E, cnt, n_b);
    const int slot = __shfl(ebase_lane, e) + lt_key + popc64(eq_key & below) - lt_e;
    // LoRA view: segment blocks in (expert, adapter) order
    const bool lora = valid && ad < L;
    const int skey = lora ? e * L + ad : 0;
    int lt_s, seg_blk;
    uint64_t eq_s, unused;
    rank_by_bits(skey, ballot64(lora), bits_for(E * L), lt_s, eq_s);
    const uint64_t seg_first = ballot64(lora && (eq_s & below) == 0);
    rank_by_bits(skey, seg_first, bits_for(E * L), seg_blk, unused);
    seg_blk = __shfl(seg_blk, eq_s ? __ffsll(static_cast<long long>(eq_s)) - 1 : lane);
    const int lslot = lora ? 16 * seg_blk + popc64(eq_s & below) : -1;
    const int ns = lora ? popc64(eq_s) : 0;
    const int n_l = 16 * popc64(seg_first);
    (void)lt_s;

    if (valid && !ids) {  // with ids given, the routing launch wrote both
        o.ids[lane] = e;
        o.tw[lane] = w;
    }
    if (valid) {
        o.sorted_b[slot] = lane;
        o.slot_of_pair[lane] = slot;
        o.slot_adapter[slot] = ad < L ? ad : -1;
        if (lora) o.sorted_l[lslot] = lane;
        o.lslot_of_pair[lane] = lslot;
    }
    // each used expert: padding rows and block-map entry
#pragma unroll 1
    for (int x = 0; x < E; ++x) {
        const int c = __builtin_amdgcn_readlane(cnt, x);
        if (c == 0) continue;
        const int base = __builtin_amdgcn_readlane(ebase_lane, x);
        if (lane >= c && lane < 16) {
            o.sorted_b[base + lane] = P;
            o.slot_adapter[base + lane] = -1;
        }
        if (lane == 0) o.blk_e_b[base >> 4] = x;
    }
    // each segment: padding rows and block-map entries
#pragma unroll 1
    for (uint64_t m = seg_first; m; m &= m - 1) {
        const int q = __ffsll(static_cast<long long>(m)) - 1;
        const int base = __builtin_amdgcn_readlane(lslot, q), nq = __builtin_amdgcn_readlane(ns, q);
        const int eq = __builtin_amdgcn_readlane(e, q), aq = __builtin_amdgcn_readlane(ad, q);
        if (lane >= nq && lane < 16) o.sorted_l[base + lane] = P;
        if (lane == 0) {
            o.blk_e_l[base >> 4] = eq;
            o.blk_a_l[base >> 4] = aq;
        }
    }
    for (int i = n_b + lane; i < o.C_b; i += 64) {
        o.sorted_b[i] = P;
        o.slot_adapter[i] = -1;
    }
    for (int i = (n_b >> 4) + lane; i < (o.C_b >> 4); i += 64) o.blk_e_b[i] = -1;
    for (int i = n_l + lane; i < o.C_l; i += 64) o.sorted_l[i] = P;
    for (int i = (n_l >> 4) + lane; i < (o.C_l >> 4); i += 64) {
        o.blk_e_l[i] = -1;
        o.blk_a_l[i] = -1;
    }
    if (lane == 0) {
        *o.n_b = n_b;
        *o.n_l = n_l;
    }
}

}  // namespace moelora
