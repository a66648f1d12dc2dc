// C ABI of libmoelora: argument checks, workspace layout and the launch
// sequence of the multi-LoRA MoE expert layer (see include/moe_lora.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/moe_lora.h"
#include "kernels.h"
#include "local_route.h"

using namespace moelora;

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Plan {
    int T, H, I, E, k, L, r, P;
    int bm_b, bm_l, C_b, C_l, nblk_b, nblk_l;
    int ksplit;  // K ranges of the down projection (partial sums summed by the combine)
    int ssplit;  // K ranges of the two shrinks (partials summed by the projection kernels)
    int ksw_gu, ksw_dn;  // 16-row blocks: waves per tile of the two projections
    int fn_gu;           // 16-row blocks: 16-column fragments per gate_up wave
    bool w_stream;       // direct-load kernels: weights read with the non-temporal policy
    bool fused;  // the shrinks run as producer waves inside the projection launches
    bool fuse_combine;  // the down projection adds its weighted rows into out (no D, no combine launch)
    bool local;  // the gate_up launch aligns the batch itself (no alignment launch)
    bool local_route;  // ... and routes it too (no routing launch)
    size_t off_ids, off_w, off_sorted_b, off_blk_e_b, off_counts, off_sorted_l, off_blk_e_l,
        off_blk_a_l, off_slot, off_lslot, off_sad, off_defer, off_s1, off_s2, off_s1hl, off_s2hl,
        off_h, off_d, total;
    bool s_hl;  // the direct-load projection kernels take S as bf16 hi/lo rows
};

int roundup_i(long v, long m) { return static_cast<int>((v + m - 1) / m * m); }

// Where a decode-sized batch is aligned inside the gate_up launch, that
// launch also routes it when each wave's top-k scan (E x top_k steps per
// token) is this short; longer scans cost the launch more than the routing
// launch takes, and the routing launch stays.
constexpr int kLocalRouteMaxWork = 32;

int default_bm_base(int P, int E) {
    if (E == 1) {  // no routing: the one expert holds all P rows
        int bm = 16;
        while (bm < P && bm < 128) bm *= 2;
        return bm;
    }
    const long avg = (P + E - 1) / E;  // mean rows per expert
    if (avg <= 8) return 16;    // weight streaming: one 16-row block per expert
    // 64-row register-staged tiles: the skewed wide-expert layer (16 rows
    // per expert on average, up to ~50) measured 505 us against 516 us with
    // 32-row tiles
    if (avg <= 16) return 64;
    // direct-to-LDS 128 x 192 tiles: at 64 rows per expert (many-adapter
    // layer) one block per expert streams its weights once: 629 us against
    // 753 us with 64-row blocks, which split most experts in two
    return 128;
}

// LoRA view blocks: 64 rows once the (expert, adapter) segments average at
// least 32 rows, so that each block's shrink reads its LoRA A once for four
// 16-row fragments (prefill-shaped layer: both shrinks 134 -> 93 us); 16 rows
// otherwise, where the padding of each segment would cost more (decode,
// many-adapter and wide-expert layers).
int default_bm_lora(int P, int E, int L) {
    return L > 0 && static_cast<long>(P) >= 32L * E * L ? 64 : 16;
}

int check_desc(const moe_lora_desc* d) {
    if (!d) return MOE_LORA_EINVAL;
    if (d->T < 0 || d->H <= 0 || d->I <= 0 || d->E <= 0 || d->L < 0) return MOE_LORA_EINVAL;
    if (d->H % 64 || d->I % 64) return MOE_LORA_EINVAL;
    if (d->E > 1024 || d->top_k < 1 || d->top_k > d->E || d->top_k > 32) return MOE_LORA_EINVAL;
    if (d->L > 0 && !(d->r == 8 || d->r == 16 || d->r == 32 || d->r == 64 || d->r == 128))
        return MOE_LORA_EINVAL;
    if (d->flags & ~(MOE_LORA_FLAG_OUT_BF16 | MOE_LORA_FLAG_SHRINK_LAUNCH | MOE_LORA_FLAG_FUSED_COMBINE |
                     MOE_LORA_FLAG_NO_SHRINK_WAIT | MOE_LORA_FLAG_ROUTE_LAUNCH))
        return MOE_LORA_EINVAL;
    if ((d->flags & MOE_LORA_FLAG_FUSED_COMBINE) && (d->flags & MOE_LORA_FLAG_OUT_BF16)) return MOE_LORA_EINVAL;
    if (d->block_m_base != 0 && !pow2_in(d->block_m_base, 16, 256)) return MOE_LORA_EINVAL;
    if (d->block_m_lora != 0 && !pow2_in(d->block_m_lora, 16, 256)) return MOE_LORA_EINVAL;
    const long P = static_cast<long>(d->T) * d->top_k;
    if (P > (1L << 24)) return MOE_LORA_EINVAL;
    if (!align_fits(d->E, d->L)) return MOE_LORA_EINVAL;
    return MOE_LORA_OK;
}

int make_plan(const moe_lora_desc* d, Plan* p) {
    const int rc = check_desc(d);
    if (rc) return rc;
    p->T = d->T; p->H = d->H; p->I = d->I; p->E = d->E; p->k = d->top_k; p->L = d->L;
    p->r = d->L > 0 ? d->r : 8;
    p->P = d->T * d->top_k;
    p->bm_b = d->block_m_base ? d->block_m_base : default_bm_base(p->P, p->E);
    p->bm_l = d->block_m_lora ? d->block_m_lora : default_bm_lora(p->P, p->E, p->L);
    if (!gemm_supported(p->I, p->H, 1, p->bm_b) || !gemm_supported(p->H, p->I, 0, p->bm_b))
        return MOE_LORA_EINVAL;
    const long P = p->P;
    p->C_b = roundup_i(P + std::min<long>(p->E, P) * (p->bm_b - 1), p->bm_b);
    p->C_l = roundup_i(P + std::min<long>(static_cast<long>(p->E) * p->L, P) * (p->bm_l - 1), p->bm_l);
    p->nblk_b = p->C_b / p->bm_b;
    p->nblk_l = p->C_l / p->bm_l;
    // launch tuning: 0 = the library's choice; results do not depend on any
    // of these beyond the order of fp32 sums
    if (d->down_ksplit < 0 || d->shrink_ksplit < 0 || d->waves_gate_up < 0 || d->waves_down < 0 ||
        d->frags_gate_up < 0)
        return MOE_LORA_EINVAL;
    p->ksplit = d->down_ksplit ? d->down_ksplit : gemm_down_ksplit(p->H, p->I, p->bm_b, p->nblk_b);
    // the direct-load kernels take the whole K range
    if (p->bm_b >= 128 && p->ksplit != 1) return MOE_LORA_EINVAL;
    if (p->ksplit > p->I / 64 || (p->I / 64) % p->ksplit) return MOE_LORA_EINVAL;
    p->ksw_gu = d->waves_gate_up ? d->waves_gate_up : 1;
    p->ksw_dn = d->waves_down ? d->waves_down : 1;
    if (p->bm_b != 16 && (p->ksw_gu != 1 || p->ksw_dn != 1)) return MOE_LORA_EINVAL;
    if (p->bm_b == 16 && (!skinny_waves_ok(p->H, 1, p->ksw_gu) || !skinny_waves_ok(p->I, p->ksplit, p->ksw_dn)))
        return MOE_LORA_EINVAL;
    // 8 fragments per gate_up wave: 16-row blocks, one wave per tile, I a
    // multiple of 64 (whole 64-column tiles)
    p->fn_gu = d->frags_gate_up ? d->frags_gate_up : 4;
    if (p->fn_gu != 4 && (p->fn_gu != 8 || p->bm_b != 16 || p->ksw_gu != 1 || p->I % 64))
        return MOE_LORA_EINVAL;
    // 128- and 256-row blocks with at most half a block of rows per expert on
    // average: nearly every expert has one block, whose column tiles read
    // each weight tile once, and those loads take the non-temporal policy
    // (many-adapter layer, 64 rows per expert: 619 -> 609 us). With more rows
    // per expert the blocks of an expert share its weight tiles through the
    // L2 (the prefill-shaped layer with the policy: 1516 -> 1996 us).
    p->w_stream = p->bm_b >= 128 && static_cast<long>(p->P) * 2 <= static_cast<long>(p->E) * p->bm_b;
    // the weighted combine runs in the down projection's epilogue (fp32
    // atomic adds into out) only on request: the atomics cost the down
    // projection more than the fixed-order combine launch takes at every
    // measured shape (decode-shaped layer +7 against 4.5 us, prefill-shaped
    // +585 against 67 us)
    p->fuse_combine = (d->flags & MOE_LORA_FLAG_FUSED_COMBINE) != 0;
    // 16-row base blocks (few rows per expert: the projections stream their
    // weights) run the shrinks inside the projection launches, as long as
    // the producer waves stay a small share of the machine (at most about
    // one per SIMD); more of them take the wave slots ahead of the projection
    // and measured slower than separate launches
    p->fused = false;
    if (p->L > 0 && p->bm_b == 16 && !(d->flags & MOE_LORA_FLAG_SHRINK_LAUNCH)) {
        const int ss = std::max(producer_ksplit(p->H), producer_ksplit(p->I));
        const long units = static_cast<long>(p->nblk_l) * ((p->r + 15) / 16) * ss;
        p->fused = units <= kMaxProducerUnits;
    }
    // decode-sized batches with 16-row blocks: every wave of the gate_up
    // launch routes the batch itself from the logits, so that the launch
    // streams weights while the routing is worked out; the routing and
    // alignment launches (about 11 us of a 300 us decode-shaped call) drop
    // out
    p->local = p->bm_b == 16 && p->bm_l == 16 && local_route_fits(p->T, p->E, p->k) && p->ksw_gu == 1 &&
               (p->L == 0 || p->fused) && !(d->flags & MOE_LORA_FLAG_ROUTE_LAUNCH);
    p->local_route = p->local && static_cast<long>(p->E) * p->k <= kLocalRouteMaxWork;
    if (p->fused) {
        p->ssplit = std::max(producer_ksplit(p->H), producer_ksplit(p->I));
        if (d->shrink_ksplit && d->shrink_ksplit != p->ssplit) return MOE_LORA_EINVAL;
    } else if (p->L > 0 && d->shrink_ksplit) {
        p->ssplit = d->shrink_ksplit;
        if (p->ssplit > kMaxShrinkSplit || p->ssplit > std::min(p->H, p->I) / 64) return MOE_LORA_EINVAL;
    } else {
        p->ssplit = p->L > 0 ? std::min(shrink_ksplit(p->nblk_l, p->H, p->bm_b),
                                        shrink_ksplit(p->nblk_l, p->I, p->bm_b)) : 1;
    }
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o += up(bytes); return at; };
    p->off_ids = take(4 * P);
    p->off_w = take(4 * P);
    p->off_sorted_b = take(4ul * p->C_b);
    p->off_blk_e_b = take(4ul * p->nblk_b);
    p->off_counts = take(64);
    p->off_sorted_l = take(4ul * p->C_l);
    p->off_blk_e_l = take(4ul * p->nblk_l);
    p->off_blk_a_l = take(4ul * p->nblk_l);
    p->off_slot = take(4 * P);
    p->off_lslot = take(4 * P);
    p->off_sad = take(4ul * p->C_b);
    p->off_defer = take(4ul * align_defer_ints(p->P, p->E, p->L));
    const size_t sbytes = p->L > 0 ? 4ul * p->ssplit * p->C_b * p->r : 0;
    p->off_s1 = take(sbytes);
    p->off_s2 = take(sbytes);
    // the LDS kernels (32- to 256-row blocks, never a split shrink) run the
    // expand in their pipeline from a bf16 hi/lo copy of S
    p->s_hl = p->L > 0 && p->bm_b >= 32 && p->ssplit == 1;
    const size_t hlbytes = p->s_hl ? 2ul * p->C_b * s_hl_stride_of(p->r) : 0;
    p->off_s1hl = take(hlbytes);
    p->off_s2hl = take(hlbytes);
    p->off_h = take(2ul * p->C_b * p->I);
    p->off_d = take(p->fuse_combine ? 0 : 4ul * p->ksplit * p->C_b * p->H);
    p->total = o;
    return MOE_LORA_OK;
}

int check_weights(const moe_lora_desc* d, const moe_lora_weights* w) {
    if (!w) return MOE_LORA_EINVAL;
    if (!w->w_gate_up || !w->w_down || !aligned16(w->w_gate_up) || !aligned16(w->w_down))
        return MOE_LORA_EINVAL;
    if (d->L > 0) {
        const void* l[4] = {w->a_gate_up, w->b_gate_up, w->a_down, w->b_down};
        for (const void* q : l)
            if (!q || !aligned16(q)) return MOE_LORA_EINVAL;
    }
    if ((w->w_gate_up_packed && (!aligned16(w->w_gate_up_packed) || !pack_skinny_supported(d->I, d->H, 1))) ||
        (w->w_down_packed && (!aligned16(w->w_down_packed) || !pack_skinny_supported(d->H, d->I, 0))))
        return MOE_LORA_EINVAL;
    return MOE_LORA_OK;
}

template <typename T>
T* at(void* base, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// ---- per-kernel timing --------------------------------------------------
const char* kKernelNames[MOE_LORA_NKERNELS] = {"route", "align", "shrink_gate_up", "gemm_gate_up",
                                               "shrink_down", "gemm_down", "combine"};
struct Timing {
    int max_calls = 0;
    int ncalls = 0;
    std::vector<hipEvent_t> ev;        // [max_calls][NKERNELS + 1]
    std::vector<uint8_t> launched;     // [max_calls][NKERNELS]: whether the call launched kernel i
} g_timing;

void timing_mark(int call, int i, hipStream_t s) {
    if (call >= 0) (void)hipEventRecord(g_timing.ev[static_cast<size_t>(call) * (MOE_LORA_NKERNELS + 1) + i], s);
}

}  // namespace

extern "C" {

const char* moe_lora_strerror(int code) {
    switch (code) {
        case MOE_LORA_OK: return "ok";
        case MOE_LORA_EINVAL: return "invalid argument (dimension, pointer, alignment or block size)";
        case MOE_LORA_EWORKSPACE: return "workspace too small";
        case MOE_LORA_EHIP: return "HIP runtime or launch error";
        case MOE_LORA_ESCRATCH: return "call needs more scratch than the library's static buffer holds";
        default: return "unknown error";
    }
}

int moe_lora_validate(const moe_lora_desc* d, const moe_lora_weights* w, size_t ws_bytes) {
    Plan p;
    int rc = make_plan(d, &p);
    if (rc) return rc;
    if (w && (rc = check_weights(d, w))) return rc;
    if (ws_bytes != static_cast<size_t>(-1) && ws_bytes < p.total) return MOE_LORA_EWORKSPACE;
    return MOE_LORA_OK;
}

int moe_lora_block_sizes(const moe_lora_desc* d, int32_t* bm_b, int32_t* bm_l) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc) return rc;
    if (bm_b) *bm_b = p.bm_b;
    if (bm_l) *bm_l = p.bm_l;
    return MOE_LORA_OK;
}

int moe_lora_plan(const moe_lora_desc* d, moe_lora_plan_info* info) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc) return rc;
    if (!info) return MOE_LORA_EINVAL;
    info->block_m_base = p.bm_b;
    info->block_m_lora = p.bm_l;
    info->down_ksplit = p.ksplit;
    info->shrink_ksplit = p.L > 0 ? p.ssplit : 0;
    info->waves_gate_up = p.bm_b == 16 ? p.ksw_gu : 0;
    info->frags_gate_up = p.bm_b == 16 ? p.fn_gu : 0;
    info->waves_down = p.bm_b == 16 ? p.ksw_dn : 0;
    info->shrinks_in_projections = p.fused ? 1 : 0;
    info->combine_in_down = p.fuse_combine ? 1 : 0;
    info->routing_in_gate_up = p.local_route ? 2 : p.local ? 1 : 0;
    return MOE_LORA_OK;
}

int moe_lora_workspace_bytes(const moe_lora_desc* d, size_t* bytes) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc) return rc;
    if (!bytes) return MOE_LORA_EINVAL;
    *bytes = p.total;
    return MOE_LORA_OK;
}

int moe_lora_align_capacity(const moe_lora_desc* d, int32_t* C_b, int32_t* C_l) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc) return rc;
    if (C_b) *C_b = p.C_b;
    if (C_l) *C_l = p.C_l;
    return MOE_LORA_OK;
}

int moe_lora_pack_weights(const moe_lora_desc* d, const void* w_gate_up, const void* w_down,
                          void* w_gate_up_packed, void* w_down_packed, void* stream) {
    const int rc = check_desc(d);
    if (rc) return rc;
    const bool gu = w_gate_up_packed != nullptr, dn = w_down_packed != nullptr;
    if ((gu && (!w_gate_up || !aligned16(w_gate_up) || !aligned16(w_gate_up_packed) ||
                !pack_skinny_supported(d->I, d->H, 1))) ||
        (dn && (!w_down || !aligned16(w_down) || !aligned16(w_down_packed) || !pack_skinny_supported(d->H, d->I, 0))))
        return MOE_LORA_EINVAL;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (gu && launch_pack_skinny(static_cast<const uint16_t*>(w_gate_up), static_cast<uint16_t*>(w_gate_up_packed),
                                 d->E, d->I, d->H, 1, s) != hipSuccess)
        return MOE_LORA_EHIP;
    if (dn && launch_pack_skinny(static_cast<const uint16_t*>(w_down), static_cast<uint16_t*>(w_down_packed), d->E,
                                 d->H, d->I, 0, s) != hipSuccess)
        return MOE_LORA_EHIP;
    return MOE_LORA_OK;
}

int moe_lora_route(const moe_lora_desc* d, const float* logits, int32_t* ids, float* w,
                   void* stream) {
    const int rc = check_desc(d);
    if (rc) return rc;
    if (d->T == 0) return MOE_LORA_OK;
    if (!logits || !ids || !w) return MOE_LORA_EINVAL;
    return launch_route(logits, d->T, d->E, d->top_k, ids, w, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? MOE_LORA_OK
               : MOE_LORA_EHIP;
}

int moe_lora_align(const moe_lora_desc* d, const int32_t* topk_ids, const int32_t* adapter_ids,
                   int32_t* sorted_b, int32_t* blk_e_b, int32_t* n_b, int32_t* sorted_l,
                   int32_t* blk_e_l, int32_t* blk_a_l, int32_t* n_l, void* workspace, size_t ws_bytes,
                   void* stream) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc) return rc;
    if (d->T == 0) return MOE_LORA_OK;
    if (!topk_ids || !adapter_ids || !sorted_b || !blk_e_b || !n_b || !sorted_l || !blk_e_l ||
        !blk_a_l || !n_l)
        return MOE_LORA_EINVAL;
    // the alignment's scratch is the forward pass's (same region of a
    // workspace of moe_lora_workspace_bytes)
    int32_t* defer = nullptr;
    if (workspace) {
        if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return MOE_LORA_EINVAL;
        if (ws_bytes < p.total) return MOE_LORA_EWORKSPACE;
        defer = at<int32_t>(workspace, p.off_defer);
    } else if (!align_single_workgroup(p.P, p.E, p.L)) {
        return MOE_LORA_EWORKSPACE;
    }
    return launch_align(topk_ids, adapter_ids, p.T, p.k, p.E, p.L, p.bm_b, p.bm_l, p.C_b, p.C_l,
                        sorted_b, blk_e_b, n_b, sorted_l, blk_e_l, blk_a_l, n_l, nullptr,
                        nullptr, nullptr, defer, static_cast<hipStream_t>(stream)) == hipSuccess
               ? MOE_LORA_OK
               : MOE_LORA_EHIP;
}

}  // extern "C"

namespace {

// The launch sequence of one layer call on a checked plan; `workspace` holds
// at least p.total bytes, 256-byte aligned.
int forward_planned(const Plan& p, const moe_lora_desc* d, const moe_lora_weights* w, const void* x,
                    const float* logits, const int32_t* adapter_ids, void* out, void* workspace,
                    hipStream_t s) {

    int32_t* ids = at<int32_t>(workspace, p.off_ids);
    float* tw = at<float>(workspace, p.off_w);
    int32_t* sorted_b = at<int32_t>(workspace, p.off_sorted_b);
    int32_t* blk_e_b = at<int32_t>(workspace, p.off_blk_e_b);
    int32_t* counts = at<int32_t>(workspace, p.off_counts);
    int32_t* sorted_l = at<int32_t>(workspace, p.off_sorted_l);
    int32_t* blk_e_l = at<int32_t>(workspace, p.off_blk_e_l);
    int32_t* blk_a_l = at<int32_t>(workspace, p.off_blk_a_l);
    int32_t* slot = at<int32_t>(workspace, p.off_slot);
    int32_t* lslot = at<int32_t>(workspace, p.off_lslot);
    int32_t* sad = at<int32_t>(workspace, p.off_sad);
    float* s1 = at<float>(workspace, p.off_s1);
    float* s2 = at<float>(workspace, p.off_s2);
    uint16_t* h = at<uint16_t>(workspace, p.off_h);
    float* dn = at<float>(workspace, p.off_d);

    int call = -1;
    if (g_timing.max_calls > 0 && g_timing.ncalls < g_timing.max_calls) {
        call = g_timing.ncalls++;
        const bool shrink_launched = p.L > 0 && !p.fused;
        uint8_t* l = &g_timing.launched[static_cast<size_t>(call) * MOE_LORA_NKERNELS];
        l[2] = l[4] = shrink_launched ? 1 : 0;  // shrink_gate_up, shrink_down
        l[1] = p.local ? 0 : 1;                 // align (with local routing, "route" times the clearing launch)
        l[6] = p.fuse_combine ? 0 : 1;          // combine
    }

    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t v) { if (e == hipSuccess) e = v; };
    timing_mark(call, 0, s);
    // counts[0..1]: n_b, n_l (alignment); counts[2..3]: producer counts of
    // the two projections; counts[4]: the call's status word; 2..4 are
    // zeroed by the routing launch
    if (p.local_route) {
        ok(launch_zero(counts + 2, 3, p.fuse_combine ? static_cast<float*>(out) : nullptr, p.T, p.H, s));
        timing_mark(call, 1, s);
    } else if (p.local) {
        ok(launch_route(logits, p.T, p.E, p.k, ids, tw, s, counts + 2, 3,
                        p.fuse_combine ? static_cast<float*>(out) : nullptr, p.H));
        timing_mark(call, 1, s);
    } else {
        ok(launch_route(logits, p.T, p.E, p.k, ids, tw, s, counts + 2, 3,
                        p.fuse_combine ? static_cast<float*>(out) : nullptr, p.H));
        timing_mark(call, 1, s);
        ok(launch_align(ids, adapter_ids, p.T, p.k, p.E, p.L, p.bm_b, p.bm_l, p.C_b, p.C_l, sorted_b,
                        blk_e_b, counts, sorted_l, blk_e_l, blk_a_l, counts + 1, slot, lslot, sad,
                        at<int32_t>(workspace, p.off_defer), s));
    }
    timing_mark(call, 2, s);

    ShrinkArgs sa{};
    sa.top_k = p.k; sa.P = p.P; sa.sorted_l = sorted_l; sa.blk_e_l = blk_e_l;
    sa.blk_a_l = blk_a_l; sa.slot_of_pair = slot; sa.E = p.E; sa.r = p.r; sa.bm_l = p.bm_l;
    sa.n_blocks = p.nblk_l; sa.ksplit = p.ssplit; sa.C_b = p.C_b;
    sa.s_hl_stride = s_hl_stride_of(p.r);
    uint16_t* s1hl = p.s_hl ? at<uint16_t>(workspace, p.off_s1hl) : nullptr;
    uint16_t* s2hl = p.s_hl ? at<uint16_t>(workspace, p.off_s2hl) : nullptr;
    if (p.L > 0 && !p.fused) {
        sa.X = static_cast<const uint16_t*>(x); sa.gather_token = 1; sa.K = p.H;
        sa.A = static_cast<const uint16_t*>(w->a_gate_up); sa.S = s1; sa.S_hl = s1hl;
        ok(launch_shrink(sa, s));
    }
    timing_mark(call, 3, s);

    GemmArgs ga{};
    ga.sorted_b = sorted_b; ga.blk_e_b = blk_e_b; ga.P = p.P; ga.top_k = p.k; ga.bm_b = p.bm_b;
    ga.n_b_live = counts;
    ga.n_blocks = p.nblk_b; ga.slot_adapter = sad; ga.L = p.L; ga.E = p.E; ga.r = p.r;
    ga.C_b = p.C_b; ga.h_out = h; ga.d_out = dn; ga.ksplit = 1; ga.s_split = p.ssplit;
    ga.X = static_cast<const uint16_t*>(x); ga.gate_up = 1;
    ga.W = static_cast<const uint16_t*>(w->w_gate_up); ga.N_out = p.I; ga.K = p.H;
    ga.Wp = p.bm_b == 16 ? static_cast<const uint16_t*>(w->w_gate_up_packed) : nullptr;
    ga.S = s1; ga.Bl = static_cast<const uint16_t*>(w->b_gate_up);
    ga.S_hl = s1hl; ga.s_hl_stride = s_hl_stride_of(p.r); ga.ksw = p.ksw_gu; ga.frags = p.fn_gu;
    ga.w_stream = p.w_stream;
    if (p.fused) {
        ga.prod_ncf = (p.r + 15) / 16;
        ga.prod_units = p.nblk_l * ga.prod_ncf * p.ssplit;
        ga.gather_token = 1; ga.sorted_l = sorted_l; ga.blk_e_l = blk_e_l; ga.blk_a_l = blk_a_l;
        ga.slot_of_pair = slot; ga.Al = static_cast<const uint16_t*>(w->a_gate_up);
        ga.bm_l = p.bm_l; ga.S_out = s1; ga.done = counts + 2; ga.n_l = counts + 1;
        ga.status = counts + 4;
        ga.max_polls = (d->flags & MOE_LORA_FLAG_NO_SHRINK_WAIT) ? 0 : kMaxProducerPolls;
    }
    if (p.local) {
        // expert-indexed blocks; the launch's first workgroup writes the
        // routing and alignment for the launches below
        ga.local = 1; ga.adapter_ids = adapter_ids; ga.T = p.T; ga.n_blocks = p.E;
        if (p.local_route) ga.logits = logits;
        else ga.local_ids = ids;
        ga.pub = LocalOut{ids, tw, sorted_b, blk_e_b, counts, sorted_l, blk_e_l, blk_a_l, counts + 1,
                          slot, lslot, sad, p.C_b, p.C_l};
    }
    ok(launch_gemm(ga, s));
    ga.local = 0; ga.logits = nullptr; ga.local_ids = nullptr; ga.adapter_ids = nullptr; ga.n_blocks = p.nblk_b;
    timing_mark(call, 4, s);

    if (p.L > 0 && !p.fused) {
        sa.X = h; sa.gather_token = 0; sa.K = p.I;
        sa.A = static_cast<const uint16_t*>(w->a_down); sa.S = s2; sa.S_hl = s2hl;
        ok(launch_shrink(sa, s));
    }
    timing_mark(call, 5, s);

    ga.X = h; ga.gate_up = 0; ga.W = static_cast<const uint16_t*>(w->w_down); ga.N_out = p.H;
    ga.Wp = p.bm_b == 16 ? static_cast<const uint16_t*>(w->w_down_packed) : nullptr;
    ga.K = p.I; ga.S = s2; ga.Bl = static_cast<const uint16_t*>(w->b_down); ga.ksplit = p.ksplit;
    ga.S_hl = s2hl; ga.ksw = p.ksw_dn;
    if (p.fuse_combine) {
        ga.out_acc = static_cast<float*>(out);
        ga.topk_w = tw;
        ga.d_out = nullptr;
    }
    if (p.fused) {
        ga.gather_token = 0; ga.Al = static_cast<const uint16_t*>(w->a_down);
        ga.S_out = s2; ga.done = counts + 3;
    }
    ok(launch_gemm(ga, s));
    timing_mark(call, 6, s);

    if (!p.fuse_combine)
        ok(launch_combine(dn, p.ksplit, p.C_b, slot, tw, p.T, p.k, p.H, out,
                          (d->flags & MOE_LORA_FLAG_OUT_BF16) != 0, s));
    timing_mark(call, 7, s);
    return e == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

// Checks shared by both forward entry points (everything but the workspace).
int check_forward(const moe_lora_desc* d, const moe_lora_weights* w, const void* x, const float* logits,
                  const int32_t* adapter_ids, const void* out, Plan* p) {
    int rc = make_plan(d, p);
    if (rc) return rc;
    if ((rc = check_weights(d, w))) return rc;
    if (p->T == 0) return MOE_LORA_OK;
    if (!x || !logits || !adapter_ids || !out) return MOE_LORA_EINVAL;
    if (!aligned16(x) || !aligned16(out)) return MOE_LORA_EINVAL;
    return MOE_LORA_OK;
}

// ---- the static scratch of moe_lora_forward_noalloc ------------------------
// Every GPU the library runs on holds one copy of this array from module load
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device with
// hipGetSymbolAddress, and only that address is ever handed to a kernel.
__device__ __attribute__((aligned(256))) uint8_t scratch[MOE_LORA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// that device), or null on a HIP error.
void* scratch_address(int dev) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_lora_forward(const moe_lora_desc* d, const moe_lora_weights* w, const void* x,
                     const float* logits, const int32_t* adapter_ids, void* out,
                     void* workspace, size_t ws_bytes, void* stream) {
    Plan p;
    const int rc = check_forward(d, w, x, logits, adapter_ids, out, &p);
    if (rc || p.T == 0) return rc;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign)) return MOE_LORA_EINVAL;
    if (ws_bytes < p.total) return MOE_LORA_EWORKSPACE;
    return forward_planned(p, d, w, x, logits, adapter_ids, out, workspace, static_cast<hipStream_t>(stream));
}

int moe_lora_forward_noalloc(const moe_lora_desc* d, const moe_lora_weights* w, const void* x,
                             const float* logits, const int32_t* adapter_ids, void* out, void* stream) {
    Plan p;
    const int rc = check_forward(d, w, x, logits, adapter_ids, out, &p);
    if (rc || p.T == 0) return rc;
    if (p.total > MOE_LORA_SCRATCH_BYTES) return MOE_LORA_ESCRATCH;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_LORA_EHIP;
    if (s) {
        // the scratch address is the current device's: the stream must be on it
        int sdev = -1;
        if (hipStreamGetDevice(s, &sdev) != hipSuccess) return MOE_LORA_EHIP;
        if (sdev != dev) return MOE_LORA_EINVAL;
    }
    void* ws = scratch_address(dev);
    if (!ws) return MOE_LORA_EHIP;
    return forward_planned(p, d, w, x, logits, adapter_ids, out, ws, s);
}

int moe_lora_read_stages(const moe_lora_desc* d, const void* workspace, size_t ws_bytes,
                         int32_t* topk_ids, float* topk_w, float* s1, uint16_t* h, float* s2,
                         float* dn, void* stream) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc) return rc;
    if (p.T == 0) return MOE_LORA_OK;
    if (!workspace) return MOE_LORA_EINVAL;
    if (ws_bytes < p.total) return MOE_LORA_EWORKSPACE;
    if (dn && p.fuse_combine) return MOE_LORA_EINVAL;  // D is not kept
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = const_cast<void*>(workspace);
    const int32_t* slot = at<int32_t>(ws, p.off_slot);
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t v) { if (e == hipSuccess) e = v; };
    if (topk_ids)
        ok(hipMemcpyAsync(topk_ids, at<int32_t>(ws, p.off_ids), 4ul * p.P, hipMemcpyDeviceToDevice, s));
    if (topk_w)
        ok(hipMemcpyAsync(topk_w, at<float>(ws, p.off_w), 4ul * p.P, hipMemcpyDeviceToDevice, s));
    const int32_t* lslot = at<int32_t>(ws, p.off_lslot);  // -1 = pair without adapter
    // with L == 0 every mask entry is -1 and the (empty) S buffers are never read
    if (s1) ok(launch_gather_rows_f32(at<float>(ws, p.off_s1), p.ssplit, p.C_b, p.r, slot, lslot, p.P, s1, s));
    if (s2) ok(launch_gather_rows_f32(at<float>(ws, p.off_s2), p.ssplit, p.C_b, p.r, slot, lslot, p.P, s2, s));
    if (h) ok(launch_gather_rows_bf16(at<uint16_t>(ws, p.off_h), p.I, slot, p.P, h, s));
    if (dn) ok(launch_gather_rows_f32(at<float>(ws, p.off_d), p.ksplit, p.C_b, p.H, slot, nullptr, p.P, dn, s));
    return e == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

int moe_lora_read_alignment(const moe_lora_desc* d, const void* workspace, size_t ws_bytes,
                            int32_t* sorted_b, int32_t* blk_e_b, int32_t* n_b, int32_t* sorted_l,
                            int32_t* blk_e_l, int32_t* blk_a_l, int32_t* n_l, void* stream) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc) return rc;
    if (p.T == 0) return MOE_LORA_OK;
    if (!workspace) return MOE_LORA_EINVAL;
    if (ws_bytes < p.total) return MOE_LORA_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = const_cast<void*>(workspace);
    hipError_t e = hipSuccess;
    auto cp = [&](int32_t* dst, size_t off, size_t n) {
        if (dst && e == hipSuccess)
            e = hipMemcpyAsync(dst, at<int32_t>(ws, off), 4 * n, hipMemcpyDeviceToDevice, s);
    };
    cp(sorted_b, p.off_sorted_b, p.C_b);
    cp(blk_e_b, p.off_blk_e_b, p.nblk_b);
    cp(n_b, p.off_counts, 1);
    cp(sorted_l, p.off_sorted_l, p.C_l);
    cp(blk_e_l, p.off_blk_e_l, p.nblk_l);
    cp(blk_a_l, p.off_blk_a_l, p.nblk_l);
    cp(n_l, p.off_counts + 4, 1);
    return e == hipSuccess ? MOE_LORA_OK : MOE_LORA_EHIP;
}

int moe_lora_read_status(const moe_lora_desc* d, const void* workspace, size_t ws_bytes,
                         int32_t* status, void* stream) {
    Plan p;
    const int rc = make_plan(d, &p);
    if (rc) return rc;
    if (!workspace || !status) return MOE_LORA_EINVAL;
    if (ws_bytes < p.total) return MOE_LORA_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = const_cast<void*>(workspace);
    return hipMemcpyAsync(status, at<int32_t>(ws, p.off_counts + 16), 4, hipMemcpyDeviceToDevice, s) ==
                   hipSuccess
               ? MOE_LORA_OK
               : MOE_LORA_EHIP;
}

int moe_lora_timing_enable(int32_t max_calls) {
    for (hipEvent_t ev : g_timing.ev) (void)hipEventDestroy(ev);
    g_timing.ev.clear();
    g_timing.ncalls = 0;
    g_timing.max_calls = 0;
    if (max_calls <= 0) return MOE_LORA_OK;
    g_timing.ev.resize(static_cast<size_t>(max_calls) * (MOE_LORA_NKERNELS + 1));
    g_timing.launched.assign(static_cast<size_t>(max_calls) * MOE_LORA_NKERNELS, 1);
    for (auto& ev : g_timing.ev)
        if (hipEventCreate(&ev) != hipSuccess) return MOE_LORA_EHIP;
    g_timing.max_calls = max_calls;
    return MOE_LORA_OK;
}

int moe_lora_timing_read(float* ms, int32_t* ncalls) {
    if (!ms || !ncalls) return MOE_LORA_EINVAL;
    for (int i = 0; i < MOE_LORA_NKERNELS; ++i) ms[i] = 0.f;
    const int n = g_timing.ncalls;
    for (int c = 0; c < n; ++c) {
        hipEvent_t* ev = &g_timing.ev[static_cast<size_t>(c) * (MOE_LORA_NKERNELS + 1)];
        if (hipEventSynchronize(ev[MOE_LORA_NKERNELS]) != hipSuccess) return MOE_LORA_EHIP;
        for (int i = 0; i < MOE_LORA_NKERNELS; ++i) {
            // a kernel the call did not launch reports 0 (its marks enclose
            // only the events' own overhead)
            if (!g_timing.launched[static_cast<size_t>(c) * MOE_LORA_NKERNELS + i]) continue;
            float t = 0.f;
            if (hipEventElapsedTime(&t, ev[i], ev[i + 1]) != hipSuccess) return MOE_LORA_EHIP;
            ms[i] += t;
        }
    }
    *ncalls = n;
    g_timing.ncalls = 0;
    return MOE_LORA_OK;
}

const char* moe_lora_kernel_name(int32_t i) {
    return (i >= 0 && i < MOE_LORA_NKERNELS) ? kKernelNames[i] : "";
}

}  // extern "C"
