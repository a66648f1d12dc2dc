// Host-side launchers of the gfx950 kernels (internal to libmoelora).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moelora {

// ---- route + align --------------------------------------------------------
// zero_words[0 .. n_zero) are set to 0 by the same launch (n_zero <= 256);
// with zero_out, rows 0..T-1 of zero_out [T][H] (fp32) are set to 0 too.
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s, int32_t* zero_words = nullptr, int n_zero = 0,
                        float* zero_out = nullptr, int H = 0);

// zero_words[0 .. n_zero) = 0 and, with zero_out, rows 0..T-1 of zero_out
// [T][H] (fp32) = 0: what the routing launch clears, for calls that route
// inside the gate_up launch.
hipError_t launch_zero(int32_t* zero_words, int n_zero, float* zero_out, int T, int H, hipStream_t s);

// Whether the alignment handles E experts x (L adapters + none) keys: in one
// workgroup (its LDS holds the key counts with at least one histogram row),
// or spread over several launches (up to 36864 keys).
bool align_fits(int E, int L);
// Whether P pairs take the one-workgroup path (which needs no workspace).
bool align_single_workgroup(int P, int E, int L);

hipError_t launch_align(const int32_t* topk_ids, const int32_t* adapter_ids, int T, int k,
                        int E, int L, int bm_b, int bm_l, int C_b, int C_l,
                        int32_t* sorted_b, int32_t* blk_e_b, int32_t* n_b,
                        int32_t* sorted_l, int32_t* blk_e_l, int32_t* blk_a_l, int32_t* n_l,
                        int32_t* slot_of_pair, int32_t* lslot_of_pair, int32_t* slot_adapter,
                        int32_t* defer, hipStream_t s);
// ints of workspace the alignment of P pairs uses: the per-range key counts
// and each pair's key and rank, or the multi-launch path's histograms and
// segment starts
int align_defer_ints(int P, int E, int L);

// ---- LoRA shrink ----------------------------------------------------------
// S[slot][j] = X[row] . A[a][e][j] for the real rows of each LoRA-view block.
// gather_token: X row of pair p is x[p / top_k] (else h[slot_of_pair[p]]).
struct ShrinkArgs {
    const uint16_t* X;   // x [T][K] or h [C_b][K]
    int gather_token;
    int K, top_k, P;
    const int32_t* sorted_l;
    const int32_t* blk_e_l;
    const int32_t* blk_a_l;
    const int32_t* slot_of_pair;
    const uint16_t* A;   // [L][E][r][K]
    int E, r, bm_l, n_blocks;
    float* S;            // [ksplit][C_b][r]: one partial sum per K range
    int ksplit, C_b;     // K ranges (workgroups per LoRA block), base-view capacity
    // optional (ksplit == 1 only): S again as bf16 rows [C_b][s_hl_stride] =
    // hi parts (r), lo parts (r), zeros; hi + lo carries S to about 2^-16
    uint16_t* S_hl;
    int s_hl_stride;
};
// Row length (elements) of the bf16 hi/lo copy of S: whole 64-wide K steps.
inline int s_hl_stride_of(int r) { return 2 * r < 64 ? 64 : 2 * r; }
hipError_t launch_shrink(const ShrinkArgs& a, hipStream_t s);
// K ranges for the shrink: several workgroups per LoRA block when there are
// few blocks (decode-sized batches), so that more CUs stream the LoRA A.
// At most kMaxShrinkSplit; the projection kernels add the partials.
constexpr int kMaxShrinkSplit = 4;
int shrink_ksplit(int n_blocks_l, int K, int bm_b);
// K ranges of a shrink run inside a projection kernel: each producer wave
// streams at most kProducerMaxK of K, so the producers finish well before the
// projection's own K loop ends (up to kMaxProducerSplit ranges).
constexpr int kProducerMaxK = 4096;
constexpr int kMaxProducerSplit = 16;
// at most this many producer waves per projection launch (LoRA-view block
// capacity x column fragments x K ranges); beyond it the shrinks get launches
// of their own
constexpr long kMaxProducerUnits = 1024;
inline int producer_ksplit(int K) {
    const int s = (K + kProducerMaxK - 1) / kProducerMaxK;
    return s < 1 ? 1 : (s > kMaxProducerSplit ? kMaxProducerSplit : s);
}

// Where a launch that routes a decode-sized batch itself writes the routing
// and alignment for the launches after it (the layouts of the routing and
// alignment kernels' outputs).
struct LocalOut {
    int32_t* ids;
    float* tw;
    int32_t *sorted_b, *blk_e_b, *n_b, *sorted_l, *blk_e_l, *blk_a_l, *n_l;
    int32_t *slot_of_pair, *lslot_of_pair, *slot_adapter;
    int C_b, C_l;
};

// ---- grouped expert GEMM with fused LoRA expand (+ SwiGLU) ---------------
struct GemmArgs {
    const uint16_t* X;        // gate_up: x [T][K]; down: h [C_b][K]
    int gate_up;              // 1: W = W_gu, epilogue SwiGLU -> h; 0: W = W_d -> D
    const int32_t* sorted_b;
    const int32_t* blk_e_b;
    int P, top_k, bm_b, n_blocks;
    const int32_t* n_b_live;  // padded length of the base view (live blocks x bm_b), from the alignment
    int xcd_slots;            // direct-load kernel: workgroups resident per XCD (set by its launcher)
    const uint16_t* W;        // gate_up: [E][2I][H]; down: [E][H][I]
    const uint16_t* Wp;       // 16-row kernel: W in its packed order (launch_pack_skinny), or null
    int N_out;                // gate_up: I (h columns); down: H
    int K;                    // gate_up: H; down: I
    // LoRA expand
    const int32_t* slot_adapter;  // [C_b] adapter of each base slot, -1 = none / padding
    int L, E, r;
    const float* S;           // [s_split][C_b][r] shrink partials (unused when L == 0)
    int s_split;              // number of shrink partials, summed in order on load
    int C_b;
    const uint16_t* Bl;       // gate_up: [L][E][2I][r]; down: [L][E][H][r]
    // outputs
    uint16_t* h_out;          // [C_b][I]
    float* d_out;             // [ksplit][C_b][H] partial sums over K ranges (down)
    // down only, instead of d_out: the weighted combine in the epilogue;
    // out_acc[t][c] += topk_w[p] * D[p][c] for every real row p = t*top_k + j
    // (fp32 atomic adds into a zeroed out_acc [T][H])
    float* out_acc;
    const float* topk_w;
    int ksplit;               // down only: the K range is cut into ksplit equal parts
    int ksw;                  // 16-row blocks: waves per tile splitting its K range (1, 2 or 4)
    int frags;                // 16-row gate_up: 16-column fragments per wave (4, or 8 with ksw 1)
    int w_stream;             // 128/256-row blocks: weight tiles read by about one block each (nt loads)
    // optional bf16 hi/lo copy of S (see ShrinkArgs); the direct-load kernel
    // then runs the expand as extra stages of its LDS pipeline
    const uint16_t* S_hl;
    int s_hl_stride;
    // LoRA shrink run inside this launch (16-row blocks only; prod_units == 0:
    // S comes from a separate shrink launch). The first prod_units
    // workgroups of the grid are producer waves: unit u computes the 16
    // columns (u % prod_ncf) of S, over K range (u / prod_ncf) % s_split, for
    // the rows of LoRA-view block u / (prod_ncf * s_split), writes them to
    // S_out and then counts itself in *done. The projection waves run their
    // base K loop first and wait for every live unit before the expand.
    int prod_units;
    int prod_ncf;
    int gather_token;             // producer X row of pair p: x[p / top_k] (1) or h[slot_of_pair[p]] (0)
    const int32_t* sorted_l;
    const int32_t* blk_e_l;
    const int32_t* blk_a_l;
    const int32_t* slot_of_pair;
    const uint16_t* Al;           // gate_up: [L][E][r][H]; down: [L][E][r][I]
    int bm_l;
    float* S_out;                 // the buffer S points at
    int32_t* done;                // producer completion count, zero at launch
    const int32_t* n_l;           // padded LoRA-view length (live LoRA blocks x bm_l)
    int32_t* status;              // the call's status word (kStatus* bits), zero at launch
    int max_polls;                // polls of a projection wave waiting for the producers
    // gate_up with 16-row blocks on a decode-sized batch (local_route_fits):
    // with local set, every wave aligns the batch itself instead of reading
    // the alignment: from local_ids (the routing launch's picks) when given,
    // else routing it first from logits [T][E]; adapters from adapter_ids [T].
    // Block b of the grid is expert b (n_blocks = E); workgroup 0 writes the
    // alignment (and, from logits, the routing) to pub for the launches that
    // follow
    int local;
    const float* logits;
    const int32_t* local_ids;
    const int32_t* adapter_ids;
    int T;
    LocalOut pub;
};
// status bit: a projection wave stopped waiting for the producers and
// computed the shrink of its own rows (output valid, slower)
constexpr int32_t kStatusShrinkFallback = 1;
constexpr int kMaxProducerPolls = 1 << 20;
// W in the 16-row projection kernel's packed order (see k_pack_skinny);
// false when the shape does not suit that kernel.
bool pack_skinny_supported(int N_out, int K, int gate_up);
hipError_t launch_pack_skinny(const uint16_t* W, uint16_t* Wp, int E, int N_out, int K, int gate_up,
                              hipStream_t s);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// Whether a tile configuration exists for these sizes.
bool gemm_supported(int N_out, int K, int gate_up, int bm_b);
// Whether ksw waves per tile (1, 2 or 4) may split the K range of a 16-row
// (skinny) projection whose workgroups each own K / ksplit.
bool skinny_waves_ok(int K, int ksplit, int ksw);
// K splits for the down projection: enough waves to fill the chip when the
// grid is small (few blocks, few column tiles, long K); 1 for the large-block
// kernels. Always divides K / 64.
int gemm_down_ksplit(int N_out, int K, int bm_b, int n_blocks);

// ---- combine + stage readers --------------------------------------------
// out[t] = sum_j w[t][j] * (sum_s D[s][slot(t, j)]), s = 0..nsplit-1 (the
// K-range partial sums of the down projection), all in a fixed order.
// out: fp32 [T][H], or bf16 bits [T][H] when out_bf16
hipError_t launch_combine(const float* D, int nsplit, int C_b, const int32_t* slot_of_pair,
                          const float* topk_w, int T, int k, int H, void* out, bool out_bf16,
                          hipStream_t s);

// dst[p][c] = sum_s src_part[s][slot(p)][c]; rows with mask[p] < 0 are 0
// (mask may be null).
hipError_t launch_gather_rows_f32(const float* src_part, int nsplit, int C_b, int ncols,
                                  const int32_t* slot_of_pair, const int32_t* mask, int P,
                                  float* dst, hipStream_t s);
hipError_t launch_gather_rows_bf16(const uint16_t* src, int ncols, const int32_t* slot_of_pair,
                                   int P, uint16_t* dst, hipStream_t s);

}  // namespace moelora
