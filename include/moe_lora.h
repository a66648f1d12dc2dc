/*
 * moe_lora.h -- C ABI of libmoelora.so: the fused multi-LoRA Mixture-of-Experts
 * expert layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (AWS ML Blog post "Efficiently serve dozens of fine-tuned models
 * with vLLM on Amazon SageMaker AI and Amazon Bedrock"; Korean summary on
 * agentlenshq.com, section "Multi-LoRA serving for MoE"):
 *   for every token t with adapter a_t (-1 or out of range = no adapter) and
 *   each of its top_k experts e (weights w renormalised over the k chosen):
 *     g  = W_gu[e] x_t + B_gu[a][e] (A_gu[a][e] x_t)        gate_up + LoRA
 *     h  = silu(g[0:I]) * g[I:2I]                              SwiGLU
 *     d  = W_d[e] h + B_d[a][e] (A_d[a][e] h)                  down + LoRA
 *     out_t = sum_j w_j d                                      combine
 *   The LoRA terms are skipped for tokens without an adapter; LoRA scale 1.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates device memory in these calls and never frees caller
 *    memory; intermediates live in the caller's workspace.
 *  - bf16 tensors are raw bf16 bit patterns (uint16). Layouts are row-major
 *    with the reduction dimension contiguous, like a PyTorch Linear weight.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *    work on it; none synchronises the host.
 *  - Calls sharing a workspace must be ordered on one stream; calls on
 *    different streams need distinct workspaces.
 *  - Return value: MOE_LORA_OK (0) or a negative error code; nothing is
 *    enqueued when a call returns an argument error.
 */
#ifndef MOE_LORA_H
#define MOE_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_LORA_OK 0
#define MOE_LORA_EINVAL (-1)     /* bad dimension, null/misaligned pointer, bad block size */
#define MOE_LORA_EWORKSPACE (-2) /* workspace smaller than moe_lora_workspace_bytes() */
#define MOE_LORA_EHIP (-3)       /* a HIP launch or runtime call failed */
#define MOE_LORA_ESCRATCH (-4)   /* moe_lora_forward_noalloc: the call needs more than
                                    MOE_LORA_SCRATCH_BYTES of scratch */

/* Shape of one layer call.
 *   T tokens (T == 0 is a no-op), H hidden size, I expert intermediate size
 *   (gate_up produces 2I), E experts, top_k experts per token (1..min(E,32)),
 *   L adapter slots (0 = no adapters), r LoRA rank (one of 8,16,32,64,128).
 *   H and I must be multiples of 64.
 *   block_m_base / block_m_lora: rows per block of the two alignment views;
 *   0 = library default; else a power of two in [16, 256].
 *   flags: a combination of
 *     MOE_LORA_FLAG_OUT_BF16        out is bf16, rounded to nearest even from
 *                                   the fp32 sum
 *     MOE_LORA_FLAG_SHRINK_LAUNCH   run the two LoRA shrinks as launches of
 *                                   their own even where the library would run
 *                                   them inside the projection launches (for
 *                                   comparison; the results agree to rounding)
 *     MOE_LORA_FLAG_FUSED_COMBINE   fold the weighted top_k sum into the down
 *                                   projection: `out` (fp32) is cleared by the
 *                                   call's first launch and each down row adds
 *                                   w * row into its token's output row with
 *                                   fp32 atomic adds. The order of those adds
 *                                   varies from call to call, so the last bits
 *                                   of `out` may differ between calls when
 *                                   top_k > 2. Without the flag the down
 *                                   projection stores its fp32 rows and a
 *                                   launch of its own sums each token's rows in
 *                                   a fixed order: bitwise repeatable (and
 *                                   faster on MI355X at every measured shape).
 *                                   Not with OUT_BF16.
 *     MOE_LORA_FLAG_NO_SHRINK_WAIT  where the shrinks run inside the
 *                                   projection launches, projection waves do
 *                                   not wait for them: each computes the shrink
 *                                   of its own rows (the path a wait that runs
 *                                   out takes; same results to rounding,
 *                                   slower; for tests of that path)
 *     MOE_LORA_FLAG_ROUTE_LAUNCH    keep the routing and alignment launches
 *                                   where the library would route the batch
 *                                   inside the gate_up launch (decode-sized
 *                                   batches, see moe_lora_plan_info; same
 *                                   results to rounding; for comparison)
 *   any other bit is an error.
 *   Launch tuning (0 = the library's choice; any valid value computes the
 *   same layer up to the order of fp32 sums; these are what a per-shape
 *   tuning table sets, AWS post, section "Tuning kernel configurations for
 *   Amazon SageMaker AI and Amazon Bedrock"):
 *     down_ksplit    K ranges of the down projection, each adding its own fp32
 *                    partial (summed in order by the combine): a divisor of
 *                    I/64; only 1 with base blocks of 128 or 256 rows
 *     shrink_ksplit  K ranges per LoRA block of the two shrinks when they have
 *                    launches of their own (1..4, at most min(H, I)/64); where
 *                    they run inside the projections only their own value
 *     waves_gate_up, waves_down
 *                    16-row base blocks: waves per tile that split its K range
 *                    (1, 2 or 4; each wave keeps >= 4 chunks of 64); other
 *                    block sizes take only 1
 *     frags_gate_up  16-row base blocks: 16-column weight fragments per gate_up
 *                    wave, 4 (32 h columns) or 8 (64 h columns: half the
 *                    waves, each with twice the bytes in flight; needs 16-row
 *                    base blocks, one wave per tile and I a multiple of 64) */
#define MOE_LORA_FLAG_OUT_BF16 1
#define MOE_LORA_FLAG_SHRINK_LAUNCH 2
#define MOE_LORA_FLAG_FUSED_COMBINE 4
#define MOE_LORA_FLAG_NO_SHRINK_WAIT 8
#define MOE_LORA_FLAG_ROUTE_LAUNCH 16
typedef struct moe_lora_desc {
    int32_t T, H, I, E, top_k, L, r;
    int32_t block_m_base, block_m_lora;
    int32_t flags;
    int32_t down_ksplit, shrink_ksplit, waves_gate_up, waves_down;
    int32_t frags_gate_up;
} moe_lora_desc;

/* Weights (device pointers, bf16 bits, 16-byte aligned).
 *   w_gate_up [E][2I][H]   rows 0..I-1 = gate, rows I..2I-1 = up
 *   w_down    [E][H][I]
 *   a_gate_up [L][E][r][H]   LoRA shrink of gate_up (x . A^T)
 *   b_gate_up [L][E][2I][r]  LoRA expand of gate_up
 *   a_down    [L][E][r][I]
 *   b_down    [L][E][H][r]
 *   w_gate_up_packed, w_down_packed: optional copies of w_gate_up / w_down
 *             written by moe_lora_pack_weights (same sizes); NULL = none.
 *             Where a call runs the 16-row kernels they read these instead,
 *             with bitwise-equal results.
 * The four LoRA pointers may be NULL when L == 0. */
typedef struct moe_lora_weights {
    const void *w_gate_up, *w_down;
    const void *a_gate_up, *b_gate_up, *a_down, *b_down;
    const void *w_gate_up_packed, *w_down_packed;
} moe_lora_weights;

/* Copies of the base weights in the order in which the 16-row projection
 * kernels (few rows per expert: decode-sized batches) stream them, for
 * callers that can hold a second copy. In the row layout each wave reads 64
 * rows at the matrix pitch, and pitches with large power-of-two factors
 * (8 or 10 KiB, e.g. hidden sizes 4096 or 5120) stream up to about a fifth
 * slower; in the packed copy the bytes a wave reads for one 64-wide K chunk
 * of its tile form one contiguous 8 KiB block, and its blocks follow each
 * other. The packed order depends only on E, H and I.
 *   w_gate_up, w_down           the row-layout weights (as in moe_lora_weights)
 *   w_gate_up_packed, w_down_packed   outputs, same sizes, 16-byte aligned,
 *                               not overlapping the inputs
 * Either pair may be NULL (that projection is not packed). Enqueued on
 * `stream`. Returns MOE_LORA_EINVAL for a shape the 16-row kernels do not
 * take (I a multiple of 32 and H of 64 are needed). */
int moe_lora_pack_weights(const moe_lora_desc *d, const void *w_gate_up, const void *w_down,
                          void *w_gate_up_packed, void *w_down_packed, void *stream);

/* Human-readable text of an error code (static storage). */
const char *moe_lora_strerror(int code);

/* Host-only argument check, touches no device. `w` may be NULL (then only the
 * descriptor is checked); ws_bytes is compared against the workspace size
 * unless it is (size_t)-1. */
int moe_lora_validate(const moe_lora_desc *d, const moe_lora_weights *w, size_t ws_bytes);

/* Block sizes the library uses for this descriptor (resolves the 0 defaults). */
int moe_lora_block_sizes(const moe_lora_desc *d, int32_t *block_m_base, int32_t *block_m_lora);

/* The launch choices the library makes for this descriptor (0 defaults
 * resolved): base / LoRA block rows, down K ranges, shrink K ranges (0 when
 * L == 0), waves per tile of the two 16-row projections (0 for other block
 * sizes), whether the shrinks run inside the projection launches, whether
 * the combine runs in the down projection, and routing_in_gate_up: 0 = the
 * routing and alignment have launches of their own; 1 = the gate_up launch
 * aligns the batch itself from the routing launch's picks (no alignment
 * launch); 2 = it also routes the batch from the logits (no routing launch
 * either; where E top_k <= 32). 1 and 2 apply to decode-sized batches:
 * T <= 16, E <= 32, top_k <= 8, T top_k <= 64, 16-row blocks, the shrinks
 * inside the projections or no LoRA, one wave per gate_up tile. The routing
 * and alignment are then written by that launch's first workgroup, in the
 * same layouts. frags_gate_up: fragments per 16-row gate_up wave (0 for
 * other block sizes). Host only. */
typedef struct moe_lora_plan_info {
    int32_t block_m_base, block_m_lora, down_ksplit, shrink_ksplit;
    int32_t waves_gate_up, waves_down, shrinks_in_projections, combine_in_down;
    int32_t routing_in_gate_up;
    int32_t frags_gate_up;
} moe_lora_plan_info;
int moe_lora_plan(const moe_lora_desc *d, moe_lora_plan_info *info);

/* Workspace bytes moe_lora_forward needs for this descriptor. */
int moe_lora_workspace_bytes(const moe_lora_desc *d, size_t *bytes);

/* Capacities of the two alignment views (lengths of sorted_b / sorted_l):
 *   C_b = roundup(P + min(E, P)(BMb - 1), BMb),
 *   C_l = roundup(P + min(E L, P)(BMl - 1), BMl),   P = T top_k. */
int moe_lora_align_capacity(const moe_lora_desc *d, int32_t *C_b, int32_t *C_l);

/* Routing (AWS post, section "Implementing multi-LoRA inference for MoE models
 * in vLLM": the router sends each token to its most relevant experts).
 *   logits   f32 [T][E]  (finite values)
 *   topk_ids i32 [T][k]  the k largest logits, largest first; on equal values
 *                        the lower expert id comes first
 *   topk_w   f32 [T][k]  softmax over the k selected logits */
int moe_lora_route(const moe_lora_desc *d, const float *logits, int32_t *topk_ids,
                   float *topk_w, void *stream);

/* Alignment: the compound expert x adapter grouping (AWS post, section
 * "Tuning kernel configurations for Amazon SageMaker AI and Amazon Bedrock":
 * the LoRA kernels carry an extra grid axis over adapters and see the sparsity
 * of several adapters on top of expert routing).
 * Pairs p = t*k + j are ordered by (expert, a', p), a' = adapter if in [0,L)
 * else L. Base view: per expert in id order, its pairs, padded with the
 * sentinel P to a multiple of block_m_base. LoRA view: per (expert, adapter)
 * segment with adapter < L, experts then adapters ascending, padded to
 * block_m_lora. Output (device):
 *   sorted_b i32 [C_b]        slot -> pair id (P = padding)
 *   blk_e_b  i32 [C_b/BMb]    block -> expert (-1 past the used blocks)
 *   n_b      i32 [1]          used length of sorted_b
 *   sorted_l i32 [C_l], blk_e_l, blk_a_l i32 [C_l/BMl], n_l i32 [1]: LoRA view
 *   workspace  device buffer of >= moe_lora_workspace_bytes() bytes, 256-byte
 *              aligned, or NULL. Up to E*(L+1) = 9712 keys: with a workspace,
 *              batches of more than 256 pairs count their keys per range on
 *              many workgroups (the counts and each pair's rank live in the
 *              workspace); NULL is accepted and one workgroup then does all
 *              of it, more slowly for large batches. Above that, up to 36864
 *              keys (e.g. 256 experts x 128 adapters), the counting is spread
 *              over several launches whose histograms live in the workspace:
 *              NULL is then MOE_LORA_EWORKSPACE.
 * The result is deterministic (no order-dependent atomics) and the same on
 * every path.
 * Limit: E*(L+1) <= 36864 and T*top_k <= 2^24. */
int moe_lora_align(const moe_lora_desc *d, const int32_t *topk_ids, const int32_t *adapter_ids,
                   int32_t *sorted_b, int32_t *blk_e_b, int32_t *n_b,
                   int32_t *sorted_l, int32_t *blk_e_l, int32_t *blk_a_l, int32_t *n_l,
                   void *workspace, size_t ws_bytes, void *stream);

/* The whole layer.
 *   x           bf16 [T][H]
 *   logits      f32  [T][E]
 *   adapter_ids i32  [T]   (-1 or any id outside [0, L) = no adapter)
 *   out         f32  [T][H] (overwritten); bf16 bits [T][H] with
 *               MOE_LORA_FLAG_OUT_BF16
 *   workspace   device buffer of >= moe_lora_workspace_bytes() bytes, 256-byte
 *               aligned; it holds the routing, alignment and intermediates of
 *               this call until the next call that uses it.
 * The gate_up and down LoRA expands add into the base projections' results
 * inside the projection kernels (AWS post, section "Kernel optimizations":
 * the LoRA add is fused into the expand). The chosen experts' outputs are
 * then aggregated (AWS post, section "Implementing multi-LoRA inference for
 * MoE models in vLLM") by a fixed-order launch, or inside the down projection
 * with MOE_LORA_FLAG_FUSED_COMBINE. With 16-row base blocks (few rows
 * per expert, the default when T*top_k/E <= 8) and at most 1024 producer
 * waves (LoRA-view block capacity x ceil(r/16) x K ranges of up to 4096),
 * the LoRA shrinks run inside the projection launches too, as producer waves
 * beside the base weight stream; the projection waves wait for them, by
 * polling a counter in the workspace, only before their expand. Such a wait
 * is bounded (about a second of polling): a wave whose wait runs out
 * computes the shrink of its own rows instead, so the output is valid
 * whatever order the hardware starts the waves in, and moe_lora_read_status
 * reports MOE_LORA_STATUS_SHRINK_FALLBACK (a performance signal). */
int moe_lora_forward(const moe_lora_desc *d, const moe_lora_weights *w, const void *x,
                     const float *logits, const int32_t *adapter_ids, void *out,
                     void *workspace, size_t ws_bytes, void *stream);

/* The whole layer without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and errors as
 * moe_lora_forward, which it shares every kernel with, except that the
 * intermediates live in a static device array of the library
 * (MOE_LORA_SCRATCH_BYTES = 64 MiB, 256-byte aligned; each GPU the library
 * runs on holds its own copy from module load until the process ends).
 *  - The call allocates nothing and calls no allocating routine. Its first
 *    call on a device looks up that device's address of the array (a host
 *    call, once per device, with the device current).
 *  - It works on the CURRENT device: a non-null `stream` must belong to it
 *    (else MOE_LORA_EINVAL).
 *  - A call whose moe_lora_workspace_bytes() exceeds MOE_LORA_SCRATCH_BYTES
 *    returns MOE_LORA_ESCRATCH and enqueues nothing (e.g. the decode-sized
 *    batches of the hidden = intermediate = 2880, 32-expert layer fit up to
 *    about 100 tokens; a 6400-token prefill batch does not).
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (each call re-initialises what it reads: its first
 *    launch clears the counters and status word, the alignment fills both
 *    views to capacity). Calls that may overlap on one GPU (different
 *    streams, or host threads without ordering) RACE on the array: order
 *    them on one stream. The read-back calls below do not apply to it. */
#define MOE_LORA_SCRATCH_BYTES ((size_t)64 << 20)
int moe_lora_forward_noalloc(const moe_lora_desc *d, const moe_lora_weights *w, const void *x,
                             const float *logits, const int32_t *adapter_ids, void *out,
                             void *stream);

/* Copy intermediates of the last moe_lora_forward on `workspace` out in pair
 * order (row p = t*k + j); any output may be NULL.
 *   topk_ids i32 [P], topk_w f32 [P]
 *   s1 f32 [P][r]  gate_up shrink x.A^T   (0 rows for pairs without adapter)
 *   h  bf16 [P][I] activation as fed to the down projection
 *   s2 f32 [P][r]  down shrink h.A^T       (0 rows for pairs without adapter)
 *   dn f32 [P][H]  down projection output incl. LoRA, before the weighting;
 *                  not kept with MOE_LORA_FLAG_FUSED_COMBINE (then a non-NULL
 *                  dn is MOE_LORA_EINVAL: the down projection added its rows
 *                  into out directly) */
int moe_lora_read_stages(const moe_lora_desc *d, const void *workspace, size_t ws_bytes,
                         int32_t *topk_ids, float *topk_w, float *s1, uint16_t *h,
                         float *s2, float *dn, void *stream);

/* Status of the last moe_lora_forward with T > 0 on `workspace`: copies one
 * int32 into `status` (a device pointer, like every tensor argument) on
 * `stream`. 0 means every projection wave found the shrink of its launch
 * done; MOE_LORA_STATUS_SHRINK_FALLBACK means at least one wave stopped
 * waiting for it and computed the shrink of its own rows (the output is
 * valid; the call was slower than it should be). Each forward call with
 * T > 0 clears the word first. */
#define MOE_LORA_STATUS_SHRINK_FALLBACK 1
int moe_lora_read_status(const moe_lora_desc *d, const void *workspace, size_t ws_bytes,
                         int32_t *status, void *stream);

/* Copy the alignment of the last moe_lora_forward on `workspace` out (same
 * arrays and layout as moe_lora_align produces); any output may be NULL. */
int moe_lora_read_alignment(const moe_lora_desc *d, const void *workspace, size_t ws_bytes,
                            int32_t *sorted_b, int32_t *blk_e_b, int32_t *n_b,
                            int32_t *sorted_l, int32_t *blk_e_l, int32_t *blk_a_l, int32_t *n_l,
                            void *stream);

/* Per-kernel timing of moe_lora_forward, for profiling only (process-global,
 * not thread-safe). moe_lora_timing_enable(n) makes the next n forward calls
 * record HIP events around each of their kernels on their stream (n = 0 turns
 * it off). moe_lora_timing_read synchronises those events and returns the
 * summed milliseconds per kernel (ms[i], i < MOE_LORA_NKERNELS, in the order
 * of moe_lora_kernel_name) and the number of calls recorded, then resets. A
 * kernel that the calls did not launch reports 0: the shrinks when they ran
 * inside the projection launches, or when L == 0. */
#define MOE_LORA_NKERNELS 7
int moe_lora_timing_enable(int32_t max_calls);
int moe_lora_timing_read(float *ms, int32_t *ncalls);
const char *moe_lora_kernel_name(int32_t i);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LORA_H */
