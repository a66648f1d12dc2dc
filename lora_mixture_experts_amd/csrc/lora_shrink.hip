// LoRA shrink S = X . A^T (rank r) over the LoRA-view blocks.
//
// Shrink is the skinny "xA" product of the AWS ML Blog post "Efficiently serve
// dozens of fine-tuned models with vLLM on Amazon SageMaker AI and Amazon
// Bedrock", section "Kernel optimizations": splitting the K reduction across
// thread groups balances the load of such skinny products. Here one
// 256-thread workgroup owns a LoRA block (rows of one expert x adapter
// segment) and one K range of it; its 4 waves split the block into (16-row
// fragment, K part) pairs, so even a block with a single real row keeps 4
// waves streaming A (small workgroups let several blocks share a CU, which
// measured faster than 16-wave workgroups). The K parts are added through LDS
// in a fixed order: no atomics, no cross-workgroup traffic, and the result is
// deterministic. Each output element is written once, in base-slot order, for
// the expand fused into the projection kernel.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moelora {

constexpr int kShrinkThreads = 256;
constexpr int kShrinkWaves = kShrinkThreads / 64;

// At most this many 16-row fragments are multiplied together against one
// load of a wave's LoRA A chunk (bounded by the registers the accumulators
// and operand buffers take); the launcher takes min(fragments per block, it).
template <int FN>
constexpr int shrink_group() { return FN <= 2 ? 4 : 8 / FN; }

template <int FN, int G>
__global__ __launch_bounds__(kShrinkThreads) void k_shrink(ShrinkArgs a) {
    const int b = blockIdx.x;
    const int e = a.blk_e_l[b];
    if (e < 0) return;
    const int ad = a.blk_a_l[b];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int kc = lane >> 4, lrow = lane & 15;
    const int nfm = a.bm_l / 16;  // 16-row fragments in the block (1..16)
    // K in chunks of 64; this workgroup owns chunks [z0, z1) (its K range)
    // and wave w the w-th quarter [q0, q1) of them, for every fragment
    const int nqa = a.K / 64, z = blockIdx.y;
    const int z0 = z * nqa / a.ksplit, z1 = (z + 1) * nqa / a.ksplit;
    const int nq = z1 - z0;
    const int q0 = z0 + wave * nq / kShrinkWaves, q1 = z0 + (wave + 1) * nq / kShrinkWaves;

    // B operand rows (LoRA A rows j = fn*16 + lrow); columns j >= r (r = 8)
    // re-read row j - 8 and are never stored, so loads stay unconditional
    const uint16_t* Abase = a.A + (static_cast<size_t>(ad) * a.E + e) * a.r * a.K;
    const uint16_t* brow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int j = fn * 16 + lrow;
        brow[fn] = Abase + static_cast<size_t>(j < a.r ? j : j - 8) * a.K + kc * 16;
    }
    const int p_first = a.sorted_l[b * a.bm_l];
    __shared__ f32x4 red[kShrinkWaves][G][FN][64];

    // groups of G fragments: each K chunk of A is loaded once per wave and
    // multiplied against the chunk of every fragment of the group
    for (int fg = 0; fg < nfm; fg += G) {
        // A operand rows (block row fm*16 + lrow); padding rows re-read the
        // block's first (real) row, merging into the same memory requests, and
        // their outputs are never stored. Lane (lrow, kc) reads 32 contiguous
        // bytes (elements 16 kc .. 16 kc + 15) of each 64-wide chunk, so a pair
        // of wave-wide loads consumes whole 128-byte lines. Fragments made
        // only of padding (or past the block) are skipped (uniform per wave).
        const uint16_t* xrow[G];
        bool live[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int fm = fg + g;
            live[g] = fm < nfm && a.sorted_l[b * a.bm_l + min(fm, nfm - 1) * 16] < a.P;
            int p = a.sorted_l[b * a.bm_l + min(fm, nfm - 1) * 16 + lrow];
            if (p >= a.P) p = p_first;
            const size_t row = a.gather_token ? static_cast<size_t>(p / a.top_k)
                                              : static_cast<size_t>(a.slot_of_pair[p]);
            xrow[g] = a.X + row * a.K + kc * 16;
        }

        f32x4 acc[G][FN];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[g][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 xb[2][G][2], wb[2][FN][2];
        auto load = [&](int buf, int q) {
            const int k0 = q * 64;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int h = 0; h < 2; ++h) wb[buf][fn][h] = ld16(brow[fn] + k0 + 8 * h);
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (live[g]) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) xb[buf][g][h] = ld16(xrow[g] + k0 + 8 * h);
                }
        };
        auto compute = [&](int buf) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    if (live[g]) {
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn)
                            acc[g][fn] = mfma16x16x32(xb[buf][g][h], wb[buf][fn][h], acc[g][fn]);
                    }
        };
        const int n = q1 - q0;
        if (n > 0) {
            // two-stage register pipeline (as in the skinny projection kernel)
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

        // add the four K quarters of each fragment in order 0..3 (wave g
        // finishes fragment fg + g) and store
        __syncthreads();  // the previous group's partials have been read
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) red[wave][g][fn][lane] = acc[g][fn];
        __syncthreads();
        for (int g = wave; g < G; g += kShrinkWaves) {
            const int fm = fg + g;
            if (fm >= nfm || a.sorted_l[b * a.bm_l + fm * 16] >= a.P) continue;
            f32x4 sum[FN];
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                sum[fn] = red[0][g][fn][lane];
                for (int w = 1; w < kShrinkWaves; ++w) sum[fn] += red[w][g][fn][lane];
            }
            int oslot[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = a.sorted_l[b * a.bm_l + fm * 16 + 4 * kc + i];
                oslot[i] = q < a.P ? a.slot_of_pair[q] : -1;
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int j = fn * 16 + lrow;
                if (j < a.r) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (oslot[i] >= 0) a.S[(static_cast<size_t>(z) * a.C_b + oslot[i]) * a.r + j] = sum[fn][i];
                }
            }
            if (a.S_hl) {
                // the bf16 copy: hi = bf16(s), lo = bf16(s - hi), then zeros to
                // the row end (only when 2r is below one 64-wide K step)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (oslot[i] < 0) continue;
                    uint16_t* row = a.S_hl + static_cast<size_t>(oslot[i]) * a.s_hl_stride;
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        const int j = fn * 16 + lrow;
                        if (j < a.r) {
                            const uint16_t hi = f32_to_bf16_rne(sum[fn][i]);
                            row[j] = hi;
                            row[a.r + j] = f32_to_bf16_rne(sum[fn][i] - bf16_to_f32(hi));
                            if constexpr (FN == 1)
                                for (int q = 2 * a.r + j; q < a.s_hl_stride; q += a.r) row[q] = 0;
                        }
                    }
                }
            }
        }
    }
}

int shrink_ksplit(int n_blocks_l, int K, int bm_b) {
    // Only for long K, few LoRA blocks and small base blocks. A CU streams a
    // LoRA A at a rate bounded by the loads it can keep in flight, so each
    // such block's K is cut into ranges on separate CUs (at least 4 chunks
    // of 64 each). The projection kernels add the partials when they load S;
    // at K below 4096 that extra load cost as much as the split saved.
    // (the wide-expert layer with 64-row base blocks: 490 us split 4 ways
    // against 505 us unsplit)
    if (bm_b > 64 || n_blocks_l <= 0 || n_blocks_l >= 128 || K < 4096) return 1;
    return std::max(1, std::min({kMaxShrinkSplit, (256 + n_blocks_l - 1) / n_blocks_l, K / 64 / 4}));
}

hipError_t launch_shrink(const ShrinkArgs& a, hipStream_t s) {
    if (a.n_blocks == 0) return hipSuccess;
    if (a.bm_l < 16 || a.bm_l > 256 || (a.bm_l & (a.bm_l - 1))) return hipErrorInvalidValue;
    if (a.ksplit < 1 || a.ksplit > a.K / 64) return hipErrorInvalidValue;
    if (a.S_hl && (a.ksplit != 1 || a.s_hl_stride != s_hl_stride_of(a.r))) return hipErrorInvalidValue;
    const dim3 grid(a.n_blocks, a.ksplit), block(kShrinkThreads);
    const int nfm = a.bm_l / 16;
#define MOELORA_SHRINK(FN)                                                                            \
    do {                                                                                              \
        const int g = std::min(nfm, shrink_group<FN>());                                              \
        if (g == 1) hipLaunchKernelGGL((k_shrink<FN, 1>), grid, block, 0, s, a);                      \
        if constexpr (shrink_group<FN>() >= 2)                                                        \
            if (g == 2) hipLaunchKernelGGL((k_shrink<FN, (shrink_group<FN>() >= 2 ? 2 : 1)>), grid, block, 0, s, a); \
        if constexpr (shrink_group<FN>() >= 4)                                                        \
            if (g == 4) hipLaunchKernelGGL((k_shrink<FN, (shrink_group<FN>() >= 4 ? 4 : 1)>), grid, block, 0, s, a); \
    } while (0)
    switch ((a.r + 15) / 16) {
        case 1: MOELORA_SHRINK(1); break;
        case 2: MOELORA_SHRINK(2); break;
        case 4: MOELORA_SHRINK(4); break;
        case 8: MOELORA_SHRINK(8); break;
        default: return hipErrorInvalidValue;
    }
#undef MOELORA_SHRINK
    return hipGetLastError();
}

}  // namespace moelora
