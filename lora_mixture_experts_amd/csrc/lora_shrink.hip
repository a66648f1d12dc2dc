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

template <int FN>
__global__ __launch_bounds__(kShrinkThreads) void k_shrink(ShrinkArgs a) {
    const int b = blockIdx.x;
    const int e = a.blk_e_l[b];
    if (e < 0) return;
    const int ad = a.blk_a_l[b];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int kc = lane >> 4, lrow = lane & 15;
    const int nfm = a.bm_l / 16;                         // 16-row fragments in the block (1..16)
    const int nkp = nfm >= kShrinkWaves ? 1 : kShrinkWaves / nfm;  // K parts per fragment
    const int fstride = kShrinkWaves / nkp;              // fragments in flight per round
    const int kp = wave % nkp;
    // K in chunks of 64; this workgroup owns chunks [z0, z1) (its K range)
    // and this wave [q0, q1) of them
    const int nqa = a.K / 64, z = blockIdx.y;
    const int z0 = z * nqa / a.ksplit, z1 = (z + 1) * nqa / a.ksplit;
    const int nq = z1 - z0;
    const int q0 = z0 + kp * nq / nkp, q1 = z0 + (kp + 1) * nq / nkp;

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
    __shared__ f32x4 red[kShrinkWaves][FN][64];

    // rounds of fstride fragments (every wave runs the same number of rounds,
    // so the barriers below match)
    for (int fm = wave / nkp; fm < nfm; fm += fstride) {
        // A operand row (block row fm*16 + lrow); padding rows re-read the
        // block's first (real) row, merging into the same memory requests, and
        // their outputs are never stored. Lane (lrow, kc) reads 32 contiguous
        // bytes (elements 16 kc .. 16 kc + 15) of each 64-wide chunk, so a pair
        // of wave-wide loads consumes whole 128-byte lines.
        int p = a.sorted_l[b * a.bm_l + fm * 16 + lrow];
        if (p >= a.P) p = p_first;
        const size_t row = a.gather_token ? static_cast<size_t>(p / a.top_k)
                                          : static_cast<size_t>(a.slot_of_pair[p]);
        const uint16_t* xrow = a.X + row * a.K + kc * 16;

        f32x4 acc[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 xb[2][2], wb[2][FN][2];
        auto load = [&](int buf, int q) {
            const int k0 = q * 64;
#pragma unroll
            for (int h = 0; h < 2; ++h) xb[buf][h] = ld16(xrow + k0 + 8 * h);
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int h = 0; h < 2; ++h) wb[buf][fn][h] = ld16(brow[fn] + k0 + 8 * h);
        };
        auto compute = [&](int buf) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) acc[fn] = mfma16x16x32(xb[buf][h], wb[buf][fn][h], acc[fn]);
        };
        // fragments made only of padding are skipped (uniform per wave)
        const bool live = a.sorted_l[b * a.bm_l + fm * 16] < a.P;
        const int n = q1 - q0;
        if (live && n > 0) {
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

        // add the K parts of the fragment in order 0..nkp-1 and store
        if (nkp > 1) {
            __syncthreads();  // the previous round's partials have been read
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) red[wave][fn][lane] = acc[fn];
            __syncthreads();
            if (kp == 0) {
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    for (int w = 1; w < nkp; ++w) acc[fn] += red[wave + w][fn][lane];
            }
        }
        if (kp != 0 || !live) continue;
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
                    if (oslot[i] >= 0) a.S[(static_cast<size_t>(z) * a.C_b + oslot[i]) * a.r + j] = acc[fn][i];
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
                        const uint16_t hi = f32_to_bf16_rne(acc[fn][i]);
                        row[j] = hi;
                        row[a.r + j] = f32_to_bf16_rne(acc[fn][i] - bf16_to_f32(hi));
                        if constexpr (FN == 1)
                            for (int q = 2 * a.r + j; q < a.s_hl_stride; q += a.r) row[q] = 0;
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
    switch ((a.r + 15) / 16) {
        case 1: hipLaunchKernelGGL(k_shrink<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(k_shrink<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(k_shrink<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(k_shrink<8>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moelora
