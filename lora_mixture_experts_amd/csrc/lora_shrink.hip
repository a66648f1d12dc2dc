// LoRA shrink S = X . A^T (rank r) over the LoRA-view blocks, split along K.
//
// Shrink is the skinny "xA" product of the AWS ML Blog post "Efficiently serve
// dozens of fine-tuned models with vLLM on Amazon SageMaker AI and Amazon
// Bedrock", section "Kernel optimizations": splitting the K reduction across
// thread groups balances the load of such skinny products. Here each
// workgroup owns (LoRA block, K split); the four waves of a workgroup share
// the block's rows and interleave 32-wide K steps; partial sums go to a
// per-split slice of S_part instead of atomics, and the consumer (the expand
// fused into the projection kernel) adds the slices in a fixed order, so the
// result is deterministic.
#include "common.h"
#include "kernels.h"

namespace moelora {

constexpr int kShrinkMaxFN = 8;  // r <= 128

template <int FN>
__global__ __launch_bounds__(256) void k_shrink(ShrinkArgs a) {
    const int b = blockIdx.x, split = blockIdx.y;
    const int e = a.blk_e_l[b];
    if (e < 0) return;
    const int ad = a.blk_a_l[b];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kc = lane >> 4, lrow = lane & 15;
    const int Ks = a.K / a.nsplit;
    const int k_begin = split * Ks;
    const int nsteps = Ks / 32;
    const uint16_t* Abase = a.A + (static_cast<size_t>(ad) * a.E + e) * a.r * a.K;

    // B operand rows (LoRA A rows j = fn*16 + lrow), zero past r
    const uint16_t* brow[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int j = fn * 16 + lrow;
        brow[fn] = j < a.r ? Abase + static_cast<size_t>(j) * a.K + k_begin + kc * 8 : nullptr;
    }

    __shared__ f32x4 red[3][kShrinkMaxFN][64];
    const int nfm_total = a.bm_l / 16;
    for (int fm = 0; fm < nfm_total; ++fm) {
        // A operand row (block row fm*16 + lrow)
        const int p = a.sorted_l[b * a.bm_l + fm * 16 + lrow];
        const uint16_t* xrow = nullptr;
        if (p < a.P) {
            const size_t row = a.gather_token ? static_cast<size_t>(p / a.top_k)
                                              : static_cast<size_t>(a.slot_of_pair[p]);
            xrow = a.X + row * a.K + k_begin + kc * 8;
        }
        // a whole 16-row fragment of padding contributes nothing
        if (!__any(xrow != nullptr)) continue;

        f32x4 acc[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        int s = wave;
        for (; s + 12 < nsteps; s += 16) {  // four steps per round, loads first
            u32x4 xa[4], wb[4][FN];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int k0 = (s + 4 * u) * 32;
                xa[u] = xrow ? ld16(xrow + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    wb[u][fn] = brow[fn] ? ld16(brow[fn] + k0) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) acc[fn] = mfma16x16x32(xa[u], wb[u][fn], acc[fn]);
        }
        for (; s < nsteps; s += 4) {
            const int k0 = s * 32;
            const u32x4 xa = xrow ? ld16(xrow + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const u32x4 wb = brow[fn] ? ld16(brow[fn] + k0) : u32x4{0, 0, 0, 0};
                acc[fn] = mfma16x16x32(xa, wb, acc[fn]);
            }
        }
        // reduce the four waves' partial sums (fixed order) and store
        if (wave > 0) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) red[wave - 1][fn][lane] = acc[fn];
        }
        __syncthreads();
        if (wave == 0) {
            // output rows of this lane: 4*kc + i
            int oslot[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = a.sorted_l[b * a.bm_l + fm * 16 + 4 * kc + i];
                oslot[i] = q < a.P ? a.slot_of_pair[q] : -1;
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                f32x4 v = acc[fn];
#pragma unroll
                for (int w = 0; w < 3; ++w) v += red[w][fn][lane];
                const int j = fn * 16 + lrow;
                if (j < a.r) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (oslot[i] >= 0)
                            a.S_part[(static_cast<size_t>(split) * a.C_b + oslot[i]) * a.r + j] = v[i];
                }
            }
        }
        __syncthreads();
    }
}

hipError_t launch_shrink(const ShrinkArgs& a, hipStream_t s) {
    if (a.n_blocks == 0) return hipSuccess;
    const dim3 grid(a.n_blocks, a.nsplit), block(256);
    const int fn = (a.r + 15) / 16;
    switch (fn) {
        case 1: hipLaunchKernelGGL(k_shrink<1>, grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL(k_shrink<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(k_shrink<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(k_shrink<8>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moelora
