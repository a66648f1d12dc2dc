// Top-k weighted combine and the stage readers.
//
// Combine: out[t] = sum_j w[t][j] * D[slot(t, j)], j ascending, no atomics,
// where D is the sum of the down projection's K-range partials (in order)
// (AWS ML Blog post "Efficiently serve dozens of fine-tuned models with vLLM
// on Amazon SageMaker AI and Amazon Bedrock", section "Implementing multi-LoRA
// inference for MoE models in vLLM": the chosen experts' outputs are
// aggregated). Each thread owns four consecutive hidden columns of one token.
// The sum is formed in fp32; the bf16 output form rounds it once, to nearest
// even, at the store.
#include "common.h"
#include "kernels.h"

namespace moelora {

template <bool BF16OUT>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ D, int nsplit, int C_b,
                                                 const int32_t* __restrict__ slot_of_pair,
                                                 const float* __restrict__ w, int k, int H,
                                                 void* __restrict__ out) {
    const int t = blockIdx.x;
    const int n = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (n >= H) return;
    const size_t part = static_cast<size_t>(C_b) * H;  // one K-range partial
    // items q = j * nsplit + s in ascending order, 8 per round: the slot loads
    // of a round, then its row loads, then the adds; d holds choice j's sum
    // over s, folded into acc (times w_j) when the next choice starts
    const int nq = k * nsplit;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, d = {0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < nq; q0 += 8) {
        int slot[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) slot[u] = slot_of_pair[t * k + min(q0 + u, nq - 1) / nsplit];
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sp = min(q0 + u, nq - 1) % nsplit;
            v[u] = *reinterpret_cast<const f32x4*>(D + sp * part + static_cast<size_t>(slot[u]) * H + n);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = q0 + u;
            if (q < nq) {
                if (q > 0 && q % nsplit == 0) {
                    acc += w[t * k + q / nsplit - 1] * d;
                    d = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                d += v[u];
            }
        }
    }
    acc += w[t * k + k - 1] * d;
    const size_t at = static_cast<size_t>(t) * H + n;
    if (BF16OUT) {
        const uint32_t lo = f32_to_bf16_rne(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[1])) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + at) = make_uint2(lo, hi);
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + at) = acc;
    }
}

hipError_t launch_combine(const float* D, int nsplit, int C_b, const int32_t* slot_of_pair,
                          const float* topk_w, int T, int k, int H, void* out, bool out_bf16,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    const dim3 grid(T, (H / 4 + 255) / 256), block(256);
    if (out_bf16)
        hipLaunchKernelGGL(k_combine<true>, grid, block, 0, s, D, nsplit, C_b, slot_of_pair, topk_w, k, H, out);
    else
        hipLaunchKernelGGL(k_combine<false>, grid, block, 0, s, D, nsplit, C_b, slot_of_pair, topk_w, k, H, out);
    return hipGetLastError();
}

// dst[p][c] = sum_s src[s][slot(p)][c]; 0 for pairs with mask[p] < 0.
__global__ __launch_bounds__(256) void k_gather_f32(const float* __restrict__ src, int nsplit,
                                                    int C_b, int ncols,
                                                    const int32_t* __restrict__ slot_of_pair,
                                                    const int32_t* __restrict__ mask,
                                                    float* __restrict__ dst) {
    const int p = blockIdx.x;
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= ncols) return;
    float v = 0.f;
    if (!mask || mask[p] >= 0) {
        const int slot = slot_of_pair[p];
        for (int s = 0; s < nsplit; ++s) v += src[(static_cast<size_t>(s) * C_b + slot) * ncols + c];
    }
    dst[static_cast<size_t>(p) * ncols + c] = v;
}

hipError_t launch_gather_rows_f32(const float* src_part, int nsplit, int C_b, int ncols,
                                  const int32_t* slot_of_pair, const int32_t* mask, int P,
                                  float* dst, hipStream_t s) {
    if (P == 0) return hipSuccess;
    const dim3 grid(P, (ncols + 255) / 256), block(256);
    hipLaunchKernelGGL(k_gather_f32, grid, block, 0, s, src_part, nsplit, C_b, ncols, slot_of_pair,
                       mask, dst);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_gather_bf16(const uint16_t* __restrict__ src, int ncols,
                                                     const int32_t* __restrict__ slot_of_pair,
                                                     uint16_t* __restrict__ dst) {
    const int p = blockIdx.x;
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= ncols) return;
    dst[static_cast<size_t>(p) * ncols + c] = src[static_cast<size_t>(slot_of_pair[p]) * ncols + c];
}

hipError_t launch_gather_rows_bf16(const uint16_t* src, int ncols, const int32_t* slot_of_pair,
                                   int P, uint16_t* dst, hipStream_t s) {
    if (P == 0) return hipSuccess;
    const dim3 grid(P, (ncols + 255) / 256), block(256);
    hipLaunchKernelGGL(k_gather_bf16, grid, block, 0, s, src, ncols, slot_of_pair, dst);
    return hipGetLastError();
}

}  // namespace moelora
