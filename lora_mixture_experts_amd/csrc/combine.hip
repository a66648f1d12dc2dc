// Top-k weighted combine and the stage readers.
//
// Combine: out[t] = sum_j w[t][j] * D[slot(t, j)], j ascending, no atomics
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
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ D,
                                                 const int32_t* __restrict__ slot_of_pair,
                                                 const float* __restrict__ w, int k, int H,
                                                 void* __restrict__ out) {
    const int t = blockIdx.x;
    const int n = (blockIdx.y * 256 + threadIdx.x) * 4;
    if (n >= H) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // up to 8 choices per round: all slot/weight loads, then all row loads,
    // then the sums in j order (no load waits on the previous choice's add)
    for (int j0 = 0; j0 < k; j0 += 8) {
        int slot[8];
        float wj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = min(j0 + u, k - 1);
            slot[u] = slot_of_pair[t * k + j];
            wj[u] = w[t * k + j];
        }
        f32x4 d[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            d[u] = *reinterpret_cast<const f32x4*>(D + static_cast<size_t>(slot[u]) * H + n);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u < k) acc += wj[u] * d[u];
    }
    const size_t at = static_cast<size_t>(t) * H + n;
    if (BF16OUT) {
        const uint32_t lo = f32_to_bf16_rne(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[1])) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(acc[3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + at) = make_uint2(lo, hi);
    } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + at) = acc;
    }
}

hipError_t launch_combine(const float* D, const int32_t* slot_of_pair, const float* topk_w,
                          int T, int k, int H, void* out, bool out_bf16, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const dim3 grid(T, (H / 4 + 255) / 256), block(256);
    if (out_bf16)
        hipLaunchKernelGGL(k_combine<true>, grid, block, 0, s, D, slot_of_pair, topk_w, k, H, out);
    else
        hipLaunchKernelGGL(k_combine<false>, grid, block, 0, s, D, slot_of_pair, topk_w, k, H, out);
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
