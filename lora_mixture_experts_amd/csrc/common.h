// Device-side helpers shared by the gfx950 kernels of libmoelora.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moelora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave index within the workgroup, marked wave-uniform (scalar) so that loops
// bounded by it compile as scalar loops with exact memory wait counts.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Pack 8 floats as bf16 (RNE) into a u32x4 (element 0 in the low half of .x).
__device__ __forceinline__ u32x4 pack_bf16x8(const float* v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = static_cast<uint32_t>(f32_to_bf16_rne(v[2 * i])) |
               (static_cast<uint32_t>(f32_to_bf16_rne(v[2 * i + 1])) << 16);
    return r;
}

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies A[l%16][kslot(l/16, 0..7)] and B[kslot(l/16, 0..7)][l%16];
// the product pairs A and B entries by (lane group, element), so any fixed
// assignment of K indices to the 4x8 slots gives the same sum as long as A and
// B use the same one. Lane l receives D[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// The same load with the non-temporal (streaming) cache policy, for data that
// the launch reads exactly once.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ uint64_t ballot64(bool pred) { return __ballot(pred); }

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Mask of lanes strictly below this lane.
__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace moelora
