// Grouped expert projections on bf16 MFMA (gfx950, v_mfma_f32_16x16x32_bf16)
// with the LoRA expand fused in, plus SwiGLU for gate_up.
//
// One launch covers every expert: a workgroup takes one block of the base
// alignment view (rows of a single expert, gathered through sorted_b) and one
// tile of output columns. After the base K loop the LoRA expand runs as extra
// MFMA K steps on the same accumulators, once per adapter present among the
// block's rows: acc += S . B^T with S (the shrink output) split into a bf16
// high part and a bf16 low part so that the rank-r product keeps ~16 bits of
// S. This is the "LoRA add fused into the expand" of the AWS ML Blog post
// "Efficiently serve dozens of fine-tuned models with vLLM on Amazon SageMaker
// AI and Amazon Bedrock" (section "Kernel optimizations"), taken one step
// further: the expand writes straight into the base accumulator in registers.
//
// gate_up: the tile's 16-column fragments alternate gate / up for the same
// activation columns, so every lane holds matching gate and up values and the
// SwiGLU epilogue h = silu(gate) * up runs in registers; h is stored in bf16.
// down: the fp32 result is stored per base slot for the weighted combine.
#include "common.h"
#include "kernels.h"

namespace moelora {

// W row of fragment f (16 rows each) of a tile whose first output column is c0.
template <bool GATEUP>
__device__ __forceinline__ int w_row_of_frag(int f, int c0, int I) {
    if (GATEUP) return ((f & 1) ? I : 0) + c0 + 16 * (f >> 1);
    return c0 + 16 * f;
}

__device__ __forceinline__ int row_adapter(const GemmArgs& a, int slot) { return a.slot_adapter[slot]; }

// S row chunk (8 values starting at j0) as hi/lo bf16 operands; zero when the
// row is not in the current adapter run or j is past r.
__device__ __forceinline__ void load_s_hilo(const GemmArgs& a, int slot, bool in_run, int j0,
                                            u32x4& hi, u32x4& lo) {
    float v[8], rest[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = 0.f;
    if (in_run && j0 < a.r) {
        const float* src = a.S + static_cast<size_t>(slot) * a.r + j0;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[q] = x0[q];
            v[4 + q] = x1[q];
        }
    }
    hi = pack_bf16x8(v);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t word = hi[q >> 1];
        const uint16_t bits = (q & 1) ? static_cast<uint16_t>(word >> 16) : static_cast<uint16_t>(word);
        rest[q] = v[q] - bf16_to_f32(bits);
    }
    lo = pack_bf16x8(rest);
}

// LoRA B operand chunk: rows of Bl[ad][e] (each r wide), 8 values at j0.
__device__ __forceinline__ u32x4 load_lora_b(const GemmArgs& a, int Nw, int ad, int e, int wrow,
                                             int j0) {
    if (j0 >= a.r) return u32x4{0, 0, 0, 0};
    const uint16_t* src = a.Bl + ((static_cast<size_t>(ad) * a.E + e) * Nw + wrow) * a.r + j0;
    return ld16(src);
}

// ===========================================================================
// Skinny variant: 16-row blocks (few rows per expert: the weights are
// streamed from HBM once and each byte feeds at most 16 rows).
//
// One wave is one workgroup and owns a 16-row x (16 FN)-column output tile
// over the whole K range, so there is no cross-wave reduction, no LDS and no
// barrier; thousands of independent waves fill the chip in a single round.
// In each 64-wide K chunk lane (n, g) reads 32 contiguous bytes of weight row
// n (elements 16 g .. 16 g + 15), so a wave-wide pair of loads consumes whole
// 128-byte lines of 16 rows; the two 16-byte halves feed two MFMA K steps and
// the activation operand uses the same K assignment. Loads of chunk q+1 are in
// flight while chunk q is multiplied.
template <bool GATEUP, int FN>
__global__ __launch_bounds__(64) void k_gemm_skinny(GemmArgs a) {
    const int b = blockIdx.y, tile = blockIdx.x;
    const int e = a.blk_e_b[b];
    if (e < 0) return;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, lrow = lane & 15;
    const int I = GATEUP ? a.N_out : 0;
    const int Nw = GATEUP ? 2 * a.N_out : a.N_out;
    constexpr int kCols = GATEUP ? FN * 8 : FN * 16;  // output columns per wave
    const int c0 = tile * kCols;
    const int K = a.K;

    const int slot = b * 16 + lrow;
    // Padding rows (sentinel P) re-read the block's first row, which is always
    // a real row: the duplicate addresses merge into the same memory request,
    // MFMA output rows depend only on their own A row, and padding rows are
    // never consumed, so no masking is needed and every load is issued
    // unconditionally (exact wait counts).
    const uint16_t* xrow;
    if (GATEUP) {
        int p = a.sorted_b[slot];
        if (p >= a.P) p = a.sorted_b[b * 16];
        xrow = a.X + static_cast<size_t>(p / a.top_k) * K + g * 16;
    } else {
        xrow = a.X + static_cast<size_t>(slot) * K + g * 16;
    }
    const uint16_t* wrow[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f)
        wrow[f] = a.W + (static_cast<size_t>(e) * Nw + w_row_of_frag<GATEUP>(f, c0, I) + lrow) * K +
                  g * 16;

    f32x4 acc[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 xb[2][2], wb[2][FN][2];
    auto load = [&](int buf, int q) {
        const int k0 = q * 64;
#pragma unroll
        for (int h = 0; h < 2; ++h) xb[buf][h] = ld16(xrow + k0 + 8 * h);
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int h = 0; h < 2; ++h) wb[buf][f][h] = ld16(wrow[f] + k0 + 8 * h);
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int f = 0; f < FN; ++f) acc[f] = mfma16x16x32(xb[buf][h], wb[buf][f][h], acc[f]);
    };

    const int nq = K / 64;
    load(0, 0);
    __builtin_amdgcn_sched_barrier(0);

    // LoRA expand first (its inputs are ready before this kernel starts), so
    // its latency overlaps the first weight loads: acc += S . B^T for every
    // adapter present among the 16 rows.
    if (a.L > 0) {
        const int my_a = row_adapter(a, slot);
        bool pending = my_a >= 0;
        while (true) {
            const uint64_t m = ballot64(pending);
            if (m == 0) break;
            const int leader = __ffsll(static_cast<long long>(m)) - 1;
            const int acur = __shfl(my_a, leader);
            const bool in_run = pending && my_a == acur;
            pending = pending && !in_run;
            for (int kk = 0; kk < a.r; kk += 32) {
                const int j0 = kk + g * 8;
                u32x4 hi, lo, bb[FN];
#pragma unroll
                for (int f = 0; f < FN; ++f)
                    bb[f] = load_lora_b(a, Nw, acur, e, w_row_of_frag<GATEUP>(f, c0, I) + lrow, j0);
                load_s_hilo(a, slot, in_run, j0, hi, lo);
#pragma unroll
                for (int f = 0; f < FN; ++f) {
                    acc[f] = mfma16x16x32(hi, bb[f], acc[f]);
                    acc[f] = mfma16x16x32(lo, bb[f], acc[f]);
                }
            }
        }
    }

    // Two-stage register pipeline with one back edge and no early exit, so
    // the prefetch stays in flight across iterations; scheduling barriers stop
    // the compiler from sinking loads next to their use. A prefetch past the
    // end re-reads the last chunk (in bounds) and is discarded.
    int q = 0;
    for (int i = 0; i + 1 < nq; i += 2, q += 2) {
        load(1, q + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(0);
        __builtin_amdgcn_sched_barrier(0);
        load(0, min(q + 2, nq - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (nq & 1) compute(0);

    const int orow0 = b * 16 + 4 * g;
    if (GATEUP) {
#pragma unroll
        for (int u = 0; u < FN / 2; ++u) {
            const int col = c0 + 16 * u + lrow;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.h_out[static_cast<size_t>(orow0 + i) * a.N_out + col] =
                    f32_to_bf16_rne(silu(acc[2 * u][i]) * acc[2 * u + 1][i]);
        }
    } else {
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            const int col = c0 + 16 * f + lrow;
#pragma unroll
            for (int i = 0; i < 4; ++i) a.d_out[static_cast<size_t>(orow0 + i) * a.N_out + col] = acc[f][i];
        }
    }
}

// ===========================================================================
// Tiled variant: BM x BNT tile (BNT = GEMM columns), BK = 64, LDS double
// buffer with an XOR swizzle of the 16-byte chunks, 2 x 2 waves.
template <int BM, int BNT>
struct TileCfg {
    static constexpr int FM = BM / 32;   // 16-row fragments per wave
    static constexpr int FN = BNT / 32;  // 16-col fragments per wave
    static constexpr int A_LD = BM / 32;   // 16-byte chunks per thread per stage
    static constexpr int B_LD = BNT / 32;
    static constexpr int A_ELEMS = BM * 64;
    static constexpr int B_ELEMS = BNT * 64;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

template <int BM, int BNT, bool GATEUP>
__global__ __launch_bounds__(256) void k_gemm_tiled(GemmArgs a) {
    using C = TileCfg<BM, BNT>;
    constexpr int FM = C::FM, FN = C::FN;
    const int b = blockIdx.x;
    const int e = a.blk_e_b[b];
    if (e < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int wm = wave >> 1, wn = wave & 1;
    const int kc = lane >> 4, lrow = lane & 15;
    const int I = GATEUP ? a.N_out : 0;
    const int Nw = GATEUP ? 2 * a.N_out : a.N_out;
    const int c0 = blockIdx.y * (GATEUP ? BNT / 2 : BNT);
    const int K = a.K;
    const int row0 = b * BM;

    __shared__ __attribute__((aligned(16))) uint16_t As[2][C::A_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][C::B_ELEMS];

    // global -> LDS assignment: thread owns rows tid/8 + 32*i, chunk tid%8
    const int ld_row = tid >> 3, ld_chunk = tid & 7;
    // padding rows re-read the block's first (real) row; their outputs are
    // never consumed
    const uint16_t* asrc[C::A_LD];
    const int p_first = a.sorted_b[row0];
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
        const int r = ld_row + 32 * i;
        const int slot = row0 + r;
        if (GATEUP) {
            const int p = a.sorted_b[slot];
            asrc[i] = a.X + static_cast<size_t>((p < a.P ? p : p_first) / a.top_k) * K + ld_chunk * 8;
        } else {
            asrc[i] = a.X + static_cast<size_t>(slot) * K + ld_chunk * 8;
        }
    }
    const uint16_t* bsrc[C::B_LD];
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
        const int r = ld_row + 32 * i;
        const int wr = w_row_of_frag<GATEUP>(r >> 4, c0, I) + (r & 15);
        bsrc[i] = a.W + (static_cast<size_t>(e) * Nw + wr) * K + ld_chunk * 8;
    }

    u32x4 ra[C::A_LD], rb[C::B_LD];
    auto gload = [&](int kt) {
        const int k0 = kt * 64;
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i) ra[i] = ld16(asrc[i] + k0);
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i) rb[i] = ld16(bsrc[i] + k0);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::A_LD; ++i)
            *reinterpret_cast<u32x4*>(&As[buf][swz(ld_row + 32 * i, ld_chunk)]) = ra[i];
#pragma unroll
        for (int i = 0; i < C::B_LD; ++i)
            *reinterpret_cast<u32x4*>(&Bs[buf][swz(ld_row + 32 * i, ld_chunk)]) = rb[i];
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / 64;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int chunk = kk * 4 + kc;
            u32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const u32x4*>(
                    &As[buf][swz(wm * (BM / 2) + i * 16 + lrow, chunk)]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = *reinterpret_cast<const u32x4*>(
                    &Bs[buf][swz(wn * (BNT / 2) + j * 16 + lrow, chunk)]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = mfma16x16x32(fa[i], fb[j], acc[i][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // LoRA expand: per distinct adapter among this wave's rows
    const int wrow_base = row0 + wm * (BM / 2);
    if (a.L > 0) {
        int my_a[FM];
        bool pending[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            my_a[i] = row_adapter(a, wrow_base + i * 16 + lrow);
            pending[i] = my_a[i] >= 0;
        }
        while (true) {
            int cand = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                if (pending[i] && my_a[i] < cand) cand = my_a[i];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) cand = min(cand, __shfl_xor(cand, off));
            if (cand == 0x7fffffff) break;
            for (int kk = 0; kk < a.r; kk += 32) {
                const int j0 = kk + kc * 8;
                u32x4 bb[FN];
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bb[j] = load_lora_b(a, Nw, cand, e,
                                        w_row_of_frag<GATEUP>(wn * FN + j, c0, I) + lrow, j0);
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const bool in_run = pending[i] && my_a[i] == cand;
                    if (!__any(in_run)) continue;
                    u32x4 hi, lo;
                    load_s_hilo(a, wrow_base + i * 16 + lrow, in_run, j0, hi, lo);
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        acc[i][j] = mfma16x16x32(hi, bb[j], acc[i][j]);
                        acc[i][j] = mfma16x16x32(lo, bb[j], acc[i][j]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
                if (pending[i] && my_a[i] == cand) pending[i] = false;
        }
    }

    // epilogue
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int orow0 = wrow_base + i * 16 + 4 * kc;
        if (GATEUP) {
#pragma unroll
            for (int j = 0; j < FN; j += 2) {
                const int col = c0 + 16 * ((wn * FN + j) >> 1) + lrow;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a.h_out[static_cast<size_t>(orow0 + q) * a.N_out + col] =
                        f32_to_bf16_rne(silu(acc[i][j][q]) * acc[i][j + 1][q]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = c0 + 16 * (wn * FN + j) + lrow;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a.d_out[static_cast<size_t>(orow0 + q) * a.N_out + col] = acc[i][j][q];
            }
        }
    }
}

// ---------------------------------------------------------------------------
static int pick_bnt(int N_out, int gate_up, int bm) {
    // GEMM columns per tile; gate_up tiles cover BNT/2 activation columns
    const int prefs_big[] = {192, 128, 64};
    for (int bnt : prefs_big) {
        if (bm == 256 && bnt > 128) continue;
        const int cols = gate_up ? bnt / 2 : bnt;
        if (N_out % cols == 0) return bnt;
    }
    return 0;
}

#ifndef MOELORA_SKINNY_FN
#define MOELORA_SKINNY_FN 4
#endif

// fragments per skinny workgroup: 8 when the column count allows, else 4
static int skinny_fn(int N_out, int gate_up) {
    const int cols8 = gate_up ? 64 : 128;
    return (MOELORA_SKINNY_FN == 8 && N_out % cols8 == 0) ? 8 : 4;
}

bool gemm_supported(int N_out, int K, int gate_up, int bm_b) {
    if (K % 64 != 0 || N_out % 32 != 0) return false;
    if (bm_b == 16) return N_out % (gate_up ? 32 : 64) == 0;
    if (bm_b == 32 || bm_b == 64 || bm_b == 128 || bm_b == 256) return pick_bnt(N_out, gate_up, bm_b) != 0;
    return false;
}

template <int BM, int BNT>
static void launch_tiled(const GemmArgs& a, hipStream_t s) {
    const int cols = a.gate_up ? BNT / 2 : BNT;
    const dim3 grid(a.n_blocks, a.N_out / cols), block(256);
    if (a.gate_up)
        hipLaunchKernelGGL((k_gemm_tiled<BM, BNT, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_gemm_tiled<BM, BNT, false>), grid, block, 0, s, a);
}

template <int BM>
static hipError_t launch_tiled_bm(const GemmArgs& a, hipStream_t s, int bnt) {
    switch (bnt) {
        case 64: launch_tiled<BM, 64>(a, s); break;
        case 128: launch_tiled<BM, 128>(a, s); break;
        case 192:
            if constexpr (BM <= 128) {
                launch_tiled<BM, 192>(a, s);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
    if (a.n_blocks == 0) return hipSuccess;
    if (!gemm_supported(a.N_out, a.K, a.gate_up, a.bm_b)) return hipErrorInvalidValue;
    if (a.bm_b == 16) {
        const int fn = skinny_fn(a.N_out, a.gate_up);
        const int cols = a.gate_up ? fn * 8 : fn * 16;
        if (a.n_blocks > 65535) return hipErrorInvalidValue;
        const dim3 grid(a.N_out / cols, a.n_blocks), block(64);
        if (fn == 8) {
            if (a.gate_up) hipLaunchKernelGGL((k_gemm_skinny<true, 8>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_gemm_skinny<false, 8>), grid, block, 0, s, a);
        } else {
            if (a.gate_up) hipLaunchKernelGGL((k_gemm_skinny<true, 4>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((k_gemm_skinny<false, 4>), grid, block, 0, s, a);
        }
        return hipGetLastError();
    }
    const int bnt = pick_bnt(a.N_out, a.gate_up, a.bm_b);
    switch (a.bm_b) {
        case 32: return launch_tiled_bm<32>(a, s, bnt);
        case 64: return launch_tiled_bm<64>(a, s, bnt);
        case 128: return launch_tiled_bm<128>(a, s, bnt);
        case 256: return launch_tiled_bm<256>(a, s, bnt);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moelora
