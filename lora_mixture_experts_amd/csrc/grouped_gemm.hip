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

__device__ __forceinline__ int row_adapter(const GemmArgs& a, int slot) {
    const int p = a.sorted_b[slot];
    if (p >= a.P) return -1;
    const int ad = a.adapter_ids[p / a.top_k];
    return (ad >= 0 && ad < a.L) ? ad : -1;
}

// S row chunk (8 values starting at j0) as hi/lo bf16 operands; zero when the
// row is not in the current adapter run or j is past r.
__device__ __forceinline__ void load_s_hilo(const GemmArgs& a, int slot, bool in_run, int j0,
                                            u32x4& hi, u32x4& lo) {
    float v[8], rest[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = 0.f;
    if (in_run && j0 < a.r) {
        for (int s = 0; s < a.nsplit; ++s) {
            const float* src = a.S_part + (static_cast<size_t>(s) * a.C_b + slot) * a.r + j0;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[q] += x0[q];
                v[4 + q] += x1[q];
            }
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
// Skinny variant: 16-row blocks (few rows per expert, weight streaming bound).
// 4 waves split the K steps; each wave keeps 4 fragments (64 columns).
template <bool GATEUP>
__global__ __launch_bounds__(256) void k_gemm_skinny(GemmArgs a) {
    constexpr int FN = 4;
    const int b = blockIdx.x;
    const int e = a.blk_e_b[b];
    if (e < 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kc = lane >> 4, lrow = lane & 15;
    const int I = GATEUP ? a.N_out : 0;
    const int Nw = GATEUP ? 2 * a.N_out : a.N_out;
    const int c0 = blockIdx.y * (GATEUP ? 32 : 64);
    const int K = a.K;

    const int slot = b * 16 + lrow;
    const int p = a.sorted_b[slot];
    const uint16_t* xrow = nullptr;
    if (GATEUP) {
        if (p < a.P) xrow = a.X + static_cast<size_t>(p / a.top_k) * K + kc * 8;
    } else {
        xrow = a.X + static_cast<size_t>(slot) * K + kc * 8;
    }
    const uint16_t* wrow[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f)
        wrow[f] = a.W + (static_cast<size_t>(e) * Nw + w_row_of_frag<GATEUP>(f, c0, I) + lrow) * K +
                  kc * 8;

    f32x4 acc[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nsteps = K / 32;
    int s = wave;
    for (; s + 12 < nsteps; s += 16) {
        u32x4 xa[4], wb[4][FN];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k0 = (s + 4 * u) * 32;
            xa[u] = xrow ? ld16(xrow + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int f = 0; f < FN; ++f) wb[u][f] = ld16_nt(wrow[f] + k0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int f = 0; f < FN; ++f) acc[f] = mfma16x16x32(xa[u], wb[u][f], acc[f]);
    }
    for (; s < nsteps; s += 4) {
        const int k0 = s * 32;
        const u32x4 xa = xrow ? ld16(xrow + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int f = 0; f < FN; ++f) acc[f] = mfma16x16x32(xa, ld16_nt(wrow[f] + k0), acc[f]);
    }

    __shared__ f32x4 red[4][FN][64];
#pragma unroll
    for (int f = 0; f < FN; ++f) red[wave][f][lane] = acc[f];
    __syncthreads();

    // finalising wave: gate_up -> wave w < 2 owns fragments (2w, 2w+1); down -> wave w owns w
    constexpr int kOwn = GATEUP ? 2 : 1;
    if (GATEUP && wave >= 2) return;
    f32x4 v[kOwn];
    int fidx[kOwn];
#pragma unroll
    for (int o = 0; o < kOwn; ++o) {
        fidx[o] = wave * kOwn + o;
        v[o] = red[0][fidx[o]][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) v[o] += red[w][fidx[o]][lane];
    }

    // LoRA expand, one pass per adapter present in the block
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
                const int j0 = kk + kc * 8;
                u32x4 hi, lo;
                load_s_hilo(a, slot, in_run, j0, hi, lo);
#pragma unroll
                for (int o = 0; o < kOwn; ++o) {
                    const u32x4 bb = load_lora_b(a, Nw, acur, e,
                                                 w_row_of_frag<GATEUP>(fidx[o], c0, I) + lrow, j0);
                    v[o] = mfma16x16x32(hi, bb, v[o]);
                    v[o] = mfma16x16x32(lo, bb, v[o]);
                }
            }
        }
    }

    const int orow0 = b * 16 + 4 * kc;
    if (GATEUP) {
        const int col = c0 + 16 * wave + lrow;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a.h_out[static_cast<size_t>(orow0 + i) * a.N_out + col] =
                f32_to_bf16_rne(silu(v[0][i]) * v[1][i]);
    } else {
        const int col = c0 + 16 * wave + lrow;
#pragma unroll
        for (int i = 0; i < 4; ++i) a.d_out[static_cast<size_t>(orow0 + i) * a.N_out + col] = v[0][i];
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
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
    const uint16_t* asrc[C::A_LD];
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
        const int r = ld_row + 32 * i;
        const int slot = row0 + r;
        if (GATEUP) {
            const int p = a.sorted_b[slot];
            asrc[i] = p < a.P ? a.X + static_cast<size_t>(p / a.top_k) * K + ld_chunk * 8 : nullptr;
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
        for (int i = 0; i < C::A_LD; ++i) ra[i] = asrc[i] ? ld16(asrc[i] + k0) : u32x4{0, 0, 0, 0};
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
        const int cols = a.gate_up ? 32 : 64;
        const dim3 grid(a.n_blocks, a.N_out / cols), block(256);
        if (a.gate_up)
            hipLaunchKernelGGL(k_gemm_skinny<true>, grid, block, 0, s, a);
        else
            hipLaunchKernelGGL(k_gemm_skinny<false>, grid, block, 0, s, a);
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
