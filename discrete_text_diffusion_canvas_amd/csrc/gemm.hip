// MFMA GEMM family for gfx950: C[m][n] = sum_k A[m][k] * W[n][k].
//
// Every dense contraction of the denoising step goes through this template:
// the QKV and output projections of each layer, the router logits, the
// grouped expert SwiGLU projections, and the tied 262K-vocabulary LM head
// with its fused temperature/entropy/argmax epilogue.
//
// Layout: A (activations) row-major [rows][K]; W (weights) row-major [N][K]
// ("K-contiguous", the model's [out][in] storage); both stream along K.
// A workgroup of 256 threads (4 waves, WM x WN) owns a BM x BN output tile,
// each wave a (TM*16) x (TN*16) sub-tile of 16x16 MFMA tiles.
//   bf16: v_mfma_f32_16x16x32_bf16, one per (m-tile, n-tile, 32-wide k-step).
//   f32:  v_mfma_f32_16x16x4_f32, eight per k-step; each lane feeds the same
//         8 consecutive k of A and W to the eight issues, so every k is paired
//         with itself and the sum over the k-step is exact in order-free form.
//   fp8 weights (OCP e4m3) are widened to bf16 when staged into LDS; the
//         per-output-row scale multiplies the accumulator in the epilogue.
// Global -> registers -> LDS with double-buffered LDS; rows of the LDS tiles
// are padded by 16 bytes so the 16 lanes reading one fragment hit distinct
// banks. Rows past M and columns past N are zero-filled and never stored.
#include "common.hpp"
#include "gemm.hpp"

namespace dg {

// ---- element types in LDS ----
template <typename T> struct Frag;
template <> struct Frag<uint16_t> { typedef u16x8 type; };
template <> struct Frag<float> { struct type { f32x4 lo, hi; }; };

__device__ __forceinline__ f32x4 mfma16(const u16x8& a, const u16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const Frag<float>::type& a, const Frag<float>::type& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], c, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], c, 0, 0, 0);
    return c;
}

// 8 consecutive elements of a row -> LDS element type
template <typename TL, int WK> struct Chunk;
// bf16 activations/weights: one 16-byte load
template <> struct Chunk<uint16_t, WK_SAME> {
    u16x8 v;
    __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u16x8*>(p); }
    __device__ __forceinline__ void zero() { v = u16x8{0, 0, 0, 0, 0, 0, 0, 0}; }
    __device__ __forceinline__ void store(uint16_t* s) const { *reinterpret_cast<u16x8*>(s) = v; }
    static constexpr int bytes = 16;
};
// e4m3 weights: one 8-byte load, widened exactly to bf16
template <> struct Chunk<uint16_t, WK_FP8> {
    u32x2 v;
    __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u32x2*>(p); }
    __device__ __forceinline__ void zero() { v = u32x2{0u, 0u}; }
    __device__ __forceinline__ void store(uint16_t* s) const {
        u16x8 o;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t b = (v[j >> 2] >> (8 * (j & 3))) & 0xffu;
            o[j] = (uint16_t)(__float_as_uint(e4m3_to_f32(b)) >> 16);
        }
        *reinterpret_cast<u16x8*>(s) = o;
    }
    static constexpr int bytes = 8;
};
// f32: two 16-byte loads
template <> struct Chunk<float, WK_SAME> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const void* p) {
        a = reinterpret_cast<const f32x4*>(p)[0];
        b = reinterpret_cast<const f32x4*>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = f32x4{0, 0, 0, 0}; b = a; }
    __device__ __forceinline__ void store(float* s) const {
        reinterpret_cast<f32x4*>(s)[0] = a;
        reinterpret_cast<f32x4*>(s)[1] = b;
    }
    static constexpr int bytes = 32;
};

template <typename TL>
__device__ __forceinline__ typename Frag<TL>::type read_frag(const TL* s);
template <>
__device__ __forceinline__ u16x8 read_frag<uint16_t>(const uint16_t* s) { return *reinterpret_cast<const u16x8*>(s); }
template <>
__device__ __forceinline__ Frag<float>::type read_frag<float>(const float* s) {
    Frag<float>::type f;
    f.lo = reinterpret_cast<const f32x4*>(s)[0];
    f.hi = reinterpret_cast<const f32x4*>(s)[1];
    return f;
}

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }

// ---------------------------------------------------------------------------
// The kernel. Grid: x = N tiles, y = group (grouped mode) or M block.
// ---------------------------------------------------------------------------
template <int WM, int WN, int TM, int TN, int BK, typename TL, int WK, int EPI>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs g) {
    constexpr int BM = WM * TM * 16;
    constexpr int BN = WN * TN * 16;
    constexpr int PAD = 16 / sizeof(TL);
    constexpr int SK = BK + PAD;                 // LDS row stride (elements)
    constexpr int CPR = BK / 8;                  // 8-element chunks per tile row
    constexpr int A_CH = BM * CPR / 256;         // A chunks per thread
    constexpr int B_CH = (BN * CPR + 255) / 256; // W chunks per thread
    static_assert(BM * CPR % 256 == 0, "A tile must split evenly");
    typedef typename Frag<TL>::type FragT;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    TL* As = reinterpret_cast<TL*>(smem_raw);
    TL* Bs = As + 2 * BM * SK;

    if (g.state && g.state[0]) return;  // finished canvas: replays are no-ops
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 15, lg = lane >> 4;

    // ---- the rows of this block ----
    int row0, mrows;
    int grp = 0;
    if (g.group_offsets) {
        grp = blockIdx.y;
        row0 = g.group_offsets[grp];
        mrows = g.group_offsets[grp + 1] - row0;
        if (mrows <= 0) return;
    } else {
        row0 = 0;
        mrows = g.M;
    }
    const int n0 = blockIdx.x * BN;
    if (n0 >= g.N) return;
    const TL* Abase = reinterpret_cast<const TL*>(g.A);
    const unsigned char* Wb = reinterpret_cast<const unsigned char*>(g.W) + (int64_t)grp * g.w_group_stride * (WK == WK_FP8 ? 1 : sizeof(TL));
    const unsigned char* W2b = g.W2 ? reinterpret_cast<const unsigned char*>(g.W2) + (int64_t)grp * g.w_group_stride * (WK == WK_FP8 ? 1 : sizeof(TL)) : nullptr;
    constexpr int WES = (WK == WK_FP8) ? 1 : sizeof(TL);  // bytes per weight element
    const int KT = g.K / BK;

    for (int mb = g.group_offsets ? 0 : blockIdx.y * BM; mb < mrows; mb += g.group_offsets ? BM : (int)(gridDim.y * BM)) {
        const int mcount = min(BM, mrows - mb);

        // per-thread chunk coordinates
        Chunk<TL, WK_SAME> ra[A_CH];
        Chunk<TL, WK> rb[B_CH];
        auto load_regs = [&](int kt) {
            const int k0 = kt * BK;
#pragma unroll
            for (int c = 0; c < A_CH; ++c) {
                int ch = tid + 256 * c;
                int r = ch / CPR, kc = (ch % CPR) * 8;
                if (r < mcount) {
                    int ar = row0 + mb + r;
                    int src = g.a_rows ? g.a_rows[ar] : ar;
                    ra[c].load(Abase + (int64_t)src * g.lda + k0 + kc);
                } else {
                    ra[c].zero();
                }
            }
#pragma unroll
            for (int c = 0; c < B_CH; ++c) {
                int ch = tid + 256 * c;
                int r = ch / CPR, kc = (ch % CPR) * 8;
                if (ch < BN * CPR) {
                    const unsigned char* base = Wb;
                    int wr;
                    if (EPI == EPI_SWIGLU) {
                        // first half of the tile: gate rows, second half: up rows
                        int half = BN / 2;
                        wr = n0 / 2 + (r % half);
                        if (r >= half) base = W2b;
                        if (wr >= g.N / 2) { rb[c].zero(); continue; }
                    } else {
                        wr = n0 + r;
                        if (wr >= g.N) { rb[c].zero(); continue; }
                    }
                    rb[c].load(base + ((int64_t)wr * g.ldw + k0 + kc) * WES);
                }
            }
        };
        auto store_lds = [&](int buf) {
            TL* as = As + buf * BM * SK;
            TL* bs = Bs + buf * BN * SK;
#pragma unroll
            for (int c = 0; c < A_CH; ++c) {
                int ch = tid + 256 * c;
                ra[c].store(as + (ch / CPR) * SK + (ch % CPR) * 8);
            }
#pragma unroll
            for (int c = 0; c < B_CH; ++c) {
                int ch = tid + 256 * c;
                if (ch < BN * CPR) rb[c].store(bs + (ch / CPR) * SK + (ch % CPR) * 8);
            }
        };

        f32x4 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // m-tiles of this wave that hold at least one real row
        const int wrow0 = wm * TM * 16;
        const int tm_live = max(0, min(TM, (mcount - wrow0 + 15) / 16));

        load_regs(0);
        store_lds(0);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < KT) load_regs(kt + 1);
            const TL* as = As + buf * BM * SK;
            const TL* bs = Bs + buf * BN * SK;
#pragma unroll
            for (int ks = 0; ks < BK / 32; ++ks) {
                FragT bfr[TN];
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bfr[j] = read_frag<TL>(bs + (wn * TN * 16 + j * 16 + lr) * SK + ks * 32 + lg * 8);
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if (i < tm_live) {
                        FragT afr = read_frag<TL>(as + (wrow0 + i * 16 + lr) * SK + ks * 32 + lg * 8);
#pragma unroll
                        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(afr, bfr[j], acc[i][j]);
                    }
                }
            }
            if (kt + 1 < KT) store_lds(buf ^ 1);
            __syncthreads();
        }

        // ---- epilogue ----
        // acc[i][j][q]: row = wrow0 + i*16 + lg*4 + q, col = wn*TN*16 + j*16 + lr (tile-local)
        if constexpr (EPI == EPI_LMHEAD) {
            lmhead_epilogue<WM, WN, TM, TN>(g, acc, mb, mcount, n0, smem_raw);
        } else {
            if constexpr (EPI != EPI_SWIGLU) {
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if (i >= tm_live) continue;
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int n = n0 + wn * TN * 16 + j * 16 + lr;
                        if (n >= g.N) continue;
                        const float sc = g.w_scale ? bf2f(g.w_scale[(int64_t)grp * g.scale_group_stride + n]) : 1.f;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r = wrow0 + i * 16 + lg * 4 + q;
                            if (r >= mcount) continue;
                            const int orow = row0 + mb + r;  // output row (slot in grouped mode)
                            const float v = acc[i][j][q] * sc;
                            if constexpr (EPI == EPI_STORE_F32) {
                                reinterpret_cast<float*>(g.C)[(int64_t)orow * g.ldc + n] = v;
                            } else if constexpr (EPI == EPI_STORE_BF16) {
                                reinterpret_cast<uint16_t*>(g.C)[(int64_t)orow * g.ldc + n] = f2bf(v);
                            } else if constexpr (EPI == EPI_RESIDUAL) {
                                g.X[(int64_t)orow * g.ldx + n] += v;
                            }
                        }
                    }
                }
            }
            if constexpr (EPI == EPI_SWIGLU) {
                // stage the fp32 tile through LDS, then h = silu(gate) * up
                __syncthreads();
                float* st = reinterpret_cast<float*>(smem_raw);  // [BM][BN+1]
                constexpr int SC = BN + 1;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    if (i >= tm_live) continue;
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r = wrow0 + i * 16 + lg * 4 + q;
                            const int c = wn * TN * 16 + j * 16 + lr;
                            st[r * SC + c] = acc[i][j][q];
                        }
                }
                __syncthreads();
                constexpr int HALF = BN / 2;
                const int hn0 = n0 / 2;
                for (int e = tid; e < BM * HALF; e += 256) {
                    const int r = e / HALF, c = e % HALF;
                    const int n = hn0 + c;
                    if (r >= mcount || n >= g.N / 2) continue;
                    float gv = st[r * SC + c], uv = st[r * SC + HALF + c];
                    if (g.w_scale) {
                        gv *= bf2f(g.w_scale[(int64_t)grp * g.scale_group_stride + n]);
                        uv *= bf2f(g.w2_scale[(int64_t)grp * g.scale_group_stride + n]);
                    }
                    const float h = silu(gv) * uv;
                    const int orow = row0 + mb + r;
                    if (g.c_f32)
                        reinterpret_cast<float*>(g.C)[(int64_t)orow * g.ldc + n] = h;
                    else
                        reinterpret_cast<uint16_t*>(g.C)[(int64_t)orow * g.ldc + n] = f2bf(h);
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Launch configurations.
// ---------------------------------------------------------------------------
template <int WM, int WN, int TM, int TN, int BK, typename TL, int WK, int EPI>
static hipError_t launch_cfg(const GemmArgs& g, int groups, hipStream_t st) {
    constexpr int BM = WM * TM * 16;
    constexpr int BN = WN * TN * 16;
    constexpr int SK = BK + 16 / sizeof(TL);
    size_t lds = (size_t)2 * (BM + BN) * SK * sizeof(TL);
    if (EPI == EPI_SWIGLU) lds = std::max(lds, (size_t)BM * (BN + 1) * sizeof(float));
    if (EPI == EPI_LMHEAD) lds = std::max(lds, lmhead_epilogue_lds<WM, WN, TM, TN>());
    auto kern = gemm_kernel<WM, WN, TM, TN, BK, TL, WK, EPI>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid((g.N + BN - 1) / BN, groups > 0 ? groups : std::max(1, std::min((g.M + BM - 1) / BM, 65535)));
    if (EPI == EPI_SWIGLU) grid.x = (g.N / 2 + BN / 2 - 1) / (BN / 2);
    kern<<<grid, 256, lds, st>>>(g);
    return hipGetLastError();
}

template <typename TL, int WK, int EPI>
static hipError_t launch_proj(const GemmArgs& g, int groups, hipStream_t st) {
    // 256 x 64 tiles, 4 waves stacked along M, 32-wide K steps
    return launch_cfg<4, 1, 4, 4, 32, TL, WK, EPI>(g, groups, st);
}

template <typename TL, int WK, int EPI>
static hipError_t launch_small_m(const GemmArgs& g, int groups, hipStream_t st) {
    // 64 x 64 tiles for grouped experts (few rows per expert)
    return launch_cfg<1, 4, 4, 1, 32, TL, WK, EPI>(g, groups, st);
}

hipError_t gemm_launch(const GemmArgs& g, int act_f32, int w_fp8, int epi, int groups, int shape,
                       hipStream_t st) {
    // weight-streaming contractions: the split-K streaming kernel (g.M bounds
    // the rows per group in grouped mode)
    if (epi != EPI_LMHEAD && shape != SHAPE_LDS) return stream_gemm_launch(g, act_f32, w_fp8, epi, groups, g.M, st);
#define DG_DISPATCH(EPIV)                                                                              \
    if (epi == EPIV) {                                                                                 \
        if (act_f32) return shape == SHAPE_SMALL_M ? launch_small_m<float, WK_SAME, EPIV>(g, groups, st) \
                                                  : launch_proj<float, WK_SAME, EPIV>(g, groups, st);    \
        if (w_fp8) return shape == SHAPE_SMALL_M ? launch_small_m<uint16_t, WK_FP8, EPIV>(g, groups, st) \
                                                : launch_proj<uint16_t, WK_FP8, EPIV>(g, groups, st);    \
        return shape == SHAPE_SMALL_M ? launch_small_m<uint16_t, WK_SAME, EPIV>(g, groups, st)           \
                                      : launch_proj<uint16_t, WK_SAME, EPIV>(g, groups, st);             \
    }
    DG_DISPATCH(EPI_STORE_F32)
    DG_DISPATCH(EPI_STORE_BF16)
    DG_DISPATCH(EPI_RESIDUAL)
    DG_DISPATCH(EPI_SWIGLU)
#undef DG_DISPATCH
    if (epi == EPI_LMHEAD) {
        // f32 models, and bf16 shapes outside the tiled kernel (d_model not a
        // multiple of 64, or a logits row stride not a multiple of 8)
        if (act_f32) return launch_cfg<2, 2, 4, 4, 32, float, WK_SAME, EPI_LMHEAD>(g, 0, st);
        return launch_cfg<2, 2, 4, 4, 32, uint16_t, WK_SAME, EPI_LMHEAD>(g, 0, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace dg
