// Weight-streaming MFMA GEMM for gfx950: C[m][n] = sum_k A[m][k] W[n][k] for
// the projections (QKV, output, router) and the grouped expert SwiGLU layers.
//
// These contractions read each weight once and are bound by HBM bandwidth or
// by memory latency (few rows per expert). A workgroup owns a 64 x 64 output
// tile; its 4 waves split the K loop (wave w takes k-steps w, w+4, ...), so
// every weight byte is loaded by exactly one wave and the 4 waves read
// adjacent pieces of each weight row at the same time. MFMA fragments are
// loaded from global memory straight into registers, DEPTH k-steps ahead of
// their use, so each wave keeps DEPTH x (m-tiles + 4) loads in flight. LDS is
// used only at the end: the 4 partial tiles are summed in a fixed order
// (deterministic) and the epilogue (store / residual add / SwiGLU) reads the
// summed tile with coalesced stores.
//
// Block order: the m-blocks that share a weight tile get linear ids that are
// congruent modulo 8 (one XCD, one L2) and adjacent in launch order, so the
// extra reads of a weight tile hit that XCD's L2.
#include "common.hpp"
#include "gemm.hpp"

namespace dg {

namespace {

constexpr int SBM = 64;  // rows per tile
constexpr int SBN = 64;  // cols per tile
constexpr int STM = 4;   // 16-row m-tiles
constexpr int STN = 4;   // 16-col n-tiles

template <typename TL, int WK> struct SFrag;
template <> struct SFrag<uint16_t, WK_SAME> {
    u16x8 v;
    __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u16x8*>(p); }
    __device__ __forceinline__ void zero() { v = u16x8{0, 0, 0, 0, 0, 0, 0, 0}; }
};
template <> struct SFrag<uint16_t, WK_FP8> {
    u32x2 v;
    __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u32x2*>(p); }
    __device__ __forceinline__ void zero() { v = u32x2{0u, 0u}; }
};
template <> struct SFrag<float, WK_SAME> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const void* p) {
        a = reinterpret_cast<const f32x4*>(p)[0];
        b = reinterpret_cast<const f32x4*>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = f32x4{0, 0, 0, 0}; b = a; }
};

__device__ __forceinline__ u16x8 widen_e4m3(const u32x2& v) {
    u16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t b = (v[j >> 2] >> (8 * (j & 3))) & 0xffu;
        o[j] = (uint16_t)(__float_as_uint(e4m3_to_f32(b)) >> 16);
    }
    return o;
}

__device__ __forceinline__ f32x4 smfma(const SFrag<uint16_t, WK_SAME>& a, const SFrag<uint16_t, WK_SAME>& b,
                                       f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, b.v),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 smfma(const SFrag<uint16_t, WK_SAME>& a, const SFrag<uint16_t, WK_FP8>& b,
                                       f32x4 c) {
    u16x8 w = widen_e4m3(b.v);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, w), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 smfma(const SFrag<float, WK_SAME>& a, const SFrag<float, WK_SAME>& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[j], b.a[j], c, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[j], b.b[j], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ float ssilu(float x) { return x / (1.f + __expf(-x)); }

}  // namespace

template <typename TL, int WK, int EPI, int DEPTH>
__global__ void __launch_bounds__(256) stream_gemm_kernel(GemmArgs g, int n_tiles, int units, int mb_max) {
    if (g.state && g.state[0]) return;
    // ---- decode the block: unit u = group * n_tiles + tile, m-block mb ----
    const int id = blockIdx.x;
    const int blk = id / (8 * mb_max), rem = id % (8 * mb_max);
    const int mb = rem / 8;
    const int u = blk * 8 + rem % 8;
    if (u >= units) return;
    const int grp = u / n_tiles, tile = u % n_tiles;
    int row0, mrows;
    if (g.group_offsets) {
        row0 = g.group_offsets[grp];
        mrows = g.group_offsets[grp + 1] - row0;
    } else {
        row0 = 0;
        mrows = g.M;
    }
    const int m0 = mb * SBM;
    if (m0 >= mrows) return;
    const int mcount = min(SBM, mrows - m0);
    const int tm_live = (mcount + 15) / 16;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    constexpr int WES = (WK == WK_FP8) ? 1 : (int)sizeof(TL);
    const int64_t wgs = g.w_group_stride * WES;  // bytes between groups' weights

    // ---- fragment sources ----
    // A rows: m-tile i, lane row lr
    const TL* arow[STM];
#pragma unroll
    for (int i = 0; i < STM; ++i) {
        const int r = m0 + i * 16 + lr;
        if (r < mcount + m0 && r < mrows) {
            const int ar = row0 + r;
            const int src = g.a_rows ? g.a_rows[ar] : ar;
            arow[i] = reinterpret_cast<const TL*>(g.A) + (int64_t)src * g.lda;
        } else {
            arow[i] = nullptr;
        }
    }
    // W rows: n-tile j, lane col lr
    const unsigned char* wrow[STN];
    const int n0 = tile * SBN;
#pragma unroll
    for (int j = 0; j < STN; ++j) {
        int wr;
        const unsigned char* base;
        int limit;
        if (EPI == EPI_SWIGLU) {
            // n-tiles 0,1: gate rows; 2,3: up rows (same output columns)
            wr = tile * (SBN / 2) + (j & 1) * 16 + lr;
            base = reinterpret_cast<const unsigned char*>(j < 2 ? g.W : g.W2);
            limit = g.N / 2;
        } else {
            wr = n0 + j * 16 + lr;
            base = reinterpret_cast<const unsigned char*>(g.W);
            limit = g.N;
        }
        wrow[j] = wr < limit ? base + (int64_t)grp * wgs + (int64_t)wr * g.ldw * WES : nullptr;
    }

    SFrag<TL, WK_SAME> fa[DEPTH][STM];
    SFrag<TL, WK> fb[DEPTH][STN];
    f32x4 acc[STM][STN];
#pragma unroll
    for (int i = 0; i < STM; ++i)
#pragma unroll
        for (int j = 0; j < STN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KS = g.K / 32;                  // k-steps of 32
    const int nmine = (KS - wave + 3) / 4;    // this wave's k-steps: wave, wave+4, ...
    auto load = [&](int d, int s) {           // s-th k-step of this wave into slot d
        if (s < nmine) {
            const int k = (wave + 4 * s) * 32 + lg * 8;
#pragma unroll
            for (int i = 0; i < STM; ++i) {
                if (i < tm_live && arow[i]) fa[d][i].load(arow[i] + k);
                else fa[d][i].zero();
            }
#pragma unroll
            for (int j = 0; j < STN; ++j) {
                if (wrow[j]) fb[d][j].load(wrow[j] + (int64_t)k * WES);
                else fb[d][j].zero();
            }
        }
    };
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load(d, d);
    for (int s0 = 0; s0 < nmine; s0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            if (s0 + d < nmine) {
#pragma unroll
                for (int i = 0; i < STM; ++i) {
                    if (i < tm_live) {
#pragma unroll
                        for (int j = 0; j < STN; ++j) acc[i][j] = smfma(fa[d][i], fb[d][j], acc[i][j]);
                    }
                }
                load(d, s0 + d + DEPTH);
            }
        }
    }

    // ---- sum the 4 waves' partial tiles in LDS, in wave order ----
    __shared__ float tile_s[SBM][SBN + 1];
    for (int w = 0; w < 4; ++w) {
        if (wave == w) {
#pragma unroll
            for (int i = 0; i < STM; ++i)
#pragma unroll
                for (int j = 0; j < STN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = i * 16 + lg * 4 + q, c = j * 16 + lr;
                        if (w == 0) tile_s[r][c] = acc[i][j][q];
                        else tile_s[r][c] += acc[i][j][q];
                    }
        }
        __syncthreads();
    }
    // ---- epilogue ----
    if constexpr (EPI == EPI_SWIGLU) {
        const int hn0 = tile * (SBN / 2);
        for (int e = tid; e < SBM * (SBN / 2); e += 256) {
            const int r = e / (SBN / 2), c = e % (SBN / 2);
            const int n = hn0 + c;
            if (r >= mcount || n >= g.N / 2) continue;
            float gv = tile_s[r][c], uv = tile_s[r][c + SBN / 2];
            if (g.w_scale) {
                gv *= bf2f(g.w_scale[(int64_t)grp * g.scale_group_stride + n]);
                uv *= bf2f(g.w2_scale[(int64_t)grp * g.scale_group_stride + n]);
            }
            const float h = ssilu(gv) * uv;
            const int64_t orow = row0 + m0 + r;
            if (g.c_f32) reinterpret_cast<float*>(g.C)[orow * g.ldc + n] = h;
            else reinterpret_cast<uint16_t*>(g.C)[orow * g.ldc + n] = f2bf(h);
        }
    } else {
        for (int e = tid; e < SBM * SBN; e += 256) {
            const int r = e / SBN, c = e % SBN;
            const int n = n0 + c;
            if (r >= mcount || n >= g.N) continue;
            float v = tile_s[r][c];
            if (g.w_scale) v *= bf2f(g.w_scale[(int64_t)grp * g.scale_group_stride + n]);
            const int64_t orow = row0 + m0 + r;
            if constexpr (EPI == EPI_STORE_F32) reinterpret_cast<float*>(g.C)[orow * g.ldc + n] = v;
            else if constexpr (EPI == EPI_STORE_BF16) reinterpret_cast<uint16_t*>(g.C)[orow * g.ldc + n] = f2bf(v);
            else if constexpr (EPI == EPI_RESIDUAL) g.X[orow * g.ldx + n] += v;
        }
    }
}

template <typename TL, int WK, int EPI>
static hipError_t launch_stream_t(const GemmArgs& g, int groups, int max_rows, hipStream_t st) {
    const int G = groups > 0 ? groups : 1;
    const int n_tiles = EPI == EPI_SWIGLU ? (g.N / 2 + SBN / 2 - 1) / (SBN / 2) : (g.N + SBN - 1) / SBN;
    const int units = G * n_tiles;
    const int mb_max = std::max(1, (max_rows + SBM - 1) / SBM);
    const int64_t blocks = (int64_t)((units + 7) / 8) * 8 * mb_max;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    constexpr int DEPTH = sizeof(TL) == 4 ? 2 : 4;
    stream_gemm_kernel<TL, WK, EPI, DEPTH><<<(unsigned)blocks, 256, 0, st>>>(g, n_tiles, units, mb_max);
    return hipGetLastError();
}

hipError_t stream_gemm_launch(const GemmArgs& g, int act_f32, int w_fp8, int epi, int groups, int max_rows,
                              hipStream_t st) {
#define DG_SDISPATCH(EPIV)                                                                  \
    if (epi == EPIV) {                                                                      \
        if (act_f32) return launch_stream_t<float, WK_SAME, EPIV>(g, groups, max_rows, st); \
        if (w_fp8) return launch_stream_t<uint16_t, WK_FP8, EPIV>(g, groups, max_rows, st); \
        return launch_stream_t<uint16_t, WK_SAME, EPIV>(g, groups, max_rows, st);           \
    }
    DG_SDISPATCH(EPI_STORE_F32)
    DG_SDISPATCH(EPI_STORE_BF16)
    DG_SDISPATCH(EPI_RESIDUAL)
    DG_SDISPATCH(EPI_SWIGLU)
#undef DG_SDISPATCH
    return hipErrorInvalidValue;
}

}  // namespace dg
