// Weight-streaming MFMA GEMM for gfx950: C[m][n] = sum_k A[m][k] W[n][k] for
// the projections (QKV, output, router) and the grouped expert SwiGLU layers.
//
// These contractions read each weight once and are bound by HBM bandwidth or
// by memory latency (few rows per expert). A workgroup owns a 64 x 64 output
// tile; its 4 waves split the K loop (wave w takes k-steps w, w+4, ...), so
// every weight byte is loaded by exactly one wave and the 4 waves read
// adjacent pieces of each weight row at the same time. MFMA fragments are
// loaded from global memory straight into registers one k-step ahead of their
// use with a branch-free loop (so the compiler keeps the loads in flight), and
// two or more waves per SIMD hide the rest of the latency. LDS is
// used only at the end: the 4 partial tiles are summed in a fixed order
// (deterministic) and the epilogue (store / residual add / SwiGLU) reads the
// summed tile with coalesced stores.
//
// Block order: the m-blocks that share a weight tile get linear ids that are
// congruent modulo 8 (one XCD, one L2) and adjacent in launch order, so the
// extra reads of a weight tile hit that XCD's L2.
#include "common.hpp"
#include "gemm.hpp"

// build-time tunable: the waves per SIMD the register allocation must allow
#ifndef DG_STREAM_WAVES
#define DG_STREAM_WAVES 2
#endif
#ifndef DG_STREAM_W_NT
#define DG_STREAM_W_NT 1
#endif

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
    __device__ __forceinline__ void load_nt(const void* p) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(p));
    }
    __device__ __forceinline__ void zero() { v = u16x8{0, 0, 0, 0, 0, 0, 0, 0}; }
};
template <> struct SFrag<uint16_t, WK_FP8> {
    u32x2 v;
    __device__ __forceinline__ void load(const void* p) { v = *reinterpret_cast<const u32x2*>(p); }
    __device__ __forceinline__ void load_nt(const void* p) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    }
    __device__ __forceinline__ void zero() { v = u32x2{0u, 0u}; }
};
template <> struct SFrag<float, WK_SAME> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const void* p) {
        a = reinterpret_cast<const f32x4*>(p)[0];
        b = reinterpret_cast<const f32x4*>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = f32x4{0, 0, 0, 0}; b = a; }
    __device__ __forceinline__ void load_nt(const void* p) { load(p); }
};

// 8 e4m3 codes -> 8 bf16 (exact): the gfx950 scaled pack conversion at
// scale 1, or bit manipulation
#ifndef DG_STREAM_F8_HWCVT
#define DG_STREAM_F8_HWCVT 1
#endif
__device__ __forceinline__ u16x8 widen_e4m3(const u32x2& v) {
#if DG_STREAM_F8_HWCVT
    u32x4 o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        o[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[h], 1.0f, false));
        o[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[h], 1.0f, true));
    }
    return __builtin_bit_cast(u16x8, o);
#else
    u16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t b = (v[j >> 2] >> (8 * (j & 3))) & 0xffu;
        o[j] = (uint16_t)(__float_as_uint(e4m3_to_f32(b)) >> 16);
    }
    return o;
#endif
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

// The K loop for TMV live m-tiles: two register slots, loads issued one
// k-step ahead, no branches (addresses are clamped to valid memory; a k-step
// past this wave's range contributes zero through a select on the W frags).
template <int TMV, typename TL, int WK>
__device__ __forceinline__ void stream_kloop(f32x4 (&acc)[STM][STN], const TL* const (&arow)[STM],
                                             const unsigned char* const (&wrow)[STN], int wave, int lg, int KS,
                                             int kbase) {
    constexpr int WES = (WK == WK_FP8) ? 1 : (int)sizeof(TL);
    SFrag<TL, WK_SAME> fa[2][TMV];
    SFrag<TL, WK> fb[2][STN];
    const int nmax = (KS + 3) / 4;
    auto load = [&](int d, int s) {
        const int ks = min(wave + 4 * s, KS - 1);
        const int k = kbase + ks * 32 + lg * 8;
#pragma unroll
        for (int i = 0; i < TMV; ++i) fa[d][i].load(arow[i] + k);
#pragma unroll
        for (int j = 0; j < STN; ++j) {  // weights are read once: non-temporal
            if (DG_STREAM_W_NT) fb[d][j].load_nt(wrow[j] + (int64_t)k * WES);
            else fb[d][j].load(wrow[j] + (int64_t)k * WES);
        }
    };
    auto consume = [&](int d, int s) {
        const bool ok = wave + 4 * s < KS;
#pragma unroll
        for (int j = 0; j < STN; ++j)
            if (!ok) fb[d][j].zero();
#pragma unroll
        for (int i = 0; i < TMV; ++i)
#pragma unroll
            for (int j = 0; j < STN; ++j) acc[i][j] = smfma(fa[d][i], fb[d][j], acc[i][j]);
    };
    load(0, 0);
    load(1, 1);
    for (int s = 0; s < nmax; s += 2) {
        consume(0, s);
        load(0, s + 2);
        consume(1, s + 1);
        load(1, s + 3);
    }
}

// Work: for every unit (group, 64-column tile) the m-blocks of 64 rows. Item
// ids place the m-blocks of one unit 8 apart, so with a persistent grid (a
// multiple of 8) they run on one XCD. Grouped mode reads the hit groups from
// g.hit ([0] = count, then group ids) and the largest m-block count from
// g.hit_mb; non-grouped mode has one group of g.M rows. With g.ksplit > 1
// (non-grouped plain f32 store, or grouped SwiGLU) the K range is cut into
// g.ksplit slices, one more item dimension, and slice s leaves its sums
// (times the e4m3 row scales, if any) in g.part[s][row][n] (SwiGLU: gate of hidden unit f at
// n = f, up at n = N/2 + f; rows are slots, g.M of them); the consumer adds
// the slices in order.
template <typename TL, int WK, int EPI>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DG_STREAM_WAVES)))
stream_gemm_kernel(GemmArgs g, int n_tiles) {
    if (g.state && g.state[0]) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    constexpr int WES = (WK == WK_FP8) ? 1 : (int)sizeof(TL);
    const int64_t wgs = g.w_group_stride * WES;  // bytes between groups' weights
    const int ngroups = g.group_offsets ? g.hit[0] : 1;
    const int mb_max = g.group_offsets ? *g.hit_mb : (g.M + SBM - 1) / SBM;
    const int units = ngroups * n_tiles;
    const int ksplit = g.ksplit > 1 ? g.ksplit : 1;
    const int64_t items = (int64_t)((units * ksplit + 7) / 8) * 8 * mb_max;
    const int KS = g.K / 32 / ksplit;  // k-steps per slice
    __shared__ float tile_s[SBM][SBN + 1];

    for (int64_t id = blockIdx.x; id < items; id += gridDim.x) {
        const int blk = (int)(id / (8 * mb_max)), rem = (int)(id % (8 * mb_max));
        const int mb = rem / 8;
        const int uk = blk * 8 + rem % 8;
        if (uk >= units * ksplit) continue;
        const int u = uk % units, kslice = uk / units;
        const int gi = u / n_tiles, tile = u % n_tiles;
        const int grp = g.group_offsets ? g.hit[1 + gi] : 0;
        int row0, mrows;
        if (g.group_offsets) {
            row0 = g.group_offsets[grp];
            mrows = g.group_offsets[grp + 1] - row0;
        } else {
            row0 = 0;
            mrows = g.M;
        }
        const int m0 = mb * SBM;
        if (m0 >= mrows) continue;
        const int mcount = min(SBM, mrows - m0);
        const int tm_live = (mcount + 15) / 16;

        // A rows of the m-tiles (rows past mcount read the block's first row:
        // their outputs are never stored)
        const TL* arow[STM];
#pragma unroll
        for (int i = 0; i < STM; ++i) {
            const int r = m0 + min(i * 16 + lr, mcount - 1);
            const int ar = row0 + r;
            const int src = g.a_rows ? g.a_rows[ar] : ar;
            arow[i] = reinterpret_cast<const TL*>(g.A) + (int64_t)src * g.lda;
        }
        // W rows of the n-tiles (past N: the last row, never stored)
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
            wr = min(wr, limit - 1);
            wrow[j] = base + (int64_t)grp * wgs + (int64_t)wr * g.ldw * WES;
        }

        f32x4 acc[STM][STN];
#pragma unroll
        for (int i = 0; i < STM; ++i)
#pragma unroll
            for (int j = 0; j < STN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int kbase = kslice * KS * 32;
        if (tm_live == 1) stream_kloop<1, TL, WK>(acc, arow, wrow, wave, lg, KS, kbase);
        else if (tm_live == 2) stream_kloop<2, TL, WK>(acc, arow, wrow, wave, lg, KS, kbase);
        else stream_kloop<4, TL, WK>(acc, arow, wrow, wave, lg, KS, kbase);

        // ---- sum the 4 waves' partial tiles in LDS, in wave order ----
        for (int w = 0; w < 4; ++w) {
            if (wave == w) {
#pragma unroll
                for (int i = 0; i < STM; ++i) {
                    if (i >= tm_live) continue;
#pragma unroll
                    for (int j = 0; j < STN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int r = i * 16 + lg * 4 + q, c = j * 16 + lr;
                            if (w == 0) tile_s[r][c] = acc[i][j][q];
                            else tile_s[r][c] += acc[i][j][q];
                        }
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
                const int64_t orow = row0 + m0 + r;
                if (ksplit > 1) {
                    float* P = g.part + ((int64_t)kslice * g.M + orow) * g.N;
                    P[n] = gv;
                    P[g.N / 2 + n] = uv;
                    continue;
                }
                const float h = ssilu(gv) * uv;
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
                if (ksplit > 1) g.part[((int64_t)kslice * g.M + orow) * g.N + n] = v;
                else if constexpr (EPI == EPI_STORE_F32) reinterpret_cast<float*>(g.C)[orow * g.ldc + n] = v;
                else if constexpr (EPI == EPI_STORE_BF16) reinterpret_cast<uint16_t*>(g.C)[orow * g.ldc + n] = f2bf(v);
                else if constexpr (EPI == EPI_RESIDUAL) g.X[orow * g.ldx + n] += v;
            }
        }
        __syncthreads();  // tile_s is reused by the next item
    }
}

template <typename TL, int WK, int EPI>
static hipError_t launch_stream_t(const GemmArgs& g, int groups, int max_rows, hipStream_t st) {
    const int G = groups > 0 ? groups : 1;
    const int n_tiles = EPI == EPI_SWIGLU ? (g.N / 2 + SBN / 2 - 1) / (SBN / 2) : (g.N + SBN - 1) / SBN;
    const int units = G * n_tiles;
    const int mb_max = std::max(1, (max_rows + SBM - 1) / SBM);
    const int ks = g.ksplit > 1 ? g.ksplit : 1;
    const bool split_ok = EPI == EPI_STORE_F32 ? !g.group_offsets : EPI == EPI_SWIGLU && g.group_offsets;
    if (ks > 1 && (!split_ok || !g.part || (g.K / 32) % ks)) return hipErrorInvalidValue;
    const int64_t items = (int64_t)((units * ks + 7) / 8) * 8 * mb_max;  // upper bound
    // persistent grid: a multiple of 8 (one slot per XCD), at most 4 per CU
    int64_t grid = std::min<int64_t>(items, 256 * 4);
    grid = std::max<int64_t>(8, (grid + 7) / 8 * 8);
    stream_gemm_kernel<TL, WK, EPI><<<(unsigned)grid, 256, 0, st>>>(g, n_tiles);
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
