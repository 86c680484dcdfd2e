// Per-layer glue kernels of the MoE transformer for gfx950: token embedding,
// RMSNorm, rotary embedding with the head-major scatter of Q/K/V, the top-k
// router, the expert histogram/permutation and the deterministic combine.
//
// The model follows the DiffusionGemma model card (zh-TW): intro list and the
// spec table (a sparse MoE with 8 of 128 experts active plus 1 shared expert
// per token). Pre-norm RMSNorm, rotate-half RoPE, softmax over the selected
// router logits and SwiGLU experts are the readings taken where the card is
// silent.
#include "common.hpp"
#include "layer.hpp"

namespace dg {

// ---------------------------------------------------------------------------
// X[i][:] = E[tok[i]][:] as f32. One workgroup per row.
// ---------------------------------------------------------------------------
template <typename TE>
__global__ void __launch_bounds__(256) embed_kernel(const TE* __restrict__ E, int d, int V,
                                                    const int32_t* __restrict__ tok, float* __restrict__ X,
                                                    const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int i = blockIdx.x;
    const int64_t t = tok[i];
    const bool ok = t >= 0 && t < V;  // an id outside the vocabulary embeds as a zero row
    const TE* src = E + (ok ? t : 0) * d;
    for (int k = threadIdx.x; k < d; k += 256) {
        float v;
        if constexpr (sizeof(TE) == 2) v = bf2f(src[k]); else v = src[k];
        X[(int64_t)i * d + k] = ok ? v : 0.f;
    }
}

// ---------------------------------------------------------------------------
// y = x / sqrt(mean(x^2) + eps) * w, f32 statistics. One workgroup of
// NORM_NT threads per row; the row (d % 4 == 0, d <= 4096) stays in
// registers as up to NORM_V4 float4 per thread between the sum of squares
// and the scaled store.
// ---------------------------------------------------------------------------
// build-time tunable: threads per row of the norm kernels (1024 measured
// faster than 512 and 256: one row per CU, more loads in flight)
#ifndef DG_NORM_THREADS
#define DG_NORM_THREADS 1024
#endif
constexpr int NORM_NT = DG_NORM_THREADS;
constexpr int NORM_V4 = 1024 / NORM_NT;  // float4 per thread: d <= 4096

// With ylo (bf16 outputs only) the row is also left as a pair: y = bf16(v)
// and ylo = bf16(v - y), which carries v to ~16 significant bits (the LM
// head's activation operand).
template <typename TO>
__device__ __forceinline__ void norm_row_store(const float4 (&x)[NORM_V4], int nv, const float* __restrict__ w,
                                               float eps, int d, TO* __restrict__ y, TO* __restrict__ ylo) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NORM_V4; ++j) {
        const int c = threadIdx.x + NORM_NT * j;
        if (c < nv) ss += (x[j].x * x[j].x + x[j].y * x[j].y) + (x[j].z * x[j].z + x[j].w * x[j].w);
    }
    ss = wave_sum(ss);
    __shared__ float red[NORM_NT / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;  // the wave sums in wave order
#pragma unroll
    for (int k = 0; k < NORM_NT / 64; ++k) tot += red[k];
    const float rs = 1.f / sqrtf(tot / (float)d + eps);
    const float4* w4 = reinterpret_cast<const float4*>(w);
#pragma unroll
    for (int j = 0; j < NORM_V4; ++j) {
        const int c = threadIdx.x + NORM_NT * j;
        if (c >= nv) continue;
        const float4 g = w4[c];
        const float v[4] = {x[j].x * rs * g.x, x[j].y * rs * g.y, x[j].z * rs * g.z, x[j].w * rs * g.w};
        if constexpr (sizeof(TO) == 2) {
            uint2 o;
            o.x = f2bf2(v[0], v[1]);
            o.y = f2bf2(v[2], v[3]);
            reinterpret_cast<uint2*>(y)[c] = o;
            if (ylo) {
                uint2 r;
                r.x = f2bf2(v[0] - __uint_as_float(o.x << 16), v[1] - __uint_as_float(o.x & 0xffff0000u));
                r.y = f2bf2(v[2] - __uint_as_float(o.y << 16), v[3] - __uint_as_float(o.y & 0xffff0000u));
                reinterpret_cast<uint2*>(ylo)[c] = r;
            }
        } else {
            reinterpret_cast<float4*>(y)[c] = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

// With nparts > 0 the row first takes a residual update: X += the sum, in
// slice order, of the K-slice partials part[s][i][.] of the product that
// produces it; the updated row is stored back to X and normalised.
template <typename TO>
__global__ void __launch_bounds__(NORM_NT) rmsnorm_kernel(float* __restrict__ X, const float* __restrict__ part, int nparts,
                                                      int n, int d, const float* __restrict__ w, float eps,
                                                      TO* __restrict__ Y, TO* __restrict__ Ylo,
                                                      const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int i = blockIdx.x, nv = d / 4;
    float4* x4 = reinterpret_cast<float4*>(X + (int64_t)i * d);
    float4 x[NORM_V4];
#pragma unroll
    for (int j = 0; j < NORM_V4; ++j) {
        const int c = threadIdx.x + NORM_NT * j;
        x[j] = c < nv ? x4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (nparts > 0) {
        const float4* p4 = reinterpret_cast<const float4*>(part + (int64_t)i * d);
        const int64_t ps = (int64_t)n * nv;  // float4 per slice
        // the loads of up to 8 slices for all of the thread's float4s go out
        // before the first add (clamped addresses, so no branch separates
        // them; the clamped duplicates are not used)
        float4 pv[NORM_V4][8];
#pragma unroll
        for (int j = 0; j < NORM_V4; ++j) {
            const int c = min(threadIdx.x + NORM_NT * j, nv - 1);
#pragma unroll
            for (int s = 0; s < 8; ++s) pv[j][s] = p4[min(s, nparts - 1) * ps + c];
        }
#pragma unroll
        for (int j = 0; j < NORM_V4; ++j) {
            const int c = threadIdx.x + NORM_NT * j;
            if (c >= nv) continue;
            float4 acc = pv[j][0];
#pragma unroll
            for (int s = 1; s < 8; ++s) {
                if (s < nparts) {
                    acc.x += pv[j][s].x; acc.y += pv[j][s].y; acc.z += pv[j][s].z; acc.w += pv[j][s].w;
                }
            }
            for (int s = 8; s < nparts; ++s) {
                const float4 v = p4[s * ps + c];
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
            x[j].x += acc.x; x[j].y += acc.y; x[j].z += acc.z; x[j].w += acc.w;
            x4[c] = x[j];
        }
    }
    norm_row_store<TO>(x, nv, w, eps, d, Y + (int64_t)i * d, Ylo ? Ylo + (int64_t)i * d : nullptr);
}

// ---------------------------------------------------------------------------
// RoPE angles of the rows i in [0, n) at positions pos0 + i: cs[i][d] =
// (cos a, sin a) with a = pos * base^(-2d/hd), d < hd/2 (rotate-half pairs).
// The angle is formed and reduced modulo 2*pi in float64 (positions reach
// 10^5), then sin/cos are taken in float32. Computed once per call and shared
// by every layer, whose rows sit at the same positions.
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(int hd, int64_t pos0, double base, float* __restrict__ cs,
                                  const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int i = blockIdx.x;
    const int half = hd / 2;
    for (int dd = threadIdx.x; dd < half; dd += blockDim.x) {
        const double inv = pow(base, -2.0 * (double)dd / (double)hd);
        double a = (double)(pos0 + i) * inv;
        a = fmod(a, 6.283185307179586476925286766559);
        float sa, ca;
        sincosf((float)a, &sa, &ca);
        cs[((int64_t)i * half + dd) * 2] = ca;
        cs[((int64_t)i * half + dd) * 2 + 1] = sa;
    }
}

// 8 consecutive elements of T <-> float (16 bytes of bf16, 32 of f32)
template <typename T> struct Vec8;
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
        const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
        reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
};
template <> struct Vec8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[8]) {
        const uint4 x = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf2f((uint16_t)(w[j] & 0xffff));
            v[2 * j + 1] = bf2f((uint16_t)(w[j] >> 16));
        }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&v)[8]) {
        uint4 x;
        x.x = f2bf2(v[0], v[1]);
        x.y = f2bf2(v[2], v[3]);
        x.z = f2bf2(v[4], v[5]);
        x.w = f2bf2(v[6], v[7]);
        *reinterpret_cast<uint4*>(p) = x;
    }
};

// 8 consecutive projection outputs at element offset `off` of qkv, or, when
// the projection was split over K (nparts > 1), the sum of its f32 partials
// part[p][.] in slice order rounded to the activation type, exactly what the
// split GEMM's own reduce would have stored in qkv
template <typename T>
__device__ __forceinline__ void qkv_load8(const T* qkv, const float* part, int nparts, int64_t pstride, int64_t off,
                                          float (&v)[8]) {
    if (nparts <= 1) {
        Vec8<T>::load(qkv + off, v);
        return;
    }
    // the loads of up to 8 slices are all issued before the adds
    constexpr int MAXP = 8;
    float4 a[MAXP], b[MAXP];
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p < nparts) {
            const float4* src = reinterpret_cast<const float4*>(part + p * pstride + off);
            a[p] = src[0];
            b[p] = src[1];
        }
    }
    v[0] = a[0].x; v[1] = a[0].y; v[2] = a[0].z; v[3] = a[0].w;
    v[4] = b[0].x; v[5] = b[0].y; v[6] = b[0].z; v[7] = b[0].w;
#pragma unroll
    for (int p = 1; p < MAXP; ++p) {
        if (p < nparts) {
            v[0] += a[p].x; v[1] += a[p].y; v[2] += a[p].z; v[3] += a[p].w;
            v[4] += b[p].x; v[5] += b[p].y; v[6] += b[p].z; v[7] += b[p].w;
        }
    }
    for (int p = MAXP; p < nparts; ++p) {
        float t[8];
        Vec8<float>::load(part + p * pstride + off, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += t[e];
    }
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf2f(f2bf(v[e]));
    }
}

// ---------------------------------------------------------------------------
// RoPE + scatter. qkv [n][(Hq+2Hkv)*hd] (row i at position pos0+i; or its
// K-slice partials, see qkv_load8) ->
//   Q  [Hq][q_ld][hd]        rows q_off + i   (rotated)
//   K  [Hkv][kv_ld][hd]      rows kv_off + i  (rotated)
//   V^T [Hkv][hd][kv_ld]     columns kv_off + i (V stored transposed)
// Columns i in [n, v_zero_to) of V^T are set to 0 (the canvas V^T is read in
// whole 64-key blocks). Rotate-half with the angles of rope_table_kernel:
//   out[d] = x[d] cos a - x[d+hd/2] sin a;  out[d+hd/2] = x[d+hd/2] cos a + x[d] sin a.
// Grid: (tiles, heads), 256 threads. A Q/K workgroup rotates 16 rows in
// 8-element chunks (one chunk pair per thread for hd = 256). A V workgroup
// transposes a 64-row x 64-dim tile through LDS: its loads are issued before
// the first LDS write, and each V^T row segment leaves as 16-byte stores of 8
// consecutive columns.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) rope_scatter_kernel(const T* __restrict__ qkv, const float* __restrict__ part,
                                                           int nparts, int n, int Hq, int Hkv, int hd,
                                                           const float* __restrict__ cs, T* __restrict__ Q,
                                                           int64_t q_ld, int64_t q_off, T* __restrict__ K,
                                                           T* __restrict__ V, int64_t kv_ld, int64_t kv_off,
                                                           int v_zero_to, const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int h = blockIdx.y;
    const int half = hd / 2, width = (Hq + 2 * Hkv) * hd;
    const int64_t pstride = (int64_t)n * width;
    if (h < Hq + Hkv) {
        const int r0 = blockIdx.x * 16;
        const int cpr = half / 8;  // 8-element chunks per half row
        const int rows = min(16, n - r0);
        for (int u = threadIdx.x; u < rows * cpr; u += 256) {
            const int i = r0 + u / cpr, d0 = (u % cpr) * 8;
            const int64_t src = (int64_t)i * width + h * hd;
            float x1[8], x2[8], y1[8], y2[8];
            qkv_load8<T>(qkv, part, nparts, pstride, src + d0, x1);
            qkv_load8<T>(qkv, part, nparts, pstride, src + half + d0, x2);
            const float4* c4 = reinterpret_cast<const float4*>(cs + ((int64_t)i * half + d0) * 2);
            const float4 c[4] = {c4[0], c4[1], c4[2], c4[3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                y1[2 * j] = x1[2 * j] * c[j].x - x2[2 * j] * c[j].y;
                y2[2 * j] = x2[2 * j] * c[j].x + x1[2 * j] * c[j].y;
                y1[2 * j + 1] = x1[2 * j + 1] * c[j].z - x2[2 * j + 1] * c[j].w;
                y2[2 * j + 1] = x2[2 * j + 1] * c[j].z + x1[2 * j + 1] * c[j].w;
            }
            T* dst = h < Hq ? Q + ((int64_t)h * q_ld + q_off + i) * hd
                            : K + ((int64_t)(h - Hq) * kv_ld + kv_off + i) * hd;
            Vec8<T>::store(dst + d0, y1);
            Vec8<T>::store(dst + half + d0, y2);
        }
    } else {
        // V: a 64-row x 64-dim tile per workgroup (x = row tile * hd/64 + dim
        // tile), transposed through LDS
        __shared__ float vt[64 * 65];
        const int dq = hd / 64;
        const int r0 = (blockIdx.x / dq) * 64, d0 = (blockIdx.x % dq) * 64;
        const int rows = min(64, max(n, v_zero_to) - r0);
        if (rows <= 0) return;
        const int hv = h - Hq - Hkv;
        float v[2][8];
#pragma unroll
        for (int j = 0; j < 2; ++j) {  // 64 rows x 8 chunks of 8 dims: two per thread
            const int u = threadIdx.x + 256 * j;
            const int r = u / 8, i = r0 + r;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
            if (r < rows && i < n)
                qkv_load8<T>(qkv, part, nparts, pstride, (int64_t)i * width + h * hd + d0 + (u % 8) * 8, v[j]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int u = threadIdx.x + 256 * j;
            const int r = u / 8, c = (u % 8) * 8;
            if (r < rows)
#pragma unroll
                for (int e = 0; e < 8; ++e) vt[r * 65 + c + e] = v[j][e];
        }
        __syncthreads();
        // output unit: (dim d, 8 consecutive columns)
        const int cgs = (rows + 7) / 8;
        const bool vec = ((kv_off + r0) % 8) == 0 && rows % 8 == 0;
        for (int u = threadIdx.x; u < 64 * cgs; u += 256) {
            const int d = u / cgs, c0 = (u % cgs) * 8;
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = c0 + e < rows ? vt[(c0 + e) * 65 + d] : 0.f;
            T* dst = V + ((int64_t)hv * hd + d0 + d) * kv_ld + kv_off + r0 + c0;
            if (vec) {
                Vec8<T>::store(dst, o);
            } else {
                for (int e = 0; e < 8 && c0 + e < rows; ++e) {
                    if constexpr (sizeof(T) == 2) dst[e] = f2bf(o[e]); else dst[e] = o[e];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Router top-k. logits r [n][E] f32 (+ bias [E]); one wavefront (workgroup) per token.
// k rounds of a wavefront argmax (value desc, expert id asc); gates are the
// softmax over the k selected logits (f32).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) router_topk_kernel(const float* __restrict__ r, int nparts, int64_t pstride,
                                                         const float* __restrict__ bias, int n, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ gates,
                                                         const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int tokn = blockIdx.x;
    const int lane = threadIdx.x;
    if (tokn >= n) return;
    constexpr int PER = 8;  // up to 512 experts
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        int e = lane + 64 * j;
        v[j] = -INFINITY;
        if (e < E) {
            // the logit: its K-slice partial sums added in slice order (the
            // loads of up to 16 slices are all issued before the adds: their
            // addresses are clamped, so no branch separates them)
            const float* src = r + (int64_t)tokn * E + e;
            float xs[16];
#pragma unroll
            for (int p = 0; p < 16; ++p) xs[p] = src[min(p, nparts - 1) * pstride];
            float x = xs[0];
#pragma unroll
            for (int p = 1; p < 16; ++p) x = p < nparts ? x + xs[p] : x;
            for (int p = 16; p < nparts; ++p) x += src[p * pstride];
            x += bias[e];
            v[j] = x == x ? x : -INFINITY;  // a NaN logit ranks last
        }
    }
    // every round picks an expert not taken yet (ties and -inf go to the lowest
    // id), so the k ids are always distinct and valid
    bool taken[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) taken[j] = false;
    float sel[16];
    int sid[16];
    for (int s = 0; s < k; ++s) {
        ArgMax best{-INFINITY, 0x7fffffff};
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            int e = lane + 64 * j;
            if (e < E && !taken[j]) best = argmax_merge(best, ArgMax{v[j], e});
        }
        best = wave_argmax(best);
        sel[s] = best.v;
        sid[s] = best.i;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (lane + 64 * j == best.i) taken[j] = true;
    }
    if (lane == 0) {
        float m = sel[0];
        float den = 0.f;
        for (int s = 0; s < k; ++s) den += __expf(sel[s] - m);
        for (int s = 0; s < k; ++s) {
            ids[(int64_t)tokn * k + s] = sid[s];
            gates[(int64_t)tokn * k + s] = __expf(sel[s] - m) / den;
        }
    }
}

// ---------------------------------------------------------------------------
// Expert histogram and permutation, one workgroup of 1024 threads (16 waves).
// Slots: routed assignments grouped by expert, inside a group in assignment
// order (token-major); then the shared expert's n slots in token order.
// offsets has E+2 entries (group g = [offsets[g], offsets[g+1]), g = E is the
// shared expert); perm[slot] = token; slot_of[token*k + j] = slot of its j-th
// expert. The groups with rows are listed in increasing id (the shared expert
// last) in two lists: hitB = [count, ids...] for groups of at least big_min
// rows (none if big_min <= 0) with hitB_mb = their largest number of 256-row
// blocks, and hit = [count, ids...] for the rest with hit_mb = their largest
// number of 64-row blocks.
//
// A stable counting sort without serial scans: the assignments are cut into
// chunks of 64 (one wavefront each). Inside a chunk the lanes holding the
// same expert id are found with one ballot per id bit, so a lane's rank among
// them is a popcount and the chunk's count per expert is written by its first
// lane. A scan over the chunks per expert and one over the experts then give
// every assignment its slot: offset(expert) + earlier chunks + rank.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) hist_permute_kernel(const int32_t* __restrict__ ids, int n, int k, int E,
                                                            int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ slot_of, int32_t* __restrict__ hit,
                                                            int32_t* __restrict__ hit_mb,
                                                            int32_t* __restrict__ hitB,
                                                            int32_t* __restrict__ hitB_mb, int big_min,
                                                            int32_t* __restrict__ hit_out,
                                                            const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    extern __shared__ __align__(16) unsigned char shraw[];
    const int total = n * k;
    const int nch = (total + 63) / 64;
    int32_t* off = reinterpret_cast<int32_t*>(shraw);            // [E + 2]
    int32_t* tot = off + E + 2;                                    // [E]
    uint16_t* cbase = reinterpret_cast<uint16_t*>(tot + E);        // [nch][E] assignments of e in earlier chunks
    uint16_t* esid = cbase + (size_t)nch * E;                      // [total] expert of each assignment
    uint8_t* ccnt = reinterpret_cast<uint8_t*>(esid + total);      // [nch][E] count of e in the chunk
    uint8_t* rank = ccnt + (size_t)nch * E;                        // [total] rank inside its chunk
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < nch * E; i += 1024) ccnt[i] = 0;
    __syncthreads();
    int nbits = 1;
    while ((1 << nbits) <= E) ++nbits;  // ids 0..E (E marks an empty lane)
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int c = wave; c < nch; c += 16) {
        const int a = c * 64 + lane;
        const int e = a < total ? ids[a] : E;
        unsigned long long peers = ~0ull;
        for (int bit = 0; bit < nbits; ++bit) {
            const unsigned long long m = __ballot((e >> bit) & 1);
            peers &= ((e >> bit) & 1) ? m : ~m;
        }
        if (a < total) {
            const int r = __popcll(peers & lt);
            esid[a] = (uint16_t)e;
            rank[a] = (uint8_t)r;
            if (r == 0) ccnt[c * E + e] = (uint8_t)__popcll(peers);
        }
    }
    __syncthreads();
    // per expert: running count over the chunks
    for (int e = tid; e < E; e += 1024) {
        int run = 0;
        for (int c = 0; c < nch; ++c) {
            cbase[c * E + e] = (uint16_t)run;
            run += ccnt[c * E + e];
        }
        tot[e] = run;
    }
    __syncthreads();
    // exclusive scan over the experts, the hit list and the largest block
    // count, by wavefront 0 (each lane takes a run of consecutive experts)
    if (wave == 0) {
        const int per = (E + 63) / 64;
        const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
        auto is_big = [&](int rows) { return big_min > 0 && rows >= big_min; };
        int sum = 0, nzs = 0, nzb = 0, mbs = 0, mbb = 0;
        for (int e = e0; e < e1; ++e) {
            const int t = tot[e];
            sum += t;
            if (t > 0) {
                if (is_big(t)) { ++nzb; mbb = max(mbb, (t + 255) / 256); }
                else { ++nzs; mbs = max(mbs, (t + 63) / 64); }
            }
        }
        int isum = sum, izs = nzs, izb = nzb;
        for (int o = 1; o < 64; o <<= 1) {
            const int vs = __shfl_up(isum, o, 64), va = __shfl_up(izs, o, 64), vb = __shfl_up(izb, o, 64);
            if (lane >= o) { isum += vs; izs += va; izb += vb; }
            mbs = max(mbs, __shfl_xor(mbs, o, 64));
            mbb = max(mbb, __shfl_xor(mbb, o, 64));
        }
        int run = isum - sum, hs = izs - nzs, hb = izb - nzb;
        for (int e = e0; e < e1; ++e) {
            off[e] = run;
            run += tot[e];
            if (tot[e] > 0) {
                if (is_big(tot[e])) hitB[1 + hb++] = e;
                else hit[1 + hs++] = e;
            }
        }
        if (lane == 63) {
            // izs / izb are now the numbers of routed groups in each list
            off[E] = isum;
            off[E + 1] = isum + n;
            if (hit_out) *hit_out = izs + izb;  // routed experts only
            int cs = izs, cb = izb;
            if (n > 0) {  // the shared expert: every token
                if (is_big(n)) { hitB[1 + cb++] = E; mbb = max(mbb, (n + 255) / 256); }
                else { hit[1 + cs++] = E; mbs = max(mbs, (n + 63) / 64); }
            }
            hit[0] = cs;
            hitB[0] = cb;
            *hit_mb = max(mbs, 1);
            *hitB_mb = max(mbb, 1);
        }
    }
    __syncthreads();
    for (int e = tid; e <= E + 1; e += 1024) offsets[e] = off[e];
    for (int a = tid; a < total; a += 1024) {
        const int e = esid[a];
        const int slot = off[e] + cbase[(a >> 6) * E + e] + rank[a];
        perm[slot] = a / k;
        slot_of[a] = slot;
    }
    for (int i = tid; i < n; i += 1024) perm[off[E] + i] = i;
}

// ---------------------------------------------------------------------------
// X[i] += Y[shared slot of i] + sum_j gate[i][j] * Y[slot_of[i][j]] (j ascending).
// One workgroup per token (d % 4 == 0, d <= 4096). With nw != NULL the new row
// is also normalised (the next layer's pre-attention RMSNorm, or the final
// norm) into A, from the registers that hold it.
// ---------------------------------------------------------------------------
template <typename TO>
__global__ void __launch_bounds__(NORM_NT) combine_kernel(float* __restrict__ X, int d, const float* __restrict__ Y,
                                                      const int32_t* __restrict__ slot_of,
                                                      const float* __restrict__ gates, int k, int shared_off,
                                                      const float* __restrict__ nw, float eps, TO* __restrict__ A,
                                                      TO* __restrict__ Alo, const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int i = blockIdx.x, nv = d / 4;
    __shared__ int sl[16];
    __shared__ float gt[16];
    if (threadIdx.x < k) {
        sl[threadIdx.x] = slot_of[(int64_t)i * k + threadIdx.x];
        gt[threadIdx.x] = gates[(int64_t)i * k + threadIdx.x];
    }
    __syncthreads();
    const float4* ysh = reinterpret_cast<const float4*>(Y + (int64_t)(shared_off + i) * d);
    float4* xr = reinterpret_cast<float4*>(X + (int64_t)i * d);
    float4 x[NORM_V4];
#pragma unroll
    for (int j = 0; j < NORM_V4; ++j) {
        const int c = threadIdx.x + NORM_NT * j;
        x[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c >= nv) continue;
        float4 acc = ysh[c];
        for (int e = 0; e < k; ++e) {
            const float4 y = reinterpret_cast<const float4*>(Y + (int64_t)sl[e] * d)[c];
            const float g = gt[e];
            acc.x += g * y.x; acc.y += g * y.y; acc.z += g * y.z; acc.w += g * y.w;
        }
        float4 v = xr[c];
        v.x += acc.x; v.y += acc.y; v.z += acc.z; v.w += acc.w;
        xr[c] = v;
        x[j] = v;
    }
    if (nw) norm_row_store<TO>(x, nv, nw, eps, d, A + (int64_t)i * d, Alo ? Alo + (int64_t)i * d : nullptr);
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
hipError_t launch_embed(const void* E, int act_f32, int d, int V, const int32_t* tok, int n, float* X,
                        const int32_t* state, hipStream_t st) {
    if (act_f32) embed_kernel<float><<<n, 256, 0, st>>>((const float*)E, d, V, tok, X, state);
    else embed_kernel<uint16_t><<<n, 256, 0, st>>>((const uint16_t*)E, d, V, tok, X, state);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* X, int n, int d, const float* w, float eps, void* Y, int act_f32,
                          const int32_t* state, hipStream_t st, void* Ylo) {
    return launch_residual_rmsnorm(const_cast<float*>(X), nullptr, 0, n, d, w, eps, Y, act_f32, state, st, Ylo);
}

hipError_t launch_residual_rmsnorm(float* X, const float* part, int nparts, int n, int d, const float* w, float eps,
                                   void* Y, int act_f32, const int32_t* state, hipStream_t st, void* Ylo) {
    if (d % 4 || d > 4 * NORM_NT * NORM_V4 || (nparts > 0 && !part) || (Ylo && act_f32)) return hipErrorInvalidValue;
    if (act_f32) rmsnorm_kernel<float><<<n, NORM_NT, 0, st>>>(X, part, nparts, n, d, w, eps, (float*)Y, nullptr, state);
    else
        rmsnorm_kernel<uint16_t><<<n, NORM_NT, 0, st>>>(X, part, nparts, n, d, w, eps, (uint16_t*)Y, (uint16_t*)Ylo,
                                                     state);
    return hipGetLastError();
}

hipError_t launch_rope_table(int n, int hd, int64_t pos0, double base, float* cs, const int32_t* state,
                             hipStream_t st) {
    rope_table_kernel<<<n, std::max(64, std::min(256, hd / 2)), 0, st>>>(hd, pos0, base, cs, state);
    return hipGetLastError();
}

hipError_t launch_rope_scatter(const void* qkv, const float* part, int nparts, int act_f32, int n, int Hq, int Hkv,
                               int hd, const float* cs, void* Q,
                               int64_t q_ld, int64_t q_off, void* K, void* V, int64_t kv_ld, int64_t kv_off,
                               int v_zero_to, const int32_t* state, hipStream_t st) {
    if (hd % 64 || hd > 256) return hipErrorInvalidValue;
    const int rows = std::max(n, v_zero_to);
    // x: 16-row tiles (Q/K) or 64-row x 64-dim tiles (V), whichever are more
    const dim3 grid(std::max((rows + 15) / 16, (rows + 63) / 64 * (hd / 64)), Hq + 2 * Hkv);
    const size_t lds = 0;
    if (act_f32)
        rope_scatter_kernel<float><<<grid, 256, lds, st>>>((const float*)qkv, part, nparts, n, Hq, Hkv, hd, cs, (float*)Q, q_ld,
                                                           q_off, (float*)K, (float*)V, kv_ld, kv_off, v_zero_to,
                                                           state);
    else
        rope_scatter_kernel<uint16_t><<<grid, 256, lds, st>>>((const uint16_t*)qkv, part, nparts, n, Hq, Hkv, hd, cs, (uint16_t*)Q,
                                                              q_ld, q_off, (uint16_t*)K, (uint16_t*)V, kv_ld, kv_off,
                                                              v_zero_to, state);
    return hipGetLastError();
}

hipError_t launch_router_topk(const float* r, int nparts, const float* bias, int n, int E, int k, int32_t* ids,
                              float* gates, const int32_t* state, hipStream_t st) {
    router_topk_kernel<<<n, 64, 0, st>>>(r, std::max(nparts, 1), (int64_t)n * E, bias, n, E, k, ids, gates, state);
    return hipGetLastError();
}

static size_t hist_permute_lds(int n, int k, int E) {
    const size_t total = (size_t)n * k, nch = (total + 63) / 64;
    // off, tot (int32); cbase (u16 [nch][E]); esid (u16 [total]); ccnt (u8 [nch][E]); rank (u8 [total])
    return (size_t)(2 * E + 2) * 4 + nch * E * 2 + total * 2 + nch * E + total;
}

int hist_permute_max_rows(int k, int E) {
    if (k < 1 || E < 1 || E > 65535) return 0;
    int best = 0;
    for (int n = 1; (size_t)n * k <= 65535 && hist_permute_lds(n, k, E) <= 160 * 1024; ++n) best = n;
    return best;
}

hipError_t launch_hist_permute(const int32_t* ids, int n, int k, int E, int32_t* offsets, int32_t* perm,
                               int32_t* slot_of, int32_t* hit, int32_t* hit_mb, int32_t* hitB, int32_t* hitB_mb,
                               int big_min, int32_t* hit_out, const int32_t* state, hipStream_t st) {
    const size_t total = (size_t)n * k;
    const size_t lds = hist_permute_lds(n, k, E);
    if (lds > 160 * 1024 || E > 65535 || total > 65535) return hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(hist_permute_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hist_permute_kernel<<<1, 1024, lds, st>>>(ids, n, k, E, offsets, perm, slot_of, hit, hit_mb, hitB, hitB_mb,
                                               big_min, hit_out, state);
    return hipGetLastError();
}

hipError_t launch_combine(float* X, int n, int d, const float* Y, const int32_t* slot_of, const float* gates, int k,
                          int shared_off, const float* norm_w, float eps, void* A, int act_f32, const int32_t* state,
                          hipStream_t st, void* Alo) {
    if (d % 4 || d > 4 * NORM_NT * NORM_V4 || k > 16 || (Alo && act_f32)) return hipErrorInvalidValue;
    if (act_f32)
        combine_kernel<float><<<n, NORM_NT, 0, st>>>(X, d, Y, slot_of, gates, k, shared_off, norm_w, eps, (float*)A,
                                                 nullptr, state);
    else
        combine_kernel<uint16_t><<<n, NORM_NT, 0, st>>>(X, d, Y, slot_of, gates, k, shared_off, norm_w, eps,
                                                    (uint16_t*)A, (uint16_t*)Alo, state);
    return hipGetLastError();
}

}  // namespace dg
