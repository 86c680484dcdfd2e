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
__global__ void __launch_bounds__(256) embed_kernel(const TE* __restrict__ E, int d, const int32_t* __restrict__ tok,
                                                    float* __restrict__ X, const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int i = blockIdx.x;
    const int64_t t = tok[i];
    const TE* src = E + t * d;
    for (int k = threadIdx.x; k < d; k += 256) {
        float v;
        if constexpr (sizeof(TE) == 2) v = bf2f(src[k]); else v = src[k];
        X[(int64_t)i * d + k] = v;
    }
}

// ---------------------------------------------------------------------------
// y = x / sqrt(mean(x^2) + eps) * w, f32 statistics. One workgroup per row.
// ---------------------------------------------------------------------------
template <typename TO>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ X, int d, const float* __restrict__ w,
                                                      float eps, TO* __restrict__ Y, const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int i = blockIdx.x;
    const float* x = X + (int64_t)i * d;
    float ss = 0.f;
    for (int k = threadIdx.x; k < d; k += 256) ss += x[k] * x[k];
    ss = wave_sum(ss);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float rs = 1.f / sqrtf(tot / (float)d + eps);
    for (int k = threadIdx.x; k < d; k += 256) {
        float v = x[k] * rs * w[k];
        if constexpr (sizeof(TO) == 2) Y[(int64_t)i * d + k] = f2bf(v); else Y[(int64_t)i * d + k] = v;
    }
}

// ---------------------------------------------------------------------------
// RoPE + scatter. qkv [n][(Hq+2Hkv)*hd] (row i at position pos0+i) ->
//   Q  [Hq][q_ld][hd]        rows q_off + i   (rotated)
//   K  [Hkv][kv_ld][hd]      rows kv_off + i  (rotated)
//   V^T [Hkv][hd][kv_ld]     columns kv_off + i (V stored transposed)
// Columns i in [n, v_zero_to) of V^T are set to 0 (the canvas V^T is read in
// whole 64-key blocks). Rotate-half: for d < hd/2, a = pos * base^(-2d/hd):
//   out[d] = x[d] cos a - x[d+hd/2] sin a;  out[d+hd/2] = x[d+hd/2] cos a + x[d] sin a.
// The angle is formed and reduced modulo 2*pi in float64 (positions reach
// 10^5), then sin/cos are taken in float32. One workgroup per row i handles
// every head; thread d owns the rotation pair (d, d + hd/2).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void rope_scatter_kernel(const T* __restrict__ qkv, int n, int Hq, int Hkv, int hd, int64_t pos0,
                                    double base, T* __restrict__ Q, int64_t q_ld, int64_t q_off,
                                    T* __restrict__ K, T* __restrict__ V, int64_t kv_ld, int64_t kv_off,
                                    int v_zero_to, const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int i = blockIdx.x;
    const int half = hd / 2;
    auto st = [&](T* p, float v) {
        if constexpr (sizeof(T) == 2) *p = f2bf(v); else *p = v;
    };
    if (i >= n) {  // zero V^T columns past the rows
        for (int e = threadIdx.x; e < Hkv * hd; e += blockDim.x)
            st(V + ((int64_t)(e / hd) * hd + e % hd) * kv_ld + kv_off + i, 0.f);
        return;
    }
    const int width = (Hq + 2 * Hkv) * hd;
    const T* src = qkv + (int64_t)i * width;
    auto ld = [&](int j) -> float {
        if constexpr (sizeof(T) == 2) return bf2f(src[j]); else return src[j];
    };
    for (int dd = threadIdx.x; dd < half; dd += blockDim.x) {
        const double inv = pow(base, -2.0 * (double)dd / (double)hd);
        double a = (double)(pos0 + i) * inv;
        a = fmod(a, 6.283185307179586476925286766559);
        float sa, ca;
        sincosf((float)a, &sa, &ca);
        for (int h = 0; h < Hq + 2 * Hkv; ++h) {
            float x1 = ld(h * hd + dd), x2 = ld(h * hd + dd + half);
            if (h < Hq + Hkv) {
                const float y1 = x1 * ca - x2 * sa;
                const float y2 = x2 * ca + x1 * sa;
                x1 = y1;
                x2 = y2;
            }
            if (h < Hq) {
                T* dst = Q + ((int64_t)h * q_ld + q_off + i) * hd;
                st(dst + dd, x1);
                st(dst + dd + half, x2);
            } else if (h < Hq + Hkv) {
                T* dst = K + ((int64_t)(h - Hq) * kv_ld + kv_off + i) * hd;
                st(dst + dd, x1);
                st(dst + dd + half, x2);
            } else {
                T* dst = V + (int64_t)(h - Hq - Hkv) * hd * kv_ld + kv_off + i;
                st(dst + (int64_t)dd * kv_ld, x1);
                st(dst + (int64_t)(dd + half) * kv_ld, x2);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Router top-k. logits r [n][E] f32 (+ bias [E]); one wavefront per token.
// k rounds of a wavefront argmax (value desc, expert id asc); gates are the
// softmax over the k selected logits (f32).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) router_topk_kernel(const float* __restrict__ r, const float* __restrict__ bias,
                                                          int n, int E, int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ gates, const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int tokn = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (tokn >= n) return;
    constexpr int PER = 8;  // up to 512 experts
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        int e = lane + 64 * j;
        v[j] = e < E ? r[(int64_t)tokn * E + e] + bias[e] : -INFINITY;
    }
    float sel[16];
    int sid[16];
    for (int s = 0; s < k; ++s) {
        ArgMax best{-INFINITY, 0x7fffffff};
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            int e = lane + 64 * j;
            if (e < E) best = argmax_merge(best, ArgMax{v[j], e});
        }
        best = wave_argmax(best);
        sel[s] = best.v;
        sid[s] = best.i;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (lane + 64 * j == best.i) v[j] = -INFINITY;
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
// expert. Counts come from LDS atomics; placement is deterministic: wave w
// handles experts w, w+16, ... and walks the assignments in chunks of 64 with
// a ballot, so the rank inside a group is a popcount.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) hist_permute_kernel(const int32_t* __restrict__ ids, int n, int k, int E,
                                                            int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ slot_of, int32_t* __restrict__ hit,
                                                            int32_t* __restrict__ hit_mb,
                                                            const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    extern __shared__ int32_t sh[];
    const int total = n * k;
    int32_t* cnt = sh;               // [E + 1]
    int32_t* off = sh + E + 1;       // [E + 2]
    int32_t* sid = off + E + 2;      // [total]
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e <= E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int a = tid; a < total; a += 1024) {
        int e = ids[a];
        sid[a] = e;
        atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0, h = 0, mbm = n > 0 ? (n + 63) / 64 : 0;
        for (int e = 0; e < E; ++e) {
            off[e] = run;
            run += cnt[e];
            if (cnt[e] > 0) {
                hit[1 + h++] = e;
                mbm = max(mbm, (cnt[e] + 63) / 64);
            }
        }
        off[E] = run;
        off[E + 1] = run + n;
        if (n > 0) hit[1 + h++] = E;   // the shared expert: every token
        hit[0] = h;
        *hit_mb = mbm;
    }
    __syncthreads();
    for (int e = tid; e <= E + 1; e += 1024) offsets[e] = off[e];
    for (int e = wave; e < E; e += 16) {
        if (cnt[e] == 0) continue;
        int base = off[e];
        for (int c = 0; c < total; c += 64) {
            const int a = c + lane;
            const bool hit = a < total && sid[a] == e;
            const unsigned long long m = __ballot(hit);
            if (hit) {
                const int rank = __popcll(m & ((1ull << lane) - 1ull));
                const int slot = base + rank;
                perm[slot] = a / k;
                slot_of[a] = slot;
            }
            base += __popcll(m);
        }
    }
    for (int i = tid; i < n; i += 1024) perm[off[E] + i] = i;
}

// ---------------------------------------------------------------------------
// X[i] += Y[shared slot of i] + sum_j gate[i][j] * Y[slot_of[i][j]] (j ascending).
// One workgroup per token.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) combine_kernel(float* __restrict__ X, int d, const float* __restrict__ Y,
                                                      const int32_t* __restrict__ slot_of,
                                                      const float* __restrict__ gates, int k, int shared_off,
                                                      const int32_t* __restrict__ state) {
    if (state && state[0]) return;
    const int i = blockIdx.x;
    __shared__ int sl[16];
    __shared__ float gt[16];
    if (threadIdx.x < k) {
        sl[threadIdx.x] = slot_of[(int64_t)i * k + threadIdx.x];
        gt[threadIdx.x] = gates[(int64_t)i * k + threadIdx.x];
    }
    __syncthreads();
    const float* ysh = Y + (int64_t)(shared_off + i) * d;
    for (int c = threadIdx.x; c < d; c += 256) {
        float acc = ysh[c];
        for (int j = 0; j < k; ++j) acc += gt[j] * Y[(int64_t)sl[j] * d + c];
        X[(int64_t)i * d + c] += acc;
    }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
hipError_t launch_embed(const void* E, int act_f32, int d, const int32_t* tok, int n, float* X,
                        const int32_t* state, hipStream_t st) {
    if (act_f32) embed_kernel<float><<<n, 256, 0, st>>>((const float*)E, d, tok, X, state);
    else embed_kernel<uint16_t><<<n, 256, 0, st>>>((const uint16_t*)E, d, tok, X, state);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* X, int n, int d, const float* w, float eps, void* Y, int act_f32,
                          const int32_t* state, hipStream_t st) {
    if (act_f32) rmsnorm_kernel<float><<<n, 256, 0, st>>>(X, d, w, eps, (float*)Y, state);
    else rmsnorm_kernel<uint16_t><<<n, 256, 0, st>>>(X, d, w, eps, (uint16_t*)Y, state);
    return hipGetLastError();
}

hipError_t launch_rope_scatter(const void* qkv, int act_f32, int n, int Hq, int Hkv, int hd, int64_t pos0,
                               double base, void* Q, int64_t q_ld, int64_t q_off, void* K, void* V, int64_t kv_ld,
                               int64_t kv_off, int v_zero_to, const int32_t* state, hipStream_t st) {
    const int rows = std::max(n, v_zero_to);
    const int threads = std::max(64, std::min(256, hd / 2));
    if (act_f32)
        rope_scatter_kernel<float><<<rows, threads, 0, st>>>((const float*)qkv, n, Hq, Hkv, hd, pos0, base, (float*)Q,
                                                             q_ld, q_off, (float*)K, (float*)V, kv_ld, kv_off,
                                                             v_zero_to, state);
    else
        rope_scatter_kernel<uint16_t><<<rows, threads, 0, st>>>((const uint16_t*)qkv, n, Hq, Hkv, hd, pos0, base,
                                                                (uint16_t*)Q, q_ld, q_off, (uint16_t*)K,
                                                                (uint16_t*)V, kv_ld, kv_off, v_zero_to, state);
    return hipGetLastError();
}

hipError_t launch_router_topk(const float* r, const float* bias, int n, int E, int k, int32_t* ids, float* gates,
                              const int32_t* state, hipStream_t st) {
    router_topk_kernel<<<(n + 3) / 4, 256, 0, st>>>(r, bias, n, E, k, ids, gates, state);
    return hipGetLastError();
}

hipError_t launch_hist_permute(const int32_t* ids, int n, int k, int E, int32_t* offsets, int32_t* perm,
                               int32_t* slot_of, int32_t* hit, int32_t* hit_mb, const int32_t* state,
                               hipStream_t st) {
    size_t lds = (size_t)(2 * E + 3 + n * k) * sizeof(int32_t);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(hist_permute_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hist_permute_kernel<<<1, 1024, lds, st>>>(ids, n, k, E, offsets, perm, slot_of, hit, hit_mb, state);
    return hipGetLastError();
}

hipError_t launch_combine(float* X, int n, int d, const float* Y, const int32_t* slot_of, const float* gates, int k,
                          int shared_off, const int32_t* state, hipStream_t st) {
    combine_kernel<<<n, 256, 0, st>>>(X, d, Y, slot_of, gates, k, shared_off, state);
    return hipGetLastError();
}

}  // namespace dg
