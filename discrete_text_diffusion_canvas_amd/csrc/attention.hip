// Attention for gfx950: decoder canvas attention (bidirectional inside the
// canvas plus cross-attention into the cached prefix, one joint softmax per
// head) and the encoder's causal, sliding-window attention.
//
// DiffusionGemma model card (zh-TW), "模型總覽" (overview): the decoder
// processes the canvas with bidirectional attention and reads the encoder's
// cached context through cross-attention; the encoder is autoregressive; the
// spec table gives a 1024-token sliding window. One joint softmax over
// [prefix rows in the window || canvas rows] is the reading taken for how the
// two attentions combine.
//
// Flash-style: a workgroup (4 waves) owns 64 query rows of one head and a
// contiguous slice of the key range (split-KV); each wave owns 16 query rows.
// Per 64-key block: K is staged in LDS row-major, V transposed ([d][key]);
// S = Q K^T with MFMA (Q fragments stay in registers), online softmax in f32,
// P goes through LDS to become the A operand of O += P V. Split slices write
// unnormalised partials (O, max, sum) that a merge kernel combines.
#include "common.hpp"
#include "layer.hpp"

namespace dg {

template <typename TL> struct AFrag;
template <> struct AFrag<uint16_t> { typedef u16x8 type; };
template <> struct AFrag<float> { struct type { f32x4 lo, hi; }; };

__device__ __forceinline__ f32x4 amfma(const u16x8& a, const u16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 amfma(const AFrag<float>::type& a, const AFrag<float>::type& b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], c, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], c, 0, 0, 0);
    return c;
}
template <typename TL>
__device__ __forceinline__ typename AFrag<TL>::type afrag_ld(const TL* p);
template <>
__device__ __forceinline__ u16x8 afrag_ld<uint16_t>(const uint16_t* p) { return *reinterpret_cast<const u16x8*>(p); }
template <>
__device__ __forceinline__ AFrag<float>::type afrag_ld<float>(const float* p) {
    AFrag<float>::type f;
    f.lo = reinterpret_cast<const f32x4*>(p)[0];
    f.hi = reinterpret_cast<const f32x4*>(p)[1];
    return f;
}
__device__ __forceinline__ float to_f(uint16_t v) { return bf2f(v); }
__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ void from_f(uint16_t* p, float v) { *p = f2bf(v); }
__device__ __forceinline__ void from_f(float* p, float v) { *p = v; }

constexpr int KB = 64;  // keys per block

template <typename TL, int HD>
__global__ void __launch_bounds__(256) attention_kernel(AttnArgs a) {
    if (a.state && a.state[0]) return;
    constexpr int PADL = 16 / sizeof(TL);
    constexpr int SKK = HD + PADL;       // K tile row stride
    constexpr int SVT = KB + PADL;       // V^T row stride
    constexpr int SP = KB + PADL;        // P row stride
    constexpr int NT_D = HD / 16;        // output n-tiles over head_dim
    constexpr int KS = HD / 32;          // k-steps over head_dim
    extern __shared__ __align__(16) unsigned char smem[];
    TL* Ks = reinterpret_cast<TL*>(smem);
    TL* Vt = Ks + KB * SKK;
    TL* Ps = Vt + HD * SVT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int h = blockIdx.y;
    const int g = h / (a.Hq / a.Hkv);
    const int q0 = blockIdx.x * 64;
    const int qw0 = q0 + wave * 16;  // this wave's first query row

    // virtual key range: segment 1 rows [s1, e1) then segment 2 rows [0, n2)
    const int64_t L1 = a.e1 - a.s1;
    const int64_t Ltot = L1 + a.n2;
    int64_t kbeg = 0, kend = Ltot;
    if (a.causal) {
        // query positions in this tile: [qpos0 + q0, qpos0 + q0 + 63]
        const int64_t qlo = a.qpos0 + q0, qhi = a.qpos0 + min(q0 + 63, a.nq - 1);
        kend = min<int64_t>(Ltot, qhi - a.s1 + 1);
        if (a.window > 0) kbeg = max<int64_t>(0, qlo - a.window + 1 - a.s1);
    }
    const int64_t span = max<int64_t>(0, kend - kbeg);
    const int64_t per = ((span + a.splits - 1) / a.splits + KB - 1) / KB * KB;
    const int64_t kb0 = kbeg + per * blockIdx.z;
    const int64_t kb1 = min<int64_t>(kend, kb0 + per);

    const TL* Qh = reinterpret_cast<const TL*>(a.Q) + (int64_t)h * a.ldq * HD;
    typename AFrag<TL>::type qf[KS];
    const int myq = qw0 + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (myq < a.nq) {
            qf[ks] = afrag_ld<TL>(Qh + (int64_t)myq * HD + ks * 32 + lg * 8);
        } else {
            if constexpr (sizeof(TL) == 2) qf[ks] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            else { qf[ks].lo = f32x4{0, 0, 0, 0}; qf[ks].hi = qf[ks].lo; }
        }
    }
    f32x4 o[NT_D];
#pragma unroll
    for (int j = 0; j < NT_D; ++j) o[j] = f32x4{0, 0, 0, 0};
    float m_run[4], l_run[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.f; }
    const float scale = 1.f / sqrtf((float)HD);

    const TL* K1 = reinterpret_cast<const TL*>(a.K1) + (int64_t)g * a.ld1 * HD;
    const TL* V1 = reinterpret_cast<const TL*>(a.V1) + (int64_t)g * a.ld1 * HD;
    const TL* K2 = a.K2 ? reinterpret_cast<const TL*>(a.K2) + (int64_t)g * a.ld2 * HD : nullptr;
    const TL* V2 = a.V2 ? reinterpret_cast<const TL*>(a.V2) + (int64_t)g * a.ld2 * HD : nullptr;

    for (int64_t kb = kb0; kb < kb1; kb += KB) {
        // ---- stage K (row-major) and V (transposed) for keys [kb, kb+64) ----
        constexpr int CH = KB * HD / 8;  // 8-element chunks
        for (int c = tid; c < CH; c += 256) {
            const int kr = c / (HD / 8), dc = (c % (HD / 8)) * 8;
            const int64_t j = kb + kr;
            TL kv[8], vv[8];
            if (j < kb1) {
                const TL* kp;
                const TL* vp;
                if (j < L1) { kp = K1 + (a.s1 + j) * HD; vp = V1 + (a.s1 + j) * HD; }
                else { kp = K2 + (j - L1) * HD; vp = V2 + (j - L1) * HD; }
                if constexpr (sizeof(TL) == 2) {
                    u16x8 x = *reinterpret_cast<const u16x8*>(kp + dc);
                    u16x8 y = *reinterpret_cast<const u16x8*>(vp + dc);
#pragma unroll
                    for (int q = 0; q < 8; ++q) { kv[q] = x[q]; vv[q] = y[q]; }
                } else {
#pragma unroll
                    for (int q = 0; q < 8; ++q) { kv[q] = kp[dc + q]; vv[q] = vp[dc + q]; }
                }
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) { kv[q] = 0; vv[q] = 0; }
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                Ks[kr * SKK + dc + q] = kv[q];
                Vt[(dc + q) * SVT + kr] = vv[q];
            }
        }
        __syncthreads();
        // ---- S = Q K^T for this wave's 16 rows x 64 keys ----
        f32x4 s[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            s[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                auto kf = afrag_ld<TL>(Ks + (nt * 16 + lr) * SKK + ks * 32 + lg * 8);
                s[nt] = amfma(qf[ks], kf, s[nt]);
            }
        }
        // ---- mask, online softmax ----
        float pmax[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pmax[i] = -INFINITY;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int64_t j = kb + nt * 16 + lr;
            int64_t kpos;
            if (j < L1) kpos = a.s1 + j; else kpos = a.pos2_0 + (j - L1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int qr = qw0 + lg * 4 + i;
                const int64_t qpos = a.qpos0 + qr;
                bool ok = j < kb1 && qr < a.nq;
                if (a.causal) ok = ok && kpos <= qpos && (a.window <= 0 || qpos - kpos < a.window);
                float v = ok ? s[nt][i] * scale : -INFINITY;
                s[nt][i] = v;
                pmax[i] = fmaxf(pmax[i], v);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int o2 = 1; o2 < 16; o2 <<= 1) pmax[i] = fmaxf(pmax[i], __shfl_xor(pmax[i], o2, 64));
        float alpha[4], mnew[4], psum[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mnew[i] = fmaxf(m_run[i], pmax[i]);
            alpha[i] = (m_run[i] == -INFINITY) ? 0.f : __expf(m_run[i] - mnew[i]);
            psum[i] = 0.f;
        }
        TL* pw = Ps + wave * 16 * SP;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float p = (mnew[i] == -INFINITY) ? 0.f : __expf(s[nt][i] - mnew[i]);
                TL pl;
                from_f(&pl, p);
                psum[i] += to_f(pl);  // the probabilities the MFMA sees
                pw[(lg * 4 + i) * SP + nt * 16 + lr] = pl;
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int o2 = 1; o2 < 16; o2 <<= 1) psum[i] += __shfl_xor(psum[i], o2, 64);
            l_run[i] = l_run[i] * alpha[i] + psum[i];
            m_run[i] = mnew[i];
        }
#pragma unroll
        for (int j = 0; j < NT_D; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[j][i] *= alpha[i];
        __syncthreads();  // P visible to the wave (and K/V reads done before restaging)
        // ---- O += P V ----
#pragma unroll
        for (int ks2 = 0; ks2 < KB / 32; ++ks2) {
            auto pf = afrag_ld<TL>(pw + lr * SP + ks2 * 32 + lg * 8);
#pragma unroll
            for (int j = 0; j < NT_D; ++j) {
                auto vf = afrag_ld<TL>(Vt + (j * 16 + lr) * SVT + ks2 * 32 + lg * 8);
                o[j] = amfma(pf, vf, o[j]);
            }
        }
        __syncthreads();
    }
    // ---- write out ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int qr = qw0 + lg * 4 + i;
        if (qr >= a.nq) continue;
        if (a.splits == 1) {
            const float inv = l_run[i] > 0.f ? 1.f / l_run[i] : 0.f;
            TL* out = reinterpret_cast<TL*>(a.O) + (int64_t)qr * a.Hq * HD + (int64_t)h * HD;
#pragma unroll
            for (int j = 0; j < NT_D; ++j) from_f(out + j * 16 + lr, o[j][i] * inv);
        } else {
            float* po = a.part_o + (((int64_t)blockIdx.z * a.nq + qr) * a.Hq + h) * HD;
#pragma unroll
            for (int j = 0; j < NT_D; ++j) po[j * 16 + lr] = o[j][i];
            if (lr == 0) {
                float* pm = a.part_ml + (((int64_t)blockIdx.z * a.nq + qr) * a.Hq + h) * 2;
                pm[0] = m_run[i];
                pm[1] = l_run[i];
            }
        }
    }
}

// Merge split-KV partials: O = sum_s O_s e^(m_s - M) / sum_s l_s e^(m_s - M).
template <typename TL>
__global__ void attn_merge_kernel(AttnArgs a, int hd) {
    if (a.state && a.state[0]) return;
    const int qr = blockIdx.x, h = blockIdx.y;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s)
        M = fmaxf(M, a.part_ml[(((int64_t)s * a.nq + qr) * a.Hq + h) * 2]);
    float L = 0.f;
    for (int s = 0; s < a.splits; ++s) {
        const float* pm = a.part_ml + (((int64_t)s * a.nq + qr) * a.Hq + h) * 2;
        if (pm[0] != -INFINITY) L += pm[1] * __expf(pm[0] - M);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    TL* out = reinterpret_cast<TL*>(a.O) + (int64_t)qr * a.Hq * hd + (int64_t)h * hd;
    for (int d = threadIdx.x; d < hd; d += blockDim.x) {
        float acc = 0.f;
        for (int s = 0; s < a.splits; ++s) {
            const float* pm = a.part_ml + (((int64_t)s * a.nq + qr) * a.Hq + h) * 2;
            if (pm[0] == -INFINITY) continue;
            acc += a.part_o[(((int64_t)s * a.nq + qr) * a.Hq + h) * hd + d] * __expf(pm[0] - M);
        }
        from_f(out + d, acc * inv);
    }
}

template <typename TL, int HD>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t st) {
    constexpr int PADL = 16 / sizeof(TL);
    size_t lds = ((size_t)KB * (HD + PADL) + (size_t)HD * (KB + PADL) + (size_t)4 * 16 * (KB + PADL)) * sizeof(TL);
    auto kern = attention_kernel<TL, HD>;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    dim3 grid((a.nq + 63) / 64, a.Hq, a.splits);
    kern<<<grid, 256, lds, st>>>(a);
    if (a.splits > 1) attn_merge_kernel<TL><<<dim3(a.nq, a.Hq), 256, 0, st>>>(a, HD);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int act_f32, hipStream_t st) {
    if (act_f32) {
        if (a.hd == 64) return launch_attn_t<float, 64>(a, st);
        if (a.hd == 128) return launch_attn_t<float, 128>(a, st);
        return hipErrorInvalidValue;
    }
    if (a.hd == 64) return launch_attn_t<uint16_t, 64>(a, st);
    if (a.hd == 128) return launch_attn_t<uint16_t, 128>(a, st);
    if (a.hd == 256) return launch_attn_t<uint16_t, 256>(a, st);
    return hipErrorInvalidValue;
}

size_t attention_partial_floats(int splits, int nq, int Hq, int hd) {
    return (size_t)splits * nq * Hq * (hd + 2);
}

}  // namespace dg
