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
// Flash-style, split-KV: a workgroup owns a set of query rows and a slice of
// the 64-key blocks; each wave owns 16 query rows, S = Q K^T and O += P V run
// on MFMA, the softmax is online in f32, P goes through LDS to become an A
// operand, and split slices write unnormalised partials (O, max, sum) that a
// merge kernel combines. V is stored transposed ([d][key]) so that the B
// operand of P V reads contiguous keys.
//
// bf16 (attn_t_kernel): the query heads of one KV group share every K/V
// tile, scores are formed transposed and P stays in registers (below).
#include "common.hpp"
#include "layer.hpp"

// build-time tunables: waves per attention workgroup (8: one 16-row tile each;
// 4: two tiles each) and the fewest 64-key blocks a KV split should hold
#ifndef DG_ATTN_WAVES
#define DG_ATTN_WAVES 8
#endif
#ifndef DG_ATTN_MIN_BLOCKS
#define DG_ATTN_MIN_BLOCKS 3
#endif
// workgroups the KV splits aim for (one per CU; 512 and 1024 measured slower
// on the decode step, the long-context decode and the long prefill)
#ifndef DG_ATTN_TARGET_WGS
#define DG_ATTN_TARGET_WGS 256
#endif
// 1: the transposed kernel keeps each wave's Q fragments in registers
#ifndef DG_ATTN_QREG
#define DG_ATTN_QREG 1
#endif

namespace dg {

// Split-KV partial outputs of the bf16 kernels are stored as bf16 (half the
// bytes written by the splits and read by the merge; the merge sums them in
// f32); f32 models keep f32 partials.
#ifndef DG_ATTN_PART_BF16
#define DG_ATTN_PART_BF16 1
#endif
template <typename TL>
constexpr bool part_bf16() { return DG_ATTN_PART_BF16 && sizeof(TL) == 2; }
template <typename TL>
__device__ __forceinline__ void store_part(float* base, int64_t idx, float v) {
    if constexpr (part_bf16<TL>()) reinterpret_cast<uint16_t*>(base)[idx] = f2bf(v);
    else base[idx] = v;
}

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

// Max / sum over the 16 lanes of a DPP row (the 16 keys of an S tile column
// group): swap neighbours, swap pairs, mirror halves of 8, mirror the row.
// Each step combines two partial results commutatively, so all 16 lanes end
// with bit-identical totals.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    return v;
}

// Online-softmax update of one wave's 16 rows from its S tile (4 n-tiles of
// 16 keys, already masked and scaled); writes P (storage type) to pw
// ([16][SP]) and rescales O. The reference max m_run of a row moves only when
// the block's max exceeds it by more than SM_SLACK (then, wave-uniformly,
// every row takes its exact new max and O, l are rescaled); otherwise the
// probabilities are exp(s - m_run) <= e^SM_SLACK. The normalisation O / l and
// the split merge use the same reference, so the result is unchanged up to
// rounding while most blocks skip the rescale of O.
constexpr float SM_SLACK = 8.f;
template <typename TL, int NT_D, int SP>
__device__ __forceinline__ void softmax_block(f32x4 (&s)[4], float (&m_run)[4], float (&l_run)[4],
                                              f32x4 (&o)[NT_D], TL* pw, int lr, int lg) {
    float pmax[4];
    bool grow = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pmax[i] = row16_max(fmaxf(fmaxf(s[0][i], s[1][i]), fmaxf(s[2][i], s[3][i])));
        grow |= pmax[i] > m_run[i] + SM_SLACK;
    }
    if (__ballot(grow)) {  // wave-uniform
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mnew = fmaxf(m_run[i], pmax[i]);
            alpha[i] = (m_run[i] == -INFINITY) ? 0.f : __expf(m_run[i] - mnew);
            m_run[i] = mnew;
            l_run[i] *= alpha[i];
        }
#pragma unroll
        for (int j = 0; j < NT_D; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[j][i] *= alpha[i];
    }
    float psum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = (m_run[i] == -INFINITY) ? 0.f : __expf(s[nt][i] - m_run[i]);
            TL pl;
            from_f(&pl, p);
            psum[i] += to_f(pl);  // the probabilities the MFMA sees
            pw[(lg * 4 + i) * SP + nt * 16 + lr] = pl;
        }
#pragma unroll
    for (int i = 0; i < 4; ++i) l_run[i] += row16_sum(psum[i]);
}

// ===========================================================================
// Generic kernel (f32, and any head_dim): one query head per workgroup,
// staging through registers.
// ===========================================================================
template <typename TL, int HD>
__global__ void __launch_bounds__(256) attention_kernel(AttnArgs a) {
    if (a.state && a.state[0]) return;
    constexpr int PADL = 16 / sizeof(TL);
    constexpr int SKK = HD + PADL;       // K tile row stride
    constexpr int SVT = KB + PADL;       // V^T row stride
    constexpr int SP = KB + PADL;        // P row stride
    constexpr int NT_D = HD / 16;
    constexpr int KS = HD / 32;
    extern __shared__ __align__(16) unsigned char smem[];
    TL* Ks = reinterpret_cast<TL*>(smem);
    TL* Vt = Ks + KB * SKK;
    TL* Ps = Vt + HD * SVT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int h = blockIdx.y;
    const int g = h / (a.Hq / a.Hkv);
    const int q0 = blockIdx.x * 64;
    const int qw0 = q0 + wave * 16;

    const int64_t L1 = a.e1 - a.s1;
    const int64_t Ltot = L1 + a.n2;
    int64_t kbeg = 0, kend = Ltot;
    if (a.causal) {
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
    const TL* V1 = reinterpret_cast<const TL*>(a.V1) + (int64_t)g * HD * a.ld1;
    const TL* K2 = a.K2 ? reinterpret_cast<const TL*>(a.K2) + (int64_t)g * a.ld2 * HD : nullptr;
    const TL* V2 = a.V2 ? reinterpret_cast<const TL*>(a.V2) + (int64_t)g * HD * a.ld2 : nullptr;

    for (int64_t kb = kb0; kb < kb1; kb += KB) {
        for (int c = tid; c < KB * HD / 8; c += 256) {   // K rows, 8 elements per chunk
            const int kr = c / (HD / 8), dc = (c % (HD / 8)) * 8;
            const int64_t j = kb + kr;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                TL kv = 0;
                if (j < kb1) kv = j < L1 ? K1[(a.s1 + j) * HD + dc + q] : K2[(j - L1) * HD + dc + q];
                Ks[kr * SKK + dc + q] = kv;
            }
        }
        for (int c = tid; c < KB * HD; c += 256) {       // V^T: consecutive threads take consecutive keys
            const int d = c / KB, kr = c % KB;
            const int64_t j = kb + kr;
            TL vv = 0;
            if (j < kb1) vv = j < L1 ? V1[(int64_t)d * a.ld1 + a.s1 + j] : V2[(int64_t)d * a.ld2 + (j - L1)];
            Vt[d * SVT + kr] = vv;
        }
        __syncthreads();
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
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int64_t j = kb + nt * 16 + lr;
            const int64_t kpos = j < L1 ? a.s1 + j : a.pos2_0 + (j - L1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int qr = qw0 + lg * 4 + i;
                const int64_t qpos = a.qpos0 + qr;
                bool ok = j < kb1 && qr < a.nq;
                if (a.causal) ok = ok && kpos <= qpos && (a.window <= 0 || qpos - kpos < a.window);
                s[nt][i] = ok ? s[nt][i] * scale : -INFINITY;
            }
        }
        TL* pw = Ps + wave * 16 * SP;
        softmax_block<TL, NT_D, SP>(s, m_run, l_run, o, pw, lr, lg);
        __syncthreads();
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
            const int64_t po = (((int64_t)blockIdx.z * a.nq + qr) * a.Hq + h) * HD;
#pragma unroll
            for (int j = 0; j < NT_D; ++j) store_part<TL>(a.part_o, po + j * 16 + lr, o[j][i]);
            if (lr == 0) {
                float* pm = a.part_ml + (((int64_t)blockIdx.z * a.nq + qr) * a.Hq + h) * 2;
                pm[0] = m_run[i];
                pm[1] = l_run[i];
            }
        }
    }
}

// ===========================================================================
// bf16 kernel: register-staged K/V blocks shared by the query heads of a KV
// group.
// ===========================================================================
namespace {

// K tile rows are HD*2 bytes (>= 256): chunk c of key row r sits at c ^ (r & 15).
__device__ __forceinline__ int kswz(int r, int c) { return c ^ (r & 15); }
// V^T tile rows are 128 bytes (64 keys): chunk c of row d sits at c ^ ((d >> 1) & 7).
__device__ __forceinline__ int vswz(int d, int c) { return c ^ ((d >> 1) & 7); }

}  // namespace

// every wave's LDS writes done and visible, without waiting for the global
// loads in flight (a __syncthreads would also wait for those)
__device__ __forceinline__ void attn_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup id -> (query tile qt, KV group g, split sp). The query tiles of
// one (group, split) read the same K/V blocks, so they get ids 8 apart: with
// workgroups dealt to the 8 XCDs in id order they share one XCD's L2 instead
// of fetching the blocks once per XCD.
__device__ __forceinline__ void attn_ids(int nqt, int& qt, int& gs) {
    const int id = blockIdx.x;
    const int lane8 = id % 8, rest = id / 8;      // rest = (gs / 8) * nqt + qt
    qt = rest % nqt;
    gs = (rest / nqt) * 8 + lane8;                // (group, split) pair; past the last: no work
}

// bf16 kernel with transposed scores. A workgroup's 128 query rows are the
// 128/R positions of all R query heads of one KV group, so every K/V tile is
// shared by the whole group; the K tile [64 keys][hd] and V^T tile [hd][64
// keys] of the next block are loaded into registers while the current block
// is computed and written into the XOR-swizzled LDS slot after it. Key blocks
// are aligned to multiples of 64 in each segment; keys outside the visible
// range are masked in the scores, and V^T values of keys at or past the end
// of a segment are read as zero, so whatever the buffers hold there cannot
// reach the output. S is formed as K Q^T: a lane then holds, for query row lr of its wave's tile,
// 16 scores of keys nt*16 + 4*lg + q (nt, q < 4). That layout is already the
// A operand of the P V product if the keys of each 32-key k-step are taken in
// the order (first run: 32*ks2 + 4*lg + q, second: 32*ks2 + 16 + 4*lg + q),
// so P stays in registers; the V^T tile is stored into LDS in that key order
// (two 8-byte halves per 16-byte chunk). Row max and sum are 16 in-lane
// values plus two cross-lane steps. Scores are kept unscaled; the softmax
// runs in base 2 with the 1/sqrt(hd) scale folded into the exponent, and the
// partial maxima leave in natural-log units for the merge.
template <int HD, int NW>
__global__ void __launch_bounds__(NW * 64) attn_t_kernel(AttnArgs a, int R) {
    if (a.state && a.state[0]) return;
    const int QP = 128 / R;                       // positions per workgroup
    const int nqt = (a.nq + QP - 1) / QP;
    int qt, gs;
    attn_ids(nqt, qt, gs);
    if (gs >= a.Hkv * a.splits) return;
    const int g = gs % a.Hkv, sp = gs / a.Hkv;
    constexpr int KROWB = HD * 2;                 // bytes per K row
    constexpr int K_BYTES = KB * KROWB;           // K tile
    constexpr int V_BYTES = HD * KB * 2;          // V^T tile (rows of 128 bytes)
    constexpr int STAGE = K_BYTES + V_BYTES;
    constexpr int K_LD = K_BYTES / 1024 / NW;     // 16-byte loads per lane and block
    constexpr int V_LD = V_BYTES / 1024 / NW;
    constexpr int TPW = 128 / (16 * NW);          // 16-row tiles per wave
    constexpr int RPW = 16 * TPW;                 // rows per wave
    constexpr int KRPI = 1024 / KROWB;            // K rows per 1 KB piece
    constexpr int KCPR = KROWB / 16;              // chunks per K row
    constexpr int NT_D = HD / 16;
    constexpr int KS = HD / 32;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* Qs = smem + STAGE;             // [128 rows][HD], swizzled

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int qx0 = qt * QP;
    auto row_head = [&](int rho) { return g * R + rho / QP; };
    auto row_pos = [&](int rho) { return qx0 + rho % QP; };

    // ---- the key blocks of this workgroup ----
    const int64_t qlo = a.qpos0 + qx0, qhi = a.qpos0 + min(qx0 + QP, a.nq) - 1;
    int64_t b1lo, b1hi;                           // segment-1 blocks [b1lo, b1hi)
    if (a.causal) {
        int64_t kmin = a.s1, kmax = min<int64_t>(a.e1 - 1, qhi);
        if (a.window > 0) kmin = max<int64_t>(kmin, qlo - a.window + 1);
        b1lo = kmin / KB;
        b1hi = kmax >= kmin ? kmax / KB + 1 : b1lo;
    } else {
        b1lo = a.s1 / KB;
        b1hi = a.e1 > a.s1 ? (a.e1 - 1) / KB + 1 : b1lo;
    }
    const int64_t nb1 = b1hi - b1lo;
    const int64_t nb2 = a.n2 > 0 ? (a.n2 + KB - 1) / KB : 0;
    const int64_t nb = nb1 + nb2;
    const int64_t per = (nb + a.splits - 1) / a.splits;
    const int64_t bb0 = per * sp, bb1 = min<int64_t>(nb, bb0 + per);

    const uint16_t* K1 = reinterpret_cast<const uint16_t*>(a.K1) + (int64_t)g * a.ld1 * HD;
    const uint16_t* V1 = reinterpret_cast<const uint16_t*>(a.V1) + (int64_t)g * HD * a.ld1;
    const uint16_t* K2 = a.K2 ? reinterpret_cast<const uint16_t*>(a.K2) + (int64_t)g * a.ld2 * HD : nullptr;
    const uint16_t* V2 = a.V2 ? reinterpret_cast<const uint16_t*>(a.V2) + (int64_t)g * HD * a.ld2 : nullptr;

    // register loads of virtual block vb (clamped to this workgroup's last
    // block, so the loop stays branch-free): K rows with the LDS swizzle
    // applied on the read side; V^T rows as plain 16-byte chunks of 8 keys
    u32x4 kr[K_LD], vr[V_LD];
    auto load = [&](int64_t vb) {
        vb = min<int64_t>(vb, bb1 - 1);
        const bool seg1 = vb < nb1;
        const int64_t row0 = seg1 ? (b1lo + vb) * KB : (vb - nb1) * KB;
        const int64_t rlim = seg1 ? a.e1 : a.n2;   // rows >= rlim: any valid row (masked)
        const uint16_t* Kb = seg1 ? K1 : K2;
        const uint16_t* Vb = seg1 ? V1 : V2;
        const int64_t vld = seg1 ? a.ld1 : a.ld2;
#pragma unroll
        for (int j = 0; j < K_LD; ++j) {
            const int r = (wave * K_LD + j) * KRPI + lane / KCPR;
            const int pos = lane % KCPR;
            int64_t kr_row = row0 + r;
            if (kr_row >= rlim) kr_row = rlim - 1;
            if (kr_row < 0) kr_row = 0;
            kr[j] = *reinterpret_cast<const u32x4*>(Kb + kr_row * HD + 8 * kswz(r, pos));
        }
        const int64_t vk0 = row0 + 8 * (lane % 8);  // first of this lane's 8 keys
#pragma unroll
        for (int j = 0; j < V_LD; ++j) {
            const int d = (wave * V_LD + j) * 8 + lane / 8;
            vr[j] = *reinterpret_cast<const u32x4*>(Vb + (int64_t)d * vld + vk0);
            if (vk0 + 8 > rlim) {  // keys at or past the segment's end read as zero
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (vk0 + e >= rlim) vr[j][e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            }
        }
    };
    // V^T row d: 16-byte slot L = 4*ks2 + l4 holds keys 32*ks2 + 4*l4 + (0..3)
    // then 32*ks2 + 16 + 4*l4 + (0..3), at position vswz(d, L). Chunk c = 4*ks2
    // + m of 8 keys gives its half h to slot 4*ks2 + 2*(m % 2) + h, byte
    // offset 8*(m / 2).
    auto store = [&]() {
        unsigned char* base = smem;
#pragma unroll
        for (int j = 0; j < K_LD; ++j) *reinterpret_cast<u32x4*>(base + (wave * K_LD + j) * 1024 + lane * 16) = kr[j];
#pragma unroll
        for (int j = 0; j < V_LD; ++j) {
            const int d = (wave * V_LD + j) * 8 + lane / 8;
            const int c = lane % 8, ks2 = c / 4, m = c % 4;
            unsigned char* row = base + K_BYTES + d * 128 + 8 * (m / 2);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int L = 4 * ks2 + 2 * (m % 2) + h;
                *reinterpret_cast<u32x2*>(row + vswz(d, L) * 16) = u32x2{vr[j][2 * h], vr[j][2 * h + 1]};
            }
        }
    };

    // ---- Q rows of the workgroup into LDS (row rho, 16-byte chunk c at kswz):
    // all loads first (rows past nq read row 0 and are zeroed), then the writes
    {
        constexpr int QL = 128 * KCPR / (NW * 64);  // 16-byte pieces per thread
        u16x8 qv[QL];
#pragma unroll
        for (int j = 0; j < QL; ++j) {
            const int e = tid + NW * 64 * j, rho = e / KCPR, c = e % KCPR;
            const int qp = row_pos(rho);
            qv[j] = *reinterpret_cast<const u16x8*>(reinterpret_cast<const uint16_t*>(a.Q) +
                                                    ((int64_t)row_head(rho) * a.ldq + (qp < a.nq ? qp : 0)) * HD +
                                                    c * 8);
        }
#pragma unroll
        for (int j = 0; j < QL; ++j) {
            const int e = tid + NW * 64 * j, rho = e / KCPR, c = e % KCPR;
            const u16x8 z = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
            *reinterpret_cast<u16x8*>(Qs + rho * KROWB + kswz(rho, c) * 16) = row_pos(rho) < a.nq ? qv[j] : z;
        }
    }
    f32x4 o[TPW][NT_D];
    float m_run[TPW], l_run[TPW];  // row lr of tile t, base-2 units (scaled)
    int qpos[TPW];                 // absolute position of row lr (< 2^31)
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
        for (int j = 0; j < NT_D; ++j) o[t][j] = f32x4{0, 0, 0, 0};
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
        qpos[t] = (int)(a.qpos0 + row_pos(wave * RPW + t * 16 + lr));
    }
    const float c2 = 1.4426950408889634f / sqrtf((float)HD);  // log2(e) / sqrt(hd)
    constexpr float SLACK2 = SM_SLACK * 1.4426950408889634f;

    if (bb0 < bb1) {
        load(bb0);
        store();
        load(bb0 + 1);
    }
    attn_lds_barrier();
#if DG_ATTN_QREG
    // the wave's Q fragments for every k-step, read from LDS once
    u16x8 qreg[KS][TPW];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int q = wave * RPW + t * 16 + lr;
            qreg[ks][t] = *reinterpret_cast<const u16x8*>(Qs + q * KROWB + kswz(q, ks * 4 + lg) * 16);
        }
#endif
    for (int64_t vb = bb0; vb < bb1; ++vb) {
        const unsigned char* Kt = smem;
        const unsigned char* Vt = Kt + K_BYTES;
        const bool seg1 = vb < nb1;
        const int64_t row0 = seg1 ? (b1lo + vb) * KB : (vb - nb1) * KB;
        // ---- S^T = K Q^T; the fragments of k-step ks + 1 are read while the
        // MFMAs of ks run ----
        f32x4 s[TPW][4];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) s[t][nt] = f32x4{0, 0, 0, 0};
        u16x8 qf[2][TPW], kf[2][4];
        auto ld_s = [&](int bsel, int ks) {
            const int c = ks * 4 + lg;
#if !DG_ATTN_QREG
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int q = wave * RPW + t * 16 + lr;
                qf[bsel][t] = *reinterpret_cast<const u16x8*>(Qs + q * KROWB + kswz(q, c) * 16);
            }
#endif
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int r = nt * 16 + lr;
                kf[bsel][nt] = *reinterpret_cast<const u16x8*>(Kt + r * KROWB + kswz(r, c) * 16);
            }
        };
        ld_s(0, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) ld_s((ks + 1) & 1, ks + 1);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
#if DG_ATTN_QREG
                    s[t][nt] = amfma(kf[ks & 1][nt], qreg[ks][t], s[t][nt]);
#else
                    s[t][nt] = amfma(kf[ks & 1][nt], qf[ks & 1][t], s[t][nt]);
#endif
                }
        }
        // ---- mask: only blocks that reach past the visible keys, or causal ----
        const bool full = !a.causal && (seg1 ? (row0 >= a.s1) & (row0 + KB <= a.e1) : (row0 + KB <= a.n2));
        if (!full) {  // uniform
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int key = (int)(row0 + nt * 16 + 4 * lg + q);
                    const bool kin = seg1 ? (key >= (int)a.s1) & (key < (int)a.e1) : (key < a.n2);
                    const int kp = seg1 ? key : (int)a.pos2_0 + key;
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        bool ok = kin;
                        if (a.causal) {
                            const int dq = qpos[t] - kp;
                            ok = ok & (dq >= 0) & ((a.window <= 0) | (dq < a.window));
                        }
                        if (!ok) s[t][nt][q] = -INFINITY;
                    }
                }
        }
        // ---- online softmax (base 2), P into registers as the A operand ----
        u16x8 pf[TPW][2];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            float mx = fmaxf(fmaxf(fmaxf(s[t][0][0], s[t][0][1]), fmaxf(s[t][0][2], s[t][0][3])),
                             fmaxf(fmaxf(s[t][1][0], s[t][1][1]), fmaxf(s[t][1][2], s[t][1][3])));
            mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[t][2][0], s[t][2][1]), fmaxf(s[t][2][2], s[t][2][3])),
                                 fmaxf(fmaxf(s[t][3][0], s[t][3][1]), fmaxf(s[t][3][2], s[t][3][3]))));
            mx = xor32_max(xor16_max(mx));
            const float pm = mx * c2;  // the row's block max, base-2 units
            if (__ballot(pm > m_run[t] + SLACK2)) {  // wave-uniform
                const float mnew = fmaxf(m_run[t], pm);
                const float alpha = m_run[t] == -INFINITY ? 0.f : exp2f(m_run[t] - mnew);
                m_run[t] = mnew;
                l_run[t] *= alpha;
                // O rows 4*lg + i: their factors sit in lanes 4*lg + i
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, 4 * lg + i, WAVE);
#pragma unroll
                    for (int j = 0; j < NT_D; ++j) o[t][j][i] *= ai;
                }
            }
            const float mr = m_run[t];
            const bool live = mr != -INFINITY;
            float psum = 0.f;
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
                u32x4 w;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {  // first / second run of 4 keys: n-tile 2*ks2 + hh
                    const f32x4 sv = s[t][2 * ks2 + hh];
                    float pv[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) pv[q] = live ? exp2f(fmaf(sv[q], c2, -mr)) : 0.f;
                    const uint32_t w0 = f2bf2(pv[0], pv[1]), w1 = f2bf2(pv[2], pv[3]);
                    w[2 * hh] = w0;
                    w[2 * hh + 1] = w1;
                    // the probabilities the MFMA sees
                    psum += (__uint_as_float(w0 << 16) + __uint_as_float(w0 & 0xffff0000u)) +
                            (__uint_as_float(w1 << 16) + __uint_as_float(w1 & 0xffff0000u));
                }
                pf[t][ks2] = __builtin_bit_cast(u16x8, w);
            }
            psum = xor32_sum(xor16_sum(psum));
            l_run[t] += psum;
        }
        // ---- O += P V: V^T fragments in groups of 4, the next group read
        // during the current MFMAs ----
#pragma unroll
        for (int ks2 = 0; ks2 < KB / 32; ++ks2) {
            u16x8 vf[2][4];
            auto ld_v = [&](int bsel, int jg) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int d = (jg * 4 + jj) * 16 + lr;
                    vf[bsel][jj] = *reinterpret_cast<const u16x8*>(Vt + d * 128 + vswz(d, ks2 * 4 + lg) * 16);
                }
            };
            ld_v(0, 0);
#pragma unroll
            for (int jg = 0; jg < NT_D / 4; ++jg) {
                if (jg + 1 < NT_D / 4) ld_v((jg + 1) & 1, jg + 1);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int t = 0; t < TPW; ++t)
                        o[t][jg * 4 + jj] = amfma(pf[t][ks2], vf[jg & 1][jj], o[t][jg * 4 + jj]);
            }
        }
        __builtin_amdgcn_s_barrier();  // every wave done with the slot
        store();
        load(vb + 2);
        attn_lds_barrier();
    }
    __syncthreads();  // retire the tail loads
    // ---- write out: O row 4*lg + i takes its (m, l) from lane 4*lg + i ----
    constexpr float LN2 = 0.6931471805599453f;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float li = __shfl(l_run[t], 4 * lg + i, WAVE);
            const float mi = __shfl(m_run[t], 4 * lg + i, WAVE);
            const int rho = wave * RPW + t * 16 + lg * 4 + i;
            if (row_pos(rho) >= a.nq) continue;
            const int hq = row_head(rho), qr = row_pos(rho);
            if (a.splits == 1) {
                const float inv = li > 0.f ? 1.f / li : 0.f;
                uint16_t* out = reinterpret_cast<uint16_t*>(a.O) + (int64_t)qr * a.Hq * HD + (int64_t)hq * HD;
#pragma unroll
                for (int j = 0; j < NT_D; ++j) out[j * 16 + lr] = f2bf(o[t][j][i] * inv);
            } else {
                const int64_t po = (((int64_t)sp * a.nq + qr) * a.Hq + hq) * HD;
#pragma unroll
                for (int j = 0; j < NT_D; ++j) store_part<uint16_t>(a.part_o, po + j * 16 + lr, o[t][j][i]);
                if (lr == 0) {
                    float* pm = a.part_ml + (((int64_t)sp * a.nq + qr) * a.Hq + hq) * 2;
                    pm[0] = mi * LN2;  // natural-log units, as the merge expects
                    pm[1] = li;
                }
            }
        }
    }
}

// Merge split-KV partials: O = sum_s O_s e^(m_s - M) / sum_s l_s e^(m_s - M).
// One wave per (query row, head); a lane owns 4 consecutive dims. Every
// split's (m, l) and partial loads are issued before the sums, which run in
// split order.
constexpr int MERGE_MAX_SPLITS = 16;
template <typename TL>
__global__ void __launch_bounds__(256) attn_merge_kernel(AttnArgs a, int hd) {
    if (a.state && a.state[0]) return;
    const int pair = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (pair >= a.nq * a.Hq) return;
    const int qr = pair / a.Hq, h = pair % a.Hq;
    const int64_t rs = (int64_t)a.nq * a.Hq;  // (row, head) pairs per split
    constexpr int MS = MERGE_MAX_SPLITS;
    const int c = lane * 4;                   // hd <= 256: one 4-dim chunk per lane
    const bool has = c < hd;
    // all loads first: every split's (m, l) and partial chunk (a split with no
    // keys left zeros there; it gets weight 0 and is skipped in the sum)
    float2 ml[MS];
    float4 po[MS];
#pragma unroll
    for (int s = 0; s < MS; ++s) {
        if (s < a.splits) {
            ml[s] = *reinterpret_cast<const float2*>(a.part_ml + (s * rs + pair) * 2);
            if (has) {
                if constexpr (part_bf16<TL>()) {
                    const uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.part_o) +
                                                                     (s * rs + pair) * hd + c);
                    po[s] = make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
                                        __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u));
                } else {
                    po[s] = *reinterpret_cast<const float4*>(a.part_o + (s * rs + pair) * hd + c);
                }
            }
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < MS; ++s)
        if (s < a.splits) M = fmaxf(M, ml[s].x);
    float L = 0.f, wgt[MS];
#pragma unroll
    for (int s = 0; s < MS; ++s) {
        wgt[s] = 0.f;
        if (s < a.splits && ml[s].x != -INFINITY) {
            wgt[s] = __expf(ml[s].x - M);
            L += ml[s].y * wgt[s];
        }
    }
    if (!has) return;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < MS; ++s) {
        if (s < a.splits && ml[s].x != -INFINITY) {
            acc.x += po[s].x * wgt[s];
            acc.y += po[s].y * wgt[s];
            acc.z += po[s].z * wgt[s];
            acc.w += po[s].w * wgt[s];
        }
    }
    TL* out = reinterpret_cast<TL*>(a.O) + (int64_t)qr * a.Hq * hd + (int64_t)h * hd;
    from_f(out + c, acc.x * inv);
    from_f(out + c + 1, acc.y * inv);
    from_f(out + c + 2, acc.z * inv);
    from_f(out + c + 3, acc.w * inv);
}

static void launch_merge_any(const AttnArgs& a, bool bf16, hipStream_t st) {
    const unsigned grid = (unsigned)(((int64_t)a.nq * a.Hq + 3) / 4);
    if (bf16) attn_merge_kernel<uint16_t><<<grid, 256, 0, st>>>(a, a.hd);
    else attn_merge_kernel<float><<<grid, 256, 0, st>>>(a, a.hd);
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
    if (a.splits > 1) launch_merge_any(a, sizeof(TL) == 2, st);
    return hipGetLastError();
}

template <int HD>
static hipError_t launch_attn_grouped(const AttnArgs& a, hipStream_t st) {
    constexpr int NW = DG_ATTN_WAVES;
    const int R = a.Hq / a.Hkv;
    constexpr int STAGE = 64 * HD * 2 * 2;
    const size_t lds = (size_t)STAGE + (size_t)128 * HD * 2;
    auto kern = attn_t_kernel<HD, NW>;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int nqt = (a.nq + 128 / R - 1) / (128 / R), ngs = a.Hkv * a.splits;
    const unsigned grid = (unsigned)(((ngs + 7) / 8) * nqt * 8);  // see attn_ids
    kern<<<grid, NW * 64, lds, st>>>(a, R);
    if (a.splits > 1) launch_merge_any(a, true, st);
    return hipGetLastError();
}

bool attention_uses_grouped(int Hq, int Hkv, int hd, int act_f32) {
    const int R = Hq / Hkv;
    return !act_f32 && (hd == 128 || hd == 256) && R >= 1 && R <= 64 && 128 % R == 0;
}

int attention_splits(int nq, int64_t keys, int Hq, int Hkv, int hd, int act_f32, int max_splits, int max_rows) {
    int s;
    if (attention_uses_grouped(Hq, Hkv, hd, act_f32)) {
        // about one workgroup per CU, each with at least DG_ATTN_MIN_BLOCKS key blocks
        const int64_t wgs = (int64_t)((nq + 128 / (Hq / Hkv) - 1) / (128 / (Hq / Hkv))) * Hkv;
        const int64_t blocks = (keys + KB - 1) / KB + 1;
        s = (int)std::min<int64_t>((DG_ATTN_TARGET_WGS + wgs - 1) / wgs,
                                   std::max<int64_t>(1, blocks / DG_ATTN_MIN_BLOCKS));
    } else {
        const int qtiles = (nq + 63) / 64;
        s = (int)std::min<int64_t>(max_splits, std::max<int64_t>(1, (keys + 511) / 512));
        while (s > 1 && qtiles * Hq * (s / 2) >= 512) s /= 2;
    }
    s = std::max(1, std::min(s, max_splits));
    while (s > 1 && (int64_t)s * nq > (int64_t)max_rows) --s;
    return s;
}

hipError_t launch_attention(const AttnArgs& a, int act_f32, hipStream_t st) {
    if (a.splits > MERGE_MAX_SPLITS || a.hd % 4 || a.hd > 256) return hipErrorInvalidValue;
    if (attention_uses_grouped(a.Hq, a.Hkv, a.hd, act_f32) && a.ld1 % 64 == 0 && (a.n2 == 0 || a.ld2 % 64 == 0)) {
        if (a.hd == 256) return launch_attn_grouped<256>(a, st);
        return launch_attn_grouped<128>(a, st);
    }
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
