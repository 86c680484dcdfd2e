// Entropy-Bounded sampler kernels for gfx950.
//
// DiffusionGemma model card (zh-TW), best practice 1 "diffusion sampling
// settings" (and recommendation 1 of the Korean card): at most 48 steps; a
// temperature falling linearly from 0.8 to 0.4 that shapes the logits; the
// lowest-entropy tokens are committed while their summed entropy stays within
// the bound 0.1; unselected tokens are re-noised; sampling stops early when
// the canvas-mean entropy is below 0.005 and the most probable tokens are
// unchanged over two consecutive steps.
//
// Candidates are the uncommitted positions (commits final) or, in the
// reselect-all commit mode that reads the charlie27.com digest's remark on
// self-correction, every position; then an unselected position returns to
// MASK whether or not it was committed before.
//
// Kernels (one denoising step, in launch order):
//   logit_stats   per (row, vocab split): base-2 entropy partials, raw argmax
//   merge_rows    per row: entropy (nats), log-sum-exp, argmax
//   eb_select     one workgroup: rank candidates by (entropy, position), float32
//                 running sum (a scan) in sorted order, cut at the bound (at
//                 least one)
//   draw_chunks   chip-wide: float64 sums of exp(z - M) per (selected row, chunk)
//   draw_pick     per selected row: Philox4x32-10 uniform, float64 inverse CDF
//                 in vocabulary order (chunk totals, then a scan in one chunk)
//   finalize      one workgroup: re-mask, canvas-mean entropy (float64, per
//                 wave then the wave sums in order), stop test, argmax fill at
//                 the end, state update
// Every kernel reads the step index and the done flag from device memory so a
// captured step can be replayed without host involvement.
#include "common.hpp"
#include "kernels.hpp"

namespace dg {

// ---------------------------------------------------------------------------
// Temperature at step t: tau0 + (tau1 - tau0) * t / (S - 1), in float64 with
// the operations in that order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double tau_at(const SamplerParams& sp, int t) {
    if (sp.max_steps <= 1) return (double)sp.temp_start;
    return (double)sp.temp_start +
           ((double)sp.temp_end - (double)sp.temp_start) * (double)t / (double)(sp.max_steps - 1);
}

// one logit of a row, widened to f32
template <typename T> struct Raw8Elem;
template <> struct Raw8Elem<uint16_t> {
    static __device__ __forceinline__ float get(const uint16_t* p, int i) { return bf2f(p[i]); }
};
template <> struct Raw8Elem<float> {
    static __device__ __forceinline__ float get(const float* p, int i) { return p[i]; }
};

// Values at or below STATS_EXCLUDED take no part in the statistics (as -inf
// would): the statistics pass writes it over MASK, over the bias token (whose
// biased value joins the row once, after the loop) and over columns past the
// end of a split, so the reduction over a chunk needs no per-column test.
// Logits at or below -2^64 are thereby treated as -inf. The value stays
// finite when tempered (|2^64 * log2(e) / tau| < 2^128 for tau > 2^-63), so
// its 2^(z2 - m2) is 0 and its entropy term 0 * (z2 - m2) is 0, not NaN.
constexpr float STATS_EXCLUDED = -0x1p64f;
constexpr uint16_t STATS_EXCLUDED_BF16 = 0xDF80;  // -2^64

// 8 consecutive logits as loaded (bf16: one 16-byte vector; f32: two),
// widened to f32 only when used, so a load in flight does not stall the code
// that issues the next ones.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
    u16x8 v;
    __device__ __forceinline__ void load(const uint16_t* p) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(p));
    }
    __device__ __forceinline__ void fill_excluded() { v = STATS_EXCLUDED_BF16; }
    // element q (0..7, may differ per lane) becomes STATS_EXCLUDED
    __device__ __forceinline__ void exclude(int q) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k == q) v[k] = STATS_EXCLUDED_BF16;
    }
    __device__ __forceinline__ float at(int j) const { return bf2f(v[j]); }
    // makes the compiler treat the vector as rewritten, so values widened
    // from it before this point are recomputed after it, not kept live
    __device__ __forceinline__ void refresh() { asm volatile("" : "+v"(v)); }
};
template <> struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
    }
    __device__ __forceinline__ void fill_excluded() { a = STATS_EXCLUDED; b = STATS_EXCLUDED; }
    __device__ __forceinline__ void exclude(int q) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (k == q) a[k] = STATS_EXCLUDED;
            if (k + 4 == q) b[k] = STATS_EXCLUDED;
        }
    }
    __device__ __forceinline__ float at(int j) const { return j < 4 ? a[j] : b[j - 4]; }
    __device__ __forceinline__ void refresh() {}
};

// ---------------------------------------------------------------------------
// Row statistics over given logits (the sampler-only entry point). Grid
// (nsplit, n), 256 threads; split i covers columns [i*split_cols, ...), a
// multiple of 2048. The split is read in chunks of 16384 columns (256 threads
// x 8 vectors x 8): a thread holds its 8 vectors of one chunk and already has
// the next chunk's loads in flight while it reduces the current one, and the
// kernel is held to 128 VGPRs so that four workgroups (and their loads) share
// a CU. Per chunk, one pass over the values:
//   sums    s = sum 2^d, t = sum 2^d d with d = x*c2 - r (one fma) against the
//           lane's running reference r (its first chunk's tempered max; any
//           reference gives the same entropy and log-sum-exp, and values below
//           it by more than 126 are negligible next to the value at r), 2^d
//           by the hardware exp; a chunk whose max lies more than 64 above r
//           is summed again against that max, so 2^d never overflows;
//   max     the lane's max of the raw values alongside (tempering by c2 > 0
//           keeps the order);
//   argmax  only when the wave's max beats the running one (wave-uniform, a
//           few chunks per row) do the lanes holding it look for its lowest
//           column.
// The bias token's value L + bias joins the row's partial once, after the
// loop. GUMBEL: the same pass also keeps the Gumbel-max candidate of the
// split, the lowest column maximising z_v - log(-log u_v) with z =
// (L + bias) / tau and u_v from Philox at counter (row, step, canvas,
// 1 + v / 4), word v % 4.
// ---------------------------------------------------------------------------
// build-time tunable: waves per SIMD the statistics pass over bf16 logits is
// compiled for (4: at most 128 VGPRs); f32 logits hold twice the registers
// per chunk (2)
#ifndef DG_STATS_WAVES_PER_EU
#define DG_STATS_WAVES_PER_EU 4
#endif
constexpr int STATS_PER = 8;                      // vectors of 8 per thread and chunk
constexpr int STATS_CHUNK = 256 * 8 * STATS_PER;  // columns per chunk

template <typename T, bool GUMBEL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? DG_STATS_WAVES_PER_EU : 2)))
logit_stats_kernel(const T* __restrict__ logits, int64_t ld, int V, int split_cols,
                   const int32_t* __restrict__ state, int step_override, SamplerParams sp, int mask_id,
                   const int32_t* __restrict__ bias_tok, const float* __restrict__ bias_val,
                   RowPart* __restrict__ parts, int nsplit) {
    if (state && state[0]) return;
    constexpr int PER = STATS_PER;
    const int row = blockIdx.y;
    const int sp_i = blockIdx.x;
    const int t = step_override >= 0 ? step_override : state[1];
    const float c2 = (float)(1.4426950408889634 / tau_at(sp, t));  // log2(e) / tau
    const int c0 = sp_i * split_cols;
    const int c1 = min(V, c0 + split_cols);
    const T* rowp = logits + (int64_t)row * ld;
    const int btok = bias_tok ? bias_tok[row] : -1;
    const float bval = bias_tok ? bias_val[row] : 0.f;
    const int tid = threadIdx.x;

    EntPart e{-INFINITY, 0.f, 0.f};
    ArgMax am{-INFINITY, 0x7fffffff};
    ArgMax gm{-INFINITY, 0x7fffffff};
    // cur: the chunk being reduced; nxt: the next one, its loads in flight
    Raw8<T> cur[PER], nxt[PER];
    // vector j of a chunk at `base`: columns base + (j*256 + tid)*8 .. +8
    // (vocabulary and split bounds are multiples of 8). Every lane loads, a
    // vector past c1 from c1 - 8 (set to STATS_EXCLUDED when its chunk is
    // reduced): loads under a branch, even a uniform one, would make the
    // compiler wait for all loads in flight, the next chunk's included,
    // before using any
    auto fetch = [&](Raw8<T> (&r)[PER], int base) {
#pragma unroll
        for (int j = 0; j < PER; ++j) r[j].load(rowp + min(base + (j * 256 + tid) * 8, c1 - 8));
    };
    if (c0 < c1) fetch(cur, c0);
    for (int base = c0; base < c1; base += STATS_CHUNK) {
        // unconditional as well (past the last chunk every lane reads c1 - 8,
        // one line per wave, never used)
        fetch(nxt, base + STATS_CHUNK);
        // MASK, the bias token and columns past c1 leave the chunk's
        // reduction (wave-uniform tests)
        if (base + STATS_CHUNK > c1) {
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (base + (j * 256 + tid) * 8 >= c1) cur[j].fill_excluded();
        }
        const bool has_mask = mask_id >= base && mask_id < base + STATS_CHUNK;
        const bool has_bias = btok >= base && btok < base + STATS_CHUNK;
        if (has_mask || has_bias) {
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int v0 = base + (j * 256 + tid) * 8;
                if (has_mask && (unsigned)(mask_id - v0) < 8u) cur[j].exclude(mask_id - v0);
                if (has_bias && (unsigned)(btok - v0) < 8u) cur[j].exclude(btok - v0);
            }
        }
        // reference of the sums: the lane's running one; on its first chunk
        // the lane's max (a max pass of its own)
        float ref2 = e.m;
        if (!(ref2 > -INFINITY)) {
            float m0 = -INFINITY;
#pragma unroll
            for (int j = 0; j < PER; ++j)
#pragma unroll
                for (int q = 0; q < 8; ++q) m0 = fmaxf(m0, cur[j].at(q));
#pragma unroll
            for (int j = 0; j < PER; ++j) cur[j].refresh();
            ref2 = m0 > STATS_EXCLUDED ? m0 * c2 : -INFINITY;
        }
        float lm = -INFINITY, ls = 0.f, lt = 0.f;
        if (ref2 > -INFINITY) {
#pragma unroll
            for (int j = 0; j < PER; ++j)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float x = cur[j].at(q);
                    lm = fmaxf(lm, x);
                    const float d = fmaf(x, c2, -ref2);
                    const float w = __builtin_amdgcn_exp2f(d);
                    ls += w;
                    lt = fmaf(w, d, lt);
                }
#pragma unroll
            for (int j = 0; j < PER; ++j) cur[j].refresh();
            if (lm * c2 - ref2 > 64.f) {
                // a value far above the reference (2^d up to 2^128 would
                // overflow): the chunk again against its own max
                ref2 = lm * c2;
                ls = 0.f;
                lt = 0.f;
#pragma unroll
                for (int j = 0; j < PER; ++j)
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const float d = fmaf(cur[j].at(q), c2, -ref2);
                        const float w = __builtin_amdgcn_exp2f(d);
                        ls += w;
                        lt = fmaf(w, d, lt);
                    }
#pragma unroll
                for (int j = 0; j < PER; ++j) cur[j].refresh();
            }
            e = ent_merge(e, EntPart{ref2, ls, lt});
        }
        const float wm = wave_max(lm);
        if (wm > am.v && wm > STATS_EXCLUDED) {
            int li = 0x7fffffff;
            if (lm == wm) {
#pragma unroll
                for (int j = PER - 1; j >= 0; --j)
#pragma unroll
                    for (int q = 7; q >= 0; --q)
                        if (cur[j].at(q) == wm) li = base + (j * 256 + tid) * 8 + q;
            }
            am = ArgMax{wm, wave_min_i(li)};
        }
        if constexpr (GUMBEL) {
#pragma unroll
            for (int j = 0; j < PER; ++j) cur[j].refresh();
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int v0 = base + (j * 256 + tid) * 8;
                if (v0 >= c1) continue;
                u32x4 w[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    w[h] = philox10(u32x4{(uint32_t)row, (uint32_t)t, (uint32_t)sp.canvas_idx,
                                          (uint32_t)(1 + v0 / 4 + h)},
                                    sp.seed_lo, sp.seed_hi);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float xq = cur[j].at(q);
                    if (!(xq > STATS_EXCLUDED)) continue;
                    const float val = xq * c2 * 0.6931471805599453f + gumbel_of(w[q >> 2][q & 3]);
                    if (val > gm.v) { gm.v = val; gm.i = v0 + q; }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) cur[j] = nxt[j];
    }
    e = wave_ent(e);
    am = wave_argmax(am);
    if constexpr (GUMBEL) gm = wave_argmax(gm);
    __shared__ EntPart se[4];
    __shared__ ArgMax sa[4], sg[4];
    const int w = tid >> 6;
    if ((tid & 63) == 0) { se[w] = e; sa[w] = am; sg[w] = gm; }
    __syncthreads();
    if (tid == 0) {
        for (int i = 1; i < 4; ++i) {
            e = ent_merge(e, se[i]);
            am = argmax_merge(am, sa[i]);
            if constexpr (GUMBEL) gm = argmax_merge(gm, sg[i]);
        }
        // the bias token, excluded from the loop: its biased value once
        if (btok >= c0 && btok < c1 && btok != mask_id) {
            const float xb = Raw8Elem<T>::get(rowp, btok) + bval;
            if (!(xb <= STATS_EXCLUDED)) {  // NaN joins (and spoils the row, as a NaN logit does)
                e = ent_merge(e, EntPart{xb * c2, 1.f, 0.f});
                if (xb > STATS_EXCLUDED) am = argmax_merge(am, ArgMax{xb, btok});
                if constexpr (GUMBEL) {
                    const u32x4 u = philox10(u32x4{(uint32_t)row, (uint32_t)t, (uint32_t)sp.canvas_idx,
                                                   (uint32_t)(1 + btok / 4)},
                                             sp.seed_lo, sp.seed_hi);
                    const uint32_t word = (btok & 3) == 0 ? u[0] : (btok & 3) == 1 ? u[1] : (btok & 3) == 2 ? u[2] : u[3];
                    if (xb > STATS_EXCLUDED)
                        gm = argmax_merge(gm, ArgMax{xb * c2 * 0.6931471805599453f + gumbel_of(word), btok});
                }
            }
        }
        RowPart p;
        p.m2 = e.m; p.s = e.s; p.t = e.t; p.lmax = am.v; p.amax = am.i == 0x7fffffff ? -1 : am.i;
        p.pad[0] = __float_as_int(gm.v);
        p.pad[1] = gm.i == 0x7fffffff ? -1 : gm.i;
        p.pad[2] = 0;
        parts[(int64_t)row * nsplit + sp_i] = p;
    }
}

// ---------------------------------------------------------------------------
// Merge the per-split partials of each row. One workgroup of 256 threads
// per row: each thread merges every 256th partial, then the waves, then the
// wave results in order.
// H = ln2 * (log2 S - T2 / S) (clamped at 0); lse = ln2 * (M2 + log2 S).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) merge_rows_kernel(
    const RowPart* __restrict__ parts, int n, int nsplit, const int32_t* __restrict__ state,
    float* __restrict__ H, float* __restrict__ lse, int32_t* __restrict__ amax, int32_t* __restrict__ gtok) {
    if (state && state[0]) return;
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    EntPart e{-INFINITY, 0.f, 0.f};
    ArgMax am{-INFINITY, 0x7fffffff}, gm{-INFINITY, 0x7fffffff};
    const RowPart* p = parts + (int64_t)row * nsplit;
    for (int i = tid; i < nsplit; i += 256) {
        RowPart q = p[i];
        if (q.amax >= 0) {
            e = ent_merge(e, EntPart{q.m2, q.s, q.t});
            am = argmax_merge(am, ArgMax{q.lmax, q.amax});
        }
        if (gtok && q.pad[1] >= 0) gm = argmax_merge(gm, ArgMax{__int_as_float(q.pad[0]), q.pad[1]});
    }
    e = wave_ent(e);
    am = wave_argmax(am);
    if (gtok) gm = wave_argmax(gm);
    __shared__ EntPart se[4];
    __shared__ ArgMax sa[4], sg[4];
    if (lane == 0) { se[w] = e; sa[w] = am; sg[w] = gm; }
    __syncthreads();
    if (tid == 0) {
        for (int i = 1; i < 4; ++i) {
            e = ent_merge(e, se[i]);
            am = argmax_merge(am, sa[i]);
            if (gtok) gm = argmax_merge(gm, sg[i]);
        }
        const float LN2 = 0.6931471805599453f;
        float l2s = log2f(e.s);
        float h = LN2 * (l2s - e.t / e.s);
        H[row] = fmaxf(h, 0.f);
        lse[row] = LN2 * (e.m + l2s);
        amax[row] = am.i == 0x7fffffff ? 0 : am.i;  // no finite logit (NaN input): id 0
        if (gtok) gtok[row] = gm.i == 0x7fffffff ? amax[row] : gm.i;
    }
}

// ---------------------------------------------------------------------------
// EB selection in one workgroup of 1024 threads (n <= 1024). Keys are
// (entropy bits, position) as 64-bit integers: entropies are >= 0, so their
// IEEE bit patterns order like the values; with the position they are
// unique, so thread i places its key at its rank (the count of smaller keys,
// n LDS broadcasts) instead of a sorting network's log^2 n barriers.
// Non-candidates (committed rows, unless every row is re-selected) rank last.
// The running sum in sorted order is a workgroup scan in f32. Writes
// the selection mask, the selected positions in sorted order (sel_list) and
// their count (state word 4).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) eb_select_kernel(
    const float* __restrict__ H, const uint8_t* __restrict__ committed, int n,
    int32_t* __restrict__ state, SamplerParams sp, uint8_t* __restrict__ selected,
    int32_t* __restrict__ sel_list) {
    if (state && state[0]) return;
    constexpr unsigned long long NONCAND = 0xffffffff00000000ull;
    __shared__ unsigned long long key[1024], skey[1024];
    __shared__ float wsum[16];
    __shared__ int kcut, has_cand;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // keys (entropy bits, position): unique, so a key's rank is the number
    // of smaller keys; non-candidates rank after every candidate
    unsigned long long k = NONCAND | (unsigned)tid;
    if (tid < n && (sp.commit_mode != 0 || !committed[tid]))
        k = ((unsigned long long)__float_as_uint(H[tid]) << 32) | (unsigned)tid;
    if (tid < n) key[tid] = k;
    if (tid == 0) { kcut = 0x7fffffff; has_cand = 0; }
    __syncthreads();
    if (tid < n) {
        int r = 0;
        for (int j = 0; j < n; ++j) r += key[j] < k;  // one LDS broadcast per j
        skey[r] = k;
        selected[tid] = 0;
    }
    __syncthreads();
    // running f32 sum of the sorted candidate entropies (a workgroup scan);
    // mode 0 keeps position i while S_i <= bound, mode 1 while S_{i-1} <= bound
    const unsigned long long sk = tid < n ? skey[tid] : NONCAND;
    const bool cand = sk < NONCAND;
    const float h = cand ? __uint_as_float((unsigned)(sk >> 32)) : 0.f;
    float incl = h;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(incl, o, WAVE);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    float off = 0.f;
    for (int i = 0; i < w; ++i) off += wsum[i];
    incl += off;
    const float excl = incl - h;
    const bool ok = cand && (sp.bound_mode == 0 ? incl <= sp.bound : excl <= sp.bound);
    if (tid < n && !ok) atomicMin(&kcut, tid);  // the first position not kept
    if (tid == 0 && cand) has_cand = 1;
    __syncthreads();
    int kk = min(kcut, n);
    if (kk == 0 && has_cand) kk = 1;  // at least one while candidates remain
    if (tid == 0) state[4] = kk;
    if (tid < kk) {
        const int pos = (int)(sk & 0xffffffffu);
        selected[pos] = 1;
        sel_list[tid] = pos;
    }
}

// ---------------------------------------------------------------------------
// Inverse-CDF draw of the selected rows, in float64: w_v = exp(z_v - M') with
// z = (L + bias) / tau and M' = z at the row's argmax (any offset cancels in
// the comparison with u * sum w). The vocabulary is cut into chunks of
// DRAW_CHUNK columns; each of the 256 threads of a chunk owns 16 consecutive
// columns, loaded as two vectors before the first exp (one load round trip,
// not one per column).
//   draw_chunks: every (selected row, chunk) pair sums its w (chip-wide grid).
//   draw_pick:   per selected row, a workgroup scan of the chunk totals (256
//                chunks at a time, in vocabulary order) finds the chunk where
//                u * S falls, and a scan inside it the column.
// ---------------------------------------------------------------------------
constexpr int DRAW_CHUNK = 4096;

template <typename T>
__device__ __forceinline__ double zval(const T* rowp, int v, int btok, double bval, double tau) {
    float l;
    if constexpr (sizeof(T) == 2) l = bf2f(rowp[v]); else l = rowp[v];
    double L = (double)l + (v == btok ? bval : 0.0);
    return L / tau;
}

// A thread's 16 consecutive logits v0 .. v0+15 (v0 a multiple of 16, V a
// multiple of 8), loaded as whole vectors before any use; a vector at or
// past V reads the row's last one and is marked absent.
template <typename T>
__device__ __forceinline__ void load16(const T* rowp, int v0, int V, float (&x)[16], bool (&in)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int vh = v0 + 8 * h;
        in[h] = vh < V;
        const int va = in[h] ? vh : V - 8;
        if constexpr (sizeof(T) == 2) {
            const u16x8 u = *reinterpret_cast<const u16x8*>(rowp + va);
#pragma unroll
            for (int q = 0; q < 8; ++q) x[8 * h + q] = bf2f(u[q]);
        } else {
            const f32x4 a = *reinterpret_cast<const f32x4*>(rowp + va);
            const f32x4 b = *reinterpret_cast<const f32x4*>(rowp + va + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) { x[8 * h + q] = a[q]; x[8 * h + 4 + q] = b[q]; }
        }
    }
}

// w_v = exp(z_v - M) of the thread's 16 columns (0 for absent columns and
// MASK), z = (L + bias) / tau in float64
__device__ __forceinline__ void chunk_weights(const float (&x)[16], const bool (&in)[2], int v0, int mask_id,
                                              int btok, double bval, double tau, double M, double (&w)[16]) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int v = v0 + q;
        const double L = (double)x[q] + (v == btok ? bval : 0.0);
        w[q] = (in[q / 8] && v != mask_id) ? exp(L / tau - M) : 0.0;
    }
}

template <typename T>
__global__ void __launch_bounds__(256) draw_chunks_kernel(
    const T* __restrict__ logits, int64_t ld, int V, int mask_id,
    const int32_t* __restrict__ bias_tok, const float* __restrict__ bias_val,
    const int32_t* __restrict__ sel_list, const int32_t* __restrict__ amax,
    const int32_t* __restrict__ state, int step_override, SamplerParams sp, double* __restrict__ chunk_sum) {
    if (state && state[0]) return;
    const int nchunk = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
    const int k = state[4];
    const int t = step_override >= 0 ? step_override : state[1];
    const double tau = tau_at(sp, t);
    __shared__ double red[4];
    for (int item = blockIdx.x; item < k * nchunk; item += gridDim.x) {
        const int r = item / nchunk, c = item % nchunk;
        const int row = sel_list[r];
        const T* rowp = logits + (int64_t)row * ld;
        const int btok = bias_tok ? bias_tok[row] : -1;
        const double bval = bias_tok ? (double)bias_val[row] : 0.0;
        const double M = zval(rowp, amax[row], btok, bval, tau);
        const int v0 = c * DRAW_CHUNK + threadIdx.x * 16;
        float x[16];
        bool in[2];
        load16(rowp, v0, V, x, in);
        double w[16];
        chunk_weights(x, in, v0, mask_id, btok, bval, tau, M, w);
        double s = 0.0;
#pragma unroll
        for (int q = 0; q < 16; ++q) s += w[q];
        s = wave_sum_d(s);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
        __syncthreads();
        if (threadIdx.x == 0) chunk_sum[(int64_t)r * nchunk + c] = (red[0] + red[1]) + (red[2] + red[3]);
        __syncthreads();
    }
}

template <typename T>
__global__ void __launch_bounds__(256) draw_pick_kernel(
    const T* __restrict__ logits, int64_t ld, int V, int mask_id,
    const int32_t* __restrict__ bias_tok, const float* __restrict__ bias_val,
    const int32_t* __restrict__ sel_list, const int32_t* __restrict__ amax,
    const int32_t* __restrict__ state, int step_override, SamplerParams sp,
    uint32_t seed_lo, uint32_t seed_hi, int canvas_idx, const double* __restrict__ chunk_sum,
    int32_t* __restrict__ tokens, uint8_t* __restrict__ committed) {
    if (state && state[0]) return;
    const int r = blockIdx.x;
    if (r >= state[4]) return;
    const int nchunk = (V + DRAW_CHUNK - 1) / DRAW_CHUNK;
    const int t = step_override >= 0 ? step_override : state[1];
    const double tau = tau_at(sp, t);
    const int row = sel_list[r];
    const T* rowp = logits + (int64_t)row * ld;
    const int btok = bias_tok ? bias_tok[row] : -1;
    const double bval = bias_tok ? (double)bias_val[row] : 0.0;
    const double M = zval(rowp, amax[row], btok, bval, tau);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    __shared__ double s_cstart, s_last_start;
    __shared__ int s_chunk, s_last_c, owner, last_owner;
    __shared__ double red[4];
    const double* cs = chunk_sum + (int64_t)r * nchunk;
    // the row's uniform and the target u * S, S the sum of the chunk totals
    u32x4 ctr;
    ctr[0] = (uint32_t)row; ctr[1] = (uint32_t)t; ctr[2] = (uint32_t)canvas_idx; ctr[3] = 0u;
    const uint32_t x0 = philox10(ctr, seed_lo, seed_hi)[0];
    const double u = (double)(x0 >> 8) * (1.0 / 16777216.0);
    double part = 0.0;
    for (int c = tid; c < nchunk; c += 256) part += cs[c];
    part = wave_sum_d(part);
    if (lane == 0) red[w] = part;
    if (tid == 0) { s_chunk = 0x7fffffff; s_last_c = -1; owner = 0x7fffffff; last_owner = -1; }
    __syncthreads();
    const double target = u * ((red[0] + red[1]) + (red[2] + red[3]));
    __syncthreads();
    // the chunk where the running sum of the chunk totals (in vocabulary
    // order, 256 chunks at a time) passes the target: the first with mass
    // whose end exceeds it; if rounding leaves none, the last with mass
    double run = 0.0;
    for (int b = 0; b < nchunk; b += 256) {
        const int c = b + tid;
        const double v = c < nchunk ? cs[c] : 0.0;
        double incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const double y = __shfl_up(incl, o, WAVE);
            if (lane >= o) incl += y;
        }
        if (lane == 63) red[w] = incl;
        __syncthreads();
        double woff = 0.0;
        for (int i = 0; i < w; ++i) woff += red[i];
        const double start = run + woff + incl - v;
        run += (red[0] + red[1]) + (red[2] + red[3]);
        if (v > 0.0 && start + v > target) atomicMin(&s_chunk, c);
        if (v > 0.0) atomicMax(&s_last_c, c);
        __syncthreads();
        if (c == s_chunk) s_cstart = start;
        if (c == s_last_c) s_last_start = start;
        __syncthreads();
        if (s_chunk != 0x7fffffff) break;  // uniform
    }
    int c = s_chunk;
    double cstart = s_cstart;
    if (c == 0x7fffffff) { c = s_last_c; cstart = s_last_start; }
    if (c < 0) {
        // no chunk holds finite positive mass (a NaN row, or a +inf logit
        // whose exp(z - M) is NaN): the argmax is committed and no chunk is
        // scanned (uniform over the workgroup)
        if (tid == 0) {
            tokens[row] = amax[row];
            committed[row] = 1;
        }
        return;
    }
    const int v0 = c * DRAW_CHUNK + tid * 16;
    float x[16];
    bool in[2];
    load16(rowp, v0, V, x, in);
    double wts[16];
    chunk_weights(x, in, v0, mask_id, btok, bval, tau, M, wts);
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < 16; ++q) s += wts[q];
    // exclusive scan of the thread sums inside the chunk
    double incl = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        double y = __shfl_up(incl, o, WAVE);
        if (lane >= o) incl += y;
    }
    if (lane == 63) red[w] = incl;
    __syncthreads();
    double woff = 0.0;
    for (int i = 0; i < w; ++i) woff += red[i];
    const double start = cstart + woff + incl - s;
    if (s > 0.0 && start + s > target) atomicMin(&owner, tid);
    if (s > 0.0) atomicMax(&last_owner, tid);
    __syncthreads();
    // the first thread whose running end exceeds the target; if rounding
    // leaves none, the last thread with mass in the chunk
    const int own = owner != 0x7fffffff ? owner : last_owner;
    if (tid == own) {
        double acc = start;
        int pick = -1, last = -1;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if (pick >= 0) break;
            const double wv = wts[q];
            if (wv > 0.0) last = v0 + q;
            acc += wv;
            if (wv > 0.0 && acc > target) pick = v0 + q;
        }
        if (pick < 0) pick = last >= 0 ? last : amax[row];  // no mass (NaN input): the argmax
        tokens[row] = pick;
        committed[row] = 1;
    }
}

// ---------------------------------------------------------------------------
// Re-mask, stop test, finish and state update. One workgroup of 1024 threads.
// state: [0] done, [1] step, [2] n_committed, [3] stable count, [4] n_selected,
//        [5] stop flag of the last step, [6] finished flag of the last step.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) finalize_kernel(
    const float* __restrict__ H, const int32_t* __restrict__ amax, int n, int mask_id,
    int32_t* __restrict__ state, int step_override, SamplerParams sp,
    int32_t* __restrict__ tokens, uint8_t* __restrict__ committed, int32_t* __restrict__ prev_amax,
    const uint8_t* __restrict__ selected, double* __restrict__ mean_out) {
    if (state && state[0]) return;
    const int tid = threadIdx.x;
    const int t = step_override >= 0 ? step_override : state[1];
    __shared__ int diff, ncom;
    __shared__ float hs[1024];
    if (tid == 0) { diff = 0; ncom = 0; }
    __syncthreads();
    int d = 0, c = 0;
    // Committed after this step's draws: under reselect-all only the rows
    // selected this step; otherwise every row committed so far.
    const bool reselect = sp.commit_mode != 0;
    for (int i = tid; i < n; i += 1024) {
        d += amax[i] != prev_amax[i];
        c += (reselect ? selected[i] : committed[i]) != 0;
        hs[i] = H[i];
    }
    if (d) atomicAdd(&diff, d);
    if (c) atomicAdd(&ncom, c);
    __syncthreads();
    // canvas mean in float64: per wave, then the 16 wave sums in order
    __shared__ double wmean[16];
    __shared__ double meanH;
    {
        const double v = tid < n ? (double)hs[tid] : 0.0;
        const double ws = wave_sum_d(v);
        if ((tid & 63) == 0) wmean[tid >> 6] = ws;
    }
    __syncthreads();
    if (tid == 0) {
        double acc = 0.0;
        for (int i = 0; i < 16; ++i) acc += wmean[i];
        meanH = acc / (double)n;
    }
    __syncthreads();
    const double mH = meanH;
    const int stable = (t > 0 && diff == 0) ? state[3] + 1 : 1;
    const bool stop = stable >= sp.stable_steps && mH < (double)sp.stop_entropy;
    const bool finished = stop || t == sp.max_steps - 1 || ncom == n;
    for (int i = tid; i < n; i += 1024) {
        if (!(reselect ? selected[i] : committed[i])) {
            tokens[i] = finished ? amax[i] : mask_id;
            committed[i] = finished ? 1 : 0;
        }
        prev_amax[i] = amax[i];
    }
    __syncthreads();
    if (tid == 0) {
        state[3] = stable;
        state[5] = stop ? 1 : 0;
        state[6] = finished ? 1 : 0;
        state[2] = finished ? n : ncom;
        state[1] = t + 1;
        if (mean_out) *mean_out = mH;
        state[0] = finished ? 1 : 0;
    }
}

// ---------------------------------------------------------------------------
// Host-side launchers.
// ---------------------------------------------------------------------------
// build-time tunable: chunks of 16384 columns per split of the statistics pass
// (a workgroup streams its split with the next chunk's loads in flight)
#ifndef DG_STATS_CHUNKS_PER_SPLIT
#define DG_STATS_CHUNKS_PER_SPLIT 8
#endif
static int nsplit_for(int V) {
    // DG_STATS_CHUNKS_PER_SPLIT x 16384 columns per split, fewer (a multiple
    // of 2048) for small vocabularies
    int cols = STATS_CHUNK * DG_STATS_CHUNKS_PER_SPLIT;
    if (V < cols) cols = ((V + 2047) / 2048) * 2048;
    return (V + cols - 1) / cols;
}

int sampler_nsplit(int V) { return nsplit_for(V); }
int draw_nchunk(int V) { return (V + DRAW_CHUNK - 1) / DRAW_CHUNK; }

hipError_t launch_logit_stats(const void* logits, int dtype_f32, int64_t ld, int n, int V,
                              const int32_t* state, int step_override, const SamplerParams& sp, int mask_id,
                              const int32_t* bias_tok, const float* bias_val, RowPart* parts,
                              hipStream_t st) {
    int ns = nsplit_for(V);
    int cols = (V + ns - 1) / ns;
    cols = ((cols + 2047) / 2048) * 2048;
    dim3 grid(ns, n);
#define DG_STATS(T, G)                                                                                          \
    logit_stats_kernel<T, G><<<grid, 256, 0, st>>>((const T*)logits, ld, V, cols, state, step_override, sp, \
                                                   mask_id, bias_tok, bias_val, parts, ns)
    if (dtype_f32) {
        if (sp.draw_mode) DG_STATS(float, true);
        else DG_STATS(float, false);
    } else {
        if (sp.draw_mode) DG_STATS(uint16_t, true);
        else DG_STATS(uint16_t, false);
    }
#undef DG_STATS
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gumbel-max draws: the selected rows sel_list[0 .. state[4]) take the
// candidate the statistics pass kept for them.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) gumbel_commit_kernel(const int32_t* __restrict__ sel_list,
                                                            const int32_t* __restrict__ gtok,
                                                            const int32_t* __restrict__ state,
                                                            int32_t* __restrict__ tokens,
                                                            uint8_t* __restrict__ committed) {
    if (state[0]) return;
    const int k = state[4];
    for (int i = threadIdx.x; i < k; i += 256) {
        const int row = sel_list[i];
        tokens[row] = gtok[row];
        committed[row] = 1;
    }
}

hipError_t launch_merge_rows(const RowPart* parts, int n, int nsplit, const int32_t* state, float* H,
                             float* lse, int32_t* amax, int32_t* gtok, hipStream_t st) {
    merge_rows_kernel<<<n, 256, 0, st>>>(parts, n, nsplit, state, H, lse, amax, gtok);
    return hipGetLastError();
}

hipError_t launch_sampler_tail(const void* logits, int dtype_f32, int64_t ld, int n, int V, int mask_id,
                               const int32_t* bias_tok, const float* bias_val, const float* H,
                               const int32_t* amax, int32_t* state, int step_override, const SamplerParams& sp,
                               uint64_t seed, int canvas_idx, int32_t* tokens, uint8_t* committed,
                               int32_t* prev_amax, uint8_t* selected, int32_t* sel_list, double* chunk_sum,
                               const int32_t* gtok, double* mean_out, hipStream_t st) {
    eb_select_kernel<<<1, 1024, 0, st>>>(H, committed, n, state, sp, selected, sel_list);
    uint32_t lo = (uint32_t)(seed & 0xffffffffu), hi = (uint32_t)(seed >> 32);
    const int grid = 512;
    if (sp.draw_mode) {
        if (!gtok) return hipErrorInvalidValue;
        gumbel_commit_kernel<<<1, 256, 0, st>>>(sel_list, gtok, state, tokens, committed);
    } else if (dtype_f32) {
        draw_chunks_kernel<float><<<grid, 256, 0, st>>>((const float*)logits, ld, V, mask_id, bias_tok, bias_val,
                                                        sel_list, amax, state, step_override, sp, chunk_sum);
        draw_pick_kernel<float><<<n, 256, 0, st>>>((const float*)logits, ld, V, mask_id, bias_tok, bias_val,
                                                   sel_list, amax, state, step_override, sp, lo, hi, canvas_idx,
                                                   chunk_sum, tokens, committed);
    } else {
        draw_chunks_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)logits, ld, V, mask_id, bias_tok,
                                                           bias_val, sel_list, amax, state, step_override, sp,
                                                           chunk_sum);
        draw_pick_kernel<uint16_t><<<n, 256, 0, st>>>((const uint16_t*)logits, ld, V, mask_id, bias_tok, bias_val,
                                                      sel_list, amax, state, step_override, sp, lo, hi,
                                                      canvas_idx, chunk_sum, tokens, committed);
    }
    finalize_kernel<<<1, 1024, 0, st>>>(H, amax, n, mask_id, state, step_override, sp, tokens, committed,
                                        prev_amax, selected, mean_out);
    return hipGetLastError();
}

}  // namespace dg
