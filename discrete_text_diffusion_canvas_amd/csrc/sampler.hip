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
//   eb_select     one workgroup: sort candidates by (entropy, position), float32
//                 running sum in sorted order, cut at the bound (at least one)
//   draw_chunks   chip-wide: float64 sums of exp(z - M) per (selected row, chunk)
//   draw_pick     per selected row: Philox4x32-10 uniform, float64 inverse CDF
//                 in vocabulary order (chunk totals, then a scan in one chunk)
//   finalize      one workgroup: re-mask, canvas-mean entropy (float64, position
//                 order), stop test, argmax fill at the end, state update
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

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&x)[8]) {
    u16x8 v = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = bf2f(v[j]);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { x[j] = a[j]; x[4 + j] = b[j]; }
}

// ---------------------------------------------------------------------------
// Row statistics over given logits (the sampler-only entry point). Grid
// (nsplit, n), 256 threads; split i covers columns [i*split_cols, ...), a
// multiple of 2048. Each thread loads its 64 columns (8 vectors of 8, wave
// loads contiguous) before computing, so every thread keeps 8 loads in flight.
// The max and its lowest column come from the tempered value z2 = x*log2(e)/tau;
// for bf16 logits z2 preserves the order and the equalities of x exactly (two
// distinct bf16 values differ by at least 2^-8 relative), for f32 logits the
// raw values are compared instead.
// GUMBEL: the same pass also keeps the Gumbel-max candidate of the split, the
// lowest column maximising z_v - log(-log u_v) with z = (L + bias) / tau and
// u_v from Philox at counter (row, step, canvas, 1 + v / 4), word v % 4.
// ---------------------------------------------------------------------------
template <typename T, bool GUMBEL>
__global__ void __launch_bounds__(256) logit_stats_kernel(
    const T* __restrict__ logits, int64_t ld, int V, int split_cols,
    const int32_t* __restrict__ state, int step_override, SamplerParams sp, int mask_id,
    const int32_t* __restrict__ bias_tok, const float* __restrict__ bias_val,
    RowPart* __restrict__ parts, int nsplit) {
    if (state && state[0]) return;
    constexpr int PER = 8;
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
    const float inv_tau = (float)(1.0 / tau_at(sp, t));
    for (int base = c0; base < c1; base += 256 * 8 * PER) {
        float x[PER][8];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            int v0 = base + (j * 256 + tid) * 8;
            if (v0 < c1) {
                load8<T>(rowp + v0, x[j]);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) x[j][q] = -INFINITY;
            }
        }
        const bool special = (btok >= base && btok < base + 256 * 8 * PER) ||
                             (mask_id >= base && mask_id < base + 256 * 8 * PER);
        float z[PER][8];
        float vm = -INFINITY;
        int vi = 0x7fffffff;
        float rm = -INFINITY;  // raw max (f32 logits)
        if (!special) {
#pragma unroll
            for (int j = 0; j < PER; ++j)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    z[j][q] = x[j][q] * c2;
                    const int col = base + (j * 256 + tid) * 8 + q;
                    if constexpr (sizeof(T) == 2) {
                        if (z[j][q] > vm) { vm = z[j][q]; vi = col; }
                    } else {
                        vm = fmaxf(vm, z[j][q]);
                        if (x[j][q] > rm) { rm = x[j][q]; vi = col; }
                    }
                }
        } else {
#pragma unroll
            for (int j = 0; j < PER; ++j)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int col = base + (j * 256 + tid) * 8 + q;
                    float l = x[j][q] + (col == btok ? bval : 0.f);
                    if (col == mask_id) l = -INFINITY;
                    z[j][q] = l * c2;
                    if constexpr (sizeof(T) == 2) {
                        if (z[j][q] > vm) { vm = z[j][q]; vi = col; }
                    } else {
                        vm = fmaxf(vm, z[j][q]);
                        if (l > rm) { rm = l; vi = col; }
                    }
                }
        }
        if constexpr (GUMBEL) {
            // z = z2 / log2(e) and the bias / MASK handling of z2 above
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
                    const float zn = z[j][q] * 0.6931471805599453f;
                    if (zn == -INFINITY || v0 + q >= c1) continue;
                    const float val = zn + gumbel_of(w[q >> 2][q & 3]);
                    if (val > gm.v) { gm.v = val; gm.i = v0 + q; }
                }
            }
        }
        if (vm == -INFINITY) continue;
        float ls = 0.f, lt = 0.f;
#pragma unroll
        for (int j = 0; j < PER; ++j)
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                float d = z[j][q] - vm;
                float w = exp2f(d);
                ls += w;
                lt += w > 0.f ? w * d : 0.f;
            }
        e = ent_merge(e, EntPart{vm, ls, lt});
        ArgMax c{sizeof(T) == 2 ? vm : rm, vi};
        am = argmax_merge(am, c);
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
        RowPart p;
        p.m2 = e.m; p.s = e.s; p.t = e.t; p.lmax = am.v; p.amax = am.i == 0x7fffffff ? -1 : am.i;
        p.pad[0] = __float_as_int(gm.v);
        p.pad[1] = gm.i == 0x7fffffff ? -1 : gm.i;
        p.pad[2] = 0;
        parts[(int64_t)row * nsplit + sp_i] = p;
    }
}

// ---------------------------------------------------------------------------
// Merge the per-split partials of each row. One wavefront per row.
// H = ln2 * (log2 S - T2 / S) (clamped at 0); lse = ln2 * (M2 + log2 S).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) merge_rows_kernel(
    const RowPart* __restrict__ parts, int n, int nsplit, const int32_t* __restrict__ state,
    float* __restrict__ H, float* __restrict__ lse, int32_t* __restrict__ amax, int32_t* __restrict__ gtok) {
    if (state && state[0]) return;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= n) return;
    EntPart e{-INFINITY, 0.f, 0.f};
    ArgMax am{-INFINITY, 0x7fffffff}, gm{-INFINITY, 0x7fffffff};
    const RowPart* p = parts + (int64_t)row * nsplit;
    for (int i = lane; i < nsplit; i += 64) {
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
    if (lane == 0) {
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
// IEEE bit patterns order like the values. Non-candidates (committed rows,
// unless every row is re-selected) sort last. Writes
// the selection mask, the selected positions in sorted order (sel_list) and
// their count (state word 4).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) eb_select_kernel(
    const float* __restrict__ H, const uint8_t* __restrict__ committed, int n,
    int32_t* __restrict__ state, SamplerParams sp, uint8_t* __restrict__ selected,
    int32_t* __restrict__ sel_list) {
    if (state && state[0]) return;
    __shared__ unsigned long long key[1024];
    __shared__ float hs[1024];
    __shared__ int kstar;
    const int tid = threadIdx.x;
    int npow = 1;
    while (npow < n) npow <<= 1;
    for (int i = tid; i < npow; i += 1024) {
        unsigned long long k = ~0ull;
        if (i < n && (sp.commit_mode != 0 || !committed[i]))
            k = ((unsigned long long)__float_as_uint(H[i]) << 32) | (unsigned)i;
        key[i] = k;
    }
    __syncthreads();
    // bitonic sort ascending
    for (int size = 2; size <= npow; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < npow; i += 1024) {
                int j = i ^ stride;
                if (j > i) {
                    bool up = (i & size) == 0;
                    unsigned long long a = key[i], b = key[j];
                    if ((a > b) == up) { key[i] = b; key[j] = a; }
                }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < n; i += 1024) {
        unsigned long long kk = key[i];
        hs[i] = kk == ~0ull ? -1.f : __uint_as_float((unsigned)(kk >> 32));
        selected[i] = 0;
    }
    __syncthreads();
    if (tid == 0) {
        // float32 running sum in sorted order; mode 0: S_k <= bound,
        // mode 1: S_{k-1} <= bound. At least one while candidates remain.
        float run = 0.f;
        int k = 0;
        for (int i = 0; i < n; ++i) {
            float h = hs[i];
            if (h < 0.f) break;
            float prev = run;
            run = run + h;
            bool ok = sp.bound_mode == 0 ? (run <= sp.bound) : (prev <= sp.bound);
            if (!ok) break;
            k = i + 1;
        }
        if (k == 0 && n > 0 && hs[0] >= 0.f) k = 1;
        kstar = k;
        state[4] = k;
    }
    __syncthreads();
    for (int i = tid; i < kstar; i += 1024) {
        int pos = (int)(key[i] & 0xffffffffu);
        selected[pos] = 1;
        sel_list[i] = pos;
    }
}

// ---------------------------------------------------------------------------
// Inverse-CDF draw of the selected rows, in float64: w_v = exp(z_v - M') with
// z = (L + bias) / tau and M' = z at the row's argmax (any offset cancels in
// the comparison with u * sum w). The vocabulary is cut into chunks of
// DRAW_CHUNK columns; each of the 256 threads of a chunk owns 16 consecutive
// columns.
//   draw_chunks: every (selected row, chunk) pair sums its w (chip-wide grid).
//   draw_pick:   per selected row, the running sum over chunk totals finds the
//                chunk where u * S falls, and a scan inside it the column.
// ---------------------------------------------------------------------------
constexpr int DRAW_CHUNK = 4096;

template <typename T>
__device__ __forceinline__ double zval(const T* rowp, int v, int btok, double bval, double tau) {
    float l;
    if constexpr (sizeof(T) == 2) l = bf2f(rowp[v]); else l = rowp[v];
    double L = (double)l + (v == btok ? bval : 0.0);
    return L / tau;
}

template <typename T>
__device__ __forceinline__ double thread_chunk_sum(const T* rowp, int v0, int V, int mask_id, int btok,
                                                   double bval, double tau, double M) {
    double s = 0.0;
    for (int q = 0; q < 16; ++q) {
        int v = v0 + q;
        if (v < V && v != mask_id) s += exp(zval(rowp, v, btok, bval, tau) - M);
    }
    return s;
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
        double s = thread_chunk_sum(rowp, c * DRAW_CHUNK + threadIdx.x * 16, V, mask_id, btok, bval, tau, M);
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
    __shared__ double s_target, s_cstart;
    __shared__ int s_chunk, owner, last_owner;
    __shared__ double red[4];
    if (tid == 0) {
        u32x4 ctr;
        ctr[0] = (uint32_t)row; ctr[1] = (uint32_t)t; ctr[2] = (uint32_t)canvas_idx; ctr[3] = 0u;
        const uint32_t x0 = philox10(ctr, seed_lo, seed_hi)[0];
        const double u = (double)(x0 >> 8) * (1.0 / 16777216.0);
        const double* cs = chunk_sum + (int64_t)r * nchunk;
        double tot = 0.0;
        for (int c = 0; c < nchunk; ++c) tot += cs[c];
        const double target = u * tot;
        double run = 0.0;
        int owner_c = -1;
        double start = 0.0;
        for (int c = 0; c < nchunk; ++c) {
            if (cs[c] > 0.0 && run + cs[c] > target) { owner_c = c; start = run; break; }
            run += cs[c];
        }
        if (owner_c < 0) {  // rounding at the very end: last chunk with mass
            run = 0.0;
            for (int c = 0; c < nchunk; ++c) {
                if (cs[c] > 0.0) { owner_c = c; start = run; }
                run += cs[c];
            }
        }
        s_target = target;
        s_cstart = start;
        s_chunk = owner_c;
        owner = 0x7fffffff;
        last_owner = -1;
        if (owner_c < 0) {
            // no chunk holds finite positive mass (a NaN row, or a +inf logit
            // whose exp(z - M) is NaN): the argmax is committed and no chunk
            // is scanned
            tokens[row] = amax[row];
            committed[row] = 1;
        }
    }
    __syncthreads();
    const int c = s_chunk;
    if (c < 0) return;  // uniform over the workgroup
    const double target = s_target;
    const int v0 = c * DRAW_CHUNK + tid * 16;
    const double s = thread_chunk_sum(rowp, v0, V, mask_id, btok, bval, tau, M);
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
    const double start = s_cstart + woff + incl - s;
    if (s > 0.0 && start + s > target) atomicMin(&owner, tid);
    if (s > 0.0) atomicMax(&last_owner, tid);
    __syncthreads();
    // the first thread whose running end exceeds the target; if rounding
    // leaves none, the last thread with mass in the chunk
    const int own = owner != 0x7fffffff ? owner : last_owner;
    if (tid == own) {
        double run = start;
        int pick = -1, last = -1;
        for (int q = 0; q < 16; ++q) {
            int v = v0 + q;
            if (v >= V || v == mask_id) continue;
            double wv = exp(zval(rowp, v, btok, bval, tau) - M);
            if (wv > 0.0) last = v;
            run += wv;
            if (run > target) { pick = v; break; }
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
    __shared__ double meanH;
    if (tid == 0) {
        double acc = 0.0;  // float64, position order
        for (int i = 0; i < n; ++i) acc += (double)hs[i];
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
static int nsplit_for(int V) {
    // 16384 columns per split (256 threads x 64), fewer for small vocabularies
    int cols = 16384;
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
    merge_rows_kernel<<<(n + 3) / 4, 256, 0, st>>>(parts, n, nsplit, state, H, lse, amax, gtok);
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
