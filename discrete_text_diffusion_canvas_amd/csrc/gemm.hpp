// Arguments and the LM-head epilogue of the MFMA GEMM family (gemm.hip).
#pragma once
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dg {

enum { WK_SAME = 0, WK_FP8 = 1 };
enum { EPI_STORE_F32 = 0, EPI_STORE_BF16 = 1, EPI_RESIDUAL = 2, EPI_SWIGLU = 3, EPI_LMHEAD = 4 };
enum { SHAPE_PROJ = 0, SHAPE_SMALL_M = 1, SHAPE_LDS = 2 };

struct GemmArgs {
    // A: activations [rows][K] (f32 or bf16), row stride lda; optional gather
    const void* A;
    const void* A2;                 // LM head: the bf16 residual x - bf16(x) of A, same layout
    int64_t lda;
    const int32_t* a_rows;          // A row of output row r is a_rows[r] (grouped gathers)
    // W: weights [N][K] per group, row stride ldw (elements); fp8 codes or same type as A
    const void* W;
    const void* W2;                 // SwiGLU: up weights (W = gate); each [N/2][K]
    int64_t ldw;
    int64_t w_group_stride;         // elements between groups' weights
    const uint16_t* w_scale;        // fp8: bf16 scale per output row (per group)
    const uint16_t* w2_scale;
    int64_t scale_group_stride;
    int M, N, K;                    // M: rows (non-grouped) / bound on rows per group (grouped);
                                    // N: output columns (SwiGLU: 2F)
    const int32_t* group_offsets;   // grouped: group g owns rows [off[g], off[g+1])
    const int32_t* hit;             // grouped: [0] = number of groups with rows, then their ids
    const int32_t* hit_mb;          // grouped: largest number of 64-row blocks of a group
    // outputs
    void* C;                        // [rows][ldc]
    int64_t ldc;
    int c_f32;                      // C element type: 1 f32, 0 bf16 (SwiGLU / LM head)
    float* X;                       // EPI_RESIDUAL: X[row][n] += C
    int64_t ldx;
    // split-K (LDS-staged dense GEMM): K slices, f32 partials [ksplit][M][N]
    int ksplit;
    float* part;
    int defer_reduce;               // dense split-K: leave the partials to the consumer
    // control
    const int32_t* state;           // canvas state (done flag, step) or NULL
    // LM head
    RowPart* parts;                 // [rows][nsplit]
    int nsplit;
    int step_override;
    SamplerParams sp;
    int mask_id;
    const int32_t* bias_tok;
    const float* bias_val;
};

hipError_t gemm_launch(const GemmArgs& g, int act_f32, int w_fp8, int epi, int groups, int shape,
                       hipStream_t st);
hipError_t stream_gemm_launch(const GemmArgs& g, int act_f32, int w_fp8, int epi, int groups, int max_rows,
                              hipStream_t st);
// The LM head with bf16 activations given as hi + lo pairs (A, A2), bf16 or
// e4m3 (w_scale) vocabulary rows, f32 statistics partials per 128 columns
// (lmhead.hip): K % 64 == 0, N % 8 == 0, ldc % 8 == 0, nsplit = N / 128.
bool lmhead_supported(const GemmArgs& g);
hipError_t lmhead_launch(const GemmArgs& g, hipStream_t st);
// LDS-staged GEMM (bf16 activations and weights, K % 64 == 0): grouped over
// the big-group list in g.hit / g.hit_mb (SwiGLU or f32 store), or dense
// (g.group_offsets NULL) with optional split-K through g.part.
bool tile_gemm_supported(const GemmArgs& g, int act_f32, int w_fp8, int epi);
hipError_t tile_gemm_launch(const GemmArgs& g, int epi, int groups, int max_rows, hipStream_t st);
// K slices for a dense M x N x K product (1 = no split)
int tile_dense_ksplit(int M, int N, int K);
// K slices of the grouped gate/up GEMM for a batch of `rows` tokens
int tile_grouped_ksplit(int rows);
// Grouped SwiGLU split over K: slot rows of groups of >= big_min rows hold
// ks_big partial slices in g.part, the others ks_small (1: already stored);
// adds them in slice order and stores silu(gate) * up to g.C (bf16)
hipError_t swiglu_reduce_launch(const GemmArgs& g, int groups, int big_min, int ks_big, int ks_small, hipStream_t st);

// ---------------------------------------------------------------------------
// LM-head epilogue: the logits of record (the accumulator in the storage
// type) are stored; then per row over this tile's columns, from the f32
// accumulators, the base-2 entropy partials of z2 = (logit + bias) *
// log2(e) / tau with the MASK column removed, and the argmax of
// (logit + bias), lowest column on ties.
// ---------------------------------------------------------------------------
template <int WM, int WN, int TM, int TN>
constexpr size_t lmhead_epilogue_lds() {
    return (size_t)WN * WM * TM * 16 * (sizeof(EntPart) + sizeof(ArgMax));
}

__device__ __forceinline__ double lm_tau_at(const SamplerParams& sp, int t) {
    if (sp.max_steps <= 1) return (double)sp.temp_start;
    return (double)sp.temp_start +
           ((double)sp.temp_end - (double)sp.temp_start) * (double)t / (double)(sp.max_steps - 1);
}

template <int WM, int WN, int TM, int TN>
__device__ __forceinline__ void lmhead_epilogue(const GemmArgs& g, f32x4 (&acc)[TM][TN], int mb, int mcount,
                                                int n0, unsigned char* smem) {
    constexpr int BM = WM * TM * 16;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 15, lg = lane >> 4;
    const int wrow0 = wm * TM * 16;
    const int t = g.step_override >= 0 ? g.step_override : (g.state ? g.state[1] : 0);
    const float c2 = (float)(1.4426950408889634 / lm_tau_at(g.sp, t));
    EntPart* pe = reinterpret_cast<EntPart*>(smem);
    ArgMax* pa = reinterpret_cast<ArgMax*>(pe + WN * BM);
    __syncthreads();  // the main loop's LDS buffers are reused
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = wrow0 + i * 16 + lg * 4 + q;
            const bool rok = r < mcount;
            const int row = mb + r;
            const int bt = (rok && g.bias_tok) ? g.bias_tok[row] : -1;
            const float bv = (rok && g.bias_tok) ? g.bias_val[row] : 0.f;
            float zv[TN];
            float vm = -INFINITY, rawm = -INFINITY;
            int vi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n0 + wn * TN * 16 + j * 16 + lr;
                const float l = acc[i][j][q];
                if (rok && n < g.N) {
                    if (g.c_f32)
                        reinterpret_cast<float*>(g.C)[(int64_t)row * g.ldc + n] = l;
                    else
                        reinterpret_cast<uint16_t*>(g.C)[(int64_t)row * g.ldc + n] = f2bf(l);
                }
                float lb = l + (n == bt ? bv : 0.f);
                bool ok = rok && n < g.N && n != g.mask_id;
                if (!ok) lb = -INFINITY;
                zv[j] = lb * c2;
                vm = fmaxf(vm, zv[j]);
                if (lb > rawm) { rawm = lb; vi = n; }
            }
            // argmax across the 16 lanes holding this row
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                float ov = __shfl_xor(rawm, o, 64);
                int oi = __shfl_xor(vi, o, 64);
                if (ov > rawm || (ov == rawm && oi < vi)) { rawm = ov; vi = oi; }
                vm = fmaxf(vm, __shfl_xor(vm, o, 64));
            }
            float s = 0.f, tt = 0.f;
            if (vm != -INFINITY) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    float d = zv[j] - vm;
                    float w = exp2f(d);
                    s += w;
                    tt += w > 0.f ? w * d : 0.f;
                }
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                s += __shfl_xor(s, o, 64);
                tt += __shfl_xor(tt, o, 64);
            }
            if (lr == 0) {
                pe[wn * BM + r] = EntPart{vm, s, tt};
                pa[wn * BM + r] = ArgMax{rawm, vi};
            }
        }
    }
    __syncthreads();
    for (int r = tid; r < BM; r += 256) {
        if (r >= mcount) continue;
        EntPart e = pe[r];
        ArgMax a = pa[r];
#pragma unroll
        for (int w = 1; w < WN; ++w) {
            e = ent_merge(e, pe[w * BM + r]);
            a = argmax_merge(a, pa[w * BM + r]);
        }
        RowPart p;
        p.m2 = e.m; p.s = e.s; p.t = e.t; p.lmax = a.v; p.amax = (a.i == 0x7fffffff || a.v == -INFINITY) ? -1 : a.i;
        p.pad[0] = p.pad[1] = p.pad[2] = 0;
        g.parts[(int64_t)(mb + r) * g.nsplit + blockIdx.x] = p;
    }
}

}  // namespace dg
