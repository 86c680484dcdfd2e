// Launchers of the per-layer glue kernels (layer.hip) and attention (attention.hip).
#pragma once
#include <algorithm>

#include "common.hpp"

namespace dg {

hipError_t launch_embed(const void* E, int act_f32, int d, int V, const int32_t* tok, int n, float* X,
                        const int32_t* state, hipStream_t st);
// Y = rmsnorm(X); with Ylo (bf16 only) also Ylo = bf16(rmsnorm(X) - Y)
hipError_t launch_rmsnorm(const float* X, int n, int d, const float* w, float eps, void* Y, int act_f32,
                          const int32_t* state, hipStream_t st, void* Ylo = nullptr);
// X += sum over the nparts K-slice partials part[s][n][d] (slice order), then
// Y = rmsnorm(X); nparts = 0: the plain norm
hipError_t launch_residual_rmsnorm(float* X, const float* part, int nparts, int n, int d, const float* w, float eps,
                                   void* Y, int act_f32, const int32_t* state, hipStream_t st, void* Ylo = nullptr);
hipError_t launch_rope_table(int n, int hd, int64_t pos0, double base, float* cs, const int32_t* state,
                             hipStream_t st);
// qkv, or (nparts > 1) its K-slice f32 partials part[nparts][n][width]
hipError_t launch_rope_scatter(const void* qkv, const float* part, int nparts, int act_f32, int n, int Hq, int Hkv,
                               int hd, const float* cs, void* Q,
                               int64_t q_ld, int64_t q_off, void* K, void* V, int64_t kv_ld, int64_t kv_off,
                               int v_zero_to, const int32_t* state, hipStream_t st);
hipError_t launch_router_topk(const float* r, int nparts, const float* bias, int n, int E, int k, int32_t* ids,
                              float* gates, const int32_t* state, hipStream_t st);
// Largest row count n for which launch_hist_permute can permute n x k
// (row, slot) pairs over E experts (its one-workgroup LDS bound).
int hist_permute_max_rows(int k, int E);
hipError_t launch_hist_permute(const int32_t* ids, int n, int k, int E, int32_t* offsets, int32_t* perm,
                               int32_t* slot_of, int32_t* hit, int32_t* hit_mb, int32_t* hitB, int32_t* hitB_mb,
                               int big_min, int32_t* hit_out, const int32_t* state, hipStream_t st);
// X += shared + gated expert rows; with norm_w, A = rmsnorm(X) (and, with Alo,
// bf16 only, Alo = bf16(rmsnorm(X) - A))
hipError_t launch_combine(float* X, int n, int d, const float* Y, const int32_t* slot_of, const float* gates, int k,
                          int shared_off, const float* norm_w, float eps, void* A, int act_f32, const int32_t* state,
                          hipStream_t st, void* Alo = nullptr);

// Attention over up to two key segments per KV head (V stored transposed):
//   segment 1: K1 [Hkv][ld1][hd], V1^T [Hkv][hd][ld1], rows [s1, e1) (cache),
//              positions = row index
//   segment 2: K2 [Hkv][ld2][hd], V2^T [Hkv][hd][ld2], rows [0, n2) (canvas),
//              positions pos2_0 + row
// ld1 and ld2 are multiples of 64; V^T columns past e1 / n2 may hold anything
// (the bf16 kernel reads them as zero; the generic kernel never reads them).
// Queries Q [Hq][ldq][hd] rows [0, nq) at positions qpos0 + row; output
// O [nq][Hq*hd]. causal: key position <= query position; window > 0: and
// query position - key position < window (per query). Softmax scale 1/sqrt(hd).
struct AttnArgs {
    const void* Q;
    int64_t ldq;
    int nq;
    int64_t qpos0;
    const void* K1;
    const void* V1;
    int64_t ld1;
    int64_t s1, e1;
    const void* K2;
    const void* V2;
    int64_t ld2;
    int n2;
    int64_t pos2_0;
    int Hq, Hkv, hd;
    int causal;
    int window;       // per-query window for causal attention (0 = none)
    void* O;
    float* part_o;    // split-KV partials [splits][nq][Hq][hd] f32
    float* part_ml;   // [splits][nq][Hq][2]
    int splits;
    const int32_t* state;
};
hipError_t launch_attention(const AttnArgs& a, int act_f32, hipStream_t st);
size_t attention_partial_floats(int splits, int nq, int Hq, int hd);
// KV splits for nq queries over `keys` keys: enough workgroups for the chip,
// at most max_splits and max_splits * nq <= max_rows partial rows
int attention_splits(int nq, int64_t keys, int Hq, int Hkv, int hd, int act_f32, int max_splits, int max_rows);

}  // namespace dg
