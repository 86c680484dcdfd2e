// The model handle and the launch order of the decoder step, the encoder
// prefill/append and canvas generation (include/dg.h).
//
// DiffusionGemma model card (zh-TW), "模型總覽" (overview): the encoder
// prefills the prompt into a KV cache; the decoder denoises a canvas with
// bidirectional attention and cross-attention into the cache; a fully
// denoised canvas is encoded and appended, then the next canvas starts.
// Best practice 1 gives the sampler that ends each step.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/dg.h"
#include "api_util.hpp"
#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"
#include "layer.hpp"

using namespace dgapi;

struct dg_model {
    dg_config cfg;
    const void* embed;
    const void* lm8 = nullptr;        // optional e4m3 LM head [vocab][d]
    const uint16_t* lm8_scale = nullptr;
    const float* final_norm;
    std::vector<dg_layer_weights> layers;
};

// expert groups with at least this many rows take the LDS-staged GEMM (bf16);
// on the 256-row decode step 33 and 49 measured the same as 65, 97 and 129
// 4% and 6% slower per step
#ifndef DG_TILE_MIN_ROWS
#define DG_TILE_MIN_ROWS 65
#endif

namespace {

constexpr int MAX_SPLITS = 16;
constexpr int SPLIT_ROWS = 256;  // partial buffers hold MAX_SPLITS x SPLIT_ROWS query rows

int lm_bn(const dg_config& c) { return 128; }
int lm_nsplit(const dg_config& c) { return (c.vocab + lm_bn(c) - 1) / lm_bn(c); }
size_t act_bytes(const dg_config& c) { return c.act_dtype == DG_F32 ? 4 : 2; }
bool is_global(const dg_config& c, int l) { return c.global_every > 0 && l % c.global_every == c.global_every - 1; }

struct Work {
    float* X;          // [T][d] residual stream
    void* A;           // [T][d] normed activations (act dtype)
    void* A_lo;        // [T][d] bf16 residual of the final-normed activations (LM head operand)
    void* QKV;         // [T][(Hq+2Hkv) hd]
    void* Q;           // [Hq][T][hd]
    void* Kc;          // [Hkv][T64][hd]
    void* Vc;          // [Hkv][hd][T64] (transposed)
    void* O;           // [T][Hq hd]
    float* rope_cs;    // [T][hd/2][2] cos, sin of the rows' RoPE angles
    float* gemm_part;  // split-K partials of the dense projections
    float* gu_part;    // split-K partials of the tiled expert gate/up GEMM
    float* part_o;     // attention split partials
    float* part_ml;
    float* rlog;       // router logits: [K slices][n][E] partial sums
    int32_t* ids;      // [T][k]
    float* gates;      // [T][k]
    int32_t* offsets;  // [E+2]
    int32_t* perm;     // [T(k+1)]
    int32_t* slot_of;  // [T k]
    int32_t* hit;      // [E+2]: groups with rows ([0] = count)
    int32_t* hit_mb;   // [1]: largest 64-row block count of a group
    int32_t* hitB;     // [E+2]: groups of many rows, for the LDS-staged GEMM ([0] = count)
    int32_t* hitB_mb;  // [1]: largest 256-row block count of those
    void* Hbuf;        // [T(k+1)][F]
    float* Y;          // [T(k+1)][d]
    dg::RowPart* parts;  // [min(T, canvas)][nsplit]
    int32_t* sel_list;
    double* chunk_sum;
    int32_t* gtok;      // [Nc]: Gumbel-max candidates of the rows
    int32_t* bias_tok;  // [T]: a batch's per-row bias tokens (-1: none)
    float* bias_val;    // [T]
    size_t bytes;
    int rows;
    int rows64;        // T rounded up to a multiple of 64 (canvas K/V row stride)
    int32_t* experts_hit = nullptr;  // optional [n_layers] routed experts hit per layer (caller's buffer)
};

// K slices of a weight-streaming GEMM over d_model inputs: the most (up to
// 16) that divide its 32-wide k-steps and leave each slice at least
// min_steps, so few output tiles still spread over many workgroups. Measured
// best: 8 steps (two per wave) for the router, 16 for the gate/up products of
// the small expert groups.
#ifndef DG_ROUTER_SLICE_STEPS
#define DG_ROUTER_SLICE_STEPS 8
#endif
#ifndef DG_SMALL_SLICE_STEPS
#define DG_SMALL_SLICE_STEPS 16
#endif
#ifndef DG_STREAM_MAX_SLICES
#define DG_STREAM_MAX_SLICES 16
#endif
int stream_ksplit(const dg_config& c, int min_steps) {
    const int ks_total = c.d_model / 32;
    int best = 1;
    for (int s = 2; s <= DG_STREAM_MAX_SLICES; ++s)
        if (ks_total % s == 0 && ks_total / s >= min_steps) best = s;
    return best;
}
int router_ksplit(const dg_config& c) { return stream_ksplit(c, DG_ROUTER_SLICE_STEPS); }
int small_ksplit(const dg_config& c) { return stream_ksplit(c, DG_SMALL_SLICE_STEPS); }

Work carve(const dg_model* m, void* base, int T) {
    const dg_config& c = m->cfg;
    const size_t ab = act_bytes(c);
    const int d = c.d_model, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
    const int E = c.n_experts, k = c.top_k, F = c.ffn_hidden;
    const int Nc = std::min(T, c.max_canvas);
    Carve cv(base);
    Work w;
    w.X = cv.take<float>((size_t)T * d);
    w.A = cv.take<char>((size_t)T * d * ab);
    w.A_lo = cv.take<char>((size_t)T * d * ab);
    w.QKV = cv.take<char>((size_t)T * (Hq + 2 * Hkv) * hd * ab);
    w.Q = cv.take<char>((size_t)T * Hq * hd * ab);
    const int T64 = (T + 63) / 64 * 64;
    w.Kc = cv.take<char>((size_t)T64 * Hkv * hd * ab);
    w.Vc = cv.take<char>((size_t)T64 * Hkv * hd * ab);
    w.O = cv.take<char>((size_t)T * Hq * hd * ab);
    w.rope_cs = cv.take<float>((size_t)T * hd);
    {   // split-K partials of the QKV and output projections (when they split)
        const int nqkv = (Hq + 2 * Hkv) * hd;
        const int ka = dg::tile_dense_ksplit(T, nqkv, d), kb = dg::tile_dense_ksplit(T, d, Hq * hd);
        const size_t parts = std::max(ka > 1 ? (size_t)ka * T * nqkv : 0, kb > 1 ? (size_t)kb * T * d : 0);
        w.gemm_part = parts ? cv.take<float>(parts) : nullptr;
    }
    {   // split-K partials of the tiled gate/up GEMM: [slices][T (k + 1) slots][2F]
        const int gks = ab == 2 ? std::max(dg::tile_grouped_ksplit(T), small_ksplit(c)) : 1;
        w.gu_part = gks > 1 ? cv.take<float>((size_t)gks * T * (k + 1) * 2 * F) : nullptr;
    }
    w.part_o = cv.take<float>((size_t)MAX_SPLITS * SPLIT_ROWS * Hq * hd);
    w.part_ml = cv.take<float>((size_t)MAX_SPLITS * SPLIT_ROWS * Hq * 2);
    w.rlog = cv.take<float>((size_t)router_ksplit(c) * T * E);
    w.ids = cv.take<int32_t>((size_t)T * k);
    w.gates = cv.take<float>((size_t)T * k);
    w.offsets = cv.take<int32_t>(E + 2);
    w.perm = cv.take<int32_t>((size_t)T * (k + 1));
    w.slot_of = cv.take<int32_t>((size_t)T * k);
    w.hit = cv.take<int32_t>(E + 2);
    w.hit_mb = cv.take<int32_t>(1);
    w.hitB = cv.take<int32_t>(E + 2);
    w.hitB_mb = cv.take<int32_t>(1);
    w.Hbuf = cv.take<char>((size_t)T * (k + 1) * F * ab);
    w.Y = cv.take<float>((size_t)T * (k + 1) * d);
    w.parts = cv.take<dg::RowPart>((size_t)Nc * lm_nsplit(c));
    w.sel_list = cv.take<int32_t>(Nc);
    w.chunk_sum = cv.take<double>((size_t)Nc * dg::draw_nchunk(c.vocab));
    w.gtok = cv.take<int32_t>(Nc);
    w.bias_tok = cv.take<int32_t>(T);
    w.bias_val = cv.take<float>(T);
    w.bytes = cv.off;
    w.rows = T;
    w.rows64 = T64;
    return w;
}

// largest chunk (<= cap) whose workspace fits in ws_bytes
int rows_fitting(const dg_model* m, size_t ws_bytes, int cap) {
    int best = 0;
    for (int T = 1; T <= cap; T *= 2)
        if (carve(m, nullptr, T).bytes <= ws_bytes) best = T;
    if (best && best < cap && carve(m, nullptr, cap).bytes <= ws_bytes) best = cap;
    return best;
}

dg::GemmArgs gargs() {
    dg::GemmArgs g;
    memset(&g, 0, sizeof g);
    g.step_override = -1;
    return g;
}

#define DG_TRY(expr, what)                                        \
    do {                                                          \
        if (dg_status _s = hip_check((expr), what)) return _s;    \
    } while (0)

// A dense projection of n rows: the LDS-staged GEMM (split over K when there
// are too few column tiles to fill the chip) where it applies, else the
// weight-streaming GEMM. With parts != NULL a split product leaves its K-slice
// partials in w.gemm_part for the consumer to add (*parts = their count;
// 1 = the result is in g.C).
hipError_t dense_gemm(dg::GemmArgs g, const Work& w, int f32, int fp8, int epi, hipStream_t st,
                      int* parts = nullptr) {
    if (parts) *parts = 1;
    if (dg::tile_gemm_supported(g, f32, fp8, epi)) {
        g.ksplit = dg::tile_dense_ksplit(g.M, g.N, g.K);
        g.part = w.gemm_part;
        if (g.ksplit > 1 && g.part && parts) {
            g.defer_reduce = 1;
            *parts = g.ksplit;
        }
        if (g.ksplit <= 1 || g.part) return dg::tile_gemm_launch(g, epi, 1, g.M, st);
        g.ksplit = 0;
        g.part = nullptr;
    }
    return dg::gemm_launch(g, f32, fp8, epi, 0, dg::SHAPE_PROJ, st);
}

// ---------------------------------------------------------------------------
// The MoE half of a layer on rows X[0..n): X += shared(b) + sum_j g_j expert_j(b)
// ---------------------------------------------------------------------------
// resid_parts > 1: the output projection left that many K-slice partials in
// w.gemm_part, added to X here before the norm.
// next_lo: with the final norm as next_norm (bf16), the normed rows are also
// left as hi + lo pairs for the LM head (w.A, w.A_lo).
dg_status moe_block(const dg_model* m, int l, const Work& w, int n, const float* next_norm, const int32_t* state,
                    hipStream_t st, int resid_parts = 1, bool next_lo = false) {
    const dg_config& c = m->cfg;
    const dg_layer_weights& L = m->layers[l];
    const int d = c.d_model, E = c.n_experts, k = c.top_k, F = c.ffn_hidden;
    const int f32 = c.act_dtype == DG_F32, fp8 = c.weight_dtype == DG_FP8_E4M3;
    DG_TRY(dg::launch_residual_rmsnorm(w.X, w.gemm_part, resid_parts > 1 ? resid_parts : 0, n, d, L.moe_norm,
                                       c.norm_eps, w.A, f32, state, st),
           "rmsnorm");
    {   // router logits (router weights are never e4m3)
        dg::GemmArgs g = gargs();
        g.A = w.A; g.lda = d; g.W = L.router; g.ldw = d; g.M = n; g.N = E; g.K = d;
        g.C = w.rlog; g.ldc = E; g.state = state;
        g.ksplit = router_ksplit(c); g.part = w.rlog;
        DG_TRY(dg::gemm_launch(g, f32, 0, dg::EPI_STORE_F32, 0, dg::SHAPE_PROJ, st), "router gemm");
    }
    DG_TRY(dg::launch_router_topk(w.rlog, router_ksplit(c), L.router_bias, n, E, k, w.ids, w.gates, state, st),
           "router topk");
    // groups of more than 64 rows go to the LDS-staged GEMM (bf16 activations)
    dg::GemmArgs gu = gargs(), dn = gargs();
    gu.A = w.A; gu.lda = d; gu.a_rows = w.perm;
    gu.W = L.w_gate; gu.W2 = L.w_up; gu.ldw = d; gu.w_group_stride = (int64_t)F * d;
    gu.w_scale = (const uint16_t*)L.gate_scale; gu.w2_scale = (const uint16_t*)L.up_scale; gu.scale_group_stride = F;
    gu.M = n; gu.N = 2 * F; gu.K = d; gu.group_offsets = w.offsets;
    gu.C = w.Hbuf; gu.ldc = F; gu.c_f32 = f32; gu.state = state;
    dn.A = w.Hbuf; dn.lda = F;
    dn.W = L.w_down; dn.ldw = F; dn.w_group_stride = (int64_t)d * F;
    dn.w_scale = (const uint16_t*)L.down_scale; dn.scale_group_stride = d;
    dn.M = n; dn.N = d; dn.K = F; dn.group_offsets = w.offsets;
    dn.C = w.Y; dn.ldc = d; dn.c_f32 = 1; dn.state = state;
    const bool tiled = dg::tile_gemm_supported(gu, f32, fp8, dg::EPI_SWIGLU) &&
                       dg::tile_gemm_supported(dn, f32, fp8, dg::EPI_STORE_F32);
    const int big_min = tiled ? DG_TILE_MIN_ROWS : 0;
    DG_TRY(dg::launch_hist_permute(w.ids, n, k, E, w.offsets, w.perm, w.slot_of, w.hit, w.hit_mb, w.hitB, w.hitB_mb,
                                   big_min, w.experts_hit ? w.experts_hit + l : nullptr, state, st),
           "hist permute");
    const int small_rows = tiled ? 64 : n;  // bound on the rows of a stream-GEMM group
    {   // gate/up with SwiGLU; products split over K leave partials for one reduce
        const int slot = timing_begin(st, DG_TIME_EXPERT_GATE_UP);
        const int ks_small = tiled && w.gu_part ? small_ksplit(c) : 1;
        const int ks_big = tiled && w.gu_part ? dg::tile_grouped_ksplit(n) : 1;
        dg::GemmArgs g = gu;
        g.M = n * (k + 1);  // slots: the rows of the partials
        g.part = w.gu_part;
        g.hit = w.hit; g.hit_mb = w.hit_mb; g.ksplit = ks_small;
        DG_TRY(dg::stream_gemm_launch(g, f32, fp8, dg::EPI_SWIGLU, E + 1, small_rows, st), "expert gate/up");
        if (tiled) {
            g.hit = w.hitB; g.hit_mb = w.hitB_mb; g.ksplit = ks_big;
            DG_TRY(dg::tile_gemm_launch(g, dg::EPI_SWIGLU, E + 1, n, st), "expert gate/up (tiled)");
        }
        if (ks_small > 1 || ks_big > 1)
            DG_TRY(dg::swiglu_reduce_launch(g, E + 1, big_min, ks_big, ks_small, st), "swiglu reduce");
        timing_end(slot, st);
    }
    {   // down
        const int slot = timing_begin(st, DG_TIME_EXPERT_DOWN);
        dg::GemmArgs g = dn;
        g.hit = w.hit; g.hit_mb = w.hit_mb;
        DG_TRY(dg::stream_gemm_launch(g, f32, fp8, dg::EPI_STORE_F32, E + 1, small_rows, st), "expert down");
        if (tiled) {
            g.hit = w.hitB; g.hit_mb = w.hitB_mb;
            DG_TRY(dg::tile_gemm_launch(g, dg::EPI_STORE_F32, E + 1, n, st), "expert down (tiled)");
        }
        timing_end(slot, st);
    }
    DG_TRY(dg::launch_combine(w.X, n, d, w.Y, w.slot_of, w.gates, k, n * k, next_norm, c.norm_eps, w.A, f32, state,
                              st, next_lo && !f32 ? w.A_lo : nullptr),
           "combine");
    return DG_OK;
}

int attn_splits(const dg_config& c, int nq, int64_t keys) {
    return dg::attention_splits(nq, keys, c.n_q_heads, c.n_kv_heads, c.head_dim, c.act_dtype == DG_F32, MAX_SPLITS,
                                MAX_SPLITS * SPLIT_ROWS);
}

// ---------------------------------------------------------------------------
// Decoder layer over the canvas rows X[0..n) at positions P..P+n-1.
// ---------------------------------------------------------------------------
// With normed_in, w.A already holds rmsnorm(X) with this layer's attention
// norm; next_norm (or NULL) is normalised into w.A by the closing combine.
// One canvas of a step: rows [row0, row0 + n) of the work buffers (row0 a
// multiple of 64 when there are several), attending its own cache.
struct Seg {
    int row0, n;
    const dg_kv* kv;
};

dg_status decoder_layer(const dg_model* m, int l, const Work& w, int n, const Seg* segs, int nseg,
                        const int32_t* state, bool normed_in, const float* next_norm, hipStream_t st,
                        bool next_lo = false) {
    const dg_config& c = m->cfg;
    const dg_layer_weights& L = m->layers[l];
    const int d = c.d_model, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
    const int f32 = c.act_dtype == DG_F32, fp8 = c.weight_dtype == DG_FP8_E4M3;
    const size_t ab = act_bytes(c);
    if (!normed_in) DG_TRY(dg::launch_rmsnorm(w.X, n, d, L.attn_norm, c.norm_eps, w.A, f32, state, st), "rmsnorm");
    int qkv_parts = 1, o_parts = 1;
    {
        dg::GemmArgs g = gargs();
        g.A = w.A; g.lda = d; g.W = L.wqkv; g.ldw = d; g.w_scale = (const uint16_t*)L.wqkv_scale;
        g.M = n; g.N = (Hq + 2 * Hkv) * hd; g.K = d; g.C = w.QKV; g.ldc = g.N; g.state = state;
        const int slot = timing_begin(st, DG_TIME_QKV);
        DG_TRY(dense_gemm(g, w, f32, fp8, f32 ? dg::EPI_STORE_F32 : dg::EPI_STORE_BF16, st, &qkv_parts), "qkv gemm");
        timing_end(slot, st);
    }
    DG_TRY(dg::launch_rope_scatter(w.QKV, w.gemm_part, qkv_parts, f32, n, Hq, Hkv, hd, w.rope_cs, w.Q, w.rows, 0,
                                   w.Kc, w.Vc, w.rows64, 0, w.rows64, state, st),
           "rope");
    for (int s = 0; s < nseg; ++s) {
        // canvas s: its query rows and canvas K/V rows, its cache
        const Seg& sg = segs[s];
        const int64_t P = sg.kv->len;
        dg::AttnArgs a;
        memset(&a, 0, sizeof a);
        a.Q = (char*)w.Q + (size_t)sg.row0 * hd * ab; a.ldq = w.rows; a.nq = sg.n; a.qpos0 = P;
        a.K1 = sg.kv->k[l]; a.V1 = sg.kv->v[l]; a.ld1 = sg.kv->capacity;
        a.s1 = is_global(c, l) ? 0 : std::max<int64_t>(0, P - c.window);
        a.e1 = P;
        a.K2 = (char*)w.Kc + (size_t)sg.row0 * hd * ab; a.V2 = (char*)w.Vc + (size_t)sg.row0 * ab;
        a.ld2 = w.rows64; a.n2 = sg.n; a.pos2_0 = P;
        a.Hq = Hq; a.Hkv = Hkv; a.hd = hd; a.causal = 0; a.window = 0;
        a.O = (char*)w.O + (size_t)sg.row0 * Hq * hd * ab; a.part_o = w.part_o; a.part_ml = w.part_ml;
        a.splits = attn_splits(c, sg.n, (a.e1 - a.s1) + sg.n);
        a.state = state;
        const int slot = timing_begin(st, DG_TIME_ATTENTION);
        DG_TRY(dg::launch_attention(a, f32, st), "attention");
        timing_end(slot, st);
    }
    {
        dg::GemmArgs g = gargs();
        g.A = w.O; g.lda = Hq * hd; g.W = L.wo; g.ldw = Hq * hd; g.w_scale = (const uint16_t*)L.wo_scale;
        g.M = n; g.N = d; g.K = Hq * hd; g.X = w.X; g.ldx = d; g.state = state;
        const int slot = timing_begin(st, DG_TIME_O_PROJ);
        DG_TRY(dense_gemm(g, w, f32, fp8, dg::EPI_RESIDUAL, st, &o_parts), "o gemm");
        timing_end(slot, st);
    }
    return moe_block(m, l, w, n, next_norm, state, st, o_parts, next_lo);
}

// ---------------------------------------------------------------------------
// Encoder over one chunk of n tokens at positions P..P+n-1 (X holds their
// embeddings); every layer's K/V rows are written into the cache.
// ---------------------------------------------------------------------------
dg_status encoder_chunk(const dg_model* m, const Work& w, int n, const dg_kv* kv, int64_t P, hipStream_t st) {
    const dg_config& c = m->cfg;
    const int d = c.d_model, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
    const int f32 = c.act_dtype == DG_F32, fp8 = c.weight_dtype == DG_FP8_E4M3;
    DG_TRY(dg::launch_rope_table(n, hd, P, c.rope_base, w.rope_cs, nullptr, st), "rope table");
    for (int l = 0; l < c.n_layers; ++l) {
        const dg_layer_weights& L = m->layers[l];
        if (l == 0) DG_TRY(dg::launch_rmsnorm(w.X, n, d, L.attn_norm, c.norm_eps, w.A, f32, nullptr, st), "rmsnorm");
        dg::GemmArgs g = gargs();
        g.A = w.A; g.lda = d; g.W = L.wqkv; g.ldw = d; g.w_scale = (const uint16_t*)L.wqkv_scale;
        g.M = n; g.N = (Hq + 2 * Hkv) * hd; g.K = d; g.C = w.QKV; g.ldc = g.N;
        int qkv_parts = 1;
        int slot = timing_begin(st, DG_TIME_QKV);
        DG_TRY(dense_gemm(g, w, f32, fp8, f32 ? dg::EPI_STORE_F32 : dg::EPI_STORE_BF16, st, &qkv_parts), "qkv gemm");
        timing_end(slot, st);
        DG_TRY(dg::launch_rope_scatter(w.QKV, w.gemm_part, qkv_parts, f32, n, Hq, Hkv, hd, w.rope_cs, w.Q, w.rows, 0,
                                       kv->k[l], kv->v[l], kv->capacity, P, 0, nullptr, st),
               "rope");
        if (l == c.n_layers - 1) break;  // nothing in the cache depends on the rest
        dg::AttnArgs a;
        memset(&a, 0, sizeof a);
        a.Q = w.Q; a.ldq = w.rows; a.nq = n; a.qpos0 = P;
        a.K1 = kv->k[l]; a.V1 = kv->v[l]; a.ld1 = kv->capacity; a.s1 = 0; a.e1 = P + n;
        a.Hq = Hq; a.Hkv = Hkv; a.hd = hd; a.causal = 1;
        a.window = is_global(c, l) ? 0 : c.window;
        a.O = w.O; a.part_o = w.part_o; a.part_ml = w.part_ml;
        int64_t span = a.window > 0 ? std::min<int64_t>(P + n, (int64_t)a.window + 64) : P + n;
        a.splits = attn_splits(c, n, span);
        slot = timing_begin(st, DG_TIME_ATTENTION);
        DG_TRY(dg::launch_attention(a, f32, st), "attention");
        timing_end(slot, st);
        dg::GemmArgs go = gargs();
        go.A = w.O; go.lda = Hq * hd; go.W = L.wo; go.ldw = Hq * hd; go.w_scale = (const uint16_t*)L.wo_scale;
        go.M = n; go.N = d; go.K = Hq * hd; go.X = w.X; go.ldx = d;
        slot = timing_begin(st, DG_TIME_O_PROJ);
        DG_TRY(dense_gemm(go, w, f32, fp8, dg::EPI_RESIDUAL, st), "o gemm");
        timing_end(slot, st);
        // the next layer's attention norm rides on this layer's combine
        if (dg_status s = moe_block(m, l, w, n, m->layers[l + 1].attn_norm, nullptr, st)) return s;
    }
    return DG_OK;
}

dg_status lm_head(const dg_model* m, const Work& w, int n, const dg::SamplerParams& sp, int step_override,
                  const int32_t* state, const int32_t* bias_tok, const float* bias_val, dg_step_stats* stats,
                  bool normed_in, hipStream_t st, int32_t* gtok = nullptr) {
    const dg_config& c = m->cfg;
    const int f32 = c.act_dtype == DG_F32;
    // bf16: the final-normed rows as hi + lo pairs (w.A, w.A_lo), written by
    // the last layer's combine when normed_in
    if (!normed_in)
        DG_TRY(dg::launch_rmsnorm(w.X, n, c.d_model, m->final_norm, c.norm_eps, w.A, f32, state, st,
                                  f32 ? nullptr : w.A_lo),
               "final norm");
    dg::GemmArgs g = gargs();
    g.A = w.A; g.A2 = f32 ? nullptr : w.A_lo; g.lda = c.d_model; g.W = m->lm8 ? m->lm8 : m->embed;
    g.ldw = c.d_model;
    g.w_scale = m->lm8_scale;
    g.M = n; g.N = c.vocab; g.K = c.d_model;
    g.C = stats->logits; g.ldc = stats->logits_ld; g.c_f32 = f32;
    g.parts = w.parts; g.nsplit = lm_nsplit(c);
    g.state = state; g.step_override = step_override; g.sp = sp; g.mask_id = c.mask_id;
    g.bias_tok = bias_tok; g.bias_val = bias_val;
    int slot = timing_begin(st, DG_TIME_LM_HEAD);
    if (!f32 && dg::lmhead_supported(g))
        DG_TRY(dg::lmhead_launch(g, st), "lm head");
    else if (m->lm8 || sp.draw_mode)
        return fail(DG_E_UNSUPPORTED, "e4m3 LM head or Gumbel-max draws: shape outside the LM-head kernel");
    else
        DG_TRY(dg::gemm_launch(g, f32, 0, dg::EPI_LMHEAD, 0, dg::SHAPE_PROJ, st), "lm head");
    timing_end(slot, st);
    DG_TRY(dg::launch_merge_rows(w.parts, n, lm_nsplit(c), state, stats->entropy, stats->lse, stats->argmax,
                                 sp.draw_mode ? gtok : nullptr, st),
           "merge rows");
    return DG_OK;
}

dg_status check_kv(const dg_model* m, const dg_kv* kv) {
    if (!kv || !kv->k || !kv->v) return fail(DG_E_INVALID, "kv cache is NULL");
    if (kv->len < 0 || kv->capacity < kv->len) return fail(DG_E_INVALID, "kv len/capacity inconsistent");
    if (kv->capacity % 64) return fail(DG_E_SHAPE, "kv capacity must be a multiple of 64");
    if (kv->capacity > (int64_t)1 << 30) return fail(DG_E_SHAPE, "kv capacity above 2^30 rows");
    for (int l = 0; l < m->cfg.n_layers; ++l)
        if (!kv->k[l] || !kv->v[l]) return fail(DG_E_INVALID, "kv layer %d pointer is NULL", l);
    return DG_OK;
}

dg_status check_logits(const dg_model* m, const dg_step_stats* s, int n) {
    if (dg_status e = check_stats(s)) return e;
    if (!s->logits) return fail(DG_E_INVALID, "stats->logits is NULL");
    if (s->logits_ld < m->cfg.vocab) return fail(DG_E_SHAPE, "logits_ld < vocab");
    (void)n;
    return DG_OK;
}

// rows [0, n): no bias token
__global__ void no_bias_kernel(int32_t* tok, float* val, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        tok[i] = -1;
        val[i] = 0.f;
    }
}

dg_status ws_for(const dg_model* m, void* ws, size_t ws_bytes, int rows, Work* out) {
    if (!ws) return fail(DG_E_INVALID, "workspace is NULL");
    Work w = carve(m, ws, rows);
    if (w.bytes > ws_bytes) return fail(DG_E_CAPACITY, "workspace %zu bytes < %zu needed", ws_bytes, w.bytes);
    *out = w;
    return DG_OK;
}

}  // namespace

extern "C" {

dg_status dg_model_create(const dg_config* c, const dg_weights* w, dg_model** out) {
    if (!c || !w || !out) return fail(DG_E_INVALID, "NULL argument");
    *out = nullptr;
    if (c->n_layers < 1 || c->d_model < 32 || c->d_model % 32 || c->d_model > 4096)
        return fail(DG_E_SHAPE, "d_model must be a multiple of 32 in 32..4096");
    if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads)
        return fail(DG_E_SHAPE, "n_q_heads must be a positive multiple of n_kv_heads");
    if (c->act_dtype != DG_F32 && c->act_dtype != DG_BF16) return fail(DG_E_UNSUPPORTED, "act_dtype");
    if (c->weight_dtype == DG_F32 ? c->act_dtype != DG_F32 : c->act_dtype != DG_BF16)
        return fail(DG_E_UNSUPPORTED, "f32 weights need f32 activations; bf16/e4m3 weights need bf16");
    if (c->weight_dtype != DG_F32 && c->weight_dtype != DG_BF16 && c->weight_dtype != DG_FP8_E4M3)
        return fail(DG_E_UNSUPPORTED, "weight_dtype");
    const int hd = c->head_dim;
    if (!(hd == 64 || hd == 128 || (hd == 256 && c->act_dtype == DG_BF16)))
        return fail(DG_E_UNSUPPORTED, "head_dim must be 64 or 128 (f32) / 64, 128 or 256 (bf16)");
    if (c->n_experts < 1 || c->n_experts > 512) return fail(DG_E_SHAPE, "n_experts outside 1..512");
    if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts) return fail(DG_E_SHAPE, "top_k outside 1..min(16, E)");
    if (c->ffn_hidden < 32 || c->ffn_hidden % 32) return fail(DG_E_SHAPE, "ffn_hidden must be a multiple of 32");
    if (c->vocab < 8 || c->vocab % 8) return fail(DG_E_SHAPE, "vocab must be a multiple of 8");
    if (c->mask_id < 0 || c->mask_id >= c->vocab) return fail(DG_E_INVALID, "mask_id outside the vocabulary");
    if (c->max_canvas < 1 || c->max_canvas > 1024) return fail(DG_E_SHAPE, "max_canvas outside 1..1024");
    if (dg::hist_permute_max_rows(c->top_k, c->n_experts) < c->max_canvas)
        return fail(DG_E_UNSUPPORTED, "max_canvas x top_k routed rows exceed the expert permutation's capacity");
    if (c->window < 0 || c->global_every < 0) return fail(DG_E_INVALID, "window/global_every must be >= 0");
    if (!(c->rope_base > 1.f) || !(c->norm_eps >= 0.f)) return fail(DG_E_INVALID, "rope_base/norm_eps");
    if (!w->embed || !w->final_norm || !w->layers) return fail(DG_E_INVALID, "weight pointer is NULL");
    auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    if (!a16(w->embed) || !a16(w->final_norm)) return fail(DG_E_INVALID, "weights must be 16-byte aligned");
    if ((w->lm_head_e4m3 == nullptr) != (w->lm_head_scale == nullptr))
        return fail(DG_E_INVALID, "lm_head_e4m3 and lm_head_scale must both be set or both NULL");
    if (w->lm_head_e4m3 && (c->act_dtype != DG_BF16 || !a16(w->lm_head_e4m3)))
        return fail(DG_E_UNSUPPORTED, "an e4m3 LM head needs bf16 activations and 16-byte alignment");
    const bool fp8 = c->weight_dtype == DG_FP8_E4M3;
    for (int l = 0; l < c->n_layers; ++l) {
        const dg_layer_weights& L = w->layers[l];
        if (!L.attn_norm || !L.moe_norm || !L.wqkv || !L.wo || !L.router || !L.router_bias || !L.w_gate ||
            !L.w_up || !L.w_down)
            return fail(DG_E_INVALID, "layer %d: weight pointer is NULL", l);
        if (!a16(L.attn_norm) || !a16(L.moe_norm) || !a16(L.wqkv) || !a16(L.wo) || !a16(L.router) ||
            !a16(L.w_gate) || !a16(L.w_up) || !a16(L.w_down))
            return fail(DG_E_INVALID, "layer %d: weights must be 16-byte aligned", l);
        if (fp8 && (!L.wqkv_scale || !L.wo_scale || !L.gate_scale || !L.up_scale || !L.down_scale))
            return fail(DG_E_INVALID, "layer %d: e4m3 weights need scales", l);
    }
    dg_model* m = new (std::nothrow) dg_model;
    if (!m) return fail(DG_E_INVALID, "out of host memory");
    m->cfg = *c;
    m->embed = w->embed;
    m->lm8 = w->lm_head_e4m3;
    m->lm8_scale = (const uint16_t*)w->lm_head_scale;
    m->final_norm = w->final_norm;
    m->layers.assign(w->layers, w->layers + c->n_layers);
    *out = m;
    return DG_OK;
}

void dg_model_destroy(dg_model* m) { delete m; }

size_t dg_workspace_bytes(const dg_model* m, int32_t max_rows) {
    if (!m || max_rows < 1 || max_rows > 4096) return 0;
    // the split-K partials make the need non-monotonic in the row count
    size_t best = 0;
    for (int T = 1; T <= max_rows; ++T) best = std::max(best, carve(m, nullptr, T).bytes);
    return best;
}

dg_status dg_embed(const dg_model* m, const int32_t* tokens, int32_t n, float* X, void* stream) {
    if (!m || !tokens || !X) return fail(DG_E_INVALID, "NULL argument");
    if (n < 1) return fail(DG_E_SHAPE, "n must be >= 1");
    return hip_check(dg::launch_embed(m->embed, m->cfg.act_dtype == DG_F32, m->cfg.d_model, m->cfg.vocab, tokens, n, X,
                                      nullptr, (hipStream_t)stream),
                     "embed");
}

dg_status dg_decoder_layer(const dg_model* m, int32_t layer, float* X, int32_t n, const dg_kv* kv,
                           int32_t* route_ids, float* route_gates, void* ws, size_t ws_bytes, void* stream) {
    if (!m || !X) return fail(DG_E_INVALID, "NULL argument");
    if (layer < 0 || layer >= m->cfg.n_layers) return fail(DG_E_INVALID, "layer out of range");
    if (n < 1 || n > m->cfg.max_canvas) return fail(DG_E_SHAPE, "n outside 1..max_canvas");
    if (dg_status s = check_kv(m, kv)) return s;
    Work w;
    if (dg_status s = ws_for(m, ws, ws_bytes, n, &w)) return s;
    hipStream_t st = (hipStream_t)stream;
    const size_t xb = (size_t)n * m->cfg.d_model * sizeof(float);
    DG_TRY(hipMemcpyAsync(w.X, X, xb, hipMemcpyDeviceToDevice, st), "copy X in");
    DG_TRY(dg::launch_rope_table(n, m->cfg.head_dim, kv->len, m->cfg.rope_base, w.rope_cs, nullptr, st), "rope table");
    const Seg seg{0, n, kv};
    if (dg_status s = decoder_layer(m, layer, w, n, &seg, 1, nullptr, false, nullptr, st)) return s;
    DG_TRY(hipMemcpyAsync(X, w.X, xb, hipMemcpyDeviceToDevice, st), "copy X out");
    const size_t kb = (size_t)n * m->cfg.top_k;
    if (route_ids) DG_TRY(hipMemcpyAsync(route_ids, w.ids, kb * 4, hipMemcpyDeviceToDevice, st), "copy ids");
    if (route_gates) DG_TRY(hipMemcpyAsync(route_gates, w.gates, kb * 4, hipMemcpyDeviceToDevice, st), "copy gates");
    return DG_OK;
}

dg_status dg_lm_head(const dg_model* m, const float* X, int32_t n, const dg_sampler_cfg* scfg, int32_t step_idx,
                     const int32_t* bias_tok, const float* bias_val, dg_step_stats* stats, void* ws,
                     size_t ws_bytes, void* stream) {
    if (!m || !X) return fail(DG_E_INVALID, "NULL argument");
    if (dg_status s = check_sampler_cfg(scfg)) return s;
    if (n < 1 || n > m->cfg.max_canvas) return fail(DG_E_SHAPE, "n outside 1..max_canvas");
    if (step_idx < 0 || step_idx >= scfg->max_steps) return fail(DG_E_INVALID, "step_idx out of range");
    if ((bias_tok == nullptr) != (bias_val == nullptr)) return fail(DG_E_INVALID, "bias pointers");
    if (dg_status s = check_logits(m, stats, n)) return s;
    Work w;
    if (dg_status s = ws_for(m, ws, ws_bytes, n, &w)) return s;
    hipStream_t st = (hipStream_t)stream;
    DG_TRY(hipMemcpyAsync(w.X, X, (size_t)n * m->cfg.d_model * 4, hipMemcpyDeviceToDevice, st), "copy X");
    return lm_head(m, w, n, to_params(scfg), step_idx, nullptr, bias_tok, bias_val, stats, false, st);
}

dg_status dg_prefill_append(const dg_model* m, dg_kv* kv, const int32_t* tokens, int32_t n, void* ws,
                            size_t ws_bytes, void* stream) {
    if (!m || !tokens) return fail(DG_E_INVALID, "NULL argument");
    if (dg_status s = check_kv(m, kv)) return s;
    if (n < 0) return fail(DG_E_SHAPE, "n must be >= 0");
    if (kv->len + n > kv->capacity) return fail(DG_E_CAPACITY, "kv cache capacity %lld < %lld", (long long)kv->capacity,
                                                (long long)(kv->len + n));
    if (n == 0) return DG_OK;
    if (!ws) return fail(DG_E_INVALID, "workspace is NULL");
    // chunk rows: what the workspace holds, at most 4096 and at most what the
    // expert permutation takes in one pass (a multiple of 256 when larger)
    int cap = std::min(dg::hist_permute_max_rows(m->cfg.top_k, m->cfg.n_experts), 4096);
    if (cap >= 256) cap -= cap % 256;
    const int T = rows_fitting(m, ws_bytes, std::min(n, cap));
    if (T < 1) return fail(DG_E_CAPACITY, "workspace too small for one row");
    Work w = carve(m, ws, T);
    hipStream_t st = (hipStream_t)stream;
    int64_t P = kv->len;
    for (int off = 0; off < n; off += T) {
        const int cn = std::min(T, n - off);
        DG_TRY(dg::launch_embed(m->embed, m->cfg.act_dtype == DG_F32, m->cfg.d_model, m->cfg.vocab, tokens + off, cn,
                                w.X, nullptr, st),
               "embed");
        if (dg_status s = encoder_chunk(m, w, cn, kv, P, st)) return s;
        P += cn;
    }
    kv->len = P;
    return DG_OK;
}

dg_status dg_canvas_step(const dg_model* m, dg_canvas* canvas, const dg_kv* kv, int32_t step_idx, uint64_t seed,
                         const dg_sampler_cfg* scfg, dg_step_stats* stats, void* ws, size_t ws_bytes,
                         void* stream) {
    if (!m) return fail(DG_E_INVALID, "model is NULL");
    if (dg_status s = check_sampler_cfg(scfg)) return s;
    if (!canvas) return fail(DG_E_INVALID, "canvas is NULL");
    const int n = canvas->n;
    if (n < 1 || n > m->cfg.max_canvas) return fail(DG_E_SHAPE, "canvas n outside 1..max_canvas");
    if (dg_status s = check_canvas(canvas, n)) return s;
    if (dg_status s = check_kv(m, kv)) return s;
    if (dg_status s = check_logits(m, stats, n)) return s;
    if (step_idx < -1 || step_idx >= scfg->max_steps) return fail(DG_E_INVALID, "step_idx out of range");
    if (scfg->draw_mode == DG_DRAW_GUMBEL_MAX && m->cfg.act_dtype != DG_BF16)
        return fail(DG_E_UNSUPPORTED, "Gumbel-max draws need bf16 activations");
    Work w;
    if (dg_status s = ws_for(m, ws, ws_bytes, n, &w)) return s;
    w.experts_hit = stats->experts_hit;
    hipStream_t st = (hipStream_t)stream;
    dg::SamplerParams sp = to_params(scfg);
    sp.seed_lo = (uint32_t)(seed & 0xffffffffu);
    sp.seed_hi = (uint32_t)(seed >> 32);
    sp.canvas_idx = canvas->canvas_idx;
    const dg_config& c = m->cfg;
    DG_TRY(dg::launch_embed(m->embed, c.act_dtype == DG_F32, c.d_model, c.vocab, canvas->tokens, n, w.X, canvas->state, st),
           "embed");
    DG_TRY(dg::launch_rope_table(n, c.head_dim, kv->len, c.rope_base, w.rope_cs, canvas->state, st), "rope table");
    for (int l = 0; l < c.n_layers; ++l) {
        const float* next = l + 1 < c.n_layers ? m->layers[l + 1].attn_norm : m->final_norm;
        const Seg seg{0, n, kv};
        if (dg_status s = decoder_layer(m, l, w, n, &seg, 1, canvas->state, l > 0, next, st, l + 1 == c.n_layers))
            return s;
    }
    if (dg_status s = lm_head(m, w, n, sp, step_idx, canvas->state, canvas->bias_tok, canvas->bias_val, stats, true,
                              st, w.gtok))
        return s;
    return hip_check(dg::launch_sampler_tail(stats->logits, c.act_dtype == DG_F32, stats->logits_ld, n, c.vocab,
                                             c.mask_id, canvas->bias_tok, canvas->bias_val, stats->entropy,
                                             stats->argmax, canvas->state, step_idx, sp, seed, canvas->canvas_idx,
                                             canvas->tokens, canvas->committed, canvas->prev_argmax, stats->selected,
                                             w.sel_list, w.chunk_sum, w.gtok, stats->mean_entropy, st),
                     "sampler tail");
}

dg_status dg_generate_canvas(const dg_model* m, dg_canvas* canvas, dg_kv* kv, const dg_sampler_cfg* scfg,
                             uint64_t seed, int32_t append_after, int32_t poll_every, dg_step_stats* stats,
                             int32_t* steps_taken, void* ws, size_t ws_bytes, void* stream) {
    if (!m || !canvas || !steps_taken) return fail(DG_E_INVALID, "NULL argument");
    if (dg_status s = check_sampler_cfg(scfg)) return s;
    if (poll_every < 1) return fail(DG_E_INVALID, "poll_every must be >= 1");
    if (dg_status s = check_canvas(canvas, canvas->n)) return s;
    if (dg_status s = check_kv(m, kv)) return s;
    if (append_after && kv->len + canvas->n > kv->capacity) return fail(DG_E_CAPACITY, "kv cache full");
    hipStream_t st = (hipStream_t)stream;
    if (dg_status s = dg_canvas_reset(canvas, m->cfg.mask_id, stream)) return s;
    int32_t hstate[DG_STATE_WORDS] = {0};
    for (int t = 0; t < scfg->max_steps; ++t) {
        if (dg_status s = dg_canvas_step(m, canvas, kv, t, seed, scfg, stats, ws, ws_bytes, stream)) return s;
        if ((t + 1) % poll_every == 0 || t + 1 == scfg->max_steps) {
            DG_TRY(hipMemcpyAsync(hstate, canvas->state, sizeof hstate, hipMemcpyDeviceToHost, st), "read state");
            DG_TRY(hipStreamSynchronize(st), "sync");
            if (hstate[DG_ST_DONE]) break;
        }
    }
    DG_TRY(hipMemcpyAsync(hstate, canvas->state, sizeof hstate, hipMemcpyDeviceToHost, st), "read state");
    DG_TRY(hipStreamSynchronize(st), "sync");
    *steps_taken = hstate[DG_ST_STEP];
    if (append_after) {
        if (dg_status s = dg_prefill_append(m, kv, canvas->tokens, canvas->n, ws, ws_bytes, stream)) return s;
    }
    return DG_OK;
}

dg_status dg_canvas_step_batch(const dg_model* m, dg_canvas* canvases, const dg_kv* kvs, int32_t nb, int32_t step_idx,
                               uint64_t seed, const dg_sampler_cfg* scfg, dg_step_stats* stats, void* ws,
                               size_t ws_bytes, void* stream) {
    if (!m || !canvases || !kvs) return fail(DG_E_INVALID, "NULL argument");
    if (nb < 1 || nb > 64) return fail(DG_E_SHAPE, "batch of %d canvases outside 1..64", nb);
    if (dg_status s = check_sampler_cfg(scfg)) return s;
    if (step_idx < 0 || step_idx >= scfg->max_steps) return fail(DG_E_INVALID, "step_idx out of range");
    if (scfg->draw_mode != DG_DRAW_INVERSE_CDF) return fail(DG_E_UNSUPPORTED, "batches draw by inverse CDF");
    const dg_config& c = m->cfg;
    Seg segs[64];
    int rows = 0;
    bool any_bias = false;
    for (int b = 0; b < nb; ++b) {
        const int n = canvases[b].n;
        if (n < 1) return fail(DG_E_SHAPE, "canvas %d: n must be >= 1", b);
        if (nb > 1 && n % 64) return fail(DG_E_SHAPE, "canvas %d: n=%d is not a multiple of 64", b, n);
        if (dg_status s = check_canvas(&canvases[b], n)) return s;
        if (dg_status s = check_kv(m, &kvs[b])) return s;
        segs[b] = Seg{rows, n, &kvs[b]};
        rows += n;
        any_bias |= canvases[b].bias_tok != nullptr;
    }
    if (rows > c.max_canvas) return fail(DG_E_SHAPE, "%d batch rows exceed max_canvas %d", rows, c.max_canvas);
    if (dg_status s = check_logits(m, stats, rows)) return s;
    if (!stats->mean_entropy) return fail(DG_E_INVALID, "stats->mean_entropy is NULL");
    Work w;
    if (dg_status s = ws_for(m, ws, ws_bytes, rows, &w)) return s;
    w.experts_hit = stats->experts_hit;
    hipStream_t st = (hipStream_t)stream;
    const dg::SamplerParams sp = to_params(scfg);
    const int f32 = c.act_dtype == DG_F32;
    for (int b = 0; b < nb; ++b) {
        const Seg& sg = segs[b];
        DG_TRY(dg::launch_embed(m->embed, f32, c.d_model, c.vocab, canvases[b].tokens, sg.n,
                                w.X + (size_t)sg.row0 * c.d_model, nullptr, st),
               "embed");
        DG_TRY(dg::launch_rope_table(sg.n, c.head_dim, sg.kv->len, c.rope_base, w.rope_cs + (size_t)sg.row0 * c.head_dim,
                                     nullptr, st),
               "rope table");
    }
    if (any_bias) {
        no_bias_kernel<<<(rows + 255) / 256, 256, 0, st>>>(w.bias_tok, w.bias_val, rows);
        DG_TRY(hipGetLastError(), "bias fill");
        for (int b = 0; b < nb; ++b) {
            if (!canvases[b].bias_tok) continue;
            const Seg& sg = segs[b];
            DG_TRY(hipMemcpyAsync(w.bias_tok + sg.row0, canvases[b].bias_tok, (size_t)sg.n * 4,
                                  hipMemcpyDeviceToDevice, st),
                   "bias tokens");
            DG_TRY(hipMemcpyAsync(w.bias_val + sg.row0, canvases[b].bias_val, (size_t)sg.n * 4,
                                  hipMemcpyDeviceToDevice, st),
                   "bias values");
        }
    }
    for (int l = 0; l < c.n_layers; ++l) {
        const float* next = l + 1 < c.n_layers ? m->layers[l + 1].attn_norm : m->final_norm;
        if (dg_status s = decoder_layer(m, l, w, rows, segs, nb, nullptr, l > 0, next, st, l + 1 == c.n_layers))
            return s;
    }
    if (dg_status s = lm_head(m, w, rows, sp, step_idx, nullptr, any_bias ? w.bias_tok : nullptr,
                              any_bias ? w.bias_val : nullptr, stats, true, st))
        return s;
    const size_t lb = (size_t)stats->logits_ld * act_bytes(c);
    for (int b = 0; b < nb; ++b) {
        const Seg& sg = segs[b];
        dg_canvas& cv = canvases[b];
        DG_TRY(dg::launch_sampler_tail((const char*)stats->logits + sg.row0 * lb, f32, stats->logits_ld, sg.n, c.vocab,
                                       c.mask_id, cv.bias_tok, cv.bias_val, stats->entropy + sg.row0,
                                       stats->argmax + sg.row0, cv.state, step_idx, sp, seed, cv.canvas_idx,
                                       cv.tokens, cv.committed, cv.prev_argmax, stats->selected + sg.row0,
                                       w.sel_list, w.chunk_sum, nullptr, stats->mean_entropy + b, st),
               "sampler tail");
    }
    return DG_OK;
}

dg_status dg_generate_batch(const dg_model* m, dg_canvas* canvases, dg_kv* kvs, int32_t nb, const dg_sampler_cfg* scfg,
                            uint64_t seed, int32_t append_after, int32_t poll_every, dg_step_stats* stats,
                            int32_t* steps_taken, void* ws, size_t ws_bytes, void* stream) {
    if (!m || !canvases || !kvs || !steps_taken) return fail(DG_E_INVALID, "NULL argument");
    if (nb < 1 || nb > 64) return fail(DG_E_SHAPE, "batch of %d canvases outside 1..64", nb);
    if (dg_status s = check_sampler_cfg(scfg)) return s;
    if (poll_every < 1) return fail(DG_E_INVALID, "poll_every must be >= 1");
    for (int b = 0; b < nb; ++b) {
        if (dg_status s = check_canvas(&canvases[b], canvases[b].n)) return s;
        if (dg_status s = check_kv(m, &kvs[b])) return s;
        if (append_after && kvs[b].len + canvases[b].n > kvs[b].capacity)
            return fail(DG_E_CAPACITY, "canvas %d: kv cache full", b);
    }
    hipStream_t st = (hipStream_t)stream;
    for (int b = 0; b < nb; ++b)
        if (dg_status s = dg_canvas_reset(&canvases[b], m->cfg.mask_id, stream)) return s;
    std::vector<int32_t> hstate((size_t)nb * DG_STATE_WORDS);
    for (int t = 0; t < scfg->max_steps; ++t) {
        if (dg_status s = dg_canvas_step_batch(m, canvases, kvs, nb, t, seed, scfg, stats, ws, ws_bytes, stream))
            return s;
        if ((t + 1) % poll_every == 0 || t + 1 == scfg->max_steps) {
            for (int b = 0; b < nb; ++b)
                DG_TRY(hipMemcpyAsync(&hstate[(size_t)b * DG_STATE_WORDS], canvases[b].state,
                                      DG_STATE_WORDS * sizeof(int32_t), hipMemcpyDeviceToHost, st),
                       "read state");
            DG_TRY(hipStreamSynchronize(st), "sync");
            bool all = true;
            for (int b = 0; b < nb; ++b) all &= hstate[(size_t)b * DG_STATE_WORDS + DG_ST_DONE] != 0;
            if (all) break;
        }
    }
    for (int b = 0; b < nb; ++b)
        DG_TRY(hipMemcpyAsync(&hstate[(size_t)b * DG_STATE_WORDS], canvases[b].state, DG_STATE_WORDS * sizeof(int32_t),
                              hipMemcpyDeviceToHost, st),
               "read state");
    DG_TRY(hipStreamSynchronize(st), "sync");
    for (int b = 0; b < nb; ++b) steps_taken[b] = hstate[(size_t)b * DG_STATE_WORDS + DG_ST_STEP];
    if (append_after)
        for (int b = 0; b < nb; ++b)
            if (dg_status s = dg_prefill_append(m, &kvs[b], canvases[b].tokens, canvases[b].n, ws, ws_bytes, stream))
                return s;
    return DG_OK;
}

struct dg_step_graph {
    hipStream_t cap = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

void dg_step_graph_destroy(dg_step_graph* g) {
    if (!g) return;
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    if (g->cap) (void)hipStreamDestroy(g->cap);
    delete g;
}

dg_status dg_step_graph_create(const dg_model* m, dg_canvas* canvas, const dg_kv* kv, const dg_sampler_cfg* scfg,
                               uint64_t seed, dg_step_stats* stats, void* ws, size_t ws_bytes, dg_step_graph** out) {
    if (!out) return fail(DG_E_INVALID, "out is NULL");
    *out = nullptr;
    dg_step_graph* g = new (std::nothrow) dg_step_graph;
    if (!g) return fail(DG_E_INVALID, "out of host memory");
    // a capture stream of its own (default priority)
    if (dg_status s = hip_check(hipStreamCreateWithFlags(&g->cap, hipStreamNonBlocking), "capture stream")) {
        dg_step_graph_destroy(g);
        return s;
    }
    if (dg_status s = hip_check(hipStreamBeginCapture(g->cap, hipStreamCaptureModeRelaxed), "begin capture")) {
        dg_step_graph_destroy(g);
        return s;
    }
    const dg_status st = dg_canvas_step(m, canvas, kv, -1, seed, scfg, stats, ws, ws_bytes, g->cap);
    const hipError_t e = hipStreamEndCapture(g->cap, &g->graph);
    if (st != DG_OK) {
        dg_step_graph_destroy(g);
        return st;
    }
    if (dg_status s = hip_check(e, "end capture")) {
        dg_step_graph_destroy(g);
        return s;
    }
    if (dg_status s = hip_check(hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0), "instantiate")) {
        dg_step_graph_destroy(g);
        return s;
    }
    *out = g;
    return DG_OK;
}

dg_status dg_step_graph_launch(dg_step_graph* g, void* stream) {
    if (!g || !g->exec) return fail(DG_E_INVALID, "graph is NULL");
    return hip_check(hipGraphLaunch(g->exec, (hipStream_t)stream), "graph launch");
}

}  // extern "C"
