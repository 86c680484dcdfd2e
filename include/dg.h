/*
 * dg.h - C ABI of the MI355X (gfx950) canvas denoising library (libdg.so).
 *
 * The library implements the block-autoregressive canvas denoising of
 * DiffusionGemma as described by its model cards:
 *   - DiffusionGemma model card (zh-TW, gemma.gh.miniasp.com), "模型總覽"
 *     (overview): an autoregressive encoder prefills the prompt into a KV
 *     cache; a decoder denoises a 256-token canvas with bidirectional
 *     attention and reads the cache through cross-attention; a fully
 *     denoised canvas is run through the encoder and appended to the cache
 *     before the next canvas starts. The spec table fixes 30 layers, a
 *     1024-token sliding window, 128 experts with 8 active plus 1 shared, a
 *     262K vocabulary and a canvas of 256.
 *   - the same card, best practice 1 "擴散取樣設定" (diffusion sampling
 *     settings): the Entropy-Bounded sampler (at most 48 steps, temperature
 *     0.8 -> 0.4 linear, entropy bound 0.1, full re-noising of unselected
 *     tokens, stop when the mean entropy is below 0.005 and the argmax is
 *     unchanged for 2 consecutive steps).
 *
 * Conventions for every entry point:
 *   - Device pointers are hipMalloc'd (or torch) memory owned by the caller;
 *     the library never allocates or frees device memory. Scratch comes from
 *     a caller-provided workspace of at least the size the matching
 *     *_workspace_bytes function returns.
 *   - Calls are asynchronous on the given HIP stream unless stated otherwise.
 *   - Every argument is validated on the host before anything is enqueued; a
 *     call that returns an error has enqueued nothing and modified nothing.
 *   - Errors are negative dg_status codes; dg_last_error() returns a
 *     thread-local message for the last failing call on this thread.
 *   - No C++ exception crosses this interface.
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16).
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dg_status;
#define DG_OK 0
#define DG_E_INVALID (-1)     /* null pointer or out-of-range scalar */
#define DG_E_SHAPE (-2)       /* inconsistent sizes */
#define DG_E_CAPACITY (-3)    /* KV cache or workspace too small */
#define DG_E_HIP (-4)         /* a HIP runtime call failed */
#define DG_E_UNSUPPORTED (-5) /* configuration outside what the kernels implement */

#define DG_F32 0
#define DG_BF16 1
#define DG_FP8_E4M3 2

#define DG_BOUND_SUM 0          /* sum of selected entropies <= bound */
#define DG_BOUND_SUM_MINUS_MAX 1 /* sum minus the largest selected entropy <= bound */

/* Commit modes. KEEP: candidates are the uncommitted positions and a commit is
 * final (the model cards' sampling settings, best practice 1: unselected
 * tokens are re-noised). RESELECT_ALL: the charlie27.com digest's section on
 * DiffusionGemma says outputs are corrected over the iterations; read as
 * every position being a candidate at every step, a selected position taking
 * a fresh draw, and every unselected position, committed before or not,
 * returning to mask_id with its commit cleared. */
#define DG_COMMIT_KEEP 0
#define DG_COMMIT_RESELECT_ALL 1

/* Draw modes of a committed token, both exact draws from softmax((L + bias) /
 * tau) without the MASK id. INVERSE_CDF: one Philox4x32-10 uniform per
 * (position, step, canvas) through the cumulative sum in vocabulary order, in
 * float64, by kernels that re-read the selected rows' logits.
 * GUMBEL_MAX: the lowest v maximising z_v - log(-log u_v), u_v = (top 23 bits
 * of Philox word v % 4 at counter (position, step, canvas, 1 + v / 4) + 1/2)
 * * 2^-23, float32, evaluated inside the statistics pass (the LM head
 * epilogue or the logit statistics), so no pass re-reads the logits. Model
 * steps support it with bf16 activations and one canvas per step. */
#define DG_DRAW_INVERSE_CDF 0
#define DG_DRAW_GUMBEL_MAX 1

/* Canvas state words (int32 device array of DG_STATE_WORDS). */
#define DG_STATE_WORDS 8
#define DG_ST_DONE 0        /* 1 once the canvas is finished */
#define DG_ST_STEP 1        /* index of the next step == steps taken */
#define DG_ST_COMMITTED 2   /* committed positions */
#define DG_ST_STABLE 3      /* consecutive steps with an unchanged argmax vector */
#define DG_ST_SELECTED 4    /* positions committed by the last step's EB selection */
#define DG_ST_STOP 5        /* 1 if the last step fired the adaptive stop */
#define DG_ST_FINISHED 6    /* 1 if the last step finished the canvas */

/* Sampler settings. dg_sampler_default() returns the model card's values
 * (best practice 1): 48 steps, 0.8 -> 0.4, bound 0.1, stop entropy 0.005,
 * 2 stable steps, DG_BOUND_SUM, DG_COMMIT_KEEP, DG_DRAW_INVERSE_CDF. */
typedef struct dg_sampler_cfg {
    int32_t max_steps;
    float temp_start;     /* temperatures in [1e-12, 3e38], else DG_E_INVALID */
    float temp_end;
    float bound;          /* nats */
    float stop_entropy;   /* nats, strict "<" */
    int32_t stable_steps; /* argmax vector unchanged over this many consecutive steps */
    int32_t bound_mode;   /* DG_BOUND_SUM or DG_BOUND_SUM_MINUS_MAX */
    int32_t commit_mode;  /* DG_COMMIT_KEEP or DG_COMMIT_RESELECT_ALL */
    int32_t draw_mode;    /* DG_DRAW_INVERSE_CDF or DG_DRAW_GUMBEL_MAX */
} dg_sampler_cfg;

/* One canvas. All pointers are device memory of n elements (state: 8).
 * An uncommitted position always holds mask_id between steps; under
 * DG_COMMIT_KEEP a commit is final.
 * bias_tok/bias_val (optional, both NULL or both set) add bias_val[i] to the
 * logit of token bias_tok[i] in row i before the temperature. */
typedef struct dg_canvas {
    int32_t* tokens;
    uint8_t* committed;
    int32_t* prev_argmax;
    int32_t* state;
    const int32_t* bias_tok;
    const float* bias_val;
    int32_t n;
    int32_t canvas_idx; /* Philox counter word 2 */
} dg_canvas;

/* Per-step outputs (device memory, n elements each unless stated). */
typedef struct dg_step_stats {
    float* entropy;        /* nats, of softmax((L + bias) / tau_t), MASK excluded. dg_canvas_step and
                              dg_lm_head take entropy, lse and argmax from the LM head's f32
                              accumulators (the logits of record are those values rounded to the act
                              dtype; draws sample the logits of record); dg_sampler_step from the
                              given logits */
    float* lse;            /* log-sum-exp of (L + bias) / tau_t */
    int32_t* argmax;       /* lowest id on ties, MASK excluded */
    uint8_t* selected;     /* 1 where the EB selection committed (or, under
                              DG_COMMIT_RESELECT_ALL, re-committed) this step */
    double* mean_entropy;  /* [1] canvas-mean entropy used by the stop test */
    void* logits;          /* dg_canvas_step: [n][logits_ld] logits of record (act dtype), written;
                              dg_sampler_step: unused */
    int64_t logits_ld;
    int32_t* experts_hit;  /* optional (NULL = not written), dg_canvas_step only: [n_layers] number of
                              routed experts that received at least one canvas row in each layer
                              (the shared expert not counted) */
} dg_step_stats;

/* Library version string. */
const char* dg_version(void);

/* Thread-local message for the last failing call on this thread ("" if none). */
const char* dg_last_error(void);

/* The model card's sampler settings (best practice 1). */
dg_sampler_cfg dg_sampler_default(void);

/* Reset a canvas to all-MASK, nothing committed, state zeroed, prev_argmax -1
 * (the placeholder canvas the news post describes the model starting from).
 * Enqueued on `stream`. */
dg_status dg_canvas_reset(dg_canvas* canvas, int32_t mask_id, void* stream);

/*
 * Event timing of one kernel of the step (measurement support, not part of
 * the method). dg_timing_enable(target) creates the event pool on first use
 * and starts recording a start/stop event pair on the caller's stream around
 * every following eager launch of the chosen kernel:
 *   DG_TIME_LM_HEAD          the LM-head GEMM with its statistics epilogue
 *                            (dg_canvas_step, dg_lm_head), or the
 *                            logit-statistics kernel of dg_sampler_step;
 *   DG_TIME_EXPERT_GATE_UP   the grouped expert gate/up GEMM with SwiGLU;
 *   DG_TIME_EXPERT_DOWN      the grouped expert down GEMM;
 *   DG_TIME_QKV              the QKV projection;
 *   DG_TIME_ATTENTION        the attention kernel (canvas + prefix in the
 *                            decoder, causal in dg_prefill_append);
 *   DG_TIME_O_PROJ           the output projection.
 * The expert and projection targets cover the decoder and the encoder.
 * DG_TIME_OFF (0) stops recording. dg_timing_read synchronises on the
 * recorded events, returns their summed elapsed milliseconds and count, and
 * clears the list. At most 8192 pairs are kept; later launches are not
 * timed. Not thread-safe.
 */
enum {
    DG_TIME_OFF = 0,
    DG_TIME_LM_HEAD = 1,
    DG_TIME_EXPERT_GATE_UP = 2,
    DG_TIME_EXPERT_DOWN = 3,
    DG_TIME_QKV = 4,
    DG_TIME_ATTENTION = 5,
    DG_TIME_O_PROJ = 6
};
dg_status dg_timing_enable(int32_t target);
dg_status dg_timing_read(double* total_ms, int32_t* launches);

/* Workspace bytes dg_sampler_step needs for n rows of `vocab` logits. */
size_t dg_sampler_workspace_bytes(int32_t n, int32_t vocab);

/*
 * dg_sampler_step - one EB sampler step on given logits (model card zh-TW,
 * best practice 1): tempered statistics, EB selection, a Philox4x32-10
 * inverse-CDF draw per selected position, re-masking, the adaptive stop test
 * and, when the canvas finishes (stop, last step, or all committed), the
 * argmax fill of the remaining positions.
 *
 *   scfg          sampler settings (host)
 *   logits        device [n][ld] of dtype logits_dtype (DG_F32 or DG_BF16)
 *   n, vocab, ld  rows (1..1024), columns (multiple of 8), row stride (>= vocab,
 *                 multiple of 8), in elements
 *   mask_id       excluded vocabulary id and the re-mask token (0..vocab-1)
 *   canvas        canvas buffers (device); canvas->n must equal n
 *   step_idx      step to run (0..max_steps-1); it is written to the state's
 *                 step word, so a caller can replay a step; -1 keeps the step
 *                 index already in device memory
 *   seed          Philox key (low word, high word)
 *   stats         outputs (device)
 *   ws, ws_bytes  workspace (device), >= dg_sampler_workspace_bytes(n, vocab)
 *   stream        hipStream_t (NULL = default stream)
 * A finished canvas (state DONE = 1) is left unchanged.
 */
dg_status dg_sampler_step(const dg_sampler_cfg* scfg, const void* logits, int32_t logits_dtype,
                          int32_t n, int32_t vocab, int64_t ld, int32_t mask_id, dg_canvas* canvas,
                          int32_t step_idx, uint64_t seed, dg_step_stats* stats, void* ws,
                          size_t ws_bytes, void* stream);


/*
 * dg_sampler_step_noalloc - dg_sampler_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, checks and results as
 * dg_sampler_step, without ws / ws_bytes: its scratch is a static device
 * array of DG_SAMPLER_STATIC_SCRATCH_BYTES bytes per GPU (also returned by
 * dg_sampler_static_scratch_bytes()), which each GPU the library runs on
 * holds until the process ends. The call allocates nothing and calls no
 * allocating routine; the array's device address is looked up on the first
 * call on each device (call it with that device current).
 *   Limit: DG_E_CAPACITY when dg_sampler_workspace_bytes(n, vocab) exceeds
 *   the array (n = 1024 rows fit up to a vocabulary of about 900K; 256 rows
 *   up to about 3.7M).
 *   Every call on a GPU shares that GPU's array, which keeps the last call's
 *   contents: calls that overlap on one GPU (different streams or threads)
 *   race; serialise them.
 */
#define DG_SAMPLER_STATIC_SCRATCH_BYTES (2u << 20)
size_t dg_sampler_static_scratch_bytes(void);
dg_status dg_sampler_step_noalloc(const dg_sampler_cfg* scfg, const void* logits, int32_t logits_dtype, int32_t n,
                                  int32_t vocab, int64_t ld, int32_t mask_id, dg_canvas* canvas,
                                  int32_t step_idx, uint64_t seed, dg_step_stats* stats, void* stream);

/* ------------------------------------------------------------------------
 * Model geometry. The spec table of the model card fixes the counts (30
 * layers, 1024-token window, 128 experts with 8 active plus 1 shared, 262K
 * vocabulary, canvas 256); widths are configuration. Layer l is global
 * (sees the whole cache) iff global_every > 0 and l % global_every ==
 * global_every - 1; other layers see the last `window` cache rows.
 * ------------------------------------------------------------------------ */
typedef struct dg_config {
    int32_t n_layers;
    int32_t d_model;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;     /* 64, 128 or 256 */
    int32_t n_experts;    /* routed experts (<= 512); the shared expert is extra */
    int32_t top_k;        /* <= 16 */
    int32_t ffn_hidden;   /* SwiGLU hidden width of every expert */
    int32_t vocab;
    int32_t mask_id;      /* placeholder token; excluded from the output distribution */
    int32_t max_canvas;   /* largest canvas (<= 1024; max_canvas x top_k routed rows must fit the
                             expert permutation, else DG_E_UNSUPPORTED) */
    int32_t window;
    int32_t global_every;
    int32_t weight_dtype; /* DG_F32, DG_BF16 or DG_FP8_E4M3: projection and expert matrices */
    int32_t act_dtype;    /* DG_F32 or DG_BF16: activations, KV cache, embedding, router, logits */
    float rope_base;
    float norm_eps;
} dg_config;

/* One layer's weights (device). Matrices are [out][in], `in` contiguous.
 *   wqkv   [(Hq + 2 Hkv) hd][d]   rows: query heads, key heads, value heads
 *   wo     [d][Hq hd]
 *   router [E][d] (act dtype), router_bias [E] f32
 *   w_gate, w_up [E + 1][F][d]; w_down [E + 1][d][F]; expert E is the shared one
 *   *_scale: DG_FP8_E4M3 only, bf16 per output row ([rows] / [E + 1][rows])
 *   attn_norm, moe_norm [d] f32 RMSNorm weights */
typedef struct dg_layer_weights {
    const float* attn_norm;
    const float* moe_norm;
    const void* wqkv;
    const void* wo;
    const void* router;
    const float* router_bias;
    const void* w_gate;
    const void* w_up;
    const void* w_down;
    const void* wqkv_scale;
    const void* wo_scale;
    const void* gate_scale;
    const void* up_scale;
    const void* down_scale;
} dg_layer_weights;

/* Whole-model weights: the tied embedding / LM-head matrix [vocab][d] (act
 * dtype), the final RMSNorm weight [d] f32, and n_layers layer records
 * (host array, copied by dg_model_create).
 * lm_head_e4m3 / lm_head_scale (optional, both NULL or both set; bf16
 * activations only): an OCP e4m3 copy of the tied matrix, [vocab][d] codes
 * with one bf16 scale per vocabulary row. When set, the LM head reads it (half
 * the bytes of the largest single weight read); the input embedding still
 * reads `embed`. */
typedef struct dg_weights {
    const void* embed;
    const float* final_norm;
    const dg_layer_weights* layers;
    const void* lm_head_e4m3;
    const void* lm_head_scale;
} dg_weights;

/* KV cache: per layer (host arrays of n_layers device pointers) K of
 * [n_kv_heads][capacity][head_dim] and V transposed, [n_kv_heads][head_dim]
 * [capacity], in the act dtype; keys after RoPE. Positions [0, len) are
 * filled; dg_prefill_append advances len on the host. capacity must be a
 * multiple of 64 and at most 2^30 rows (DG_E_SHAPE otherwise). Rows at or
 * beyond len may hold anything (a reused cache, NaN): attention reads whole
 * 64-key blocks, masks the scores of keys outside the visible range and
 * reads the values of keys at or beyond len as zero. */
typedef struct dg_kv {
    void* const* k;
    void* const* v;
    int64_t capacity;
    int64_t len;
} dg_kv;

typedef struct dg_model dg_model;

/* Validate the configuration and weight pointers and create a host-side
 * handle (no device memory is allocated; the weights are borrowed). */
dg_status dg_model_create(const dg_config* cfg, const dg_weights* w, dg_model** out);
void dg_model_destroy(dg_model* m);

/* Workspace bytes for steps over up to max_rows canvas rows, or prefill
 * chunks of max_rows tokens (1 <= max_rows <= 4096). Larger workspaces let
 * dg_prefill_append use larger chunks. */
size_t dg_workspace_bytes(const dg_model* m, int32_t max_rows);

/*
 * dg_prefill_append - the encoder (model card zh-TW, overview: the encoder
 * prefills the prompt into the KV cache; a finished canvas is run through the
 * encoder and appended). Runs n tokens (device int32, positions kv->len ..
 * kv->len + n - 1) through the layers with causal attention (a per-query
 * sliding window on local layers) and appends every layer's rotated K and V
 * at rows kv->len ..; the last layer's attention output and MoE are skipped.
 * Tokens are processed in chunks of the workspace's max_rows, at most 4096
 * and at most the rows whose top_k routed slots the expert permutation holds
 * in one workgroup (2048 for 128 experts, top-8). Updates
 * kv->len on the host when enqueued. DG_E_CAPACITY if len + n > capacity.
 * Token ids outside [0, vocab) are not checked on the host (they are device
 * data); the embedding reads them as zero rows.
 */
dg_status dg_prefill_append(const dg_model* m, dg_kv* kv, const int32_t* tokens, int32_t n, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * dg_canvas_step - one denoising step (model card zh-TW, overview and best
 * practice 1): the decoder over all canvas positions at once against the KV
 * cache rows [0, kv->len) (canvas positions kv->len ..), the tied LM head
 * with the fused tempered statistics (logits of record are written to
 * stats->logits), then the EB sampler step exactly as dg_sampler_step.
 * step_idx as in dg_sampler_step. The canvas K/V are not cached.
 */
dg_status dg_canvas_step(const dg_model* m, dg_canvas* canvas, const dg_kv* kv, int32_t step_idx,
                         uint64_t seed, const dg_sampler_cfg* scfg, dg_step_stats* stats, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * dg_generate_canvas - denoise one canvas to completion (model card zh-TW,
 * overview: block-autoregressive multi-canvas sampling): reset the canvas to
 * all-MASK, run dg_canvas_step for t = 0, 1, ... until the device marks it
 * finished (at most max_steps), then, if append_after != 0, run the finished
 * tokens through the encoder with dg_prefill_append. Synchronises on
 * `stream` every `poll_every` steps (>= 1) to read the done flag; returns
 * the number of steps taken in *steps_taken (host).
 */
dg_status dg_generate_canvas(const dg_model* m, dg_canvas* canvas, dg_kv* kv, const dg_sampler_cfg* scfg,
                             uint64_t seed, int32_t append_after, int32_t poll_every, dg_step_stats* stats,
                             int32_t* steps_taken, void* ws, size_t ws_bytes, void* stream);

/*
 * dg_canvas_step_batch - one denoising step of nb canvases of several users
 * at once (model card zh-TW, capabilities: low-batch serving), each with its
 * own KV cache: canvases[b] attends kvs[b] (rows [0, kvs[b].len), canvas
 * positions kvs[b].len ..) and only its own rows; the projections, router,
 * expert GEMMs and LM head run once over all canvas rows, so each weight
 * byte is read once per step for the whole batch. Every canvas then takes
 * the sampler step of dg_sampler_step on its rows with its own state, bias
 * and canvas_idx.
 *   canvases, kvs: arrays of nb (1..64) structs; sum of canvases[b].n <=
 *     max_canvas; with nb > 1 every n is a multiple of 64.
 *   step_idx: the step index of every canvas (0 <= step_idx < max_steps;
 *     the batch moves in lockstep). A finished canvas's rows are still
 *     computed, but its sampler step changes nothing.
 *   stats: one set for the batch; canvas b owns rows [r_b, r_b + n_b) of
 *     entropy, lse, argmax, selected and logits (r_b = sum of the earlier
 *     n), and mean_entropy[b] (nb entries). experts_hit counts over all rows.
 *   ws: dg_workspace_bytes(m, sum of n) bytes at least.
 * Errors as dg_canvas_step; DG_E_SHAPE for the batch limits above.
 */
dg_status dg_canvas_step_batch(const dg_model* m, dg_canvas* canvases, const dg_kv* kvs, int32_t nb, int32_t step_idx,
                               uint64_t seed, const dg_sampler_cfg* scfg, dg_step_stats* stats, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * dg_generate_batch - denoise nb canvases to completion together: reset them
 * all, run dg_canvas_step_batch for t = 0, 1, ... until every canvas is
 * finished (polling the device every poll_every steps) or max_steps, then,
 * if append_after != 0, append each canvas to its own cache with
 * dg_prefill_append. steps_taken[b] (host, nb entries) receives the steps
 * canvas b took before it finished.
 */
dg_status dg_generate_batch(const dg_model* m, dg_canvas* canvases, dg_kv* kvs, int32_t nb, const dg_sampler_cfg* scfg,
                            uint64_t seed, int32_t append_after, int32_t poll_every, dg_step_stats* stats,
                            int32_t* steps_taken, void* ws, size_t ws_bytes, void* stream);

/*
 * A denoising step captured as a HIP graph (the model card's step, zh-TW best
 * practice 1, replayed without host launches). dg_step_graph_create records
 * one dg_canvas_step with the step index read from canvas->state (step_idx
 * -1) on a stream of its own and instantiates it; every pointer (model,
 * canvas, kv arrays, stats, workspace) and the KV length kv->len at creation
 * are baked in, so the graph is valid until the next dg_prefill_append on
 * that cache (then destroy it and create another). dg_step_graph_launch
 * enqueues one step on `stream`; after the canvas is finished a launch is a
 * no-op on the device. Validation errors are those of dg_canvas_step
 * (nothing is recorded then); HIP errors map to DG_E_HIP. The object is a
 * host allocation owned by the caller until dg_step_graph_destroy.
 */
typedef struct dg_step_graph dg_step_graph;
dg_status dg_step_graph_create(const dg_model* m, dg_canvas* canvas, const dg_kv* kv, const dg_sampler_cfg* scfg,
                               uint64_t seed, dg_step_stats* stats, void* ws, size_t ws_bytes, dg_step_graph** out);
dg_status dg_step_graph_launch(dg_step_graph* graph, void* stream);
void dg_step_graph_destroy(dg_step_graph* graph);

/*
 * Component entry points (the stages of dg_canvas_step, exposed so each can
 * be checked on its own; same validation and ownership rules):
 *   dg_embed:          X[i][:] = embed[tokens[i]][:]                 (X f32 [n][d];
 *                      ids outside [0, vocab) give zero rows)
 *   dg_decoder_layer:  X <- decoder layer `layer` over n canvas rows at
 *                      positions kv->len .. (X f32 [n][d], in place); if
 *                      route_ids/route_gates are not NULL the router's top-k
 *                      ids (int32 [n][k]) and gates (f32 [n][k]) are copied out
 *   dg_lm_head:        logits and tempered statistics of rmsnorm(X) for step
 *                      step_idx (no selection): stats->logits, entropy, lse, argmax
 */
dg_status dg_embed(const dg_model* m, const int32_t* tokens, int32_t n, float* X, void* stream);
dg_status dg_decoder_layer(const dg_model* m, int32_t layer, float* X, int32_t n, const dg_kv* kv,
                           int32_t* route_ids, float* route_gates, void* ws, size_t ws_bytes, void* stream);
dg_status dg_lm_head(const dg_model* m, const float* X, int32_t n, const dg_sampler_cfg* scfg, int32_t step_idx,
                     const int32_t* bias_tok, const float* bias_val, dg_step_stats* stats, void* ws,
                     size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
