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
 * 2 stable steps, DG_BOUND_SUM. */
typedef struct dg_sampler_cfg {
    int32_t max_steps;
    float temp_start;
    float temp_end;
    float bound;          /* nats */
    float stop_entropy;   /* nats, strict "<" */
    int32_t stable_steps; /* argmax vector unchanged over this many consecutive steps */
    int32_t bound_mode;   /* DG_BOUND_SUM or DG_BOUND_SUM_MINUS_MAX */
} dg_sampler_cfg;

/* One canvas. All pointers are device memory of n elements (state: 8).
 * Commits are final: an uncommitted position always holds mask_id.
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
    float* entropy;        /* nats, of softmax((L + bias) / tau_t), MASK excluded */
    float* lse;            /* log-sum-exp of (L + bias) / tau_t */
    int32_t* argmax;       /* lowest id on ties, MASK excluded */
    uint8_t* selected;     /* 1 where the EB selection committed this step */
    double* mean_entropy;  /* [1] canvas-mean entropy used by the stop test */
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
 * Event timing of each step's dominant kernel (measurement support, not part
 * of the method). dg_timing_enable(1) creates the event pool on first use and
 * starts recording a start/stop event pair on the caller's stream around the
 * dominant kernel of every following eager step (the logit-statistics kernel
 * of dg_sampler_step); dg_timing_read synchronises on the recorded events,
 * returns their summed elapsed milliseconds and count, and clears the list.
 * At most 8192 pairs are kept; later launches are not timed. Not thread-safe.
 */
dg_status dg_timing_enable(int32_t on);
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

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
