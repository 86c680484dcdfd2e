// C ABI of libdg: host-side validation, workspace carving and launch order.
// The public contract is include/dg.h.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/dg.h"
#include "api_util.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace dgapi {

thread_local std::string g_err;

dg_status fail(dg_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

dg_status hip_check(hipError_t e, const char* what) {
    if (e == hipSuccess) return DG_OK;
    return fail(DG_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

dg_status check_sampler_cfg(const dg_sampler_cfg* s) {
    if (!s) return fail(DG_E_INVALID, "sampler config is NULL");
    if (s->max_steps < 1 || s->max_steps > 1 << 20) return fail(DG_E_INVALID, "max_steps out of range");
    // at least 1e-12: the statistics pass tempers its excluded-column value
    // -2^64 by log2(e)/tau and needs the product finite
    if (!(s->temp_start >= 1e-12f) || !(s->temp_end >= 1e-12f) || !(s->temp_start <= 3.0e38f) ||
        !(s->temp_end <= 3.0e38f))
        return fail(DG_E_INVALID, "temperatures must lie in [1e-12, 3e38]");
    if (!(s->bound >= 0.f)) return fail(DG_E_INVALID, "bound must be >= 0");
    if (!(s->stop_entropy >= 0.f)) return fail(DG_E_INVALID, "stop_entropy must be >= 0");
    if (s->stable_steps < 1) return fail(DG_E_INVALID, "stable_steps must be >= 1");
    if (s->bound_mode != DG_BOUND_SUM && s->bound_mode != DG_BOUND_SUM_MINUS_MAX)
        return fail(DG_E_INVALID, "unknown bound_mode");
    if (s->commit_mode != DG_COMMIT_KEEP && s->commit_mode != DG_COMMIT_RESELECT_ALL)
        return fail(DG_E_INVALID, "unknown commit_mode");
    if (s->draw_mode != DG_DRAW_INVERSE_CDF && s->draw_mode != DG_DRAW_GUMBEL_MAX)
        return fail(DG_E_INVALID, "unknown draw_mode");
    return DG_OK;
}

dg::SamplerParams to_params(const dg_sampler_cfg* s) {
    dg::SamplerParams p;
    p.max_steps = s->max_steps;
    p.temp_start = s->temp_start;
    p.temp_end = s->temp_end;
    p.bound = s->bound;
    p.stop_entropy = s->stop_entropy;
    p.stable_steps = s->stable_steps;
    p.bound_mode = s->bound_mode;
    p.commit_mode = s->commit_mode;
    p.draw_mode = s->draw_mode;
    p.seed_lo = p.seed_hi = 0;
    p.canvas_idx = 0;
    return p;
}

dg_status check_canvas(const dg_canvas* c, int n) {
    if (!c) return fail(DG_E_INVALID, "canvas is NULL");
    if (!c->tokens || !c->committed || !c->prev_argmax || !c->state)
        return fail(DG_E_INVALID, "canvas buffer pointer is NULL");
    if ((c->bias_tok == nullptr) != (c->bias_val == nullptr))
        return fail(DG_E_INVALID, "bias_tok and bias_val must both be set or both NULL");
    if (c->n != n) return fail(DG_E_SHAPE, "canvas n=%d does not match %d rows", c->n, n);
    if (c->canvas_idx < 0) return fail(DG_E_INVALID, "canvas_idx must be >= 0");
    return DG_OK;
}

dg_status check_stats(const dg_step_stats* s) {
    if (!s || !s->entropy || !s->lse || !s->argmax || !s->selected)
        return fail(DG_E_INVALID, "step stats pointer is NULL");
    return DG_OK;
}

__global__ void canvas_reset_kernel(int32_t* tokens, uint8_t* committed, int32_t* prev, int32_t* state,
                                    int n, int mask_id) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        tokens[i] = mask_id;
        committed[i] = 0;
        prev[i] = -1;
    }
    if (i < DG_STATE_WORDS) state[i] = 0;
}

// ---- optional event timing of the dominant kernel of each step ----
struct Timing {
    int target = DG_TIME_OFF;
    static constexpr int kMax = 8192;
    hipEvent_t ev[2 * kMax];
    int used = 0;
    bool created = false;
};
Timing g_timing;

}  // namespace dgapi

namespace dgapi {

// Records the start event of a launch of kernel `target`; returns the slot or -1.
int timing_begin(hipStream_t st, int target) {
    if (g_timing.target == DG_TIME_OFF || g_timing.target != target || g_timing.used >= Timing::kMax) return -1;
    int slot = g_timing.used++;
    hipEventRecord(g_timing.ev[2 * slot], st);
    return slot;
}
void timing_end(int slot, hipStream_t st) {
    if (slot >= 0) hipEventRecord(g_timing.ev[2 * slot + 1], st);
}

}  // namespace dgapi

namespace {
using namespace dgapi;

size_t sampler_ws(int n, int V) {
    return align256((size_t)n * dg::sampler_nsplit(V) * sizeof(dg::RowPart)) +
           align256((size_t)n * sizeof(int32_t)) + align256((size_t)n * dg::draw_nchunk(V) * sizeof(double)) +
           align256((size_t)n * sizeof(int32_t));
}

}  // namespace

extern "C" {

const char* dg_version(void) { return "dg 0.1 gfx950"; }

const char* dg_last_error(void) { return g_err.c_str(); }

dg_sampler_cfg dg_sampler_default(void) {
    dg_sampler_cfg c;
    c.max_steps = 48;
    c.temp_start = 0.8f;
    c.temp_end = 0.4f;
    c.bound = 0.1f;
    c.stop_entropy = 0.005f;
    c.stable_steps = 2;
    c.bound_mode = DG_BOUND_SUM;
    c.commit_mode = DG_COMMIT_KEEP;
    c.draw_mode = DG_DRAW_INVERSE_CDF;
    return c;
}

dg_status dg_canvas_reset(dg_canvas* c, int32_t mask_id, void* stream) {
    if (!c) return fail(DG_E_INVALID, "canvas is NULL");
    if (dg_status s = check_canvas(c, c->n)) return s;
    if (c->n < 1 || c->n > 1024) return fail(DG_E_SHAPE, "canvas n=%d outside 1..1024", c->n);
    if (mask_id < 0) return fail(DG_E_INVALID, "mask_id must be >= 0");
    int threads = 256;
    int blocks = (c->n + threads - 1) / threads;
    canvas_reset_kernel<<<blocks, threads, 0, (hipStream_t)stream>>>(c->tokens, c->committed, c->prev_argmax,
                                                                      c->state, c->n, mask_id);
    return hip_check(hipGetLastError(), "canvas_reset launch");
}

dg_status dg_timing_enable(int32_t target) {
    if (target < DG_TIME_OFF || target > DG_TIME_O_PROJ) return fail(DG_E_INVALID, "unknown timing target %d", target);
    if (target != DG_TIME_OFF && !g_timing.created) {
        for (int i = 0; i < 2 * Timing::kMax; ++i)
            if (dg_status s = hip_check(hipEventCreate(&g_timing.ev[i]), "hipEventCreate")) return s;
        g_timing.created = true;
    }
    g_timing.target = target;
    g_timing.used = 0;
    return DG_OK;
}

dg_status dg_timing_read(double* total_ms, int32_t* launches) {
    if (!total_ms || !launches) return fail(DG_E_INVALID, "NULL output");
    double tot = 0.0;
    for (int i = 0; i < g_timing.used; ++i) {
        float ms = 0.f;
        if (dg_status s = hip_check(hipEventSynchronize(g_timing.ev[2 * i + 1]), "hipEventSynchronize")) return s;
        if (dg_status s = hip_check(hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]),
                                    "hipEventElapsedTime"))
            return s;
        tot += ms;
    }
    *total_ms = tot;
    *launches = g_timing.used;
    g_timing.used = 0;
    return DG_OK;
}

size_t dg_sampler_workspace_bytes(int32_t n, int32_t vocab) {
    if (n < 1 || vocab < 8) return 0;
    return sampler_ws(n, vocab);
}

}  // extern "C"

// Scratch memory of dg_sampler_step_noalloc: one copy per GPU, held until the
// process ends. Every call on a GPU shares it; the kernels write each part
// (row partials, selected-row list, draw chunk sums, Gumbel candidates)
// before reading it, so nothing needs to start at zero.
static __device__ __align__(256) unsigned char scratch[DG_SAMPLER_STATIC_SCRATCH_BYTES];

namespace {

// Argument checks shared by dg_sampler_step and dg_sampler_step_noalloc
// (everything but the workspace).
dg_status check_sampler_args(const dg_sampler_cfg* scfg, const void* logits, int32_t logits_dtype, int32_t n,
                             int32_t vocab, int64_t ld, int32_t mask_id, const dg_canvas* canvas, int32_t step_idx,
                             const dg_step_stats* stats) {
    if (dg_status s = check_sampler_cfg(scfg)) return s;
    if (!logits) return fail(DG_E_INVALID, "logits is NULL");
    if (logits_dtype != DG_F32 && logits_dtype != DG_BF16) return fail(DG_E_UNSUPPORTED, "logits dtype");
    if (n < 1 || n > 1024) return fail(DG_E_SHAPE, "n=%d outside 1..1024", n);
    if (vocab < 8 || vocab % 8) return fail(DG_E_SHAPE, "vocab=%d must be a positive multiple of 8", vocab);
    if (ld < vocab || ld % 8) return fail(DG_E_SHAPE, "ld must be >= vocab and a multiple of 8");
    if (mask_id < 0 || mask_id >= vocab) return fail(DG_E_INVALID, "mask_id outside 0..vocab-1");
    if ((uintptr_t)logits % 16) return fail(DG_E_INVALID, "logits must be 16-byte aligned");
    if (dg_status s = check_canvas(canvas, n)) return s;
    if (dg_status s = check_stats(stats)) return s;
    if (step_idx < -1 || step_idx >= scfg->max_steps) return fail(DG_E_INVALID, "step_idx out of range");
    return DG_OK;
}

// The sampler step's launches over scratch memory `ws` (device address, at
// least sampler_ws(n, vocab) bytes); arguments already checked.
dg_status sampler_step_launch(const dg_sampler_cfg* scfg, const void* logits, int32_t logits_dtype, int32_t n,
                              int32_t vocab, int64_t ld, int32_t mask_id, dg_canvas* canvas, int32_t step_idx,
                              uint64_t seed, dg_step_stats* stats, void* ws, hipStream_t st) {
    dg::SamplerParams sp = to_params(scfg);
    sp.seed_lo = (uint32_t)(seed & 0xffffffffu);
    sp.seed_hi = (uint32_t)(seed >> 32);
    sp.canvas_idx = canvas->canvas_idx;
    Carve cv(ws);
    dg::RowPart* parts = cv.take<dg::RowPart>((size_t)n * dg::sampler_nsplit(vocab));
    int32_t* sel_list = cv.take<int32_t>(n);
    double* chunk_sum = cv.take<double>((size_t)n * dg::draw_nchunk(vocab));
    int32_t* gtok = sp.draw_mode ? cv.take<int32_t>(n) : nullptr;
    int f32 = logits_dtype == DG_F32;
    int slot = timing_begin(st, DG_TIME_LM_HEAD);
    if (dg_status s = hip_check(dg::launch_logit_stats(logits, f32, ld, n, vocab, canvas->state, step_idx, sp, mask_id,
                                                       canvas->bias_tok, canvas->bias_val, parts, st),
                                "logit_stats"))
        return s;
    timing_end(slot, st);
    if (dg_status s = hip_check(dg::launch_merge_rows(parts, n, dg::sampler_nsplit(vocab), canvas->state,
                                                      stats->entropy, stats->lse, stats->argmax, gtok, st),
                                "merge_rows"))
        return s;
    return hip_check(dg::launch_sampler_tail(logits, f32, ld, n, vocab, mask_id, canvas->bias_tok,
                                             canvas->bias_val, stats->entropy, stats->argmax, canvas->state,
                                             step_idx, sp, seed, canvas->canvas_idx, canvas->tokens,
                                             canvas->committed, canvas->prev_argmax, stats->selected, sel_list,
                                             chunk_sum, gtok, stats->mean_entropy, st),
                     "sampler tail");
}

constexpr size_t kStaticScratchBytes = (size_t)DG_SAMPLER_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's scratch array, looked up once per device
// (with that device current). The array's host-side name is not a device
// address and is never passed to a kernel.
dg_status static_scratch(void** out) {
    int dev = -1;
    if (dg_status s = hip_check(hipGetDevice(&dev), "hipGetDevice")) return s;
    if (dev < 0 || dev >= kMaxDevices) return fail(DG_E_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (dg_status s = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))
            return s;
        if (!p) return fail(DG_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DG_OK;
}

}  // namespace

extern "C" {

dg_status dg_sampler_step(const dg_sampler_cfg* scfg, const void* logits, int32_t logits_dtype, int32_t n,
                          int32_t vocab, int64_t ld, int32_t mask_id, dg_canvas* canvas, int32_t step_idx,
                          uint64_t seed, dg_step_stats* stats, void* ws, size_t ws_bytes, void* stream) {
    if (dg_status s = check_sampler_args(scfg, logits, logits_dtype, n, vocab, ld, mask_id, canvas, step_idx, stats))
        return s;
    if (!ws || ws_bytes < sampler_ws(n, vocab)) return fail(DG_E_CAPACITY, "workspace too small");
    return sampler_step_launch(scfg, logits, logits_dtype, n, vocab, ld, mask_id, canvas, step_idx, seed, stats, ws,
                               (hipStream_t)stream);
}

size_t dg_sampler_static_scratch_bytes(void) { return kStaticScratchBytes; }

dg_status dg_sampler_step_noalloc(const dg_sampler_cfg* scfg, const void* logits, int32_t logits_dtype, int32_t n,
                                  int32_t vocab, int64_t ld, int32_t mask_id, dg_canvas* canvas, int32_t step_idx,
                                  uint64_t seed, dg_step_stats* stats, void* stream) {
    if (dg_status s = check_sampler_args(scfg, logits, logits_dtype, n, vocab, ld, mask_id, canvas, step_idx, stats))
        return s;
    const size_t need = sampler_ws(n, vocab);
    if (need > kStaticScratchBytes)
        return fail(DG_E_CAPACITY, "n=%d x vocab=%d needs %zu bytes of scratch, above the static %zu", n, vocab, need,
                    kStaticScratchBytes);
    void* ws = nullptr;
    if (dg_status s = static_scratch(&ws)) return s;
    return sampler_step_launch(scfg, logits, logits_dtype, n, vocab, ld, mask_id, canvas, step_idx, seed, stats, ws,
                               (hipStream_t)stream);
}

}  // extern "C"
