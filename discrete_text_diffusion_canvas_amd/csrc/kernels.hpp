// Internal declarations shared between the kernel translation units and the
// C-ABI layer. Not part of the public interface (include/dg.h is).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

struct RowPart;

// Sampler parameters as the kernels see them.
struct SamplerParams {
    int max_steps;
    float temp_start;
    float temp_end;
    float bound;
    float stop_entropy;
    int stable_steps;
    int bound_mode;   // 0: sum <= bound; 1: sum minus the largest <= bound
    int commit_mode;  // 0: commits are final; 1: every position re-selected each step
    int draw_mode;    // 0: inverse CDF; 1: Gumbel-max (fused into the statistics pass)
    uint32_t seed_lo, seed_hi;  // Philox key (Gumbel-max draws)
    int canvas_idx;             // Philox counter word 2 (Gumbel-max draws)
};

// ---- sampler.hip ----
int sampler_nsplit(int V);
int draw_nchunk(int V);
hipError_t launch_logit_stats(const void* logits, int dtype_f32, int64_t ld, int n, int V,
                              const int32_t* state, int step_override, const SamplerParams& sp, int mask_id,
                              const int32_t* bias_tok, const float* bias_val, RowPart* parts,
                              hipStream_t st);
// gtok (optional): each row's Gumbel-max candidate from the partials' pad words
hipError_t launch_merge_rows(const RowPart* parts, int n, int nsplit, const int32_t* state, float* H,
                             float* lse, int32_t* amax, int32_t* gtok, hipStream_t st);
hipError_t launch_sampler_tail(const void* logits, int dtype_f32, int64_t ld, int n, int V, int mask_id,
                               const int32_t* bias_tok, const float* bias_val, const float* H,
                               const int32_t* amax, int32_t* state, int step_override, const SamplerParams& sp,
                               uint64_t seed, int canvas_idx, int32_t* tokens, uint8_t* committed,
                               int32_t* prev_amax, uint8_t* selected, int32_t* sel_list, double* chunk_sum,
                               const int32_t* gtok, double* mean_out, hipStream_t st);

}  // namespace dg
