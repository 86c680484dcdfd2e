// Host-side helpers shared by the C-ABI translation units: error reporting
// and the workspace bump allocator.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <string>

#include "../../include/dg.h"
#include "kernels.hpp"

namespace dgapi {

dg_status check_sampler_cfg(const dg_sampler_cfg* s);
dg::SamplerParams to_params(const dg_sampler_cfg* s);
dg_status check_canvas(const dg_canvas* c, int n);
dg_status check_stats(const dg_step_stats* s);

dg_status fail(dg_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dg_status hip_check(hipError_t e, const char* what);

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bump allocator over a caller-provided workspace; with a NULL base it only
// measures.
struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* p) : base((char*)p) {}
    template <typename T>
    T* take(size_t count) {
        T* p = (T*)(base ? base + off : nullptr);
        off += align256(count * sizeof(T));
        return p;
    }
};

// event timing of the dominant kernel of a step (api.hip)
int timing_begin(hipStream_t st, int target);
void timing_end(int slot, hipStream_t st);

}  // namespace dgapi
