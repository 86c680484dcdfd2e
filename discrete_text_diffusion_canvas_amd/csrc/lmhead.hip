// The tied LM head for gfx950 (bf16): logits L = rmsnorm(x) E^T over the
// 262K vocabulary with the fused tempered-statistics epilogue.
//
// DiffusionGemma model card (zh-TW): spec table (262K vocabulary) and best
// practice 1 (the temperature shapes the logits the sampler reads). The
// statistics per row (max, partition sum, entropy partial, argmax) are
// computed from the logits of record in the epilogue, so probabilities are
// never written to memory.
//
// bf16 models run the LM head on the tiled GEMM (gemm_tile.hip, its LM-head
// epilogue); this kernel serves f32 models.
//
// Shape: all canvas rows (<= 256) x 128 vocabulary rows per workgroup, 4 waves
// as 2 x 2 (each 128 x 64, 8 x 4 MFMA tiles of 16x16x32 bf16). K advances in
// stages of 64; each stage of A (256 x 64) and E (128 x 64) is copied from
// global memory straight into LDS (global_load_lds_dwordx4, 16 bytes per lane)
// with STAGES-1 stages in flight. A 128-byte LDS row holds 8 chunks of 16
// bytes; chunk c of row r is stored at position c ^ ((r >> 1) & 7), so the 16
// lanes reading one fragment column hit 16 distinct 4-bank groups.
#include "common.hpp"
#include "gemm.hpp"

namespace dg {

namespace {

#ifndef DG_LM_BK
#define DG_LM_BK 64
#endif
#ifndef DG_LM_STAGES
#define DG_LM_STAGES 3
#endif
constexpr int LBM = 256;   // rows (canvas)
constexpr int LBN = 128;   // vocabulary rows per workgroup
constexpr int LBK = DG_LM_BK;    // k per stage (64; 32 allows more stages)
constexpr int LSTAGES = DG_LM_STAGES;
constexpr int ROWB = LBK * 2;                         // bytes per LDS row
constexpr int A_BYTES = LBM * ROWB;                   // 32 KB
constexpr int B_BYTES = LBN * ROWB;                   // 16 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;        // 48 KB
constexpr int A_INSTR = A_BYTES / 1024 / 4;           // per wave
constexpr int B_INSTR = B_BYTES / 1024 / 4;           // per wave
constexpr int LOADS_PER_STAGE = A_INSTR + B_INSTR;
constexpr int RPI = 1024 / ROWB;                      // LDS rows per 1 KB copy instruction
constexpr int CPR = ROWB / 16;                        // 16-byte chunks per row
static_assert(LOADS_PER_STAGE * (LSTAGES - 1) < 64, "vmcnt range");

// s_waitcnt with only vmcnt limited (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// 128-byte rows (8 chunks): chunk c of row r at c ^ ((r >> 1) & 7);
// 64-byte rows (4 chunks): chunk c of row r at c ^ ((r >> 2) & 3).
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (CPR == 8) return c ^ ((r >> 1) & 7);
    else return c ^ ((r >> 2) & 3);
}

}  // namespace

// Epilogue of one 256 x 128 tile. The accumulators go to LDS as the logits
// of record (bf16-rounded unless the logits are f32), row-major with a stride
// of LBN + 4 floats. From there (1) the logits leave in 16-byte coalesced
// stores and (2) one thread per canvas row walks its 128 logits in vocabulary
// order for the tile's partial statistics: the max and the 2^x partition sum
// and entropy partial of the tempered logits (log2 units), and the raw argmax
// (first index among equal values) with the row's bias token added and the
// mask token excluded.
constexpr int TS = LBN + 4;
static_assert((size_t)LBM * TS * 4 <= (size_t)LSTAGES * STAGE_BYTES, "epilogue tile must fit the stage buffers");

__device__ __forceinline__ void lmhead_tile_epilogue(const GemmArgs& g, const f32x4 (&acc)[8][4], int mcount,
                                                     int n0, unsigned char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lg = lane >> 4;
    float* T = reinterpret_cast<float*>(smem);
    __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float l = acc[i][j][q];
                T[(wm * 128 + i * 16 + lg * 4 + q) * TS + wn * 64 + j * 16 + lr] = g.c_f32 ? l : round_bf(l);
            }
    __syncthreads();

    const int N = g.N;
    if (g.c_f32) {
        float* C = reinterpret_cast<float*>(g.C);
        const bool vec = (g.ldc % 4) == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0;
        for (int idx = tid; idx < mcount * (LBN / 4); idx += 256) {
            const int r = idx / (LBN / 4), ch = idx % (LBN / 4);
            const int n = n0 + ch * 4;
            const float4 v = *reinterpret_cast<const float4*>(T + r * TS + ch * 4);
            float* dst = C + (int64_t)r * g.ldc + n;
            if (vec && n + 3 < N) {
                *reinterpret_cast<float4*>(dst) = v;
            } else {
                const float e[4] = {v.x, v.y, v.z, v.w};
                for (int u = 0; u < 4; ++u)
                    if (n + u < N) dst[u] = e[u];
            }
        }
    } else {
        uint16_t* C = reinterpret_cast<uint16_t*>(g.C);
        const bool vec = (g.ldc % 8) == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0;
        for (int idx = tid; idx < mcount * (LBN / 8); idx += 256) {
            const int r = idx / (LBN / 8), ch = idx % (LBN / 8);
            const int n = n0 + ch * 8;
            const float4 a = *reinterpret_cast<const float4*>(T + r * TS + ch * 8);
            const float4 b = *reinterpret_cast<const float4*>(T + r * TS + ch * 8 + 4);
            const float e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint16_t* dst = C + (int64_t)r * g.ldc + n;
            if (vec && n + 7 < N) {
                uint4 w;
                w.x = f2bf2(e[0], e[1]);
                w.y = f2bf2(e[2], e[3]);
                w.z = f2bf2(e[4], e[5]);
                w.w = f2bf2(e[6], e[7]);
                *reinterpret_cast<uint4*>(dst) = w;
            } else {
                for (int u = 0; u < 8; ++u)
                    if (n + u < N) dst[u] = f2bf(e[u]);
            }
        }
    }

    const int r = tid;
    if (r >= mcount) return;
    const int t = g.step_override >= 0 ? g.step_override : (g.state ? g.state[1] : 0);
    const float c2 = (float)(1.4426950408889634 / lm_tau_at(g.sp, t));
    const int bt = g.bias_tok ? g.bias_tok[r] : -1;
    const float bv = g.bias_tok ? g.bias_val[r] : 0.f;
    const float* row = T + r * TS;
    float vm = -INFINITY, rawm = -INFINITY;
    int vi = 0x7fffffff;
#pragma unroll 4
    for (int c = 0; c < LBN; c += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(row + c);
        const float e[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int n = n0 + c + u;
            float lb = e[u] + (n == bt ? bv : 0.f);
            if (n >= N || n == g.mask_id) lb = -INFINITY;
            vm = fmaxf(vm, lb * c2);
            if (lb > rawm) { rawm = lb; vi = n; }
        }
    }
    float s = 0.f, tt = 0.f;
    if (vm != -INFINITY) {
#pragma unroll 4
        for (int c = 0; c < LBN; c += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(row + c);
            const float e[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int n = n0 + c + u;
                float lb = e[u] + (n == bt ? bv : 0.f);
                if (n >= N || n == g.mask_id) lb = -INFINITY;
                const float d = lb * c2 - vm;
                const float w = exp2f(d);
                s += w;
                tt += w > 0.f ? w * d : 0.f;
            }
        }
    }
    RowPart p;
    p.m2 = vm; p.s = s; p.t = tt; p.lmax = rawm;
    p.amax = (vi == 0x7fffffff || rawm == -INFINITY) ? -1 : vi;
    p.pad[0] = p.pad[1] = p.pad[2] = 0;
    g.parts[(int64_t)r * g.nsplit + blockIdx.x] = p;
}

__global__ void __launch_bounds__(256) lmhead_kernel(GemmArgs g) {
    if (g.state && g.state[0]) return;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * LBN;
    const int M = g.M, N = g.N;
    const uint16_t* A = reinterpret_cast<const uint16_t*>(g.A);
    const uint16_t* E = reinterpret_cast<const uint16_t*>(g.W);
    const int KT = g.K / LBK;

    // Per-lane global sources for this wave's load instructions. Instruction
    // j of this wave covers LDS rows [8*(wave*NI + j), +8); lane i fills
    // row +i/8, position i%8, i.e. logical chunk swz(row, i%8).
    const int pos = lane % CPR;
    const uint16_t* asrc[A_INSTR];
    const uint16_t* bsrc[B_INSTR];
#pragma unroll
    for (int j = 0; j < A_INSTR; ++j) {
        const int r = RPI * (wave * A_INSTR + j) + lane / CPR;
        const int rr = r < M ? r : 0;  // rows past M read row 0; never stored
        asrc[j] = A + (int64_t)rr * g.lda + 8 * swz(r, pos);
    }
#pragma unroll
    for (int j = 0; j < B_INSTR; ++j) {
        const int r = RPI * (wave * B_INSTR + j) + lane / CPR;
        const int vr = min(n0 + r, N - 1);  // past the vocabulary: a valid row, discarded
        bsrc[j] = E + (int64_t)vr * g.ldw + 8 * swz(r, pos);
    }
    auto issue = [&](int kt) {
        unsigned char* st = smem + (kt % LSTAGES) * STAGE_BYTES;
        const int k0 = kt * LBK;
#pragma unroll
        for (int j = 0; j < A_INSTR; ++j)
            __builtin_amdgcn_global_load_lds(asrc[j] + k0, st + (wave * A_INSTR + j) * 1024, 16, 0, 0);
#pragma unroll
        for (int j = 0; j < B_INSTR; ++j)
            __builtin_amdgcn_global_load_lds(bsrc[j] + k0, st + A_BYTES + (wave * B_INSTR + j) * 1024, 16, 0, 0);
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < LSTAGES - 1; ++s)
        if (s < KT) issue(s);
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + LSTAGES - 1 < KT) {
            issue(kt + LSTAGES - 1);
            wait_vmcnt<LOADS_PER_STAGE * (LSTAGES - 1)>();
        } else if (KT - 1 - kt >= 3 && LSTAGES > 4) {
            wait_vmcnt<LOADS_PER_STAGE * 3>();
        } else if (KT - 1 - kt >= 2 && LSTAGES > 3) {
            wait_vmcnt<LOADS_PER_STAGE * 2>();
        } else if (kt + 1 < KT) {
            wait_vmcnt<LOADS_PER_STAGE>();
        } else {
            wait_vmcnt<0>();
        }
        // this wave's copies of stage kt have landed (vmcnt); the barrier makes
        // every wave's copies visible. A bare s_barrier: the fence of
        // __syncthreads would wait for the stages still in flight.
        __builtin_amdgcn_s_barrier();
        const unsigned char* st = smem + (kt % LSTAGES) * STAGE_BYTES;
        const unsigned char* as = st;
        const unsigned char* bs = st + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < LBK / 32; ++ks) {
            const int c = ks * 4 + lg;  // logical 16-byte chunk of this lane
            u16x8 bfr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = wn * 64 + j * 16 + lr;
                bfr[j] = *reinterpret_cast<const u16x8*>(bs + r * ROWB + swz(r, c) * 16);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = wm * 128 + i * 16 + lr;
                const u16x8 afr = *reinterpret_cast<const u16x8*>(as + r * ROWB + swz(r, c) * 16);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, afr),
                                                                        __builtin_bit_cast(bf16x8, bfr[j]),
                                                                        acc[i][j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_barrier();  // all waves done reading before the buffer is refilled
    }
    wait_vmcnt<0>();
    lmhead_tile_epilogue(g, acc, min(M, LBM), n0, smem);
}

hipError_t launch_lmhead_bf16(const GemmArgs& g, hipStream_t st) {
    if (g.M > LBM || g.K % LBK) return hipErrorInvalidValue;
    const size_t lds = (size_t)LSTAGES * STAGE_BYTES;
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(lmhead_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    lmhead_kernel<<<(g.N + LBN - 1) / LBN, 256, lds, st>>>(g);
    return hipGetLastError();
}

}  // namespace dg
