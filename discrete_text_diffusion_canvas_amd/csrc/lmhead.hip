// The tied LM head for gfx950 (bf16): logits L = rmsnorm(x) E^T over the
// 262K vocabulary with the fused tempered-statistics epilogue.
//
// DiffusionGemma model card (zh-TW): spec table (262K vocabulary) and best
// practice 1 (the temperature shapes the logits the sampler reads). The
// statistics per row (max, partition sum, entropy partial, argmax) are
// computed from the logits of record in the epilogue, so probabilities are
// never written to memory.
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

constexpr int LBM = 256;   // rows (canvas)
constexpr int LBN = 128;   // vocabulary rows per workgroup
constexpr int LBK = 64;    // k per stage
constexpr int LSTAGES = 3;
constexpr int ROWB = LBK * 2;                         // bytes per LDS row (128)
constexpr int A_BYTES = LBM * ROWB;                   // 32 KB
constexpr int B_BYTES = LBN * ROWB;                   // 16 KB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;        // 48 KB
constexpr int A_INSTR = A_BYTES / 1024 / 4;           // per wave: 8
constexpr int B_INSTR = B_BYTES / 1024 / 4;           // per wave: 4
constexpr int LOADS_PER_STAGE = A_INSTR + B_INSTR;    // 12 per wave

// s_waitcnt with only vmcnt limited (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

}  // namespace

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
    const int pos = lane & 7;
    const uint16_t* asrc[A_INSTR];
    const uint16_t* bsrc[B_INSTR];
#pragma unroll
    for (int j = 0; j < A_INSTR; ++j) {
        const int r = 8 * (wave * A_INSTR + j) + (lane >> 3);
        const int rr = r < M ? r : 0;  // rows past M read row 0; never stored
        asrc[j] = A + (int64_t)rr * g.lda + 8 * swz(r, pos);
    }
#pragma unroll
    for (int j = 0; j < B_INSTR; ++j) {
        const int r = 8 * (wave * B_INSTR + j) + (lane >> 3);
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
        for (int ks = 0; ks < 2; ++ks) {
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
    lmhead_epilogue<2, 2, 8, 4>(g, acc, 0, min(M, LBM), n0, smem);
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
