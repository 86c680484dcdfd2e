// The tied LM head for gfx950 with bf16 activations: logits L = x E^T over
// the 262K vocabulary, the tempered statistics of every row in the epilogue.
//
// DiffusionGemma model card (zh-TW): the spec table (262K vocabulary) and
// best practice 1 (a temperature from 0.8 to 0.4 shapes the logits whose
// per-position entropies the sampler compares with its bound). At tau = 0.4
// the entropy of a row moves by up to ~10x the relative error of its logits,
// so the activation side is carried at ~16 significant bits: the final
// RMSNorm leaves x = hi + lo as two bf16 arrays (hi = bf16(x), lo =
// bf16(x - hi)) and the K loop accumulates hi E^T + lo E^T in f32. The logits
// then carry the error of an f32 product, not of bf16 activations.
//
// Shape: a workgroup owns 256 canvas rows x 256 vocabulary rows; 8 waves (two
// per SIMD), wave w the rows [32 w, +32) x all 256 columns with
// v_mfma_f32_32x32x16_bf16 (8 accumulator tiles of 32 x 32, 128 registers;
// each weight fragment read from LDS feeds 2 MFMAs: hi and lo). A wave's
// activation rows are its own, so their hi and lo fragments go from global
// memory (L2) straight into registers, kept as a ring of the next four 16-k
// steps (each slot refilled four steps ahead as soon as its MFMAs have read
// it); only the vocabulary tile is shared and is
// staged through LDS: each lane loads 16-byte pieces (8 bytes when the matrix
// is e4m3, widened to bf16 with the hardware convert) one stage ahead and
// writes them into one of two XOR-swizzled slots (chunk c of row r at
// c ^ ((r >> 1) & 7): 16 consecutive rows reading one chunk hit distinct
// banks), one barrier per stage. Work items (m-block, vocabulary tile) are
// walked by a persistent grid; the m-blocks of one tile get ids 8 apart, one
// XCD, so the tile's weight rows come from that XCD's L2 after the first.
//
// Epilogue, per half tile of 128 columns (the statistics partial of merge_rows):
// the accumulators go through LDS as an f32 tile; the bf16 logits of record
// leave in 16-byte stores, and one thread per canvas row takes, from the f32
// values, the raw max and its lowest column, then the base-2 partition sum
// and entropy partial of the tempered (biased, MASK-excluded) logits. With
// Gumbel-max draws the row's best z - log(-log u) over the logits of record is
// kept as well.
#include "common.hpp"
#include "gemm.hpp"

#include <type_traits>

namespace dg {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int LBM = 256;                          // canvas rows per work item
constexpr int LBN = 256;                          // vocabulary rows per work item
// build-time tunables: row groups of the 8 waves (8: a wave owns 32 rows x
// 256 columns; 4: 64 rows x 128 columns, measured 41% slower) and the k-steps
// of the activation ring (4 measured faster than 2)
#ifndef DG_LM_WR
#define DG_LM_WR 8
#endif
#ifndef DG_LM_RING
#define DG_LM_RING 4
#endif
constexpr int LNW = 8;                            // waves, two per SIMD
constexpr int LWR = DG_LM_WR;                     // row groups of waves
constexpr int LWC = LNW / LWR;                    // column groups
constexpr int LRT = LBM / LWR / 32;               // 32-row tiles per wave
constexpr int LCT = LBN / LWC / 32;               // 32-column tiles per wave
constexpr int LHC = LCT / 2;                      // column tiles per fragment half
constexpr int RING = DG_LM_RING;                  // k-steps held in the activation ring
constexpr int LKB = 64;                           // k per stage
constexpr int LROWB = LKB * 2;                    // bytes of an LDS weight row
constexpr int LB_BYTES = LBN * LROWB;             // one stage of the weight tile
constexpr int LB_INSTR = LB_BYTES / 1024 / LNW;   // 1 KB pieces per wave and stage
constexpr int TST = 129;                          // epilogue tile row stride (floats, odd)
static_assert(LWR * LWC == LNW && LRT * 32 * LWR == LBM && LCT * 32 * LWC == LBN, "wave grid covers the tile");
static_assert(LBN == 256 && (LWC == 1 || LWC == 2), "epilogue halves of 128 columns");
constexpr size_t LM_LDS = std::max<size_t>(2 * (size_t)LB_BYTES, (size_t)LBM * TST * sizeof(float));

__device__ __forceinline__ int lswz(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ void lm_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// 8 e4m3 codes -> 8 bf16 (exact), the gfx950 scaled pack conversion at scale 1
__device__ __forceinline__ u32x4 lm_widen8_e4m3(u32x2 v) {
    u32x4 o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        o[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[h], 1.0f, false));
        o[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[h], 1.0f, true));
    }
    return o;
}

}  // namespace

template <bool WF8, bool GUMBEL>
__global__ void __launch_bounds__(LNW * 64) lmhead_kernel(GemmArgs g) {
    if (g.state && g.state[0]) return;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int N = g.N, M = g.M;
    const int n_tiles = (N + LBN - 1) / LBN;
    const int mb_max = (M + LBM - 1) / LBM;
    const int64_t items = (int64_t)((n_tiles + 7) / 8) * 8 * mb_max;
    const int KT = g.K / LKB;
    const uint16_t* Ahi = reinterpret_cast<const uint16_t*>(g.A);
    const uint16_t* Alo = reinterpret_cast<const uint16_t*>(g.A2);
    const int step = g.step_override >= 0 ? g.step_override : (g.state ? g.state[1] : 0);
    const double tau = lm_tau_at(g.sp, step);
    const float c2 = (float)(1.4426950408889634 / tau);  // log2(e) / tau
    const float inv_tau = (float)(1.0 / tau);
    using WT = std::conditional_t<WF8, uint8_t, uint16_t>;  // one weight
    using WR = std::conditional_t<WF8, u32x2, u32x4>;       // a lane's 8 weights
    // wave w: row group w % LWR, column group w / LWR
    const int wr_g = LWC == 1 ? wave : wave % LWR, wc_g = LWC == 1 ? 0 : wave / LWR;
    const int wrow0 = wr_g * 32 * LRT;                      // the wave's first row of the item
    const int wcol0 = wc_g * 32 * LCT;                      // its first column of the tile

    for (int64_t id = blockIdx.x; id < items; id += gridDim.x) {
        const int blk = (int)(id / (8 * mb_max)), rem = (int)(id % (8 * mb_max));
        const int mb = rem / 8, tile = blk * 8 + rem % 8;
        const int m0 = mb * LBM;
        if (tile >= n_tiles || m0 >= M) continue;  // uniform over the workgroup
        const int mcount = min(LBM, M - m0);
        const int n0 = tile * LBN;
        const bool live = wrow0 < mcount;          // uniform over the wave

        // Sources are recomputed at every stage rather than held in registers
        // (the accumulators and the two stages of activation fragments leave
        // few to spare). Activations: this lane's row of each row tile (rows
        // past mcount read the last one, never stored), k-half 8 hi of each
        // 16-k step. Weights: load j of this wave covers LDS row 8 (wave
        // LB_INSTR + j) + lane / 8 at position lane % 8 (logical chunk
        // lswz(row, lane % 8)); rows past N read the last one.
        WR rb[LB_INSTR];
        // activation fragments as a ring of the next RING 16-k steps: slot
        // s % RING holds step s; once the MFMAs of step s have read it, it is
        // refilled with step s + RING (of this stage or the next)
        u32x4 ra[RING][LRT][2];  // [k-step % RING][row tile][0: hi, 1: lo]
        auto load_b = [&](int kt) {
            const int64_t k0 = (int64_t)min(kt, KT - 1) * LKB;  // past the last stage: re-read it (unused)
#pragma unroll
            for (int j = 0; j < LB_INSTR; ++j) {
                const int r = 8 * (wave * LB_INSTR + j) + (lane >> 3);
                const int wr = min(n0 + r, N - 1);
                const WT* src = reinterpret_cast<const WT*>(g.W) + (int64_t)wr * g.ldw + k0 + 8 * lswz(r, lane & 7);
                rb[j] = __builtin_nontemporal_load(reinterpret_cast<const WR*>(src));
            }
        };
        // k-step s of stage kt into ring slot s % RING (past the last stage:
        // the last one again, unused)
        auto load_a = [&](int s, int kt) {
            const int64_t k0 = (int64_t)min(kt, KT - 1) * LKB + 16 * s + 8 * hi;
#pragma unroll
            for (int t = 0; t < LRT; ++t) {
                const int64_t ao = (int64_t)(m0 + min(wrow0 + 32 * t + l32, mcount - 1)) * g.lda + k0;
                ra[s % RING][t][0] = *reinterpret_cast<const u32x4*>(Ahi + ao);
                ra[s % RING][t][1] = *reinterpret_cast<const u32x4*>(Alo + ao);
            }
        };
        auto store_b = [&](int slot) {
            unsigned char* st = smem + slot * LB_BYTES;
#pragma unroll
            for (int j = 0; j < LB_INSTR; ++j) {
                u32x4 v;
                if constexpr (WF8) v = lm_widen8_e4m3(rb[j]);
                else v = rb[j];
                *reinterpret_cast<u32x4*>(st + (wave * LB_INSTR + j) * 1024 + lane * 16) = v;
            }
        };
        f32x16 acc[LRT][LCT];
#pragma unroll
        for (int t = 0; t < LRT; ++t)
#pragma unroll
            for (int j = 0; j < LCT; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[t][j][q] = 0.f;
        // stage kt from LDS slot `slot`; each k-step's activation slot is
        // refilled RING steps ahead right after use. The wave's weight
        // fragments of a k-step come in two halves; a half's reads for the
        // next k-step are issued as soon as the MFMAs of this step are done
        // with it, so they land while the other half's MFMAs run (scheduling
        // barriers keep that order).
        auto rd = [&](const unsigned char* bs, u32x4 (&dst)[LHC], int s, int jh) {
            const int c = 2 * s + hi;
#pragma unroll
            for (int jj = 0; jj < LHC; ++jj) {
                const int r = wcol0 + 32 * (LHC * jh + jj) + l32;
                dst[jj] = *reinterpret_cast<const u32x4*>(bs + r * LROWB + lswz(r, c) * 16);
            }
        };
        auto mm = [&](const u32x4 (&bh)[LHC], int s, int jh, int hl) {
#pragma unroll
            for (int jj = 0; jj < LHC; ++jj)
#pragma unroll
                for (int t = 0; t < LRT; ++t)
                    acc[t][LHC * jh + jj] = mfma32(ra[s % RING][t][hl], bh[jj], acc[t][LHC * jh + jj]);
        };
        auto compute = [&](int slot, int kt) {
            const unsigned char* bs = smem + slot * LB_BYTES;
            u32x4 bA[LHC], bB[LHC];
            rd(bs, bA, 0, 0);
            rd(bs, bB, 0, 1);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                mm(bA, s, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                mm(bB, s, 1, 0);
                __builtin_amdgcn_sched_barrier(0);
                mm(bA, s, 0, 1);
                __builtin_amdgcn_sched_barrier(0);
                if (s < 3) rd(bs, bA, s + 1, 0);
                __builtin_amdgcn_sched_barrier(0);
                mm(bB, s, 1, 1);
                __builtin_amdgcn_sched_barrier(0);
                if (s < 3) rd(bs, bB, s + 1, 1);
                if (s + RING < 4) load_a(s + RING, kt);
                else load_a(s + RING - 4, kt + 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // stage kt: its weight registers go to LDS slot kt % 2 (last read two
        // stages ago, before the previous barrier), the registers are
        // refilled with stage kt + 1, one barrier publishes the slot, then
        // the MFMAs
        if (live) {
#pragma unroll
            for (int s = 0; s < RING; ++s) load_a(s, 0);
        }
        load_b(0);
        for (int kt = 0; kt < KT; ++kt) {
            store_b(kt & 1);
            load_b(kt + 1);
            lm_lds_barrier();
            if (live) compute(kt & 1, kt);
        }
        __syncthreads();  // retire the tail loads; every wave done with the slots

        // ---- epilogue, per half of 128 columns ----
        // acc[t][j][q] is row wrow0 + 32 t + 8 (q / 4) + 4 hi + q % 4 of the
        // item, column wcol0 + 32 j + l32 of the tile. The half goes through LDS as
        // f32 (T[row][col], odd row stride: a thread per row reads without
        // bank conflicts); then the logits of record leave as bf16 in 16-byte
        // stores (16 threads per row) and thread r computes row r's partials.
        float* T = reinterpret_cast<float*>(smem);
        uint16_t* C = reinterpret_cast<uint16_t*>(g.C);
        // statistics: two threads per row (lanes 2r' and 2r'+1 of a wave),
        // each over 64 of the half's 128 columns, combined by a neighbour swap
        const int r_own = tid >> 1, hf = tid & 1;               // this thread's row of the item, its 64 columns
        const bool own_ok = r_own < mcount;
        const int bt = own_ok && g.bias_tok ? g.bias_tok[m0 + r_own] : -1;
        const float bv = own_ok && g.bias_tok ? g.bias_val[m0 + r_own] : 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ptile = 2 * tile + h;
            if (ptile >= g.nsplit) break;   // uniform: no columns in this half
            const int cb = n0 + 128 * h;    // first column of the half
            __syncthreads();                // the LDS is free (K loop, or the previous half)
            if (live) {
                // the wave's column tiles that fall in this half (with one
                // column group, tiles 4h .. 4h+3; with two, all tiles of the
                // waves of group h)
#pragma unroll
                for (int jj = 0; jj < LCT; ++jj) {
                    const int ct = wcol0 + 32 * jj - 128 * h;  // the tile's first column in the half
                    if (ct < 0 || ct >= 128) continue;
                    float sc = 1.f;
                    if constexpr (WF8) sc = bf2f(g.w_scale[min(cb + ct + l32, N - 1)]);
#pragma unroll
                    for (int t = 0; t < LRT; ++t)
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const int row = wrow0 + 32 * t + 8 * (q / 4) + 4 * hi + (q % 4);
                            T[row * TST + ct + l32] = acc[t][jj][q] * sc;
                        }
                }
            }
            __syncthreads();
            // (1) logits of record, bf16: 16 threads per row, 8 columns each
            for (int e = tid; e < mcount * 16; e += LNW * 64) {
                const int row = e >> 4, c8 = (e & 15) * 8, col = cb + c8;
                if (col >= N) continue;  // N % 8 == 0: a chunk is inside or past N
                const float* tp = T + row * TST + c8;
                u32x4 o;
#pragma unroll
                for (int u = 0; u < 4; ++u) o[u] = f2bf2(tp[2 * u], tp[2 * u + 1]);
                *reinterpret_cast<u32x4*>(C + (int64_t)(m0 + row) * g.ldc + col) = o;
            }
            // (2) row r_own's partials over the half, from the f32 values:
            // raw max and its lowest column, then the base-2 partition sum
            // and entropy partial against that max. Thread hf takes columns
            // 64 hf + ((j + 32 hf) % 64), j = 0..63: the two threads of a row
            // (and the 32 rows of a wave) read distinct LDS banks.
            {
                const float* tp = T + r_own * TST + 64 * hf;
                const bool special = (bt >= cb && bt < cb + 128) || (g.mask_id >= cb && g.mask_id < cb + 128) ||
                                     cb + 128 > N;
                auto colv = [&](int j) { return (j + 32 * hf) & 63; };
                float rawm = -INFINITY;
                int vi = 0x7fffffff;
                if (!special) {
#pragma unroll 4
                    for (int j = 0; j < 64; ++j) {
                        const int c = colv(j);
                        const float l = tp[c];
                        const int col = cb + 64 * hf + c;
                        if (l > rawm || (l == rawm && col < vi)) { rawm = l; vi = col; }
                    }
                } else {
#pragma unroll 4
                    for (int j = 0; j < 64; ++j) {
                        const int c = colv(j);
                        const int col = cb + 64 * hf + c;
                        float l = tp[c] + (col == bt ? bv : 0.f);
                        if (col >= N || col == g.mask_id) l = -INFINITY;
                        if (l > rawm || (l == rawm && col < vi)) { rawm = l; vi = col; }
                    }
                }
                // the row's max and lowest column over both threads
                {
                    const ArgMax o{__builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, rawm), 0xB1, 0xF, 0xF, false)),
                                   __builtin_amdgcn_update_dpp(0, vi, 0xB1, 0xF, 0xF, false)};
                    const ArgMax m = argmax_merge(ArgMax{rawm, vi}, o);
                    rawm = m.v;
                    vi = m.i;
                }
                const float vm = rawm * c2;
                float sa = 0.f, ta = 0.f;
                if (rawm != -INFINITY) {
                    if (!special) {
    #pragma unroll 4
                    for (int j = 0; j < 64; ++j) {
                            const float d = fmaf(tp[colv(j)], c2, -vm);
                            const float w = __builtin_amdgcn_exp2f(d);
                            sa += w;
                            ta = fmaf(w, d, ta);
                        }
                    } else {
    #pragma unroll 4
                    for (int j = 0; j < 64; ++j) {
                            const int c = colv(j);
                            const int col = cb + 64 * hf + c;
                            float l = tp[c] + (col == bt ? bv : 0.f);
                            if (col >= N || col == g.mask_id) l = -INFINITY;
                            const float d = l * c2 - vm;
                            const float w = __builtin_amdgcn_exp2f(d);
                            sa += w;
                            ta += w > 0.f ? w * d : 0.f;
                        }
                    }
                }
                sa += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, sa), 0xB1, 0xF,
                                                                            0xF, false));
                ta += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, ta), 0xB1, 0xF,
                                                                            0xF, false));
                // Gumbel-max candidate over the logits of record: the lowest
                // column maximising z - log(-log u), u from Philox at (row,
                // step, canvas, 1 + v / 4), word v % 4
                float gv = -INFINITY;
                int gi = 0x7fffffff;
                if constexpr (GUMBEL) {
                    const int grow = m0 + r_own;
                    for (int c = 64 * hf; c < 64 * hf + 64 && cb + c < N; c += 4) {
                        const u32x4 wd = philox10(u32x4{(uint32_t)grow, (uint32_t)step, (uint32_t)g.sp.canvas_idx,
                                                        (uint32_t)(1 + (cb + c) / 4)},
                                                  g.sp.seed_lo, g.sp.seed_hi);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int col = cb + c + u;
                            if (col == g.mask_id) continue;
                            const float val =
                                (round_bf(T[r_own * TST + c + u]) + (col == bt ? bv : 0.f)) * inv_tau + gumbel_of(wd[u]);
                            if (val > gv) { gv = val; gi = col; }
                        }
                    }
                    const ArgMax o{__builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, gv), 0xB1, 0xF, 0xF, false)),
                                   __builtin_amdgcn_update_dpp(0, gi, 0xB1, 0xF, 0xF, false)};
                    const ArgMax m = argmax_merge(ArgMax{gv, gi}, o);
                    gv = m.v;
                    gi = m.i;
                }
                if (own_ok && hf == 0) {
                    RowPart p;
                    p.m2 = rawm == -INFINITY ? -INFINITY : vm;
                    p.s = sa;
                    p.t = ta;
                    p.lmax = rawm;
                    p.amax = (vi == 0x7fffffff || rawm == -INFINITY) ? -1 : vi;
                    p.pad[0] = __float_as_int(gv);
                    p.pad[1] = gi == 0x7fffffff ? -1 : gi;
                    p.pad[2] = 0;
                    g.parts[(int64_t)(m0 + r_own) * g.nsplit + ptile] = p;
                }
            }
        }
        __syncthreads();  // the LDS is refilled by the next item
    }
}

bool lmhead_supported(const GemmArgs& g) {
    return !g.c_f32 && g.A2 && g.K % LKB == 0 && g.lda % 8 == 0 && g.ldw % 8 == 0 && g.ldc % 8 == 0 &&
           g.N % 8 == 0 && g.ksplit <= 1 && g.nsplit == (g.N + 127) / 128;
}

template <bool WF8, bool GUMBEL>
static hipError_t launch_lm(const GemmArgs& g, hipStream_t st) {
    auto kern = lmhead_kernel<WF8, GUMBEL>;
    static bool attr = false;
    static int per_cu = 0;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)LM_LDS);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), LNW * 64,
                                                         LM_LDS);
        if (e != hipSuccess) return e;
        per_cu = std::max(per_cu, 1);
        attr = true;
    }
    const int n_tiles = (g.N + LBN - 1) / LBN;
    const int mb = (g.M + LBM - 1) / LBM;
    const int64_t items = (int64_t)((n_tiles + 7) / 8) * 8 * mb;
    int64_t grid = std::min<int64_t>(items, 256 * per_cu);
    grid = std::max<int64_t>(8, (grid + 7) / 8 * 8);
    kern<<<(unsigned)grid, LNW * 64, LM_LDS, st>>>(g);
    return hipGetLastError();
}

hipError_t lmhead_launch(const GemmArgs& g, hipStream_t st) {
    if (!lmhead_supported(g)) return hipErrorInvalidValue;
    const bool f8 = g.w_scale != nullptr, gum = g.sp.draw_mode != 0;
    if (f8) return gum ? launch_lm<true, true>(g, st) : launch_lm<true, false>(g, st);
    return gum ? launch_lm<false, true>(g, st) : launch_lm<false, false>(g, st);
}

}  // namespace dg
