// LDS-staged grouped GEMM for gfx950 (bf16): C[m][n] = sum_k A[m][k] W[n][k]
// for the expert groups that received many rows.
//
// The expert SwiGLU layers of the MoE (DiffusionGemma model card (zh-TW),
// intro list and spec table: 8 of 128 experts active plus 1 shared expert)
// read each hit expert's weights once. When a group holds many rows, the
// register-fragment streaming kernel (gemm_stream.hip) would re-read the
// weight tile once per 64-row block and load as many activation bytes as
// weight bytes through the fragment path, whose total throughput is bounded
// well below HBM bandwidth. Here a workgroup owns up to 256 rows of one group
// (one m-block) and BN weight rows, so each weight byte is fetched once, and
// both operands arrive as whole 128-byte row segments:
//
//   * stages of 64 k: each lane loads 16-byte pieces of the A rows (gathered
//     through the permutation) and of the BN weight rows into registers, two
//     stages ahead, 8 lanes per 128-byte row segment, then writes them into
//     one of two LDS slots; chunk c of LDS row r is stored at
//     c ^ ((r >> 1) & 7) so MFMA fragment reads are conflict-free. (Register
//     loads keep overlapping with the MFMAs; LDS-direct copies measured here
//     serialise with them.) One barrier per stage;
//   * BN/16 waves: wave w owns rows [64 (w % 4), + 64) x columns
//     [64 (w / 4), + 64) (4 x 4 MFMA 16x16x32 tiles; with BN = 128 two waves
//     share a SIMD); a wave whose rows lie past the group's rows skips its
//     MFMAs (its copies of those rows read one valid row);
//   * the epilogue transposes the tile through LDS and leaves in 16-byte
//     coalesced stores: SwiGLU (BN/2 gate + BN/2 up columns of the same
//     hidden units) to bf16, or a plain f32 store.
//
// e4m3 weights (WF8): a lane loads 8 bytes (8 weights) per 16-byte LDS piece
// and widens them to bf16 before the LDS store (every e4m3 value is exact in
// bf16), so the MFMAs and the LDS layout are those of the bf16 path; the
// per-output-row scale multiplies the f32 accumulators after the K loop,
// before any epilogue or partial store.
//
// Work items (group from the big-group list, m-block, n-tile) are walked by a
// persistent grid; the m-blocks of one (group, n-tile) get ids 8 apart so they
// run on one XCD and the repeated weight reads hit its L2.
#include "common.hpp"
#include "gemm.hpp"

#include <type_traits>

// build-time tunables: weight rows per workgroup of the gate/up and down GEMMs
// (gate/up without a K split: groups of more than 256 rows, i.e. prefill
// chunks and batches of canvases; 128 measured 6% faster than 64 on a
// 131072-token prefill and 5% on four canvases)
#ifndef DG_TILE_BN_GU
#define DG_TILE_BN_GU 128
#endif
#ifndef DG_TILE_BN_DN
#define DG_TILE_BN_DN 128
#endif
#ifndef DG_TILE_BN_DENSE
#define DG_TILE_BN_DENSE 128
#endif
// rows per m-block of the dense products (256: one block for a 256-token
// canvas; 64: four blocks sharing each weight tile through L2, measured
// slower on the 256 x 8192 x 2816 projection)
#ifndef DG_TILE_BM_DENSE
#define DG_TILE_BM_DENSE 256
#endif
// weight loads as non-temporal (streamed once; measured faster HBM streaming)
#ifndef DG_TILE_W_NT
#define DG_TILE_W_NT 1
#endif
// gate/up split over K (decode-sized batches): tile width and slices
#ifndef DG_TILE_BN_GU_SPLIT
#define DG_TILE_BN_GU_SPLIT 128
#endif
#ifndef DG_GU_KSPLIT
#define DG_GU_KSPLIT 2
#endif
// stages the operand registers are loaded ahead
#ifndef DG_TILE_DEPTH
#define DG_TILE_DEPTH 2
#endif
// e4m3 -> bf16 widening of the weight tiles: 1 = the gfx950 scaled pack
// conversion at scale 1, 0 = bit manipulation
#ifndef DG_TILE_F8_HWCVT
#define DG_TILE_F8_HWCVT 1
#endif
// e4m3 weights on this kernel at all (0: they stay on the streaming kernel)
#ifndef DG_TILE_FP8
#define DG_TILE_FP8 1
#endif


namespace dg {

namespace {

constexpr int TBM = 256;                       // rows per m-block (largest)
constexpr int TBK = 64;                        // k per stage
constexpr int TROWB = TBK * 2;                 // bytes per LDS row

__device__ __forceinline__ int tswz(int r, int c) { return c ^ ((r >> 1) & 7); }

// every wave's LDS writes done and visible, without waiting for the global
// loads in flight (a __syncthreads would also wait for those)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float tsilu(float x) { return x / (1.f + __expf(-x)); }

// 8 e4m3 codes (byte j of the pair = weight j) -> 8 bf16, exact
__device__ __forceinline__ u32x4 widen8_e4m3(u32x2 v) {
    u32x4 o;
#if DG_TILE_F8_HWCVT
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        o[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[h], 1.0f, false));
        o[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[h], 1.0f, true));
    }
#else
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t a = (v[j >> 1] >> (16 * (j & 1))) & 0xffu, b = (v[j >> 1] >> (16 * (j & 1) + 8)) & 0xffu;
        o[j] = (__float_as_uint(e4m3_to_f32(a)) >> 16) | (__float_as_uint(e4m3_to_f32(b)) & 0xffff0000u);
    }
#endif
    return o;
}

// waves of a BM x BN workgroup: BM/64 row blocks; 256 rows: BN/64 (at most
// 2) column blocks; 64 rows: 4 column blocks
template <int BN, int BM>
constexpr int tile_waves() { return BM == 64 ? 4 : BN >= 128 ? 8 : BN / 16; }
// columns of one epilogue pass through LDS
template <int BN>
constexpr int tile_epi_cols() { return BN < 128 ? BN : 128; }
// two stage slots, or the epilogue tile if larger
template <int BN, int BM>
constexpr size_t tile_lds_bytes() {
    return std::max<size_t>(2 * (size_t)(BM + BN) * TROWB, (size_t)BM * (tile_epi_cols<BN>() + 4) * 4);
}

}  // namespace

// columns n..n+3 of output row `row` (columns past N are dropped)
template <int EPI>
__device__ __forceinline__ void tile_store4(const GemmArgs& g, int64_t row, int n, const float4& v) {
    const float vv[4] = {v.x, v.y, v.z, v.w};
    const bool full = n + 4 <= g.N;
    if constexpr (EPI == EPI_STORE_F32) {
        float* dst = reinterpret_cast<float*>(g.C) + row * g.ldc + n;
        if (full) *reinterpret_cast<float4*>(dst) = v;
        else for (int q = 0; q < 4 && n + q < g.N; ++q) dst[q] = vv[q];
    } else if constexpr (EPI == EPI_STORE_BF16) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(g.C) + row * g.ldc + n;
        if (full) {
            uint2 o;
            o.x = f2bf2(vv[0], vv[1]);
            o.y = f2bf2(vv[2], vv[3]);
            *reinterpret_cast<uint2*>(dst) = o;
        } else {
            for (int q = 0; q < 4 && n + q < g.N; ++q) dst[q] = f2bf(vv[q]);
        }
    } else if constexpr (EPI == EPI_RESIDUAL) {
        float* dst = g.X + row * g.ldx + n;
        if (full) {
            float4 x = *reinterpret_cast<const float4*>(dst);
            x.x += v.x; x.y += v.y; x.z += v.z; x.w += v.w;
            *reinterpret_cast<float4*>(dst) = x;
        } else {
            for (int q = 0; q < 4 && n + q < g.N; ++q) dst[q] += vv[q];
        }
    }
}

// Sum of the K-slice partials part[s][row][n] in slice order, then the
// epilogue. One thread per 4 columns.
template <int EPI>
__global__ void __launch_bounds__(256) tile_reduce_kernel(GemmArgs g) {
    if (g.state && g.state[0]) return;
    const int n4 = g.N / 4;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)g.M * n4) return;
    const int row = (int)(e / n4), n = (int)(e % n4) * 4;
    float4 acc = *reinterpret_cast<const float4*>(g.part + (int64_t)row * g.N + n);
    for (int s = 1; s < g.ksplit; ++s) {
        const float4 p = *reinterpret_cast<const float4*>(g.part + ((int64_t)s * g.M + row) * g.N + n);
        acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
    }
    tile_store4<EPI>(g, row, n, acc);
}

// Grouped split-K SwiGLU: for every slot whose group's GEMM was split, gate
// and up summed over the K slices in slice order, then h = silu(gate) * up to
// bf16. Groups of at least big_min rows were cut into ks_big slices, the
// others into ks_small; a count of 1 means that GEMM stored h itself. The
// group of a slot is found by bisection of g.group_offsets (copied to LDS
// first when there are at most SWR_LDS_OFF of them, so the bisection does not
// wait on a chain of global loads); the loads of up to 8 slices go out before
// the first add.
constexpr int SWR_LDS_OFF = 1024;
__global__ void __launch_bounds__(256) tile_swiglu_reduce_kernel(GemmArgs g, int groups, int big_min, int ks_big,
                                                                 int ks_small) {
    if (g.state && g.state[0]) return;
    __shared__ int off_s[SWR_LDS_OFF];
    const bool in_lds = groups + 1 <= SWR_LDS_OFF;
    if (in_lds) {
        for (int q = threadIdx.x; q <= groups; q += 256) off_s[q] = g.group_offsets[q];
        __syncthreads();
    }
    const int* off = in_lds ? off_s : g.group_offsets;
    const int F = g.N / 2, f4 = F / 4;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int total = off[groups];
    if (e >= (int64_t)total * f4) return;
    const int slot = (int)(e / f4), f = (int)(e % f4) * 4;
    int lo = 0, hi = groups;  // group gr with off[gr] <= slot < off[gr + 1]
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (off[mid] <= slot) lo = mid; else hi = mid;
    }
    const int ks = off[lo + 1] - off[lo] >= big_min ? ks_big : ks_small;
    if (ks <= 1) return;
    float4 gp[8], up[8];  // slices past ks load slice ks - 1 again (unused)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const float* P = g.part + ((int64_t)min(s, ks - 1) * g.M + slot) * g.N;
        gp[s] = *reinterpret_cast<const float4*>(P + f);
        up[s] = *reinterpret_cast<const float4*>(P + F + f);
    }
    float4 ga = gp[0], ua = up[0];
#pragma unroll
    for (int s = 1; s < 8; ++s) {
        if (s < ks) {
            ga.x += gp[s].x; ga.y += gp[s].y; ga.z += gp[s].z; ga.w += gp[s].w;
            ua.x += up[s].x; ua.y += up[s].y; ua.z += up[s].z; ua.w += up[s].w;
        }
    }
    for (int s = 8; s < ks; ++s) {
        const float* P = g.part + ((int64_t)s * g.M + slot) * g.N;
        const float4 gq = *reinterpret_cast<const float4*>(P + f);
        const float4 uq = *reinterpret_cast<const float4*>(P + F + f);
        ga.x += gq.x; ga.y += gq.y; ga.z += gq.z; ga.w += gq.w;
        ua.x += uq.x; ua.y += uq.y; ua.z += uq.z; ua.w += uq.w;
    }
    uint2 o;
    o.x = f2bf2(tsilu(ga.x) * ua.x, tsilu(ga.y) * ua.y);
    o.y = f2bf2(tsilu(ga.z) * ua.z, tsilu(ga.w) * ua.w);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.C) + (int64_t)slot * g.ldc + f) = o;
}

template <int BN, int EPI, int DEPTH, int BM, bool WF8>
__global__ void __launch_bounds__((tile_waves<BN, BM>() * 64)) tile_gemm_kernel(GemmArgs g, int n_tiles) {
    if (g.state && g.state[0]) return;
    static_assert(BM == 64 || BM == 256, "m-blocks of 64 or 256 rows");
    constexpr int TA_BYTES = BM * TROWB;
    constexpr int B_BYTES = BN * TROWB;
    constexpr int STAGE = TA_BYTES + B_BYTES;
    constexpr int NW = tile_waves<BN, BM>();      // waves
    constexpr int NT = NW * 64;                   // threads
    constexpr int TA_INSTR = TA_BYTES / 1024 / NW;  // 1 KB row pieces of A per wave and stage
    constexpr int B_INSTR = B_BYTES / 1024 / NW;
    constexpr int RB = BM / 64, CB = NW / RB;     // row blocks, column blocks
    constexpr int WC = BN / CB;                   // columns per wave
    constexpr int TN = WC / 16;                   // 16-column tiles per wave
    static_assert(TA_INSTR >= 1 && B_INSTR >= 1 && TN >= 1, "tile shape");
    constexpr int EP = tile_epi_cols<BN>();       // columns per epilogue pass
    constexpr int NPASS = BN / EP;
    constexpr int TS = EP + 4;  // epilogue tile row stride (floats)
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % RB, wn = wave / RB;     // row block, column block
    const int lr = lane & 15, lg = lane >> 4;
    const int pos = lane & 7;
    const bool grouped = g.group_offsets != nullptr;
    const int ngroups = grouped ? g.hit[0] : 1;
    // grouped: hit_mb counts 256-row blocks (an upper bound for 64-row ones)
    const int mb_max = grouped ? *g.hit_mb * (TBM / BM) : (g.M + BM - 1) / BM;
    const int ksplit = g.ksplit > 1 ? g.ksplit : 1;
    const int units = ngroups * n_tiles;
    const int64_t items = (int64_t)((units * ksplit + 7) / 8) * 8 * mb_max;
    const int KT = g.K / TBK / ksplit;  // stages per K slice
    const uint16_t* Ab = reinterpret_cast<const uint16_t*>(g.A);

    for (int64_t id = blockIdx.x; id < items; id += gridDim.x) {
        const int blk = (int)(id / (8 * mb_max)), rem = (int)(id % (8 * mb_max));
        const int mb = rem / 8;
        const int uk = blk * 8 + rem % 8;
        if (uk >= units * ksplit) continue;
        const int u = uk % units, ks = uk / units;
        const int gi = u / n_tiles, tile = u % n_tiles;
        const int grp = grouped ? g.hit[1 + gi] : 0;
        const int row0 = grouped ? g.group_offsets[grp] : 0;
        const int mrows = grouped ? g.group_offsets[grp + 1] - row0 : g.M;
        const int kbase = ks * KT * TBK;  // first k of this slice
        const int m0 = mb * BM;
        if (m0 >= mrows) continue;  // uniform over the workgroup
        const int mcount = min(BM, mrows - m0);
        const bool live = wm * 64 < mcount;

        // load sources: load j of this wave covers LDS rows
        // 8*(wave*TA_INSTR + j) + lane/8 (A) and 8*(wave*B_INSTR + j) + lane/8
        // (W), position lane%8, i.e. logical chunk tswz(row, lane%8)
        const uint16_t* asrc[TA_INSTR];
#pragma unroll
        for (int j = 0; j < TA_INSTR; ++j) {
            const int r = 8 * (wave * TA_INSTR + j) + (lane >> 3);
            const int rr = min(r, mcount - 1);  // past the rows: a valid row, never stored
            const int ar = row0 + m0 + rr;
            const int src = g.a_rows ? g.a_rows[ar] : ar;
            asrc[j] = Ab + (int64_t)src * g.lda + 8 * tswz(r, pos);
        }
        // weight row of tile-local column r (the B row r of the LDS tile)
        auto w_row = [&](int r, bool& second) {
            if constexpr (EPI == EPI_SWIGLU) {
                // per EP rows (one epilogue pass): EP/2 gate rows, then the up
                // rows of the same hidden units
                const int pp = r / EP, rr = r % EP;
                second = rr >= EP / 2;
                return min(tile * (BN / 2) + pp * (EP / 2) + (rr % (EP / 2)), g.N / 2 - 1);
            } else {
                second = false;
                return min(tile * BN + r, g.N - 1);
            }
        };
        using WT = std::conditional_t<WF8, uint8_t, uint16_t>;  // one weight
        using WR = std::conditional_t<WF8, u32x2, u32x4>;       // a lane's 8 weights
        const WT* bsrc[B_INSTR];
#pragma unroll
        for (int j = 0; j < B_INSTR; ++j) {
            const int r = 8 * (wave * B_INSTR + j) + (lane >> 3);
            bool second;
            const int wr = w_row(r, second);
            const WT* base = reinterpret_cast<const WT*>(second ? g.W2 : g.W);
            bsrc[j] = base + (int64_t)grp * g.w_group_stride + (int64_t)wr * g.ldw + 8 * tswz(r, pos);
        }
        // DEPTH register slots of one stage each, loaded DEPTH stages ahead;
        // loads past the last stage re-read it (branch-free, so the waits stay
        // exact)
        u32x4 ra[DEPTH][TA_INSTR];
        WR rb[DEPTH][B_INSTR];
        auto load = [&](int d, int kt) {
            const int k0 = kbase + min(kt, KT - 1) * TBK;
#pragma unroll
            for (int j = 0; j < TA_INSTR; ++j) ra[d][j] = *reinterpret_cast<const u32x4*>(asrc[j] + k0);
#pragma unroll
            for (int j = 0; j < B_INSTR; ++j) {
                const WR* src = reinterpret_cast<const WR*>(bsrc[j] + k0);
                rb[d][j] = DG_TILE_W_NT ? __builtin_nontemporal_load(src) : *src;
            }
        };
        auto store = [&](int d, int slot) {
            unsigned char* st = smem + slot * STAGE;
#pragma unroll
            for (int j = 0; j < TA_INSTR; ++j)
                *reinterpret_cast<u32x4*>(st + (wave * TA_INSTR + j) * 1024 + lane * 16) = ra[d][j];
#pragma unroll
            for (int j = 0; j < B_INSTR; ++j) {
                u32x4 v;
                if constexpr (WF8) v = widen8_e4m3(rb[d][j]);
                else v = rb[d][j];
                *reinterpret_cast<u32x4*>(st + TA_BYTES + (wave * B_INSTR + j) * 1024 + lane * 16) = v;
            }
        };

        f32x4 acc[4][TN];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto compute = [&](int d) {
            const unsigned char* as = smem + d * STAGE;
            const unsigned char* bs = as + TA_BYTES;
#pragma unroll
            for (int ks = 0; ks < TBK / 32; ++ks) {
                const int c = ks * 4 + lg;
                if constexpr (TN <= 4) {
                    u16x8 bfr[TN];
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int r = wn * WC + j * 16 + lr;
                        bfr[j] = *reinterpret_cast<const u16x8*>(bs + r * TROWB + tswz(r, c) * 16);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = wm * 64 + i * 16 + lr;
                        const u16x8 afr = *reinterpret_cast<const u16x8*>(as + r * TROWB + tswz(r, c) * 16);
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, afr), __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j], 0, 0, 0);
                    }
                } else {
                    // wide wave tiles: the 4 A fragments stay, one B fragment at a time
                    u16x8 afr[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = wm * 64 + i * 16 + lr;
                        afr[i] = *reinterpret_cast<const u16x8*>(as + r * TROWB + tswz(r, c) * 16);
                    }
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int r = wn * WC + j * 16 + lr;
                        const u16x8 bfr = *reinterpret_cast<const u16x8*>(bs + r * TROWB + tswz(r, c) * 16);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, afr[i]), __builtin_bit_cast(bf16x8, bfr), acc[i][j], 0, 0, 0);
                    }
                }
            }
        };
        // stage kt: its registers (slot kt % DEPTH) go to LDS slot kt % 2, the
        // register slot is refilled with stage kt + DEPTH, one barrier
        // publishes the LDS slot (written here, it was last read two stages
        // ago, before the previous barrier), then the MFMAs read it
        auto step = [&](int d, int slot, int kt) {
            store(d, slot);
            load(d, kt + DEPTH);
            lds_barrier();
            if (live) compute(slot);
        };
        constexpr int UNROLL = DEPTH % 2 ? 2 * DEPTH : DEPTH;
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load(d, d);
        int kt = 0;
        for (; kt + UNROLL <= KT; kt += UNROLL) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) step(u % DEPTH, u % 2, kt + u);
        }
#pragma unroll
        for (int u = 0; u + 1 < UNROLL; ++u)
            if (kt + u < KT) step(u % DEPTH, u % 2, kt + u);
        __syncthreads();  // retire the tail loads; every wave done with the slots
        if constexpr (WF8) {
            // per-output-row scales: column wn*WC + j*16 + lr of the tile
            if (live) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    bool second;
                    const int wr = w_row(wn * WC + j * 16 + lr, second);
                    const uint16_t* sc = second ? g.w2_scale : g.w_scale;
                    const float s = __uint_as_float((uint32_t)sc[(int64_t)grp * g.scale_group_stride + wr] << 16);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i][j] *= s;
                }
            }
        }

        // ---- epilogue: per pass of EP columns, the tile through LDS, then
        // coalesced row stores; ptile numbers EP-column tiles ----
        float* T = reinterpret_cast<float*>(smem);
#pragma unroll 1
        for (int p = 0; p < NPASS; ++p) {
        const int ptile = tile * NPASS + p;
        __syncthreads();
        if (live) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int c = wn * WC + j * 16 - p * EP;  // a whole 16-column tile is in the pass or not
                if (c < 0 || c >= EP) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        T[(wm * 64 + i * 16 + lg * 4 + q) * TS + c + lr] = acc[i][j][q];
            }
        }
        __syncthreads();
        if (ksplit > 1) {
            // raw f32 partial of this K slice: part[ks][row][n] (SwiGLU: gate
            // columns f at n = f, up columns at n = N/2 + f)
            constexpr int CH = EP / 4;
            float* P = g.part + (int64_t)ks * g.M * g.N;
            for (int e = tid; e < mcount * CH; e += NT) {
                const int r = e / CH, c0 = (e % CH) * 4;
                int n;
                if constexpr (EPI == EPI_SWIGLU) {
                    const int f = ptile * (EP / 2) + (c0 % (EP / 2));
                    if (f >= g.N / 2) continue;
                    n = (c0 < EP / 2 ? 0 : g.N / 2) + f;
                } else {
                    n = ptile * EP + c0;
                    if (n >= g.N) continue;
                }
                const float4 v = *reinterpret_cast<const float4*>(T + r * TS + c0);
                *reinterpret_cast<float4*>(P + (int64_t)(row0 + m0 + r) * g.N + n) = v;  // N % 8 == 0
            }
        } else if constexpr (EPI == EPI_SWIGLU) {
            constexpr int CH = EP / 2 / 8;  // 8-column chunks of hidden units per row
            uint16_t* C = reinterpret_cast<uint16_t*>(g.C);
            const int f0 = ptile * (EP / 2), F = g.N / 2;
            for (int e = tid; e < mcount * CH; e += NT) {
                const int r = e / CH, c0 = (e % CH) * 8;
                const int f = f0 + c0;
                if (f >= F) continue;
                const float* gt = T + r * TS + c0;
                const float* up = gt + EP / 2;
                uint16_t h[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) h[q] = f2bf(tsilu(gt[q]) * up[q]);
                uint16_t* dst = C + (int64_t)(row0 + m0 + r) * g.ldc + f;
                if (f + 8 <= F) {
                    uint4 v;
                    v.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                    v.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                    v.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
                    v.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
                    *reinterpret_cast<uint4*>(dst) = v;
                } else {
                    for (int q = 0; q < 8 && f + q < F; ++q) dst[q] = h[q];
                }
            }
        } else {
            constexpr int CH = EP / 4;  // float4 chunks per row
            const int n0 = ptile * EP;
            for (int e = tid; e < mcount * CH; e += NT) {
                const int r = e / CH, c0 = (e % CH) * 4;
                const int n = n0 + c0;
                if (n >= g.N) continue;
                const float4 v = *reinterpret_cast<const float4*>(T + r * TS + c0);
                const int64_t row = row0 + m0 + r;
                tile_store4<EPI>(g, row, n, v);
            }
        }
        }  // passes
        __syncthreads();  // the LDS is refilled by the next item
    }
}

template <int BN, int EPI, int DEPTH = DG_TILE_DEPTH, int BM = TBM, bool WF8 = false>
static hipError_t launch_tile_t(const GemmArgs& g, int groups, int max_rows, hipStream_t st) {
    const int n_tiles = EPI == EPI_SWIGLU ? (g.N / 2 + BN / 2 - 1) / (BN / 2) : (g.N + BN - 1) / BN;
    const int mb_max = std::max(1, (max_rows + BM - 1) / BM);
    const int ks = g.ksplit > 1 ? g.ksplit : 1;
    const int64_t items = (int64_t)((groups * n_tiles * ks + 7) / 8) * 8 * mb_max;  // upper bound
    const size_t lds = tile_lds_bytes<BN, BM>();
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(tile_gemm_kernel<BN, EPI, DEPTH, BM, WF8>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    // persistent grid: as many workgroups as fit on the 256 CUs, a multiple of 8
    static int per_cu = 0;
    if (!per_cu) {
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(tile_gemm_kernel<BN, EPI, DEPTH, BM, WF8>), tile_waves<BN, BM>() * 64, lds);
        if (e != hipSuccess) return e;
        per_cu = std::max(per_cu, 1);
    }
    int64_t grid = std::min<int64_t>(items, 256 * per_cu);
    grid = std::max<int64_t>(8, (grid + 7) / 8 * 8);
    tile_gemm_kernel<BN, EPI, DEPTH, BM, WF8><<<(unsigned)grid, tile_waves<BN, BM>() * 64, lds, st>>>(g, n_tiles);
    if (ks > 1 && !g.group_offsets && !g.defer_reduce) {  // grouped or deferred: the caller's reduce
        const int64_t n = (int64_t)g.M * (g.N / 4);
        tile_reduce_kernel<EPI><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(g);
    }
    return hipGetLastError();
}

bool tile_gemm_supported(const GemmArgs& g, int act_f32, int w_fp8, int epi) {
    if (act_f32 || (w_fp8 != 0) != (g.w_scale != nullptr) || (w_fp8 && !DG_TILE_FP8)) return false;
    if (w_fp8 && epi == EPI_SWIGLU && !g.w2_scale) return false;
    if (g.K % TBK || g.lda % 8 || g.ldw % 8) return false;
    switch (epi) {
        case EPI_SWIGLU: return !g.c_f32 && g.ldc % 8 == 0 && (g.N / 2) % 8 == 0;
        case EPI_STORE_F32: return g.ldc % 4 == 0 && g.N % 4 == 0;
        case EPI_STORE_BF16: return g.ldc % 4 == 0 && g.N % 4 == 0;
        case EPI_RESIDUAL: return g.ldx % 4 == 0 && g.N % 4 == 0;
        default: return false;
    }
}

int tile_dense_ksplit(int M, int N, int K) {
    // split until there are enough work items for most CUs (each slice keeps
    // at least 4 stages); every split adds M x N f32 partials to write and read
    const int items = (N + DG_TILE_BN_DENSE - 1) / DG_TILE_BN_DENSE * ((M + DG_TILE_BM_DENSE - 1) / DG_TILE_BM_DENSE);
    int ks = 1;
    while (items * ks < 160 && (K / TBK) % (ks * 2) == 0 && K / TBK / (ks * 2) >= 4) ks *= 2;
    return ks;
}

int tile_grouped_ksplit(int rows) { return rows <= TBM ? DG_GU_KSPLIT : 1; }

hipError_t swiglu_reduce_launch(const GemmArgs& g, int groups, int big_min, int ks_big, int ks_small, hipStream_t st) {
    if (!g.part || (g.N / 2) % 4 || g.c_f32) return hipErrorInvalidValue;
    const int64_t n = (int64_t)g.M * (g.N / 8);
    tile_swiglu_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(g, groups, big_min, ks_big, ks_small);
    return hipGetLastError();
}

template <bool WF8>
static hipError_t tile_gemm_launch_w(const GemmArgs& g, int epi, int groups, int max_rows, hipStream_t st) {
    constexpr int D = DG_TILE_DEPTH;
    if (g.group_offsets) {
        if (g.ksplit > 1) {
            // SwiGLU over K slices: partials [ksplit][M slots][2F], M = all
            // slots; swiglu_reduce_launch finishes them
            if (epi != EPI_SWIGLU || !g.part || (g.K / TBK) % g.ksplit || (g.N / 2) % 4) return hipErrorInvalidValue;
            return launch_tile_t<DG_TILE_BN_GU_SPLIT, EPI_SWIGLU, D, TBM, WF8>(g, groups, max_rows, st);
        }
        if (epi == EPI_SWIGLU) return launch_tile_t<DG_TILE_BN_GU, EPI_SWIGLU, D, TBM, WF8>(g, groups, max_rows, st);
        if (epi == EPI_STORE_F32)
            return launch_tile_t<DG_TILE_BN_DN, EPI_STORE_F32, D, TBM, WF8>(g, groups, max_rows, st);
        return hipErrorInvalidValue;
    }
    if (g.ksplit > 1 && (!g.part || (g.K / TBK) % g.ksplit)) return hipErrorInvalidValue;
    constexpr int BMD = DG_TILE_BM_DENSE;
    if (epi == EPI_STORE_BF16) return launch_tile_t<DG_TILE_BN_DENSE, EPI_STORE_BF16, D, BMD, WF8>(g, 1, g.M, st);
    if (epi == EPI_RESIDUAL) return launch_tile_t<DG_TILE_BN_DENSE, EPI_RESIDUAL, D, BMD, WF8>(g, 1, g.M, st);
    if (epi == EPI_STORE_F32) return launch_tile_t<DG_TILE_BN_DENSE, EPI_STORE_F32, D, BMD, WF8>(g, 1, g.M, st);
    return hipErrorInvalidValue;
}

hipError_t tile_gemm_launch(const GemmArgs& g, int epi, int groups, int max_rows, hipStream_t st) {
    if (!g.w_scale) return tile_gemm_launch_w<false>(g, epi, groups, max_rows, st);
    if (epi == EPI_SWIGLU && !g.w2_scale) return hipErrorInvalidValue;
    return tile_gemm_launch_w<true>(g, epi, groups, max_rows, st);
}

}  // namespace dg
