// Grouped expert GEMMs: up (gathered x rows -> GELU(x W1^T + b1)) and
// down (H rows -> H W2^T + b2), one weight panel per expert group.
//
// "The expert group activated per token" (wmrh.cn), sec. 3.1: each expert
// is FFN(x) = W2 GELU(W1 x + b1) + b2; "AI-Research-SKILLs MoE training
// guide", sec. 3.1: Linear(h, 4h) -> GELU -> Linear(4h, h) on the rows
// routed to that expert; "MoE architecture deep dive", sec. 3: the shared
// expert sees every token (group E here).
//
// Work decomposition.  The per-expert row counts exist only on the device,
// so each block rebuilds the tile table (tiles per group, n-tile major,
// m-tile minor) in LDS from offsets[] and then walks it persistently.
// Logical tile L of round r goes to block (xcd, local) with
// L = r * grid + xcd * grid/8 + local: the 8 XCDs each take a contiguous
// run of tiles, so the m-tiles that share one weight panel run on the same
// XCD and hit its L2.
//
// The kernels, by group size (the host picks one per GEMM, see the
// variant ids in kernels.h):
//   gemm_ring     groups of <= 16 rows (decode): weights through a
//                 four-stage LDS ring in 1-2 KB row runs, non-temporal;
//   gemm_stream   groups of <= 32 rows: weights straight into MFMA
//                 fragments, K split over four waves;
//   gemm_bf16_lds / _dma / _dma64   BM x BN x 64 tiles staged through LDS
//                 (registers, or direct-to-LDS loads), 4 or 8 waves with
//                 v_mfma_f32_32x32x16_bf16;
//   gemm_bf16_w4  256 x 256 tiles, one wave per SIMD holding 128 x 128 in
//                 256 accumulators (16x16x32 MFMAs issued in a fixed
//                 order), half-height tiles for a group's last <= 128 rows,
//                 optionally split over K, or 224-row tiles for groups
//                 split evenly;
//   gemm_bf16_x2  128 x 256 tiles, two blocks per CU (selectable only:
//                 slower than gemm_bf16_w4 on every measured shape);
//   gemm_f32_simt the fp32 layer on the vector ALUs.
// Common to the tiled kernels: 16-byte-chunk XOR swizzles that keep the
// fragment reads free of bank conflicts (checked with rocprof's LDS
// conflict counter on gfx950, whose ds_read_b128 passes do not follow a
// plain 64-bank model), the A operand of the up pass gathered on load
// through slot_token[], bias and activation in the epilogue.
#include "kernels.h"

namespace {

constexpr int BK = 64;

// Global -> registers: this thread's 16-byte chunks of the A and B tiles
// at k offset ko.  Tile rows past the group's end carry offset 0 (row 0,
// always valid memory): they only feed output rows that are never stored,
// so they need no zeroing (and no wait on the load).
template <int AC, int BC>
__device__ __forceinline__ void tile_gload(u32x4 (&ra)[AC], u32x4 (&rb)[BC],
                                           const uint16_t *A,
                                           const int (&aoff)[AC],
                                           const uint16_t *const (&bp)[BC],
                                           int ko) {
#pragma unroll
    for (int i = 0; i < AC; ++i) ra[i] = *(const u32x4 *)(A + aoff[i] + ko);
#pragma unroll
    for (int i = 0; i < BC; ++i) rb[i] = *(const u32x4 *)(bp[i] + ko);
}

// Registers -> one LDS stage; chunk c of row r lands at r*8 + (c ^ (r/2 % 8)).
template <int AC, int BC, int BM, int RPP>
__device__ __forceinline__ void tile_sstore(const u32x4 (&ra)[AC],
                                            const u32x4 (&rb)[BC], u32x4 *sA,
                                            int lrow, int lc) {
    u32x4 *sB = sA + BM * 8;
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        const int rr = lrow + i * RPP;
        sA[rr * 8 + (lc ^ ((rr >> 1) & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) {
        const int rr = lrow + i * RPP;
        sB[rr * 8 + (lc ^ ((rr >> 1) & 7))] = rb[i];
    }
}

// LDS -> registers: the MFMA fragments of sub-step kk (16 k values) of one
// stage for this wave's TM row tiles (A) and TN column tiles (B).
// BMX: rows of the tile being computed, at most the BM rows the stage
// holds (the eight-wave kernel runs a group of <= 256 rows in its 320-row
// stages as a 256-row tile).
template <int BM, int BN, int WM, int WN, int TM, int TN, int BMX = BM>
__device__ __forceinline__ void load_frags(bf16x8 (&af)[TM], bf16x8 (&bf)[TN],
                                           const u32x4 *stage, int wm, int wn,
                                           int lane, int kk) {
    static_assert(BMX <= BM && TM * 32 * WM == BMX, "tile rows");
    const u32x4 *sA = stage;
    const u32x4 *sB = stage + BM * 8;
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int ar = wm * (BMX / WM) + i * 32 + (lane & 31);
        af[i] = as_bf16x8(sA[ar * 8 + (c ^ ((ar >> 1) & 7))]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int br = wn * (BN / WN) + j * 32 + (lane & 31);
        bf[j] = as_bf16x8(sB[br * 8 + (c ^ ((br >> 1) & 7))]);
    }
}

// acc[i][j] += B_j^T A_i for one 16-deep sub-step (weight fragment as the
// MFMA A operand: each lane ends with 4 consecutive features of one row).
template <int TM, int TN>
__device__ __forceinline__ void mfma_block(floatx16 (&acc)[TM][TN],
                                           const bf16x8 (&af)[TM],
                                           const bf16x8 (&bf)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i],
                                                               acc[i][j], 0, 0, 0);
}

// Epilogue of the 32x32-MFMA tile kernels.  The lane holds row
// m = lane%32 of each 32x32 block and features 8*q + 4*(lane/32) + 0..3
// (q = 0..3).  Ungated: bias, then GELU or SiLU on the up pass, one 8-byte
// store per q.  Gated (SwiGLU up pass): blocks j and j+1 of a wave are the
// gate and up halves of one 64-column chunk c of the virtual panel, so the
// lane forms SiLU(gate + b1) * (up + b3) for features 32*c + 8*q +
// 4*(lane/32) + 0..3 itself (the host only picks tiles whose waves cover
// whole 64-column chunks).
template <int BM, int BN, int WM, int WN, int TM, int TN, bool UP>
__device__ __forceinline__ void store_tile(const GemmParams &p,
                                           const floatx16 (&acc)[TM][TN],
                                           bool routed, int g, int row0,
                                           int nrows, int n0, int wm, int wn,
                                           int lane) {
    uint16_t *out = (uint16_t *)p.out;
    if (UP && p.gated) {
        const int F = p.N >> 1;
        const uint16_t *b1 = routed
            ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * F : nullptr)
            : (const uint16_t *)p.bias_s;
        const uint16_t *b3 = routed
            ? (p.bias3 ? (const uint16_t *)p.bias3 + (size_t)g * F : nullptr)
            : (const uint16_t *)p.bias_s3;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = wm * (BM / WM) + i * 32 + (lane & 31);
            if (m >= nrows) continue;
            uint16_t *orow = out + (size_t)(row0 + m) * p.ldo;
#pragma unroll
            for (int j = 0; j + 1 < TN; j += 2) {
                const int f0 = (n0 + wn * (BN / WN) + j * 32) >> 1;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int f = f0 + 8 * q + 4 * (lane >> 5);
                    float h[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float gv = acc[i][j][4 * q + r];
                        float uv = acc[i][j + 1][4 * q + r];
                        if (b1) gv += bf16_to_f32(b1[f + r]);
                        if (b3) uv += bf16_to_f32(b3[f + r]);
                        h[r] = silu_f(gv) * uv;
                    }
                    u32x2 o;
                    o.x = pack_bf16x2(h[0], h[1]);
                    o.y = pack_bf16x2(h[2], h[3]);
                    *(u32x2 *)(orow + f) = o;
                }
            }
        }
        return;
    }
    const uint16_t *bg = routed
        ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * p.N : nullptr)
        : (const uint16_t *)p.bias_s;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int m = wm * (BM / WM) + i * 32 + (lane & 31);
        if (m >= nrows) continue;
        uint16_t *orow = out + (size_t)(row0 + m) * p.ldo;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * (BN / WN) + j * 32 + 8 * q +
                              4 * (lane >> 5);
                float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
                float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
                if (bg) {
                    const u32x2 bb = *(const u32x2 *)(bg + n);
                    v0 += bf16_lo(bb.x);
                    v1 += bf16_hi(bb.x);
                    v2 += bf16_lo(bb.y);
                    v3 += bf16_hi(bb.y);
                }
                if (UP) {
                    v0 = act_up(p.act, v0);
                    v1 = act_up(p.act, v1);
                    v2 = act_up(p.act, v2);
                    v3 = act_up(p.act, v3);
                }
                u32x2 o;
                o.x = pack_bf16x2(v0, v1);
                o.y = pack_bf16x2(v2, v3);
                *(u32x2 *)(orow + n) = o;
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, bool UP>
__global__ __launch_bounds__(WM *WN * 64, 1) void gemm_bf16_lds(GemmParams p) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / (WM * 32);
    constexpr int TN = BN / (WN * 32);
    constexpr int AC = BM * 8 / NT;      // 16-byte A chunks per thread
    constexpr int BC = BN * 8 / NT;      // 16-byte B chunks per thread
    constexpr int RPP = NT / 8;          // tile rows per load pass
    constexpr int STAGE = (BM + BN) * 8; // 16-byte units per stage
    static_assert(AC >= 1 && BC >= 1, "tile too small for the block");
    extern __shared__ u32x4 smem[];
    __shared__ TileTable tt;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int N = p.N, K = p.K, KT = K / BK;
    const int NTN = N / BN;
    const int G = p.E + p.n_shared;
    build_tile_table(tt, p.offsets, p.E, p.n_shared, p.shared_base, p.T, BM,
                     NTN);
    const int total = tt.base[G];
    const int nb = gridDim.x, per = nb >> 3;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const uint16_t *A = (const uint16_t *)p.A;
    const int lrow = tid >> 3, lc = tid & 7;

    for (int r = 0;; ++r) {
        const int L = r * nb + xcd * per + loc;
        if (L >= total) break;
        const int g = find_group(tt, G, L);
        const int local = L - tt.base[g];
        const int mt = tt.mt[g];
        const int n_tile = local / mt, m_tile = local - n_tile * mt;
        const int row0 = tt.start[g] + m_tile * BM;
        const int nrows = min(BM, tt.rows[g] - m_tile * BM);
        const int n0 = n_tile * BN;
        const bool routed = g < p.E;

        int aoff[AC];
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int rr = lrow + i * RPP;
            aoff[i] = lc * 8;
            if (rr < nrows) {
                const int slot = row0 + rr;
                int src = slot;
                if (UP) src = routed ? p.slot_token[slot] : slot - p.shared_base;
                aoff[i] = src * K + lc * 8;
            }
        }
        const uint16_t *bp[BC];
#pragma unroll
        for (int i = 0; i < BC; ++i)
            bp[i] = (const uint16_t *)weight_row(p, routed, g,
                                                 n0 + lrow + i * RPP, 2) +
                    lc * 8;

        floatx16 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        // Software pipeline: global loads of step kt+1 are in flight while
        // step kt computes; within a step the LDS fragments of sub-step
        // kk+1 are read while the MFMAs of sub-step kk run, and the first
        // fragments of the next step are read right after the barrier,
        // under the last sub-step's MFMAs.
        u32x4 ra[AC], rb[BC];
        tile_gload<AC, BC>(ra, rb, A, aoff, bp, 0);
        tile_sstore<AC, BC, BM, RPP>(ra, rb, smem, lrow, lc);
        __syncthreads();
        bf16x8 fa[2][TM], fb[2][TN];
        load_frags<BM, BN, WM, WN, TM, TN>(fa[0], fb[0], smem, wm, wn, lane, 0);
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < KT;
            if (more)
                tile_gload<AC, BC>(ra, rb, A, aoff, bp, (kt + 1) * BK);
            const u32x4 *stage = smem + cur * STAGE;
#pragma unroll
            for (int kk = 0; kk < BK / 16 - 1; ++kk) {
                load_frags<BM, BN, WM, WN, TM, TN>(fa[(kk + 1) & 1],
                                                   fb[(kk + 1) & 1], stage,
                                                   wm, wn, lane, kk + 1);
                mfma_block<TM, TN>(acc, fa[kk & 1], fb[kk & 1]);
            }
            if (more)
                tile_sstore<AC, BC, BM, RPP>(ra, rb, smem + (cur ^ 1) * STAGE,
                                             lrow, lc);
            __syncthreads();
            constexpr int LAST = (BK / 16 - 1) & 1;
            if (more)
                load_frags<BM, BN, WM, WN, TM, TN>(fa[LAST ^ 1], fb[LAST ^ 1],
                                                   smem + (cur ^ 1) * STAGE,
                                                   wm, wn, lane, 0);
            mfma_block<TM, TN>(acc, fa[LAST], fb[LAST]);
        }
        __syncthreads();   // LDS is reused by the next tile's prologue
        store_tile<BM, BN, WM, WN, TM, TN, UP>(p, acc, routed, g, row0, nrows,
                                               n0, wm, wn, lane);
    }
}

// ---------------------------------------------------------------------
// bf16 kernel with direct global->LDS loads (global_load_lds_dwordx4) into
// an NS-stage ring of BM x 32 / BN x 32 tiles.  Loads run NS-1 stages ahead
// of the MFMAs without holding registers, which hides L2-miss latency that
// a one-step register prefetch cannot.  One wave instruction fills 16 rows
// (64 bytes each) of a tile; lane i writes row i/4, 16-byte slot i%4, and
// fetches the k-chunk (i%4) ^ ((row/4) % 4) so that the fragment reads
// (32 rows at one chunk) are free of bank conflicts.
constexpr int BKD = 32;

__device__ __forceinline__ void dma16(const uint16_t *src, u32x4 *lds_row16) {
    __builtin_amdgcn_global_load_lds(
        (const void *)src,
        (__attribute__((address_space(3))) void *)lds_row16, 16, 0, 0);
}

// The same load with the non-temporal hint, for weight panels that only
// one row tile reads: their lines are not kept in the caches at the
// expense of the gathered token rows, which every column tile of the group
// reads again.  (Measured on the Expert-Choice-shaped layer, one 256-row
// tile per expert: up GEMM 136 -> 131 us, 192-column down GEMM 124 -> 104,
// layer 292 -> 272 us; DeepSeek-shaped up GEMM, 320-row tiles, 2.48 -> 2.41
// ms.  Where two or more row tiles share a panel through L2 it is slower:
// with every weight load non-temporal the DeepSeek-shaped down GEMM, whose
// groups of 257..384 rows run as two tiles on one panel, took 2.44 -> 2.78
// ms, and even there its one-tile groups alone gained nothing.)
__device__ __forceinline__ void dma16_nt(const void *src, u32x4 *lds) {
    __builtin_amdgcn_global_load_lds(
        src, (__attribute__((address_space(3))) void *)lds, 16, 0,
        2 /* non-temporal */);
}

// s_waitcnt vmcnt(n) only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) |
                               (0xF << 8));
}


// LDS -> registers: both 16-deep sub-steps of one BKD = 32 stage.
template <int BM, int BN, int WM, int WN, int TM, int TN>
__device__ __forceinline__ void read_stage(bf16x8 (&fa)[2][TM],
                                           bf16x8 (&fb)[2][TN],
                                           const u32x4 *stage, int wm, int wn,
                                           int lane) {
    const u32x4 *sA = stage;
    const u32x4 *sB = stage + BM * 4;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int c = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int ar = wm * (BM / WM) + i * 32 + (lane & 31);
            fa[kk][i] = as_bf16x8(sA[ar * 4 + (c ^ ((ar >> 2) & 3))]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int br = wn * (BN / WN) + j * 32 + (lane & 31);
            fb[kk][j] = as_bf16x8(sB[br * 4 + (c ^ ((br >> 2) & 3))]);
        }
    }
}

template <int BM, int BN, int WM, int WN, bool UP, int NS>
__global__ __launch_bounds__(WM *WN * 64, 1) void gemm_bf16_dma(GemmParams p) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / (WM * 32);
    constexpr int TN = BN / (WN * 32);
    constexpr int IA = BM / 16 / NW;      // A load instructions per wave
    constexpr int IB = BN / 16 / NW;      // B load instructions per wave
    constexpr int PER = IA + IB;          // per wave per stage
    constexpr int STAGE = (BM + BN) * 4;  // 16-byte units per stage
    static_assert(IA * NW * 16 == BM && IB * NW * 16 == BN, "tile split");
    static_assert(NS >= 3 && (NS - 2) * PER < 64, "vmcnt range");
    extern __shared__ u32x4 smem[];
    __shared__ TileTable tt;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int N = p.N, K = p.K, KT = K / BKD;
    const int NTN = N / BN;
    const int G = p.E + p.n_shared;
    build_tile_table(tt, p.offsets, p.E, p.n_shared, p.shared_base, p.T, BM,
                     NTN);
    const int total = tt.base[G];
    const int nb = gridDim.x, per = nb >> 3;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const uint16_t *A = (const uint16_t *)p.A;
    const int lr = lane >> 2;                       // row within 16
    const int lp = lane & 3;                        // 16-byte slot

    for (int r = 0;; ++r) {
        const int L = r * nb + xcd * per + loc;
        if (L >= total) break;
        const int g = find_group(tt, G, L);
        const int local = L - tt.base[g];
        const int mt = tt.mt[g];
        const int n_tile = local / mt, m_tile = local - n_tile * mt;
        const int row0 = tt.start[g] + m_tile * BM;
        const int nrows = min(BM, tt.rows[g] - m_tile * BM);
        const int n0 = n_tile * BN;
        const bool routed = g < p.E;

        // per-lane sources of each load instruction; tile rows past the
        // group's end read row 0 and are never stored
        int aoff[IA];
        const uint16_t *bp[IB];
#pragma unroll
        for (int j = 0; j < IA; ++j) {
            const int rr = (wave + j * NW) * 16 + lr;
            const int ch = lp ^ ((rr >> 2) & 3);
            int src = 0;
            if (rr < nrows) {
                const int slot = row0 + rr;
                src = slot;
                if (UP) src = routed ? p.slot_token[slot] : slot - p.shared_base;
            }
            aoff[j] = src * K + ch * 8;
        }
#pragma unroll
        for (int j = 0; j < IB; ++j) {
            const int rr = (wave + j * NW) * 16 + lr;
            const int ch = lp ^ ((rr >> 2) & 3);
            bp[j] = (const uint16_t *)weight_row(p, routed, g, n0 + rr, 2) +
                    ch * 8;
        }
        auto issue = [&](int ks) __attribute__((always_inline)) {
            u32x4 *st = smem + (ks % NS) * STAGE;
            const int ko = ks * BKD;
#pragma unroll
            for (int j = 0; j < IA; ++j)
                dma16(A + aoff[j] + ko, st + (wave + j * NW) * 64);
#pragma unroll
            for (int j = 0; j < IB; ++j)
                dma16(bp[j] + ko, st + BM * 4 + (wave + j * NW) * 64);
        };

        floatx16 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        // Stage kt's fragments sit in registers while stage kt+1's are
        // read from LDS, so every wave's LDS reads overlap its own (and its
        // SIMD neighbour's) MFMAs instead of all waves reading, then all
        // computing, between barriers.  At iteration kt: wait until this
        // wave's loads of stage kt+1 have landed, barrier (all waves' loads
        // landed; all waves finished reading stage kt-1), refill the slot of
        // stage kt-1 with stage kt+NS-1, read stage kt+1, compute stage kt.
        wait_vmcnt<0>();   // previous tile's stores and loads are done
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < KT) issue(s);
        bf16x8 fa[2][2][TM], fb[2][2][TN];   // [buffer][sub-step][tile]
        if (KT > 1) wait_vmcnt<(NS - 2) * PER>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        read_stage<BM, BN, WM, WN, TM, TN>(fa[0], fb[0], smem, wm, wn, lane);
        auto step = [&](int kt, bf16x8 (&fa_cur)[2][TM],
                        bf16x8 (&fb_cur)[2][TN], bf16x8 (&fa_nxt)[2][TM],
                        bf16x8 (&fb_nxt)[2][TN]) __attribute__((always_inline)) {
            if (kt + 1 < KT) {
                if (kt + NS - 2 < KT) wait_vmcnt<(NS - 3) * PER>();
                else wait_vmcnt<0>();
                __builtin_amdgcn_s_barrier();
                if (kt + NS - 1 < KT) issue(kt + NS - 1);
                read_stage<BM, BN, WM, WN, TM, TN>(
                    fa_nxt, fb_nxt, smem + ((kt + 1) % NS) * STAGE, wm, wn,
                    lane);
            }
            mfma_block<TM, TN>(acc, fa_cur[0], fb_cur[0]);
            mfma_block<TM, TN>(acc, fa_cur[1], fb_cur[1]);
        };
        for (int kt = 0; kt < KT; kt += 2) {
            step(kt, fa[0], fb[0], fa[1], fb[1]);
            if (kt + 1 < KT) step(kt + 1, fa[1], fb[1], fa[0], fb[0]);
        }
        __syncthreads();   // the ring is reused by the next tile
        store_tile<BM, BN, WM, WN, TM, TN, UP>(p, acc, routed, g, row0, nrows,
                                               n0, wm, wn, lane);
    }
}

// ---------------------------------------------------------------------
// bf16 kernel with direct global->LDS loads and 64-deep stages: every row
// of a stage is one whole 128-byte line, so each L1->L2 request moves a
// full line (32-deep stages move half lines and double the L2 request
// rate, which is what saturates the L2 first).  Two stages: the loads of
// stage kt+1 are issued at the start of step kt and land during its
// MFMAs.  One wave instruction fills 8 rows; lane i writes row i/8, slot
// i%8 and fetches k-chunk (i%8) ^ ((row/2) % 8), the swizzle that keeps
// the fragment reads conflict-free.
template <int BM, int BN, int WM, int WN, bool UP>
__global__ __launch_bounds__(WM *WN * 64, 1) void gemm_bf16_dma64(GemmParams p) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / (WM * 32);
    constexpr int TN = BN / (WN * 32);
    constexpr int IA = BM / 8 / NW;       // A load instructions per wave
    constexpr int IB = BN / 8 / NW;       // B load instructions per wave
    constexpr int STAGE = (BM + BN) * 8;  // 16-byte units per stage
    static_assert(IA * NW * 8 == BM && IB * NW * 8 == BN, "tile split");
    extern __shared__ u32x4 smem[];
    __shared__ TileTable tt;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
    const int wm = wave / WN, wn = wave % WN;
    const int N = p.N, K = p.K, KT = K / BK;
    const int NTN = N / BN;
    const int G = p.E + p.n_shared;
    build_tile_table(tt, p.offsets, p.E, p.n_shared, p.shared_base, p.T, BM,
                     NTN);
    const int total = tt.base[G];
    const int nb = gridDim.x, per = nb >> 3;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const uint16_t *A = (const uint16_t *)p.A;
    const int lr = lane >> 3;                       // row within 8
    const int lp = lane & 7;                        // 16-byte slot

    for (int r = 0;; ++r) {
        const int L = r * nb + xcd * per + loc;
        if (L >= total) break;
        const int g = find_group(tt, G, L);
        const int local = L - tt.base[g];
        const int mt = tt.mt[g];
        const int n_tile = local / mt, m_tile = local - n_tile * mt;
        const int row0 = tt.start[g] + m_tile * BM;
        const int nrows = min(BM, tt.rows[g] - m_tile * BM);
        const int n0 = n_tile * BN;
        const bool routed = g < p.E;

        int aoff[IA];
        const uint16_t *bp[IB];
#pragma unroll
        for (int j = 0; j < IA; ++j) {
            const int rr = (wave + j * NW) * 8 + lr;
            const int ch = lp ^ ((rr >> 1) & 7);
            int src = 0;
            if (rr < nrows) {
                const int slot = row0 + rr;
                src = slot;
                if (UP) src = routed ? p.slot_token[slot] : slot - p.shared_base;
            }
            aoff[j] = src * K + ch * 8;
        }
#pragma unroll
        for (int j = 0; j < IB; ++j) {
            const int rr = (wave + j * NW) * 8 + lr;
            const int ch = lp ^ ((rr >> 1) & 7);
            bp[j] = (const uint16_t *)weight_row(p, routed, g, n0 + rr, 2) +
                    ch * 8;
        }
        // a weight panel that only this row tile reads is streamed
        // non-temporally (uniform per tile)
        const bool nt_b = mt == 1;
        // 8-row groups wholly past the group's end are not loaded (their
        // stale LDS rows only feed outputs that are never stored)
        auto issue = [&](int ks) __attribute__((always_inline)) {
            u32x4 *st = smem + (ks & 1) * STAGE;
            const int ko = ks * BK;
#pragma unroll
            for (int j = 0; j < IA; ++j)
                if ((wave + j * NW) * 8 < nrows)
                    dma16(A + aoff[j] + ko, st + (wave + j * NW) * 64);
            if (nt_b) {
#pragma unroll
                for (int j = 0; j < IB; ++j)
                    dma16_nt(bp[j] + ko, st + BM * 8 + (wave + j * NW) * 64);
            } else {
#pragma unroll
                for (int j = 0; j < IB; ++j)
                    dma16(bp[j] + ko, st + BM * 8 + (wave + j * NW) * 64);
            }
        };

        wait_vmcnt<0>();   // previous tile's stores are done
        issue(0);
        wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        // The tile's MFMAs over BMX rows (BMX = BM, or 256 for a group of
        // at most 256 rows in 320-row stages: 8 instead of 10 row blocks per
        // SIMD, the DeepSeek-shaped groups being 256 +- 17 rows).  Each
        // height has its own accumulators, live only in its own branch.
        auto compute = [&](auto bmx) __attribute__((always_inline)) {
            constexpr int BMX = decltype(bmx)::value;
            constexpr int TMX = BMX / (WM * 32);
            floatx16 acc[TMX][TN];
#pragma unroll
            for (int i = 0; i < TMX; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
            bf16x8 fa[2][TMX], fb[2][TN];
            for (int kt = 0; kt < KT; ++kt) {
                // the other slot was last read in step kt-1, before its barrier
                if (kt + 1 < KT) issue(kt + 1);
                const u32x4 *stage = smem + (kt & 1) * STAGE;
                load_frags<BM, BN, WM, WN, TMX, TN, BMX>(fa[0], fb[0], stage,
                                                         wm, wn, lane, 0);
#pragma unroll
                for (int kk = 0; kk < BK / 16; ++kk) {
                    if (kk + 1 < BK / 16)
                        load_frags<BM, BN, WM, WN, TMX, TN, BMX>(
                            fa[(kk + 1) & 1], fb[(kk + 1) & 1], stage, wm, wn,
                            lane, kk + 1);
                    mfma_block<TMX, TN>(acc, fa[kk & 1], fb[kk & 1]);
                }
                wait_vmcnt<0>();
                __builtin_amdgcn_s_barrier();
            }
            store_tile<BMX, BN, WM, WN, TMX, TN, UP>(p, acc, routed, g, row0,
                                                     nrows, n0, wm, wn, lane);
        };
        if (BM == 320 && nrows <= 256)
            compute(std::integral_constant<int, BM == 320 ? 256 : BM>{});
        else
            compute(std::integral_constant<int, BM>{});
    }
}

// ---------------------------------------------------------------------
// Four-wave 256 x 256 tile kernel for large groups (prefill).  One wave per
// SIMD owns a 128 x 128 quarter as 8 x 8 v_mfma_f32_16x16x32_bf16 blocks.
// The MFMAs are written as asm with the accumulator as an AGPR operand:
// with the builtin, hipcc splits the 256 accumulators between AGPRs and
// VGPRs and copies them back and forth every step.  As volatile asm they
// also keep the order written here, which is the issue schedule: K is
// walked in 64-deep stages through two LDS slots filled by direct-to-LDS
// loads, and while one 32-deep sub-step's 64 MFMAs issue, the 16 fragment
// reads of the next sub-step go between its first 48 MFMAs and the 16
// loads of the stage after next between every fourth (in the second
// sub-step of a stage).  A burst of loads would stall the only wave of the
// SIMD at the memory pipe; spread out, their issue hides under the MFMAs.
// The slots are two arrays named statically (two stages per loop trip), so
// the compiler sees that the loads into one and the reads of the other do
// not alias and adds no waits between them.
namespace w4 {
constexpr int BM = 256, BN = 256, SK = 64;   // stage depth SK
constexpr int CPR = 8;                   // 16-byte chunks per row and stage
constexpr int STAGE = (BM + BN) * CPR;   // 16-byte units per stage (64 KB)
constexpr int LPW = BM / 8 / 4;          // loads per wave, operand and stage

__device__ __forceinline__ void dma16b(const char *src, u32x4 *lds_row8) {
    __builtin_amdgcn_global_load_lds(
        (const void *)src,
        (__attribute__((address_space(3))) void *)lds_row8, 16, 0, 0);
}

__device__ __forceinline__ void mfma_agpr(floatx4 &acc, const bf16x8 &a,
                                          const bf16x8 &b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(acc)
                 : "v"(a), "v"(b));
}
}  // namespace w4

// bias[f0 + 16 b + t] (t < 4) of NB 16-column blocks into v[4 b + t], as
// bf16 -> f32; zeros without a bias.  The 8-byte loads are issued together
// under one uniform branch, so one wait covers them.
template <int NB>
__device__ __forceinline__ void load_bias4(const uint16_t *bias, int f0,
                                           float *v) {
    if (bias) {
        u32x2 bb[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) bb[b] = *(const u32x2 *)(bias + f0 + 16 * b);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            v[4 * b + 0] = bf16_lo(bb[b].x);
            v[4 * b + 1] = bf16_hi(bb[b].x);
            v[4 * b + 2] = bf16_lo(bb[b].y);
            v[4 * b + 3] = bf16_hi(bb[b].y);
        }
    } else {
#pragma unroll
        for (int b = 0; b < 4 * NB; ++b) v[b] = 0.0f;
    }
}

// One tile.  Full: 256 rows, the waves 2 x 2 quarters of 128 x 128.  Half
// (a tile of at most 128 rows, normally a group's last): the waves split
// the 256 columns, 128 x 64 each, so the tile costs half the MFMAs and
// half the A loads.  The issue schedule of a 32-deep sub-step: its MFMAs
// with the next sub-step's fragment reads spread over the first three
// quarters (full) or half (half), and in a stage's second sub-step the
// loads of the stage after next spread over the MFMAs.
// PART: write the fp32 sums over stages kt0 .. kt0 + KT - 1 to the tail
// partial buffer (plane ks) instead of finishing the tile.
// WR: rows of a wave's part of a full tile, 128 (256-row tiles) or 112
// (224-row tiles of evenly split groups: seven MFMA row blocks a wave).
// BN: tile columns, 256 or 192 (ungated only: a wave's 48 or 96 columns
// are not whole 64-column gate/up chunks); the slots keep room for 256.
// NT: weight rows loaded with the non-temporal hint (for GEMMs whose
// groups are one row tile each).
template <bool UP, bool HALF, bool PART, int WR = 128, int BN = 256,
          bool NT = false>
__device__ __forceinline__ void w4_tile(const GemmParams &p, u32x4 *slot0,
                                        u32x4 *slot1, int g, int row0,
                                        int nrows, int n0, bool routed,
                                        int wave, int lane, int kt0, int KT,
                                        int ks) {
    using namespace w4;
    static_assert(WR == 128 || ((WR == 112 || WR == 96 || WR == 80) && !HALF),
                  "wave rows");
    static_assert(BN == 256 || BN == 192, "tile columns");
    constexpr int TN = HALF ? BN / 64 : BN / 32;  // 16-column blocks per wave
    constexpr int WC = TN * 16;               // columns per wave
    constexpr int RB = HALF ? 8 : WR / 16;    // 16-row blocks per wave
    constexpr int TR = HALF ? 128 : 2 * WR;   // tile rows
    constexpr int LA = TR / 32;               // A loads per wave and stage
    constexpr int LB = BN / 32;               // B loads per wave and stage
    constexpr int NL = LA + LB;               // loads per wave and stage
    constexpr int NF = RB + TN;               // fragment reads per sub-step
    constexpr int NM = RB * TN;               // MFMAs per sub-step
    // a read after every RD MFMAs, a load after every DM (192 columns: as
    // densely as the fewer MFMAs need)
    constexpr int RD = BN == 192 ? 2 : HALF ? 2 : 3;
    constexpr int DM = BN == 192 ? (NM - 2) / (NL - 1)
                                 : HALF ? 2 : WR == 128 ? 4 : 3;
    static_assert(RD * (NF - 1) < NM && DM * (NL - 1) + 1 < NM, "issue slots");
    // The lane index is made opaque here, once per tile, so that the
    // per-lane addresses below are recomputed for each tile instead of
    // being hoisted out of the kernel's tile loop, where ~100 of them stay
    // live across it and are spilled to scratch.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    const int wm = HALF ? 0 : wave >> 1;
    const int wn = HALF ? wave : wave & 1;
    const int N = p.N, K = p.K;
    const char *A = (const char *)p.A;
    // Load j of a wave fills rows 8 (wave + 4 j) + lane/8 of an operand,
    // lane%8 being the 16-byte slot; the lane fetches k-chunk
    // (lane%8) ^ ((row/2) % 8), which depends on the lane only.  With that
    // swizzle the fragment reads (16 rows at one chunk) are conflict-free.
    const int lr = lane >> 3;
    const int ch = (lane & 7) ^ ((4 * wave + (lr >> 1)) & 7);
    const uint32_t b_lane = (uint32_t)(lr * K + ch * 8) * 2u;
    const int l16 = lane & 15;
    const int sw = (l16 >> 1) & 7;

    // A rows past the group's end re-read the tile's first row: their
    // products land in rows that are never stored
    uint32_t a_off[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        int rr = (wave + 4 * j) * 8 + lr;
        if (rr >= nrows) rr = 0;
        const int slot = row0 + rr;
        int src = slot;
        if (UP) src = routed ? p.slot_token[slot] : slot - p.shared_base;
        a_off[j] = (uint32_t)(src * K + ch * 8) * 2u;
    }
    const char *bbase[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j)
        bbase[j] = weight_row(p, routed, g, n0 + (wave + 4 * j) * 8, 2);

    // load q (q < LA: A rows, else B rows) of stage kt0 + kl into a slot
    auto dma_one = [&](int kl, u32x4 *st, int q) __attribute__((always_inline)) {
        const size_t ko = (size_t)(kt0 + kl) * SK * 2;
        if (q < LA)
            dma16b(A + ko + a_off[q], st + (wave + 4 * q) * 64);
        else if (NT)
            dma16_nt(bbase[q - LA] + ko + b_lane,
                     st + BM * CPR + (wave + 4 * (q - LA)) * 64);
        else
            dma16b(bbase[q - LA] + ko + b_lane,
                   st + BM * CPR + (wave + 4 * (q - LA)) * 64);
    };
    // fragment q (q < 8: A block q, else B block q - 8), sub-step kk
    auto frag_one = [&](bf16x8 (&fa)[RB], bf16x8 (&fb)[TN], const u32x4 *st,
                        int kk, int q) __attribute__((always_inline)) {
        const int c = (kk * 4 + (lane >> 4)) ^ sw;
        if (q < RB)
            fa[q] = as_bf16x8(st[(wm * WR + q * 16 + l16) * CPR + c]);
        else
            fb[q - RB] = as_bf16x8(
                st[BM * CPR + (wn * WC + (q - RB) * 16 + l16) * CPR + c]);
    };

    floatx4 acc[RB][TN];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa0[RB], fb0[TN], fa1[RB], fb1[TN];

    // every wave is done with both slots (previous tile) before the first
    // loads of this one
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < NL; ++q) dma_one(0, slot0, q);
#pragma unroll
    for (int q = 0; q < NL; ++q) dma_one(min(1, KT - 1), slot1, q);
    wait_vmcnt<NL>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < NF; ++q) frag_one(fa0, fb0, slot0, 0, q);

    // Stage s: sub-step 2s on fa0 while the second half of stage s is read
    // into fa1; then sub-step 2s+1 on fa1 while the first half of stage s+1
    // is read into fa0 and stage s+2 is loaded into the slot that stage s
    // leaves.  Loads past the end re-load the last stage, reads past the
    // end fill registers that are never used.
    auto stage = [&](int s, u32x4 *cur, u32x4 *nxt) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
#pragma unroll
        for (int q = 0; q < NM; ++q) {
            mfma_agpr(acc[q / TN][q % TN], fb0[q % TN], fa0[q / TN]);
            if (q % RD == 0 && q / RD < NF) frag_one(fa1, fb1, cur, 1, q / RD);
        }
        // own reads done, stage s+1 landed (this wave's part), then every
        // wave's part
        __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4));
        __builtin_amdgcn_s_barrier();
        const int nx = min(s + 2, KT - 1);
#pragma unroll
        for (int q = 0; q < NM; ++q) {
            mfma_agpr(acc[q / TN][q % TN], fb1[q % TN], fa1[q / TN]);
            if (q % RD == 0 && q / RD < NF) frag_one(fa0, fb0, nxt, 0, q / RD);
            if (q % DM == 1 && q / DM < NL) dma_one(nx, cur, q / DM);
        }
    };
    // The compiler does not know that the asm are MFMAs, so the wait states
    // they need against other instructions are inserted here, in the loop
    // body, where neither the accumulator zeroing before the loop nor the
    // reads after it can be placed: a few before the first MFMA (a VALU
    // write of its srcC), and after the last MFMA enough for a read of its
    // result (an 8-pass XDL op).
    for (int s = 0; s < KT; s += 2) {
        asm volatile("s_nop 4");
        stage(s, slot0, slot1);
        stage(s + 1, slot1, slot0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    }

    if (PART) {
        // fp32 partial sums of this K range, rows of the group's tail
        const int G = p.E + p.n_shared;
        float *dst = p.part + ((size_t)ks * G + g) * 128 * N;
        __builtin_amdgcn_s_waitcnt(0);   // re-loads landed before the next tile
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int r = i * 16 + l16;
            if (r >= nrows) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int c = n0 + wn * WC + j * 16 + 4 * (lane >> 4);
                *(float4 *)(dst + (size_t)r * N + c) =
                    make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        }
        return;
    }

    // Epilogue through LDS.  A wave's MFMA layout gives each lane 4
    // consecutive columns of 16 rows per block, so direct stores would
    // write 32-byte pieces of 16 rows per instruction.  Instead each wave
    // converts its part (bias, then the activation or SwiGLU, to bf16) into
    // a staging copy of the output tile in the idle slots (rows 0-127 in
    // slot0, 128-255 in slot1; 512-byte rows whose 16-byte chunks are
    // XOR-swizzled by the row), and the block then writes whole row
    // segments with 16-byte stores.
    __builtin_amdgcn_s_waitcnt(0);   // re-loads landed, own reads done
    __builtin_amdgcn_s_barrier();    // and every wave's
    const int cq = 4 * (lane >> 4);
    // 4 values at tile row R (0..TR-1), output column c (c % 4 == 0); R < 128
    // is uniform for a row block, so the slot choice is too
    auto put = [&](int R, int c, const float (&v)[4]) __attribute__((always_inline)) {
        char *stg = (char *)(R < 128 ? slot0 : slot1);
        const int rl = R & 127;
        const int sc = (c >> 3) ^ (rl & 15);
        u32x2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *(u32x2 *)(stg + rl * 512 + sc * 16 + ((c >> 2) & 1) * 8) = o;
    };
    const bool gated = BN == 256 && UP && p.gated;
    if (gated) if constexpr (BN == 256) {
        // a wave's columns are whole 64-column chunks of the virtual panel:
        // blocks 4c, 4c+1 are the gate rows and 4c+2, 4c+3 the up rows of
        // the tile's output features WC wn / 2 + 32 c + 16 jj + ...
        constexpr int NC = WC / 64;
        const int F = N >> 1;
        const uint16_t *b1 = routed
            ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * F : nullptr)
            : (const uint16_t *)p.bias_s;
        const uint16_t *b3 = routed
            ? (p.bias3 ? (const uint16_t *)p.bias3 + (size_t)g * F : nullptr)
            : (const uint16_t *)p.bias_s3;
        // 4 consecutive features per (c, jj): one 8-byte load each, all
        // issued before the first use (no wait per element)
        float bv1[NC][2][4], bv3[NC][2][4];
        const int fb = (n0 >> 1) + (WC / 2) * wn + cq;
        load_bias4<NC * 2>(b1, fb, &bv1[0][0][0]);
        load_bias4<NC * 2>(b3, fb, &bv3[0][0][0]);
        // BIAS is a compile-time flag: x + 0.0f is not folded away
        auto swiglu = [&](auto bias) __attribute__((always_inline)) {
            constexpr bool BIAS = decltype(bias)::value;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        float h[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            float gv = acc[i][4 * c + jj][t];
                            float uv = acc[i][4 * c + 2 + jj][t];
                            if (BIAS) {
                                gv += bv1[c][jj][t];
                                uv += bv3[c][jj][t];
                            }
                            h[t] = silu_f(gv) * uv;
                        }
                        put(wm * WR + i * 16 + l16, (WC / 2) * wn + 32 * c + 16 * jj + cq, h);
                    }
                // one row block at a time: the accumulators are read as they
                // are converted, not all at once
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (b1 || b3) swiglu(std::true_type{});
        else swiglu(std::false_type{});
    }
    if (!gated) {
        const uint16_t *bg = routed
            ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * N : nullptr)
            : (const uint16_t *)p.bias_s;
        // the activation is chosen once, outside the element loops, so
        // those stay straight-line code
        const int act = !UP ? -1 : p.act == ACT_SILU ? ACT_SILU : ACT_GELU;
        float bv[TN][4];
        load_bias4<TN>(bg, n0 + wn * WC + cq, &bv[0][0]);
        // BIAS is a compile-time flag: x + 0.0f is not folded away
        auto convert = [&](auto fn, auto bias) __attribute__((always_inline)) {
            constexpr bool BIAS = decltype(bias)::value;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        v[t] = fn(BIAS ? acc[i][j][t] + bv[j][t] : acc[i][j][t]);
                    put(wm * WR + i * 16 + l16, wn * WC + j * 16 + cq, v);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto with_act = [&](auto bias) __attribute__((always_inline)) {
            if (act == ACT_GELU)
                convert([](float z) __attribute__((always_inline)) { return gelu_erf(z); }, bias);
            else if (act == ACT_SILU)
                convert([](float z) __attribute__((always_inline)) { return silu_f(z); }, bias);
            else
                convert([](float z) __attribute__((always_inline)) { return z; }, bias);
        };
        // (only for the up GEMM: in the down GEMM's epilogue the second
        // copy made the compiler spill)
        if (!UP || bg) with_act(std::true_type{});
        else with_act(std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    // 16-byte chunks per output row: BN / 8 (32 or 24), or 16 (gated)
    const int cpr = gated ? 16 : BN / 8;
    const int rpp = 256 / cpr;                 // rows per block pass
    const int rr = tid / cpr, cc = tid % cpr;
    uint16_t *out = (uint16_t *)p.out + (gated ? n0 >> 1 : n0) + cc * 8;
    for (int r0 = 0; r0 < TR; r0 += rpp) {
        const int row = r0 + rr;
        // (24 chunks a row: the last 16 threads have no row in a pass)
        if (row < nrows && (BN == 256 || rr < rpp)) {
            const char *sb = (const char *)(row < 128 ? slot0 : slot1);
            const int rl = row & 127;
            const u32x4 v = *(const u32x4 *)(sb + rl * 512 + ((cc ^ (rl & 15)) * 16));
            *(u32x4 *)(out + (size_t)(row0 + row) * p.ldo) = v;
        }
    }
}

// TM_ROWS = 256: full tiles, a group's last <= 128 rows as a half tile.
// With four or more rounds of tiles, the full tiles of every group come
// first and the half tiles after them: the 4-5 row tiles of one (expert,
// column) panel then run side by side at one pace and share the panel's
// k-slices through L2 (a half tile among them finishes early and breaks
// that: the Mixtral up GEMM fetched 3.3 GB instead of 2.1), and the cheaper
// half tiles fill the end of the schedule.  With fewer rounds the tiles
// stay in group order, where the half tiles spread over the last round
// (the Mixtral down GEMM's 2.25 rounds: 5 % faster that way).
// TM_ROWS = 128: every tile half-height (for groups of up to ~128 rows).
// Even split (TM_ROWS = 256, tails not split over K): a group whose last
// 256-row block would hold 1..128 rows and that needs m >= 3 tiles, if m
// tiles of 224 rows hold it, runs as those m tiles instead.  The m tiles
// take the same time, so all of a weight panel's row tiles run side by
// side and share it through L2; the half tiles instead come after every
// full tile, and by then their panels have left L2 (the Mixtral up GEMM
// fetched ~0.9 GB more than its weights and rows for them).
// Two-tile groups (257..384 rows) split the same way: two tiles of 160 or
// 192 rows instead of a full tile and a half tile, the half tile being the
// one that would re-read the weight panel long after (DeepSeek-shaped
// groups of 256 +- 17 rows: about half of them).  A one-tile group of
// 129..224 rows runs as one tile of 160, 192 or 224 rows (fewer padded
// MFMA rows than a 256-row tile).
__device__ __forceinline__ int w4_even_rows(int rows) {
    const int m = (rows + 255) >> 8, rem = rows & 255;
    // a group of 129..224 rows, one tile: trimmed to its height
    if (m == 1 && rem > 128)
        return rows <= 160 ? 160 : rows <= 192 ? 192 : rows <= 224 ? 224 : 0;
    if (rem < 1 || rem > 128) return 0;
    if (m == 2) return rows <= 320 ? 160 : 192;
    return m >= 3 && m * 224 >= rows ? 224 : 0;
}
__device__ __forceinline__ bool w4_even_group(int rows) {
    return w4_even_rows(rows) != 0;
}

// TN_COLS: tile columns (256, or 192 for an ungated GEMM with N a multiple
// of 192).  NT: weights streamed with the non-temporal hint.
template <bool UP, int TM_ROWS, int TN_COLS = 256, bool NT = false>
__global__ __launch_bounds__(256, 1) void gemm_bf16_w4(GemmParams p) {
    using namespace w4;
    __shared__ u32x4 slot0[STAGE], slot1[STAGE];
    __shared__ TileTable tf, th;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KT = p.K / SK;
    const int NTN = p.N / TN_COLS;
    const int G = p.E + p.n_shared;
    if (TM_ROWS == 128) {
        build_tile_table(tf, p.offsets, p.E, p.n_shared, p.shared_base, p.T,
                         128, NTN);
    } else {
        // full-height tiles: whole 256-row blocks and a last block of more
        // than 128 rows (or an evenly split group's 224-row tiles); half
        // tiles: a last block of 1..128 rows
        const bool ev = p.tail_split <= 1;
        build_tile_table_by(tf, p.offsets, p.E, p.n_shared, p.shared_base,
                            p.T, NTN, [ev](int rows) {
                                if (ev && w4_even_group(rows)) return (rows + 255) >> 8;
                                return (rows >> 8) + ((rows & 255) > 128);
                            });
        build_tile_table_by(th, p.offsets, p.E, p.n_shared, p.shared_base,
                            p.T, NTN, [ev](int rows) {
                                if (ev && w4_even_group(rows)) return 0;
                                const int rem = rows & 255;
                                return rem > 0 && rem <= 128 ? 1 : 0;
                            });
    }
    // S > 1: the half tiles run as S units each over a 1/S range of K
    const int S = TM_ROWS == 256 && p.tail_split > 1 ? p.tail_split : 1;
    const int total_f = __builtin_amdgcn_readfirstlane(tf.base[G]);
    const int total = total_f + (TM_ROWS == 128
                                     ? 0
                                     : S * __builtin_amdgcn_readfirstlane(th.base[G]));
    const int nb = gridDim.x, per = nb >> 3;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const bool halves_last = TM_ROWS == 256 && (S > 1 || total >= 4 * nb);
    for (int r = 0;; ++r) {
        const int L = r * nb + xcd * per + loc;
        if (L >= total) break;
        int g, n_tile, m_tile, ks = 0;
        if (!halves_last) {
            // group order: the group's tiles n-tile major, m-tile minor,
            // the half tile (if any) last of each column
            g = 0;
            int lo = 0, hi = G;
            while (hi - lo > 1) {     // largest g with tile base <= L
                const int mid = (lo + hi) >> 1;
                if (tf.base[mid] + (TM_ROWS == 256 ? th.base[mid] : 0) <= L) lo = mid;
                else hi = mid;
            }
            g = __builtin_amdgcn_readfirstlane(lo);
            const int base = tf.base[g] + (TM_ROWS == 256 ? th.base[g] : 0);
            const int mt = tf.mt[g] + (TM_ROWS == 256 ? th.mt[g] : 0);
            const int local = __builtin_amdgcn_readfirstlane(L - base);
            n_tile = local / mt;
            m_tile = local - n_tile * mt;
        } else {
            const bool first = L < total_f;
            const TileTable &tt = first ? tf : th;
            int Lg = first ? L : L - total_f;
            if (!first) {             // unit ks of half tile Lg / S
                ks = Lg % S;
                Lg /= S;
            }
            g = __builtin_amdgcn_readfirstlane(find_group(tt, G, Lg));
            const int local = Lg - __builtin_amdgcn_readfirstlane(tt.base[g]);
            const int mt = __builtin_amdgcn_readfirstlane(tt.mt[g]);
            n_tile = local / mt;
            // a half tile follows the group's full tiles
            m_tile = first ? local - n_tile * mt
                           : __builtin_amdgcn_readfirstlane(tf.mt[g]);
        }
        const int grows = __builtin_amdgcn_readfirstlane(tf.rows[g]);
        const int ev_rows = TM_ROWS == 256 && S == 1 ? w4_even_rows(grows) : 0;
        const int tm = ev_rows ? ev_rows : TM_ROWS;
        const int row0 = __builtin_amdgcn_readfirstlane(tf.start[g]) + m_tile * tm;
        const int nrows = min(tm, grows - m_tile * tm);
        const int n0 = n_tile * TN_COLS;
        const bool routed = g < p.E;
        if (S > 1 && L >= total_f)
            w4_tile<UP, true, true, 128, TN_COLS, NT>(p, slot0, slot1, g, row0, nrows, n0,
                                    routed, wave, lane, ks * (KT / S), KT / S,
                                    ks);
        else if (TM_ROWS == 128 || nrows <= 128)
            w4_tile<UP, true, false, 128, TN_COLS, NT>(p, slot0, slot1, g, row0, nrows, n0,
                                     routed, wave, lane, 0, KT, 0);
        else if (tm == 224)
            w4_tile<UP, false, false, 112, TN_COLS, NT>(p, slot0, slot1, g, row0, nrows, n0,
                                           routed, wave, lane, 0, KT, 0);
        else if (tm == 192)
            w4_tile<UP, false, false, 96, TN_COLS, NT>(p, slot0, slot1, g, row0, nrows, n0,
                                          routed, wave, lane, 0, KT, 0);
        else if (tm == 160)
            w4_tile<UP, false, false, 80, TN_COLS, NT>(p, slot0, slot1, g, row0, nrows, n0,
                                          routed, wave, lane, 0, KT, 0);
        else
            w4_tile<UP, false, false, 128, TN_COLS, NT>(p, slot0, slot1, g, row0, nrows, n0,
                                      routed, wave, lane, 0, KT, 0);
    }
}

// ---------------------------------------------------------------------
// The four-wave 256 x 256 tile with v_mfma_f32_32x32x16_bf16 instead of
// 16x16x32.  Same LDS stages (64-deep, two slots, the same direct loads and
// swizzle), the same one wave per SIMD with 256 AGPR accumulators, but a
// wave's 128 x 128 quarter is 4 x 4 blocks of 32 x 32, half as many MFMA
// instructions for the same work.  Measured on gfx950 with one wave per
// SIMD and fragment reads prefetched a step ahead: 16x16x32 with one
// ds_read_b128 per four MFMAs issues at 18.4 clocks per 16-clock MFMA,
// 32x32x16 with one read per two MFMAs (the same bytes per FLOP) at 32.9
// per 32-clock MFMA.  A 64-deep stage is four 16-deep steps; the fragments
// of steps 2 and 3 are read during step 1, so that after the mid-stage
// barrier nothing reads the slot any more and the loads of the stage after
// next go into it during steps 2 and 3 while step 2 reads the next stage's
// first fragments from the other slot.  Tile heights are multiples of 64
// (32-row MFMA blocks, two wave rows): 256, 192 and 128 full-width tiles
// and the 128 x 256 half tile (the waves then split the columns).
namespace w4x {
using w4::BM;
using w4::BN;
using w4::CPR;
using w4::LPW;
using w4::SK;

__device__ __forceinline__ void mfma32_agpr(floatx16 &acc, const bf16x8 &a,
                                            const bf16x8 &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+a"(acc)
                 : "v"(a), "v"(b));
}
}  // namespace w4x

// bias[f0 + 8 q + t] (q, t < 4) into v[q][t] as bf16 -> f32 (zeros without
// a bias): the 16 columns a lane of a 32 x 32 output block holds.
__device__ __forceinline__ void load_bias_q4(const uint16_t *bias, int f0,
                                             float (&v)[4][4]) {
    if (bias) {
        u32x2 bb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) bb[q] = *(const u32x2 *)(bias + f0 + 8 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[q][0] = bf16_lo(bb[q].x);
            v[q][1] = bf16_hi(bb[q].x);
            v[q][2] = bf16_lo(bb[q].y);
            v[q][3] = bf16_hi(bb[q].y);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int t = 0; t < 4; ++t) v[q][t] = 0.0f;
    }
}

// One tile.  HALF: at most 128 rows, waves 128 x 64.  Otherwise 2 WR rows,
// waves 2 x 2 quarters of WR x 128.  PART: fp32 sums of stages kt0 ..
// kt0 + KT - 1 into the tail partial buffer (plane ks), as w4_tile.
template <bool UP, bool HALF, bool PART, int WR = 128>
__device__ __forceinline__ void w4x_tile(const GemmParams &p, u32x4 *slot0,
                                         u32x4 *slot1, int g, int row0,
                                         int nrows, int n0, bool routed,
                                         int wave, int lane, int kt0, int KT,
                                         int ks) {
    using namespace w4x;
    static_assert(WR == 128 || ((WR == 96 || WR == 64) && !HALF), "wave rows");
    constexpr int TN = HALF ? 2 : 4;          // 32-column blocks per wave
    constexpr int WC = HALF ? 64 : 128;       // columns per wave
    constexpr int RB = HALF ? 4 : WR / 32;    // 32-row blocks per wave
    constexpr int WRR = HALF ? 128 : WR;      // rows per wave
    constexpr int TR = HALF ? 128 : 2 * WR;   // tile rows
    constexpr int LA = TR / 32;               // A loads per wave and stage
    constexpr int NL = LA + LPW;              // loads per wave and stage
    constexpr int NF = RB + TN;               // fragment reads per step
    constexpr int NM = RB * TN;               // MFMAs per step
    constexpr int DM = (2 * NM) / NL;         // a load every DM MFMAs
    static_assert(DM >= 1 && DM * NL <= 2 * NM, "load slots");
    // the lane index made opaque once per tile (addresses recomputed per
    // tile, not hoisted out of the tile loop and spilled)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    const int wm = HALF ? 0 : wave >> 1;
    const int wn = HALF ? wave : wave & 1;
    const int N = p.N, K = p.K;
    const char *A = (const char *)p.A;
    const int lr = lane >> 3;
    const int ch = (lane & 7) ^ ((4 * wave + (lr >> 1)) & 7);
    const uint32_t b_lane = (uint32_t)(lr * K + ch * 8) * 2u;
    const int l32 = lane & 31;
    const int hk = lane >> 5;                 // k half of a 16-deep step
    const int sw = (l32 >> 1) & 7;            // row swizzle of l32's rows

    uint32_t a_off[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        int rr = (wave + 4 * j) * 8 + lr;
        if (rr >= nrows) rr = 0;
        const int slot = row0 + rr;
        int src = slot;
        if (UP) src = routed ? p.slot_token[slot] : slot - p.shared_base;
        a_off[j] = (uint32_t)(src * K + ch * 8) * 2u;
    }
    const char *bbase[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j)
        bbase[j] = weight_row(p, routed, g, n0 + (wave + 4 * j) * 8, 2);

    auto dma_one = [&](int kl, u32x4 *st, int q) __attribute__((always_inline)) {
        const size_t ko = (size_t)(kt0 + kl) * SK * 2;
        if (q < LA)
            w4::dma16b(A + ko + a_off[q], st + (wave + 4 * q) * 64);
        else
            w4::dma16b(bbase[q - LA] + ko + b_lane,
                       st + BM * CPR + (wave + 4 * (q - LA)) * 64);
    };
    // fragment q (q < RB: A block q, else B block q - RB) of 16-deep step t
    auto frag_one = [&](bf16x8 (&fa)[RB], bf16x8 (&fb)[TN], const u32x4 *st,
                        int t, int q) __attribute__((always_inline)) {
        const int c = (t * 2 + hk) ^ sw;
        if (q < RB)
            fa[q] = as_bf16x8(st[(wm * WRR + q * 32 + l32) * CPR + c]);
        else
            fb[q - RB] = as_bf16x8(
                st[BM * CPR + (wn * WC + (q - RB) * 32 + l32) * CPR + c]);
    };

    floatx16 acc[RB][TN];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    bf16x8 a0[RB], b0[TN], a1[RB], b1[TN], a2[RB], b2[TN], a3[RB], b3[TN];

    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < NL; ++q) dma_one(0, slot0, q);
#pragma unroll
    for (int q = 0; q < NL; ++q) dma_one(min(1, KT - 1), slot1, q);
    wait_vmcnt<NL>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < NF; ++q) frag_one(a0, b0, slot0, 0, q);

    // MFMAs of one step on (fa, fb), with R reads (index r: r < NF the
    // fragments of ra/rb at step rt, else of rc/rd at step rt + 1, all from
    // rs) spread over them, and (LD) loads d0 .. of the stage after next.
    auto step = [&](const bf16x8 (&fa)[RB], const bf16x8 (&fb)[TN],
                    auto nreads, bf16x8 (&ra)[RB], bf16x8 (&rb)[TN],
                    bf16x8 (&rc)[RB], bf16x8 (&rd)[TN], const u32x4 *rs,
                    int rt, auto ld, int d0, int kload, u32x4 *lslot)
                    __attribute__((always_inline)) {
        constexpr int R = decltype(nreads)::value;
        constexpr bool LD = decltype(ld)::value;
#pragma unroll
        for (int x = 0; x < NM; ++x) {
            mfma32_agpr(acc[x / TN][x % TN], fb[x % TN], fa[x / TN]);
#pragma unroll
            for (int r = (x * R) / NM; r < ((x + 1) * R) / NM; ++r) {
                if (r < NF) frag_one(ra, rb, rs, rt, r);
                else frag_one(rc, rd, rs, rt + 1, r - NF);
            }
            if (LD && x % DM == 0 && d0 + x / DM < NL && x / DM < (NM + DM - 1) / DM)
                dma_one(kload, lslot, d0 + x / DM);
        }
    };
    constexpr int LD2 = (NM + DM - 1) / DM;   // loads issued in step 2
    auto stage = [&](int s, u32x4 *cur, u32x4 *nxt) __attribute__((always_inline)) {
        const int nx = min(s + 2, KT - 1);
        // step 0 (fragments a0/b0): read step 1's from cur
        step(a0, b0, std::integral_constant<int, NF>{}, a1, b1, a1, b1, cur, 1,
             std::false_type{}, 0, nx, cur);
        // step 1: read steps 2 and 3 from cur
        step(a1, b1, std::integral_constant<int, 2 * NF>{}, a2, b2, a3, b3, cur,
             2, std::false_type{}, 0, nx, cur);
        // own reads done, stage s+1 landed (this wave's part), then every
        // wave's part: nothing reads cur after this barrier
        __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4));
        __builtin_amdgcn_s_barrier();
        // step 2: read the next stage's step 0 from nxt, load stage s+2
        step(a2, b2, std::integral_constant<int, NF>{}, a0, b0, a0, b0, nxt, 0,
             std::true_type{}, 0, nx, cur);
        // step 3: the rest of the loads
        step(a3, b3, std::integral_constant<int, 0>{}, a0, b0, a0, b0, nxt, 0,
             std::true_type{}, LD2, nx, cur);
    };
    for (int s = 0; s < KT; s += 2) {
        asm volatile("s_nop 4");
        stage(s, slot0, slot1);
        stage(s + 1, slot1, slot0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    }
    // lane l holds, for row l32 of each 32 x 32 block, output columns
    // 8 q + 4 hk + 0..3 (q = 0..3): acc[i][j][4 q + t]
    if (PART) {
        const int G = p.E + p.n_shared;
        float *dst = p.part + ((size_t)ks * G + g) * 128 * N;
        __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int r = wm * WRR + i * 32 + l32;
            if (r >= nrows) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = n0 + wn * WC + j * 32 + 8 * q + 4 * hk;
                    *(float4 *)(dst + (size_t)r * N + c) =
                        make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                    acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                }
        }
        return;
    }
    // Epilogue through LDS, as w4_tile: bias and activation (or SwiGLU) to
    // bf16 into a staging copy of the output tile in the idle slots (rows
    // 0-127 in slot0, 128-255 in slot1, 512-byte rows with 16-byte chunks
    // XOR-swizzled by the row), then whole row segments with 16-byte stores.
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    auto put = [&](int R, int c, const float (&v)[4]) __attribute__((always_inline)) {
        char *stg = (char *)(R < 128 ? slot0 : slot1);
        const int rl = R & 127;
        const int sc = (c >> 3) ^ (rl & 15);
        u32x2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *(u32x2 *)(stg + rl * 512 + sc * 16 + ((c >> 2) & 1) * 8) = o;
    };
    const bool gated = UP && p.gated;
    if (gated) {
        // wave columns are whole 64-column chunks of the virtual panel:
        // block 2c the gate rows and 2c + 1 the up rows of output features
        // WC wn / 2 + 32 c + 8 q + 4 hk + t
        constexpr int NC = WC / 64;
        const int F = N >> 1;
        const uint16_t *bp1 = routed
            ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * F : nullptr)
            : (const uint16_t *)p.bias_s;
        const uint16_t *bp3 = routed
            ? (p.bias3 ? (const uint16_t *)p.bias3 + (size_t)g * F : nullptr)
            : (const uint16_t *)p.bias_s3;
        const int fb0 = (n0 >> 1) + (WC / 2) * wn + 4 * hk;
        float bv1[NC][4][4], bv3[NC][4][4];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            load_bias_q4(bp1 ? bp1 + 32 * c : nullptr, fb0, bv1[c]);
            load_bias_q4(bp3 ? bp3 + 32 * c : nullptr, fb0, bv3[c]);
        }
        auto swiglu = [&](auto bias) __attribute__((always_inline)) {
            constexpr bool BIAS = decltype(bias)::value;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float h[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            float gv = acc[i][2 * c][4 * q + t];
                            float uv = acc[i][2 * c + 1][4 * q + t];
                            if (BIAS) {
                                gv += bv1[c][q][t];
                                uv += bv3[c][q][t];
                            }
                            h[t] = silu_f(gv) * uv;
                        }
                        put(wm * WRR + i * 32 + l32,
                            (WC / 2) * wn + 32 * c + 8 * q + 4 * hk, h);
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (bp1 || bp3) swiglu(std::true_type{});
        else swiglu(std::false_type{});
    } else {
        const uint16_t *bg = routed
            ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * N : nullptr)
            : (const uint16_t *)p.bias_s;
        const int act = !UP ? -1 : p.act == ACT_SILU ? ACT_SILU : ACT_GELU;
        // bias of columns wn WC + 32 j + 8 q + 4 hk + t
        float bv[TN][4][4];
#pragma unroll
        for (int j = 0; j < TN; ++j)
            load_bias_q4(bg ? bg + 32 * j : nullptr, n0 + wn * WC + 4 * hk, bv[j]);
        auto convert = [&](auto fn, auto bias) __attribute__((always_inline)) {
            constexpr bool BIAS = decltype(bias)::value;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            v[t] = fn(BIAS ? acc[i][j][4 * q + t] + bv[j][q][t]
                                           : acc[i][j][4 * q + t]);
                        put(wm * WRR + i * 32 + l32, wn * WC + j * 32 + 8 * q + 4 * hk, v);
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto with_act = [&](auto bias) __attribute__((always_inline)) {
            if (act == ACT_GELU)
                convert([](float z) __attribute__((always_inline)) { return gelu_erf(z); }, bias);
            else if (act == ACT_SILU)
                convert([](float z) __attribute__((always_inline)) { return silu_f(z); }, bias);
            else
                convert([](float z) __attribute__((always_inline)) { return z; }, bias);
        };
        if (!UP || bg) with_act(std::true_type{});
        else with_act(std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    const int cpr = gated ? 16 : 32;
    const int rpp = 256 / cpr;
    const int rr = tid / cpr, cc = tid % cpr;
    uint16_t *out = (uint16_t *)p.out + (gated ? n0 >> 1 : n0) + cc * 8;
    for (int r0 = 0; r0 < TR; r0 += rpp) {
        const int row = r0 + rr;
        if (row < nrows) {
            const char *sb = (const char *)(row < 128 ? slot0 : slot1);
            const int rl = row & 127;
            const u32x4 v = *(const u32x4 *)(sb + rl * 512 + ((cc ^ (rl & 15)) * 16));
            *(u32x4 *)(out + (size_t)(row0 + row) * p.ldo) = v;
        }
    }
}

// Row tiles of a group of `rows` rows for the 32x32 four-wave kernel
// without split tails: m = ceil(rows / 256) tiles whose heights (256, 192
// or 128, in that order) hold the group with the least padding; a group of
// at most 128 rows is one half tile instead (counted in th, not here).
struct W4xSplit {
    int n256, n192, n128;
};
__device__ __forceinline__ W4xSplit w4x_split(int rows) {
    W4xSplit s = {0, 0, 0};
    if (rows <= 128) return s;
    const int m = (rows + 255) >> 8;
    const int x = (256 * m - rows) >> 6;      // 64-row reductions
    s.n128 = max(0, x - m);
    s.n192 = x - 2 * s.n128;
    s.n256 = m - s.n192 - s.n128;
    return s;
}

template <bool UP, int TM_ROWS>
__global__ __launch_bounds__(256, 1) void gemm_bf16_w4x(GemmParams p) {
    using namespace w4;
    __shared__ u32x4 slot0[STAGE], slot1[STAGE];
    __shared__ TileTable tf, th;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KT = p.K / SK;
    const int NTN = p.N / BN;
    const int G = p.E + p.n_shared;
    // S > 1: the half tiles run as S units each over a 1/S range of K, and
    // full tiles are whole 256-row blocks; S == 1: mixed heights
    const int S = TM_ROWS == 256 && p.tail_split > 1 ? p.tail_split : 1;
    if (TM_ROWS == 128) {
        build_tile_table(tf, p.offsets, p.E, p.n_shared, p.shared_base, p.T,
                         128, NTN);
    } else {
        build_tile_table_by(tf, p.offsets, p.E, p.n_shared, p.shared_base,
                            p.T, NTN, [S](int rows) {
                                if (S > 1) return (rows >> 8) + ((rows & 255) > 128);
                                const W4xSplit w = w4x_split(rows);
                                return w.n256 + w.n192 + w.n128;
                            });
        build_tile_table_by(th, p.offsets, p.E, p.n_shared, p.shared_base,
                            p.T, NTN, [S](int rows) {
                                if (S > 1) {
                                    const int rem = rows & 255;
                                    return rem > 0 && rem <= 128 ? 1 : 0;
                                }
                                return rows > 0 && rows <= 128 ? 1 : 0;
                            });
    }
    const int total_f = __builtin_amdgcn_readfirstlane(tf.base[G]);
    const int total = total_f + (TM_ROWS == 128
                                     ? 0
                                     : S * __builtin_amdgcn_readfirstlane(th.base[G]));
    const int nb = gridDim.x, per = nb >> 3;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    const bool halves_last = TM_ROWS == 256 && (S > 1 || total >= 4 * nb);
    for (int r = 0;; ++r) {
        const int L = r * nb + xcd * per + loc;
        if (L >= total) break;
        int g, n_tile, m_tile, ks = 0;
        bool half;
        if (!halves_last) {
            int lo = 0, hi = G;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (tf.base[mid] + (TM_ROWS == 256 ? th.base[mid] : 0) <= L) lo = mid;
                else hi = mid;
            }
            g = __builtin_amdgcn_readfirstlane(lo);
            const int base = tf.base[g] + (TM_ROWS == 256 ? th.base[g] : 0);
            const int mt = tf.mt[g] + (TM_ROWS == 256 ? th.mt[g] : 0);
            const int local = __builtin_amdgcn_readfirstlane(L - base);
            n_tile = local / mt;
            m_tile = local - n_tile * mt;
            half = TM_ROWS == 128 || m_tile >= tf.mt[g];
        } else {
            const bool first = L < total_f;
            const TileTable &tt = first ? tf : th;
            int Lg = first ? L : L - total_f;
            if (!first) {
                ks = Lg % S;
                Lg /= S;
            }
            g = __builtin_amdgcn_readfirstlane(find_group(tt, G, Lg));
            const int local = Lg - __builtin_amdgcn_readfirstlane(tt.base[g]);
            const int mt = __builtin_amdgcn_readfirstlane(tt.mt[g]);
            n_tile = local / mt;
            m_tile = first ? local - n_tile * mt
                           : __builtin_amdgcn_readfirstlane(tf.mt[g]);
            half = !first;
        }
        const int grows = __builtin_amdgcn_readfirstlane(tf.rows[g]);
        const int gstart = __builtin_amdgcn_readfirstlane(tf.start[g]);
        int tm = TM_ROWS, off = m_tile * TM_ROWS;
        if (TM_ROWS == 256 && !half) {
            if (S > 1) {
                tm = 256;
                off = m_tile * 256;
            } else {
                const W4xSplit w = w4x_split(grows);
                if (m_tile < w.n256) {
                    tm = 256;
                    off = m_tile * 256;
                } else if (m_tile < w.n256 + w.n192) {
                    tm = 192;
                    off = w.n256 * 256 + (m_tile - w.n256) * 192;
                } else {
                    tm = 128;
                    off = w.n256 * 256 + w.n192 * 192 + (m_tile - w.n256 - w.n192) * 128;
                }
            }
        } else if (TM_ROWS == 256 && half) {
            // the group's rows after its full tiles
            off = S > 1 ? (tf.mt[g]) * 256 : 0;
            tm = 128;
        }
        const int row0 = gstart + off;
        const int nrows = min(tm, grows - off);
        const int n0 = n_tile * BN;
        const bool routed = g < p.E;
        if (S > 1 && L >= total_f)
            w4x_tile<UP, true, true>(p, slot0, slot1, g, row0, nrows, n0,
                                     routed, wave, lane, ks * (KT / S), KT / S,
                                     ks);
        else if (half || TM_ROWS == 128)
            w4x_tile<UP, true, false>(p, slot0, slot1, g, row0, nrows, n0,
                                      routed, wave, lane, 0, KT, 0);
        else if (tm == 256)
            w4x_tile<UP, false, false, 128>(p, slot0, slot1, g, row0, nrows, n0,
                                            routed, wave, lane, 0, KT, 0);
        else if (tm == 192)
            w4x_tile<UP, false, false, 96>(p, slot0, slot1, g, row0, nrows, n0,
                                           routed, wave, lane, 0, KT, 0);
        else
            w4x_tile<UP, false, false, 64>(p, slot0, slot1, g, row0, nrows, n0,
                                           routed, wave, lane, 0, KT, 0);
    }
}

// ---------------------------------------------------------------------
// Two blocks per CU: 128 x 256 tiles, four waves of 128 x 64 (8 x 4
// v_mfma_f32_16x16x32_bf16 blocks, 128 accumulators as AGPR operands, as in
// the four-wave kernel).  With one wave per SIMD the four-wave kernel's
// epilogue (bias, activation, bf16 conversion: ~6000 vector instructions a
// wave and tile) and its tile prologue leave the matrix cores idle; here each
// SIMD holds a wave of each of two independent blocks, so one block's
// epilogue and load waits run under the other's MFMAs.  The price is half the
// reuse per LDS byte, so the stages are 32 deep (64-byte row pieces) and the
// LDS ring three slots of 24 KB (A 128 rows, B 256 rows), 72 KB a block.
// Stage s+2 is requested when stage s is about to be used (two stages in
// flight); a stage's fragments are read at the start of its own step, the
// other block covering that latency.  Three statically named slot arrays
// (three steps per loop trip) keep the compiler from seeing an alias between
// the loads into one slot and the reads of another.
namespace x2 {
constexpr int BM = 128, BN = 256, SK = 32;   // stage depth SK
constexpr int ROWB = SK * 2;                 // bytes of a row per stage
constexpr int SLOT = (BM + BN) * ROWB;       // 24 KB
constexpr int LA = BM / 16 / 4;              // A loads per wave and stage
constexpr int LB = BN / 16 / 4;              // B loads per wave and stage
}  // namespace x2

template <bool UP>
__device__ __forceinline__ void x2_tile(const GemmParams &p, char *s0,
                                        char *s1, char *s2, int g, int row0,
                                        int nrows, int n0, bool routed,
                                        int wave) {
    using namespace x2;
    // opaque once per tile, so that the per-lane offsets are recomputed
    // here instead of living across the tile loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int K = p.K, N = p.N, KT = K / SK;
    const char *A = (const char *)p.A;
    // Load j of a wave fills rows 16 (wave + 4 j) + lane/4 of an operand;
    // position lane%4 of the row's 64 bytes receives k-chunk
    // (lane%4) ^ (row/2 % 4) = (lane%4) ^ (lane/8 % 4).  With that swizzle
    // the fragment reads (16 rows at one chunk) run without bank conflicts
    // (measured: the swizzle by row/4 % 4, free of conflicts on a plain
    // 64-bank model, costs every read a second pass on gfx950).
    const int lr = lane >> 2;
    const int ch = (lane & 3) ^ ((lane >> 3) & 3);
    uint32_t a_off[LA];
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        int rr = 16 * (wave + 4 * j) + lr;
        if (rr >= nrows) rr = 0;     // products land in rows never stored
        const int slot = row0 + rr;
        int src = slot;
        if (UP) src = routed ? p.slot_token[slot] : slot - p.shared_base;
        a_off[j] = (uint32_t)(src * K + ch * 8) * 2u;
    }
    const char *bbase[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j)
        bbase[j] = weight_row(p, routed, g, n0 + 16 * (wave + 4 * j), 2);
    const uint32_t b_lane = (uint32_t)(lr * K + ch * 8) * 2u;
    auto dma = [&](int kt, char *slot) __attribute__((always_inline)) {
        const size_t ko = (size_t)kt * SK * 2;
#pragma unroll
        for (int j = 0; j < LA; ++j)
            w4::dma16b(A + ko + a_off[j], (u32x4 *)(slot + (wave + 4 * j) * 1024));
#pragma unroll
        for (int j = 0; j < LB; ++j)
            w4::dma16b(bbase[j] + ko + b_lane,
                       (u32x4 *)(slot + BM * ROWB + (wave + 4 * j) * 1024));
    };
    const int l16 = lane & 15;
    const int fpos = ((lane >> 4) ^ ((l16 >> 1) & 3)) * 16;
    const int a_rd = l16 * ROWB + fpos;
    const int b_rd = (BM + 64 * wave + l16) * ROWB + fpos;

    floatx4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa[8], fb[4];

    // every wave has read its staged outputs of the previous tile
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    dma(0, s0);
    dma(min(1, KT - 1), s1);
    // Step s: stage s landed (own loads, then everyone's), which also means
    // every wave is past step s-1, so the slot of stage s-1 takes stage s+2;
    // then stage s's fragments and its 32 MFMAs.  Loads past the end re-load
    // the last stage into a slot that is no longer read.
    auto step = [&](int s, const char *cur, char *nxt2) __attribute__((always_inline)) {
        wait_vmcnt<LA + LB>();
        __builtin_amdgcn_s_barrier();
        dma(min(s + 2, KT - 1), nxt2);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fb[j] = as_bf16x8(*(const u32x4 *)(cur + b_rd + j * 16 * ROWB));
#pragma unroll
        for (int i = 0; i < 8; ++i)
            fa[i] = as_bf16x8(*(const u32x4 *)(cur + a_rd + i * 16 * ROWB));
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) w4::mfma_agpr(acc[i][j], fb[j], fa[i]);
    };
    // wait states of the asm MFMAs: before the first (a VALU write of its
    // srcC) and after the last (a read of an 8-pass result)
    // whole trips of three steps (a conditional step inside the trip makes
    // the compiler lose track of which slot each load writes and wait for
    // all of them), then the last KT % 3 steps
    const int KT3 = KT - KT % 3;
    int s = 0;
    for (; s < KT3; s += 3) {
        asm volatile("s_nop 4");
        step(s, s0, s2);
        step(s + 1, s1, s0);
        step(s + 2, s2, s1);
    }
    if (s < KT) {
        asm volatile("s_nop 4");
        step(s, s0, s2);
        if (s + 1 < KT) step(s + 1, s1, s0);
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");

    // Epilogue: the re-loads have landed and every wave is done with the
    // slots; each wave stages its own 128 x 64 outputs (128 x 32 gated) as
    // bf16 in 16 KB of the slots, rows 0-63 and 64-127 in two 8 KB halves,
    // 16-byte chunks XOR-swizzled by the row, and writes them back as whole
    // row segments, with no block barrier between.
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    const bool gated = UP && p.gated;
    const int RS = gated ? 64 : 128;        // staged bytes per row
    const int CPR = RS / 16;
    const int SH = gated ? 2 : 1;           // rows per 256 bytes: 1 << SH
    char *h0 = wave == 3 ? s0 + 16384 : (wave == 0 ? s0 : wave == 1 ? s1 : s2);
    char *h1 = wave == 3 ? s1 + 16384 : h0 + 8192;
    const int cq = 4 * (lane >> 4);
    auto put = [&](int rl, int c, const float (&v)[4]) __attribute__((always_inline)) {
        char *base = rl < 64 ? h0 : h1;
        const int r = rl & 63;
        const int sc = (c >> 3) ^ ((r >> SH) & (CPR - 1));
        u32x2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *(u32x2 *)(base + r * RS + sc * 16 + ((c >> 2) & 1) * 8) = o;
    };
    if (gated) {
        const int F = N >> 1;
        const uint16_t *b1 = routed
            ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * F : nullptr)
            : (const uint16_t *)p.bias_s;
        const uint16_t *b3 = routed
            ? (p.bias3 ? (const uint16_t *)p.bias3 + (size_t)g * F : nullptr)
            : (const uint16_t *)p.bias_s3;
        float bv1[2][4], bv3[2][4];
        const int fb0 = (n0 >> 1) + 32 * wave + cq;
        load_bias4<2>(b1, fb0, &bv1[0][0]);
        load_bias4<2>(b3, fb0, &bv3[0][0]);
        // blocks 0, 1: gate rows, 2, 3: up rows of features 16 jj + ...
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                float h[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    h[t] = silu_f(acc[i][jj][t] + bv1[jj][t]) *
                           (acc[i][2 + jj][t] + bv3[jj][t]);
                put(i * 16 + l16, 16 * jj + cq, h);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        const uint16_t *bg = routed
            ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * N : nullptr)
            : (const uint16_t *)p.bias_s;
        const int act = !UP ? -1 : p.act == ACT_SILU ? ACT_SILU : ACT_GELU;
        float bv[4][4];
        load_bias4<4>(bg, n0 + 64 * wave + cq, &bv[0][0]);
        auto convert = [&](auto fn) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = fn(acc[i][j][t] + bv[j][t]);
                    put(i * 16 + l16, 16 * j + cq, v);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if (act == ACT_GELU)
            convert([](float z) __attribute__((always_inline)) { return gelu_erf(z); });
        else if (act == ACT_SILU)
            convert([](float z) __attribute__((always_inline)) { return silu_f(z); });
        else
            convert([](float z) __attribute__((always_inline)) { return z; });
    }
    // the wave reads back only what it wrote: LDS keeps a wave's order
    const int rpp = 64 / CPR;                 // rows per pass
    const int rr = lane / CPR, cc = lane % CPR;
    uint16_t *out = (uint16_t *)p.out + (gated ? (n0 >> 1) + 32 * wave : n0 + 64 * wave) + cc * 8;
    for (int r0 = 0; r0 < BM; r0 += rpp) {
        const int row = r0 + rr;
        const char *base = row < 64 ? h0 : h1;
        const int r = row & 63;
        const u32x4 v = *(const u32x4 *)(base + r * RS + ((cc ^ ((r >> SH) & (CPR - 1))) * 16));
        if (row < nrows) *(u32x4 *)(out + (size_t)(row0 + row) * p.ldo) = v;
    }
}

template <bool UP>
__global__ __launch_bounds__(256, 2) void gemm_bf16_x2(GemmParams p) {
    using namespace x2;
    __shared__ __attribute__((aligned(16))) char slot0[SLOT], slot1[SLOT], slot2[SLOT];
    __shared__ TileTable tt;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int NTN = p.N / BN;
    const int G = p.E + p.n_shared;
    build_tile_table(tt, p.offsets, p.E, p.n_shared, p.shared_base, p.T, BM, NTN);
    const int total = __builtin_amdgcn_readfirstlane(tt.base[G]);
    // XCD-aware order: the blocks of one XCD take consecutive tiles, which
    // are the row tiles of one (group, 256-column) weight panel
    const int nb = gridDim.x, per = nb >> 3;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    for (int r = 0;; ++r) {
        const int L = r * nb + xcd * per + loc;
        if (L >= total) break;
        const int g = __builtin_amdgcn_readfirstlane(find_group(tt, G, L));
        const int local = L - __builtin_amdgcn_readfirstlane(tt.base[g]);
        const int mt = __builtin_amdgcn_readfirstlane(tt.mt[g]);
        const int n_tile = local / mt;
        const int m_tile = local - n_tile * mt;
        const int row0 = __builtin_amdgcn_readfirstlane(tt.start[g]) + m_tile * BM;
        const int nrows = min(BM, __builtin_amdgcn_readfirstlane(tt.rows[g]) - m_tile * BM);
        x2_tile<UP>(p, slot0, slot1, slot2, g, row0, nrows, n_tile * BN,
                    g < p.E, wave);
    }
}

// Finishing the split tails: for each group whose last 1..128 rows ran as
// split units, out[row] = epilogue(sum over ks in order of the fp32 partial
// rows + bias), 8 outputs per thread and step.  Block (group, 128-column
// chunk of the output).  Gated: output feature f pairs virtual columns
// 64 (f / 32) + f % 32 (gate) and that + 32 (up).
template <bool UP>
__global__ __launch_bounds__(256) void w4_tail_reduce(GemmParams p) {
    const int G = p.E + p.n_shared;
    const bool gated = UP && p.gated;
    const int N = p.N;
    const int OC = gated ? N >> 1 : N;
    const int nch = OC / 128;
    const int g = blockIdx.x / nch, c0 = (blockIdx.x - g * nch) * 128;
    const bool routed = g < p.E;
    const int st = routed ? p.offsets[g] : p.shared_base;
    const int rw = routed ? p.offsets[g + 1] - st : p.T;
    const int rem = rw & 255;
    if (rem == 0 || rem > 128) return;
    const int S = p.tail_split;
    const size_t plane = (size_t)G * 128 * N;
    const float *part = p.part + (size_t)g * 128 * N;
    const int Fb = gated ? N >> 1 : N;         // bias row length
    const uint16_t *b1 = routed
        ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * Fb : nullptr)
        : (const uint16_t *)p.bias_s;
    const uint16_t *b3 = !gated ? nullptr
        : routed ? (p.bias3 ? (const uint16_t *)p.bias3 + (size_t)g * Fb : nullptr)
                 : (const uint16_t *)p.bias_s3;
    uint16_t *out = (uint16_t *)p.out;
    for (int i = threadIdx.x; i < rem * 16; i += blockDim.x) {
        const int r = i >> 4, c = c0 + (i & 15) * 8;
        const float *src = part + (size_t)r * N;
        float v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int f = c + t;
            if (gated) {
                const int cg = 64 * (f >> 5) + (f & 31);
                float gv = src[cg], uv = src[cg + 32];
                for (int k = 1; k < S; ++k) {
                    gv += src[k * plane + cg];
                    uv += src[k * plane + cg + 32];
                }
                if (b1) gv += bf16_to_f32(b1[f]);
                if (b3) uv += bf16_to_f32(b3[f]);
                v[t] = silu_f(gv) * uv;
            } else {
                float s = src[f];
                for (int k = 1; k < S; ++k) s += src[k * plane + f];
                if (b1) s += bf16_to_f32(b1[f]);
                v[t] = UP ? act_up(p.act, s) : s;
            }
        }
        u32x4 o;
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = pack_bf16x2(v[2 * t], v[2 * t + 1]);
        *(u32x4 *)(out + (size_t)(st + rw - rem + r) * p.ldo + c) = o;
    }
}

// ---------------------------------------------------------------------
// Weight-streaming kernel for groups of at most a few dozen rows (decode).
// Work units are (group, 32-column slab) over the full K; the grid is
// persistent and walks the units with a stride, so equal-cost units spread
// evenly over the resident blocks.  A unit loops over 32-row chunks of its
// group (normally one).  The four waves split K into quarters; each wave
// streams its weight rows straight into v_mfma_f32_16x16x32_bf16 fragments
// (no LDS staging: every weight byte feeds exactly one MFMA).  In that
// layout four lanes read one 64-byte run of a weight row, and the token
// rows are read as 16-row halves, the second half only when the chunk has
// more than 16 rows.  Two batches of SU sub-steps are kept in flight, and
// the four partial accumulators are summed through LDS in a fixed order
// before the epilogue.
template <int MT, int TN, int SU>
__device__ __forceinline__ void stream_chunk(floatx4 (&acc)[2][TN],
                                             const uint16_t *const (&wt)[TN],
                                             const uint16_t *a0,
                                             const uint16_t *a1, int kq) {
    u32x4 av[2][SU][MT], bv[2][SU][TN];
    auto load = [&](int buf, int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < SU; ++s) {
#pragma unroll
            for (int n = 0; n < TN; ++n)
                bv[buf][s][n] = *(const u32x4 *)(wt[n] + k0 + s * 32);
            av[buf][s][0] = *(const u32x4 *)(a0 + k0 + s * 32);
            if (MT == 2) av[buf][s][MT - 1] = *(const u32x4 *)(a1 + k0 + s * 32);
        }
    };
    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < SU; ++s)
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < TN; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(bv[buf][s][n]), as_bf16x8(av[buf][s][m]),
                        acc[m][n], 0, 0, 0);
    };
    constexpr int STEP = 32 * SU;
    load(0, 0);
    for (int k0 = 0; k0 < kq; k0 += 2 * STEP) {
        if (k0 + STEP < kq) load(1, k0 + STEP);
        __builtin_amdgcn_sched_barrier(0);
        compute(0);
        __builtin_amdgcn_sched_barrier(0);
        if (k0 + STEP < kq) {
            if (k0 + 2 * STEP < kq) load(0, k0 + 2 * STEP);
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// FP8 (OCP E4M3) weight rows, bf16 activations.  Each lane loads 16
// weight bytes, the run k = 16q .. 16q+15 of a 64-deep sub-step (q =
// lane/16), and feeds two MFMAs with them (bytes 0-7, then 8-15), decoded
// exactly to bf16 (every E4M3 value is a bf16 value: the fp32 decode's
// upper half).  The token rows are read at the same k (two 16-byte loads),
// so both operands agree on the k order inside each MFMA.  The
// per-output-channel scale is applied in the epilogue.
__device__ __forceinline__ uint32_t upper_halves(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
    const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
    const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
    const f2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
    u32x4 r;
    r[0] = upper_halves(a[0], a[1]);
    r[1] = upper_halves(b[0], b[1]);
    r[2] = upper_halves(c[0], c[1]);
    r[3] = upper_halves(d[0], d[1]);
    return r;
}

template <int MT, int TN, int SU>
__device__ __forceinline__ void stream_chunk_fp8(floatx4 (&acc)[2][TN],
                                                 const uint8_t *const (&wt)[TN],
                                                 const uint16_t *a0,
                                                 const uint16_t *a1, int kq) {
    u32x4 av[2][SU][MT][2], bv[2][SU][TN];
    auto load = [&](int buf, int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < SU; ++s) {
#pragma unroll
            for (int n = 0; n < TN; ++n)
                bv[buf][s][n] = *(const u32x4 *)(wt[n] + k0 + s * 64);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                av[buf][s][0][h] = *(const u32x4 *)(a0 + k0 + s * 64 + 8 * h);
                if (MT == 2)
                    av[buf][s][MT - 1][h] =
                        *(const u32x4 *)(a1 + k0 + s * 64 + 8 * h);
            }
        }
    };
    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < SU; ++s)
#pragma unroll
            for (int n = 0; n < TN; ++n) {
                const u32x4 q = bv[buf][s][n];
                const u32x4 lo = e4m3x8_to_bf16x8(q[0], q[1]);
                const u32x4 hi = e4m3x8_to_bf16x8(q[2], q[3]);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(lo), as_bf16x8(av[buf][s][m][0]), acc[m][n],
                        0, 0, 0);
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(hi), as_bf16x8(av[buf][s][m][1]), acc[m][n],
                        0, 0, 0);
                }
            }
    };
    constexpr int STEP = 64 * SU;
    load(0, 0);
    for (int k0 = 0; k0 < kq; k0 += 2 * STEP) {
        if (k0 + STEP < kq) load(1, k0 + STEP);
        __builtin_amdgcn_sched_barrier(0);
        compute(0);
        __builtin_amdgcn_sched_barrier(0);
        if (k0 + STEP < kq) {
            if (k0 + 2 * STEP < kq) load(0, k0 + 2 * STEP);
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// FP8 = false: bf16 weights; true: E4M3 weights with per-channel scales.
// NB = columns per unit (NB/16 MFMA tiles): wider units re-read the token
// rows fewer times per weight byte.
template <bool UP, bool FP8, int NB>
__global__ __launch_bounds__(256, 2) void gemm_stream(GemmParams p) {
    constexpr int TN = NB / 16;
    // sub-steps per load batch: 32-deep (bf16) or 64-deep (FP8) ones
    constexpr int SU = NB == 32 ? 4 : 2;
    __shared__ float part[4][32][NB + 1];
    __shared__ TileTable tt;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int N = p.N, K = p.K;
    const int NTN = N / NB;
    const int G = p.E + p.n_shared;
    build_tile_table(tt, p.offsets, p.E, p.n_shared, p.shared_base, p.T, 32,
                     NTN);
    const uint16_t *A = (const uint16_t *)p.A;
    const int kq = K / 4;                     // this wave's K range
    const int kbeg = wave * kq;
    // k offset of this lane inside a sub-step: 8 bf16 of a 32-deep one, or
    // 16 of a 64-deep one for FP8 weights
    const int kg = FP8 ? (lane >> 4) * 16 : (lane >> 4) * 8;
    const int r16 = lane & 15;
    uint16_t *out = (uint16_t *)p.out;

    for (int u = blockIdx.x; u < G * NTN; u += gridDim.x) {
        const int g = u / NTN, n_tile = u - g * NTN;
        if (tt.rows[g] == 0) continue;
        const bool routed = g < p.E;
        const int esz = FP8 ? 1 : 2;         // bytes per weight
        const int n0 = n_tile * NB;
        // this lane's weight row of every 16-row MFMA tile of the unit
        const char *wt[TN];
#pragma unroll
        for (int n = 0; n < TN; ++n)
            wt[n] = weight_row(p, routed, g, n0 + 16 * n + r16, esz) +
                    (size_t)(kbeg + kg) * esz;

        for (int mc = 0; mc < tt.mt[g]; ++mc) {
            const int row0 = tt.start[g] + mc * 32;
            const int nrows = min(32, tt.rows[g] - mc * 32);
            int src[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int rr = h * 16 + r16;
                src[h] = 0;
                if (rr < nrows) {
                    const int slot = row0 + rr;
                    src[h] = slot;
                    if (UP)
                        src[h] = routed ? p.slot_token[slot]
                                        : slot - p.shared_base;
                }
            }
            const uint16_t *a0 = A + (size_t)src[0] * K + kbeg + kg;
            const uint16_t *a1 = A + (size_t)src[1] * K + kbeg + kg;
            floatx4 acc[2][TN];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < TN; ++n)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[m][n][v] = 0.0f;
            if (FP8) {
                const uint8_t *q[TN];
#pragma unroll
                for (int n = 0; n < TN; ++n) q[n] = (const uint8_t *)wt[n];
                if (nrows > 16)
                    stream_chunk_fp8<2, TN, NB == 32 ? 2 : 1>(acc, q, a0, a1,
                                                              kq);
                else
                    stream_chunk_fp8<1, TN, SU>(acc, q, a0, a1, kq);
            } else {
                const uint16_t *b[TN];
#pragma unroll
                for (int n = 0; n < TN; ++n) b[n] = (const uint16_t *)wt[n];
                if (nrows > 16)
                    stream_chunk<2, TN, SU>(acc, b, a0, a1, kq);
                else
                    stream_chunk<1, TN, SU>(acc, b, a0, a1, kq);
            }
            // lane holds row m = 16*mt + lane%16, features
            // 16*nt + 4*(lane/16) + 0..3
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < TN; ++n)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        part[wave][16 * m + r16][16 * n + 4 * (lane >> 4) + v] =
                            acc[m][n][v];
            __syncthreads();
            if (UP && p.gated) {
                // a 64-column unit of the virtual panel: columns 0-31 are
                // the gate rows and 32-63 the up rows of features
                // 32*n_tile + 0..31
                const int F = N >> 1, f0 = n0 >> 1;
                const uint16_t *b1 = routed
                    ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * F : nullptr)
                    : (const uint16_t *)p.bias_s;
                const uint16_t *b3 = routed
                    ? (p.bias3 ? (const uint16_t *)p.bias3 + (size_t)g * F : nullptr)
                    : (const uint16_t *)p.bias_s3;
                const float *s1 = FP8 ? (routed ? p.scale + (size_t)g * F : p.scale_s)
                                      : nullptr;
                const float *s3 = FP8 ? (routed ? p.scale3 + (size_t)g * F : p.scale_s3)
                                      : nullptr;
                for (int e = tid; e < 32 * 16; e += 256) {
                    const int m = e >> 4;
                    const int c = (e & 15) * 2;
                    if (m < nrows) {
                        float h[2];
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            float gv = part[0][m][c + i] + part[1][m][c + i];
                            gv += part[2][m][c + i];
                            gv += part[3][m][c + i];
                            float uv = part[0][m][32 + c + i] + part[1][m][32 + c + i];
                            uv += part[2][m][32 + c + i];
                            uv += part[3][m][32 + c + i];
                            if (FP8) {
                                gv *= s1[f0 + c + i];
                                uv *= s3[f0 + c + i];
                            }
                            if (b1) gv += bf16_to_f32(b1[f0 + c + i]);
                            if (b3) uv += bf16_to_f32(b3[f0 + c + i]);
                            h[i] = silu_f(gv) * uv;
                        }
                        *(uint32_t *)(out + (size_t)(row0 + m) * p.ldo + f0 + c) =
                            pack_bf16x2(h[0], h[1]);
                    }
                }
            } else {
                const uint16_t *bg = routed
                    ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * N : nullptr)
                    : (const uint16_t *)p.bias_s;
                const float *sg = FP8 ? (routed ? p.scale + (size_t)g * N : p.scale_s)
                                      : nullptr;
                for (int e = tid; e < 32 * NB / 2; e += 256) {
                    const int m = e / (NB / 2);
                    const int c = (e - m * (NB / 2)) * 2;
                    if (m < nrows) {
                        float v0 = part[0][m][c] + part[1][m][c];
                        v0 += part[2][m][c];
                        v0 += part[3][m][c];
                        float v1 = part[0][m][c + 1] + part[1][m][c + 1];
                        v1 += part[2][m][c + 1];
                        v1 += part[3][m][c + 1];
                        if (FP8) {
                            v0 *= sg[n0 + c];
                            v1 *= sg[n0 + c + 1];
                        }
                        if (bg) {
                            v0 += bf16_to_f32(bg[n0 + c]);
                            v1 += bf16_to_f32(bg[n0 + c + 1]);
                        }
                        if (UP) {
                            v0 = act_up(p.act, v0);
                            v1 = act_up(p.act, v1);
                        }
                        *(uint32_t *)(out + (size_t)(row0 + m) * p.ldo + n0 + c) =
                            pack_bf16x2(v0, v1);
                    }
                }
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------
// Weight-ring kernel for groups of at most 16 rows (decode).  HBM delivers
// the most when each row of a weight panel is read in runs of a few KB
// requested together, which the MFMA operand layout cannot give when
// loading straight into registers (one load instruction covers 64 bytes of
// each of 16 rows).  Here the weights pass through LDS instead: a stage is
// 16 weight rows x CB bytes, fetched with non-temporal direct-to-LDS loads
// in whole 1 KB runs per wave instruction, into a ring of four stages
// (three in flight).  A unit is (group, 16-row chunk of the group, 64
// output columns = four groups of 16 weight rows; gated: 32 features, their
// gate rows then their up rows) over the whole of K, walked k range by k
// range and, inside each, row group by row group; the token rows of a k
// range are loaded into registers once, with its first stage, and serve
// its four stages.  The ring runs on across the units of a block, so
// nothing drains between units; every step issues a fixed set of loads
// (past the last stage they re-read one line), so the waits are fixed
// counts.  The four waves split each stage's k range in quarters; a unit's
// partial sums are added through LDS (the slot its last stage leaves) in a
// fixed order.  Each LDS row of a stage is padded by four 16-byte chunks
// and its chunks XOR-swizzled by the row, so that the fragment reads (16
// rows, one chunk) fall in distinct bank groups while every sub-step's
// read is at a fixed offset from one address.
namespace ring {
constexpr int MAXTOK = MOE_RING_MAXTOK;

__device__ __forceinline__ void dma16nt(const char *src, u32x4 *lds) {
    __builtin_amdgcn_global_load_lds(
        (const void *)src, (__attribute__((address_space(3))) void *)lds, 16,
        0, 2 /* non-temporal */);
}

__device__ __forceinline__ void dma4(const char *src, u32x4 *lds) {
    __builtin_amdgcn_global_load_lds(
        (const void *)src, (__attribute__((address_space(3))) void *)lds, 4,
        0, 0);
}
}  // namespace ring

template <bool UP, bool FP8, int CB, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_ring(GemmParams p) {
    constexpr int CPR = CB / 16;          // 16-byte chunks of a row per stage
    // LDS rows of CPR + 4 chunks, and chunk c of row r at c ^ ((r / 2) % 4)
    // (low two bits): the fragment reads (16 rows at one chunk) then run
    // without bank conflicts on gfx950, which rows padded by one chunk did
    // not (two passes a read, rocprof counters)
    constexpr int RS = CPR + 4;           // LDS row stride (chunks)
    constexpr int CPS = 16 * RS;          // chunks per stage
    constexpr int EPI = 32;               // epilogue chunks per slot
    constexpr int NI = CB / 256;          // 1 KB weight loads per wave
    constexpr int SS = CB / 256;          // sub-steps per wave per stage
    constexpr int NA = FP8 ? 2 * SS : SS; // token-row loads per k range
    constexpr int PW = 2 + NI;            // loads of a stage (constants, weights)
    constexpr int PA = PW + NA;           // ... of the first stage of a k range
    constexpr int esz = FP8 ? 1 : 2;
    static_assert(PW + PA < 64, "vmcnt range");
    static_assert(CPS * 16 >= 4 * 4 * 16 * 16 * 4, "reduction fits a stage");
    // A slot: the stage, then the unit's epilogue constants, 128 dwords
    // (every wave loads the same copy): 0-31 the bf16 biases of the 64
    // columns (gated: 0-15 the 32 gate biases, 32-47 the 32 up biases),
    // 64-127 the FP8 scales (gated: 64-95 gate, 96-127 up).
    __shared__ u32x4 sl0[CPS + EPI], sl1[CPS + EPI], sl2[CPS + EPI],
        sl3[CPS + EPI];
    __shared__ int stok[ring::MAXTOK];
    __shared__ TileTable tt;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q = lane >> 4;
    const int G = p.E + p.n_shared;
    const bool gated = UP && p.gated;
    const int KC = p.K * esz / CB;        // k ranges
    const int SPU = 4 * KC;               // stages per unit
    const int NS = p.N / 64;              // 64-column slabs
    if (UP) {
        const int ns = p.offsets[p.E];
        for (int i = tid; i < ns; i += 256) stok[i] = p.slot_token[i];
    }
    build_tile_table(tt, p.offsets, p.E, p.n_shared, p.shared_base, p.T, 16,
                     NS);
    const int units = tt.base[G];
    // bf16: as few blocks as give every block the same number of units (a
    // block with one unit fewer than the rest would leave its share of the
    // bandwidth idle for a unit's time: Mixtral-shaped up GEMM 162 -> 152
    // us).  FP8 units carry half the bytes, and there the blocks left idle
    // cost more than the uneven last unit (81 against 86 us): every block.
    const int per = (units + (int)gridDim.x - 1) / (int)gridDim.x;
    const int nb = FP8 ? (int)gridDim.x : per > 0 ? (units + per - 1) / per : 0;
    const int bid = blockIdx.x;
    const int nmine = bid < units && bid < nb ? (units - 1 - bid) / nb + 1 : 0;
    const int total = nmine * SPU;
    if (total == 0) return;

    struct Unit { int g, slab, row0, nrows; };
    auto unit_of = [&](int ui) __attribute__((always_inline)) {
        const int u = bid + ui * nb;
        Unit r;
        r.g = __builtin_amdgcn_readfirstlane(find_group(tt, G, u));
        const int local = u - __builtin_amdgcn_readfirstlane(tt.base[r.g]);
        const int mt = __builtin_amdgcn_readfirstlane(tt.mt[r.g]);
        r.slab = local / mt;
        const int mc = local - r.slab * mt;
        r.row0 = __builtin_amdgcn_readfirstlane(tt.start[r.g]) + 16 * mc;
        r.nrows = min(16, __builtin_amdgcn_readfirstlane(tt.rows[r.g]) - 16 * mc);
        return r;
    };

    // Issue cursor: the next stage to issue is row group (stage index & 3)
    // of k range ikc of unit iu.  On entering a unit: the first weight row
    // of each row group, this lane's token row (at the lane's k offset) and
    // the sources of this lane's two epilogue-constant dwords.
    const size_t rowb = (size_t)p.K * esz;
    int iu = 0, ikc = 0;
    const char *wr[4] = {nullptr, nullptr, nullptr, nullptr};
    const char *e0 = nullptr, *e1 = nullptr;
    const uint16_t *arow = nullptr;
    auto enter = [&](int ui) __attribute__((always_inline)) {
        const Unit U = unit_of(ui);
        const bool routed = U.g < p.E;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
            wr[rg] = weight_row(p, routed, U.g, 64 * U.slab + 16 * rg, esz);
        const int slotrow = U.row0 + (l16 < U.nrows ? l16 : 0);
        int src = slotrow;
        if (UP) src = routed ? stok[slotrow] : slotrow - p.shared_base;
        arow = (const uint16_t *)p.A + (size_t)src * p.K +
               (FP8 ? (CB / 4) * wave + 16 * q : (CB / 8) * wave + 8 * q);
        // constants: the unit's 64 columns, or (gated) its 32 features
        const int F = gated ? p.N >> 1 : p.N;
        const int c0 = gated ? 32 * U.slab : 64 * U.slab;
        const uint16_t *b1 = routed
            ? (p.bias ? (const uint16_t *)p.bias + (size_t)U.g * F : nullptr)
            : (const uint16_t *)p.bias_s;
        const uint16_t *b3 = !gated ? nullptr : routed
            ? (p.bias3 ? (const uint16_t *)p.bias3 + (size_t)U.g * F : nullptr)
            : (const uint16_t *)p.bias_s3;
        const float *s1 = !FP8 ? nullptr : routed ? p.scale + (size_t)U.g * F : p.scale_s;
        const float *s3 = !(FP8 && gated) ? nullptr
            : routed ? p.scale3 + (size_t)U.g * F : p.scale_s3;
        e0 = nullptr;
        e1 = nullptr;
        if (gated) {
            if (lane < 16) e0 = b1 ? (const char *)(b1 + c0) + 4 * lane : nullptr;
            else if (lane >= 32 && lane < 48)
                e0 = b3 ? (const char *)(b3 + c0) + 4 * (lane - 32) : nullptr;
            if (lane < 32) e1 = s1 ? (const char *)(s1 + c0 + lane) : nullptr;
            else e1 = s3 ? (const char *)(s3 + c0 + lane - 32) : nullptr;
        } else {
            if (lane < 32) e0 = b1 ? (const char *)(b1 + c0) + 4 * lane : nullptr;
            e1 = s1 ? (const char *)(s1 + c0 + lane) : nullptr;
        }
        if (!e0) e0 = wr[0];
        if (!e1) e1 = wr[0];
    };

    // Issue the next stage (row group RG of k range ikc): the constants and
    // 16 weight rows x CB bytes into slot (this wave: rows 4 wave .. +3),
    // and for row group 0 this wave's quarter of the k range's token rows
    // into ab.  Past the last stage the cursor stays on the last unit and
    // each weight load re-reads one line (its lane offset is multiplied by
    // zero: a select between two addresses would give the compiler a
    // second path and cost exact waits).
    auto issue = [&](auto rgc, bool real, u32x4 *slot, u32x4 (&ab)[NA]) __attribute__((always_inline)) {
        constexpr int RG = decltype(rgc)::value;
        if (RG == 0 && real && ikc == 0) enter(iu);
        u32x4 *ep = slot + CPS;
        ring::dma4(e0, ep);
        ring::dma4(e1, ep + 16);
        const char *wb = wr[RG] + (size_t)ikc * CB + 4 * wave * rowb;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            // 1 KB of row 4 wave + jr (half h of a 2 KB run); the lane
            // fetches the chunk that the row's swizzle puts at its position
            const int jr = NI == 8 ? j >> 1 : j, h = NI == 8 ? (j & 1) : 0;
            const int sw = ((4 * wave + jr) >> 1) & 3;
            const uint32_t loff = (uint32_t)(lane ^ sw) * 16 * (uint32_t)real;
            ring::dma16nt(wb + jr * rowb + h * 1024 + loff,
                          slot + (4 * wave + jr) * RS + h * 64);
        }
        if (RG == 0) {
            const uint16_t *a = arow + (size_t)ikc * (FP8 ? CB : CB / 2);
#pragma unroll
            for (int s = 0; s < SS; ++s) {
                if (FP8) {
                    ab[2 * s] = *(const u32x4 *)(a + 64 * s);
                    ab[2 * s + 1] = *(const u32x4 *)(a + 64 * s + 8);
                } else {
                    ab[s] = *(const u32x4 *)(a + 32 * s);
                }
            }
        }
        if (RG == 3 && real && ++ikc == KC) {
            ikc = 0;
            ++iu;
        }
    };

    floatx4 acc[4];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) acc[rg] = floatx4{0.f, 0.f, 0.f, 0.f};
    uint16_t *out = (uint16_t *)p.out;

    // The unit's partial sums are complete: add the four waves' through
    // the slot its last stage left, finish, store.
    auto finish = [&](int ui, u32x4 *slot) __attribute__((always_inline)) {
        const Unit U = unit_of(ui);
        // [wave][row group][16 tokens][16 columns]: 16 KB, inside the
        // stage part of the slot; every wave has read the stage first
        float *red = (float *)slot;
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[((wave * 4 + rg) * 16 + l16) * 16 + 4 * q + v] = acc[rg][v];
        __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        const uint32_t *ep = (const uint32_t *)(slot + CPS);
        const uint16_t *eb = (const uint16_t *)ep;
        const float *es = (const float *)(ep + 64);
        const bool routed = U.g < p.E;
        const int m = tid >> 4;
        auto sum = [&](int col) __attribute__((always_inline)) {
            // virtual column col (0..63) of the unit: row group col / 16
            const int rg = col >> 4, c = col & 15;
            float x = red[((0 * 4 + rg) * 16 + m) * 16 + c] +
                      red[((1 * 4 + rg) * 16 + m) * 16 + c];
            x += red[((2 * 4 + rg) * 16 + m) * 16 + c];
            x += red[((3 * 4 + rg) * 16 + m) * 16 + c];
            return x;
        };
        if (gated) {
            // features 2 (tid & 15), +1 of the unit's 32
            const bool has_b1 = routed ? p.bias != nullptr : p.bias_s != nullptr;
            const bool has_b3 = routed ? p.bias3 != nullptr : p.bias_s3 != nullptr;
            float h[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int f = 2 * (tid & 15) + i;
                float gv = sum(f), uv = sum(32 + f);
                if (FP8) {
                    gv *= es[f];
                    uv *= es[32 + f];
                }
                if (has_b1) gv += bf16_to_f32(eb[f]);
                if (has_b3) uv += bf16_to_f32(eb[64 + f]);
                h[i] = silu_f(gv) * uv;
            }
            if (m < U.nrows)
                *(uint32_t *)(out + (size_t)(U.row0 + m) * p.ldo + 32 * U.slab +
                              2 * (tid & 15)) = pack_bf16x2(h[0], h[1]);
        } else {
            // columns 4 (tid & 15) .. +3 of the unit's 64
            const bool has_b = routed ? p.bias != nullptr : p.bias_s != nullptr;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 4 * (tid & 15) + i;
                float x = sum(c);
                if (FP8) x *= es[c];
                if (has_b) x += bf16_to_f32(eb[c]);
                v[i] = UP ? act_up(p.act, x) : x;
            }
            if (m < U.nrows) {
                u32x2 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                *(u32x2 *)(out + (size_t)(U.row0 + m) * p.ldo + 64 * U.slab +
                           4 * (tid & 15)) = o;
            }
        }
    };

    auto compute = [&](auto rgc, const u32x4 *slot, const u32x4 (&ab)[NA]) __attribute__((always_inline)) {
        constexpr int RG = decltype(rgc)::value;
        const u32x4 *brow = slot + l16 * RS + (CPR / 4) * wave + (q ^ ((l16 >> 1) & 3));
#pragma unroll
        for (int s = 0; s < SS; ++s) {
            // this lane's 16 weight bytes: row l16, chunk 4 s + q of the
            // wave's quarter of the stage
            const u32x4 b = brow[4 * s];
            if (FP8) {
                acc[RG] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(e4m3x8_to_bf16x8(b[0], b[1])), as_bf16x8(ab[2 * s]),
                    acc[RG], 0, 0, 0);
                acc[RG] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(e4m3x8_to_bf16x8(b[2], b[3])), as_bf16x8(ab[2 * s + 1]),
                    acc[RG], 0, 0, 0);
            } else {
                acc[RG] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(b), as_bf16x8(ab[s]), acc[RG], 0, 0, 0);
            }
        }
    };

    // Step t (t % 8 == I): stage t landed everywhere (this wave's loads of
    // the next two stages may still be in flight), stage t + 3 issued into
    // the slot that stage t - 1 left, stage t (row group I % 4, token rows
    // of set I / 4) consumed; the last stage of a unit finishes it (steps
    // past the last stage change only acc).
    int cu = 0, ckc = 0;
    u32x4 abs0[NA], abs1[NA];
    auto step = [&](auto ic, int t, u32x4 *cur, u32x4 *nxt) __attribute__((always_inline)) {
        constexpr int I = decltype(ic)::value;
        constexpr int RG = I % 4, NRG = (I + 3) % 4;
        // loads issued after stage t: stages t + 1 and t + 2
        constexpr int AFTER = ((I + 1) % 4 == 0 || (I + 2) % 4 == 0) ? PW + PA : 2 * PW;
        wait_vmcnt<AFTER>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (((I + 3) / 4) % 2 == 0)
            issue(std::integral_constant<int, NRG>{}, t + 3 < total, nxt, abs0);
        else
            issue(std::integral_constant<int, NRG>{}, t + 3 < total, nxt, abs1);
        __builtin_amdgcn_sched_barrier(0);
        if (I / 4 == 0) compute(std::integral_constant<int, RG>{}, cur, abs0);
        else compute(std::integral_constant<int, RG>{}, cur, abs1);
        if (RG == 3 && ++ckc == KC) {
            if (t < total) finish(cu, cur);
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) acc[rg] = floatx4{0.f, 0.f, 0.f, 0.f};
            ckc = 0;
            ++cu;
        }        // keep this step's MFMAs ahead of the next step's barrier
        __builtin_amdgcn_sched_barrier(0);
    };

    issue(std::integral_constant<int, 0>{}, true, sl0, abs0);
    issue(std::integral_constant<int, 1>{}, 1 < total, sl1, abs0);
    issue(std::integral_constant<int, 2>{}, 2 < total, sl2, abs0);
    // whole rounds of eight steps (two k ranges)
    for (int t = 0; t < total; t += 8) {
        step(std::integral_constant<int, 0>{}, t, sl0, sl3);
        step(std::integral_constant<int, 1>{}, t + 1, sl1, sl0);
        step(std::integral_constant<int, 2>{}, t + 2, sl2, sl1);
        step(std::integral_constant<int, 3>{}, t + 3, sl3, sl2);
        step(std::integral_constant<int, 4>{}, t + 4, sl0, sl3);
        step(std::integral_constant<int, 5>{}, t + 5, sl1, sl0);
        step(std::integral_constant<int, 6>{}, t + 6, sl2, sl1);
        step(std::integral_constant<int, 7>{}, t + 7, sl3, sl2);
    }
    __builtin_amdgcn_s_waitcnt(0);   // the trailing re-reads have landed
}

// fp32 grouped GEMM on the vector ALUs (64 x 64 x 16 tiles, 4 x 4 outputs
// per thread, sequential fp32 FMA over k).
template <bool UP>
__global__ __launch_bounds__(256) void gemm_f32_simt(GemmParams p) {
    constexpr int BM = 64, BN = 64, BKF = 16;
    __shared__ float As[BKF][BM + 4];
    __shared__ float Bs[BKF][BN + 4];
    __shared__ TileTable tt;
    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
    const int N = p.N, K = p.K;
    const int G = p.E + p.n_shared;
    build_tile_table(tt, p.offsets, p.E, p.n_shared, p.shared_base, p.T, BM,
                     N / BN);
    const int total = tt.base[G];
    const float *A = (const float *)p.A;
    const int lr = tid >> 2, lk = (tid & 3) * 4;
    for (int L = blockIdx.x; L < total; L += gridDim.x) {
        const int g = find_group(tt, G, L);
        const int local = L - tt.base[g];
        const int mt = tt.mt[g];
        const int n_tile = local / mt, m_tile = local - n_tile * mt;
        const int row0 = tt.start[g] + m_tile * BM;
        const int nrows = min(BM, tt.rows[g] - m_tile * BM);
        const int n0 = n_tile * BN;
        const bool routed = g < p.E;
        const bool gated = UP && p.gated;
        const float *arow = nullptr;
        if (lr < nrows) {
            const int slot = row0 + lr;
            int src = slot;
            if (UP) src = routed ? p.slot_token[slot] : slot - p.shared_base;
            arow = A + (size_t)src * K;
        }
        const float *brow = (const float *)weight_row(p, routed, g, n0 + lr, 4);
        // this thread's 4 tile columns: 4*tx .. 4*tx+3, or (gated) the
        // gate columns 2*tx, 2*tx+1 and their up columns 32 + 2*tx, +1
        const int cb0 = gated ? 2 * tx : 4 * tx;
        const int cb1 = gated ? 32 + 2 * tx : 4 * tx + 2;
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
        for (int k0 = 0; k0 < K; k0 += BKF) {
            const float4 av = arow ? *(const float4 *)(arow + k0 + lk)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 bv = *(const float4 *)(brow + k0 + lk);
            As[lk + 0][lr] = av.x;
            As[lk + 1][lr] = av.y;
            As[lk + 2][lr] = av.z;
            As[lk + 3][lr] = av.w;
            Bs[lk + 0][lr] = bv.x;
            Bs[lk + 1][lr] = bv.y;
            Bs[lk + 2][lr] = bv.z;
            Bs[lk + 3][lr] = bv.w;
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < BKF; ++kk) {
                const float4 a4 = *(const float4 *)&As[kk][ty * 4];
                const float2 b01 = *(const float2 *)&Bs[kk][cb0];
                const float2 b23 = *(const float2 *)&Bs[kk][cb1];
                const float a[4] = {a4.x, a4.y, a4.z, a4.w};
                const float b[4] = {b01.x, b01.y, b23.x, b23.y};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
            __syncthreads();
        }
        float *out = (float *)p.out;
        if (gated) {
            const int F = N >> 1, f = (n0 >> 1) + 2 * tx;
            const float *b1 = routed
                ? (p.bias ? (const float *)p.bias + (size_t)g * F : nullptr)
                : (const float *)p.bias_s;
            const float *b3 = routed
                ? (p.bias3 ? (const float *)p.bias3 + (size_t)g * F : nullptr)
                : (const float *)p.bias_s3;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = ty * 4 + i;
                if (m >= nrows) continue;
                float h[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float gv = acc[i][j], uv = acc[i][2 + j];
                    if (b1) gv += b1[f + j];
                    if (b3) uv += b3[f + j];
                    h[j] = silu_f(gv) * uv;
                }
                *(float2 *)(out + (size_t)(row0 + m) * p.ldo + f) =
                    make_float2(h[0], h[1]);
            }
            continue;
        }
        const float *bg = routed
            ? (p.bias ? (const float *)p.bias + (size_t)g * N : nullptr)
            : (const float *)p.bias_s;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = ty * 4 + i;
            if (m >= nrows) continue;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + tx * 4 + j;
                float z = acc[i][j];
                if (bg) z += bg[n];
                v[j] = UP ? act_up(p.act, z) : z;
            }
            *(float4 *)(out + (size_t)(row0 + m) * p.ldo + n0 + tx * 4) =
                make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

template <int BM, int BN, int WM, int WN, bool UP, int NS>
hipError_t launch_dma(const GemmParams &p, int grid, hipStream_t s) {
    const int lds = NS * (BM + BN) * 64;
    auto kern = gemm_bf16_dma<BM, BN, WM, WN, UP, NS>;
    hipError_t err = hipFuncSetAttribute((const void *)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(WM * WN * 64), lds, s, p);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool UP>
hipError_t launch_dma64(const GemmParams &p, int grid, hipStream_t s) {
    const int lds = 2 * (BM + BN) * 128;
    auto kern = gemm_bf16_dma64<BM, BN, WM, WN, UP>;
    hipError_t err = hipFuncSetAttribute((const void *)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(WM * WN * 64), lds, s, p);
    return hipGetLastError();
}

template <bool UP, int TM_ROWS, bool X32 = false, int TN_COLS = 256,
          bool NT = false>
hipError_t launch_w4(const GemmParams &p, int grid, hipStream_t s) {
    if (X32)
        hipLaunchKernelGGL((gemm_bf16_w4x<UP, TM_ROWS>), dim3(grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((gemm_bf16_w4<UP, TM_ROWS, TN_COLS, NT>), dim3(grid),
                           dim3(256), 0, s, p);
    if (TM_ROWS == 256 && p.tail_split > 1) {
        const int G = p.E + p.n_shared;
        const int oc = UP && p.gated ? p.N / 2 : p.N;
        hipLaunchKernelGGL(w4_tail_reduce<UP>, dim3(G * (oc / 128)), dim3(256),
                           0, s, p);
    }
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool UP>
hipError_t launch_lds(const GemmParams &p, int grid, hipStream_t s) {
    const int lds = 2 * (BM + BN) * 8 * 16;
    auto kern = gemm_bf16_lds<BM, BN, WM, WN, UP>;
    hipError_t err = hipFuncSetAttribute((const void *)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(WM * WN * 64), lds, s, p);
    return hipGetLastError();
}

}  // namespace

GemmVariantInfo gemm_variant_info(int variant) {
    switch (variant) {
    case GEMM_BF16_256x256: return {256, 256, 512, 2 * 512 * 128};
    case GEMM_BF16_128x256: return {128, 256, 256, 2 * 384 * 128};
    case GEMM_BF16_32x256: return {32, 256, 256, 2 * 288 * 128};
    case GEMM_BF16_64x64: return {64, 64, 256, 2 * 128 * 128};
    case GEMM_BF16_DMA_256x256: return {256, 256, 512, 4 * 512 * 64};
    case GEMM_BF16_DMA_128x256: return {128, 256, 256, 4 * 384 * 64};
    case GEMM_BF16_STREAM_32x64: return {32, 32, 256, 0};
    case GEMM_FP8_STREAM_32x64: return {32, 32, 256, 0};
    case GEMM_BF16_STREAM_64x64: return {32, 64, 256, 0};
    case GEMM_FP8_STREAM_64x64: return {32, 64, 256, 0};
    case GEMM_BF16_DMA64_256x256: return {256, 256, 512, 2 * 512 * 128};
    case GEMM_BF16_DMA64_128x256: return {128, 256, 256, 2 * 384 * 128};
    case GEMM_BF16_DMA64_320x256: return {320, 256, 512, 2 * 576 * 128};
    case GEMM_BF16_W4_256x256: return {256, 256, 256, 2 * 512 * 128};
    case GEMM_BF16_W4_128x256: return {128, 256, 256, 2 * 512 * 128};
    case GEMM_BF16_W4X_256x256: return {256, 256, 256, 2 * 512 * 128};
    case GEMM_BF16_W4X_128x256: return {128, 256, 256, 2 * 512 * 128};
    case GEMM_BF16_W4_256x192: return {256, 192, 256, 2 * 512 * 128};
    case GEMM_BF16_TALL_320x192: return {320, 192, 256, 2 * 512 * 128};
    case GEMM_BF16_TALL_288x224: return {288, 224, 256, 2 * 512 * 128};
    case GEMM_BF16_X2_128x256: return {128, 256, 256, 3 * 384 * 64};
    case GEMM_BF16_RING_16x16: return {16, 16, 256, 4 * 16 * MOE_RING_CB_BF16};
    case GEMM_FP8_RING_16x16: return {16, 16, 256, 4 * 16 * MOE_RING_CB_FP8};
    case GEMM_BF16_RING2_16x16: return {16, 16, 256, 4 * 16 * 1024};
    case GEMM_FP8_RING2_16x16: return {16, 16, 256, 4 * 16 * 1024};
    default: return {64, 64, 256, 0};
    }
}

hipError_t launch_gemm(const GemmParams &p, int variant, bool up, int grid,
                       hipStream_t s) {
    switch (variant) {
    case GEMM_BF16_256x256:
        return up ? launch_lds<256, 256, 2, 4, true>(p, grid, s)
                  : launch_lds<256, 256, 2, 4, false>(p, grid, s);
    case GEMM_BF16_128x256:
        return up ? launch_lds<128, 256, 2, 2, true>(p, grid, s)
                  : launch_lds<128, 256, 2, 2, false>(p, grid, s);
    case GEMM_BF16_32x256:
        return up ? launch_lds<32, 256, 1, 4, true>(p, grid, s)
                  : launch_lds<32, 256, 1, 4, false>(p, grid, s);
    case GEMM_BF16_64x64:
        return up ? launch_lds<64, 64, 2, 2, true>(p, grid, s)
                  : launch_lds<64, 64, 2, 2, false>(p, grid, s);
    case GEMM_BF16_DMA_256x256:
        return up ? launch_dma<256, 256, 2, 4, true, 4>(p, grid, s)
                  : launch_dma<256, 256, 2, 4, false, 4>(p, grid, s);
    case GEMM_BF16_DMA_128x256:
        return up ? launch_dma<128, 256, 2, 2, true, 4>(p, grid, s)
                  : launch_dma<128, 256, 2, 2, false, 4>(p, grid, s);
    case GEMM_BF16_DMA64_256x256:
        return up ? launch_dma64<256, 256, 2, 4, true>(p, grid, s)
                  : launch_dma64<256, 256, 2, 4, false>(p, grid, s);
    case GEMM_BF16_DMA64_128x256:
        return up ? launch_dma64<128, 256, 2, 2, true>(p, grid, s)
                  : launch_dma64<128, 256, 2, 2, false>(p, grid, s);
    case GEMM_BF16_DMA64_320x256:
        return up ? launch_dma64<320, 256, 2, 4, true>(p, grid, s)
                  : launch_dma64<320, 256, 2, 4, false>(p, grid, s);
    case GEMM_BF16_W4_256x256:
        return up ? launch_w4<true, 256>(p, grid, s)
                  : launch_w4<false, 256>(p, grid, s);
    case GEMM_BF16_W4_128x256:
        return up ? launch_w4<true, 128>(p, grid, s)
                  : launch_w4<false, 128>(p, grid, s);
    case GEMM_BF16_W4X_256x256:
        return up ? launch_w4<true, 256, true>(p, grid, s)
                  : launch_w4<false, 256, true>(p, grid, s);
    case GEMM_BF16_W4X_128x256:
        return up ? launch_w4<true, 128, true>(p, grid, s)
                  : launch_w4<false, 128, true>(p, grid, s);
    case GEMM_BF16_W4_256x192:
        // picked where every group is one row tile (expert choice with at
        // most 256 rows per expert): weights streamed non-temporally
        return up ? launch_w4<true, 256, false, 192, true>(p, grid, s)
                  : launch_w4<false, 256, false, 192, true>(p, grid, s);
    case GEMM_BF16_TALL_320x192: return launch_gemm_tall(p, 192, up, grid, s);
    case GEMM_BF16_TALL_288x224: return launch_gemm_tall(p, 224, up, grid, s);
    case GEMM_BF16_X2_128x256:
        if (up)
            hipLaunchKernelGGL(gemm_bf16_x2<true>, dim3(grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL(gemm_bf16_x2<false>, dim3(grid), dim3(256), 0, s, p);
        return hipGetLastError();

    case GEMM_BF16_RING_16x16:
        if (up)
            hipLaunchKernelGGL((gemm_ring<true, false, MOE_RING_CB_BF16, 1>),
                               dim3(grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_ring<false, false, MOE_RING_CB_BF16, 1>),
                               dim3(grid), dim3(256), 0, s, p);
        return hipGetLastError();
    case GEMM_FP8_RING_16x16:
        if (up)
            hipLaunchKernelGGL((gemm_ring<true, true, MOE_RING_CB_FP8, 1>),
                               dim3(grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_ring<false, true, MOE_RING_CB_FP8, 1>),
                               dim3(grid), dim3(256), 0, s, p);
        return hipGetLastError();
    case GEMM_BF16_RING2_16x16:
        if (up)
            hipLaunchKernelGGL((gemm_ring<true, false, 1024, 2>),
                               dim3(grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_ring<false, false, 1024, 2>),
                               dim3(grid), dim3(256), 0, s, p);
        return hipGetLastError();
    case GEMM_FP8_RING2_16x16:
        if (up)
            hipLaunchKernelGGL((gemm_ring<true, true, 1024, 2>),
                               dim3(grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_ring<false, true, 1024, 2>),
                               dim3(grid), dim3(256), 0, s, p);
        return hipGetLastError();
    case GEMM_BF16_STREAM_32x64:
        if (up)
            hipLaunchKernelGGL((gemm_stream<true, false, 32>), dim3(grid),
                               dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_stream<false, false, 32>), dim3(grid),
                               dim3(256), 0, s, p);
        return hipGetLastError();
    case GEMM_BF16_STREAM_64x64:
        if (up)
            hipLaunchKernelGGL((gemm_stream<true, false, 64>), dim3(grid),
                               dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_stream<false, false, 64>), dim3(grid),
                               dim3(256), 0, s, p);
        return hipGetLastError();
    case GEMM_FP8_STREAM_64x64:
        if (up)
            hipLaunchKernelGGL((gemm_stream<true, true, 64>), dim3(grid),
                               dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_stream<false, true, 64>), dim3(grid),
                               dim3(256), 0, s, p);
        return hipGetLastError();
    case GEMM_FP8_STREAM_32x64:
        if (up)
            hipLaunchKernelGGL((gemm_stream<true, true, 32>), dim3(grid),
                               dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_stream<false, true, 32>), dim3(grid),
                               dim3(256), 0, s, p);
        return hipGetLastError();
    default:
        if (up)
            hipLaunchKernelGGL(gemm_f32_simt<true>, dim3(grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL(gemm_f32_simt<false>, dim3(grid), dim3(256), 0, s, p);
        return hipGetLastError();
    }
}
