// Four-wave grouped GEMM with tall, narrow tiles: 320 x 192 or 288 x 224.
//
// "MoE architecture deep dive" (juejin.cn), sec. 3: fine-grained experts
// (DeepSeek-V3: 256 routed experts of width 2048 plus a shared one, top-8)
// give each expert about T k / E rows, 256 at T = 8192, in groups that
// scatter a few tens of rows either side.  "The expert group activated per
// token" (wmrh.cn), sec. 3.1: each expert is W2 GELU(W1 x + b1) + b2.
//
// The four-wave 256 x 256 tile holds a wave's 128 x 128 quarter in its 256
// accumulator registers, so a group of 257..384 rows takes two row tiles
// that each stream the expert's weight panel.  Here a wave holds 160 x 96
// (320 x 192 tiles, 240 accumulators) or 144 x 112 (288 x 224 tiles, 252
// accumulators), so such a group (most of the DeepSeek-shaped groups above
// 256 rows) is one tile that reads each weight panel once.  A stage of
// 64-deep rows is still 512 rows of 128 bytes (A rows from the start of an
// LDS slot, the BN weight rows at its end): 64 KB, the same two-slot ring,
// the same direct-to-LDS loads, XOR swizzle and issue schedule as the
// 256 x 256 kernel, with 7.9 (320 x 192) or 8.3 (288 x 224) MFLOP per
// stage against 8.4.
//
// A group of R rows runs as m = ceil(R / TRMAX) row tiles of the smallest
// height in {64, 128, 192, 256, 288, 320} (at most TRMAX) that holds
// ceil(R / m) rows.  Column tiles need not divide N: the last one is
// ragged (N = 2048 with 192-column tiles: 10 full and one of 128 columns);
// its weight loads past N re-read the last valid 8 rows and its columns
// past N are not stored.  In the 320 x 192 form with N >= 2048 a group of at
// most 256 rows (one row tile) takes 256-column tiles instead.  The epilogue (bias, GELU / SiLU for the up GEMM,
// bf16) stores straight from the accumulators: a lane's 4 consecutive
// columns of one row as an 8-byte store.
//
// A group that is one row tile (every DeepSeek-shaped routed group of up to
// 320 / 288 rows) streams its weight panel with the non-temporal hint:
// nothing else reads it, and the gathered token rows, which each of the
// group's column tiles reads again, then stay in L2.  On a probe of this
// load schedule (A rows shared by the 32 CUs of an XCD, every CU streaming
// its own weight panel from HBM) that raised the weight stream from 4.0 to
// 5.2 TB/s; the 256 x 256 kernel cannot use it for groups of 257..384
// rows, whose two row tiles share their panel through L2.
#include "kernels.h"

namespace {

namespace tall {
constexpr int SK = 64;              // stage depth (k)

// Direct global -> LDS load of 16 bytes per lane (the wave fills 1 KB from
// lds on), plain or with the non-temporal hint.
__device__ __forceinline__ void load16(const void *src, u32x4 *lds) {
    __builtin_amdgcn_global_load_lds(
        src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void load16_nt(const void *src, u32x4 *lds) {
    __builtin_amdgcn_global_load_lds(
        src, (__attribute__((address_space(3))) void *)lds, 16, 0,
        2 /* non-temporal */);
}

// s_waitcnt vmcnt(n) only.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) |
                               (0xF << 8));
}

// v_mfma_f32_16x16x32_bf16 into AGPR accumulators, as asm (with the builtin
// the accumulators get split between AGPRs and VGPRs and copied every step;
// as volatile asm the MFMAs also keep the issue order written here).
__device__ __forceinline__ void mfma16(floatx4 &acc, const bf16x8 &a,
                                       const bf16x8 &b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(acc)
                 : "v"(a), "v"(b));
}
constexpr int CPR = 8;              // 16-byte chunks per row and stage
constexpr int SROWS = 512;          // A and B rows per stage slot
constexpr int STAGE = SROWS * CPR;  // 16-byte units per slot (64 KB)

// Row-tile height of a group of `rows` rows split into mt tiles.
template <int TRMAX>
__device__ __forceinline__ int height(int rows, int mt) {
    const int per = (rows + mt - 1) / mt;
    if (per <= 64) return 64;
    if (per <= 128) return 128;
    if (per <= 192) return 192;
    if (per <= 256) return 256;
    if (per <= 288 || TRMAX == 288) return 288;
    return 320;
}
}  // namespace tall

// One tile of TR = 2 WR rows and BN columns; the waves are 2 x 2 parts of
// WR x BN / 2.  row0 / nrows: the tile's first slot row and its rows in the
// group; n0: its first column.  NT: the weights with the non-temporal hint
// (a group of one row tile: nothing else reads its panel, and the streamed
// weights then leave the gathered rows that every column tile reads in L2).
template <bool UP, int WR, int BN, bool NT>
__device__ __forceinline__ void tall_tile(const GemmParams &p, u32x4 *slot0,
                                          u32x4 *slot1, int g, int row0,
                                          int nrows, int n0, bool routed,
                                          int wave) {
    using namespace tall;
    constexpr int TN = BN / 32;         // 16-column blocks per wave
    constexpr int WC = BN / 2;          // columns per wave
    constexpr int RB = WR / 16;         // 16-row blocks per wave
    constexpr int TR = 2 * WR;          // tile rows
    constexpr int BOFF = SROWS - BN;    // first weight row of a slot
    static_assert(WR % 16 == 0 && TR <= BOFF, "A rows fit before the B rows");
    static_assert(RB * TN <= 64, "at most 256 accumulators a wave");
    constexpr int LA = TR / 32;         // A loads per wave and stage
    constexpr int LB = BN / 32;         // B loads per wave and stage
    constexpr int NL = LA + LB;
    constexpr int NF = RB + TN;         // fragment reads per sub-step
    constexpr int NM = RB * TN;         // MFMAs per sub-step
    // a fragment read after every RD MFMAs, a load after every DM, spread
    // over the sub-step as far as its MFMAs allow
    constexpr int RD = (NM - 1) / (NF - 1) < 3 ? (NM - 1) / (NF - 1) : 3;
    constexpr int DM = (NM - 2) / (NL - 1) < 4 ? (NM - 2) / (NL - 1) : 4;
    static_assert(RD >= 1 && DM >= 1 && RD * (NF - 1) < NM &&
                      DM * (NL - 1) + 1 < NM,
                  "issue slots");
    // The lane index is made opaque once per tile, so that the per-lane
    // addresses below are recomputed per tile rather than hoisted out of
    // the tile loop and spilled.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int N = p.N, K = p.K;
    const int KT = K / SK;
    const char *A = (const char *)p.A;
    // Load j of a wave fills operand rows 8 (wave + 4 j) + lane / 8, lane % 8
    // being the 16-byte slot; the lane fetches k-chunk (lane % 8) ^ ((row /
    // 2) % 8), which depends on the lane only, so that the fragment reads
    // (16 rows at one chunk) are free of bank conflicts.
    const int lr = lane >> 3;
    const int ch = (lane & 7) ^ ((4 * wave + (lr >> 1)) & 7);
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
    // weight rows in runs of 8 (N is a multiple of 16, so a run is wholly
    // inside or wholly past N); a run past N re-reads the last one
    const uint32_t b_lane = (uint32_t)(lr * K + ch * 8) * 2u;
    const char *bbase[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j)
        bbase[j] = weight_row(p, routed, g, min(n0 + (wave + 4 * j) * 8, N - 8), 2);

    auto dma_one = [&](int kt, u32x4 *st, int q) __attribute__((always_inline)) {
        const size_t ko = (size_t)kt * SK * 2;
        if (q < LA)
            load16(A + ko + a_off[q], st + (wave + 4 * q) * 64);
        else if (NT)
            load16_nt(bbase[q - LA] + ko + b_lane,
                      st + BOFF * CPR + (wave + 4 * (q - LA)) * 64);
        else
            load16(bbase[q - LA] + ko + b_lane,
                   st + BOFF * CPR + (wave + 4 * (q - LA)) * 64);
    };
    // fragment q (q < RB: A block q, else B block q - RB) of sub-step kk
    auto frag_one = [&](bf16x8 (&fa)[RB], bf16x8 (&fb)[TN], const u32x4 *st,
                        int kk, int q) __attribute__((always_inline)) {
        const int c = (kk * 4 + (lane >> 4)) ^ sw;
        if (q < RB)
            fa[q] = as_bf16x8(st[(wm * WR + q * 16 + l16) * CPR + c]);
        else
            fb[q - RB] = as_bf16x8(
                st[(BOFF + wn * WC + (q - RB) * 16 + l16) * CPR + c]);
    };

    floatx4 acc[RB][TN];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa0[RB], fb0[TN], fa1[RB], fb1[TN];

    // every wave is done with both slots (previous tile) and its stores
    // have left before the first loads of this one
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < NL; ++q) dma_one(0, slot0, q);
#pragma unroll
    for (int q = 0; q < NL; ++q) dma_one(min(1, KT - 1), slot1, q);
    wait_vm<NL>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < NF; ++q) frag_one(fa0, fb0, slot0, 0, q);

    // Stage s: sub-step 2s on fa0 while the second half of stage s is read
    // into fa1; then sub-step 2s+1 on fa1 while the first half of stage s+1
    // is read into fa0 and stage s+2 is loaded into the slot that stage s
    // leaves.  Loads past the end re-load the last stage, reads past the
    // end fill registers that are never used.
    auto stage = [&](int s, u32x4 *cur, u32x4 *nxt) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
#pragma unroll
        for (int q = 0; q < NM; ++q) {
            mfma16(acc[q / TN][q % TN], fb0[q % TN], fa0[q / TN]);
            if (q % RD == 0 && q / RD < NF) frag_one(fa1, fb1, cur, 1, q / RD);
        }
        // own reads done, own part of stage s+1 landed, then every wave's
        __builtin_amdgcn_s_waitcnt(0x0 | (0x7 << 4));
        __builtin_amdgcn_s_barrier();
        const int nx = min(s + 2, KT - 1);
#pragma unroll
        for (int q = 0; q < NM; ++q) {
            mfma16(acc[q / TN][q % TN], fb1[q % TN], fa1[q / TN]);
            if (q % RD == 0 && q / RD < NF) frag_one(fa0, fb0, nxt, 0, q / RD);
            if (q >= 1 && (q - 1) % DM == 0 && (q - 1) / DM < NL)
                dma_one(nx, cur, (q - 1) / DM);
        }
    };
    // The asm MFMAs get their wait states here: a few before the first
    // (a VALU write of its srcC), and after the last enough for a read of
    // its result (an 8-pass XDL op).
    for (int s = 0; s < KT; s += 2) {
        asm volatile("s_nop 4");
        stage(s, slot0, slot1);
        stage(s + 1, slot1, slot0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    }

    // Epilogue: bias, activation (up) and bf16, stored from the
    // accumulators.  Lane l holds rows 16 i + l % 16 and columns
    // 16 j + 4 (l / 16) .. + 3 of its wave's part.
    const int cq = 4 * (lane >> 4);
    const int cw = n0 + wn * WC + cq;        // column of block 0
    const uint16_t *bg = routed
        ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * N : nullptr)
        : (const uint16_t *)p.bias_s;
    float bv[TN][4];
    {
        u32x2 bb[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bb[j] = bg && cw + 16 * j < N ? *(const u32x2 *)(bg + cw + 16 * j)
                                          : u32x2{0u, 0u};
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            bv[j][0] = bf16_lo(bb[j].x);
            bv[j][1] = bf16_hi(bb[j].x);
            bv[j][2] = bf16_lo(bb[j].y);
            bv[j][3] = bf16_hi(bb[j].y);
        }
    }
    uint16_t *out = (uint16_t *)p.out;
    auto convert = [&](auto fn) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int r = wm * WR + i * 16 + l16;
            uint16_t *orow = out + (size_t)(row0 + r) * p.ldo;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                float v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = fn(acc[i][j][t] + bv[j][t]);
                if (r < nrows && cw + 16 * j < N) {
                    u32x2 o;
                    o.x = pack_bf16x2(v[0], v[1]);
                    o.y = pack_bf16x2(v[2], v[3]);
                    *(u32x2 *)(orow + cw + 16 * j) = o;
                }
            }
            // one row block at a time: the accumulators are read as they
            // are converted, not all at once
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (!UP)
        convert([](float z) __attribute__((always_inline)) { return z; });
    else if (p.act == ACT_SILU)
        convert([](float z) __attribute__((always_inline)) { return silu_f(z); });
    else
        convert([](float z) __attribute__((always_inline)) { return gelu_erf(z); });
}

// The tile of height h (one of the heights tall::height returns).
template <bool UP, int BN, bool NT>
__device__ __forceinline__ void run_tile(int h, const GemmParams &p,
                                         u32x4 *slot0, u32x4 *slot1, int g,
                                         int row0, int nrows, int n0,
                                         bool routed, int wave) {
    constexpr int TRMAX = BN == 192 ? 320 : 288;
    switch (h) {
    case 64: tall_tile<UP, 32, BN, NT>(p, slot0, slot1, g, row0, nrows, n0, routed, wave); break;
    case 128: tall_tile<UP, 64, BN, NT>(p, slot0, slot1, g, row0, nrows, n0, routed, wave); break;
    case 192: tall_tile<UP, 96, BN, NT>(p, slot0, slot1, g, row0, nrows, n0, routed, wave); break;
    case 256: tall_tile<UP, 128, BN, NT>(p, slot0, slot1, g, row0, nrows, n0, routed, wave); break;
    case 288: tall_tile<UP, 144, BN, NT>(p, slot0, slot1, g, row0, nrows, n0, routed, wave); break;
    default:
        if constexpr (TRMAX >= 320)
            tall_tile<UP, 160, BN, NT>(p, slot0, slot1, g, row0, nrows, n0, routed, wave);
        break;
    }
}

// A one-tile group of at most 256 rows on 256-column tiles (weights with
// the non-temporal hint).
template <bool UP>
__device__ __forceinline__ void run_wide_tile(int h, const GemmParams &p,
                                              u32x4 *slot0, u32x4 *slot1,
                                              int g, int row0, int nrows,
                                              int n0, bool routed, int wave) {
    switch (h) {
    case 64: tall_tile<UP, 32, 256, true>(p, slot0, slot1, g, row0, nrows, n0, routed, wave); break;
    case 128: tall_tile<UP, 64, 256, true>(p, slot0, slot1, g, row0, nrows, n0, routed, wave); break;
    case 192: tall_tile<UP, 96, 256, true>(p, slot0, slot1, g, row0, nrows, n0, routed, wave); break;
    default: tall_tile<UP, 128, 256, true>(p, slot0, slot1, g, row0, nrows, n0, routed, wave); break;
    }
}

// Persistent over the tiles: group-major, then column tile, then row tile,
// so that the row tiles of a weight panel are consecutive.  Logical tile L
// of round r goes to block (xcd, local) with L = r * grid + xcd * grid/8 +
// local: each XCD takes a contiguous run of tiles, and the tiles that
// share a group's gathered rows (its column tiles) run on one XCD and hit
// its L2.
template <bool UP, int BN>
__global__ __launch_bounds__(256, 1) void gemm_bf16_tall(GemmParams p) {
    using namespace tall;
    constexpr int TRMAX = BN == 192 ? 320 : 288;
    __shared__ u32x4 slot0[STAGE], slot1[STAGE];
    __shared__ TileTable tt;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // 320 x 192 form with N >= 2048: a group of at most 256 rows runs on
    // 256-column tiles (fewer, fuller tiles: DeepSeek-shaped up GEMM 2.26 ->
    // 2.20 ms, layer with the tall down GEMM 4.955 -> 4.926 ms).  Not for a
    // narrow N: on the Switch-shaped down GEMM (N = 768) three column tiles
    // a group instead of four left a quarter of the CUs idle (68 -> 83 us).
    const bool WIDE = BN == 192 && p.N >= 2048;
    const int NTN = (p.N + BN - 1) / BN;
    const int NTW = (p.N + 255) / 256;
    const int G = p.E + p.n_shared;
    // tt.mt: every tile of the group (row tiles x its column tiles)
    build_tile_table_by(tt, p.offsets, p.E, p.n_shared, p.shared_base, p.T,
                        1, [NTN, NTW, WIDE](int rows) {
                            const int m = (rows + TRMAX - 1) / TRMAX;
                            return m * (WIDE && rows <= 256 ? NTW : NTN);
                        });
    const int total = __builtin_amdgcn_readfirstlane(tt.base[G]);
    const int nb = gridDim.x, per = nb >> 3;
    const int xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
    for (int r = 0;; ++r) {
        const int L = r * nb + xcd * per + loc;
        if (L >= total) break;
        const int g = __builtin_amdgcn_readfirstlane(find_group(tt, G, L));
        const int local = L - __builtin_amdgcn_readfirstlane(tt.base[g]);
        const int grows = __builtin_amdgcn_readfirstlane(tt.rows[g]);
        const bool wide = WIDE && grows <= 256;
        const int mt = __builtin_amdgcn_readfirstlane(tt.mt[g]) / (wide ? NTW : NTN);
        const int n_tile = local / mt;
        const int m_tile = local - n_tile * mt;
        const int h = height<TRMAX>(grows, mt);
        const int row0 = __builtin_amdgcn_readfirstlane(tt.start[g]) + m_tile * h;
        const int nrows = min(h, grows - m_tile * h);
        if (nrows <= 0) continue;
        const bool routed = g < p.E;
        if (wide) {
            run_wide_tile<UP>(h, p, slot0, slot1, g, row0, nrows, n_tile * 256,
                              routed, wave);
            continue;
        }
        const int n0 = n_tile * BN;
        // one row tile: its panel is read by no other tile
        if (mt == 1)
            run_tile<UP, BN, true>(h, p, slot0, slot1, g, row0, nrows, n0, routed, wave);
        else
            run_tile<UP, BN, false>(h, p, slot0, slot1, g, row0, nrows, n0, routed, wave);
    }
}

}  // namespace

hipError_t launch_gemm_tall(const GemmParams &p, int bn, bool up, int grid,
                            hipStream_t s) {
    if (bn == 192) {
        if (up)
            hipLaunchKernelGGL((gemm_bf16_tall<true, 192>), dim3(grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_bf16_tall<false, 192>), dim3(grid), dim3(256), 0, s, p);
    } else {
        if (up)
            hipLaunchKernelGGL((gemm_bf16_tall<true, 224>), dim3(grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((gemm_bf16_tall<false, 224>), dim3(grid), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}
