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
// bf16 kernel: BM x BN x 64 tiles, A and B staged through LDS (double
// buffered, one barrier per k-step) with a 16-byte-chunk XOR swizzle that
// keeps ds_read_b128 conflict-free; v_mfma_f32_32x32x16_bf16 with the
// weight fragment as the MFMA A operand so each lane ends with 4
// consecutive output features of one row (8-byte packed stores).  The A
// operand of the up pass is gathered on load through slot_token[].
#include "kernels.h"

namespace {

constexpr int BK = 64;

// Global -> registers: this thread's 16-byte chunks of the A and B tiles
// at k offset ko (A rows with offset -1 are zero).
template <int AC, int BC>
__device__ __forceinline__ void tile_gload(u32x4 (&ra)[AC], u32x4 (&rb)[BC],
                                           const uint16_t *A,
                                           const uint16_t *Wg,
                                           const int (&aoff)[AC],
                                           const int (&boff)[BC], int ko) {
#pragma unroll
    for (int i = 0; i < AC; ++i) {
        // rows past the group's end read row 0 (always valid) and are zeroed
        u32x4 v = *(const u32x4 *)(A + max(aoff[i], 0) + ko);
        if (aoff[i] < 0) v = u32x4{0, 0, 0, 0};
        ra[i] = v;
    }
#pragma unroll
    for (int i = 0; i < BC; ++i) rb[i] = *(const u32x4 *)(Wg + boff[i] + ko);
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
        const uint16_t *Wg = routed
            ? (const uint16_t *)p.W + (size_t)g * N * K
            : (const uint16_t *)p.Ws;
        const uint16_t *bg = routed
            ? (p.bias ? (const uint16_t *)p.bias + (size_t)g * N : nullptr)
            : (const uint16_t *)p.bias_s;

        int aoff[AC];
#pragma unroll
        for (int i = 0; i < AC; ++i) {
            const int rr = lrow + i * RPP;
            aoff[i] = -1;
            if (rr < nrows) {
                const int slot = row0 + rr;
                int src = slot;
                if (UP) src = routed ? p.slot_token[slot] : slot - p.shared_base;
                aoff[i] = src * K + lc * 8;
            }
        }
        int boff[BC];
#pragma unroll
        for (int i = 0; i < BC; ++i) boff[i] = (n0 + lrow + i * RPP) * K + lc * 8;

        floatx16 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        u32x4 ra[AC], rb[BC];
        tile_gload<AC, BC>(ra, rb, A, Wg, aoff, boff, 0);
        tile_sstore<AC, BC, BM, RPP>(ra, rb, smem, lrow, lc);
        __syncthreads();
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < KT)
                tile_gload<AC, BC>(ra, rb, A, Wg, aoff, boff, (kt + 1) * BK);
            const u32x4 *sA = smem + cur * STAGE;
            const u32x4 *sB = sA + BM * 8;
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                const int c = kk * 2 + (lane >> 5);
                bf16x8 af[TM], bfr[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int ar = wm * (BM / WM) + i * 32 + (lane & 31);
                    af[i] = as_bf16x8(sA[ar * 8 + (c ^ ((ar >> 1) & 7))]);
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int br = wn * (BN / WN) + j * 32 + (lane & 31);
                    bfr[j] = as_bf16x8(sB[br * 8 + (c ^ ((br >> 1) & 7))]);
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            bfr[j], af[i], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < KT)
                tile_sstore<AC, BC, BM, RPP>(ra, rb, smem + (cur ^ 1) * STAGE,
                                             lrow, lc);
            __syncthreads();
        }

        // Epilogue.  Lane holds row m = lane%32 of each 32x32 tile and
        // features 8*q + 4*(lane/32) + 0..3 for q = 0..3.
        uint16_t *out = (uint16_t *)p.out;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = wm * (BM / WM) + i * 32 + (lane & 31);
            if (m >= nrows) continue;
            uint16_t *orow = out + (size_t)(row0 + m) * N;
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
                        v0 = gelu_erf(v0);
                        v1 = gelu_erf(v1);
                        v2 = gelu_erf(v2);
                        v3 = gelu_erf(v3);
                    }
                    u32x2 o;
                    o.x = pack_bf16x2(v0, v1);
                    o.y = pack_bf16x2(v2, v3);
                    *(u32x2 *)(orow + n) = o;
                }
            }
        }
    }
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
        const float *Wg = routed ? (const float *)p.W + (size_t)g * N * K
                                 : (const float *)p.Ws;
        const float *bg = routed
            ? (p.bias ? (const float *)p.bias + (size_t)g * N : nullptr)
            : (const float *)p.bias_s;
        const float *arow = nullptr;
        if (lr < nrows) {
            const int slot = row0 + lr;
            int src = slot;
            if (UP) src = routed ? p.slot_token[slot] : slot - p.shared_base;
            arow = A + (size_t)src * K;
        }
        const float *brow = Wg + (size_t)(n0 + lr) * K;
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
                const float4 b4 = *(const float4 *)&Bs[kk][tx * 4];
                const float a[4] = {a4.x, a4.y, a4.z, a4.w};
                const float b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
            __syncthreads();
        }
        float *out = (float *)p.out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = ty * 4 + i;
            if (m >= nrows) continue;
            float4 o;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + tx * 4 + j;
                float z = acc[i][j];
                if (bg) z += bg[n];
                v[j] = UP ? gelu_erf(z) : z;
            }
            o = make_float4(v[0], v[1], v[2], v[3]);
            *(float4 *)(out + (size_t)(row0 + m) * N + n0 + tx * 4) = o;
        }
    }
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
    default:
        if (up)
            hipLaunchKernelGGL(gemm_f32_simt<true>, dim3(grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL(gemm_f32_simt<false>, dim3(grid), dim3(256), 0, s, p);
        return hipGetLastError();
    }
}
