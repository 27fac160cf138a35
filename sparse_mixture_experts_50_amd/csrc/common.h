// Device-side helpers shared by the HIP kernels of the MoE layer (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_MAX_E 256
#define MOE_MAX_GROUPS (MOE_MAX_E + 1)   // routed experts + one shared

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
// Native 16-byte vector (promotes to registers, unlike the struct uint4).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ bfloat16
__device__ __forceinline__ float bf16_lo(uint32_t w) {
    return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
    return __uint_as_float(w & 0xFFFF0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}
// float -> bfloat16, round to nearest even, by gfx950's v_cvt_pk_bf16_f32
// (one instruction per pair; bit-identical to the integer rounding
// u + 0x7FFF + ((u >> 16) & 1) on finite inputs, checked on the device over
// every low-half pattern, ties included).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(
        uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return pack_bf16x2(f, 0.0f) & 0xFFFFu;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

// GELU of the erf form, z * Phi(z) with Phi(z) = erfc(-z / sqrt 2) / 2.
// erfc by the Chebyshev-fitted form of Numerical Recipes (Press et al.,
// 2nd ed., sec. 6.2, "erfcc"): for x >= 0,
//   erfc(x) = t exp(-x^2 + P(t)),  t = 1 / (1 + x / 2),
// P a degree-9 polynomial, with fractional error below 1.2e-7 for every x.
// The error being relative, the deep negative tail (where Phi is tiny) is
// as accurate as the rest.  With x = |z| / sqrt 2 and q = erfc(x) / 2,
// Phi(z) = q for z < 0 and 1 - q otherwise, so z Phi(z) = max(z, 0) - |z| q
// for either sign, without a select.  The hardware exponential is base 2,
// so P's coefficients below are those of the book times log2(e), with
// log2(1/2) = -1 added to the constant term for the halving, and the 1/sqrt 2
// of x is folded into the reciprocal's and the square's factors: about 19
// vector instructions per value, two of them transcendental.  No branch: a
// tile epilogue evaluates hundreds of these per lane in straight-line code,
// so independent evaluations interleave and hide the latencies.
__device__ __forceinline__ float gelu_erf(float z) {
    const float az = fabsf(z);
    const float t = __builtin_amdgcn_rcpf(fmaf(az, 0.35355339f, 1.0f));
    float r = fmaf(0.24651730f, t, -1.18611491f);
    r = fmaf(r, t, 2.14747453f);
    r = fmaf(r, t, -1.63775313f);
    r = fmaf(r, t, 0.40232158f);
    r = fmaf(r, t, -0.26875687f);
    r = fmaf(r, t, 0.13963005f);
    r = fmaf(r, t, 0.53970063f);
    r = fmaf(r, t, 1.44272923f);
    r = fmaf(r, t, -2.82574821f);
    // log2 of erfc(x) / (2 t) = -x^2 log2(e) + (scaled P)(t), x^2 = z^2 / 2
    const float q = t * __builtin_amdgcn_exp2f(fmaf(z * -0.72134752f, z, r));
    return fmaf(-az, q, fmaxf(z, 0.0f));
}

// ------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// ---------------------------------------------------------- tile table
// Groups g = 0..E-1 are the routed experts (rows offsets[g]..offsets[g+1]),
// group E (when n_shared) is the shared expert with rows
// shared_base..shared_base+T.  Tiles of a group are enumerated n-tile major,
// m-tile minor, so consecutive tiles share one weight panel.
struct TileTable {
    int base[MOE_MAX_GROUPS + 1];   // first tile of each group
    int start[MOE_MAX_GROUPS];      // first slot row of each group
    int rows[MOE_MAX_GROUPS];
    int mt[MOE_MAX_GROUPS];         // m-tiles of each group
};

// Build the table in LDS with the whole block; ends with __syncthreads().
// mt_of(rows): the group's row tiles (ceil(rows / BM) for plain tiles).
template <typename F>
__device__ __forceinline__ void build_tile_table_by(
    TileTable &tt, const int32_t *__restrict__ offsets, int E, int n_shared,
    int shared_base, int T, int n_tiles_n, F mt_of) {
    const int G = E + n_shared;
    for (int g = threadIdx.x; g < G; g += blockDim.x) {
        int st, rw;
        if (g < E) {
            st = offsets[g];
            rw = offsets[g + 1] - st;
        } else {
            st = shared_base;
            rw = T;
        }
        const int mt = mt_of(rw);
        tt.start[g] = st;
        tt.rows[g] = rw;
        tt.mt[g] = mt;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int per = (G + 63) / 64;
        const int g0 = lane * per;
        int local = 0;
        for (int i = 0; i < per; ++i)
            if (g0 + i < G) local += tt.mt[g0 + i] * n_tiles_n;
        int incl = local;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        int run = incl - local;
        for (int i = 0; i < per; ++i) {
            if (g0 + i < G) {
                tt.base[g0 + i] = run;
                run += tt.mt[g0 + i] * n_tiles_n;
            }
        }
        if (lane == 63) tt.base[G] = incl;
    }
    __syncthreads();
}

__device__ __forceinline__ void build_tile_table(
    TileTable &tt, const int32_t *__restrict__ offsets, int E, int n_shared,
    int shared_base, int T, int BM, int n_tiles_n) {
    build_tile_table_by(tt, offsets, E, n_shared, shared_base, T, n_tiles_n,
                        [BM](int rows) { return (rows + BM - 1) / BM; });
}

// Largest g with base[g] <= L (base[G] > L assumed).
__device__ __forceinline__ int find_group(const TileTable &tt, int G, int L) {
    int lo = 0, hi = G;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (tt.base[mid] <= L) lo = mid; else hi = mid;
    }
    return lo;
}

// Arguments of one grouped GEMM pass (up: gathered x -> H with GELU;
// down: H -> Yp).  Weight panels are row-major [N][K] per group.
struct GemmParams {
    const void *A;            // up: x [T][K]; down: H [slots][K]
    const int32_t *slot_token;
    const int32_t *offsets;   // [E+1]
    const void *W;            // [E][N][K]
    const void *bias;         // [E][N] or null
    const void *Ws;           // shared [N][K] or null
    const void *bias_s;       // shared [N] or null
    void *out;                // [slots][N]
    const float *scale;       // FP8 weights: per-output-channel [E][N]
    const float *scale_s;     // FP8 shared expert [N]
    // SwiGLU up GEMM (gated != 0): W is the gate matrix W1 and W3 the up
    // matrix, both [E][N/2][K]; the N = 2*d_ff columns are a virtual panel
    // of 64-row chunks (32 rows of W1, then the same 32 rows of W3), and
    // the output holds N/2 features per row
    const void *W3, *bias3, *Ws3, *bias_s3;
    const float *scale3, *scale_s3;
    int E, n_shared, T, shared_base;
    int N, K;
    int act;                  // up epilogue: ACT_GELU, ACT_SILU, ACT_SWIGLU
    int gated;                // 1 for the SwiGLU up GEMM
    int ldo;                  // output row stride (elements)
    // Four-wave 256-row kernel, tail_split > 1: each half-height tile (a
    // group's last 1..128 rows) runs as tail_split units over consecutive
    // ranges of K, writing fp32 partial sums to part, laid out
    // [tail_split][E + n_shared][128][N] (rows of the group's tail); the
    // tail reduction adds them in order and finishes the rows.
    float *part;
    int tail_split;
};

enum { ACT_GELU = 0, ACT_SILU = 1, ACT_SWIGLU = 2 };

// SiLU(z) = z / (1 + e^-z) with the hardware exponential and reciprocal
// (relative error a few 1e-7).
__device__ __forceinline__ float silu_f(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Activation of an ungated up GEMM output.
__device__ __forceinline__ float act_up(int act, float z) {
    return act == ACT_SILU ? silu_f(z) : gelu_erf(z);
}

// Start of weight row v (elements of esz bytes) of group g's panel; for a
// gated up GEMM v indexes the interleaved W1 / W3 panel.
__device__ __forceinline__ const char *weight_row(const GemmParams &p,
                                                  bool routed, int g, int v,
                                                  int esz) {
    if (!p.gated) {
        const char *W = routed ? (const char *)p.W + (size_t)g * p.N * p.K * esz
                               : (const char *)p.Ws;
        return W + (size_t)v * p.K * esz;
    }
    const int F = p.N >> 1;
    const int c = v >> 6, r = v & 63;
    const size_t row = (size_t)(32 * c + (r & 31));
    const char *base = r < 32 ? (const char *)(routed ? p.W : p.Ws)
                              : (const char *)(routed ? p.W3 : p.Ws3);
    if (routed) base += (size_t)g * F * p.K * esz;
    return base + row * p.K * esz;
}
