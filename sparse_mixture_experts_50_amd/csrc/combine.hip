// Routing-weighted combine:
//   y[t] = sum over kept j (in j order) of w[t,j] * Yp[slot_of[t,j]]
//          + Yp[shared_base + t]            (with a shared expert)
// fp32 accumulation, one rounding to the output dtype.  A dropped
// assignment (slot -1) adds nothing and the other weights stay as they are.
//
// "MoE architecture deep dive" (juejin.cn), sec. 1.1: Output is the sum of
// normalized_weight_i * Expert_i(x); sec. 3: plus the shared expert;
// sec. 2.3: an overflowing token skips the expert.  "AI-Research-SKILLs MoE
// training guide", sec. 3.1: weighted merge of the expert outputs.
//
// One block per token row; 16-byte vectors (8 bf16 or 4 fp32 lanes).  The
// output row is written exactly once (no atomics), so the result does not
// depend on scheduling.
#include "kernels.h"

namespace {

constexpr int MAX_K = MOE_MAX_E;     // expert choice: k = E <= 256

// 16 bytes of row `row_off` (elements) at vector index v: 8 bf16 or 4 fp32.
// Each expert-output row is read once, by one block, in whole 1 KB runs per
// wave.  NT: non-temporal loads, for expert outputs larger than the
// last-level cache (which otherwise still holds them from the down
// projection).
template <bool BF16, bool NT>
__device__ __forceinline__ u32x4 load_vec(const void *yp, size_t row_off,
                                          int v) {
    const u32x4 *q = BF16 ? (const u32x4 *)((const uint16_t *)yp + row_off) + v
                          : (const u32x4 *)((const float *)yp + row_off) + v;
    if (NT) return __builtin_nontemporal_load(q);
    return *q;
}

template <bool BF16>
__device__ __forceinline__ void fma_vec(float *acc, float w, u32x4 q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (BF16) {
            acc[2 * i] = fmaf(w, bf16_lo(q[i]), acc[2 * i]);
            acc[2 * i + 1] = fmaf(w, bf16_hi(q[i]), acc[2 * i + 1]);
        } else {
            acc[i] = fmaf(w, __uint_as_float(q[i]), acc[i]);
        }
    }
}

template <bool BF16>
__device__ __forceinline__ void add_vec(float *acc, u32x4 q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (BF16) {
            acc[2 * i] += bf16_lo(q[i]);
            acc[2 * i + 1] += bf16_hi(q[i]);
        } else {
            acc[i] += __uint_as_float(q[i]);
        }
    }
}

// One block per token.  Wave 0 first compacts the token's kept
// assignments (slot >= 0) into LDS in j order, so every thread then walks
// only the rows it adds, with no per-j global loads; the sum order is the
// j order either way.
template <bool BF16, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    constexpr int VW = BF16 ? 8 : 4;
    __shared__ int s_slot[MAX_K];
    __shared__ float s_w[MAX_K];
    __shared__ int s_n;
    const int t = blockIdx.x;
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        const unsigned long long lt = (1ull << lane) - 1ull;
        int n = 0;
        for (int j0 = 0; j0 < p.k; j0 += 64) {
            const int j = j0 + lane;
            const int s = j < p.k ? p.slot_of[(size_t)t * p.k + j] : -1;
            const float w = j < p.k ? p.topk_w[(size_t)t * p.k + j] : 0.0f;
            const unsigned long long m = __ballot(s >= 0);
            if (s >= 0) {
                const int pos = n + __popcll(m & lt);
                s_slot[pos] = s;
                s_w[pos] = w;
            }
            n += __popcll(m);
        }
        if (lane == 0) s_n = n;
    }
    __syncthreads();
    const int n = s_n;
    const int nv = p.d / VW;
    for (int v = threadIdx.x; v < nv; v += blockDim.x) {
        float acc[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[i] = 0.0f;
        // eight (then four) rows in flight, added in order
        int i = 0;
        for (; i + 8 <= n; i += 8) {
            u32x4 q[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                q[u] = load_vec<BF16, NT>(p.yp, (size_t)s_slot[i + u] * p.d, v);
#pragma unroll
            for (int u = 0; u < 8; ++u) fma_vec<BF16>(acc, s_w[i + u], q[u]);
        }
        for (; i + 4 <= n; i += 4) {
            u32x4 q[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                q[u] = load_vec<BF16, NT>(p.yp, (size_t)s_slot[i + u] * p.d, v);
#pragma unroll
            for (int u = 0; u < 4; ++u) fma_vec<BF16>(acc, s_w[i + u], q[u]);
        }
        for (; i < n; ++i)
            fma_vec<BF16>(acc, s_w[i],
                          load_vec<BF16, NT>(p.yp, (size_t)s_slot[i] * p.d, v));
        if (p.n_shared)
            add_vec<BF16>(acc, load_vec<BF16, NT>(
                p.yp, (size_t)(p.shared_base + t) * p.d, v));
        if (BF16) {
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
            *((u32x4 *)((uint16_t *)p.y + (size_t)t * p.d) + v) = o;
        } else {
            *((float4 *)((float *)p.y + (size_t)t * p.d) + v) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
}

}  // namespace

hipError_t launch_combine(const CombineParams &p, int dtype, hipStream_t s) {
    // one 16-byte vector per thread where the row allows it
    const int nv = p.d / (dtype == 1 ? 8 : 4);
    const int threads = nv >= 256 ? 256 : (nv + 63) / 64 * 64;
    // expert outputs beyond the 256 MB last-level cache: non-temporal
    const double rows = (double)p.T * p.k + (double)p.n_shared * p.T;
    const bool nt = rows * p.d * (dtype == 1 ? 2 : 4) > 256.0 * 1024 * 1024;
    if (dtype == 1) {
        if (nt)
            hipLaunchKernelGGL((combine_kernel<true, true>), dim3(p.T), dim3(threads), 0, s, p);
        else
            hipLaunchKernelGGL((combine_kernel<true, false>), dim3(p.T), dim3(threads), 0, s, p);
    } else {
        hipLaunchKernelGGL((combine_kernel<false, false>), dim3(p.T), dim3(threads), 0, s, p);
    }
    return hipGetLastError();
}
