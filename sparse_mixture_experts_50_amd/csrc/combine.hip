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

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    constexpr int VW = BF16 ? 8 : 4;
    const int t = blockIdx.x;
    const int nv = p.d / VW;
    int slots[8];
    float wts[8];
    const int kk = p.k;
    for (int v = threadIdx.x; v < nv; v += blockDim.x) {
        float acc[VW];
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[i] = 0.0f;
        for (int j0 = 0; j0 < kk; j0 += 8) {
            const int nj = min(8, kk - j0);
            for (int j = 0; j < nj; ++j) {
                slots[j] = p.slot_of[(size_t)t * kk + j0 + j];
                wts[j] = p.topk_w[(size_t)t * kk + j0 + j];
            }
            for (int j = 0; j < nj; ++j) {
                const int s = slots[j];
                if (s < 0) continue;
                const float w = wts[j];
                if (BF16) {
                    const uint4 q = *((const uint4 *)((const uint16_t *)p.yp +
                                                      (size_t)s * p.d) + v);
                    acc[0] = fmaf(w, bf16_lo(q.x), acc[0]);
                    acc[1] = fmaf(w, bf16_hi(q.x), acc[1]);
                    acc[2] = fmaf(w, bf16_lo(q.y), acc[2]);
                    acc[3] = fmaf(w, bf16_hi(q.y), acc[3]);
                    acc[4] = fmaf(w, bf16_lo(q.z), acc[4]);
                    acc[5] = fmaf(w, bf16_hi(q.z), acc[5]);
                    acc[6] = fmaf(w, bf16_lo(q.w), acc[6]);
                    acc[7] = fmaf(w, bf16_hi(q.w), acc[7]);
                } else {
                    const float4 q = *((const float4 *)((const float *)p.yp +
                                                        (size_t)s * p.d) + v);
                    acc[0] = fmaf(w, q.x, acc[0]);
                    acc[1] = fmaf(w, q.y, acc[1]);
                    acc[2] = fmaf(w, q.z, acc[2]);
                    acc[3] = fmaf(w, q.w, acc[3]);
                }
            }
        }
        if (p.n_shared) {
            const size_t srow = (size_t)(p.shared_base + t) * p.d;
            if (BF16) {
                const uint4 q = *((const uint4 *)((const uint16_t *)p.yp + srow) + v);
                acc[0] += bf16_lo(q.x);
                acc[1] += bf16_hi(q.x);
                acc[2] += bf16_lo(q.y);
                acc[3] += bf16_hi(q.y);
                acc[4] += bf16_lo(q.z);
                acc[5] += bf16_hi(q.z);
                acc[6] += bf16_lo(q.w);
                acc[7] += bf16_hi(q.w);
            } else {
                const float4 q = *((const float4 *)((const float *)p.yp + srow) + v);
                acc[0] += q.x;
                acc[1] += q.y;
                acc[2] += q.z;
                acc[3] += q.w;
            }
        }
        if (BF16) {
            uint4 o;
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            o.z = pack_bf16x2(acc[4], acc[5]);
            o.w = pack_bf16x2(acc[6], acc[7]);
            *((uint4 *)((uint16_t *)p.y + (size_t)t * p.d) + v) = o;
        } else {
            *((float4 *)((float *)p.y + (size_t)t * p.d) + v) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    }
}

}  // namespace

hipError_t launch_combine(const CombineParams &p, int dtype, hipStream_t s) {
    if (dtype == 1)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(p.T), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(p.T), dim3(256), 0, s, p);
    return hipGetLastError();
}
