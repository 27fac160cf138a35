// Router: logits = x . Wr^T (+ add) (- sub), softmax, top-k, renormalise.
//
// "MoE architecture deep dive" (juejin.cn), sec. 1.2: gate weights are
// Softmax(x . W_g); sec. 1.3: take the K largest and renormalise them to
// sum 1; sec. 2.4: routing uses logits - b_i.  "AI-Research-SKILLs MoE
// training guide", sec. 3.1: the router is an nn.Linear (additive bias).
//
// One block (16 waves) routes 32 tokens.  bf16 logits come from MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate); fp32 logits from plain FMA.
// The logits never leave the chip: each wave then takes 2 tokens and does
// max, exp-sum, selection and renormalisation across its 64 lanes.  The
// selection compares fp32 logits (softmax is monotonic), ties to the lower
// expert index.  Each block also writes its column sums of the softmax
// probabilities, reduced later in a fixed order for p_i.
//
// Expert choice ("AI-Research-SKILLs MoE training guide", sec. 4.2): no
// top-k; every token writes the probabilities of all E experts and resets
// its slot row to -1, and the block writes its logits transposed to [E][T]
// (32 consecutive tokens per expert row), the layout in which each expert
// later ranks its column.
#include "kernels.h"

namespace {

constexpr int RT = MOE_ROUTER_TOKENS;
constexpr int RW = 16;            // waves per router block

// Softmax + top-k phase over logits staged in LDS (KS partial planes).
template <int EP, int KS>
__device__ __forceinline__ void route_tokens(const float (*lg)[RT][EP],
                                             const RouterParams &p,
                                             float (*pp)[EP]) {
    static_assert(RT % RW == 0, "tokens per wave");
    constexpr int PER = EP >= 64 ? EP / 64 : 1;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * RT;
    float psum[PER];
    float addv[PER], subv[PER];
    bool valid[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        valid[i] = e < p.E && e < EP;
        psum[i] = 0.0f;
        addv[i] = (valid[i] && p.add) ? p.add[e] : 0.0f;
        subv[i] = (valid[i] && p.sub) ? p.sub[e] : 0.0f;
    }
    float zsum = 0.0f, hsum = 0.0f;
    for (int q = 0; q < RT / RW; ++q) {
        const int tl = wave * (RT / RW) + q;
        const int t = t0 + tl;
        if (t >= p.T) break;
        float v[PER];
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + 64 * i;
            float s = 0.0f;
            if (valid[i]) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) s += lg[ks][tl][e];
                s = s + addv[i];
                s = s - subv[i];
            }
            v[i] = valid[i] ? s : -INFINITY;
            m = fmaxf(m, v[i]);
        }
        m = wave_max(m);
        float ex[PER];
        float ls = 0.0f;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            ex[i] = valid[i] ? expf(v[i] - m) : 0.0f;
            ls += ex[i];
        }
        const float S = wave_sum(ls);
        float pl = 0.0f;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            psum[i] += ex[i] / S;
            if (valid[i]) pl += ex[i] * (v[i] - m);
        }
        // monitors: logsumexp = m + ln S; entropy (nats) = ln S - sum p (l - m)
        const float lnS = logf(S);
        const float lse = m + lnS;
        zsum += lse * lse;
        hsum += lnS - wave_sum(pl) / S;

        if (p.scores) {          // expert choice: all experts, weight p
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int e = lane + 64 * i;
                if (valid[i]) {
                    p.topk_idx[(size_t)t * p.E + e] = e;
                    p.topk_w[(size_t)t * p.E + e] = ex[i] / S;
                    p.slot_of[(size_t)t * p.E + e] = -1;  // picks come later
                }
            }
            continue;
        }

        // top-k: k rounds of a wave-wide (max logit, min index) search
        bool taken[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) taken[i] = false;
        int my_e = 0;
        float my_ex = 0.0f;
        for (int j = 0; j < p.k; ++j) {
            float bv = -INFINITY;
            int be = 0x7FFFFFFF;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int e = lane + 64 * i;
                if (valid[i] && !taken[i] &&
                    (v[i] > bv || (v[i] == bv && e < be))) {
                    bv = v[i];
                    be = e;
                }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oe = __shfl_xor(be, o, 64);
                if (ov > bv || (ov == bv && oe < be)) {
                    bv = ov;
                    be = oe;
                }
            }
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (be == lane + 64 * i) taken[i] = true;
            if (lane == j) {
                my_e = be;
                my_ex = expf(bv - m);
            }
        }
        const float wsum = wave_sum(lane < p.k ? my_ex : 0.0f);
        if (lane < p.k) {
            p.topk_idx[(size_t)t * p.k + lane] = my_e;
            p.topk_w[(size_t)t * p.k + lane] = my_ex / wsum;
        }
    }
    // block column sums of the probabilities, fixed order over waves
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        if (e < EP) pp[wave][e] = psum[i];
    }
    __shared__ float zh[RW][2];
    if (lane == 0) {
        zh[wave][0] = zsum;
        zh[wave][1] = hsum;
    }
    __syncthreads();
    if (threadIdx.x < 2) {
        float s = zh[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < RW; ++w) s += zh[w][threadIdx.x];
        p.zh_part[(size_t)blockIdx.x * 2 + threadIdx.x] = s;
    }
    for (int e = threadIdx.x; e < p.E; e += blockDim.x) {
        float s = pp[0][e];
#pragma unroll
        for (int w = 1; w < RW; ++w) s += pp[w][e];
        p.p_part[(size_t)blockIdx.x * p.E + e] = s;
    }
    if (p.scores) {
        // the same additions in the same order as v[] above, so the
        // scores equal the logits the softmax saw bit for bit
        for (int i = threadIdx.x; i < p.E * RT; i += blockDim.x) {
            const int e = i / RT, tl = i % RT, t = t0 + tl;
            if (t >= p.T) continue;
            float s = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) s += lg[ks][tl][e];
            s = s + (p.add ? p.add[e] : 0.0f);
            s = s - (p.sub ? p.sub[e] : 0.0f);
            p.scores[(size_t)e * p.T + t] = s;
        }
    }
}

// bf16 logits with MFMA.  EP = E rounded up to 32/64/128/256.  The 16
// waves split the 32-expert tiles and, beyond that, the depth d, so even a
// single block (a 32-token decode step) keeps 16 waves of loads in flight.
template <int EP>
__global__ __launch_bounds__(RW * 64) void router_bf16(RouterParams p) {
    constexpr int NTE = EP / 32;                  // 32-expert tiles
    constexpr int KS = NTE >= RW ? 1 : RW / NTE;  // k-splits across waves
    constexpr int TPW = NTE >= RW ? NTE / RW : 1; // tiles per wave
    __shared__ float lg[KS][RT][EP];
    __shared__ float pp[RW][EP];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * RT;
    const int ks = NTE >= RW ? 0 : wave / NTE;
    const int tok = min(t0 + (lane & 31), p.T - 1);
    const int kg = (lane >> 5) * 8;
    const uint16_t *xrow = (const uint16_t *)p.x + (size_t)tok * p.d + kg;
    const uint16_t *wrow[TPW];
    int tile[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        tile[i] = NTE >= RW ? wave + RW * i : wave % NTE;
        const int e = min(tile[i] * 32 + (lane & 31), p.E - 1);
        wrow[i] = (const uint16_t *)p.wr + (size_t)e * p.d + kg;
    }
    floatx16 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

    // Rows past T and experts past E read a clamped valid row: their
    // logits land in lanes that the selection never looks at, so the loads
    // need no predicate (predicated loads serialise the k-loop).
#pragma unroll 8
    for (int k0 = ks * 16; k0 < p.d; k0 += 16 * KS) {
        const u32x4 av = *(const u32x4 *)(xrow + k0);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const u32x4 bv = *(const u32x4 *)(wrow[i] + k0);
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(av), as_bf16x8(bv), acc[i], 0, 0, 0);
        }
    }
    // D[token][expert]: lane holds expert column lane%32 and token rows
    // 8*(v/4) + 4*(lane/32) + v%4.
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int e = tile[i] * 32 + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int tl = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            lg[ks][tl][e] = acc[i][v];
        }
    }
    __syncthreads();
    route_tokens<EP, KS>(lg, p, pp);
}

// fp32 logits with plain FMA (sequential over d).
template <int EP>
__global__ __launch_bounds__(RW * 64) void router_f32(RouterParams p) {
    __shared__ float lg[1][RT][EP];
    __shared__ float pp[RW][EP];
    const int t0 = blockIdx.x * RT;
    const float *x = (const float *)p.x;
    const float *wr = (const float *)p.wr;
    for (int pair = threadIdx.x; pair < RT * EP; pair += blockDim.x) {
        const int tl = pair / EP;
        const int e = pair % EP;
        const int t = t0 + tl;
        float s = 0.0f;
        if (t < p.T && e < p.E) {
            const float4 *xr = (const float4 *)(x + (size_t)t * p.d);
            const float4 *wv = (const float4 *)(wr + (size_t)e * p.d);
            for (int c = 0; c < p.d / 4; ++c) {
                const float4 a = xr[c];
                const float4 b = wv[c];
                s = fmaf(a.x, b.x, s);
                s = fmaf(a.y, b.y, s);
                s = fmaf(a.z, b.z, s);
                s = fmaf(a.w, b.w, s);
            }
        }
        lg[0][tl][e] = s;
    }
    __syncthreads();
    route_tokens<EP, 1>(lg, p, pp);
}

}  // namespace

hipError_t launch_router(const RouterParams &p, int dtype, hipStream_t s) {
    const int blocks = (p.T + RT - 1) / RT;
    const dim3 grid(blocks), block(RW * 64);
    const int EP = p.E <= 32 ? 32 : p.E <= 64 ? 64 : p.E <= 128 ? 128 : 256;
    if (dtype == 1) {
        switch (EP) {
        case 32: hipLaunchKernelGGL(router_bf16<32>, grid, block, 0, s, p); break;
        case 64: hipLaunchKernelGGL(router_bf16<64>, grid, block, 0, s, p); break;
        case 128: hipLaunchKernelGGL(router_bf16<128>, grid, block, 0, s, p); break;
        default: hipLaunchKernelGGL(router_bf16<256>, grid, block, 0, s, p); break;
        }
    } else {
        switch (EP) {
        case 32: hipLaunchKernelGGL(router_f32<32>, grid, block, 0, s, p); break;
        case 64: hipLaunchKernelGGL(router_f32<64>, grid, block, 0, s, p); break;
        case 128: hipLaunchKernelGGL(router_f32<128>, grid, block, 0, s, p); break;
        default: hipLaunchKernelGGL(router_f32<256>, grid, block, 0, s, p); break;
        }
    }
    return hipGetLastError();
}
