// Router: logits = x . Wr^T (+ add) (- sub), softmax, top-k, renormalise.
//
// "MoE architecture deep dive" (juejin.cn), sec. 1.2: gate weights are
// Softmax(x . W_g); sec. 1.3: take the K largest and renormalise them to
// sum 1; sec. 2.4: routing uses logits - b_i.  "AI-Research-SKILLs MoE
// training guide", sec. 3.1: the router is an nn.Linear (additive bias).
//
// bf16: two kernels.  The logits kernel spreads the logits GEMM over many
// blocks: each block takes 32 (E <= 64, router_logits) or 128 (E > 64,
// router_logits_lds, router rows staged in LDS) tokens, all experts and one
// of S consecutive depth ranges, with MFMA 32x32x16 (fp32 accumulation),
// and writes fp32 partial sums; a single block per 32 tokens would pull
// every token row through one CU.  router_route sums the S
// partials in order (deterministic), then routes 32 tokens per block: for
// E <= 32 one lane per token walks its E logits in registers (no cross-lane
// traffic); for larger E each wave takes 2 tokens across its 64 lanes.
// fp32: one kernel with FMA logits.  The selection compares fp32 logits
// (softmax is monotonic), ties to the lower expert index.  Each 32-token
// block also writes its column sums of the softmax probabilities, reduced
// later in a fixed order for p_i, and its logsumexp / entropy sums.
//
// Expert choice ("AI-Research-SKILLs MoE training guide", sec. 4.2): no
// top-k; every token writes the probabilities of all E experts and resets
// its slot row to -1, and the block writes its logits transposed to [E][T]
// (32 consecutive tokens per expert row), the layout in which each expert
// later ranks its column.
#include "kernels.h"
#include "permute_block.h"

namespace {

constexpr int RT = MOE_ROUTER_TOKENS;
constexpr int RW = 16;            // waves per router block

// LG_PAD: the logit planes staged in LDS have rows of EP + 1 floats.  The
// expert-choice score pass reads them token-minor (a column of 32 tokens at
// one expert per 32 lanes), which with EP-float rows put every lane of a
// column on one bank; the MFMA result writes (two token rows 4 apart per
// instruction) and the one-lane-per-token reads of the small-E path share
// banks the same way.
// Softmax + top-k phase over logits staged in LDS (KS partial planes).
// hist: LDS counts of each expert's picks among the block's tokens, zeroed
// by the caller before its last barrier; written out as the block's row of
// p.blk (top-k only).
template <int EP, int KS>
__device__ __forceinline__ void route_tokens(const float (*lg)[RT][EP + 1],
                                             const RouterParams &p,
                                             float (*pp)[EP], int *hist) {
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
            // an id outside [0, E) (only from non-finite logits) is never
            // counted and never dispatched
            if ((unsigned)my_e < (unsigned)p.E) atomicAdd(&hist[my_e], 1);
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
        if (!p.scores) p.blk[(size_t)blockIdx.x * p.E + e] = hist[e];
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

// The MFMA k-loop of the router kernels: n steps at k = kbeg + i * kstep,
// each one 32x32x16 MFMA per expert tile (A: 8 x values of the lane's
// token row, B: 8 weights of the lane's expert row).  The loads of U steps
// are issued before their MFMAs (a loop of load, wait, MFMA per step waits
// out one memory latency each).  A step past n loads the last step again
// and runs its MFMA with a zero A operand, which adds exactly zero (the
// weights are finite): no branch, so the loads stay ahead of the MFMAs,
// and the sums are those of the plain loop, in the same order.
template <int TPW, int U>
__device__ __forceinline__ void router_kloop(const uint16_t *xrow,
                                             const uint16_t *const (&wrow)[TPW],
                                             int kbeg, int kstep, int n,
                                             floatx16 (&acc)[TPW]) {
    const int klast = kbeg + (n - 1) * kstep;
    for (int i0 = 0; i0 < n; i0 += U) {
        u32x4 av[U], bv[U][TPW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = min(kbeg + (i0 + u) * kstep, klast);
            av[u] = *(const u32x4 *)(xrow + k);
#pragma unroll
            for (int i = 0; i < TPW; ++i) bv[u][i] = *(const u32x4 *)(wrow[i] + k);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + u >= n) av[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < TPW; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    as_bf16x8(av[u]), as_bf16x8(bv[u][i]), acc[i], 0, 0, 0);
        }
    }
}

// Partial logits over one depth range.  EP = E rounded up to 32..256.
// E <= 64: a block is one 32-token tile; its 4 waves split the expert tiles
// and then the depth range (KW interleaved 16-deep steps each), reduced
// through LDS in wave order.  E > 64: a block is four 32-token tiles, one
// per wave, each wave covering every expert tile over the whole range.
// Rows past T and experts past E read a clamped valid row: their sums land
// in entries that are never written out, so the loads need no predicate.
template <int EP>
__global__ __launch_bounds__(256) void router_logits(RouterParams p) {
    constexpr int ET = EP / 32;                 // 32-expert tiles
    constexpr bool SMALL = EP <= 64;
    constexpr int KW = SMALL ? 4 / ET : 1;      // depth splits in a block
    constexpr int TPW = SMALL ? 1 : ET;         // tiles per wave
    __shared__ float red[SMALL ? KW : 1][32][SMALL ? EP : 1];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int s = blockIdx.y;
    const int k_lo = s * p.kc, k_hi = min(p.d, k_lo + p.kc);
    const int tt = SMALL ? blockIdx.x : blockIdx.x * 4 + wave;   // token tile
    const int t0 = tt * 32;
    const int kw = SMALL ? wave / ET : 0;
    const int tok = min(t0 + (lane & 31), p.T - 1);
    const int kg = (lane >> 5) * 8;
    const uint16_t *xrow = (const uint16_t *)p.x + (size_t)tok * p.d + kg;
    const uint16_t *wrow[TPW];
    int etile[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        etile[i] = SMALL ? wave % ET : i;
        const int e = min(etile[i] * 32 + (lane & 31), p.E - 1);
        wrow[i] = (const uint16_t *)p.wr + (size_t)e * p.d + kg;
    }
    floatx16 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    {
        const int kb = k_lo + kw * 16;
        const int n = kb < k_hi ? (k_hi - kb + 16 * KW - 1) / (16 * KW) : 0;
        router_kloop<TPW, TPW <= 2 ? 8 : 2>(xrow, wrow, kb, 16 * KW, n, acc);
    }
    // D[token][expert]: lane holds expert column lane%32 and token rows
    // 8*(v/4) + 4*(lane/32) + v%4.
    float *part = p.part + (size_t)s * p.T * p.E;
    if (SMALL) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int tl = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            red[kw][tl][etile[0] * 32 + (lane & 31)] = acc[0][v];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < 32 * p.E; i += 256) {
            const int tl = i / p.E, e = i - tl * p.E;
            if (t0 + tl >= p.T) continue;
            float sum = red[0][tl][e];
#pragma unroll
            for (int w = 1; w < KW; ++w) sum += red[w][tl][e];
            part[(size_t)(t0 + tl) * p.E + e] = sum;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int e = etile[i] * 32 + (lane & 31);
        if (e >= p.E) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = t0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (t < p.T) part[(size_t)t * p.E + e] = acc[i][v];
        }
    }
}

// Partial logits over one depth range for E > 64 (EP = 128 or 256).  A
// block takes 128 MT tokens, 32 MT per wave (MT 32-token MFMA tiles), and
// every expert: each wave holds MT x EP / 32 accumulator tiles of 32x32.
// The router rows of each 64-deep step are staged in LDS once per block
// (two buffers, loaded into registers one step ahead, one barrier per
// step) and every wave reads its B fragments there (with MT = 2 each feeds
// two MFMAs).  Against one 32-token tile per wave reading the router rows
// straight from L2, the router matrix is pulled from L2 a quarter (MT = 2)
// or half (MT = 1) as often per token.  MT = 1 is launched: its 128
// accumulators let two blocks share a CU and hide each other's load waits
// (DeepSeek-shaped logits 62.5 -> 55.4 us against MT = 2's one block of
// 256 accumulators per wave).  Staged rows are 128 bytes of eight 16-byte
// chunks, chunk c of row r at c ^ ((r / 2) % 8), so that 32 lanes reading
// 32 rows at one chunk hit distinct bank groups.
template <int EP, int MT>
__global__ __launch_bounds__(256, MT == 1 ? 2 : 1) void router_logits_lds(RouterParams p) {
    constexpr int ET = EP / 32;                 // 32-expert tiles
    constexpr int CH = EP * 8;                  // 16-byte chunks per step
    constexpr int PT = CH / 256;                // chunks per thread per step
    __shared__ u32x4 wst0[CH], wst1[CH];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.y;
    const int k_lo = s * p.kc, k_hi = min(p.d, k_lo + p.kc);
    const int t0 = blockIdx.x * (128 * MT) + wave * (32 * MT);
    const int kg = (lane >> 5) * 8;
    const uint16_t *xr[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int tok = min(t0 + 32 * m + (lane & 31), p.T - 1);
        xr[m] = (const uint16_t *)p.x + (size_t)tok * p.d + kg;
    }
    const uint16_t *wsrc[PT];
    int wdst[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int idx = tid + 256 * i, r = idx >> 3, c = idx & 7;
        const int e = min(r, p.E - 1);
        wsrc[i] = (const uint16_t *)p.wr + (size_t)e * p.d + 8 * c;
        wdst[i] = r * 8 + (c ^ ((r >> 1) & 7));
    }
    floatx16 acc[MT][ET];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int et = 0; et < ET; ++et)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[m][et][v] = 0.0f;

    u32x4 wreg[PT], areg[MT][4];
    auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PT; ++i) wreg[i] = *(const u32x4 *)(wsrc[i] + k0);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                areg[m][j] = *(const u32x4 *)(xr[m] + k0 + 16 * j);
    };
    load(k_lo);
    int buf = 0;
    for (int k0 = k_lo; k0 < k_hi; k0 += 64) {
        u32x4 *st = buf ? wst1 : wst0;
#pragma unroll
        for (int i = 0; i < PT; ++i) st[wdst[i]] = wreg[i];
        u32x4 a[2][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) a[m][j] = areg[m][j];
        __syncthreads();
        if (k0 + 64 < k_hi) load(k0 + 64);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 2 * j + (lane >> 5);
#pragma unroll
            for (int et = 0; et < ET; ++et) {
                const int r = 32 * et + (lane & 31);
                const u32x4 bv = st[r * 8 + (c ^ ((r >> 1) & 7))];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    acc[m][et] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(a[m][j]), as_bf16x8(bv), acc[m][et], 0, 0, 0);
            }
        }
        buf ^= 1;
    }
    // D[token][expert]: lane holds expert column lane%32 and token rows
    // 8*(v/4) + 4*(lane/32) + v%4 of its tile
    float *part = p.part + (size_t)s * p.T * p.E;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int et = 0; et < ET; ++et) {
            const int e = 32 * et + (lane & 31);
            if (e >= p.E) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int t = t0 + 32 * m + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (t < p.T) part[(size_t)t * p.E + e] = acc[m][et][v];
            }
        }
}

// One lane per token (E <= EP = 32): softmax, statistics and selection on
// the token's logits held in registers, written as selects rather than
// branches (padding experts hold -inf and never win a pick, k <= E); the
// probabilities go to pr (LDS), from which the picked weights are
// renormalised (the softmax denominator cancels).  lg: the block's summed
// logits; addv / subv: the router and balancing biases (0 where absent).
template <int EP>
__device__ __forceinline__ void route_lanes(const float (*lg)[EP + 1],
                                            const RouterParams &p,
                                            const float *addv,
                                            const float *subv,
                                            float (*pr)[EP + 1],
                                            float (*zh)[2], int *hist) {
    const int tl = threadIdx.x;          // 0..31
    const int t = blockIdx.x * RT + tl;
    float z = 0.0f, h = 0.0f;
    if (t < p.T) {
        float v[EP], ex[EP];
        float m = -INFINITY;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
            float s = lg[tl][e];
            s = s + addv[e];
            s = s - subv[e];
            v[e] = e < p.E ? s : -INFINITY;
            m = fmaxf(m, v[e]);
        }
        float S = 0.0f, pl = 0.0f;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
            const bool real = e < p.E;
            ex[e] = real ? expf(v[e] - m) : 0.0f;
            S += ex[e];
            pl += real ? ex[e] * (v[e] - m) : 0.0f;
        }
        const float inv = 1.0f / S;
#pragma unroll
        for (int e = 0; e < EP; ++e) pr[tl][e] = ex[e] * inv;
        // monitors: logsumexp = m + ln S; entropy (nats) = ln S - sum p (l - m)
        const float lnS = logf(S);
        const float lse = m + lnS;
        z = lse * lse;
        h = lnS - pl / S;
        if (p.scores) {          // expert choice: all experts, weight p
            for (int e = 0; e < p.E; ++e) {
                p.topk_idx[(size_t)t * p.E + e] = e;
                p.topk_w[(size_t)t * p.E + e] = pr[tl][e];
                p.slot_of[(size_t)t * p.E + e] = -1;  // picks come later
                p.scores[(size_t)e * p.T + t] = lg[tl][e] + addv[e] - subv[e];
            }
        } else {
            // k rounds of (max logit, lowest index) over the untaken
            // experts; the rounds run twice (the sum of the picked
            // probabilities is needed before the first weight is written)
            // rather than reading the picks back from memory
            auto pick = [&](uint32_t taken) __attribute__((always_inline)) {
                float bv = -INFINITY;
                int be = -1;
#pragma unroll
                for (int e = 0; e < EP; ++e) {
                    const bool better = !((taken >> e) & 1u) &&
                                        (be < 0 || v[e] > bv);
                    bv = better ? v[e] : bv;
                    be = better ? e : be;
                }
                return be;
            };
            uint32_t taken = 0;
            float wsum = 0.0f;
            for (int j = 0; j < p.k; ++j) {
                const int be = pick(taken);
                taken |= 1u << be;
                wsum += pr[tl][be];
            }
            const float winv = 1.0f / wsum;
            taken = 0;
            for (int j = 0; j < p.k; ++j) {
                const int be = pick(taken);
                taken |= 1u << be;
                p.topk_idx[(size_t)t * p.k + j] = be;
                p.topk_w[(size_t)t * p.k + j] = pr[tl][be] * winv;
                if (be < p.E) atomicAdd(&hist[be], 1);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < EP; ++e) pr[tl][e] = 0.0f;
    }
    zh[tl][0] = z;
    zh[tl][1] = h;
}

// Sum the S partial logit planes of this block's 32 tokens in order into
// lg (tokens past T take the last token's sums; they are never routed).
template <int EP>
__device__ __forceinline__ void sum_partials(const RouterParams &p,
                                             float (*lg)[EP + 1]) {
    const int t0 = blockIdx.x * RT;
    const size_t plane = (size_t)p.T * p.E;
    for (int i = threadIdx.x; i < RT * p.E; i += blockDim.x) {
        const int tl = i / p.E, e = i - tl * p.E;
        const int t = min(t0 + tl, p.T - 1);
        const float *src = p.part + (size_t)t * p.E + e;
        // every load issued before the in-order sum
        float a[MOE_ROUTER_MAX_SPLITS];
#pragma unroll
        for (int k = 0; k < MOE_ROUTER_MAX_SPLITS; ++k)
            a[k] = k < p.S ? src[k * plane] : 0.0f;
        float s = a[0];
#pragma unroll
        for (int k = 1; k < MOE_ROUTER_MAX_SPLITS; ++k)
            if (k < p.S) s += a[k];
        lg[tl][e] = s;
    }
}

// Route 32 tokens from their split partial logits, one lane per token
// (E <= 32: a handful of logits per lane beats a chain of 64-lane
// reductions), in a 256-thread block; then the block's probability column
// sums and lse^2 / entropy sums in token order.
template <int EP>
__device__ __forceinline__ void route_tile_lanes(const RouterParams &p) {
    static_assert(EP <= 32, "one lane per token");
    __shared__ float lg[RT][EP + 1];      // rows of EP + 1 floats (LG_PAD)
    __shared__ float pr[RT][EP + 1];
    __shared__ float zh[RT][2];
    __shared__ float addv[EP], subv[EP];
    __shared__ int hist[EP];
    if (threadIdx.x < EP) {
        const int e = threadIdx.x;
        addv[e] = (e < p.E && p.add) ? p.add[e] : 0.0f;
        subv[e] = (e < p.E && p.sub) ? p.sub[e] : 0.0f;
        hist[e] = 0;
    }
    sum_partials<EP>(p, lg);
    __syncthreads();
    if (threadIdx.x < RT) route_lanes<EP>(lg, p, addv, subv, pr, zh, hist);
    __syncthreads();
    // block sums in token order: probability columns, then lse^2, entropy
    for (int e = threadIdx.x; e < p.E; e += blockDim.x) {
        float s = pr[0][e];
        for (int tl = 1; tl < RT; ++tl) s += pr[tl][e];
        p.p_part[(size_t)blockIdx.x * p.E + e] = s;
        if (!p.scores) p.blk[(size_t)blockIdx.x * p.E + e] = hist[e];
    }
    if (threadIdx.x >= 64 && threadIdx.x < 66) {
        const int c = threadIdx.x - 64;
        float s = zh[0][c];
        for (int tl = 1; tl < RT; ++tl) s += zh[tl][c];
        p.zh_part[(size_t)blockIdx.x * 2 + c] = s;
    }
}

// Sum the S partial logit planes of 32 tokens in order, then route them:
// one lane per token in a 256-thread block (E <= 32), or 2 tokens per wave
// in a 1024-thread block.
template <int EP>
__global__ __launch_bounds__(EP <= 32 ? 256 : RW * 64) void router_route(RouterParams p) {
    if constexpr (EP <= 32) {
        route_tile_lanes<EP>(p);
    } else {
        __shared__ float lg[1][RT][EP + 1];   // rows of EP + 1 floats (LG_PAD)
        __shared__ float pp[RW][EP];
        __shared__ int hist[EP];
        for (int e = threadIdx.x; e < EP; e += blockDim.x) hist[e] = 0;
        sum_partials<EP>(p, lg[0]);
        __syncthreads();
        route_tokens<EP, 1>(lg, p, pp, hist);
    }
}

// A decode-sized step's routing and dispatch in one launch (bf16 split
// router, E <= 32, one 32-token tile, T*k <= 256): router_route's work for
// the tile, then the single-block permute on the picks it wrote, so the
// results equal router_route + permute_small bit for bit.  The logits stay
// spread over the partial-logit kernel's blocks (one block pulling every
// token and router row through its CU took 22 us against 5).
template <int EP>
__global__ __launch_bounds__(256) void route_permute_small(RouterParams p,
                                                           PermuteParams q) {
    route_tile_lanes<EP>(p);
    // the picks and sums this block wrote to global memory are visible to
    // the whole block after the barrier
    __syncthreads();
    permute_one_block<256>(q);
}

// bf16, fused: one block (16 waves) computes and routes 32 tokens.  The
// waves split the 32-expert tiles and, beyond that, the depth d; the logits
// stay in LDS.  Used when there are enough such blocks to fill the GPU and
// each pulls little through its CU (short d, few experts).
template <int EP>
__global__ __launch_bounds__(RW * 64) void router_fused(RouterParams p) {
    constexpr int NTE = EP / 32;                  // 32-expert tiles
    constexpr int KS = NTE >= RW ? 1 : RW / NTE;  // k-splits across waves
    constexpr int TPW = NTE >= RW ? NTE / RW : 1; // tiles per wave
    __shared__ float lg[KS][RT][EP + 1];  // rows of EP + 1 floats (LG_PAD)
    __shared__ float pp[RW][EP];
    __shared__ int hist[EP];
    for (int e = threadIdx.x; e < EP; e += blockDim.x) hist[e] = 0;

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
    // (one load-wait-MFMA chain per step: the block's 32 waves per CU hide
    // the latency; the batched loop of router_logits measured 15-25 %
    // slower here)
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
    route_tokens<EP, KS>(lg, p, pp, hist);
}

// fp32 logits with plain FMA (sequential over d).
template <int EP>
__global__ __launch_bounds__(RW * 64) void router_f32(RouterParams p) {
    __shared__ float lg[1][RT][EP + 1];   // rows of EP + 1 floats (LG_PAD)
    __shared__ float pp[RW][EP];
    __shared__ int hist[EP];
    for (int e = threadIdx.x; e < EP; e += blockDim.x) hist[e] = 0;
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
    route_tokens<EP, 1>(lg, p, pp, hist);
}

}  // namespace

RouterPlan router_plan(int T, int d, int E, int cus) {
    RouterPlan r;
    r.ep = E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256;
    // fused when its 32-token blocks fill at least half the GPU and each
    // reads at most ~400 KB (32 token rows and every router row): the
    // Mixtral-shaped prefill (128 blocks of 328 KB) runs as fast fused as
    // split (23 against 14 + 10 us) and saves a launch; a decode step (one
    // block) or E = 256 at d = 7168 (4 MB per block) is split
    const long long fblocks = ((long long)T + RT - 1) / RT;
    const double fbytes = 2.0 * d * (RT + E);
    r.split = !(2 * fblocks >= cus && fbytes <= 400e3);
    const bool small = r.ep <= 64;
    r.tokens = small ? 32 : 128;
    const int kw = small ? 4 / (r.ep / 32) : 1;
    const long long blocks = T > 0 ? (T + r.tokens - 1) / r.tokens : 1;
    // about two blocks per CU, each wave keeping at least 8 16-deep MFMA
    // steps of its range (E > 64: four 64-deep staged steps)
    const long long want = (long long)cus * 2;
    int S = (int)((want + blocks - 1) / blocks);
    const int most = small ? d / (16 * 8 * kw) : d / 256;
    if (S > most) S = most;
    if (S > MOE_ROUTER_MAX_SPLITS) S = MOE_ROUTER_MAX_SPLITS;
    if (S < 1) S = 1;
    // whole steps per range (d is a multiple of 64): 16 deep, or 64 deep
    // for the staged kernel
    const int step = small ? 16 : 64;
    int kc = (d + S - 1) / S;
    kc = (kc + step - 1) / step * step;
    r.S = (d + kc - 1) / kc;
    r.kc = kc;
    return r;
}

hipError_t launch_router(const RouterParams &p, int dtype, hipStream_t s) {
    const int blocks = (p.T + RT - 1) / RT;
    const dim3 grid(blocks), block(RW * 64);
    const int EP = p.E <= 32 ? 32 : p.E <= 64 ? 64 : p.E <= 128 ? 128 : 256;
    if (dtype == 1 && !p.S) {
        switch (EP) {
        case 32: hipLaunchKernelGGL(router_fused<32>, grid, block, 0, s, p); break;
        case 64: hipLaunchKernelGGL(router_fused<64>, grid, block, 0, s, p); break;
        case 128: hipLaunchKernelGGL(router_fused<128>, grid, block, 0, s, p); break;
        default: hipLaunchKernelGGL(router_fused<256>, grid, block, 0, s, p); break;
        }
        return hipGetLastError();
    }
    if (dtype == 1) {
        const int tokens = EP <= 64 ? 32 : 128;
        const dim3 lgrid((p.T + tokens - 1) / tokens, p.S);
        switch (EP) {
        case 32:
            hipLaunchKernelGGL(router_logits<32>, lgrid, dim3(256), 0, s, p);
            hipLaunchKernelGGL(router_route<32>, grid, dim3(256), 0, s, p);
            break;
        case 64:
            hipLaunchKernelGGL(router_logits<64>, lgrid, dim3(256), 0, s, p);
            hipLaunchKernelGGL(router_route<64>, grid, block, 0, s, p);
            break;
        case 128:
            hipLaunchKernelGGL((router_logits_lds<128, 1>), lgrid, dim3(256), 0, s, p);
            hipLaunchKernelGGL(router_route<128>, grid, block, 0, s, p);
            break;
        default:
            hipLaunchKernelGGL((router_logits_lds<256, 1>), lgrid, dim3(256), 0, s, p);
            hipLaunchKernelGGL(router_route<256>, grid, block, 0, s, p);
            break;
        }
        return hipGetLastError();
    }
    switch (EP) {
    case 32: hipLaunchKernelGGL(router_f32<32>, grid, block, 0, s, p); break;
    case 64: hipLaunchKernelGGL(router_f32<64>, grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL(router_f32<128>, grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL(router_f32<256>, grid, block, 0, s, p); break;
    }
    return hipGetLastError();
}

bool route_permute_small_ok(const RouterParams &p) {
    return p.S > 0 && p.S <= MOE_ROUTER_MAX_SPLITS && p.E <= 32 &&
           p.T <= RT && p.T * p.k <= MOE_PERMUTE_ONE_BLOCK && !p.scores;
}

hipError_t launch_route_permute_small(const RouterParams &p,
                                      const PermuteParams &q, hipStream_t s) {
    const dim3 lgrid(1, p.S);
    hipLaunchKernelGGL(router_logits<32>, lgrid, dim3(256), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(route_permute_small<32>, dim3(1), dim3(256), 0, s, p, q);
    return hipGetLastError();
}
