// Counting, capacity, stable dispatch and statistics of a whole layer in
// one block, for T*k <= 256 assignments (one permute chunk) and one router
// token tile: the single-block form of permute.hip's dispatch (same
// arithmetic, same results), shared by the single-launch permute and by the
// router kernel that also routes and dispatches a decode step.
#pragma once

#include "kernels.h"

namespace {

// The six monitors from counts, kept and the reduced router sums z, h
// (thread 0 of the block).
__device__ void write_monitor(const PermuteParams &p, float z, float h,
                              const int *cnt_s, const int *kept_s) {
    int cmax = cnt_s[0], cmin = cnt_s[0], used = 0, kept = 0;
    for (int e = 0; e < p.E; ++e) {
        cmax = max(cmax, cnt_s[e]);
        cmin = min(cmin, cnt_s[e]);
        used += cnt_s[e] > 0;
        kept += kept_s[e];
    }
    const float n = (float)p.T * (float)p.k;
    p.monitor[0] = z / (float)p.T;
    p.monitor[1] = h / (float)p.T * 1.44269504088896340736f;  // nats -> bits
    p.monitor[2] = cmin > 0 ? (float)cmax / (float)cmin : INFINITY;
    p.monitor[3] = (float)used / (float)p.E;
    p.monitor[4] = (n - (float)kept) / n;
    p.monitor[5] = (float)cmax / (float)p.T;
}

// Sum of the per-router-block lse^2 and entropy partials in block order
// (single-block callers only; thread 0 gets the result).
__device__ void sum_zh_serial(const PermuteParams &p, float *z, float *h) {
    float zs = 0.0f, hs = 0.0f;
    for (int b = 0; b < p.n_rtiles; ++b) {
        zs += p.zh_part[(size_t)b * 2];
        hs += p.zh_part[(size_t)b * 2 + 1];
    }
    *z = zs;
    *h = hs;
}

// NT threads (a multiple of 64, at least MOE_MAX_E).  Reads p.topk_idx,
// p.p_part and p.zh_part; writes counts, kept, offsets, slot_token,
// slot_of, f, p, l_aux and the monitors.
template <int NT>
__device__ __forceinline__ void permute_one_block(const PermuteParams &p) {
    static_assert(NT % 64 == 0 && NT >= MOE_MAX_E, "block shape");

    __shared__ int h[MOE_MAX_E];
    __shared__ int off_s[MOE_MAX_E + 1];
    __shared__ float fp_s[MOE_MAX_E];
    __shared__ int cnt_s[MOE_MAX_E];
    __shared__ int kept_s[MOE_MAX_E];
    __shared__ int wsum[NT / 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = p.T * p.k;
    for (int e = tid; e < p.E; e += NT) h[e] = 0;
    __syncthreads();
    for (int a = tid; a < n; a += NT) {
        const int e = p.topk_idx[a];
        if ((unsigned)e < (unsigned)p.E) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    // counts, capacity, statistics, offsets (thread e = expert e)
    const int e = tid;
    int cnt = 0, kept = 0;
    if (e < p.E) {
        cnt = h[e];
        kept = (p.capacity >= 0 && cnt > p.capacity) ? p.capacity : cnt;
        p.counts[e] = cnt;
        p.kept[e] = kept;
        float ps = 0.0f;
        for (int b = 0; b < p.n_rtiles; ++b) ps += p.p_part[(size_t)b * p.E + e];
        const float pe = ps / (float)p.T;
        const float fe = (float)cnt / ((float)p.T * (float)p.k);
        p.p[e] = pe;
        p.f[e] = fe;
        fp_s[e] = fe * pe;
        cnt_s[e] = cnt;
        kept_s[e] = kept;
    }
    int incl = kept;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (e < p.E) {
        off_s[e] = before + incl - kept;
        p.offsets[e] = before + incl - kept;
        h[e] = 0;                       // becomes the running rank
    }
    if (e == p.E - 1) {
        off_s[p.E] = before + incl;
        p.offsets[p.E] = before + incl;
    }
    if (tid == 0) {
        float s = 0.0f;
        for (int i = 0; i < p.E; ++i) s += fp_s[i];
        p.l_aux[0] = p.alpha * (float)p.E * s;
        if (p.monitor) {
            float z, h;
            sum_zh_serial(p, &z, &h);
            write_monitor(p, z, h, cnt_s, kept_s);
        }
    }
    __syncthreads();
    if (wave == 0) {
        const unsigned long long lt = (1ull << lane) - 1ull;
        for (int base = 0; base < n; base += 64) {
            const int a = base + lane;
            int ex = a < n ? p.topk_idx[a] : -1;
            if ((unsigned)ex >= (unsigned)p.E) ex = -1;
            const bool ok = ex >= 0;
            int rank = 0;
            unsigned long long pending = __ballot(ok);
            while (pending) {
                const int leader = __ffsll((long long)pending) - 1;
                const int le = __shfl(ex, leader, 64);
                const unsigned long long same = __ballot(ex == le);
                const int r0 = h[le];
                if (ex == le) rank = r0 + __popcll(same & lt);
                __builtin_amdgcn_wave_barrier();
                if (lane == leader) h[le] = r0 + __popcll(same);
                __builtin_amdgcn_wave_barrier();
                pending &= ~same;
            }
            if (a < n) {
                int slot = -1;
                if (ok && (p.capacity < 0 || rank < p.capacity)) {
                    slot = off_s[ex] + rank;
                    p.slot_token[slot] = a / p.k;
                }
                p.slot_of[a] = slot;
            }
        }
    }
    __syncthreads();
    for (int sl = tid; sl < n; sl += NT)
        if (sl >= off_s[p.E]) p.slot_token[sl] = -1;
}

}  // namespace
