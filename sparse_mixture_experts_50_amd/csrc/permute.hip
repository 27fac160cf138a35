// Counting, capacity, stable dispatch and load-balance statistics.
//
// "AI-Research-SKILLs MoE training guide", sec. 4.3: expert counts are the
// bincount of the selected indices, f is that count over the number of
// selections, p the mean gate probability; "MoE architecture deep dive",
// sec. 2.2: L_aux = alpha * N * sum f_i p_i; sec. 2.3: an expert takes at
// most floor(T/E * cf) tokens, the overflow skips the experts; sec. 2.4:
// the per-expert bias moves up for an overloaded expert.
//
// Three launches (one when T*k fits a single chunk), no float atomics,
// deterministic:
//   hist    one block per 256-assignment chunk: LDS-atomic histogram
//   scan    one block: per-expert exclusive scan over chunks (rank bases),
//           counts, kept = min(count, C), offsets, f, p, L_aux
//   scatter one wave per chunk: within-wave stable ranks by ballot over
//           equal experts, slot = offset + rank, overflow -> -1
// Assignments are numbered a = t*k + j, so chunk order is token-major and
// the resulting permutation is stable in (t, j).
#include "kernels.h"

namespace {

constexpr int CH = MOE_PERMUTE_CHUNK;

// The six monitors from counts and kept (thread 0 of the block; the
// per-router-block lse^2 and entropy sums are reduced in block order).
__device__ void write_monitor(const PermuteParams &p, const int *cnt_s,
                              const int *kept_s) {
    float z = 0.0f, h = 0.0f;
    for (int b = 0; b < p.n_rtiles; ++b) {
        z += p.zh_part[(size_t)b * 2];
        h += p.zh_part[(size_t)b * 2 + 1];
    }
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

__global__ __launch_bounds__(256) void permute_hist(PermuteParams p) {
    __shared__ int h[MOE_MAX_E];
    for (int e = threadIdx.x; e < p.E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int n = p.T * p.k;
    const int a0 = blockIdx.x * CH;
    const int a1 = min(n, a0 + CH);
    for (int a = a0 + threadIdx.x; a < a1; a += blockDim.x) {
        const int e = p.topk_idx[a];
        // an id outside [0, E) (only possible from non-finite logits) is
        // never counted and never dispatched
        if ((unsigned)e < (unsigned)p.E) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < p.E; e += blockDim.x)
        p.blk[(size_t)blockIdx.x * p.E + e] = h[e];
}

__global__ __launch_bounds__(256) void permute_scan(PermuteParams p) {
    __shared__ int kept_s[MOE_MAX_E];
    __shared__ int cnt_s[MOE_MAX_E];
    __shared__ float fp_s[MOE_MAX_E];
    __shared__ int wsum[4];
    const int e = threadIdx.x;
    int cnt = 0, kept = 0;
    if (e < p.E) {
        // batches of 8 independent loads keep the serial scans short
        int b = 0;
        for (; b + 8 <= p.n_chunks; b += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = p.blk[(size_t)(b + u) * p.E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                p.blk[(size_t)(b + u) * p.E + e] = cnt;  // rank base
                cnt += v[u];
            }
        }
        for (; b < p.n_chunks; ++b) {
            const size_t i = (size_t)b * p.E + e;
            const int v = p.blk[i];
            p.blk[i] = cnt;           // rank base of expert e in chunk b
            cnt += v;
        }
        kept = (p.capacity >= 0 && cnt > p.capacity) ? p.capacity : cnt;
        p.counts[e] = cnt;
        p.kept[e] = kept;
        float ps = 0.0f;
        b = 0;
        for (; b + 8 <= p.n_rtiles; b += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = p.p_part[(size_t)(b + u) * p.E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) ps += v[u];
        }
        for (; b < p.n_rtiles; ++b) ps += p.p_part[(size_t)b * p.E + e];
        const float pe = ps / (float)p.T;
        const float fe = (float)cnt / ((float)p.T * (float)p.k);
        p.p[e] = pe;
        p.f[e] = fe;
        fp_s[e] = fe * pe;
    }
    kept_s[e] = kept;
    cnt_s[e] = cnt;
    // exclusive scan of kept over experts (256 threads = 4 waves)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
    if (e < p.E) p.offsets[e] = before + incl - kept;
    if (e == p.E - 1) p.offsets[p.E] = before + incl;
    if (threadIdx.x == 0) {
        float s = 0.0f;
        for (int i = 0; i < p.E; ++i) s += fp_s[i];
        p.l_aux[0] = p.alpha * (float)p.E * s;
        if (p.monitor) write_monitor(p, cnt_s, kept_s);
    }
}

__global__ __launch_bounds__(64) void permute_scatter(PermuteParams p) {
    __shared__ int run[MOE_MAX_E];
    const int lane = threadIdx.x;
    const int b = blockIdx.x;
    for (int e = lane; e < p.E; e += 64) run[e] = p.blk[(size_t)b * p.E + e];
    __syncthreads();
    const int n = p.T * p.k;
    const int a0 = b * CH;
    const int a1 = min(n, a0 + CH);
    const int total = p.offsets[p.E];
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int base = a0; base < a1; base += 64) {
        const int a = base + lane;
        int e = a < a1 ? p.topk_idx[a] : -1;
        if ((unsigned)e >= (unsigned)p.E) e = -1;
        const bool ok = e >= 0;
        int rank = 0;
        unsigned long long pending = __ballot(ok);
        while (pending) {
            const int leader = __ffsll((long long)pending) - 1;
            const int le = __shfl(e, leader, 64);
            const unsigned long long same = __ballot(e == le);
            const int r0 = run[le];
            if (e == le) rank = r0 + __popcll(same & lt);
            __syncthreads();   // all lanes have read run[le]
            if (lane == leader) run[le] = r0 + __popcll(same);
            __syncthreads();
            pending &= ~same;
        }
        if (a < a1) {
            int slot = -1;
            if (ok && (p.capacity < 0 || rank < p.capacity)) {
                slot = p.offsets[e] + rank;
                p.slot_token[slot] = a / p.k;
            }
            p.slot_of[a] = slot;
        }
    }
    // slots past the last kept one hold -1
    for (int s = a0 + lane; s < a1; s += 64)
        if (s >= total) p.slot_token[s] = -1;
}

// All three steps in one block when every assignment fits one chunk
// (T*k <= 256, e.g. a decode step): same arithmetic, one launch.
__global__ __launch_bounds__(256) void permute_small(PermuteParams p) {
    __shared__ int h[MOE_MAX_E];
    __shared__ int off_s[MOE_MAX_E + 1];
    __shared__ float fp_s[MOE_MAX_E];
    __shared__ int cnt_s[MOE_MAX_E];
    __shared__ int kept_s[MOE_MAX_E];
    __shared__ int wsum[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int n = p.T * p.k;
    for (int e = tid; e < p.E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    for (int a = tid; a < n; a += blockDim.x) {
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
        if (p.monitor) write_monitor(p, cnt_s, kept_s);
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
    for (int sl = tid; sl < n; sl += blockDim.x)
        if (sl >= off_s[p.E]) p.slot_token[sl] = -1;
}

__global__ void bias_update_kernel(int E, const int32_t *counts, float target,
                                   float gamma, float *bias) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < E) {
        const float c = (float)counts[e];
        const float sgn = c > target ? 1.0f : (c < target ? -1.0f : 0.0f);
        bias[e] = __fadd_rn(bias[e], gamma * sgn);
    }
}

}  // namespace

hipError_t launch_permute(const PermuteParams &p, hipStream_t s) {
    if (p.n_chunks == 1) {
        hipLaunchKernelGGL(permute_small, dim3(1), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(permute_hist, dim3(p.n_chunks), dim3(256), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(permute_scan, dim3(1), dim3(256), 0, s, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(permute_scatter, dim3(p.n_chunks), dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bias_update(int E, const int32_t *counts, float target,
                              float gamma, float *bias, hipStream_t s) {
    hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0,
                       s, E, counts, target, gamma, bias);
    return hipGetLastError();
}
