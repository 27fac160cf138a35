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
//
// Expert choice ("AI-Research-SKILLs MoE training guide", sec. 4.2): every
// token is a candidate of every expert (counts = T, k = E) and expert e
// keeps its C largest logits instead of its first C tokens.  Two launches:
//   scan    as above, with counts = T
//   select  one block per expert: exact radix select of the C-th largest
//           logit (passes of 11, 11 and 10 bits over order-preserving
//           keys), then the picks in token order; equal keys go to the
//           lower token index
#include "kernels.h"

namespace {

constexpr int CH = MOE_PERMUTE_CHUNK;

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

// One block of 1024 threads, thread = (segment, expert): S = 1024 / E
// segments split the chunk list and the router-block list, so each thread
// walks n/S entries instead of n; partial results meet in LDS and are
// summed in segment order (deterministic).
constexpr int SCAN_THREADS = 1024;

__global__ __launch_bounds__(SCAN_THREADS) void permute_scan(PermuteParams p) {
    __shared__ int seg_i[SCAN_THREADS];
    __shared__ float seg_f[SCAN_THREADS];
    __shared__ float zh_w[SCAN_THREADS / 64][2];
    __shared__ int kept_s[MOE_MAX_E];
    __shared__ int cnt_s[MOE_MAX_E];
    __shared__ float fp_s[MOE_MAX_E];
    __shared__ int wsum[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int S = SCAN_THREADS / p.E;              // E <= 256: S >= 4
    const int e = tid % p.E, seg = tid / p.E;
    const bool active = seg < S;

    // 1. chunk counts of expert e over this segment's chunks
    const int L = (p.n_chunks + S - 1) / S;
    const int c0 = min(p.n_chunks, seg * L), c1 = min(p.n_chunks, c0 + L);
    int part = 0;
    if (active) {
        int b = c0;
        for (; b + 32 <= c1; b += 32) {
            int v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = p.blk[(size_t)(b + u) * p.E + e];
#pragma unroll
            for (int u = 0; u < 32; ++u) part += v[u];
        }
        for (; b < c1; ++b) part += p.blk[(size_t)b * p.E + e];
        seg_i[seg * p.E + e] = part;
    }
    // 2. probability column sums over this segment's router blocks
    if (active) {
        float ps = 0.0f;
        int b = seg;
        for (; b + 31 * S < p.n_rtiles; b += 32 * S) {
            float v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = p.p_part[(size_t)(b + u * S) * p.E + e];
#pragma unroll
            for (int u = 0; u < 32; ++u) ps += v[u];
        }
        for (; b < p.n_rtiles; b += S) ps += p.p_part[(size_t)b * p.E + e];
        seg_f[seg * p.E + e] = ps;
    }
    // 3. router z / entropy partials: all threads, then waves in order
    float zs = 0.0f, hs = 0.0f;
    if (p.monitor) {
        for (int b = tid; b < p.n_rtiles; b += SCAN_THREADS) {
            zs += p.zh_part[(size_t)b * 2];
            hs += p.zh_part[(size_t)b * 2 + 1];
        }
        zs = wave_sum(zs);
        hs = wave_sum(hs);
        if (lane == 0) {
            zh_w[wave][0] = zs;
            zh_w[wave][1] = hs;
        }
    }
    __syncthreads();
    // 4a. inclusive scan of the segment counts over the segments, per
    // expert: log2(S) steps through LDS instead of a loop over up to S - 1
    // earlier segments per thread (S = 128 at E = 8)
    for (int d = 1; d < S; d <<= 1) {
        int v = 0;
        if (active && seg >= d) v = seg_i[(seg - d) * p.E + e];
        __syncthreads();
        if (active) seg_i[seg * p.E + e] += v;
        __syncthreads();
    }
    // 4. rank bases: the segment's base plus a running count over its
    // chunks, 32 counts loaded before any base is written (one memory round
    // trip per 32 chunks rather than per chunk)
    if (active && p.n_chunks > 0) {
        int run = seg_i[seg * p.E + e] - part;   // earlier segments' counts
        int b = c0;
        for (; b + 32 <= c1; b += 32) {
            int v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = p.blk[(size_t)(b + u) * p.E + e];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                p.blk[(size_t)(b + u) * p.E + e] = run;   // rank base in chunk b+u
                run += v[u];
            }
        }
        for (; b < c1; ++b) {
            const size_t i = (size_t)b * p.E + e;
            const int v = p.blk[i];
            p.blk[i] = run;
            run += v;
        }
    }
    // 5. per expert (threads 0..E-1): counts, kept, f, p
    int cnt = 0, kept = 0;
    if (tid < p.E) {
        if (p.scores) {
            cnt = p.T;                    // expert choice: every token
        } else {
            cnt = seg_i[(S - 1) * p.E + tid];   // inclusive over every segment
        }
        float ps = 0.0f;
        for (int q = 0; q < S; ++q) ps += seg_f[q * p.E + tid];
        kept = (p.capacity >= 0 && cnt > p.capacity) ? p.capacity : cnt;
        p.counts[tid] = cnt;
        p.kept[tid] = kept;
        const float pe = ps / (float)p.T;
        const float fe = (float)cnt / ((float)p.T * (float)p.k);
        p.p[tid] = pe;
        p.f[tid] = fe;
        fp_s[tid] = fe * pe;
        kept_s[tid] = kept;
        cnt_s[tid] = cnt;
    }
    // 6. offsets: exclusive scan of kept over experts (waves 0-3)
    int incl = kept;
    if (tid < 256) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        if (lane == 63) wsum[wave] = incl;
    }
    __syncthreads();
    if (tid < p.E) {
        int before = 0;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        p.offsets[tid] = before + incl - kept;
        if (tid == p.E - 1) p.offsets[p.E] = before + incl;
    }
    if (tid == 0) {
        float sfp = 0.0f;
        for (int i = 0; i < p.E; ++i) sfp += fp_s[i];
        p.l_aux[0] = p.alpha * (float)p.E * sfp;
        if (p.monitor) {
            float z = 0.0f, h = 0.0f;
            for (int w = 0; w < SCAN_THREADS / 64; ++w) {
                z += zh_w[w][0];
                h += zh_w[w][1];
            }
            write_monitor(p, z, h, cnt_s, kept_s);
        }
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
    // bits of an expert id: the lanes holding the same expert as this one
    // are those whose ballot agrees with this lane's on every bit
    const int nbits = p.E > 1 ? 32 - __clz(p.E - 1) : 1;
    for (int base = a0; base < a1; base += 64) {
        const int a = base + lane;
        int e = a < a1 ? p.topk_idx[a] : -1;
        if ((unsigned)e >= (unsigned)p.E) e = -1;
        const bool ok = e >= 0;
        unsigned long long same = __ballot(ok);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = (e >> bit) & 1;
            const unsigned long long m = __ballot(on);
            same &= on ? m : ~m;
        }
        // rank: the expert's running count plus the earlier lanes of the
        // same expert; the group's last lane advances the count (every lane
        // of the wave has read it before: one wave, LDS in program order)
        int rank = 0;
        if (ok) {
            const int before = __popcll(same & lt);
            rank = run[e] + before;
            if (before == __popcll(same) - 1) run[e] = rank + 1;
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
    for (int sl = tid; sl < n; sl += blockDim.x)
        if (sl >= off_s[p.E]) p.slot_token[sl] = -1;
}

// Float -> unsigned key with the same order (-0 is ranked with +0, as
// the two compare equal).
__device__ __forceinline__ unsigned order_key(float v) {
    unsigned u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int EC_THREADS = 1024;
constexpr int EC_WAVES = EC_THREADS / 64;
constexpr int EC_KR = 8;          // keys per lane kept in registers
constexpr int EC_BINS = 2048;     // 11-bit digits: passes of 11, 11, 10 bits

// One 64-token step of a wave's in-order pick emission: keys above thr
// are picked, equal keys while fewer than `need` equal ones came before.
// sb / eb count the picks and the equal keys before this step.
__device__ __forceinline__ void ec_pick_step(const PermuteParams &p, int e,
                                             int C, unsigned thr, int need,
                                             int t, bool in, unsigned u,
                                             int &sb, int &eb) {
    const int lane = threadIdx.x & 63;
    const unsigned long long lt = (1ull << lane) - 1ull;
    const bool gt = in && u > thr;
    const bool eq = in && u == thr;
    const unsigned long long em = __ballot(eq);
    const bool sel = gt || (eq && eb + __popcll(em & lt) < need);
    const unsigned long long sm = __ballot(sel);
    if (sel) {
        const int slot = e * C + sb + __popcll(sm & lt);
        p.slot_token[slot] = t;
        p.slot_of[(size_t)t * p.E + e] = slot;
    }
    sb += __popcll(sm);
    eb += __popcll(em);
}

// Expert choice, block e: wave w owns the contiguous token segment
// [w*L, (w+1)*L) (L a multiple of 64) and lane l its tokens w*L + 64i + l.
// Keys of the first EC_KR*1024 tokens are staged in LDS; beyond that
// (T > 8192) they are re-read.  The router has already set
// slot_of[t][e] = -1 everywhere, so only the C picks are written here.
__global__ __launch_bounds__(EC_THREADS) void ec_select(PermuteParams p) {
    __shared__ unsigned keys[EC_KR * EC_THREADS];
    __shared__ __attribute__((aligned(16))) int hist[EC_BINS];
    __shared__ int w_gt[EC_WAVES], w_eq[EC_WAVES];
    __shared__ unsigned s_digit;
    __shared__ int s_need;
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = p.T, C = p.capacity;
    if (C == 0) return;
    const float *sc = p.scores + (size_t)e * T;
    const int L = ((T + EC_WAVES - 1) / EC_WAVES + 63) / 64 * 64;
    const int s0 = wave * L;
    const int s1 = min(T, s0 + L);
    const int n_i = L / 64;
    const int n_r = min(n_i, EC_KR);      // 64-token steps staged in LDS
    // LDS slot of step i of this lane (wave-private, so no barrier needed)
    unsigned *kw = keys + wave * (EC_KR * 64) + lane;
    for (int i = 0; i < n_r; ++i) {
        const int t = s0 + 64 * i + lane;
        kw[64 * i] = t < s1 ? order_key(sc[t]) : 0u;
    }

    // thr = the C-th largest key; need = how many keys equal to thr are
    // picked (every key above thr is).  Invariant of each pass: at least
    // `need` keys match `prefix` on the bits fixed so far.
    unsigned prefix = 0, mask = 0;
    int need = C;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
        const unsigned dmask = pass == 2 ? 0x3FFu : 0x7FFu;
        for (int i = tid; i < EC_BINS; i += EC_THREADS) hist[i] = 0;
        __syncthreads();
        for (int i = 0; i < n_i; ++i) {
            const int t = s0 + 64 * i + lane;
            if (t < s1) {
                const unsigned u = i < n_r ? kw[64 * i] : order_key(sc[t]);
                if ((u & mask) == prefix)
                    atomicAdd(&hist[(u >> shift) & dmask], 1);
            }
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds bins [2016-32l, 2047-32l], scanned high to low
            const int lo = EC_BINS - 32 - 32 * lane;
            int sum = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int4 v = *(const int4 *)&hist[lo + 4 * q];
                sum += v.x + v.y + v.z + v.w;
            }
            int incl = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o, 64);
                if (lane >= o) incl += v;
            }
            int before = incl - sum;
            if (before < need && need <= incl) {   // exactly one lane
                for (int j = 31; j >= 0; --j) {
                    const int c = hist[lo + j];
                    if (need <= before + c) {
                        s_digit = (unsigned)(lo + j);
                        s_need = need - before;
                        break;
                    }
                    before += c;
                }
            }
        }
        __syncthreads();
        // s_digit / s_need are rewritten only after the next pass's
        // histogram barrier, which every thread reaches after this read
        prefix |= s_digit << shift;
        mask |= dmask << shift;
        need = s_need;
    }

    // picks in token order: count per wave, one barrier, then every wave
    // emits its own segment
    int n_gt = 0, n_eq = 0;
    for (int i = 0; i < n_i; ++i) {
        const int t = s0 + 64 * i + lane;
        const bool in = t < s1;
        const unsigned u = !in ? 0u : i < n_r ? kw[64 * i] : order_key(sc[t]);
        n_gt += __popcll(__ballot(in && u > prefix));
        n_eq += __popcll(__ballot(in && u == prefix));
    }
    if (lane == 0) {
        w_gt[wave] = n_gt;
        w_eq[wave] = n_eq;
    }
    __syncthreads();
    int gt_before = 0, eq_before = 0;
    for (int w = 0; w < wave; ++w) {
        gt_before += w_gt[w];
        eq_before += w_eq[w];
    }
    int sb = gt_before + min(eq_before, need);   // picks before this wave
    int eb = eq_before;                          // equal keys before it
    for (int i = 0; i < n_i; ++i) {
        const int t = s0 + 64 * i + lane;
        const bool in = t < s1;
        const unsigned u = !in ? 0u : i < n_r ? kw[64 * i] : order_key(sc[t]);
        ec_pick_step(p, e, C, prefix, need, t, in, u, sb, eb);
    }
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
    hipLaunchKernelGGL(permute_scan, dim3(1), dim3(SCAN_THREADS), 0, s, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(permute_scatter, dim3(p.n_chunks), dim3(64), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_expert_choice(const PermuteParams &p, hipStream_t s) {
    hipLaunchKernelGGL(permute_scan, dim3(1), dim3(SCAN_THREADS), 0, s, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(ec_select, dim3(p.E), dim3(EC_THREADS), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bias_update(int E, const int32_t *counts, float target,
                              float gamma, float *bias, hipStream_t s) {
    hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0,
                       s, E, counts, target, gamma, bias);
    return hipGetLastError();
}
