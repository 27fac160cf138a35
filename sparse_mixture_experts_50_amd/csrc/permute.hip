// Counting, capacity, stable dispatch and load-balance statistics.
//
// "AI-Research-SKILLs MoE training guide", sec. 4.3: expert counts are the
// bincount of the selected indices, f is that count over the number of
// selections, p the mean gate probability; "MoE architecture deep dive",
// sec. 2.2: L_aux = alpha * N * sum f_i p_i; sec. 2.3: an expert takes at
// most floor(T/E * cf) tokens, the overflow skips the experts; sec. 2.4:
// the per-expert bias moves up for an overloaded expert.
//
// A chunk is the 32 k assignments of one router token tile, whose
// expert histogram the router block already counted in LDS (with LDS
// atomics) and wrote to blk.  One launch, no float atomics, deterministic:
//   dispatch one block per chunk: from the whole histogram its rank bases
//            (counts of the earlier chunks) and the expert offsets
//            (exclusive scan of kept = min(count, C)); integer sums, so
//            every block finds the same offsets.  Then one wave ranks
//            equal experts by ballot: slot = offset + rank, overflow -> -1
//   stats    one more block: counts, kept, offsets, f, p, L_aux, monitor
// (a single block does all of it when T*k fits one block).
// Assignments are numbered a = t*k + j, so chunk order is token-major and
// the resulting permutation is stable in (t, j).
//
// Expert choice ("AI-Research-SKILLs MoE training guide", sec. 4.2): every
// token is a candidate of every expert (counts = T, k = E) and expert e
// keeps its C largest logits instead of its first C tokens.  One launch:
//   stats   one block, as above, with counts = T
//   select  one block per expert: exact radix select of the C-th largest
//           logit (passes of 11, 11 and 10 bits over order-preserving
//           keys), then the picks in token order; equal keys go to the
//           lower token index
#include "kernels.h"
#include "permute_block.h"

namespace {

// Assignments per chunk: one router token tile's.
constexpr int CH = MOE_ROUTER_TOKENS;
// Most experts per token under top-k routing.
constexpr int MOE_MAX_TOPK = 64;

// Blocks of 1024 threads, thread = (segment, expert): S = 1024 / E
// segments split the chunk list and the router-block list, so each thread
// walks n/S entries instead of n; partial results meet in LDS and are
// summed in segment order (deterministic).
constexpr int SCAN_THREADS = 1024;

// Counts, kept, offsets, f, p, L_aux and the monitor, in one block.
__device__ __forceinline__ void stats_block(const PermuteParams &p) {
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

    // 1-2. chunk counts of expert e over this segment's chunks, and its
    // probability column sum over the segment's router blocks (blocks
    // seg, seg + S, ... added in that order); both in batches of 16 loads
    // issued before any is added (past the end a batch re-reads the last
    // entry and adds zero instead, which is exact: the probabilities are
    // never -0)
    const int L = (p.n_chunks + S - 1) / S;
    const int c0 = min(p.n_chunks, seg * L), c1 = min(p.n_chunks, c0 + L);
    const int nr = seg < p.n_rtiles ? (p.n_rtiles - 1 - seg) / S + 1 : 0;
    if (active) {
        const bool has_c = c0 < c1, has_r = nr > 0;
        const int nb = max((c1 - c0 + 15) / 16, (nr + 15) / 16);
        int part = 0;
        float ps = 0.0f;
        for (int it = 0; it < nb; ++it) {
            int vi[16];
            float vf[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int c = max(min(c0 + it * 16 + u, c1 - 1), 0);
                vi[u] = has_c ? p.blk[(size_t)c * p.E + e] : 0;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int r = max(min(it * 16 + u, nr - 1), 0);
                vf[u] = has_r ? p.p_part[(size_t)(seg + r * S) * p.E + e] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                part += c0 + it * 16 + u < c1 ? vi[u] : 0;
                ps += it * 16 + u < nr ? vf[u] : 0.0f;
            }
        }
        seg_i[seg * p.E + e] = part;
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
    // 4. per expert (threads 0..E-1): counts, kept, f, p
    int cnt = 0, kept = 0;
    if (tid < p.E) {
        int cs = 0;
        float ps = 0.0f;
        for (int q = 0; q < S; ++q) {
            cs += seg_i[q * p.E + tid];
            ps += seg_f[q * p.E + tid];
        }
        cnt = p.scores ? p.T : cs;        // expert choice: every token
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
    // 5. offsets: exclusive scan of kept over experts (waves 0-3)
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

// Chunk b: rank bases (its experts' counts over chunks 0..b-1) and the
// expert offsets from the whole histogram, then one wave places the
// chunk's assignments.
__device__ __forceinline__ void chunk_block(const PermuteParams &p, int b) {
    __shared__ int tot_s[MOE_MAX_E];
    __shared__ int run[MOE_MAX_E];
    __shared__ int off_s[MOE_MAX_E + 1];
    __shared__ int idx_s[CH * MOE_MAX_TOPK];
    __shared__ int wsum[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int E = p.E;
    const int n = p.T * p.k;
    const int a0 = b * CH * p.k;
    const int a1 = min(n, a0 + CH * p.k);
    // the chunk's expert ids, requested first so that they arrive while
    // the histogram is read
    for (int a = a0 + tid; a < a1; a += SCAN_THREADS) idx_s[a - a0] = p.topk_idx[a];
    for (int i = tid; i < E; i += SCAN_THREADS) {
        tot_s[i] = 0;
        run[i] = 0;
    }
    __syncthreads();
    // 1. counts of expert e over this segment's chunks, all of them and
    // those before b, in batches of 16 loads (a partial batch re-reads the
    // segment's last chunk and adds zero for it)
    const int S = SCAN_THREADS / E;                // E <= 256: S >= 4
    const int e = tid % E, seg = tid / E;
    if (seg < S) {
        const int L = (p.n_chunks + S - 1) / S;
        const int c0 = min(p.n_chunks, seg * L), c1 = min(p.n_chunks, c0 + L);
        int tot = 0, bef = 0;
        int c = c0;
        for (; c + 16 <= c1; c += 16) {
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = p.blk[(size_t)(c + u) * E + e];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                tot += v[u];
                bef += c + u < b ? v[u] : 0;
            }
        }
        for (; c < c1; c += 16) {
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = p.blk[(size_t)min(c + u, c1 - 1) * E + e];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int x = c + u < c1 ? v[u] : 0;
                tot += x;
                bef += c + u < b ? x : 0;
            }
        }
        if (tot) atomicAdd(&tot_s[e], tot);
        if (bef) atomicAdd(&run[e], bef);
    }
    __syncthreads();
    // 2. offsets: exclusive scan of kept = min(count, C) over experts
    int kept = 0, incl = 0;
    if (tid < 256) {
        if (tid < E) {
            const int cnt = tot_s[tid];
            kept = (p.capacity >= 0 && cnt > p.capacity) ? p.capacity : cnt;
        }
        incl = kept;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        if (lane == 63) wsum[wave] = incl;
    }
    __syncthreads();
    if (tid < E) {
        int before = 0;
        for (int w = 0; w < wave; ++w) before += wsum[w];
        off_s[tid] = before + incl - kept;
        if (tid == E - 1) off_s[E] = before + incl;
    }
    __syncthreads();
    if (wave != 0) return;
    // 3. one wave: stable ranks by ballot over equal experts
    const int total = off_s[E];
    const unsigned long long lt = (1ull << lane) - 1ull;
    // bits of an expert id: the lanes holding the same expert as this one
    // are those whose ballot agrees with this lane's on every bit
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 1;
    for (int base = a0; base < a1; base += 64) {
        const int a = base + lane;
        int ea = a < a1 ? idx_s[a - a0] : -1;
        if ((unsigned)ea >= (unsigned)E) ea = -1;
        const bool ok = ea >= 0;
        unsigned long long same = __ballot(ok);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = (ea >> bit) & 1;
            const unsigned long long m = __ballot(on);
            same &= on ? m : ~m;
        }
        // rank: the expert's running count plus the earlier lanes of the
        // same expert; the group's last lane advances the count (every lane
        // of the wave has read it before: one wave, LDS in program order)
        int rank = 0;
        if (ok) {
            const int before = __popcll(same & lt);
            rank = run[ea] + before;
            if (before == __popcll(same) - 1) run[ea] = rank + 1;
        }
        if (a < a1) {
            int slot = -1;
            if (ok && (p.capacity < 0 || rank < p.capacity)) {
                slot = off_s[ea] + rank;
                p.slot_token[slot] = a / p.k;
            }
            p.slot_of[a] = slot;
        }
    }
    // slots past the last kept one hold -1
    for (int s = a0 + lane; s < a1; s += 64)
        if (s >= total) p.slot_token[s] = -1;
}

// Top-k dispatch: blocks 0..n_chunks-1 place their chunks, block n_chunks
// writes the statistics.  At most 64 registers a lane, so that two blocks
// fit a CU and the statistics block, the last, does not wait for a chunk
// block to end.
__global__ __launch_bounds__(SCAN_THREADS, 8) void permute_dispatch(PermuteParams p) {
    if ((int)blockIdx.x == p.n_chunks)
        stats_block(p);
    else
        chunk_block(p, blockIdx.x);
}

// Counting, scan and dispatch in one block when T*k <= 256 (e.g. a decode
// step): the same arithmetic over the same assignments, one launch.
__global__ __launch_bounds__(256) void permute_small(PermuteParams p) {
    permute_one_block<256>(p);
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

// Expert choice, expert e (block 1 + e): wave w owns the token segment
// [w*L, (w+1)*L) (L a multiple of 64) and lane l its tokens w*L + 64i + l.
// Keys of the first EC_KR*1024 tokens are staged in LDS; beyond that
// (T > 8192) they are re-read.  The router has already set
// slot_of[t][e] = -1 everywhere, so only the C picks are written here.
__device__ __forceinline__ void ec_select_block(const PermuteParams &p, int e) {
    __shared__ unsigned keys[EC_KR * EC_THREADS];
    __shared__ __attribute__((aligned(16))) int hist[EC_BINS];
    __shared__ int w_gt[EC_WAVES], w_eq[EC_WAVES];
    __shared__ unsigned s_digit;
    __shared__ int s_need;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = p.T, C = p.capacity;
    if (C == 0) return;
    const float *sc = p.scores + (size_t)e * T;
    const int L = ((T + EC_WAVES - 1) / EC_WAVES + 63) / 64 * 64;
    const int s0 = wave * L;
    const int s1 = min(T, s0 + L);
    const int n_i = L / 64;
    const int n_r = min(n_i, EC_KR);      // 64-token steps staged in LDS
    // LDS slot of step i of this lane (wave-private, so no barrier needed).
    // The EC_KR loads are issued together (addresses clamped into the
    // row, the values past the segment then replaced by 0) rather than one
    // wait per step.
    unsigned *kw = keys + wave * (EC_KR * 64) + lane;
    {
        float v[EC_KR];
#pragma unroll
        for (int i = 0; i < EC_KR; ++i) v[i] = sc[min(s0 + 64 * i + lane, T - 1)];
#pragma unroll
        for (int i = 0; i < EC_KR; ++i) {
            const int t = s0 + 64 * i + lane;
            if (i < n_r) kw[64 * i] = t < s1 ? order_key(v[i]) : 0u;
        }
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

// Expert choice: block 0 writes the statistics (counts = T, kept = C,
// offsets e*C: it reads no pick, the picks read none of it), block 1 + e
// picks expert e's tokens.  The statistics block goes first: where the
// E + 1 blocks outnumber the CUs (one such block fits a CU), the block
// left waiting is a pick that starts when the short statistics block ends.
static_assert(EC_THREADS == SCAN_THREADS, "one block shape");
__global__ __launch_bounds__(EC_THREADS) void ec_dispatch(PermuteParams p) {
    if (blockIdx.x == 0)
        stats_block(p);
    else
        ec_select_block(p, (int)blockIdx.x - 1);
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
    if ((long long)p.T * p.k <= MOE_PERMUTE_ONE_BLOCK) {
        hipLaunchKernelGGL(permute_small, dim3(1), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(permute_dispatch, dim3(p.n_chunks + 1), dim3(SCAN_THREADS),
                       0, s, p);
    return hipGetLastError();
}

hipError_t launch_expert_choice(const PermuteParams &p, hipStream_t s) {
    hipLaunchKernelGGL(ec_dispatch, dim3(p.E + 1), dim3(EC_THREADS), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bias_update(int E, const int32_t *counts, float target,
                              float gamma, float *bias, hipStream_t s) {
    hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0,
                       s, E, counts, target, gamma, bias);
    return hipGetLastError();
}
