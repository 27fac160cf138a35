/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts FFN layer
 * forward.
 *
 * The layer (sources are the pages' titles and sections):
 *   1. router logits  l[t,e] = x[t,:] . Wr[e,:] + add[e] - b[e], softmax
 *      ("MoE architecture deep dive", sec. 1.2 gating network; sec. 2.4
 *      aux-loss-free balancing subtracts b);
 *   2. top-k with renormalised weights (same page, sec. 1.3 steps 2-3;
 *      "AI-Research-SKILLs MoE training guide", sec. 3.1 and 4.2);
 *   3. per-expert counts, optional capacity C = floor(T/E * cf), stable
 *      token-order dispatch; overflow assignments skip the expert
 *      ("MoE architecture deep dive", sec. 2.3);
 *   4. each expert: W2 GELU(W1 x + b1) + b2 with exact erf GELU
 *      ("The expert group activated per token", sec. 3.1 FFN formula), or
 *      with SiLU, or gated: W2 (SiLU(W1 x + b1) * (W3 x + b3)) + b2
 *      (SwiGLU) ("AI-Research-SKILLs MoE training guide", sec. 6.1
 *      Mixtral block: its code uses Linear, SiLU, Linear, its text SwiGLU);
 *      optional always-on shared expert ("MoE architecture deep dive",
 *      sec. 3, DeepSeek-V3 shared expert);
 *   5. y[t] = sum_j w[t,j] Expert_{idx[t,j]}(x[t]) (+ Shared(x[t]))
 *      ("MoE architecture deep dive", sec. 1.1);
 *   6. f_i = count_i / (T k), p_i = mean_t p[t,i],
 *      L_aux = alpha * E * sum f_i p_i (same page, sec. 2.2; "AI-Research-
 *      SKILLs MoE training guide", sec. 4.3);
 *   7. balancing-bias step b_i += gamma * sign(count_i - target)
 *      ("MoE architecture deep dive", sec. 2.4).
 *
 * Expert-Choice routing (desc->routing == MOE_ROUTE_EXPERT_CHOICE;
 * "AI-Research-SKILLs MoE training guide", sec. 4.2, Expert Choice):
 * instead of steps 2-3 every expert picks its own C = desc->capacity
 * tokens, the C largest router logits l[t,e] in its column (ties to the
 * lower token index), so each expert holds exactly C tokens.  A pick is
 * weighted by the token's softmax probability p[t,e], not renormalised; a
 * token no expert picked gets y = 0 (plus the shared expert).  The mode
 * reuses the top-k data layout with k = E: each token is a candidate of
 * every expert, in expert order, and the capacity rule becomes the
 * per-expert top-C.  So for every t and e:
 *   topk_idx[t][e] = e,  topk_w[t][e] = p[t,e],
 *   slot_of[t][e]  = e*C + (rank of t among the picks of e in token
 *                    order), or -1 if e did not pick t,
 *   slot_token[e*C + r] = the r-th picked token of e (ascending),
 *   counts[e] = T, kept[e] = C, offsets[e] = e*C,
 * and f, p, L_aux and the monitors follow from those counts with k = E
 * (f_i = 1/E, L_aux = alpha * sum_i p_i = alpha).  The expert FFN and
 * combine steps are the same as for top-k.
 *
 * Conventions for every entry point:
 *   - Pointers named in the structs and arguments are DEVICE pointers unless
 *     stated otherwise; arrays are row-major and contiguous.
 *   - The caller owns every buffer, including the workspace sized by
 *     moe_workspace_size().  The library allocates nothing and only
 *     enqueues work on `stream` (a hipStream_t; NULL is the default
 *     stream).  No call synchronises the device or reads device data back
 *     to the host.  The one piece of state kept between calls is a
 *     per-device cache of the compute-unit count (filled on first use,
 *     atomically, with a value that never changes).
 *   - Tuning variables.  The environment variables MOE_ROUTER_SPLIT (0 / 1:
 *     fused or split bf16 router), MOE_TAIL_SPLIT (1..8: cap of the
 *     four-wave GEMM's K split of half-height tiles) and
 *     MOE_GEMM_VARIANT_UP / MOE_GEMM_VARIANT_DOWN (a tile variant id,
 *     used only where valid for the shape) are read at every call.  The
 *     first two change the workspace layout, so they are part of the
 *     workspace contract: keep them unchanged between moe_workspace_size()
 *     and the calls that use that workspace (a call whose workspace is then
 *     too small returns MOE_ERR_WORKSPACE).  Unset, every choice is a
 *     function of the descriptor and the device.
 *   - Arguments are validated on the host before any HIP call; a failed
 *     check returns a negative moe_status and enqueues nothing.  A failed
 *     kernel launch returns MOE_ERR_HIP.  T == 0 is valid: once the
 *     descriptor passes its checks the call returns MOE_OK, enqueues
 *     nothing and does not look at the pointers.  Non-finite inputs are not
 *     checked.
 *   - Calls on distinct streams with distinct workspaces may run
 *     concurrently.
 *   - The residual is not applied: a token whose every assignment
 *     overflowed capacity gets y = 0 exactly, so the caller's x + y passes
 *     it through unchanged.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, k out of range */
    MOE_ERR_UNSUPPORTED = -2, /* shape or dtype this library cannot run */
    MOE_ERR_WORKSPACE = -3,   /* workspace missing or too small */
    MOE_ERR_HIP = -4,         /* a HIP launch failed */
    MOE_ERR_SCRATCH = -5      /* moe_forward_noalloc: the shape needs more
                                 than MOE_NOALLOC_SCRATCH_BYTES of scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
    MOE_ROUTE_TOPK = 0,          /* tokens choose k experts (default) */
    MOE_ROUTE_EXPERT_CHOICE = 1  /* experts choose C tokens */
} moe_routing_mode;

typedef enum {
    MOE_ACT_GELU = 0,    /* h = GELU(W1 x + b1), exact erf form */
    MOE_ACT_SILU = 1,    /* h = SiLU(W1 x + b1), SiLU(z) = z / (1 + e^-z) */
    MOE_ACT_SWIGLU = 2   /* h = SiLU(W1 x + b1) * (W3 x + b3) */
} moe_activation;

/* Layer shape, host struct passed by pointer.
 *   T         tokens (>= 0)
 *   d         model width; multiple of 64
 *   E         routed experts, 1 <= E <= 256
 *   k         experts per token, 1 <= k <= min(E, 64); must equal E for
 *             expert choice
 *   d_ff      expert hidden width; multiple of 64
 *   n_shared  0 or 1 always-on shared expert (weight 1)
 *   dtype     MOE_F32 or MOE_BF16 for x, all weight matrices, the expert
 *             Linear biases and y (arithmetic accumulates in fp32)
 *   capacity  top-k: -1 = no limit, else C >= 0 assignments kept per
 *             expert (see moe_capacity); expert choice: tokens picked per
 *             expert, 0 <= C <= T (required)
 *   aux_alpha coefficient of L_aux (0.01 is the pages' usual value)
 *   routing   a moe_routing_mode
 *   expert_fp8 0: w1, w2, ws1, ws2 are in dtype; 1: they are OCP FP8 E4M3
 *             bytes with fp32 per-output-channel scales (moe_weights
 *             *_scale), a weight being e4m3(byte) * scale[row].  Needs
 *             dtype MOE_BF16 and d, d_ff multiples of 1024; activations,
 *             biases and y stay bf16.  The pages quote FP8 serving of the
 *             Mixtral layer ("MoE inference with vLLM"; "AI-Research-
 *             SKILLs MoE training guide", sec. 9); its target is the
 *             weight-streaming decode shape, whose bytes it halves.
 *   activation a moe_activation (applies to routed and shared experts);
 *             MOE_ACT_SWIGLU needs d_ff a multiple of 128 for bf16 */
typedef struct moe_desc {
    int32_t T, d, E, k, d_ff;
    int32_t n_shared;
    int32_t dtype;
    int32_t capacity;
    float aux_alpha;
    int32_t routing;
    int32_t expert_fp8;
    int32_t activation;
} moe_desc;

/* Weights: caller-owned, read-only device buffers; NULL = absent.
 *   w_router    [E][d]        dtype                 (required)
 *   b_router    [E]           fp32, ADDED to logits (nn.Linear bias, or a
 *                             fixed per-expert skew)
 *   expert_bias [E]           fp32, SUBTRACTED from logits (aux-loss-free
 *                             balancing); enters softmax, selection and
 *                             weights
 *   w1, b1      [E][d_ff][d], [E][d_ff]   dtype (w1 required)
 *   w2, b2      [E][d][d_ff], [E][d]      dtype (w2 required)
 *   ws1..bs2    shared expert, same shapes without the E axis; ws1/ws2
 *               required iff n_shared == 1
 *   w1_scale    [E][d_ff] fp32, w2_scale [E][d], ws1_scale [d_ff],
 *   ws2_scale   [d]: per-output-channel scales of FP8 expert matrices
 *               (required iff expert_fp8, for the matrices present)
 *   w3, b3      [E][d_ff][d], [E][d_ff]  SwiGLU up projection (w3
 *               required iff activation == MOE_ACT_SWIGLU); ws3, bs3 the
 *               shared expert's; w3_scale [E][d_ff], ws3_scale [d_ff] for
 *               FP8.  W1 is then the gate projection. */
typedef struct moe_weights {
    const void *w_router;
    const float *b_router;
    const float *expert_bias;
    const void *w1, *b1;
    const void *w2, *b2;
    const void *ws1, *bs1, *ws2, *bs2;
    const float *w1_scale, *w2_scale, *ws1_scale, *ws2_scale;
    const void *w3, *b3, *ws3, *bs3;
    const float *w3_scale, *ws3_scale;
} moe_weights;

/* Routing results and statistics: caller-owned device buffers.
 *   topk_idx   [T][k] int32  selected experts, descending probability,
 *                            ties to the lower index
 *   topk_w     [T][k] fp32   renormalised weights (sum 1 per token)
 *   counts     [E]    int32  assignments per expert, before capacity
 *   kept       [E]    int32  min(counts, C)
 *   offsets    [E+1]  int32  exclusive prefix sum of kept
 *   slot_token [T*k]  int32  token of each expert-sorted slot; slots at
 *                            and beyond offsets[E] hold -1 (expert
 *                            choice: [E*C], every slot used; may be NULL
 *                            when E*C == 0)
 *   slot_of    [T][k] int32  slot of each assignment, -1 if it overflowed
 *   f, p       [E]    fp32   f_i = counts_i/(T k), p_i = mean_t p[t,i]
 *   l_aux      [1]    fp32   alpha * E * sum_i f_i p_i
 *   monitor    [6]    fp32   optional (NULL = not computed) router and load
 *                            monitors, in this order:
 *                            z-loss = mean_t (logsumexp_e logit[t,e])^2
 *                            ("AI-Research-SKILLs MoE training guide",
 *                            sec. 4.3), routing entropy in bits =
 *                            mean_t -sum_e p log2 p ("The expert group
 *                            activated per token", sec. 4.4), load imbalance
 *                            = max count / min count (+inf if an expert is
 *                            empty), utilization = nonempty experts / E,
 *                            drop rate = assignments over capacity / (T k)
 *                            (training guide, sec. 10.1), max share =
 *                            largest count / T ("MoE architecture deep
 *                            dive", sec. 4: collapse above 0.4) */
typedef struct moe_routing {
    int32_t *topk_idx;
    float *topk_w;
    int32_t *counts, *kept, *offsets;
    int32_t *slot_token, *slot_of;
    float *f, *p, *l_aux;
    float *monitor;
} moe_routing;

/* Host.  floor((double)T / E * cf): the capacity formula of "MoE
 * architecture deep dive", sec. 2.3.  Returns -1 if cf < 0 (no limit) and
 * MOE_ERR_INVALID_ARG if T < 0 or E < 1. */
int32_t moe_capacity(int32_t T, int32_t E, double cf);

/* Host.  Bytes of workspace the calls below need for this shape, or 0 if
 * the descriptor is invalid; a function of the descriptor alone (and of the
 * MOE_ROUTER_SPLIT and MOE_TAIL_SPLIT tuning variables, when set; a call
 * whose workspace is then too small returns MOE_ERR_WORKSPACE).  One
 * workspace serves every entry point;
 * moe_router_topk writes router partial sums into it that moe_permute reads,
 * and moe_grouped_ffn writes the expert outputs that moe_combine reads, so
 * run a sequence of calls with one workspace. */
size_t moe_workspace_size(const moe_desc *desc);

/* Host.  The grouped-GEMM kernel variant moe_ffn_up (up != 0) or
 * moe_ffn_down would run for this descriptor on the current device (an
 * internal id, for diagnostics and benchmark reports), or a negative
 * status if the descriptor is invalid.  Depends on the descriptor, the
 * device's CU count and the MOE_GEMM_VARIANT_UP / _DOWN tuning variables. */
int moe_gemm_variant(const moe_desc *desc, int up);

/* Host.  Number of K ranges S the four-wave 256-row grouped GEMM splits
 * each half-height (last <= 128 rows of a group) tile into for moe_ffn_up
 * (up != 0) or moe_ffn_down: 1 when there is no split or another variant
 * runs, else 2..8 with (K / 64) divisible by 2 S, so every unit covers a
 * whole number of 64-deep stage pairs.  A negative status if the
 * descriptor is invalid.  For diagnostics and tests. */
int moe_gemm_tail_split(const moe_desc *desc, int up);

/* Router GEMM with bias, softmax, top-k and renormalisation (layer steps
 * 1-2); bf16 layers run it as one kernel or, for deep or few-token shapes,
 * as partial logits over depth ranges (fp32, in the workspace) followed by
 * the routing kernel.  Reads x [T][d] and the router weights; writes
 * r->topk_idx, r->topk_w and per-token-tile probability column sums into
 * the workspace (consumed by moe_permute for p_i).  Expert choice: writes
 * topk_idx = e and topk_w = p[t,e] for all E experts, sets every entry of
 * r->slot_of (required) to -1, and writes the logits, transposed to
 * [E][T], into the workspace for moe_permute.  Top-k: also writes each
 * 32-token tile's count of picks per expert into the workspace. */
int moe_router_topk(const moe_desc *desc, const void *x,
                    const moe_weights *w, moe_routing *r, void *ws,
                    size_t ws_bytes, void *stream);

/* Counts, capacity, stable dispatch and statistics (layer steps 3 and 6).
 * Reads r->topk_idx and what moe_router_topk left in the workspace (the
 * probability partial sums and each 32-token tile's expert counts); writes
 * counts, kept, offsets, slot_token, slot_of, f, p, l_aux and, if
 * r->monitor is not NULL, the six monitors.  Expert choice: each expert's
 * top-C selection over the workspace logits replaces the capacity cut
 * (r->topk_idx is not read), and only the picked entries of slot_of are
 * written, over the -1 that moe_router_topk left there. */
int moe_permute(const moe_desc *desc, moe_routing *r, void *ws,
                size_t ws_bytes, void *stream);

/* moe_router_topk followed by moe_permute (layer steps 1-3 and 6), with
 * the same arguments, checks and results.  Where a decode-sized step
 * allows (bf16, top-k routing, E <= 32, T <= 32, T*k <= 256) the routing
 * and the dispatch run in one workgroup after the partial logits: two
 * kernel launches instead of three, with results equal to the two calls'
 * bit for bit.  The pages give fewer kernel launches as the reason for
 * fused MoE kernels in serving ("MoE inference with vLLM";
 * "AI-Research-SKILLs MoE training guide", sec. 9.2). */
int moe_route_dispatch(const moe_desc *desc, const void *x,
                       const moe_weights *w, moe_routing *r, void *ws,
                       size_t ws_bytes, void *stream);

/* Grouped expert FFNs (layer step 4): for every kept slot s of expert e,
 *   Yp[s] = W2_e GELU(W1_e x[slot_token[s]] + b1_e) + b2_e,
 * and, with a shared expert, Yp[R + t] = Shared(x[t]) for every token,
 * where R = T*k routed slots (expert choice: R = E*C).  Yp is written
 * into the workspace (dtype, [R + n_shared*T][d]); the hidden activations
 * are rounded to dtype between the two GEMMs.  Equivalent to moe_ffn_up
 * followed by moe_ffn_down. */
int moe_grouped_ffn(const moe_desc *desc, const void *x,
                    const moe_weights *w, const moe_routing *r, void *ws,
                    size_t ws_bytes, void *stream);

/* First half of moe_grouped_ffn: H[s] = GELU(W1_e x[token(s)] + b1_e)
 * (or the SiLU / SwiGLU form of desc->activation) into the workspace (one
 * kernel launch). */
int moe_ffn_up(const moe_desc *desc, const void *x, const moe_weights *w,
               const moe_routing *r, void *ws, size_t ws_bytes,
               void *stream);

/* Second half of moe_grouped_ffn: Yp[s] = W2_e H[s] + b2_e (one launch). */
int moe_ffn_down(const moe_desc *desc, const moe_weights *w,
                 const moe_routing *r, void *ws, size_t ws_bytes,
                 void *stream);

/* Weighted combine (layer step 5): y[t] = sum over kept j, in j order, of
 * topk_w[t,j] * Yp[slot_of[t,j]], plus Yp[R + t] with a shared expert;
 * fp32 accumulation, one rounding to dtype.  y is [T][d], dtype. */
int moe_combine(const moe_desc *desc, const moe_routing *r, void *y,
                void *ws, size_t ws_bytes, void *stream);

/* The whole forward: moe_route_dispatch (= moe_router_topk and
 * moe_permute), moe_grouped_ffn and moe_combine on one stream. */
int moe_forward(const moe_desc *desc, const void *x, const moe_weights *w,
                moe_routing *r, void *y, void *ws, size_t ws_bytes,
                void *stream);

/* Bytes of the static device scratch moe_forward_noalloc uses (16 MiB per
 * GPU the library runs on, held until the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)

/* moe_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments and results as
 * moe_forward, minus ws / ws_bytes: the scratch (router partials, dispatch
 * histograms, hidden activations, expert outputs) lives in a file-scope
 * device array of MOE_NOALLOC_SCRATCH_BYTES per GPU, whose address is
 * looked up once per device on the first call there.  Allocates nothing:
 * no hipMalloc, hipFree or allocating library call.  Returns
 * MOE_ERR_SCRATCH, enqueuing nothing, when moe_workspace_size(desc)
 * exceeds the buffer (decode-sized layers fit: the Mixtral-shaped T = 32
 * step needs 2.4 MB).  No part of the scratch has to start at zero.  Every
 * call on one GPU shares that GPU's buffer, which keeps the last call's
 * contents: calls that overlap on one GPU (distinct streams, or host
 * threads) race and must be serialised by the caller. */
int moe_forward_noalloc(const moe_desc *desc, const void *x,
                        const moe_weights *w, moe_routing *r, void *y,
                        void *stream);

/* Balancing-bias step (layer step 7), in place on fp32 state:
 * bias[e] = bias[e] + gamma * sign(counts[e] - target), sign(0) = 0, one
 * fp32 add.  Apply after a forward; it affects the next call. */
int moe_bias_update(int32_t E, const int32_t *counts, float target,
                    float gamma, float *expert_bias, void *stream);

/* Host.  Static English text of a moe_status value. */
const char *moe_status_string(int status);

/* Host.  Library version string. */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
