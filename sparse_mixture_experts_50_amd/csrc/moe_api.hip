// Host side of the C ABI declared in include/moe.h: argument checks,
// workspace layout, kernel-variant choice and launches.  Every check runs
// before the first HIP call, so a rejected call enqueues nothing.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct WsLayout {
    size_t p_part, zh_part, blk, scores, rpart, tpart, h, yp, total;
    int n_rtiles, n_chunks;
    size_t rows;
};

int elem_bytes(int dtype) { return dtype == MOE_F32 ? 4 : 2; }

bool expert_choice(const moe_desc *d) {
    return d->routing == MOE_ROUTE_EXPERT_CHOICE;
}

// Routed expert rows: T*k assignments, or E*C picks for expert choice.
long long routed_rows(const moe_desc *d) {
    return expert_choice(d) ? (long long)d->E * d->capacity
                            : (long long)d->T * d->k;
}

int check_desc(const moe_desc *d) {
    if (!d) return MOE_ERR_INVALID_ARG;
    if (d->T < 0 || d->E < 1 || d->k < 1 || d->k > d->E || d->d < 1 ||
        d->d_ff < 1 || d->capacity < -1 ||
        (d->n_shared != 0 && d->n_shared != 1) ||
        (d->routing != MOE_ROUTE_TOPK && !expert_choice(d)))
        return MOE_ERR_INVALID_ARG;
    if (expert_choice(d) &&
        (d->k != d->E || d->capacity < 0 || d->capacity > d->T))
        return MOE_ERR_INVALID_ARG;
    if (d->expert_fp8 != 0 && d->expert_fp8 != 1) return MOE_ERR_INVALID_ARG;
    if (d->activation < MOE_ACT_GELU || d->activation > MOE_ACT_SWIGLU)
        return MOE_ERR_INVALID_ARG;
    // the gated bf16 up GEMM runs on tiles whose waves cover whole 64-column
    // chunks of the 2*d_ff virtual panel (256-column tiles, 64-column
    // streaming units)
    if (d->activation == MOE_ACT_SWIGLU && d->dtype == MOE_BF16 &&
        d->d_ff % 128 != 0)
        return MOE_ERR_UNSUPPORTED;
    if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    // FP8 weights run on the weight-streaming kernel: its four K quarters
    // hold whole 256-deep load batches
    if (d->expert_fp8 && (d->dtype != MOE_BF16 || d->d % 1024 != 0 ||
                          d->d_ff % 1024 != 0))
        return MOE_ERR_UNSUPPORTED;
    if (d->E > MOE_MAX_E || (!expert_choice(d) && d->k > 64))
        return MOE_ERR_UNSUPPORTED;
    if (d->d % 64 != 0 || d->d_ff % 64 != 0) return MOE_ERR_UNSUPPORTED;
    // 32-bit element offsets inside the kernels
    if ((double)d->T * d->k >= 2147483647.0) return MOE_ERR_UNSUPPORTED;
    const double rows = (double)routed_rows(d) + (double)d->n_shared * d->T;
    if (rows * d->d_ff >= 2147483647.0 || rows * d->d >= 2147483647.0 ||
        2.0 * d->d * d->d_ff >= 2147483647.0)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// Expected row tiles of one routed group: E[ceil(X / bm)] with the group
// size X ~ Normal(avg, avg (1 - 1/E)) (a binomial share of the T k
// assignments), i.e. the sum over j of P(X > j bm); capped at the capacity.
// Expert-choice groups hold exactly C rows.  full / half: the same split
// for a kernel whose last <= 128 rows of a group take a half tile.
struct TileCount {
    double tiles, full, half;
};
TileCount group_tiles(const moe_desc *d, int bm) {
    const double avg = (double)routed_rows(d) / d->E;
    TileCount c = {0.0, 0.0, 0.0};
    if (expert_choice(d) || avg <= 0.0) {
        c.tiles = ceil(avg / bm);
        c.full = floor(avg / bm);
        c.half = (avg - c.full * bm) > 0 ? 1.0 : 0.0;
        if (avg - c.full * bm > 128) {
            c.full += 1.0;
            c.half = 0.0;
        }
        return c;
    }
    const double sd = sqrt(avg * (1.0 - 1.0 / d->E));
    const double cap = d->capacity >= 0 ? (double)d->capacity : 1e30;
    auto above = [&](double x) {      // P(X > x), 0 at or above the cap
        if (x >= cap) return 0.0;
        return 0.5 * erfc((x - avg) / (sd * sqrt(2.0)));
    };
    for (int j = 0; j * (double)bm < avg + 8.0 * sd + bm && j < 1 << 20; ++j) {
        const double pj = above(j * (double)bm);
        c.tiles += pj;
        // the tile starting at j bm is half height when the group ends
        // within its first 128 rows
        const double ph = pj - above(j * (double)bm + 128.0);
        c.half += ph;
        c.full += pj - ph;
    }
    return c;
}

int variant_override(bool up, const moe_desc *d, int N);

// The four-wave 256-row kernels (16x16x32 and 32x32x16 MFMA forms), the
// ones with split tails.
bool w4_256(int v) {
    return v == GEMM_BF16_W4_256x256 || v == GEMM_BF16_W4X_256x256;
}
// Any four-wave kernel (256-row or every tile 128 rows, 256 or 192
// columns).
bool w4_any(int v) {
    return w4_256(v) || v == GEMM_BF16_W4_128x256 ||
           v == GEMM_BF16_W4X_128x256 || v == GEMM_BF16_W4_256x192;
}
bool w4_fits(const moe_desc *d, bool up);

// Whether the four-wave 256-row kernel may run this GEMM: forced by the
// tuning variable, or inside the range where pick_variant weighs it
// against the eight-wave kernels (a function of the descriptor only; the
// device-dependent cost comparison may still pick another kernel).
bool w4_256_possible(const moe_desc *d, bool up, int N) {
    const int forced = variant_override(up, d, N);
    if (forced >= 0) return w4_256(forced);
    const double avg = (double)routed_rows(d) / d->E;
    const int K = up ? d->d : d->d_ff;
    const bool small_down = !up && avg > 192.0 && avg <= 384.0;
    return N % 256 == 0 && (avg >= 768.0 || small_down) && K >= 2048 &&
           w4_fits(d, up);
}

// How many K ranges the four-wave 256-row kernel splits each half-height
// tile into (1: none).  When the full tiles fill whole rounds and the half
// tiles would run as a sparse extra round (the Mixtral down GEMM: 512 full
// tiles, two rounds of the 256 CUs, then 64 half tiles), each half tile
// runs as S units over 1/S of K so that the last round fills the CUs; the
// units' fp32 partials are added by the tail reduction.  A function of the
// shape only (sized for 256 CUs), so the workspace size is too.
int tail_split(const moe_desc *d, bool up) {
    if (d->dtype != MOE_BF16 || d->expert_fp8) return 1;
    const int N = up ? (d->activation == MOE_ACT_SWIGLU ? 2 * d->d_ff : d->d_ff)
                     : d->d;
    const int K = up ? d->d : d->d_ff;
    if (N % 256 != 0 || K % 128 != 0 || K < 256) return 1;
    // no split (and no partials in the workspace) where the four-wave
    // 256-row kernel cannot be the pick
    if (!w4_256_possible(d, up, N)) return 1;
    const TileCount g = group_tiles(d, 256);
    const int rem = d->T & 255;
    const double shared_half = (double)d->n_shared * (rem > 0 && rem <= 128);
    const double H = (g.half * d->E + shared_half) * (N / 256);
    if (H < 1.0) return 1;
    int S = (int)floor(256.0 / H);
    if (S > 8) S = 8;
    if (S < 1) S = 1;
    // tuning and test knob: MOE_TAIL_SPLIT=1..8 caps the split (1: none);
    // read here, so the workspace size follows it.  The cap comes first:
    // the unit ranges below must still be whole stage pairs.
    const char *v = getenv("MOE_TAIL_SPLIT");
    if (v && v[0] >= '1' && v[0] <= '8' && v[1] == 0 && S > v[0] - '0')
        S = v[0] - '0';
    // each unit walks KT / S 64-deep stages, two per loop trip
    while (S > 1 && (K / 64) % (2 * S) != 0) --S;
    if (S > 1 && (double)S * (d->E + d->n_shared) * 128.0 * N * 4.0 > 512e6)
        S = 1;
    return S;
}

size_t tail_part_bytes(const moe_desc *d, bool up) {
    const int S = tail_split(d, up);
    if (S < 2) return 0;
    const int N = up ? (d->activation == MOE_ACT_SWIGLU ? 2 * d->d_ff : d->d_ff)
                     : d->d;
    return (size_t)S * (d->E + d->n_shared) * 128 * N * sizeof(float);
}

// The router's logits split depends on the shape only (sized for the
// MI355X's 256 CUs), so the workspace size is a pure function of the
// descriptor.
RouterPlan plan(const moe_desc *d) {
    RouterPlan r = router_plan(d->T, d->d, d->E, 256);
    // tuning and test knob: MOE_ROUTER_SPLIT=0 / 1 forces the fused or the
    // split bf16 router (read here, so the workspace size follows it)
    const char *v = getenv("MOE_ROUTER_SPLIT");
    if (v && (v[0] == '0' || v[0] == '1') && v[1] == 0) r.split = v[0] == '1';
    return r;
}

WsLayout layout(const moe_desc *d) {
    WsLayout L;
    const size_t es = elem_bytes(d->dtype);
    L.n_rtiles = (d->T + MOE_ROUTER_TOKENS - 1) / MOE_ROUTER_TOKENS;
    // a dispatch chunk is a router token tile's assignments (expert
    // choice dispatches by per-expert selection, not by chunks)
    L.n_chunks = expert_choice(d) ? 0 : L.n_rtiles;
    L.rows = (size_t)routed_rows(d) + (size_t)d->n_shared * d->T;
    size_t off = 0;
    L.p_part = off;
    off += align_up((size_t)L.n_rtiles * d->E * sizeof(float));
    L.zh_part = off;
    off += align_up((size_t)L.n_rtiles * 2 * sizeof(float));
    L.blk = off;
    off += align_up((size_t)L.n_chunks * d->E * sizeof(int32_t));
    L.scores = off;       // expert choice: logits transposed, [E][T] fp32
    if (expert_choice(d)) off += align_up((size_t)d->E * d->T * sizeof(float));
    L.rpart = off;        // bf16 router: partial logits, [S][T][E] fp32
    if (d->dtype == MOE_BF16 && plan(d).split)
        off += align_up((size_t)plan(d).S * d->T * d->E * sizeof(float));
    L.tpart = off;        // split tails of the four-wave GEMM: fp32 partials
    {
        const size_t a = tail_part_bytes(d, true), b = tail_part_bytes(d, false);
        off += align_up(a > b ? a : b);
    }
    L.h = off;
    off += align_up(L.rows * d->d_ff * es);
    L.yp = off;
    off += align_up(L.rows * d->d * es);
    L.total = off > 0 ? off : kAlign;
    return L;
}

int check_ws(const moe_desc *d, void *ws, size_t ws_bytes) {
    if (!ws) return MOE_ERR_WORKSPACE;
    if (ws_bytes < layout(d).total) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

char *at(void *ws, size_t off) { return (char *)ws + off; }

int to_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Compute units of the current device (host query, cached per device).
// The cache is the library's one piece of state kept between calls: a
// per-device constant, written with relaxed atomics, so concurrent first
// calls at worst both query the device and store the same value.
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount,
                                  dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Tuning override: MOE_GEMM_VARIANT_UP / MOE_GEMM_VARIANT_DOWN name a
// GemmVariant; it is used only if valid for this dtype and width.
bool gated_up(const moe_desc *d, bool up) {
    return up && d->activation == MOE_ACT_SWIGLU;
}

// Variants whose waves hold whole 64-column chunks of the gated panel.
bool gate_capable(int v) {
    return v != GEMM_BF16_64x64 && v != GEMM_BF16_STREAM_32x64 &&
           v != GEMM_FP8_STREAM_32x64 && v != GEMM_BF16_W4_256x192 &&
           !tall_variant(v);
}

// The four-wave kernel walks K in pairs of 64-deep stages and addresses
// its A operand with 32-bit byte offsets.
bool w4_fits(const moe_desc *d, bool up) {
    const long long K = up ? d->d : d->d_ff;
    const long long rows = up ? d->T : routed_rows(d) + (long long)d->n_shared * d->T;
    return K >= 128 && K % 128 == 0 && rows * K * 2 < (1ll << 32);
}

// The two-block kernel walks K in 32-deep stages, with the same 32-bit A
// offsets.
bool x2_fits(const moe_desc *d, bool up) {
    const long long K = up ? d->d : d->d_ff;
    const long long rows = up ? d->T : routed_rows(d) + (long long)d->n_shared * d->T;
    return K >= 32 && K % 32 == 0 && rows * K * 2 < (1ll << 32);
}

// The weight-ring kernels take K in stages of whole row runs and stage
// the routed slots' token indices in LDS.
bool ring_fits(const moe_desc *d, bool up, int variant) {
    const bool fp8 = variant == GEMM_FP8_RING_16x16 || variant == GEMM_FP8_RING2_16x16;
    const long long K = up ? d->d : d->d_ff;
    if ((K * (fp8 ? 1 : 2)) % ring_cb(variant) != 0) return false;
    return !up || routed_rows(d) <= MOE_RING_MAXTOK;
}

int variant_override(bool up, const moe_desc *d, int N) {
    const char *v = getenv(up ? "MOE_GEMM_VARIANT_UP" : "MOE_GEMM_VARIANT_DOWN");
    if (!v || !*v) return -1;
    const int id = atoi(v);
    if (d->dtype == MOE_F32) return -1;
    if (gated_up(d, up) && !gate_capable(id)) return -1;
    const bool fp8_id = id == GEMM_FP8_STREAM_32x64 ||
                        id == GEMM_FP8_STREAM_64x64 ||
                        id == GEMM_FP8_RING_16x16 || id == GEMM_FP8_RING2_16x16;
    if (ring_variant(id) && !ring_fits(d, up, id)) return -1;
    if (d->expert_fp8) return fp8_id ? id : -1;
    if (id < GEMM_BF16_256x256 || id > GEMM_BF16_TALL_288x224 ||
        id == GEMM_F32_64x64 || fp8_id)
        return -1;
    // the tall-tile kernel takes a ragged last column tile
    if (!tall_variant(id) && N % gemm_variant_info(id).bn != 0) return -1;
    if ((w4_any(id) || tall_variant(id)) && !w4_fits(d, up))
        return -1;
    if (id == GEMM_BF16_X2_128x256 && !x2_fits(d, up)) return -1;
    // the streaming kernels split K in four quarters of whole load batches
    // (4 x 32 deep for 32-column units, 2 x 32 for 64-column ones)
    if (id == GEMM_BF16_STREAM_32x64 && (d->d % 512 != 0 || d->d_ff % 512 != 0))
        return -1;
    if (id == GEMM_BF16_STREAM_64x64 && (d->d % 256 != 0 || d->d_ff % 256 != 0))
        return -1;
    return id;
}

// Expected cost of a grouped GEMM: whole rounds of tiles over the
// persistent grid, each round costing a tile's time, in units of one tile
// row.  A tile streams its 256-column weight panel and runs its prologue
// and epilogue whatever its height: worth about 128 rows for the
// eight-wave kernels and 40 for the four-wave one (measured on the
// Mixtral-shaped GEMMs), whose half-height tiles cost about 0.65 of a full
// one.
double tile_cost(const moe_desc *d, int N, int bm, int slots, double over,
                 bool halves) {
    const TileCount g = group_tiles(d, bm);
    const double shared = (double)d->n_shared * ceil((double)d->T / bm);
    const double per_group = halves ? g.full + 0.65 * g.half : g.tiles;
    const double tiles = (per_group * d->E + shared) * (N / 256);
    // an expected few percent of a round past a whole number (a rare
    // group just over a tile boundary) is not charged a whole round
    return ceil(tiles / slots - 0.05) * (bm + over);
}

// Variant choice, from sweeps of group size, depth and width on MI355X:
// streaming up to 32 rows per expert; 32-row tiles to 48; the four-wave
// kernel with 128-row tiles to 128 (one or two half tiles per group; the
// eight-wave 256-row kernel where K does not suit it); the eight-wave
// 256-row kernel to 192; above that the cheapest of 256- and 320-row
// eight-wave tiles and the four-wave 256-row kernel.  The last only for
// K >= 2048 (shallower GEMMs are dominated by its one-wave-per-SIMD
// epilogue) and groups of >= 768 rows: then the row tiles of one expert
// run side by side and share each weight panel through L2; with one or
// two tiles per expert (DeepSeek-shaped layers, multi-GB expert weights)
// the tiles stream distinct weights and the taller 320-row tile, with more
// FLOPs per weight byte, is faster; for such an up projection (K >= 2048)
// the four-wave 320 x 192 tile is faster still.
int pick_variant(const moe_desc *d, int N, bool up) {
    if (d->dtype == MOE_F32) return GEMM_F32_64x64;
    const double avg = (double)routed_rows(d) / d->E;
    // The weight ring reads each weight byte once per 16-row chunk of a
    // group, so it is used where groups are expected to fit one chunk
    // (and the shared expert too), in its two-blocks-per-CU form.  Measured
    // on the Mixtral-shaped decode GEMMs it is 8-18 % faster than the
    // register-streaming kernel, except for the gated up projection (whose
    // units read the W1 and W3 panels at the same offsets), 8 % slower.
    const bool ring_rows = avg <= 12.0 && (d->n_shared == 0 || d->T <= 16);
    if (d->expert_fp8)
        return ring_rows && !gated_up(d, up) && ring_fits(d, up, GEMM_FP8_RING2_16x16)
                   ? GEMM_FP8_RING2_16x16 : GEMM_FP8_STREAM_64x64;
    if (N % 256 != 0) return GEMM_BF16_64x64;
    const int K = up ? d->d : d->d_ff;
    // the streaming kernel splits K in four quarters of whole 64-deep
    // load batches; 64-column units re-read the token rows half as often
    // as 32-column ones
    if (avg <= 32.0 && d->d % 256 == 0 && d->d_ff % 256 == 0) {
        if (ring_rows && !gated_up(d, up) && ring_fits(d, up, GEMM_BF16_RING2_16x16))
            return GEMM_BF16_RING2_16x16;
        return GEMM_BF16_STREAM_64x64;
    }
    if (avg <= 48.0) return GEMM_BF16_32x256;
    // A shallow up projection (K <= 1536) spends much of each tile in its
    // epilogue, which is latency-bound: kernels with two or more waves per
    // SIMD hide it.  Under a capacity limit of at most 192 rows the groups
    // are small and uneven (the limit exists because routing is skewed:
    // the Switch-shaped layer keeps 0-160 rows per expert, 62 on average)
    // and 32-row tiles waste the least (Switch up GEMM 70 us against 77
    // for 128-row four-wave tiles); without one, from ~100 rows per expert
    // the eight-wave 256-row kernel (6-20 % faster on five swept shapes).
    if (up && K <= 1536) {
        if (expert_choice(d) == false && d->capacity >= 0 && d->capacity <= 192 &&
            K <= 1024)
            return GEMM_BF16_32x256;
        if (avg > 96.0 && avg <= 192.0) return GEMM_BF16_DMA64_256x256;
    }
    // Expert choice with 129..256 rows per expert, no shared expert, K >=
    // 2048 and N a multiple of 192: every group is one full (or trimmed)
    // tile of the four-wave kernel, so E (N / 256) tiles fill only part of
    // the CUs' one round; with 192-column tiles, if E (N / 192) still fit
    // one round, each tile has three quarters of the work (the
    // Expert-Choice-shaped down GEMM: 64 x 4 = 256 tiles instead of 192,
    // layer 0.326 -> 0.318 ms).  Not for groups of up to 128 rows: the
    // Switch-shaped down GEMM (0-160 rows, mostly half tiles) ran 7 us
    // slower than on 128 x 256 tiles.
    if (!up && !gated_up(d, up) && N % 192 == 0 && K >= 2048 &&
        expert_choice(d) && d->capacity > 128 && d->capacity <= 256 &&
        d->n_shared == 0 && w4_fits(d, up) &&
        (long long)d->E * (N / 192) <= device_cus())
        return GEMM_BF16_W4_256x192;
    // A down projection (K >= 2048) under a top-k capacity limit of 129..320
    // rows: every group is one tall row tile, whose weight panel then
    // streams with the non-temporal hint (the Switch-shaped down GEMM, 0..160
    // rows per expert: layer 0.187 -> 0.177 ms against 128-row four-wave
    // tiles; its up GEMM, K = 768, ran 86 us against 70 on 32-row tiles).
    // Under a limit of at most 128 rows the 128-row four-wave tiles below
    // stay (not measured against this).
    if (!up && !expert_choice(d) && d->capacity > 128 && d->capacity <= 320 &&
        K >= 2048 && w4_fits(d, up))
        return GEMM_BF16_TALL_320x192;
    if (avg <= 128.0)
        return w4_fits(d, up) ? GEMM_BF16_W4_128x256 : GEMM_BF16_DMA64_256x256;
    if (avg <= 192.0) return GEMM_BF16_DMA64_256x256;
    // One- and two-tile groups (up to 384 rows) of a down projection with
    // K >= 2048: the four-wave kernel runs a group of 257..384 rows as two
    // tiles of 160 or 192 rows side by side on one weight panel.  On the
    // DeepSeek-shaped down GEMM (groups of 256 +- 17 rows, K = 2048) it is
    // 0.2 ms faster than the eight-wave 320-row kernel; on the up GEMM
    // (K = 7168) the two are within 2 %.
    // DeepSeek-shaped down projection (193..320 rows per expert on average,
    // K and N >= 2048): the tall kernel, every group one row tile with
    // non-temporal weights (256-column tiles up to 256 rows, 320 x 192
    // above): layer 4.955 -> 4.926 ms against the four-wave kernel below.
    if (!up && avg > 192.0 && avg <= 320.0 && K >= 2048 && N >= 2048 &&
        w4_fits(d, up))
        return GEMM_BF16_TALL_320x192;
    if (!up && avg <= 384.0 && K >= 2048 && w4_fits(d, up))
        return GEMM_BF16_W4_256x256;
    // Ungated up projections with K >= 2048 whose groups average 193..320
    // rows (DeepSeek-shaped: 256 +- 17): 320 x 192 tiles hold nearly every
    // routed group in one row tile, whose weight panel then streams with the
    // non-temporal hint and leaves the group's gathered rows in L2 (up GEMM
    // 2.34 -> 2.21 ms against the 320-row eight-wave kernel, layer 5.02 ->
    // 4.97 ms).  Not for down projections (288 x 224 and 320 x 192 tiles both
    // measured slower there than the four-wave kernel) or shallow K (the
    // Expert-Choice up GEMM, K = 768: 129-137 us against 126-128).
    if (up && !gated_up(d, up) && K >= 2048 && avg > 192.0 && avg <= 320.0 &&
        w4_fits(d, up))
        return GEMM_BF16_TALL_320x192;
    const int slots = device_cus();
    int best = GEMM_BF16_DMA64_256x256;
    double cost = tile_cost(d, N, 256, slots, 128.0, false);
    const double c320 = tile_cost(d, N, 320, slots, 128.0, false);
    if (c320 < cost) {
        best = GEMM_BF16_DMA64_320x256;
        cost = c320;
    }
    if (w4_fits(d, up) && K >= 2048 && avg >= 768.0 &&
        tile_cost(d, N, 256, slots, 40.0, true) < cost)
        best = GEMM_BF16_W4_256x256;
    return best;
}

int gemm_grid(const moe_desc *d, int variant, int N) {
    const GemmVariantInfo vi = gemm_variant_info(variant);
    if (ring_variant(variant)) return device_cus() * ring_occupancy(variant);
    if (stream_variant(variant)) {              // persistent over units
        const long long units = (long long)(d->E + d->n_shared) * (N / vi.bn);
        const long long slots = (long long)device_cus() * 2;
        return (int)(units < slots ? units : slots);
    }
    const long long mtiles = (routed_rows(d) + vi.bm - 1) / vi.bm +
                             d->E +
                             (long long)d->n_shared * ((d->T + vi.bm - 1) / vi.bm);
    const long long ub = mtiles * ((N + vi.bn - 1) / vi.bn);
    int per_cu = 1;
    if (vi.lds_bytes == 0) per_cu = 4;
    else if (vi.lds_bytes <= 80 * 1024) per_cu = 2;
    long long g = (long long)device_cus() * per_cu;
    if (ub < g) g = ub;
    g = (g + 7) / 8 * 8;
    return (int)(g < 8 ? 8 : g);
}

int check_weights_router(const moe_weights *w) {
    if (!w || !w->w_router) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int check_weights_ffn(const moe_desc *d, const moe_weights *w) {
    if (!w || !w->w1 || !w->w2) return MOE_ERR_INVALID_ARG;
    if (d->n_shared && (!w->ws1 || !w->ws2)) return MOE_ERR_INVALID_ARG;
    if (d->expert_fp8 && (!w->w1_scale || !w->w2_scale ||
                          (d->n_shared && (!w->ws1_scale || !w->ws2_scale))))
        return MOE_ERR_INVALID_ARG;
    if (d->activation == MOE_ACT_SWIGLU) {
        if (!w->w3 || (d->n_shared && !w->ws3)) return MOE_ERR_INVALID_ARG;
        if (d->expert_fp8 &&
            (!w->w3_scale || (d->n_shared && !w->ws3_scale)))
            return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

int check_routing_router(const moe_desc *d, const moe_routing *r) {
    if (!r || !r->topk_idx || !r->topk_w) return MOE_ERR_INVALID_ARG;
    if (expert_choice(d) && !r->slot_of) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// slot_token holds routed_rows() entries, so with no routed rows (expert
// choice with C = 0) it may be NULL.
int check_routing_permute(const moe_desc *d, const moe_routing *r) {
    if (!r || (!r->topk_idx && !expert_choice(d)) || !r->counts ||
        !r->kept || !r->offsets || (!r->slot_token && routed_rows(d) > 0) ||
        !r->slot_of || !r->f || !r->p || !r->l_aux)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int check_routing_ffn(const moe_desc *d, const moe_routing *r) {
    if (!r || !r->offsets || (!r->slot_token && routed_rows(d) > 0))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

int check_routing_combine(const moe_routing *r) {
    if (!r || !r->slot_of || !r->topk_w) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

RouterParams router_params(const moe_desc *desc, const void *x,
                           const moe_weights *w, moe_routing *r, void *ws) {
    const WsLayout L = layout(desc);
    RouterParams p;
    p.x = x;
    p.wr = w->w_router;
    p.add = w->b_router;
    p.sub = w->expert_bias;
    p.topk_idx = r->topk_idx;
    p.topk_w = r->topk_w;
    p.p_part = (float *)at(ws, L.p_part);
    p.zh_part = (float *)at(ws, L.zh_part);
    p.scores = expert_choice(desc) ? (float *)at(ws, L.scores) : nullptr;
    p.slot_of = r->slot_of;
    p.blk = (int32_t *)at(ws, L.blk);
    const RouterPlan rp = plan(desc);
    p.part = (float *)at(ws, L.rpart);
    p.S = rp.split ? rp.S : 0;
    p.kc = rp.kc;
    p.T = desc->T;
    p.d = desc->d;
    p.E = desc->E;
    p.k = desc->k;
    return p;
}

PermuteParams permute_params(const moe_desc *desc, moe_routing *r, void *ws) {
    const WsLayout L = layout(desc);
    PermuteParams p;
    p.topk_idx = r->topk_idx;
    p.p_part = (const float *)at(ws, L.p_part);
    p.zh_part = (const float *)at(ws, L.zh_part);
    p.blk = (int32_t *)at(ws, L.blk);
    p.scores = expert_choice(desc) ? (const float *)at(ws, L.scores) : nullptr;
    p.counts = r->counts;
    p.kept = r->kept;
    p.offsets = r->offsets;
    p.slot_token = r->slot_token;
    p.slot_of = r->slot_of;
    p.f = r->f;
    p.p = r->p;
    p.l_aux = r->l_aux;
    p.monitor = r->monitor;
    p.T = desc->T;
    p.E = desc->E;
    p.k = desc->k;
    p.capacity = desc->capacity;
    p.n_rtiles = L.n_rtiles;
    p.n_chunks = L.n_chunks;
    p.alpha = desc->aux_alpha;
    return p;
}

// moe_router_topk then moe_permute, as one launch where a decode-sized
// step allows it (the same results either way).  Arguments checked by the
// caller.
int route_and_permute(const moe_desc *desc, const void *x,
                      const moe_weights *w, moe_routing *r, void *ws,
                      size_t ws_bytes, void *stream) {
    const RouterParams rp = router_params(desc, x, w, r, ws);
    if (desc->dtype == MOE_BF16 && !expert_choice(desc) &&
        route_permute_small_ok(rp))
        return to_status(launch_route_permute_small(
            rp, permute_params(desc, r, ws), (hipStream_t)stream));
    int st = moe_router_topk(desc, x, w, r, ws, ws_bytes, stream);
    if (st != MOE_OK) return st;
    return moe_permute(desc, r, ws, ws_bytes, stream);
}

GemmParams gemm_params(const moe_desc *d, const moe_weights *w,
                       const moe_routing *r, bool up, const void *x, void *ws) {
    const WsLayout L = layout(d);
    GemmParams p = {};
    p.slot_token = r->slot_token;
    p.offsets = r->offsets;
    p.E = d->E;
    p.n_shared = d->n_shared;
    p.T = d->T;
    p.shared_base = (int)routed_rows(d);
    if (up) {
        p.A = x;
        p.W = w->w1;
        p.bias = w->b1;
        p.Ws = w->ws1;
        p.bias_s = w->bs1;
        p.out = at(ws, L.h);
        p.scale = w->w1_scale;
        p.scale_s = w->ws1_scale;
        p.act = d->activation;
        p.gated = d->activation == MOE_ACT_SWIGLU;
        if (p.gated) {
            p.W3 = w->w3;
            p.bias3 = w->b3;
            p.Ws3 = w->ws3;
            p.bias_s3 = w->bs3;
            p.scale3 = w->w3_scale;
            p.scale_s3 = w->ws3_scale;
        }
        // a gated up GEMM has 2*d_ff (virtual) columns and d_ff outputs
        p.N = p.gated ? 2 * d->d_ff : d->d_ff;
        p.ldo = d->d_ff;
        p.K = d->d;
    } else {
        p.A = at(ws, L.h);
        p.W = w->w2;
        p.bias = w->b2;
        p.Ws = w->ws2;
        p.bias_s = w->bs2;
        p.out = at(ws, L.yp);
        p.scale = w->w2_scale;
        p.scale_s = w->ws2_scale;
        p.N = d->d;
        p.ldo = d->d;
        p.K = d->d_ff;
    }
    return p;
}

int run_gemm(const moe_desc *d, const moe_weights *w, const moe_routing *r,
             bool up, const void *x, void *ws, hipStream_t s) {
    const GemmParams p = gemm_params(d, w, r, up, x, ws);
    int variant = variant_override(up, d, p.N);
    if (variant < 0) variant = pick_variant(d, p.N, up);
    // check_desc keeps a gated N = 2*d_ff a multiple of 256, so pick_variant
    // never lands on a variant that cannot pair gate and up columns
    if (gated_up(d, up) && !gate_capable(variant)) return MOE_ERR_UNSUPPORTED;
    const int grid = gemm_grid(d, variant, p.N);
    if (w4_256(variant)) {
        GemmParams q = p;
        q.tail_split = tail_split(d, up);
        // a split unit covers KT / S stages in whole stage pairs; any other
        // split would drop or repeat part of K
        if (q.tail_split > 1 && (q.K / 64) % (2 * q.tail_split) != 0)
            return MOE_ERR_UNSUPPORTED;
        if (q.tail_split > 1) q.part = (float *)at(ws, layout(d).tpart);
        return to_status(launch_gemm(q, variant, up, grid, s));
    }
    return to_status(launch_gemm(p, variant, up, grid, s));
}

// ---------------------------------------------------------------------
// Static scratch of moe_forward_noalloc: a file-scope device array that
// each GPU the library runs on holds until the process ends.  In host code
// `scratch` is only a host-side stand-in for the symbol: its device
// address on the current device comes from hipGetSymbolAddress, once per
// device, and only that address is handed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

// Device address of `scratch` on the current device (nullptr and the
// failing status on error).  The lookup runs once per device; concurrent
// first calls may both look it up and store the same address.
void *static_scratch(int *status) {
    static std::atomic<void *> addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        *status = MOE_ERR_HIP;
        return nullptr;
    }
    void *ptr = addr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess ||
            !ptr) {
            *status = MOE_ERR_HIP;
            return nullptr;
        }
        addr[dev].store(ptr, std::memory_order_release);
    }
    *status = MOE_OK;
    return ptr;
}

}  // namespace

extern "C" {

int32_t moe_capacity(int32_t T, int32_t E, double cf) {
    if (T < 0 || E < 1) return MOE_ERR_INVALID_ARG;
    if (cf < 0.0) return -1;
    const double c = floor(((double)T / (double)E) * cf);
    if (c > 2147483647.0) return 2147483647;
    return (int32_t)c;
}

int moe_gemm_variant(const moe_desc *desc, int up) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    const int N = up ? (desc->activation == MOE_ACT_SWIGLU ? 2 * desc->d_ff
                                                           : desc->d_ff)
                     : desc->d;
    int v = variant_override(up != 0, desc, N);
    if (v < 0) v = pick_variant(desc, N, up != 0);
    return v;
}

int moe_gemm_tail_split(const moe_desc *desc, int up) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    const int N = up ? (desc->activation == MOE_ACT_SWIGLU ? 2 * desc->d_ff
                                                           : desc->d_ff)
                     : desc->d;
    int v = variant_override(up != 0, desc, N);
    if (v < 0) v = pick_variant(desc, N, up != 0);
    return w4_256(v) ? tail_split(desc, up != 0) : 1;
}

size_t moe_workspace_size(const moe_desc *desc) {
    if (check_desc(desc) != MOE_OK) return 0;
    return layout(desc).total;
}

int moe_router_topk(const moe_desc *desc, const void *x, const moe_weights *w,
                    moe_routing *r, void *ws, size_t ws_bytes, void *stream) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    if (!x) return MOE_ERR_INVALID_ARG;
    if ((st = check_weights_router(w)) != MOE_OK) return st;
    if ((st = check_routing_router(desc, r)) != MOE_OK) return st;
    if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
    const RouterParams p = router_params(desc, x, w, r, ws);
    return to_status(launch_router(p, desc->dtype, (hipStream_t)stream));
}

int moe_permute(const moe_desc *desc, moe_routing *r, void *ws,
                size_t ws_bytes, void *stream) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    if ((st = check_routing_permute(desc, r)) != MOE_OK) return st;
    if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
    const PermuteParams p = permute_params(desc, r, ws);
    if (expert_choice(desc))
        return to_status(launch_expert_choice(p, (hipStream_t)stream));
    return to_status(launch_permute(p, (hipStream_t)stream));
}

int moe_route_dispatch(const moe_desc *desc, const void *x,
                       const moe_weights *w, moe_routing *r, void *ws,
                       size_t ws_bytes, void *stream) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    if (!x) return MOE_ERR_INVALID_ARG;
    if ((st = check_weights_router(w)) != MOE_OK) return st;
    if ((st = check_routing_router(desc, r)) != MOE_OK) return st;
    if ((st = check_routing_permute(desc, r)) != MOE_OK) return st;
    if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
    return route_and_permute(desc, x, w, r, ws, ws_bytes, stream);
}

int moe_ffn_up(const moe_desc *desc, const void *x, const moe_weights *w,
               const moe_routing *r, void *ws, size_t ws_bytes,
               void *stream) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    if (!x) return MOE_ERR_INVALID_ARG;
    if ((st = check_weights_ffn(desc, w)) != MOE_OK) return st;
    if ((st = check_routing_ffn(desc, r)) != MOE_OK) return st;
    if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
    return run_gemm(desc, w, r, true, x, ws, (hipStream_t)stream);
}

int moe_ffn_down(const moe_desc *desc, const moe_weights *w,
                 const moe_routing *r, void *ws, size_t ws_bytes,
                 void *stream) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    if ((st = check_weights_ffn(desc, w)) != MOE_OK) return st;
    if ((st = check_routing_ffn(desc, r)) != MOE_OK) return st;
    if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
    return run_gemm(desc, w, r, false, nullptr, ws, (hipStream_t)stream);
}

int moe_grouped_ffn(const moe_desc *desc, const void *x, const moe_weights *w,
                    const moe_routing *r, void *ws, size_t ws_bytes,
                    void *stream) {
    int st = moe_ffn_up(desc, x, w, r, ws, ws_bytes, stream);
    if (st != MOE_OK) return st;
    return moe_ffn_down(desc, w, r, ws, ws_bytes, stream);
}

int moe_combine(const moe_desc *desc, const moe_routing *r, void *y, void *ws,
                size_t ws_bytes, void *stream) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    if (!y) return MOE_ERR_INVALID_ARG;
    if ((st = check_routing_combine(r)) != MOE_OK) return st;
    if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
    const WsLayout L = layout(desc);
    CombineParams p;
    p.yp = at(ws, L.yp);
    p.slot_of = r->slot_of;
    p.topk_w = r->topk_w;
    p.y = y;
    p.T = desc->T;
    p.d = desc->d;
    p.k = desc->k;
    p.n_shared = desc->n_shared;
    p.shared_base = (int)routed_rows(desc);
    return to_status(launch_combine(p, desc->dtype, (hipStream_t)stream));
}

int moe_forward(const moe_desc *desc, const void *x, const moe_weights *w,
                moe_routing *r, void *y, void *ws, size_t ws_bytes,
                void *stream) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    if (!x || !y) return MOE_ERR_INVALID_ARG;
    if ((st = check_weights_router(w)) != MOE_OK) return st;
    if ((st = check_weights_ffn(desc, w)) != MOE_OK) return st;
    if ((st = check_routing_router(desc, r)) != MOE_OK) return st;
    if ((st = check_routing_permute(desc, r)) != MOE_OK) return st;
    if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
    if ((st = route_and_permute(desc, x, w, r, ws, ws_bytes, stream)) != MOE_OK)
        return st;
    if ((st = moe_grouped_ffn(desc, x, w, r, ws, ws_bytes, stream)) != MOE_OK)
        return st;
    return moe_combine(desc, r, y, ws, ws_bytes, stream);
}

int moe_forward_noalloc(const moe_desc *desc, const void *x,
                        const moe_weights *w, moe_routing *r, void *y,
                        void *stream) {
    int st = check_desc(desc);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    const size_t need = layout(desc).total;
    if (need > kStaticScratchBytes) return MOE_ERR_SCRATCH;
    void *ws = static_scratch(&st);
    if (st != MOE_OK) return st;
    return moe_forward(desc, x, w, r, y, ws, kStaticScratchBytes, stream);
}

int moe_bias_update(int32_t E, const int32_t *counts, float target,
                    float gamma, float *expert_bias, void *stream) {
    if (E < 1 || E > MOE_MAX_E || !counts || !expert_bias)
        return MOE_ERR_INVALID_ARG;
    return to_status(launch_bias_update(E, counts, target, gamma, expert_bias,
                                        (hipStream_t)stream));
}

const char *moe_status_string(int status) {
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH:
        return "layer needs more scratch than the static buffer holds";
    default: return "unknown status";
    }
}

const char *moe_version(void) { return "moe-gfx950 0.2.0"; }

}  // extern "C"
