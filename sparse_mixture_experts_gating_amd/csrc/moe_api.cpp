// C ABI of the MoE layer (declared in include/moe.h): argument checks,
// workspace carving, launch sequencing and per-kernel event timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "moe.h"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

// ---------------------------------------------------------------------------
// timing
// ---------------------------------------------------------------------------
enum Kind {
    K_ROUTE, K_GATE_LOGITS, K_EC_SELECT, K_PERM_COUNT, K_PERM_SCAN, K_PERM_SCATTER, K_EC_PERMUTE, K_GATHER,
    K_TILE_PLAN, K_GEMM1, K_GEMM2, K_GEMM1_SHARED, K_GEMM2_SHARED, K_COMBINE, K_ROUTER_STATS, K_PERM_SMALL,
    K_ROUTE_GATE, K_COUNT
};
const char *kKindNames[K_COUNT] = {"route", "gate_logits", "ec_select", "permute_count", "permute_scan",
                                   "permute_scatter", "ec_permute", "gather_rows", "tile_plan", "gemm1_act",
                                   "gemm2", "gemm1_act_shared", "gemm2_shared", "combine", "router_stats",
                                   "permute_small", "route_gate"};

struct Pending {
    hipEvent_t a, b;
    int kind;
};
std::mutex g_tmu;
std::atomic<bool> g_timing{false};  // read outside the lock by every launch
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
double g_total_ms[K_COUNT];
int64_t g_launches[K_COUNT];

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launches of the allocation-free entry points record no events (creating
// one allocates); set for the duration of such a call on this thread.
thread_local bool t_untimed = false;

// Runs one launch; with timing on, brackets it with events on its stream.
template <class F>
moe_status launch(int kind, hipStream_t s, F &&f) {
    hipEvent_t a = nullptr, b = nullptr;
    if (!t_untimed && g_timing.load(std::memory_order_relaxed)) {
        std::lock_guard<std::mutex> lk(g_tmu);
        a = take_event();
        b = take_event();
        if (a && b && hipEventRecord(a, s) != hipSuccess) a = nullptr;
    }
    f();
    hipError_t e = hipGetLastError();
    if (a && b && hipEventRecord(b, s) == hipSuccess) {
        std::lock_guard<std::mutex> lk(g_tmu);
        g_pending.push_back({a, b, kind});
    }
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s launch failed: %s", kKindNames[kind], hipGetErrorString(e));
    return MOE_OK;
}

#define TRY(expr)                          \
    do {                                   \
        moe_status _st = (expr);           \
        if (_st != MOE_OK) return _st;     \
    } while (0)

// ---------------------------------------------------------------------------
// configuration
// ---------------------------------------------------------------------------
struct Derived {
    int64_t T, d, E, k, F, Fs;
    int64_t Ns, Fsum;  // shared experts and their stacked hidden width Ns * Fs
    int gating, act;
    bool bf16, ec;
    int capacity;      // Switch / expert choice, else 0
    int group_chunks;  // Switch: chunks per capacity group, 0 = all
    int64_t slots;     // token choice: T*k; expert choice: E*C (entries of topk_idx / topk_w)
    int64_t a_max;     // rows of x_perm / y_perm
    int64_t S;         // slot_row columns: k or E
    int64_t nc;        // permutation chunks
    size_t elem;       // bytes per element of dtype
};

bool token_choice_capacity(const moe_config *c) {
    return c->gating == MOE_GATE_SWITCH ||
           ((c->gating == MOE_GATE_TOPK_SOFTMAX || c->gating == MOE_GATE_SOFTMAX_TOPK) && c->capacity_factor > 0.f);
}

int capacity_of(const moe_config *c) {
    if (token_choice_capacity(c)) {
        const double G = c->capacity_group > 0 ? (double)c->capacity_group : (double)c->num_tokens;
        const int cap = (int)((double)c->capacity_factor * G * (double)c->top_k / (double)c->num_experts);
        return cap < c->min_capacity ? c->min_capacity : cap;
    }
    if (c->gating == MOE_GATE_EXPERT_CHOICE)
        return (int)((double)c->capacity_factor * (double)c->num_tokens / (double)c->num_experts);
    return 0;
}

moe_status derive(const moe_config *c, Derived *o) {
    if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
    if (c->num_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "num_tokens < 0");
    if (c->d_model < 1 || c->num_experts < 1 || c->d_ff < 1 || c->d_ff_shared < 0)
        return fail(MOE_ERR_INVALID_ARG, "d_model, num_experts and d_ff must be >= 1, d_ff_shared >= 0");
    if (c->gating < 0 || c->gating > 3) return fail(MOE_ERR_INVALID_ARG, "unknown gating %d", c->gating);
    if (c->act < 0 || c->act > 2) return fail(MOE_ERR_INVALID_ARG, "unknown activation %d", c->act);
    if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
    o->T = c->num_tokens;
    o->d = c->d_model;
    o->E = c->num_experts;
    o->F = c->d_ff;
    o->Fs = c->d_ff_shared;
    o->Ns = o->Fs > 0 ? c->num_shared : 0;
    if (o->Fs > 0 && c->num_shared < 1)
        return fail(MOE_ERR_INVALID_ARG, "num_shared must be >= 1 when d_ff_shared > 0");
    o->Fsum = o->Ns * o->Fs;
    o->gating = c->gating;
    o->act = c->act;
    o->bf16 = c->dtype == MOE_BF16;
    o->ec = c->gating == MOE_GATE_EXPERT_CHOICE;
    o->elem = o->bf16 ? 2 : 4;
    o->k = o->ec ? 0 : c->top_k;
    if (o->E > 1024) return fail(MOE_ERR_UNSUPPORTED, "num_experts %lld > 1024", (long long)o->E);
    if (!o->ec && (c->top_k < 1 || c->top_k > c->num_experts))
        return fail(MOE_ERR_INVALID_ARG, "top_k %d outside [1, num_experts=%d]", c->top_k, c->num_experts);
    o->capacity = 0;
    o->group_chunks = 0;
    if (c->min_capacity < 0) return fail(MOE_ERR_INVALID_ARG, "min_capacity < 0");
    if (c->capacity_factor < 0.f) return fail(MOE_ERR_INVALID_ARG, "capacity_factor < 0");
    if (c->gating == MOE_GATE_SWITCH && c->top_k != 1) return fail(MOE_ERR_INVALID_ARG, "Switch gating needs top_k == 1");
    if (c->gating == MOE_GATE_SWITCH && !(c->capacity_factor > 0.f))
        return fail(MOE_ERR_INVALID_ARG, "Switch gating needs capacity_factor > 0");
    if (token_choice_capacity(c)) {
        if (c->capacity_group < 0) return fail(MOE_ERR_INVALID_ARG, "capacity_group < 0");
        if (c->capacity_group % kChunk != 0)
            return fail(MOE_ERR_UNSUPPORTED, "capacity_group %d is not a multiple of %d", c->capacity_group, kChunk);
        o->capacity = capacity_of(c);
        if (o->T > 0 && o->capacity < 1) return fail(MOE_ERR_INVALID_ARG, "capacity int(cf*G/E) is 0");
        o->group_chunks = c->capacity_group / kChunk;
    }
    if (o->ec) {
        if (!(c->capacity_factor > 0.f)) return fail(MOE_ERR_INVALID_ARG, "expert choice needs capacity_factor > 0");
        o->capacity = capacity_of(c);
        if (o->T > 0 && (o->capacity < 1 || o->capacity > o->T))
            return fail(MOE_ERR_INVALID_ARG, "expert capacity %d outside [1, T=%lld]", o->capacity, (long long)o->T);
        if (o->capacity > kEcMaxCapacity)
            return fail(MOE_ERR_UNSUPPORTED, "expert capacity %d > %d", o->capacity, kEcMaxCapacity);
    }
    const int kq = o->bf16 ? 64 : 16;
    if (o->d % kq || o->F % kq || o->Fs % kq)
        return fail(MOE_ERR_UNSUPPORTED, "d_model, d_ff and d_ff_shared must be multiples of %d for this dtype", kq);
    // the GEMM tiles address up to 256 rows from a tile base with 32-bit byte offsets
    if (std::max(std::max(o->d, o->F), o->Fsum) > (1 << 21))
        return fail(MOE_ERR_UNSUPPORTED, "d_model, d_ff and num_shared * d_ff_shared must be at most %d", 1 << 21);
    // the shared experts' down projections are read through one buffer resource
    if (o->Ns > 1 && o->Fsum * o->d * (int64_t)o->elem > 0x7fffffff)
        return fail(MOE_ERR_UNSUPPORTED, "the shared down projections exceed 2^31 bytes");
    o->slots = o->ec ? o->E * o->capacity : o->T * o->k;
    o->a_max = o->slots;
    o->S = o->ec ? o->E : o->k;
    o->nc = (o->T + kChunk - 1) / kChunk;
    if (o->T * (o->ec ? o->E : o->k) >= (int64_t)1 << 31 || o->slots >= (int64_t)1 << 31)
        return fail(MOE_ERR_UNSUPPORTED, "too many token slots for 32-bit row indices");
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Carve {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t o = off;
        off += align_up(bytes);
        return o;
    }
};

struct PermuteWs {
    size_t counts, pre, base, ranks;
};
PermuteWs carve_permute(const Derived &D, Carve &c) {
    PermuteWs w{};
    if (D.ec) return w;
    const size_t ce = (size_t)D.nc * D.E * 4;
    w.counts = c.take(ce);
    w.pre = c.take(ce);
    w.base = c.take(ce);
    w.ranks = c.take((size_t)D.T * D.k * 4);
    return w;
}

struct LossWs {
    size_t part, cnt;
};
LossWs carve_losses(const Derived &D, Carve &c) {
    const int64_t nb = (D.T + kStatTokens - 1) / kStatTokens;
    LossWs w{};
    w.part = c.take((size_t)nb * (D.E + 1) * 4);
    w.cnt = c.take((size_t)nb * D.E * 4);
    return w;
}

struct FfnWs {
    size_t mstart, mtile, h, hs, part, cnt;
    int64_t part_floats;
    int ncnt, max_mt;
};
FfnWs carve_ffn(const Derived &D, Carve &c) {
    FfnWs w{};
    w.mstart = c.take((size_t)(D.E + 1) * 4);
    w.max_mt = (int)max_mtiles(D.a_max, (int)D.E);
    w.mtile = c.take((size_t)w.max_mt * 16);
    w.h = c.take((size_t)D.a_max * D.F * D.elem);
    w.hs = D.Fs ? c.take((size_t)D.T * D.Fsum * D.elem) : 0;
    if (D.bf16) {
        // split-K partial tiles: one largest tile per CU (the bf16 shapes with
        // several workgroups per CU have proportionally smaller tiles)
        int cus = device_cus();
        if (cus <= 0) cus = 256;
        w.part_floats = (int64_t)cus * kSplitUnitFloats;
        w.ncnt = cus * kSplitSlotsPerCu;
        w.part = c.take((size_t)w.part_floats * 4);
        w.cnt = c.take((size_t)w.ncnt * 4);
    }
    return w;
}

// Token choice over many experts (bf16, 128..256 experts, at least 1024
// tokens): the forward pass computes the router logits as a dense GEMM split
// along K into partial sums (workspace), then one light kernel adds the
// parts, writes the logits and gates.  The fused tile router would stream all
// router weights through LDS once per 32 tokens.
bool router_as_gemm(const Derived &D) { return D.bf16 && !D.ec && D.E >= 128 && D.E <= 256 && D.T >= 1024; }

struct ForwardWs {
    size_t logits, idx, w, counts, offsets, row_token, slot_row, x_perm, y_perm, y_shared, rpart, logits_t;
    PermuteWs perm;
    FfnWs ffn;
};
ForwardWs carve_forward(const Derived &D, Carve &c) {
    ForwardWs w{};
    w.logits = c.take((size_t)D.T * D.E * 4);
    w.idx = c.take((size_t)D.slots * 4);
    w.w = c.take((size_t)D.slots * 4);
    w.counts = c.take((size_t)D.E * 4);
    w.offsets = c.take((size_t)(D.E + 1) * 4);
    w.row_token = c.take((size_t)D.a_max * 4);
    w.slot_row = c.take((size_t)D.T * D.S * 4);
    w.x_perm = c.take((size_t)D.a_max * D.d * D.elem);
    w.y_perm = c.take((size_t)D.a_max * D.d * D.elem);
    w.y_shared = D.Fs ? c.take((size_t)D.T * D.d * D.elem) : 0;
    w.perm = carve_permute(D, c);
    w.ffn = carve_ffn(D, c);
    w.rpart = router_as_gemm(D) ? c.take((size_t)kRouterMaxSplit * D.T * D.E * 4) : 0;
    // expert choice (bf16 routers): the logits transposed, [E][T]
    w.logits_t = D.ec && D.bf16 ? c.take((size_t)D.T * D.E * 4) : 0;
    return w;
}

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

moe_status need_ptr(const void *p, const char *name, bool aligned = true) {
    if (!p) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
    if (aligned && misaligned(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return MOE_OK;
}

moe_status check_weights_ffn(const Derived &D, const moe_weights *w) {
    if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
    TRY(need_ptr(w->w1, "w1"));
    TRY(need_ptr(w->w2, "w2"));
    if (D.act == MOE_ACT_SWIGLU) {
        TRY(need_ptr(w->w3, "w3"));
        if (w->b1 || w->b2) return fail(MOE_ERR_INVALID_ARG, "expert biases are only defined for ReLU/GELU experts");
    }
    if (D.Fs) {
        TRY(need_ptr(w->ws1, "ws1"));
        TRY(need_ptr(w->ws3, "ws3"));
        TRY(need_ptr(w->ws2, "ws2"));
    }
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// stage bodies (arguments already checked)
// ---------------------------------------------------------------------------
moe_status do_route(const Derived &D, const void *x, const moe_weights *w, const moe_routing *r, hipStream_t s,
                    const void *w_noise = nullptr, const float *noise = nullptr) {
    if (D.T == 0) return MOE_OK;
    RouteArgs a{x, w->w_router, w->b_router, (int)D.T, (int)D.d, (int)D.E, (int)D.k, D.gating, D.bf16,
                r->logits, r->topk_idx, r->topk_w, w_noise, noise};
    TRY(launch(K_ROUTE, s, [&] { launch_route(a, s); }));
    if (D.ec)
        TRY(launch(K_EC_SELECT, s, [&] {
            launch_ec_select(r->logits, (int)D.T, (int)D.E, D.capacity, r->topk_idx, r->topk_w, s);
        }));
    return MOE_OK;
}

// plan non-null: the one-workgroup permutation, or else the scan of the
// three-kernel one, also builds the grouped GEMMs' tile plan, and
// *plan_built is set.
moe_status do_permute(const Derived &D, const void *x, const moe_routing *r, void *x_perm, char *ws,
                      const PermuteWs &pw, hipStream_t s, bool gather = true, const TilePlanArgs *plan = nullptr,
                      bool *plan_built = nullptr) {
    if (D.T == 0) return MOE_OK;
    if (D.ec) {
        TRY(launch(K_EC_PERMUTE, s, [&] {
            launch_ec_permute(r->topk_idx, (int)D.T, (int)D.E, D.capacity, r->counts, r->offsets, r->row_token,
                              r->slot_row, s);
        }));
    } else {
        PermuteArgs a{r->topk_idx, (int)D.T, (int)D.E, (int)D.k, D.capacity, D.group_chunks,
                      (int32_t *)(ws + pw.counts), (int32_t *)(ws + pw.pre), (int32_t *)(ws + pw.base),
                      (int32_t *)(ws + pw.ranks), r->counts, r->offsets, r->row_token, r->slot_row};
        const TilePlanArgs none{0, nullptr, nullptr, 0, nullptr, 0, false};
        if (permute_small_fits((int)D.T, (int)D.E, (int)D.k)) {
            TRY(launch(K_PERM_SMALL, s, [&] { launch_permute_small(a, plan ? *plan : none, s); }));
        } else {
            TRY(launch(K_PERM_COUNT, s, [&] { launch_permute_count(a, s); }));
            TRY(launch(K_PERM_SCAN, s, [&] { launch_permute_scan(a, plan ? *plan : none, s); }));
            TRY(launch(K_PERM_SCATTER, s, [&] { launch_permute_scatter(a, s); }));
        }
        if (plan && plan_built) *plan_built = true;
    }
    if (gather)
        TRY(launch(K_GATHER, s, [&] {
            launch_gather_rows(x, r->row_token, r->offsets, (int)D.E, D.a_max, (int)D.d, (int)D.elem, x_perm, s);
        }));
    return MOE_OK;
}

// The forward pass skips the gather kernel when the first GEMM can load the
// routed token rows itself: float32 (the VALU kernel addresses rows through
// the row map with 64-bit pointers), or bf16 with all of x addressable by one
// buffer resource (32-bit byte offsets below 2^31).
bool gather_in_gemm(const Derived &D) { return !D.bf16 || (int64_t)D.T * D.d * 2 <= 0x7fffffff; }

int pick_shape(const Derived &D) {
    if (D.ec) return D.capacity <= 160 ? kGemmSmallM : kGemmPrefill;
    if (D.T <= 32) return kGemmDecode;
    int64_t max_rows = D.T, kept_max = D.T * D.k;
    if (D.capacity > 0) {
        const int64_t groups = D.group_chunks ? (D.T + D.group_chunks * kChunk - 1) / (D.group_chunks * kChunk) : 1;
        max_rows = std::min<int64_t>(D.T, groups * D.capacity);
        kept_max = std::min<int64_t>(kept_max, groups * D.capacity * D.E);
    }
    const double avg = (double)D.T * D.k / D.E;
    if (avg <= 160.0 || max_rows <= 384) {
        // When even the 128-row tiles of the down projection (N = d, 256
        // columns a tile) cannot fill the CUs, each tile's K loop is the
        // critical path and smaller tiles spread the work over more CUs, as
        // long as the extra m-tiles do not re-stream weights from HBM: few
        // rows per expert (32-row tiles, one each) or weights that stay in
        // the 256 MB MALL (64-row tiles, half the weight re-reads of 32-row
        // ones).  Measured: Switch layer 0.085 -> 0.061 ms on 32-row tiles,
        // then 0.070 -> 0.063 ms on 64-row ones (alternating runs); Mixtral
        // shape T = 64 0.67 -> 0.60 ms on 32-row tiles, but T = 128 and 256
        // faster on 128-row tiles (0.69 vs 0.73, 0.69 vs 0.76 ms).
        const int64_t tiles = ((kept_max + 127) / 128 + D.E) * ((D.d + 255) / 256);
        const double wbytes = (double)D.E * D.F * D.d * D.elem * (D.act == MOE_ACT_SWIGLU ? 3 : 2);
        const bool few_rows = avg <= 24.0, cached = wbytes <= 128e6;
        if (tiles < device_cus() && few_rows) return kGemmDecode;
        return tiles < device_cus() && cached ? kGemmMid : kGemmSmallM;
    }
    return kGemmPrefill;
}

// average rows per expert under four 256-row tiles: most tiles are ragged
bool ragged_layer(const Derived &D) { return D.a_max < 4 * 256 * D.E; }

// Tile plan of the grouped GEMMs for this layer, in the FFN workspace.
// Ragged layers spread the tiles of experts with less than a tile of rows
// among the others (DeepSeek-style layer: down projection -2.5%).
TilePlanArgs plan_args(const Derived &D, char *ws, const FfnWs &fw) {
    return TilePlanArgs{gemm_block_m(pick_shape(D), D.bf16), (int32_t *)(ws + fw.mstart), (int4 *)(ws + fw.mtile),
                        fw.max_mt, D.bf16 ? (int32_t *)(ws + fw.cnt) : nullptr, D.bf16 ? fw.ncnt : 0,
                        ragged_layer(D)};
}

// x_perm null: the first GEMM reads the routed rows straight from x through
// the row map (float32, or bf16 with x within one buffer resource; see
// gather_in_gemm).
// plan_built: the permutation already wrote the tile plan (plan_args).
moe_status do_ffn(const Derived &D, const void *x_perm, const void *x, const moe_routing *r, const moe_weights *w,
                  void *y_perm, void *y_shared, char *ws, const FfnWs &fw, hipStream_t s, bool plan_built = false) {
    if (D.T == 0) return MOE_OK;
    const int shape = pick_shape(D);
    const TilePlanArgs plan = plan_args(D, ws, fw);
    int32_t *mstart = plan.mstart;
    int4 *mtile = plan.mtile;
    void *H = ws + fw.h;
    const SplitKWs split{D.bf16 ? (float *)(ws + fw.part) : nullptr, fw.part_floats,
                         D.bf16 ? (int32_t *)(ws + fw.cnt) : nullptr, fw.ncnt};
    if (!plan_built)
        TRY(launch(K_TILE_PLAN, s, [&] {
            launch_tile_plan(r->counts, r->offsets, (int)D.E, plan.BM, mstart, mtile, fw.max_mt, split.cnt,
                             split.ncnt, plan.interleave, s);
        }));
    GemmArgs g1{x_perm, w->w1, w->w3, w->b1, H, r->offsets, mstart, mtile, fw.max_mt, (int)D.E, D.a_max, (int)D.F,
                (int)D.d, D.act == MOE_ACT_SWIGLU ? kActSwiglu : D.act, D.bf16, split};
    if (x_perm == nullptr) {
        g1.A = x;
        g1.arow = r->row_token;
        g1.a_rows = D.T;
    }
    TRY(launch(K_GEMM1, s, [&] { launch_grouped_gemm(g1, shape, s); }));
    GemmArgs g2{H, w->w2, nullptr, w->b2, y_perm, r->offsets, mstart, mtile, fw.max_mt, (int)D.E, D.a_max, (int)D.d,
                (int)D.F, kActNone, D.bf16, split};
    TRY(launch(K_GEMM2, s, [&] { launch_grouped_gemm(g2, shape, s); }));
    if (D.Fs) {
        // The Ns shared experts as one SwiGLU expert of width Ns * Fs: their
        // stacked [Ns][Fs][d] gate and up weights are its [Ns*Fs][d] rows, and
        // the down projection takes its K axis from the Ns [d][Fs] blocks in
        // turn (K-sliced B), so the experts' outputs add up in one accumulation.
        const int sshape = D.T <= 32 ? kGemmDecode : kGemmPrefill;
        void *Hs = ws + fw.hs;
        GemmArgs s1{x, w->ws1, w->ws3, nullptr, Hs, nullptr, nullptr, nullptr, 0, 1, D.T, (int)D.Fsum, (int)D.d,
                    kActSwiglu, D.bf16, split};
        TRY(launch(K_GEMM1_SHARED, s, [&] { launch_grouped_gemm(s1, sshape, s); }));
        GemmArgs s2{Hs, w->ws2, nullptr, nullptr, y_shared, nullptr, nullptr, nullptr, 0, 1, D.T, (int)D.d,
                    (int)D.Fsum, kActNone, D.bf16, split};
        if (D.Ns > 1) s2.kslice = (int)D.Fs;
        TRY(launch(K_GEMM2_SHARED, s, [&] { launch_grouped_gemm(s2, sshape, s); }));
    }
    return MOE_OK;
}

moe_status do_combine(const Derived &D, const void *y_perm, const void *y_shared, const moe_routing *r, void *y,
                      hipStream_t s) {
    if (D.T == 0) return MOE_OK;
    CombineArgs a{y_perm, y_shared, r->topk_w, r->slot_row, (int)D.T, (int)D.d, (int)D.S, D.ec, D.bf16, y};
    return launch(K_COMBINE, s, [&] { launch_combine(a, s); });
}

moe_status check_routing(const Derived &D, const moe_routing *r, bool need_perm) {
    if (!r) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
    TRY(need_ptr(r->topk_idx, "routing.topk_idx", false));
    TRY(need_ptr(r->topk_w, "routing.topk_w", false));
    if (need_perm) {
        TRY(need_ptr(r->counts, "routing.counts", false));
        TRY(need_ptr(r->offsets, "routing.offsets", false));
        TRY(need_ptr(r->row_token, "routing.row_token", false));
        TRY(need_ptr(r->slot_row, "routing.slot_row", false));
    }
    return MOE_OK;
}

// ---------------------------------------------------------------------------
// fixed scratch of the allocation-free permutation
// ---------------------------------------------------------------------------
// Device memory of the library itself, one copy per GPU, held until the
// process ends.  On the host, `scratch` names only a stand-in for the device
// array: kernels receive the device address that hipGetSymbolAddress returns
// for the current device, never the name.
constexpr size_t kNoAllocScratchBytes = (size_t)MOE_PERMUTE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxScratchDevices];  // device address per device, null until first use

// The current device's copy of `scratch`, looked up once per device.
moe_status scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(MOE_ERR_UNSUPPORTED, "device %d: the fixed scratch is kept for devices 0..%d", dev,
                    kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                        hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

moe_status check_route_limits(const Derived &D) {
    if (D.E > 256) return fail(MOE_ERR_UNSUPPORTED, "the fused router handles at most 256 experts");
    return MOE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// exported entry points
// ---------------------------------------------------------------------------
extern "C" {

const char *moe_last_error(void) { return g_err.c_str(); }

moe_status moe_capacity(const moe_config *cfg, int32_t *capacity) {
    g_err.clear();
    if (!capacity) return fail(MOE_ERR_INVALID_ARG, "capacity is NULL");
    Derived D;
    TRY(derive(cfg, &D));
    *capacity = D.capacity;
    return MOE_OK;
}

moe_status moe_workspace_size(const moe_config *cfg, int32_t stage, size_t *bytes) {
    g_err.clear();
    if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
    Derived D;
    TRY(derive(cfg, &D));
    Carve c;
    if (stage == MOE_STAGE_FORWARD) carve_forward(D, c);
    else if (stage == MOE_STAGE_PERMUTE) carve_permute(D, c);
    else if (stage == MOE_STAGE_FFN) carve_ffn(D, c);
    else if (stage == MOE_STAGE_LOSSES) carve_losses(D, c);
    else return fail(MOE_ERR_INVALID_ARG, "unknown stage %d", stage);
    *bytes = c.off;
    return MOE_OK;
}

moe_status moe_route(const moe_config *cfg, const void *x, const moe_weights *w, moe_routing *routing,
                     void *stream) {
    g_err.clear();
    Derived D;
    TRY(derive(cfg, &D));
    if (D.T == 0) return MOE_OK;  // empty batch: nothing to launch
    TRY(check_route_limits(D));
    TRY(need_ptr(x, "x"));
    if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
    TRY(need_ptr(w->w_router, "w_router"));
    TRY(check_routing(D, routing, false));
    if (D.ec) TRY(need_ptr(routing->logits, "routing.logits (required for expert choice)", false));
    return do_route(D, x, w, routing, (hipStream_t)stream);
}

moe_status moe_route_noisy(const moe_config *cfg, const void *x, const moe_weights *w, const void *w_noise,
                           const float *noise, moe_routing *routing, void *stream) {
    g_err.clear();
    Derived D;
    TRY(derive(cfg, &D));
    if (D.T == 0) return MOE_OK;  // empty batch: nothing to launch
    if (D.ec) return fail(MOE_ERR_UNSUPPORTED, "the noisy router is defined for token-choice gating");
    TRY(check_route_limits(D));
    TRY(need_ptr(x, "x"));
    if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
    TRY(need_ptr(w->w_router, "w_router"));
    TRY(need_ptr(w_noise, "w_noise"));
    TRY(need_ptr(noise, "noise", false));
    TRY(check_routing(D, routing, false));
    return do_route(D, x, w, routing, (hipStream_t)stream, w_noise, noise);
}

moe_status moe_router_losses(const moe_config *cfg, const float *logits, const int32_t *topk_idx, float *out,
                             void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    Derived D;
    TRY(derive(cfg, &D));
    if (D.ec) return fail(MOE_ERR_UNSUPPORTED, "router losses are defined for token-choice gating");
    if (D.E > 256) return fail(MOE_ERR_UNSUPPORTED, "router losses handle at most 256 experts");
    if (D.T == 0) return fail(MOE_ERR_INVALID_ARG, "router losses need at least one token");
    TRY(need_ptr(logits, "logits", false));
    TRY(need_ptr(topk_idx, "topk_idx", false));
    TRY(need_ptr(out, "out", false));
    Carve c;
    const LossWs lw = carve_losses(D, c);
    TRY(need_ptr(ws, "ws"));
    if (ws_bytes < c.off) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, c.off);
    hipStream_t s = (hipStream_t)stream;
    char *base = (char *)ws;
    return launch(K_ROUTER_STATS, s, [&] {
        launch_router_stats(logits, topk_idx, (int)D.T, (int)D.E, (int)D.k, (float *)(base + lw.part),
                            (int32_t *)(base + lw.cnt), out, s);
    });
}

moe_status moe_route_from_logits(const moe_config *cfg, const float *logits, moe_routing *routing, void *stream) {
    g_err.clear();
    Derived D;
    TRY(derive(cfg, &D));
    if (D.T == 0) return MOE_OK;  // empty batch: nothing to launch
    TRY(check_route_limits(D));
    TRY(need_ptr(logits, "logits", false));
    TRY(check_routing(D, routing, false));
    if (D.T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    if (D.ec)
        return launch(K_EC_SELECT, s, [&] {
            launch_ec_select(logits, (int)D.T, (int)D.E, D.capacity, routing->topk_idx, routing->topk_w, s);
        });
    return launch(K_GATE_LOGITS, s, [&] {
        launch_gate_logits(logits, (int)D.T, (int)D.E, (int)D.k, D.gating, routing->topk_idx, routing->topk_w, s);
    });
}

moe_status moe_permute(const moe_config *cfg, const void *x, moe_routing *routing, void *x_perm, void *ws,
                       size_t ws_bytes, void *stream) {
    g_err.clear();
    Derived D;
    TRY(derive(cfg, &D));
    if (D.T == 0) return MOE_OK;  // empty batch: nothing to launch
    TRY(check_routing(D, routing, true));
    TRY(need_ptr(x, "x"));
    TRY(need_ptr(x_perm, "x_perm"));
    Carve c;
    const PermuteWs pw = carve_permute(D, c);
    if (c.off > 0) {
        TRY(need_ptr(ws, "ws"));
        if (ws_bytes < c.off)
            return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, c.off);
    }
    return do_permute(D, x, routing, x_perm, (char *)ws, pw, (hipStream_t)stream);
}

moe_status moe_permute_noalloc(const moe_config *cfg, const void *x, moe_routing *routing, void *x_perm,
                               void *stream) {
    g_err.clear();
    Derived D;
    TRY(derive(cfg, &D));
    if (D.T == 0) return MOE_OK;  // empty batch: nothing to launch
    TRY(check_routing(D, routing, true));
    TRY(need_ptr(x, "x"));
    TRY(need_ptr(x_perm, "x_perm"));
    Carve c;
    const PermuteWs pw = carve_permute(D, c);
    if (c.off > kNoAllocScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED, "permutation scratch of %zu bytes exceeds the fixed %zu bytes", c.off,
                    kNoAllocScratchBytes);
    void *ws = nullptr;
    TRY(scratch_of_current_device(&ws));
    // every scratch entry the kernels read is written earlier in this call,
    // so nothing is cleared between calls
    t_untimed = true;
    const moe_status st = do_permute(D, x, routing, x_perm, (char *)ws, pw, (hipStream_t)stream);
    t_untimed = false;
    return st;
}

moe_status moe_expert_ffn(const moe_config *cfg, const void *x_perm, const void *x, const moe_routing *routing,
                          const moe_weights *w, void *y_perm, void *y_shared, void *ws, size_t ws_bytes,
                          void *stream) {
    g_err.clear();
    Derived D;
    TRY(derive(cfg, &D));
    if (D.T == 0) return MOE_OK;  // empty batch: nothing to launch
    if (!routing) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
    TRY(need_ptr(routing->counts, "routing.counts", false));
    TRY(need_ptr(routing->offsets, "routing.offsets", false));
    TRY(need_ptr(x_perm, "x_perm"));
    TRY(need_ptr(y_perm, "y_perm"));
    TRY(check_weights_ffn(D, w));
    if (D.Fs) {
        TRY(need_ptr(x, "x (shared expert input)"));
        TRY(need_ptr(y_shared, "y_shared"));
    }
    Carve c;
    const FfnWs fw = carve_ffn(D, c);
    TRY(need_ptr(ws, "ws"));
    if (ws_bytes < c.off) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, c.off);
    return do_ffn(D, x_perm, x, routing, w, y_perm, y_shared, (char *)ws, fw, (hipStream_t)stream);
}

moe_status moe_combine(const moe_config *cfg, const void *y_perm, const void *y_shared, const moe_routing *routing,
                       void *y, void *stream) {
    g_err.clear();
    Derived D;
    TRY(derive(cfg, &D));
    if (D.T == 0) return MOE_OK;  // empty batch: nothing to launch
    if (!routing) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
    TRY(need_ptr(routing->topk_w, "routing.topk_w", false));
    TRY(need_ptr(routing->slot_row, "routing.slot_row", false));
    TRY(need_ptr(y_perm, "y_perm"));
    TRY(need_ptr(y, "y"));
    if (D.Fs) TRY(need_ptr(y_shared, "y_shared"));
    else if (y_shared && misaligned(y_shared)) return fail(MOE_ERR_INVALID_ARG, "y_shared is not 16-byte aligned");
    return do_combine(D, y_perm, y_shared, routing, y, (hipStream_t)stream);
}

moe_status moe_forward(const moe_config *cfg, const void *x, const moe_weights *w, void *y, moe_routing *routing,
                       void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    Derived D;
    TRY(derive(cfg, &D));
    if (D.T == 0) return MOE_OK;  // empty batch: nothing to launch
    TRY(check_route_limits(D));
    TRY(need_ptr(x, "x"));
    TRY(need_ptr(y, "y"));
    if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
    TRY(need_ptr(w->w_router, "w_router"));
    TRY(check_weights_ffn(D, w));
    Carve c;
    const ForwardWs fw = carve_forward(D, c);
    TRY(need_ptr(ws, "ws"));
    if (ws_bytes < c.off) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, c.off);
    char *base = (char *)ws;
    moe_routing r;
    if (routing) {
        TRY(check_routing(D, routing, true));
        r = *routing;
        if (!r.logits) r.logits = (float *)(base + fw.logits);
    } else {
        r.logits = (float *)(base + fw.logits);
        r.topk_idx = (int32_t *)(base + fw.idx);
        r.topk_w = (float *)(base + fw.w);
        r.counts = (int32_t *)(base + fw.counts);
        r.offsets = (int32_t *)(base + fw.offsets);
        r.row_token = (int32_t *)(base + fw.row_token);
        r.slot_row = (int32_t *)(base + fw.slot_row);
    }
    if (D.T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    void *x_perm = base + fw.x_perm;
    void *y_perm = base + fw.y_perm;
    void *y_shared = D.Fs ? base + fw.y_shared : nullptr;
    const bool fused = gather_in_gemm(D);
    const TilePlanArgs plan = plan_args(D, base, fw.ffn);
    bool plan_built = false;
    if (fused && route_permute_fits((int)D.T, (int)D.E, D.bf16, D.ec)) {
        // one router block: it also permutes its selections and writes the
        // tile plan (Mixtral-shape decode: one launch fewer)
        const RouteArgs a{x, w->w_router, w->b_router, (int)D.T, (int)D.d, (int)D.E, (int)D.k, D.gating, D.bf16,
                          r.logits, r.topk_idx, r.topk_w, nullptr, nullptr};
        RoutePermuteArgs pa;
        pa.capacity = D.capacity;
        pa.group_chunks = D.group_chunks;
        pa.counts = r.counts;
        pa.offsets = r.offsets;
        pa.row_token = r.row_token;
        pa.slot_row = r.slot_row;
        pa.plan = plan;
        TRY(launch(K_ROUTE, s, [&] { launch_route_permute(a, pa, s); }));
        plan_built = true;
    } else if (D.ec) {
        // expert choice: the router also writes the logits transposed (each
        // expert's column contiguous) and fills the row map with -1; the
        // selection kernel then writes the permutation's chosen entries and
        // the tile plan (every expert has exactly C rows)
        RouteArgs a{x, w->w_router, w->b_router, (int)D.T, (int)D.d, (int)D.E, (int)D.k, D.gating, D.bf16,
                    r.logits, r.topk_idx, r.topk_w, nullptr, nullptr};
        float *lt = D.bf16 ? (float *)(base + fw.logits_t) : nullptr;
        a.logits_t = lt;
        a.fill_rows = lt ? r.slot_row : nullptr;
        bool transposed = false;
        TRY(launch(K_ROUTE, s, [&] { transposed = launch_route(a, s); }));
        EcPermuteArgs pa;
        pa.counts = r.counts;
        pa.offsets = r.offsets;
        pa.row_token = r.row_token;
        pa.slot_row = r.slot_row;
        pa.plan = plan;
        pa.prefilled = transposed;
        TRY(launch(K_EC_SELECT, s, [&] {
            launch_ec_select(r.logits, (int)D.T, (int)D.E, D.capacity, r.topk_idx, r.topk_w, s, &pa,
                             transposed ? lt : nullptr);
        }));
        plan_built = true;
        if (!fused)
            TRY(launch(K_GATHER, s, [&] {
                launch_gather_rows(x, r.row_token, r.offsets, (int)D.E, D.a_max, (int)D.d, (int)D.elem, x_perm, s);
            }));
    } else {
        if (router_as_gemm(D)) {
            const int S = router_gemm_split((int)D.T, (int)D.E, (int)D.d);
            float *part = (float *)(base + fw.rpart);
            TRY(launch(K_ROUTE, s, [&] {
                launch_router_gemm(x, w->w_router, (int)D.T, (int)D.d, (int)D.E, part, S, s);
            }));
            TRY(launch(K_ROUTE_GATE, s, [&] {
                launch_gate_partials(part, S, w->b_router, (int)D.T, (int)D.E, (int)D.k, D.gating, r.logits,
                                     r.topk_idx, r.topk_w, s);
            }));
        } else {
            TRY(do_route(D, x, w, &r, s));
        }
        TRY(do_permute(D, x, &r, x_perm, base, fw.perm, s, !fused, &plan, &plan_built));
    }
    TRY(do_ffn(D, fused ? nullptr : x_perm, x, &r, w, y_perm, y_shared, base, fw.ffn, s, plan_built));
    return do_combine(D, y_perm, y_shared, &r, y, s);
}

moe_status moe_timing_enable(int32_t on) {
    g_err.clear();
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing.store(on != 0, std::memory_order_relaxed);
    return MOE_OK;
}

moe_status moe_timing_reset(void) {
    g_err.clear();
    std::lock_guard<std::mutex> lk(g_tmu);
    for (auto &p : g_pending) {
        (void)hipEventSynchronize(p.b);
        g_pool.push_back(p.a);
        g_pool.push_back(p.b);
    }
    g_pending.clear();
    for (int i = 0; i < K_COUNT; ++i) {
        g_total_ms[i] = 0.0;
        g_launches[i] = 0;
    }
    return MOE_OK;
}

moe_status moe_timing_read(int32_t kind, double *total_ms, int64_t *launches) {
    g_err.clear();
    if (kind < 0 || kind >= K_COUNT) return fail(MOE_ERR_INVALID_ARG, "unknown kernel kind %d", kind);
    if (!total_ms || !launches) return fail(MOE_ERR_INVALID_ARG, "output pointer is NULL");
    std::lock_guard<std::mutex> lk(g_tmu);
    for (auto &p : g_pending) {
        hipError_t e = hipEventSynchronize(p.b);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.a, p.b);
        if (e != hipSuccess) {
            for (auto &q : g_pending) {  // the events go back to the pool; their timings are lost
                g_pool.push_back(q.a);
                g_pool.push_back(q.b);
            }
            g_pending.clear();
            return fail(MOE_ERR_HIP, "event timing failed: %s", hipGetErrorString(e));
        }
        g_total_ms[p.kind] += ms;
        g_launches[p.kind] += 1;
        g_pool.push_back(p.a);
        g_pool.push_back(p.b);
    }
    g_pending.clear();
    *total_ms = g_total_ms[kind];
    *launches = g_launches[kind];
    return MOE_OK;
}

const char *moe_kernel_name(int32_t kind) {
    if (kind < 0 || kind >= K_COUNT) return nullptr;
    return kKindNames[kind];
}

}  // extern "C"
