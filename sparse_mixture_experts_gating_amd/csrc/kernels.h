// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum ActKind { kActRelu = 0, kActGelu = 1, kActSwiglu = 2, kActNone = 3 };
enum GateKind { kGateTopkSoftmax = 0, kGateSoftmaxTopk = 1, kGateSwitch = 2, kGateExpertChoice = 3 };

constexpr int kEcMaxCapacity = 4096;  // LDS sort buffer of the expert-choice select
constexpr int kChunk = 64;            // tokens per permutation chunk (one wave)

// ---- route ----
struct RouteArgs {
    const void *x;
    const void *wg;
    const float *bias;
    int T, d, E, k, gating;
    bool bf16;
    float *logits;  // may be null for token choice
    int32_t *idx;
    float *w;
    const void *wn;       // noisy router: noise projection [E][d], else null
    const float *noise;   // noisy router: [T][E] standard-normal draw, else null
    // expert choice in the forward pass (bf16 routers): also write the
    // logits transposed, [E][T], so that each expert's column is contiguous
    // for the selection, and fill the row map [T][E] with -1 (the selection
    // then writes only its chosen entries); null: neither
    float *logits_t = nullptr;
    int32_t *fill_rows = nullptr;
};
// Returns whether it wrote logits_t and fill_rows (bf16 routers whose tile
// has room for the transposed logits; false when logits_t is null).
bool launch_route(const RouteArgs &a, hipStream_t s);
void launch_gate_logits(const float *logits, int T, int E, int k, int gating, int32_t *idx, float *w,
                        hipStream_t s);
constexpr int kStatTokens = 256;  // tokens per block of the router statistics
void launch_router_stats(const float *logits, const int32_t *idx, int T, int E, int k, float *part,
                         int32_t *cnt, float *out, hipStream_t s);
// Expert-choice selection; with slot_row set it also writes what the
// expert-choice permutation writes (counts, offsets, row_token, slot_row
// [T][E]) and, with plan.mstart set, the grouped GEMMs' tile plan, so the
// forward pass needs no permutation launch.  Declared after TilePlanArgs.
struct EcPermuteArgs;
// logits_t: the same logits transposed ([E][T], from the router), or null.
void launch_ec_select(const float *logits, int T, int E, int C, int32_t *ec_idx, float *ec_score,
                      hipStream_t s, const EcPermuteArgs *perm = nullptr, const float *logits_t = nullptr);

// ---- permute ----
struct PermuteArgs {
    const int32_t *idx;  // [T][k]
    int T, E, k;
    int capacity;        // 0 = none
    int group_chunks;    // chunks per capacity group (0 = all)
    int32_t *chunk_counts, *chunk_pre, *chunk_base;  // [NC][E]
    int32_t *ranks;      // [T][k]
    int32_t *counts, *offsets, *row_token, *slot_row;
};
// One-workgroup permutation (count, scan and scatter in LDS) for batches whose
// chunk tables fit: E <= kMaxSmallExperts, small_tables_bytes(T, E) <= kSmallLdsBytes and
// T * k <= kSmallMaxSlots.  Writes counts, offsets, row_token and slot_row.
constexpr int kMaxSmallExperts = 1024;
constexpr int kSmallLdsBytes = 40 * 1024;
// LDS of the one-workgroup permutation's chunk tables: masks (8 bytes),
// prefixes and bases (4 bytes each) of nc = ceil(T / 64) chunks, in rows of
// E + 1 entries (the padding entry spreads one expert's column over the LDS
// banks: with rows of E = 16 the masks of a column shared two banks)
inline int64_t small_tables_bytes(int64_t T, int E) { return (T + kChunk - 1) / kChunk * (E + 1) * 16; }
constexpr int kSmallMaxSlots = 16384;
bool permute_small_fits(int T, int E, int k);
// The grouped GEMMs' tile plan (see launch_tile_plan), built at the end of
// the one-workgroup permutation when mstart is not null.
struct TilePlanArgs {
    int BM;
    int32_t *mstart;
    int4 *mtile;
    int max_mt;
    int32_t *cnt;
    int ncnt;
    bool interleave;
};

struct EcPermuteArgs {
    int32_t *counts = nullptr, *offsets = nullptr, *row_token = nullptr, *slot_row = nullptr;
    TilePlanArgs plan{};
    bool prefilled = false;  // slot_row already holds -1 everywhere (written by the router)
};

// The router of a batch that fits one router block (bf16, token choice,
// T <= 16, E <= 16) can also permute its selections in that block: it writes
// what the permutation writes (counts, offsets, row_token, slot_row; the
// first `capacity` per capacity group of group_chunks chunks kept) and the
// tile plan when plan.mstart is set.
struct RoutePermuteArgs {
    int capacity = 0, group_chunks = 0;
    int32_t *counts = nullptr, *offsets = nullptr, *row_token = nullptr, *slot_row = nullptr;
    TilePlanArgs plan{};
};
bool route_permute_fits(int T, int E, bool bf16, bool expert_choice);
void launch_route_permute(const RouteArgs &a, const RoutePermuteArgs &p, hipStream_t s);
void launch_permute_small(const PermuteArgs &a, const TilePlanArgs &plan, hipStream_t s);
void launch_permute_count(const PermuteArgs &a, hipStream_t s);
void launch_permute_scan(const PermuteArgs &a, const TilePlanArgs &plan, hipStream_t s);
void launch_permute_scatter(const PermuteArgs &a, hipStream_t s);
void launch_ec_permute(const int32_t *ec_idx, int T, int E, int C, int32_t *counts, int32_t *offsets,
                       int32_t *row_token, int32_t *slot_row, hipStream_t s);
void launch_gather_rows(const void *x, const int32_t *row_token, const int32_t *offsets, int E, int64_t rows_max,
                        int d, int elem_bytes, void *x_perm, hipStream_t s);

// ---- expert FFN ----
// Tile plan: mstart[e] = sum over experts e' < e of ceil(counts[e'] / BM), mstart[E] = total.
// mstart[e] = first m-tile of expert e (exclusive scan of ceil(counts/BM)),
// mstart[E] = total; mtile[m] for every m-tile m < min(total, max_mt) =
// {mstart[g], g, offsets[g], offsets[g+1]} of its expert g.  Also clears the split-K arrival counters cnt[0 .. ncnt) (cnt may
// be null).  E <= kMaxPlanExperts.
constexpr int kMaxPlanExperts = 1024;
// interleave: light experts (fewer rows than BM) spread evenly among the
// heavy experts' m-tiles instead of expert order (build_tile_plan); only for
// layers with fewer than 1024 routed rows per expert on average.
void launch_tile_plan(const int32_t *counts, const int32_t *offsets, int E, int BM, int32_t *mstart, int4 *mtile,
                      int max_mt, int32_t *cnt, int ncnt, bool interleave, hipStream_t s);
// capacity of the m-tile table for rows routed rows over E experts (any BM >= 32)
inline int64_t max_mtiles(int64_t rows, int E) { return (rows + 31) / 32 + E; }

// Split-K workspace of the bf16 grouped GEMM: float32 partial tiles of the
// last, partial round of tiles plus one arrival counter per split tile.
constexpr int64_t kSplitUnitFloats = 256 * 256;  // largest BM x (gate + up) N tile
constexpr int kSplitSlotsPerCu = 4;              // counters per CU (several workgroups per CU)
struct SplitKWs {
    float *part;       // null: no split K
    int64_t part_floats;
    int32_t *cnt;
    int ncnt;
};
int device_cus();  // compute units of the current device

struct GemmArgs {
    const void *A;          // [rows][K] dtype (row r of group g at offsets[g] + i)
    const void *B0;         // [G][N][K] (SwiGLU: gate projection)
    const void *B1;         // [G][N][K] up projection (SwiGLU) or null
    const float *bias;      // [G][N] or null
    void *C;                // [rows][N] dtype
    const int32_t *offsets; // [G+1] or null: one group of `rows` rows
    const int32_t *mstart;  // [G+1] tile plan for the kernel's BM, or null with offsets null
    const int4 *mtile;      // m-tile table of that plan, or null with offsets null
    int max_mt;             // its capacity
    int G;                  // groups (experts)
    int64_t rows;           // rows of the single group when offsets is null; else A_max (grid bound)
    int N, K;
    int act;                // ActKind; kActSwiglu uses B1
    bool bf16;
    SplitKWs split;         // bf16 only; part null = off
    // A holds a_rows source rows, and row r of the grouped operand is A row
    // arow[r] (the routed token rows, gathered by the tile loads
    // themselves).  bf16 needs a_rows * K * 2 < 2^31 (one buffer resource).
    const int32_t *arow = nullptr;
    int64_t a_rows = 0;
    // K-sliced B (one group, not SwiGLU): B holds K / kslice matrices
    // [N][kslice] one after another, slice s supplying columns s * kslice ..
    // (s+1) * kslice - 1 of the K axis; 0 = B is [G][N][K].
    int kslice = 0;
};
enum GemmShape { kGemmPrefill = 0, kGemmSmallM = 1, kGemmDecode = 2, kGemmMid = 3 };
// Router logits of many experts as a dense GEMM: x [T][d] times wg [E][d]^T
// (E <= 256), split into S K parts whose float32 sums go to partout [S][T][E];
// launch_gate_partials adds them up and gates.
constexpr int kRouterMaxSplit = 8;
int router_gemm_split(int T, int E, int d);
void launch_router_gemm(const void *x, const void *wg, int T, int d, int E, float *partout, int S, hipStream_t s);
void launch_gate_partials(const float *part, int S, const float *bias, int T, int E, int k, int gating,
                          float *logits, int32_t *idx, float *w, hipStream_t s);
int gemm_block_m(int shape, bool bf16);
void launch_grouped_gemm(const GemmArgs &a, int shape, hipStream_t s);

// ---- combine ----
struct CombineArgs {
    const void *y_perm;    // [A_max][d]
    const void *y_shared;  // [T][d] or null
    const float *w;        // token choice: [T][k]; expert choice: [E*C] scores by row
    const int32_t *slot_row;  // [T][S]
    int T, d, S;           // S = k (token choice) or E (expert choice)
    bool expert_choice;
    bool bf16;
    void *y;               // [T][d]
};
void launch_combine(const CombineArgs &a, hipStream_t s);

}  // namespace moe
