// Grouped GEMMs of the expert FFNs on gfx950.
//
// For every expert g, the rows offsets[g] .. offsets[g+1]-1 of A (the
// expert-contiguous token rows) are multiplied by that expert's weights
// only, C = act(A_g B_g^T), so unselected experts do no work ([lecture]
// study-site lecture-03 "Mixture of Experts", section "Token Routing").
// With SwiGLU the first GEMM multiplies each A tile by the gate and the up
// projection in the same K loop and writes silu(gate) * up ([yj-zh]
// youngju.dev "Mixture of Experts（MoE）架构深度解析" SwiGLUExpert; [yj-ja]
// youngju.dev "Sparse Mixture of Experts（MoE）アーキテクチャ深層分析" SwiGLUExpert).
//
// Tiles: a device-side plan (mstart, m-tile table) lists the m-tiles of every expert; the
// grid covers the worst case and surplus blocks exit.  Inside an expert with
// Me m-tiles, tiles run in groups of Me x gN (m fastest, gN ~ 32 / Me weight
// panels; bands of 8 m-tiles when Me > 8), and every XCD receives runs of 32
// consecutive tiles: a run shares the expert's activation tiles and a few
// weight panels in that XCD's L2.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

constexpr int kXcds = 8;
constexpr int kXcdRun = 32;  // consecutive logical tiles per XCD
constexpr int kGridQuantum = kXcds * kXcdRun;

// Blocks are dispatched round-robin over the XCDs (block b -> XCD b % 8):
// the i-th block an XCD receives gets logical tile 256*(i/32) + 32*xcd + i%32.
__device__ inline int xcd_remap(int b) {
    const int xcd = b % kXcds, slot = b / kXcds;
    return (slot / kXcdRun) * kGridQuantum + xcd * kXcdRun + slot % kXcdRun;
}

struct TileCoord {
    int g, nt;
    int64_t row0, row_end;
    bool valid;
};

// Position of tile `local` among the mt x ntn tiles of one group.  A group
// of more than kBandM m-tiles is cut into bands of kBandM m-tiles (the last
// one shorter), each band's tiles in runs of kBandM x 32/kBandM; so a run of
// 32 never holds 32 m-tiles of one weight panel, which would re-read the
// group's activation rows once per panel (DeepSeek-style shared experts,
// 32 m-tiles x 16 panels: gate/up 392 -> 382 us, down 300 -> 291 us).
constexpr int kBandM = 8;
__device__ inline void group_tile(int local, int mt, int ntn, int *m, int *n) {
    int mb0 = 0;  // first m-tile of the band
    if (mt > kBandM) {
        const int b = local / (kBandM * ntn);
        mb0 = b * kBandM;
        local -= b * kBandM * ntn;
        mt = min(kBandM, mt - mb0);
    }
    int gn = kXcdRun / mt;
    if (gn < 1) gn = 1;
    const int per = mt * gn;
    const int grp = local / per, within = local % per;
    *m = mb0 + within % mt;
    *n = grp * gn + within / mt;
}

// The m-tile table holds, for every m-tile of the plan, its expert's first
// m-tile (x), the expert index (y) and the expert's rows [z, w).  Tile t of the grid belongs to m-tile t / ntn,
// so one table load (next to the total) places it; no search over experts.
// UNIT > 0: the group's rows are cut into blocks of UNIT rows, and its mt
// m-tiles take equal shares of the blocks (the first ones one more when they
// do not divide evenly), instead of BM rows each and the remainder last.  An
// expert of 1030 rows then runs five tiles of 13 row blocks of 16 instead of
// four full tiles and one of 6 rows; with the row-block skip the padding
// MFMAs all but vanish and the tiles of a group stay equally long.
template <int BM, int UNIT = 0>
__device__ inline TileCoord find_tile(int tile, const int32_t *offsets, const int32_t *mstart, const int4 *mtile,
                                      int max_mt, int G, int64_t rows, int ntn) {
    TileCoord c;
    c.valid = false;
    int m, n;
    if (offsets == nullptr) {
        const int mtiles = (int)((rows + BM - 1) / BM);
        if (tile >= mtiles * ntn) return c;
        group_tile(tile, mtiles, ntn, &m, &n);
        c.g = 0;
        c.nt = n;
        c.row0 = (int64_t)m * BM;
        c.row_end = rows;
        c.valid = true;
        return c;
    }
    const int mt = tile / ntn;
    const int4 info = mtile[mt < max_mt ? mt : max_mt - 1];
    const int total = mstart[G];
    if (tile >= total * ntn) return c;
    const int local = tile - info.x * ntn;
    const int mt_g = (int)((info.w - info.z + BM - 1) / BM);
    group_tile(local, mt_g, ntn, &m, &n);
    c.g = info.y;
    c.nt = n;
    if constexpr (UNIT > 0) {
        // blocks <= mt_g * BM / UNIT, so no m-tile gets more than BM rows
        const int nblk = (info.w - info.z + UNIT - 1) / UNIT;
        const int q = nblk / mt_g, r = nblk % mt_g;
        c.row0 = info.z + (int64_t)UNIT * (m * q + min(m, r));
        c.row_end = min((int64_t)info.w, info.z + (int64_t)UNIT * ((m + 1) * q + min(m + 1, r)));
    } else {
        c.row0 = info.z + (int64_t)m * BM;
        c.row_end = info.w;
    }
    c.valid = true;
    return c;
}


struct GemmParams {
    const bf16 *A;
    const bf16 *B0;
    const bf16 *B1;
    const float *bias;
    bf16 *C;
    const int32_t *offsets;
    const int32_t *mstart;
    const int4 *mtile;  // m-tile table of the plan (offsets non-null)
    int max_mt;         // its capacity
    int G;
    int64_t rows;
    int N, K;
    int act;
    // split K of the last, partial round of tiles (null part: off)
    float *part;      // [slots][BM * NB] float32 partial accumulators
    int32_t *cnt;     // [slots] arrival counters, zero between launches
    int slots;        // workgroups resident at once
    int max_split;    // at most this many K parts per tile
    int max_slabs;    // partial tiles the part area holds
    // gathered A: row r of the grouped operand is row arow[r] of A, whose
    // a_bytes bytes one buffer resource covers (null: rows in place)
    const int32_t *arow;
    int64_t a_bytes;
    // K-sliced B (one group): K = (K / kslice) slices of kslice, slice s a
    // [N][kslice] matrix at B0 + s * N * kslice; 0 = B is [N][K]
    int kslice;
    // float32 partial products (one group, the router's logits): every tile
    // is split into fixed_split K parts, and part q writes its [rows][N]
    // float32 sums to partout + q * rows * N (no activation, no epilogue)
    float *partout;
    int fixed_split;
};

// Work item of one workgroup.  The tiles fill rounds of `slots` workgroups;
// when the last round is partial (rem tiles), each of its tiles is split into
// S = slots / rem parts along K, so that the last round is as wide as the
// others and each part runs 1/S of the K loop.  The parts of a tile are
// consecutive logical indices, mostly inside one run of 32 (one XCD); their
// partial sums are written and read at device scope, so parts that straddle
// two XCDs are as correct.  rem * S may exceed the slots: the launch adds
// workgroups for every part.
struct WorkItem {
    int tile;    // logical tile
    int part;    // K part (0 when not split)
    int S;       // K parts of this tile
    int unit;    // index of the split tile among the split ones (S > 1)
    bool valid;
};

__device__ inline WorkItem work_item(int w, int ntiles, const GemmParams &p) {
    WorkItem it{w, 0, 1, 0, w < ntiles};
    if (p.fixed_split > 0) {  // every tile in fixed_split K parts, consecutive work items
        it.tile = w / p.fixed_split;
        it.part = w % p.fixed_split;
        it.S = p.fixed_split;
        it.valid = it.tile < ntiles;
        return it;
    }
    if (p.part == nullptr || ntiles <= 0) return it;
    const int rem = ntiles % p.slots;
    if (rem == 0) return it;
    // The part count S minimises the split tiles' makespan, ceil(rem*S /
    // slots) rounds of 1/S of a tile (any count, not only powers of two:
    // the Mixtral-shape down projection's last round of 80 tiles takes 3
    // parts, 1043 -> 980 us).
    int S = 1, best_r = 1, best_s = 1;
    for (int s = 2; s <= p.max_split && rem * s <= p.max_slabs; ++s) {
        const int r = (rem * s + p.slots - 1) / p.slots;
        if (r * best_s < best_r * s) {
            best_r = r;
            best_s = s;
            S = s;
        }
    }
    if (S < 2) return it;
    const int full = ntiles - rem;
    if (w < full) return it;
    const int u = w - full;
    it.valid = u < rem * S;
    it.unit = u / S;
    it.tile = full + it.unit;
    it.part = u % S;
    it.S = S;
    return it;
}

__device__ inline int total_tiles(int BM, int ntn, const int32_t *offsets, const int32_t *mstart, int G,
                                  int64_t rows) {
    if (offsets == nullptr) return (int)((rows + BM - 1) / BM) * ntn;
    return mstart[G] * ntn;
}

// Calls f(std::integral_constant<int, NA>) with NA = min(n, TM), n >= 0.
template <int NA, int TM, typename F>
__device__ inline void dispatch_active(int n, F &&f) {
    if constexpr (NA >= TM) {
        f(std::integral_constant<int, TM>{});
    } else {
        if (n <= NA) f(std::integral_constant<int, NA>{});
        else dispatch_active<NA + 1, TM>(n, f);
    }
}

// Two K tiles are in flight in registers (loads issued two steps ahead) and
// the MFMA fragments are double-buffered.  m-tiles are balanced (find_tile
// with UNIT = MF), and in a tile of fewer than BM rows each wave runs only
// the MFMAs of its row blocks that hold rows.
// IL: 0 = compiler schedule; 1 = the next substep's LDS reads interleaved
// 1:1 with this substep's MFMAs.
// MF: MFMA tile edge, 32 (v_mfma_f32_32x32x16_bf16) or 16
// (v_mfma_f32_16x16x32_bf16).  Both give the same flops per cycle, but with
// switching operands the 16x16x32 form sustains more flops under the socket
// power limit (2.06 vs 1.79 PFLOP/s in a register-only loop; 2.5% on the
// whole grouped GEMM).
// RMAP: waves w and w + 4, which share a SIMD, take different row halves (wm)
// instead of the same one.  JOUT: MFMA order with the B fragment in the outer
// loop (each B fragment feeds NA MFMAs in a row, the A fragments change every
// MFMA) instead of the A fragment.
// SL: B is K-sliced (p.kslice > 0): the rows of each K tile are read from
// its slice (the shared experts' down projections side by side along K).
// PO: float32 partial products out (p.partout, p.fixed_split): each work
// item writes its K part's sums and ends there.
template <int BM, int BN, int WM, int WN, bool GLU, int IL = 0, int MF = 32, bool RMAP = false, int BK = 64,
          bool JOUT = false, bool SL = false, bool PO = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(GemmParams p) {
    constexpr int NT = 64 * WM * WN;  // threads
    static_assert(BK == 64 || BK == 128, "K tile");
    constexpr int KCH = BK / 8;  // 16-byte chunks per LDS operand row
    constexpr int NB = GLU ? 2 * BN : BN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    static_assert(MF == 32 || MF == 16, "MFMA shape");
    constexpr int KSUB = MF == 32 ? 16 : 32;   // k per MFMA
    constexpr int NSUB = BK / KSUB;            // k-substeps per K tile
    constexpr int AR = MF * MF / 64;           // accumulator registers per MFMA tile
    using acc_t = float __attribute__((ext_vector_type(AR)));
    constexpr int TM = WTM / MF, TN = WTN / MF;
    constexpr int TB = GLU ? 2 * TN : TN;  // B fragments per k-substep (gate then up)
    constexpr int RSTEP = NT / KCH;        // rows between a thread's successive 16-byte chunks
    constexpr int A_PER_T = BM / RSTEP, B_PER_T = NB / RSTEP;
    constexpr int FS = 2;                  // fragment register sets
    static_assert(A_PER_T >= 1 && B_PER_T >= 1 && BM % RSTEP == 0 && NB % RSTEP == 0, "tile/threads");
    static_assert(RSTEP % 16 == 0, "a thread's rows share one LDS swizzle");
    static_assert(!GLU || BN % RSTEP == 0, "gate/up split must fall between a thread's chunks");
    static_assert(TM >= 1 && TN >= 1, "wave tile");
    __shared__ __attribute__((aligned(16))) bf16 lds[2][(BM + NB) * BK];
    __shared__ int last_part;

    const int ntn = (p.N + BN - 1) / BN;
    const WorkItem wi = work_item(xcd_remap(blockIdx.x),
                                  total_tiles(BM, ntn, p.offsets, p.mstart, p.G, p.rows), p);
    if (!wi.valid) return;
    const TileCoord tc = find_tile<BM, MF>(wi.tile, p.offsets, p.mstart, p.mtile, p.max_mt, p.G,
                                                        p.rows, ntn);
    if (!tc.valid) return;
    const int n0 = tc.nt * BN;
    const int64_t K = p.K;
    // K tiles [kbeg, kbeg + KT) of this work item
    const int KT_all = p.K / BK;
    const int kbeg = (int)((int64_t)KT_all * wi.part / wi.S);
    const int KT = (int)((int64_t)KT_all * (wi.part + 1) / wi.S) - kbeg;

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int wm = RMAP ? wave / WN : wave % WM, wn = RMAP ? wave % WN : wave / WM;
    // MF-row blocks of this wave that hold rows of the tile: in a tile of
    // fewer than BM rows a wave runs the MFMAs (and A-fragment reads) of only
    // its first NA blocks; the blocks past them lie wholly past the tile's
    // last row.
    const int64_t wrows = tc.row_end - (tc.row0 + (int64_t)wm * WTM);
    const int nact = wrows <= 0 ? 0 : (wrows >= WTM ? TM : (int)((wrows + MF - 1) / MF));

    // Loads: buffer loads from uniform tile bases with 32-bit per-chunk byte
    // offsets; the K offset goes in the scalar offset.  The byte limit of
    // each buffer ends at the expert's last row (A) or the matrix's last row
    // (B), so rows past it read as zeros: padding rows of a partial tile feed
    // the MFMAs zeros rather than copies of real rows, which keeps their
    // switching power low.  Thread tid moves chunk (tid % KCH) of rows
    // tid/KCH + RSTEP*i.
    const int r0 = tid / KCH, ch0 = tid % KCH;
    const int64_t k0 = (int64_t)kbeg * BK;
    // Gathered A: one resource over all of A and a per-row byte offset from
    // the row map; padding rows get an offset past the limit (zeros).
    static_assert(!(SL && GLU), "K-sliced B is for the down projection");
    const char *abase = p.arow ? (const char *)(p.A + k0) : (const char *)(p.A + tc.row0 * K + k0);
    // B row stride: K, or the slice width (then every K offset, k0 included,
    // goes into the per-tile scalar offset)
    const int64_t bstride = SL ? p.kslice : K;
    const char *b0base = SL ? (const char *)(p.B0 + (int64_t)n0 * bstride)
                            : (const char *)(p.B0 + ((int64_t)tc.g * p.N + n0) * K + k0);
    const char *b1base = GLU ? (const char *)(p.B1 + ((int64_t)tc.g * p.N + n0) * K + k0) : nullptr;
    const __amdgpu_buffer_rsrc_t arsrc =
        buffer_rsrc(abase, p.arow ? p.a_bytes - k0 * 2 : (tc.row_end - tc.row0) * K * 2);
    const __amdgpu_buffer_rsrc_t b0rsrc =
        buffer_rsrc(b0base, SL ? ((K / bstride) * p.N - n0) * bstride * 2 : (int64_t)(p.N - n0) * K * 2);
    const __amdgpu_buffer_rsrc_t b1rsrc = GLU ? buffer_rsrc(b1base, (int64_t)(p.N - n0) * K * 2) : b0rsrc;
    // byte offset of K tile kt (of this work item) inside B: its slice, then
    // its column.  The slice width is a multiple of BK, and all of B spans
    // less than 2^31 bytes, so 32-bit tile arithmetic suffices (a 64-bit
    // division per K tile had cost the 256-row kernel 103 spilled VGPRs).
    const int tps = SL ? p.kslice / BK : 1;              // K tiles per slice
    const int slice_bytes = SL ? p.N * p.kslice * 2 : 0;  // bytes per slice
    auto bk_off = [&](int kt) {
        if constexpr (SL) {
            const int t = kbeg + kt;
            return (t / tps) * slice_bytes + (t % tps) * (BK * 2);
        } else {
            return kt * BK * 2;
        }
    };
    uint32_t aoff[A_PER_T], boff[B_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
        const int64_t r = r0 + RSTEP * i;
        if (p.arow == nullptr) aoff[i] = (uint32_t)((r * K + ch0 * 8) * 2);
        else aoff[i] = (tc.row0 + r < tc.row_end ? (uint32_t)(p.arow[tc.row0 + r] * K * 2) : 0x80000000u) + ch0 * 16;
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
        int r = r0 + RSTEP * i;
        if (GLU && r >= BN) r -= BN;
        boff[i] = (uint32_t)(((int64_t)r * bstride + ch0 * 8) * 2);
    }
    // LDS: chunk c of row r sits at chunk slot c ^ swz(r); swz is the same for
    // all of a thread's rows (they differ by multiples of 16), so one base
    // address plus compile-time strides covers them.
    const int sdst = r0 * BK + ((ch0 ^ swz_k<BK>(r0)) * 8);
    // MFMA operand lanes: lane l holds row (l % MF) of a fragment and the
    // 16-byte k chunk l / MF of the k-substep; rows of one wave's fragments
    // differ by multiples of 16, so they share one swizzle.
    const int sw_a = swz_k<BK>(wm * WTM + lane % MF);
    const int sw_b = swz_k<BK>(wn * WTN + lane % MF);
    const int fa0 = (wm * WTM + lane % MF) * BK, fb0 = (BM + wn * WTN + lane % MF) * BK;

    acc_t acc[TM][TB];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = acc_t{};

    // Two register sets keep two K tiles in flight (prefetch distance 2); the
    // loads are issued unconditionally (the tail re-reads the last tile) so the
    // compiler's wait counts stay exact.  Two LDS buffers alternate: while the
    // MFMAs consume one, the next tile is stored into the other.
    u32x4 ra[2][A_PER_T], rb[2][B_PER_T];
    auto gload = [&](int kt, int set) {
        const int ko = kt * BK * 2, kob = bk_off(kt);
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) ra[set][i] = buffer_load16(arsrc, aoff[i], ko);
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const bool up = GLU && RSTEP * i >= BN;
            rb[set][i] = buffer_load16(up ? b1rsrc : b0rsrc, boff[i], kob);
        }
    };
    auto lstore = [&](int buf, int set) {
        bf16 *L = lds[buf];
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) store16(L + sdst + i * RSTEP * BK, ra[set][i]);
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) store16(L + BM * BK + sdst + i * RSTEP * BK, rb[set][i]);
    };
    bf16x8 fa[FS][TM], fb[FS][TB];
    auto fload = [&](const bf16 *L, int ks, int slot, auto na) {
        constexpr int NA = decltype(na)::value;
        const int ch = ks * (KSUB / 8) + lane / MF;
        const bf16 *La = L + fa0 + ((ch ^ sw_a) * 8);
        const bf16 *Lb = L + fb0 + ((ch ^ sw_b) * 8);
#pragma unroll
        for (int i = 0; i < NA; ++i) fa[slot][i] = __builtin_bit_cast(bf16x8, load16(La + i * MF * BK));
#pragma unroll
        for (int j = 0; j < TB; ++j)
            fb[slot][j] = __builtin_bit_cast(bf16x8,
                                             load16(Lb + ((j >= TN ? BN : 0) + (j % TN) * MF) * BK));
    };
    auto mfma = [&](int slot, int i, int j) {
        if constexpr (MF == 32)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
        else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
    };
    auto mfmas = [&](int slot, auto na) {
        constexpr int NA = decltype(na)::value;
        if constexpr (JOUT) {
#pragma unroll
            for (int j = 0; j < TB; ++j)
#pragma unroll
                for (int i = 0; i < NA; ++i) mfma(slot, i, j);
        } else {
#pragma unroll
            for (int i = 0; i < NA; ++i)
#pragma unroll
                for (int j = 0; j < TB; ++j) mfma(slot, i, j);
        }
    };
    // MFMAs of one K tile whose k-substep-0 fragments are already in slot 0:
    // each substep first loads the next substep's fragments into the other
    // slot, then runs its MFMAs
    auto compute = [&](const bf16 *L, auto na) {
        constexpr int NA = decltype(na)::value;
#pragma unroll
        for (int ks = 0; ks < NSUB; ++ks) {
            if (ks + 1 < NSUB) fload(L, ks + 1, (ks + 1) & 1, na);
            mfmas(ks & 1, na);
            if constexpr (IL == 1) {
                if (ks + 1 < NSUB) {
#pragma unroll
                    for (int g = 0; g < NA + TB; ++g) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // The K loop with the MFMA work of the first NA row blocks of this wave
    // (the loads, LDS stores and barriers are the same for every NA, so every
    // wave meets every barrier).
    auto kloop = [&](auto na) {
        constexpr bool MMA = decltype(na)::value > 0;
        gload(0, 0);
        gload(KT > 1 ? 1 : 0, 1);
        lstore(0, 0);
        __syncthreads();
        // Pairs of K tiles with no control flow inside, so the compiler's wait
        // counts see exactly one register set in flight when the other is
        // stored.  Loads and stores past the last tile re-read and re-store
        // tile KT-1 into a buffer nobody reads afterwards.
        int kt = 0;
        for (; kt + 1 < KT; kt += 2) {
            // even step: LDS buffer 0 holds tile kt, register set 1 holds tile kt+1
            gload(min(kt + 2, KT - 1), 0);
            if constexpr (MMA) fload(lds[0], 0, 0, na);
            lstore(1, 1);
            if constexpr (MMA) compute(lds[0], na);
            __syncthreads();
            // odd step: LDS buffer 1 holds tile kt+1, register set 0 holds tile kt+2 (or KT-1)
            gload(min(kt + 3, KT - 1), 1);
            if constexpr (MMA) fload(lds[1], 0, 0, na);
            lstore(0, 0);
            if constexpr (MMA) compute(lds[1], na);
            __syncthreads();
        }
        if (kt < KT) {  // odd tile count: the last tile is in LDS buffer 0
            if constexpr (MMA) {
                fload(lds[0], 0, 0, na);
                compute(lds[0], na);
            }
        }
    };
    dispatch_active<0, TM>(nact, kloop);

    if constexpr (PO) {
        // accumulator r of an MFMA tile holds D[row][lane % MF] with row =
        // 8*(r/4) + 4*(lane/32) + r%4 (32x32) or 4*(lane/16) + r (16x16)
        static_assert(!GLU, "partial products of one projection");
        float *out = p.partout + (int64_t)wi.part * p.rows * p.N;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int col = n0 + wn * WTN + j * MF + lane % MF;
#pragma unroll
                for (int r = 0; r < AR; ++r) {
                    const int64_t row = tc.row0 + wm * WTM + i * MF +
                                        (MF == 32 ? 8 * (r / 4) + 4 * (lane / 32) + r % 4 : 4 * (lane / 16) + r);
                    if (row < tc.row_end && col < p.N) out[row * p.N + col] = acc[i][j][r];
                }
            }
        return;
    }

    if (wi.S > 1) {
        // Publish this part's accumulators; the last part to arrive adds the
        // S parts in part order (the sum does not depend on arrival order)
        // and runs the epilogue.  Layout: 16-byte chunk q4 of acc[i][j] of
        // thread tid at ((i * TB + j) * (AR / 4) + q4) * NT + tid.
        //
        // The parts may run on different XCDs, whose L2s are not coherent
        // with each other.  The partials are therefore written and read at
        // device scope (sc1: stores written through to the device coherence
        // point, loads served from it), and each thread waits for its stores
        // to complete before the workgroup barrier and the arrival count.
        // This avoids a device-scope fence, which writes back this XCD's
        // whole L2 and serialised badly when many parts arrive together
        // (Mixtral-shape prefill: gate/up 1760 -> 1715 us, down 927 -> 864
        // us; 32-row decode tiles: 160 -> 348 us with the fence).
        constexpr int PER_UNIT = BM * NB;
        constexpr int kDeviceScope = 16;  // cache policy: sc1
        const float *parts = p.part + (int64_t)wi.unit * wi.S * PER_UNIT;
        const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(parts, (int64_t)wi.S * PER_UNIT * 4);
        const int mine = wi.part * PER_UNIT * 4;  // byte offset of this part's slab
        // Row blocks past the tile's rows (i >= nact, the same in every part
        // of the tile) hold zeros and are neither written nor read.
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= nact) continue;
#pragma unroll
            for (int j = 0; j < TB; ++j)
#pragma unroll
                for (int q4 = 0; q4 < AR / 4; ++q4) {
                    const f32x4 v = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2],
                                     acc[i][j][4 * q4 + 3]};
                    const int o = (((i * TB + j) * (AR / 4) + q4) * NT + tid) * 16;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), prs, o, mine, kDeviceScope);
                }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores are complete
        __syncthreads();
        if (tid == 0) last_part = atomicAdd(p.cnt + wi.unit, 1) == wi.S - 1;
        __syncthreads();
        if (!last_part) return;
        // parts added in part order; this part's own sums come from its
        // registers (the same values it wrote), so it reads S - 1 slabs
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (i >= nact) continue;
#pragma unroll
            for (int j = 0; j < TB; ++j)
#pragma unroll
                for (int q4 = 0; q4 < AR / 4; ++q4) {
                    const int o = (((i * TB + j) * (AR / 4) + q4) * NT + tid) * 16;
                    const f32x4 own = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2],
                                       acc[i][j][4 * q4 + 3]};
                    auto term = [&](int sp) __attribute__((always_inline)) {
                        return sp == wi.part ? own
                                             : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                             prs, o, sp * PER_UNIT * 4, kDeviceScope));
                    };
                    f32x4 v = term(0);
                    for (int sp = 1; sp < wi.S; ++sp) v += term(sp);
                    acc[i][j][4 * q4] = v[0];
                    acc[i][j][4 * q4 + 1] = v[1];
                    acc[i][j][4 * q4 + 2] = v[2];
                    acc[i][j][4 * q4 + 3] = v[3];
                }
        }
        if (tid == 0) p.cnt[wi.unit] = 0;  // ready for the next launch
    }

    // Epilogue: the activated tile goes through LDS (free after the K loop)
    // so that the global stores are whole 16-byte chunks of rows.
    // Accumulator r of an MFMA tile holds D[row][lane % MF] with
    // row = 8*(r/4) + 4*(lane/32) + r%4 (32x32) or 4*(lane/16) + r (16x16):
    // each group of four accumulators is four consecutive rows of one column.
    // Lanes l and l^1 hold adjacent columns; they trade two values (DPP quad
    // permutation 1,0,3,2) so that the even lane owns rows +0,+1 and the odd
    // lane rows +2,+3 of both columns, and each writes bf16 pairs (4 bytes).
    // LDS: BM rows of BN bf16; 16-byte chunk c of row r at slot c ^ ((r/2) % 8),
    // so the eight rows one write instruction touches hit distinct banks.
    static_assert(BM * BN * 2 <= (int)sizeof(lds), "output tile fits in the staging buffers");
    static_assert(BN % 64 == 0, "at least eight 16-byte chunks per output row");
    constexpr int CPR = BN / 8;  // 16-byte chunks per output row
    bf16 *Ct = &lds[0][0];
    const float *bias = p.bias ? p.bias + (int64_t)tc.g * p.N : nullptr;
    const bool odd = lane & 1;
    auto swap1 = [](float x) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    };
    __syncthreads();  // every wave is done with the operand tiles
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int cl = wn * WTN + j * MF + lane % MF;  // column inside the tile
            const float bcol = bias && n0 + cl < p.N ? bias[n0 + cl] : 0.f;
#pragma unroll
            for (int g = 0; g < AR / 4; ++g) {
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v[r] = acc[i][j][4 * g + r];
                    if constexpr (GLU) v[r] = silu_fast(v[r]) * acc[i][TN + j][4 * g + r];
                    else v[r] = apply_act(p.act, v[r] + bcol);
                }
                const float xs = swap1(odd ? v[0] : v[2]), ys = swap1(odd ? v[1] : v[3]);
                const int rb = wm * WTM + i * MF + (MF == 32 ? 8 * g + 4 * (lane / 32) : 4 * (lane / 16));
                const int ra0 = rb + (odd ? 2 : 0), ra1 = ra0 + 1;
                const int ce = cl & ~1;  // even column of the pair
                const bf16x2 p0 = {(bf16)(odd ? xs : v[0]), (bf16)(odd ? v[2] : xs)};
                const bf16x2 p1 = {(bf16)(odd ? ys : v[1]), (bf16)(odd ? v[3] : ys)};
                *(bf16x2 *)(Ct + ra0 * BN + (((ce / 8) ^ ((ra0 / 2) & 7)) * 8) + ce % 8) = p0;
                *(bf16x2 *)(Ct + ra1 * BN + (((ce / 8) ^ ((ra1 / 2) & 7)) * 8) + ce % 8) = p1;
            }
        }
    __syncthreads();
    for (int q = tid; q < BM * CPR; q += NT) {
        const int rl = q / CPR, c = q % CPR;
        const int64_t row = tc.row0 + rl;
        const int col = n0 + c * 8;
        if (row < tc.row_end && col < p.N)
            store16(p.C + row * p.N + col, load16(Ct + rl * BN + ((c ^ ((rl / 2) & 7)) * 8)));
    }
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes bytes
// 16 l .. 16 l + 15 after the wave-uniform LDS address `dst` (one wave
// instruction fills 1 KiB); offsets at or past the buffer's limit write zeros.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, bf16 *dst, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

// GEMMs of the 256-row tiles with their operands loaded from global memory
// straight into LDS (buffer_load_dwordx4 ... lds), so that no registers
// stage them: the register-staged kernel above spends 64 VGPRs a thread on
// its two load sets.  GLU: the SwiGLU gate/up GEMM, each tile 128 outputs
// of gate and of up; else the plain down projection (no bias, no
// activation), each tile 256 outputs.  8 waves (2 per SIMD) in 2 (rows) x 4
// (columns); each wave 128 rows x 64 B rows (32 gate + 32 up, or 64) on
// v_mfma_f32_16x16x32_bf16, with the fragments double-buffered.  Waves w and
// w + 4, which share a SIMD, take different row halves, and in a tile of
// fewer than BM rows each wave runs only its row blocks that hold rows (as
// above).  Each load instruction fills RPI whole LDS rows, and every lane
// fetches the 16-byte chunk that its swizzled slot holds.
//
// Two LDS buffers, one barrier per K tile (two k-substeps of 32):
//   1. the MFMAs of substep 0 (fragments in slot 0), with the fragment
//      reads of substep 1 into slot 1 between them;
//   2. wait for this wave's loads of tile kt+1 and its reads of tile kt;
//      barrier, so every wave's loads have landed and every wave has read
//      tile kt;
//   3. the MFMAs of substep 1, with the loads of tile kt+2 into tile kt's
//      buffer and the substep-0 reads of tile kt+1 into slot 0 between them.
// The program order of each MFMA batch is pinned in groups (sched_barrier):
// group g issues load g, then fragment reads 3g .. 3g+2, then its share of
// the MFMAs (B fragment in the outer loop).  K runs in pairs of K tiles, so
// K % 128 == 0, and split parts cut on pairs.
//
// Alternating launches against the register-staged kernel: Mixtral-shape
// gate/up 1703 -> 1606 us, DeepSeek-style shared experts 392 -> 341 us,
// DeepSeek-style routed gate/up unchanged (4391 -> 4435 us).  Fragment reads
// 2 or 4 per group instead of 3: 1% and 4% slower.  The down projection on
// this schedule first gained nothing (880 -> 888 us); with the wave priority
// of the post-barrier batch (below) it runs 928 -> 858 us.
template <int BM, int BN, bool GLU>
__global__ __launch_bounds__(512) void gemm_lds_kernel(GemmParams p) {
    constexpr int WM = 2, WN = 4, NT = 64 * WM * WN, NW = WM * WN;
    // B rows of a tile: BN gate rows, then BN up rows (GLU), or BN rows
    constexpr int BK = 64, NB = GLU ? 2 * BN : BN;
    constexpr int WTM = BM / WM, WTB = NB / WN;
    constexpr int MF = 16, KSUB = 32;
    // TN: output column blocks of a wave
    constexpr int TM = WTM / MF, TB = WTB / MF, TN = GLU ? TB / 2 : TB;
    constexpr int KCH = BK / 8, RPI = 64 / KCH;          // 16-byte chunks a row; rows a load instruction fills
    constexpr int AI = BM / RPI / NW, BI = NB / RPI / NW;  // load instructions per wave and K tile
    constexpr int RPG = 3;                                 // fragment reads per group
    static_assert(AI >= 1 && BI >= 1 && BK / KSUB == 2, "tile");
    static_assert(!GLU || BN % (BI * RPI) == 0, "a wave's B load rows lie in one of gate / up");
    // two LDS objects, so that the compiler sees that the fragment reads of
    // one buffer do not alias the direct loads into the other
    __shared__ __attribute__((aligned(16))) bf16 lds0[(BM + NB) * BK];
    __shared__ __attribute__((aligned(16))) bf16 lds1[(BM + NB) * BK];
    __shared__ int last_part;

    const int ntn = (p.N + BN - 1) / BN;
    const WorkItem wi = work_item(xcd_remap(blockIdx.x), total_tiles(BM, ntn, p.offsets, p.mstart, p.G, p.rows), p);
    if (!wi.valid) return;
    const TileCoord tc = find_tile<BM, MF>(wi.tile, p.offsets, p.mstart, p.mtile, p.max_mt, p.G, p.rows, ntn);
    if (!tc.valid) return;
    const int n0 = tc.nt * BN;
    const int64_t K = p.K;
    const int KP_all = p.K / (2 * BK);
    const int kbeg = 2 * (int)((int64_t)KP_all * wi.part / wi.S);
    const int KT = 2 * (int)((int64_t)KP_all * (wi.part + 1) / wi.S) - kbeg;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t wrows = tc.row_end - (tc.row0 + (int64_t)wm * WTM);
    const int nact = wrows <= 0 ? 0 : (wrows >= WTM ? TM : (int)((wrows + MF - 1) / MF));

    // buffer resources and byte offsets as in the register-staged kernel
    const int64_t k0 = (int64_t)kbeg * BK;
    const char *abase = p.arow ? (const char *)(p.A + k0) : (const char *)(p.A + tc.row0 * K + k0);
    const __amdgpu_buffer_rsrc_t arsrc =
        buffer_rsrc(abase, p.arow ? p.a_bytes - k0 * 2 : (tc.row_end - tc.row0) * K * 2);
    const bool bup = GLU && wave * BI * RPI >= BN;  // this wave loads up rows (else gate rows)
    const bf16 *bmat = bup ? p.B1 : p.B0;
    const __amdgpu_buffer_rsrc_t brsrc =
        buffer_rsrc(bmat + ((int64_t)tc.g * p.N + n0) * K + k0, (int64_t)(p.N - n0) * K * 2);
    // lane L of a load instruction fills LDS row RPI*q + L/KCH, slot L%KCH,
    // with the global chunk that slot holds: chunk = slot ^ swz(row)
    const int lrow = lane / KCH, lslot = lane % KCH;
    uint32_t aoff[AI], boff[BI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int r = (wave * AI + i) * RPI + lrow;
        const int c = lslot ^ swz_k<BK>(r);
        if (p.arow == nullptr) aoff[i] = (uint32_t)(((int64_t)r * K + c * 8) * 2);
        else aoff[i] = (tc.row0 + r < tc.row_end ? (uint32_t)(p.arow[tc.row0 + r] * K * 2) : 0x80000000u) + c * 16;
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const int r = (wave * BI + i) * RPI + lrow;  // LDS B row
        const int c = lslot ^ swz_k<BK>(r);
        boff[i] = (uint32_t)(((int64_t)(GLU ? r % BN : r) * K + c * 8) * 2);
    }
    auto load_a = [&](bf16 *L, int i, int ko) __attribute__((always_inline)) {
        buffer_load16_lds(arsrc, L + (wave * AI + i) * RPI * BK, aoff[i], ko);
    };
    auto load_b = [&](bf16 *L, int i, int ko) __attribute__((always_inline)) {
        buffer_load16_lds(brsrc, L + BM * BK + (wave * BI + i) * RPI * BK, boff[i], ko);
    };
    auto issue = [&](int kt, bf16 *L) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < AI; ++i) load_a(L, i, kt * BK * 2);
#pragma unroll
        for (int i = 0; i < BI; ++i) load_b(L, i, kt * BK * 2);
    };
    // fragment lanes: row lane % 16 of each 16-row block, 16-byte k chunk
    // lane / 16 of a 32-k substep; B rows: gate wn*32 .., up BN + wn*32 ..
    const int sw_a = swz_k<BK>(wm * WTM + lane % MF);
    const int sw_b = swz_k<BK>(wn * TN * MF + lane % MF);
    const int fa0 = (wm * WTM + lane % MF) * BK;
    const int fb0 = (BM + wn * TN * MF + lane % MF) * BK;
    auto bofs = [](int j) __attribute__((always_inline)) {
        return GLU ? ((j >= TN ? BN : 0) + (j % TN) * MF) * BK : j * MF * BK;
    };

    f32x4 acc[TM][TB];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = f32x4{};
    bf16x8 fa[2][TM], fb[2][TB];
    // one MFMA batch (substep of slot ms), with the fragment reads of slot
    // rs (buffer R, substep rks) and, if LOADS, the loads of tile ldkt into
    // LD between its MFMAs
    auto batch = [&](const bf16 *R, int rks, int rs, int ms, bf16 *LD, int ldkt, auto na, auto loads)
                     __attribute__((always_inline)) {
        constexpr int NA = decltype(na)::value;
        constexpr int NR = NA + TB, NM = NA * TB, NL = decltype(loads)::value ? AI + BI : 0;
        constexpr int NG = NR > NL ? NR : NL;
        constexpr int PER = (NM + NG - 1) / NG;
        const int ch = rks * (KSUB / 8) + lane / MF;
        const bf16 *La = R + fa0 + ((ch ^ sw_a) * 8);
        const bf16 *Lb = R + fb0 + ((ch ^ sw_b) * 8);
        // The batch after the barrier (the one with the loads) runs at wave
        // priority 1 and every batch ends at 0: a wave still in that batch
        // wins the issue slot over its SIMD partner that has moved on to the
        // next K tile's first batch, which keeps the two waves of a SIMD in
        // step for the next barrier.  Alternating launches (Mixtral-shape
        // gate/up): 1652 -> 1582 us; priority in the other batch instead:
        // +3.6%; in both: +2.5%; in the register-staged down projection
        // (whole batch, first substep, or barrier to first substep): +74%,
        // +17%, +1%.
        if constexpr (decltype(loads)::value) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g < NL) {
                if (g < AI) load_a(LD, g, ldkt * BK * 2);
                else load_b(LD, g - AI, ldkt * BK * 2);
            }
#pragma unroll
            for (int r = g * RPG; r < (g + 1) * RPG && r < NR; ++r) {
                if (r < NA) fa[rs][r] = __builtin_bit_cast(bf16x8, load16(La + r * MF * BK));
                else fb[rs][r - NA] = __builtin_bit_cast(bf16x8, load16(Lb + bofs(r - NA)));
            }
#pragma unroll
            for (int q = g * PER; q < (g + 1) * PER && q < NM; ++q)
                acc[q % NA][q / NA] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ms][q % NA], fb[ms][q / NA],
                                                                               acc[q % NA][q / NA], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };
    // K tile kt in buffer L, tile kt+1 landing in Lo; substep 0's fragments
    // of tile kt are in slot 0
    auto step = [&](bf16 *L, bf16 *Lo, int kt, auto na) __attribute__((always_inline)) {
        constexpr bool MMA = decltype(na)::value > 0;
        if constexpr (MMA) {
            // slot 0's reads (issued a whole batch ago) are complete; saying
            // so here keeps the compiler from waiting on the reads it issues
            // next (the LDS counter saturates at 15 outstanding)
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            __builtin_amdgcn_sched_barrier(0);
            batch(L, 1, 1, 0, L, 0, na, std::false_type{});
        }
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
        __syncthreads();
        // past the last tile the loads re-read tile KT-1 into a buffer that
        // nobody reads afterwards (no branches around the loads)
        if constexpr (MMA) batch(Lo, 0, 0, 1, L, min(kt + 2, KT - 1), na, std::true_type{});
        else issue(min(kt + 2, KT - 1), L);
    };
    // the K loop with the MFMA work of the first NA row blocks of this wave
    // (loads and barriers are the same for every NA)
    auto kloop = [&](auto na) __attribute__((always_inline)) {
        constexpr int NA = decltype(na)::value;
        issue(0, lds0);
        issue(min(1, KT - 1), lds1);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (AI + BI));  // vmcnt(AI+BI): tile 0 landed
        __syncthreads();
        if constexpr (NA > 0) {
            const bf16 *La = lds0 + fa0 + (((lane / MF) ^ sw_a) * 8);
            const bf16 *Lb = lds0 + fb0 + (((lane / MF) ^ sw_b) * 8);
#pragma unroll
            for (int i = 0; i < NA; ++i) fa[0][i] = __builtin_bit_cast(bf16x8, load16(La + i * MF * BK));
#pragma unroll
            for (int j = 0; j < TB; ++j) fb[0][j] = __builtin_bit_cast(bf16x8, load16(Lb + bofs(j)));
        }
        for (int kt = 0; kt < KT; kt += 2) {
            step(lds0, lds1, kt, na);
            step(lds1, lds0, kt + 1, na);
        }
        __builtin_amdgcn_s_waitcnt(0x0070);  // the last loads have landed before the LDS is reused
    };
    dispatch_active<0, TM>(nact, kloop);

    if (wi.S > 1) {
        // split K: as in the register-staged kernel (device-scope partials,
        // the last part to arrive adds them in part order)
        constexpr int PER_UNIT = BM * NB;
        constexpr int kDeviceScope = 16;
        const float *parts = p.part + (int64_t)wi.unit * wi.S * PER_UNIT;
        const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(parts, (int64_t)wi.S * PER_UNIT * 4);
        const int mine = wi.part * PER_UNIT * 4;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int o = ((i * TB + j) * NT + tid) * 16;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), prs, o, mine,
                                                       kDeviceScope);
            }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (tid == 0) last_part = atomicAdd(p.cnt + wi.unit, 1) == wi.S - 1;
        __syncthreads();
        if (!last_part) return;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int o = ((i * TB + j) * NT + tid) * 16;
                f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, o, 0, kDeviceScope));
                for (int sp = 1; sp < wi.S; ++sp)
                    v += __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, o, sp * PER_UNIT * 4, kDeviceScope));
                acc[i][j] = v;
            }
        if (tid == 0) p.cnt[wi.unit] = 0;
    }

    // Epilogue as in the register-staged kernel: silu(gate) * up, bf16
    // pairs traded between lanes l and l^1, the tile staged in LDS (rows
    // 0 .. BM/2-1 in lds0, the rest in lds1) for 16-byte row stores.
    static_assert(BM / 2 * BN * 2 <= (int)sizeof(lds0), "half the output tile fits in a staging buffer");
    constexpr int CPR = BN / 8;  // BN output columns either way
    auto Ct = [&](int r) __attribute__((always_inline)) { return r < BM / 2 ? lds0 + r * BN : lds1 + (r - BM / 2) * BN; };
    const bool odd = lane & 1;
    auto swap1 = [](float x) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    };
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int cl = wn * TN * MF + j * MF + lane % MF;
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (GLU) v[r] = silu_fast(acc[i][j][r]) * acc[i][TN + j][r];
                else v[r] = acc[i][j][r];
            }
            const float xs = swap1(odd ? v[0] : v[2]), ys = swap1(odd ? v[1] : v[3]);
            const int rb = wm * WTM + i * MF + 4 * (lane / 16);
            const int ra0 = rb + (odd ? 2 : 0), ra1 = ra0 + 1;
            const int ce = cl & ~1;
            const bf16x2 p0 = {(bf16)(odd ? xs : v[0]), (bf16)(odd ? v[2] : xs)};
            const bf16x2 p1 = {(bf16)(odd ? ys : v[1]), (bf16)(odd ? v[3] : ys)};
            *(bf16x2 *)(Ct(ra0) + (((ce / 8) ^ ((ra0 / 2) & 7)) * 8) + ce % 8) = p0;
            *(bf16x2 *)(Ct(ra1) + (((ce / 8) ^ ((ra1 / 2) & 7)) * 8) + ce % 8) = p1;
        }
    __syncthreads();
    for (int q = tid; q < BM * CPR; q += NT) {
        const int rl = q / CPR, c = q % CPR;
        const int64_t row = tc.row0 + rl;
        const int col = n0 + c * 8;
        if (row < tc.row_end && col < p.N)
            store16(p.C + row * p.N + col, load16(Ct(rl) + ((c ^ ((rl / 2) & 7)) * 8)));
    }
}

struct GemmParamsF32 {
    const float *A;
    const float *B0;
    const float *B1;
    const float *bias;
    float *C;
    const int32_t *offsets;
    const int32_t *mstart;
    const int4 *mtile;
    int max_mt;
    int G;
    int64_t rows;
    int N, K;
    int act;
    int kslice;  // K-sliced B as in GemmParams; 0 = B is [N][K]
    // gathered A: row r of the grouped operand is row arow[r] of A (null:
    // rows in place)
    const int32_t *arow;
};

constexpr int kF32BM = 32;

// Float32 grouped GEMM on the vector ALU: 32x32 tiles (small tiles, so that
// the few rows of a float32 layer still spread over many CUs), K steps of
// 64, each of the 256 threads 2x2 outputs (2x2 more for the up projection).
// The next K step's operands are loaded into registers (16-byte loads)
// while the current one is computed from LDS.  Rows past the group's end and
// columns past N read a valid row (results discarded); K positions past K
// read zeros.
template <bool GLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParamsF32 p) {
    constexpr int BM = kF32BM, BN = 32, BK = 64;
    constexpr int NU = GLU ? 2 : 1;
    __shared__ float As[BK][BM + 1];
    __shared__ float Bs[NU][BK][BN + 1];
    const int ntn = (p.N + BN - 1) / BN;
    const TileCoord tc = find_tile<BM>(xcd_remap(blockIdx.x), p.offsets, p.mstart, p.mtile, p.max_mt, p.G, p.rows, ntn);
    if (!tc.valid) return;
    const int n0 = tc.nt * BN;
    const int64_t K = p.K;
    const float *Bg[NU];
    Bg[0] = p.B0 + (int64_t)tc.g * p.N * K;
    if constexpr (GLU) Bg[NU - 1] = p.B1 + (int64_t)tc.g * p.N * K;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    float acc[NU][2][2] = {};
    // loader: float4 q = tid + 256 * i holds k = 4 * (q % 16) .. +3 of tile row q / 16
    const float *arow[2], *brow[NU][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = (tid + 256 * i) / 16;
        int64_t gr = tc.row0 + r;
        if (gr >= tc.row_end) gr = tc.row_end - 1;
        arow[i] = p.A + (p.arow ? (int64_t)p.arow[gr] : gr) * K;
        int n = n0 + r;
        if (n >= p.N) n = p.N - 1;
#pragma unroll
        for (int u = 0; u < NU; ++u) brow[u][i] = Bg[u] + (int64_t)n * (p.kslice ? p.kslice : K);
    }
    const int kq = 4 * (tid % 16);
    float4 ra[2], rb[NU][2];
    auto gload = [&](int k0) {
        const int k = k0 + kq;
        const bool in = k < p.K;  // K is a multiple of 16: a float4 is all in or all out
        // K-sliced B (the shared experts' down projections): column k is
        // column k % kslice of slice k / kslice; a float4 stays in one slice
        const int64_t bk = p.kslice ? (int64_t)(k / p.kslice) * p.N * p.kslice + k % p.kslice : k;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            ra[i] = in ? *(const float4 *)(arow[i] + k) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < NU; ++u)
                rb[u][i] = in ? *(const float4 *)(brow[u][i] + bk) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = (tid + 256 * i) / 16;
            As[kq][r] = ra[i].x;
            As[kq + 1][r] = ra[i].y;
            As[kq + 2][r] = ra[i].z;
            As[kq + 3][r] = ra[i].w;
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                Bs[u][kq][r] = rb[u][i].x;
                Bs[u][kq + 1][r] = rb[u][i].y;
                Bs[u][kq + 2][r] = rb[u][i].z;
                Bs[u][kq + 3][r] = rb[u][i].w;
            }
        }
    };
    gload(0);
    for (int k0 = 0; k0 < p.K; k0 += BK) {
        lstore();
        __syncthreads();
        if (k0 + BK < p.K) gload(k0 + BK);
#pragma unroll 16
        for (int kk = 0; kk < BK; ++kk) {
            float a[2], b[NU][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = As[kk][ty * 2 + i];
#pragma unroll
                for (int u = 0; u < NU; ++u) b[u][i] = Bs[u][kk][tx * 2 + i];
            }
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[u][i][j] = fmaf(a[i], b[u][j], acc[u][i][j]);
        }
        __syncthreads();
    }
    const float *bias = p.bias ? p.bias + (int64_t)tc.g * p.N : nullptr;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t row = tc.row0 + ty * 2 + i;
        if (row >= tc.row_end) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + tx * 2 + j;
            if (col >= p.N) continue;
            float v = acc[0][i][j];
            if constexpr (GLU) v = silu(v) * acc[NU - 1][i][j];
            else v = apply_act(p.act, v + (bias ? bias[col] : 0.f));
            p.C[row * p.N + col] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// tile plan
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_plan_kernel(const int32_t *__restrict__ counts,
                                                        const int32_t *__restrict__ offsets, int E, int BM,
                                                        int32_t *__restrict__ mstart, int4 *__restrict__ mtile,
                                                        int max_mt, int32_t *__restrict__ cnt, int ncnt,
                                                        int interleave) {
    __shared__ int scratch[3 * (kMaxPlanExperts + 1)];
    build_tile_plan(counts, offsets, E, BM, mstart, mtile, max_mt, cnt, ncnt, interleave != 0, scratch);
}

void launch_tile_plan(const int32_t *counts, const int32_t *offsets, int E, int BM, int32_t *mstart, int4 *mtile,
                      int max_mt, int32_t *cnt, int ncnt, bool interleave, hipStream_t s) {
    hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(256), 0, s, counts, offsets, E, BM, mstart, mtile, max_mt, cnt,
                       cnt ? ncnt : 0, interleave ? 1 : 0);
}

int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices] = {};  // 0: not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int gemm_block_m(int shape, bool bf16) {
    if (!bf16) return kF32BM;
    if (shape == kGemmDecode) return 32;
    if (shape == kGemmMid) return 64;
    if (shape == kGemmSmallM) return 128;
    return 256;
}

static int64_t grid_for(const GemmArgs &a, int BM, int BN) {
    const int64_t ntn = (a.N + BN - 1) / BN;
    int64_t mtiles;
    if (a.offsets == nullptr) mtiles = (a.rows + BM - 1) / BM;
    else mtiles = (a.rows + (int64_t)a.G * (BM - 1)) / BM;
    int64_t g = mtiles * ntn;
    g = (g + kGridQuantum - 1) / kGridQuantum * kGridQuantum;
    return g;
}

// Split K of the last round needs the number of co-resident workgroups of
// `kern` (nthreads a workgroup; cached in per_cu_cache) and room for that
// many BM x NB partial tiles; otherwise it stays off.  Only for K loops of
// at least 4096 (at least 2048 per part).  Sets p's split fields and returns
// the workgroups to add to the grid.
static int64_t split_k_setup(const GemmArgs &a, void (*kern)(GemmParams), int nthreads, int BM, int NB, int BK,
                             std::atomic<int> &per_cu_cache, GemmParams &p) {
    const int KT = a.K / BK;
    const int min_part = 2048 / BK;  // K tiles per part at least (1024 or 512 measured slower on decode tiles)
    if (a.split.part == nullptr || KT < 2 * min_part) return 0;
    int per_cu = per_cu_cache.load(std::memory_order_relaxed);
    if (per_cu < 0) {
        int n = 0;
        per_cu = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, nthreads, 0) == hipSuccess ? n : 0;
        per_cu_cache.store(per_cu, std::memory_order_relaxed);
    }
    const int64_t slots = (int64_t)device_cus() * per_cu;
    if (slots <= 0 || slots > a.split.ncnt || slots * BM * NB > a.split.part_floats) return 0;
    p.part = a.split.part;
    p.cnt = a.split.cnt;
    p.slots = (int)slots;
    p.max_split = std::min(8, KT / min_part);
    p.max_slabs = (int)std::min<int64_t>(a.split.part_floats / ((int64_t)BM * NB), 1 << 30);
    // the split parts add rem * (S - 1) work items beyond the tiles, fewer
    // than slots * (max_split - 1) and than max_slabs (rem * S slabs);
    // surplus workgroups exit at once
    const int64_t extra = std::min<int64_t>(slots * std::max(1, p.max_split - 1), p.max_slabs);
    return (extra + kGridQuantum - 1) / kGridQuantum * kGridQuantum;
}

template <int BM, int BN, int WM, int WN, bool GLU, int MF = 16, bool RMAP = false, int IL = 0, int BK = 64,
          bool JOUT = false, bool SL = false, bool PO = false>
static void launch_bf16_t(const GemmArgs &a, hipStream_t s, float *partout = nullptr, int fixed_split = 0) {
    constexpr int NB = GLU ? 2 * BN : BN;
    static_assert((int64_t)BM * NB <= kSplitUnitFloats, "split-K unit");
    auto kern = gemm_bf16_kernel<BM, BN, WM, WN, GLU, IL, MF, RMAP, BK, JOUT, SL, PO>;
    GemmParams p{(const bf16 *)a.A, (const bf16 *)a.B0, (const bf16 *)a.B1, a.bias, (bf16 *)a.C,
                 a.offsets, a.mstart, a.mtile, a.max_mt, a.G, a.rows, a.N, a.K, a.act, nullptr, nullptr, 0, 1, 0,
                 a.arow, a.a_rows * a.K * 2, SL ? a.kslice : 0, PO ? partout : nullptr, PO ? fixed_split : 0};
    int64_t grid = grid_for(a, BM, BN);
    if (grid == 0) return;
    if constexpr (PO) {
        // every tile in fixed_split parts (consecutive work items), whole grid quanta
        const int64_t need = ((a.rows + BM - 1) / BM) * ((a.N + BN - 1) / BN) * fixed_split;
        grid = (need + kGridQuantum - 1) / kGridQuantum * kGridQuantum;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WM * WN), 0, s, p);
        return;
    }
    // workgroups of this kernel per CU, queried once (atomic: callers may
    // launch from several host threads)
    static std::atomic<int> per_cu_cache{-1};
    grid += split_k_setup(a, kern, 64 * WM * WN, BM, NB, BK, per_cu_cache, p);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WM * WN), 0, s, p);
}

// 256-row tiles with direct-to-LDS loads (K % 128 == 0): the SwiGLU
// gate/up GEMM (128 outputs of gate and up) or the plain down projection
// (256 outputs)
template <int BN, bool GLU>
static void launch_lds(const GemmArgs &a, hipStream_t s) {
    constexpr int BM = 256, NB = GLU ? 2 * BN : BN;
    static_assert((int64_t)BM * NB <= kSplitUnitFloats, "split-K unit");
    auto kern = gemm_lds_kernel<BM, BN, GLU>;
    GemmParams p{(const bf16 *)a.A, (const bf16 *)a.B0, (const bf16 *)a.B1, nullptr, (bf16 *)a.C,
                 a.offsets, a.mstart, a.mtile, a.max_mt, a.G, a.rows, a.N, a.K, a.act, nullptr, nullptr, 0, 1, 0,
                 a.arow, a.a_rows * a.K * 2, 0, nullptr, 0};
    int64_t grid = grid_for(a, BM, BN);
    if (grid == 0) return;
    static std::atomic<int> per_cu_cache{-1};
    grid += split_k_setup(a, kern, 512, BM, NB, 64, per_cu_cache, p);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), 0, s, p);
}

template <bool GLU>
static void launch_f32_t(const GemmArgs &a, hipStream_t s) {
    GemmParamsF32 p{(const float *)a.A, (const float *)a.B0, (const float *)a.B1, a.bias, (float *)a.C,
                    a.offsets, a.mstart, a.mtile, a.max_mt, a.G, a.rows, a.N, a.K, a.act, a.kslice, a.arow};
    const int64_t grid = grid_for(a, kF32BM, 32);
    if (grid == 0) return;
    hipLaunchKernelGGL((gemm_f32_kernel<GLU>), dim3((unsigned)grid), dim3(256), 0, s, p);
}

int router_gemm_split(int T, int E, int d) {
    // 128-row tiles over all E <= 256 columns; enough K parts for about one
    // work item per CU, each part at least 512 deep
    const int tiles = (T + 127) / 128 * ((E + 255) / 256);
    int cus = device_cus();
    if (cus <= 0) cus = 256;
    int S = (cus + tiles - 1) / tiles;
    S = std::max(1, std::min(S, std::min(kRouterMaxSplit, d / 512)));
    return S;
}

void launch_router_gemm(const void *x, const void *wg, int T, int d, int E, float *partout, int S, hipStream_t s) {
    GemmArgs a{x, wg, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, T, E, d, kActNone, true,
               SplitKWs{nullptr, 0, nullptr, 0}};
    launch_bf16_t<128, 256, 2, 4, false, 32, true, 1, 64, false, false, true>(a, s, partout, S);
}

void launch_grouped_gemm(const GemmArgs &a, int shape, hipStream_t s) {
    const bool glu = a.act == kActSwiglu;
    if (!a.bf16) {
        if (glu) launch_f32_t<true>(a, s);
        else launch_f32_t<false>(a, s);
        return;
    }
    // Tile shapes measured on the Mixtral-shape prefill GEMMs (T=4096, k=2,
    // d=4096, F=14336): 8 waves (2 per SIMD) with 256-row tiles, two K tiles
    // in flight, fragments double-buffered, on 16x16x32 MFMAs.  The 128- and
    // 32-row tiles stay on 32x32x16, which measured faster for them.
    // Alternating single launches of two variants (so both see the same
    // power and clock state) measured: 16x16x32 MFMAs 2.5% faster than
    // 32x32x16 on both GEMMs; row halves split across the two waves of a
    // SIMD (RMAP) 3% faster on the down projection and 1% slower on the
    // gate/up one; LDS reads interleaved 1:1 with the MFMAs (IL = 1) 2.5%
    // faster on the down projection, no change on the gate/up one (2%
    // faster on it too once the m-tiles were balanced and split by rows).
    // Balanced m-tiles with the row-block skip: gate/up 1865 -> 1790
    // us, down 950 -> 884 us (the padding rows of each expert's last tile
    // had been 13.5% of the MFMAs).  The skip alone, on tiles of BM rows
    // and a short last one, had gained 1% and doubled the gate/up GEMM's L2
    // misses: the short tiles finished early and broke the lock-step of a
    // 32-tile XCD group.  Balanced tiles of one group are equally long, and
    // the split rows (RMAP) give each SIMD one wave of each row half, so the
    // skipped blocks shorten every SIMD's work alike.
    if (a.kslice > 0) {
        // K-sliced B: the shared experts' down projection (one group, decode
        // or prefill tiles, same schedules as below)
        if (shape == kGemmDecode) launch_bf16_t<32, 128, 1, 4, false, 32, false, 0, 64, false, true>(a, s);
        else launch_bf16_t<256, 256, 2, 4, false, 16, true, 1, 64, false, true>(a, s);
        return;
    }
    if (shape == kGemmMid) {
        // 64-row tiles for layers whose weights stay in the MALL and whose
        // experts hold a few dozen to a few hundred rows: each m-tile streams
        // its expert's weight panels from L2 / MALL, so twice the rows per
        // tile halve that traffic.  Narrow outputs (the down projection,
        // N = d < 1024) take 64-column tiles, so that there are enough tiles
        // for the CUs.  Measured against 32-row tiles: Switch layer (T = 4096,
        // d = 512, E = 16, capacity 80 per row) GEMM1 22.2 -> 17.9 us, GEMM2
        // 17.7 -> 17.1 us (64 x 128 tiles: 20.7 us), layer 0.070 -> 0.063 ms.
        if (glu) launch_bf16_t<64, 128, 2, 4, true, 32, true, 1>(a, s);
        else if (a.N >= 1024) launch_bf16_t<64, 128, 2, 4, false, 32, true, 1>(a, s);
        else launch_bf16_t<64, 64, 2, 2, false, 32, true>(a, s);
        return;
    }
    if (shape == kGemmDecode) {
        // gate/up: K tiles of 128 (256 bytes of each weight row per load
        // round rather than 128: a plain read of the decode tile's weight
        // rows in that pattern streams at 5.4 instead of 5.0 TB/s; Mixtral
        // decode gate/up 355 -> 323 us) and LDS reads interleaved with the
        // MFMAs (324 -> 318 us).  The down projection stays on K tiles of 64
        // (with 128 its LDS allows one workgroup per CU instead of three:
        // 155 -> 166 us) and on the compiler's schedule (interleaved: Switch
        // down projection 17.5 -> 18.3 us).
        if (glu && a.K % 128 == 0) launch_bf16_t<32, 128, 1, 4, true, 32, false, 1, 128>(a, s);
        else if (glu) launch_bf16_t<32, 128, 1, 4, true, 32, false, 1>(a, s);
        else launch_bf16_t<32, 128, 1, 4, false, 32>(a, s);
    } else if (shape == kGemmSmallM) {
        // 8 waves (2 per SIMD) rather than 4: on the expert-choice layer
        // (128 rows per expert) the down projection 112 -> 90 us, gate/up
        // 171 -> 165 us; on the Switch layer 41 -> 28 and 50 -> 38 us.
        // Splitting these short tiles along K measured 2x slower.  LDS reads
        // interleaved with the MFMAs: expert-choice GEMMs about -1%.
        if (glu) launch_bf16_t<128, 128, 2, 4, true, 32, true, 1>(a, s);
        else launch_bf16_t<128, 256, 2, 4, false, 32, true, 1>(a, s);
    } else {
        if (glu && a.K % 128 == 0) launch_lds<128, true>(a, s);
        else if (glu) launch_bf16_t<256, 128, 2, 4, true, 16, true, 1, 64, true>(a, s);
        else if (a.K % 128 == 0 && a.bias == nullptr && a.act == kActNone) launch_lds<256, false>(a, s);
        else launch_bf16_t<256, 256, 2, 4, false, 16, true, 1>(a, s);
    }
}

}  // namespace moe
