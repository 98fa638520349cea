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
// Tiles: a device-side plan (mstart) lists the m-tiles of every expert; the
// grid covers the worst case and surplus blocks exit.  Tile order is (expert,
// n-tile, m-tile) with m fastest, remapped so that runs of consecutive tiles
// land on one XCD and share its L2 copy of the weight panel.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kXcds = 8;
constexpr int kXcdRun = 4;  // consecutive logical tiles per XCD
constexpr int kGridQuantum = kXcds * kXcdRun;

// Blocks are dispatched round-robin over the XCDs (block b -> XCD b % 8).
// Within each group of 32 blocks, XCD x receives logical tiles 4x .. 4x+3.
__device__ inline int xcd_remap(int b) {
    const int grp = b / kGridQuantum, within = b % kGridQuantum;
    return grp * kGridQuantum + (within % kXcds) * kXcdRun + within / kXcds;
}

struct TileCoord {
    int g, nt;
    int64_t row0, row_end;
    bool valid;
};

template <int BM>
__device__ inline TileCoord find_tile(int tile, const int32_t *offsets, const int32_t *mstart, int G,
                                      int64_t rows, int ntn) {
    TileCoord c;
    c.valid = false;
    if (offsets == nullptr) {
        const int mtiles = (int)((rows + BM - 1) / BM);
        if (tile >= mtiles * ntn) return c;
        c.g = 0;
        c.nt = tile / mtiles;
        c.row0 = (int64_t)(tile % mtiles) * BM;
        c.row_end = rows;
        c.valid = true;
        return c;
    }
    const int total = mstart[G];
    if (tile >= total * ntn) return c;
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mstart[mid] * ntn <= tile) lo = mid;
        else hi = mid - 1;
    }
    const int local = tile - mstart[lo] * ntn;
    const int mt_g = mstart[lo + 1] - mstart[lo];
    c.g = lo;
    c.nt = local / mt_g;
    c.row0 = offsets[lo] + (int64_t)(local % mt_g) * BM;
    c.row_end = offsets[lo + 1];
    c.valid = true;
    return c;
}

// LDS tiles hold rows of 64 bf16 (128 bytes = eight 16-byte chunks).  Chunk c
// of row r is stored at chunk slot c ^ swz(r) so that the 16-byte reads of 16
// consecutive rows at one chunk index touch distinct banks.
__device__ inline int swz(int r) { return (r >> 1) & 7; }

struct GemmParams {
    const bf16 *A;
    const bf16 *B0;
    const bf16 *B1;
    const float *bias;
    bf16 *C;
    const int32_t *offsets;
    const int32_t *mstart;
    int G;
    int64_t rows;
    int N, K;
    int act;
};

template <int BM, int BN, int WM, int WN, bool GLU>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmParams p) {
    constexpr int BK = 64;
    constexpr int NB = GLU ? 2 * BN : BN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int A_PER_T = BM * 8 / 256, B_PER_T = NB * 8 / 256;
    static_assert(WM * WN == 4, "four waves");
    static_assert(A_PER_T >= 1 && B_PER_T >= 1, "tile too small");
    __shared__ __attribute__((aligned(16))) bf16 lds[2][(BM + NB) * BK];

    const int ntn = (p.N + BN - 1) / BN;
    const TileCoord tc = find_tile<BM>(xcd_remap(blockIdx.x), p.offsets, p.mstart, p.G, p.rows, ntn);
    if (!tc.valid) return;
    const int n0 = tc.nt * BN;
    const int64_t K = p.K;
    const bf16 *B0g = p.B0 + (int64_t)tc.g * p.N * K;
    const bf16 *B1g = GLU ? p.B1 + (int64_t)tc.g * p.N * K : nullptr;

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int wm = wave % WM, wn = wave / WM;

    // global source of each thread's chunks (row clamped into the group)
    const bf16 *asrc[A_PER_T];
    int adst[A_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
        const int q = tid + i * 256, r = q / 8, ch = q % 8;
        int64_t gr = tc.row0 + r;
        if (gr >= tc.row_end) gr = tc.row_end - 1;
        asrc[i] = p.A + gr * K + ch * 8;
        adst[i] = r * BK + ((ch ^ swz(r)) * 8);
    }
    const bf16 *bsrc[B_PER_T];
    int bdst[B_PER_T];
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
        const int q = tid + i * 256, r = q / 8, ch = q % 8;
        const bool up = GLU && r >= BN;
        int n = n0 + (up ? r - BN : r);
        if (n >= p.N) n = p.N - 1;
        bsrc[i] = (up ? B1g : B0g) + (int64_t)n * K + ch * 8;
        bdst[i] = (BM + r) * BK + ((ch ^ swz(r)) * 8);
    }

    f32x16 acc[TM][TN];
    f32x16 accu[GLU ? TM : 1][GLU ? TN : 1];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            acc[i][j] = f32x16{};
            if constexpr (GLU) accu[i][j] = f32x16{};
        }

    u32x4 ra[A_PER_T], rb[B_PER_T];
    auto gload = [&](int kt) {
        const int64_t ko = (int64_t)kt * BK;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) ra[i] = load16(asrc[i] + ko);
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) rb[i] = load16(bsrc[i] + ko);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) store16(&lds[buf][adst[i]], ra[i]);
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) store16(&lds[buf][bdst[i]], rb[i]);
    };

    const int KT = p.K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        const bf16 *L = lds[cur];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ks * 2 + lane / 32;
            bf16x8 af[TM], bfr[TN], bu[GLU ? TN : 1];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + lane % 32;
                af[i] = __builtin_bit_cast(bf16x8, load16(L + r * BK + ((ch ^ swz(r)) * 8)));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 32 + lane % 32;
                bfr[j] = __builtin_bit_cast(bf16x8, load16(L + (BM + r) * BK + ((ch ^ swz(r)) * 8)));
                if constexpr (GLU)
                    bu[j] = __builtin_bit_cast(bf16x8, load16(L + (BM + BN + r) * BK + ((ch ^ swz(r)) * 8)));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
                    if constexpr (GLU)
                        accu[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bu[j], accu[i][j], 0, 0, 0);
                }
        }
        if (kt + 1 < KT) lstore(cur ^ 1);
        __syncthreads();
    }

    // epilogue: D[8*q + 4*(lane/32) + j][lane%32] of each 32x32 tile is acc[4*q + j]
    const float *bias = p.bias ? p.bias + (int64_t)tc.g * p.N : nullptr;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WTN + j * 32 + lane % 32;
            if (col >= p.N) continue;
            const float bcol = bias ? bias[col] : 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int64_t row = tc.row0 + wm * WTM + i * 32 + 8 * q + 4 * (lane / 32) + jj;
                    if (row >= tc.row_end) continue;
                    float v = acc[i][j][4 * q + jj];
                    if constexpr (GLU) v = silu(v) * accu[i][j][4 * q + jj];
                    else v = apply_act(p.act, v + bcol);
                    p.C[row * p.N + col] = (bf16)v;
                }
        }
}

// ---------------------------------------------------------------------------
// float32 grouped GEMM on the vector ALUs: 64x64 tiles, 4x4 outputs per
// thread, K in steps of 16 through LDS.
// ---------------------------------------------------------------------------
struct GemmParamsF32 {
    const float *A;
    const float *B0;
    const float *B1;
    const float *bias;
    float *C;
    const int32_t *offsets;
    const int32_t *mstart;
    int G;
    int64_t rows;
    int N, K;
    int act;
};

constexpr int kF32BM = 64;

template <bool GLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParamsF32 p) {
    constexpr int BM = kF32BM, BN = 64, BK = 16;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    __shared__ float Bu[GLU ? BK : 1][BN + 4];
    const int ntn = (p.N + BN - 1) / BN;
    const TileCoord tc = find_tile<BM>(xcd_remap(blockIdx.x), p.offsets, p.mstart, p.G, p.rows, ntn);
    if (!tc.valid) return;
    const int n0 = tc.nt * BN;
    const int64_t K = p.K;
    const float *B0g = p.B0 + (int64_t)tc.g * p.N * K;
    const float *B1g = GLU ? p.B1 + (int64_t)tc.g * p.N * K : nullptr;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    float acc[4][4] = {}, accu[GLU ? 4 : 1][GLU ? 4 : 1] = {};
    // loader: element (r, kk) with r = q / 16, kk = q % 16 for q = tid + 256 * i
    for (int k0 = 0; k0 < p.K; k0 += BK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + 256 * i, r = q / BK, kk = q % BK;
            int64_t gr = tc.row0 + r;
            if (gr >= tc.row_end) gr = tc.row_end - 1;
            As[kk][r] = p.A[gr * K + k0 + kk];
            int n = n0 + r;
            if (n >= p.N) n = p.N - 1;
            Bs[kk][r] = B0g[(int64_t)n * K + k0 + kk];
            if constexpr (GLU) Bu[kk][r] = B1g[(int64_t)n * K + k0 + kk];
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4], bu[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = As[kk][ty * 4 + i];
                b[i] = Bs[kk][tx * 4 + i];
                if constexpr (GLU) bu[i] = Bu[kk][tx * 4 + i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
                    if constexpr (GLU) accu[i][j] = fmaf(a[i], bu[j], accu[i][j]);
                }
        }
        __syncthreads();
    }
    const float *bias = p.bias ? p.bias + (int64_t)tc.g * p.N : nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = tc.row0 + ty * 4 + i;
        if (row >= tc.row_end) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + tx * 4 + j;
            if (col >= p.N) continue;
            float v = acc[i][j];
            if constexpr (GLU) v = silu(v) * accu[i][j];
            else v = apply_act(p.act, v + (bias ? bias[col] : 0.f));
            p.C[row * p.N + col] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// tile plan
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void tile_plan_kernel(const int32_t *__restrict__ counts, int E, int BM,
                                                       int32_t *__restrict__ mstart) {
    const int lane = threadIdx.x;
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        const int v = e < E ? (counts[e] + BM - 1) / BM : 0;
        int incl = v;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int n = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += n;
        }
        if (e < E) mstart[e] = base + incl - v;
        base += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) mstart[E] = base;
}

void launch_tile_plan(const int32_t *counts, int E, int BM, int32_t *mstart, hipStream_t s) {
    hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(64), 0, s, counts, E, BM, mstart);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
int gemm_block_m(int shape, bool bf16) {
    if (!bf16) return kF32BM;
    if (shape == kGemmDecode) return 32;
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

template <int BM, int BN, int WM, int WN, bool GLU>
static void launch_bf16_t(const GemmArgs &a, hipStream_t s) {
    GemmParams p{(const bf16 *)a.A, (const bf16 *)a.B0, (const bf16 *)a.B1, a.bias, (bf16 *)a.C,
                 a.offsets, a.mstart, a.G, a.rows, a.N, a.K, a.act};
    const int64_t grid = grid_for(a, BM, BN);
    if (grid == 0) return;
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, GLU>), dim3((unsigned)grid), dim3(256), 0, s, p);
}

template <bool GLU>
static void launch_f32_t(const GemmArgs &a, hipStream_t s) {
    GemmParamsF32 p{(const float *)a.A, (const float *)a.B0, (const float *)a.B1, a.bias, (float *)a.C,
                    a.offsets, a.mstart, a.G, a.rows, a.N, a.K, a.act};
    const int64_t grid = grid_for(a, kF32BM, 64);
    if (grid == 0) return;
    hipLaunchKernelGGL((gemm_f32_kernel<GLU>), dim3((unsigned)grid), dim3(256), 0, s, p);
}

void launch_grouped_gemm(const GemmArgs &a, int shape, hipStream_t s) {
    const bool glu = a.act == kActSwiglu;
    if (!a.bf16) {
        if (glu) launch_f32_t<true>(a, s);
        else launch_f32_t<false>(a, s);
        return;
    }
    if (shape == kGemmDecode) {
        if (glu) launch_bf16_t<32, 128, 1, 4, true>(a, s);
        else launch_bf16_t<32, 128, 1, 4, false>(a, s);
    } else if (shape == kGemmSmallM) {
        if (glu) launch_bf16_t<128, 128, 2, 2, true>(a, s);
        else launch_bf16_t<128, 256, 2, 2, false>(a, s);
    } else {
        if (glu) launch_bf16_t<256, 128, 2, 2, true>(a, s);
        else launch_bf16_t<256, 256, 2, 2, false>(a, s);
    }
}

}  // namespace moe
