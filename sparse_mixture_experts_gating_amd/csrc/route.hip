// Router GEMM fused with wave-level gating, gating on given logits, and
// expert-choice selection, for gfx950.
//
// Pages (titles as published):
//   [devtips] devtips.kr "MoE (Mixture of Experts) 아키텍처 완전 정복" -- MoELayer
//   [yj-zh]   youngju.dev "Mixture of Experts（MoE）架构深度解析" -- GatingNetwork,
//             SwitchRouter, MixtralMoELayer, ExpertChoiceRouter
//   [yj-ja]   youngju.dev "Sparse Mixture of Experts（MoE）アーキテクチャ深層分析" --
//             gating formula, TopKGating, ExpertChoiceGating
#include "common.h"
#include "kernels.h"
#include "perm_small.h"

namespace moe {

// One wave gates one token whose E float32 logits start at `row`.
// Lane l holds experts l, l+64, l+128, l+192 (E <= 256).  Selection repeats a
// wave-wide maximum of unique rank keys (value desc, index asc) k times, so
// the slots come out in rank order.  Weights:
//   topk-softmax: softmax over the k selected logits ([yj-zh] GatingNetwork);
//   softmax-topk / switch: softmax over all E logits taken at the selected
//   experts ([yj-ja] gating formula; [yj-zh] SwitchRouter probs.max).
__device__ void gate_one_token(const float *row, int E, int k, int gating, int64_t t,
                               int32_t *__restrict__ idx_out, float *__restrict__ w_out) {
    const int lane = threadIdx.x % kWave;
    uint64_t key[4];
    float val[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + kWave * q;
        if (e < E) {
            val[q] = row[e];
            key[q] = rank_key(val[q], (uint32_t)e);
        } else {
            val[q] = 0.f;
            key[q] = 0ull;  // below every finite key
        }
    }
    int32_t sel_idx[4] = {0, 0, 0, 0};
    float sel_val[4] = {0.f, 0.f, 0.f, 0.f};
    float top = 0.f;
    for (int j = 0; j < k; ++j) {
        uint64_t m = key[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) m = key[q] > m ? key[q] : m;
        m = wave_max_u64(m);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (key[q] == m) key[q] = 0ull;
        const float v = key_value((uint32_t)(m >> 32));
        if (j == 0) top = v;
        if (lane == (j & (kWave - 1))) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if ((j >> 6) == q) {
                    sel_idx[q] = (int32_t)rank_key_index(m);
                    sel_val[q] = v;
                }
        }
    }
    float part = 0.f;
    if (gating == kGateTopkSoftmax) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + kWave * q < k) part += expf(sel_val[q] - top);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + kWave * q < E) part += expf(val[q] - top);
    }
    const float z = wave_sum(part);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j = lane + kWave * q;
        if (j < k) {
            idx_out[t * k + j] = sel_idx[q];
            w_out[t * k + j] = expf(sel_val[q] - top) / z;
        }
    }
}

// Router GEMM on bf16 MFMA (v_mfma_f32_16x16x32_bf16) + gating epilogue for
// few experts (16*NT at most; launched for up to 16).  A block owns 16 tokens
// and its WK waves split the model dimension into WK contiguous ranges.  Each
// wave computes 16 tokens x 16*NT experts over its range straight from global
// memory, issuing U chunks of x and of the router weights before their MFMAs
// so that enough bytes are in flight to stream x at HBM rate (x rows are read
// once; the router weights stay in L1/L2).  Partial sums meet in LDS in a
// fixed order, the bias is added, logits are written, and each wave gates
// whole tokens.
__device__ inline float softplus(float u) { return fmaxf(u, 0.f) + log1pf(expf(-fabsf(u))); }

// NOISY adds the noise projection as a second MFMA accumulator set and forms
// x.Wg + b + softplus(x.Wn) * noise ([yj-ja] TopKGating, training branch).
// PERM (a batch of one block, T <= 16): the block then permutes its own
// selections (permute_small_block) and writes the tile plan, which saves
// the permutation launch of a decode step.
template <int NT, int WK, bool NOISY, bool PERM = false>
__global__ __launch_bounds__(64 * WK) void route_bf16_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ wg, const float *__restrict__ bias,
    int T, int d, int E, int k, int gating, float *__restrict__ logits,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out, const bf16 *__restrict__ wn,
    const float *__restrict__ noise, RoutePermuteArgs perm) {
    constexpr int TOK = 16;
    constexpr int EP = 16 * NT;
    constexpr int LD = EP + 4;
    constexpr int U = (NOISY ? 2 * NT : NT) <= 2 ? 8 : 4;  // chunks in flight per wave
    __shared__ float part[WK * TOK * LD];
    __shared__ float partn[NOISY ? WK * TOK * LD : 1];
    const int wk = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t tok0 = (int64_t)blockIdx.x * TOK;
    const int r = lane % 16, kq = (lane / 16) * 8;
    int64_t trow = tok0 + r;
    if (trow >= T) trow = T - 1;
    const bf16 *xa = x + trow * d + kq;
    int64_t woff[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        int e = nt * 16 + r;
        if (e >= E) e = E - 1;
        woff[nt] = (int64_t)e * d + kq;
    }
    f32x4 acc[NT], accn[NOISY ? NT : 1];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (NOISY) accn[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int nk = d / 32;
    const int kb = nk * wk / WK, ke = nk * (wk + 1) / WK;
    auto step = [&](const bf16x8 &a, const bf16x8 *b, const bf16x8 *bn) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[nt], acc[nt], 0, 0, 0);
            if constexpr (NOISY) accn[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bn[nt], accn[nt], 0, 0, 0);
        }
    };
    int kc = kb;
    for (; kc + U <= ke; kc += U) {
        bf16x8 a[U], b[U][NT], bn[U][NOISY ? NT : 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            a[u] = __builtin_bit_cast(bf16x8, load16(xa + (kc + u) * 32));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                b[u][nt] = __builtin_bit_cast(bf16x8, load16(wg + woff[nt] + (kc + u) * 32));
                if constexpr (NOISY) bn[u][nt] = __builtin_bit_cast(bf16x8, load16(wn + woff[nt] + (kc + u) * 32));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) step(a[u], b[u], bn[u]);
    }
    for (; kc < ke; ++kc) {
        bf16x8 b[NT], bn[NOISY ? NT : 1];
        const bf16x8 a = __builtin_bit_cast(bf16x8, load16(xa + kc * 32));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            b[nt] = __builtin_bit_cast(bf16x8, load16(wg + woff[nt] + kc * 32));
            if constexpr (NOISY) bn[nt] = __builtin_bit_cast(bf16x8, load16(wn + woff[nt] + kc * 32));
        }
        step(a, b, bn);
    }
    // D[row = 4*(lane/16) + j][col = lane%16] of each 16x16 tile
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            part[(wk * TOK + 4 * (lane / 16) + j) * LD + nt * 16 + r] = acc[nt][j];
            if constexpr (NOISY) partn[(wk * TOK + 4 * (lane / 16) + j) * LD + nt * 16 + r] = accn[nt][j];
        }
    __syncthreads();
    for (int i = threadIdx.x; i < TOK * EP; i += 64 * WK) {
        const int tt = i / EP, e = i % EP;
        float s = part[tt * LD + e];
#pragma unroll
        for (int w = 1; w < WK; ++w) s += part[(w * TOK + tt) * LD + e];
        if (e < E) {
            if (bias) s += bias[e];
            if constexpr (NOISY) {
                float u = partn[tt * LD + e];
#pragma unroll
                for (int w = 1; w < WK; ++w) u += partn[(w * TOK + tt) * LD + e];
                const int64_t t = tok0 + tt < T ? tok0 + tt : T - 1;
                s += softplus(u) * noise[t * E + e];
            }
            if (logits && tok0 + tt < T) logits[(tok0 + tt) * E + e] = s;
        }
        part[tt * LD + e] = s;
    }
    __syncthreads();
    if (gating == kGateExpertChoice) return;
    for (int tt = wk; tt < TOK; tt += WK) {
        const int64_t t = tok0 + tt;
        if (t < T) gate_one_token(part + tt * LD, E, k, gating, t, idx_out, w_out);
    }
    if constexpr (PERM) {
        extern __shared__ unsigned long long perm_lds[];
        __syncthreads();  // every token's selection is written (and visible to the block)
        permute_small_block<64 * WK>(idx_out, T, E, k, perm.capacity, perm.group_chunks, perm.counts,
                                     perm.offsets, perm.row_token, perm.slot_row, perm.plan, perm_lds);
    }
}

// float32 router (VALU): one wave per token, lane per expert, plus gating.
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ wg, const float *__restrict__ bias,
    int T, int d, int E, int k, int gating, float *__restrict__ logits,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out, const float *__restrict__ wn,
    const float *__restrict__ noise) {
    __shared__ float rows[4][256];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    const bool live = t < T;
    if (live) {
        for (int e = lane; e < E; e += kWave) {
            const float *xr = x + t * d;
            const float *wr = wg + (int64_t)e * d;
            float s = 0.f;
            for (int i = 0; i < d; ++i) s = fmaf(xr[i], wr[i], s);
            if (bias) s += bias[e];
            if (wn) {
                const float *nr = wn + (int64_t)e * d;
                float u = 0.f;
                for (int i = 0; i < d; ++i) u = fmaf(xr[i], nr[i], u);
                s += softplus(u) * noise[t * E + e];
            }
            rows[wave][e] = s;
            if (logits) logits[t * E + e] = s;
        }
    }
    __syncthreads();
    if (live && gating != kGateExpertChoice) gate_one_token(rows[wave], E, k, gating, t, idx_out, w_out);
}

// Gating alone on given float32 logits [T][E]: one wave per token.
__global__ __launch_bounds__(256) void gate_logits_kernel(const float *__restrict__ logits, int T, int E,
                                                           int k, int gating, int32_t *__restrict__ idx_out,
                                                           float *__restrict__ w_out) {
    const int wave = threadIdx.x / kWave;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t < T) gate_one_token(logits + t * E, E, k, gating, t, idx_out, w_out);
}

// ---------------------------------------------------------------------------
// Router statistics ([yj-ja] compute_load_balancing_loss, router_z_loss):
// each block owns kStatTokens consecutive tokens; each wave walks its tokens
// in order accumulating softmax probabilities (lane l: experts l + 64q),
// logsumexp^2 and selection counts; the waves' partials meet in LDS in wave
// order.  A one-block pass then sums the block partials in block order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_stats_kernel(const float *__restrict__ logits,
                                                           const int32_t *__restrict__ idx, int T, int E, int k,
                                                           float *__restrict__ part, int32_t *__restrict__ cnt) {
    __shared__ float sp[4][257];
    __shared__ int sc[4][256];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    float pacc[4] = {0.f, 0.f, 0.f, 0.f};
    int cacc[4] = {0, 0, 0, 0};
    float zacc = 0.f;
    for (int tt = wave; tt < kStatTokens; tt += 4) {
        const int64_t t = (int64_t)blockIdx.x * kStatTokens + tt;
        if (t >= T) break;
        const float *row = logits + t * E;
        float v[4];
        float m = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane + kWave * q;
            v[q] = e < E ? row[e] : -INFINITY;
            m = fmaxf(m, v[q]);
        }
        m = wave_max(m);
        float ex[4], s = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ex[q] = lane + kWave * q < E ? expf(v[q] - m) : 0.f;
            s += ex[q];
        }
        s = wave_sum(s);
#pragma unroll
        for (int q = 0; q < 4; ++q) pacc[q] += ex[q] / s;
        const float lse = m + logf(s);
        zacc += lse * lse;
        for (int j = 0; j < k; ++j) {
            const int e = idx[t * k + j];
            if (e >= 0 && e < E && lane == (e & (kWave - 1))) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if ((e >> 6) == q) ++cacc[q];
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        sp[wave][lane + kWave * q] = pacc[q];
        sc[wave][lane + kWave * q] = cacc[q];
    }
    if (lane == 0) sp[wave][256] = zacc;
    __syncthreads();
    const int e = threadIdx.x;
    float* pb = part + (int64_t)blockIdx.x * (E + 1);
    if (e < E) {
        pb[e] = ((sp[0][e] + sp[1][e]) + sp[2][e]) + sp[3][e];
        cnt[(int64_t)blockIdx.x * E + e] = sc[0][e] + sc[1][e] + sc[2][e] + sc[3][e];
    }
    if (e == 0) pb[E] = ((sp[0][256] + sp[1][256]) + sp[2][256]) + sp[3][256];
}

__global__ __launch_bounds__(256) void router_stats_finalize_kernel(const float *__restrict__ part,
                                                                    const int32_t *__restrict__ cnt, int nb, int T,
                                                                    int E, int k, float *__restrict__ out) {
    __shared__ float prod[256];
    const int e = threadIdx.x;
    if (e < E) {
        float ps = 0.f;
        int64_t cs = 0;
        for (int b = 0; b < nb; ++b) {
            ps += part[(int64_t)b * (E + 1) + e];
            cs += cnt[(int64_t)b * E + e];
        }
        const float P = ps / (float)T;
        const float f = (float)((double)cs / ((double)T * k));
        out[2 + e] = P;
        prod[e] = f * P;
    }
    __syncthreads();
    if (e == 0) {
        float a = 0.f, z = 0.f;
        for (int i = 0; i < E; ++i) a += prod[i];
        for (int b = 0; b < nb; ++b) z += part[(int64_t)b * (E + 1) + E];
        out[0] = (float)E * a;
        out[1] = z / (float)T;
    }
}

void launch_router_stats(const float *logits, const int32_t *idx, int T, int E, int k, float *part, int32_t *cnt,
                         float *out, hipStream_t s) {
    const int nb = (T + kStatTokens - 1) / kStatTokens;
    hipLaunchKernelGGL(router_stats_kernel, dim3(nb), dim3(256), 0, s, logits, idx, T, E, k, part, cnt);
    hipLaunchKernelGGL(router_stats_finalize_kernel, dim3(1), dim3(256), 0, s, part, cnt, nb, T, E, k, out);
}

// ---------------------------------------------------------------------------
// Expert choice ([yj-zh] ExpertChoiceRouter; [yj-ja] ExpertChoiceGating):
// block e scores every token with softmax over the token axis of column e
// and keeps the C best tokens by (logit desc, token asc).
//   1. column max m and sum z of exp(l - m) (fixed-order block reductions);
//   2. radix select (4 x 8-bit digits of the order key) of the C-th key;
//   3. ordered compaction: keys above the threshold, then the lowest-index
//      tokens equal to it until C are taken;
//   4. bitonic sort of the C unique 64-bit rank keys in LDS, descending;
//   5. write tokens and scores exp(l - m) / z in rank order.
// ---------------------------------------------------------------------------
constexpr int kEcThreads = 1024;

__device__ inline float block_reduce_max(float v, float *sh) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    v = wave_max(v);
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float r = sh[0];
    for (int w = 1; w < kEcThreads / kWave; ++w) r = fmaxf(r, sh[w]);
    __syncthreads();
    return r;
}
__device__ inline float block_reduce_sum(float v, float *sh) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    v = wave_sum(v);
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float r = sh[0];
    for (int w = 1; w < kEcThreads / kWave; ++w) r += sh[w];
    __syncthreads();
    return r;
}
// Exclusive prefix sum over the block's threads (in thread order).
__device__ inline int block_exclusive_scan(int v, int *sh, int *total) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += n;
    }
    if (lane == kWave - 1) sh[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < kEcThreads / kWave; ++w) {
        if (w < wave) base += sh[w];
        tot += sh[w];
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// CACHE: the expert's column of logits (T <= kEcColMax) is read from global
// memory once, with the stride E, into LDS, and every pass reads it there.
// Histograms are per wave (atomics contend only inside a wave) and are
// summed in wave order.
constexpr int kEcColMax = 16384;
template <bool CACHE>
__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(const float *__restrict__ logits, int T, int E,
                                                               int C, int32_t *__restrict__ ec_idx,
                                                               float *__restrict__ ec_score) {
    constexpr int NW = kEcThreads / kWave;
    __shared__ float shf[NW];
    __shared__ int shi[NW];
    __shared__ uint32_t hist[NW][256];
    __shared__ uint32_t sel_prefix, sel_need;
    __shared__ uint64_t cand[kEcMaxCapacity];
    __shared__ float colc[CACHE ? kEcColMax : 1];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, wave = tid / kWave;
    const float *col = logits + e;
    if constexpr (CACHE) {
        for (int t = tid; t < T; t += kEcThreads) colc[t] = col[(int64_t)t * E];
        __syncthreads();
    }
    auto val = [&](int t) { return CACHE ? colc[t] : col[(int64_t)t * E]; };

    float m = -INFINITY;
    for (int t = tid; t < T; t += kEcThreads) m = fmaxf(m, val(t));
    m = block_reduce_max(m, shf);
    float z = 0.f;
    for (int t = tid; t < T; t += kEcThreads) z += expf(val(t) - m);
    z = block_reduce_sum(z, shf);

    uint32_t prefix = 0, mask = 0, need = (uint32_t)C;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < NW * 256; i += kEcThreads) (&hist[0][0])[i] = 0;
        __syncthreads();
        for (int t = tid; t < T; t += kEcThreads) {
            const uint32_t u = order_key(val(t));
            if ((u & mask) == prefix) atomicAdd(&hist[wave][(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        for (int b = tid; b < 256; b += kEcThreads) {
            uint32_t sum = 0;
            for (int w = 0; w < NW; ++w) sum += hist[w][b];
            hist[0][b] = sum;
        }
        __syncthreads();
        if (wave == 0) {
            // The bucket holding the `need`-th largest key: the first bucket,
            // from the top, whose running count reaches `need` (bucket 0 if
            // none among 255..1 does).  Lane l takes buckets 255-4l .. 252-4l;
            // a wave prefix sum over the lanes' totals gives the running counts.
            const int lane = tid;
            uint32_t sq[4], acc4 = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc4 += hist[0][255 - (4 * lane + q)];
                sq[q] = acc4;
            }
            uint32_t incl = acc4;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t nb = __shfl_up(incl, o, kWave);
                if (lane >= o) incl += nb;
            }
            const uint32_t excl = incl - acc4;
            int qsel = -1;
#pragma unroll
            for (int q = 3; q >= 0; --q)
                if (4 * lane + q <= 254 && excl + sq[q] >= need) qsel = q;
            const uint64_t hit = __ballot(qsel >= 0);
            const int winner = hit ? __ffsll((unsigned long long)hit) - 1 : kWave - 1;
            if (lane == winner) {
                const int q = hit ? qsel : 3;
                const uint32_t before = excl + (q == 0 ? 0u : q == 1 ? sq[0] : q == 2 ? sq[1] : sq[2]);
                sel_need = need - before;
                sel_prefix = prefix | ((uint32_t)(255 - (4 * lane + q)) << shift);
            }
        }
        __syncthreads();
        need = sel_need;
        prefix = sel_prefix;
        mask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t thr = prefix;       // order key of the C-th best token
    const int n_gt = C - (int)need;    // tokens strictly above it; `need` ties are taken

    const int chunk = (T + kEcThreads - 1) / kEcThreads;
    const int t0 = tid * chunk;
    const int t1 = min(T, t0 + chunk);
    int gt = 0, eq = 0;
    for (int t = t0; t < t1; ++t) {
        const uint32_t u = order_key(val(t));
        gt += u > thr;
        eq += u == thr;
    }
    int tot;
    int gt_base = block_exclusive_scan(gt, shi, &tot);
    int eq_base = block_exclusive_scan(eq, shi, &tot);
    for (int t = t0; t < t1; ++t) {
        const float v = val(t);
        const uint32_t u = order_key(v);
        if (u > thr) {
            if (gt_base < n_gt) cand[gt_base] = rank_key(v, (uint32_t)t);
            ++gt_base;
        } else if (u == thr) {
            if (eq_base < (int)need) cand[n_gt + eq_base] = rank_key(v, (uint32_t)t);
            ++eq_base;
        }
    }
    int P = 1;
    while (P < C) P <<= 1;
    if (P <= 2 * kWave) {
        // Up to 128 candidates: wave 0 sorts them in registers, two per lane
        // (elements lane and lane + 64), with a bitonic network of register
        // compares and lane exchanges; zero keys pad to 128 and sort last.
        __syncthreads();
        if (wave == 0) {
            const int lane = tid;
            uint64_t v0 = lane < C ? cand[lane] : 0ull, v1 = lane + kWave < C ? cand[lane + kWave] : 0ull;
            for (int size = 2; size <= 2 * kWave; size <<= 1) {
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    if (stride == kWave) {  // partners in one lane: element lane (lower) and lane + 64
                        const bool desc = (lane & size) == 0;
                        const uint64_t hi = v0 > v1 ? v0 : v1, lo = v0 > v1 ? v1 : v0;
                        v0 = desc ? hi : lo;
                        v1 = desc ? lo : hi;
                    } else {
                        const uint64_t p0 = shfl_xor_u64(v0, stride), p1 = shfl_xor_u64(v1, stride);
                        const bool lower = (lane & stride) == 0;
                        const bool d0 = (lane & size) == 0, d1 = ((lane + kWave) & size) == 0;
                        // the lower index keeps the larger key when descending
                        v0 = (lower == d0) ? (v0 > p0 ? v0 : p0) : (v0 < p0 ? v0 : p0);
                        v1 = (lower == d1) ? (v1 > p1 ? v1 : p1) : (v1 < p1 ? v1 : p1);
                    }
                }
            }
            cand[lane] = v0;
            cand[lane + kWave] = v1;
        }
        __syncthreads();
    } else {
    for (int i = C + tid; i < P; i += kEcThreads) cand[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P / 2; i += kEcThreads) {
                const int lo = 2 * stride * (i / stride) + (i % stride);
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t a = cand[lo], b = cand[hi];
                if ((a < b) == desc) {
                    cand[lo] = b;
                    cand[hi] = a;
                }
            }
            __syncthreads();
        }
    }
    }
    for (int j = tid; j < C; j += kEcThreads) {
        const uint64_t kk = cand[j];
        const float v = key_value((uint32_t)(kk >> 32));
        ec_idx[(int64_t)e * C + j] = (int32_t)rank_key_index(kk);
        ec_score[(int64_t)e * C + j] = expf(v - m) / z;
    }
}

// ---------------------------------------------------------------------------
// Router GEMM with LDS-staged operand tiles and the gating epilogue.
// A block owns TOK tokens and all E experts (padded to EP; with the noisy
// router, EP more columns hold the noise projection x.Wn).  Each K chunk of
// 64 moves the x rows and the weight rows through registers into one of two
// XOR-swizzled LDS buffers (rows past T or E read as zeros through the
// buffer-load limit), and the NTH/64 waves split the columns: wave w computes
// TOK tokens x EPX/(NTH/64) columns on v_mfma_f32_16x16x32_bf16.  The float32
// logits then meet in LDS, the bias (and softplus(x.Wn) * noise) is added in
// a fixed order, and each wave gates whole tokens.
// ---------------------------------------------------------------------------
template <int TOK, int EP, bool NOISY, int PD = 4, int NTH = 256>
__global__ __launch_bounds__(NTH) void router_tile_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ wg, const float *__restrict__ bias, int T, int d, int E,
    int k, int gating, float *__restrict__ logits, int32_t *__restrict__ idx_out, float *__restrict__ w_out,
    const bf16 *__restrict__ wn, const float *__restrict__ noise) {
    constexpr int BK = 64;
    constexpr int NW = NTH / kWave;           // waves
    constexpr int RP = NTH / 8;               // rows one pass of 16-byte chunks covers
    constexpr int EPX = NOISY ? 2 * EP : EP;  // B rows: router weights, then the noise projection
    constexpr int ROWS = TOK + EPX;           // LDS rows per buffer
    constexpr int WTN = EPX / NW;             // columns per wave
    constexpr int TM = TOK / 16, TN = WTN / 16;
    // 16-byte chunks per thread and K chunk; with fewer x rows than one pass,
    // the threads past them load duplicates and skip their LDS stores
    constexpr int XPT = TOK >= RP ? TOK / RP : 1, WPT = EPX / RP;
    static_assert(TM >= 1 && TN >= 1 && WPT >= 1 && (TOK % RP == 0 || RP % TOK == 0), "router tile");
    static_assert(2 * ROWS * BK * 2 >= TOK * EPX * 4, "the logits tile reuses the staging buffers");
    __shared__ __attribute__((aligned(16))) bf16 lds[2][ROWS * BK];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int64_t tok0 = (int64_t)blockIdx.x * TOK;
    const int r0 = tid / 8, ch0 = tid % 8;  // thread moves chunk ch0 of rows r0 + RP*i
    const int xr0 = r0 % TOK;               // its x row (a duplicate when r0 >= TOK)
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x + tok0 * d, (T - tok0) * (int64_t)d * 2);
    const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(wg, (int64_t)E * d * 2);
    const __amdgpu_buffer_rsrc_t nr = NOISY ? buffer_rsrc(wn, (int64_t)E * d * 2) : wr;
    uint32_t xoff[XPT], woff[WPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) xoff[i] = (uint32_t)(((int64_t)(xr0 + RP * i) * d + ch0 * 8) * 2);
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        const int r = r0 + RP * i;
        woff[i] = (uint32_t)(((int64_t)(NOISY && r >= EP ? r - EP : r) * d + ch0 * 8) * 2);
    }
    // rows r0 + RP*i (and TOK + r0 + RP*i, TOK a multiple of 16) share swz(r0)
    const int sdst = r0 * BK + ((ch0 ^ swz(r0)) * 8);
    const bool xstore = r0 < TOK;
    // PD register sets: chunk c is loaded into set c % PD, PD chunks ahead of
    // its MFMAs, so PD - 1 chunks stay in flight while one is computed.
    u32x4 rx[PD][XPT], rw[PD][WPT];
    auto gload = [&](int kc, int set) {
        const int ko = kc * BK * 2;
#pragma unroll
        for (int i = 0; i < XPT; ++i) rx[set][i] = buffer_load16(xr, xoff[i], ko);
#pragma unroll
        for (int i = 0; i < WPT; ++i) rw[set][i] = buffer_load16(NOISY && RP * i >= EP ? nr : wr, woff[i], ko);
    };
    auto lstore = [&](bf16 *L, int set) {
        if (xstore) {
#pragma unroll
            for (int i = 0; i < XPT; ++i) store16(L + sdst + i * RP * BK, rx[set][i]);
        }
#pragma unroll
        for (int i = 0; i < WPT; ++i) store16(L + TOK * BK + sdst + i * RP * BK, rw[set][i]);
    };
    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fragment lanes: row lane % 16, 16-byte k chunk lane / 16 of a 32-k substep
    const int sw = swz(lane % 16);
    const int fa0 = (lane % 16) * BK, fb0 = (TOK + wave * WTN + lane % 16) * BK;
    auto compute = [&](const bf16 *L) {
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int c = ((ks * 4 + lane / 16) ^ sw) * 8;
            bf16x8 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = __builtin_bit_cast(bf16x8, load16(L + fa0 + i * 16 * BK + c));
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = __builtin_bit_cast(bf16x8, load16(L + fb0 + j * 16 * BK + c));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };
    const int nk = d / BK;
#pragma unroll
    for (int c = 0; c < PD; ++c) gload(min(c, nk - 1), c);
    lstore(lds[0], 0);
    __syncthreads();
    // chunk kc: refill its set's predecessor (set kc % PD, stored at the end
    // of the previous chunk) with chunk kc + PD, compute chunk kc from LDS,
    // store chunk kc + 1 into the other LDS buffer.  Past the last chunk the
    // loads re-read chunk nk - 1 and the stores fill a buffer nobody reads.
    for (int k0 = 0; k0 < nk; k0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            const int kc = k0 + u;
            if (kc < nk) {
                gload(min(kc + PD, nk - 1), u);
                compute(lds[kc & 1]);
                lstore(lds[(kc + 1) & 1], (u + 1) % PD);
                __syncthreads();
            }
        }
    }
    // float32 logits tile [TOK][EPX] in the (now free) staging buffers;
    // D[4*(lane/16) + q][lane % 16] of each 16x16 tile is acc[q]
    float *Lf = reinterpret_cast<float *>(&lds[0][0]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                Lf[(i * 16 + 4 * (lane / 16) + q) * EPX + wave * WTN + j * 16 + lane % 16] = acc[i][j][q];
    __syncthreads();
    for (int tt = wave; tt < TOK; tt += NW) {
        const int64_t t = tok0 + tt;
        if (t >= T) break;
        float *row = Lf + tt * EPX;
        // lane l owns experts l + 64q, the entries gate_one_token reads back
        for (int e = lane; e < E; e += kWave) {
            float v = row[e];
            if (bias) v += bias[e];
            if constexpr (NOISY) v += softplus(row[EP + e]) * noise[t * E + e];
            row[e] = v;
            if (logits) logits[t * E + e] = v;
        }
        if (gating != kGateExpertChoice) gate_one_token(row, E, k, gating, t, idx_out, w_out);
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int TOK, int EP>
static void launch_router_tile_t(const RouteArgs &a, hipStream_t s) {
    const int grid = (a.T + TOK - 1) / TOK;
    // register sets in flight: four, or two when a set is large (noisy, 256 experts)
    constexpr int PDN = (TOK + 2 * EP) / 32 <= 10 ? 4 : 2;
    if (a.wn)
        hipLaunchKernelGGL((router_tile_kernel<TOK, EP, true, PDN>), dim3(grid), dim3(256), 0, s, (const bf16 *)a.x,
                           (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           (const bf16 *)a.wn, a.noise);
    else if constexpr (EP >= 128)  // 8 waves: 2 per SIMD (DeepSeek-style router 124 -> 109 us)
        hipLaunchKernelGGL((router_tile_kernel<TOK, EP, false, 4, 512>), dim3(grid), dim3(512), 0, s,
                           (const bf16 *)a.x, (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits,
                           a.idx, a.w, nullptr, nullptr);
    else
        hipLaunchKernelGGL((router_tile_kernel<TOK, EP, false>), dim3(grid), dim3(256), 0, s, (const bf16 *)a.x,
                           (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           nullptr, nullptr);
}

template <int TOK>
static void launch_router_tile(const RouteArgs &a, hipStream_t s) {
    if (a.E <= 64) launch_router_tile_t<TOK, 64>(a, s);
    else if (a.E <= 128) launch_router_tile_t<TOK, 128>(a, s);
    else launch_router_tile_t<TOK, 256>(a, s);
}

template <int NT, int WK>
static void launch_route_bf16_wk(const RouteArgs &a, const RoutePermuteArgs *perm, hipStream_t s) {
    const int grid = (a.T + 15) / 16;
    if (perm) {  // one block (route_permute_fits): route, then permute in the same block
        const size_t lds = (size_t)((a.T + kChunk - 1) / kChunk) * a.E * 16;
        hipLaunchKernelGGL((route_bf16_kernel<NT, WK, false, true>), dim3(1), dim3(64 * WK), lds, s,
                           (const bf16 *)a.x, (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits,
                           a.idx, a.w, nullptr, nullptr, *perm);
    } else if (a.wn) {
        hipLaunchKernelGGL((route_bf16_kernel<NT, WK, true>), dim3(grid), dim3(64 * WK), 0, s, (const bf16 *)a.x,
                           (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           (const bf16 *)a.wn, a.noise, RoutePermuteArgs{});
    } else {
        hipLaunchKernelGGL((route_bf16_kernel<NT, WK, false>), dim3(grid), dim3(64 * WK), 0, s, (const bf16 *)a.x,
                           (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           nullptr, nullptr, RoutePermuteArgs{});
    }
}

// K-split depth: 16 waves once each holds at least eight 32-wide chunks.
template <int NT>
static void launch_route_bf16_t(const RouteArgs &a, hipStream_t s, const RoutePermuteArgs *perm = nullptr) {
    const int nk = a.d / 32;
    if (nk >= 128) launch_route_bf16_wk<NT, 16>(a, perm, s);
    else if (nk >= 32) launch_route_bf16_wk<NT, 8>(a, perm, s);
    else launch_route_bf16_wk<NT, 4>(a, perm, s);
}

bool route_permute_fits(int T, int E, bool bf16, bool expert_choice) {
    return bf16 && !expert_choice && T >= 1 && T <= 16 && E <= 16;
}

void launch_route_permute(const RouteArgs &a, const RoutePermuteArgs &p, hipStream_t s) {
    launch_route_bf16_t<1>(a, s, &p);
}

void launch_route(const RouteArgs &a, hipStream_t s) {
    if (a.T == 0) return;
    if (!a.bf16) {
        hipLaunchKernelGGL(route_f32_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, (const float *)a.x,
                           (const float *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           (const float *)a.wn, a.noise);
        return;
    }
    // Up to 16 experts: per-wave K slices straight from global memory.  More
    // experts: LDS-staged tiles, so that a block's tokens share each weight
    // row instead of every 16-token wave re-reading all of them from L2.
    if (a.E <= 16) {
        launch_route_bf16_t<1>(a, s);
        return;
    }
    // 32-token blocks unless that already gives a block per CU twice over
    if (a.T >= 64 * 512) launch_router_tile<64>(a, s);
    else launch_router_tile<32>(a, s);
}

void launch_gate_logits(const float *logits, int T, int E, int k, int gating, int32_t *idx, float *w,
                        hipStream_t s) {
    if (T == 0) return;
    hipLaunchKernelGGL(gate_logits_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, gating, idx, w);
}

void launch_ec_select(const float *logits, int T, int E, int C, int32_t *ec_idx, float *ec_score,
                      hipStream_t s) {
    if (T <= kEcColMax)
        hipLaunchKernelGGL(ec_select_kernel<true>, dim3(E), dim3(kEcThreads), 0, s, logits, T, E, C, ec_idx, ec_score);
    else
        hipLaunchKernelGGL(ec_select_kernel<false>, dim3(E), dim3(kEcThreads), 0, s, logits, T, E, C, ec_idx, ec_score);
}

}  // namespace moe
