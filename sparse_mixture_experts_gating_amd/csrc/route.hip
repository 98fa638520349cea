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
#include "plan.h"
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

// One lane gates one token of E <= EMAX <= kLaneGateMax experts (logits at
// `row`, in LDS or global memory), with the selection and weights of
// gate_one_token: slot j takes the largest logit not taken by slots 0..j-1
// (order_key; the lowest index among equal keys), so the slots come out in
// rank order; the softmax sums run in slot order (topk-softmax) or expert
// order (softmax-topk, switch).  For few experts a wave gates up to 64
// tokens this way in fewer instructions than the wave-wide selection (DPP
// maxima of 64-bit keys) takes for one.
constexpr int kLaneGateMax = 16;
template <int EMAX>
__device__ __forceinline__ void gate_token_lane(const float *row, int E, int k, int gating, int64_t t,
                                       int32_t *__restrict__ idx_out, float *__restrict__ w_out) {
    static_assert(EMAX <= kLaneGateMax, "experts of one lane");
    float v[EMAX];
    uint32_t key[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
        v[e] = e < E ? row[e] : 0.f;
        key[e] = order_key(v[e]);
    }
    // k <= E (checked by the API); the slots are unrolled so that their
    // values stay in registers, and k, uniform over the wave, ends them
    float sel[EMAX];
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < EMAX; ++j) {
        if (j >= k) continue;
        int best = 0;
        uint32_t bk = 0;
        float bv = 0.f;
        bool any = false;
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
            const bool ok = e < E && !((taken >> e) & 1u) && (!any || key[e] > bk);
            any = any || ok;
            best = ok ? e : best;
            bk = ok ? key[e] : bk;
            bv = ok ? v[e] : bv;
        }
        taken |= 1u << best;
        sel[j] = bv;
        idx_out[t * k + j] = best;
    }
    const float top = sel[0];
    float z = 0.f;
    if (gating == kGateTopkSoftmax) {
#pragma unroll
        for (int j = 0; j < EMAX; ++j)
            if (j < k) z += expf(sel[j] - top);
    } else {
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E) z += expf(v[e] - top);
    }
#pragma unroll
    for (int j = 0; j < EMAX; ++j)
        if (j < k) w_out[t * k + j] = expf(sel[j] - top) / z;
}
template <int EMAX_HI = kLaneGateMax>
__device__ __forceinline__ void gate_token_lane_any(const float *row, int E, int k, int gating, int64_t t,
                                           int32_t *__restrict__ idx_out, float *__restrict__ w_out) {
    if (E <= 8) gate_token_lane<8>(row, E, k, gating, t, idx_out, w_out);
    else gate_token_lane<EMAX_HI>(row, E, k, gating, t, idx_out, w_out);
}

// EG lanes (EG = 8 or 16) gate one token of E <= EG experts whose logits are
// at `row` (LDS), with the selection and weights of gate_token_lane.  Lane
// e takes its expert's slot as the number of experts ranked above it (a
// larger order_key, or an equal key at a lower index), so each lane runs a
// few dozen independent instructions where one lane per token runs k
// dependent passes over all experts (about 2 us at the end of every router
// block).  The largest logit is the rank-0 expert's value; the softmax sums
// run in slot order (topk-softmax: the selected logits pass through `sel`,
// EG floats of LDS per token) or expert order (softmax-topk, switch),
// exactly as in gate_token_lane.  `live` is false for the padding tokens
// of a ragged last block (they write nothing).
template <int EG>
__device__ __forceinline__ void gate_token_group(const float *row, float *sel, int E, int k, int gating,
                                                 bool live, int64_t t, int32_t *__restrict__ idx_out,
                                                 float *__restrict__ w_out) {
    const int e = threadIdx.x % EG;
    float v[EG];
    uint32_t key[EG];
#pragma unroll
    for (int j = 0; j < EG; ++j) {
        v[j] = j < E ? row[j] : 0.f;
        key[j] = order_key(v[j]);
    }
    const float mine = e < E ? row[e] : 0.f;
    const uint32_t kmine = order_key(mine);
    int rank = 0;
    uint32_t mk = 0;
#pragma unroll
    for (int j = 0; j < EG; ++j)
        if (j < E) {
            rank += (key[j] > kmine || (key[j] == kmine && j < e)) ? 1 : 0;
            mk = key[j] > mk ? key[j] : mk;
        }
    float top = 0.f;
#pragma unroll
    for (int j = EG - 1; j >= 0; --j)
        if (j < E && key[j] == mk) top = v[j];  // the lowest index among equal maxima
    const bool chosen = e < E && rank < k;
    float z = 0.f;
    if (gating == kGateTopkSoftmax) {
        if (chosen) sel[rank] = mine;
        __builtin_amdgcn_wave_barrier();  // the slot values are written before they are read back
#pragma unroll
        for (int j = 0; j < EG; ++j)
            if (j < k) z += expf(sel[j] - top);
    } else {
#pragma unroll
        for (int j = 0; j < EG; ++j)
            if (j < E) z += expf(v[j] - top);
    }
    if (live && chosen) {
        idx_out[t * k + rank] = e;
        w_out[t * k + rank] = expf(mine - top) / z;
    }
}

// Router GEMM on bf16 MFMA (v_mfma_f32_16x16x32_bf16) + gating epilogue for
// few experts (16*NT at most; launched for up to 16).  A block owns 16 tokens
// and its WK waves split the model dimension into WK contiguous ranges.  Each
// wave computes 16 tokens x 16*NT experts over its range straight from global
// memory, issuing U chunks of x and of the router weights before their MFMAs
// so that enough bytes are in flight to stream x at HBM rate (x rows are read
// once; the router weights stay in L1/L2).  Partial sums meet in LDS in a
// fixed order, the bias is added, logits are written, and the first TOK lanes
// gate one token each.
__device__ inline float softplus(float u) { return fmaxf(u, 0.f) + log1pf(expf(-fabsf(u))); }

// NOISY adds the noise projection as a second MFMA accumulator set and forms
// x.Wg + b + softplus(x.Wn) * noise ([yj-ja] TopKGating, training branch).
// PERM (a batch of one block, T <= 16): the block then permutes its own
// selections (permute_small_block) and writes the tile plan, which saves
// the permutation launch of a decode step.
// PAIR (at most 8 experts, d % 64 == 0, no noise): each 64-wide k step is
// cut into two 32-wide segments that share one MFMA.  Row r of the A operand
// is token r % 8 of an 8-token group over segment r / 8, column c of B is
// expert c % 8 over segment c / 8, so the two diagonal 8 x 8 blocks of the
// product hold the two segments' partial sums and the others are discarded.
// One load instruction then covers 128 contiguous bytes of each of 8 token
// rows (whole cache lines, where the layout above reads half lines of 16
// rows), both token groups of a block share each B load, and no B lane
// loads a duplicate expert row.  Prefill router of the Mixtral-shape layer
// (4096 tokens, d = 4096, bare kernels): 11.0 -> 10.0 us.
template <int NT, int WK, bool NOISY, bool PERM = false, bool PAIR = false>
__global__ __launch_bounds__(64 * WK) void route_bf16_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ wg, const float *__restrict__ bias,
    int T, int d, int E, int k, int gating, float *__restrict__ logits,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out, const bf16 *__restrict__ wn,
    const float *__restrict__ noise, RoutePermuteArgs perm, float *__restrict__ logits_t,
    int32_t *__restrict__ fill_rows) {
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
    if constexpr (PAIR) {
        static_assert(NT == 1 && !NOISY, "paired segments: up to 8 experts, no noise projection");
        constexpr int UP = 4;  // 64-wide steps in flight per wave
        const int seg = r / 8;
        const bf16 *xp[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            int64_t t = tok0 + 8 * g + r % 8;
            if (t >= T) t = T - 1;
            xp[g] = x + t * d + seg * 32 + kq;
        }
        int e = r % 8;
        if (e >= E) e = E - 1;
        const bf16 *wp = wg + (int64_t)e * d + seg * 32 + kq;
        f32x4 pacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        const int n64 = d / 64;
        const int kb = n64 * wk / WK, ke = n64 * (wk + 1) / WK;
        for (int kc = kb; kc < ke; kc += UP) {
            bf16x8 a[UP][2], b[UP];
#pragma unroll
            for (int u = 0; u < UP; ++u) {
                // steps past this wave's range re-read its last step (unused)
                const int ko = min(kc + u, ke - 1) * 64;
#pragma unroll
                for (int g = 0; g < 2; ++g) a[u][g] = __builtin_bit_cast(bf16x8, load16(xp[g] + ko));
                b[u] = __builtin_bit_cast(bf16x8, load16(wp + ko));
            }
#pragma unroll
            for (int u = 0; u < UP; ++u)
                if (kc + u < ke)
#pragma unroll
                    for (int g = 0; g < 2; ++g)
                        pacc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][g], b[u], pacc[g], 0, 0, 0);
        }
        // D[row 4*(lane/16) + j][col r]: the diagonal blocks (row / 8 ==
        // col / 8) go to the partial table, segment 0 in columns 0..7 and
        // segment 1 in columns 8..15
        if (lane / 32 == seg) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    part[(wk * TOK + 8 * g + (4 * (lane / 16) + j) % 8) * LD + r] = pacc[g][j];
        }
    } else {
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
    }
    __syncthreads();
    for (int i = threadIdx.x; i < TOK * EP; i += 64 * WK) {
        const int tt = i / EP, e = i % EP;
        float s;
        if constexpr (PAIR) {
            if (e >= 8) continue;
            s = part[tt * LD + e] + part[tt * LD + 8 + e];
#pragma unroll
            for (int w = 1; w < WK; ++w) s += part[(w * TOK + tt) * LD + e] + part[(w * TOK + tt) * LD + 8 + e];
        } else {
            s = part[tt * LD + e];
#pragma unroll
            for (int w = 1; w < WK; ++w) s += part[(w * TOK + tt) * LD + e];
        }
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
    if (gating == kGateExpertChoice) {
        if (logits_t) {
            // transposed logits (16 consecutive tokens of each expert) and
            // the -1 fill of these tokens' rows of the row map
            for (int i = threadIdx.x; i < TOK * E; i += 64 * WK) {
                const int e = i / TOK, tt = i % TOK;
                if (tok0 + tt < T) logits_t[(int64_t)e * T + tok0 + tt] = part[tt * LD + e];
            }
            for (int i = threadIdx.x; i < TOK * E; i += 64 * WK)
                if (tok0 + i / E < T) fill_rows[tok0 * E + i] = -1;
        }
        return;
    }
    // EG lanes per token (16 tokens x EG <= 256 threads <= the block)
    static_assert(EP <= 16 && 64 * WK >= TOK * 16, "group gating covers the block's tokens and experts");
    __shared__ float selv[TOK * 16];
    if (E <= 8) {
        if (threadIdx.x < TOK * 8) {
            const int tt = threadIdx.x / 8;
            gate_token_group<8>(part + tt * LD, selv + tt * 16, E, k, gating, tok0 + tt < T, tok0 + tt, idx_out,
                                w_out);
        }
    } else if (threadIdx.x < TOK * 16) {
        const int tt = threadIdx.x / 16;
        gate_token_group<16>(part + tt * LD, selv + tt * 16, E, k, gating, tok0 + tt < T, tok0 + tt, idx_out,
                             w_out);
    }
    if constexpr (PERM) {
        extern __shared__ unsigned long long perm_lds[];
        __syncthreads();  // every token's selection is written (and visible to the block)
        permute_small_block<64 * WK>(idx_out, T, E, k, perm.capacity, perm.group_chunks, perm.counts,
                                     perm.offsets, perm.row_token, perm.slot_row, perm.plan, perm_lds);
    }
}

// float32 router (VALU) plus gating, one wave per token.  Up to 64 experts
// (d % 16 == 0, 16-byte aligned rows): lane l takes expert l / S and the
// 4-float chunks l % S, l % S + S, ... of the model dimension in order, with
// S = 64 / (E rounded up to a power of two); an expert's S partial sums meet
// in an xor butterfly over its S lanes, which leaves the same sum in each
// (a + b == b + a), so the order is fixed.  Basic top-2 layer (8 experts,
// d = 128): 15 -> 6 us, where one lane per expert walked the whole row with
// 4-byte loads.  More experts: one lane per expert over the whole row.
__global__ __launch_bounds__(256) void route_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ wg, const float *__restrict__ bias,
    int T, int d, int E, int k, int gating, float *__restrict__ logits,
    int32_t *__restrict__ idx_out, float *__restrict__ w_out, const float *__restrict__ wn,
    const float *__restrict__ noise) {
    __shared__ float rows[4][256];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    const bool live = t < T;
    if (live && E <= kWave) {
        int ep = 1;
        while (ep < E) ep <<= 1;
        const int S = kWave / ep, e = lane / S, sl = lane % S;
        const int ec = e < E ? e : E - 1;
        const float4 *xr = (const float4 *)(x + t * d);
        const float4 *wr = (const float4 *)(wg + (int64_t)ec * d);
        const float4 *nr = wn ? (const float4 *)(wn + (int64_t)ec * d) : nullptr;
        float sum = 0.f, u = 0.f;
        for (int c = sl; c < d / 4; c += S) {
            const float4 a = xr[c], b = wr[c];
            sum = fmaf(a.x, b.x, sum);
            sum = fmaf(a.y, b.y, sum);
            sum = fmaf(a.z, b.z, sum);
            sum = fmaf(a.w, b.w, sum);
            if (nr) {
                const float4 q = nr[c];
                u = fmaf(a.x, q.x, u);
                u = fmaf(a.y, q.y, u);
                u = fmaf(a.z, q.z, u);
                u = fmaf(a.w, q.w, u);
            }
        }
        for (int o = 1; o < S; o <<= 1) {
            sum += __shfl_xor(sum, o, kWave);
            if (nr) u += __shfl_xor(u, o, kWave);
        }
        if (sl == 0 && e < E) {
            float v = sum;
            if (bias) v += bias[e];
            if (nr) v += softplus(u) * noise[t * E + e];
            rows[wave][e] = v;
            if (logits) logits[t * E + e] = v;
        }
    } else if (live) {
        for (int e = lane; e < E; e += kWave) {
            const float *xr = x + t * d;
            const float *wr = wg + (int64_t)e * d;
            float v = 0.f;
            for (int i = 0; i < d; ++i) v = fmaf(xr[i], wr[i], v);
            if (bias) v += bias[e];
            if (wn) {
                const float *nr = wn + (int64_t)e * d;
                float u = 0.f;
                for (int i = 0; i < d; ++i) u = fmaf(xr[i], nr[i], u);
                v += softplus(u) * noise[t * E + e];
            }
            rows[wave][e] = v;
            if (logits) logits[t * E + e] = v;
        }
    }
    __syncthreads();
    if (gating == kGateExpertChoice) return;
    if (E <= kLaneGateMax) {
        const int64_t tl = (int64_t)blockIdx.x * 4 + threadIdx.x;
        if (threadIdx.x < 4 && tl < T) gate_token_lane_any(rows[threadIdx.x], E, k, gating, tl, idx_out, w_out);
    } else if (live) {
        gate_one_token(rows[wave], E, k, gating, t, idx_out, w_out);
    }
}

// Logits from the router GEMM's K parts: l[t][e] = sum of the S parts in
// part order, plus the bias, written out and gated from LDS with the same
// selection and weights as the fused routers.  One wave per token.  VEC (E a
// multiple of 4, logits and bias 16-byte aligned): lane l owns experts
// 4l .. 4l+3, and all S of its 16-byte part loads are issued before any is
// added (with the parts' loads in one dependent chain, the gating of the
// DeepSeek-style layer's 8192 tokens took 23 us); the sum runs in the same
// order either way.
template <int S, bool VEC>
__global__ __launch_bounds__(256) void gate_partials_kernel(const float *__restrict__ part,
                                                            const float *__restrict__ bias, int T, int E, int k,
                                                            int gating, float *__restrict__ logits,
                                                            int32_t *__restrict__ idx_out, float *__restrict__ w_out) {
    __shared__ __attribute__((aligned(16))) float rows[4][256];  // 16-byte row stores below
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int64_t slab = (int64_t)T * E;
    if constexpr (VEC) {
        const int e0 = 4 * lane;
        if (e0 < E) {
            f32x4 p[S];
#pragma unroll
            for (int q = 0; q < S; ++q) p[q] = *(const f32x4 *)(part + q * slab + t * E + e0);
            f32x4 v = p[0];
#pragma unroll
            for (int q = 1; q < S; ++q) v += p[q];
            if (bias) v += *(const f32x4 *)(bias + e0);
            *(f32x4 *)(&rows[wave][e0]) = v;
            *(f32x4 *)(logits + t * E + e0) = v;
        }
    } else {
        for (int e = lane; e < E; e += kWave) {
            float p[S];
#pragma unroll
            for (int q = 0; q < S; ++q) p[q] = part[q * slab + t * E + e];
            float v = p[0];
#pragma unroll
            for (int q = 1; q < S; ++q) v += p[q];
            if (bias) v += bias[e];
            rows[wave][e] = v;
            logits[t * E + e] = v;
        }
    }
    // gate_one_token reads back the entries each lane wrote; the barrier
    // keeps the compiler from moving those LDS reads above the writes
    __builtin_amdgcn_wave_barrier();
    gate_one_token(rows[wave], E, k, gating, t, idx_out, w_out);
}

template <int S>
static void launch_gate_partials_s(const float *part, const float *bias, int T, int E, int k, int gating,
                                   float *logits, int32_t *idx, float *w, hipStream_t s) {
    const bool vec = (E & 3) == 0 && ((uintptr_t)logits & 15u) == 0 && ((uintptr_t)bias & 15u) == 0 &&
                     ((uintptr_t)part & 15u) == 0;
    auto kern = vec ? gate_partials_kernel<S, true> : gate_partials_kernel<S, false>;
    hipLaunchKernelGGL(kern, dim3((T + 3) / 4), dim3(256), 0, s, part, bias, T, E, k, gating, logits, idx, w);
}

void launch_gate_partials(const float *part, int S, const float *bias, int T, int E, int k, int gating,
                          float *logits, int32_t *idx, float *w, hipStream_t s) {
    if (T == 0) return;
    static_assert(kRouterMaxSplit == 8, "one instantiation per part count");
    switch (S) {
        case 1: launch_gate_partials_s<1>(part, bias, T, E, k, gating, logits, idx, w, s); break;
        case 2: launch_gate_partials_s<2>(part, bias, T, E, k, gating, logits, idx, w, s); break;
        case 3: launch_gate_partials_s<3>(part, bias, T, E, k, gating, logits, idx, w, s); break;
        case 4: launch_gate_partials_s<4>(part, bias, T, E, k, gating, logits, idx, w, s); break;
        case 5: launch_gate_partials_s<5>(part, bias, T, E, k, gating, logits, idx, w, s); break;
        case 6: launch_gate_partials_s<6>(part, bias, T, E, k, gating, logits, idx, w, s); break;
        case 7: launch_gate_partials_s<7>(part, bias, T, E, k, gating, logits, idx, w, s); break;
        default: launch_gate_partials_s<8>(part, bias, T, E, k, gating, logits, idx, w, s); break;
    }
}

// Gating alone on given float32 logits [T][E]: one lane per token for up to
// kLaneGateMax experts, else one wave per token.
__global__ __launch_bounds__(256) void gate_logits_lane_kernel(const float *__restrict__ logits, int T, int E,
                                                                int k, int gating, int32_t *__restrict__ idx_out,
                                                                float *__restrict__ w_out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < T) gate_token_lane_any(logits + t * E, E, k, gating, t, idx_out, w_out);
}
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
//   1. radix select (4 x 8-bit digits of the order key) of the C-th key
//      over the tokens at or above a cheap lower bound of it, with the
//      column max m and the sum z of exp(l - m) (fixed-order reductions)
//      computed in its first two passes;
//   2. ordered compaction: keys above the threshold, then the lowest-index
//      tokens equal to it until C are taken;
//   3. the C unique 64-bit rank keys in descending order (rank sort up to
//      128 of them, else a bitonic sort in LDS);
//   4. write tokens and scores exp(l - m) / z in rank order.
// ---------------------------------------------------------------------------
constexpr int kEcThreads = 1024;

// Exclusive prefix sum over the block's threads (in thread order).
__device__ inline int block_exclusive_scan(int v, int *sh, int *total) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
    const int incl = wave_incl_scan(v);
    if (lane == kWave - 1) sh[wave] = incl;
    __syncthreads();
    // the waves' totals, one per lane, scanned the same way
    constexpr int NW = kEcThreads / kWave;
    const int ws = wave_incl_scan(lane < NW ? sh[lane] : 0);
    const int base = wave > 0 ? __builtin_amdgcn_readlane(ws, wave - 1) : 0;
    *total = __builtin_amdgcn_readlane(ws, NW - 1);
    __syncthreads();
    return base + incl - v;
}

// CACHE: the expert's column of logits (T <= kEcColMax) is read from global
// memory once, with the stride E, into LDS, and every pass reads it there.
// Histograms are per wave (atomics contend only inside a wave) and are
// summed in wave order.
constexpr int kEcColMax = 16384;
template <bool CACHE>
__global__ __launch_bounds__(kEcThreads) void ec_select_kernel(const float *__restrict__ logits,
                                                               const float *__restrict__ logits_t, int T, int E,
                                                               int C, int32_t *__restrict__ ec_idx,
                                                               float *__restrict__ ec_score, EcPermuteArgs perm) {
    constexpr int NW = kEcThreads / kWave;
    __shared__ float shf[NW];
    __shared__ int shi[NW];
    __shared__ float shz[NW];
    __shared__ uint32_t shk[NW];
    __shared__ uint32_t hist[2][NW][256];  // per-wave histograms, two passes' worth
    __shared__ uint32_t sel_prefix[2], sel_need[2];
    __shared__ uint64_t cand[kEcMaxCapacity];
    __shared__ float colc[CACHE ? kEcColMax : 1];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, wave = tid / kWave;
    // the expert's column: contiguous in the transposed logits, else with
    // stride E (each element its own cache line: the column read had been a
    // quarter of the kernel)
    const float *col = logits_t ? logits_t + (int64_t)e * T : logits + e;
    const int64_t cs = logits_t ? 1 : E;
    for (int i = tid; i < NW * 256; i += kEcThreads) hist[0][0][i] = 0;
    if constexpr (CACHE) {
        // eight loads in flight per thread before their LDS stores
        for (int t0 = tid; t0 < T; t0 += 8 * kEcThreads) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u * kEcThreads;
                v[u] = t < T ? col[(int64_t)t * cs] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u * kEcThreads;
                if (t < T) colc[t] = v[u];
            }
        }
        __syncthreads();
    }
    auto val = [&](int t) { return CACHE ? colc[t] : col[(int64_t)t * cs]; };
    // This thread's tokens: the contiguous chunk t0 .. t1 - 1, held in
    // registers when the column is cached (at most kEcColMax / kEcThreads =
    // 16 of them), so that every pass below is register arithmetic.
    const int chunk = (T + kEcThreads - 1) / kEcThreads;
    const int t0 = tid * chunk, t1 = min(T, t0 + chunk), nmine = max(0, t1 - t0);
    constexpr int kMaxChunk = CACHE ? kEcColMax / kEcThreads : 1;
    float cv[kMaxChunk];
    if constexpr (CACHE) {
#pragma unroll
        for (int j = 0; j < kMaxChunk; ++j) cv[j] = j < nmine ? colc[t0 + j] : 0.f;
    }
    auto for_mine = [&](auto f) __attribute__((always_inline)) {
        if constexpr (CACHE) {
#pragma unroll
            for (int j = 0; j < kMaxChunk; ++j)
                if (j < nmine) f(t0 + j, cv[j]);
        } else {
            for (int t = t0; t < t1; ++t) f(t, val(t));
        }
    };
    const int lane = tid % kWave;
    // fixed-tree reductions over the waves' values, one per lane
    auto waves_max = [&](const float *sh) {
        float r = lane < NW ? sh[lane] : -INFINITY;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) r = fmaxf(r, __shfl_xor(r, o, kWave));
        return __shfl(r, 0, kWave);
    };
    auto waves_sum = [&](const float *sh) {
        float r = lane < NW ? sh[lane] : 0.f;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) r += __shfl_xor(r, o, kWave);
        return __shfl(r, 0, kWave);
    };

    // A lower bound of the C-th largest key when C <= NG = kEcThreads / 8:
    // the smallest of the largest keys of NG disjoint groups of tokens (the
    // chunks of 8 consecutive threads).  At least NG distinct tokens reach
    // it, so the C best all do, and the radix passes count only the tokens
    // at or above it (Gaussian logits, T = 8192, C = 128: about 6% of them).
    // Taken on order keys, so that -0.0 and 0.0 stay apart.
    constexpr int NG = kEcThreads / 8;
    uint32_t floor_key = 0;
    const bool filtered = C <= NG;
    if (filtered) {
        uint32_t km = 0;  // no token: the lowest key (then no filtering)
        for_mine([&](int, float v) { km = max(km, order_key(v)); });
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) km = max(km, (uint32_t)__shfl_xor((int)km, o, kWave));
#pragma unroll
        for (int o = 8; o < kWave; o <<= 1) km = min(km, (uint32_t)__shfl_xor((int)km, o, kWave));
        if (lane == 0) shk[wave] = km;
        __syncthreads();  // also orders the hist[0] clearing before pass 0
        uint32_t f = lane < NW ? shk[lane] : 0xFFFFFFFFu;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) f = min(f, (uint32_t)__shfl_xor((int)f, o, kWave));
        floor_key = (uint32_t)__shfl((int)f, 0, kWave);
    } else {
        __syncthreads();  // hist[0] cleared
    }
    // Radix select with two barriers per pass: the histograms of a pass are
    // cleared during the pass before (hist[pass & 1], cleared in pass - 1
    // or above), wave 0 alone sums the histograms and picks the bucket, and
    // the picks alternate between two slots.  The column max m rides along
    // in pass 0 and the sum z of exp(l - m) in pass 1 (each thread's chunk
    // in order, then a wave reduction, then a fixed tree over the waves).
    float m = -INFINITY, z = 0.f;
    uint32_t prefix = 0, mask = 0, need = (uint32_t)C;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        // filtered: few keys take part, and all waves share one histogram
        // (row 0); else one histogram per wave (atomics contend only inside
        // a wave), summed by wave 0
        uint32_t(*H)[256] = hist[pass & 1];
        uint32_t *Hw = H[filtered ? 0 : wave];
        const int nrows = filtered ? 1 : NW;
        uint32_t *Hn = &hist[(pass + 1) & 1][0][0];
        for (int i = tid; i < nrows * 256; i += kEcThreads) Hn[i] = 0;
        if (pass == 0) for_mine([&](int, float v) { m = fmaxf(m, v); });
        if (pass == 1) for_mine([&](int, float v) { z += expf(v - m); });
        for_mine([&](int, float v) {
            const uint32_t u = order_key(v);
            if (u >= floor_key && (u & mask) == prefix) atomicAdd(&Hw[(u >> shift) & 255u], 1u);
        });
        if (pass == 0) {
            const float wm = wave_max(m);
            if (lane == 0) shf[wave] = wm;
        } else if (pass == 1) {
            const float wz = wave_sum(z);
            if (lane == 0) shz[wave] = wz;
        }
        __syncthreads();
        if (pass == 0) m = waves_max(shf);
        else if (pass == 1) z = waves_sum(shz);
        if (wave == 0) {
            // The bucket holding the `need`-th largest key: the first bucket,
            // from the top, whose running count reaches `need` (bucket 0 if
            // none among 255..1 does).  Lane l takes buckets 255-4l .. 252-4l
            // (summed over the histograms); a wave prefix sum over the
            // lanes' totals gives the running counts.
            uint32_t sq[4], acc4 = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int b = 255 - (4 * lane + q);
                uint32_t hb = 0;
                for (int w = 0; w < nrows; ++w) hb += H[w][b];
                acc4 += hb;
                sq[q] = acc4;
            }
            const uint32_t incl = (uint32_t)wave_incl_scan((int)acc4);
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
                sel_need[pass & 1] = need - before;
                sel_prefix[pass & 1] = prefix | ((uint32_t)(255 - (4 * lane + q)) << shift);
            }
        }
        __syncthreads();
        need = sel_need[pass & 1];
        prefix = sel_prefix[pass & 1];
        mask |= 255u << shift;
    }
    const uint32_t thr = prefix;       // order key of the C-th best token
    const int n_gt = C - (int)need;    // tokens strictly above it; `need` ties are taken

    int gt = 0, eq = 0;
    for_mine([&](int, float v) {
        const uint32_t u = order_key(v);
        gt += u > thr;
        eq += u == thr;
    });
    // one scan for both counts, packed in 16-bit halves (every prefix is
    // at most T, so both halves fit while T < 2^15)
    int tot, gt_base, eq_base;
    if (T < 32768) {
        const int both = block_exclusive_scan((gt << 16) | eq, shi, &tot);
        gt_base = both >> 16;
        eq_base = both & 0xFFFF;
    } else {
        gt_base = block_exclusive_scan(gt, shi, &tot);
        eq_base = block_exclusive_scan(eq, shi, &tot);
    }
    // (branch-free counters: incremented in branches, the compiler kept
    // the two in a private array)
    for_mine([&](int t, float v) {
        const uint32_t u = order_key(v);
        const bool g = u > thr, q = u == thr;
        if (g && gt_base < n_gt) cand[gt_base] = rank_key(v, (uint32_t)t);
        if (q && eq_base < (int)need) cand[n_gt + eq_base] = rank_key(v, (uint32_t)t);
        gt_base += g;
        eq_base += q;
    });
    int P = 1;
    while (P < C) P <<= 1;
    if (P <= 2 * kWave) {
        // Up to 128 candidates with unique keys (the token index is part of
        // the key): candidate i goes to position #(candidates with a larger
        // key).  The threads split the comparisons: thread tid compares
        // candidate tid % 128 with the 16 candidates 16 (tid / 128) .. + 15
        // (broadcast LDS reads), and the 8 partial counts meet in LDS.  (A
        // bitonic network in one wave, 28 dependent rounds of lane
        // exchanges, took 1.6x as long.)
        constexpr int NC = 2 * kWave, JP = NC * NC / kEcThreads;
        static_assert(kEcThreads / NC * JP == NC, "the threads cover every pair");
        __shared__ int rnk[NC];
        __shared__ uint64_t srt[NC];
        if (tid < NC) rnk[tid] = 0;
        __syncthreads();
        const int i = tid % NC, j0 = (tid / NC) * JP;
        if (i < C) {
            const uint64_t ki = cand[i];
            int c = 0;
#pragma unroll
            for (int j = j0; j < j0 + JP; ++j) c += j < C && cand[j] > ki;
            atomicAdd(&rnk[i], c);
        }
        __syncthreads();
        if (tid < C) srt[rnk[tid]] = cand[tid];
        __syncthreads();
        if (tid < C) cand[tid] = srt[tid];
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
    if (perm.slot_row == nullptr) return;
    // The permutation of expert choice: expert e owns rows e*C .. e*C + C - 1
    // in rank order; column e of slot_row is -1 except at its C tokens.
    // The -1 fill (unless the router wrote it, row by row) completes (each
    // thread's stores, then the barrier) before the rows are written over it.
    if (!perm.prefilled) {
        for (int t = tid; t < T; t += kEcThreads) perm.slot_row[(int64_t)t * E + e] = -1;
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
    }
    for (int j = tid; j < C; j += kEcThreads) {
        const int t = (int)rank_key_index(cand[j]);
        perm.row_token[(int64_t)e * C + j] = t;
        perm.slot_row[(int64_t)t * E + e] = e * C + j;
    }
    if (tid == 0) {
        perm.counts[e] = C;
        perm.offsets[e] = e * C;
        if (e == 0) perm.offsets[E] = E * C;
    }
    if (e == 0 && perm.plan.mstart != nullptr) {
        // every expert has C rows: the plan needs no other block's results
        // counts [E], offsets [E+1] and the plan's 3(E+1) scratch ints in the
        // candidate buffer (free once every thread has read its rows)
        static_assert(kEcMaxCapacity * 2 >= 5 * kMaxPlanExperts + 4, "plan scratch fits");
        int32_t *pc = reinterpret_cast<int32_t *>(cand);
        __syncthreads();
        for (int i = tid; i <= E; i += kEcThreads) {
            if (i < E) pc[i] = C;
            pc[E + i] = i * C;
        }
        __syncthreads();
        build_tile_plan(pc, pc + E, E, perm.plan.BM, perm.plan.mstart, perm.plan.mtile, perm.plan.max_mt,
                        perm.plan.cnt, perm.plan.ncnt, perm.plan.interleave, pc + 2 * E + 1);
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
// Whether the router tile's staging buffers also hold the transposed logits
// tile [EP][TOK] next to the logits tile [TOK][EPX] (the rows of both
// operand buffers, 64 bf16 each, two buffers).
constexpr bool router_tile_transposes(int TOK, int EP, int EPX) {
    return 2 * (TOK + EPX) * 64 * 2 >= (TOK * EPX + EP * TOK) * 4;
}
template <int TOK, int EP, bool NOISY, int PD = 4, int NTH = 256>
__global__ __launch_bounds__(NTH) void router_tile_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ wg, const float *__restrict__ bias, int T, int d, int E,
    int k, int gating, float *__restrict__ logits, int32_t *__restrict__ idx_out, float *__restrict__ w_out,
    const bf16 *__restrict__ wn, const float *__restrict__ noise, float *__restrict__ logits_t,
    int32_t *__restrict__ fill_rows) {
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
    // expert choice: the transposed tile [EP][TOK] after it, when it fits
    // (entry tt of expert e at slot tt ^ (e % TOK), so that both the
    // per-expert writes and the per-token reads spread over the banks)
    float *LfT = Lf + TOK * EPX;
    static_assert(!router_tile_transposes(TOK, EP, EPX) || 2 * ROWS * BK * 2 >= (TOK * EPX + EP * TOK) * 4,
                  "transposed tile");
    if (!router_tile_transposes(TOK, EP, EPX)) logits_t = nullptr;
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
            if (logits_t) LfT[e * TOK + (tt ^ (e % TOK))] = v;
        }
        if (gating != kGateExpertChoice) gate_one_token(row, E, k, gating, t, idx_out, w_out);
    }
    if (logits_t) {
        // expert choice: the transposed logits, TOK consecutive tokens of
        // each expert, and the -1 fill of these tokens' rows of the row map
        __syncthreads();
        for (int i = tid; i < TOK * E; i += NTH) {
            const int e = i / TOK, tt = i % TOK;
            if (tok0 + tt < T) logits_t[(int64_t)e * T + tok0 + tt] = LfT[e * TOK + (tt ^ (e % TOK))];
        }
        for (int i = tid; i < TOK * E; i += NTH)
            if (tok0 + i / E < T) fill_rows[tok0 * E + i] = -1;
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int TOK, int EP>
static bool launch_router_tile_t(const RouteArgs &a, hipStream_t s) {
    const int grid = (a.T + TOK - 1) / TOK;
    // register sets in flight: four, or two when a set is large (noisy, 256 experts)
    constexpr int PDN = (TOK + 2 * EP) / 32 <= 10 ? 4 : 2;
    if (a.wn)
        hipLaunchKernelGGL((router_tile_kernel<TOK, EP, true, PDN>), dim3(grid), dim3(256), 0, s, (const bf16 *)a.x,
                           (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           (const bf16 *)a.wn, a.noise, a.logits_t, a.fill_rows);
    else if constexpr (EP >= 128)  // 8 waves: 2 per SIMD (DeepSeek-style router 124 -> 109 us)
        hipLaunchKernelGGL((router_tile_kernel<TOK, EP, false, 4, 512>), dim3(grid), dim3(512), 0, s,
                           (const bf16 *)a.x, (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits,
                           a.idx, a.w, nullptr, nullptr, a.logits_t, a.fill_rows);
    else
        hipLaunchKernelGGL((router_tile_kernel<TOK, EP, false>), dim3(grid), dim3(256), 0, s, (const bf16 *)a.x,
                           (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           nullptr, nullptr, a.logits_t, a.fill_rows);
    return a.logits_t != nullptr && router_tile_transposes(TOK, EP, a.wn ? 2 * EP : EP);
}

template <int TOK>
static bool launch_router_tile(const RouteArgs &a, hipStream_t s) {
    if (a.E <= 64) return launch_router_tile_t<TOK, 64>(a, s);
    if (a.E <= 128) return launch_router_tile_t<TOK, 128>(a, s);
    return launch_router_tile_t<TOK, 256>(a, s);
}

template <int NT, int WK>
static void launch_route_bf16_wk(const RouteArgs &a, const RoutePermuteArgs *perm, hipStream_t s) {
    const int grid = (a.T + 15) / 16;
    // paired K segments: up to 8 experts, token choice, no noise projection
    const bool pair = NT == 1 && a.E <= 8 && a.d % 64 == 0 && a.gating != kGateExpertChoice && !a.wn;
    if (perm) {  // one block (route_permute_fits): route, then permute in the same block
        const size_t lds = (size_t)small_tables_bytes(a.T, a.E);
        auto kern = pair ? route_bf16_kernel<NT, WK, false, true, NT == 1> : route_bf16_kernel<NT, WK, false, true>;
        hipLaunchKernelGGL(kern, dim3(1), dim3(64 * WK), lds, s, (const bf16 *)a.x, (const bf16 *)a.wg, a.bias, a.T,
                           a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w, nullptr, nullptr, *perm, nullptr, nullptr);
    } else if (pair) {
        hipLaunchKernelGGL((route_bf16_kernel<NT, WK, false, false, NT == 1>), dim3(grid), dim3(64 * WK), 0, s,
                           (const bf16 *)a.x, (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits,
                           a.idx, a.w, nullptr, nullptr, RoutePermuteArgs{}, nullptr, nullptr);
    } else if (a.wn) {
        hipLaunchKernelGGL((route_bf16_kernel<NT, WK, true>), dim3(grid), dim3(64 * WK), 0, s, (const bf16 *)a.x,
                           (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           (const bf16 *)a.wn, a.noise, RoutePermuteArgs{}, a.logits_t, a.fill_rows);
    } else {
        hipLaunchKernelGGL((route_bf16_kernel<NT, WK, false>), dim3(grid), dim3(64 * WK), 0, s, (const bf16 *)a.x,
                           (const bf16 *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           nullptr, nullptr, RoutePermuteArgs{}, a.logits_t, a.fill_rows);
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

bool launch_route(const RouteArgs &a, hipStream_t s) {
    if (a.T == 0) return false;
    if (!a.bf16) {
        hipLaunchKernelGGL(route_f32_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, (const float *)a.x,
                           (const float *)a.wg, a.bias, a.T, a.d, a.E, a.k, a.gating, a.logits, a.idx, a.w,
                           (const float *)a.wn, a.noise);
        return false;
    }
    // Up to 16 experts: per-wave K slices straight from global memory.  More
    // experts: LDS-staged tiles, so that a block's tokens share each weight
    // row instead of every 16-token wave re-reading all of them from L2.
    if (a.E <= 16) {
        launch_route_bf16_t<1>(a, s);
        return a.logits_t != nullptr;
    }
    // 32-token blocks unless that already gives a block per CU twice over
    if (a.T >= 64 * 512) return launch_router_tile<64>(a, s);
    return launch_router_tile<32>(a, s);
}

void launch_gate_logits(const float *logits, int T, int E, int k, int gating, int32_t *idx, float *w,
                        hipStream_t s) {
    if (T == 0) return;
    if (E <= kLaneGateMax)
        hipLaunchKernelGGL(gate_logits_lane_kernel, dim3((T + 255) / 256), dim3(256), 0, s, logits, T, E, k, gating,
                           idx, w);
    else
        hipLaunchKernelGGL(gate_logits_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, gating, idx, w);
}

void launch_ec_select(const float *logits, int T, int E, int C, int32_t *ec_idx, float *ec_score,
                      hipStream_t s, const EcPermuteArgs *perm, const float *logits_t) {
    const EcPermuteArgs pa = perm ? *perm : EcPermuteArgs{};
    if (T <= kEcColMax)
        hipLaunchKernelGGL(ec_select_kernel<true>, dim3(E), dim3(kEcThreads), 0, s, logits, logits_t, T, E, C, ec_idx,
                           ec_score, pa);
    else
        hipLaunchKernelGGL(ec_select_kernel<false>, dim3(E), dim3(kEcThreads), 0, s, logits, logits_t, T, E, C,
                           ec_idx, ec_score, pa);
}

}  // namespace moe
