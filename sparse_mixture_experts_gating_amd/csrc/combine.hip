// Gate-weighted combine on gfx950: y[t] = sum over slots of w * y_perm[row]
// (+ shared expert output), the mixture y = sum_i G(x)_i E_i(x) of [yj-ja]
// youngju.dev "Sparse Mixture of Experts（MoE）アーキテクチャ深層分析" (gating
// formula), gathered per token instead of scattered with atomics, so the sum
// runs in a fixed order (slot order; expert order for expert choice) and is
// deterministic.  One wave per token (or per column range of a token),
// eight elements per lane per step.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

template <typename T>
__device__ inline void load8(const T *p, float *v);
template <>
__device__ inline void load8<bf16>(const bf16 *p, float *v) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, load16(p));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)b[i];
}
template <>
__device__ inline void load8<float>(const float *p, float *v) {
    const u32x4 a = load16(p), b = load16(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = __uint_as_float(a[i]);
        v[4 + i] = __uint_as_float(b[i]);
    }
}
template <typename T>
__device__ inline void store8(T *p, const float *v);
template <>
__device__ inline void store8<bf16>(bf16 *p, const float *v) {
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (bf16)v[i];
    store16(p, __builtin_bit_cast(u32x4, b));
}
template <>
__device__ inline void store8<float>(float *p, const float *v) {
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = __float_as_uint(v[i]);
        b[i] = __float_as_uint(v[4 + i]);
    }
    store16(p, a);
    store16(p + 4, b);
}

// A wave owns one token's columns, or one of `parts` equal ranges of them
// (few tokens: more waves in flight, shorter dependent load chains).  It
// first compacts the token's kept slots (row >= 0) into LDS, in slot order,
// with their gates; then, for each 8-element column chunk, it issues the
// loads of up to kBatch kept rows at once and adds them in slot order, so
// several loads are in flight per lane.
constexpr int kBatch = 8;
template <typename T, bool EC>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ y_perm, const T *__restrict__ y_shared,
                                                      const float *__restrict__ w,
                                                      const int32_t *__restrict__ slot_row, int Tn, int d, int S,
                                                      int parts, T *__restrict__ y) {
    // per-wave tables of the kept rows and gates, S entries each (dynamic
    // LDS sized to S, so that few slots leave room for more waves per CU)
    extern __shared__ int32_t comb_lds[];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    int32_t *krow = comb_lds + wave * S;
    float *kw = reinterpret_cast<float *>(comb_lds + 4 * S) + wave * S;
    const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
    const int64_t t = gw / parts;
    if (t >= Tn) return;
    // columns [c_lo, c_hi) of this wave: whole 8-element chunks
    const int cpp = (d / 8 + parts - 1) / parts * 8;
    const int c_lo = (int)(gw % parts) * cpp, c_hi = min(d, c_lo + cpp);
    const int32_t *sr = slot_row + t * S;
    int nv = 0;
    for (int s0 = 0; s0 < S; s0 += kWave) {
        const int s = s0 + lane;
        const int row = s < S ? sr[s] : -1;
        const bool keep = row >= 0;
        const uint64_t m = __ballot(keep);
        if (keep) {
            const int pos = nv + __popcll(m & ((1ull << lane) - 1ull));
            krow[pos] = row;
            // expert choice: the score sits at the row (w[row]); it is
            // loaded next to the row's outputs below, so that its latency
            // does not precede theirs
            if constexpr (!EC) kw[pos] = w[t * S + s];
        }
        nv += __popcll(m);
    }
    // lanes read entries other lanes wrote: one wave's LDS operations execute
    // in order, so only the compiler must not move the reads above the writes
    __builtin_amdgcn_wave_barrier();
    for (int c0 = c_lo + lane * 8; c0 < c_hi; c0 += kWave * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < nv; j0 += kBatch) {
            float v[kBatch][8];
            float gs[EC ? kBatch : 1];
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (j0 + b < nv) {
                    const int64_t row = krow[j0 + b];
                    load8<T>(y_perm + row * d + c0, v[b]);
                    if constexpr (EC) gs[b] = w[row];
                }
#pragma unroll
            for (int b = 0; b < kBatch; ++b)
                if (j0 + b < nv) {
                    float g;
                    if constexpr (EC) g = gs[b];
                    else g = kw[j0 + b];
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[b][i], acc[i]);
                }
        }
        if (y_shared) {
            float v[8];
            load8<T>(y_shared + t * d + c0, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += v[i];
        }
        store8<T>(y + t * d + c0, acc);
    }
}

void launch_combine(const CombineArgs &a, hipStream_t s) {
    if (a.T == 0) return;
    // Column ranges per token: enough waves for about four per CU, each range
    // at least one pass of the wave (512 columns).  Mixtral-shape decode (16
    // tokens): 8 ranges.
    // Expert choice (about one kept row per token among E slots): two ranges
    // per token, so that twice the waves share each token's short chain of
    // map, row and score loads (expert-choice layer 20.5 -> 19.5 us; two
    // ranges for the token-choice layers of 4096 and 8192 tokens measured
    // 1-8% slower).
    const int64_t want = a.expert_choice ? 2 : (4LL * device_cus() + a.T - 1) / a.T;
    const int parts = (int)std::max<int64_t>(1, std::min<int64_t>(want, a.d / (kWave * 8)));
    const dim3 grid((unsigned)((a.T * parts + 3) / 4));
    const size_t lds = (size_t)4 * a.S * (sizeof(int32_t) + sizeof(float));
    auto go = [&](auto ec) {
        constexpr bool EC = decltype(ec)::value;
        if (a.bf16)
            hipLaunchKernelGGL((combine_kernel<bf16, EC>), grid, dim3(256), lds, s, (const bf16 *)a.y_perm,
                               (const bf16 *)a.y_shared, a.w, a.slot_row, a.T, a.d, a.S, parts, (bf16 *)a.y);
        else
            hipLaunchKernelGGL((combine_kernel<float, EC>), grid, dim3(256), lds, s, (const float *)a.y_perm,
                               (const float *)a.y_shared, a.w, a.slot_row, a.T, a.d, a.S, parts, (float *)a.y);
    };
    if (a.expert_choice) go(std::true_type{});
    else go(std::false_type{});
}

}  // namespace moe
