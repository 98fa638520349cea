// Counts, capacity and the stable expert-contiguous permutation, and the
// coalesced gather of token rows, for gfx950.
//
// Token t's assignment to expert e goes to row offsets[e] + (number of kept
// assignments to e by tokens before t): rows of one expert are in ascending
// token order, the order x[mask] gives in [yj-zh] youngju.dev "Mixture of
// Experts（MoE）架构深度解析" MoELayer.  With a capacity C, inside each
// capacity group only the first C tokens of every expert are kept
// ([yj-zh] SwitchRouter).  Everything is integer arithmetic with no order
// dependence, so results are bit-exact and deterministic:
//   count   : each wave owns 64 consecutive tokens; lanes OR their bit into a
//             per-expert 64-bit LDS mask; popcounts give per-chunk counts and
//             each assignment's rank inside the chunk;
//   scan    : per expert, a running sum over chunks (reset at group starts)
//             gives the in-group prefix and the kept-row base of each chunk,
//             then an exclusive scan over experts gives offsets;
//   scatter : row = offsets[e] + base[chunk][e] + rank, or -1 when
//             prefix + rank >= C.
#include "common.h"
#include "kernels.h"
#include "perm_small.h"
#include "plan.h"

namespace moe {

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t *__restrict__ idx, int T, int E, int k,
                                                            int32_t *__restrict__ chunk_counts,
                                                            int32_t *__restrict__ ranks) {
    extern __shared__ unsigned long long masks[];  // [4][E]
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    unsigned long long *my = masks + (int64_t)wave * E;
    for (int e = lane; e < E; e += kWave) my[e] = 0ull;
    __syncthreads();
    const int64_t c = (int64_t)blockIdx.x * 4 + wave;
    const int64_t t = c * kChunk + lane;
    const int64_t nc = ((int64_t)T + kChunk - 1) / kChunk;
    const bool live = t < T;
    const unsigned long long bit = 1ull << lane;
    if (live)
        for (int j = 0; j < k; ++j) {
            const int e = idx[t * k + j];
            if (e >= 0 && e < E) atomicOr(&my[e], bit);
        }
    __syncthreads();
    if (live)
        for (int j = 0; j < k; ++j) {
            const int e = idx[t * k + j];
            ranks[t * k + j] = (e >= 0 && e < E) ? __popcll(my[e] & (bit - 1ull)) : 0;
        }
    if (c < nc)
        for (int e = lane; e < E; e += kWave) chunk_counts[c * E + e] = __popcll(my[e]);
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(int nc, int E, int capacity, int group_chunks,
                                                                    const int32_t *__restrict__ chunk_counts,
                                                                    int32_t *__restrict__ chunk_pre,
                                                                    int32_t *__restrict__ chunk_base,
                                                                    int32_t *__restrict__ counts,
                                                                    int32_t *__restrict__ offsets,
                                                                    TilePlanArgs plan) {
    __shared__ int wsum[kScanThreads / kWave];
    __shared__ int lcnt[kScanThreads], loff[kScanThreads + 1];
    const int e = threadIdx.x;
    int kept_total = 0;
    if (e < E) {
        int run = 0;
        int c = 0;
        constexpr int U = 8;
        for (; c + U <= nc; c += U) {
            int cnt[U];
#pragma unroll
            for (int u = 0; u < U; ++u) cnt[u] = chunk_counts[(int64_t)(c + u) * E + e];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int cc = c + u;
                if (group_chunks > 0 && cc % group_chunks == 0) run = 0;
                chunk_pre[(int64_t)cc * E + e] = run;
                int kept = cnt[u];
                if (capacity > 0) {
                    const int room = capacity - run;
                    kept = room <= 0 ? 0 : (room < cnt[u] ? room : cnt[u]);
                }
                chunk_base[(int64_t)cc * E + e] = kept_total;
                kept_total += kept;
                run += cnt[u];
            }
        }
        for (; c < nc; ++c) {
            const int cnt = chunk_counts[(int64_t)c * E + e];
            if (group_chunks > 0 && c % group_chunks == 0) run = 0;
            chunk_pre[(int64_t)c * E + e] = run;
            int kept = cnt;
            if (capacity > 0) {
                const int room = capacity - run;
                kept = room <= 0 ? 0 : (room < cnt ? room : cnt);
            }
            chunk_base[(int64_t)c * E + e] = kept_total;
            kept_total += kept;
            run += cnt;
        }
        counts[e] = kept_total;
    }
    // exclusive scan of counts over experts (thread order == expert order)
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int incl = wave_incl_scan(kept_total);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < kScanThreads / kWave; ++w) {
        if (w < wave) base += wsum[w];
        total += wsum[w];
    }
    if (e < E) {
        offsets[e] = base + incl - kept_total;
        lcnt[e] = kept_total;
        loff[e] = base + incl - kept_total;
    }
    if (e == 0) {
        offsets[E] = total;
        loff[E] = total;
    }
    // the grouped GEMMs' tile plan from the counts and offsets in LDS (one
    // launch fewer than the separate plan kernel: DeepSeek-style layer)
    if (plan.mstart != nullptr) {
        __shared__ int plan_scratch[3 * (kMaxPlanExperts + 1)];
        __syncthreads();
        build_tile_plan(lcnt, loff, E, plan.BM, plan.mstart, plan.mtile, plan.max_mt, plan.cnt, plan.ncnt,
                        plan.interleave, plan_scratch);
    }
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(const int32_t *__restrict__ idx, int T, int E, int k,
                                                              int capacity, const int32_t *__restrict__ ranks,
                                                              const int32_t *__restrict__ chunk_pre,
                                                              const int32_t *__restrict__ chunk_base,
                                                              const int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ row_token,
                                                              int32_t *__restrict__ slot_row) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * k) return;
    const int64_t t = i / k;
    const int e = idx[i];
    if (e < 0 || e >= E) {
        slot_row[i] = -1;
        return;
    }
    const int64_t ce = (t / kChunk) * E + e;
    const int r = ranks[i];
    if (capacity > 0 && chunk_pre[ce] + r >= capacity) {
        slot_row[i] = -1;
        return;
    }
    const int row = offsets[e] + chunk_base[ce] + r;
    slot_row[i] = row;
    row_token[row] = (int32_t)t;
}

// ---------------------------------------------------------------------------
// Small batches: the three phases above in one workgroup, with the per-chunk
// masks, prefixes and bases in LDS (nc * E * 16 bytes), so a decode-sized or
// mid-sized batch pays one launch instead of three (four with the grouped
// GEMMs' tile plan, which the forward pass builds here too).  Same formulas,
// so the same counts, offsets, rows and drops.
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 1024;

__global__ __launch_bounds__(kSmallThreads) void permute_small_kernel(const int32_t *__restrict__ idx, int T, int E,
                                                                      int k, int capacity, int group_chunks,
                                                                      int32_t *__restrict__ counts,
                                                                      int32_t *__restrict__ offsets,
                                                                      int32_t *__restrict__ row_token,
                                                                      int32_t *__restrict__ slot_row,
                                                                      TilePlanArgs plan) {
    extern __shared__ unsigned long long lds_u64[];
    permute_small_block<kSmallThreads>(idx, T, E, k, capacity, group_chunks, counts, offsets, row_token, slot_row,
                                       plan, lds_u64);
}

bool permute_small_fits(int T, int E, int k) {
    return E <= kMaxSmallExperts && small_tables_bytes(T, E) <= kSmallLdsBytes && (int64_t)T * k <= kSmallMaxSlots;
}

void launch_permute_small(const PermuteArgs &a, const TilePlanArgs &plan, hipStream_t s) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kSmallThreads), (size_t)small_tables_bytes(a.T, a.E), s,
                       a.idx, a.T, a.E, a.k, a.capacity, a.group_chunks, a.counts, a.offsets, a.row_token, a.slot_row,
                       plan);
}

void launch_permute_count(const PermuteArgs &a, hipStream_t s) {
    const int64_t nc = ((int64_t)a.T + kChunk - 1) / kChunk;
    const size_t shmem = (size_t)4 * a.E * sizeof(unsigned long long);
    hipLaunchKernelGGL(permute_count_kernel, dim3((unsigned)((nc + 3) / 4)), dim3(256), shmem, s, a.idx, a.T, a.E,
                       a.k, a.chunk_counts, a.ranks);
}

void launch_permute_scan(const PermuteArgs &a, const TilePlanArgs &plan, hipStream_t s) {
    const int nc = (a.T + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, nc, a.E, a.capacity, a.group_chunks,
                       a.chunk_counts, a.chunk_pre, a.chunk_base, a.counts, a.offsets, plan);
}

void launch_permute_scatter(const PermuteArgs &a, hipStream_t s) {
    const int64_t n = (int64_t)a.T * a.k;
    if (n == 0) return;
    hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.idx, a.T, a.E,
                       a.k, a.capacity, a.ranks, a.chunk_pre, a.chunk_base, a.offsets, a.row_token, a.slot_row);
}

// ---------------------------------------------------------------------------
// Expert choice: expert e owns rows e*C .. e*C+C-1 in its selection order;
// slot_row is the dense token x expert map of rows (-1 = not chosen), the
// inverse of the dispatch matrix of [yj-ja] youngju.dev "Sparse Mixture of
// Experts（MoE）アーキテクチャ深層分析" ExpertChoiceGating.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void ec_fill_kernel(int T, int E, int C, int32_t *__restrict__ counts,
                                                      int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ slot_row) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < (int64_t)T * E) slot_row[i] = -1;
    if (i < E) counts[i] = C;
    if (i <= E) offsets[i] = (int32_t)(i * C);
}

__global__ __launch_bounds__(256) void ec_scatter_kernel(const int32_t *__restrict__ ec_idx, int T, int E, int C,
                                                         int32_t *__restrict__ row_token,
                                                         int32_t *__restrict__ slot_row) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)E * C) return;
    const int e = (int)(i / C);
    const int t = ec_idx[i];
    row_token[i] = t;
    if (t >= 0 && t < T) slot_row[(int64_t)t * E + e] = (int32_t)i;
}

void launch_ec_permute(const int32_t *ec_idx, int T, int E, int C, int32_t *counts, int32_t *offsets,
                       int32_t *row_token, int32_t *slot_row, hipStream_t s) {
    int64_t n = (int64_t)T * E;
    if (n < E + 1) n = E + 1;
    hipLaunchKernelGGL(ec_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, E, C, counts, offsets,
                       slot_row);
    const int64_t m = (int64_t)E * C;
    hipLaunchKernelGGL(ec_scatter_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, s, ec_idx, T, E, C,
                       row_token, slot_row);
}

// ---------------------------------------------------------------------------
// Gather: x_perm[r] = x[row_token[r]] for r < offsets[E]; one wave per row,
// 16-byte loads and stores, four in flight per lane.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_rows_kernel(const char *__restrict__ x,
                                                          const int32_t *__restrict__ row_token,
                                                          const int32_t *__restrict__ offsets, int E,
                                                          int64_t row_bytes, char *__restrict__ out) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= offsets[E]) return;
    const char *src = x + (int64_t)row_token[r] * row_bytes;
    char *dst = out + r * row_bytes;
    constexpr int64_t step = kWave * 16;
    int64_t o = (int64_t)lane * 16;
    for (; o + 3 * step < row_bytes; o += 4 * step) {
        const u32x4 v0 = load16(src + o), v1 = load16(src + o + step);
        const u32x4 v2 = load16(src + o + 2 * step), v3 = load16(src + o + 3 * step);
        store16(dst + o, v0);
        store16(dst + o + step, v1);
        store16(dst + o + 2 * step, v2);
        store16(dst + o + 3 * step, v3);
    }
    for (; o < row_bytes; o += step) store16(dst + o, load16(src + o));
}

void launch_gather_rows(const void *x, const int32_t *row_token, const int32_t *offsets, int E, int64_t rows_max,
                        int d, int elem_bytes, void *x_perm, hipStream_t s) {
    if (rows_max == 0) return;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((rows_max + 3) / 4)), dim3(256), 0, s, (const char *)x,
                       row_token, offsets, E, (int64_t)d * elem_bytes, (char *)x_perm);
}

}  // namespace moe
