// One-workgroup permutation of up to kSmallMaxSlots token-expert
// assignments, shared by the permutation kernel and the router of a batch
// that fits one router block (the router then permutes its own gating).
#pragma once

#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

// Run by all NTH threads of one workgroup.  idx [T][k] may have been written
// by this workgroup before a barrier.  lds_u64: 16 nc E bytes of LDS, nc =
// ceil(T / kChunk) token chunks.  Writes counts [E], offsets [E + 1],
// row_token and slot_row [T][k] (-1: dropped) and, when plan.mstart is set,
// the grouped GEMMs' tile plan.  The layout and its order are those of the
// count / scan / scatter kernels: each expert's rows in ascending token
// order, the first `capacity` of each capacity group kept.
template <int NTH>
__device__ void permute_small_block(const int32_t *__restrict__ idx, int T, int E, int k, int capacity,
                                    int group_chunks, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                    int32_t *__restrict__ row_token, int32_t *__restrict__ slot_row,
                                    const TilePlanArgs &plan, unsigned long long *lds_u64) {
    const int nc = (T + kChunk - 1) / kChunk;
    unsigned long long *masks = lds_u64;                   // [nc][E]
    int32_t *pre = (int32_t *)(masks + (int64_t)nc * E);  // [nc][E] in-group prefix before the chunk
    int32_t *base = pre + (int64_t)nc * E;                  // [nc][E] kept rows of e before the chunk
    __shared__ int wsum[NTH / kWave];
    __shared__ int offs[kMaxSmallExperts + 1];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    for (int i = tid; i < nc * E; i += NTH) masks[i] = 0ull;
    __syncthreads();
    // chunk masks: bit l of masks[c][e] = token 64c + l chose e
    for (int c = wave; c < nc; c += NTH / kWave) {
        const int t = c * kChunk + lane;
        if (t < T)
            for (int j = 0; j < k; ++j) {
                const int e = idx[(int64_t)t * k + j];
                if (e >= 0 && e < E) atomicOr(&masks[c * E + e], 1ull << lane);
            }
    }
    __syncthreads();
    // per expert, one wave: wave-wide scans over windows of 64 chunks give
    //   P(c)   = assignments to e in chunks 0..c                (into base)
    //   pre(c) = P(c) - cnt(c) - P(first chunk of c's group - 1)  (into pre)
    //   base(c) = kept assignments to e in chunks before c      (into base)
    __shared__ int ktot[kMaxSmallExperts];
    for (int e = wave; e < E; e += NTH / kWave) {
        int carry = 0;
        for (int c0 = 0; c0 < nc; c0 += kWave) {
            const int c = c0 + lane;
            const int incl = wave_incl_scan(c < nc ? __popcll(masks[c * E + e]) : 0);
            if (c < nc) base[c * E + e] = carry + incl;
            carry += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        for (int c0 = 0; c0 < nc; c0 += kWave) {
            const int c = c0 + lane;
            if (c < nc) {
                const int head = group_chunks > 0 ? c - c % group_chunks : 0;
                pre[c * E + e] = base[c * E + e] - __popcll(masks[c * E + e]) - (head > 0 ? base[(head - 1) * E + e] : 0);
            }
        }
        carry = 0;
        for (int c0 = 0; c0 < nc; c0 += kWave) {
            const int c = c0 + lane;
            int kept = 0;
            if (c < nc) {
                const int cnt = __popcll(masks[c * E + e]);
                kept = cnt;
                if (capacity > 0) {
                    const int room = capacity - pre[c * E + e];
                    kept = room <= 0 ? 0 : (room < cnt ? room : cnt);
                }
            }
            const int incl = wave_incl_scan(kept);
            if (c < nc) base[c * E + e] = carry + incl - kept;
            carry += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        if (lane == 0) {
            ktot[e] = carry;
            counts[e] = carry;
        }
    }
    __syncthreads();
    const int kept_total = tid < E ? ktot[tid] : 0;
    // exclusive scan of the kept counts over experts (thread order)
    const int incl = wave_incl_scan(kept_total);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < NTH / kWave; ++w) {
        if (w < wave) before += wsum[w];
        total += wsum[w];
    }
    if (tid < E) {
        offs[tid] = before + incl - kept_total;
        offsets[tid] = before + incl - kept_total;
    }
    if (tid == 0) {
        offsets[E] = total;
        offs[E] = total;
    }
    __syncthreads();
    // rows: offsets[e] + base + rank inside the chunk, or -1 past the capacity
    const int64_t n = (int64_t)T * k;
    for (int64_t i = tid; i < n; i += NTH) {
        const int t = (int)(i / k);
        const int e = idx[i];
        if (e < 0 || e >= E) {
            slot_row[i] = -1;
            continue;
        }
        const int ce = (t / kChunk) * E + e;
        const int r = __popcll(masks[ce] & ((1ull << (t % kChunk)) - 1ull));
        if (capacity > 0 && pre[ce] + r >= capacity) {
            slot_row[i] = -1;
            continue;
        }
        const int row = offs[e] + base[ce] + r;
        slot_row[i] = row;
        row_token[row] = t;
    }
    if (plan.mstart != nullptr) {
        __shared__ int plan_scratch[3 * (kMaxSmallExperts + 1)];
        build_tile_plan(ktot, offs, E, plan.BM, plan.mstart, plan.mtile, plan.max_mt, plan.cnt, plan.ncnt,
                        plan.interleave, plan_scratch);
    }
}

}  // namespace moe
