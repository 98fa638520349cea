// One-workgroup permutation of up to kSmallMaxSlots token-expert
// assignments, shared by the permutation kernel and the router of a batch
// that fits one router block (the router then permutes its own gating).
#pragma once

#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

// Run by all NTH threads of one workgroup.  idx [T][k] may have been written
// by this workgroup before a barrier.  lds_u64: small_tables_bytes(T, E)
// bytes of LDS: three tables of nc = ceil(T / kChunk) token-chunk rows of
// ES = E + 1 entries (the padding entry keeps one expert's column off a
// single LDS bank).  Writes counts [E], offsets [E + 1],
// row_token and slot_row [T][k] (-1: dropped) and, when plan.mstart is set,
// the grouped GEMMs' tile plan.  The layout and its order are those of the
// count / scan / scatter kernels: each expert's rows in ascending token
// order, the first `capacity` of each capacity group kept.
template <int NTH>
__device__ void permute_small_block(const int32_t *__restrict__ idx, int T, int E, int k, int capacity,
                                    int group_chunks, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                    int32_t *__restrict__ row_token, int32_t *__restrict__ slot_row,
                                    const TilePlanArgs &plan, unsigned long long *lds_u64) {
    const int nc = (T + kChunk - 1) / kChunk, ES = E + 1;
    unsigned long long *masks = lds_u64;                    // [nc][ES]
    int32_t *pre = (int32_t *)(masks + (int64_t)nc * ES);  // [nc][ES] in-group prefix before the chunk
    int32_t *base = pre + (int64_t)nc * ES;                  // [nc][ES] kept rows of e before the chunk
    __shared__ int wsum[NTH / kWave];
    __shared__ int offs[kMaxSmallExperts + 1];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    for (int i = tid; i < nc * ES; i += NTH) masks[i] = 0ull;
    __syncthreads();
    // chunk masks: bit l of masks[c][e] = token 64c + l chose e.  Thread
    // tid takes slots tid + u * NTH, kLoads idx loads in flight before the
    // first atomic; its first kLoads slots stay in registers for the
    // scatter below, which then loads nothing again when the batch has at
    // most kLoads * NTH slots.
    constexpr int NW = NTH / kWave, kLoads = 8;
    const int n = T * k;  // <= kSmallMaxSlots
    int first_ev[kLoads];
    for (int i0 = tid; i0 < n; i0 += kLoads * NTH) {
        int ev[kLoads];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int i = i0 + u * NTH;
            ev[u] = i < n ? idx[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int i = i0 + u * NTH, e = ev[u];
            if (e >= 0 && e < E) {
                const int t = i / k;
                atomicOr(&masks[(t / kChunk) * ES + e], 1ull << (t % kChunk));
            }
            if (i0 == tid) first_ev[u] = e;
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
            const int incl = wave_incl_scan(c < nc ? __popcll(masks[c * ES + e]) : 0);
            if (c < nc) base[c * ES + e] = carry + incl;
            carry += __builtin_amdgcn_readlane(incl, kWave - 1);
        }
        for (int c0 = 0; c0 < nc; c0 += kWave) {
            const int c = c0 + lane;
            if (c < nc) {
                const int head = group_chunks > 0 ? c - c % group_chunks : 0;
                pre[c * ES + e] =
                    base[c * ES + e] - __popcll(masks[c * ES + e]) - (head > 0 ? base[(head - 1) * ES + e] : 0);
            }
        }
        carry = 0;
        for (int c0 = 0; c0 < nc; c0 += kWave) {
            const int c = c0 + lane;
            int kept = 0;
            if (c < nc) {
                const int cnt = __popcll(masks[c * ES + e]);
                kept = cnt;
                if (capacity > 0) {
                    const int room = capacity - pre[c * ES + e];
                    kept = room <= 0 ? 0 : (room < cnt ? room : cnt);
                }
            }
            const int incl = wave_incl_scan(kept);
            if (c < nc) base[c * ES + e] = carry + incl - kept;
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
    // the waves' totals, one per lane, scanned the same way
    const int ws = wave_incl_scan(lane < NW ? wsum[lane] : 0);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int before = wv > 0 ? __builtin_amdgcn_readlane(ws, wv - 1) : 0;
    const int total = __builtin_amdgcn_readlane(ws, NW - 1);
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
    // (the same slots per thread as above: the first kLoads from registers)
    for (int i0 = tid; i0 < n; i0 += kLoads * NTH) {
        int ev[kLoads];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int i = i0 + u * NTH;
            ev[u] = i0 == tid ? first_ev[u] : (i < n ? idx[i] : -1);
        }
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int i = i0 + u * NTH, e = ev[u];
            if (i >= n) break;
            int row = -1;
            if (e >= 0 && e < E) {
                const int t = i / k;
                const int ce = (t / kChunk) * ES + e;
                const int r = __popcll(masks[ce] & ((1ull << (t % kChunk)) - 1ull));
                if (capacity <= 0 || pre[ce] + r < capacity) {
                    row = offs[e] + base[ce] + r;
                    row_token[row] = t;
                }
            }
            slot_row[i] = row;
        }
    }
    if (plan.mstart != nullptr) {
        __shared__ int plan_scratch[3 * (kMaxSmallExperts + 1)];
        build_tile_plan(ktot, offs, E, plan.BM, plan.mstart, plan.mtile, plan.max_mt, plan.cnt, plan.ncnt,
                        plan.interleave, plan_scratch);
    }
}

}  // namespace moe
