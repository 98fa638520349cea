// Device-side tile plan of the grouped expert GEMMs, shared by the plan
// kernel and the one-workgroup permutation.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// Number of light experts placed before heavy m-tile h when nl light experts
// are spread over Mh heavy m-tiles: light j goes after q_j = floor((2j+1) Mh
// / (2 nl)) heavy m-tiles, and q_j <= h  <=>  2j+1 < 2 nl (h+1) / Mh.
// 32-bit arithmetic: the interleaved plan is used for ragged layers only
// (fewer than 1024 rows per expert on average, so Mh < 2^16 m-tiles), and nl
// <= 1024 keeps 2 nl (h+1) and (2j+1) Mh below 2^28.
__device__ inline int lights_before(uint32_t h, uint32_t Mh, uint32_t nl) {
    if (nl == 0) return 0;
    if (Mh == 0) return (int)nl;
    const uint32_t c = (2 * nl * (h + 1) + Mh - 1) / Mh;
    return (int)(c / 2 < nl ? c / 2 : nl);
}

// The tile plan of the grouped GEMMs, built by one workgroup (any size; wave
// 0 runs the scans) from the per-expert kept counts and row offsets, which
// may sit in global memory or in LDS.  scratch: 3 * (E + 1) ints of LDS.
// Writes mstart[0..E], the m-tile table mtile[0 .. min(total, max_mt)) and
// clears the split-K arrival counters cnt[0 .. ncnt).
__device__ inline void build_tile_plan(const int32_t *counts, const int32_t *offsets, int E, int BM,
                                       int32_t *__restrict__ mstart, int4 *__restrict__ mtile, int max_mt,
                                       int32_t *__restrict__ cnt, int ncnt, bool interleave, int *scratch) {
    int *ms = scratch;               // first m-tile of each expert (expert order)
    int *hs = scratch + (E + 1);     // heavy m-tiles before each expert
    int *ls = scratch + 2 * (E + 1); // light experts before each expert
    const int tid = threadIdx.x, lane = tid % kWave, nthreads = blockDim.x;
    for (int i = tid; i < ncnt; i += nthreads) cnt[i] = 0;
    if (tid < kWave) {
        int base = 0, hbase = 0, lbase = 0;
        for (int e0 = 0; e0 < E; e0 += kWave) {
            const int e = e0 + lane;
            const int c = e < E ? counts[e] : 0;
            const int v = (c + BM - 1) / BM;
            const int hv = c >= BM ? v : 0, lv = c > 0 && c < BM ? 1 : 0;
            const int incl = wave_incl_scan(v), hincl = wave_incl_scan(hv), lincl = wave_incl_scan(lv);
            if (e < E) {
                mstart[e] = base + incl - v;
                ms[e] = base + incl - v;
                hs[e] = hbase + hincl - hv;
                ls[e] = lbase + lincl - lv;
            }
            base += __builtin_amdgcn_readlane(incl, kWave - 1);
            hbase += __builtin_amdgcn_readlane(hincl, kWave - 1);
            lbase += __builtin_amdgcn_readlane(lincl, kWave - 1);
        }
        if (lane == 0) {
            mstart[E] = base;
            ms[E] = base;
            hs[E] = hbase;
            ls[E] = lbase;
        }
    }
    __syncthreads();
    if (!interleave) {
        for (int e = tid; e < E; e += nthreads) {
            const int first = ms[e], n = ms[e + 1] - first;
            const int4 info = make_int4(first, e, offsets[e], offsets[e + 1]);
            for (int m = 0; m < n && first + m < max_mt; ++m) mtile[first + m] = info;
        }
        return;
    }
    // Interleaved order: the light experts (fewer rows than one tile: their
    // tiles stream weights for a few rows) are spread evenly among the
    // m-tiles of the heavy experts (whose tiles are MFMA-bound), so that
    // every round of tiles mixes both kinds.  A heavy expert's m-tiles stay
    // in order; a light expert between two of them splits it into runs, and
    // each run is one table group (its own first m-tile and row range).
    const uint32_t Mh = hs[E], nl = ls[E];
    for (int e = tid; e < E; e += nthreads) {
        const int c = offsets[e + 1] - offsets[e];
        if (c <= 0) continue;
        if (c < BM) {
            const uint32_t j = ls[e];
            const uint32_t pos = (2 * j + 1) * Mh / (2 * nl) + j;
            if (pos < (uint32_t)max_mt) mtile[pos] = make_int4((int)pos, e, offsets[e], offsets[e + 1]);
            continue;
        }
        const int n = ms[e + 1] - ms[e];
        const int off0 = offsets[e], off1 = offsets[e + 1];
        // L is constant along a run, so x = h0 + L(h0) = h0 + L(h) for any h of it
        uint32_t L = lights_before(hs[e], Mh, nl);
        int m0 = 0;
        for (int m = 0; m < n; ++m) {
            const uint32_t h = hs[e] + m;
            const uint32_t Lnext = m + 1 < n ? lights_before(h + 1, Mh, nl) : L;
            if (m + 1 < n && Lnext == L) continue;
            // run m0 .. m: consecutive table positions from that of m-tile m0
            const int x = (int)(hs[e] + m0 + L);
            const int z = off0 + m0 * BM;
            const int w = min(off1, off0 + (m + 1) * BM);
            for (int q = m0; q <= m; ++q)
                if (x + q - m0 < max_mt) mtile[x + q - m0] = make_int4(x, e, z, w);
            m0 = m + 1;
            L = Lnext;
        }
    }
}

}  // namespace moe
