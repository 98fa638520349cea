// Shared device helpers for the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Element types the kernels are instantiated for.
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static inline float load(const float *p) { return *p; }
    __device__ static inline void store(float *p, float v) { *p = v; }
};
template <> struct Elem<bf16> {
    __device__ static inline float load(const bf16 *p) { return (float)(*p); }
    // float -> bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950)
    __device__ static inline void store(bf16 *p, float v) { *p = (bf16)v; }
};

__device__ inline u32x4 load16(const void *p) { return *(const u32x4 *)p; }
__device__ inline void store16(void *p, u32x4 v) { *(u32x4 *)p = v; }

// Order-preserving unsigned image of a float32: a > b  <=>  key(a) > key(b),
// with -0.0 mapped to the image of +0.0 so that the two tie.
__device__ inline uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_value(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}
// Unique rank key: larger value first, then lower index first.
__device__ inline uint64_t rank_key(float v, uint32_t idx) {
    return ((uint64_t)order_key(v) << 32) | (uint64_t)(~idx);
}
__device__ inline uint32_t rank_key_index(uint64_t key) { return ~(uint32_t)(key & 0xffffffffu); }

__device__ inline uint64_t shfl_xor_u64(uint64_t v, int mask) {
    uint32_t lo = __shfl_xor((uint32_t)v, mask, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), mask, kWave);
    return ((uint64_t)hi << 32) | lo;
}
__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}
// Butterfly sum: every lane ends with the same value, in a fixed order.
// Inclusive prefix sum over the 64 lanes of a wave, in lane order, on DPP
// lane moves: shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then the
// total of rows 0 and 2 to rows 1 and 3 (row_bcast:15) and the total of
// lanes 0..31 to rows 2 and 3 (row_bcast:31).  Lanes a move does not write
// add 0.  All 64 lanes must be active.  (Lane exchanges through LDS take
// one dependent round trip per step: the expert-choice bucket search took
// 1.4x as long with them.)
__device__ inline int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }
// silu on the hardware transcendentals: e^-z = 2^(-z log2 e) (v_exp_f32) and
// one reciprocal (v_rcp_f32), each about 1 ulp; for outputs rounded to bf16
// (2^-9 relative) this matches the full-precision form.  Large negative z
// gives 2^+inf = inf, rcp(inf) = 0, so the result tends to -0 as silu does.
__device__ inline float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}
__device__ inline float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

__device__ inline float apply_act(int act, float z) {
    if (act == kActRelu) return z > 0.f ? z : 0.f;
    if (act == kActGelu) return gelu_erf(z);
    return z;
}


// Raw buffer resource over `bytes` bytes from `base` (limit clamped to 2^31 - 1;
// callers address at most a 256-row tile from the base).  Loads at offsets
// at or past the limit return zeros.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int64_t bytes) {
    const int64_t lim = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)lim, 0x00020000);
}
__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0));
}

// LDS tiles hold rows of 64 bf16 (128 bytes = eight 16-byte chunks).  Chunk c
// of row r is stored at chunk slot c ^ swz(r) so that the 16-byte reads of 16
// consecutive rows at one chunk index touch distinct banks.
__device__ inline int swz(int r) { return (r >> 1) & 7; }
// Rows of BK bf16: 64 as above; 128 (sixteen chunks): slot c ^ (r % 16), so
// that 16 consecutive rows at one chunk index touch distinct bank groups
// whatever the bank count.  Both depend on r % 16 only.
template <int BK>
__device__ inline int swz_k(int r) { return BK == 64 ? swz(r) : (r & 15); }

}  // namespace moe
