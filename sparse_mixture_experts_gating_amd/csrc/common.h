// Shared device helpers for the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// Wave reductions on DPP lane moves (all 64 lanes must be active): an
// inclusive scan inside each row of 16 lanes (row_shr by 1, 2, 4 and 8),
// then row 0's and row 2's results to rows 1 and 3 (row_bcast:15) and lanes
// 0..31's result to rows 2 and 3 (row_bcast:31), so lane 63 ends with the
// whole wave's; every lane then reads lane 63.  Lanes a move does not write
// see the identity (0, or -inf for the float maximum).  The order of the
// float sum is fixed.  (Through LDS lane exchanges, one dependent round
// trip per step, the gating of one token took several times as long.)
template <int CTRL, int ROWS, bool BOUND>
__device__ inline uint32_t dpp_u32(uint32_t v, uint32_t identity) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROWS, 0xf, BOUND);
}
template <int CTRL, int ROWS, bool BOUND>
__device__ inline float dpp_f32(float v, float identity) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL, ROWS, 0xf, BOUND));
}
__device__ inline uint64_t wave_max_u64(uint64_t v) {
    auto step = [](uint64_t x, uint64_t o) { return o > x ? o : x; };
    auto mv = [](uint64_t x, auto ctrl) {
        constexpr int C = decltype(ctrl)::value;
        constexpr int R = C == 0x142 ? 0xa : C == 0x143 ? 0xc : 0xf;
        constexpr bool B = C < 0x140;
        const uint32_t lo = dpp_u32<C, R, B>((uint32_t)x, 0u), hi = dpp_u32<C, R, B>((uint32_t)(x >> 32), 0u);
        return ((uint64_t)hi << 32) | lo;
    };
    v = step(v, mv(v, std::integral_constant<int, 0x111>{}));
    v = step(v, mv(v, std::integral_constant<int, 0x112>{}));
    v = step(v, mv(v, std::integral_constant<int, 0x114>{}));
    v = step(v, mv(v, std::integral_constant<int, 0x118>{}));
    v = step(v, mv(v, std::integral_constant<int, 0x142>{}));
    v = step(v, mv(v, std::integral_constant<int, 0x143>{}));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}
// Inclusive prefix sum over the 64 lanes of a wave, in lane order (the
// same DPP moves; lane 63 holds the total).
__device__ inline int wave_incl_scan(int x) {
    x += (int)dpp_u32<0x111, 0xf, true>((uint32_t)x, 0u);   // row_shr:1
    x += (int)dpp_u32<0x112, 0xf, true>((uint32_t)x, 0u);   // row_shr:2
    x += (int)dpp_u32<0x114, 0xf, true>((uint32_t)x, 0u);   // row_shr:4
    x += (int)dpp_u32<0x118, 0xf, true>((uint32_t)x, 0u);   // row_shr:8
    x += (int)dpp_u32<0x142, 0xa, false>((uint32_t)x, 0u);  // row_bcast:15
    x += (int)dpp_u32<0x143, 0xc, false>((uint32_t)x, 0u);  // row_bcast:31
    return x;
}
__device__ inline float wave_sum(float v) {
    v += dpp_f32<0x111, 0xf, true>(v, 0.f);
    v += dpp_f32<0x112, 0xf, true>(v, 0.f);
    v += dpp_f32<0x114, 0xf, true>(v, 0.f);
    v += dpp_f32<0x118, 0xf, true>(v, 0.f);
    v += dpp_f32<0x142, 0xa, false>(v, 0.f);
    v += dpp_f32<0x143, 0xc, false>(v, 0.f);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ inline float wave_max(float v) {
    v = fmaxf(v, dpp_f32<0x111, 0xf, false>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<0x112, 0xf, false>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<0x114, 0xf, false>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<0x118, 0xf, false>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<0x142, 0xa, false>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<0x143, 0xc, false>(v, -INFINITY));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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
