// Shared device helpers for the gfx950 kernels: scheme traits, bf16 handling,
// wavefront reductions. Everything here is written for 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

enum Scheme : int { SYM4_G128 = 0, AFF4_G64 = 1, AFF8_G64 = 2 };

// Per-scheme constants.
//   KV     weights covered by one 16-byte code vector
//   VPG    16-byte vectors per quantization group
//   BIAS   magic offset folded into the dot products (see unpack below):
//          sum_k (BIAS_ELEM + u_k) x_k = sum_k u_k x_k + BIAS * sum_k x_k
template <int S> struct Traits;
template <> struct Traits<SYM4_G128> {
    static constexpr int BITS = 4, GROUP = 128, KV = 32, VPG = 4;
    static constexpr float BIAS = 136.f;  // 128 (exponent trick) + 8 (signed -> offset nibble)
    static constexpr bool AFFINE = false;
};
template <> struct Traits<AFF4_G64> {
    static constexpr int BITS = 4, GROUP = 64, KV = 32, VPG = 2;
    static constexpr float BIAS = 128.f;
    static constexpr bool AFFINE = true;
};
template <> struct Traits<AFF8_G64> {
    static constexpr int BITS = 8, GROUP = 64, KV = 16, VPG = 4;
    static constexpr float BIAS = 2176.f;  // 128 (low nibble) + 16 * 128 (high nibble)
    static constexpr bool AFFINE = true;
};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN payloads unspecified).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// fp32 accumulate of a 2-wide bf16 dot product: acc + a.lo*b.lo + a.hi*b.hi.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Two 4-bit fields at bits [0,4) and [16,20) of `v` become the bf16 pair
// (128 + lo, 128 + hi): exponent 2^7 with the nibble in the low mantissa bits.
// One v_and_or_b32.
__device__ __forceinline__ uint32_t nib_pair_to_bf16(uint32_t v) {
    return (v & 0x000F000Fu) | 0x43004300u;
}

// Sum over groups of L consecutive lanes (L = 8, 16, 32 or 64); every lane of a
// group ends up with the group total. Fixed order -> deterministic.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(L == 8 || L == 16 || L == 32 || L == 64, "lanes per row");
    // xor 1, xor 2 (quad permutes), then half-row and row mirrors
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    if constexpr (L >= 16)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_min(float v) {
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float gelu_tanh(float g) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * g * (1.f + tanhf(c * (g + 0.044715f * g * g * g)));
}

}  // namespace w4
