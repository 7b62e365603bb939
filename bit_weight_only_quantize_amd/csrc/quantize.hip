// quantize_pack: fp32 weights -> group-wise codes + scales (+ biases).
//
// sym4_g128 follows the airllm article §4.2 (group_quantize with bits = 4):
// absmax/7 scale with a 1e-8 floor, round half to even, clamp to +-7, two
// codes per byte with the even element in the low nibble.
// aff4_g64 / aff8_g64 follow the TurboFieldfare article, section 量化和精度
// (affine, 64 weights per group, bf16 scale and bf16 bias); the min/max rule
// (scale = (max-min)/(2^b-1), bias = min, both rounded to bf16, codes computed
// against the rounded values) is this library's reading of that format.
//
// Every step is plain IEEE fp32 (correctly rounded division, no contraction), so
// the codes are bit-identical to any host implementation of the same steps.
#pragma clang fp contract(off)

#include "common.hpp"
#include "launch.hpp"

namespace w4 {

// One wavefront quantizes 128 consecutive weights of a row: one sym4 group, two
// aff4 groups (one per half wavefront) or two aff8 groups (each lane one weight
// of group lane/32... see below). Each lane owns two adjacent weights.
template <int S>
__global__ __launch_bounds__(256) void quantize_pack_kernel(const float* __restrict__ W, int64_t N,
                                                            int64_t K, uint8_t* __restrict__ codes,
                                                            void* __restrict__ scale,
                                                            uint16_t* __restrict__ bias) {
    using T = Traits<S>;
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // 128-weight unit
    const int64_t units_per_row = K / 128 + (K % 128 ? 1 : 0);
    if (unit >= N * units_per_row) return;
    const int64_t row = unit / units_per_row;
    const int64_t k0 = (unit % units_per_row) * 128;
    const int64_t k = k0 + 2 * lane;
    const bool valid = k < K;  // K % 64 == 0, so a half-unit is either all valid or all not
    float2 w = valid ? *reinterpret_cast<const float2*>(W + row * K + k) : make_float2(0.f, 0.f);

    if constexpr (S == SYM4_G128) {
        float a = wave_max(fmaxf(fabsf(w.x), fabsf(w.y)));
        float s = fmaxf(a / 7.0f, 1e-8f);
        float q0 = fminf(fmaxf(rintf(w.x / s), -7.f), 7.f);
        float q1 = fminf(fmaxf(rintf(w.y / s), -7.f), 7.f);
        uint32_t b = ((uint32_t)(int)q0 & 0xFu) | (((uint32_t)(int)q1 & 0xFu) << 4);
        codes[row * (K / 2) + k / 2] = (uint8_t)b;
        if (lane == 0) static_cast<float*>(scale)[row * (K / 128) + k0 / 128] = s;
    } else {
        // 64-weight groups: lanes 0..31 hold group 2u, lanes 32..63 group 2u+1.
        float mn = fminf(w.x, w.y), mx = fmaxf(w.x, w.y);
        for (int o = 16; o >= 1; o >>= 1) {
            mn = fminf(mn, __shfl_xor(mn, o, 64));
            mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        }
        const float levels = (float)((1 << T::BITS) - 1);
        float s32 = fmaxf((mx - mn) / levels, 1e-8f);
        uint32_t sb = f32_to_bf16_rne(s32), bb = f32_to_bf16_rne(mn);
        float sf = bf16_bits_to_f32(sb), bf = bf16_bits_to_f32(bb);
        float q0 = fminf(fmaxf(rintf((w.x - bf) / sf), 0.f), levels);
        float q1 = fminf(fmaxf(rintf((w.y - bf) / sf), 0.f), levels);
        if (valid) {
            if constexpr (T::BITS == 4) {
                codes[row * (K / 2) + k / 2] = (uint8_t)((uint32_t)q0 | ((uint32_t)q1 << 4));
            } else {
                uint16_t two = (uint16_t)((uint32_t)q0 | ((uint32_t)q1 << 8));
                *reinterpret_cast<uint16_t*>(codes + row * K + k) = two;
            }
            if ((lane & 31) == 0) {
                const int64_t g = row * (K / 64) + k / 64;
                static_cast<uint16_t*>(scale)[g] = (uint16_t)sb;
                bias[g] = (uint16_t)bb;
            }
        }
    }
}

hipError_t launch_quantize_pack(int scheme, const float* W, int64_t N, int64_t K, void* codes,
                                void* scale, void* bias, hipStream_t st) {
    const int64_t units = N * (K / 128 + (K % 128 ? 1 : 0));
    const int64_t blocks = (units + 3) / 4;
    if (blocks == 0) return hipSuccess;
    dim3 grid((unsigned)blocks), block(256);
    switch (scheme) {
        case SYM4_G128:
            hipLaunchKernelGGL(quantize_pack_kernel<SYM4_G128>, grid, block, 0, st, W, N, K,
                               (uint8_t*)codes, scale, (uint16_t*)bias);
            break;
        case AFF4_G64:
            hipLaunchKernelGGL(quantize_pack_kernel<AFF4_G64>, grid, block, 0, st, W, N, K,
                               (uint8_t*)codes, scale, (uint16_t*)bias);
            break;
        default:
            hipLaunchKernelGGL(quantize_pack_kernel<AFF8_G64>, grid, block, 0, st, W, N, K,
                               (uint8_t*)codes, scale, (uint16_t*)bias);
            break;
    }
    return hipGetLastError();
}

}  // namespace w4
