// Single-token decode GEMV (M = 1), single-shot: every lane issues all of its
// code loads at kernel start, so a launch keeps the whole matrix in flight and
// the latency of HBM is paid once.
//
// Per lane: R rows x NV 16-byte code vectors (vector j of a row is vector
// sl + LPR*j, so the LPR lanes of a row read consecutive 16-byte pieces).
// Activations come either from LDS (staged and pair-permuted once per
// workgroup, XL = 0) or straight from global memory (L1/L2-resident, permuted
// in registers, XL = 1). The arithmetic is the skinny core's: nibble pairs ->
// bf16 (128 + u) -> v_dot2_f32_bf16, offset removed per vector from the
// activation sum, DPP reduction across the LPR lanes of a row.
#pragma once

#include "common.hpp"
#include "skinny.hpp"

namespace w4 {

// Activation pairs and sum for code vector v of a 4-bit row, read from global
// memory: 32 bf16 -> 16 pair dwords (x[t], x[t+4]) per 8-element block.
template <int S>
__device__ __forceinline__ void load_x_pairs_global(const uint16_t* __restrict__ x, int v,
                                                    uint32_t (&xp)[Traits<S>::BITS == 4 ? 16 : 8],
                                                    float& xsum) {
    using T = Traits<S>;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (int64_t)v * T::KV);
    constexpr uint32_t ONES = 0x3F803F80u;  // bf16 pair (1, 1)
    float s = 0.f;
    if constexpr (T::BITS == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4_t d = src[j];
            xp[4 * j + 0] = (d[0] & 0xFFFFu) | (d[2] << 16);
            xp[4 * j + 1] = (d[0] >> 16) | (d[2] & 0xFFFF0000u);
            xp[4 * j + 2] = (d[1] & 0xFFFFu) | (d[3] << 16);
            xp[4 * j + 3] = (d[1] >> 16) | (d[3] & 0xFFFF0000u);
            s = dot2_bf16(ONES, d[0], s);
            s = dot2_bf16(ONES, d[1], s);
            s = dot2_bf16(ONES, d[2], s);
            s = dot2_bf16(ONES, d[3], s);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4_t d = src[j];
            xp[4 * j + 0] = (d[0] & 0xFFFFu) | (d[1] << 16);
            xp[4 * j + 1] = (d[0] >> 16) | (d[1] & 0xFFFF0000u);
            xp[4 * j + 2] = (d[2] & 0xFFFFu) | (d[3] << 16);
            xp[4 * j + 3] = (d[2] >> 16) | (d[3] & 0xFFFF0000u);
            s = dot2_bf16(ONES, d[0], s);
            s = dot2_bf16(ONES, d[1], s);
            s = dot2_bf16(ONES, d[2], s);
            s = dot2_bf16(ONES, d[3], s);
        }
    }
    xsum = s;
}

// D += dot(code vector c, activation pairs xp) with the (128 + u) encoding.
template <int S>
__device__ __forceinline__ void dot_vector(const u32x4_t& c, const uint32_t* xp, float& D,
                                           float& Dh) {
    using T = Traits<S>;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (T::BITS == 4) {
            uint32_t w = c[j];
            if constexpr (S == SYM4_G128) w ^= 0x88888888u;
            D = dot2_bf16(nib_pair_to_bf16(w), xp[4 * j + 0], D);
            D = dot2_bf16(nib_pair_to_bf16(w >> 4), xp[4 * j + 1], D);
            D = dot2_bf16(nib_pair_to_bf16(w >> 8), xp[4 * j + 2], D);
            D = dot2_bf16(nib_pair_to_bf16(w >> 12), xp[4 * j + 3], D);
        } else {
            const uint32_t w = c[j];
            const uint32_t xa = xp[2 * j], xb = xp[2 * j + 1];
            D = dot2_bf16(nib_pair_to_bf16(w >> 8), xb, dot2_bf16(nib_pair_to_bf16(w), xa, D));
            Dh = dot2_bf16(nib_pair_to_bf16(w >> 12), xb, dot2_bf16(nib_pair_to_bf16(w >> 4), xa, Dh));
        }
    }
}

// Register-resident state of one lane: R rows x NV code vectors and their scales.
template <int S, int NV, int R>
struct Gemv1Regs {
    u32x4_t c[R][NV];
    float sc[R][NV];
    float bi[R][NV];
};

template <int S, int LPR, int NV, int R>
__device__ __forceinline__ void gemv1_load(Gemv1Regs<S, NV, R>& G, const uint8_t* const (&crow)[R],
                                           const uint8_t* const (&srow)[R],
                                           const uint8_t* const (&brow)[R], int VR, int sl) {
    using T = Traits<S>;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int v = sl + LPR * j;
        const int g = v / T::VPG;
        if (v < VR) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                G.c[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(crow[r]) + v);
                if constexpr (T::AFFINE) {
                    G.sc[r][j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(srow[r])[g]);
                    G.bi[r][j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(brow[r])[g]);
                } else {
                    G.sc[r][j] = reinterpret_cast<const float*>(srow[r])[g];
                }
            }
        }
    }
}

template <int S, int LPR, int NV, int R, int XL>
__device__ __forceinline__ void gemv1_compute(const Gemv1Regs<S, NV, R>& G, int VR, int sl,
                                              const uint16_t* __restrict__ x,
                                              const uint32_t* __restrict__ xs,
                                              const float* __restrict__ XS, float (&acc)[R]) {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    constexpr int XW = L::XW;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int v = sl + LPR * j;
        if (v >= VR) break;
        uint32_t xp[XW];
        float X;
        if constexpr (XL == 1) {
            load_x_pairs_global<S>(x, v, xp, X);
        } else {
#pragma unroll
            for (int p = 0; p < XW / 4; ++p) {
                const uint4 q = *reinterpret_cast<const uint4*>(xs + L::piece(v, p));
                xp[4 * p] = q.x; xp[4 * p + 1] = q.y; xp[4 * p + 2] = q.z; xp[4 * p + 3] = q.w;
            }
            X = XS[v];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float D = 0.f, Dh = 0.f;
            dot_vector<S>(G.c[r][j], xp, D, Dh);
            if constexpr (T::BITS == 8) D = fmaf(16.f, Dh, D);
            const float s = G.sc[r][j];
            const float corr = T::AFFINE ? fmaf(-T::BIAS, s, G.bi[r][j]) : -T::BIAS * s;
            acc[r] = fmaf(s, D, acc[r]);
            acc[r] = fmaf(corr, X, acc[r]);
        }
    }
}

// Dense M = 1 GEMV: y[n] = sum_k x[k] w[n][k].
template <int S, int LPR, int NV, int R, int XL>
__global__ __launch_bounds__(256) void gemv1_kernel(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scale,
                                                    const uint8_t* __restrict__ bias, int N, int K,
                                                    const uint16_t* __restrict__ x,
                                                    float* __restrict__ y) {
    using T = Traits<S>;
    extern __shared__ __align__(16) uint32_t smem[];
    constexpr int RSW = 64 / LPR;
    const int VR = K / T::KV;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane / LPR, sl = lane % LPR;
    const int64_t rowbytes = (int64_t)K * T::BITS / 8;
    const int64_t groups = K / T::GROUP;
    constexpr int SB = T::AFFINE ? 2 : 4;
    const uint8_t* crow[R];
    const uint8_t* srow[R];
    const uint8_t* brow[R];
    int n[R];
    const int base = blockIdx.x * (4 * RSW * R) + wave * (RSW * R) + slot;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        n[r] = base + r * RSW;
        const int64_t nl = n[r] < N ? n[r] : N - 1;
        crow[r] = codes + nl * rowbytes;
        srow[r] = scale + nl * groups * SB;
        brow[r] = T::AFFINE ? bias + nl * groups * 2 : nullptr;
    }
    Gemv1Regs<S, NV, R> G;
    gemv1_load<S, LPR, NV, R>(G, crow, srow, brow, VR, sl);  // whole share in flight
    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + K / 2);
    if constexpr (XL == 0) {
        stage_x<S, 1, 1, 256>(x, K, nullptr, 1, K, xs, XS);
        __syncthreads();
    }
    float acc[R];
    gemv1_compute<S, LPR, NV, R, XL>(G, VR, sl, x, xs, XS, acc);
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = group_sum<LPR>(acc[r]);
    if (sl == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (n[r] < N) y[n[r]] = acc[r];
    }
}

}  // namespace w4
