// Skinny fused-dequant dot-product core (decode GEMV, M <= MT tokens per pass).
//
// The airllm article §2.2 fuses the dequantization into the matmul kernel: the
// weights are converted in registers right after they are loaded, so no
// dequantized copy ever reaches memory. This core does exactly that for a
// wavefront-slot of LPR lanes per weight row:
//
//   * codes stream from HBM as 16-byte vectors (32 four-bit or 16 eight-bit
//     weights), coalesced: the LPR lanes of a row read consecutive vectors;
//   * a pair of nibbles becomes a bf16 pair (128 + u) with one v_and_or_b32
//     (exponent 2^7, nibble in the low mantissa bits: exact);
//   * v_dot2_f32_bf16 multiplies it with a pair of activations and accumulates
//     in fp32;
//   * the constant offset is removed once per group from the group's activation
//     sum:  sum (BIAS + u) x = sum u x + BIAS * X,  so per group
//        sym:    s * (D - 136 X)              (codes XOR 8 turn two's complement
//                                              nibbles into u = q + 8)
//        affine: s * D + (b - BIAS * s) * X   (w = s u + b);
//   * partial sums are reduced across the LPR lanes with DPP.
//
// Activations are staged once per workgroup in LDS, already permuted into the
// pairs the unpack produces ((x[t], x[t+4]) for a 4-bit word, (x[t], x[t+2]) for
// an 8-bit word), together with per-vector sums X. Pieces of a lane's block are
// XOR-swizzled so that the 8 lanes served by one LDS cycle hit distinct banks.
#pragma once

#include "common.hpp"

namespace w4 {

template <int S, int V>
struct XLayout {
    using T = Traits<S>;
    static constexpr int XW = T::BITS == 4 ? 16 : 8;  // activation dwords per code vector
    static constexpr int P = V * XW / 4;              // 16-byte pieces per lane block
    // dword offset of piece p (0..XW/4-1) of vector v inside one token's row
    __device__ __forceinline__ static int piece(int v, int p) {
        const int b = v / V;
        const int pp = (v % V) * (XW / 4) + p;
        const int h = (P >= 8) ? (b & 7) : ((b * P / 8) & (P - 1));
        return b * (V * XW) + 4 * (pp ^ h);
    }
};

// Stage activation rows x[m][0..K) (bf16) for m < mt into LDS:
//   xs[m * (K/2) + ...]  permuted pairs (see XLayout), zero for m >= mt
//   XS[m * VR + v]       fp32 sum of the vector's activations (sequential order)
template <int S, int MT, int V, int NT>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int64_t ldx,
                                        const int* __restrict__ tok, int mt, int K,
                                        uint32_t* __restrict__ xs, float* __restrict__ XS) {
    using T = Traits<S>;
    using L = XLayout<S, V>;
    const int VR = K / T::KV;
    const int xstride = K / 2;
    for (int idx = threadIdx.x; idx < MT * VR; idx += NT) {
        const int m = idx / VR, v = idx - m * VR;
        uint32_t* dst = xs + m * xstride;
        if (m >= mt) {
            for (int p = 0; p < L::XW / 4; ++p)
                *reinterpret_cast<uint4*>(dst + L::piece(v, p)) = make_uint4(0, 0, 0, 0);
            XS[m * VR + v] = 0.f;
            continue;
        }
        const int64_t row = tok ? (int64_t)tok[m] : (int64_t)m;
        const uint4* src = reinterpret_cast<const uint4*>(x + row * ldx + (int64_t)v * T::KV);
        float sum = 0.f;
        if constexpr (T::BITS == 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // 8 activations per code dword
                const uint4 d = src[j];
                uint4 o;
                o.x = (d.x & 0xFFFFu) | (d.z << 16);          // (x0, x4)
                o.y = (d.x >> 16) | (d.z & 0xFFFF0000u);      // (x1, x5)
                o.z = (d.y & 0xFFFFu) | (d.w << 16);          // (x2, x6)
                o.w = (d.y >> 16) | (d.w & 0xFFFF0000u);      // (x3, x7)
                *reinterpret_cast<uint4*>(dst + L::piece(v, j)) = o;
                sum += bf16_bits_to_f32(d.x & 0xFFFFu); sum += bf16_bits_to_f32(d.x >> 16);
                sum += bf16_bits_to_f32(d.y & 0xFFFFu); sum += bf16_bits_to_f32(d.y >> 16);
                sum += bf16_bits_to_f32(d.z & 0xFFFFu); sum += bf16_bits_to_f32(d.z >> 16);
                sum += bf16_bits_to_f32(d.w & 0xFFFFu); sum += bf16_bits_to_f32(d.w >> 16);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {  // 8 activations = two 4-weight code dwords
                const uint4 d = src[j];
                uint4 o;
                o.x = (d.x & 0xFFFFu) | (d.y << 16);          // (x0, x2)
                o.y = (d.x >> 16) | (d.y & 0xFFFF0000u);      // (x1, x3)
                o.z = (d.z & 0xFFFFu) | (d.w << 16);          // (x4, x6)
                o.w = (d.z >> 16) | (d.w & 0xFFFF0000u);      // (x5, x7)
                *reinterpret_cast<uint4*>(dst + L::piece(v, j)) = o;
                sum += bf16_bits_to_f32(d.x & 0xFFFFu); sum += bf16_bits_to_f32(d.x >> 16);
                sum += bf16_bits_to_f32(d.y & 0xFFFFu); sum += bf16_bits_to_f32(d.y >> 16);
                sum += bf16_bits_to_f32(d.z & 0xFFFFu); sum += bf16_bits_to_f32(d.z >> 16);
                sum += bf16_bits_to_f32(d.w & 0xFFFFu); sum += bf16_bits_to_f32(d.w >> 16);
            }
        }
        XS[m * VR + v] = sum;
    }
}

// Staging of one token's activations by NT threads (thread index `tid`):
// fetch(): up to XV vectors per thread into registers; commit(): pair
// permutation (v_perm_b32), per-vector sums (v_dot2 with ones) and the LDS
// writes. Same layout as stage_x with V = 1.
template <int S, int XV, int NT>
struct XStage {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    static constexpr int Q = T::BITS == 4 ? 4 : 2;  // 16-byte activation loads per code vector
    u32x4_t d[XV][Q];

    // Loads are unconditional (index clamped into the row) so that no branch
    // blurs the compiler's in-order wait counts; extra lanes re-read vector VR-1.
    __device__ __forceinline__ void fetch(const uint16_t* __restrict__ x, int VR, int tid) {
#pragma unroll
        for (int t = 0; t < XV; ++t) {
            const int v = min(tid + NT * t, VR - 1);
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + (int64_t)v * T::KV);
#pragma unroll
            for (int q = 0; q < Q; ++q) d[t][q] = src[q];
        }
    }

    __device__ __forceinline__ void commit(int VR, uint32_t* __restrict__ xs, float* __restrict__ XS,
                                           int tid) const {
        constexpr uint32_t ONES = 0x3F803F80u;  // bf16 pair (1, 1)
#pragma unroll
        for (int t = 0; t < XV; ++t) {
            const int v = tid + NT * t;
            if (v < VR) {
                float sum = 0.f;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const u32x4_t e = d[t][q];
                    uint4 o;
                    if constexpr (T::BITS == 4) {  // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
                        o.x = __builtin_amdgcn_perm(e[2], e[0], 0x05040100u);
                        o.y = __builtin_amdgcn_perm(e[2], e[0], 0x07060302u);
                        o.z = __builtin_amdgcn_perm(e[3], e[1], 0x05040100u);
                        o.w = __builtin_amdgcn_perm(e[3], e[1], 0x07060302u);
                    } else {                       // (x0,x2) (x1,x3) (x4,x6) (x5,x7)
                        o.x = __builtin_amdgcn_perm(e[1], e[0], 0x05040100u);
                        o.y = __builtin_amdgcn_perm(e[1], e[0], 0x07060302u);
                        o.z = __builtin_amdgcn_perm(e[3], e[2], 0x05040100u);
                        o.w = __builtin_amdgcn_perm(e[3], e[2], 0x07060302u);
                    }
                    *reinterpret_cast<uint4*>(xs + L::piece(v, q)) = o;
                    sum = dot2_bf16(ONES, e[0], sum);
                    sum = dot2_bf16(ONES, e[1], sum);
                    sum = dot2_bf16(ONES, e[2], sum);
                    sum = dot2_bf16(ONES, e[3], sum);
                }
                XS[v] = sum;
            }
        }
    }
};

// One lane's share of R weight rows against MT staged tokens.
template <int S, int MT, int LPR, int V, int R>
struct SkinnyCore {
    using T = Traits<S>;
    using L = XLayout<S, V>;
    struct Buf {
        u32x4_t c[R][V];
        float s[R];
        float b[R];
    };

    const uint8_t* crow[R];  // codes of each row
    const uint8_t* srow[R];  // scales of each row (fp32 or bf16)
    const uint8_t* brow[R];  // biases of each row (bf16, affine only)
    int VR;                  // 16-byte vectors per row
    int sl;                  // lane index inside the row slot (0..LPR-1)

    __device__ __forceinline__ int steps() const { return (VR + LPR * V - 1) / (LPR * V); }

    __device__ __forceinline__ void load(Buf& B, int step) const {
        const int v0 = (step * LPR + sl) * V;
        if (v0 < VR) {
            const int g = v0 / T::VPG;
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int i = 0; i < V; ++i)
                    B.c[r][i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t*>(crow[r]) + (v0 + i));
                if constexpr (T::AFFINE) {
                    B.s[r] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(srow[r])[g]);
                    B.b[r] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(brow[r])[g]);
                } else {
                    B.s[r] = reinterpret_cast<const float*>(srow[r])[g];
                }
            }
        }
    }

    __device__ __forceinline__ void compute(const Buf& B, int step, const uint32_t* __restrict__ xs,
                                            const float* __restrict__ XS, int xstride,
                                            float (&acc)[R][MT]) const {
        const int v0 = (step * LPR + sl) * V;
        if (v0 >= VR) return;
        float D[R][MT];
        float Dh[R][MT];  // high-nibble sums (8-bit codes only)
        float X[MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) D[r][m] = Dh[r][m] = 0.f;
#pragma unroll
        for (int m = 0; m < MT; ++m) X[m] = 0.f;

#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int v = v0 + i;
            uint4 xp[MT][L::XW / 4];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
#pragma unroll
                for (int p = 0; p < L::XW / 4; ++p)
                    xp[m][p] = *reinterpret_cast<const uint4*>(xs + m * xstride + L::piece(v, p));
                X[m] += XS[m * VR + v];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint32_t cw[4] = {B.c[r][i][0], B.c[r][i][1], B.c[r][i][2], B.c[r][i][3]};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (T::BITS == 4) {
                        uint32_t c = cw[j];
                        if constexpr (S == SYM4_G128) c ^= 0x88888888u;
                        const uint32_t w0 = nib_pair_to_bf16(c);
                        const uint32_t w1 = nib_pair_to_bf16(c >> 4);
                        const uint32_t w2 = nib_pair_to_bf16(c >> 8);
                        const uint32_t w3 = nib_pair_to_bf16(c >> 12);
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            const uint4 q = xp[m][j];
                            float d = D[r][m];
                            d = dot2_bf16(w0, q.x, d);
                            d = dot2_bf16(w1, q.y, d);
                            d = dot2_bf16(w2, q.z, d);
                            d = dot2_bf16(w3, q.w, d);
                            D[r][m] = d;
                        }
                    } else {
                        const uint32_t c = cw[j];
                        const uint32_t l0 = nib_pair_to_bf16(c);        // bytes 0,2 low nibbles
                        const uint32_t l1 = nib_pair_to_bf16(c >> 8);   // bytes 1,3 low nibbles
                        const uint32_t h0 = nib_pair_to_bf16(c >> 4);   // bytes 0,2 high nibbles
                        const uint32_t h1 = nib_pair_to_bf16(c >> 12);  // bytes 1,3 high nibbles
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            const uint4 q = xp[m][j >> 1];
                            const uint32_t xa = (j & 1) ? q.z : q.x;
                            const uint32_t xb = (j & 1) ? q.w : q.y;
                            D[r][m] = dot2_bf16(l1, xb, dot2_bf16(l0, xa, D[r][m]));
                            Dh[r][m] = dot2_bf16(h1, xb, dot2_bf16(h0, xa, Dh[r][m]));
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float s = B.s[r];
            const float corr = T::AFFINE ? fmaf(-T::BIAS, s, B.b[r]) : -T::BIAS * s;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float d = (T::BITS == 8) ? fmaf(16.f, Dh[r][m], D[r][m]) : D[r][m];
                acc[r][m] = fmaf(s, d, acc[r][m]);
                acc[r][m] = fmaf(corr, X[m], acc[r][m]);
            }
        }
    }

    // Full pass over the row: software-pipelined (next step's loads in flight
    // while the current one is computed). `first` must already hold step 0.
    __device__ __forceinline__ void run(Buf& A, Buf& Bb, const uint32_t* xs, const float* XS,
                                        int xstride, float (&acc)[R][MT]) const {
        const int ns = steps();
        for (int st = 0; st < ns; st += 2) {
            if (st + 1 < ns) load(Bb, st + 1);
            compute(A, st, xs, XS, xstride, acc);
            if (st + 1 < ns) {
                if (st + 2 < ns) load(A, st + 2);
                compute(Bb, st + 1, xs, XS, xstride, acc);
            }
        }
    }
};

}  // namespace w4
