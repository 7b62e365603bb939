// Single-token decode GEMV, one wavefront per weight row (K >= 64 code vectors).
//
// Design for gfx950 (airllm article §2.2: dequantize in registers right after
// the load; §3.3: decode is memory-bound):
//   * a wavefront owns R whole rows, so row addresses are wave-uniform (SGPRs)
//     and lane l reads 16-byte code vectors l, l+64, ... of each row: every load
//     instruction moves 1 KiB of contiguous codes;
//   * all code and scale loads of a lane are issued up front (single shot),
//     right behind its share of the activations, so the whole matrix is in
//     flight at once;
//   * the activation vector is staged once per workgroup in LDS as bf16 pairs
//     matching the unpack order, with per-vector sums for the offset removal.
//     Every row wavefront stages a share of it and issues those loads before
//     its weight loads: vmcnt retires a wavefront's loads in order, so waiting
//     for the activations then does not wait for the weights, and the weight
//     bytes stay in flight across the staging barrier. (Dedicated staging
//     wavefronts were measured slower: their loads queue behind the row
//     wavefronts' weight traffic and they take wave slots from row waves, so
//     fewer workgroups fit on a CU at once.)
//   * a code vector is consumed as soon as the wavefront's own loads for it
//     have retired;
//   * one v_and_or_b32 (affine) or v_bitop3_b32 (sym: and + xor with 0x43084308,
//     which also moves the two's-complement code to q + 8) turns a nibble pair
//     into a bf16 pair (128 + u); v_dot2_f32_bf16 accumulates in fp32;
//   * the 64-lane reduction is DPP only (quad perms, row mirrors, row_bcast15/31).
// Several matrices that share the activation vector (Q/K/V, gate/up) can be
// served by one launch: blocks are split among up to kMaxGroup matrices.
#pragma once

#include "common.hpp"
#include "skinny.hpp"

namespace w4 {

constexpr int kMaxGroup = 4;

struct GemvGroupArgs {
    const uint8_t* codes[kMaxGroup];
    const uint8_t* scale[kMaxGroup];
    const uint8_t* bias[kMaxGroup];
    float* y[kMaxGroup];
    int N[kMaxGroup];
    int tile_start[kMaxGroup + 1];  // first block of each matrix; tile_start[count] = grid
    int count;
    uint16_t* h;  // gated launches: bf16(gelu_tanh(y[0]) * y[1]) [M][N] instead of y
};

// Opaque VGPR copy of a constant: keeps the compiler from folding it into
// literal operands (VOP3 encodings on gfx9 take no literals), so the unpack
// stays one three-operand instruction per nibble pair.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
    return r;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 ROW_MASK, 0xF, false));
}

// Full 64-lane sum; lane 63 holds the total (DPP only, no LDS traffic).
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
    v += dpp_f<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141, 0xF>(v);  // row_half_mirror
    v += dpp_f<0x140, 0xF>(v);  // row_mirror: every lane holds its 16-lane row sum
    v += dpp_f<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
    v += dpp_f<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
    return v;
}

// D = sum over one 16-byte code vector of (BIAS_ELEM + u) * x, x given as the
// staged bf16 pairs xp (XW dwords); 8-bit codes fold the high nibbles in as 16x.
template <int S>
__device__ __forceinline__ float dot_code_vector(const u32x4_t& c, const uint32_t* xp,
                                                 uint32_t MASK, uint32_t MAGIC) {
    using T = Traits<S>;
    float D = 0.f, Dh = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w = c[d];
        if constexpr (T::BITS == 4) {
            // sym: (nib & 0xF) ^ 0x..08 = 0x43 | (q + 8); affine: | 0x43 -> 128 + u
            auto pair = [&](uint32_t s) {
                return S == SYM4_G128 ? ((s & MASK) ^ MAGIC) : ((s & MASK) | MAGIC);
            };
            D = dot2_bf16(pair(w), xp[4 * d + 0], D);
            D = dot2_bf16(pair(w >> 4), xp[4 * d + 1], D);
            D = dot2_bf16(pair(w >> 8), xp[4 * d + 2], D);
            D = dot2_bf16(pair(w >> 12), xp[4 * d + 3], D);
        } else {
            const uint32_t xa = xp[2 * d], xb = xp[2 * d + 1];
            D = dot2_bf16((w & MASK) | MAGIC, xa, D);
            D = dot2_bf16(((w >> 8) & MASK) | MAGIC, xb, D);
            Dh = dot2_bf16(((w >> 4) & MASK) | MAGIC, xa, Dh);
            Dh = dot2_bf16(((w >> 12) & MASK) | MAGIC, xb, Dh);
        }
    }
    if constexpr (T::BITS == 8) D = fmaf(16.f, Dh, D);
    return D;
}

// acc += s * D + (b - BIAS * s) * X   (affine)   or   s * D - BIAS * s * X   (sym)
template <int S>
__device__ __forceinline__ float apply_group(float acc, float D, float X, float s, float b) {
    using T = Traits<S>;
    const float corr = T::AFFINE ? fmaf(-T::BIAS, s, b) : -T::BIAS * s;
    acc = fmaf(s, D, acc);
    return fmaf(corr, X, acc);
}

template <int S>
__device__ __forceinline__ uint32_t unpack_magic() {
    return opaque(S == SYM4_G128 ? 0x43084308u : 0x43004300u);
}

// Staged activation pairs of vector v (XW dwords) from an LDS region.
template <int S>
__device__ __forceinline__ void read_pairs(const uint32_t* xs, int v,
                                           uint32_t (&xp)[Traits<S>::BITS == 4 ? 16 : 8]) {
    using L = XLayout<S, 1>;
#pragma unroll
    for (int p = 0; p < L::XW / 4; ++p) {
        const uint4 q = *reinterpret_cast<const uint4*>(xs + L::piece(v, p));
        xp[4 * p] = q.x; xp[4 * p + 1] = q.y; xp[4 * p + 2] = q.z; xp[4 * p + 3] = q.w;
    }
}

// x is deliberately not __restrict__: loads from a read-only no-alias kernel
// argument count as constant memory, which the compiler may schedule after the
// weight loads regardless of any fence, and then the activation wait would
// also wait for every weight byte.
template <int S, int NV, int R, int XV, int RW>
__global__ __launch_bounds__(64 * RW) void gemv_wave_kernel(GemvGroupArgs a, int K,
                                                            const uint16_t* x) {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    constexpr int XW = L::XW;
    extern __shared__ __align__(16) uint32_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int VR = K / T::KV;

    // which matrix of the group this block serves (uniform)
    const int t = blockIdx.x;
    int i = 0;
#pragma unroll
    for (int q = 1; q < kMaxGroup; ++q)
        if (q < a.count && t >= a.tile_start[q]) i = q;
    const int N = a.N[i];
    const int row0 = (t - a.tile_start[i]) * (RW * R) + wave * R;
    const int64_t rowbytes = (int64_t)K * T::BITS / 8;
    const int64_t groups = K / T::GROUP;
    constexpr int SB = T::AFFINE ? 2 : 4;

    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + K / 2);
    // this wavefront's share of the activations, loaded before any weight byte
    XStage<S, XV, 64 * RW> xstage;
    xstage.fetch(x, VR, threadIdx.x);
    asm volatile("" ::: "memory");  // keep the weight loads behind these

    u32x4_t c[R][NV];
    float sc[R][NV], bi[R][NV];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = row0 + r < N ? row0 + r : N - 1;
        const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(a.codes[i] + n * rowbytes);
        const uint8_t* sp = a.scale[i] + n * groups * SB;
        const uint8_t* bp = T::AFFINE ? a.bias[i] + n * groups * 2 : nullptr;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            // unconditional (clamped) loads keep the wait counts exact; the
            // duplicates past the row end are never used
            const int v = min(lane + 64 * j, VR - 1);
            c[r][j] = __builtin_nontemporal_load(cp + v);
            const int g = v / T::VPG;
            if constexpr (T::AFFINE) {
                sc[r][j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(sp)[g]);
                bi[r][j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(bp)[g]);
            } else {
                sc[r][j] = reinterpret_cast<const float*>(sp)[g];
            }
        }
    }

    xstage.commit(VR, xs, XS, threadIdx.x);  // waits for the activations only
    __syncthreads();  // activations staged; weight loads still in flight

    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int v = lane + 64 * j;
        if (v >= VR) break;
        uint32_t xp[XW];
        read_pairs<S>(xs, v, xp);
        const float X = XS[v];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = apply_group<S>(acc[r], dot_code_vector<S>(c[r][j], xp, MASK, MAGIC), X,
                                    sc[r][j], T::AFFINE ? bi[r][j] : 0.f);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float tot = wave_sum_to_lane63(acc[r]);
        if (lane == 63 && row0 + r < N) a.y[i][row0 + r] = tot;
    }
}

}  // namespace w4

namespace w4 {

// Multi-token decode GEMV (2 <= M <= 64) on the same design: a row wavefront
// loads its R rows' codes once (registers) and reuses them for every token;
// the staging wavefronts stage MT tokens at a time into one of two LDS buffers
// while the row wavefronts consume the other. Per token tile a row wavefront
// unpacks each code vector once and issues 16 v_dot2 per token.
// LDS: 2 * MT * (K/2 + K/KV) dwords (up to the 160 KiB of a gfx950 CU).
// Workgroup (row block, blockIdx.y) takes tokens [blockIdx.y * TPW, + TPW):
// launches with few row blocks split the tokens to fill the chip.
template <int S, int NV, int R, int MT, int XV, int SW>
__global__ __launch_bounds__(256 + 64 * SW) void gemv_wave_mt_kernel(GemvGroupArgs a, int K, int M,
                                                                     const uint16_t* __restrict__ x,
                                                                     int TPW) {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    constexpr int XW = L::XW;
    extern __shared__ __align__(16) uint32_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int VR = K / T::KV;
    const int tokw = K / 2 + VR;             // dwords per staged token
    const int tb = blockIdx.y * TPW;         // this workgroup's first token
    const int Mw = min(M - tb, TPW);         // and its token count (>= 1)
    const int tiles = (Mw + MT - 1) / MT;

    const int t = blockIdx.x;
    int i = 0;
#pragma unroll
    for (int q = 1; q < kMaxGroup; ++q)
        if (q < a.count && t >= a.tile_start[q]) i = q;
    const int N = a.N[i];
    const int row0 = (t - a.tile_start[i]) * (4 * R) + wave * R;

    if (wave >= 4) {
        // staging wavefronts: tile s -> buffer s % 2, one barrier per tile
        const int sl = threadIdx.x - 256;
        for (int s = 0; s < tiles; ++s) {
            uint32_t* buf = smem + (s & 1) * MT * tokw;
            XStage<S, XV, 64 * SW> st[MT];  // all loads of the tile first, then the LDS writes
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int tok = tb + min(s * MT + m, Mw - 1);  // rows past Mw re-stage the last (unused)
                st[m].fetch(x + (int64_t)tok * K, VR, sl);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
                st[m].commit(VR, buf + m * tokw, reinterpret_cast<float*>(buf + m * tokw + K / 2), sl);
            __syncthreads();
        }
        return;
    }

    const int64_t rowbytes = (int64_t)K * T::BITS / 8;
    const int64_t groups = K / T::GROUP;
    constexpr int SB = T::AFFINE ? 2 : 4;
    u32x4_t c[R][NV];
    float sc[R][NV], bi[R][NV];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = row0 + r < N ? row0 + r : N - 1;
        const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(a.codes[i] + n * rowbytes);
        const uint8_t* sp = a.scale[i] + n * groups * SB;
        const uint8_t* bp = T::AFFINE ? a.bias[i] + n * groups * 2 : nullptr;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int v = min(lane + 64 * j, VR - 1);
            c[r][j] = __builtin_nontemporal_load(cp + v);
            const int g = v / T::VPG;
            if constexpr (T::AFFINE) {
                sc[r][j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(sp)[g]);
                bi[r][j] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(bp)[g]);
            } else {
                sc[r][j] = reinterpret_cast<const float*>(sp)[g];
                bi[r][j] = 0.f;
            }
        }
    }
    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    for (int s = 0; s < tiles; ++s) {
        __syncthreads();  // tile s staged
        const uint32_t* buf = smem + (s & 1) * MT * tokw;
        float acc[R][MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int v = lane + 64 * j;
            if (v >= VR) break;
            uint32_t w[R][16];  // unpacked bf16 pairs of each row's code vector
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t cw = c[r][j][d];
                    if constexpr (T::BITS == 4) {
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            const uint32_t sft = cw >> (4 * h);
                            w[r][4 * d + h] = S == SYM4_G128 ? ((sft & MASK) ^ MAGIC) : ((sft & MASK) | MAGIC);
                        }
                    } else {
                        w[r][4 * d + 0] = (cw & MASK) | MAGIC;          // low nibbles, bytes 0/2
                        w[r][4 * d + 1] = ((cw >> 8) & MASK) | MAGIC;   // low nibbles, bytes 1/3
                        w[r][4 * d + 2] = ((cw >> 4) & MASK) | MAGIC;   // high nibbles, bytes 0/2
                        w[r][4 * d + 3] = ((cw >> 12) & MASK) | MAGIC;  // high nibbles, bytes 1/3
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                uint32_t xp[XW];
                read_pairs<S>(buf + m * tokw, v, xp);
                const float X = reinterpret_cast<const float*>(buf + m * tokw + K / 2)[v];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float D = 0.f;
                    if constexpr (T::BITS == 4) {
#pragma unroll
                        for (int q = 0; q < 16; ++q) D = dot2_bf16(w[r][q], xp[q], D);
                    } else {
                        float Dh = 0.f;
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            D = dot2_bf16(w[r][4 * d + 0], xp[2 * d], D);
                            D = dot2_bf16(w[r][4 * d + 1], xp[2 * d + 1], D);
                            Dh = dot2_bf16(w[r][4 * d + 2], xp[2 * d], Dh);
                            Dh = dot2_bf16(w[r][4 * d + 3], xp[2 * d + 1], Dh);
                        }
                        D = fmaf(16.f, Dh, D);
                    }
                    acc[r][m] = apply_group<S>(acc[r][m], D, X, sc[r][j], bi[r][j]);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float tot = wave_sum_to_lane63(acc[r][m]);
                const int tok = s * MT + m;
                if (lane == 63 && row0 + r < N && tok < Mw) a.y[i][(int64_t)(tb + tok) * N + row0 + r] = tot;
            }
    }
}

}  // namespace w4
