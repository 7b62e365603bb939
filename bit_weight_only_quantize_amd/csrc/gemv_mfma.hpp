// Skinny decode GEMM (2 <= M <= 16 tokens) on the matrix cores.
//
// airllm article §2.2: the weights are dequantized in registers right after the
// load, no dequantized copy is written; §3.3: decode stays memory-bound. With
// several tokens the per-token dot products would make a VALU kernel compute-
// and LDS-bound (every token re-reads its activations), so here the unpacked
// codes feed v_mfma_f32_16x16x32_bf16 directly from registers:
//
//   * D[token][row] = A[token][k] * B[k][row]: A is 16 tokens x 32 k of
//     activations, B the 32 k x 16 weight rows; lane l holds weight row l % 16
//     and k = 8 (l / 16) + 0..7 of B, and rows 4 (l / 16) + 0..3 (tokens) of D,
//     so a lane's outputs all belong to one weight row and one group scale;
//   * a step is one quantization group: 16 bytes of codes per lane (sym, 128
//     weights x 16 rows per wavefront load) or 8 bytes (affine, 64 weights) --
//     an MFMA's 32 k must not straddle two groups, and with four lanes per row
//     an affine group of 64 only fits 8-byte lane loads;
//   * a code word (8 nibbles) unpacks with the magic-exponent trick into four
//     bf16 pairs (k, k+4) = 128 + u, so the activations are permuted the same
//     way (v_perm_b32) and the offset is removed per group with the group's
//     activation sums X, which one extra MFMA against a ones operand delivers
//     already in the D layout:  acc += s * D + (b - BIAS s) * X;
//   * activations come straight from global memory (L2-resident, 16-byte
//     loads issued before the step's code loads) and are reused by the RT row
//     tiles of a wavefront; the block's group scales are staged once in LDS
//     (one coalesced pass instead of a scattered 2-4 byte load per step);
//   * the WK wavefronts of a workgroup take contiguous step ranges of the same
//     rows (split K, DEPTH steps in flight per wavefront) and their partial sums
//     are added through LDS in a fixed order, so results are deterministic.
#pragma once

#include "common.hpp"
#include "gemv_wave.hpp"

namespace w4 {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int S>
struct MfmaStep {
    static constexpr int LB = S == SYM4_G128 ? 16 : 8;  // code bytes per lane per step
    static constexpr int WPL = LB / 4;                  // code words per lane per step
    static constexpr int KSTEP = 8 * LB;                // k per step (one group)
    using code_t = typename std::conditional<LB == 16, u32x4_t, u32x2_t>::type;
};

// bf16x8 from four packed bf16 pairs
__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4_t v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8_t, v);
}

// At most kMfmaMaxGroups groups per row (the staging registers hold four
// 64-group slices).
constexpr int kMfmaMaxGroups = 256;

// LDS: the workgroup's scales as [group][row] words (affine: bf16 scale in the
// low half, bf16 bias in the high half), later reused for the split-K sums.
template <int S, int RT, int WK>
size_t gemv_mfma_lds_bytes(int64_t K) {
    const size_t scales = (size_t)(K / Traits<S>::GROUP) * 16 * RT * 4;
    const size_t red = (size_t)(WK > 1 ? WK - 1 : 1) * RT * 4 * 64 * 4;
    return scales > red ? scales : red;
}

template <int S, int RT, int WK, int DEPTH>
__global__ __launch_bounds__(64 * WK) void gemv_mfma_kernel(GemvGroupArgs a, int K, int M,
                                                            const uint16_t* x) {
    using T = Traits<S>;
    using P = MfmaStep<S>;
    using code_t = typename P::code_t;
    constexpr int WPL = P::WPL;
    constexpr int ROWS = 16 * RT;
    extern __shared__ __align__(16) uint32_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c16 = lane & 15;

    const int t = blockIdx.x;
    int i = 0;
#pragma unroll
    for (int q = 1; q < kMaxGroup; ++q)
        if (q < a.count && t >= a.tile_start[q]) i = q;
    const int N = a.N[i];
    const int row0 = (t - a.tile_start[i]) * ROWS;
    const int groups = K / T::GROUP;  // == steps
    const int J = (groups + WK - 1) / WK;
    const int s0 = wave * J;
    const int s1 = min(s0 + J, groups);

    // 1. the block's scales (and biases) -> LDS, loads issued first
    constexpr int SR = (ROWS + WK - 1) / WK;  // rows staged per wavefront
    const int sgl = (groups + 63) / 64;       // group slices per row
    uint32_t sv[SR][4];
#pragma unroll
    for (int k = 0; k < SR; ++k) {
        const int r = wave + WK * k;
        const int n = min(row0 + min(r, ROWS - 1), N - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j >= sgl) break;  // uniform
            const int gi = min(lane + 64 * j, groups - 1);
            const uint32_t e = (uint32_t)n * (uint32_t)groups + (uint32_t)gi;
            if constexpr (T::AFFINE)
                sv[k][j] = (uint32_t)reinterpret_cast<const uint16_t*>(a.scale[i])[e] |
                           ((uint32_t)reinterpret_cast<const uint16_t*>(a.bias[i])[e] << 16);
            else
                sv[k][j] = reinterpret_cast<const uint32_t*>(a.scale[i])[e];
        }
    }
    asm volatile("" ::: "memory");  // keep the step loads behind these

    // 2. per-lane bases: 32-bit offsets from wave-uniform pointers
    const uint8_t* cbase = a.codes[i];
    uint32_t coff[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n = min(row0 + 16 * rt + c16, N - 1);
        coff[rt] = (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)(g * P::LB);
    }
    // tokens past M re-read row M-1; their outputs are never stored
    const uint32_t xoff = (uint32_t)min(c16, M - 1) * (uint32_t)K + (uint32_t)(g * 2 * P::LB);

    struct Buf {
        u32x4_t xv[WPL];
        code_t c[RT];
    };
    auto load = [&](Buf& B, int s) {
        // activations first: in-order vmcnt then never waits for code bytes
#pragma unroll
        for (int d = 0; d < WPL; ++d)
            B.xv[d] = *reinterpret_cast<const u32x4_t*>(x + xoff + (uint32_t)s * P::KSTEP + 8 * d);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            B.c[rt] = *reinterpret_cast<const code_t*>(cbase + coff[rt] + (uint32_t)s * (P::KSTEP / 2));
    };

    Buf buf[DEPTH];
#pragma unroll
    for (int p = 0; p < DEPTH - 1; ++p)
        if (s0 + p < s1) load(buf[p], s0 + p);

    // scales land in LDS while the first steps' bytes are in flight
#pragma unroll
    for (int k = 0; k < SR; ++k) {
        const int r = wave + WK * k;
        if (r < ROWS) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < sgl && lane + 64 * j < groups) lds[(lane + 64 * j) * ROWS + r] = sv[k][j];
        }
    }
    __syncthreads();

    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    const uint32_t ONE2 = 0x3F803F80u;  // bf16 pair (1, 1)
    const bf16x8_t ONES = as_bf16x8(ONE2, ONE2, ONE2, ONE2);
    f32x4_t acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const Buf& B, int s) {
        uint32_t sw[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) sw[rt] = lds[s * ROWS + 16 * rt + c16];
        bf16x8_t A[WPL];
        f32x4_t DX = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < WPL; ++d) {
            const u32x4_t e = B.xv[d];  // (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) ...
            A[d] = as_bf16x8(__builtin_amdgcn_perm(e[2], e[0], 0x05040100u),
                             __builtin_amdgcn_perm(e[2], e[0], 0x07060302u),
                             __builtin_amdgcn_perm(e[3], e[1], 0x05040100u),
                             __builtin_amdgcn_perm(e[3], e[1], 0x07060302u));
            DX = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[d], ONES, DX, 0, 0, 0);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4_t D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 0; d < WPL; ++d) {
                const uint32_t w = B.c[rt][d];
                auto pair = [&](uint32_t v) {
                    return S == SYM4_G128 ? ((v & MASK) ^ MAGIC) : ((v & MASK) | MAGIC);
                };
                const bf16x8_t Bw = as_bf16x8(pair(w), pair(w >> 4), pair(w >> 8), pair(w >> 12));
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[d], Bw, D, 0, 0, 0);
            }
            float sc, corr;
            if constexpr (T::AFFINE) {
                sc = __uint_as_float(sw[rt] << 16);
                corr = fmaf(-T::BIAS, sc, __uint_as_float(sw[rt] & 0xFFFF0000u));
            } else {
                sc = __uint_as_float(sw[rt]);
                corr = -T::BIAS * sc;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[rt][r] = fmaf(corr, DX[r], fmaf(sc, D[r], acc[rt][r]));
        }
    };

    // DEPTH steps in flight: step s + DEPTH - 1 is loaded while step s is
    // computed; the ring is unrolled so every buffer index is static
    for (int s = s0; s < s1; s += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const int step = s + u;
            if (step < s1) {
                if (step + DEPTH - 1 < s1) load(buf[(u + DEPTH - 1) % DEPTH], step + DEPTH - 1);
                compute(buf[u], step);
            }
        }
    }

    // split-K partial sums: waves 1.. hand theirs to wave 0 through LDS (the
    // scale area, free once every wavefront is past its last step)
    if constexpr (WK > 1) {
        __syncthreads();
        float* red = reinterpret_cast<float*>(lds);
        if (wave > 0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[(((wave - 1) * RT + rt) * 4 + r) * 64 + lane] = acc[rt][r];
        }
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int w = 0; w < WK - 1; ++w)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[rt][r] += red[((w * RT + rt) * 4 + r) * 64 + lane];
    }
    float* y = a.y[i];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n = row0 + 16 * rt + c16;
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m < M) y[(int64_t)m * N + n] = acc[rt][r];
        }
    }
}

}  // namespace w4
