// Prefill GEMM with the dequantization fused in: Y = X * dequant(W)^T.
//
// airllm article §3.3: prefill is compute-dense (decode is memory-bound), so
// this is the one product on the hot path built on the matrix cores; §2.2: the
// weights are converted right after they are loaded instead of materializing a
// dequantized copy in HBM.
//
// Tiling for gfx950 (256 CUs in 8 XCDs, 160 KiB LDS, bf16 MFMA 32x32x16):
//   * a workgroup computes a 256 (M) x 128 (N) tile with 4 wavefronts, each a
//     128 x 64 sub-tile of 4 x 2 MFMA blocks (fp32 accumulators);
//   * per 32-wide k step the X tile (bf16, 16 KiB) is copied and the W tile's
//     codes (2 KiB) are dequantized to bf16 -- w = s*q (sym) or s*u + b (affine),
//     computed in fp32 and rounded to nearest even -- into a double-buffered LDS
//     stage (48 KiB), 16-byte chunks XOR-swizzled so the MFMA operand reads are
//     free of bank conflicts; the next step's global loads are in flight while
//     the current step's MFMAs run;
//   * tiles are ordered so that consecutive tiles land on one XCD and share an
//     X row block (workgroups are dispatched round-robin over the 8 XCDs), which
//     keeps the X block resident in that XCD's L2;
//   * the epilogue rounds the fp32 accumulators to bf16 (nearest even).
#include "common.hpp"
#include "launch.hpp"

namespace w4 {

constexpr int GBM = 256, GBN = 128, GBK = 32;

// 16-byte chunk c (0..3) of LDS row `row` (64 bytes per row)
__device__ __forceinline__ int gchunk(int row, int c) { return row * 4 + (c ^ ((row >> 1) & 3)); }

template <int S>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scale,
                                                   const uint8_t* __restrict__ bias, int M, int N,
                                                   int K, const uint16_t* __restrict__ X,
                                                   uint16_t* __restrict__ Y, int tiles_m,
                                                   int tiles_n) {
    using T = Traits<S>;
    extern __shared__ __align__(16) uint4 gsm[];
    uint4* As = gsm;                      // [2][GBM * 4]
    uint4* Bs = gsm + 2 * GBM * 4;        // [2][GBN * 4]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous range of tiles, N-fastest, so an XCD's workgroups share X rows.
    const int ntiles = tiles_m * tiles_n;
    const int per = (ntiles + 7) / 8;
    const int L = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (L >= ntiles) return;
    const int m0 = (L / tiles_n) * GBM, n0 = (L % tiles_n) * GBN;

    // ---- per-thread load assignment
    // X: 4 chunks of 16 bytes: rows tid/4 + 64 i, chunk tid % 4
    const int ac = tid & 3;
    const uint16_t* xrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = min(m0 + (tid >> 2) + 64 * i, M - 1);
        xrow[i] = X + (int64_t)r * K + ac * 8;
    }
    // W: row tid/2, 16 weights (8 bytes of codes) at k offset 16 * (tid % 2)
    const int brow = tid >> 1, bh = tid & 1;
    const int bn = min(n0 + brow, N - 1);
    const uint8_t* crow = codes + (int64_t)bn * (K / 2) + bh * 8;
    const int64_t groups = K / T::GROUP;
    constexpr int SB = T::AFFINE ? 2 : 4;
    const uint8_t* srow = scale + (int64_t)bn * groups * SB;
    const uint8_t* bro = T::AFFINE ? bias + (int64_t)bn * groups * 2 : nullptr;

    u32x4_t xa[4];
    uint2 wc;
    float ws, wb;
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const u32x4_t*>(xrow[i] + k0);
        wc = *reinterpret_cast<const uint2*>(crow + k0 / 2);
        const int g = (k0 + bh * 16) / T::GROUP;
        if constexpr (T::AFFINE) {
            ws = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(srow)[g]);
            wb = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(bro)[g]);
        } else {
            ws = reinterpret_cast<const float*>(srow)[g];
            wb = -8.f * ws;  // q = u - 8 after the xor below
        }
    };
    auto lstore = [&](int stage) {
        uint4* A = As + stage * GBM * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4_t v = xa[i];
            A[gchunk((tid >> 2) + 64 * i, ac)] = make_uint4(v[0], v[1], v[2], v[3]);
        }
        // dequantize 16 weights -> 8 bf16 pairs (natural k order)
        uint32_t out[8];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            uint32_t c = d ? wc.y : wc.x;
            if constexpr (S == SYM4_G128) c ^= 0x88888888u;  // two's complement -> q + 8
            const uint32_t lo = c & 0x0F0F0F0Fu;             // elements 0, 2, 4, 6
            const uint32_t hi = (c >> 4) & 0x0F0F0F0Fu;      // elements 1, 3, 5, 7
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float e0 = (float)((lo >> (8 * b)) & 0xFFu);
                const float e1 = (float)((hi >> (8 * b)) & 0xFFu);
                const bf16x2_t p = {(__bf16)fmaf(e0, ws, wb), (__bf16)fmaf(e1, ws, wb)};
                out[4 * d + b] = __builtin_bit_cast(uint32_t, p);
            }
        }
        uint4* B = Bs + stage * GBN * 4;
        B[gchunk(brow, 2 * bh)] = make_uint4(out[0], out[1], out[2], out[3]);
        B[gchunk(brow, 2 * bh + 1)] = make_uint4(out[4], out[5], out[6], out[7]);
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int ksteps = K / GBK;
    gload(0);
    lstore(0);
    __syncthreads();
    const int arow = wm * 128 + (lane & 31), brw = wn * 64 + (lane & 31), half = lane >> 5;
    for (int s = 0; s < ksteps; ++s) {
        const int st = s & 1;
        if (s + 1 < ksteps) gload((s + 1) * GBK);
        const uint4* A = As + st * GBM * 4;
        const uint4* B = Bs + st * GBN * 4;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8_t af[4], bf[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = __builtin_bit_cast(bf16x8_t, A[gchunk(arow + 32 * i, 2 * kk + half)]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = __builtin_bit_cast(bf16x8_t, B[gchunk(brw + 32 * j, 2 * kk + half)]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < ksteps) lstore(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue: D[i][j] of a 32x32 block sits in lane j + 32 * ((i / 4) % 2),
    // register 4 * (i / 8) + i % 4.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + 32 * j + (lane & 31);
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
                if (m < M) {
                    const bf16x2_t p = {(__bf16)acc[i][j][r], (__bf16)0.f};
                    Y[(int64_t)m * N + n] = (uint16_t)__builtin_bit_cast(uint32_t, p);
                }
            }
        }
}

hipError_t launch_gemm(int scheme, const void* codes, const void* scale, const void* bias,
                       int64_t N, int64_t K, const uint16_t* X, int64_t M, uint16_t* Y,
                       hipStream_t st) {
    const int tm = (int)((M + GBM - 1) / GBM), tn = (int)((N + GBN - 1) / GBN);
    const int per = (tm * tn + 7) / 8;
    const size_t lds = 2 * (GBM + GBN) * 64;
    if (scheme == SYM4_G128)
        hipLaunchKernelGGL(gemm_kernel<SYM4_G128>, dim3(8 * per), dim3(256), lds, st,
                           (const uint8_t*)codes, (const uint8_t*)scale, (const uint8_t*)bias,
                           (int)M, (int)N, (int)K, X, Y, tm, tn);
    else
        hipLaunchKernelGGL(gemm_kernel<AFF4_G64>, dim3(8 * per), dim3(256), lds, st,
                           (const uint8_t*)codes, (const uint8_t*)scale, (const uint8_t*)bias,
                           (int)M, (int)N, (int)K, X, Y, tm, tn);
    return hipGetLastError();
}

}  // namespace w4
