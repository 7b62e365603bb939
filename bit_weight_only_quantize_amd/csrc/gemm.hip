// Prefill GEMM with the dequantization fused in: Y = X * dequant(W)^T.
//
// airllm article §3.3: prefill is compute-dense (decode is memory-bound), so
// this is the one product on the hot path built on the matrix cores; §2.2: the
// weights are converted right after they are loaded instead of materializing a
// dequantized copy in HBM.
//
// Design for gfx950 (256 CUs in 8 XCDs, 160 KiB LDS, bf16 MFMA 32x32x16):
//   * a workgroup computes a 256 (M) x 128 (N) tile with 8 wavefronts: 4 MFMA
//     wavefronts (a 2 x 2 grid of 128 x 64 sub-tiles, fp32 accumulators) and 4
//     producer wavefronts, one of each per SIMD, so the dequantization VALU work
//     of the producer issues in the shadow of the consumer's MFMAs;
//   * producers stream 64-wide k steps: the X tile (bf16, 32 KiB) is copied and
//     the W tile's codes (4 KiB) are dequantized -- w = s*q (sym) or s*u + b
//     (affine), in fp32, rounded to nearest even bf16 -- into a 3-stage LDS ring
//     (144 KiB); global loads run three steps ahead of their LDS stores;
//   * 16-byte chunks are XOR-swizzled by row so MFMA operand reads from LDS are
//     free of bank conflicts; one barrier per k step separates the ring stages;
//   * tiles are ordered so consecutive tiles land on one XCD and share an X row
//     block (workgroups are dispatched round-robin over the 8 XCDs), keeping
//     that block resident in the XCD's L2;
//   * the epilogue rounds the fp32 accumulators to bf16 (nearest even).
#include "common.hpp"
#include "launch.hpp"

namespace w4 {

constexpr int GBM = 256, GBN = 128, GBK = 64, GSTAGES = 3;
constexpr int GCH = GBK / 8;  // 16-byte chunks per LDS row

// LDS chunk index of chunk c (0..7) of row `row`
__device__ __forceinline__ int gchunk(int row, int c) { return row * GCH + (c ^ (row & 7)); }

template <int S>
__global__ __launch_bounds__(512) void gemm_kernel(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scale,
                                                   const uint8_t* __restrict__ bias, int M, int N,
                                                   int K, const uint16_t* __restrict__ X,
                                                   uint16_t* __restrict__ Y, int tiles_m,
                                                   int tiles_n) {
    using T = Traits<S>;
    extern __shared__ __align__(16) uint4 gsm[];
    constexpr int STAGE = (GBM + GBN) * GCH;  // chunks per ring stage
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous range of tiles, N-fastest, so an XCD's workgroups share X rows.
    const int ntiles = tiles_m * tiles_n;
    const int per = (ntiles + 7) / 8;
    const int L = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (L >= ntiles) return;
    const int m0 = (L / tiles_n) * GBM, n0 = (L % tiles_n) * GBN;
    const int ksteps = K / GBK;

    if (wave >= 4) {
        // ---------------- producers: 256 threads
        const int p = tid - 256;
        const uint16_t* xrow[8];
        int arow[8], ac[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = p + 256 * i;
            arow[i] = q >> 3;
            ac[i] = q & 7;
            const int r = min(m0 + arow[i], M - 1);
            xrow[i] = X + (int64_t)r * K + ac[i] * 8;
        }
        const int brow = p >> 1, bh = p & 1;
        const int bn = min(n0 + brow, N - 1);
        const uint8_t* crow = codes + (int64_t)bn * (K / 2) + bh * 16;
        const int64_t groups = K / T::GROUP;
        constexpr int SB = T::AFFINE ? 2 : 4;
        const uint8_t* srow = scale + (int64_t)bn * groups * SB;
        const uint8_t* bro = T::AFFINE ? bias + (int64_t)bn * groups * 2 : nullptr;

        // Loaded values are kept raw until lstore: converting a scale right after
        // its load would make the wavefront wait (vmcnt retires in order) for the
        // whole load batch issued before it, defeating the prefetch.
        struct Regs {
            u32x4_t xa[8];
            u32x4_t wc;
            uint32_t ws, wb;  // raw scale / bias bits
        };
        auto gload = [&](Regs& R, int s) {
            const int k0 = s * GBK;
#pragma unroll
            for (int i = 0; i < 8; ++i) R.xa[i] = *reinterpret_cast<const u32x4_t*>(xrow[i] + k0);
            R.wc = *reinterpret_cast<const u32x4_t*>(crow + k0 / 2);
            const int g = k0 / T::GROUP;
            if constexpr (T::AFFINE) {
                R.ws = reinterpret_cast<const uint16_t*>(srow)[g];
                R.wb = reinterpret_cast<const uint16_t*>(bro)[g];
            } else {
                R.ws = reinterpret_cast<const uint32_t*>(srow)[g];
            }
        };
        auto lstore = [&](const Regs& R, int s) {
            const float ws = T::AFFINE ? bf16_bits_to_f32(R.ws) : __uint_as_float(R.ws);
            const float wb = T::AFFINE ? bf16_bits_to_f32(R.wb) : -8.f * ws;  // sym: q = u - 8
            uint4* A = gsm + (s % GSTAGES) * STAGE;
            uint4* B = A + GBM * GCH;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                A[gchunk(arow[i], ac[i])] = make_uint4(R.xa[i][0], R.xa[i][1], R.xa[i][2], R.xa[i][3]);
            // 32 weights (4 code dwords) -> 4 chunks of 8 bf16 in natural k order
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t c = R.wc[d];
                if constexpr (S == SYM4_G128) c ^= 0x88888888u;  // two's complement -> q + 8
                const uint32_t lo = c & 0x0F0F0F0Fu;             // elements 0, 2, 4, 6
                const uint32_t hi = (c >> 4) & 0x0F0F0F0Fu;      // elements 1, 3, 5, 7
                uint32_t o[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float e0 = (float)((lo >> (8 * b)) & 0xFFu);
                    const float e1 = (float)((hi >> (8 * b)) & 0xFFu);
                    const bf16x2_t pr = {(__bf16)fmaf(e0, ws, wb), (__bf16)fmaf(e1, ws, wb)};
                    o[b] = __builtin_bit_cast(uint32_t, pr);
                }
                B[gchunk(brow, 4 * bh + d)] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        };
        // Three register buffers: while the consumers work on step s, steps
        // s+3 .. s+5 are in flight from global memory (the producers are
        // latency-bound: every N tile re-reads its X block from L2).
        // prologue: stages 0 and 1 stored, steps 2..4 in registers
        Regs ra, rb, rc;
        gload(ra, 0);
        if (ksteps > 1) gload(rb, 1);
        if (ksteps > 2) gload(rc, 2);
        lstore(ra, 0);
        if (ksteps > 3) gload(ra, 3);
        if (ksteps > 1) lstore(rb, 1);
        if (ksteps > 4) gload(rb, 4);
        __syncthreads();
        // iteration s: store step s+2 (loaded three steps earlier), load step s+5
        for (int s = 0; s < ksteps; s += 3) {
            if (s + 2 < ksteps) lstore(rc, s + 2);
            if (s + 5 < ksteps) gload(rc, s + 5);
            __syncthreads();
            if (s + 1 < ksteps) {
                if (s + 3 < ksteps) lstore(ra, s + 3);
                if (s + 6 < ksteps) gload(ra, s + 6);
                __syncthreads();
            }
            if (s + 2 < ksteps) {
                if (s + 4 < ksteps) lstore(rb, s + 4);
                if (s + 7 < ksteps) gload(rb, s + 7);
                __syncthreads();
            }
        }
        return;
    }

    // ---------------- MFMA consumers: 4 wavefronts, 128 x 64 each
    const int wm = wave >> 1, wn = wave & 1;
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int arow = wm * 128 + (lane & 31), brw = wn * 64 + (lane & 31), half = lane >> 5;
    // Fragments are double-buffered across (step, kk): the reads for the next
    // k slice are in flight while this slice's MFMAs issue. Stage s+1 is already
    // complete during step s (the ring is 3 deep), so the pipeline runs across
    // step boundaries; the barrier only has to follow the last read of stage s.
    bf16x8_t af[2][4], bf[2][2];
    auto frags = [&](int buf, int s, int kk) {
        const uint4* A = gsm + (s % GSTAGES) * STAGE;
        const uint4* B = A + GBM * GCH;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[buf][i] = __builtin_bit_cast(bf16x8_t, A[gchunk(arow + 32 * i, 2 * kk + half)]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            bf[buf][j] = __builtin_bit_cast(bf16x8_t, B[gchunk(brw + 32 * j, 2 * kk + half)]);
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bf[buf][j], acc[i][j], 0, 0, 0);
    };
    // The scheduling barriers keep each fragment read batch ahead of the
    // MFMAs it overlaps; left alone, the scheduler moves the reads in among
    // those MFMAs and waits on them right away.
    __syncthreads();  // prologue stages ready
    frags(0, 0, 0);
    for (int s = 0; s < ksteps; ++s) {
        frags(1, s, 1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(0);
        frags(0, s, 2);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(1);
        frags(1, s, 3);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(0);
        if (s + 1 < ksteps) frags(0, s + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(1);
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
                    const bf16x2_t pr = {(__bf16)acc[i][j][r], (__bf16)0.f};
                    Y[(int64_t)m * N + n] = (uint16_t)__builtin_bit_cast(uint32_t, pr);
                }
            }
        }
}

hipError_t launch_gemm(int scheme, const void* codes, const void* scale, const void* bias,
                       int64_t N, int64_t K, const uint16_t* X, int64_t M, uint16_t* Y,
                       hipStream_t st) {
    const int tm = (int)((M + GBM - 1) / GBM), tn = (int)((N + GBN - 1) / GBN);
    const int per = (tm * tn + 7) / 8;
    const size_t lds = (size_t)GSTAGES * (GBM + GBN) * GCH * 16;
    auto kern = scheme == SYM4_G128 ? gemm_kernel<SYM4_G128> : gemm_kernel<AFF4_G64>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(kern, dim3(8 * per), dim3(512), lds, st, (const uint8_t*)codes,
                       (const uint8_t*)scale, (const uint8_t*)bias, (int)M, (int)N, (int)K, X, Y,
                       tm, tn);
    return hipGetLastError();
}

}  // namespace w4
