// Decode GEMV / skinny GEMM with the dequantization fused into the product.
//
// airllm article §2.2: dequantize inside the matmul kernel, in registers, right
// after the weights are loaded; §3.3: decode is memory-bound, so the kernel is
// built to stream the packed codes at HBM speed. See skinny.hpp for the
// per-lane arithmetic.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "skinny.hpp"
#include "gemv_wave.hpp"

namespace w4 {

constexpr int kThreads = 256;  // 4 wavefronts per workgroup

template <int S, int MT, int LPR, int V, int R>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scale,
                                                        const uint8_t* __restrict__ bias, int N,
                                                        int K, const uint16_t* __restrict__ x,
                                                        int M, float* __restrict__ y) {
    using T = Traits<S>;
    using Core = SkinnyCore<S, MT, LPR, V, R>;
    extern __shared__ __align__(16) uint32_t smem[];
    constexpr int RSW = 64 / LPR;  // row slots per wavefront
    const int VR = K / T::KV;
    const int xstride = K / 2;
    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + MT * xstride);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane / LPR, sl = lane % LPR;
    const int64_t rowbytes = (int64_t)K * T::BITS / 8;
    const int64_t groups = K / T::GROUP;
    constexpr int SB = T::AFFINE ? 2 : 4;

    Core core;
    core.VR = VR;
    core.sl = sl;
    int n[R];
    const int base = blockIdx.x * (4 * RSW * R) + wave * (RSW * R) + slot;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        n[r] = base + r * RSW;
        const int64_t nl = n[r] < N ? n[r] : N - 1;  // rows past the end re-read the last row
        core.crow[r] = codes + nl * rowbytes;
        core.srow[r] = scale + nl * groups * SB;
        core.brow[r] = T::AFFINE ? bias + nl * groups * 2 : nullptr;
    }
    typename Core::Buf A, B;
    for (int t0 = 0; t0 < M; t0 += MT) {
        const int mt = min(MT, M - t0);
        core.load(A, 0);  // first code vectors in flight while the activations are staged
        if (t0) __syncthreads();
        stage_x<S, MT, V, kThreads>(x + (int64_t)t0 * K, K, nullptr, mt, K, xs, XS);
        __syncthreads();
        float acc[R][MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
        core.run(A, B, xs, XS, xstride, acc);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = group_sum<LPR>(acc[r][m]);
        if (sl == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    if (n[r] < N && m < mt) y[(int64_t)(t0 + m) * N + n[r]] = acc[r][m];
        }
    }
}

static size_t lds_bytes(int scheme, int64_t K, int mt) {
    const int kv = scheme == AFF8_G64 ? 16 : 32;
    return (size_t)mt * (size_t)(K / 2 + K / kv) * 4;
}

GemvPlan plan_gemv(int scheme, int64_t N, int64_t K, int64_t M) {
    const int kv = scheme == AFF8_G64 ? 16 : 32;
    const int vpg = scheme == AFF4_G64 ? 2 : 4;
    const int64_t VR = K / kv;
    GemvPlan best{64, 1, 2, 1, 0, 0};
    double best_score = -1;
    int mt = M >= 4 ? 4 : (M >= 2 ? 2 : 1);
    while (mt > 1 && lds_bytes(scheme, K, mt) > 65536) mt /= 2;
    const int lprs8[] = {64, 16};
    const int lprs4[] = {64, 32, 16, 8};
    const int* lprs = scheme == AFF8_G64 ? lprs8 : lprs4;
    const int nl = scheme == AFF8_G64 ? 2 : 4;
    for (int li = 0; li < nl; ++li) {
        const int lpr = lprs[li];
        for (int v = 2; v >= 1; --v) {
            if (scheme == AFF8_G64 && v != 1) continue;
            if (v > vpg) continue;
            for (int r = 4; r >= 2; r -= 2) {
                if (scheme == AFF8_G64 && r != 2) continue;
                const int64_t rows_wg = 4LL * (64 / lpr) * r;
                const int64_t wgs = (N + rows_wg - 1) / rows_wg;
                const int64_t steps = (VR + lpr * v - 1) / (lpr * v);
                const double lane_eff = (double)VR / (double)(steps * lpr * v);
                const double row_eff = (double)N / (double)(wgs * rows_wg);
                const double fill = wgs >= 512 ? 1.0 : (double)wgs / 512.0;
                const double score = lane_eff * row_eff * fill;
                if (score > best_score + 1e-9) {
                    best_score = score;
                    best = GemvPlan{lpr, v, r, mt, wgs, lds_bytes(scheme, K, mt)};
                }
            }
        }
    }
    return best;
}

template <int S, int MT, int LPR, int V, int R>
static hipError_t go(const GemvPlan& p, const void* codes, const void* scale, const void* bias,
                     int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                     hipStream_t st) {
    hipLaunchKernelGGL((gemv_kernel<S, MT, LPR, V, R>), dim3((unsigned)p.blocks), dim3(kThreads),
                       p.lds, st, (const uint8_t*)codes, (const uint8_t*)scale,
                       (const uint8_t*)bias, (int)N, (int)K, x, (int)M, y);
    return hipGetLastError();
}

template <int S, int MT, int LPR, int V>
static hipError_t pick_r(const GemvPlan& p, const void* c, const void* s, const void* b,
                         int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                         hipStream_t st) {
    if constexpr (S == AFF8_G64) return go<S, MT, LPR, V, 2>(p, c, s, b, N, K, x, M, y, st);
    else if (p.r == 4) return go<S, MT, LPR, V, 4>(p, c, s, b, N, K, x, M, y, st);
    else return go<S, MT, LPR, V, 2>(p, c, s, b, N, K, x, M, y, st);
}

template <int S, int MT, int LPR>
static hipError_t pick_v(const GemvPlan& p, const void* c, const void* s, const void* b,
                         int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                         hipStream_t st) {
    if constexpr (S == AFF8_G64) return pick_r<S, MT, LPR, 1>(p, c, s, b, N, K, x, M, y, st);
    else if (p.v == 2) return pick_r<S, MT, LPR, 2>(p, c, s, b, N, K, x, M, y, st);
    else return pick_r<S, MT, LPR, 1>(p, c, s, b, N, K, x, M, y, st);
}

template <int S, int MT>
static hipError_t pick_lpr(const GemvPlan& p, const void* c, const void* s, const void* b,
                           int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                           hipStream_t st) {
    if constexpr (S == AFF8_G64) {
        if (p.lpr == 64) return pick_v<S, MT, 64>(p, c, s, b, N, K, x, M, y, st);
        return pick_v<S, MT, 16>(p, c, s, b, N, K, x, M, y, st);
    } else {
        switch (p.lpr) {
            case 64: return pick_v<S, MT, 64>(p, c, s, b, N, K, x, M, y, st);
            case 32: return pick_v<S, MT, 32>(p, c, s, b, N, K, x, M, y, st);
            case 16: return pick_v<S, MT, 16>(p, c, s, b, N, K, x, M, y, st);
            default: return pick_v<S, MT, 8>(p, c, s, b, N, K, x, M, y, st);
        }
    }
}

template <int S>
static hipError_t pick_mt(const GemvPlan& p, const void* c, const void* s, const void* b,
                          int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                          hipStream_t st) {
    switch (p.mt) {
        case 4: return pick_lpr<S, 4>(p, c, s, b, N, K, x, M, y, st);
        case 2: return pick_lpr<S, 2>(p, c, s, b, N, K, x, M, y, st);
        default: return pick_lpr<S, 1>(p, c, s, b, N, K, x, M, y, st);
    }
}

// ---------------------------------------------------------------- M = 1, wave per row
// Instantiated code-vector counts per lane (ceil(VR / 64) rounded up to one of these).
// 16-byte code vectors per lane for rows of VR vectors; 0 if too many. The
// one-token kernel also takes 11 and 14 per lane (rows of up to 896 vectors:
// the 8-bit scheme at K = 11008 or 13824, the 4-bit ones up to K = 28672),
// the multi-token kernel, which keeps more per lane, at most 8.
static int wave_nv(int64_t VR, bool one_token = false) {
    const int64_t need = (VR + 63) / 64;
    const int nvs[] = {1, 2, 3, 4, 6, 7, 8, 11, 14};
    for (int nv : nvs)
        if (nv >= need && (nv <= 8 || one_token)) return nv;
    return 0;
}

bool gemv_wave_ok(int scheme, int64_t K) {
    const int kv = scheme == AFF8_G64 ? 16 : 32;
    const int64_t VR = K / kv;
    return VR >= 64 && wave_nv(VR, true) > 0;
}

// Row wavefronts stage the activations themselves (no staging wavefronts): a
// workgroup is RW row wavefronts, each issuing its share of the activation
// loads before its weight loads.
template <int S, int NV, int R, int RW>
static void go_wave(const GemvGroupArgs& a, int blocks, int K, const uint16_t* x, size_t lds,
                    hipStream_t st) {
    constexpr int XV = (NV + RW - 1) / RW;  // activation vectors per lane
    hipLaunchKernelGGL((gemv_wave_kernel<S, NV, R, XV, RW>), dim3(blocks), dim3(64 * RW), lds, st,
                       a, K, x);
}

template <int S, int R, int RW>
static void pick_nv(int nv, const GemvGroupArgs& a, int blocks, int K, const uint16_t* x,
                    size_t lds, hipStream_t st) {
    switch (nv) {
        case 1: go_wave<S, 1, R, RW>(a, blocks, K, x, lds, st); break;
        case 2: go_wave<S, 2, R, RW>(a, blocks, K, x, lds, st); break;
        case 3: go_wave<S, 3, R, RW>(a, blocks, K, x, lds, st); break;
        case 4: go_wave<S, 4, R, RW>(a, blocks, K, x, lds, st); break;
        case 6: go_wave<S, 6, R, RW>(a, blocks, K, x, lds, st); break;
        case 7: go_wave<S, 7, R, RW>(a, blocks, K, x, lds, st); break;
        case 8: go_wave<S, 8, R, RW>(a, blocks, K, x, lds, st); break;
        default:  // 11 or 14: one row per wavefront only (two take nv <= 4)
            if constexpr (R == 1) {
                if (nv == 11) go_wave<S, 11, R, RW>(a, blocks, K, x, lds, st);
                else go_wave<S, 14, R, RW>(a, blocks, K, x, lds, st);
            }
            break;
    }
}

template <int S>
static void pick_shape(int R, int RW, int nv, const GemvGroupArgs& a, int blocks, int K,
                       const uint16_t* x, size_t lds, hipStream_t st) {
    if (R == 2 && RW == 4) pick_nv<S, 2, 4>(nv, a, blocks, K, x, lds, st);
    else if (R == 2) pick_nv<S, 2, 8>(nv, a, blocks, K, x, lds, st);
    else if (RW == 4) pick_nv<S, 1, 4>(nv, a, blocks, K, x, lds, st);
    else pick_nv<S, 1, 8>(nv, a, blocks, K, x, lds, st);
}

hipError_t launch_gemv_wave(int scheme, int count, const void* const* codes,
                            const void* const* scale, const void* const* bias, const int64_t* N,
                            int64_t K, const uint16_t* x, float* const* y, hipStream_t st) {
    const int kv = scheme == AFF8_G64 ? 16 : 32;
    const int64_t VR = K / kv;
    const int nv = wave_nv(VR, true);
    int64_t total_rows = 0;
    for (int i = 0; i < count; ++i) total_rows += N[i];
    // Measured on the decode shapes: two rows per wavefront pay off once a
    // launch has enough rows to fill every CU several times over and rows are
    // short; otherwise one. Small launches keep 4-wavefront workgroups so that
    // more CUs get work.
    const int R = (total_rows >= 12288 && nv <= 4) ? 2 : 1;
    const int RW = ((R == 2 && nv <= 2) || total_rows < 4096) ? 4 : 8;
    GemvGroupArgs a{};
    int blocks = 0;
    for (int i = 0; i < count; ++i) {
        a.codes[i] = (const uint8_t*)codes[i];
        a.scale[i] = (const uint8_t*)scale[i];
        a.bias[i] = (const uint8_t*)bias[i];
        a.y[i] = y[i];
        a.N[i] = (int)N[i];
        a.tile_start[i] = blocks;
        blocks += (int)((N[i] + RW * R - 1) / (RW * R));
    }
    a.tile_start[count] = blocks;
    a.count = count;
    if (blocks == 0) return hipSuccess;
    const size_t lds = (size_t)(K / 2 + VR) * 4;
    switch (scheme) {
        case SYM4_G128: pick_shape<SYM4_G128>(R, RW, nv, a, blocks, (int)K, x, lds, st); break;
        case AFF4_G64: pick_shape<AFF4_G64>(R, RW, nv, a, blocks, (int)K, x, lds, st); break;
        default: pick_shape<AFF8_G64>(R, RW, nv, a, blocks, (int)K, x, lds, st); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- 2 <= M <= 64, wave per row
constexpr size_t kMaxLds = 160 * 1024;

template <typename Kern>
static void allow_lds(Kern k, size_t bytes) {
    if (bytes > 64 * 1024)
        (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)kMaxLds);
}

// Token tile: as many tokens as the LDS double buffer and the staging
// wavefronts' registers (MT x XV activation vectors in flight) allow.
static int mt_tile(int64_t M, int64_t K, int kv, int nv) {
    int mt = M <= 2 ? 2 : (M <= 4 ? 4 : 8);
    const int xv = (nv + 1) / 2;
    while (mt > 2 && (mt * xv > 8 || (size_t)2 * mt * (K / 2 + K / kv) * 4 > kMaxLds)) mt /= 2;
    return mt;
}

bool gemv_wave_mt_ok(int scheme, int64_t K, int64_t M) {
    const int kv = scheme == AFF8_G64 ? 16 : 32;
    const int64_t VR = K / kv;
    if (M < 2 || M > 64 || VR < 64 || wave_nv(VR) == 0) return false;
    if (scheme == AFF8_G64 && wave_nv(VR) > 2) return false;
    return (size_t)2 * 2 * (K / 2 + VR) * 4 <= kMaxLds;
}

template <int S, int NV, int MT>
static void go_mt(const GemvGroupArgs& a, int blocks, int K, int M, const uint16_t* x, size_t lds,
                  hipStream_t st) {
    constexpr int R = NV <= 3 ? 2 : 1;
    constexpr int SW = 2, XV = (NV + 1) / 2;
    auto kern = gemv_wave_mt_kernel<S, NV, R, MT, XV, SW>;
    allow_lds(kern, lds);
    // few row blocks (a router: 128 rows in 16 blocks): split the token tiles
    // over workgroups too, up to about two workgroups per CU
    const int ttiles = (M + MT - 1) / MT;
    const int ts = std::max(1, std::min(ttiles, 512 / std::max(blocks, 1)));
    const int tpw = MT * ((ttiles + ts - 1) / ts);
    const int gy = (M + tpw - 1) / tpw;
    hipLaunchKernelGGL(kern, dim3(blocks, gy), dim3(256 + 64 * SW), lds, st, a, K, M, x, tpw);
}

template <int S, int NV>
static void pick_mt_tile(int mt, const GemvGroupArgs& a, int blocks, int K, int M,
                         const uint16_t* x, size_t lds, hipStream_t st) {
    constexpr int XV = (NV + 1) / 2;
    if constexpr (8 * XV <= 8)
        if (mt == 8) return go_mt<S, NV, 8>(a, blocks, K, M, x, lds, st);
    if constexpr (4 * XV <= 8)
        if (mt >= 4) return go_mt<S, NV, 4>(a, blocks, K, M, x, lds, st);
    go_mt<S, NV, 2>(a, blocks, K, M, x, lds, st);
}

template <int S>
static void pick_nv_mt(int nv, int mt, const GemvGroupArgs& a, int blocks, int K, int M,
                       const uint16_t* x, size_t lds, hipStream_t st) {
    if constexpr (S == AFF8_G64) {
        if (nv == 1) pick_mt_tile<S, 1>(mt, a, blocks, K, M, x, lds, st);
        else pick_mt_tile<S, 2>(mt, a, blocks, K, M, x, lds, st);
    } else {
        switch (nv) {
            case 1: pick_mt_tile<S, 1>(mt, a, blocks, K, M, x, lds, st); break;
            case 2: pick_mt_tile<S, 2>(mt, a, blocks, K, M, x, lds, st); break;
            case 3: pick_mt_tile<S, 3>(mt, a, blocks, K, M, x, lds, st); break;
            case 4: pick_mt_tile<S, 4>(mt, a, blocks, K, M, x, lds, st); break;
            case 6: pick_mt_tile<S, 6>(mt, a, blocks, K, M, x, lds, st); break;
            case 7: pick_mt_tile<S, 7>(mt, a, blocks, K, M, x, lds, st); break;
            default: pick_mt_tile<S, 8>(mt, a, blocks, K, M, x, lds, st); break;
        }
    }
}

hipError_t launch_gemv_wave_mt(int scheme, int count, const void* const* codes,
                               const void* const* scale, const void* const* bias, const int64_t* N,
                               int64_t K, const uint16_t* x, int64_t M, float* const* y,
                               hipStream_t st) {
    const int kv = scheme == AFF8_G64 ? 16 : 32;
    const int64_t VR = K / kv;
    const int nv = wave_nv(VR);
    const int R = nv <= 3 ? 2 : 1;
    const int mt = mt_tile(M, K, kv, nv);
    GemvGroupArgs a{};
    int blocks = 0;
    for (int i = 0; i < count; ++i) {
        a.codes[i] = (const uint8_t*)codes[i];
        a.scale[i] = (const uint8_t*)scale[i];
        a.bias[i] = (const uint8_t*)bias[i];
        a.y[i] = y[i];
        a.N[i] = (int)N[i];
        a.tile_start[i] = blocks;
        blocks += (int)((N[i] + 4 * R - 1) / (4 * R));
    }
    a.tile_start[count] = blocks;
    a.count = count;
    if (blocks == 0) return hipSuccess;
    const size_t lds = (size_t)2 * mt * (K / 2 + VR) * 4;
    switch (scheme) {
        case SYM4_G128: pick_nv_mt<SYM4_G128>(nv, mt, a, blocks, (int)K, (int)M, x, lds, st); break;
        case AFF4_G64: pick_nv_mt<AFF4_G64>(nv, mt, a, blocks, (int)K, (int)M, x, lds, st); break;
        default: pick_nv_mt<AFF8_G64>(nv, mt, a, blocks, (int)K, (int)M, x, lds, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_gemv(int scheme, const void* codes, const void* scale, const void* bias,
                       int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                       hipStream_t st) {
    if (M == 1 && gemv_wave_ok(scheme, K))
        return launch_gemv_wave(scheme, 1, &codes, &scale, &bias, &N, K, x, &y, st);
    if (gemv_mfma_ok(scheme, K, M)) {
        const hipError_t e = launch_gemv_mfma(scheme, 1, &codes, &scale, &bias, &N, K, x, M, &y, st);
        if (e != hipErrorNotSupported) return e;  // else nothing was launched
    }
    if (gemv_wave_mt_ok(scheme, K, M))
        return launch_gemv_wave_mt(scheme, 1, &codes, &scale, &bias, &N, K, x, M, &y, st);
    const GemvPlan p = plan_gemv(scheme, N, K, M);
    switch (scheme) {
        case SYM4_G128: return pick_mt<SYM4_G128>(p, codes, scale, bias, N, K, x, M, y, st);
        case AFF4_G64: return pick_mt<AFF4_G64>(p, codes, scale, bias, N, K, x, M, y, st);
        default: return pick_mt<AFF8_G64>(p, codes, scale, bias, N, K, x, M, y, st);
    }
}

}  // namespace w4
