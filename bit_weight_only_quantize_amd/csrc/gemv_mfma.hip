// Launch side of the skinny MFMA decode GEMM (2 <= M <= 16, 4-bit schemes).
#include <algorithm>

#include "gemv_mfma.hpp"
#include "launch.hpp"

namespace w4 {

// y[i] = sum of the KP partial outputs part[p][i], p = 0 .. KP-1 in order
// (all loads issued first; KP <= 8)
__global__ __launch_bounds__(256) void ksplit_sum_kernel(const float* __restrict__ part, int KP,
                                                         int64_t MN, float* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MN) return;
    float v[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) v[p] = part[(int64_t)min(p, KP - 1) * MN + i];
    float s = v[0];
#pragma unroll
    for (int p = 1; p < 8; ++p) s = p < KP ? s + v[p] : s;
    y[i] = s;
}

bool gemv_mfma_ok(int scheme, int64_t K, int64_t M) {
    if (scheme != SYM4_G128 && scheme != AFF4_G64 && scheme != AFF8_G64) return false;
    const int group = scheme == SYM4_G128 ? 128 : 64;
    return M >= 2 && M <= 16 && K >= group && K / group <= kMfmaMaxGroups;
}

template <int S, int RT, int WK>
static void go_mfma(const GemvGroupArgs& a, int blocks, int K, int M, const uint16_t* x,
                    hipStream_t st) {
    const size_t lds = gemv_mfma_lds_bytes<S, RT, WK>(K);
    switch (mfma_slices(K / Traits<S>::GROUP)) {
        case 1: hipLaunchKernelGGL((gemv_mfma_kernel<S, RT, WK, 2, 1>), dim3(blocks), dim3(64 * WK), lds, st, a, K, M, x); break;
        case 2: hipLaunchKernelGGL((gemv_mfma_kernel<S, RT, WK, 2, 2>), dim3(blocks), dim3(64 * WK), lds, st, a, K, M, x); break;
        default: hipLaunchKernelGGL((gemv_mfma_kernel<S, RT, WK, 2, 4>), dim3(blocks), dim3(64 * WK), lds, st, a, K, M, x); break;
    }
}

// Activations in LDS (gemv_mfma_lds_kernel): one workgroup per CU holds TP =
// ceil(tiles / CUs) tiles; 16 wavefronts stage x (in as few chunks of steps
// as LDS allows), and TP * WK of them stream codes, each tile's steps split
// over WK of them. Measured on the 7B shapes with the code stream alone:
// about 24 steps (KB) of code loads in flight per CU read fastest, more read
// slower (16 wavefronts x 4 steps on one tile: 1.6 TB/s against 2.4 with 4
// x 4). Launches of more than 16 tiles per CU take the split-K kernel.
struct LdsPlan {
    int KP = 1, TP = 0, WK = 1, CS = 0, SG = 16, spw = 0, grid = 0;
    bool chunked = false;
    size_t lds = 0;
};

// gated: tiles come in (gate, up) pairs that one workgroup must hold together,
// so TP is even and x must fit in one pass (no chunks, no K parts)
template <int S>
static bool plan_mfma_lds(int tiles, int64_t K, int64_t M, bool split, LdsPlan& P,
                          bool gated = false) {
    constexpr int kCUs = 256, kWaves = 16;
    constexpr size_t kLds = 160 * 1024;
    if (tiles == 0) return false;
    const MfmaLdsLayout<S> whole((int)K, (int)M, 1);
    const int steps = whole.steps, GPS = whole.GPS;
    // the staging lanes of one group of all tokens must fit the workgroup
    if (64 * kWaves < whole.mp * (Traits<S>::GROUP / 8)) return false;
    // a run of CS steps on TP tiles per workgroup: the K-slice split WK puts
    // about 24 steps of code loads in flight per CU; returns the LDS bytes
    // (activations, sums and scale blocks), 0 if they do not fit
    int TP1 = (tiles + kCUs - 1) / kCUs;
    // the K-slice split follows the tiles per CU before a gated plan rounds
    // TP up to even, so that gated and plain launches sum in the same order
    const int tp_wk = TP1;
    auto fit = [&](LdsPlan& q) -> size_t {
        const int depth = q.chunked ? 2 : 4;
        const int tpw = gated ? tp_wk : q.TP;
        int WK = (24 + tpw * depth / 2) / (tpw * depth);
        WK = std::max(1, std::min({WK, kWaves / q.TP, q.CS}));
        // every K-slice of a full run non-empty
        while (WK > 1 && (WK - 1) * ((q.CS + WK - 1) / WK) >= q.CS) --WK;
        q.WK = WK;
        q.spw = (q.CS + WK - 1) / WK;
        const int sgmax = std::min(q.spw * GPS, whole.groups);
        if (sgmax > (q.chunked ? 64 : 128)) return 0;  // chunked: registers (see below)
        q.SG = sgmax <= 16 ? 16 : sgmax <= 32 ? 32 : sgmax <= 64 ? 64 : 128;
        size_t lds = MfmaLdsLayout<S>((int)K, (int)M, q.CS).bytes() + (size_t)q.TP * WK * 16 * (q.SG + 1) * 4;
        lds = std::max(lds, WK > 1 ? (size_t)q.TP * WK * 64 * 16 : (size_t)0);
        if (gated) lds = std::max(lds, (size_t)q.TP * 64 * 16);  // the pairs' hand-over
        return lds <= kLds ? lds : 0;
    };
    // an odd TP would have to grow by one: fewer workgroups than CUs for the
    // same rows measured slower than the plain launch plus the activation
    // (13B gate/up at M = 8: 7 -> 8 tiles per workgroup); one tile per CU
    // becomes two on half the CUs
    if (gated && (TP1 & 1)) {
        if (TP1 > 1) return false;
        TP1 = 2;
    }
    if (TP1 > kWaves) return false;
    LdsPlan q;
    q.TP = TP1;
    q.CS = steps;
    if ((q.lds = fit(q))) {
        q.grid = (tiles + TP1 - 1) / TP1;
        P = q;
        return true;
    }
    if (gated) return false;
    // x does not fit. With room for partial outputs: K parts on different
    // CUs, each part's x one chunk; the plan with the fewest code steps per
    // CU (TP x part steps), the fewest parts on a tie, all in one round of
    // workgroups
    if (split) {
        LdsPlan best;
        for (int KP = 2; KP <= 8; ++KP) {
            LdsPlan c;
            c.KP = KP;
            c.CS = (steps + KP - 1) / KP;
            if ((KP - 1) * c.CS >= steps) continue;  // an empty last part
            c.TP = (tiles + kCUs / KP - 1) / (kCUs / KP);
            if (c.TP > kWaves) continue;
            if (!(c.lds = fit(c))) continue;
            c.grid = KP * ((tiles + c.TP - 1) / c.TP);
            if (best.KP == 1 || c.TP * c.CS < best.TP * best.CS) best = c;
        }
        if (best.KP > 1) {
            P = best;
            return true;
        }
    }
    // else the fewest chunks whose activations, sums and scale blocks fit
    q.chunked = true;
    for (int chunks = 2; chunks <= steps; ++chunks) {
        q.CS = (steps + chunks - 1) / chunks;
        if ((q.lds = fit(q))) {
            q.grid = (tiles + TP1 - 1) / TP1;
            P = q;
            return true;
        }
    }
    return false;
}

template <int S>
static bool try_mfma_gated(const void* const* codes, const void* const* scale,
                           const void* const* bias, int64_t N, int64_t K, const uint16_t* x,
                           int64_t M, uint16_t* h, hipStream_t st) {
    constexpr size_t kLds = 160 * 1024;
    GemvGroupArgs a{};
    for (int i = 0; i < 2; ++i) {
        a.codes[i] = (const uint8_t*)codes[i];
        a.scale[i] = (const uint8_t*)scale[i];
        a.bias[i] = (const uint8_t*)bias[i];
        a.N[i] = (int)N;
    }
    a.count = 2;
    a.h = h;
    const int tiles = 2 * (int)((N + 15) / 16);
    LdsPlan P;
    if (!plan_mfma_lds<S>(tiles, K, M, false, P, true)) return false;
    auto go = [&](auto kern) {
        if (P.lds > 64 * 1024)
            (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
        hipLaunchKernelGGL(kern, dim3(P.grid), dim3(1024), P.lds, st, a, (int)K, (int)M, x, tiles,
                           P.TP, P.WK, P.CS, P.KP, (float*)nullptr);
    };
    // the same depth / staging choices as the plain launch below
    auto by_depth = [&](auto sgc) {
        constexpr int G = decltype(sgc)::value;
        if constexpr (G <= 32 && S != AFF4_G64) {
            if (M >= 12) {
                if (P.spw >= 4) go(gemv_mfma_lds_kernel<S, 4, G, false, false, 8, true>);
                else go(gemv_mfma_lds_kernel<S, 2, G, false, false, 8, true>);
                return;
            }
        }
        // (the affine 4-bit variant with 128-group scale blocks takes two steps
        // in flight: with four, the pairs' hand-over spills a register)
        if constexpr (!(S == AFF4_G64 && G == 128)) {
            if (P.spw >= 4) {
                go(gemv_mfma_lds_kernel<S, 4, G, false, false, 4, true>);
                return;
            }
        }
        go(gemv_mfma_lds_kernel<S, 2, G, false, false, 4, true>);
    };
    if (P.SG == 16) by_depth(std::integral_constant<int, 16>{});
    else if (P.SG == 32) by_depth(std::integral_constant<int, 32>{});
    else if (P.SG == 64) by_depth(std::integral_constant<int, 64>{});
    else by_depth(std::integral_constant<int, 128>{});
    return true;
}

hipError_t launch_gemv_mfma_gated(int scheme, const void* const* gate, const void* const* up,
                                  int64_t N, int64_t K, const uint16_t* x, int64_t M, uint16_t* h,
                                  hipStream_t st) {
    if (!gemv_mfma_ok(scheme, K, M) || N <= 0) return hipErrorNotSupported;
    const void* c[2] = {gate[0], up[0]};
    const void* s[2] = {gate[1], up[1]};
    const void* b[2] = {gate[2], up[2]};
    const bool ok = scheme == SYM4_G128  ? try_mfma_gated<SYM4_G128>(c, s, b, N, K, x, M, h, st)
                    : scheme == AFF4_G64 ? try_mfma_gated<AFF4_G64>(c, s, b, N, K, x, M, h, st)
                                         : try_mfma_gated<AFF8_G64>(c, s, b, N, K, x, M, h, st);
    return ok ? hipGetLastError() : hipErrorNotSupported;
}

template <int S>
static bool try_mfma_lds(int count, const void* const* codes, const void* const* scale,
                         const void* const* bias, const int64_t* N, int64_t K,
                         const uint16_t* x, int64_t M, float* const* y, float* part,
                         hipStream_t st) {
    constexpr size_t kLds = 160 * 1024;
    GemvGroupArgs a{};
    int tiles = 0;
    for (int i = 0; i < count; ++i) {
        a.codes[i] = (const uint8_t*)codes[i];
        a.scale[i] = (const uint8_t*)scale[i];
        a.bias[i] = (const uint8_t*)bias[i];
        a.y[i] = y[i];
        a.N[i] = (int)N[i];
        a.tile_start[i] = tiles;
        tiles += (int)((N[i] + 15) / 16);
    }
    a.tile_start[count] = tiles;
    a.count = count;
    LdsPlan P;
    if (!plan_mfma_lds<S>(tiles, K, M, part != nullptr && count == 1, P)) return false;
    auto go = [&](auto kern) {
        if (P.lds > 64 * 1024)
            (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
        hipLaunchKernelGGL(kern, dim3(P.grid), dim3(1024), P.lds, st, a, (int)K, (int)M, x, tiles,
                           P.TP, P.WK, P.CS, P.KP, part);
    };
    // four steps in flight (eight read slower, see above); slices under four
    // steps take two. The chunk loop costs the registers of two more steps in
    // flight, so chunked launches keep two.
    auto by_depth = [&](auto sgc) {
        constexpr int G = decltype(sgc)::value;
        if constexpr (G <= 64) {
            if (P.chunked) {
                go(gemv_mfma_lds_kernel<S, 2, G, true>);
                return;
            }
        }
        // 12 or more tokens: 8 staging loads in flight per lane (the 7B stack
        // at M = 16: +3.6%; at M = 4 it cost 2%). The registers only allow it
        // with scale blocks of up to 32 groups and without the affine 4-bit
        // regrouping (those variants spill)
        if constexpr (G <= 32 && S != AFF4_G64) {
            if (M >= 12) {
                if (P.KP > 1) {
                    if (P.spw >= 4) go(gemv_mfma_lds_kernel<S, 4, G, false, true, 8>);
                    else go(gemv_mfma_lds_kernel<S, 2, G, false, true, 8>);
                } else {
                    if (P.spw >= 4) go(gemv_mfma_lds_kernel<S, 4, G, false, false, 8>);
                    else go(gemv_mfma_lds_kernel<S, 2, G, false, false, 8>);
                }
                return;
            }
        }
        if (P.KP > 1) {
            if (P.spw >= 4) go(gemv_mfma_lds_kernel<S, 4, G, false, true>);
            else go(gemv_mfma_lds_kernel<S, 2, G, false, true>);
        } else {
            if (P.spw >= 4) go(gemv_mfma_lds_kernel<S, 4, G, false>);
            else go(gemv_mfma_lds_kernel<S, 2, G, false>);
        }
    };
    if (P.SG == 16) by_depth(std::integral_constant<int, 16>{});
    else if (P.SG == 32) by_depth(std::integral_constant<int, 32>{});
    else if (P.SG == 64) by_depth(std::integral_constant<int, 64>{});
    else by_depth(std::integral_constant<int, 128>{});
    if (P.KP > 1) {
        const int64_t MN = M * N[0];
        hipLaunchKernelGGL(ksplit_sum_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st,
                           (const float*)part, P.KP, MN, y[0]);
    }
    return true;
}

size_t gemv_mfma_split_bytes(int scheme, int64_t N, int64_t K, int64_t M) {
    if (!gemv_mfma_ok(scheme, K, M) || N <= 0) return 0;
    const int tiles = (int)((N + 15) / 16);
    LdsPlan P;
    const bool ok = scheme == SYM4_G128  ? plan_mfma_lds<SYM4_G128>(tiles, K, M, true, P)
                    : scheme == AFF4_G64 ? plan_mfma_lds<AFF4_G64>(tiles, K, M, true, P)
                                         : plan_mfma_lds<AFF8_G64>(tiles, K, M, true, P);
    return ok && P.KP > 1 ? (size_t)P.KP * (size_t)(M * N) * sizeof(float) : 0;
}

hipError_t launch_gemv_mfma(int scheme, int count, const void* const* codes,
                            const void* const* scale, const void* const* bias, const int64_t* N,
                            int64_t K, const uint16_t* x, int64_t M, float* const* y,
                            hipStream_t st, float* part) {
    if (scheme == AFF8_G64) {
        // 8-bit codes: the LDS kernel only (the split-K kernel has no 8-bit
        // step); NotSupported sends the caller to the VALU paths
        if (try_mfma_lds<AFF8_G64>(count, codes, scale, bias, N, K, x, M, y, part, st))
            return hipGetLastError();
        return hipErrorNotSupported;
    }
    if (scheme == SYM4_G128 ? try_mfma_lds<SYM4_G128>(count, codes, scale, bias, N, K, x, M, y, part, st)
                            : try_mfma_lds<AFF4_G64>(count, codes, scale, bias, N, K, x, M, y, part, st))
        return hipGetLastError();
    // The split-K kernel takes what the LDS kernel does not: more than 16 row
    // tiles per CU, i.e. more than 65536 rows (the 13B tied head). Measured on
    // the 13B head and the 7B/13B decode shapes at M = 4, 8, 16: two row tiles
    // per wavefront amortize the activation loads over that many rows (four do
    // not pay), with two split-K wavefronts for sym and four for affine.
    constexpr int RT = 2;
    GemvGroupArgs a{};
    int blocks = 0;
    for (int i = 0; i < count; ++i) {
        a.codes[i] = (const uint8_t*)codes[i];
        a.scale[i] = (const uint8_t*)scale[i];
        a.bias[i] = (const uint8_t*)bias[i];
        a.y[i] = y[i];
        a.N[i] = (int)N[i];
        a.tile_start[i] = blocks;
        blocks += (int)((N[i] + 16 * RT - 1) / (16 * RT));
    }
    a.tile_start[count] = blocks;
    a.count = count;
    if (blocks == 0) return hipSuccess;
    if (scheme == SYM4_G128) go_mfma<SYM4_G128, RT, 2>(a, blocks, (int)K, (int)M, x, st);
    else go_mfma<AFF4_G64, RT, 4>(a, blocks, (int)K, (int)M, x, st);
    return hipGetLastError();
}

}  // namespace w4
