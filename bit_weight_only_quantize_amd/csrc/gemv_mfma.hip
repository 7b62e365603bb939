// Launch side of the skinny MFMA decode GEMM (2 <= M <= 16, 4-bit schemes).
#include <algorithm>

#include "gemv_mfma.hpp"
#include "launch.hpp"

namespace w4 {

bool gemv_mfma_ok(int scheme, int64_t K, int64_t M) {
    if (scheme != SYM4_G128 && scheme != AFF4_G64) return false;
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

template <int S>
static void pick_mfma(int RT, int WK, const GemvGroupArgs& a, int blocks, int K, int M,
                      const uint16_t* x, hipStream_t st) {
    if (RT == 2) {
        if (WK == 8) go_mfma<S, 2, 8>(a, blocks, K, M, x, st);
        else if (WK == 4) go_mfma<S, 2, 4>(a, blocks, K, M, x, st);
        else go_mfma<S, 2, 2>(a, blocks, K, M, x, st);
    } else {
        if (WK == 8) go_mfma<S, 1, 8>(a, blocks, K, M, x, st);
        else go_mfma<S, 1, 4>(a, blocks, K, M, x, st);
    }
}

// Activations in LDS (gemv_mfma_lds_kernel): one workgroup per CU holds TP =
// ceil(tiles / CUs) tiles; 16 wavefronts stage x (in as few chunks of steps
// as LDS allows), and TP * WK of them stream codes, each tile's steps split
// over WK of them. Measured on the 7B shapes with the code stream alone:
// about 24 steps (KB) of code loads in flight per CU read fastest, more read
// slower (16 wavefronts x 4 steps on one tile: 1.6 TB/s against 2.4 with 4
// x 4). Launches of more than 16 tiles per CU take the split-K kernel.
template <int S>
static bool try_mfma_lds(int count, const void* const* codes, const void* const* scale,
                         const void* const* bias, const int64_t* N, int64_t K,
                         const uint16_t* x, int64_t M, float* const* y, hipStream_t st) {
    constexpr int kCUs = 256, kWaves = 16;
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
    if (tiles == 0) return false;
    const int TP = (tiles + kCUs - 1) / kCUs;
    if (TP > kWaves) return false;
    const MfmaLdsLayout<S> whole((int)K, (int)M, 1);
    const int steps = whole.steps, GPS = whole.GPS;
    // the staging lanes of one group of all tokens must fit the workgroup
    if (64 * kWaves < whole.mp * (Traits<S>::GROUP / 8)) return false;
    // fewest chunks whose activations, sums and scale blocks fit in LDS; the
    // tile split WK puts about 24 steps of code loads in flight per CU
    int CS = 0, SG = 0, spw = 0, WK = 1;
    size_t lds = 0;
    for (int chunks = 1; chunks <= steps; ++chunks) {
        CS = (steps + chunks - 1) / chunks;
        const int depth = chunks > 1 ? 2 : 4;
        WK = (24 + TP * depth / 2) / (TP * depth);
        WK = std::max(1, std::min({WK, kWaves / TP, CS}));
        // every K-slice of a full chunk non-empty
        while (WK > 1 && (WK - 1) * ((CS + WK - 1) / WK) >= CS) --WK;
        spw = (CS + WK - 1) / WK;
        const int sgmax = std::min(spw * GPS, whole.groups);
        if (sgmax > (chunks > 1 ? 64 : 128)) continue;  // chunked: registers (see below)
        SG = sgmax <= 16 ? 16 : sgmax <= 32 ? 32 : sgmax <= 64 ? 64 : 128;
        lds = MfmaLdsLayout<S>((int)K, (int)M, CS).bytes() + (size_t)TP * WK * 16 * (SG + 1) * 4;
        lds = std::max(lds, WK > 1 ? (size_t)TP * WK * 64 * 16 : (size_t)0);
        if (lds <= kLds) break;
        lds = 0;
    }
    if (lds == 0) return false;
    const int grid = (tiles + TP - 1) / TP;
    auto go = [&](auto kern) {
        if (lds > 64 * 1024)
            (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kWaves), lds, st, a, (int)K, (int)M, x, tiles, TP, WK, CS);
    };
    // four steps in flight (eight read slower, see above); slices under four
    // steps take two. The chunk loop costs the registers of two more steps in
    // flight, so chunked launches keep two.
    auto by_depth = [&](auto sgc) {
        constexpr int G = decltype(sgc)::value;
        if constexpr (G <= 64) {
            if (CS < steps) {
                go(gemv_mfma_lds_kernel<S, 2, G, true>);
                return;
            }
        }
        if (spw >= 4) go(gemv_mfma_lds_kernel<S, 4, G, false>);
        else go(gemv_mfma_lds_kernel<S, 2, G, false>);
    };
    if (SG == 16) by_depth(std::integral_constant<int, 16>{});
    else if (SG == 32) by_depth(std::integral_constant<int, 32>{});
    else if (SG == 64) by_depth(std::integral_constant<int, 64>{});
    else by_depth(std::integral_constant<int, 128>{});
    return true;
}

hipError_t launch_gemv_mfma(int scheme, int count, const void* const* codes,
                            const void* const* scale, const void* const* bias, const int64_t* N,
                            int64_t K, const uint16_t* x, int64_t M, float* const* y,
                            hipStream_t st) {
    if (scheme == SYM4_G128 ? try_mfma_lds<SYM4_G128>(count, codes, scale, bias, N, K, x, M, y, st)
                            : try_mfma_lds<AFF4_G64>(count, codes, scale, bias, N, K, x, M, y, st))
        return hipGetLastError();
    int64_t total_rows = 0;
    for (int i = 0; i < count; ++i) total_rows += N[i];
    // The split-K kernel takes what the LDS kernel does not: more than 16 row
    // tiles per CU (the 13B tied head) and launches too small for one
    // workgroup of staging lanes. Measured on the 7B (sym) and 13B (affine)
    // decode shapes at M = 4, 8, 16: two row tiles per wavefront amortize the
    // activation loads once a launch has many rows (four do not pay); such
    // launches run best with fewer split-K wavefronts (sym 2, affine 4),
    // while eight give the smaller launches enough loads in flight.
    const bool big = scheme == AFF4_G64 || total_rows >= 16384;
    const int RT = big ? 2 : 1;
    const int WK = big ? (scheme == SYM4_G128 ? 2 : 4) : 8;
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
    if (scheme == SYM4_G128) pick_mfma<SYM4_G128>(RT, WK, a, blocks, (int)K, (int)M, x, st);
    else pick_mfma<AFF4_G64>(RT, WK, a, blocks, (int)K, (int)M, x, st);
    return hipGetLastError();
}

}  // namespace w4
