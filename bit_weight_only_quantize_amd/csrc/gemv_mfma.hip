// Launch side of the skinny MFMA decode GEMM (2 <= M <= 16, 4-bit schemes).
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

hipError_t launch_gemv_mfma(int scheme, int count, const void* const* codes,
                            const void* const* scale, const void* const* bias, const int64_t* N,
                            int64_t K, const uint16_t* x, int64_t M, float* const* y,
                            hipStream_t st) {
    int64_t total_rows = 0;
    for (int i = 0; i < count; ++i) total_rows += N[i];
    // Measured on the 7B (sym) and 13B (affine) decode shapes at M = 4, 8, 16:
    // two row tiles per wavefront amortize the activation loads once a launch
    // has many rows (four do not pay); such launches run best with fewer
    // split-K wavefronts (sym 2, affine 4), while eight give the smaller
    // launches enough loads in flight.
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
