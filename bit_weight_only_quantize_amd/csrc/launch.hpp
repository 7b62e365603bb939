// Host-side launchers shared between the translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

hipError_t launch_quantize_pack(int scheme, const float* W, int64_t N, int64_t K, void* codes,
                                void* scale, void* bias, hipStream_t st);

// Largest K the skinny kernels can stage in LDS for one token.
constexpr int64_t kMaxSkinnyK = 28672;

struct GemvPlan {
    int lpr, v, r, mt;
    int64_t blocks;
    size_t lds;
};
GemvPlan plan_gemv(int scheme, int64_t N, int64_t K, int64_t M);

// M = 1, one wavefront per row, up to 4 matrices sharing x in one launch.
bool gemv_wave_ok(int scheme, int64_t K);
hipError_t launch_gemv_wave(int scheme, int count, const void* const* codes,
                            const void* const* scale, const void* const* bias, const int64_t* N,
                            int64_t K, const uint16_t* x, float* const* y, hipStream_t st);

hipError_t launch_gemv(int scheme, const void* codes, const void* scale, const void* bias,
                       int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                       hipStream_t st);

}  // namespace w4
