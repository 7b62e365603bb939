// Dense gated FFN for one token in a single launch: gate and up projections,
// h = bf16(gelu_tanh(g) * u), then the down projection y = W_down h.
//
// airllm article §3.1: fusing the layer's kernels into fewer launches is where
// its decode latency came from; TurboFieldfare article (M2 time table): 55.6 of
// 162.8 ms per token went to command-buffer waits. On MI355X a launch of a
// decode projection pays a fill and drain of ~1-1.5 us (a 48 MB streaming read
// reaches 5.6-5.9 TB/s, a 1 GiB one 7.1 TB/s). The weights of the down
// projection do not depend on h, only the activations do, so here the down
// rows' code loads go out before h is complete and the whole FFN streams as
// one launch.
//
// Work is an ordered list of items walked by a persistent grid no larger than
// what the GPU holds at once (occupancy API x CUs); workgroup b takes items b,
// b + gridDim.x, ... in increasing order:
//   [gate/up items] [down items]
//   gate/up item  RW*R (gate, up) row pairs, wave-per-row GEMV (activations
//                 staged in LDS by every wavefront): h stored as bf16 pairs
//                 in kHRep copies (device-scope stores), then a split count of
//                 finished items whose completion raises a replicated "every h
//                 row in" flag
//   down item     RW*RD output rows: issues its row loads, waits for the flag,
//                 stages h (device-scope loads of its copy) in LDS, reduces
//                 y[n] in registers
// A down item only waits for gate/up items, which come first in the list;
// with every workgroup resident each wait ends. Waits are also bounded (a poll
// limit the host sets): a workgroup that gives up records it in the error word,
// leaves its rows of y unwritten and carries on, so the kernel always exits.
// The last workgroup out resets the hand-off words and copies the error word
// to the status word.
#include <algorithm>

#include "common.hpp"
#include "gemv_wave.hpp"
#include "handoff.hpp"
#include "launch.hpp"
#include "skinny.hpp"

namespace w4 {

struct FfnArgs {
    const uint8_t *gc, *gs, *gb;  // gate codes, scales, biases [F][D]
    const uint8_t *uc, *us, *ub;  // up [F][D]
    const uint8_t *dc, *ds, *db;  // down [D][F]
    const uint16_t* x;            // [D] bf16
    uint16_t* hc;                 // [kHRep][F] bf16 hand-off copies (workspace)
    uint16_t* h;                  // [F] bf16 out, or null
    float* y;                     // [D] out
    unsigned* sync;               // kLayerSyncWords words (workspace)
    int D, F, n_gu, n_down;
    long long wait_limit;
    int withhold;                 // testing: never raise the "every h row in" flag
};

constexpr int kFfnRW = 4;  // wavefronts per workgroup
constexpr int kFfnThreads = 64 * kFfnRW;
constexpr int kFfnRD = 2;  // down rows per wavefront
// (gate, up) row pairs per wavefront: four (one 8-byte store of h per copy)
// while the row is at most 128 code vectors, else two (registers)
template <int NVG>
constexpr int ffn_pairs() { return NVG <= 2 ? 4 : 2; }

template <int S>
__device__ __forceinline__ void ffn_scale(const uint8_t* s, const uint8_t* b, int g, float& sc,
                                          float& bi) {
    if constexpr (Traits<S>::AFFINE) {
        sc = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(s)[g]);
        bi = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(b)[g]);
    } else {
        sc = reinterpret_cast<const float*>(s)[g];
        bi = 0.f;
    }
}

// ---------------------------------------------------------------- gate/up item
// R (gate, up) row pairs per wavefront. HANDOFF: h goes to the kHRep copies
// (device-scope stores) and the item counts itself; else h goes to a.h only.
// XV: activation vectors staged per thread (the row's D / KV vectors <= 256 XV).
template <int S, int NV, int R, bool HANDOFF, int XV = 1>
__device__ void ffn_gate_up_item(const FfnArgs& a, int item, uint32_t* smem, int* sflag) {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    constexpr int SB = T::AFFINE ? 2 : 4;
    const int tid = item_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int D = a.D, F = a.F, VR = D / T::KV;
    const int64_t rowbytes = (int64_t)D * T::BITS / 8, groups = D / T::GROUP;
    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + D / 2);
    XStage<S, XV, kFfnThreads> xstage;
    xstage.fetch(a.x, VR, tid);
    asm volatile("" ::: "memory");  // the weight loads go out behind the activations
    const int row0 = item * (kFfnRW * R) + wave * R;
    u32x4_t c[2 * R][NV];
    float sc[2 * R][NV], bi[2 * R][NV];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = min(row0 + r, F - 1);
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) {
            const u32x4_t* cp = reinterpret_cast<const u32x4_t*>((gu ? a.uc : a.gc) + n * rowbytes);
            const uint8_t* sp = (gu ? a.us : a.gs) + n * groups * SB;
            const uint8_t* bp = T::AFFINE ? (gu ? a.ub : a.gb) + n * groups * 2 : nullptr;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int v = min(lane + 64 * j, VR - 1);
                c[2 * r + gu][j] = __builtin_nontemporal_load(cp + v);
                ffn_scale<S>(sp, bp, v / T::VPG, sc[2 * r + gu][j], bi[2 * r + gu][j]);
            }
        }
    }
    xstage.commit(VR, xs, XS, tid);  // waits for the activations only
    __syncthreads();
    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    float acc[2 * R] = {};
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int v = lane + 64 * j;
        if (v >= VR) break;
        uint32_t xp[L::XW];
        read_pairs<S>(xs, v, xp);
        const float X = XS[v];
#pragma unroll
        for (int q = 0; q < 2 * R; ++q)
            acc[q] = apply_group<S>(acc[q], dot_code_vector<S>(c[q][j], xp, MASK, MAGIC), X,
                                    sc[q][j], bi[q][j]);
    }
    // the wavefront's R rows are adjacent (row0 a multiple of R, F a multiple
    // of 64): one R * 2-byte store per copy of h
    uint32_t hw[R / 2];
#pragma unroll
    for (int r = 0; r < R; r += 2) {
        const float g0 = wave_sum_to_lane63(acc[2 * r]);
        const float u0 = wave_sum_to_lane63(acc[2 * r + 1]);
        const float g1 = wave_sum_to_lane63(acc[2 * r + 2]);
        const float u1 = wave_sum_to_lane63(acc[2 * r + 3]);
        hw[r / 2] = f32_to_bf16_rne(gelu_tanh(g0) * u0) | (f32_to_bf16_rne(gelu_tanh(g1) * u1) << 16);
    }
    if (lane == 63 && row0 < F) {
        if constexpr (R == 4) {
            const uint64_t v = hw[0] | ((uint64_t)hw[1] << 32);
            if constexpr (HANDOFF) {
#pragma unroll
                for (int c2 = 0; c2 < kHRep; ++c2) put64(a.hc + (int64_t)c2 * F + row0, v);
            }
            if (a.h) *reinterpret_cast<uint64_t*>(a.h + row0) = v;
        } else {
            if constexpr (HANDOFF) {
#pragma unroll
                for (int c2 = 0; c2 < kHRep; ++c2) put32(a.hc + (int64_t)c2 * F + row0, hw[0]);
            }
            if (a.h) *reinterpret_cast<uint32_t*>(a.h + row0) = hw[0];
        }
    }
    if constexpr (!HANDOFF) return;
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) *sflag = split_count(a.sync, kSyncHSub, kSyncHTop, item, a.n_gu);
    __syncthreads();
    if (*sflag && !a.withhold && threadIdx.x < kSyncRep)  // every h row is in
        put32(a.sync + kSyncHDoneRep + threadIdx.x * kSyncLine, 1u);
}

// ---------------------------------------------------------------- down item
template <int S, int NVD>
__device__ void ffn_down_item(const FfnArgs& a, int item, uint32_t* smem, int* sflag) {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    constexpr int R = kFfnRD;
    constexpr int SB = T::AFFINE ? 2 : 4;
    const int tid = item_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int D = a.D, F = a.F, VR = F / T::KV;
    const int64_t rowbytes = (int64_t)F / 2, groups = F / T::GROUP;
    const int row0 = item * (kFfnRW * R) + wave * R;
    // the rows do not depend on h: every code and scale load goes out first
    u32x4_t c[R][NVD];
    float sc[R][NVD], bi[R][NVD];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = min(row0 + r, D - 1);
        const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(a.dc + n * rowbytes);
        const uint8_t* sp = a.ds + n * groups * SB;
        const uint8_t* bp = T::AFFINE ? a.db + n * groups * 2 : nullptr;
#pragma unroll
        for (int j = 0; j < NVD; ++j) {
            const int v = min(lane + 64 * j, VR - 1);
            c[r][j] = __builtin_nontemporal_load(cp + v);
            ffn_scale<S>(sp, bp, v / T::VPG, sc[r][j], bi[r][j]);
        }
    }
    asm volatile("" ::: "memory");
    if (!wg_wait_flag(a.sync, a.wait_limit, kSyncHDoneRep, kGaveUpH, sflag)) return;  // uniform
    // stage this workgroup's copy of h: 16-byte pieces (8 elements) in the
    // unpack's pair order, lane i of a load instruction reading piece i of a
    // 1 KiB run (two 8-byte device-scope loads per piece) ...
    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + F / 2);
    const uint16_t* hsrc = a.hc + (int64_t)(blockIdx.x % kHRep) * F;
    const int pieces = F / 8;
    for (int i = tid; i < pieces; i += kFfnThreads) {
        const uint64_t lo = get64(hsrc + (int64_t)i * 8), hi = get64(hsrc + (int64_t)i * 8 + 4);
        const uint32_t e0 = (uint32_t)lo, e1 = (uint32_t)(lo >> 32), e2 = (uint32_t)hi,
                       e3 = (uint32_t)(hi >> 32);
        uint4 o;  // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
        o.x = __builtin_amdgcn_perm(e2, e0, 0x05040100u);
        o.y = __builtin_amdgcn_perm(e2, e0, 0x07060302u);
        o.z = __builtin_amdgcn_perm(e3, e1, 0x05040100u);
        o.w = __builtin_amdgcn_perm(e3, e1, 0x07060302u);
        *reinterpret_cast<uint4*>(xs + L::piece(i / 4, i % 4)) = o;
    }
    __syncthreads();
    // ... then each vector's sum from its four pieces, in element order (the
    // order the activation staging of the GEMV kernels uses)
    constexpr uint32_t ONES = 0x3F803F80u;
    for (int v = tid; v < VR; v += kFfnThreads) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 o = *reinterpret_cast<const uint4*>(xs + L::piece(v, q));
            sum = dot2_bf16(ONES, __builtin_amdgcn_perm(o.y, o.x, 0x05040100u), sum);  // (x0,x1)
            sum = dot2_bf16(ONES, __builtin_amdgcn_perm(o.w, o.z, 0x05040100u), sum);  // (x2,x3)
            sum = dot2_bf16(ONES, __builtin_amdgcn_perm(o.y, o.x, 0x07060302u), sum);  // (x4,x5)
            sum = dot2_bf16(ONES, __builtin_amdgcn_perm(o.w, o.z, 0x07060302u), sum);  // (x6,x7)
        }
        XS[v] = sum;
    }
    __syncthreads();
    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    float acc[R] = {};
#pragma unroll
    for (int j = 0; j < NVD; ++j) {
        const int v = lane + 64 * j;
        if (v >= VR) break;
        uint32_t xp[L::XW];
        read_pairs<S>(xs, v, xp);
        const float X = XS[v];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = apply_group<S>(acc[r], dot_code_vector<S>(c[r][j], xp, MASK, MAGIC), X,
                                    sc[r][j], bi[r][j]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float tot = wave_sum_to_lane63(acc[r]);
        if (lane == 63 && row0 + r < D) a.y[row0 + r] = tot;
    }
}

// ---------------------------------------------------------------- the kernel
template <int S, int NVG, int NVD>
__global__ __launch_bounds__(kFfnThreads) void ffn_kernel(FfnArgs a) {
    extern __shared__ __align__(16) uint32_t smem[];
    __shared__ int sflag;
    const int n = a.n_gu + a.n_down;
    for (int it = blockIdx.x; it < n; it += gridDim.x) {
        if (it < a.n_gu) ffn_gate_up_item<S, NVG, ffn_pairs<NVG>(), true>(a, it, smem, &sflag);
        else ffn_down_item<S, NVD>(a, it - a.n_gu, smem, &sflag);
        __syncthreads();  // LDS and sflag reuse by the next item
    }
    if (threadIdx.x == 0) {
        stores_done();  // this thread's earlier counts and polls have completed
        sflag = split_count(a.sync, kSyncExitSub, kSyncExitTop, blockIdx.x, gridDim.x);
    }
    __syncthreads();
    if (sflag && threadIdx.x < 64) {
        const int lane = threadIdx.x;
        if (lane == 0) {
            const unsigned err = atomicExch(a.sync + kSyncErr, 0u);
            put32(a.sync + kSyncStatus, err);
            put32(a.sync + kSyncHTop, 0u);
            put32(a.sync + kSyncExitTop, 0u);
        }
        if (lane < kSyncRep) {
            put32(a.sync + kSyncHSub + lane * kSyncLine, 0u);
            put32(a.sync + kSyncHDoneRep + lane * kSyncLine, 0u);
            put32(a.sync + kSyncExitSub + lane * kSyncLine, 0u);
        }
    }
}

// The gate/up rows on their own (one token): h = bf16(gelu_tanh(g) * u) to a.h,
// one workgroup per RW * 2 row pairs; the down projection follows as a GEMV
// launch.
template <int S, int NV, int XV>
__global__ __launch_bounds__(kFfnThreads) void ffn_gate_up_kernel(FfnArgs a) {
    extern __shared__ __align__(16) uint32_t smem[];
    ffn_gate_up_item<S, NV, 2, false, XV>(a, blockIdx.x, smem, nullptr);
}

// h = bf16(gelu_tanh(g) * u) elementwise: the launch sequence (gate and up in
// one GEMV launch, this, down) where the gate/up launch cannot carry it.
__global__ __launch_bounds__(256) void ffn_act_kernel(const float* __restrict__ g,
                                                      const float* __restrict__ u,
                                                      uint16_t* __restrict__ h, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        h[i] = (uint16_t)f32_to_bf16_rne(gelu_tanh(g[i]) * u[i]);
}

// ---------------------------------------------------------------- host side
static size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

static int ffn_nv(int64_t VR) { return (int)((VR + 63) / 64); }

bool ffn_fused_ok(int scheme, int64_t D, int64_t F) {
    if (scheme != SYM4_G128 && scheme != AFF4_G64) return false;
    const int64_t g = scheme == SYM4_G128 ? 128 : 64;
    if (D % g || F % g) return false;
    const int nvg = ffn_nv(D / 32), nvd = ffn_nv(F / 32);
    return nvg >= 2 && nvg <= 4 && nvd >= 6 && nvd <= 8;
}

FfnWorkspace ffn_workspace_layout(int scheme, int64_t M, int64_t D, int64_t F) {
    FfnWorkspace w{};
    size_t o = 0;
    w.sync = o;  o += al256(kLayerSyncWords * 4);
    w.h = o;     o += al256((size_t)std::max<int64_t>(kHRep, M) * F * 2);
    w.g = o;     o += al256((size_t)M * F * 4);
    w.u = o;     o += al256((size_t)M * F * 4);
    w.part = o;  o += M > 1 && M <= 16 ? al256(gemv_mfma_split_bytes(scheme, D, F, M)) : 0;
    w.total = o;
    return w;
}

template <int S, int NVG, int NVD>
static hipError_t go_ffn(const FfnArgs& a, size_t lds, hipStream_t st) {
    auto kern = ffn_kernel<S, NVG, NVD>;
    hipError_t e = hipSuccess;
    const int grid = persistent_grid((const void*)kern, kFfnThreads, lds, a.n_gu + a.n_down, &e);
    if (grid < 1) return e;  // nothing launched
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kFfnThreads), lds, st, a);
    return hipGetLastError();
}

template <int S, int NVG>
static hipError_t pick_ffn_nvd(int nvd, const FfnArgs& a, size_t lds, hipStream_t st) {
    if (nvd == 6) return go_ffn<S, NVG, 6>(a, lds, st);
    if (nvd == 7) return go_ffn<S, NVG, 7>(a, lds, st);
    return go_ffn<S, NVG, 8>(a, lds, st);
}

template <int S>
static hipError_t pick_ffn(int nvg, int nvd, const FfnArgs& a, size_t lds, hipStream_t st) {
    if (nvg == 2) return pick_ffn_nvd<S, 2>(nvd, a, lds, st);
    if (nvg == 3) return pick_ffn_nvd<S, 3>(nvd, a, lds, st);
    return pick_ffn_nvd<S, 4>(nvd, a, lds, st);
}

hipError_t launch_ffn_fused(int scheme, const void* const* gate, const void* const* up,
                            const void* const* down, int64_t D, int64_t F, const uint16_t* x,
                            uint16_t* h, float* y, void* ws, long long wait_limit, int withhold,
                            hipStream_t st) {
    if (!ffn_fused_ok(scheme, D, F)) return hipErrorNotSupported;
    const FfnWorkspace L = ffn_workspace_layout(scheme, 1, D, F);
    uint8_t* base = (uint8_t*)ws;
    FfnArgs a{};
    a.gc = (const uint8_t*)gate[0]; a.gs = (const uint8_t*)gate[1]; a.gb = (const uint8_t*)gate[2];
    a.uc = (const uint8_t*)up[0];   a.us = (const uint8_t*)up[1];   a.ub = (const uint8_t*)up[2];
    a.dc = (const uint8_t*)down[0]; a.ds = (const uint8_t*)down[1]; a.db = (const uint8_t*)down[2];
    a.x = x;
    a.hc = (uint16_t*)(base + L.h);
    a.h = h;
    a.y = y;
    a.sync = (unsigned*)(base + L.sync);
    a.D = (int)D;
    a.F = (int)F;
    a.n_gu = (int)((F + kFfnRW * 4 - 1) / (kFfnRW * 4));  // four pairs per wavefront ...
    a.n_down = (int)((D + kFfnRW * kFfnRD - 1) / (kFfnRW * kFfnRD));
    a.wait_limit = wait_limit;
    a.withhold = withhold;
    const size_t lds = (size_t)std::max(D / 2 + D / 32, F / 2 + F / 32) * 4;
    const int nvg = ffn_nv(D / 32), nvd = ffn_nv(F / 32);
    if (nvg > 2) a.n_gu = (int)((F + kFfnRW * 2 - 1) / (kFfnRW * 2));  // ... or two
    return scheme == SYM4_G128 ? pick_ffn<SYM4_G128>(nvg, nvd, a, lds, st)
                               : pick_ffn<AFF4_G64>(nvg, nvd, a, lds, st);
}

template <int S, int NV>
static void go_ffn_gate_up_nv(const FfnArgs& a, int blocks, size_t lds, hipStream_t st) {
    constexpr int XV = NV * 64 > 256 ? 2 : 1;  // D / KV vectors <= 64 NV
    hipLaunchKernelGGL((ffn_gate_up_kernel<S, NV, XV>), dim3(blocks), dim3(kFfnThreads), lds, st, a);
}

template <int S>
static hipError_t go_ffn_gate_up(int nv, const FfnArgs& a, int blocks, size_t lds, hipStream_t st) {
    if constexpr (Traits<S>::BITS == 4) {  // D / 32 <= 256 vectors
        switch (nv) {
            case 1: go_ffn_gate_up_nv<S, 1>(a, blocks, lds, st); break;
            case 2: go_ffn_gate_up_nv<S, 2>(a, blocks, lds, st); break;
            case 3: go_ffn_gate_up_nv<S, 3>(a, blocks, lds, st); break;
            default: go_ffn_gate_up_nv<S, 4>(a, blocks, lds, st); break;
        }
    } else {  // 8-bit: D / 16 <= 512 vectors
        switch (nv) {
            case 1: go_ffn_gate_up_nv<S, 1>(a, blocks, lds, st); break;
            case 2: go_ffn_gate_up_nv<S, 2>(a, blocks, lds, st); break;
            case 3: go_ffn_gate_up_nv<S, 3>(a, blocks, lds, st); break;
            case 4: go_ffn_gate_up_nv<S, 4>(a, blocks, lds, st); break;
            case 5: go_ffn_gate_up_nv<S, 5>(a, blocks, lds, st); break;
            case 6: go_ffn_gate_up_nv<S, 6>(a, blocks, lds, st); break;
            case 7: go_ffn_gate_up_nv<S, 7>(a, blocks, lds, st); break;
            default: go_ffn_gate_up_nv<S, 8>(a, blocks, lds, st); break;
        }
    }
    return hipGetLastError();
}

bool ffn_gate_up_ok(int scheme, int64_t D, int64_t F) {
    if (scheme == AFF8_G64) return D % 64 == 0 && F % 64 == 0 && D / 16 <= 512;
    if (scheme != SYM4_G128 && scheme != AFF4_G64) return false;
    const int64_t g = scheme == SYM4_G128 ? 128 : 64;
    return D % g == 0 && F % g == 0 && D / 32 <= 256;
}

hipError_t launch_ffn_gate_up(int scheme, const void* const* gate, const void* const* up, int64_t D,
                              int64_t F, const uint16_t* x, uint16_t* h, hipStream_t st) {
    if (!ffn_gate_up_ok(scheme, D, F)) return hipErrorNotSupported;
    FfnArgs a{};
    a.gc = (const uint8_t*)gate[0]; a.gs = (const uint8_t*)gate[1]; a.gb = (const uint8_t*)gate[2];
    a.uc = (const uint8_t*)up[0];   a.us = (const uint8_t*)up[1];   a.ub = (const uint8_t*)up[2];
    a.x = x;
    a.h = h;
    a.D = (int)D;
    a.F = (int)F;
    const int blocks = (int)((F + kFfnRW * 2 - 1) / (kFfnRW * 2));
    const int64_t VR = D / (scheme == AFF8_G64 ? 16 : 32);  // 16-byte code vectors per row
    const size_t lds = (size_t)(D / 2 + VR) * 4;
    const int nv = ffn_nv(VR);
    return scheme == SYM4_G128 ? go_ffn_gate_up<SYM4_G128>(nv, a, blocks, lds, st)
           : scheme == AFF4_G64 ? go_ffn_gate_up<AFF4_G64>(nv, a, blocks, lds, st)
                                : go_ffn_gate_up<AFF8_G64>(nv, a, blocks, lds, st);
}

hipError_t launch_ffn_act(const float* g, const float* u, uint16_t* h, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(ffn_act_kernel, dim3((unsigned)blocks), dim3(256), 0, st, g, u, h, n);
    return hipGetLastError();
}

}  // namespace w4
