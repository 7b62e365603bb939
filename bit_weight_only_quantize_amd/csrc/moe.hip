// Mixture-of-experts decode path on 4-bit experts.
//
// TurboFieldfare article (Gemma 4 26B-A4B section and 量化和精度): 128 routed
// experts per layer, 8 chosen per token by an 8-bit router with no logit
// softcap; a dense shared expert whose output is added without a routing
// weight; shared and routed FFNs computed side by side; experts stored at a
// fixed stride. Only the selected experts' bytes are read.
//
// Route:  router GEMV (fp32 logits) -> one wavefront per token: softmax over all
//         E raw logits, top-k by logit (ties to the lower index), weights = the
//         selected probabilities (not renormalized).
// Experts: bucket (token, slot) pairs by expert (stable, deterministic) ->
//         gate/up pass (both rows of an n in one lane; epilogue
//         h = bf16(gelu_tanh(g) * u)) over active experts + the shared expert ->
//         down pass into per-pair partial rows + the shared output ->
//         combine y = shared + sum_j w_j * partial_j in a fixed order.
// No floating-point atomics anywhere: results are bit-reproducible.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "skinny.hpp"
#include "moe1.hpp"

namespace w4 {

// ---------------------------------------------------------------- routing
// One workgroup (64 threads) per token, E <= 1024. Every logit is ranked against
// all E logits (staged in LDS): rank = #{j : l_j > l_e or (l_j == l_e and j < e)},
// i.e. its position in a stable sort by logit descending. rank < k selects the
// expert into slot `rank`. Softmax over all E raw logits; no renormalization.
__global__ __launch_bounds__(64) void topk_softmax_kernel(const float* __restrict__ logits, int E,
                                                          int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ wts) {
    __shared__ float ls[1024];
    const int m = blockIdx.x, lane = threadIdx.x;
    const float* l = logits + (int64_t)m * E;
    float mx = -INFINITY;
    for (int e = lane; e < E; e += 64) {
        ls[e] = l[e];
        mx = fmaxf(mx, ls[e]);
    }
    mx = wave_max(mx);
    __syncthreads();
    float s = 0.f;
    for (int e = lane; e < E; e += 64) s += expf(ls[e] - mx);
    for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o, 64);  // same order in every lane
    const float inv = 1.f / s;
    for (int e = lane; e < E; e += 64) {
        const float v = ls[e];
        int rank = 0;
        for (int j = 0; j < E; ++j) {
            const float u = ls[j];
            rank += (u > v) | ((u == v) & (j < e));
        }
        if (rank < k) {
            ids[(int64_t)m * k + rank] = e;
            wts[(int64_t)m * k + rank] = expf(v - mx) * inv;
        }
    }
}

hipError_t launch_route(int scheme, const void* codes, const void* scale, const void* bias,
                        int64_t E, int64_t K, const uint16_t* x, int64_t M, int k, float* logits,
                        int32_t* ids, float* wts, hipStream_t st) {
    hipError_t e = launch_gemv(scheme, codes, scale, bias, E, K, x, M, logits, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_softmax_kernel, dim3((unsigned)M), dim3(64), 0, st, logits, (int)E, k,
                       ids, wts);
    return hipGetLastError();
}

// ---------------------------------------------------------------- bucketing
// Single workgroup. Pair p = m * k + j (token m, slot j). For every expert e, the
// pairs routed to it in increasing p; experts with at least one pair listed in
// increasing e. Ids outside [0, E) are ignored.
__global__ __launch_bounds__(1024) void moe_bucket_kernel(const int32_t* __restrict__ ids, int P,
                                                          int E, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ active,
                                                          int32_t* __restrict__ n_active,
                                                          int32_t* __restrict__ pairs) {
    __shared__ int cnt[1024];
    __shared__ int off[1025];
    __shared__ int act[1025];
    const int t = threadIdx.x;
    for (int e = t; e < E; e += blockDim.x) {
        int c = 0;
        for (int p = 0; p < P; ++p) c += ids[p] == e;
        cnt[e] = c;
    }
    __syncthreads();
    if (t == 0) {  // exclusive scans (E <= 1024: a single pass is cheap)
        int o = 0, a = 0;
        for (int e = 0; e < E; ++e) {
            off[e] = o;
            o += cnt[e];
            if (cnt[e]) act[a++] = e;
        }
        off[E] = o;
        act[E] = a;
    }
    __syncthreads();
    for (int e = t; e <= E; e += blockDim.x) offsets[e] = off[e];
    for (int i = t; i < E; i += blockDim.x) active[i] = i < act[E] ? act[i] : -1;
    if (t == 0) *n_active = act[E];
    for (int e = t; e < E; e += blockDim.x) {
        int w = off[e];
        for (int p = 0; p < P; ++p)
            if (ids[p] == e) pairs[w++] = p;
    }
}

// ---------------------------------------------------------------- expert passes
struct MoeMat {  // one stacked matrix (expert stride in bytes), or a single one
    const uint8_t* codes;
    const uint8_t* scale;
    const uint8_t* bias;
    int64_t stride_c, stride_s;  // bytes between experts
    int N, K;
};

struct MoeArgs {
    MoeMat gate, up, down, sgate, sup, sdown;
    int has_shared;
    int M, k, E;
    const uint16_t* x;        // [M][D]
    const int32_t* offsets;   // [E+1]
    const int32_t* active;    // [E]
    const int32_t* n_active;  // [1]
    const int32_t* pairs;     // [M*k]
    uint16_t* h;              // [M*k][F] bf16
    uint16_t* hs;             // [M][Fs] bf16
    float* part;              // [M*k][D]
    float* sout;              // [M][D]
    int amax;                 // routed slots in the grid = min(E, M*k)
    int tiles_r, tiles_s;     // row tiles per routed slot / for the shared expert
};

template <int S>
__device__ __forceinline__ void row_ptrs(const MoeMat& W, int e, int n, const uint8_t*& c,
                                         const uint8_t*& s, const uint8_t*& b) {
    using T = Traits<S>;
    const int64_t groups = W.K / T::GROUP;
    constexpr int SB = T::AFFINE ? 2 : 4;
    c = W.codes + e * W.stride_c + (int64_t)n * W.K * T::BITS / 8;
    s = W.scale + e * W.stride_s + (int64_t)n * groups * SB;
    b = T::AFFINE ? W.bias + e * W.stride_s + (int64_t)n * groups * 2 : nullptr;
}

// gate/up pass: one lane slot owns (gate row n, up row n); block = 4 * (64/LPR) n.
template <int S, int MT, int LPR, int V>
__global__ __launch_bounds__(256) void moe_gate_up_kernel(MoeArgs a) {
    using Core = SkinnyCore<S, MT, LPR, V, 2>;
    constexpr int RSW = 64 / LPR, NPB = 4 * RSW;
    extern __shared__ __align__(16) uint32_t smem[];
    __shared__ int tok[MT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane / LPR, sl = lane % LPR;
    int bid = blockIdx.x, e, n0, count, first;
    const MoeMat *G, *U;
    bool shared;
    if (bid < a.amax * a.tiles_r) {
        const int s = bid / a.tiles_r;
        if (s >= *a.n_active) return;
        e = a.active[s];
        n0 = (bid % a.tiles_r) * NPB;
        first = a.offsets[e];
        count = a.offsets[e + 1] - first;
        G = &a.gate;
        U = &a.up;
        shared = false;
    } else {
        e = 0;
        n0 = (bid - a.amax * a.tiles_r) * NPB;
        first = 0;
        count = a.M;
        G = &a.sgate;
        U = &a.sup;
        shared = true;
    }
    const int F = G->N, D = G->K;
    const int n = n0 + wave * RSW + slot;
    const int nl = n < F ? n : F - 1;
    Core core;
    core.VR = D / Traits<S>::KV;
    core.sl = sl;
    row_ptrs<S>(*G, e, nl, core.crow[0], core.srow[0], core.brow[0]);
    row_ptrs<S>(*U, e, nl, core.crow[1], core.srow[1], core.brow[1]);
    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + MT * (D / 2));
    typename Core::Buf A, B;
    for (int t0 = 0; t0 < count; t0 += MT) {
        const int mt = min(MT, count - t0);
        core.load(A, 0);
        if (t0) __syncthreads();
        if (threadIdx.x < MT) {
            const int i = t0 + (int)threadIdx.x < count ? t0 + threadIdx.x : t0;
            tok[threadIdx.x] = shared ? i : a.pairs[first + i] / a.k;
        }
        __syncthreads();
        stage_x<S, MT, V, 256>(a.x, D, tok, mt, D, xs, XS);
        __syncthreads();
        float acc[2][MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[0][m] = acc[1][m] = 0.f;
        core.run(A, B, xs, XS, D / 2, acc);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            acc[0][m] = group_sum<LPR>(acc[0][m]);
            acc[1][m] = group_sum<LPR>(acc[1][m]);
        }
        if (sl == 0 && n < F) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < mt) {
                    const uint16_t hv = (uint16_t)f32_to_bf16_rne(gelu_tanh(acc[0][m]) * acc[1][m]);
                    if (shared) a.hs[(int64_t)(t0 + m) * F + n] = hv;
                    else a.h[(int64_t)a.pairs[first + t0 + m] * F + n] = hv;
                }
            }
        }
    }
}

// down pass: rows n of W_down[e] against the h rows of the expert's pairs.
template <int S, int MT, int LPR, int V, int R>
__global__ __launch_bounds__(256) void moe_down_kernel(MoeArgs a) {
    using Core = SkinnyCore<S, MT, LPR, V, R>;
    constexpr int RSW = 64 / LPR, NPB = 4 * RSW * R;
    extern __shared__ __align__(16) uint32_t smem[];
    __shared__ int tok[MT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane / LPR, sl = lane % LPR;
    int bid = blockIdx.x, e, n0, count, first;
    const MoeMat* W;
    bool shared;
    if (bid < a.amax * a.tiles_r) {
        const int s = bid / a.tiles_r;
        if (s >= *a.n_active) return;
        e = a.active[s];
        n0 = (bid % a.tiles_r) * NPB;
        first = a.offsets[e];
        count = a.offsets[e + 1] - first;
        W = &a.down;
        shared = false;
    } else {
        e = 0;
        n0 = (bid - a.amax * a.tiles_r) * NPB;
        first = 0;
        count = a.M;
        W = &a.sdown;
        shared = true;
    }
    const int D = W->N, F = W->K;
    const uint16_t* hin = shared ? a.hs : a.h;
    Core core;
    core.VR = F / Traits<S>::KV;
    core.sl = sl;
    int n[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        n[r] = n0 + wave * RSW * R + slot + r * RSW;
        const int nl = n[r] < D ? n[r] : D - 1;
        row_ptrs<S>(*W, e, nl, core.crow[r], core.srow[r], core.brow[r]);
    }
    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + MT * (F / 2));
    typename Core::Buf A, B;
    for (int t0 = 0; t0 < count; t0 += MT) {
        const int mt = min(MT, count - t0);
        core.load(A, 0);
        if (t0) __syncthreads();
        if (threadIdx.x < MT) {
            const int i = t0 + (int)threadIdx.x < count ? t0 + threadIdx.x : t0;
            tok[threadIdx.x] = shared ? i : a.pairs[first + i];
        }
        __syncthreads();
        stage_x<S, MT, V, 256>(hin, F, tok, mt, F, xs, XS);
        __syncthreads();
        float acc[R][MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
        core.run(A, B, xs, XS, F / 2, acc);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = group_sum<LPR>(acc[r][m]);
        if (sl == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (n[r] >= D) continue;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m >= mt) continue;
                    if (shared) a.sout[(int64_t)(t0 + m) * D + n[r]] = acc[r][m];
                    else a.part[(int64_t)a.pairs[first + t0 + m] * D + n[r]] = acc[r][m];
                }
            }
        }
    }
}

// y[m][n] = shared[m][n] + sum_j w[m][j] * part[m*k + j][n]   (fixed j order)
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ part,
                                                          const float* __restrict__ sout,
                                                          const float* __restrict__ wts,
                                                          const int32_t* __restrict__ ids, int M,
                                                          int k, int D, int E, int has_shared,
                                                          float* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * D) return;
    const int m = (int)(i / D), n = (int)(i % D);
    float acc = has_shared ? sout[i] : 0.f;
    for (int j = 0; j < k; ++j) {
        const int e = ids[(int64_t)m * k + j];
        if (e < 0 || e >= E) continue;
        acc = fmaf(wts[(int64_t)m * k + j], part[((int64_t)m * k + j) * D + n], acc);
    }
    y[i] = acc;
}

// ---------------------------------------------------------------- host side
static size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

MoeWorkspace moe_workspace_layout(int64_t M, int k, int64_t E, int64_t D, int64_t F, int64_t Fs) {
    MoeWorkspace w{};
    size_t o = 0;
    w.offsets = o; o += al((E + 1) * 4);
    w.active = o;  o += al(E * 4);
    w.n_active = o; o += al(4);
    w.pairs = o;   o += al(M * k * 4);
    w.h = o;       o += al(M * k * F * 2);
    w.hs = o;      o += al(M * Fs * 2);
    w.part = o;    o += al(M * k * D * 4);
    w.sout = o;    o += al(M * D * 4);
    w.total = o;
    return w;
}

static MoeMat mm(const void* c, const void* s, const void* b, int64_t N, int64_t K, int scheme) {
    const int64_t groups = K / (scheme == SYM4_G128 ? 128 : 64);
    MoeMat m{};
    m.codes = (const uint8_t*)c;
    m.scale = (const uint8_t*)s;
    m.bias = (const uint8_t*)b;
    m.stride_c = N * K / 2;
    m.stride_s = N * groups * (scheme == SYM4_G128 ? 4 : 2);
    m.N = (int)N;
    m.K = (int)K;
    return m;
}

template <int S>
static hipError_t moe_passes(const MoeArgs& a0, int64_t Fs, hipStream_t st) {
    MoeArgs a = a0;
    const int D = a.gate.K, F = a.gate.N;
    // gate/up: LPR 64 (one wavefront per (gate, up) row pair), 4 n per block
    a.tiles_r = (F + 3) / 4;
    a.tiles_s = a.has_shared ? (int)((Fs + 3) / 4) : 0;
    int blocks = a.amax * a.tiles_r + a.tiles_s;
    const int kv = Traits<S>::KV;
    const int Dmax = D;
    if (a.M == 1) {
        size_t lds = (size_t)1 * (Dmax / 2 + Dmax / kv) * 4;
        hipLaunchKernelGGL((moe_gate_up_kernel<S, 1, 64, 1>), dim3(blocks), dim3(256), lds, st, a);
    } else {
        size_t lds = (size_t)4 * (Dmax / 2 + Dmax / kv) * 4;
        hipLaunchKernelGGL((moe_gate_up_kernel<S, 4, 64, 1>), dim3(blocks), dim3(256), lds, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // down: LPR 16, V 2, R 2 -> 32 rows per block (K = F routed, Fs shared)
    const int Kmax = a.has_shared ? (int)std::max<int64_t>(F, Fs) : F;
    a.tiles_r = (D + 31) / 32;
    a.tiles_s = a.has_shared ? a.tiles_r : 0;
    blocks = a.amax * a.tiles_r + a.tiles_s;
    if (a.M == 1) {
        size_t lds = (size_t)1 * (Kmax / 2 + Kmax / kv) * 4;
        hipLaunchKernelGGL((moe_down_kernel<S, 1, 16, 2, 2>), dim3(blocks), dim3(256), lds, st, a);
    } else {
        size_t lds = (size_t)4 * (Kmax / 2 + Kmax / kv) * 4;
        hipLaunchKernelGGL((moe_down_kernel<S, 4, 16, 2, 2>), dim3(blocks), dim3(256), lds, st, a);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- M = 1 fast path
static Moe1Mat m1m(const void* const* t, int64_t N, int64_t K, int scheme) {
    const int64_t groups = K / (scheme == SYM4_G128 ? 128 : 64);
    Moe1Mat m{};
    m.codes = (const uint8_t*)t[0];
    m.scale = (const uint8_t*)t[1];
    m.bias = (const uint8_t*)t[2];
    m.stride_c = N * K / 2;
    m.stride_s = N * groups * (scheme == SYM4_G128 ? 4 : 2);
    return m;
}

bool moe1_ok(int64_t M, int k, int64_t D, int64_t F, int64_t Fs) {
    return M == 1 && k <= 8 && D >= 2048 && D <= 4096 && F >= 32 && F <= 1024 && Fs <= 4096 &&
           (Fs == 0 || Fs >= 32);
}

template <int S, int NVD, int NVS>
static void go_down1(const Moe1Args& a, int blocks, size_t lds, hipStream_t st) {
    hipLaunchKernelGGL((moe1_down_kernel<S, NVD, NVS, 1, NVD + NVS>), dim3(blocks), dim3(320), lds,
                       st, a);
}

template <int S, int NVD>
static void pick_nvs(int nvs, const Moe1Args& a, int blocks, size_t lds, hipStream_t st) {
    if (nvs == 0) go_down1<S, NVD, 0>(a, blocks, lds, st);
    else if (nvs == 1) go_down1<S, NVD, 1>(a, blocks, lds, st);
    else go_down1<S, NVD, 2>(a, blocks, lds, st);
}

template <int S>
static hipError_t moe1_passes(Moe1Args a, hipStream_t st) {
    constexpr int R = 2;
    const int kv = Traits<S>::KV;
    a.tiles_r = (a.F + 4 * R - 1) / (4 * R);
    a.tiles_s = a.has_shared ? (a.Fs + 4 * R - 1) / (4 * R) : 0;
    const int blocks = a.k * a.tiles_r + a.tiles_s;
    const size_t lds = (size_t)(a.D / 2 + a.D / kv) * 4;
    if (a.D / kv <= 64)
        hipLaunchKernelGGL((moe1_gate_up_kernel<S, 1, R, 1>), dim3(blocks), dim3(320), lds, st, a);
    else
        hipLaunchKernelGGL((moe1_gate_up_kernel<S, 2, R, 2>), dim3(blocks), dim3(320), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int VRF = a.F / kv, VRS = a.has_shared ? a.Fs / kv : 0;
    const int nvd = (VRF + 7) / 8, nvs = (VRS + 63) / 64;
    const size_t lds2 = (size_t)(8 * (a.F / 2 + VRF) + (a.has_shared ? a.Fs / 2 + VRS : 0)) * 4;
    const int blocks2 = (a.D + 3) / 4;
    switch (nvd) {
        case 1: pick_nvs<S, 1>(nvs, a, blocks2, lds2, st); break;
        case 2: pick_nvs<S, 2>(nvs, a, blocks2, lds2, st); break;
        case 3: pick_nvs<S, 3>(nvs, a, blocks2, lds2, st); break;
        default: pick_nvs<S, 4>(nvs, a, blocks2, lds2, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_moe(int scheme, const MoeMats& W, const uint16_t* x, int64_t M, const int32_t* ids,
                      const float* wts, int k, void* ws, float* y, hipStream_t st) {
    const int64_t E = W.E, D = W.D, F = W.F, Fs = W.Fs;
    const MoeWorkspace L = moe_workspace_layout(M, k, E, D, F, Fs);
    uint8_t* base = (uint8_t*)ws;
    if (moe1_ok(M, k, D, F, Fs)) {
        Moe1Args a{};
        a.gate = m1m(W.gate, F, D, scheme);
        a.up = m1m(W.up, F, D, scheme);
        a.down = m1m(W.down, D, F, scheme);
        a.has_shared = Fs > 0;
        if (Fs > 0) {
            a.sgate = m1m(W.sgate, Fs, D, scheme);
            a.sup = m1m(W.sup, Fs, D, scheme);
            a.sdown = m1m(W.sdown, D, Fs, scheme);
        }
        a.k = k; a.E = (int)E; a.D = (int)D; a.F = (int)F; a.Fs = (int)Fs;
        a.x = x; a.ids = ids; a.wts = wts;
        a.h = (uint16_t*)(base + L.h);
        a.hs = (uint16_t*)(base + L.hs);
        a.y = y;
        return scheme == SYM4_G128 ? moe1_passes<SYM4_G128>(a, st) : moe1_passes<AFF4_G64>(a, st);
    }
    MoeArgs a{};
    a.gate = mm(W.gate[0], W.gate[1], W.gate[2], F, D, scheme);
    a.up = mm(W.up[0], W.up[1], W.up[2], F, D, scheme);
    a.down = mm(W.down[0], W.down[1], W.down[2], D, F, scheme);
    a.has_shared = Fs > 0;
    if (Fs > 0) {
        a.sgate = mm(W.sgate[0], W.sgate[1], W.sgate[2], Fs, D, scheme);
        a.sup = mm(W.sup[0], W.sup[1], W.sup[2], Fs, D, scheme);
        a.sdown = mm(W.sdown[0], W.sdown[1], W.sdown[2], D, Fs, scheme);
    }
    a.M = (int)M;
    a.k = k;
    a.E = (int)E;
    a.x = x;
    a.offsets = (const int32_t*)(base + L.offsets);
    a.active = (const int32_t*)(base + L.active);
    a.n_active = (const int32_t*)(base + L.n_active);
    a.pairs = (const int32_t*)(base + L.pairs);
    a.h = (uint16_t*)(base + L.h);
    a.hs = (uint16_t*)(base + L.hs);
    a.part = (float*)(base + L.part);
    a.sout = (float*)(base + L.sout);
    a.amax = (int)std::min<int64_t>(E, M * k);
    const int P = (int)(M * k);
    hipLaunchKernelGGL(moe_bucket_kernel, dim3(1), dim3(1024), 0, st, ids, P, (int)E,
                       (int32_t*)(base + L.offsets), (int32_t*)(base + L.active),
                       (int32_t*)(base + L.n_active), (int32_t*)(base + L.pairs));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = scheme == SYM4_G128 ? moe_passes<SYM4_G128>(a, Fs, st) : moe_passes<AFF4_G64>(a, Fs, st);
    if (e != hipSuccess) return e;
    const int64_t tot = M * D;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                       a.part, a.sout, wts, ids, (int)M, k, (int)D, (int)E, a.has_shared, y);
    return hipGetLastError();
}

}  // namespace w4
