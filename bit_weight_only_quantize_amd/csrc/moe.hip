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
// Experts: one token: a two-launch fast path (moe1.hpp). Several tokens:
//         bucket (token, slot) pairs by expert (stable, deterministic) ->
//         gate/up pass on the matrix cores (a gate tile and an up tile of the
//         same rows, so a lane holds g and u of one (token, f); epilogue
//         h = bf16(gelu_tanh(g) * u)) over active experts + the shared expert ->
//         down pass into per-pair partial rows + the shared output ->
//         combine y = shared + sum_j w_j * partial_j in a fixed order.
// No floating-point atomics anywhere: results are bit-reproducible.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"
#include "gemv_mfma.hpp"
#include "skinny.hpp"
#include "moe1.hpp"
#include "moe_routed.hpp"

namespace w4 {

// ---------------------------------------------------------------- routing
// One wavefront per token over precomputed logits. EPL is as small as E
// allows: a single wavefront on a CU whose instruction cache is cold pays for
// every line of code it executes.
template <int EPL>
__global__ __launch_bounds__(64) void topk_softmax_kernel(const float* __restrict__ logits, int E,
                                                          int k, int32_t* __restrict__ ids,
                                                          float* __restrict__ wts) {
    const int m = blockIdx.x, lane = threadIdx.x;
    const float* l = logits + (int64_t)m * E;
    float v[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {  // all loads issued at once (clamped), padding -inf
        const int e = lane + 64 * j;
        const float x = l[min(e, E - 1)];
        v[j] = e < E ? x : -INFINITY;
    }
    topk_rounds<EPL>(v, E, k, ids + (int64_t)m * k, wts + (int64_t)m * k);
}

hipError_t launch_route(int scheme, const void* codes, const void* scale, const void* bias,
                        int64_t E, int64_t K, const uint16_t* x, int64_t M, int k, float* logits,
                        int32_t* ids, float* wts, hipStream_t st) {
    // The router GEMV, then one single-wavefront workgroup per token. (One
    // 1024-thread workgroup per token streaming the router and selecting
    // without the logits' round trip through memory measured slower in the
    // Gemma-shaped layer at 32 tokens: 16.9 us against 6.1 + 4.7 us.)
    hipError_t e = launch_gemv(scheme, codes, scale, bias, E, K, x, M, logits, st);
    if (e != hipSuccess) return e;
    if (E <= 128)
        hipLaunchKernelGGL(topk_softmax_kernel<2>, dim3((unsigned)M), dim3(64), 0, st, logits, (int)E,
                           k, ids, wts);
    else if (E <= 256)
        hipLaunchKernelGGL(topk_softmax_kernel<4>, dim3((unsigned)M), dim3(64), 0, st, logits, (int)E,
                           k, ids, wts);
    else
        hipLaunchKernelGGL(topk_softmax_kernel<16>, dim3((unsigned)M), dim3(64), 0, st, logits,
                           (int)E, k, ids, wts);
    return hipGetLastError();
}

// ---------------------------------------------------------------- bucketing
// One 1024-thread workgroup. Pair p = m * k + j (token m, slot j), P <=
// kMoeMaxPairs, expert ids already in LDS (sid, -1 for ids outside [0, E)).
// For every expert e, the pairs routed to it (in no fixed order); the experts
// with at least one pair get work descriptors {e, first pair index, pair
// count}, one per kMoeDescPairs pairs, in increasing e; the remaining
// descriptors up to `slots` are {-1, 0, 0} and descriptor `slots` holds
// {number of descriptors in use, 0, 0}. Counts use LDS integer atomics
// (exact in any order).
__device__ __forceinline__ void bucket_pairs(const int* sid, int P, int E, int slots,
                                             int4* __restrict__ work, int32_t* __restrict__ pairs) {
    __shared__ int cnt[1024], off[1024], act[1024];
    __shared__ int n_act;
    const int t = threadIdx.x;
    for (int e = t; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int p = t; p < P; p += blockDim.x)
        if (sid[p] >= 0) atomicAdd(&cnt[sid[p]], 1);
    __syncthreads();
    if (t < 64) {  // exclusive scans of counts and of descriptor counts: 16 experts per lane
        int c[16], loc = 0, la = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = 16 * t + i;
            c[i] = e < E ? cnt[e] : 0;
            loc += c[i];
            la += (c[i] + kMoeDescPairs - 1) / kMoeDescPairs;
        }
        int incl = loc, inca = la;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d), oa = __shfl_up(inca, d);
            if (t >= d) { incl += o; inca += oa; }
        }
        int o = incl - loc, oa = inca - la;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = 16 * t + i;
            if (e < E) { off[e] = o; act[e] = c[i] > 0 ? oa : -1; }
            o += c[i];
            oa += (c[i] + kMoeDescPairs - 1) / kMoeDescPairs;
        }
        if (t == 63) n_act = inca;
    }
    __syncthreads();
    for (int e = t; e < E; e += blockDim.x)
        if (act[e] >= 0)
            for (int i = 0; i * kMoeDescPairs < cnt[e]; ++i)
                work[act[e] + i] = make_int4(e, off[e] + i * kMoeDescPairs,
                                             min(kMoeDescPairs, cnt[e] - i * kMoeDescPairs), 0);
    // a pair's place inside its expert's list comes from an LDS atomic, in
    // no fixed order: the expert passes compute every pair's outputs from its
    // own activation row alone, so the order changes no result bit
    for (int e = t; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    for (int p = t; p < P; p += blockDim.x) {
        const int e = sid[p];
        if (e >= 0) pairs[off[e] + atomicAdd(&cnt[e], 1)] = p;
    }
    for (int s = n_act + t; s < slots; s += blockDim.x) work[s] = make_int4(-1, 0, 0, 0);
    if (t == 0) work[slots] = make_int4(n_act, 0, 0, 0);
}

__global__ __launch_bounds__(1024) void moe_bucket_kernel(const int32_t* __restrict__ ids, int P,
                                                          int E, int slots, int4* __restrict__ work,
                                                          int32_t* __restrict__ pairs) {
    __shared__ __align__(16) int sid[kMoeMaxPairs];
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const int v = ids[p];
        sid[p] = v >= 0 && v < E ? v : -1;
    }
    __syncthreads();
    bucket_pairs(sid, P, E, slots, work, pairs);
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
    const int4* work;         // [amax + 1] {expert, first pair, pair count <= 16} or {-1, ..}
    const int32_t* pairs;     // [M*k]
    uint16_t* h;              // [M*k][F] bf16
    uint16_t* hs;             // [M][Fs] bf16
    float* part;              // [M*k][D]
    float* sout;              // [M][D]
    int amax;                 // descriptor slots (moe_slots)
    int tiles_r, tiles_s;     // row tiles per routed slot / for the shared expert
};

// Expert passes for M > 1 on the skinny MFMA core: a workgroup owns 16 * WR
// (gate, up) rows or 32 * WR down rows of one active expert (or of the shared
// expert, whose "bucket" is every token), WR wavefronts across its rows times
// WK splitting K, and takes the expert's tokens 16 at a time as the activation
// rows, so each expert's weights are read once per token tile.

template <int S>
__device__ __forceinline__ MfmaTile expert_tile(const MoeMat& W, int e, int row0) {
    return MfmaTile{W.codes + e * W.stride_c, W.scale + e * W.stride_s,
                    Traits<S>::AFFINE ? W.bias + e * W.stride_s : nullptr, row0, W.N};
}

// gate/up: wavefront w gets tiles (gate rows f0 + 16w.., up rows f0 + 16w..), so
// a lane holds g and u of the same (token, f) and writes h = bf16(gelu(g) * u).
template <int S, int WR, int WK, int SL, int DEPTH = 2>
__global__ __launch_bounds__(64 * WR * WK) void moe_gate_up_kernel(MoeArgs a) {
    extern __shared__ __align__(16) uint32_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int bid = blockIdx.x;
    int e = 0, f0, count, first = 0;
    bool shared;
    if (bid < a.amax * a.tiles_r) {
        const int4 w = a.work[bid / a.tiles_r];
        if (w.x < 0) return;  // whole workgroup
        e = w.x;
        f0 = (bid % a.tiles_r) * 16 * WR;
        first = w.y;
        count = w.z;
        shared = false;
    } else {
        f0 = (bid - a.amax * a.tiles_r) * 16 * WR;
        count = a.M;
        shared = true;
    }
    const MoeMat& G = shared ? a.sgate : a.gate;
    const MoeMat& U = shared ? a.sup : a.up;
    const int F = G.N, D = G.K;
    MfmaTile tl[2 * WR];
#pragma unroll
    for (int w = 0; w < WR; ++w) {
        tl[2 * w] = expert_tile<S>(G, e, f0 + 16 * w);
        tl[2 * w + 1] = expert_tile<S>(U, e, f0 + 16 * w);
    }
    for (int t0 = 0; t0 < count; t0 += 16) {
        if (t0) __syncthreads();  // LDS reuse across token tiles
        const int t = min(t0 + c16, count - 1);
        const int tok = shared ? t : a.pairs[first + t] / a.k;
        f32x4_t acc[2];
        mfma_tiles<S, 2, WK, DEPTH, WR, SL>(tl, D, a.x, (uint32_t)tok * (uint32_t)D, lds, acc);
        const int f = f0 + 16 * (wave % WR) + c16;
        if (wave < WR && f < F) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = t0 + 4 * g + r;
                if (m >= count) continue;
                const uint16_t hv = (uint16_t)f32_to_bf16_rne(gelu_tanh(acc[0][r]) * acc[1][r]);
                if (shared) a.hs[(int64_t)m * F + f] = hv;
                else a.h[(int64_t)a.pairs[first + m] * F + f] = hv;
            }
        }
    }
}

// down: wavefront w gets rows n0 + 32w .. of W_down[e] (two tiles) against the
// h rows of the expert's pairs.
template <int S, int WR, int WK, int SL, int DEPTH = 2>
__global__ __launch_bounds__(64 * WR * WK) void moe_down_kernel(MoeArgs a) {
    extern __shared__ __align__(16) uint32_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int bid = blockIdx.x;
    int e = 0, n0, count, first = 0;
    bool shared;
    if (bid < a.amax * a.tiles_r) {
        const int4 w = a.work[bid / a.tiles_r];
        if (w.x < 0) return;  // whole workgroup
        e = w.x;
        n0 = (bid % a.tiles_r) * 32 * WR;
        first = w.y;
        count = w.z;
        shared = false;
    } else {
        n0 = (bid - a.amax * a.tiles_r) * 32 * WR;
        count = a.M;
        shared = true;
    }
    const MoeMat& W = shared ? a.sdown : a.down;
    const int Dm = W.N, F = W.K;
    const uint16_t* hin = shared ? a.hs : a.h;
    MfmaTile tl[2 * WR];
#pragma unroll
    for (int w = 0; w < 2 * WR; ++w) tl[w] = expert_tile<S>(W, e, n0 + 16 * w);
    for (int t0 = 0; t0 < count; t0 += 16) {
        if (t0) __syncthreads();  // LDS reuse across token tiles
        const int t = min(t0 + c16, count - 1);
        const int row = shared ? t : a.pairs[first + t];
        f32x4_t acc[2];
        mfma_tiles<S, 2, WK, DEPTH, WR, SL>(tl, F, hin, (uint32_t)row * (uint32_t)F, lds, acc);
        if (wave >= WR) continue;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int n = n0 + 32 * wave + 16 * rt + c16;
            if (n >= Dm) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = t0 + 4 * g + r;
                if (m >= count) continue;
                if (shared) a.sout[(int64_t)m * Dm + n] = acc[rt][r];
                else a.part[(int64_t)a.pairs[first + m] * Dm + n] = acc[rt][r];
            }
        }
    }
}

// y[m][n] = shared[m][n] + sum_j w[m][j] * part[m*k + j][n]   (fixed j order;
// slots with an id outside [0, E) are skipped). A thread owns 4 consecutive
// outputs (D % 4 == 0); every slot's loads are issued before the first FMA,
// eight slots at a time, and an unused slot's partial (never written: it may
// hold anything) is dropped by a select, not multiplied by zero.
constexpr int kCombineSlots = 8;
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ part,
                                                          const float* __restrict__ sout,
                                                          const float* __restrict__ wts,
                                                          const int32_t* __restrict__ ids, int M,
                                                          int k, int D, int E, int has_shared,
                                                          float* __restrict__ y) {
    const int D4 = D / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * D4) return;
    const int m = (int)(i / D4), n4 = (int)(i % D4);
    const f32x4_t* part4 = reinterpret_cast<const f32x4_t*>(part);
    f32x4_t acc = has_shared ? reinterpret_cast<const f32x4_t*>(sout)[i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += kCombineSlots) {
        int e[kCombineSlots];
        float w[kCombineSlots];
        f32x4_t p[kCombineSlots];
#pragma unroll
        for (int u = 0; u < kCombineSlots; ++u) {
            const int64_t pj = (int64_t)m * k + min(j0 + u, k - 1);
            e[u] = ids[pj];
            w[u] = wts[pj];
            p[u] = part4[pj * D4 + n4];
        }
#pragma unroll
        for (int u = 0; u < kCombineSlots; ++u) {
            const bool use = j0 + u < k && e[u] >= 0 && e[u] < E;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = use ? fmaf(w[u], p[u][r], acc[r]) : acc[r];
        }
    }
    reinterpret_cast<f32x4_t*>(y)[i] = acc;
}

// ---------------------------------------------------------------- host side
static size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

MoeWorkspace moe_workspace_layout(int64_t M, int k, int64_t E, int64_t D, int64_t F, int64_t Fs) {
    MoeWorkspace w{};
    size_t o = 0;
    w.work = o;    o += al(((size_t)moe_slots(E, M * k) + 1) * 16);
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

template <int S, int WR, int WK, int DEPTH>
static void moe_gate_up_launch(MoeArgs a, int64_t Fs, hipStream_t st) {
    const int D = a.gate.K, F = a.gate.N;
    // gate/up: 16 * WR (gate, up) rows per workgroup
    a.tiles_r = (F + 16 * WR - 1) / (16 * WR);
    a.tiles_s = a.has_shared ? (int)((Fs + 16 * WR - 1) / (16 * WR)) : 0;
    const int blocks = a.amax * a.tiles_r + a.tiles_s;
    const size_t lds = gemv_mfma_lds_bytes<S, 2, WK, WR>(D);
    switch (mfma_slices(D / Traits<S>::GROUP)) {
        case 1: hipLaunchKernelGGL((moe_gate_up_kernel<S, WR, WK, 1, DEPTH>), dim3(blocks), dim3(64 * WR * WK), lds, st, a); break;
        case 2: hipLaunchKernelGGL((moe_gate_up_kernel<S, WR, WK, 2, DEPTH>), dim3(blocks), dim3(64 * WR * WK), lds, st, a); break;
        default: hipLaunchKernelGGL((moe_gate_up_kernel<S, WR, WK, 4, DEPTH>), dim3(blocks), dim3(64 * WR * WK), lds, st, a); break;
    }
}

template <int S, int WR, int WK, int DEPTH>
static void moe_down_launch(MoeArgs a, int64_t Fs, hipStream_t st) {
    const int D = a.gate.K, F = a.gate.N;
    // down: 32 * WR rows per workgroup (K = F routed, Fs shared)
    const int64_t Kmax = a.has_shared ? std::max<int64_t>(F, Fs) : F;
    a.tiles_r = (D + 32 * WR - 1) / (32 * WR);
    a.tiles_s = a.has_shared ? a.tiles_r : 0;
    const int blocks = a.amax * a.tiles_r + a.tiles_s;
    const size_t lds = gemv_mfma_lds_bytes<S, 2, WK, WR>(Kmax);
    switch (mfma_slices(Kmax / Traits<S>::GROUP)) {
        case 1: hipLaunchKernelGGL((moe_down_kernel<S, WR, WK, 1, DEPTH>), dim3(blocks), dim3(64 * WR * WK), lds, st, a); break;
        case 2: hipLaunchKernelGGL((moe_down_kernel<S, WR, WK, 2, DEPTH>), dim3(blocks), dim3(64 * WR * WK), lds, st, a); break;
        default: hipLaunchKernelGGL((moe_down_kernel<S, WR, WK, 4, DEPTH>), dim3(blocks), dim3(64 * WR * WK), lds, st, a); break;
    }
}

static GMat gmat(const MoeMat& m) { return GMat{m.codes, m.scale, m.bias, m.stride_c, m.stride_s, m.N, m.K}; }

// Measured on the Gemma-shaped layer at M = 32 over (WR, WK, DEPTH) in
// {1, 2, 4, 8} x {1, 2, 4} x {2, 4}: one row wavefront, two split-K wavefronts
// and four steps in flight read fastest for both passes (by 1-2% over 1, 4,
// 2; wider row blocks, 4-8 row wavefronts, up to 40% slower).
// One launch of moe_routed_kernel over the routed descriptors and/or the
// shared expert's token descriptors, where it applies (rows a multiple of 64,
// K of 128, at most 128 groups per row): false otherwise.
// nw wavefronts per workgroup (gate/up: 4 measured 0.5% over 8)
template <int S, bool GU, int RT, int nw = 4>
static bool moe_routed_launch_rt(const MoeArgs& a, bool routed, bool shared, hipStream_t st) {
    constexpr int rows = 16 * nw * RT;
    MoeRoutedArgs r{};
    int kmax = 0, blocks = 0;
    bool ok = true;
    if (shared) {
        r.S0 = gmat(GU ? a.sgate : a.sdown);
        if (GU) r.S1 = gmat(a.sup);
        ok = ok && r.S0.N % rows == 0 && r.S0.K % 128 == 0;
        kmax = std::max(kmax, r.S0.K);
        blocks += (a.M + kMoeDescPairs - 1) / kMoeDescPairs * (r.S0.N / rows);
    }
    if (routed) {
        r.W0 = gmat(GU ? a.gate : a.down);
        if (GU) r.W1 = gmat(a.up);
        ok = ok && r.W0.N % rows == 0 && r.W0.K % 128 == 0;
        kmax = std::max(kmax, r.W0.K);
        blocks += a.amax * (r.W0.N / rows);
    }
    const int groups = kmax / Traits<S>::GROUP;
    if (!ok || groups > 128) return false;
    const int sg = groups <= 16 ? 16 : groups <= 32 ? 32 : groups <= 64 ? 64 : 128;
    const size_t lds = moe_routed_lds_bytes(kmax, Traits<S>::GROUP, sg, nw, GU ? 2 : RT);
    if (lds > 160 * 1024) return false;
    r.xin = GU ? a.x : a.h;
    r.xsh = GU ? a.x : a.hs;
    r.k = GU ? a.k : 1;
    r.work = a.work;
    r.pairs = a.pairs;
    r.h = a.h;
    r.hs = a.hs;
    r.part = a.part;
    r.sout = a.sout;
    r.M = a.M;
    r.kmax = kmax;
    auto go = [&](auto kern) {
        if (lds > 64 * 1024)
            (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * nw), lds, st, r);
    };
    const bool deep = kmax / 128 >= 4;  // four steps in flight, two for shorter rows
    switch (sg) {
        case 16: deep ? go(moe_routed_kernel<S, GU, 4, 16, RT, nw>) : go(moe_routed_kernel<S, GU, 2, 16, RT, nw>); break;
        case 32: deep ? go(moe_routed_kernel<S, GU, 4, 32, RT, nw>) : go(moe_routed_kernel<S, GU, 2, 32, RT, nw>); break;
        case 64: deep ? go(moe_routed_kernel<S, GU, 4, 64, RT, nw>) : go(moe_routed_kernel<S, GU, 2, 64, RT, nw>); break;
        default: deep ? go(moe_routed_kernel<S, GU, 4, 128, RT, nw>) : go(moe_routed_kernel<S, GU, 2, 128, RT, nw>); break;
    }
    return true;
}

template <int S, bool GU>
static bool moe_routed_launch(const MoeArgs& a, bool routed, bool shared, hipStream_t st) {
    if constexpr (GU) {
        return moe_routed_launch_rt<S, GU, 1>(a, routed, shared, st);
    } else {
        // down: two row tiles per wavefront and eight wavefronts per
        // workgroup, 256 rows (the Gemma-shaped layer at M = 32: one tile,
        // four wavefronts 10.5k tok/s; two tiles 10.9k, then 11.3k with the
        // later changes; eight wavefronts 11.45k; four tiles hold 240
        // registers, one wavefront per SIMD, 9.9k; sixteen wavefronts 11.1k)
        return moe_routed_launch_rt<S, GU, 2, 8>(a, routed, shared, st) ||
               moe_routed_launch_rt<S, GU, 1>(a, routed, shared, st);
    }
}

// A pass: routed and shared descriptors in one launch where one LDS layout
// fits both (measured on the Gemma-shaped layer at M = 32: 8.7k -> 9.5k tok/s
// for gate/up; down, whose shared K = 2048 sizes the layout for routed K =
// 768 too, 3.6% more again), else one launch each; the
// per-expert-block kernel for what the routed kernel does not take.
template <int S, bool GU>
static void moe_pass(const MoeArgs& a, int64_t Fs, hipStream_t st) {
    bool routed = false, shared = false;
    if (a.has_shared) routed = shared = moe_routed_launch<S, GU>(a, true, true, st);
    if (!routed) {
        routed = moe_routed_launch<S, GU>(a, true, false, st);
        shared = a.has_shared && moe_routed_launch<S, GU>(a, false, true, st);
    }
    if (routed && (shared || !a.has_shared)) return;
    MoeArgs b = a;
    if (routed) b.amax = 0;           // its shared blocks only
    if (shared) b.has_shared = 0;     // its routed blocks only
    if (GU) moe_gate_up_launch<S, 1, 2, 4>(b, Fs, st);
    else moe_down_launch<S, 1, 2, 4>(b, Fs, st);
}

// The expert passes for several tokens: each pass on moe_routed_kernel (one
// workgroup per work descriptor and 64 rows, the descriptor's activation
// rows staged in LDS; the shared expert in a launch of its own as
// descriptors of 8 tokens), or where it does not apply on the
// per-expert-block kernel.
template <int S>
static hipError_t moe_passes(const MoeArgs& a, int64_t Fs, hipStream_t st) {
    moe_pass<S, true>(a, Fs, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    moe_pass<S, false>(a, Fs, st);
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
static void go_down1(const Moe1Args& a, int xv, int blocks, size_t lds, hipStream_t st) {
    if (xv == 1)
        hipLaunchKernelGGL((moe1_down_kernel<S, NVD, NVS, 1, 1, 4>), dim3(blocks), dim3(256), lds, st, a);
    else
        hipLaunchKernelGGL((moe1_down_kernel<S, NVD, NVS, 1, 2, 4>), dim3(blocks), dim3(256), lds, st, a);
}

template <int S, int NVD>
static void pick_nvs(int nvs, const Moe1Args& a, int xv, int blocks, size_t lds, hipStream_t st) {
    if (nvs == 0) go_down1<S, NVD, 0>(a, xv, blocks, lds, st);
    else if (nvs == 1) go_down1<S, NVD, 1>(a, xv, blocks, lds, st);
    else go_down1<S, NVD, 2>(a, xv, blocks, lds, st);
}

// Row wavefronts per workgroup of both passes; each also stages a share of its
// pass's activations (x: at most 128 vectors; h and hs: at most 384).
constexpr int kMoe1RW = 4;

template <int S, bool SEL = false>
static hipError_t moe1_passes(Moe1Args a, hipStream_t st) {
    constexpr int R = 2;
    const int kv = Traits<S>::KV;
    a.tiles_r = (a.F + kMoe1RW * R - 1) / (kMoe1RW * R);
    a.tiles_s = a.has_shared ? (a.Fs + kMoe1RW * R - 1) / (kMoe1RW * R) : 0;
    const int blocks = a.k * a.tiles_r + a.tiles_s;
    const size_t lds = (size_t)(a.D / 2 + a.D / kv) * 4;
    if (a.D / kv <= 64)
        hipLaunchKernelGGL((moe1_gate_up_kernel<S, 1, R, 1, kMoe1RW, SEL>), dim3(blocks), dim3(64 * kMoe1RW), lds, st, a);
    else
        hipLaunchKernelGGL((moe1_gate_up_kernel<S, 2, R, 1, kMoe1RW, SEL>), dim3(blocks), dim3(64 * kMoe1RW), lds, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (SEL) {  // the down pass reads the selection the gate/up pass published
        a.ids = a.ids_out;
        a.wts = a.wts_out;
    }
    const int VRF = a.F / kv, VRS = a.has_shared ? a.Fs / kv : 0;
    const int nvd = (VRF + 7) / 8, nvs = (VRS + 63) / 64;
    const int xv = (a.k * VRF + VRS + 64 * kMoe1RW - 1) / (64 * kMoe1RW);
    const size_t lds2 = (size_t)(8 * (a.F / 2 + VRF) + (a.has_shared ? a.Fs / 2 + VRS : 0)) * 4;
    const int blocks2 = (a.D + kMoe1RW - 1) / kMoe1RW;
    switch (nvd) {
        case 1: pick_nvs<S, 1>(nvs, a, xv, blocks2, lds2, st); break;
        case 2: pick_nvs<S, 2>(nvs, a, xv, blocks2, lds2, st); break;
        case 3: pick_nvs<S, 3>(nvs, a, xv, blocks2, lds2, st); break;
        default: pick_nvs<S, 4>(nvs, a, xv, blocks2, lds2, st); break;
    }
    return hipGetLastError();
}

static Moe1Args moe1_args(int scheme, const MoeMats& W, const uint16_t* x, int k, void* ws, float* y) {
    const int64_t E = W.E, D = W.D, F = W.F, Fs = W.Fs;
    const MoeWorkspace L = moe_workspace_layout(1, k, E, D, F, Fs);
    uint8_t* base = (uint8_t*)ws;
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
    a.x = x;
    a.h = (uint16_t*)(base + L.h);
    a.hs = (uint16_t*)(base + L.hs);
    a.y = y;
    return a;
}

hipError_t launch_moe_logits(int scheme, const MoeMats& W, const uint16_t* x, int64_t M,
                             const float* logits, int k, int32_t* ids, float* wts, void* ws,
                             float* y, hipStream_t st) {
    const int64_t E = W.E;
    if (moe1_ok(M, k, W.D, W.F, W.Fs) && E <= 128) {
        Moe1Args a = moe1_args(scheme, W, x, k, ws, y);
        a.logits = logits;
        a.ids_out = ids;
        a.wts_out = wts;
        return scheme == SYM4_G128 ? moe1_passes<SYM4_G128, true>(a, st)
                                   : moe1_passes<AFF4_G64, true>(a, st);
    }
    // otherwise the top-k launch (one wavefront per token, all tokens at
    // once), then the passes for those ids. For several tokens this measured
    // 5.6% faster on the Gemma-shaped layer at M = 32 than selecting and
    // bucketing in one workgroup, whose 16 wavefronts take two tokens each.
    if (E <= 128)
        hipLaunchKernelGGL(topk_softmax_kernel<2>, dim3((unsigned)M), dim3(64), 0, st, logits, (int)E, k, ids, wts);
    else if (E <= 256)
        hipLaunchKernelGGL(topk_softmax_kernel<4>, dim3((unsigned)M), dim3(64), 0, st, logits, (int)E, k, ids, wts);
    else
        hipLaunchKernelGGL(topk_softmax_kernel<16>, dim3((unsigned)M), dim3(64), 0, st, logits, (int)E, k, ids, wts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_moe(scheme, W, x, M, ids, wts, k, ws, y, st);
}

// The M > 1 path after routing: bucketing, the expert passes and the combine.
static hipError_t moe_multi(int scheme, const MoeMats& W, const uint16_t* x, int64_t M,
                            const int32_t* ids, const float* wts, int k, void* ws, float* y,
                            hipStream_t st) {
    const int64_t E = W.E, D = W.D, F = W.F, Fs = W.Fs;
    const MoeWorkspace L = moe_workspace_layout(M, k, E, D, F, Fs);
    uint8_t* base = (uint8_t*)ws;
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
    a.work = (const int4*)(base + L.work);
    a.pairs = (const int32_t*)(base + L.pairs);
    a.h = (uint16_t*)(base + L.h);
    a.hs = (uint16_t*)(base + L.hs);
    a.part = (float*)(base + L.part);
    a.sout = (float*)(base + L.sout);
    a.amax = moe_slots(E, M * k);
    const int P = (int)(M * k);
    hipLaunchKernelGGL(moe_bucket_kernel, dim3(1), dim3(1024), 0, st, ids, P, (int)E, a.amax,
                       (int4*)(base + L.work), (int32_t*)(base + L.pairs));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = scheme == SYM4_G128 ? moe_passes<SYM4_G128>(a, Fs, st) : moe_passes<AFF4_G64>(a, Fs, st);
    if (e != hipSuccess) return e;
    const int64_t tot = M * D / 4;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                       a.part, a.sout, wts, ids, (int)M, k, (int)D, (int)E, a.has_shared, y);
    return hipGetLastError();
}

hipError_t launch_moe(int scheme, const MoeMats& W, const uint16_t* x, int64_t M, const int32_t* ids,
                      const float* wts, int k, void* ws, float* y, hipStream_t st) {
    if (moe1_ok(M, k, W.D, W.F, W.Fs)) {
        Moe1Args a = moe1_args(scheme, W, x, k, ws, y);
        a.ids = ids;
        a.wts = wts;
        return scheme == SYM4_G128 ? moe1_passes<SYM4_G128>(a, st) : moe1_passes<AFF4_G64>(a, st);
    }
    return moe_multi(scheme, W, x, M, ids, wts, k, ws, y, st);
}

}  // namespace w4
