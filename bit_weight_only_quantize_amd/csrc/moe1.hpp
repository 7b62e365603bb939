// Single-token MoE expert passes (M = 1, top_k <= 8): two launches per layer,
// no bucketing and no partial buffers.
//
// TurboFieldfare article (model section, 量化和精度): 8 experts of 128 per token,
// a shared expert added without a routing weight, shared and routed FFNs side
// by side. Both passes follow the wave-per-row GEMV design: weight loads issued
// up front; every row wavefront stages a share of the activations into LDS,
// issuing those loads after the (small) routing loads and before its weight
// loads, so the activation latency overlaps the routing latency and waiting
// for the activations does not wait for the weights.
//
// gate/up pass: blocks cover (slot j < k or the shared expert) x row tiles; a
//   row wavefront owns R (gate row n, up row n) pairs and writes
//   h[j][n] = bf16(gelu_tanh(g) * u) from its reduction lane.
// down pass (+ combine): a row wavefront owns R output rows n; its 64 lanes are
//   8 groups of 8, group g reads row n of W_down[ids[g]] (K = F), every lane also
//   reads row n of the shared down projection (K = Fs). In-wave reduction:
//   y[n] = sum_lanes( shared partial + [lane is its group's first] * w_g * group_sum )
//   -- a fixed order, so the result is reproducible bit for bit.
#pragma once

#include "common.hpp"
#include "gemv_wave.hpp"
#include "skinny.hpp"
#include "topk.hpp"

namespace w4 {

struct Moe1Mat {
    const uint8_t* codes;
    const uint8_t* scale;
    const uint8_t* bias;
    int64_t stride_c, stride_s;  // bytes between experts
};

struct Moe1Args {
    Moe1Mat gate, up, down, sgate, sup, sdown;
    int has_shared, k, E, D, F, Fs;
    const uint16_t* x;   // [D]
    const int32_t* ids;  // [k]
    const float* wts;    // [k]
    // selection inside the gate/up pass (SEL): router logits [E] in, the
    // selected ids and weights out (written by workgroup 0)
    const float* logits;
    int32_t* ids_out;
    float* wts_out;
    uint16_t* h;         // [k][F] bf16
    uint16_t* hs;        // [Fs] bf16
    float* y;            // [D]
    int tiles_r, tiles_s;
};

template <int S>
__device__ __forceinline__ void m1_row(const Moe1Mat& W, int e, int64_t n, int K, const uint8_t*& c,
                                       const uint8_t*& s, const uint8_t*& b) {
    using T = Traits<S>;
    const int64_t groups = K / T::GROUP;
    constexpr int SB = T::AFFINE ? 2 : 4;
    c = W.codes + e * W.stride_c + n * K / 2;
    s = W.scale + e * W.stride_s + n * groups * SB;
    b = T::AFFINE ? W.bias + e * W.stride_s + n * groups * 2 : nullptr;
}

template <int S>
__device__ __forceinline__ void m1_scale(const uint8_t* s, const uint8_t* b, int g, float& sc,
                                         float& bi) {
    if constexpr (Traits<S>::AFFINE) {
        sc = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(s)[g]);
        bi = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(b)[g]);
    } else {
        sc = reinterpret_cast<const float*>(s)[g];
        bi = 0.f;
    }
}

// ---------------------------------------------------------------- gate/up
// SEL: the workgroup selects the token's experts itself from the router
// logits (E <= 128, the same top-k as the routing kernel, by ranks over the
// workgroup's threads), so no launch of its own is needed for the selection;
// workgroup 0 publishes the selection for the down pass and the caller.
template <int S, int NV, int R, int XV, int RW, bool SEL>
__global__ __launch_bounds__(64 * RW) void moe1_gate_up_kernel(Moe1Args a) {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    extern __shared__ __align__(16) uint32_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int D = a.D, VR = D / T::KV;
    const int bid = blockIdx.x;
    const bool shared = bid >= a.k * a.tiles_r;
    const int slot = shared ? 0 : bid / a.tiles_r;
    const int tile = shared ? bid - a.k * a.tiles_r : bid % a.tiles_r;
    // the expert id (or the router logits it is selected from), then this
    // wavefront's share of the activations (they do not depend on the id), then
    // the weights: the loads drain in issue order, so waiting for the first
    // ones does not wait for the later ones
    int e = 0;
    if constexpr (!SEL) e = shared ? 0 : a.ids[slot];
    float lt = 0.f, l64 = 0.f;
    if constexpr (SEL) {
        const float* lgt = a.logits;
        if (!shared) topk_ranked_load([&](int e) { return lgt[e]; }, a.E, lt, l64);  // block-uniform
    }
    XStage<S, XV, 64 * RW> xstage;
    xstage.fetch(a.x, VR, threadIdx.x);
    asm volatile("" ::: "memory");  // keep the weight loads behind these
    if constexpr (SEL) {
        if (!shared) {  // block-uniform
            __shared__ int32_t sel_id[8];
            __shared__ float sel_w[8];
            __shared__ uint64_t keys[128];
            __shared__ int part[256];
            __shared__ float stat[2];
            topk_ranked_select(lt, l64, a.E, a.k, sel_id, sel_w, keys, part, stat);
            __syncthreads();
            e = sel_id[slot];
            if (bid == 0 && (int)threadIdx.x < a.k) {
                a.ids_out[threadIdx.x] = sel_id[threadIdx.x];
                a.wts_out[threadIdx.x] = sel_w[threadIdx.x];
            }
        }
    }
    if (!shared && (e < 0 || e >= a.E)) return;  // whole block: nothing routed to this slot
    const int N = shared ? a.Fs : a.F;
    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + D / 2);
    const Moe1Mat& G = shared ? a.sgate : a.gate;
    const Moe1Mat& U = shared ? a.sup : a.up;
    const int row0 = tile * RW * R + wave * R;
    u32x4_t c[2 * R][NV];
    float sc[2 * R][NV], bi[2 * R][NV];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = min(row0 + r, N - 1);
#pragma unroll
        for (int gu = 0; gu < 2; ++gu) {
            const uint8_t *cp, *sp, *bp;
            m1_row<S>(gu ? U : G, e, n, D, cp, sp, bp);
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int v = min(lane + 64 * j, VR - 1);
                c[2 * r + gu][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cp) + v);
                m1_scale<S>(sp, bp, v / T::VPG, sc[2 * r + gu][j], bi[2 * r + gu][j]);
            }
        }
    }
    xstage.commit(VR, xs, XS, threadIdx.x);  // waits for the activations only
    __syncthreads();  // activations staged; weight loads still in flight
    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    float acc[2 * R];
#pragma unroll
    for (int q = 0; q < 2 * R; ++q) acc[q] = 0.f;
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
    uint16_t* out = shared ? a.hs : a.h + (int64_t)slot * a.F;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float g = wave_sum_to_lane63(acc[2 * r]);
        const float u = wave_sum_to_lane63(acc[2 * r + 1]);
        if (lane == 63 && row0 + r < N)
            out[row0 + r] = (uint16_t)f32_to_bf16_rne(gelu_tanh(g) * u);
    }
}

// ---------------------------------------------------------------- down + combine
// LDS: 8 slot regions of (F/2 pair dwords + F/KV sums), then the shared region.
// The k slot rows of h and the shared row hs are staged by all RW wavefronts,
// XV 16-element vectors per thread.
template <int S, int NVD, int NVS, int R, int XV, int RW>
__global__ __launch_bounds__(64 * RW) void moe1_down_kernel(Moe1Args a) {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    constexpr int Q = T::BITS == 4 ? 4 : 2;
    constexpr int NT = 64 * RW;
    extern __shared__ __align__(16) uint32_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int F = a.F, Fs = a.Fs, D = a.D, k = a.k;
    const int VRF = F / T::KV, VRS = a.has_shared ? Fs / T::KV : 0;
    const int regw = F / 2 + VRF;  // dwords per slot region
    uint32_t* sbase = smem + 8 * regw;

    // routing of this lane's slot group first, then this thread's share of h
    // and hs and the shared expert's rows (independent of the routing), then
    // the routed rows. The routing loads are unconditional (clamped slot) and
    // the slot test comes at use: a load under it would compile into a branch
    // whose join waits for it before anything else is issued.
    const int g = lane >> 3, sl = lane & 7;
    const int gq = max(min(g, k - 1), 0);
    int e = a.ids[gq];
    const float w_raw = a.wts[gq];
    const int total = k * VRF + VRS;
    u32x4_t d[XV][Q];
#pragma unroll
    for (int t = 0; t < XV; ++t) {
        const int i = min((int)threadIdx.x + NT * t, total - 1);
        const uint16_t* src = i < k * VRF ? a.h + (int64_t)(i / VRF) * F + (i % VRF) * T::KV
                                          : a.hs + (int64_t)(i - k * VRF) * T::KV;
#pragma unroll
        for (int q = 0; q < Q; ++q) d[t][q] = reinterpret_cast<const u32x4_t*>(src)[q];
    }
    asm volatile("" ::: "memory");  // keep the weight loads behind these
    const int row0 = blockIdx.x * RW * R + wave * R;
    u32x4_t cr[R][NVD], cs[R][NVS > 0 ? NVS : 1];
    float sr[R][NVD], br[R][NVD], ss[R][NVS > 0 ? NVS : 1], bs[R][NVS > 0 ? NVS : 1];
    if constexpr (NVS > 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t n = min(row0 + r, D - 1);
            const uint8_t *cp, *sp, *bp;
            m1_row<S>(a.sdown, 0, n, Fs, cp, sp, bp);
#pragma unroll
            for (int t = 0; t < NVS; ++t) {
                const int v = min(lane + 64 * t, VRS - 1);
                cs[r][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cp) + v);
                m1_scale<S>(sp, bp, v / T::VPG, ss[r][t], bs[r][t]);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // nothing that waits for the routing moves above this
    const bool valid = g < k && e >= 0 && e < a.E;
    const float wg = valid ? w_raw : 0.f;
    if (!valid) e = 0;  // a readable expert; its contribution is multiplied by 0
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = min(row0 + r, D - 1);
        const uint8_t *cp, *sp, *bp;
        m1_row<S>(a.down, e, n, F, cp, sp, bp);
#pragma unroll
        for (int t = 0; t < NVD; ++t) {
            const int v = min(sl + 8 * t, VRF - 1);
            cr[r][t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cp) + v);
            m1_scale<S>(sp, bp, v / T::VPG, sr[r][t], br[r][t]);
        }
    }
    // commit the staged rows (waits for them only; the weights stay in flight)
    {
        constexpr uint32_t ONES = 0x3F803F80u;
#pragma unroll
        for (int t = 0; t < XV; ++t) {
            const int i = (int)threadIdx.x + NT * t;
            if (i >= total) break;
            const bool sh = i >= k * VRF;
            uint32_t* reg = sh ? sbase : smem + (i / VRF) * regw;
            const int v = sh ? i - k * VRF : i % VRF;
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const u32x4_t ev = d[t][q];
                uint4 o;
                if constexpr (T::BITS == 4) {
                    o.x = __builtin_amdgcn_perm(ev[2], ev[0], 0x05040100u);
                    o.y = __builtin_amdgcn_perm(ev[2], ev[0], 0x07060302u);
                    o.z = __builtin_amdgcn_perm(ev[3], ev[1], 0x05040100u);
                    o.w = __builtin_amdgcn_perm(ev[3], ev[1], 0x07060302u);
                } else {
                    o.x = __builtin_amdgcn_perm(ev[1], ev[0], 0x05040100u);
                    o.y = __builtin_amdgcn_perm(ev[1], ev[0], 0x07060302u);
                    o.z = __builtin_amdgcn_perm(ev[3], ev[2], 0x05040100u);
                    o.w = __builtin_amdgcn_perm(ev[3], ev[2], 0x07060302u);
                }
                *reinterpret_cast<uint4*>(reg + L::piece(v, q)) = o;
                sum = dot2_bf16(ONES, ev[0], sum);
                sum = dot2_bf16(ONES, ev[1], sum);
                sum = dot2_bf16(ONES, ev[2], sum);
                sum = dot2_bf16(ONES, ev[3], sum);
            }
            reinterpret_cast<float*>(reg + (sh ? Fs / 2 : F / 2))[v] = sum;
        }
    }
    __syncthreads();
    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    const uint32_t* xr = smem + g * regw;
    const float* XR = reinterpret_cast<const float*>(xr + F / 2);
    const float* XSS = reinterpret_cast<const float*>(sbase + Fs / 2);
    float accr[R], accs[R];
#pragma unroll
    for (int r = 0; r < R; ++r) accr[r] = accs[r] = 0.f;
#pragma unroll
    for (int t = 0; t < NVD; ++t) {
        const int v = sl + 8 * t;
        if (v >= VRF || !valid) break;  // an empty slot contributes exactly 0
        uint32_t xp[L::XW];
        read_pairs<S>(xr, v, xp);
        const float X = XR[v];
#pragma unroll
        for (int r = 0; r < R; ++r)
            accr[r] = apply_group<S>(accr[r], dot_code_vector<S>(cr[r][t], xp, MASK, MAGIC), X,
                                     sr[r][t], br[r][t]);
    }
    if constexpr (NVS > 0) {
#pragma unroll
        for (int t = 0; t < NVS; ++t) {
            const int v = lane + 64 * t;
            if (v >= VRS) break;
            uint32_t xp[L::XW];
            read_pairs<S>(sbase, v, xp);
            const float X = XSS[v];
#pragma unroll
            for (int r = 0; r < R; ++r)
                accs[r] = apply_group<S>(accs[r], dot_code_vector<S>(cs[r][t], xp, MASK, MAGIC), X,
                                         ss[r][t], bs[r][t]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        // sum over the 8 lanes of the slot group (every lane of the group gets it)
        float d = accr[r];
        d += dpp_f<0xB1, 0xF>(d);
        d += dpp_f<0x4E, 0xF>(d);
        d += dpp_f<0x141, 0xF>(d);
        const float v = accs[r] + (sl == 0 ? wg * d : 0.f);
        const float tot = wave_sum_to_lane63(v);
        if (lane == 63 && row0 + r < D) a.y[row0 + r] = tot;
    }
}

}  // namespace w4
