// One-token MoE layer in a single launch: router GEMV, top-k, shared and routed
// gate/up, and the down projections with the weighted combine.
//
// TurboFieldfare article (Gemma 4 26B-A4B section, 量化和精度): 128 routed
// experts, 8 chosen per token by an 8-bit router with no softcap; a shared expert
// added without routing weight; shared and routed FFNs side by side. Its M2
// time table puts 55.6 of 162.8 ms per token in command-buffer waits; the
// analogue here is the fill and drain of dependent launches, which this path
// replaces by hand-offs between the workgroups of one launch.
//
// Work is an ordered list of items, walked by a persistent grid no larger than
// what the GPU holds at once (occupancy API x CUs), each workgroup taking
// items blockIdx.x, blockIdx.x + gridDim.x, ... in increasing order:
//   [router rows] [shared gate/up rows] [routed gate/up rows] [down rows]
// An item only ever waits for items with smaller indices. With every
// workgroup resident, the smallest waiting item's producers are all running
// (or done), so every wait ends; a wait is also bounded (a poll limit the host
// can set) and a workgroup that gives up records it in an error word and
// carries on without the missing input, so the kernel always exits. The
// launch is refused (and the caller takes the launch sequence) if the kernel
// needs scratch: scratch-backed waves are rationed by the runtime in a way the
// occupancy query does not see, so residency would not be guaranteed.
//
//   router item   8 router rows (wave-per-row GEMV, activations staged in
//                 LDS), each logit stored with a "written" mark; the first
//                 router item then polls all E logits, runs the top-k and
//                 stores the ids and weights, marked, into kSyncRep replicas
//   gate/up item  8 (gate, up) row pairs of the shared expert (no wait) or of
//                 the expert in one routed slot (once its id is in the
//                 replica the item polls): h = bf16(gelu_tanh(g) * u), stored
//                 in kHRep copies; then a split count of finished items whose
//                 completion raises a replicated "every h row in" flag
//   down item     8 output rows: issues its shared-down row loads, polls the
//                 selection, issues the down-row loads of the k selected
//                 experts, then waits for every h row, stages one copy of h in
//                 LDS and reduces y[n] = shared(n) + sum_j w_j * down_j(n) in a
//                 fixed order
// Hand-offs follow handoff.hpp (device-scope atomic stores and loads, split
// counters, replicated flags). Polling the hand-off data itself from every
// thread instead of one poller per workgroup floods the coherent path (3x
// slower). The last workgroup to finish resets the hand-off words, so each
// call leaves them zero.
#include <algorithm>

#include "common.hpp"
#include "gemv_wave.hpp"
#include "handoff.hpp"
#include "launch.hpp"
#include "moe1.hpp"
#include "skinny.hpp"
#include "topk.hpp"

namespace w4 {

struct LayerArgs {
    const uint8_t* rc;  // router codes, scales, biases ([E][D], 8-bit affine)
    const uint8_t* rs;
    const uint8_t* rb;
    Moe1Mat gate, up, down, sgate, sup, sdown;
    int has_shared, k, E, D, F, Fs;
    const uint16_t* x;  // [D]
    int32_t* ids;       // [k] out
    float* wts;         // [k] out
    uint16_t* h;        // [kHRep][k * F + Fs] bf16: slot rows, then the shared row
    float* y;           // [D] out
    unsigned* sync;     // kLayerSyncWords words (workspace)
    int n_router, n_sgu, n_rgu, n_down, tiles_r;
    long long wait_limit;
    int withhold;       // testing: never publish the selection
};

constexpr int kLayerRW = 4;  // wavefronts per workgroup
constexpr int kLayerThreads = 64 * kLayerRW;
constexpr int kRouterRows = 2 * kLayerRW, kGuRows = 2 * kLayerRW, kDownRows = 2 * kLayerRW;

// Thread 0 polls until the k selection words of its replica line (ids from
// word 0, weights from word kLayerMaxK) are all written, at most `limit`
// times; on success ids and weights land in sid / swt (LDS).
__device__ bool poll_selection(const LayerArgs& a, int k, int32_t* sid, float* swt) {
    const unsigned* line = a.sync + kSyncSel + (blockIdx.x % kSyncRep) * kSyncLine;
    for (long long n = 0;; ++n) {
        uint32_t w[2 * kLayerMaxK];
#pragma unroll
        for (int q = 0; q < kLayerMaxK; ++q) {
            const uint64_t v = get64(line + 2 * q);
            w[2 * q] = (uint32_t)v;
            w[2 * q + 1] = (uint32_t)(v >> 32);
        }
        bool all = true;
#pragma unroll
        for (int j = 0; j < kLayerMaxK; ++j)
            if (j < k) all = all && w[j] != 0 && w[kLayerMaxK + j] != 0;
        if (all) {
#pragma unroll
            for (int j = 0; j < kLayerMaxK; ++j) {
                sid[j] = (int32_t)w[j] - 1;
                swt[j] = __uint_as_float(w[kLayerMaxK + j] & 0x7FFFFFFFu);
            }
            return true;
        }
        if (n >= a.wait_limit) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

// ---------------------------------------------------------------- router item
// Rows item*8 .. item*8+7 of the router; item 0 also selects the experts.
template <int RS, int NVR>
__device__ void router_item(const LayerArgs& a, int item, uint32_t* smem) {
    using T = Traits<RS>;
    using L = XLayout<RS, 1>;
    constexpr int R = 2;
    const int tid = item_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int D = a.D, VR = D / T::KV;
    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + D / 2);
    XStage<RS, 1, kLayerThreads> xstage;  // VR <= 256 vectors
    xstage.fetch(a.x, VR, tid);
    asm volatile("" ::: "memory");
    const int row0 = item * kRouterRows + wave * R;
    const int64_t rowbytes = (int64_t)D * T::BITS / 8, groups = D / T::GROUP;
    constexpr int SB = T::AFFINE ? 2 : 4;
    u32x4_t c[R][NVR];
    float sc[R][NVR], bi[R][NVR];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t n = min(row0 + r, a.E - 1);
        const u32x4_t* cp = reinterpret_cast<const u32x4_t*>(a.rc + n * rowbytes);
        const uint8_t* sp = a.rs + n * groups * SB;
        const uint8_t* bp = T::AFFINE ? a.rb + n * groups * 2 : nullptr;
#pragma unroll
        for (int j = 0; j < NVR; ++j) {
            const int v = min(lane + 64 * j, VR - 1);
            c[r][j] = __builtin_nontemporal_load(cp + v);
            m1_scale<RS>(sp, bp, v / T::VPG, sc[r][j], bi[r][j]);
        }
    }
    xstage.commit(VR, xs, XS, tid);
    __syncthreads();
    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<RS>();
    float acc[R] = {};
#pragma unroll
    for (int j = 0; j < NVR; ++j) {
        const int v = lane + 64 * j;
        if (v >= VR) break;
        uint32_t xp[L::XW];
        read_pairs<RS>(xs, v, xp);
        const float X = XS[v];
#pragma unroll
        for (int r = 0; r < R; ++r)
            acc[r] = apply_group<RS>(acc[r], dot_code_vector<RS>(c[r][j], xp, MASK, MAGIC), X,
                                     sc[r][j], bi[r][j]);
    }
    unsigned* lg = a.sync + kSyncLogits;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float tot = wave_sum_to_lane63(acc[r]);
        if (lane == 63 && row0 + r < a.E)
            put64(lg + 2 * (row0 + r), (uint64_t)__float_as_uint(tot) | (1ull << 32));
    }
    if (item != 0 || wave != 0) return;
    // item 0, one wavefront: wait for every logit, select, publish
    uint64_t p[2];
    bool ok = false;
    for (long long n = 0;; ++n) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = lane + 64 * j;
            p[j] = e < a.E ? get64(lg + 2 * e) : (1ull << 32);
        }
        ok = __all((p[0] >> 32) != 0 && (p[1] >> 32) != 0);
        if (ok || n >= a.wait_limit) break;
        __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) {
        if (lane == 0) atomicOr(a.sync + kSyncErr, kGaveUpLogits);
        return;
    }
    __shared__ int32_t sel_id[kLayerMaxK];
    __shared__ float sel_w[kLayerMaxK];
    float v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) v[j] = lane + 64 * j < a.E ? __uint_as_float((uint32_t)p[j]) : -INFINITY;
    topk_rounds<2>(v, a.E, a.k, sel_id, sel_w);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (lane < a.k) {
        a.ids[lane] = sel_id[lane];
        a.wts[lane] = sel_w[lane];
    }
    if (a.withhold) return;
    // kSyncRep replicas x (k ids + 1, k weights with bit 31 set): never zero
    for (int t = lane; t < kSyncRep * 2 * kLayerMaxK; t += 64) {
        const int r = t / (2 * kLayerMaxK), w = t % (2 * kLayerMaxK), j = w % kLayerMaxK;
        if (j >= a.k) continue;
        const uint32_t val = w < kLayerMaxK ? (uint32_t)(sel_id[j] + 1)
                                            : (__float_as_uint(sel_w[j]) | 0x80000000u);
        put32(a.sync + kSyncSel + r * kSyncLine + w, val);
    }
}

// ---------------------------------------------------------------- gate/up item
// 8 (gate, up) row pairs: tile t of the shared expert (shared) or of the
// expert in routed slot `slot`. `item`: this item's index among the gate/up
// items (for the split count).
template <int S, int NV>
__device__ void gate_up_item(const LayerArgs& a, bool shared, int slot, int tile, int item,
                             uint32_t* smem, int* sflag) {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    constexpr int R = 2;
    const int tid = item_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int D = a.D, VR = D / T::KV;
    uint32_t* xs = smem;
    float* XS = reinterpret_cast<float*>(smem + D / 2);
    XStage<S, 1, kLayerThreads> xstage;
    xstage.fetch(a.x, VR, tid);
    asm volatile("" ::: "memory");
    int e = 0;
    bool live = true;
    if (!shared) {
        if (threadIdx.x == 0) {
            const unsigned* w = a.sync + kSyncSel + (blockIdx.x % kSyncRep) * kSyncLine + slot;
            int id = -1;
            for (long long n = 0;; ++n) {
                const uint32_t v = get32(w);
                if (v != 0) { id = (int)v - 1; break; }
                if (n >= a.wait_limit) break;
                __builtin_amdgcn_s_sleep(2);
            }
            if (id < 0) atomicOr(a.sync + kSyncErr, kGaveUpIds);
            *sflag = id;
        }
        __syncthreads();
        e = *sflag;
        __syncthreads();
        live = e >= 0 && e < a.E;  // gave up, or an id outside the stack: nothing to compute
    }
    if (live) {
        const int N = shared ? a.Fs : a.F;
        const Moe1Mat& G = shared ? a.sgate : a.gate;
        const Moe1Mat& U = shared ? a.sup : a.up;
        const int row0 = tile * kGuRows + wave * R;
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
        xstage.commit(VR, xs, XS, tid);
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
        // the wavefront's two rows are adjacent (row0 even, N a multiple of the
        // group): one 32-bit coherent store per copy of h
        uint32_t pair = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float g = wave_sum_to_lane63(acc[2 * r]);
            const float u = wave_sum_to_lane63(acc[2 * r + 1]);
            pair |= f32_to_bf16_rne(gelu_tanh(g) * u) << (16 * r);
        }
        const int64_t hrow = (int64_t)a.k * a.F + a.Fs;
        uint16_t* out = a.h + (shared ? (int64_t)a.k * a.F : (int64_t)slot * a.F) + row0;
        if (lane == 63 && row0 < N) {
#pragma unroll
            for (int c2 = 0; c2 < kHRep; ++c2) put32(out + c2 * hrow, pair);
        }
    }
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) *sflag = split_count(a.sync, kSyncHSub, kSyncHTop, item, a.n_sgu + a.n_rgu);
    __syncthreads();
    if (*sflag && threadIdx.x < kSyncRep)  // every h row is in
        put32(a.sync + kSyncHDoneRep + threadIdx.x * kSyncLine, 1u);
}

// ---------------------------------------------------------------- down item
// Output rows item*8 .. item*8+7: a wavefront owns two rows; its lanes are 8
// groups of 8, group g reading the rows of slot g's down matrix (K = F), every
// lane also reading the shared down rows (K = Fs). LDS: 8 slot regions of h,
// then hs.
template <int S, int NVD, int NVS>
__device__ void down_item(const LayerArgs& a, int item, uint32_t* smem, int* sflag) {
    using T = Traits<S>;
    using L = XLayout<S, 1>;
    constexpr int Q = 4;  // 16-byte activation pieces per 32-weight code vector
    constexpr int R = 2;
    static_assert(T::BITS == 4, "expert passes take 4-bit codes");
    __shared__ int32_t sid[kLayerMaxK];
    __shared__ float swt[kLayerMaxK];
    const int tid = item_tid();
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int F = a.F, Fs = a.Fs, D = a.D, k = a.k;
    const int VRF = F / T::KV, VRS = a.has_shared ? Fs / T::KV : 0;
    const int regw = F / 2 + VRF;
    uint32_t* sbase = smem + 8 * regw;
    const int row0 = item * kDownRows + wave * R;
    const int g = lane >> 3, sl = lane & 7;
    // the shared rows depend on nothing: their loads go out first
    u32x4_t cs[R][NVS > 0 ? NVS : 1];
    float ss[R][NVS > 0 ? NVS : 1], bs[R][NVS > 0 ? NVS : 1];
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
    asm volatile("" ::: "memory");
    if (threadIdx.x == 0) {
        const bool ok = poll_selection(a, k, sid, swt);
        if (!ok) atomicOr(a.sync + kSyncErr, kGaveUpIds);
        *sflag = ok;
    }
    __syncthreads();
    if (!*sflag) return;  // block-uniform
    int e = g < k ? sid[g] : -1;
    const float w_raw = g < k ? swt[g] : 0.f;
    const bool valid = e >= 0 && e < a.E;
    const float wg = valid ? w_raw : 0.f;
    if (!valid) e = 0;  // a readable expert; its contribution is multiplied by 0
    u32x4_t cr[R][NVD];
    float sr[R][NVD], br[R][NVD];
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
    asm volatile("" ::: "memory");
    const bool have_h = wg_wait_flag(a.sync, a.wait_limit, kSyncHDoneRep, kGaveUpH, sflag);
    // stage one copy of h: the k slot rows and the shared row (16-element vectors)
    const int total = k * VRF + VRS;
    if (have_h) {
        constexpr uint32_t ONES = 0x3F803F80u;
        const uint16_t* hc = a.h + (int64_t)(blockIdx.x % kHRep) * ((int64_t)k * F + Fs);
        for (int i = tid; i < total; i += kLayerThreads) {
            const bool sh = i >= k * VRF;
            const uint16_t* src = sh ? hc + (int64_t)k * F + (int64_t)(i - k * VRF) * T::KV
                                     : hc + (int64_t)(i / VRF) * F + (i % VRF) * T::KV;
            uint32_t* reg = sh ? sbase : smem + (i / VRF) * regw;
            const int v = sh ? i - k * VRF : i % VRF;
            u32x4_t ev[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const uint64_t lo = get64(src + 8 * q), hi = get64(src + 8 * q + 4);
                ev[q] = u32x4_t{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
            }
            float sum = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                uint4 o;
                o.x = __builtin_amdgcn_perm(ev[q][2], ev[q][0], 0x05040100u);
                o.y = __builtin_amdgcn_perm(ev[q][2], ev[q][0], 0x07060302u);
                o.z = __builtin_amdgcn_perm(ev[q][3], ev[q][1], 0x05040100u);
                o.w = __builtin_amdgcn_perm(ev[q][3], ev[q][1], 0x07060302u);
                *reinterpret_cast<uint4*>(reg + L::piece(v, q)) = o;
                sum = dot2_bf16(ONES, ev[q][0], sum);
                sum = dot2_bf16(ONES, ev[q][1], sum);
                sum = dot2_bf16(ONES, ev[q][2], sum);
                sum = dot2_bf16(ONES, ev[q][3], sum);
            }
            reinterpret_cast<float*>(reg + (sh ? Fs / 2 : F / 2))[v] = sum;
        }
    }
    __syncthreads();
    if (!have_h) return;  // block-uniform
    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    const uint32_t* xr = smem + g * regw;
    const float* XR = reinterpret_cast<const float*>(xr + F / 2);
    const float* XSS = reinterpret_cast<const float*>(sbase + Fs / 2);
    float accr[R] = {}, accs[R] = {};
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
        float d = accr[r];
        d += dpp_f<0xB1, 0xF>(d);
        d += dpp_f<0x4E, 0xF>(d);
        d += dpp_f<0x141, 0xF>(d);
        const float v = accs[r] + (sl == 0 ? wg * d : 0.f);
        const float tot = wave_sum_to_lane63(v);
        if (lane == 63 && row0 + r < D) a.y[row0 + r] = tot;
    }
}

// ---------------------------------------------------------------- the kernel
template <int S, int RS, int NVR, int NV, int NVD, int NVS>
__global__ __launch_bounds__(kLayerThreads, 4) void moe_layer_kernel(LayerArgs a) {
    extern __shared__ __align__(16) uint32_t smem[];
    __shared__ int sflag;
    const int n0 = a.n_router, n1 = n0 + a.n_sgu, n2 = n1 + a.n_rgu, n3 = n2 + a.n_down;
    for (int it = blockIdx.x; it < n3; it += gridDim.x) {
        if (it < n0) router_item<RS, NVR>(a, it, smem);
        else if (it < n1) gate_up_item<S, NV>(a, true, 0, it - n0, it - n0, smem, &sflag);
        else if (it < n2) gate_up_item<S, NV>(a, false, (it - n1) / a.tiles_r, (it - n1) % a.tiles_r, it - n0, smem, &sflag);
        else down_item<S, NVD, NVS>(a, it - n2, smem, &sflag);
        __syncthreads();  // LDS and sflag reuse by the next item
    }
    // the last workgroup out resets the hand-off words and reports this call's
    // give-ups (if any) in the status word
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
        for (int w = lane; w < 2 * kLayerMaxE; w += 64) put32(a.sync + kSyncLogits + w, 0u);
        for (int w = lane; w < kSyncRep * 2 * kLayerMaxK; w += 64)
            put32(a.sync + kSyncSel + (w / (2 * kLayerMaxK)) * kSyncLine + w % (2 * kLayerMaxK), 0u);
        if (lane < kSyncRep) {
            put32(a.sync + kSyncHSub + lane * kSyncLine, 0u);
            put32(a.sync + kSyncHDoneRep + lane * kSyncLine, 0u);
            put32(a.sync + kSyncExitSub + lane * kSyncLine, 0u);
        }
    }
}

// ---------------------------------------------------------------- host side
bool moe_layer_ok(int rscheme, int k, int64_t E, int64_t D, int64_t F, int64_t Fs) {
    return rscheme == AFF8_G64 && k >= 1 && k <= kLayerMaxK && E >= k && E <= kLayerMaxE &&
           D >= 2048 && D <= 4096 && F >= 32 && F <= 1024 && Fs <= 4096 && (Fs == 0 || Fs >= 32);
}

static size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

MoeLayerWorkspace moe_layer_workspace_layout(int64_t M, int k, int64_t E, int64_t D, int64_t F,
                                             int64_t Fs) {
    MoeLayerWorkspace w{};
    size_t o = 0;
    w.sync = o;   o += al256(kLayerSyncWords * 4);
    w.h = o;      o += al256((size_t)kHRep * ((size_t)k * F + Fs) * 2);
    w.multi = o;  o += al256((size_t)M * E * 4) + moe_workspace_layout(M, k, E, D, F, Fs).total;
    w.total = o;
    return w;
}

template <int S, int RS, int NVR, int NV, int NVD, int NVS>
static hipError_t go_layer(const LayerArgs& a, size_t lds, hipStream_t st) {
    auto kern = moe_layer_kernel<S, RS, NVR, NV, NVD, NVS>;
    hipError_t e = hipSuccess;
    const int grid = persistent_grid((const void*)kern, kLayerThreads, lds,
                                     a.n_router + a.n_sgu + a.n_rgu + a.n_down, &e);
    if (grid < 1) return e;  // nothing launched
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kLayerThreads), lds, st, a);
    return hipGetLastError();
}

template <int S, int RS, int NVR, int NV, int NVD>
static hipError_t pick_nvs(int nvs, const LayerArgs& a, size_t lds, hipStream_t st) {
    if (nvs == 0) return go_layer<S, RS, NVR, NV, NVD, 0>(a, lds, st);
    if (nvs == 1) return go_layer<S, RS, NVR, NV, NVD, 1>(a, lds, st);
    return go_layer<S, RS, NVR, NV, NVD, 2>(a, lds, st);
}

template <int S, int RS, int NVR, int NV>
static hipError_t pick_nvd(int nvd, int nvs, const LayerArgs& a, size_t lds, hipStream_t st) {
    switch (nvd) {
        case 1: return pick_nvs<S, RS, NVR, NV, 1>(nvs, a, lds, st);
        case 2: return pick_nvs<S, RS, NVR, NV, 2>(nvs, a, lds, st);
        case 3: return pick_nvs<S, RS, NVR, NV, 3>(nvs, a, lds, st);
        default: return pick_nvs<S, RS, NVR, NV, 4>(nvs, a, lds, st);
    }
}

// D = 2048: one 4-bit code vector per lane and row for gate/up, two 8-bit ones
// for the router; D in (2048, 4096]: twice that.
template <int S>
static hipError_t pick_layer(const LayerArgs& a, size_t lds, hipStream_t st) {
    const int VRF = a.F / Traits<S>::KV, VRS = a.has_shared ? a.Fs / Traits<S>::KV : 0;
    const int nvd = (VRF + 7) / 8, nvs = (VRS + 63) / 64;
    if (a.D <= 2048) return pick_nvd<S, AFF8_G64, 2, 1>(nvd, nvs, a, lds, st);
    return pick_nvd<S, AFF8_G64, 4, 2>(nvd, nvs, a, lds, st);
}

hipError_t launch_moe_layer(int scheme, int rscheme, const MoeMats& W, const void* const* router,
                            const uint16_t* x, int k, int32_t* ids, float* wts, void* ws,
                            float* y, long long wait_limit, int withhold, hipStream_t st) {
    if (rscheme != AFF8_G64) return hipErrorNotSupported;  // the fused path takes an 8-bit router
    const int64_t E = W.E, D = W.D, F = W.F, Fs = W.Fs;
    const MoeLayerWorkspace L = moe_layer_workspace_layout(1, k, E, D, F, Fs);
    uint8_t* base = (uint8_t*)ws;
    auto m1 = [&](const void* const* t, int64_t N, int64_t K) {
        const int64_t groups = K / (scheme == SYM4_G128 ? 128 : 64);
        Moe1Mat m{};
        m.codes = (const uint8_t*)t[0];
        m.scale = (const uint8_t*)t[1];
        m.bias = (const uint8_t*)t[2];
        m.stride_c = N * K / 2;
        m.stride_s = N * groups * (scheme == SYM4_G128 ? 4 : 2);
        return m;
    };
    LayerArgs a{};
    a.rc = (const uint8_t*)router[0];
    a.rs = (const uint8_t*)router[1];
    a.rb = (const uint8_t*)router[2];
    a.gate = m1(W.gate, F, D);
    a.up = m1(W.up, F, D);
    a.down = m1(W.down, D, F);
    a.has_shared = Fs > 0;
    if (Fs > 0) {
        a.sgate = m1(W.sgate, Fs, D);
        a.sup = m1(W.sup, Fs, D);
        a.sdown = m1(W.sdown, D, Fs);
    }
    a.k = k; a.E = (int)E; a.D = (int)D; a.F = (int)F; a.Fs = (int)Fs;
    a.x = x;
    a.ids = ids;
    a.wts = wts;
    a.h = (uint16_t*)(base + L.h);
    a.y = y;
    a.sync = (unsigned*)(base + L.sync);
    a.n_router = (int)((E + kRouterRows - 1) / kRouterRows);
    a.n_sgu = Fs > 0 ? (int)((Fs + kGuRows - 1) / kGuRows) : 0;
    a.tiles_r = (int)((F + kGuRows - 1) / kGuRows);
    a.n_rgu = k * a.tiles_r;
    a.n_down = (int)((D + kDownRows - 1) / kDownRows);
    a.wait_limit = wait_limit;
    a.withhold = withhold;
    const int kvr = 16, kv = 32;
    const size_t lds_router = (size_t)(D / 2 + D / kvr) * 4;
    const size_t lds_gu = (size_t)(D / 2 + D / kv) * 4;
    const size_t lds_down = (size_t)(8 * (F / 2 + F / kv) + (Fs > 0 ? Fs / 2 + Fs / kv : 0)) * 4;
    const size_t lds = std::max({lds_router, lds_gu, lds_down});
    return scheme == SYM4_G128 ? pick_layer<SYM4_G128>(a, lds, st) : pick_layer<AFF4_G64>(a, lds, st);
}

}  // namespace w4
