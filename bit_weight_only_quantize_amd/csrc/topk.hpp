// Router top-k in one wavefront, shared by the routing kernels and the
// single-token expert pass that selects its own experts.
//
// TurboFieldfare article (Gemma 4 26B-A4B section): 8 experts of 128 chosen
// per token by the router's logits, softmax weights, no softcap.
#pragma once

#include "common.hpp"

namespace w4 {

// Wave-wide reductions over DPP (row steps, then row_bcast15/31 into lane 63)
// and a readlane broadcast: no LDS round trips. Lanes a DPP step does not
// write keep their own value (old = src), the identity for max and min.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_keep(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, ROW_MASK, 0xF, false);
}
template <typename Op>
__device__ __forceinline__ int wave_reduce_i(int v, Op op) {
    v = op(v, dpp_keep<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
    v = op(v, dpp_keep<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
    v = op(v, dpp_keep<0x141, 0xF>(v));  // row_half_mirror
    v = op(v, dpp_keep<0x140, 0xF>(v));  // row_mirror
    v = op(v, dpp_keep<0x142, 0xA>(v));  // row_bcast15
    v = op(v, dpp_keep<0x143, 0xC>(v));  // row_bcast31
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_max_dpp(float v) {
    return __int_as_float(wave_reduce_i(__float_as_int(v), [](int a, int b) {
        return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
    }));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
    return __int_as_float(wave_reduce_i(__float_as_int(v), [](int a, int b) {
        return __float_as_int(__int_as_float(a) + __int_as_float(b));
    }));
}
__device__ __forceinline__ int wave_min_dpp(int v) {
    return wave_reduce_i(v, [](int a, int b) { return a < b ? a : b; });
}

// Top-k of one token's E <= 64 * EPL logits, in one wavefront: v holds lane's
// logits e = lane + 64 j (-inf past E). The selection is the first k of a
// stable sort by logit descending: k rounds of a wave-wide arg-max (highest
// logit, then lowest expert index), each winner masked out. Weights: softmax
// over all E raw logits, not renormalized. Register and DPP work only.
template <int EPL>
__device__ __forceinline__ void topk_rounds(const float (&v)[EPL], int E, int k,
                                            int32_t* __restrict__ ids, float* __restrict__ wts) {
    const int lane = threadIdx.x & 63;
    float mx = v[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) mx = fmaxf(mx, v[j]);
    mx = wave_max_dpp(mx);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) s += expf(v[j] - mx);
    const float inv = 1.f / wave_sum_dpp(s);
    unsigned taken = 0;
    for (int r = 0; r < k; ++r) {
        float bv = -INFINITY;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {  // this lane's best untaken (lowest index on ties)
            const int e = lane + 64 * j;
            const bool ok = e < E && !((taken >> j) & 1u) && (v[j] > bv || be == 0x7FFFFFFF);
            bv = ok ? v[j] : bv;
            be = ok ? e : be;
        }
        const float gv = wave_max_dpp(bv);
        const int ge = wave_min_dpp(be != 0x7FFFFFFF && bv == gv ? be : 0x7FFFFFFF);
        if ((ge & 63) == lane) taken |= 1u << (ge >> 6);
        if (lane == 0) {
            ids[r] = ge;
            wts[r] = expf(gv - mx) * inv;
        }
    }
}

// Key ordering logits descending, ties (-0 equal to +0) to the lower expert
// index (non-NaN logits): larger key = earlier rank.
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
    uint32_t b = v == 0.f ? 0u : __float_as_uint(v);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (0xFFFFFFFFu - (uint32_t)e);
}

// The same selection as topk_rounds<2> (E <= 128) by 256 threads of a
// workgroup at once: an expert's rank is the number of experts whose key is
// larger, each thread counting over 64 of the 128 keys, so the k ranks come
// out of two barriers instead of k dependent wave-wide arg-max rounds. The
// softmax statistics are those of topk_rounds<2> (wavefront 0, same lane
// layout and order), so ids and weights equal its outputs bit for bit.
// Two steps, so that a caller can issue the logit loads first and other loads
// behind them: topk_ranked_load gives thread t the logits of experts t and t +
// 64 (clamped indices, every thread, no branch), topk_ranked_select ranks them.
// ids / wts: ranks 0..k-1 (any memory); keys (128 u64), part (256 int), stat
// (2 float): LDS. Every thread of the workgroup takes part (blockDim.x >= 256;
// threads beyond 255 only pass the barriers).
template <typename Get>
__device__ __forceinline__ void topk_ranked_load(Get lg, int E, float& lt, float& l64) {
    const int t = threadIdx.x;
    lt = lg(min(t, E - 1));
    l64 = lg(min(t + 64, E - 1));
}

__device__ __forceinline__ void topk_ranked_select(float lt, float l64, int E, int k,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ wts, uint64_t* keys,
                                                   int* part, float* stat) {
    const int t = threadIdx.x;
    if (t < 128) keys[t] = rank_key(t < E ? lt : -INFINITY, t);
    if (t < 64) {
        const float v[2] = {t < E ? lt : -INFINITY, t + 64 < E ? l64 : -INFINITY};
        float mx = fmaxf(v[0], v[1]);
        mx = wave_max_dpp(mx);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) s += expf(v[j] - mx);
        const float inv = 1.f / wave_sum_dpp(s);
        if (t == 0) {
            stat[0] = mx;
            stat[1] = inv;
        }
    }
    __syncthreads();
    if (t < 256) {
        const int a = t & 127, h = t >> 7;
        const uint64_t ka = keys[a];
        int r = 0;
#pragma unroll 16
        for (int b = 64 * h; b < 64 * h + 64; ++b) r += keys[b] > ka ? 1 : 0;
        part[t] = r;
    }
    __syncthreads();
    if (t < E) {
        const int r = part[t] + part[t + 128];
        if (r < k) {
            ids[r] = t;
            wts[r] = expf(lt - stat[0]) * stat[1];
        }
    }
}

}  // namespace w4
