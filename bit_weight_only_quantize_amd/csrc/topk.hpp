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

}  // namespace w4
