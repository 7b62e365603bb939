// INT4 KV cache: the per-head-vector codec and the two products that read the
// cache with the dequantization fused in.
//
// Shimmy article, §3.2 (TurboShimmy INT4 KV): every head vector is quantized
// on its own with scale = max|v| / 7.5 (f32) and integers round(v / scale)
// clamped to [-8, 7], stored plus 8 as nibbles (element 2j low); attention
// dequantizes (nibble - 8) * scale on the GPU while it computes. Rounding is
// the page's f32::round (halves away from zero); an all-zero vector gets
// scale 0 and nibbles 8.
//
// Cache layout: codes [Hkv][T_max][D / 2] bytes and scales [Hkv][T_max] f32,
// one head's positions contiguous, so both products stream a head's cache as
// contiguous memory. D = 128.
//
// Products (query head h reads kv head h / (Hq / Hkv)):
//   scores[h][t] = sum_i q[h][i] * k[t][i]         (kv_scores_kernel)
//   out[h][i]    = sum_t p[h][t] * v[t][i]         (kv_wsum_kernel + kv_wsum_add_kernel)
// Both are HBM-bound: 68 bytes of codes and scale per cached vector.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"

namespace w4 {

// ---------------------------------------------------------------- quantize
// One wavefront per head vector: lane l holds elements 2l and 2l + 1, the
// wavefront's max |v| comes from a butterfly, and lane l writes byte l. A
// launch serves one cache, or two (the keys' and the values' of the same
// positions: vectors nvec .. 2 nvec - 1 go to the second).
struct KvAppend {
    const float* x[2];
    uint8_t* codes[2];
    float* scales[2];
};

__global__ __launch_bounds__(256) void kv_quantize_kernel(KvAppend a, int ncache, int nvec, int H,
                                                          int64_t pos, int64_t T_max) {
    const int lane = threadIdx.x & 63;
    int v = blockIdx.x * 4 + (threadIdx.x >> 6);  // vector index (cache, n * H + h)
    if (v >= ncache * nvec) return;               // whole wavefront
    const int cache = v >= nvec ? 1 : 0;
    v -= cache * nvec;
    const float* __restrict__ x = a.x[cache];
    uint8_t* __restrict__ codes = a.codes[cache];
    float* __restrict__ scales = a.scales[cache];
    const float2 e = reinterpret_cast<const float2*>(x + (int64_t)v * kKvHeadDim)[lane];
    float m = fmaxf(fabsf(e.x), fabsf(e.y));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float s = m / 7.5f;  // f32 division, correctly rounded
    auto code = [&](float a) -> uint32_t {
        const float q = s > 0.f ? fminf(fmaxf(roundf(a / s), -8.f), 7.f) : 0.f;  // roundf: halves away
        return (uint32_t)((int)q + 8);
    };
    const int n = v / H, h = v - n * H;
    const int64_t row = (int64_t)h * T_max + pos + n;
    codes[row * (kKvHeadDim / 2) + lane] = (uint8_t)(code(e.x) | (code(e.y) << 4));
    if (lane == 0) scales[row] = s;
}

// ---------------------------------------------------------------- scores
// A wavefront takes one query head and a chunk of positions, 16 cached keys per
// load instruction (1 KB contiguous): lane (key j = lane / 4, part c = lane %
// 4) holds 32 elements of key j, i.e. bytes 16c..16c+15 of its row. The
// nibbles convert exactly (v_cvt_f32_ubyte of the masked bytes) and meet the
// query in f32 FMAs: sum q (u - 8) = sum q u - 8 sum q, the second sum taken
// once. Four lanes of a key add their parts by cross-lane steps; the key's
// scale multiplies the total.
// Positions per wavefront, 4 of its 16-key loads in flight. Measured on the
// 7B-shaped cache (32 heads, 8193 positions): chunks of 64, 256 or 512 and 8
// loads in flight were all slower or the same, for both products. The cache
// is read once per product, so its loads are nontemporal (4% faster here;
// the same hint slowed the MoE expert passes by 8%).
constexpr int kKvChunk = 128;
constexpr int kKvDepth = 4;

// value of the lane N places along in the same row of 16 (DPP row_ror:N)
template <int N>
__device__ __forceinline__ float dpp_row_ror(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}

__device__ __forceinline__ float kv_dot32(const u32x4_t c, const float* qe, const float* qo) {
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t lo = c[d] & 0x0F0F0F0Fu, hi = (c[d] >> 4) & 0x0F0F0F0Fu;
        // keep the byte masks: one v_cvt_f32_ubyte per nibble afterwards
        asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            acc = fmaf(qe[4 * d + b], (float)((lo >> (8 * b)) & 0xFFu), acc);
            acc = fmaf(qo[4 * d + b], (float)((hi >> (8 * b)) & 0xFFu), acc);
        }
    }
    return acc;
}

// Positions pos .. T - 1 that arrive with the product's own launch (the append
// fused into the product; pos == T: none). Their cached bytes are not read:
// the lanes that handle a new position quantize it from the input, with the
// arithmetic of kv_quantize_kernel, and use the codes and scale from registers;
// the first query head of each kv group writes them into the cache. No lane of
// the launch reads a position >= pos from the cache, so the writes race with
// nothing.
struct KvNew {
    const float* x;   // [T - pos][Hkv][kKvHeadDim] fp32
    uint8_t* codes;   // the cache the new positions go to
    float* scales;
    int pos;
};

// One new head vector quantized by the whole wavefront with the lane layout and
// arithmetic of kv_quantize_kernel (lane l: elements 2l and 2l + 1, byte l; max
// |v| by the same butterfly), then handed out in the products' layout: lane
// (j, c) gets bytes 16c .. 16c + 15, i.e. elements 32c .. 32c + 31. s_out is the
// vector's scale on every lane.
__device__ __forceinline__ u32x4_t kv_quantize_wave(const float* __restrict__ src, int lane, float& s_out) {
    const float2 e = reinterpret_cast<const float2*>(src)[lane];
    float m = fmaxf(fabsf(e.x), fabsf(e.y));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float s = m / 7.5f;
    auto code = [&](float a) -> uint32_t {
        const float q = s > 0.f ? fminf(fmaxf(roundf(a / s), -8.f), 7.f) : 0.f;
        return (uint32_t)((int)q + 8);
    };
    const uint32_t b = code(e.x) | (code(e.y) << 4);
    // word i of the vector (bytes 4i .. 4i + 3) assembled on lane 4i
    const uint32_t wd = b | (__shfl_down(b, 1) << 8) | (__shfl_down(b, 2) << 16) | (__shfl_down(b, 3) << 24);
    const int c = lane & 3;
    u32x4_t w;
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] = __shfl(wd, 16 * c + 4 * d);
    s_out = s;
    return w;
}

template <int CHUNK, int DEPTH>
__global__ __launch_bounds__(256) void kv_scores_kernel(const float* __restrict__ q, int Hq,
                                                        int group, int T, int64_t T_max,
                                                        const uint8_t* __restrict__ codes,
                                                        const float* __restrict__ scales,
                                                        float* __restrict__ scores, int nch,
                                                        KvNew nw) {
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // (chunk, head) with heads fastest
    if (w >= nch * Hq) return;                           // whole wavefront
    const int h = w % Hq, ch = w / Hq;
    const int g = h / group;
    const int j = lane >> 2, c = lane & 3;
    // this lane's 32 query elements, even and odd
    float qe[16], qo[16];
    const float2* qp = reinterpret_cast<const float2*>(q + (int64_t)h * kKvHeadDim + 32 * c);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float2 e = qp[i];
        qe[i] = e.x;
        qo[i] = e.y;
    }
    // 8 * sum q, the same instructions wherever it is needed (exact: an fma or a
    // product and a difference with it give the same bits); taken after the
    // first cache loads are issued, so they do not wait for q
    auto q8sum = [&]() {
        float qs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) qs += qe[i] + qo[i];
        return 8.f * qs;
    };
    const int t0 = ch * CHUNK;
    const uint8_t* base = codes + (int64_t)g * T_max * (kKvHeadDim / 2) + 16 * c;
    const float* sbase = scales + (int64_t)g * T_max;
    constexpr int IT = CHUNK / 16;
    const int Tc = nw.pos;  // cached positions read here: 0 .. Tc - 1
    if (Tc > t0) {  // wave-uniform: this chunk holds cached positions
        // the scales of every step first, then the code loads DEPTH steps ahead:
        // the steps then wait on code loads only
        float sb[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) sb[it] = sbase[min(t0 + 16 * it + j, Tc - 1)];
        __builtin_amdgcn_sched_barrier(0);  // issued before the code loads, in this order
        u32x4_t cb[DEPTH];
        auto load = [&](int it, int slot) {  // clamped: keys past Tc reload Tc - 1
            const int t = min(t0 + 16 * min(it, IT - 1) + j, Tc - 1);
            cb[slot] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + (int64_t)t * (kKvHeadDim / 2)));
        };
#pragma unroll
        for (int p = 0; p < DEPTH; ++p) load(p, p);
        __builtin_amdgcn_sched_barrier(0);  // all DEPTH in flight before the first wait
        const float q8 = q8sum();
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int slot = it % DEPTH;
            float d = kv_dot32(cb[slot], qe, qo) - q8;
            const float s = sb[it];
            if (it + DEPTH < IT) load(it + DEPTH, slot);
            d += __shfl_xor(d, 1);
            d += __shfl_xor(d, 2);
            // every lane stores (no branch in the load pipeline): the 4 lanes of
            // a key store the same value, keys past Tc rewrite the score of Tc - 1
            scores[(int64_t)h * T + min(t0 + 16 * it + j, Tc - 1)] = s * d;
            __builtin_amdgcn_sched_barrier(0);  // steps in order: each waits for its own codes only
        }
    }
    // new positions of this chunk, one at a time (wave-uniform loop); the four
    // lanes of the position's key score it exactly as above
    if (max(Tc, t0) >= min(T, t0 + CHUNK)) return;  // wave-uniform: no new position here
    // the compiler must not share this q sum's instructions with the one above
    // and hoist them before the branch: that would wait for q before the first
    // cache load is issued
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(qe[i]), "+v"(qo[i]));
    const float q8 = q8sum();
    const int Hkv = Hq / group;
    for (int t = max(Tc, t0); t < min(T, t0 + CHUNK); ++t) {
        float s;
        const u32x4_t cw = kv_quantize_wave(nw.x + ((int64_t)(t - Tc) * Hkv + g) * kKvHeadDim, lane, s);
        float d = kv_dot32(cw, qe, qo) - q8;
        d += __shfl_xor(d, 1);
        d += __shfl_xor(d, 2);
        if (j == ((t - t0) & 15)) {
            scores[(int64_t)h * T + t] = s * d;
            if (h % group == 0) {
                const int64_t row = (int64_t)g * T_max + t;
                *reinterpret_cast<u32x4_t*>(nw.codes + row * (kKvHeadDim / 2) + 16 * c) = cw;
                if (c == 0) nw.scales[row] = s;
            }
        }
    }
}

// ---------------------------------------------------------------- weighted sum
// The same lane layout over the values: a lane accumulates p_t * scale_t times
// its 32 nibbles (as 0..15) and the weight sum W = sum p_t scale_t, so its
// elements are acc - 8 W. After the chunk the 16 lanes of each part add their
// accumulators (cross-lane steps over lane bits 2..5, a fixed order), and the
// chunk's 128 partial outputs go to part[h][chunk][128]; kv_wsum_add_kernel
// adds the chunks in a fixed order.
template <int CHUNK, int DEPTH>
__global__ __launch_bounds__(256) void kv_wsum_kernel(const float* __restrict__ pw, int Hq,
                                                      int group, int T, int64_t T_max,
                                                      const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ scales,
                                                      float* __restrict__ part, int nch, KvNew nw) {
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= nch * Hq) return;
    const int h = w % Hq, ch = w / Hq;
    const int g = h / group;
    const int j = lane >> 2, c = lane & 3;
    const int t0 = ch * CHUNK;
    const uint8_t* base = codes + (int64_t)g * T_max * (kKvHeadDim / 2) + 16 * c;
    const float* sbase = scales + (int64_t)g * T_max;
    const float* prow = pw + (int64_t)h * T;
    constexpr int IT = CHUNK / 16;
    const int Tc = nw.pos;  // cached positions read here: 0 .. Tc - 1
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    float W = 0.f;
    // one position's share: weight wt times this lane's 32 nibbles (as 0..15)
    auto accumulate = [&](const u32x4_t cw, float wt) {
        asm("" : "+v"(wt));  // wt is rounded on its own: never contracted into W's sum
        W += wt;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t lo = cw[d] & 0x0F0F0F0Fu, hi = (cw[d] >> 4) & 0x0F0F0F0Fu;
            asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                acc[8 * d + 2 * b] = fmaf(wt, (float)((lo >> (8 * b)) & 0xFFu), acc[8 * d + 2 * b]);
                acc[8 * d + 2 * b + 1] = fmaf(wt, (float)((hi >> (8 * b)) & 0xFFu), acc[8 * d + 2 * b + 1]);
            }
        }
    };
    if (Tc > t0) {  // wave-uniform: this chunk holds cached positions
        // The weights' operands of every step first (unconditional loads at
        // clamped positions), then the code loads DEPTH steps ahead: the steps
        // wait on code loads only. A load under the "key < Tc" condition would
        // become a branch that waits for every load in flight.
        float pb[IT], sb[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int t = min(t0 + 16 * it + j, Tc - 1);
            pb[it] = prow[t];
            sb[it] = sbase[t];
        }
        __builtin_amdgcn_sched_barrier(0);  // issued before the code loads, in this order
        u32x4_t cb[DEPTH];
        auto load = [&](int it, int slot) {
            const int t = min(t0 + 16 * min(it, IT - 1) + j, Tc - 1);
            cb[slot] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + (int64_t)t * (kKvHeadDim / 2)));
        };
#pragma unroll
        for (int p = 0; p < DEPTH; ++p) load(p, p);
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int slot = it % DEPTH;
            const u32x4_t cw = cb[slot];
            float pv = pb[it], sv = sb[it];
            asm("" : "+v"(pv), "+v"(sv));  // keeps the loads out of the select (no branch)
            const float wt = t0 + 16 * it + j < Tc ? pv * sv : 0.f;  // keys past Tc: 0
            if (it + DEPTH < IT) load(it + DEPTH, slot);
            accumulate(cw, wt);
            __builtin_amdgcn_sched_barrier(0);  // steps in order: each waits for its own codes only
        }
    }
    // New positions (see KvNew), one at a time; only the four lanes of the
    // position's key weigh it. A lane's new positions come after all of its
    // cached ones, and the zero-weight steps add exact zeros to sums that are
    // never -0, so the totals equal those of a read from the cache.
    const int Hkv = Hq / group;
    for (int t = max(Tc, t0); t < min(T, t0 + CHUNK); ++t) {  // wave-uniform
        float s;
        const u32x4_t cw = kv_quantize_wave(nw.x + ((int64_t)(t - Tc) * Hkv + g) * kKvHeadDim, lane, s);
        const bool mine = j == ((t - t0) & 15);
        accumulate(cw, mine ? prow[t] * s : 0.f);
        if (mine && h % group == 0) {
            const int64_t row = (int64_t)g * T_max + t;
            *reinterpret_cast<u32x4_t*>(nw.codes + row * (kKvHeadDim / 2) + 16 * c) = cw;
            if (c == 0) nw.scales[row] = s;
        }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = fmaf(-8.f, W, acc[i]);
    // lanes c, c + 4, ..., c + 60 hold part c of 16 keys: add them. Inside a
    // row of 16 lanes, rotations by 4 and by 8 (DPP, no LDS) leave every lane
    // with its row's sum for its part; across the 4 rows, lane (row R, r =
    // lane / 4 % 4) then adds only elements 8r .. 8r + 7 of its part (two
    // cross-lane steps on 8 values instead of four on 32), and row 0 stores.
    // Each output comes from one fixed lane: deterministic.
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        acc[i] += dpp_row_ror<4>(acc[i]);
        acc[i] += dpp_row_ror<8>(acc[i]);
    }
    const int r = (lane >> 2) & 3;
    float o8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        o8[i] = r == 0 ? acc[i] : r == 1 ? acc[8 + i] : r == 2 ? acc[16 + i] : acc[24 + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        o8[i] += __shfl_xor(o8[i], 16);
        o8[i] += __shfl_xor(o8[i], 32);
    }
    if (lane < 16) {
        float4* dst = reinterpret_cast<float4*>(part + ((int64_t)h * nch + ch) * kKvHeadDim + 32 * c + 8 * r);
        dst[0] = make_float4(o8[0], o8[1], o8[2], o8[3]);
        dst[1] = make_float4(o8[4], o8[5], o8[6], o8[7]);
    }
}

// out[h][e] = the sum of part[h][ch][e] over the chunks: 16 lanes per output,
// lane k taking chunks k, k + 16, ... (eight loads in flight, added in chunk
// order), then the 16 lane sums added by cross-lane steps in a fixed order.
__global__ __launch_bounds__(256) void kv_wsum_add_kernel(const float* __restrict__ part, int Hq,
                                                          int nch, float* __restrict__ out) {
    const int i = blockIdx.x * 16 + (threadIdx.x >> 4);  // h * 128 + element
    const int k = threadIdx.x & 15;
    const bool live = i < Hq * kKvHeadDim;
    const int ic = live ? i : 0;
    const int h = ic / kKvHeadDim, e = ic - h * kKvHeadDim;
    const float* p = part + (int64_t)h * nch * kKvHeadDim + e;
    float s = 0.f;
    for (int c0 = k; c0 < nch; c0 += 16 * 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int ch = c0 + 16 * u;
            v[u] = p[(int64_t)min(ch, nch - 1) * kKvHeadDim];
            v[u] = ch < nch ? v[u] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o);
    if (live && k == 0) out[i] = s;
}

// ---------------------------------------------------------------- host side
int kv_chunks(int64_t T) { return (int)((T + kKvChunk - 1) / kKvChunk); }

hipError_t launch_kv_quantize(const float* const* x, int ncache, int64_t n, int64_t H,
                              int64_t pos, int64_t T_max, uint8_t* const* codes,
                              float* const* scales, hipStream_t st) {
    const int nvec = (int)(n * H);
    KvAppend a{};
    for (int i = 0; i < ncache; ++i) {
        a.x[i] = x[i];
        a.codes[i] = codes[i];
        a.scales[i] = scales[i];
    }
    const int total = ncache * nvec;
    hipLaunchKernelGGL(kv_quantize_kernel, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, st, a,
                       ncache, nvec, (int)H, pos, T_max);
    return hipGetLastError();
}

// xnew: the fp32 vectors of positions pos .. T - 1, quantized into codes/scales
// by this launch (null: none, pos ignored)
hipError_t launch_kv_scores(const float* q, int64_t Hq, int64_t Hkv, int64_t T, int64_t T_max,
                            const uint8_t* codes, const float* scales, float* scores,
                            const float* xnew, int64_t pos, hipStream_t st) {
    const int nch = kv_chunks(T);
    const int64_t waves = (int64_t)nch * Hq;
    const KvNew nw{xnew, const_cast<uint8_t*>(codes), const_cast<float*>(scales),
                   (int)(xnew ? pos : T)};
    hipLaunchKernelGGL((kv_scores_kernel<kKvChunk, kKvDepth>), dim3((unsigned)((waves + 3) / 4)),
                       dim3(256), 0, st, q, (int)Hq, (int)(Hq / Hkv), (int)T, T_max, codes, scales,
                       scores, nch, nw);
    return hipGetLastError();
}

hipError_t launch_kv_weighted_sum(const float* p, int64_t Hq, int64_t Hkv, int64_t T,
                                  int64_t T_max, const uint8_t* codes, const float* scales,
                                  float* out, float* part, const float* xnew, int64_t pos,
                                  hipStream_t st) {
    const int nch = kv_chunks(T);
    const int64_t waves = (int64_t)nch * Hq;
    const KvNew nw{xnew, const_cast<uint8_t*>(codes), const_cast<float*>(scales),
                   (int)(xnew ? pos : T)};
    hipLaunchKernelGGL((kv_wsum_kernel<kKvChunk, kKvDepth>), dim3((unsigned)((waves + 3) / 4)),
                       dim3(256), 0, st, p, (int)Hq, (int)(Hq / Hkv), (int)T, T_max, codes, scales,
                       part, nch, nw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kv_wsum_add_kernel, dim3((unsigned)((Hq * kKvHeadDim + 15) / 16)),
                       dim3(256), 0, st, part, (int)Hq, nch, out);
    return hipGetLastError();
}

}  // namespace w4
