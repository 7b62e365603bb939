// Gate/up expert pass for several tokens as one grouped, persistent launch.
//
// TurboFieldfare article (Gemma 4 26B-A4B section): each token runs 8 of 128
// experts plus the shared expert; only the selected experts' weights are read.
// With a few tokens per active expert (32 tokens x 8 slots over ~112 experts:
// about 2 each), one workgroup per (expert, row block) leaves every workgroup
// a few kilobytes of weights behind a chain of dependent loads (descriptor,
// pair list, activations, codes). Here one workgroup per CU takes an even
// share of all the layer's work items -- one 16-row tile of one active expert
// slot (at most 16 tokens), or of the shared expert for 16 tokens -- and each
// streaming wavefront walks its items as one sequence of 128-weight steps, so
// the code prefetch runs across item boundaries. The activations x (all M <=
// 32 tokens) are staged once per workgroup in LDS in the MFMA A-operand
// layout; a step loads the gate and the up codes of the item's 16 rows; the
// epilogue writes h = bf16(gelu(g) * u).
//
// (The same scheme for the down pass, whose activations are each pair's own h
// row and so come from L2 with every step, measured slower than the
// per-expert-block kernel: the gathers of those rows, four 16-byte loads per
// lane per kilobyte of codes, dominate; sharing them over four row tiles per
// item still left it behind.)
//
// The MFMA step is the skinny GEMM's (16 tokens x 32 k x 16 rows, codes
// unpacked in registers, group sums from one MFMA against a ones operand).
#pragma once

#include "gemv_mfma.hpp"

namespace w4 {

struct GMat {  // stacked expert matrices (byte strides), or one matrix (strides 0)
    const uint8_t* codes;
    const uint8_t* scale;
    const uint8_t* bias;
    int64_t stride_c, stride_s;
    int N, K;
};

struct MoeGArgs {
    GMat r0, r1;  // routed gate, up
    GMat s0, s1;  // shared expert gate, up
    int has_shared;
    int M, k, slots, P;
    const uint16_t* x;      // [M][D]
    const int4* work;       // [slots + 1]: {expert, first pair, count <= 16}, then {n_desc, ...}
    const int32_t* pairs;   // [P]
    uint16_t* h;            // [P][F]
    uint16_t* hs;           // [M][Fs]
    int NS;                 // streaming wavefronts per workgroup
};

// Column swizzle of row lr (0..15 within a step) of the staged activations
// for rows of mp (power of two, 2..32) units: rows of 16 or more units take
// lr rotated left by one in 4 bits, shorter rows their top bits rotated.
__device__ __forceinline__ int gswz(int mp, int lr) {
    if (mp >= 16) return ((lr << 1) | (lr >> 3)) & 15;
    const int b = 31 - __builtin_clz(mp);
    const int x = lr >> (4 - b);
    return ((x << 1) | (x >> (b - 1))) & (mp - 1);
}

// LDS words of the gate/up pass's activation stage (A units, no sums).
__host__ __device__ inline int moe_gx_words(int D, int M) {
    int mp = 2;
    while (mp < M) mp *= 2;
    return (D / 128) * 16 * mp * 4;
}

// 1024 threads: all stage x, the first NS stream codes. An item is the gate
// and the up tile of the same 16 rows.
template <int S, int DEPTH>
__global__ __launch_bounds__(1024) void moe_grouped_kernel(MoeGArgs a) {
    using T = Traits<S>;
    using P = MfmaStep<S>;
    constexpr int GPS = P::GPS;
    constexpr int NM = 2;  // gate, up
    const int NT = blockDim.x;
    extern __shared__ __align__(16) uint32_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int M = a.M;
    int mp = 2;
    while (mp < M) mp *= 2;
    const int aw = moe_gx_words(a.r0.K, M);
    int4* swork = reinterpret_cast<int4*>(lds + aw);
    int* spairs = reinterpret_cast<int*>(swork + a.slots + 1);

    // 1. descriptors, the pair list and x (A layout) -> LDS
    for (int i = threadIdx.x; i <= a.slots; i += NT) swork[i] = a.work[i];
    for (int i = threadIdx.x; i < a.P; i += NT) spairs[i] = a.pairs[i];
    {
        constexpr int NV = 16;  // 16-byte vectors per 128 weights (one step) of one token
        const int D = a.r0.K;
        const int C = mp * NV, GS = NT / C;  // lanes per step of all tokens; steps at a time
        const int c = threadIdx.x % C;
        const int st0 = (int)threadIdx.x < GS * C ? (int)threadIdx.x / C : D / 128;
        const int t = c / NV, iv = c % NV;
        const bool live = t < M;
        const uint16_t* xl = a.x + (int64_t)min(t, M - 1) * D + iv * 8;
        // vector iv of a step is piece (d, gg) of the A operand: the inverse
        // of the codes' k order (for GPS = 2 each group's half of the step)
        int d, gg;
        if constexpr (GPS == 1) {
            gg = iv >> 2;
            d = iv & 3;
        } else {
            const int q = iv >> 3, i8 = iv & 7;  // group q of the step, vector i8 in it
            gg = (i8 >> 2) | (((i8 >> 1) & 1) << 1);
            d = 2 * q + (i8 & 1);
        }
        const int lr = d * 4 + gg;
        const int col = t ^ gswz(mp, lr);
        constexpr int U = 4;
        const int nst = D / 128;
        for (int sb = st0; sb < nst; sb += GS * U) {
            u32x4_t r[U];
#pragma unroll
            for (int j = 0; j < U; ++j) r[j] = *gmem<u32x4_t>(xl + min(sb + j * GS, nst - 1) * 128);
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int s = sb + j * GS;
                if (live && s < nst) {
                    const u32x4_t o = {__builtin_amdgcn_perm(r[j][2], r[j][0], 0x05040100u),
                                       __builtin_amdgcn_perm(r[j][2], r[j][0], 0x07060302u),
                                       __builtin_amdgcn_perm(r[j][3], r[j][1], 0x05040100u),
                                       __builtin_amdgcn_perm(r[j][3], r[j][1], 0x07060302u)};
                    *reinterpret_cast<u32x4_t*>(lds + 4 * ((s * 16 + lr) * mp + col)) = o;
                }
            }
        }
    }
    __syncthreads();

    // 2. this workgroup's items: an even share of routed items (descriptor j,
    //    row tile r) then shared items (row tile r, token tile tt)
    const int n_desc = __builtin_amdgcn_readfirstlane(swork[a.slots].x);
    const int tpe = a.r0.N / 16;
    const int TT = (M + 15) / 16;
    const int tps = a.has_shared ? a.s0.N / 16 : 0;
    const int Tr = n_desc * tpe, Ttot = Tr + tps * TT;
    const int i0 = (int)((int64_t)Ttot * blockIdx.x / gridDim.x);
    const int i1 = (int)((int64_t)Ttot * (blockIdx.x + 1) / gridDim.x);
    if (wave >= a.NS) return;  // staging-only wavefronts: no barrier follows
    const int ni = i1 - i0 > wave ? (i1 - i0 - wave + a.NS - 1) / a.NS : 0;
    if (ni == 0) return;
    const int spi_r = a.r0.K / 128, spi_s = a.has_shared ? a.s0.K / 128 : 0;
    // steps of this wavefront: its items n = 0 .. ni-1 are i0 + wave + n * NS
    int nr = 0;  // routed ones among them
    {
        const int first = i0 + wave;
        nr = first < Tr ? min(ni, (Tr - first + a.NS - 1) / a.NS) : 0;
    }
    const int Q = nr * spi_r + (ni - nr) * spi_s;

    struct Item {
        int sh, e, row0, first, cnt, spi;
    };
    auto item = [&](int n) {
        const int it = i0 + wave + n * a.NS;
        Item r;
        if (it < Tr) {
            const int j = it / tpe;
            const int4 w = swork[j];
            r.sh = 0;
            r.e = __builtin_amdgcn_readfirstlane(w.x);
            r.first = __builtin_amdgcn_readfirstlane(w.y);
            r.cnt = __builtin_amdgcn_readfirstlane(w.z);
            r.row0 = (it - j * tpe) * 16;
            r.spi = spi_r;
        } else {
            const int u = it - Tr, rr = u / TT, tt = u - rr * TT;
            r.sh = 1;
            r.e = 0;
            r.row0 = rr * 16;
            r.first = tt * 16;
            r.cnt = min(16, M - tt * 16);
            r.spi = spi_s;
        }
        return r;
    };
    // the activation row of token slot `slot` of an item: a pair (routed) or a token
    auto act_row = [&](const Item& it, int slot) {
        const int s = min(slot, it.cnt - 1);
        return it.sh ? it.first + s : spairs[it.first + s];
    };

    // load side: item ln, step ls; per-lane row pointers of that item
    struct Buf {
        u32x4_t c[NM];
        uint32_t sc[NM], bi[T::AFFINE ? NM : 1];
    };
    int ln = 0, ls = 0;
    Item lit = item(0);
    const uint8_t* lc[NM];
    const uint8_t* lsp[NM];
    const uint8_t* lbp[NM];
    auto set_load_item = [&]() {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const GMat& W = lit.sh ? (m ? a.s1 : a.s0) : (m ? a.r1 : a.r0);
            const int row = lit.row0 + c16;  // N % 16 == 0
            const int groups = W.K / T::GROUP;
            lc[m] = W.codes + lit.e * W.stride_c + (int64_t)row * (W.K / 2);
            lsp[m] = W.scale + lit.e * W.stride_s + (int64_t)row * groups * (T::AFFINE ? 2 : 4);
            lbp[m] = T::AFFINE ? W.bias + lit.e * W.stride_s + (int64_t)row * groups * 2 : nullptr;
        }
    };
    set_load_item();
    auto load = [&](Buf& B) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            B.c[m] = *gmem<u32x4_t>(lc[m] + ls * 64 + 16 * g);
            if constexpr (T::AFFINE) {
                B.sc[m] = *gmem<uint32_t>(lsp[m] + ls * 4);  // the step's two bf16 scales
                B.bi[m] = *gmem<uint32_t>(lbp[m] + ls * 4);  // and biases
            } else {
                B.sc[m] = *gmem<uint32_t>(lsp[m] + ls * 4);
            }
        }
        // advance (wave-uniform); past the last item the last step is reloaded
        if (ls + 1 < lit.spi) {
            ++ls;
        } else if (ln + 1 < ni) {
            ++ln;
            ls = 0;
            lit = item(ln);
            set_load_item();
        }
    };

    // compute side: item cn, step cs
    int cn = 0, cs = 0;
    Item cit = lit;
    int ctok = 0;  // the lane's token (A row) of the item
    auto set_comp_item = [&]() { ctok = cit.sh ? act_row(cit, c16) : act_row(cit, c16) / a.k; };
    set_comp_item();
    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    const uint32_t ONE2 = 0x3F803F80u;
    const bf16x8_t ONES = as_bf16x8(ONE2, ONE2, ONE2, ONE2);
    auto unpack = [&](uint32_t w) {
        auto pair = [&](uint32_t v) {
            return S == SYM4_G128 ? ((v & MASK) ^ MAGIC) : ((v & MASK) | MAGIC);
        };
        return as_bf16x8(pair(w), pair(w >> 4), pair(w >> 8), pair(w >> 12));
    };
    f32x4_t acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto epilogue = [&]() {
        // token slots past the item's count hold the last slot's values (their
        // A rows were clamped to it): the store repeats that slot's, no branch
        const int row = cit.row0 + c16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int dst = act_row(cit, 4 * g + r);
            const int F = cit.sh ? a.s0.N : a.r0.N;
            uint16_t* out = (cit.sh ? a.hs : a.h) + (int64_t)dst * F;
            out[row] = (uint16_t)f32_to_bf16_rne(gelu_tanh(acc[0][r]) * acc[1][r]);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    };

    auto compute = [&](const Buf& B) {
        bf16x8_t A[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
            A[d] = *reinterpret_cast<const bf16x8_t*>(
                lds + 4 * ((cs * 16 + d * 4 + g) * mp + (ctok ^ gswz(mp, d * 4 + g))));
        f32x4_t DX[GPS];
#pragma unroll
        for (int q = 0; q < GPS; ++q) {
            DX[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 4 / GPS * q; d < 4 / GPS * (q + 1); ++d)
                DX[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[d], ONES, DX[q], 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            uint32_t w[4] = {B.c[m][0], B.c[m][1], B.c[m][2], B.c[m][3]};
            if constexpr (GPS == 2) {
                // lanes 0-31 hold group A, lanes 32-63 group B: swap the upper
                // half of words 0/1 with the lower half of words 2/3
                const auto p02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
                const auto p13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
                w[0] = p02[0]; w[2] = p02[1];
                w[1] = p13[0]; w[3] = p13[1];
            }
#pragma unroll
            for (int q = 0; q < GPS; ++q) {
                f32x4_t Dm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 4 / GPS * q; d < 4 / GPS * (q + 1); ++d)
                    Dm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[d], unpack(w[d]), Dm, 0, 0, 0);
                float sc, corr;
                if constexpr (T::AFFINE) {
                    sc = bf16_bits_to_f32((B.sc[m] >> (16 * q)) & 0xFFFFu);
                    corr = fmaf(-T::BIAS, sc, bf16_bits_to_f32((B.bi[m] >> (16 * q)) & 0xFFFFu));
                } else {
                    sc = __uint_as_float(B.sc[m]);
                    corr = -T::BIAS * sc;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[m][r] = fmaf(corr, DX[q][r], fmaf(sc, Dm[r], acc[m][r]));
            }
        }
        // advance (wave-uniform): an item's last step writes its outputs
        if (cs + 1 < cit.spi) {
            ++cs;
        } else {
            epilogue();
            if (cn + 1 < ni) {
                ++cn;
                cs = 0;
                cit = item(cn);
                set_comp_item();
            }
        }
    };

    // 3. the steps: DEPTH - 1 ahead; whole rounds in the loop, the rest after
    Buf cb[DEPTH];
#pragma unroll
    for (int p = 0; p < DEPTH - 1; ++p) {
        load(cb[p]);
        __builtin_amdgcn_sched_barrier(0);
    }
    const int full = Q / DEPTH * DEPTH;
    for (int q0 = 0; q0 < full; q0 += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            load(cb[(u + DEPTH - 1) % DEPTH]);
            __builtin_amdgcn_sched_barrier(0);
            compute(cb[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u)
        if (full + u < Q) compute(cb[u]);
}

}  // namespace w4
