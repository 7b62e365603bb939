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
// lane per kilobyte of codes, dominate. The down pass below stages them in
// LDS per work descriptor instead.)
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

namespace w4 {

// Routed down pass for several tokens: one workgroup per (work descriptor j,
// block of 16 rows per wavefront of the expert's W_down). The descriptor's pairs (at
// most 16) are the MFMA tokens: their h rows are gathered from L2 once per
// workgroup into LDS in the A-operand layout (the skinny kernel's layout and
// swizzle, with every (group, pair) activation sum), then wavefront w streams
// row tile w over all K, its scales in a private LDS block, DEPTH steps of
// code loads in flight, and writes part[pair][row]. A small LDS footprint (a
// 768-wide h: 25 KB of activations) lets several workgroups share a CU, so one
// workgroup's staging overlaps the others' streaming.
struct MoeDownArgs {
    GMat W;                 // routed W_down (stacked)
    const uint16_t* h;      // [P][F]
    const int4* work;       // descriptors (count <= 16); x < 0 past the last
    const int32_t* pairs;   // [P]
    float* part;            // [P][D]
};

// LDS bytes of moe_down_routed_kernel for K = F and SGMAX
__host__ __device__ inline size_t moe_down_lds_bytes(int K, int group, int sgmax, int waves) {
    const int steps = K / 128;
    const int gps = 128 / group;
    return ((size_t)steps * 16 * 16 * 4 + (size_t)steps * gps * 16 + (size_t)waves * 16 * (sgmax + 1)) * 4;
}

template <int S, int DEPTH, int SGMAX>
__global__ __launch_bounds__(1024) void moe_down_routed_kernel(MoeDownArgs a) {
    using T = Traits<S>;
    using P = MfmaStep<S>;
    constexpr int GPS = P::GPS;
    constexpr int NV = T::GROUP / 8;  // 16-byte activation vectors per group
    constexpr int U = 4;
    constexpr uint32_t ONE2 = 0x3F803F80u;
    extern __shared__ __align__(16) uint32_t lds[];
    const int NT = blockDim.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int4 wd = a.work[blockIdx.y];
    const int e = __builtin_amdgcn_readfirstlane(wd.x);
    if (e < 0) return;  // whole workgroup: an unused descriptor slot
    const int first = __builtin_amdgcn_readfirstlane(wd.y), cnt = __builtin_amdgcn_readfirstlane(wd.z);
    const int K = a.W.K, N = a.W.N;
    const int groups = K / T::GROUP, steps = K / 128;
    int mp = 2;
    while (mp < cnt) mp *= 2;
    const int aw = steps * 16 * mp * 4;
    float* xd = reinterpret_cast<float*>(lds + steps * 16 * 16 * 4);
    uint32_t* sl = lds + steps * 16 * 16 * 4 + steps * GPS * 16 + wave * 16 * (SGMAX + 1);
    (void)aw;

    const int row0 = (blockIdx.x * (NT / 64) + wave) * 16;  // N % (16 * wavefronts) == 0
    const uint8_t* codes = a.W.codes + (int64_t)e * a.W.stride_c;
    const uint8_t* scale = a.W.scale + (int64_t)e * a.W.stride_s;
    const uint8_t* bias = T::AFFINE ? a.W.bias + (int64_t)e * a.W.stride_s : nullptr;
    const uint8_t* crow = codes + (int64_t)(row0 + c16) * (K / 2);

    // staging lanes: one token (pair) t and one 16-byte vector iv of a group;
    // NV consecutive lanes cover a group of one pair (coalesced; the group's
    // sum is a DPP reduction over them). Pairs past cnt store nothing.
    const int C = mp * NV, GS = NT / C;
    const int c = threadIdx.x % C;
    const int gi0 = (int)threadIdx.x < GS * C ? (int)threadIdx.x / C : groups;
    const int t = c / NV, iv = c % NV;
    const bool live = t < cnt;
    const uint16_t* xl = a.h + (int64_t)a.pairs[first + min(t, cnt - 1)] * K + iv * 8;
    const int gg = GPS == 1 ? (iv >> 2) : ((iv >> 2) | (((iv >> 1) & 1) << 1));
    u32x4_t xr[U];
    auto stage_load = [&](int gb) {
#pragma unroll
        for (int j = 0; j < U; ++j) xr[j] = *gmem<u32x4_t>(xl + min(gb + j * GS, groups - 1) * T::GROUP);
    };
    auto stage_store = [&](int gb) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float part = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) part = dot2_bf16(ONE2, xr[j][q], part);
            const float sum = group_sum<NV>(part);
            const int gi = gb + j * GS;
            if (live && gi < groups) {
                const int st = gi / GPS, q = gi - st * GPS;
                const int d = GPS == 1 ? (iv & 3) : (2 * q + (iv & 1));
                const u32x4_t o = {__builtin_amdgcn_perm(xr[j][2], xr[j][0], 0x05040100u),
                                   __builtin_amdgcn_perm(xr[j][2], xr[j][0], 0x07060302u),
                                   __builtin_amdgcn_perm(xr[j][3], xr[j][1], 0x05040100u),
                                   __builtin_amdgcn_perm(xr[j][3], xr[j][1], 0x07060302u)};
                const int lr = d * 4 + gg;
                *reinterpret_cast<u32x4_t*>(lds + 4 * ((st * 16 + lr) * mp + (t ^ gswz(mp, lr)))) = o;
                if (iv == 0) xd[(st * GPS + q) * 16 + t] = sum;
            }
        }
    };
    // 1. the first activation loads first (their waits then cover L2 only)
    stage_load(gi0);
    __builtin_amdgcn_sched_barrier(0);
    // 2. the tile's scales (affine: bf16 scale low, bias high) for the
    //    wavefront's LDS block, lanes over a row's groups
    constexpr int SR = (SGMAX + 63) / 64;
    uint32_t sv[SR][16];
#pragma unroll
    for (int hh = 0; hh < SR; ++hh) {
        const int gl = min(lane + 64 * hh, groups - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t ei = (uint32_t)(row0 + r) * (uint32_t)groups + (uint32_t)gl;
            if constexpr (T::AFFINE)
                sv[hh][r] = (uint32_t)gmem<uint16_t>(scale)[ei] | ((uint32_t)gmem<uint16_t>(bias)[ei] << 16);
            else
                sv[hh][r] = gmem<uint32_t>(scale)[ei];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 3. the first DEPTH - 1 steps' codes, in the loop's order
    using Buf = u32x4_t;
    auto load = [&](Buf& B, int s) { B = *gmem<u32x4_t>(crow + (uint32_t)min(s, steps - 1) * 64 + 16 * g); };
    Buf cb[DEPTH];
#pragma unroll
    for (int p = 0; p < DEPTH - 1; ++p) {
        load(cb[p], p);
        __builtin_amdgcn_sched_barrier(0);
    }
    // 4. activations and sums, then the scales (unconditional stores)
    stage_store(gi0);
    for (int gb = gi0 + GS * U; gb < groups; gb += GS * U) {
        stage_load(gb);
        stage_store(gb);
    }
#pragma unroll
    for (int hh = 0; hh < SR; ++hh)
#pragma unroll
        for (int r = 0; r < 16; ++r) sl[r * (SGMAX + 1) + min(lane + 64 * hh, SGMAX)] = sv[hh][r];
    __syncthreads();

    // 5. the tile's steps
    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    const int tm = min(c16, cnt - 1);  // A rows past cnt read the last pair; their outputs are dropped
    auto unpack = [&](uint32_t w) {
        auto pair = [&](uint32_t v) {
            return S == SYM4_G128 ? ((v & MASK) ^ MAGIC) : ((v & MASK) | MAGIC);
        };
        return as_bf16x8(pair(w), pair(w >> 4), pair(w >> 8), pair(w >> 12));
    };
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const Buf& B, int s) {
        bf16x8_t A[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
            A[d] = *reinterpret_cast<const bf16x8_t*>(
                lds + 4 * ((s * 16 + d * 4 + g) * mp + (tm ^ gswz(mp, d * 4 + g))));
        uint32_t w[4] = {B[0], B[1], B[2], B[3]};
        if constexpr (GPS == 2) {
            const auto p02 = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);
            const auto p13 = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
            w[0] = p02[0]; w[2] = p02[1];
            w[1] = p13[0]; w[3] = p13[1];
        }
#pragma unroll
        for (int q = 0; q < GPS; ++q) {
            f32x4_t D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int d = 4 / GPS * q; d < 4 / GPS * (q + 1); ++d)
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[d], unpack(w[d]), D, 0, 0, 0);
            const f32x4_t DX = *reinterpret_cast<const f32x4_t*>(xd + (s * GPS + q) * 16 + 4 * g);
            const uint32_t swd = sl[c16 * (SGMAX + 1) + s * GPS + q];
            float sc, corr;
            if constexpr (T::AFFINE) {
                sc = bf16_bits_to_f32(swd & 0xFFFFu);
                corr = fmaf(-T::BIAS, sc, __uint_as_float(swd & 0xFFFF0000u));
            } else {
                sc = __uint_as_float(swd);
                corr = -T::BIAS * sc;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = fmaf(corr, DX[r], fmaf(sc, D[r], acc[r]));
        }
    };
    const int full = steps / DEPTH * DEPTH;
    for (int r0 = 0; r0 < full; r0 += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            load(cb[(u + DEPTH - 1) % DEPTH], r0 + u + DEPTH - 1);
            __builtin_amdgcn_sched_barrier(0);
            compute(cb[u], r0 + u);
        }
    }
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u)
        if (full + u < steps) compute(cb[u], full + u);

    // 6. part[pair][row] for the descriptor's pairs (slots past cnt hold
    //    garbage: their group sums were never staged)
    const int n = row0 + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int slot = 4 * g + r;
        if (slot < cnt) a.part[(int64_t)a.pairs[first + slot] * N + n] = acc[r];
    }
}

}  // namespace w4
