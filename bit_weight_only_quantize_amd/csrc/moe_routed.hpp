// Routed expert passes for several tokens.
//
// TurboFieldfare article (Gemma 4 26B-A4B section): each token runs 8 of 128
// experts plus the shared expert; only the selected experts' weights are read.
// With a few tokens per active expert (32 tokens x 8 slots over ~112 experts:
// about 2 each), a pass is many small skinny products, one per active expert,
// each over that expert's few activation rows. Here a workgroup owns one work
// descriptor (an expert and at most kMoeDescPairs of its pairs) and 64 rows
// of the pass's matrices: it gathers the descriptor's activation rows into
// LDS once, in the MFMA A-operand layout, and its wavefronts stream one row
// tile each with the scales staged per tile -- the skinny LDS kernel's step,
// so a step costs one 16-byte code load per matrix.
//
// Measured against the alternatives on the Gemma-shaped layer at M = 32: a
// per-expert-block kernel that loads the activation pieces from L2 with every
// step (gate/up 91 us, down 87 us per layer) and a persistent grouped gate/up
// pass with x for all tokens staged per CU and scales loaded per step (75 us).
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

// Column swizzle of row lr (0..15 within a step) of the staged activations
// for rows of mp (power of two, 2..32) units: rows of 16 or more units take
// lr rotated left by one in 4 bits, shorter rows their top bits rotated.
__device__ __forceinline__ int gswz(int mp, int lr) {
    if (mp >= 16) return ((lr << 1) | (lr >> 3)) & 15;
    const int b = 31 - __builtin_clz(mp);
    const int x = lr >> (4 - b);
    return ((x << 1) | (x >> (b - 1))) & (mp - 1);
}



// Routed expert passes for several tokens: one workgroup per (work
// descriptor j, block of 16 * RT rows per wavefront of the expert's
// matrices). The
// descriptor's pairs (at most kMoeDescPairs) are the MFMA tokens: their
// activation rows -- x of the pair's token for gate/up, the pair's own h row
// for down -- are gathered from L2 once per workgroup into LDS in the
// A-operand layout (the skinny kernel's layout and swizzle, with every
// (group, pair) activation sum). Wavefront w then streams its row tile of
// gate and up, or its RT row tiles of down, over all K, its scales in a
// private LDS block, DEPTH steps of code loads in flight, and writes its outputs:
// h[pair][row] = bf16(gelu(g) * u), or part[pair][row]. A small LDS footprint
// and few wavefronts (NW: 4 for gate/up, 8 for down) let several workgroups
// share a CU, so one workgroup's staging overlaps the others' streaming.
// A launch covers the shared expert (S0.codes set) as ceil(M /
// kMoeDescPairs) token descriptors of its own matrices (token t of descriptor
// s is token s * kMoeDescPairs + t), the routed descriptor slots (W0.codes
// set), or both; one workgroup per (descriptor, row block), the shared
// expert's first. Both kinds in one launch share its LDS layout (kmax).
struct MoeRoutedArgs {
    GMat W0, W1;            // gate, up (gate/up pass) or down (W1 unused)
    GMat S0, S1;            // the shared expert's, same roles
    const uint16_t* xin;    // routed activations: gate/up x [M][D]; down h [P][F]
    const uint16_t* xsh;    // shared activations: gate/up x [M][D]; down hs [M][Fs]
    int k;                  // gate/up: slots per token (pair -> token); down: 1 (pair -> h row)
    const int4* work;       // descriptors (count <= kMoeDescPairs); x < 0 past the last
    const int32_t* pairs;   // [P]
    uint16_t* h;            // gate/up out [P][F]
    uint16_t* hs;           // gate/up out [M][Fs]
    float* part;            // down out [P][D]
    float* sout;            // down out [M][D]
    int M, kmax;            // tokens, longest K (LDS layout)
};

constexpr int kRoutedMp = 8;  // activation rows staged per descriptor (>= kMoeDescPairs)
static_assert(kRoutedMp >= kMoeDescPairs, "a descriptor's pairs must fit the stage");

// LDS bytes of moe_routed_kernel for reduction length K
__host__ __device__ inline size_t moe_routed_lds_bytes(int K, int group, int sgmax, int waves, int nm) {
    const int steps = K / 128;
    const int gps = 128 / group;
    return ((size_t)steps * 16 * kRoutedMp * 4 + (size_t)steps * gps * 16 +
            (size_t)waves * nm * 16 * (sgmax + 1)) * 4;
}

template <int S, bool GU, int DEPTH, int SGMAX, int RT = 1, int NW = 4>
__global__ __launch_bounds__(64 * NW) void moe_routed_kernel(MoeRoutedArgs a) {
    using T = Traits<S>;
    using P = MfmaStep<S>;
    constexpr int GPS = P::GPS;
    // matrices streamed per wavefront: gate and up, or RT row tiles of down
    constexpr int NM = GU ? 2 : RT;
    static_assert(!GU || RT == 1, "gate/up streams one row tile of each matrix");
    constexpr int NV = T::GROUP / 8;  // 16-byte activation vectors per group
    constexpr int U = 4;
    constexpr uint32_t ONE2 = 0x3F803F80u;
    extern __shared__ __align__(16) uint32_t lds[];
    const int NT = blockDim.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    // workgroup b: the shared expert's (descriptor, row block) pairs first,
    // then the routed ones
    const int rows = (NT / 64) * 16 * RT;  // per workgroup
    const int sdesc = a.S0.codes ? (a.M + kMoeDescPairs - 1) / kMoeDescPairs : 0;
    const int rbs = a.S0.codes ? a.S0.N / rows : 0, rbr = a.W0.codes ? a.W0.N / rows : 0;
    int b = blockIdx.x;
    const bool sh = b < sdesc * rbs;
    int e = 0, first, cnt, rb;
    if (sh) {
        const int j = b / rbs;
        rb = b - j * rbs;
        first = j * kMoeDescPairs;
        cnt = min(kMoeDescPairs, a.M - first);
    } else {
        b -= sdesc * rbs;
        const int j = b / rbr;
        rb = b - j * rbr;
        const int4 wd = a.work[j];
        e = __builtin_amdgcn_readfirstlane(wd.x);
        if (e < 0) return;  // whole workgroup: an unused descriptor slot
        first = __builtin_amdgcn_readfirstlane(wd.y);
        cnt = __builtin_amdgcn_readfirstlane(wd.z);
    }
    const GMat& W0 = sh ? a.S0 : a.W0;
    const int K = W0.K, N = W0.N;
    const int groups = K / T::GROUP, steps = K / 128;
    int mp = 2;
    while (mp < cnt) mp *= 2;
    const int smax = a.kmax / 128;  // the LDS layout is the longest K's
    float* xd = reinterpret_cast<float*>(lds + smax * 16 * kRoutedMp * 4);
    uint32_t* sl = lds + smax * 16 * kRoutedMp * 4 + smax * GPS * 16 + wave * NM * 16 * (SGMAX + 1);

    const int row0 = rb * rows + wave * 16 * RT;  // N % rows == 0; tile m at row0 + 16 m
    const uint8_t* crow[NM];
    const uint8_t* scl[NM];
    const uint8_t* bil[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const GMat& W = sh ? (GU && m ? a.S1 : a.S0) : (GU && m ? a.W1 : a.W0);
        crow[m] = W.codes + (int64_t)e * W.stride_c + (int64_t)(row0 + (GU ? 0 : 16 * m) + c16) * (K / 2);
        scl[m] = W.scale + (int64_t)e * W.stride_s;
        bil[m] = T::AFFINE ? W.bias + (int64_t)e * W.stride_s : nullptr;
    }

    // staging lanes: one pair slot t and one 16-byte vector iv of a group;
    // NV consecutive lanes cover a group of one slot (coalesced; the group's
    // sum is a DPP reduction over them). Slots past cnt store nothing.
    const int C = mp * NV, GS = NT / C;
    const int c = threadIdx.x % C;
    const int gi0 = (int)threadIdx.x < GS * C ? (int)threadIdx.x / C : groups;
    const int t = c / NV, iv = c % NV;
    const bool live = t < cnt;
    const int xrow = sh ? first + min(t, cnt - 1) : a.pairs[first + min(t, cnt - 1)] / a.k;
    const uint16_t* xl = (sh ? a.xsh : a.xin) + (int64_t)xrow * K + iv * 8;
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
    // 2. the tiles' scales: a tile's 16 rows are consecutive in the scale
    //    (and bias) arrays, so 16-byte vectors over the lanes cover them in
    //    SV loads per array (16 * groups elements, a multiple of a vector);
    //    step 4 spreads them into the wavefront's LDS blocks
    constexpr int EB = T::AFFINE ? 2 : 4;  // bytes per element
    constexpr int EPV = 16 / EB;           // elements per vector
    constexpr int SV = (16 * SGMAX / EPV + 63) / 64;
    const int nvec = 16 * groups / EPV;
    u32x4_t svs[NM][SV];
    u32x4_t svb[T::AFFINE ? NM : 1][SV];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int64_t e0 = (int64_t)(row0 + (GU ? 0 : 16 * m)) * groups * EB;
#pragma unroll
        for (int j = 0; j < SV; ++j) {
            const int v = min(lane + 64 * j, nvec - 1);
            svs[m][j] = *gmem<u32x4_t>(scl[m] + e0 + 16 * v);
            if constexpr (T::AFFINE) svb[m][j] = *gmem<u32x4_t>(bil[m] + e0 + 16 * v);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // 3. the first DEPTH - 1 steps' codes, in the loop's order
    struct Buf {
        u32x4_t c[NM];
    };
    auto load = [&](Buf& B, int s) {
        s = min(s, steps - 1);
#pragma unroll
        for (int m = 0; m < NM; ++m) B.c[m] = *gmem<u32x4_t>(crow[m] + (uint32_t)s * 64 + 16 * g);
    };
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
    // element idx of a tile's block is row idx / groups, group idx % groups
    // (the quotient from a float product: exact, as idx < 16 * 128 and the
    // fraction stays at least 1/(2 groups) away from an integer); lanes past
    // the block store into the padding column (unconditional stores keep the
    // load waits exact). Affine words: bf16 scale low, bias high.
    const float rg = 1.0f / (float)groups;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int j = 0; j < SV; ++j) {
            const int v = lane + 64 * j;
            const bool ok = v < nvec;
#pragma unroll
            for (int q = 0; q < EPV; ++q) {
                const int idx = v * EPV + q;
                const int r = (int)(((float)idx + 0.5f) * rg);
                const int gi = idx - r * groups;
                uint32_t w;
                if constexpr (T::AFFINE) {
                    const uint32_t s2 = svs[m][j][q / 2], b2 = svb[m][j][q / 2];
                    w = (q & 1) ? ((s2 >> 16) | (b2 & 0xFFFF0000u)) : ((s2 & 0xFFFFu) | (b2 << 16));
                } else {
                    w = svs[m][j][q];
                }
                sl[(m * 16 + (ok ? r : 15)) * (SGMAX + 1) + (ok ? gi : SGMAX)] = w;
            }
        }
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
    f32x4_t acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const Buf& B, int s) {
        bf16x8_t A[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
            A[d] = *reinterpret_cast<const bf16x8_t*>(
                lds + 4 * ((s * 16 + d * 4 + g) * mp + (tm ^ gswz(mp, d * 4 + g))));
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            uint32_t w[4] = {B.c[m][0], B.c[m][1], B.c[m][2], B.c[m][3]};
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
                const uint32_t swd = sl[(m * 16 + c16) * (SGMAX + 1) + s * GPS + q];
                float sc, corr;
                if constexpr (T::AFFINE) {
                    sc = bf16_bits_to_f32(swd & 0xFFFFu);
                    corr = fmaf(-T::BIAS, sc, __uint_as_float(swd & 0xFFFF0000u));
                } else {
                    sc = __uint_as_float(swd);
                    corr = -T::BIAS * sc;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[m][r] = fmaf(corr, DX[r], fmaf(sc, D[r], acc[m][r]));
            }
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
    // the output stage's pair ids (see 6.), issued under the last steps
    int pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pv[r] = a.pairs[first + min(4 * g + r, cnt - 1)];
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u)
        if (full + u < steps) compute(cb[u], full + u);

    // 6. outputs of the descriptor's pairs (slots past cnt hold garbage:
    //    their group sums were never staged)
    const int n = row0 + c16;
    // the four pair ids first, unconditionally (clamped): a load under the
    // slot test compiles into a branch that waits for it, one round trip per slot
    // (for the shared expert's descriptors, first + slot < M <= the pair count)
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(pv[r]));  // the loads stay unconditional
    int64_t prs[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) prs[r] = sh ? first + min(4 * g + r, cnt - 1) : pv[r];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int slot = 4 * g + r;
        if (slot < cnt) {
            const int64_t pr = prs[r];
            if constexpr (GU) {
                (sh ? a.hs : a.h)[pr * N + n] = (uint16_t)f32_to_bf16_rne(gelu_tanh(acc[0][r]) * acc[1][r]);
            } else {
#pragma unroll
                for (int m = 0; m < NM; ++m) (sh ? a.sout : a.part)[pr * N + n + 16 * m] = acc[m][r];
            }
        }
    }
}

}  // namespace w4
