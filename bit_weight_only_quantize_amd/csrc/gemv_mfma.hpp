// Skinny decode GEMM (2 <= M <= 16 tokens) on the matrix cores.
//
// airllm article §2.2: the weights are dequantized in registers right after the
// load, no dequantized copy is written; §3.3: decode stays memory-bound. With
// several tokens the per-token dot products would make a VALU kernel compute-
// and LDS-bound (every token re-reads its activations), so here the unpacked
// codes feed v_mfma_f32_16x16x32_bf16 directly from registers:
//
//   * D[token][row] = A[token][k] * B[k][row]: A is 16 tokens x 32 k of
//     activations, B the 32 k x 16 weight rows; lane l holds weight row l % 16
//     and k = 8 (l / 16) + 0..7 of B, and rows 4 (l / 16) + 0..3 (tokens) of D,
//     so a lane's outputs all belong to one weight row and one group scale;
//   * a step is 128 weights of 16 rows: 16 bytes of codes per lane, one group
//     (sym) or two (affine). An MFMA's 32 k must not straddle two groups: for
//     affine, lanes 0-31 hold group A's words and lanes 32-63 group B's, so two
//     v_permlane32_swap per lane regroup them into operand registers of a
//     single group (the activation pieces are loaded in the matching k order);
//   * a code word (8 nibbles) unpacks with the magic-exponent trick into four
//     bf16 pairs (k, k+4) = 128 + u, so the activations are permuted the same
//     way (v_perm_b32) and the offset is removed per group with the group's
//     activation sums X, which one extra MFMA against a ones operand delivers
//     already in the D layout:  acc += s * D + (b - BIAS s) * X;
//   * activations come straight from global memory (L2-resident, 16-byte
//     loads issued before the step's code loads) and are reused by the RT row
//     tiles of a wavefront; the block's group scales are staged once in LDS
//     (one coalesced pass instead of a scattered 2-4 byte load per step);
//   * the WK wavefronts of a workgroup split K over the same rows, taking
//     interleaved steps (the workgroup reads WK consecutive 64-byte pieces of
//     every row at a time), DEPTH steps in flight each; their partial sums are
//     added through LDS in a fixed order, so results are deterministic.
#pragma once

#include "common.hpp"
#include "gemv_wave.hpp"

namespace w4 {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int S>
struct MfmaStep {
    // A step is 16 bytes of codes per lane: 128 weights of 16 rows for the
    // 4-bit schemes, 64 for the 8-bit one. Groups per step; activation
    // pieces (MFMAs) per step: 4, or 2 for 8-bit codes, whose bytes are
    // converted exactly (two per MFMA operand word pair)
    static constexpr int GPS = S == AFF4_G64 ? 2 : 1;
    static constexpr int PPS = S == AFF8_G64 ? 2 : 4;
    // k offset of activation piece d (8 weights, A operand of word d after the
    // regrouping) for lane group g, relative to the step's first k
    __device__ __forceinline__ static int xpiece(int g, int d) {
        if constexpr (GPS == 1) return 32 * g + 8 * d;
        // group A: own words of lanes 0-31, lanes 32-63 take lanes 0-31's third
        // and fourth words; group B symmetric
        return 32 * (g & 1) + 16 * (g >> 1) + 8 * (d & 1) + 64 * (d >> 1);
    }
};

// Global-address-space view of a pointer: loads through it are global_load,
// never flat_load (a flat load also counts against the LDS counter and makes
// the compiler wait for every outstanding memory operation). Pointers picked
// from a struct array with a runtime index lose the address space otherwise.
template <typename V>
__device__ __forceinline__ const __attribute__((address_space(1))) V* gmem(const void* p) {
    return (const __attribute__((address_space(1))) V*)p;
}

// bf16x8 from four packed bf16 pairs
__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4_t v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8_t, v);
}

// At most kMfmaMaxGroups groups per row (scales are staged in at most four
// 64-group slices).
constexpr int kMfmaMaxGroups = 256;

// 64-group slices to stage per row: 1, 2 or 4.
inline int mfma_slices(int64_t groups) { return groups <= 64 ? 1 : (groups <= 128 ? 2 : 4); }

// One row tile of 16 weight rows: rows row0 .. row0+15 of an N x K matrix
// (rows past N are read clamped and their outputs dropped by the caller).
struct MfmaTile {
    const uint8_t* codes;
    const uint8_t* scale;
    const uint8_t* bias;
    int row0, N;
};

// LDS: the workgroup's scales as [group][row] words (affine: bf16 scale in the
// low half, bf16 bias in the high half), later reused for the split-K sums.
template <int S, int RT, int WK, int WR = 1>
size_t gemv_mfma_lds_bytes(int64_t K) {
    const size_t scales = ((size_t)(K / Traits<S>::GROUP) * 16 * RT * WR + 1) * 4;  // + trash word
    const size_t red = (size_t)(WK > 1 ? WK - 1 : 1) * WR * RT * 4 * 64 * 4;
    return scales > red ? scales : red;
}

// The workgroup's product of WR x RT row tiles with up to 16 activation rows
// over the whole K. Wavefront w works on tiles tl[(w % WR) * RT ..] over the
// w / WR-th of WK contiguous step ranges. Every wavefront must call it (it
// synchronizes); the split-K sums end up in the acc of the wavefronts with
// w < WR (the others hold partial sums). Lane l's activation row starts at
// element xoff of the wave-uniform xbase (tokens past the valid ones point at a
// valid row; the caller drops their outputs).
template <int S, int RT, int WK, int DEPTH, int WR, int SL, bool IL = true>
__device__ __forceinline__ void mfma_tiles(const MfmaTile (&tl)[WR * RT], int K,
                                           const uint16_t* xbase, uint32_t xoff, uint32_t* lds,
                                           f32x4_t (&acc)[RT]) {
    using T = Traits<S>;
    using P = MfmaStep<S>;
    constexpr int GPS = P::GPS;
    constexpr int NW = WR * WK;       // wavefronts
    constexpr int ROWS = 16 * RT * WR;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wr = wave % WR, wk = wave / WR;
    const int g = lane >> 4, c16 = lane & 15;
    const int groups = K / T::GROUP;
    const int steps = (groups + GPS - 1) / GPS;  // an odd affine count ends with a half step
    const bool odd = GPS == 2 && (groups & 1);
    // wavefront wk's steps: wk, wk + WK, ... (interleaved, so that the
    // workgroup reads WK consecutive 64-byte pieces of every row at a time) or
    // one contiguous range
    const int J = (steps + WK - 1) / WK;
    const int nj = IL ? (wk < steps ? (steps - 1 - wk) / WK + 1 : 0) : max(0, min(J, steps - wk * J));
    auto step_of = [&](int j) {  // clamped: loads past the last step re-load it
        const int jj = min(j, max(nj - 1, 0));
        return min(IL ? wk + jj * WK : wk * J + jj, steps - 1);
    };

    // 1. the tiles' scales (and biases) -> LDS, loads issued first; SL slices
    //    of 64 groups per row (SL * 64 >= groups): one coalesced pass instead of
    //    scattered 2-4 byte loads every step. Every load is unconditional
    //    (indices clamped) so that no branch makes the compiler's wait counts
    //    conservative.
    constexpr int SR = (ROWS + NW - 1) / NW;  // rows staged per wavefront
    uint32_t sv[SR][SL];
#pragma unroll
    for (int k = 0; k < SR; ++k) {
        const int r = min(wave + NW * k, ROWS - 1);
        // the row's tile by selects (a runtime index into the tile array
        // would put the array in scratch memory)
        MfmaTile tt = tl[0];
#pragma unroll
        for (int q = 1; q < WR * RT; ++q)
            if (r / 16 == q) tt = tl[q];
        const int n = min(tt.row0 + r % 16, tt.N - 1);
#pragma unroll
        for (int j = 0; j < SL; ++j) {
            const int gi = min(lane + 64 * j, groups - 1);
            const uint32_t e = (uint32_t)n * (uint32_t)groups + (uint32_t)gi;
            if constexpr (T::AFFINE)
                sv[k][j] = (uint32_t)gmem<uint16_t>(tt.scale)[e] |
                           ((uint32_t)gmem<uint16_t>(tt.bias)[e] << 16);
            else
                sv[k][j] = gmem<uint32_t>(tt.scale)[e];
        }
    }
    asm volatile("" ::: "memory");  // keep the step loads behind these

    // 2. per-lane code offsets from this wavefront's tiles' (uniform) bases
    const uint8_t* cb[RT];
    uint32_t coff[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        MfmaTile tt = tl[rt];
#pragma unroll
        for (int q = 1; q < WR; ++q)
            if (wr == q) tt = tl[q * RT + rt];
        const int n = min(tt.row0 + c16, tt.N - 1);
        cb[rt] = tt.codes;
        coff[rt] = (uint32_t)n * (uint32_t)(K / 2);
    }

    struct Buf {
        u32x4_t xv[4];
        u32x4_t c[RT];
    };
    auto load = [&](Buf& B, int s) {
        // a half step (odd affine group count, last step) has no group B: its
        // loads are redirected into group A (results unused), never past a row
        const bool half = odd && s == steps - 1;
        const int gl = half ? (g & 1) : g;
        // activations first: in-order vmcnt then never waits for code bytes
#pragma unroll
        for (int d = 0; d < 4; ++d)
            B.xv[d] = *gmem<u32x4_t>(xbase + (xoff + (uint32_t)s * 128 +
                                              (uint32_t)P::xpiece(g, half ? (d & 1) : d)));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            B.c[rt] = *gmem<u32x4_t>(cb[rt] + coff[rt] + (uint32_t)s * 64 + 16 * gl);
        }
    };

    // DEPTH steps in flight. Loads are unconditional (a wavefront past its
    // last step re-loads that step, results unused): a load under a branch
    // would make the compiler wait for every outstanding load, prefetched
    // steps included.
    Buf buf[DEPTH];
#pragma unroll
    for (int p = 0; p < DEPTH - 1; ++p) load(buf[p], step_of(p));

    // scales land in LDS while the first steps' bytes are in flight; staged
    // values past the rows or groups go to a trash word (no branch, see above)
#pragma unroll
    for (int k = 0; k < SR; ++k) {
        const int r = wave + NW * k;
#pragma unroll
        for (int j = 0; j < SL; ++j) {
            const int gi = lane + 64 * j;
            lds[r < ROWS && gi < groups ? gi * ROWS + r : groups * ROWS] = sv[k][j];
        }
    }
    __syncthreads();

    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    const uint32_t ONE2 = 0x3F803F80u;  // bf16 pair (1, 1)
    const bf16x8_t ONES = as_bf16x8(ONE2, ONE2, ONE2, ONE2);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto unpack = [&](uint32_t w) {
        auto pair = [&](uint32_t v) {
            return S == SYM4_G128 ? ((v & MASK) ^ MAGIC) : ((v & MASK) | MAGIC);
        };
        return as_bf16x8(pair(w), pair(w >> 4), pair(w >> 8), pair(w >> 12));
    };
    auto compute = [&](const Buf& B, int s) {
        const bool half = odd && s == steps - 1;
        uint32_t sw[RT][GPS];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int q = 0; q < GPS; ++q)
                sw[rt][q] = lds[min(GPS * s + q, groups - 1) * ROWS + 16 * (wr * RT + rt) + c16];
        bf16x8_t A[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const u32x4_t e = B.xv[d];  // (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) ...
            A[d] = as_bf16x8(__builtin_amdgcn_perm(e[2], e[0], 0x05040100u),
                             __builtin_amdgcn_perm(e[2], e[0], 0x07060302u),
                             __builtin_amdgcn_perm(e[3], e[1], 0x05040100u),
                             __builtin_amdgcn_perm(e[3], e[1], 0x07060302u));
        }
        // group activation sums, one per group of the step, in the D layout
        f32x4_t DX[GPS];
#pragma unroll
        for (int q = 0; q < GPS; ++q) {
            DX[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (q == 1 && half) continue;
#pragma unroll
            for (int d = 4 / GPS * q; d < 4 / GPS * (q + 1); ++d)
                DX[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[d], ONES, DX[q], 0, 0, 0);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            uint32_t w[4] = {B.c[rt][0], B.c[rt][1], B.c[rt][2], B.c[rt][3]};
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
                if (q == 1 && half) continue;
                f32x4_t D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 4 / GPS * q; d < 4 / GPS * (q + 1); ++d)
                    D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[d], unpack(w[d]), D, 0, 0, 0);
                float sc, corr;
                if constexpr (T::AFFINE) {
                    sc = __uint_as_float(sw[rt][q] << 16);
                    corr = fmaf(-T::BIAS, sc, __uint_as_float(sw[rt][q] & 0xFFFF0000u));
                } else {
                    sc = __uint_as_float(sw[rt][q]);
                    corr = -T::BIAS * sc;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[rt][r] = fmaf(corr, DX[q][r], fmaf(sc, D[r], acc[rt][r]));
            }
        }
    };

    // step s + DEPTH - 1 is loaded while step s is computed; the ring is
    // unrolled so every buffer index is static
    for (int j0 = 0; j0 < nj; j0 += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const int j = j0 + u;
            load(buf[(u + DEPTH - 1) % DEPTH], step_of(j + DEPTH - 1));
            // keep the prefetch ahead of this step's compute: left alone, the
            // scheduler sinks the loads below the MFMAs and the loop degenerates
            // into load, wait, compute
            __builtin_amdgcn_sched_barrier(0);
            if (j < nj) compute(buf[u], step_of(j));
        }
    }

    // split-K partial sums: wavefronts wk > 0 hand theirs to wavefront wr
    // through LDS (the scale area, free once every wavefront is past its last
    // step), added in a fixed order
    if constexpr (WK > 1) {
        __syncthreads();
        float* red = reinterpret_cast<float*>(lds);
        if (wk > 0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red[((((wk - 1) * WR + wr) * RT + rt) * 4 + r) * 64 + lane] = acc[rt][r];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int w = 0; w < WK - 1; ++w)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[rt][r] += red[(((w * WR + wr) * RT + rt) * 4 + r) * 64 + lane];
        }
    }
}

// Dense decode GEMM: RT row tiles of one matrix of the group per workgroup.
template <int S, int RT, int WK, int DEPTH, int SL>
__global__ __launch_bounds__(64 * WK) void gemv_mfma_kernel(GemvGroupArgs a, int K, int M,
                                                            const uint16_t* x) {
    extern __shared__ __align__(16) uint32_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int t = blockIdx.x;
    int i = 0;
#pragma unroll
    for (int q = 1; q < kMaxGroup; ++q)
        if (q < a.count && t >= a.tile_start[q]) i = q;
    const int N = a.N[i];
    const int row0 = (t - a.tile_start[i]) * (16 * RT);
    MfmaTile tl[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) tl[rt] = MfmaTile{a.codes[i], a.scale[i], a.bias[i], row0 + 16 * rt, N};
    // tokens past M re-read row M-1; their outputs are never stored
    const uint32_t xoff = (uint32_t)min(c16, M - 1) * (uint32_t)K;
    f32x4_t acc[RT];
    mfma_tiles<S, RT, WK, DEPTH, 1, SL>(tl, K, x, xoff, lds, acc);
    if (wave != 0) return;
    float* y = a.y[i];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int n = row0 + 16 * rt + c16;
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m < M) y[(int64_t)m * N + n] = acc[rt][r];
        }
    }
}

// ---------------------------------------------------------------- activations in LDS
// Variant for launches of at most 16 tiles per CU. One workgroup per CU
// stages x in LDS, already permuted into the MFMA A-operand layout and with
// every (group, token) activation sum, so a step costs a wavefront one
// 16-byte code load, four LDS reads, one LDS scale read per group and the
// MFMAs of one 16-row tile: no per-step activation loads, permutes or sum
// MFMAs, which cost more than the weight stream itself in the kernel above
// once M reaches 8-16. The workgroup owns TP consecutive 16-row tiles; each
// tile's steps are split over WK wavefronts (K-slices) whose partial sums
// meet in LDS at the end, so a CU has TP * WK wavefronts streaming codes.
// When x does not fit, the steps go in chunks of CS: the workgroup stages a
// chunk, its wavefronts run their slices of it, and the next chunk replaces
// it after a barrier.
//   LDS words: A unit (s, d, g, t) -- the 8 activations of piece d of lane
//   group g at chunk step s for token t, as the MFMA operand (x0,x4)(x1,x5)
//   (x2,x6)(x3,x7) -- in row (s * 4 + d) * 4 + g of Mp units (M rounded up
//   to a power of two), at column t ^ swz(Mp, d * 4 + g); then the sums as
//   floats [(s * GPS + q) * 16 + t]; then one scale block per wavefront.
//   The swizzle sends the 16 rows of a step that the staging lanes of one
//   (group, token) pair write to 16 different bank slots, and keeps every
//   row a permutation of its tokens for the readers. After the last chunk
//   the same memory holds the K-slices' partial tiles.
template <int S>
struct MfmaLdsLayout {
    static constexpr int GPS = MfmaStep<S>::GPS;
    static constexpr int RPS = 4 * MfmaStep<S>::PPS;  // A rows per step
    int groups, steps, mp, aw, sw;  // whole-K groups and steps; A and sums words of a chunk
    __host__ __device__ MfmaLdsLayout(int K, int M, int CS) {
        groups = K / Traits<S>::GROUP;
        steps = (groups + GPS - 1) / GPS;
        mp = 2;
        while (mp < M) mp *= 2;
        aw = CS * RPS * mp * 4;
        sw = CS * GPS * 16;
    }
    // bytes of A and sums for a chunk of CS steps
    __host__ __device__ size_t bytes() const { return (size_t)(aw + sw) * 4; }
};

// Column swizzle of row lr (0..15 within a step) for rows of mp = 2^b units:
// the row's top b bits, rotated left by one. Units of one row slot (lr mod
// 16/mp) then differ in their column for every top-bits value, and the two
// pairs a 16-lane group of the 4-bit g64 staging holds (tokens t, t + 1) land
// on opposite column parities.
__device__ __forceinline__ int lds_swz(int mp, int lr) {
    const int b = 31 - __builtin_clz(mp);
    const int x = lr >> (4 - b);
    return ((x << 1) | (x >> (b - 1))) & (mp - 1);
}

// blockDim.x >= 64 * TP * WK; wavefront w < TP * WK works on tile
// blockIdx.x * TP + w % TP over K-slice w / TP (ceil(chunk steps / WK) steps
// of every chunk; in a short last chunk a slice can be empty); all wavefronts
// stage activations. DEPTH steps of code loads in flight per streaming
// wavefront. SGMAX (at most 128) bounds the groups of a slice: the scale
// block's row stride. CHUNKED: x goes in several chunks (CS < steps).
// PARTS (K parts: KP > 1, one matrix, not CHUNKED): the grid is KP runs of
// gridDim.x / KP workgroups; run p covers steps [p * CS, p * CS + CS) of every
// tile, as one chunk, and writes its partial outputs to part + p * M * N
// ([M][N]). A template switch, so that the other launches keep constant
// chunk offsets.
//
// GATED (one pass, no K parts): matrices 0 (gate) and 1 (up) of equal N, tiles
// interleaved (tile 2j = rows 16j.. of gate, 2j + 1 the same rows of up) with
// an even TP, so a workgroup holds both halves of each pair; the up wavefront
// hands its tile to the gate wavefront through LDS, which stores
// h = bf16(gelu_tanh(g) * u) to a.h instead of y.
template <int S, int DEPTH, int SGMAX, bool CHUNKED, bool PARTS = false, int UW = 4,
          bool GATED = false>
__global__ __launch_bounds__(1024) void gemv_mfma_lds_kernel(GemvGroupArgs a, int K, int M,
                                                              const uint16_t* x, int tiles,
                                                              int TP, int WK, int CS, int KP,
                                                              float* part) {
    using T = Traits<S>;
    using P = MfmaStep<S>;
    constexpr int GPS = P::GPS;
    constexpr int NV = T::GROUP / 8;  // 16-byte activation vectors per group
    constexpr int U = CHUNKED ? 2 : UW;  // staging vectors in flight per lane (registers)
    constexpr uint32_t ONE2 = 0x3F803F80u;
    const int NT = blockDim.x;
    extern __shared__ __align__(16) uint32_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const MfmaLdsLayout<S> Lo(K, M, CS);
    constexpr int RPS = MfmaLdsLayout<S>::RPS, PPS = P::PPS;
    const int groups = Lo.groups, steps = Lo.steps, mp = Lo.mp;
    const bool odd = GPS == 2 && (groups & 1);
    float* xd = reinterpret_cast<float*>(lds + Lo.aw);
    uint32_t* sl = lds + Lo.aw + Lo.sw + wave * 16 * (SGMAX + 1);  // streaming wavefronts only

    // the first TP * WK wavefronts stream codes: this one's tile and K-slice
    // (the last workgroup's wavefronts past the last tile redo the last tile
    // and store nothing); the others only help stage the activations
    const bool comp = wave < TP * WK;
    const int tw = wave % TP, ks = min(wave / TP, WK - 1);
    const int gpp = PARTS ? (int)gridDim.x / KP : 0;  // workgroups per K part
    const int kp = PARTS ? (int)blockIdx.x / gpp : 0;
    const int tile_raw = ((int)blockIdx.x - kp * gpp) * TP + tw;
    const int tile = min(tile_raw, tiles - 1);
    int i = 0;
    if constexpr (GATED) {
        i = tile & 1;
    } else {
#pragma unroll
        for (int q = 1; q < kMaxGroup; ++q)
            if (q < a.count && tile >= a.tile_start[q]) i = q;
    }
    const int N = a.N[i];
    const int row0 = GATED ? (tile >> 1) * 16 : (tile - a.tile_start[i]) * 16;
    const uint8_t* codes = a.codes[i];
    const uint8_t* scale = a.scale[i];
    const uint8_t* bias = a.bias[i];
    const int n = min(row0 + c16, N - 1);
    const uint8_t* crow = codes + (int64_t)n * (K * T::BITS / 8);
    const int tm = min(c16, M - 1);  // tokens past M read token M-1; their outputs are dropped

    // staging lanes: a lane keeps one token t and one 16-byte vector iv of a
    // group (NV consecutive lanes cover a group of one token: coalesced, and
    // the group's sum is a DPP reduction over them) and walks the chunk's
    // groups gi0, gi0 + GS, ...; C lanes cover a group of all tokens, the
    // workgroup's first GS * C threads stage (GS >= 1), the rest load clamped
    // addresses and store nothing, as do lanes of tokens past M
    const int C = mp * NV, GS = NT / C;
    const int c = threadIdx.x % C;
    const int gi0 = (int)threadIdx.x < GS * C ? (int)threadIdx.x / C : groups;
    const int t = c / NV, iv = c % NV;
    const bool live = t < M;
    const uint16_t* xl = x + (int64_t)min(t, M - 1) * K + iv * 8;
    // vector iv of a group is piece d of lane group gg (the inverse of the
    // codes' piece order); for GPS = 2, d also depends on q
    const int gg = S == AFF8_G64 ? (iv >> 1) : GPS == 1 ? (iv >> 2) : ((iv >> 2) | (((iv >> 1) & 1) << 1));

    const uint32_t MASK = opaque(0x000F000Fu);
    const uint32_t MAGIC = unpack_magic<S>();
    auto unpack = [&](uint32_t w) {
        auto pair = [&](uint32_t v) {
            return S == SYM4_G128 ? ((v & MASK) ^ MAGIC) : ((v & MASK) | MAGIC);
        };
        return as_bf16x8(pair(w), pair(w >> 4), pair(w >> 8), pair(w >> 12));
    };

    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // one pass when x (or the K part's x) fits (CHUNKED false: no loop for
    // the compiler to hoist lane constants out of, which would cost registers
    // the ring needs)
    const int cbeg = kp * CS;
    const int c_end = CHUNKED ? steps : cbeg + 1;
    for (int c0 = cbeg; c0 < c_end; c0 += CHUNKED ? CS : 1) {
        const int cn = min(CS, steps - c0);                        // chunk steps
        const int cg0 = c0 * GPS, cgn = min(groups, (c0 + cn) * GPS) - cg0;  // chunk groups
        const int spw = (cn + WK - 1) / WK;
        const int lb = ks * spw;                   // slice start (chunk step)
        const int ns = min(cn, lb + spw) - lb;     // slice steps, <= 0 if empty
        const int lbl = min(lb, cn - 1), nsl = max(ns, 1);  // addresses of an empty slice
        if (c0 > cbeg) __syncthreads();            // the previous chunk's LDS reads are done

        u32x4_t xr[U];
        auto stage_load = [&](int gb) {
#pragma unroll
            for (int j = 0; j < U; ++j)
                xr[j] = *gmem<u32x4_t>(xl + (cg0 + min(gb + j * GS, cgn - 1)) * T::GROUP);
        };
        auto stage_store = [&](int gb) {
#pragma unroll
            for (int j = 0; j < U; ++j) {
                float part = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) part = dot2_bf16(ONE2, xr[j][e], part);
                const float sum = group_sum<NV>(part);
                const int gi = gb + j * GS;
                if (live && gi < cgn) {
                    const int st = gi / GPS, q = gi - st * GPS;
                    const int d = S == AFF8_G64 ? (iv & 1) : GPS == 1 ? (iv & 3) : (2 * q + (iv & 1));
                    // 4-bit: the (k, k + 4) pair order of the nibble unpack;
                    // 8-bit: bytes convert in order, the vector stays as loaded
                    const u32x4_t o = S == AFF8_G64 ? xr[j] : u32x4_t{__builtin_amdgcn_perm(xr[j][2], xr[j][0], 0x05040100u),
                                       __builtin_amdgcn_perm(xr[j][2], xr[j][0], 0x07060302u),
                                       __builtin_amdgcn_perm(xr[j][3], xr[j][1], 0x05040100u),
                                       __builtin_amdgcn_perm(xr[j][3], xr[j][1], 0x07060302u)};
                    const int lr = d * 4 + gg;
                    *reinterpret_cast<u32x4_t*>(lds + 4 * ((st * RPS + lr) * mp + (t ^ lds_swz(mp, lr)))) = o;
                    if (iv == 0) xd[(st * GPS + q) * 16 + t] = sum;
                }
            }
        };
        // codes of slice step ls (lane: row c16, 16-byte piece g of the step;
        // a half step redirects group B's piece into group A; plain loads:
        // nontemporal ones measured slower here); steps past the slice reload
        // its last
        using Buf = u32x4_t;
        auto load = [&](Buf& B, int ls) {
            const int s = c0 + lbl + min(ls, nsl - 1);
            const bool half = odd && s == steps - 1;
            const int gl = half ? (g & 1) : g;
            B = *gmem<u32x4_t>(crow + (uint32_t)s * 64 + 16 * gl);
        };

        // 1. the chunk's first round of activation loads goes out first: the
        //    load counter drains in order, so its waits then cover these L2
        //    reads only, not the HBM loads issued after it
        stage_load(gi0);
        __builtin_amdgcn_sched_barrier(0);
        // staging-only wavefronts: the rest of the staging, the barrier, and
        // (branch taken per wavefront, so each path's load waits stay exact)
        if (!comp) {
            stage_store(gi0);
            for (int gb = gi0 + GS * U; gb < cgn; gb += GS * U) {
                stage_load(gb);
                stage_store(gb);
            }
            __syncthreads();
            continue;
        }
        // 2. the slice's scales (affine: bf16 scale low, bf16 bias high) of
        //    the tile's 16 rows, for the wavefront's LDS block of 16 rows x
        //    (SGMAX + 1) words (odd stride: the 16 rows a step reads sit in
        //    16 banks); lanes walk a row's groups (coalesced), 64 at a time
        const int sg0 = (c0 + lbl) * GPS, sg = min(groups, (c0 + lbl + nsl) * GPS) - sg0;
        constexpr int SR = (SGMAX + 63) / 64;
        uint32_t sv[SR][16];
#pragma unroll
        for (int h = 0; h < SR; ++h) {
            const int sgl = min(lane + 64 * h, sg - 1);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t e = (uint32_t)min(row0 + r, N - 1) * (uint32_t)groups + (uint32_t)(sg0 + sgl);
                if constexpr (T::AFFINE)
                    sv[h][r] = (uint32_t)gmem<uint16_t>(scale)[e] | ((uint32_t)gmem<uint16_t>(bias)[e] << 16);
                else
                    sv[h][r] = gmem<uint32_t>(scale)[e];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // 3. the first DEPTH - 1 steps' code loads, in flight during the
        //    staging; issued step by step (the loop's order) so the
        //    load-counter wait the compiler puts at the loop head is the same
        //    from both predecessors
        Buf cb[DEPTH];
#pragma unroll
        for (int p = 0; p < DEPTH - 1; ++p) {
            load(cb[p], p);
            __builtin_amdgcn_sched_barrier(0);
        }
        // 4. activations and sums into LDS, then the scales (unconditional:
        //    a branch would leave the scale loads possibly in flight at the
        //    join and blur the load waits after it; lanes past the slice
        //    write columns nobody reads, or the padding column)
        stage_store(gi0);
        for (int gb = gi0 + GS * U; gb < cgn; gb += GS * U) {
            stage_load(gb);
            stage_store(gb);
        }
#pragma unroll
        for (int h = 0; h < SR; ++h)
#pragma unroll
            for (int r = 0; r < 16; ++r) sl[r * (SGMAX + 1) + min(lane + 64 * h, SGMAX)] = sv[h][r];
        __syncthreads();

        // 5. the slice's steps
        auto compute = [&](const Buf& B, int ls) {
            const int sc_ = lb + ls;  // chunk step
            const bool half = odd && c0 + sc_ == steps - 1;
            bf16x8_t A[PPS];
#pragma unroll
            for (int d = 0; d < PPS; ++d)
                A[d] = *reinterpret_cast<const bf16x8_t*>(
                    lds + 4 * ((sc_ * RPS + d * 4 + g) * mp + (tm ^ lds_swz(mp, d * 4 + g))));
            uint32_t w[4] = {B[0], B[1], B[2], B[3]};
            if constexpr (S == AFF8_G64) {
                // one group per step, two MFMAs over the byte codes converted
                // exactly (v_cvt_f32_ubyte, then a bf16 pair): D = sum x * q,
                // so w = s q + b adds b times the activation sum
                f32x4_t D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    uint32_t o[4];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t c = w[2 * d + h];
#pragma unroll
                        for (int b = 0; b < 2; ++b) {
                            const bf16x2_t pr = {(__bf16)(float)((c >> (16 * b)) & 0xFFu),
                                                 (__bf16)(float)((c >> (16 * b + 8)) & 0xFFu)};
                            o[2 * h + b] = __builtin_bit_cast(uint32_t, pr);
                        }
                    }
                    D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[d], as_bf16x8(o[0], o[1], o[2], o[3]), D, 0, 0, 0);
                }
                const f32x4_t DX = *reinterpret_cast<const f32x4_t*>(xd + sc_ * 16 + 4 * g);
                const uint32_t swd = sl[c16 * (SGMAX + 1) + min(ls, sg - 1)];
                const float sc = bf16_bits_to_f32(swd & 0xFFFFu);
                const float corr = __uint_as_float(swd & 0xFFFF0000u);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf(corr, DX[r], fmaf(sc, D[r], acc[r]));
                return;
            }
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
                if (q == 1 && half) continue;
                f32x4_t D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int d = PPS / GPS * q; d < PPS / GPS * (q + 1); ++d)
                    D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[d], unpack(w[d]), D, 0, 0, 0);
                const f32x4_t DX = *reinterpret_cast<const f32x4_t*>(xd + (sc_ * GPS + q) * 16 + 4 * g);
                const uint32_t swd = sl[c16 * (SGMAX + 1) + min(ls * GPS + q, sg - 1)];
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
        // step ls + DEPTH - 1 is loaded while step ls is computed; the ring
        // is unrolled so every buffer index is static. Whole rounds run in
        // the loop (nothing in it is conditional: a skipped load would make
        // the compiler's load-counter waits conservative); the last round,
        // after it, loads once and computes only the slice's remaining steps
        if (ns > 0) {  // wave-uniform
            const int rounds = (ns + DEPTH - 1) / DEPTH;
            for (int r0 = 0; r0 < (rounds - 1) * DEPTH; r0 += DEPTH) {
#pragma unroll
                for (int u = 0; u < DEPTH; ++u) {
                    load(cb[(u + DEPTH - 1) % DEPTH], r0 + u + DEPTH - 1);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(cb[u], r0 + u);
                }
            }
            const int r0 = (rounds - 1) * DEPTH;
            load(cb[DEPTH - 1], r0 + DEPTH - 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < DEPTH; ++u)
                if (r0 + u < ns) compute(cb[u], r0 + u);
        }
    }

    // staging-only wavefronts leave (a barrier waits for surviving
    // wavefronts only)
    if (!comp) return;
    // K-slices meet: every streaming wavefront parks its partial tile in LDS
    // (the activations are no longer read), slice 0 adds the others, stores
    if (WK > 1) {
        __syncthreads();
        *reinterpret_cast<f32x4_t*>(lds + 4 * threadIdx.x) = acc;
        __syncthreads();
        if (ks != 0) return;  // wave-uniform, after the last barrier
        for (int k = 1; k < WK; ++k) {
            const f32x4_t o = *reinterpret_cast<const f32x4_t*>(lds + 4 * ((k * TP + tw) * 64 + lane));
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += o[r];
        }
    }
    if constexpr (GATED) {
        // pairs meet: the up wavefront parks its tile, the gate wavefront
        // (tw even, its partner tw + 1 in this workgroup) finishes the pair
        __syncthreads();  // LDS reads of the reduction / activations are done
        if (i == 1) *reinterpret_cast<f32x4_t*>(lds + 4 * (tw * 64 + lane)) = acc;
        __syncthreads();
        if (i == 1 || tile_raw >= tiles) return;
        const f32x4_t u = *reinterpret_cast<const f32x4_t*>(lds + 4 * ((tw + 1) * 64 + lane));
        const int nn = row0 + c16;
        if (nn < N) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g + r;
                if (m < M) a.h[(int64_t)m * N + nn] = (uint16_t)f32_to_bf16_rne(gelu_tanh(acc[r]) * u[r]);
            }
        }
        return;
    }
    if (tile_raw >= tiles) return;
    float* y = PARTS ? part + (int64_t)kp * M * N : a.y[i];
    const int nn = row0 + c16;
    if (nn < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m < M) y[(int64_t)m * N + nn] = acc[r];
        }
    }
}

}  // namespace w4
