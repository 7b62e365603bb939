// Prefill GEMM with the dequantization fused in: Y = X * dequant(W)^T.
//
// airllm article §3.3: prefill is compute-dense (decode is memory-bound), so
// this is the one product on the hot path built on the matrix cores; §2.2: the
// weights are converted right after they are loaded instead of materializing a
// dequantized copy in HBM.
//
// Design for gfx950 (256 CUs in 8 XCDs, 160 KiB LDS, bf16 MFMA 32x32x16):
//   * a workgroup computes a 256 (M) x 128 (N) tile with 4 wavefronts, one per
//     SIMD, each owning all 256 rows of 32 columns (8 MFMA blocks of 32 x 32,
//     fp32 accumulators): every weight of the tile is dequantized once, at the
//     price of each X fragment being read by all four wavefronts;
//   * LDS bandwidth is the scarce resource (about 128 B/clk per CU for reads,
//     half that for ds_write_b128), so only the activations are staged there:
//     the X tile of each 64-wide k step (32 KiB) and the step's packed codes
//     (4 KiB) arrive by direct global->LDS loads (global_load_lds_dwordx4: no
//     registers, no ds_write) in a 4-stage ring, issued four steps ahead;
//   * each wavefront dequantizes its own B fragments in registers straight from
//     the codes -- w = s*q (sym) or s*u + b (affine), in fp32, rounded to nearest
//     even bf16 -- so no bf16 weight tile is ever written to or read from LDS;
//   * inside a step the contraction order of k is permuted so that one 16-byte
//     code read per column and lane covers the step's four k slices: slice kk of
//     lane half h takes the 8 weights of code word 4h + kk, and the A fragment
//     reads the matching 16-byte chunk of X;
//   * X chunks are XOR-swizzled by row (chosen through the source chunk each
//     lane of a direct load fetches) so MFMA operand reads are free of bank
//     conflicts;
//   * one barrier per step, in the middle of it: after it the next step's ring
//     stage is complete for every wavefront, the loads four steps ahead start
//     into the stage just drained (spread over the following MFMAs), and the
//     next step's first fragments are read and dequantized while this step's
//     last MFMAs run;
//   * tiles are ordered so consecutive tiles land on one XCD and share an X row
//     block (workgroups are dispatched round-robin over the 8 XCDs), keeping
//     that block resident in the XCD's L2;
//   * the epilogue rounds the fp32 accumulators to bf16 (nearest even).
#include "common.hpp"
#include "launch.hpp"

namespace w4 {

constexpr int GBM = 256, GBN = 128, GBK = 64, GSTAGES = 4;
// wavefront grid over the tile: WMN along M x WNN along N; each wavefront owns
// RM x CN outputs, NI x NJ MFMA blocks of 32 x 32
constexpr int WMN = 1, WNN = 4, RM = GBM / WMN, CN = GBN / WNN, NI = RM / 32, NJ = CN / 32;
constexpr int X_BYTES = GBM * GBK * 2;  // X tile of one step
constexpr int C_BYTES = GBN * GBK / 2;  // packed codes of one step
constexpr int STAGE_BYTES = X_BYTES + C_BYTES;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

// s_waitcnt vmcnt(n) lgkmcnt(0)
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}

// scheduling-group masks
constexpr int SG_VALU = 0x2, SG_MFMA = 0x8, SG_VMEM = 0x20, SG_DSR = 0x100;

template <int S>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* codes, const uint8_t* scale,
                                                   const uint8_t* bias, int M, int N, int K,
                                                   const uint16_t* X, uint16_t* __restrict__ Y,
                                                   int tiles_m, int tiles_n) {
    using T = Traits<S>;
    extern __shared__ __align__(16) uint8_t gsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a
    // contiguous range of tiles, N-fastest, so an XCD's workgroups share X rows.
    const int ntiles = tiles_m * tiles_n;
    const int per = (ntiles + 7) / 8;
    const int L = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (L >= ntiles) return;
    const int m0 = (L / tiles_n) * GBM, n0 = (L % tiles_n) * GBN;
    const int ksteps = K / GBK;

    // ---- direct-load sources of this wavefront. Rows and columns past the
    // matrix edge are clamped to the last one; their results are never stored.
    // X: load i covers tile rows 64*wave + 8*i + lane/8, and the lane fetches
    // the chunk that the swizzle puts at position lane%8 of its row.
    const uint16_t* xsrc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 64 * wave + 8 * i + (lane >> 3);
        const int c = (lane & 7) ^ ((lane >> 3) & 7);
        xsrc[i] = X + (int64_t)min(m0 + r, M - 1) * K + c * 8;
    }
    // codes: the load covers tile columns 32*wave + lane%32, half lane/32 of
    // the step's 32 code bytes per column
    const uint8_t* csrc =
        codes + (int64_t)min(n0 + 32 * wave + (lane & 31), N - 1) * (K / 2) + (lane >> 5) * 16;

    // ---- compute-side coordinates
    const int wm = wave / WNN, wn = wave % WNN;
    const int half = lane >> 5, l32 = lane & 31;
    const int64_t groups = K / T::GROUP;
    int64_t sidx[NJ];  // scale index of this lane's column j at group 0
#pragma unroll
    for (int j = 0; j < NJ; ++j) sidx[j] = (int64_t)min(n0 + wn * CN + 32 * j + l32, N - 1) * groups;

    // raw scale / bias bits of one step for the lane's two columns
    struct Sc {
        uint32_t s[NJ], b[NJ];
    };
    constexpr int NSC = T::AFFINE ? 2 * NJ : NJ;  // scale loads per batch
    constexpr int NB = NSC + 9;             // memory operations per batch

    // Batch t: the scale loads, then the direct loads of step t into ring stage
    // t % 4, issued in three parts spread over a step so that no wavefront
    // stalls behind a burst of loads: part 0 (scales, X loads 0..3), part 1
    // (X loads 4..7), part 2 (codes). A step past the end reloads the last step
    // into a stage nobody reads again: every batch is issued, so the in-order
    // load counter always holds whole batches and the waits below can count them.
    auto issue = [&](int t, Sc& sc, int part) {
        const int tc = min(t, ksteps - 1);
        uint8_t* st = gsm + (t % GSTAGES) * STAGE_BYTES;
        if (part == 0) {
            const int g = tc * GBK / T::GROUP;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if constexpr (T::AFFINE) {
                    sc.s[j] = reinterpret_cast<const uint16_t*>(scale)[sidx[j] + g];
                    sc.b[j] = reinterpret_cast<const uint16_t*>(bias)[sidx[j] + g];
                } else {
                    sc.s[j] = reinterpret_cast<const uint32_t*>(scale)[sidx[j] + g];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (part < 2) {
#pragma unroll
            for (int i = 4 * part; i < 4 * part + 4; ++i)
                __builtin_amdgcn_global_load_lds((gbl_void_t*)(xsrc[i] + tc * GBK),
                                                 (lds_void_t*)(st + (64 * wave + 8 * i) * 128), 16, 0, 0);
        } else {
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(csrc + tc * (GBK / 2)),
                                             (lds_void_t*)(st + X_BYTES + wave * 1024), 16, 0, 0);
        }
    };

    f32x16_t acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    bf16x8_t af[2][NI], bq[2][NJ];
    u32x4_t cw[NJ];  // this lane's 16 code bytes of the step, per column j
    // A fragments of slice kk: row wm*RM + 32i + l32, chunk 4*half + kk
    auto load_a = [&](int t, int kk, int buf) {
        const uint8_t* st = gsm + (t % GSTAGES) * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = wm * RM + 32 * i + l32;
            af[buf][i] = *reinterpret_cast<const bf16x8_t*>(st + r * 128 + (((4 * half + kk) ^ (r & 7)) << 4));
        }
    };
    auto load_codes = [&](int t) {
        const uint8_t* st = gsm + (t % GSTAGES) * STAGE_BYTES + X_BYTES;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            cw[j] = *reinterpret_cast<const u32x4_t*>(st + (NJ * wn + j) * 1024 + lane * 16);
    };
    // B fragments of slice kk: the 8 weights of code word kk (byte b holds
    // elements 2b, low nibble, and 2b + 1)
    auto dequant = [&](int kk, const Sc& sc, int buf) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float ws = T::AFFINE ? bf16_bits_to_f32(sc.s[j]) : __uint_as_float(sc.s[j]);
            const float wb = T::AFFINE ? bf16_bits_to_f32(sc.b[j]) : -8.f * ws;  // sym: q = u - 8
            uint32_t c = cw[j][kk];
            if constexpr (S == SYM4_G128) c ^= 0x88888888u;  // two's complement -> q + 8
            uint32_t lo = c & 0x0F0F0F0Fu;
            uint32_t hi = (c >> 4) & 0x0F0F0F0Fu;
            // hide the masks from the optimizer: it would otherwise fold them
            // into one bit-field extract per nibble instead of converting the
            // bytes of lo and hi directly (v_cvt_f32_ubyte0..3)
            asm("" : "+v"(lo), "+v"(hi));
            uint32_t o[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float e0 = (float)((lo >> (8 * b)) & 0xFFu);
                const float e1 = (float)((hi >> (8 * b)) & 0xFFu);
                const bf16x2_t pr = {(__bf16)fmaf(e0, ws, wb), (__bf16)fmaf(e1, ws, wb)};
                o[b] = __builtin_bit_cast(uint32_t, pr);
            }
            bq[buf][j] = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
        }
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bq[buf][j], acc[i][j], 0, 0, 0);
    };
    // The barrier orders the LDS traffic by itself (the counter waits before it
    // make each wavefront's loads and reads complete); the empty asm keeps the
    // compiler from moving memory operations across it.
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // interleave: each MFMA is followed by a share of the VALU, LDS reads and
    // global loads
    constexpr int VPM = (24 * NJ + NI * NJ - 1) / (NI * NJ);  // VALU per MFMA
    auto interleave = [&](int vm) {
#pragma unroll
        for (int r = 0; r < NI * NJ; ++r) {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            if (r < NI) __builtin_amdgcn_sched_group_barrier(SG_DSR, 1, 0);
            if (r >= NI * NJ - 4 && r - (NI * NJ - 4) < vm) __builtin_amdgcn_sched_group_barrier(SG_VMEM, 1, 0);
            __builtin_amdgcn_sched_group_barrier(SG_VALU, VPM, 0);
        }
    };

    // One step. Slices 0..2 run their MFMAs while slice kk+1 is read and
    // dequantized, and parts 1 and 2 of batch t+3 are issued. Then: this
    // wavefront's batch t+1 has landed (batches t+2 and t+3 may still be in
    // flight) and its LDS reads are done; the barrier makes that true for every
    // wavefront, so stage t+1 is readable and stage t, fully read, takes batch
    // t+4 (part 0 now). The last slice's MFMAs cover the reads and
    // dequantization of step t+1's first slice.
    auto step = [&](int t, Sc& cur, Sc& nxt, Sc& prev) {
#pragma unroll
        for (int kk = 0; kk < 3; ++kk) {
            if (kk == 0) issue(t + 3, prev, 1);
            if (kk == 1) issue(t + 3, prev, 2);
            load_a(t, kk + 1, (kk + 1) & 1);
            dequant(kk + 1, cur, (kk + 1) & 1);
            mfmas(kk & 1);
            interleave(kk == 0 ? 4 : kk == 1 ? 1 : 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vm_lgkm0<2 * NB>();
        barrier();
        issue(t + 4, cur, 0);
        load_codes(t + 1);
        load_a(t + 1, 0, 0);
        dequant(0, nxt, 0);
        mfmas(1);
        __builtin_amdgcn_sched_group_barrier(SG_DSR, NJ + NI, 0);
        __builtin_amdgcn_sched_group_barrier(SG_VMEM, NSC, 0);
#pragma unroll
        for (int r = 0; r < NI * NJ; ++r) {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            if (r < 4) __builtin_amdgcn_sched_group_barrier(SG_VMEM, 1, 0);
            __builtin_amdgcn_sched_group_barrier(SG_VALU, VPM, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    Sc sc0, sc1, sc2, sc3;
    for (int part = 0; part < 3; ++part) issue(0, sc0, part);
    for (int part = 0; part < 3; ++part) issue(1, sc1, part);
    for (int part = 0; part < 3; ++part) issue(2, sc2, part);
    issue(3, sc3, 0);
    // batch 0 landed: batches 1 and 2 and part 0 of batch 3 may be in flight
    wait_vm_lgkm0<2 * NB + NSC + 4>();
    barrier();
    load_codes(0);
    load_a(0, 0, 0);
    dequant(0, sc0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // whole rounds of four steps keep the loop free of exits: its header joins
    // one path only, so the compiler's own load-counter waits stay exact
    int t = 0;
    for (; t + 4 <= ksteps; t += 4) {
        step(t, sc0, sc1, sc3);
        step(t + 1, sc1, sc2, sc0);
        step(t + 2, sc2, sc3, sc1);
        step(t + 3, sc3, sc0, sc2);
    }
    if (t < ksteps) step(t, sc0, sc1, sc3);
    if (t + 1 < ksteps) step(t + 1, sc1, sc2, sc0);
    if (t + 2 < ksteps) step(t + 2, sc2, sc3, sc1);
    // no direct load may still be writing this workgroup's LDS when it retires
    wait_vm_lgkm0<0>();

    // ---- epilogue: D[i][j] of a 32x32 block sits in lane j + 32 * ((i / 4) % 2),
    // register 4 * (i / 8) + i % 4.
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int n = n0 + wn * CN + 32 * j + l32;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * RM + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
                if (m < M) {
                    const bf16x2_t pr = {(__bf16)acc[i][j][r], (__bf16)0.f};
                    Y[(int64_t)m * N + n] = (uint16_t)__builtin_bit_cast(uint32_t, pr);
                }
            }
        }
}

hipError_t launch_gemm(int scheme, const void* codes, const void* scale, const void* bias,
                       int64_t N, int64_t K, const uint16_t* X, int64_t M, uint16_t* Y,
                       hipStream_t st) {
    const int tm = (int)((M + GBM - 1) / GBM), tn = (int)((N + GBN - 1) / GBN);
    const int per = (tm * tn + 7) / 8;
    const size_t lds = (size_t)GSTAGES * STAGE_BYTES;
    auto kern = scheme == SYM4_G128 ? gemm_kernel<SYM4_G128> : gemm_kernel<AFF4_G64>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(kern, dim3(8 * per), dim3(256), lds, st, (const uint8_t*)codes,
                       (const uint8_t*)scale, (const uint8_t*)bias, (int)M, (int)N, (int)K, X, Y,
                       tm, tn);
    return hipGetLastError();
}

}  // namespace w4
