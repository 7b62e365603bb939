// Host-side launchers shared between the translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4 {

hipError_t launch_quantize_pack(int scheme, const float* W, int64_t N, int64_t K, void* codes,
                                void* scale, void* bias, hipStream_t st);

// Largest K the skinny kernels can stage in LDS for one token.
constexpr int64_t kMaxSkinnyK = 28672;
constexpr int kKvHeadDim = 128;  // INT4 KV cache: values per head vector

struct GemvPlan {
    int lpr, v, r, mt;
    int64_t blocks;
    size_t lds;
};
GemvPlan plan_gemv(int scheme, int64_t N, int64_t K, int64_t M);

// M = 1, one wavefront per row, up to 4 matrices sharing x in one launch.
bool gemv_wave_ok(int scheme, int64_t K);
hipError_t launch_gemv_wave(int scheme, int count, const void* const* codes,
                            const void* const* scale, const void* const* bias, const int64_t* N,
                            int64_t K, const uint16_t* x, float* const* y, hipStream_t st);

// 2 <= M <= 16, 4-bit schemes: unpacked codes feed bf16 MFMA from registers.
bool gemv_mfma_ok(int scheme, int64_t K, int64_t M);
// part: room for K-part partial outputs (gemv_mfma_split_bytes of them) or
// null; with it, a single matrix whose activations do not fit LDS takes K
// parts on different CUs and a summing launch instead of chunks
hipError_t launch_gemv_mfma(int scheme, int count, const void* const* codes,
                            const void* const* scale, const void* const* bias, const int64_t* N,
                            int64_t K, const uint16_t* x, int64_t M, float* const* y,
                            hipStream_t st, float* part = nullptr);
// gate and up ([N][K] each, 4-bit) for 2 <= M <= 16 in one launch whose
// epilogue writes h = bf16(gelu_tanh(gate x) * (up x)), bf16 [M][N]; the
// same bits as the two GEMVs and the activation. hipErrorNotSupported
// (nothing launched) where x does not fit one pass.
hipError_t launch_gemv_mfma_gated(int scheme, const void* const* gate, const void* const* up,
                                  int64_t N, int64_t K, const uint16_t* x, int64_t M, uint16_t* h,
                                  hipStream_t st);
// bytes of partial outputs the K-part plan needs (0: no K parts for this shape)
size_t gemv_mfma_split_bytes(int scheme, int64_t N, int64_t K, int64_t M);

// 2 <= M <= 64, same design with token tiles staged in LDS.
bool gemv_wave_mt_ok(int scheme, int64_t K, int64_t M);
hipError_t launch_gemv_wave_mt(int scheme, int count, const void* const* codes,
                               const void* const* scale, const void* const* bias, const int64_t* N,
                               int64_t K, const uint16_t* x, int64_t M, float* const* y,
                               hipStream_t st);

hipError_t launch_gemv(int scheme, const void* codes, const void* scale, const void* bias,
                       int64_t N, int64_t K, const uint16_t* x, int64_t M, float* y,
                       hipStream_t st);

// ---- prefill GEMM (4-bit schemes), bf16 out
hipError_t launch_gemm(int scheme, const void* codes, const void* scale, const void* bias,
                       int64_t N, int64_t K, const uint16_t* X, int64_t M, uint16_t* Y,
                       hipStream_t st);

// ---- mixture of experts
struct MoeMats {
    int64_t E, D, F, Fs;  // experts, d_model, expert FFN width, shared FFN width (0 = none)
    const void* gate[3];  // codes, scale, bias of the stacked matrices
    const void* up[3];
    const void* down[3];
    const void* sgate[3];
    const void* sup[3];
    const void* sdown[3];
};

// Routed (token, slot) pairs per call: M <= 256 tokens times top_k <= 32.
constexpr int kMoeMaxPairs = 256 * 32;
constexpr int kMoeDescPairs = 8;  // pairs per work descriptor (at most one MFMA token tile)
// work descriptors for P pairs over E experts (one per 16 pairs of an expert)
inline int moe_slots(int64_t E, int64_t P) {
    return (int)((E < P ? E : P) + (P + kMoeDescPairs - 1) / kMoeDescPairs);
}

struct MoeWorkspace {  // byte offsets inside the caller's workspace
    size_t work, pairs, h, hs, part, sout, total;
};
MoeWorkspace moe_workspace_layout(int64_t M, int k, int64_t E, int64_t D, int64_t F, int64_t Fs);

hipError_t launch_route(int scheme, const void* codes, const void* scale, const void* bias,
                        int64_t E, int64_t K, const uint16_t* x, int64_t M, int k, float* logits,
                        int32_t* ids, float* wts, hipStream_t st);
hipError_t launch_moe(int scheme, const MoeMats& W, const uint16_t* x, int64_t M, const int32_t* ids,
                      const float* wts, int k, void* ws, float* y, hipStream_t st);
// Top-k selection from router logits [M][E], then launch_moe; ids/wts are
// outputs. One token with E <= 128: the selection runs inside the gate/up pass.
hipError_t launch_moe_logits(int scheme, const MoeMats& W, const uint16_t* x, int64_t M,
                             const float* logits, int k, int32_t* ids, float* wts, void* ws,
                             float* y, hipStream_t st);

// ---- one-token MoE layer in one launch (router, top-k, shared and routed
// experts); hand-off words at the start of its workspace, zero between calls.
// A device-scope atomic or coherent access to one line costs ~10 ns and
// serializes with every other access to that line, so a count with many
// contributors is split over kSyncRep sub-counters on lines of their own, and
// what many workgroups poll is replicated on kSyncRep lines. Values that are
// polled carry their own "written" mark (never zero once written), so a
// consumer polls the data itself instead of a separate flag.
constexpr int kSyncLine = 32;  // words per 128-byte line
constexpr int kSyncRep = 32;   // sub-counters / replicas
constexpr int kHRep = 8;       // copies of h (one per XCD's readers)
constexpr int kLayerMaxE = 128, kLayerMaxK = 8;
enum : int {
    kSyncErr = 1,       // give-ups of this call (bits)
    kSyncStatus = 2,    // give-ups of the last call (bits), kept for the host
    kSyncHTop = 3,      // h sub-counters completed
    kSyncExitTop = 4,   // exit sub-counters completed
    kSyncLogits = 1 * kSyncLine,  // kLayerMaxE (value, 1) word pairs: 8 lines
    kSyncSel = kSyncLogits + 2 * kLayerMaxE,  // + r * kSyncLine: ids + 1, then weights | 2^31
    kSyncHSub = kSyncSel + kSyncRep * kSyncLine,       // + r * kSyncLine: gate/up items done
    kSyncHDoneRep = kSyncHSub + kSyncRep * kSyncLine,  // + r * kSyncLine: every h row in
    kSyncExitSub = kSyncHDoneRep + kSyncRep * kSyncLine,  // + r * kSyncLine: workgroups out
    kLayerSyncWords = kSyncExitSub + kSyncRep * kSyncLine,
};
constexpr unsigned kGaveUpLogits = 1, kGaveUpIds = 2, kGaveUpH = 4;
struct MoeLayerWorkspace {  // byte offsets
    size_t sync, h, multi, total;  // multi: where the launch sequence's area starts
};
bool moe_layer_ok(int rscheme, int k, int64_t E, int64_t D, int64_t F, int64_t Fs);
// The single launch's area (sync words, logit replicas, h copies), then the
// launch sequence's (router logits [M][E], then the w4a16_moe_gemv workspace):
// the two never overlap, so either path may follow the other on one workspace.
MoeLayerWorkspace moe_layer_workspace_layout(int64_t M, int k, int64_t E, int64_t D, int64_t F,
                                             int64_t Fs);
// router: codes, scale, bias of the [E][D] router (8-bit affine)
hipError_t launch_moe_layer(int scheme, int rscheme, const MoeMats& W, const void* const* router,
                            const uint16_t* x, int k, int32_t* ids, float* wts, void* ws,
                            float* y, long long wait_limit, int withhold, hipStream_t st);

// ---- dense gated FFN: h = bf16(gelu_tanh(W_gate x) * (W_up x)), y = W_down h
struct FfnWorkspace {  // byte offsets: hand-off words, h (copies, or the
    size_t sync, h, g, u, part, total;  // sequence's h), g and u, down K parts
};
FfnWorkspace ffn_workspace_layout(int scheme, int64_t M, int64_t D, int64_t F);
// one token in one persistent launch (4-bit schemes, D / 32 in (64, 256],
// F / 32 in (320, 512]); hipErrorNotSupported (nothing launched) otherwise
bool ffn_fused_ok(int scheme, int64_t D, int64_t F);
hipError_t launch_ffn_fused(int scheme, const void* const* gate, const void* const* up,
                            const void* const* down, int64_t D, int64_t F, const uint16_t* x,
                            uint16_t* h, float* y, void* ws, long long wait_limit, int withhold,
                            hipStream_t st);
// one token, the gate/up rows alone (4-bit: D / 32 <= 256; 8-bit: D / 16 <= 512): h to h
bool ffn_gate_up_ok(int scheme, int64_t D, int64_t F);
hipError_t launch_ffn_gate_up(int scheme, const void* const* gate, const void* const* up, int64_t D,
                              int64_t F, const uint16_t* x, uint16_t* h, hipStream_t st);
hipError_t launch_ffn_act(const float* g, const float* u, uint16_t* h, int64_t n, hipStream_t st);

// ---- INT4 KV cache (head vectors of kKvHeadDim values)
int kv_chunks(int64_t T);  // position chunks of the weighted sum (partials per head)
hipError_t launch_kv_quantize(const float* const* x, int ncache, int64_t n, int64_t H,
                              int64_t pos, int64_t T_max, uint8_t* const* codes,
                              float* const* scales, hipStream_t st);
// xnew (fp32 [T - pos][Hkv][128], or null): positions pos .. T - 1 are quantized
// into codes/scales by the product's own launch and never read from the cache
constexpr int kKvFuseMax = 16;  // the entry points fuse appends of up to this many positions
hipError_t launch_kv_scores(const float* q, int64_t Hq, int64_t Hkv, int64_t T, int64_t T_max,
                            const uint8_t* codes, const float* scales, float* scores,
                            const float* xnew, int64_t pos, hipStream_t st);
hipError_t launch_kv_weighted_sum(const float* p, int64_t Hq, int64_t Hkv, int64_t T,
                                  int64_t T_max, const uint8_t* codes, const float* scales,
                                  float* out, float* part, const float* xnew, int64_t pos,
                                  hipStream_t st);

}  // namespace w4
