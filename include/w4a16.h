/*
 * w4a16.h - group-wise 4-bit weight-only quantization with the dequantization
 * fused into the matrix products, for AMD MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [airllm]          airllm article, cf-1.com/news/5708464: §2.1 (groups of 128
 *                     consecutive weights), §2.2 (row-grouped layout; dequant fused
 *                     into the matmul kernel, converted in registers right after the
 *                     weight load), §3.3 (prefill compute-dense, decode memory-bound),
 *                     §4.2 (group_quantize: scale = absmax/7, clamp_min 1e-8,
 *                     round, clamp to +-7, two codes per byte, low nibble first).
 *   [TurboFieldfare]  TurboFieldfare / Gemma 4 26B-A4B article,
 *                     cnblogs.com/32bin/p/23195374: section 量化和精度 (affine
 *                     4-bit, 64 weights per group, one bf16 scale and one bf16 bias
 *                     per group; 8-bit router; codes used exactly as stored); the
 *                     model section (128 routed experts, 8 per token, an always-on
 *                     shared expert added without routing weight); the .gturbo
 *                     layout (128 experts per layer at a fixed stride).
 *
 * Conventions shared by every entry point
 *   - Weights W are [N][K] (output rows x input columns). Groups run along K inside
 *     one row. K must be a multiple of the scheme's group size.
 *   - 4-bit codes: uint8 [N][K/2]; byte j of a row holds element 2j in its low
 *     nibble and element 2j+1 in its high nibble. Symmetric codes are two's
 *     complement nibbles in [-7, 7]; affine codes are unsigned [0, 15].
 *     8-bit codes: uint8 [N][K], one per byte, unsigned [0, 255].
 *   - Scales: W4_SYM4_G128 -> fp32 [N][K/128]; affine -> bf16 [N][K/64] scale and
 *     bf16 [N][K/64] bias. A weight is scale*q (sym) or scale*q + bias (affine).
 *   - Activations are bf16 (raw uint16 bit patterns), row-major [M][K].
 *   - Every pointer except those documented as host pointers is a DEVICE pointer.
 *     The caller owns every buffer; the library never allocates, frees or keeps a
 *     pointer after the call returns (w4a16_moe_gemv_noalloc works in a static
 *     array of the library's own instead of a caller workspace). Work is enqueued on `stream` (a hipStream_t
 *     passed as void*, NULL = the default stream); no call synchronizes the device.
 *   - Device pointers must be 16-byte aligned (W4_EALIGN otherwise).
 *   - Arguments are validated on the host before anything is enqueued; on error
 *     nothing is launched and the return value is negative. w4_last_error() gives
 *     a message for the last failing call on the calling thread.
 *   - M == 0 or N == 0 is a successful no-op. NaN/Inf inputs give unspecified
 *     (but memory-safe) results.
 *   - Results are deterministic: no floating-point atomics; a call repeated on the
 *     same inputs returns the same bits.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---- */
#define W4_OK          0
#define W4_EINVAL     (-1) /* null pointer, unknown scheme or flag */
#define W4_ESHAPE     (-2) /* K not a multiple of the group, sizes out of range */
#define W4_EALIGN     (-3) /* a device pointer not 16-byte aligned */
#define W4_EHIP       (-4) /* HIP runtime or launch error */
#define W4_EWORKSPACE (-5) /* workspace missing or too small */

/* ---- quantization schemes ---- */
#define W4_SYM4_G128 0 /* symmetric 4-bit, group 128, fp32 scale = absmax/7 [airllm] §4.2 */
#define W4_AFF4_G64  1 /* affine 4-bit, group 64, bf16 scale + bf16 bias [TurboFieldfare] 量化和精度 */
#define W4_AFF8_G64  2 /* affine 8-bit, group 64, bf16 scale + bf16 bias (router) [TurboFieldfare] 量化和精度 */

/*
 * A quantized matrix, or a stack of `num_experts` matrices of identical shape
 * stored back to back at a fixed stride ([TurboFieldfare]: 128 fixed-stride expert
 * blobs per layer). All three arrays are [num_experts][N][...] as described above.
 * `bias` is NULL for W4_SYM4_G128 and required otherwise.
 */
typedef struct w4_matrix {
    int32_t scheme;      /* W4_SYM4_G128, W4_AFF4_G64 or W4_AFF8_G64 */
    int32_t num_experts; /* >= 1 */
    int64_t N;           /* rows per matrix (output features) */
    int64_t K;           /* columns (input features) */
    const void* codes;
    const void* scale;
    const void* bias;
} w4_matrix;

/*
 * Host-only. Byte sizes of the three storage arrays of one N x K matrix.
 * Any of the output pointers (host) may be NULL. Returns W4_EINVAL for an unknown
 * scheme, W4_ESHAPE for N < 0, K < 0 or K not a multiple of the group.
 */
int w4_packed_sizes(int scheme, int64_t N, int64_t K,
                    size_t* codes_bytes, size_t* scale_bytes, size_t* bias_bytes);

/*
 * quantize_pack. W: fp32 [N][K]. Writes codes/scale/bias in the storage form above.
 * sym  ([airllm] §4.2): per group a = max|w|; s = max(a/7, 1e-8) in fp32;
 *      q = clamp(rint(w/s), -7, 7) (round half to even).
 * aff  ([TurboFieldfare] 量化和精度; the min/max rule is a reading):
 *      s = bf16(max((max-min)/(2^b-1), 1e-8)), b = bf16(min) (round to nearest even);
 *      q = clamp(rint((w-b)/s), 0, 2^b-1) using the stored bf16 values.
 * All arithmetic is IEEE fp32 with correctly rounded division and no contraction,
 * so the output is bit-identical to a host implementation of the same steps.
 */
int w4_quantize_pack(int scheme, const float* W, int64_t N, int64_t K,
                     void* codes, void* scale, void* bias, void* stream);

/*
 * Decode GEMV / skinny GEMM with the dequantization fused into the product
 * ([airllm] §2.2, §3.3): y[m][n] = sum_k x[m][k] * w[n][k] for m < M, n < N,
 * accumulated in fp32. x: bf16 [M][K]; y: fp32 [M][N]. 1 <= M <= 64.
 * W must be a single matrix (num_experts == 1).
 */
int w4a16_gemv(const w4_matrix* W, const uint16_t* x, int64_t M, float* y, void* stream);

/*
 * Several decode GEMVs that share one activation input x, served by a single
 * launch when M == 1 (the Q, K and V projections of a layer, or its gate and up
 * projections). [airllm] §3.1 fuses operators to cut kernel launches;
 * [TurboFieldfare] runs the projections that share an input side by side.
 * Ws: host array of `count` descriptors (1 <= count <= 4), all single matrices
 * with the same scheme and K; ys: host array of device pointers, ys[i] fp32
 * [M][Ws[i]->N]. Results are identical to `count` separate w4a16_gemv calls.
 */
int w4a16_gemv_multi(const w4_matrix* const* Ws, int count, const uint16_t* x, int64_t M,
                     float* const* ys, void* stream);

/*
 * Host-only. Bytes of device workspace with which w4a16_gemv_ws splits the
 * reduction over K of W (one matrix) across CUs for M tokens; 0 when it does
 * not (then w4a16_gemv_ws runs w4a16_gemv's path and needs no workspace). A
 * split applies at 2 <= M <= 16 when the activations
 * (M * K bf16) do not fit one CU's LDS, e.g. K = 11008 at M = 16 or
 * K = 13824 at M = 8. Invalid arguments give 0.
 */
size_t w4_gemv_workspace_bytes(const w4_matrix* W, int64_t M);

/*
 * w4a16_gemv (same operation, arguments and limits) with a caller-provided
 * workspace: device memory of at least w4_gemv_workspace_bytes(W, M) bytes
 * (W4_EWORKSPACE otherwise; may be NULL when that is 0); its contents on entry
 * do not matter and on return are unspecified. Decode is memory-bound
 * ([airllm] §3.3): where x does not fit a CU's LDS, w4a16_gemv stages it in
 * chunks that each drain the weight stream, while here K is cut into parts
 * whose activations each fit, every part's tiles stream on their own CUs into
 * partial outputs in the workspace, and a second launch adds the parts in a
 * fixed order. Deterministic; the sums are ordered differently from
 * w4a16_gemv's, so the two agree to the error bound, not bit for bit.
 */
int w4a16_gemv_ws(const w4_matrix* W, const uint16_t* x, int64_t M, float* y, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Prefill GEMM ([airllm] §3.3: prefill is compute-dense): Y = X * dequant(W)^T with
 * bf16 inputs, fp32 accumulation and bf16 output (round to nearest even).
 * X: bf16 [M][K]; Y: bf16 [M][N]; any M >= 0. W: single matrix, 4-bit scheme.
 */
int w4a16_gemm(const w4_matrix* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream);

/*
 * MoE router ([TurboFieldfare], model section and 量化和精度): logits = x * Wr^T
 * (fp32 accumulate; Wr is [E][K], usually W4_AFF8_G64), then per token the top_k
 * experts by logit, largest first, ties to the lower expert index, and their
 * softmax probabilities over all E raw logits (no softcap, not renormalized).
 * x: bf16 [M][K]. Outputs: logits fp32 [M][E], ids int32 [M][top_k] and weights
 * fp32 [M][top_k] (all required). 1 <= top_k <= min(E, 32), E <= 1024.
 */
int w4_moe_route(const w4_matrix* router, const uint16_t* x, int64_t M, int top_k,
                 float* logits, int32_t* ids, float* weights, void* stream);

/*
 * Host-only. Workspace bytes w4a16_moe_gemv needs for these sizes
 * (E experts, d_model D, expert FFN width F, shared FFN width Fs, 0 = none).
 */
size_t w4_moe_workspace_bytes(int64_t M, int top_k, int64_t E, int64_t D, int64_t F, int64_t Fs);

/*
 * Mixture-of-experts FFN that reads only the selected experts
 * ([TurboFieldfare]: 8 of 128 experts per token; shared expert added unweighted;
 * shared and routed FFNs computed side by side):
 *   y[m] = sum_j weights[m][j] * FFN_{ids[m][j]}(x[m])  +  FFN_shared(x[m])
 *   FFN(x) = W_down * h,  h = bf16(gelu_tanh(W_gate x) * (W_up x))
 * gate, up: stacks [E][F][D]; down: stack [E][D][F]. shared_gate/up: [Fs][D],
 * shared_down: [D][Fs]; pass all three shared pointers NULL for no shared expert.
 * All six matrices must use the same 4-bit scheme, with D, F, Fs multiples of its
 * group. ids/weights as produced by w4_moe_route; a slot whose id lies outside
 * [0, E) contributes nothing. 1 <= M <= 256, 1 <= top_k <= 32, E <= 1024.
 * x: bf16 [M][D]; y: fp32 [M][D]. workspace: device memory of at least
 * w4_moe_workspace_bytes(...) bytes (W4_EWORKSPACE otherwise); its contents on
 * entry do not matter and on return are unspecified.
 */
int w4a16_moe_gemv(const w4_matrix* gate, const w4_matrix* up, const w4_matrix* down,
                   const w4_matrix* shared_gate, const w4_matrix* shared_up,
                   const w4_matrix* shared_down,
                   const uint16_t* x, int64_t M, const int32_t* ids, const float* weights,
                   int top_k, void* workspace, size_t workspace_bytes, float* y, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. w4a16_moe_gemv with the
 * same arguments, results and errors, except that its workspace is a
 * library-owned static device array of W4_MOE_SCRATCH_BYTES per GPU (set up on
 * the first call on each device and held until the process ends) instead of a
 * caller buffer. The call allocates nothing. W4_EWORKSPACE when the sizes need
 * more than W4_MOE_SCRATCH_BYTES (w4_moe_workspace_bytes gives the need).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (e.g. on two streams) race and must be serialized by the caller. Nothing in
 * it needs to start at zero; its contents between calls are unspecified.
 */
#define W4_MOE_SCRATCH_BYTES ((size_t)16 << 20)
int w4a16_moe_gemv_noalloc(const w4_matrix* gate, const w4_matrix* up, const w4_matrix* down,
                           const w4_matrix* shared_gate, const w4_matrix* shared_up,
                           const w4_matrix* shared_down,
                           const uint16_t* x, int64_t M, const int32_t* ids, const float* weights,
                           int top_k, float* y, void* stream);

/*
 * Router selection and the MoE FFN in one call, from router logits computed
 * beforehand (e.g. by w4a16_gemv on the router): the selection of
 * w4_moe_route ([TurboFieldfare], model section: top_k experts by logit,
 * largest first, ties to the lower expert index; softmax probabilities over all
 * E raw logits, no softcap, not renormalized), then w4a16_moe_gemv with it.
 * For one token with E <= 128 the selection runs inside the expert launches
 * instead of in a launch of its own.
 * logits: fp32 [M][E], E = the experts' count. Outputs: ids int32 [M][top_k],
 * weights fp32 [M][top_k], y fp32 [M][D]; ids and weights equal what
 * w4_moe_route selects from the same logits, bit for bit. Everything else
 * (matrices, shapes, workspace, errors) as for w4a16_moe_gemv;
 * 1 <= top_k <= min(E, 32).
 */
int w4a16_moe_gemv_logits(const w4_matrix* gate, const w4_matrix* up, const w4_matrix* down,
                          const w4_matrix* shared_gate, const w4_matrix* shared_up,
                          const w4_matrix* shared_down,
                          const uint16_t* x, int64_t M, const float* logits, int top_k,
                          int32_t* ids, float* weights, void* workspace, size_t workspace_bytes,
                          float* y, void* stream);

/*
 * One MoE layer from its input ([TurboFieldfare], model section and 量化和精度):
 * router logits = x * Wr^T, per token the top_k experts with their softmax
 * weights (exactly as w4_moe_route), then the FFN of w4a16_moe_gemv with them.
 * Results (ids, weights, y) equal those of w4_moe_route followed by
 * w4a16_moe_gemv, bit for bit, on either of the two paths below.
 * By default one token takes three launches (the router GEMV; the gate/up
 * pass, each of whose workgroups selects the experts from the logits itself;
 * the down pass with the weighted combine) and several tokens the launches of
 * w4_moe_route and w4a16_moe_gemv. With w4_moe_layer_set_single_launch(1), one
 * token with an 8-bit affine router, E <= 128, top_k <= 8, 2048 <= D <= 4096,
 * 32 <= F <= 1024 and Fs <= 4096 runs as ONE launch instead ([TurboFieldfare]'s
 * M2 time table spends a third of each token in waits between dependent GPU
 * submissions): the router rows, the selection, the shared and selected
 * experts' gate/up rows and the down rows are work items of a grid no larger
 * than the GPU holds at once, handing results to each other through
 * device-scope words in the workspace, the down rows' weights streaming while
 * the gate/up rows are computed. On this GPU each such hand-off costs about
 * what a launch boundary costs, so the default stays the launch sequence.
 * router: [E][D] single matrix; the experts as for w4a16_moe_gemv.
 * x: bf16 [M][D]; ids int32 [M][top_k], weights fp32 [M][top_k], y fp32 [M][D].
 * workspace: device memory of at least w4_moe_layer_workspace_bytes(...) bytes
 * (sized for the largest M it will serve), all zero before its first use
 * (e.g. one hipMemset when it is allocated); every call leaves the single
 * launch's hand-off words zero again, and either path may follow the other on
 * one workspace. Calls sharing a workspace must not overlap. A wait inside
 * the single launch that exceeds the poll limit (w4_moe_layer_set_wait) gives
 * up instead of hanging: the call then completes with unspecified y and
 * reports it through w4_moe_layer_status.
 */
size_t w4_moe_layer_workspace_bytes(int64_t M, int top_k, int64_t E, int64_t D, int64_t F,
                                    int64_t Fs);
int w4a16_moe_layer(const w4_matrix* router, const w4_matrix* gate, const w4_matrix* up,
                    const w4_matrix* down, const w4_matrix* shared_gate,
                    const w4_matrix* shared_up, const w4_matrix* shared_down,
                    const uint16_t* x, int64_t M, int top_k, int32_t* ids, float* weights,
                    float* y, void* workspace, size_t workspace_bytes, void* stream);

/* Host-side setting read by later w4a16_moe_layer calls from any thread:
 * enable != 0 selects the single launch for one token where it applies. */
void w4_moe_layer_set_single_launch(int enable);

/*
 * Outcome of the last single-launch w4a16_moe_layer call that used `workspace`
 * (device pointer): *status (host) = 0 if every hand-off completed, else a set
 * of W4_MOE_LAYER_GAVE_UP_* bits. Copies one word to the host and synchronizes
 * `stream`.
 */
#define W4_MOE_LAYER_GAVE_UP_LOGITS 1 /* the wait for the router logits gave up */
#define W4_MOE_LAYER_GAVE_UP_IDS 2 /* a wait for the expert selection gave up */
#define W4_MOE_LAYER_GAVE_UP_H   4 /* a wait for the gate/up rows gave up */
int w4_moe_layer_status(const void* workspace, int32_t* status, void* stream);

/*
 * Testing hook (host-side setting read by later w4a16_moe_layer calls from any
 * thread): each wait inside the single launch polls at most max_polls times
 * (<= 0 restores the default of 2^21 polls, a few seconds); withhold != 0 makes the launch
 * never publish its expert selection, so that every wait for it gives up.
 */
void w4_moe_layer_set_wait(int64_t max_polls, int withhold);

/*
 * Dense gated FFN of one decode layer: per token h = bf16(gelu_tanh(W_gate x) *
 * (W_up x)) (round to nearest even; the pages name no activation, this is the
 * gated GELU of the Gemma family, the one the expert FFN uses), then y = W_down h
 * (fp32 accumulate). [airllm] §3.1 credits its decode speed to fusing a layer's
 * operators into fewer kernel launches; [TurboFieldfare]'s M2 time table
 * spends a third of each token waiting between dependent GPU submissions.
 * One token (D / 32 <= 256 with 4-bit codes, D / 16 <= 512 with 8-bit ones)
 * takes two launches: the gate/up rows with the activation in their epilogue
 * (h written once, bf16), then the down GEMV. 2 to 16 tokens take two as well
 * where the skinny kernel can pair each gate tile with the up tile of the same
 * rows in one workgroup (its epilogue writes h). Other shapes, or
 * W4_FFN_PATH_SEQUENCE: three launches (gate and up in one GEMV launch, the
 * activation, down with K parts for 2 <= M <= 16 where h does not fit a CU).
 * W4_FFN_PATH_SINGLE_LAUNCH
 * runs one token with a 4-bit scheme, D / 32 in (64, 256] and F / 32 in
 * (320, 512] (e.g. the 7B and 13B shapes) as ONE launch: the gate/up rows and
 * the down rows are work items of a grid no larger than the GPU holds at once,
 * the down rows' weights streaming before h is complete, h handed over through
 * device-scope words and copies in the workspace. On this GPU that hand-off
 * (and the down rows' arithmetic, which can only start once h is complete)
 * costs more than the launch boundary it removes, so it is not the default.
 * All paths give the same bits for one token.
 * gate, up: single matrices [F][D]; down: [D][F]; one scheme for all three.
 * x: bf16 [M][D]; h: bf16 [M][F] out, or NULL; y: fp32 [M][D] out; 0 <= M <= 64,
 * D, F <= 28672. workspace: device memory of at least w4_ffn_workspace_bytes(down,
 * M) bytes (sized for the largest M it will serve), all zero before its first
 * use (e.g. one hipMemset when it is allocated); every call leaves its hand-off
 * words zero again. Calls sharing a workspace must not overlap. A wait inside
 * the single launch that exceeds the poll limit (w4_ffn_set_wait) gives up
 * instead of hanging: the call then completes with those rows of y unwritten
 * and reports it through w4_ffn_status.
 */
size_t w4_ffn_workspace_bytes(const w4_matrix* down, int64_t M);
int w4a16_ffn(const w4_matrix* gate, const w4_matrix* up, const w4_matrix* down,
              const uint16_t* x, int64_t M, uint16_t* h, float* y, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * The gate/up half of w4a16_ffn on its own: h = bf16(gelu_tanh(W_gate x) *
 * (W_up x)), bf16 [M][F] (required), the launches w4a16_ffn takes for that half
 * (one where the gate/up rows carry the activation in their epilogue, else a
 * GEMV launch and the activation). workspace: at least w4_ffn_gate_up_workspace_bytes(gate,
 * M) bytes, contents irrelevant. Same limits and errors as w4a16_ffn.
 */
size_t w4_ffn_gate_up_workspace_bytes(const w4_matrix* gate, int64_t M);
int w4a16_ffn_gate_up(const w4_matrix* gate, const w4_matrix* up, const uint16_t* x, int64_t M,
                      uint16_t* h, void* workspace, size_t workspace_bytes, void* stream);

/* Host-side setting read by later w4a16_ffn and w4a16_ffn_gate_up calls from
 * any thread (W4_EINVAL for another value). */
#define W4_FFN_PATH_DEFAULT 0       /* two launches for one token where they apply */
#define W4_FFN_PATH_SINGLE_LAUNCH 1 /* one persistent launch for one token where it applies */
#define W4_FFN_PATH_SEQUENCE 2      /* always the three-launch sequence */
int w4_ffn_set_path(int path);

/*
 * Outcome of the last single-launch w4a16_ffn call that used `workspace` (device
 * pointer): *status (host) = 0 if every hand-off completed, else
 * W4_FFN_GAVE_UP_H. Copies one word to the host and synchronizes `stream`.
 */
#define W4_FFN_GAVE_UP_H 4 /* a wait for the gate/up rows gave up */
int w4_ffn_status(const void* workspace, int32_t* status, void* stream);

/*
 * Testing hook (host-side setting read by later w4a16_ffn calls from any
 * thread): each wait inside the single launch polls at most max_polls times
 * (<= 0 restores the default of 2^21 polls, a few seconds); withhold != 0 makes
 * the launch never announce that h is complete, so that every wait gives up.
 */
void w4_ffn_set_wait(int64_t max_polls, int withhold);

/*
 * INT4 KV cache ([Shimmy] §3.2, TurboShimmy INT4 KV): each head vector of
 * W4_KV_HEAD_DIM fp32 values is quantized on its own: scale = max|v| / 7.5
 * (fp32), integers round(v / scale) (halves away from zero, as the page's
 * f32::round) clamped to [-8, 7], stored plus 8 as nibbles, element 2j in the
 * low nibble of byte j; an all-zero vector gets scale 0 and every nibble 8. A
 * cached value reads back as (nibble - 8) * scale.
 * Cache layout (caller-allocated, [Shimmy] §3.1 sizes it per layer): codes
 * uint8 [Hkv][T_max][W4_KV_HEAD_DIM / 2], scales fp32 [Hkv][T_max]; one head's
 * positions are contiguous. Query head h reads key/value head h / (Hq / Hkv).
 */
#define W4_KV_HEAD_DIM 128

/*
 * Quantize n new positions of Hkv head vectors into the cache: x fp32
 * [n][Hkv][W4_KV_HEAD_DIM] -> codes/scales at positions pos .. pos + n - 1.
 * 0 <= pos, pos + n <= T_max (W4_ESHAPE otherwise). n == 0 is a no-op.
 */
int w4_kv_quantize(const float* x, int64_t n, int64_t Hkv, int64_t pos, int64_t T_max,
                   uint8_t* codes, float* scales, void* stream);

/*
 * The same for the keys and the values of the same positions in one launch
 * ([Shimmy] §3.2: K and V are quantized on append): k, v fp32
 * [n][Hkv][W4_KV_HEAD_DIM] into their own caches of one shape. Results equal two
 * w4_kv_quantize calls bit for bit.
 */
int w4_kv_append(const float* k, const float* v, int64_t n, int64_t Hkv, int64_t pos,
                 int64_t T_max, uint8_t* k_codes, float* k_scales, uint8_t* v_codes,
                 float* v_scales, void* stream);

/*
 * scores[h][t] = sum_i q[h][i] * k[t][i] for the first T cached positions, with
 * the dequantization fused into the product ([Shimmy] §3.2: the shader
 * dequantizes while it computes the attention scores). q fp32 [Hq][D]; scores
 * fp32 [Hq][T]. Scaling by 1/sqrt(D), masking and the softmax are the caller's.
 * 1 <= T <= T_max; Hq a multiple of Hkv (W4_ESHAPE otherwise). Deterministic.
 */
int w4_kv_scores(const float* q, int64_t Hq, int64_t Hkv, int64_t T, int64_t T_max,
                 const uint8_t* codes, const float* scales, float* scores, void* stream);

/*
 * The key append fused into the scores ([Shimmy] §3.2 quantizes on append;
 * [airllm] §3.1 fuses the operators of a step): k_new fp32
 * [n][Hkv][W4_KV_HEAD_DIM] is quantized into positions pos .. pos + n - 1 of the
 * key cache, and scores fp32 [Hq][T] are written over the T = pos + n positions.
 * Cache contents and scores equal w4_kv_quantize then w4_kv_scores bit for bit.
 * For n <= 16 this is one launch, which takes the new positions' codes and
 * scales from registers and reads only positions < pos from the cache; for
 * larger n the append launch, then the scores launch. 1 <= n, pos + n <= T_max,
 * other shapes and errors as for w4_kv_quantize and w4_kv_scores.
 */
int w4_kv_scores_append(const float* q, const float* k_new, int64_t n, int64_t Hq, int64_t Hkv,
                        int64_t pos, int64_t T_max, uint8_t* k_codes, float* k_scales,
                        float* scores, void* stream);

/* Host-only. Workspace bytes w4_kv_weighted_sum needs for Hq heads over T positions. */
size_t w4_kv_weighted_sum_workspace_bytes(int64_t Hq, int64_t T);

/*
 * out[h][i] = sum_t p[h][t] * v[t][i] over the first T cached positions (the
 * value side of attention, dequantization fused in). p fp32 [Hq][T] (e.g. the
 * softmax of the scores); out fp32 [Hq][D]. Positions are summed in chunks whose
 * partial outputs go to the workspace (device memory of at least
 * w4_kv_weighted_sum_workspace_bytes(Hq, T) bytes, W4_EWORKSPACE otherwise;
 * contents on entry do not matter, on return unspecified), then added in a fixed
 * order. Shapes and errors as for w4_kv_scores.
 */
int w4_kv_weighted_sum(const float* p, int64_t Hq, int64_t Hkv, int64_t T, int64_t T_max,
                       const uint8_t* codes, const float* scales, float* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * The value append fused into the weighted sum, as w4_kv_scores_append does for
 * the keys: v_new fp32 [n][Hkv][W4_KV_HEAD_DIM] goes into positions pos .. pos +
 * n - 1 of the value cache, and out fp32 [Hq][W4_KV_HEAD_DIM] is the weighted sum
 * over the T = pos + n positions with p fp32 [Hq][T]. The workspace needs
 * w4_kv_weighted_sum_workspace_bytes(Hq, T) bytes. Cache contents and out equal
 * w4_kv_quantize then w4_kv_weighted_sum bit for bit. For n <= 16 the append
 * adds no launch; for larger n it is a launch of its own first.
 */
int w4_kv_weighted_sum_append(const float* p, const float* v_new, int64_t n, int64_t Hq,
                              int64_t Hkv, int64_t pos, int64_t T_max, uint8_t* v_codes,
                              float* v_scales, float* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* w4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
