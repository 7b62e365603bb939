// C-ABI entry points: host-side validation, error reporting and dispatch.
// Every check runs before anything is enqueued, so a failing call launches nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/w4a16.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return W4_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(W4_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int group_of(int scheme) { return scheme == W4_SYM4_G128 ? 128 : 64; }
int bits_of(int scheme) { return scheme == W4_AFF8_G64 ? 8 : 4; }
bool known(int scheme) {
    return scheme == W4_SYM4_G128 || scheme == W4_AFF4_G64 || scheme == W4_AFF8_G64;
}

// Checks a w4_matrix descriptor; `experts` = required num_experts (0 = any >= 1).
int check_matrix(const w4_matrix* W, const char* name, int experts) {
    if (!W) return fail(W4_EINVAL, "%s: null descriptor", name);
    if (!known(W->scheme)) return fail(W4_EINVAL, "%s: unknown scheme %d", name, (int)W->scheme);
    if (W->num_experts < 1 || (experts && W->num_experts != experts))
        return fail(W4_ESHAPE, "%s: num_experts %d", name, (int)W->num_experts);
    if (W->N < 0 || W->K <= 0) return fail(W4_ESHAPE, "%s: N=%lld K=%lld", name, (long long)W->N,
                                          (long long)W->K);
    if (W->K % group_of(W->scheme))
        return fail(W4_ESHAPE, "%s: K=%lld is not a multiple of the group size %d", name,
                    (long long)W->K, group_of(W->scheme));
    if (W->N > 0x7fffffffLL || W->K > 0x7fffffffLL)
        return fail(W4_ESHAPE, "%s: N and K must fit in 31 bits", name);
    if (W->N == 0) return W4_OK;  // an empty matrix needs no storage
    if (!W->codes || !W->scale) return fail(W4_EINVAL, "%s: null codes or scale", name);
    if (W->scheme != W4_SYM4_G128 && !W->bias)
        return fail(W4_EINVAL, "%s: affine scheme needs a bias array", name);
    if (!aligned16(W->codes) || !aligned16(W->scale) || (W->bias && !aligned16(W->bias)))
        return fail(W4_EALIGN, "%s: codes/scale/bias must be 16-byte aligned", name);
    return W4_OK;
}

}  // namespace

extern "C" {

const char* w4_last_error(void) { return g_err; }

int w4_packed_sizes(int scheme, int64_t N, int64_t K, size_t* codes_bytes, size_t* scale_bytes,
                    size_t* bias_bytes) {
    if (!known(scheme)) return fail(W4_EINVAL, "unknown scheme %d", scheme);
    if (N < 0 || K < 0 || K % group_of(scheme))
        return fail(W4_ESHAPE, "N=%lld K=%lld (K must be a multiple of %d)", (long long)N,
                    (long long)K, group_of(scheme));
    const size_t groups = (size_t)N * (size_t)(K / group_of(scheme));
    if (codes_bytes) *codes_bytes = (size_t)N * (size_t)K * bits_of(scheme) / 8;
    if (scale_bytes) *scale_bytes = groups * (scheme == W4_SYM4_G128 ? 4 : 2);
    if (bias_bytes) *bias_bytes = scheme == W4_SYM4_G128 ? 0 : groups * 2;
    return ok();
}

int w4_quantize_pack(int scheme, const float* W, int64_t N, int64_t K, void* codes, void* scale,
                     void* bias, void* stream) {
    if (!known(scheme)) return fail(W4_EINVAL, "unknown scheme %d", scheme);
    if (N < 0 || K <= 0 || K % group_of(scheme))
        return fail(W4_ESHAPE, "N=%lld K=%lld (K must be a positive multiple of %d)",
                    (long long)N, (long long)K, group_of(scheme));
    if (N == 0) return ok();
    if (!W || !codes || !scale || (scheme != W4_SYM4_G128 && !bias))
        return fail(W4_EINVAL, "null pointer argument");
    if (!aligned16(W) || !aligned16(codes) || !aligned16(scale) || (bias && !aligned16(bias)))
        return fail(W4_EALIGN, "device pointers must be 16-byte aligned");
    return hip_status(w4::launch_quantize_pack(scheme, W, N, K, codes, scale, bias,
                                               (hipStream_t)stream),
                      "quantize_pack launch");
}

int w4a16_gemv(const w4_matrix* W, const uint16_t* x, int64_t M, float* y, void* stream) {
    int rc = check_matrix(W, "W", 1);
    if (rc) return rc;
    if (M < 0 || M > 64) return fail(W4_ESHAPE, "M=%lld out of range [0, 64]", (long long)M);
    if (M == 0 || W->N == 0) return ok();
    if (W->K > w4::kMaxSkinnyK)
        return fail(W4_ESHAPE, "K=%lld exceeds the GEMV limit %lld", (long long)W->K,
                    (long long)w4::kMaxSkinnyK);
    if (!x || !y) return fail(W4_EINVAL, "null x or y");
    if (!aligned16(x) || !aligned16(y)) return fail(W4_EALIGN, "x and y must be 16-byte aligned");
    return hip_status(w4::launch_gemv(W->scheme, W->codes, W->scale, W->bias, W->N, W->K, x, M, y,
                                      (hipStream_t)stream),
                      "gemv launch");
}

size_t w4_gemv_workspace_bytes(const w4_matrix* W, int64_t M) {
    if (!W || W->num_experts != 1 || W->N <= 0 || W->K <= 0 || M < 2 || M > 16) return 0;
    const int64_t group = W->scheme == W4_SYM4_G128 ? 128 : 64;
    if (W->K % group || W->K > w4::kMaxSkinnyK) return 0;
    return w4::gemv_mfma_split_bytes(W->scheme, W->N, W->K, M);
}

int w4a16_gemv_ws(const w4_matrix* W, const uint16_t* x, int64_t M, float* y, void* workspace,
                  size_t workspace_bytes, void* stream) {
    int rc = check_matrix(W, "W", 1);
    if (rc) return rc;
    if (M < 0 || M > 64) return fail(W4_ESHAPE, "M=%lld out of range [0, 64]", (long long)M);
    if (M == 0 || W->N == 0) return ok();
    if (W->K > w4::kMaxSkinnyK)
        return fail(W4_ESHAPE, "K=%lld exceeds the GEMV limit %lld", (long long)W->K,
                    (long long)w4::kMaxSkinnyK);
    if (!x || !y) return fail(W4_EINVAL, "null x or y");
    if (!aligned16(x) || !aligned16(y)) return fail(W4_EALIGN, "x and y must be 16-byte aligned");
    const size_t need = w4_gemv_workspace_bytes(W, M);
    if (need == 0)
        return hip_status(w4::launch_gemv(W->scheme, W->codes, W->scale, W->bias, W->N, W->K, x, M,
                                          y, (hipStream_t)stream),
                          "gemv launch");
    if (!workspace || workspace_bytes < need)
        return fail(W4_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(W4_EALIGN, "workspace must be 16-byte aligned");
    const void* c = W->codes;
    const void* sc = W->scale;
    const void* b = W->bias;
    const int64_t N = W->N;
    return hip_status(w4::launch_gemv_mfma(W->scheme, 1, &c, &sc, &b, &N, W->K, x, M, &y,
                                           (hipStream_t)stream, (float*)workspace),
                      "gemv launch");  // need > 0: the K-part plan exists, so it launches
}

// Up to four non-empty matrices sharing x (same scheme and K), validated.
static hipError_t gemv_multi_dispatch(int scheme, int n, const void* const* c,
                                      const void* const* sc, const void* const* b,
                                      const int64_t* N, int64_t K, const uint16_t* x, int64_t M,
                                      float* const* y, hipStream_t st) {
    if (M == 1 && w4::gemv_wave_ok(scheme, K))
        return w4::launch_gemv_wave(scheme, n, c, sc, b, N, K, x, y, st);
    if (w4::gemv_mfma_ok(scheme, K, M)) {
        const hipError_t e = w4::launch_gemv_mfma(scheme, n, c, sc, b, N, K, x, M, y, st);
        if (e != hipErrorNotSupported) return e;
    }
    if (w4::gemv_wave_mt_ok(scheme, K, M))
        return w4::launch_gemv_wave_mt(scheme, n, c, sc, b, N, K, x, M, y, st);
    for (int i = 0; i < n; ++i) {
        const hipError_t e = w4::launch_gemv(scheme, c[i], sc[i], b[i], N[i], K, x, M, y[i], st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int w4a16_gemv_multi(const w4_matrix* const* Ws, int count, const uint16_t* x, int64_t M,
                     float* const* ys, void* stream) {
    if (!Ws || !ys) return fail(W4_EINVAL, "null Ws or ys");
    if (count < 1 || count > 4) return fail(W4_ESHAPE, "count=%d out of range [1, 4]", count);
    for (int i = 0; i < count; ++i) {
        char name[16];
        snprintf(name, sizeof(name), "Ws[%d]", i);
        int rc = check_matrix(Ws[i], name, 1);
        if (rc) return rc;
        if (Ws[i]->scheme != Ws[0]->scheme || Ws[i]->K != Ws[0]->K)
            return fail(W4_ESHAPE, "Ws[%d]: scheme and K must match Ws[0]", i);
        if (Ws[i]->N > 0 && (!ys[i] || !aligned16(ys[i])))
            return fail(ys[i] ? W4_EALIGN : W4_EINVAL, "ys[%d] null or misaligned", i);
    }
    if (M < 0 || M > 64) return fail(W4_ESHAPE, "M=%lld out of range [0, 64]", (long long)M);
    if (M == 0) return ok();
    const int64_t K = Ws[0]->K;
    if (K > w4::kMaxSkinnyK)
        return fail(W4_ESHAPE, "K=%lld exceeds the GEMV limit %lld", (long long)K,
                    (long long)w4::kMaxSkinnyK);
    if (!x) return fail(W4_EINVAL, "null x");
    if (!aligned16(x)) return fail(W4_EALIGN, "x must be 16-byte aligned");
    hipStream_t st = (hipStream_t)stream;
    // the non-empty members, for the kernels that serve several matrices per launch
    const void* c[4];
    const void* sc[4];
    const void* b[4];
    int64_t N[4];
    float* y[4];
    int n = 0;
    for (int i = 0; i < count; ++i) {
        if (Ws[i]->N == 0) continue;
        c[n] = Ws[i]->codes; sc[n] = Ws[i]->scale; b[n] = Ws[i]->bias; N[n] = Ws[i]->N;
        y[n] = ys[i];
        ++n;
    }
    if (n == 0) return ok();
    return hip_status(gemv_multi_dispatch(Ws[0]->scheme, n, c, sc, b, N, K, x, M, y, st),
                      "gemv_multi launch");
}

int w4a16_gemm(const w4_matrix* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream) {
    int rc = check_matrix(W, "W", 1);
    if (rc) return rc;
    if (W->scheme == W4_AFF8_G64) return fail(W4_EINVAL, "w4a16_gemm takes a 4-bit scheme");
    if (M < 0 || M > 0x7fffffffLL) return fail(W4_ESHAPE, "M=%lld out of range", (long long)M);
    if (M == 0 || W->N == 0) return ok();
    if (!X || !Y) return fail(W4_EINVAL, "null X or Y");
    if (!aligned16(X) || !aligned16(Y)) return fail(W4_EALIGN, "X and Y must be 16-byte aligned");
    return hip_status(w4::launch_gemm(W->scheme, W->codes, W->scale, W->bias, W->N, W->K, X, M, Y,
                                      (hipStream_t)stream),
                      "gemm launch");
}

int w4_moe_route(const w4_matrix* router, const uint16_t* x, int64_t M, int top_k, float* logits,
                 int32_t* ids, float* weights, void* stream) {
    int rc = check_matrix(router, "router", 1);
    if (rc) return rc;
    const int64_t E = router->N;
    if (E < 1 || E > 1024) return fail(W4_ESHAPE, "router: E=%lld out of range [1, 1024]", (long long)E);
    if (top_k < 1 || top_k > 32 || top_k > E)
        return fail(W4_ESHAPE, "top_k=%d out of range [1, min(E, 32)]", top_k);
    if (M < 0 || M > 4096) return fail(W4_ESHAPE, "M=%lld out of range [0, 4096]", (long long)M);
    if (M == 0) return ok();
    if (router->K > w4::kMaxSkinnyK)
        return fail(W4_ESHAPE, "router K=%lld exceeds %lld", (long long)router->K,
                    (long long)w4::kMaxSkinnyK);
    if (!x || !logits || !ids || !weights) return fail(W4_EINVAL, "null x, logits, ids or weights");
    if (!aligned16(x) || !aligned16(logits) || !aligned16(ids) || !aligned16(weights))
        return fail(W4_EALIGN, "x, logits, ids and weights must be 16-byte aligned");
    return hip_status(w4::launch_route(router->scheme, router->codes, router->scale, router->bias, E,
                                       router->K, x, M, top_k, logits, ids, weights,
                                       (hipStream_t)stream),
                      "moe_route launch");
}

size_t w4_moe_workspace_bytes(int64_t M, int top_k, int64_t E, int64_t D, int64_t F, int64_t Fs) {
    if (M < 0 || top_k < 0 || E < 0 || D < 0 || F < 0 || Fs < 0) return 0;
    return w4::moe_workspace_layout(M, top_k, E, D, F, Fs).total;
}

// Checks shared by the two MoE entry points; fills W and the scheme.
static int moe_check(const w4_matrix* gate, const w4_matrix* up, const w4_matrix* down,
                     const w4_matrix* shared_gate, const w4_matrix* shared_up,
                     const w4_matrix* shared_down, int64_t M, int top_k, w4::MoeMats& W,
                     int& scheme) {
    int rc;
    if ((rc = check_matrix(gate, "gate", 0)) || (rc = check_matrix(up, "up", 0)) ||
        (rc = check_matrix(down, "down", 0)))
        return rc;
    scheme = gate->scheme;
    if (scheme == W4_AFF8_G64) return fail(W4_EINVAL, "experts must use a 4-bit scheme");
    const int64_t E = gate->num_experts, F = gate->N, D = gate->K;
    if (up->scheme != scheme || down->scheme != scheme)
        return fail(W4_EINVAL, "gate, up and down must share one scheme");
    if (up->num_experts != E || down->num_experts != E)
        return fail(W4_ESHAPE, "gate, up and down must have the same number of experts");
    if (up->N != F || up->K != D || down->N != D || down->K != F)
        return fail(W4_ESHAPE, "expected gate/up [E][F][D] and down [E][D][F]");
    if (E > 1024) return fail(W4_ESHAPE, "E=%lld exceeds 1024", (long long)E);
    const bool any_shared = shared_gate || shared_up || shared_down;
    const bool all_shared = shared_gate && shared_up && shared_down;
    if (any_shared && !all_shared) return fail(W4_EINVAL, "pass all three shared matrices or none");
    int64_t Fs = 0;
    if (all_shared) {
        if ((rc = check_matrix(shared_gate, "shared_gate", 1)) ||
            (rc = check_matrix(shared_up, "shared_up", 1)) ||
            (rc = check_matrix(shared_down, "shared_down", 1)))
            return rc;
        Fs = shared_gate->N;
        if (shared_gate->scheme != scheme || shared_up->scheme != scheme ||
            shared_down->scheme != scheme)
            return fail(W4_EINVAL, "shared expert must use the experts' scheme");
        if (shared_gate->K != D || shared_up->K != D || shared_up->N != Fs ||
            shared_down->N != D || shared_down->K != Fs || Fs < 1)
            return fail(W4_ESHAPE, "expected shared gate/up [Fs][D] and down [D][Fs]");
    }
    if (top_k < 1 || top_k > 32) return fail(W4_ESHAPE, "top_k=%d out of range [1, 32]", top_k);
    if (M < 0 || M > 256) return fail(W4_ESHAPE, "M=%lld out of range [0, 256]", (long long)M);
    if (M > 0 && D > 0 && F < 1) return fail(W4_ESHAPE, "F must be positive");
    if (D > w4::kMaxSkinnyK / 4 || F > w4::kMaxSkinnyK / 4 || Fs > w4::kMaxSkinnyK / 4)
        return fail(W4_ESHAPE, "D, F and Fs must not exceed %lld", (long long)(w4::kMaxSkinnyK / 4));
    W = w4::MoeMats{};
    W.E = E; W.D = D; W.F = F; W.Fs = Fs;
    const w4_matrix* mats[6] = {gate, up, down, shared_gate, shared_up, shared_down};
    const void** dst[6] = {W.gate, W.up, W.down, W.sgate, W.sup, W.sdown};
    for (int i = 0; i < 6; ++i) {
        if (!mats[i]) continue;
        dst[i][0] = mats[i]->codes;
        dst[i][1] = mats[i]->scale;
        dst[i][2] = mats[i]->bias;
    }
    return W4_OK;
}

int w4a16_moe_gemv(const w4_matrix* gate, const w4_matrix* up, const w4_matrix* down,
                   const w4_matrix* shared_gate, const w4_matrix* shared_up,
                   const w4_matrix* shared_down, const uint16_t* x, int64_t M,
                   const int32_t* ids, const float* weights, int top_k, void* workspace,
                   size_t workspace_bytes, float* y, void* stream) {
    w4::MoeMats W;
    int scheme = 0;
    const int rc = moe_check(gate, up, down, shared_gate, shared_up, shared_down, M, top_k, W, scheme);
    if (rc) return rc;
    if (M == 0 || W.D == 0) return ok();
    if (!x || !ids || !weights || !y || !workspace)
        return fail(W4_EINVAL, "null x, ids, weights, y or workspace");
    if (!aligned16(x) || !aligned16(ids) || !aligned16(weights) || !aligned16(y) ||
        !aligned16(workspace))
        return fail(W4_EALIGN, "x, ids, weights, y and workspace must be 16-byte aligned");
    const size_t need = w4::moe_workspace_layout(M, top_k, W.E, W.D, W.F, W.Fs).total;
    if (workspace_bytes < need)
        return fail(W4_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    return hip_status(w4::launch_moe(scheme, W, x, M, ids, weights, top_k, workspace, y,
                                     (hipStream_t)stream),
                      "moe_gemv launch");
}

// Library-owned workspace of w4a16_moe_gemv_noalloc: one static device array
// per GPU. In host code `scratch` only names the symbol; its device address on
// the current GPU comes from hipGetSymbolAddress, taken once per device on the
// first call there and kept in moe_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[W4_MOE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int moe_scratch_ptr(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(W4_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(W4_EINVAL, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(W4_EHIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W4_OK;
}
}  // namespace

int w4a16_moe_gemv_noalloc(const w4_matrix* gate, const w4_matrix* up, const w4_matrix* down,
                           const w4_matrix* shared_gate, const w4_matrix* shared_up,
                           const w4_matrix* shared_down, const uint16_t* x, int64_t M,
                           const int32_t* ids, const float* weights, int top_k, float* y,
                           void* stream) {
    w4::MoeMats W;
    int scheme = 0;
    const int rc = moe_check(gate, up, down, shared_gate, shared_up, shared_down, M, top_k, W, scheme);
    if (rc) return rc;
    if (M == 0 || W.D == 0) return ok();
    if (!x || !ids || !weights || !y) return fail(W4_EINVAL, "null x, ids, weights or y");
    if (!aligned16(x) || !aligned16(ids) || !aligned16(weights) || !aligned16(y))
        return fail(W4_EALIGN, "x, ids, weights and y must be 16-byte aligned");
    const size_t need = w4::moe_workspace_layout(M, top_k, W.E, W.D, W.F, W.Fs).total;
    if (need > W4_MOE_SCRATCH_BYTES)
        return fail(W4_EWORKSPACE, "these sizes need %zu bytes of workspace; the static scratch holds %zu",
                    need, (size_t)W4_MOE_SCRATCH_BYTES);
    void* ws = nullptr;
    const int sr = moe_scratch_ptr(&ws);
    if (sr) return sr;
    return hip_status(w4::launch_moe(scheme, W, x, M, ids, weights, top_k, ws, y, (hipStream_t)stream),
                      "moe_gemv_noalloc launch");
}

int w4a16_moe_gemv_logits(const w4_matrix* gate, const w4_matrix* up, const w4_matrix* down,
                          const w4_matrix* shared_gate, const w4_matrix* shared_up,
                          const w4_matrix* shared_down, const uint16_t* x, int64_t M,
                          const float* logits, int top_k, int32_t* ids, float* weights,
                          void* workspace, size_t workspace_bytes, float* y, void* stream) {
    w4::MoeMats W;
    int scheme = 0;
    const int rc = moe_check(gate, up, down, shared_gate, shared_up, shared_down, M, top_k, W, scheme);
    if (rc) return rc;
    if (top_k > W.E) return fail(W4_ESHAPE, "top_k=%d exceeds E=%lld", top_k, (long long)W.E);
    if (M == 0 || W.D == 0) return ok();
    if (!x || !logits || !ids || !weights || !y || !workspace)
        return fail(W4_EINVAL, "null x, logits, ids, weights, y or workspace");
    if (!aligned16(x) || !aligned16(logits) || !aligned16(ids) || !aligned16(weights) ||
        !aligned16(y) || !aligned16(workspace))
        return fail(W4_EALIGN, "x, logits, ids, weights, y and workspace must be 16-byte aligned");
    const size_t need = w4::moe_workspace_layout(M, top_k, W.E, W.D, W.F, W.Fs).total;
    if (workspace_bytes < need)
        return fail(W4_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    return hip_status(w4::launch_moe_logits(scheme, W, x, M, logits, top_k, ids, weights,
                                            workspace, y, (hipStream_t)stream),
                      "moe_gemv_logits launch");
}

// ---------------------------------------------------------------- MoE layer
static std::atomic<long long> g_layer_polls{0};
static std::atomic<int> g_layer_withhold{0};
static std::atomic<int> g_layer_single{0};

void w4_moe_layer_set_single_launch(int enable) { g_layer_single.store(enable != 0); }
constexpr long long kLayerDefaultPolls = 1LL << 21;  // each a device-scope load + 128 cycles of sleep: seconds

void w4_moe_layer_set_wait(int64_t max_polls, int withhold) {
    g_layer_polls.store(max_polls > 0 ? (long long)max_polls : 0);
    g_layer_withhold.store(withhold != 0);
}

size_t w4_moe_layer_workspace_bytes(int64_t M, int top_k, int64_t E, int64_t D, int64_t F,
                                    int64_t Fs) {
    if (M < 0 || top_k < 1 || top_k > 32 || E < 1 || D < 0 || F < 0 || Fs < 0) return 0;
    return w4::moe_layer_workspace_layout(M, top_k, E, D, F, Fs).total;
}

int w4a16_moe_layer(const w4_matrix* router, const w4_matrix* gate, const w4_matrix* up,
                    const w4_matrix* down, const w4_matrix* shared_gate,
                    const w4_matrix* shared_up, const w4_matrix* shared_down,
                    const uint16_t* x, int64_t M, int top_k, int32_t* ids, float* weights,
                    float* y, void* workspace, size_t workspace_bytes, void* stream) {
    w4::MoeMats W;
    int scheme = 0;
    int rc = moe_check(gate, up, down, shared_gate, shared_up, shared_down, M, top_k, W, scheme);
    if (rc) return rc;
    if ((rc = check_matrix(router, "router", 1))) return rc;
    if (router->N != W.E || router->K != W.D)
        return fail(W4_ESHAPE, "router must be [E][D] = [%lld][%lld]", (long long)W.E, (long long)W.D);
    if (W.E > 1024 || top_k > W.E) return fail(W4_ESHAPE, "top_k=%d, E=%lld", top_k, (long long)W.E);
    if (M == 0 || W.D == 0) return ok();
    if (W.D > w4::kMaxSkinnyK) return fail(W4_ESHAPE, "D=%lld exceeds %lld", (long long)W.D, (long long)w4::kMaxSkinnyK);
    if (!x || !ids || !weights || !y || !workspace)
        return fail(W4_EINVAL, "null x, ids, weights, y or workspace");
    if (!aligned16(x) || !aligned16(ids) || !aligned16(weights) || !aligned16(y) || !aligned16(workspace))
        return fail(W4_EALIGN, "x, ids, weights, y and workspace must be 16-byte aligned");
    const w4::MoeLayerWorkspace L = w4::moe_layer_workspace_layout(M, top_k, W.E, W.D, W.F, W.Fs);
    if (workspace_bytes < L.total)
        return fail(W4_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
    hipStream_t st = (hipStream_t)stream;
    const void* R[3] = {router->codes, router->scale, router->bias};
    if (M == 1 && g_layer_single.load() && w4::moe_layer_ok(router->scheme, top_k, W.E, W.D, W.F, W.Fs)) {
        const long long polls = g_layer_polls.load();
        const hipError_t e = w4::launch_moe_layer(scheme, router->scheme, W, R, x, top_k, ids, weights,
                                                  workspace, y, polls > 0 ? polls : kLayerDefaultPolls,
                                                  g_layer_withhold.load(), st);
        if (e != hipErrorNotSupported) return hip_status(e, "moe_layer launch");
        // refused before launching anything: the launch sequence below
    }
    float* logits = (float*)((uint8_t*)workspace + L.multi);
    void* ws = (uint8_t*)workspace + L.multi + (((size_t)M * W.E * 4 + 255) & ~(size_t)255);
    hipError_t e;
    if (M == 1) {
        // router GEMV, then the top-k inside the gate/up pass and the down pass
        e = w4::launch_gemv(router->scheme, router->codes, router->scale, router->bias, W.E, W.D, x,
                            1, logits, st);
        if (e != hipSuccess) return hip_status(e, "moe_layer router launch");
        return hip_status(w4::launch_moe_logits(scheme, W, x, 1, logits, top_k, ids, weights, ws, y, st),
                          "moe_layer expert launches");
    }
    e = w4::launch_route(router->scheme, router->codes, router->scale, router->bias, W.E, W.D, x, M,
                         top_k, logits, ids, weights, st);
    if (e != hipSuccess) return hip_status(e, "moe_layer route launch");
    return hip_status(w4::launch_moe(scheme, W, x, M, ids, weights, top_k, ws, y, st),
                      "moe_layer expert launches");
}

int w4_moe_layer_status(const void* workspace, int32_t* status, void* stream) {
    if (!workspace || !status) return fail(W4_EINVAL, "null workspace or status");
    if (!aligned16(workspace)) return fail(W4_EALIGN, "workspace must be 16-byte aligned");
    uint32_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, (const uint8_t*)workspace + 4 * (size_t)w4::kSyncStatus, 4,
                                  hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "moe_layer status");
    *status = (int32_t)v;
    return ok();
}

// ---------------------------------------------------------------- dense gated FFN
static std::atomic<long long> g_ffn_polls{0};
static std::atomic<bool> g_ffn_withhold{false};
static std::atomic<int> g_ffn_path{W4_FFN_PATH_DEFAULT};
constexpr long long kFfnDefaultPolls = 1LL << 21;

void w4_ffn_set_wait(int64_t max_polls, int withhold) {
    g_ffn_polls.store(max_polls > 0 ? (long long)max_polls : 0);
    g_ffn_withhold.store(withhold != 0);
}

int w4_ffn_set_path(int path) {
    if (path != W4_FFN_PATH_DEFAULT && path != W4_FFN_PATH_SINGLE_LAUNCH && path != W4_FFN_PATH_SEQUENCE)
        return fail(W4_EINVAL, "unknown FFN path %d", path);
    g_ffn_path.store(path);
    return ok();
}

size_t w4_ffn_workspace_bytes(const w4_matrix* down, int64_t M) {
    if (!down || down->num_experts != 1 || down->N <= 0 || down->K <= 0 || M < 1 || M > 64 ||
        !known(down->scheme))
        return 0;
    return w4::ffn_workspace_layout(down->scheme, M, down->N, down->K).total;
}

// The gate/up half of the FFN into hh (bf16 [M][F]); g, u: fp32 [M][F] each
// (workspace) for the sequence.
static hipError_t ffn_gate_up_launches(const w4_matrix* gate, const w4_matrix* up, const uint16_t* x,
                                       int64_t M, uint16_t* hh, float* g, float* u, int path,
                                       hipStream_t st) {
    const int scheme = gate->scheme;
    const int64_t D = gate->K, F = gate->N;
    const void* G[3] = {gate->codes, gate->scale, gate->bias};
    const void* U[3] = {up->codes, up->scale, up->bias};
    if (path != W4_FFN_PATH_SEQUENCE) {
        // gate/up rows with the activation in their epilogue
        const hipError_t e = M == 1 ? w4::launch_ffn_gate_up(scheme, G, U, D, F, x, hh, st)
                                    : w4::launch_gemv_mfma_gated(scheme, G, U, F, D, x, M, hh, st);
        if (e != hipErrorNotSupported) return e;
    }
    // gate and up in one GEMV launch, then the activation
    const void* c2[2] = {gate->codes, up->codes};
    const void* s2[2] = {gate->scale, up->scale};
    const void* b2[2] = {gate->bias, up->bias};
    const int64_t N2[2] = {F, F};
    float* y2[2] = {g, u};
    hipError_t e = gemv_multi_dispatch(scheme, 2, c2, s2, b2, N2, D, x, M, y2, st);
    if (e == hipSuccess) e = w4::launch_ffn_act(g, u, hh, M * F, st);
    return e;
}

static int ffn_check_gate_up(const w4_matrix* gate, const w4_matrix* up, int64_t M) {
    int rc;
    if ((rc = check_matrix(gate, "gate", 1)) || (rc = check_matrix(up, "up", 1))) return rc;
    if (gate->scheme != up->scheme) return fail(W4_ESHAPE, "gate and up must share one scheme");
    if (up->N != gate->N || up->K != gate->K)
        return fail(W4_ESHAPE, "gate and up must both be [F][D]");
    if (M < 0 || M > 64) return fail(W4_ESHAPE, "M=%lld out of range [0, 64]", (long long)M);
    if (gate->K > w4::kMaxSkinnyK || gate->N > w4::kMaxSkinnyK)
        return fail(W4_ESHAPE, "D=%lld and F=%lld must not exceed %lld", (long long)gate->K,
                    (long long)gate->N, (long long)w4::kMaxSkinnyK);
    return W4_OK;
}

size_t w4_ffn_gate_up_workspace_bytes(const w4_matrix* gate, int64_t M) {
    if (!gate || gate->num_experts != 1 || gate->N <= 0 || gate->K <= 0 || M < 1 || M > 64 ||
        !known(gate->scheme))
        return 0;
    return 2 * (((size_t)M * gate->N * 4 + 255) & ~(size_t)255);
}

int w4a16_ffn_gate_up(const w4_matrix* gate, const w4_matrix* up, const uint16_t* x, int64_t M,
                      uint16_t* h, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = ffn_check_gate_up(gate, up, M);
    if (rc) return rc;
    if (M == 0) return ok();
    if (!x || !h || !workspace) return fail(W4_EINVAL, "null x, h or workspace");
    if (!aligned16(x) || !aligned16(h) || !aligned16(workspace))
        return fail(W4_EALIGN, "x, h and workspace must be 16-byte aligned");
    const size_t need = w4_ffn_gate_up_workspace_bytes(gate, M);
    if (workspace_bytes < need)
        return fail(W4_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    float* g = (float*)workspace;
    float* u = (float*)((uint8_t*)workspace + need / 2);
    return hip_status(ffn_gate_up_launches(gate, up, x, M, h, g, u, g_ffn_path.load(), (hipStream_t)stream),
                      "ffn gate/up launch");
}

int w4a16_ffn(const w4_matrix* gate, const w4_matrix* up, const w4_matrix* down, const uint16_t* x,
              int64_t M, uint16_t* h, float* y, void* workspace, size_t workspace_bytes,
              void* stream) {
    int rc = ffn_check_gate_up(gate, up, M);
    if (rc || (rc = check_matrix(down, "down", 1))) return rc;
    if (gate->scheme != down->scheme) return fail(W4_ESHAPE, "gate, up and down must share one scheme");
    const int64_t D = gate->K, F = gate->N;
    if (down->N != D || down->K != F)
        return fail(W4_ESHAPE, "down must be [D][F] = [%lld][%lld]", (long long)D, (long long)F);
    if (M == 0) return ok();
    if (!x || !y || !workspace) return fail(W4_EINVAL, "null x, y or workspace");
    if (!aligned16(x) || !aligned16(y) || !aligned16(workspace) || (h && !aligned16(h)))
        return fail(W4_EALIGN, "x, y, h and workspace must be 16-byte aligned");
    const w4::FfnWorkspace L = w4::ffn_workspace_layout(gate->scheme, M, D, F);
    if (workspace_bytes < L.total)
        return fail(W4_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
    hipStream_t st = (hipStream_t)stream;
    uint8_t* base = (uint8_t*)workspace;
    const int scheme = gate->scheme;
    const void* G[3] = {gate->codes, gate->scale, gate->bias};
    const void* U[3] = {up->codes, up->scale, up->bias};
    const void* Dn[3] = {down->codes, down->scale, down->bias};
    const int path = g_ffn_path.load();
    uint16_t* hh = h ? h : (uint16_t*)(base + L.h);
    if (M == 1 && path == W4_FFN_PATH_SINGLE_LAUNCH) {
        const long long polls = g_ffn_polls.load();
        const hipError_t e = w4::launch_ffn_fused(scheme, G, U, Dn, D, F, x, h, y, workspace,
                                                  polls > 0 ? polls : kFfnDefaultPolls,
                                                  g_ffn_withhold.load(), st);
        if (e != hipErrorNotSupported) return hip_status(e, "ffn launch");
        // refused before launching anything: the launches below
    }
    hipError_t e = ffn_gate_up_launches(gate, up, x, M, hh, (float*)(base + L.g),
                                        (float*)(base + L.u), path, st);
    if (e != hipSuccess) return hip_status(e, "ffn gate/up launches");
    if (M >= 2 && M <= 16 && w4::gemv_mfma_split_bytes(scheme, D, F, M) > 0)
        e = w4::launch_gemv_mfma(scheme, 1, &Dn[0], &Dn[1], &Dn[2], &D, F, hh, M, &y, st,
                                 (float*)(base + L.part));
    else
        e = w4::launch_gemv(scheme, down->codes, down->scale, down->bias, D, F, hh, M, y, st);
    return hip_status(e, "ffn down launch");
}

int w4_ffn_status(const void* workspace, int32_t* status, void* stream) {
    return w4_moe_layer_status(workspace, status, stream);  // the same word of the same layout
}

// ---------------------------------------------------------------- INT4 KV cache
static int kv_check_cache(int64_t Hq, int64_t Hkv, int64_t T, int64_t T_max, const void* codes,
                          const void* scales) {
    if (Hq < 1 || Hkv < 1 || Hq % Hkv)
        return fail(W4_ESHAPE, "Hq=%lld must be a positive multiple of Hkv=%lld", (long long)Hq,
                    (long long)Hkv);
    if (T < 0 || T > T_max || T_max > 0x7fffffffLL || Hq * w4::kv_chunks(T_max) > 0x7fffffffLL)
        return fail(W4_ESHAPE, "T=%lld, T_max=%lld out of range", (long long)T, (long long)T_max);
    if (!codes || !scales) return fail(W4_EINVAL, "null codes or scales");
    if (!aligned16(codes) || !aligned16(scales)) return fail(W4_EALIGN, "codes and scales must be 16-byte aligned");
    return W4_OK;
}

static int kv_check_append(int64_t n, int64_t Hkv, int64_t pos, int64_t T_max) {
    if (n < 0 || Hkv < 1 || pos < 0 || T_max < 1 || pos + n > T_max || T_max > 0x7fffffffLL ||
        2 * n * Hkv > 0x7fffffffLL)
        return fail(W4_ESHAPE, "n=%lld Hkv=%lld pos=%lld T_max=%lld out of range", (long long)n,
                    (long long)Hkv, (long long)pos, (long long)T_max);
    return W4_OK;
}

int w4_kv_quantize(const float* x, int64_t n, int64_t Hkv, int64_t pos, int64_t T_max,
                   uint8_t* codes, float* scales, void* stream) {
    int rc = kv_check_append(n, Hkv, pos, T_max);
    if (rc) return rc;
    if (n == 0) return ok();
    if (!x || !codes || !scales) return fail(W4_EINVAL, "null x, codes or scales");
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
        return fail(W4_EALIGN, "x, codes and scales must be 16-byte aligned");
    return hip_status(w4::launch_kv_quantize(&x, 1, n, Hkv, pos, T_max, &codes, &scales,
                                             (hipStream_t)stream),
                      "kv_quantize launch");
}

int w4_kv_append(const float* k, const float* v, int64_t n, int64_t Hkv, int64_t pos,
                 int64_t T_max, uint8_t* k_codes, float* k_scales, uint8_t* v_codes,
                 float* v_scales, void* stream) {
    int rc = kv_check_append(n, Hkv, pos, T_max);
    if (rc) return rc;
    if (n == 0) return ok();
    if (!k || !v || !k_codes || !k_scales || !v_codes || !v_scales)
        return fail(W4_EINVAL, "null k, v, codes or scales");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_codes) || !aligned16(k_scales) ||
        !aligned16(v_codes) || !aligned16(v_scales))
        return fail(W4_EALIGN, "k, v, codes and scales must be 16-byte aligned");
    const float* x[2] = {k, v};
    uint8_t* c[2] = {k_codes, v_codes};
    float* s[2] = {k_scales, v_scales};
    return hip_status(w4::launch_kv_quantize(x, 2, n, Hkv, pos, T_max, c, s, (hipStream_t)stream),
                      "kv_append launch");
}

int w4_kv_scores(const float* q, int64_t Hq, int64_t Hkv, int64_t T, int64_t T_max,
                 const uint8_t* codes, const float* scales, float* scores, void* stream) {
    int rc = kv_check_cache(Hq, Hkv, T, T_max, codes, scales);
    if (rc) return rc;
    if (T == 0) return ok();
    if (!q || !scores) return fail(W4_EINVAL, "null q or scores");
    if (!aligned16(q) || !aligned16(scores)) return fail(W4_EALIGN, "q and scores must be 16-byte aligned");
    return hip_status(w4::launch_kv_scores(q, Hq, Hkv, T, T_max, codes, scales, scores, nullptr, 0,
                                           (hipStream_t)stream),
                      "kv_scores launch");
}

int w4_kv_scores_append(const float* q, const float* k_new, int64_t n, int64_t Hq, int64_t Hkv,
                        int64_t pos, int64_t T_max, uint8_t* k_codes, float* k_scales,
                        float* scores, void* stream) {
    int rc = kv_check_append(n, Hkv, pos, T_max);
    if (rc) return rc;
    if (n < 1) return fail(W4_ESHAPE, "n=%lld: at least one new position", (long long)n);
    const int64_t T = pos + n;
    rc = kv_check_cache(Hq, Hkv, T, T_max, k_codes, k_scales);
    if (rc) return rc;
    if (!q || !k_new || !scores) return fail(W4_EINVAL, "null q, k_new or scores");
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(scores))
        return fail(W4_EALIGN, "q, k_new and scores must be 16-byte aligned");
    const hipStream_t st = (hipStream_t)stream;
    if (n <= w4::kKvFuseMax)
        return hip_status(w4::launch_kv_scores(q, Hq, Hkv, T, T_max, k_codes, k_scales, scores, k_new,
                                               pos, st),
                          "kv_scores_append launch");
    hipError_t e = w4::launch_kv_quantize(&k_new, 1, n, Hkv, pos, T_max, &k_codes, &k_scales, st);
    if (e == hipSuccess)
        e = w4::launch_kv_scores(q, Hq, Hkv, T, T_max, k_codes, k_scales, scores, nullptr, 0, st);
    return hip_status(e, "kv_scores_append launches");
}

size_t w4_kv_weighted_sum_workspace_bytes(int64_t Hq, int64_t T) {
    if (Hq < 1 || T < 1 || T > 0x7fffffffLL) return 0;
    return (size_t)Hq * (size_t)w4::kv_chunks(T) * w4::kKvHeadDim * sizeof(float);
}

int w4_kv_weighted_sum(const float* p, int64_t Hq, int64_t Hkv, int64_t T, int64_t T_max,
                       const uint8_t* codes, const float* scales, float* out, void* workspace,
                       size_t workspace_bytes, void* stream) {
    int rc = kv_check_cache(Hq, Hkv, T, T_max, codes, scales);
    if (rc) return rc;
    if (T < 1) return fail(W4_ESHAPE, "T=%lld: the weighted sum needs at least one position", (long long)T);
    if (!p || !out) return fail(W4_EINVAL, "null p or out");
    if (!aligned16(p) || !aligned16(out)) return fail(W4_EALIGN, "p and out must be 16-byte aligned");
    const size_t need = w4_kv_weighted_sum_workspace_bytes(Hq, T);
    if (!workspace || workspace_bytes < need)
        return fail(W4_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(W4_EALIGN, "workspace must be 16-byte aligned");
    return hip_status(w4::launch_kv_weighted_sum(p, Hq, Hkv, T, T_max, codes, scales, out,
                                                 (float*)workspace, nullptr, 0, (hipStream_t)stream),
                      "kv_weighted_sum launch");
}

int w4_kv_weighted_sum_append(const float* p, const float* v_new, int64_t n, int64_t Hq,
                              int64_t Hkv, int64_t pos, int64_t T_max, uint8_t* v_codes,
                              float* v_scales, float* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
    int rc = kv_check_append(n, Hkv, pos, T_max);
    if (rc) return rc;
    if (n < 1) return fail(W4_ESHAPE, "n=%lld: at least one new position", (long long)n);
    const int64_t T = pos + n;
    rc = kv_check_cache(Hq, Hkv, T, T_max, v_codes, v_scales);
    if (rc) return rc;
    if (!p || !v_new || !out) return fail(W4_EINVAL, "null p, v_new or out");
    if (!aligned16(p) || !aligned16(v_new) || !aligned16(out))
        return fail(W4_EALIGN, "p, v_new and out must be 16-byte aligned");
    const size_t need = w4_kv_weighted_sum_workspace_bytes(Hq, T);
    if (!workspace || workspace_bytes < need)
        return fail(W4_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(W4_EALIGN, "workspace must be 16-byte aligned");
    const hipStream_t st = (hipStream_t)stream;
    if (n <= w4::kKvFuseMax)
        return hip_status(w4::launch_kv_weighted_sum(p, Hq, Hkv, T, T_max, v_codes, v_scales, out,
                                                     (float*)workspace, v_new, pos, st),
                          "kv_weighted_sum_append launch");
    hipError_t e = w4::launch_kv_quantize(&v_new, 1, n, Hkv, pos, T_max, &v_codes, &v_scales, st);
    if (e == hipSuccess)
        e = w4::launch_kv_weighted_sum(p, Hq, Hkv, T, T_max, v_codes, v_scales, out,
                                       (float*)workspace, nullptr, 0, st);
    return hip_status(e, "kv_weighted_sum_append launches");
}

}  // extern "C"
