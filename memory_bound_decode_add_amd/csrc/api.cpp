// The C ABI of libfdec: argument validation, workspace sizing, launch sequencing and
// graph capture.  Every check runs before the first HIP call, so a rejected call
// enqueues nothing.  Kernels live in the .hip files; see fdec.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "fdec_internal.h"

using namespace fdec;

namespace {

thread_local std::string t_last_error;

// Test and tuning controls (include/fdec_test.h): read once per call.
std::atomic<int> g_fail_launches{0};
std::atomic<int> g_forced_split{0};
std::atomic<int> g_col_waves{0};
std::atomic<int> g_col_cols{0};
std::atomic<int> g_mfma_kernel{0};
std::atomic<int> g_mfma_tiles{0};
std::atomic<int> g_mfma_gw{0};
std::atomic<int> g_mfma_waves{0};

constexpr size_t kAlign = 256;   // sub-buffer alignment inside workspaces

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    t_last_error = std::string(fdec_status_str(status)) + ": " + buf;
    return status;
}

int ok() {
    t_last_error.clear();
    return FDEC_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(FDEC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct Span {
    const void* p;
    size_t bytes;
};
bool overlap(Span a, Span b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// ---- shared checks ----
int check_w4(const fdec_w4* W, const char* name) {
    if (!W) return fail(FDEC_ERR_NULL, "%s is NULL", name);
    if (!W->qweight || !W->scales) return fail(FDEC_ERR_NULL, "%s.qweight or %s.scales is NULL", name, name);
    if (W->K <= 0 || W->K % 128) return fail(FDEC_ERR_SHAPE, "%s.K = %d must be a positive multiple of 128", name, W->K);
    if (W->N <= 0 || W->N % 8) return fail(FDEC_ERR_SHAPE, "%s.N = %d must be a positive multiple of 8", name, W->N);
    if (!aligned16(W->qweight) || !aligned16(W->scales))
        return fail(FDEC_ERR_ALIGN, "%s arrays must be 16-byte aligned", name);
    return FDEC_OK;
}
Span w4_qspan(const fdec_w4* W) { return {W->qweight, size_t(W->K) / 8 * W->N * 4}; }
Span w4_sspan(const fdec_w4* W) { return {W->scales, size_t(W->K) / 128 * W->N * 2}; }

int check_m(int M, int max_m = 16) {
    if (M < 1 || M > max_m) return fail(FDEC_ERR_SHAPE, "M = %d must be in [1, %d]", M, max_m);
    return FDEC_OK;
}

// The W4 GEMV entry points take up to kMaxGemvRows rows: past 16 the matrix-core kernel
// stages 32 or 64 rows and feeds each weight load to two or four 16-row MFMA blocks.
constexpr int kMaxGemvRows = kMfmaMaxRows;

bool w4_gemv_shape_ok(int M, int K, int N) {
    return M >= 1 && M <= kMaxGemvRows && K > 0 && K % 128 == 0 && N > 0 && N % 8 == 0;
}

int check_norm(const fdec_bf16* x, const fdec_bf16* residual, const fdec_bf16* weight, float eps,
               int M, int H, const fdec_bf16* h_out, const fdec_bf16* y_out) {
    if (M < 0) return fail(FDEC_ERR_SHAPE, "M = %d must be >= 0", M);
    if (H < 8 || H > 16384 || H % 8) return fail(FDEC_ERR_SHAPE, "H = %d must be a multiple of 8 in [8, 16384]", H);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(FDEC_ERR_ARG, "eps must be finite and >= 0");
    if (!weight) return fail(FDEC_ERR_NULL, "add_rmsnorm: weight is required");
    if (M == 0) return FDEC_OK;   // empty batch: the [0, H] tensors may be NULL
    if (!x || !residual || !h_out || !y_out)
        return fail(FDEC_ERR_NULL, "add_rmsnorm: x, residual, h_out and y_out are required");
    if (!aligned16(x) || !aligned16(residual) || !aligned16(weight) || !aligned16(h_out) || !aligned16(y_out))
        return fail(FDEC_ERR_ALIGN, "add_rmsnorm: every tensor must be 16-byte aligned");
    const size_t t = size_t(M) * H * 2;
    const Span X{x, t}, R{residual, t}, W{weight, size_t(H) * 2}, Hs{h_out, t}, Y{y_out, t};
    if (overlap(Y, X) || overlap(Y, R) || overlap(Y, W) || overlap(Y, Hs))
        return fail(FDEC_ERR_ALIAS, "y_out overlaps another tensor");
    if (overlap(Hs, X) || overlap(Hs, W) || (overlap(Hs, R) && h_out != residual))
        return fail(FDEC_ERR_ALIAS, "h_out may only alias residual exactly");
    return FDEC_OK;
}

int check_gemv(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, const fdec_w4* W,
               const float* out_scale, const fdec_bf16* residual, int M, const fdec_bf16* y,
               void* ws, size_t ws_bytes, bool swiglu, size_t need_ws, int max_m = 16) {
    int st;
    if ((st = check_w4(W, "W")) != FDEC_OK) return st;
    if ((st = check_m(M, max_m)) != FDEC_OK) return st;
    if (!g || (swiglu && !u) || !y) return fail(FDEC_ERR_NULL, "activation input and y are required");
    if (ldgu < W->K || ldgu % 8) return fail(FDEC_ERR_SHAPE, "ld = %lld must be >= K and a multiple of 8", (long long)ldgu);
    if (!aligned16(g) || (u && !aligned16(u)) || !aligned16(y) || (residual && !aligned16(residual)))
        return fail(FDEC_ERR_ALIGN, "activation, residual and y must be 16-byte aligned");
    if (out_scale && !aligned4(out_scale)) return fail(FDEC_ERR_ALIGN, "out_scale must be 4-byte aligned");
    if (ws_bytes < need_ws) return fail(FDEC_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu required", ws_bytes, need_ws);
    if (need_ws > 0 && !ws) return fail(FDEC_ERR_NULL, "workspace is NULL");
    if (ws && !aligned16(ws)) return fail(FDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t in_bytes = (size_t(M - 1) * ldgu + W->K) * 2;
    const Span Y{y, size_t(M) * W->N * 2};
    const Span ins[] = {{g, in_bytes}, {u, in_bytes}, w4_qspan(W), w4_sspan(W), {out_scale, 4}, {ws, ws_bytes}};
    for (const Span& s : ins)
        if (overlap(Y, s)) return fail(FDEC_ERR_ALIAS, "y overlaps an input or the workspace");
    if (residual && overlap(Y, Span{residual, Y.bytes}) && residual != y)
        return fail(FDEC_ERR_ALIAS, "y may only alias residual exactly");
    const Span WS{ws, need_ws};
    const Span others[] = {{g, in_bytes}, {u, in_bytes}, w4_qspan(W), w4_sspan(W), {out_scale, 4}, {residual, Y.bytes}};
    for (const Span& s : others)
        if (overlap(WS, s)) return fail(FDEC_ERR_ALIAS, "the workspace overlaps an input");
    return FDEC_OK;
}

int injected() { return fail(FDEC_ERR_HIP, "launch failure injected by fdec_test_fail_launches"); }

// ---- FP4 weights ----
int check_fp4(const fdec_fp4* W) {
    if (!W) return fail(FDEC_ERR_NULL, "W is NULL");
    if (!W->qweight || !W->scales) return fail(FDEC_ERR_NULL, "W.qweight or W.scales is NULL");
    if (W->K <= 0 || W->K % 32) return fail(FDEC_ERR_SHAPE, "W.K = %d must be a positive multiple of 32", W->K);
    if (W->N <= 0 || W->N % 8) return fail(FDEC_ERR_SHAPE, "W.N = %d must be a positive multiple of 8", W->N);
    if (!aligned16(W->qweight) || !aligned16(W->scales)) return fail(FDEC_ERR_ALIGN, "W arrays must be 16-byte aligned");
    return FDEC_OK;
}
Span fp4_qspan(const fdec_fp4* W) { return {W->qweight, size_t(W->K) / 8 * W->N * 4}; }
Span fp4_sspan(const fdec_fp4* W) { return {W->scales, size_t(W->K) / 16 * W->N}; }

int check_fp4_gemv(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, const fdec_fp4* W, const float* out_scale,
                   const fdec_bf16* residual, int M, const fdec_bf16* y, void* ws, size_t ws_bytes, bool swiglu) {
    int st;
    if ((st = check_fp4(W)) != FDEC_OK) return st;
    if ((st = check_m(M, kMaxGemvRows)) != FDEC_OK) return st;
    if (!g || (swiglu && !u) || !y) return fail(FDEC_ERR_NULL, "activation input and y are required");
    if (ldgu < W->K || ldgu % 8) return fail(FDEC_ERR_SHAPE, "ld = %lld must be >= K and a multiple of 8", (long long)ldgu);
    if (!aligned16(g) || (u && !aligned16(u)) || !aligned16(y) || (residual && !aligned16(residual)))
        return fail(FDEC_ERR_ALIGN, "activation, residual and y must be 16-byte aligned");
    if (out_scale && !aligned4(out_scale)) return fail(FDEC_ERR_ALIGN, "out_scale must be 4-byte aligned");
    const size_t in_bytes = (size_t(M - 1) * ldgu + W->K) * 2;
    const Span Y{y, size_t(M) * W->N * 2};
    const Span ins[] = {{g, in_bytes}, {u, in_bytes}, fp4_qspan(W), fp4_sspan(W), {out_scale, 4}};
    for (const Span& sp : ins)
        if (overlap(Y, sp)) return fail(FDEC_ERR_ALIAS, "y overlaps an input");
    if (residual && overlap(Y, Span{residual, Y.bytes}) && residual != y)
        return fail(FDEC_ERR_ALIAS, "y may only alias residual exactly");
    if (!fp4_gemv_supported(M, W->K, W->N))
        return fail(FDEC_ERR_UNSUPPORTED,
                    "the FP4 GEMV takes M <= 4 with K <= 16384, or 3 <= M <= 64 with K %% 128 == 0 (M = %d, K = %d)", M,
                    W->K);
    const size_t need = fp4_gemv_workspace_bytes(M, W->K, W->N);
    if (ws_bytes < need) return fail(FDEC_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu required", ws_bytes, need);
    if (need > 0 && !ws) return fail(FDEC_ERR_NULL, "workspace is NULL");
    if (ws && !aligned16(ws)) return fail(FDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    const Span WS{ws, need};
    const Span others[] = {{g, in_bytes}, {u, in_bytes}, fp4_qspan(W), fp4_sspan(W), {out_scale, 4}, {residual, Y.bytes},
                           Y};
    for (const Span& sp : others)
        if (overlap(WS, sp)) return fail(FDEC_ERR_ALIAS, "the workspace overlaps an input or y");
    return FDEC_OK;
}

// ---- the layer ----
struct LayerDims {
    int H, I;
};

int check_layer(const fdec_mlp_layer* L, int M, LayerDims* d) {
    if (!L) return fail(FDEC_ERR_NULL, "layer is NULL");
    int st;
    if ((st = check_m(M)) != FDEC_OK) return st;
    if ((st = check_w4(&L->gate_up, "gate_up")) != FDEC_OK) return st;
    if ((st = check_w4(&L->down, "down")) != FDEC_OK) return st;
    if (!L->norm_weight) return fail(FDEC_ERR_NULL, "norm_weight is NULL");
    if (!aligned16(L->norm_weight)) return fail(FDEC_ERR_ALIGN, "norm_weight must be 16-byte aligned");
    if (L->out_scale && !aligned4(L->out_scale)) return fail(FDEC_ERR_ALIGN, "out_scale must be 4-byte aligned");
    const int H = L->gate_up.K, I = L->down.K;
    if (L->gate_up.N != 2 * I || L->down.N != H)
        return fail(FDEC_ERR_SHAPE, "gate_up must be [H, 2I] and down [I, H] (H = %d, I = %d)", H, I);
    if (H > 16384) return fail(FDEC_ERR_SHAPE, "H = %d exceeds 16384", H);
    if (!(L->eps >= 0.f) || !std::isfinite(L->eps)) return fail(FDEC_ERR_ARG, "eps must be finite and >= 0");
    d->H = H;
    d->I = I;
    return FDEC_OK;
}

// The two GEMV plans of a layer, made once per call: the workspace is checked against
// them and they are what gets launched.
// y as the matrix-core GEMVs stage it (written by the norm kernel, copied by a row-block
// gate_up): fp16 [M][H] and the [M][H/128] powers of two.
size_t staged_bytes(int M, int H) { return align_up(size_t(M) * H * 2) + align_up(size_t(M) * (H / 128) * 4); }

// Workspace of the three-kernel layer: y staged (when the gate_up runs on the row-block
// kernel at 5..16 rows), then the K-slice partial sums of whichever GEMV is running.
struct LayerPlan {
    GemvPlan gu, dn;
    bool staged;
    size_t ws;
};
LayerPlan plan_layer(int M, int H, int I, const Overrides& ov) {
    LayerPlan lp;
    lp.gu = plan_gemv(M, H, 2 * I, ov, kIdentity);
    lp.dn = plan_gemv(M, I, H, ov, kSwiGLU);
    lp.staged = lp.gu.kind == kMfma && lp.gu.mr == 16 && M > 4;
    lp.ws = (lp.staged ? staged_bytes(M, H) : 0) + std::max(lp.gu.partial_bytes, lp.dn.partial_bytes);
    return lp;
}
size_t mlp_ws(int M, int H, int I) { return plan_layer(M, H, I, Overrides{}).ws; }

int check_layer_buffers(const fdec_mlp_layer* L, int M, LayerDims d, const fdec_bf16* x,
                        const fdec_bf16* residual, const fdec_bf16* y_norm, const fdec_bf16* gate_up,
                        const fdec_bf16* out, void* ws, size_t ws_bytes, size_t need) {
    if (!x || !residual || !y_norm || !gate_up || !out)
        return fail(FDEC_ERR_NULL, "x, residual, y_norm, gate_up and out are required");
    if (!aligned16(x) || !aligned16(residual) || !aligned16(y_norm) || !aligned16(gate_up) || !aligned16(out))
        return fail(FDEC_ERR_ALIGN, "every activation buffer must be 16-byte aligned");
    if (ws_bytes < need) return fail(FDEC_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu required", ws_bytes, need);
    if (need > 0 && !ws) return fail(FDEC_ERR_NULL, "workspace is NULL");
    if (ws && !aligned16(ws)) return fail(FDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t t = size_t(M) * d.H * 2;
    const Span X{x, t}, R{residual, t}, Y{y_norm, t}, G{gate_up, size_t(M) * d.I * 4}, O{out, t}, WS{ws, need};
    const Span wts[] = {w4_qspan(&L->gate_up), w4_sspan(&L->gate_up), w4_qspan(&L->down), w4_sspan(&L->down),
                        {L->norm_weight, size_t(d.H) * 2}, {L->out_scale, 4}};
    const Span outs[] = {R, Y, G, O, WS};
    for (const Span& o : outs)
        for (const Span& w : wts)
            if (overlap(o, w)) return fail(FDEC_ERR_ALIAS, "an output buffer overlaps a weight");
    if (overlap(R, X) || overlap(R, Y) || overlap(R, G) || overlap(R, O) || overlap(R, WS) || overlap(Y, X) ||
        overlap(Y, G) || overlap(Y, O) || overlap(Y, WS) || overlap(G, X) || overlap(G, O) || overlap(G, WS) ||
        overlap(O, WS) || overlap(X, WS) || (overlap(O, X) && out != x))
        return fail(FDEC_ERR_ALIAS, "activation buffers overlap (only out == x is allowed)");
    return FDEC_OK;
}

hipError_t enqueue_layer(const fdec_mlp_layer* L, int M, LayerDims d, const LayerPlan& lp, const fdec_bf16* x,
                         fdec_bf16* residual, fdec_bf16* y_norm, fdec_bf16* gate_up, fdec_bf16* out,
                         void* ws, hipStream_t s) {
    char* ys = lp.staged ? static_cast<char*>(ws) : nullptr;
    float* yesc = lp.staged ? reinterpret_cast<float*>(ys + align_up(size_t(M) * d.H * 2)) : nullptr;
    void* pws = lp.staged ? static_cast<void*>(static_cast<char*>(ws) + staged_bytes(M, d.H)) : ws;
    hipError_t e = launch_add_rmsnorm_staged(x, residual, L->norm_weight, L->eps, M, d.H, residual, y_norm, ys,
                                             yesc, s);
    if (e != hipSuccess) return e;
    e = launch_gemv(kIdentity, y_norm, nullptr, d.H, L->gate_up.qweight, L->gate_up.scales, M, d.H, 2 * d.I,
                    nullptr, nullptr, gate_up, pws, lp.gu, s, ys, yesc);
    if (e != hipSuccess) return e;
    return launch_gemv(kSwiGLU, gate_up, gate_up + d.I, 2 * int64_t(d.I), L->down.qweight, L->down.scales, M,
                       d.I, d.H, L->out_scale, L->residual_in_epilogue ? residual : nullptr, out, pws, lp.dn, s);
}

int check_chain(const fdec_mlp_layer* layers, int n_layers, int M, LayerDims* d) {
    if (!layers) return fail(FDEC_ERR_NULL, "layers is NULL");
    if (n_layers < 1) return fail(FDEC_ERR_SHAPE, "n_layers = %d must be >= 1", n_layers);
    int st;
    for (int l = 0; l < n_layers; ++l) {
        LayerDims dl;
        if ((st = check_layer(&layers[l], M, &dl)) != FDEC_OK) return st;
        if (l == 0) *d = dl;
        if (dl.H != d->H || dl.I != d->I) return fail(FDEC_ERR_SHAPE, "layer %d has different H or I", l);
        if (l + 1 < n_layers && layers[l].residual_in_epilogue)
            return fail(FDEC_ERR_ARG, "layer %d: only the last layer may add the residual in its epilogue", l);
    }
    return FDEC_OK;
}

// ---- the two-kernel layer ----
// Workspace: h (the new residual) staged between the two kernels.  The first kernel
// cannot write h into the residual buffer itself: every workgroup of it reads that buffer.
// Up to 4 rows the layer is two kernels (the norm runs as the gate_up GEMV's prologue),
// and the workspace stages h.  From 5 rows the gate_up GEMV is the matrix-core kernel,
// whose K-sliced workgroups cannot each normalise whole rows: the layer is the norm
// (h into the residual buffer in place, y into the workspace), the gate_up GEMV with the
// SwiGLU epilogue, and the down GEMV; the workspace holds y and then the K-slice partial
// sums of whichever GEMV is running.
bool layer2_fused_norm(int M) { return M <= 4; }
// From 5 rows the workspace holds y (bf16), y staged (as above), then the K-slice partial
// sums of whichever GEMV is running.
size_t mlp2_ws(int M, int H, int I, const Overrides& ov) {
    if (layer2_fused_norm(M)) return align_up(size_t(M) * H * 2);
    GemvPlan pp;
    if (!plan_pair(M, H, I, ov, pp)) return 0;
    return align_up(size_t(M) * H * 2) + staged_bytes(M, H) +
           std::max(pp.partial_bytes, plan_gemv(M, I, H, ov, kIdentity).partial_bytes);
}

int check_layer2(const fdec_mlp_layer* L, int M, LayerDims* d, const Overrides& ov) {
    int st = check_layer(L, M, d);
    if (st != FDEC_OK) return st;
    if (!layer2_fused_norm(M)) {
        GemvPlan pp;
        if (!plan_pair(M, d->H, d->I, ov, pp))
            return fail(FDEC_ERR_UNSUPPORTED, "no matrix-core gate_up plan for M = %d, H = %d, I = %d", M, d->H, d->I);
        return FDEC_OK;
    }
    if (!norm_gemv_swiglu_supported(M, d->H, d->I) || !gemv_column_supported(M, d->I, d->H, ov))
        return fail(FDEC_ERR_UNSUPPORTED,
                    "the two-kernel layer needs the column GEMV for both projections (M = %d, H = %d, I = %d)", M,
                    d->H, d->I);
    return FDEC_OK;
}

int check_layer2_buffers(const fdec_mlp_layer* L, int M, LayerDims d, const fdec_bf16* x,
                         const fdec_bf16* residual, const fdec_bf16* act, const fdec_bf16* out, void* ws,
                         size_t ws_bytes, size_t need) {
    if (!x || !residual || !act || !out) return fail(FDEC_ERR_NULL, "x, residual, act and out are required");
    if (!aligned16(x) || !aligned16(residual) || !aligned16(act) || !aligned16(out))
        return fail(FDEC_ERR_ALIGN, "every activation buffer must be 16-byte aligned");
    if (ws_bytes < need) return fail(FDEC_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu required", ws_bytes, need);
    if (!ws) return fail(FDEC_ERR_NULL, "workspace is NULL");
    if (!aligned16(ws)) return fail(FDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t t = size_t(M) * d.H * 2;
    const Span X{x, t}, R{residual, t}, A{act, size_t(M) * d.I * 2}, O{out, t}, WS{ws, need};
    const Span wts[] = {w4_qspan(&L->gate_up), w4_sspan(&L->gate_up), w4_qspan(&L->down), w4_sspan(&L->down),
                        {L->norm_weight, size_t(d.H) * 2}, {L->out_scale, 4}};
    const Span outs[] = {R, A, O, WS};
    for (const Span& o : outs)
        for (const Span& w : wts)
            if (overlap(o, w)) return fail(FDEC_ERR_ALIAS, "an output buffer overlaps a weight");
    if (overlap(R, X) || overlap(R, A) || overlap(R, O) || overlap(R, WS) || overlap(A, X) || overlap(A, O) ||
        overlap(A, WS) || overlap(O, WS) || overlap(X, WS) || (overlap(O, X) && out != x))
        return fail(FDEC_ERR_ALIAS, "activation buffers overlap (only out == x is allowed)");
    return FDEC_OK;
}

hipError_t enqueue_layer2(const fdec_mlp_layer* L, int M, LayerDims d, const Overrides& ov, const fdec_bf16* x,
                          fdec_bf16* residual, fdec_bf16* act, fdec_bf16* out, void* ws, hipStream_t s) {
    if (!layer2_fused_norm(M)) {
        uint16_t* y = static_cast<uint16_t*>(ws);
        char* ys = static_cast<char*>(ws) + align_up(size_t(M) * d.H * 2);
        float* yesc = reinterpret_cast<float*>(ys + align_up(size_t(M) * d.H * 2));
        void* pws = static_cast<char*>(ws) + align_up(size_t(M) * d.H * 2) + staged_bytes(M, d.H);
        GemvPlan pp;
        if (!plan_pair(M, d.H, d.I, ov, pp)) return hipErrorInvalidValue;
        const GemvPlan dp = plan_gemv(M, d.I, d.H, ov, kIdentity);
        // the norm also writes y staged when the row-block gate_up will read it that way
        const bool staged = pp.kind == kMfma && pp.mr == 16;
        hipError_t e = launch_add_rmsnorm_staged(x, residual, L->norm_weight, L->eps, M, d.H, residual, y,
                                                 staged ? ys : nullptr, staged ? yesc : nullptr, s);
        if (e != hipSuccess) return e;
        e = launch_mfma_pair(y, L->gate_up.qweight, L->gate_up.scales, M, d.H, d.I, act, pws, pp, s,
                             staged ? ys : nullptr, staged ? yesc : nullptr);
        if (e != hipSuccess) return e;
        return launch_gemv(kIdentity, act, nullptr, d.I, L->down.qweight, L->down.scales, M, d.I, d.H, L->out_scale,
                           L->residual_in_epilogue ? residual : nullptr, out, pws, dp, s);
    }
    uint16_t* h = static_cast<uint16_t*>(ws);
    hipError_t e = launch_norm_gemv_swiglu(x, residual, L->norm_weight, L->eps, L->gate_up.qweight,
                                           L->gate_up.scales, M, d.H, d.I, h, act, s);
    if (e != hipSuccess) return e;
    return launch_gemv_copy(kIdentity, act, d.I, L->down.qweight, L->down.scales, M, d.I, d.H, L->out_scale,
                            L->residual_in_epilogue ? h : nullptr, out, h, residual, size_t(M) * d.H * 2, ov, s);
}

int check_chain2(const fdec_mlp_layer* layers, int n_layers, int M, LayerDims* d, const Overrides& ov) {
    int st = check_chain(layers, n_layers, M, d);
    if (st != FDEC_OK) return st;
    return check_layer2(&layers[0], M, d, ov);
}

// ---- unfused ----
size_t unfused_norm_ws(int M, int H) {
    return 2 * align_up(size_t(M) * H * 4) + align_up(size_t(M) * 3 * 4);
}
// p: the plan of the sequence's identity-prologue GEMV (M, K, N)
size_t unfused_act_ws(int M, int K, const GemvPlan& p) { return 2 * align_up(size_t(M) * K * 2) + p.partial_bytes; }

hipError_t enqueue_unfused_act(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, const fdec_w4* W,
                               const float* out_scale, const fdec_bf16* residual, int M, fdec_bf16* y,
                               void* ws, const GemvPlan& p, hipStream_t s) {
    const int K = W->K, N = W->N;
    uint16_t* t = static_cast<uint16_t*>(ws);
    uint16_t* act = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + align_up(size_t(M) * K * 2));
    void* gws = static_cast<char*>(ws) + 2 * align_up(size_t(M) * K * 2);
    hipError_t e;
    if ((e = launch_silu_bf16(g, ldgu, M, K, t, s)) != hipSuccess) return e;
    if ((e = launch_mul_bf16(t, K, u, ldgu, M, K, act, s)) != hipSuccess) return e;
    if ((e = launch_gemv(kIdentity, act, nullptr, K, W->qweight, W->scales, M, K, N, nullptr, nullptr, y, gws, p,
                         s)) != hipSuccess)
        return e;
    if ((e = launch_scale_bf16(y, int64_t(M) * N, out_scale, s)) != hipSuccess) return e;
    if (residual) return launch_add_bf16(y, residual, int64_t(M) * N, s);
    return hipSuccess;
}

hipError_t enqueue_eager_norm(const fdec_bf16* x, const fdec_bf16* r, const fdec_bf16* w, float eps, int M, int H,
                              fdec_bf16* h, fdec_bf16* y, void* ws, hipStream_t s) {
    float* a = static_cast<float*>(ws);
    float* b = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(size_t(M) * H * 4));
    float* rows = reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * align_up(size_t(M) * H * 4));
    return launch_eager_rmsnorm(x, r, w, eps, M, H, h, y, a, b, rows, s);
}

}  // namespace

namespace fdec {
Overrides current_overrides() {
    Overrides ov;
    ov.split = g_forced_split.load();
    ov.col_waves = g_col_waves.load();
    ov.col_cols = g_col_cols.load();
    ov.mfma_kernel = g_mfma_kernel.load();
    ov.mfma_tiles = g_mfma_tiles.load();
    ov.mfma_gw = g_mfma_gw.load();
    ov.mfma_waves = g_mfma_waves.load();
    return ov;
}
}  // namespace fdec

struct fdec_graph_s {
    hipGraph_t graph = nullptr;       // the captured graph the executable was made from
    hipGraphExec_t exec = nullptr;
    int kernels = 0;
    int form = 0;                     // 1: three-kernel layers, 2: two-kernel layers
    int n_layers = 0, M = 0, H = 0, I = 0;
};

namespace {

// Captures the chain of the given form on s into *out; nothing runs.  Form 1 uses
// y_norm and gate_up, form 2 uses act.
// The plans and overrides were taken once by the entry point (they fixed the workspace).
struct ChainPlan {
    LayerPlan lp;      // form 1
    Overrides ov;      // form 2
};

hipError_t capture_chain(int form, const ChainPlan& cp, const fdec_mlp_layer* layers, int n_layers, int M,
                         LayerDims d, fdec_bf16* x, fdec_bf16* residual, fdec_bf16* y_norm, fdec_bf16* gate_up,
                         fdec_bf16* act, void* ws, hipStream_t s, hipGraph_t* out) {
    *out = nullptr;
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return e;
    hipError_t le = hipSuccess;
    for (int l = 0; l < n_layers && le == hipSuccess; ++l)
        le = form == 1 ? enqueue_layer(&layers[l], M, d, cp.lp, x, residual, y_norm, gate_up, x, ws, s)
                       : enqueue_layer2(&layers[l], M, d, cp.ov, x, residual, act, x, ws, s);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(s, &g);
    if (le != hipSuccess || e != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return le != hipSuccess ? le : e;
    }
    *out = g;
    return hipSuccess;
}

int make_graph(int form, const ChainPlan& cp, const fdec_mlp_layer* layers, int n_layers, int M, LayerDims d,
               fdec_bf16* x, fdec_bf16* residual, fdec_bf16* y_norm, fdec_bf16* gate_up, fdec_bf16* act, void* ws,
               hipStream_t s, fdec_graph* out) {
    fdec_graph_s* G = new (std::nothrow) fdec_graph_s;
    if (!G) return fail(FDEC_ERR_ARG, "out of host memory");
    hipError_t e =
        capture_chain(form, cp, layers, n_layers, M, d, x, residual, y_norm, gate_up, act, ws, s, &G->graph);
    if (e != hipSuccess) {
        delete G;
        return hip_status(e, "graph capture");
    }
    size_t nodes = 0;
    if (hipGraphGetNodes(G->graph, nullptr, &nodes) != hipSuccess) nodes = 0;
    G->kernels = int(nodes);
    e = hipGraphInstantiate(&G->exec, G->graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(G->graph);
        delete G;
        return hip_status(e, "hipGraphInstantiate");
    }
    G->form = form;
    G->n_layers = n_layers;
    G->M = M;
    G->H = d.H;
    G->I = d.I;
    *out = G;
    return ok();
}

// Re-captures the chain with new layers and buffers and writes the new kernel
// arguments into the existing executable graph (hipGraphExecUpdate): the launch
// shapes are those of the graph, so no re-instantiation is needed.
int update_graph(fdec_graph G, int form, const ChainPlan& cp, const fdec_mlp_layer* layers, int n_layers, int M,
                 LayerDims d, fdec_bf16* x, fdec_bf16* residual, fdec_bf16* y_norm, fdec_bf16* gate_up,
                 fdec_bf16* act, void* ws, hipStream_t s) {
    if (G->form != form || G->n_layers != n_layers || G->M != M || G->H != d.H || G->I != d.I)
        return fail(FDEC_ERR_UNSUPPORTED,
                    "an update keeps the graph's form and shapes (form %d, %d layers, M = %d, H = %d, I = %d); "
                    "got form %d, %d layers, M = %d, H = %d, I = %d",
                    G->form, G->n_layers, G->M, G->H, G->I, form, n_layers, M, d.H, d.I);
    hipGraph_t ng = nullptr;
    hipError_t e = capture_chain(form, cp, layers, n_layers, M, d, x, residual, y_norm, gate_up, act, ws, s, &ng);
    if (e != hipSuccess) return hip_status(e, "graph capture");
    hipGraphNode_t err_node = nullptr;
    hipGraphExecUpdateResult res = hipGraphExecUpdateSuccess;
    e = hipGraphExecUpdate(G->exec, ng, &err_node, &res);
    if (e != hipSuccess || res != hipGraphExecUpdateSuccess) {
        (void)hipGetLastError();
        // keep the handle on the graph it had: a fresh executable from the kept graph
        hipGraphExec_t fresh = nullptr;
        if (hipGraphInstantiate(&fresh, G->graph, nullptr, nullptr, 0) == hipSuccess) {
            (void)hipGraphExecDestroy(G->exec);
            G->exec = fresh;
        }
        (void)hipGraphDestroy(ng);
        return fail(FDEC_ERR_UNSUPPORTED, "hipGraphExecUpdate refused the update (%s, result %d)",
                    hipGetErrorString(e), int(res));
    }
    (void)hipGraphDestroy(G->graph);
    G->graph = ng;
    size_t nodes = 0;                  // HIP may take a chain with other kernels (and nodes)
    if (hipGraphGetNodes(ng, nullptr, &nodes) == hipSuccess) G->kernels = int(nodes);
    return ok();
}

}  // namespace

extern "C" {

FDEC_API int fdec_abi_version(void) { return FDEC_ABI_VERSION; }

FDEC_API const char* fdec_status_str(int status) {
    switch (status) {
        case FDEC_OK: return "FDEC_OK";
        case FDEC_ERR_NULL: return "FDEC_ERR_NULL";
        case FDEC_ERR_SHAPE: return "FDEC_ERR_SHAPE";
        case FDEC_ERR_ALIGN: return "FDEC_ERR_ALIGN";
        case FDEC_ERR_ALIAS: return "FDEC_ERR_ALIAS";
        case FDEC_ERR_WORKSPACE: return "FDEC_ERR_WORKSPACE";
        case FDEC_ERR_UNSUPPORTED: return "FDEC_ERR_UNSUPPORTED";
        case FDEC_ERR_HIP: return "FDEC_ERR_HIP";
        case FDEC_ERR_ARG: return "FDEC_ERR_ARG";
        default: return "FDEC_ERR_UNKNOWN";
    }
}

FDEC_API const char* fdec_last_error(void) { return t_last_error.c_str(); }

FDEC_API void fdec_set_gemv_split(int32_t k) { g_forced_split.store(k > 0 ? k : 0); }
FDEC_API void fdec_set_gemv_tiling(int32_t waves, int32_t cols_per_workgroup) {
    g_col_waves.store(waves > 0 ? waves : 0);
    g_col_cols.store(cols_per_workgroup > 0 ? cols_per_workgroup : 0);
}
FDEC_API void fdec_test_fail_launches(int32_t on) { g_fail_launches.store(on ? 1 : 0); }
FDEC_API void fdec_set_mfma_plan(int32_t kernel, int32_t tiles, int32_t groups_per_wave) {
    g_mfma_kernel.store(kernel >= 1 && kernel <= 3 ? kernel : 0);
    g_mfma_tiles.store(tiles == 4 || tiles == 8 ? tiles : 0);
    g_mfma_gw.store(groups_per_wave >= 1 && groups_per_wave <= 4 ? groups_per_wave : 0);
}

FDEC_API void fdec_set_kmfma_waves(int32_t waves) { g_mfma_waves.store(waves >= 6 && waves <= 8 ? waves : 0); }

FDEC_API size_t fdec_test_gemv_workspace_bytes(int32_t M, int32_t K, int32_t N) {
    if (!w4_gemv_shape_ok(M, K, N)) return 0;
    const Overrides ov = current_overrides();
    return std::max(plan_gemv(M, K, N, ov, kSwiGLU).partial_bytes, plan_gemv(M, K, N, ov, kIdentity).partial_bytes);
}

FDEC_API int32_t fdec_test_gemv_kernel(int32_t M, int32_t K, int32_t N, int32_t swiglu) {
    if (!w4_gemv_shape_ok(M, K, N)) return -1;
    return int32_t(plan_gemv(M, K, N, current_overrides(), swiglu ? kSwiGLU : kIdentity).kind);
}

FDEC_API size_t fdec_test_mlp_workspace_bytes(int32_t M, int32_t H, int32_t I) {
    if (M < 1 || M > 16 || H <= 0 || H % 128 || I <= 0 || I % 128) return 0;
    return plan_layer(M, H, I, current_overrides()).ws;
}

FDEC_API int fdec_test_empty_kernel(int32_t wgs, int32_t threads, fdec_stream stream) {
    if (wgs < 1 || wgs > 65536 || threads < 64 || threads > 1024 || threads % 64)
        return fail(FDEC_ERR_SHAPE, "empty kernel: wgs = %d, threads = %d out of range", wgs, threads);
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_empty(wgs, threads, static_cast<hipStream_t>(stream)), "empty kernel launch");
}

FDEC_API int fdec_test_read_ceiling(const void* stream_buf, size_t stream_bytes, int32_t per_wg, const void* bcast0,
                                    const void* bcast1, size_t bcast_bytes, const void* pieces, size_t pieces_bytes,
                                    int32_t rows, int32_t row_bytes, int32_t piece_bytes, int32_t wgs, uint32_t* sink,
                                    fdec_stream stream) {
    if (!stream_buf || !bcast0 || !bcast1 || !pieces || !sink) return fail(FDEC_ERR_NULL, "read ceiling: NULL buffer");
    if (!aligned16(stream_buf) || !aligned16(bcast0) || !aligned16(bcast1) || !aligned16(pieces) || !aligned4(sink) ||
        row_bytes % 16)
        return fail(FDEC_ERR_ALIGN, "read ceiling: buffers must be 16-byte aligned and row_bytes a multiple of 16");
    if (wgs < 1 || wgs > 65536 || bcast_bytes % 16 || !read_ceiling_fits(per_wg, int(bcast_bytes / 16), rows, piece_bytes))
        return fail(FDEC_ERR_SHAPE, "read ceiling: sizes outside the probe's limits");
    if (uint64_t(wgs) * uint64_t(per_wg) * 16 > stream_bytes)
        return fail(FDEC_ERR_SHAPE, "read ceiling: wgs * per_wg chunks exceed the stream buffer");
    // the last workgroup's last piece of the last row ends inside `pieces`
    const uint64_t last_end = uint64_t(rows - 1) * uint64_t(row_bytes) +
                              ((uint64_t(wgs) * uint64_t(piece_bytes) - 1) / 16 + 1) * 16;
    if (last_end > pieces_bytes || uint64_t(wgs) * uint64_t(piece_bytes) > uint64_t(row_bytes))
        return fail(FDEC_ERR_SHAPE, "read ceiling: the pieces exceed their rows or buffer");
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_read_ceiling(stream_buf, per_wg, bcast0, bcast1, int(bcast_bytes / 16), pieces, rows,
                                          row_bytes, piece_bytes, wgs, sink, static_cast<hipStream_t>(stream)),
                      "read ceiling launch");
}

FDEC_API int fdec_workspace_init(void* ws, size_t ws_bytes, fdec_stream stream) {
    if (ws_bytes == 0) return ok();
    if (!ws) return fail(FDEC_ERR_NULL, "workspace is NULL");
    if (!aligned16(ws)) return fail(FDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)), "fill kernel");
}

FDEC_API int fdec_add_rmsnorm(const fdec_bf16* x, const fdec_bf16* residual, const fdec_bf16* weight, float eps,
                              int32_t M, int32_t H, fdec_bf16* h_out, fdec_bf16* y_out, fdec_stream stream) {
    const int st = check_norm(x, residual, weight, eps, M, H, h_out, y_out);
    if (st != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_add_rmsnorm(x, residual, weight, eps, M, H, h_out, y_out,
                                         static_cast<hipStream_t>(stream)),
                      "add_rmsnorm launch");
}

FDEC_API size_t fdec_w4_gemv_workspace_bytes(int32_t M, int32_t K, int32_t N) {
    return w4_gemv_shape_ok(M, K, N) ? gemv_workspace_bytes(M, K, N) : 0;
}

FDEC_API int fdec_swiglu_w4_gemv(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, const fdec_w4* W,
                                 const float* out_scale, const fdec_bf16* residual, int32_t M, fdec_bf16* y,
                                 void* ws, size_t ws_bytes, fdec_stream stream) {
    if (!W) return fail(FDEC_ERR_NULL, "W is NULL");
    const bool shape_ok = w4_gemv_shape_ok(M, W->K, W->N);
    const GemvPlan p = shape_ok ? plan_gemv(M, W->K, W->N, current_overrides(), kSwiGLU) : GemvPlan{};
    const int st = check_gemv(g, u, ldgu, W, out_scale, residual, M, y, ws, ws_bytes, true, p.partial_bytes,
                              kMaxGemvRows);
    if (st != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_gemv(kSwiGLU, g, u, ldgu, W->qweight, W->scales, M, W->K, W->N, out_scale, residual,
                                  y, ws, p, static_cast<hipStream_t>(stream)),
                      "gemv launch");
}

}  // extern "C"

// ---- the allocation-free SwiGLU GEMV: its K-slice partial sums live in a static device
// array instead of a caller workspace ----
namespace {

constexpr size_t kScratchBytes = FDEC_NOALLOC_SCRATCH_BYTES;
// Every GPU the library runs on holds its own copy until the process ends.  In host code
// the name `scratch` is only a host-side stand-in: the device address of this GPU's copy
// comes from hipGetSymbolAddress, taken once per device and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on device `dev`, which must be the current device.
hipError_t scratch_address(int dev, void** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

FDEC_API int fdec_swiglu_w4_gemv_noalloc(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, const fdec_w4* W,
                                         const float* out_scale, const fdec_bf16* residual, int32_t M,
                                         fdec_bf16* y, fdec_stream stream) {
    if (!W) return fail(FDEC_ERR_NULL, "W is NULL");
    const bool shape_ok = w4_gemv_shape_ok(M, W->K, W->N);
    const GemvPlan p = shape_ok ? plan_gemv(M, W->K, W->N, current_overrides(), kSwiGLU) : GemvPlan{};
    // the same checks as fdec_swiglu_w4_gemv with no workspace, then the scratch limit
    int st = check_gemv(g, u, ldgu, W, out_scale, residual, M, y, nullptr, 0, true, 0, kMaxGemvRows);
    if (st != FDEC_OK) return st;
    if (p.partial_bytes > kScratchBytes)
        return fail(FDEC_ERR_WORKSPACE, "this shape needs %zu bytes of partial sums; the static scratch holds %zu",
                    p.partial_bytes, kScratchBytes);
    if (g_fail_launches.load()) return injected();
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (p.partial_bytes > 0) {
        int dev = -1;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return hip_status(e, "hipGetDevice");
        if (dev < 0 || dev >= kMaxDevices) return fail(FDEC_ERR_UNSUPPORTED, "device %d is beyond %d", dev, kMaxDevices);
        if (s) {
            hipDevice_t sdev = -1;
            if ((e = hipStreamGetDevice(s, &sdev)) != hipSuccess) return hip_status(e, "hipStreamGetDevice");
            if (int(sdev) != dev)
                return fail(FDEC_ERR_ARG, "the stream belongs to device %d, the current device is %d", int(sdev), dev);
        }
        if ((e = scratch_address(dev, &ws)) != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        // y and the inputs may not overlap the scratch (they cannot: it is the library's own)
    }
    return hip_status(launch_gemv(kSwiGLU, g, u, ldgu, W->qweight, W->scales, M, W->K, W->N, out_scale, residual, y,
                                  ws, p, s),
                      "gemv launch");
}

FDEC_API int fdec_w4_gemv(const fdec_bf16* x, const fdec_w4* W, const float* out_scale, int32_t M, fdec_bf16* y,
                          void* ws, size_t ws_bytes, fdec_stream stream) {
    if (!W) return fail(FDEC_ERR_NULL, "W is NULL");
    const bool shape_ok = w4_gemv_shape_ok(M, W->K, W->N);
    const GemvPlan p = shape_ok ? plan_gemv(M, W->K, W->N, current_overrides(), kIdentity) : GemvPlan{};
    const int st = check_gemv(x, nullptr, W->K, W, out_scale, nullptr, M, y, ws, ws_bytes, false, p.partial_bytes,
                              kMaxGemvRows);
    if (st != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_gemv(kIdentity, x, nullptr, W->K, W->qweight, W->scales, M, W->K, W->N, out_scale,
                                  nullptr, y, ws, p, static_cast<hipStream_t>(stream)),
                      "gemv launch");
}

FDEC_API size_t fdec_mlp_workspace_bytes(int32_t M, int32_t H, int32_t I) {
    if (M < 1 || M > 16 || H <= 0 || H % 128 || I <= 0 || I % 128) return 0;
    return mlp_ws(M, H, I);
}

FDEC_API int fdec_mlp_decode(const fdec_mlp_layer* layer, int32_t M, const fdec_bf16* x, fdec_bf16* residual,
                             fdec_bf16* y_norm, fdec_bf16* gate_up, fdec_bf16* out, void* ws, size_t ws_bytes,
                             fdec_stream stream) {
    LayerDims d;
    int st = check_layer(layer, M, &d);
    if (st != FDEC_OK) return st;
    const LayerPlan lp = plan_layer(M, d.H, d.I, current_overrides());
    st = check_layer_buffers(layer, M, d, x, residual, y_norm, gate_up, out, ws, ws_bytes, lp.ws);
    if (st != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(enqueue_layer(layer, M, d, lp, x, residual, y_norm, gate_up, out, ws,
                                    static_cast<hipStream_t>(stream)),
                      "layer launch");
}

FDEC_API int fdec_mlp_chain(const fdec_mlp_layer* layers, int32_t n_layers, int32_t M, fdec_bf16* x,
                            fdec_bf16* residual, fdec_bf16* y_norm, fdec_bf16* gate_up, void* ws, size_t ws_bytes,
                            fdec_stream stream) {
    LayerDims d;
    int st = check_chain(layers, n_layers, M, &d);
    if (st != FDEC_OK) return st;
    const LayerPlan lp = plan_layer(M, d.H, d.I, current_overrides());
    for (int l = 0; l < n_layers; ++l)
        if ((st = check_layer_buffers(&layers[l], M, d, x, residual, y_norm, gate_up, x, ws, ws_bytes, lp.ws)) !=
            FDEC_OK)
            return st;
    if (g_fail_launches.load()) return injected();
    for (int l = 0; l < n_layers; ++l) {
        const hipError_t e = enqueue_layer(&layers[l], M, d, lp, x, residual, y_norm, gate_up, x, ws,
                                           static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_status(e, "chain launch");
    }
    return ok();
}

FDEC_API int fdec_mlp_graph_create(const fdec_mlp_layer* layers, int32_t n_layers, int32_t M, fdec_bf16* x,
                                   fdec_bf16* residual, fdec_bf16* y_norm, fdec_bf16* gate_up, void* ws,
                                   size_t ws_bytes, fdec_stream stream, fdec_graph* out) {
    if (!out) return fail(FDEC_ERR_NULL, "out is NULL");
    if (!stream) return fail(FDEC_ERR_ARG, "graph capture needs a non-null stream");
    LayerDims d;
    int st = check_chain(layers, n_layers, M, &d);
    if (st != FDEC_OK) return st;
    ChainPlan cp;
    cp.ov = current_overrides();
    cp.lp = plan_layer(M, d.H, d.I, cp.ov);
    for (int l = 0; l < n_layers; ++l)
        if ((st = check_layer_buffers(&layers[l], M, d, x, residual, y_norm, gate_up, x, ws, ws_bytes, cp.lp.ws)) !=
            FDEC_OK)
            return st;
    if (g_fail_launches.load()) return injected();
    return make_graph(1, cp, layers, n_layers, M, d, x, residual, y_norm, gate_up, nullptr, ws,
                      static_cast<hipStream_t>(stream), out);
}

FDEC_API int fdec_mlp_graph_update(fdec_graph graph, const fdec_mlp_layer* layers, int32_t n_layers, int32_t M,
                                   fdec_bf16* x, fdec_bf16* residual, fdec_bf16* y_norm, fdec_bf16* gate_up,
                                   void* ws, size_t ws_bytes, fdec_stream stream) {
    if (!graph || !graph->exec) return fail(FDEC_ERR_NULL, "graph is NULL");
    if (!stream) return fail(FDEC_ERR_ARG, "graph capture needs a non-null stream");
    LayerDims d;
    int st = check_chain(layers, n_layers, M, &d);
    if (st != FDEC_OK) return st;
    ChainPlan cp;
    cp.ov = current_overrides();
    cp.lp = plan_layer(M, d.H, d.I, cp.ov);
    for (int l = 0; l < n_layers; ++l)
        if ((st = check_layer_buffers(&layers[l], M, d, x, residual, y_norm, gate_up, x, ws, ws_bytes, cp.lp.ws)) !=
            FDEC_OK)
            return st;
    if (g_fail_launches.load()) return injected();
    return update_graph(graph, 1, cp, layers, n_layers, M, d, x, residual, y_norm, gate_up, nullptr, ws,
                        static_cast<hipStream_t>(stream));
}

FDEC_API int fdec_graph_launch(fdec_graph graph, fdec_stream stream) {
    if (!graph || !graph->exec) return fail(FDEC_ERR_NULL, "graph is NULL");
    if (g_fail_launches.load()) return injected();
    return hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)), "hipGraphLaunch");
}

FDEC_API int fdec_graph_kernel_count(fdec_graph graph) { return graph ? graph->kernels : -1; }

FDEC_API int fdec_graph_destroy(fdec_graph graph) {
    if (!graph) return ok();
    hipError_t e1 = graph->exec ? hipGraphExecDestroy(graph->exec) : hipSuccess;
    hipError_t e2 = graph->graph ? hipGraphDestroy(graph->graph) : hipSuccess;
    delete graph;
    return hip_status(e1 != hipSuccess ? e1 : e2, "graph destroy");
}

FDEC_API int fdec_add_rmsnorm_w4_gemv_swiglu(const fdec_bf16* x, const fdec_bf16* residual,
                                             const fdec_bf16* norm_weight, float eps, const fdec_w4* gate_up,
                                             int32_t M, fdec_bf16* h_out, fdec_bf16* act_out, fdec_stream stream) {
    int st;
    if ((st = check_w4(gate_up, "gate_up")) != FDEC_OK) return st;
    if ((st = check_m(M)) != FDEC_OK) return st;
    const int H = gate_up->K;
    if (gate_up->N % 16) return fail(FDEC_ERR_SHAPE, "gate_up.N = %d must be 2I with I a multiple of 8", gate_up->N);
    const int I = gate_up->N / 2;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(FDEC_ERR_ARG, "eps must be finite and >= 0");
    if (!x || !residual || !norm_weight || !h_out || !act_out)
        return fail(FDEC_ERR_NULL, "x, residual, norm_weight, h_out and act_out are required");
    if (!aligned16(x) || !aligned16(residual) || !aligned16(norm_weight) || !aligned16(h_out) || !aligned16(act_out))
        return fail(FDEC_ERR_ALIGN, "every tensor must be 16-byte aligned");
    const size_t t = size_t(M) * H * 2;
    const Span X{x, t}, R{residual, t}, NW{norm_weight, size_t(H) * 2}, Hs{h_out, t}, A{act_out, size_t(M) * I * 2};
    const Span ins[] = {X, R, NW, w4_qspan(gate_up), w4_sspan(gate_up)};
    for (const Span& in : ins)
        if (overlap(Hs, in) || overlap(A, in)) return fail(FDEC_ERR_ALIAS, "h_out or act_out overlaps an input");
    if (overlap(Hs, A)) return fail(FDEC_ERR_ALIAS, "h_out overlaps act_out");
    if (!norm_gemv_swiglu_supported(M, H, I))
        return fail(FDEC_ERR_UNSUPPORTED, "no column-kernel variant for M = %d, H = %d, I = %d", M, H, I);
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_norm_gemv_swiglu(x, residual, norm_weight, eps, gate_up->qweight, gate_up->scales, M, H,
                                              I, h_out, act_out, static_cast<hipStream_t>(stream)),
                      "fused gate_up launch");
}

FDEC_API size_t fdec_mlp2_workspace_bytes(int32_t M, int32_t H, int32_t I) {
    if (M < 1 || M > 16 || H <= 0 || H % 128 || I <= 0 || I % 128) return 0;
    return mlp2_ws(M, H, I, Overrides{});
}

FDEC_API size_t fdec_w4_gemv_swiglu_workspace_bytes(int32_t M, int32_t K, int32_t I) {
    GemvPlan p;
    if (K <= 0 || K % 128 || !plan_pair(M, K, I, Overrides{}, p)) return 0;
    return p.partial_bytes;
}

FDEC_API int fdec_w4_gemv_swiglu(const fdec_bf16* x, const fdec_w4* gate_up, int32_t M, fdec_bf16* act_out,
                                 void* ws, size_t ws_bytes, fdec_stream stream) {
    int st;
    if ((st = check_w4(gate_up, "gate_up")) != FDEC_OK) return st;
    if ((st = check_m(M, kMaxGemvRows)) != FDEC_OK) return st;
    if (gate_up->N % 16) return fail(FDEC_ERR_SHAPE, "gate_up.N = %d must be 2I with I a multiple of 8", gate_up->N);
    const int K = gate_up->K, I = gate_up->N / 2;
    if (!x || !act_out) return fail(FDEC_ERR_NULL, "x and act_out are required");
    if (!aligned16(x) || !aligned16(act_out)) return fail(FDEC_ERR_ALIGN, "x and act_out must be 16-byte aligned");
    GemvPlan p;
    if (!plan_pair(M, K, I, current_overrides(), p)) return fail(FDEC_ERR_UNSUPPORTED, "no plan for M = %d, K = %d, I = %d", M, K, I);
    if (ws_bytes < p.partial_bytes)
        return fail(FDEC_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu required", ws_bytes, p.partial_bytes);
    if (p.partial_bytes > 0 && !ws) return fail(FDEC_ERR_NULL, "workspace is NULL");
    if (ws && !aligned16(ws)) return fail(FDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    const Span X{x, size_t(M) * K * 2}, A{act_out, size_t(M) * I * 2}, WS{ws, p.partial_bytes};
    const Span ins[] = {X, w4_qspan(gate_up), w4_sspan(gate_up)};
    for (const Span& in : ins)
        if (overlap(A, in) || overlap(WS, in)) return fail(FDEC_ERR_ALIAS, "act_out or the workspace overlaps an input");
    if (overlap(A, WS)) return fail(FDEC_ERR_ALIAS, "act_out overlaps the workspace");
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_mfma_pair(x, gate_up->qweight, gate_up->scales, M, K, I, act_out, ws, p,
                                       static_cast<hipStream_t>(stream)),
                      "gate_up SwiGLU launch");
}

FDEC_API int fdec_mlp_decode2(const fdec_mlp_layer* layer, int32_t M, const fdec_bf16* x, fdec_bf16* residual,
                              fdec_bf16* act, fdec_bf16* out, void* ws, size_t ws_bytes, fdec_stream stream) {
    LayerDims d;
    const Overrides ov = current_overrides();
    int st = check_layer2(layer, M, &d, ov);
    if (st != FDEC_OK) return st;
    st = check_layer2_buffers(layer, M, d, x, residual, act, out, ws, ws_bytes, mlp2_ws(M, d.H, d.I, ov));
    if (st != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(enqueue_layer2(layer, M, d, ov, x, residual, act, out, ws, static_cast<hipStream_t>(stream)),
                      "layer launch");
}

FDEC_API int fdec_mlp_chain2(const fdec_mlp_layer* layers, int32_t n_layers, int32_t M, fdec_bf16* x,
                             fdec_bf16* residual, fdec_bf16* act, void* ws, size_t ws_bytes, fdec_stream stream) {
    LayerDims d;
    const Overrides ov = current_overrides();
    int st = check_chain2(layers, n_layers, M, &d, ov);
    if (st != FDEC_OK) return st;
    const size_t need = mlp2_ws(M, d.H, d.I, ov);
    for (int l = 0; l < n_layers; ++l)
        if ((st = check_layer2_buffers(&layers[l], M, d, x, residual, act, x, ws, ws_bytes, need)) != FDEC_OK)
            return st;
    if (g_fail_launches.load()) return injected();
    for (int l = 0; l < n_layers; ++l) {
        const hipError_t e =
            enqueue_layer2(&layers[l], M, d, ov, x, residual, act, x, ws, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_status(e, "chain launch");
    }
    return ok();
}

FDEC_API int fdec_mlp_graph_create2(const fdec_mlp_layer* layers, int32_t n_layers, int32_t M, fdec_bf16* x,
                                    fdec_bf16* residual, fdec_bf16* act, void* ws, size_t ws_bytes,
                                    fdec_stream stream, fdec_graph* out) {
    if (!out) return fail(FDEC_ERR_NULL, "out is NULL");
    if (!stream) return fail(FDEC_ERR_ARG, "graph capture needs a non-null stream");
    LayerDims d;
    ChainPlan cp;
    cp.ov = current_overrides();
    int st = check_chain2(layers, n_layers, M, &d, cp.ov);
    if (st != FDEC_OK) return st;
    const size_t need = mlp2_ws(M, d.H, d.I, cp.ov);
    for (int l = 0; l < n_layers; ++l)
        if ((st = check_layer2_buffers(&layers[l], M, d, x, residual, act, x, ws, ws_bytes, need)) != FDEC_OK)
            return st;
    if (g_fail_launches.load()) return injected();
    return make_graph(2, cp, layers, n_layers, M, d, x, residual, nullptr, nullptr, act, ws,
                      static_cast<hipStream_t>(stream), out);
}

FDEC_API int fdec_mlp_graph_update2(fdec_graph graph, const fdec_mlp_layer* layers, int32_t n_layers, int32_t M,
                                    fdec_bf16* x, fdec_bf16* residual, fdec_bf16* act, void* ws, size_t ws_bytes,
                                    fdec_stream stream) {
    if (!graph || !graph->exec) return fail(FDEC_ERR_NULL, "graph is NULL");
    if (!stream) return fail(FDEC_ERR_ARG, "graph capture needs a non-null stream");
    LayerDims d;
    ChainPlan cp;
    cp.ov = current_overrides();
    int st = check_chain2(layers, n_layers, M, &d, cp.ov);
    if (st != FDEC_OK) return st;
    const size_t need = mlp2_ws(M, d.H, d.I, cp.ov);
    for (int l = 0; l < n_layers; ++l)
        if ((st = check_layer2_buffers(&layers[l], M, d, x, residual, act, x, ws, ws_bytes, need)) != FDEC_OK)
            return st;
    if (g_fail_launches.load()) return injected();
    return update_graph(graph, 2, cp, layers, n_layers, M, d, x, residual, nullptr, nullptr, act, ws,
                        static_cast<hipStream_t>(stream));
}

FDEC_API size_t fdec_unfused_gemv_workspace_bytes(int32_t mode, int32_t M, int32_t K, int32_t N) {
    if (M < 1 || M > 16 || K <= 0 || K % 128 || N <= 0 || N % 8) return 0;
    if (mode == FDEC_UNFUSED_PRODUCT) return M == 1 ? size_t(M) * K * N * 4 : 0;
    if (mode == FDEC_UNFUSED_ACT) return unfused_act_ws(M, K, plan_gemv(M, K, N, Overrides{}, kIdentity));
    return 0;
}

FDEC_API int fdec_unfused_swiglu_w4_gemv(int32_t mode, const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu,
                                         const fdec_w4* W, const float* out_scale, const fdec_bf16* residual,
                                         int32_t M, fdec_bf16* y, void* ws, size_t ws_bytes, fdec_stream stream) {
    if (mode != FDEC_UNFUSED_PRODUCT && mode != FDEC_UNFUSED_ACT) return fail(FDEC_ERR_ARG, "unknown mode %d", mode);
    if (!W) return fail(FDEC_ERR_NULL, "W is NULL");
    if (mode == FDEC_UNFUSED_PRODUCT && M != 1)
        return fail(FDEC_ERR_UNSUPPORTED, "the materialised-product sequence is defined for M == 1 only (M = %d)", M);
    const bool shape_ok = M >= 1 && M <= 16 && W->K > 0 && W->K % 128 == 0 && W->N > 0 && W->N % 8 == 0;
    const GemvPlan p = shape_ok ? plan_gemv(M, W->K, W->N, current_overrides(), kIdentity) : GemvPlan{};
    const size_t need = !shape_ok ? 0
                        : mode == FDEC_UNFUSED_PRODUCT ? size_t(M) * W->K * W->N * 4
                                                       : unfused_act_ws(M, W->K, p);
    const int st = check_gemv(g, u, ldgu, W, out_scale, residual, M, y, ws, ws_bytes, true, need);
    if (st != FDEC_OK) return st;
    if (residual == y) return fail(FDEC_ERR_ALIAS, "the unfused sequence needs y distinct from residual");
    if (g_fail_launches.load()) return injected();
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mode == FDEC_UNFUSED_PRODUCT)
        return hip_status(launch_unfused_product(g, u, W->qweight, W->scales, W->K, W->N, out_scale, residual, y,
                                                 static_cast<float*>(ws), s),
                          "unfused product launch");
    return hip_status(enqueue_unfused_act(g, u, ldgu, W, out_scale, residual, M, y, ws, p, s), "unfused act launch");
}

FDEC_API size_t fdec_unfused_add_rmsnorm_workspace_bytes(int32_t M, int32_t H) {
    if (M < 0 || H < 8 || H > 16384 || H % 8) return 0;
    return unfused_norm_ws(M, H);
}

FDEC_API int fdec_unfused_add_rmsnorm(const fdec_bf16* x, const fdec_bf16* residual, const fdec_bf16* weight,
                                      float eps, int32_t M, int32_t H, fdec_bf16* h_out, fdec_bf16* y_out, void* ws,
                                      size_t ws_bytes, fdec_stream stream) {
    int st = check_norm(x, residual, weight, eps, M, H, h_out, y_out);
    if (st != FDEC_OK) return st;
    const size_t need = unfused_norm_ws(M, H);
    if (ws_bytes < need) return fail(FDEC_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu required", ws_bytes, need);
    if (need > 0 && !ws) return fail(FDEC_ERR_NULL, "workspace is NULL");
    if (ws && !aligned16(ws)) return fail(FDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t t = size_t(M) * H * 2;
    const Span WS{ws, need};
    if (overlap(WS, {x, t}) || overlap(WS, {residual, t}) || overlap(WS, {weight, size_t(H) * 2}) ||
        overlap(WS, {h_out, t}) || overlap(WS, {y_out, t}))
        return fail(FDEC_ERR_ALIAS, "the workspace overlaps a tensor");
    if (g_fail_launches.load()) return injected();
    return hip_status(enqueue_eager_norm(x, residual, weight, eps, M, H, h_out, y_out, ws,
                                         static_cast<hipStream_t>(stream)),
                      "eager norm launch");
}

namespace {
// norm scratch, then the ACT sequence's scratch (its down GEMV plan lp.dn), then the
// gate_up GEMV's workspace (plan lp.gu)
size_t unfused_mlp_ws(int M, int H, int I, const LayerPlan& lp) {
    return align_up(unfused_norm_ws(M, H)) + align_up(unfused_act_ws(M, I, lp.dn)) + align_up(lp.gu.partial_bytes);
}
}  // namespace

FDEC_API size_t fdec_unfused_mlp_workspace_bytes(int32_t M, int32_t H, int32_t I) {
    if (M < 1 || M > 16 || H <= 0 || H % 128 || I <= 0 || I % 128) return 0;
    return unfused_mlp_ws(M, H, I, plan_layer(M, H, I, Overrides{}));
}

FDEC_API int fdec_unfused_mlp_decode(const fdec_mlp_layer* layer, int32_t M, const fdec_bf16* x,
                                     fdec_bf16* residual, fdec_bf16* y_norm, fdec_bf16* gate_up, fdec_bf16* out,
                                     void* ws, size_t ws_bytes, fdec_stream stream) {
    LayerDims d;
    int st = check_layer(layer, M, &d);
    if (st != FDEC_OK) return st;
    const LayerPlan lp = plan_layer(M, d.H, d.I, current_overrides());
    const size_t need = unfused_mlp_ws(M, d.H, d.I, lp);
    st = check_layer_buffers(layer, M, d, x, residual, y_norm, gate_up, out, ws, ws_bytes, need);
    if (st != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    void* norm_ws = w;
    void* act_ws = w + align_up(unfused_norm_ws(M, d.H));
    void* gu_ws = static_cast<char*>(act_ws) + align_up(unfused_act_ws(M, d.I, lp.dn));
    hipError_t e = enqueue_eager_norm(x, residual, layer->norm_weight, layer->eps, M, d.H, residual, y_norm,
                                      norm_ws, s);
    if (e == hipSuccess)
        e = launch_gemv(kIdentity, y_norm, nullptr, d.H, layer->gate_up.qweight, layer->gate_up.scales, M, d.H,
                        2 * d.I, nullptr, nullptr, gate_up, gu_ws, lp.gu, s);
    if (e == hipSuccess)
        e = enqueue_unfused_act(gate_up, gate_up + d.I, 2 * int64_t(d.I), &layer->down, layer->out_scale,
                                layer->residual_in_epilogue ? residual : nullptr, M, out, act_ws, lp.dn, s);
    return hip_status(e, "unfused layer launch");
}

// ---- prefill sizes: the fused SwiGLU elementwise pass and the W4 GEMM ----
namespace {
int check_prefill_gemm(const fdec_bf16* x, const fdec_w4* W, const float* out_scale, const fdec_bf16* residual,
                       int M, const fdec_bf16* y) {
    int st;
    if ((st = check_w4(W, "W")) != FDEC_OK) return st;
    if (M < 1 || M > (1 << 24)) return fail(FDEC_ERR_SHAPE, "M = %d must be in [1, 2^24]", M);
    if (!x || !y) return fail(FDEC_ERR_NULL, "x and y are required");
    if (!aligned16(x) || !aligned16(y) || (residual && !aligned16(residual)))
        return fail(FDEC_ERR_ALIGN, "x, y and residual must be 16-byte aligned");
    if (out_scale && !aligned4(out_scale)) return fail(FDEC_ERR_ALIGN, "out_scale must be 4-byte aligned");
    const Span X{x, size_t(M) * W->K * 2}, Y{y, size_t(M) * W->N * 2};
    const Span ins[] = {X, w4_qspan(W), w4_sspan(W), {out_scale, 4}};
    for (const Span& in : ins)
        if (overlap(Y, in)) return fail(FDEC_ERR_ALIAS, "y overlaps an input");
    if (residual && overlap(Y, Span{residual, Y.bytes}) && residual != y)
        return fail(FDEC_ERR_ALIAS, "y may only alias residual exactly");
    return FDEC_OK;
}
}  // namespace

FDEC_API int fdec_w4_gemm(const fdec_bf16* x, const fdec_w4* W, const float* out_scale, const fdec_bf16* residual,
                          int32_t M, fdec_bf16* y, fdec_stream stream) {
    const int st = check_prefill_gemm(x, W, out_scale, residual, M, y);
    if (st != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_w4_gemm(x, W->K, W->qweight, W->scales, M, W->K, W->N, out_scale, residual, y,
                                     static_cast<hipStream_t>(stream)),
                      "gemm launch");
}

FDEC_API int fdec_swiglu(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, int32_t M, int32_t K,
                         fdec_bf16* act, fdec_stream stream) {
    if (M < 0 || K <= 0 || K % 8) return fail(FDEC_ERR_SHAPE, "M = %d, K = %d: M >= 0, K a positive multiple of 8", M, K);
    if (M == 0) return ok();
    if (!g || !u || !act) return fail(FDEC_ERR_NULL, "g, u and act are required");
    if (ldgu < K || ldgu % 8) return fail(FDEC_ERR_SHAPE, "ld = %lld must be >= K and a multiple of 8", (long long)ldgu);
    if (!aligned16(g) || !aligned16(u) || !aligned16(act)) return fail(FDEC_ERR_ALIGN, "every tensor must be 16-byte aligned");
    const size_t in_bytes = (size_t(M - 1) * ldgu + K) * 2;
    const Span A{act, size_t(M) * K * 2};
    if (overlap(A, {g, in_bytes}) || overlap(A, {u, in_bytes})) return fail(FDEC_ERR_ALIAS, "act overlaps g or u");
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_swiglu_act(g, u, ldgu, M, K, act, static_cast<hipStream_t>(stream)), "swiglu launch");
}

FDEC_API size_t fdec_swiglu_w4_gemm_workspace_bytes(int32_t M, int32_t K) {
    if (M < 1 || K <= 0 || K % 128) return 0;
    return size_t(M) * K * 2;
}

FDEC_API int fdec_swiglu_w4_gemm(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, const fdec_w4* W,
                                 const float* out_scale, const fdec_bf16* residual, int32_t M, fdec_bf16* y,
                                 void* ws, size_t ws_bytes, fdec_stream stream) {
    if (!W) return fail(FDEC_ERR_NULL, "W is NULL");
    int st = check_prefill_gemm(g, W, out_scale, residual, M, y);
    if (st != FDEC_OK) return st;
    if (!u) return fail(FDEC_ERR_NULL, "u is required");
    if (ldgu < W->K || ldgu % 8) return fail(FDEC_ERR_SHAPE, "ld = %lld must be >= K and a multiple of 8", (long long)ldgu);
    if (!aligned16(u)) return fail(FDEC_ERR_ALIGN, "u must be 16-byte aligned");
    const size_t need = size_t(M) * W->K * 2;
    if (ws_bytes < need) return fail(FDEC_ERR_WORKSPACE, "workspace of %zu bytes is below the %zu required", ws_bytes, need);
    if (!ws) return fail(FDEC_ERR_NULL, "workspace is NULL");
    if (!aligned16(ws)) return fail(FDEC_ERR_ALIGN, "workspace must be 16-byte aligned");
    const size_t in_bytes = (size_t(M - 1) * ldgu + W->K) * 2;
    const Span WS{ws, need};
    const Span others[] = {{g, in_bytes}, {u, in_bytes}, w4_qspan(W), w4_sspan(W), {out_scale, 4},
                           {residual, size_t(M) * W->N * 2}, {y, size_t(M) * W->N * 2}};
    for (const Span& o : others)
        if (overlap(WS, o)) return fail(FDEC_ERR_ALIAS, "the workspace overlaps an input or y");
    if (overlap({y, size_t(M) * W->N * 2}, {u, in_bytes})) return fail(FDEC_ERR_ALIAS, "y overlaps u");
    if (g_fail_launches.load()) return injected();
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint16_t* act = static_cast<uint16_t*>(ws);
    hipError_t e = launch_swiglu_act(g, u, ldgu, M, W->K, act, s);
    if (e == hipSuccess)
        e = launch_w4_gemm(act, W->K, W->qweight, W->scales, M, W->K, W->N, out_scale, residual, y, s);
    return hip_status(e, "swiglu gemm launch");
}

FDEC_API size_t fdec_fp4_gemv_workspace_bytes(int32_t M, int32_t K, int32_t N) {
    if (M < 1 || M > kMaxGemvRows || K <= 0 || K % 32 || N <= 0 || N % 8) return 0;
    return fp4_gemv_workspace_bytes(M, K, N);
}

FDEC_API int fdec_swiglu_fp4_gemv(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, const fdec_fp4* W,
                                  const float* out_scale, const fdec_bf16* residual, int32_t M, fdec_bf16* y,
                                  void* ws, size_t ws_bytes, fdec_stream stream) {
    const int st = check_fp4_gemv(g, u, ldgu, W, out_scale, residual, M, y, ws, ws_bytes, true);
    if (st != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_fp4_gemv(kSwiGLU, g, u, ldgu, W->qweight, W->scales, M, W->K, W->N, out_scale, residual,
                                      y, ws, nullptr, static_cast<hipStream_t>(stream)),
                      "fp4 gemv launch");
}

FDEC_API int fdec_fp4_gemv(const fdec_bf16* x, const fdec_fp4* W, const float* out_scale, const fdec_bf16* residual,
                           int32_t M, fdec_bf16* y, void* ws, size_t ws_bytes, fdec_stream stream) {
    if (!W) return fail(FDEC_ERR_NULL, "W is NULL");
    const int st = check_fp4_gemv(x, nullptr, W->K, W, out_scale, residual, M, y, ws, ws_bytes, false);
    if (st != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_fp4_gemv(kIdentity, x, nullptr, W->K, W->qweight, W->scales, M, W->K, W->N, out_scale,
                                      residual, y, ws, nullptr, static_cast<hipStream_t>(stream)),
                      "fp4 gemv launch");
}

namespace {
// The activation's per-tensor scale of the FP4-activation GEMVs: a device fp32, read by
// every workgroup, never written.
int check_act_scale(const float* act_scale, const fdec_bf16* y, int M, const fdec_fp4* W, const void* ws, size_t ws_bytes) {
    if (!act_scale) return fail(FDEC_ERR_NULL, "act_scale is required");
    if (!aligned4(act_scale)) return fail(FDEC_ERR_ALIGN, "act_scale must be 4-byte aligned");
    const Span A{act_scale, 4};
    if (overlap(A, {y, size_t(M) * W->N * 2}) || overlap(A, {ws, ws_bytes}))
        return fail(FDEC_ERR_ALIAS, "act_scale overlaps y or the workspace");
    return FDEC_OK;
}
}  // namespace

FDEC_API int fdec_swiglu_fp4a4_gemv(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, const fdec_fp4* W,
                                    const float* act_scale, const float* out_scale, const fdec_bf16* residual,
                                    int32_t M, fdec_bf16* y, void* ws, size_t ws_bytes, fdec_stream stream) {
    int st = check_fp4_gemv(g, u, ldgu, W, out_scale, residual, M, y, ws, ws_bytes, true);
    if (st != FDEC_OK) return st;
    if ((st = check_act_scale(act_scale, y, M, W, ws, ws_bytes)) != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_fp4_gemv(kSwiGLU, g, u, ldgu, W->qweight, W->scales, M, W->K, W->N, out_scale, residual,
                                      y, ws, act_scale, static_cast<hipStream_t>(stream)),
                      "fp4a4 gemv launch");
}

FDEC_API int fdec_fp4a4_gemv(const fdec_bf16* x, const fdec_fp4* W, const float* act_scale, const float* out_scale,
                             const fdec_bf16* residual, int32_t M, fdec_bf16* y, void* ws, size_t ws_bytes,
                             fdec_stream stream) {
    if (!W) return fail(FDEC_ERR_NULL, "W is NULL");
    int st = check_fp4_gemv(x, nullptr, W->K, W, out_scale, residual, M, y, ws, ws_bytes, false);
    if (st != FDEC_OK) return st;
    if ((st = check_act_scale(act_scale, y, M, W, ws, ws_bytes)) != FDEC_OK) return st;
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_fp4_gemv(kIdentity, x, nullptr, W->K, W->qweight, W->scales, M, W->K, W->N, out_scale,
                                      residual, y, ws, act_scale, static_cast<hipStream_t>(stream)),
                      "fp4a4 gemv launch");
}

FDEC_API int fdec_nvfp4_quantize(const fdec_bf16* x, int64_t ldx, int32_t M, int32_t K, const float* act_scale,
                                 uint32_t* codes, uint8_t* scales, fdec_stream stream) {
    if (M < 0 || K <= 0 || K % 16) return fail(FDEC_ERR_SHAPE, "M = %d, K = %d: M >= 0, K a positive multiple of 16", M, K);
    if (M == 0) return ok();
    if (!x || !act_scale || !codes || !scales) return fail(FDEC_ERR_NULL, "x, act_scale, codes and scales are required");
    if (ldx < K || ldx % 8) return fail(FDEC_ERR_SHAPE, "ldx = %lld must be >= K and a multiple of 8", (long long)ldx);
    if (!aligned16(x) || !aligned4(codes) || !aligned4(act_scale))
        return fail(FDEC_ERR_ALIGN, "x must be 16-byte aligned, codes and act_scale 4-byte aligned");
    const Span X{x, (size_t(M - 1) * ldx + K) * 2}, C{codes, size_t(M) * (K / 8) * 4}, S{scales, size_t(M) * (K / 16)},
        A{act_scale, 4};
    if (overlap(C, X) || overlap(C, A) || overlap(S, X) || overlap(S, A) || overlap(C, S))
        return fail(FDEC_ERR_ALIAS, "codes and scales may overlap nothing");
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_nvfp4_quantize(x, ldx, M, K, act_scale, codes, scales, static_cast<hipStream_t>(stream)),
                      "fp4 quantize launch");
}

FDEC_API int fdec_fp4_dequant(const fdec_fp4* W, float* w_out, fdec_stream stream) {
    int st = check_fp4(W);
    if (st != FDEC_OK) return st;
    if (!w_out) return fail(FDEC_ERR_NULL, "w_out is NULL");
    if (!aligned4(w_out)) return fail(FDEC_ERR_ALIGN, "w_out must be 4-byte aligned");
    const Span O{w_out, size_t(W->K) * W->N * 4};
    if (overlap(O, fp4_qspan(W)) || overlap(O, fp4_sspan(W))) return fail(FDEC_ERR_ALIAS, "w_out overlaps W");
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_fp4_dequant(W->qweight, W->scales, W->K, W->N, w_out, static_cast<hipStream_t>(stream)),
                      "fp4 dequant launch");
}

FDEC_API int fdec_w4_unpack(const fdec_w4* W, int8_t* q_out, fdec_stream stream) {
    int st = check_w4(W, "W");
    if (st != FDEC_OK) return st;
    if (!q_out) return fail(FDEC_ERR_NULL, "q_out is NULL");
    const Span Q{q_out, size_t(W->K) * W->N};
    if (overlap(Q, w4_qspan(W)) || overlap(Q, w4_sspan(W))) return fail(FDEC_ERR_ALIAS, "q_out overlaps W");
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_w4_unpack(W->qweight, W->K, W->N, q_out, static_cast<hipStream_t>(stream)),
                      "unpack launch");
}

FDEC_API int fdec_w4_dequant(const fdec_w4* W, float* w_out, fdec_stream stream) {
    int st = check_w4(W, "W");
    if (st != FDEC_OK) return st;
    if (!w_out) return fail(FDEC_ERR_NULL, "w_out is NULL");
    if (!aligned4(w_out)) return fail(FDEC_ERR_ALIGN, "w_out must be 4-byte aligned");
    const Span O{w_out, size_t(W->K) * W->N * 4};
    if (overlap(O, w4_qspan(W)) || overlap(O, w4_sspan(W))) return fail(FDEC_ERR_ALIAS, "w_out overlaps W");
    if (g_fail_launches.load()) return injected();
    return hip_status(launch_w4_dequant(W->qweight, W->scales, W->K, W->N, w_out, static_cast<hipStream_t>(stream)),
                      "dequant launch");
}

}  // extern "C"
