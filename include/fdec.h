/*
 * fdec.h -- fused decode-MLP kernels for AMD MI355X (gfx950): the C ABI.
 *
 * The library implements the memory-bound hot path of single-token decode in an
 * LLM's MLP half:
 *   - a residual add fused with RMSNorm, writing both the new residual and the
 *     normalised activations from one kernel;
 *   - a decode-batch (M = 1..64) GEMV over int4 group-quantised weights, with the
 *     SwiGLU activation silu(g) * u computed in the GEMV's prologue (the activation
 *     and the (M, K, N) broadcast product are never written to memory) and an fp32
 *     output scale (and optional residual add) folded into its epilogue;
 *   - the three-kernel layer add_rmsnorm -> gate_up GEMV -> SwiGLU-down GEMV, and a
 *     multi-layer chain captured once into a hipGraph and replayed with one call;
 *   - the unfused sequences the fused kernels replace, for comparison.
 *
 * Sources, cited by page title and section:
 *   [P1] "PyTorch Community Proposes Fusion Fix as Large Intermediate Buffers May
 *        Slow Single-Token Decoding in Quantized LLMs": a single-row matmul that the
 *        compiler turns into a broadcast multiply plus a reduction can materialise
 *        the fp32 (1, K, N) product (about 94 MB at K = 9216, N = 2560); the fix
 *        realises the small activation instead; the int4 case with a SwiGLU
 *        pre-operation is the one measured.
 *   [P3] "PyTorch folds NVFP4 output scaling into NVGEMM candidates for decode
 *        workloads": an output-scale multiplier held in a zero-dimensional fp32
 *        device tensor is applied inside the matmul; the fallback keeps the matmul
 *        and the multiply as separate launches.
 *   [P4] "09 - Operator fusion", section 5 "Technical explanation": reduction +
 *        elementwise fusion (RMSNorm), GEMM prologue fusion (dequantise int4 weights
 *        as they are loaded), GEMM epilogue fusion, horizontal fusion (gate_proj and
 *        up_proj as one gate_up matmul), the residual's two consumers (one kernel
 *        writes both outputs) and the three-kernel fused layer.
 *   [P5] "Kernel Fusion, torch.compile and CUDA Graphs, Measured": "Step 1" (SiLU
 *        and the Qwen2 RMSNorm), "Step 2: fusing them by hand in Triton" (the
 *        two-output add + RMSNorm, h rounded to bf16 first), "Step 3" (the down
 *        projection computing silu(g) * u while reading its weights), "Step 4: CUDA
 *        graphs and the decode step" (capture once, replay; fixed addresses; no host
 *        synchronisation inside the captured work).
 *
 * Conventions shared by every entry point
 *   Types.     bf16 tensors are passed as fdec_bf16 (the 16-bit pattern).  Streams
 *              are hipStream_t passed as void*; NULL is the legacy null stream.
 *   Layout.    Every matrix is row-major and densely packed unless a leading
 *              dimension is given.  int4 weights: see fdec_w4.
 *   Ownership. The caller owns every buffer, including workspaces, all in device
 *              memory.  The library allocates no device memory in any compute call.
 *              The only objects it owns are graph handles (fdec_graph), freed by
 *              fdec_graph_destroy.
 *   Async.     Every compute call only enqueues work on the given stream and
 *              returns; FDEC_OK means "validated and enqueued".  No call
 *              synchronises the host, so every call may be captured into a graph.
 *              A device-side fault surfaces at the caller's next synchronisation.
 *   Errors.    Functions return an fdec_status (0 = OK, negative = error).  All
 *              arguments are checked before any HIP call, so an invalid call enqueues
 *              nothing and leaves every output untouched.  A HIP runtime error after
 *              validation returns FDEC_ERR_HIP.  fdec_last_error() gives a
 *              thread-local message for the last failing call.  Nothing aborts,
 *              exits or throws across this ABI.
 *   Alignment. Every tensor pointer must be 16-byte aligned (128-bit loads and
 *              stores); out_scale must be 4-byte aligned.
 *   Aliasing.  Outputs must not overlap inputs, except where a parameter says so.
 *   Workspace. Entry points that reduce across workgroups take a workspace of at
 *              least the size their *_workspace_bytes query returns.  It holds the fp32
 *              partial sums of K slices, which a second kernel on the same stream sums;
 *              its contents need no initialisation.  One workspace serves one call at
 *              a time: calls that may run concurrently (different streams) need
 *              different workspaces.
 */
#ifndef FDEC_H
#define FDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define FDEC_API __attribute__((visibility("default")))
#else
#define FDEC_API
#endif

#define FDEC_ABI_VERSION 1

typedef uint16_t fdec_bf16;   /* bf16 bit pattern */
typedef void* fdec_stream;    /* hipStream_t */

typedef enum {
    FDEC_OK = 0,
    FDEC_ERR_NULL = -1,         /* a required pointer is NULL */
    FDEC_ERR_SHAPE = -2,        /* a size is out of range or not a required multiple */
    FDEC_ERR_ALIGN = -3,        /* a pointer or leading dimension is misaligned */
    FDEC_ERR_ALIAS = -4,        /* an output overlaps an input it may not overlap */
    FDEC_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required */
    FDEC_ERR_UNSUPPORTED = -6,  /* a valid request this library does not implement */
    FDEC_ERR_HIP = -7,          /* the HIP runtime reported an error */
    FDEC_ERR_ARG = -8           /* any other invalid argument (e.g. eps < 0) */
} fdec_status;

/*
 * int4 group-quantised weight matrix W [K, N] ([P1]; [P4] section 5, prologue fusion).
 *   qweight: uint32 [N][K/8], row-major (a linear layer's [out_features,
 *            in_features] orientation: the K values of one output column are
 *            contiguous).  Word (n, kb) holds the weights k = 8*kb + j, j = 0..7, of
 *            column n; weight j sits in bits [4j, 4j+4) as a two's-complement nibble
 *            (values -8..7, symmetric, no zero point).
 *   scales:  bf16 [K/128][N], row-major.  Scale (g, n) multiplies the weights
 *            k in [128 g, 128 g + 128) of column n:  W[k, n] = q[k, n] * s[k/128, n].
 *   Requirements: K a positive multiple of 128, N a positive multiple of 8.
 *   The struct itself lives in host memory; the two arrays in device memory.
 */
typedef struct {
    const uint32_t* qweight;
    const fdec_bf16* scales;
    int32_t K;
    int32_t N;
} fdec_w4;

FDEC_API int fdec_abi_version(void);
FDEC_API const char* fdec_status_str(int status);
FDEC_API const char* fdec_last_error(void);

/* Zero-fill a workspace on `stream` (a fill kernel, not a memset node, so it may be
 * captured).  ws may be NULL only if ws_bytes is 0.  ws must be 16-byte aligned.  No
 * entry point needs it (workspaces need no initialisation); it is kept for callers that
 * want a defined workspace content. */
FDEC_API int fdec_workspace_init(void* ws, size_t ws_bytes, fdec_stream stream);

/*
 * Fused residual add + RMSNorm, two outputs ([P5] Step 2; [P4] section 5: reduction +
 * elementwise, and one kernel writing both outputs of the residual).
 *   h = bf16(x + residual)                                   (the new residual)
 *   y = bf16(h * weight / sqrt(mean_H(h * h) + eps))          (computed in fp32)
 *   x, residual, h_out, y_out: bf16 [M][H];  weight: bf16 [H].
 *   M >= 0 (M == 0 enqueues nothing, and x, residual, h_out, y_out may then be NULL);
 *   8 <= H <= 16384, H % 8 == 0;  eps >= 0, finite.
 *   h_out may equal residual (in-place residual update); no other overlap allowed.
 */
FDEC_API int fdec_add_rmsnorm(const fdec_bf16* x, const fdec_bf16* residual,
                              const fdec_bf16* weight, float eps, int32_t M, int32_t H,
                              fdec_bf16* h_out, fdec_bf16* y_out, fdec_stream stream);

/*
 * SwiGLU-prologue int4 GEMV with a folded fp32 output scale ([P1]; [P3]; [P5] Step 3).
 *   y[m, n] = bf16( s * sum_k silu(g[m,k]) * u[m,k] * W[k, n]  (+ residual[m, n]) )
 *   with s = *out_scale (a device fp32 scalar read when the kernel runs, so a value
 *   changed in device memory between graph replays takes effect), or 1 if out_scale
 *   is NULL; silu(v) = v / (1 + exp(-v)); one rounding to bf16 at the end.
 *   g, u:     bf16 [M][ldgu] (row m starts at m * ldgu elements; columns 0..K-1 used).
 *             g and u may point into one buffer (the two halves of a gate_up output).
 *   W:        K x N int4 weights (fdec_w4).
 *   residual: bf16 [M][N] or NULL.
 *   y:        bf16 [M][N].  May not overlap g, u, W or out_scale; may equal residual.
 *   1 <= M <= 64;  ldgu >= K, ldgu % 8 == 0.  17..64 rows run on the matrix cores as
 *   two or four blocks of 16 rows that share every weight load (W is read once).
 *   The activation silu(g) * u is formed in registers and is never written; the
 *   (M, K, N) product is never formed.
 *   ws: at least fdec_w4_gemv_workspace_bytes(M, K, N) bytes (see Workspace above).
 */
FDEC_API size_t fdec_w4_gemv_workspace_bytes(int32_t M, int32_t K, int32_t N);
FDEC_API int fdec_swiglu_w4_gemv(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu,
                                 const fdec_w4* W, const float* out_scale,
                                 const fdec_bf16* residual, int32_t M, fdec_bf16* y,
                                 void* ws, size_t ws_bytes, fdec_stream stream);

/*
 * fdec_swiglu_w4_gemv_noalloc: fdec_swiglu_w4_gemv for callers that cannot allocate
 * device memory or pass a workspace (code under graph capture that must not allocate,
 * tight serving loops, harnesses that forbid allocation).  Same arguments, results
 * (bit for bit: the same kernels and plan), checks and errors, without ws/ws_bytes: the
 * K-slice partial sums go to a static device array of FDEC_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that each GPU holds from the library's load until the process ends.  No
 * hipMalloc, hipFree or other allocation happens in the call.
 *   A shape whose plan needs more partial-sum space than the scratch holds returns
 *   FDEC_ERR_WORKSPACE (use fdec_swiglu_w4_gemv with a workspace).  The stream must
 *   belong to the current device.  The first call on a device that needs the scratch
 *   looks up its device address (hipGetSymbolAddress, once per device); make that first
 *   call outside graph capture.
 *   Every call on a GPU shares that GPU's one scratch: calls that may overlap in time on
 *   one GPU (different streams, or graphs replayed concurrently) race and must not be
 *   issued.  The kernels write every partial they read, so no clearing is needed.
 */
#define FDEC_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
FDEC_API int fdec_swiglu_w4_gemv_noalloc(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu,
                                         const fdec_w4* W, const float* out_scale,
                                         const fdec_bf16* residual, int32_t M, fdec_bf16* y,
                                         fdec_stream stream);

/*
 * The same GEMV with the identity prologue: y = bf16( s * x @ W ), s as above
 * (NULL = 1).  Used for the horizontally fused gate_up projection ([P4] section 5,
 * horizontal fusion), whose columns [0, I) are gate_proj and [I, 2I) up_proj.
 *   x: bf16 [M][K];  y: bf16 [M][N], no overlap with x.  1 <= M <= 64 (row blocks as
 *   above).
 */
FDEC_API int fdec_w4_gemv(const fdec_bf16* x, const fdec_w4* W, const float* out_scale,
                          int32_t M, fdec_bf16* y, void* ws, size_t ws_bytes,
                          fdec_stream stream);

/*
 * One decode-MLP layer as three kernels ([P4] section 5, the fusion boundary
 * problem; [P5] Step 3):
 *   1. (residual, y_norm) = add_rmsnorm(x, residual, norm_weight, eps)   -- residual
 *      is updated in place to h = bf16(x + residual);
 *   2. gate_up = w4_gemv(y_norm, gate_up weights)            [M][2I], no scale;
 *   3. out = swiglu_w4_gemv(gate_up[:, :I], gate_up[:, I:], down weights,
 *            out_scale, residual_in_epilogue ? h : NULL).
 * With residual_in_epilogue == 0 the residual add is deferred to the next layer's
 * add_rmsnorm (out is then that layer's x).
 *   H = gate_up.K = down.N;  I = down.K;  gate_up.N = 2I.  1 <= M <= 16.
 *   x, residual, y_norm, out: bf16 [M][H];  gate_up: bf16 [M][2I].
 *   out may equal x (x is only read by step 1); no other overlap allowed.
 *   ws: at least fdec_mlp_workspace_bytes(M, H, I) bytes.
 */
typedef struct {
    const fdec_bf16* norm_weight;   /* bf16 [H] */
    float eps;
    fdec_w4 gate_up;                /* K = H, N = 2I */
    fdec_w4 down;                   /* K = I, N = H */
    const float* out_scale;         /* device fp32 scalar for step 3, or NULL (= 1) */
    int32_t residual_in_epilogue;   /* 1: out = h + MLP(y); 0: out = MLP(y) */
} fdec_mlp_layer;

FDEC_API size_t fdec_mlp_workspace_bytes(int32_t M, int32_t H, int32_t I);
FDEC_API int fdec_mlp_decode(const fdec_mlp_layer* layer, int32_t M, const fdec_bf16* x,
                             fdec_bf16* residual, fdec_bf16* y_norm, fdec_bf16* gate_up,
                             fdec_bf16* out, void* ws, size_t ws_bytes, fdec_stream stream);

/*
 * A chain of n_layers layers launched eagerly (3 kernels per layer).  Layer l reads
 * x (its input) and residual and writes out = x in place, so after the call x holds
 * the last layer's output and residual the last h.  Every layer must have
 * residual_in_epilogue == 0 except possibly the last.  All layers share H, I and M.
 */
FDEC_API int fdec_mlp_chain(const fdec_mlp_layer* layers, int32_t n_layers, int32_t M,
                            fdec_bf16* x, fdec_bf16* residual, fdec_bf16* y_norm,
                            fdec_bf16* gate_up, void* ws, size_t ws_bytes,
                            fdec_stream stream);

/*
 * The same chain captured once into a hipGraph ([P5] Step 4).  fdec_mlp_graph_create
 * captures the 3 * n_layers kernels on `stream` (which must not be the null stream)
 * and instantiates the graph; nothing runs during creation.  fdec_graph_launch
 * replays it with one call on any stream.  The graph keeps the raw pointers: the
 * caller keeps every buffer alive at the same address, and writes new inputs into x
 * and residual before each launch.  Scale values in device memory are read at each
 * replay.  The layer array is copied; it may be freed after creation.
 */
typedef struct fdec_graph_s* fdec_graph;
FDEC_API int fdec_mlp_graph_create(const fdec_mlp_layer* layers, int32_t n_layers,
                                   int32_t M, fdec_bf16* x, fdec_bf16* residual,
                                   fdec_bf16* y_norm, fdec_bf16* gate_up, void* ws,
                                   size_t ws_bytes, fdec_stream stream, fdec_graph* out);
FDEC_API int fdec_graph_launch(fdec_graph graph, fdec_stream stream);

/*
 * fdec_mlp_graph_update: re-points a graph made by fdec_mlp_graph_create at other
 * layers (weights, scales, norm weights, out_scale pointers, residual flags) and other
 * buffers (x, residual, y_norm, gate_up, ws), without a new instantiation.  [P5]
 * section "In the real world" describes this for llama.cpp: changed kernel parameters
 * are patched into the graph instead of capturing it again.  The chain is captured on
 * `stream` (not the null stream; nothing runs) and its kernel arguments are written
 * into the existing executable graph with hipGraphExecUpdate.
 *   Same argument checks as fdec_mlp_graph_create.  The update must keep the graph's
 *   launch shapes: the same form (three-kernel layers), n_layers, M, H and I, else
 *   FDEC_ERR_UNSUPPORTED and the graph is unchanged.  If HIP refuses the update, the
 *   call returns FDEC_ERR_UNSUPPORTED and the handle keeps replaying what it replayed
 *   before.  No launch of the graph may be pending when it is called (synchronise the
 *   stream it was launched on first).  The old buffers may be freed once it returns
 *   FDEC_OK.
 * fdec_mlp_graph_update2: the same for a graph made by fdec_mlp_graph_create2.
 */
FDEC_API int fdec_mlp_graph_update(fdec_graph graph, const fdec_mlp_layer* layers, int32_t n_layers,
                                   int32_t M, fdec_bf16* x, fdec_bf16* residual,
                                   fdec_bf16* y_norm, fdec_bf16* gate_up, void* ws,
                                   size_t ws_bytes, fdec_stream stream);
FDEC_API int fdec_graph_kernel_count(fdec_graph graph);
FDEC_API int fdec_graph_destroy(fdec_graph graph);

/*
 * The layer as two kernels: the other fusion placement of [P4] section 5 ("the fusion
 * boundary problem": the gate_up GEMM with a silu * up epilogue writing act, the
 * GEMM-with-prologue and reduction-with-consumer rows of its fusion list), taken one
 * step further by running the add + RMSNorm as that GEMM's prologue.
 *
 * fdec_add_rmsnorm_w4_gemv_swiglu: one kernel computing
 *     h   = bf16(x + residual)                                   -> h_out [M][H]
 *     y   = h * norm_weight / sqrt(mean_H(h^2) + eps)            (fp32, never written)
 *     g   = y @ dequant(gate_up)[:, :I],  u = y @ dequant(gate_up)[:, I:]   (fp32)
 *     act = bf16(silu(g) * u)                                    -> act_out [M][I]
 *   Every workgroup reads the whole rows of x and residual, so h_out may alias neither
 *   (nor any other input); act_out may not overlap anything.  H = gate_up.K,
 *   gate_up.N = 2I with I a multiple of 8.  Implemented for the column GEMV only
 *   (M <= 4 and H small enough for its register budget: H <= 16384 / ceil-pow2(M) and
 *   about I / 256 pairs per workgroup); otherwise FDEC_ERR_UNSUPPORTED.
 *
 * fdec_mlp_decode2: the layer of fdec_mlp_decode with SwiGLU as the gate_up GEMV's
 * epilogue (the gate/up pair is never written; act [M][I] is), same results up to the
 * roundings it leaves out.
 *   M <= 4, two kernels (y_norm is not written either):
 *     1. fdec_add_rmsnorm_w4_gemv_swiglu(x, residual) -> h (into ws), act;
 *     2. out = bf16(out_scale * act @ dequant(down) [+ h]); the same kernel copies h into
 *        residual, so afterwards residual = h as with fdec_mlp_decode.
 *     FDEC_ERR_UNSUPPORTED where either projection does not fit the column GEMV.
 *   5 <= M <= 16, three kernels (the matrix-core gate_up is split over K, so its
 *   workgroups cannot each normalise whole rows):
 *     1. fdec_add_rmsnorm(x, residual) -> residual = h (in place), y = bf16(...) into
 *        the first M * H * 2 bytes of ws;
 *     2. fdec_w4_gemv_swiglu(y, gate_up) -> act;
 *     3. out = bf16(out_scale * act @ dequant(down) [+ h]).
 *   act: bf16 [M][I] (caller-owned scratch).  out may equal x.  ws: at least
 *   fdec_mlp2_workspace_bytes(M, H, I) bytes.
 * fdec_mlp_chain2 / fdec_mlp_graph_create2: the chain of fdec_mlp_chain and
 * fdec_mlp_graph_create built from the two-kernel layer (2 * n_layers kernels).
 */
/*
 * fdec_w4_gemv_swiglu: the gate_up projection with SwiGLU as its epilogue ([P4]
 * section 5, "the fusion boundary problem": the gate_up GEMM with a silu * up epilogue
 * writing act; [P4] section 5, horizontal fusion: gate columns [0, I), up [I, 2I)):
 *     g = x @ dequant(gate_up)[:, :I],  u = x @ dequant(gate_up)[:, I:]   (fp32, never written)
 *     act = bf16(silu(g) * u)                                   -> act_out [M][I]
 *   x: bf16 [M][K] (K = gate_up.K);  gate_up.N = 2I, I a multiple of 8;  1 <= M <= 64.
 *   Matrix-core kernel; when K is split into slices the slices' fp32 sums go to ws and a
 *   second kernel adds them (in slice order) and applies the epilogue.  ws: at least
 *   fdec_w4_gemv_swiglu_workspace_bytes(M, K, I) bytes (0 when K is not split).
 *   act_out may not overlap x, the weights or ws.
 */
FDEC_API size_t fdec_w4_gemv_swiglu_workspace_bytes(int32_t M, int32_t K, int32_t I);
FDEC_API int fdec_w4_gemv_swiglu(const fdec_bf16* x, const fdec_w4* gate_up, int32_t M,
                                 fdec_bf16* act_out, void* ws, size_t ws_bytes,
                                 fdec_stream stream);

FDEC_API int fdec_add_rmsnorm_w4_gemv_swiglu(const fdec_bf16* x, const fdec_bf16* residual,
                                             const fdec_bf16* norm_weight, float eps,
                                             const fdec_w4* gate_up, int32_t M, fdec_bf16* h_out,
                                             fdec_bf16* act_out, fdec_stream stream);
FDEC_API size_t fdec_mlp2_workspace_bytes(int32_t M, int32_t H, int32_t I);
FDEC_API int fdec_mlp_decode2(const fdec_mlp_layer* layer, int32_t M, const fdec_bf16* x,
                              fdec_bf16* residual, fdec_bf16* act, fdec_bf16* out, void* ws,
                              size_t ws_bytes, fdec_stream stream);
FDEC_API int fdec_mlp_chain2(const fdec_mlp_layer* layers, int32_t n_layers, int32_t M,
                             fdec_bf16* x, fdec_bf16* residual, fdec_bf16* act, void* ws,
                             size_t ws_bytes, fdec_stream stream);
FDEC_API int fdec_mlp_graph_create2(const fdec_mlp_layer* layers, int32_t n_layers,
                                    int32_t M, fdec_bf16* x, fdec_bf16* residual,
                                    fdec_bf16* act, void* ws, size_t ws_bytes,
                                    fdec_stream stream, fdec_graph* out);
FDEC_API int fdec_mlp_graph_update2(fdec_graph graph, const fdec_mlp_layer* layers,
                                    int32_t n_layers, int32_t M, fdec_bf16* x,
                                    fdec_bf16* residual, fdec_bf16* act, void* ws,
                                    size_t ws_bytes, fdec_stream stream);

/*
 * Prefill sizes ([P5] "Kernel Fusion, torch.compile and CUDA Graphs, Measured": at a
 * 2,048-token prefill the MLP half is compute-bound and the fusion win shrinks).  A tiled
 * GEMM would recompute a fused SwiGLU prologue once per column tile, so at these sizes the
 * activation is formed once by its own elementwise kernel and the GEMM reads it as stored.
 *
 * fdec_swiglu: act[m][k] = bf16(silu(g[m][k]) * u[m][k]), one rounding ([P5] Step 1: the
 *   fused SwiGLU, 6 bytes per element).  g, u: bf16 [M][ldgu] (ldgu >= K, % 8 == 0);
 *   act: bf16 [M][K], K % 8 == 0; act may not overlap g or u.  M == 0 enqueues nothing.
 * fdec_w4_gemm: y = bf16(s * x @ dequant(W) (+ residual)), s = *out_scale or 1, for any
 *   number of rows 1 <= M <= 2^24 (matrix cores, bf16 operands: the int4 weights are exact
 *   in bf16 and x is used as stored; fp32 accumulation, the group scales applied to each
 *   group's fp32 sum).  x: bf16 [M][K];  y: bf16 [M][N], may equal residual, no other
 *   overlap.  No workspace.
 * fdec_swiglu_w4_gemm: fdec_swiglu into the workspace (act, M * K * 2 bytes =
 *   fdec_swiglu_w4_gemm_workspace_bytes(M, K)), then fdec_w4_gemm on it:
 *   y = bf16(s * bf16(silu(g) * u) @ dequant(W) (+ residual)).
 */
FDEC_API int fdec_swiglu(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu, int32_t M,
                         int32_t K, fdec_bf16* act, fdec_stream stream);
FDEC_API int fdec_w4_gemm(const fdec_bf16* x, const fdec_w4* W, const float* out_scale,
                          const fdec_bf16* residual, int32_t M, fdec_bf16* y,
                          fdec_stream stream);
FDEC_API size_t fdec_swiglu_w4_gemm_workspace_bytes(int32_t M, int32_t K);
FDEC_API int fdec_swiglu_w4_gemm(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu,
                                 const fdec_w4* W, const float* out_scale,
                                 const fdec_bf16* residual, int32_t M, fdec_bf16* y,
                                 void* ws, size_t ws_bytes, fdec_stream stream);

/*
 * FP4 weights: [P3] ("PyTorch folds NVFP4 output scaling into NVGEMM candidates for
 * decode workloads") restricts its fold to packed FP4 inputs with E4M3 1x16 block scales
 * and a zero-dimensional fp32 multiplier.  Read here as weight-only quantisation behind
 * the same SwiGLU (or identity) prologue: the activation stays the unrounded prologue
 * value, as on the int4 path.
 *   qweight: uint32 [N][K/8]; the E2M1 code of weight k = 8 kb + j of column n sits in
 *            bits [4j, 4j+4) of word (n, kb): bit 3 sign, bits 2..1 exponent (bias 1),
 *            bit 0 mantissa; values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives.
 *   scales:  E4M3 ('fn', no infinities) bytes [N][K/16]; byte (n, b) scales k in
 *            [16 b, 16 b + 16) of column n.  NaN scales are outside the contract.
 *   K % 32 == 0, N % 8 == 0; both arrays 16-byte aligned.
 *
 * fdec_swiglu_fp4_gemv: y[m, n] = bf16(s * sum_k silu(g[m,k]) u[m,k] w[k,n] (+ residual)),
 *   w = e2m1 * e4m3 block scale; arguments, aliasing and errors as fdec_swiglu_w4_gemv.
 *   Implemented for 3 <= M <= 64 with K % 128 == 0 (the matrix-core kernel, past 16
 *   rows with two or four 16-row blocks per weight load; its K slices use a workspace
 *   of fdec_fp4_gemv_workspace_bytes(M, K, N) bytes, 0 when not needed), and otherwise
 *   for M <= 4 with K <= 16384 (a chunk-owning VALU kernel, no workspace; always at
 *   M <= 2); FDEC_ERR_UNSUPPORTED otherwise, FDEC_ERR_SHAPE outside [1, 64].
 * fdec_fp4_gemv: the identity prologue, y = bf16(s * x @ w (+ residual)); x [M][K].
 * fdec_fp4_dequant: test hook; writes w as fp32 [K][N] (exact).
 */
typedef struct {
    const uint32_t* qweight;
    const uint8_t* scales;
    int32_t K, N;
} fdec_fp4;
FDEC_API size_t fdec_fp4_gemv_workspace_bytes(int32_t M, int32_t K, int32_t N);
FDEC_API int fdec_swiglu_fp4_gemv(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu,
                                  const fdec_fp4* W, const float* out_scale,
                                  const fdec_bf16* residual, int32_t M, fdec_bf16* y,
                                  void* ws, size_t ws_bytes, fdec_stream stream);
FDEC_API int fdec_fp4_gemv(const fdec_bf16* x, const fdec_fp4* W, const float* out_scale,
                           const fdec_bf16* residual, int32_t M, fdec_bf16* y, void* ws,
                           size_t ws_bytes, fdec_stream stream);
FDEC_API int fdec_fp4_dequant(const fdec_fp4* W, float* w_out, fdec_stream stream);

/*
 * FP4 activations as well ("PyTorch folds NVFP4 output scaling into NVGEMM candidates for
 * decode workloads": the scaled matmul takes packed FP4 for both of its inputs, each with
 * E4M3 1x16 block scales, and a zero-dimensional fp32 output multiplier).  The
 * activation is quantised while it is formed, with its per-tensor scale G (act_scale: a
 * device fp32 > 0, a calibrated constant), one E4M3 block scale per 16 values along K:
 *     s_b = e4m3(amax_b / (6 G)),   q_k = e2m1(x_k / (s_b G))   (q_k = 0 where s_b = 0),
 * each step an fp32 operation, both roundings to nearest with ties to the even code and
 * saturating (E4M3 at 448, E2M1 at 6).  The products use the exact values q_k s_b (G is
 * not applied: out_scale carries it, with the weights' per-tensor scale):
 *     y[m, n] = bf16(out_scale * sum_k q[m,k] s[m,k/16] w[k,n] (+ residual[m, n])).
 *
 * fdec_swiglu_fp4a4_gemv: act = silu(g) * u (fp32), quantised as above; arguments, shapes,
 *   kernels, workspace and errors as fdec_swiglu_fp4_gemv, plus act_scale (required,
 *   4-byte aligned, overlapping neither y nor the workspace).
 * fdec_fp4a4_gemv: the identity prologue (x [M][K] bf16).
 * fdec_nvfp4_quantize: test hook; the same quantisation of x [M][ldx] bf16 (K % 16 == 0,
 *   ldx >= K, ldx % 8 == 0, x 16-byte aligned): codes [M][K/8] words, the code of k =
 *   8 kb + j in bits [4j, 4j+4) of word (m, kb) (as the weights are packed); scales
 *   [M][K/16] E4M3 bytes.  codes and scales may overlap nothing.
 */
FDEC_API int fdec_swiglu_fp4a4_gemv(const fdec_bf16* g, const fdec_bf16* u, int64_t ldgu,
                                    const fdec_fp4* W, const float* act_scale,
                                    const float* out_scale, const fdec_bf16* residual, int32_t M,
                                    fdec_bf16* y, void* ws, size_t ws_bytes, fdec_stream stream);
FDEC_API int fdec_fp4a4_gemv(const fdec_bf16* x, const fdec_fp4* W, const float* act_scale,
                             const float* out_scale, const fdec_bf16* residual, int32_t M,
                             fdec_bf16* y, void* ws, size_t ws_bytes, fdec_stream stream);
FDEC_API int fdec_nvfp4_quantize(const fdec_bf16* x, int64_t ldx, int32_t M, int32_t K,
                                 const float* act_scale, uint32_t* codes, uint8_t* scales,
                                 fdec_stream stream);

/*
 * The unfused sequences the fused kernels replace, kept for comparison.
 *
 * FDEC_UNFUSED_PRODUCT ([P1], the materialised broadcast product; M == 1 only,
 *   since the decomposition applies to single-row matmuls):
 *   kernel 1 writes P[k, n] = act[k] * W[k, n] in fp32 ([1][K][N], the workspace);
 *   kernel 2 reduces P over k and writes z = bf16(sum) to y;
 *   kernel 3 applies the output scale in place: y = bf16(s * z)  ([P3] fallback);
 *   kernel 4 (only if residual != NULL): y = bf16(y + residual).
 *   Workspace: exactly M*K*N*4 bytes (94,371,840 at K = 9216, N = 2560).
 * FDEC_UNFUSED_ACT (eager SwiGLU as two kernels, [P5] Step 1, then the GEMV):
 *   kernel 1 t = bf16(silu(g)); kernel 2 act = bf16(t * u); kernel 3 z = bf16(act @ W)
 *   (the identity-prologue GEMV); kernel 4 y = bf16(s * z); kernel 5 the residual add.
 *   Workspace: 2*M*K*2 bytes for t and act, plus the GEMV workspace.
 * Arguments otherwise as fdec_swiglu_w4_gemv.
 */
typedef enum { FDEC_UNFUSED_PRODUCT = 0, FDEC_UNFUSED_ACT = 1 } fdec_unfused_mode;
FDEC_API size_t fdec_unfused_gemv_workspace_bytes(int32_t mode, int32_t M, int32_t K,
                                                  int32_t N);
FDEC_API int fdec_unfused_swiglu_w4_gemv(int32_t mode, const fdec_bf16* g,
                                         const fdec_bf16* u, int64_t ldgu,
                                         const fdec_w4* W, const float* out_scale,
                                         const fdec_bf16* residual, int32_t M,
                                         fdec_bf16* y, void* ws, size_t ws_bytes,
                                         fdec_stream stream);

/*
 * Residual add + RMSNorm as nine eager kernels, the way the Qwen2 model code spells
 * it ([P5] Step 1): h = bf16(x + r); f = fp32(h); sq = f * f; ms = mean(sq);
 * v = ms + eps; rstd = rsqrt(v); t = f * rstd; tb = bf16(t); y = bf16(tb * weight).
 * 42 bytes per element.  Arguments as fdec_add_rmsnorm plus a workspace of
 * fdec_unfused_add_rmsnorm_workspace_bytes(M, H) bytes for the fp32 intermediates.
 */
FDEC_API size_t fdec_unfused_add_rmsnorm_workspace_bytes(int32_t M, int32_t H);
FDEC_API int fdec_unfused_add_rmsnorm(const fdec_bf16* x, const fdec_bf16* residual,
                                      const fdec_bf16* weight, float eps, int32_t M,
                                      int32_t H, fdec_bf16* h_out, fdec_bf16* y_out,
                                      void* ws, size_t ws_bytes, fdec_stream stream);

/*
 * The layer as the unfused sequence: the nine-kernel norm, the gate_up GEMV, the
 * ACT-mode SwiGLU-down sequence (silu, mul, GEMV, scale, residual add).  Arguments
 * and outputs as fdec_mlp_decode; workspace fdec_unfused_mlp_workspace_bytes(M, H, I).
 */
FDEC_API size_t fdec_unfused_mlp_workspace_bytes(int32_t M, int32_t H, int32_t I);
FDEC_API int fdec_unfused_mlp_decode(const fdec_mlp_layer* layer, int32_t M,
                                     const fdec_bf16* x, fdec_bf16* residual,
                                     fdec_bf16* y_norm, fdec_bf16* gate_up,
                                     fdec_bf16* out, void* ws, size_t ws_bytes,
                                     fdec_stream stream);

/*
 * Test hooks: run the in-register int4 decode on the whole matrix and write the result
 * ([P4] section 5, prologue fusion).  The column, split-K and matrix-core GEMV kernels
 * all decode with this one routine (packed word -> fp16 values that keep a known
 * offset); the hooks run it and remove the offsets.  q_out: int8 [K][N] (the integer
 * weights); w_out: fp32 [K][N] (q * scale, exact).  Output may not overlap W.
 */
FDEC_API int fdec_w4_unpack(const fdec_w4* W, int8_t* q_out, fdec_stream stream);
FDEC_API int fdec_w4_dequant(const fdec_w4* W, float* w_out, fdec_stream stream);

/* Test, tuning and measurement controls are declared in fdec_test.h (not for production
 * use). */

#ifdef __cplusplus
}
#endif
#endif /* FDEC_H */
