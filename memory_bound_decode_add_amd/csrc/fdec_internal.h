// Internal declarations shared by the host library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fdec.h"
#include "../../include/fdec_test.h"

namespace fdec {

// The int4 GEMV has three kernels.
//  * Column-owning (M <= 4, K <= 16384): each wave owns whole output columns over the
//    full K, each workgroup stages the activation of the full K once in LDS; no
//    cross-workgroup reduction and no workspace.
//  * Split-K (any M <= 16, any K): a 256-thread workgroup owns a 64-column tile and a
//    slice of K; a second kernel sums the slices.
constexpr int kGemvThreads = 256;
constexpr int kGemvCols = 64;
constexpr int kGroup = 128;
constexpr int kColMaxTasks = 8;      // activation tasks (row, 512-wide block) per wave, column kernel
constexpr int kColMaxTasksNorm = 4;  // the same with the add + RMSNorm prologue (three loads per task)
constexpr int kColMaxWaves = 14;     // dot waves per workgroup, column kernel (with the staging waves, 16 at most)
constexpr int kColMaxChunks = 8;
constexpr int kColScLoads = 4;       // 16-byte scale loads per thread, column kernel     // 32-wide K chunks per lane, column kernel
constexpr size_t kMaxLds = 160 * 1024;
constexpr int kFinishBatch = 16;     // K slices a finish kernel requests at once

enum GemvKind { kColumnOwning = 0, kSplitK = 1, kMfma = 2, kKMfma = 3, kRing = 4 };
constexpr int kMfmaWaves = 8;       // waves per workgroup, matrix-core kernel
constexpr int kMfmaMaxSliceGroups = 36;   // 128-wide groups per K slice at 16 rows (LDS: 4 KB each)
constexpr int kMfmaMaxRows = 64;          // four row blocks of 16

struct GemvPlan {
    int kind;
    int mr;           // rows the kernel is compiled for
    int groups;       // K / 128
    // column-owning kernel
    int waves;        // waves per workgroup
    int cpw;          // most columns any wave owns (1..4)
    int cols;         // columns per workgroup
    int stagers;      // staging waves per workgroup
    int ni;           // 32-wide K chunks per lane
    int wgs;          // workgroups
    // split-K kernel (the matrix-core kernel reuses tiles = column ranges, gps = groups
    // per K slice, splits, cpw = 16-column tiles per wave, waves)
    int tiles;        // ceil(N / 64)
    int gw;           // groups per wave (1, 2 or 4)
    int gps;          // groups per split = 4 * gw
    int splits;       // ceil(groups / gps)
    size_t partial_bytes;   // fp32 partial sums of the K slices (0 when splits == 1)
    size_t lds_bytes;       // dynamic LDS per workgroup
};

// Test/tuning overrides of the GEMV plan (include/fdec_test.h).  Every compute call
// takes one snapshot at entry and plans, checks and launches with it.
struct Overrides {
    int split = 0;        // fdec_set_gemv_split
    int col_waves = 0;    // fdec_set_gemv_tiling
    int col_cols = 0;
    int mfma_kernel = 0;  // fdec_set_mfma_plan
    int mfma_tiles = 0;
    int mfma_gw = 0;
    int mfma_waves = 0;   // fdec_set_kmfma_waves
};
Overrides current_overrides();


// kAddRmsNorm: the activation is rmsnorm(x + r) * w over the whole row (the fused
// layer's gate_up), and the epilogue writes silu(gate) * up of column pairs (i, I + i).
enum Prologue { kIdentity = 0, kSwiGLU = 1, kAddRmsNorm = 2 };
bool plan_mfma(int M, int K, int N, GemvPlan& p, int min_rows = 5);   // min_rows <= M <= 64
// The gate_up projection [K, 2I] with the SwiGLU epilogue: act[m][i] = bf16(silu(g) u)
// from the unrounded sums of columns i and I + i (matrix-core kernel, 1 <= M <= 64).
bool plan_mfma_pair(int M, int K, int I, GemvPlan& p);
// The matrix-core kernel whose waves split K (5..16 rows).  max_gw: most 128-wide groups
// per wave (at most 2 with the SwiGLU prologue).
bool plan_kmfma(int M, int K, int N, int max_gw, GemvPlan& p, const Overrides& ov = Overrides{});
// The pair plan GEMVs run: plan_mfma_pair, or the ring kernel's when chosen (5..16 rows).
bool plan_pair(int M, int K, int I, const Overrides& ov, GemvPlan& p);
// Launches a pair plan of either kind.  xs / xesc: x already staged (launch_add_rmsnorm_staged's
// layout), which the row-block kernel copies instead of staging x itself; the ring
// kernel ignores them.
hipError_t launch_mfma_pair(const uint16_t* x, const uint32_t* qw, const uint16_t* sc, int M, int K, int I,
                            uint16_t* act, void* ws, const GemvPlan& p, hipStream_t s, const void* xs = nullptr,
                            const float* xesc = nullptr);
// act[m][i] = bf16(silu(g) * u) from the K slices' fp32 partials of the pairs' gate and
// up columns (P pairs per column range: gate at range * 2P + i % P, up P further).
hipError_t launch_splitk_finish_swiglu(const float* partial, int splits, int64_t split_stride, int64_t row_stride,
                                       int M, int I, int P, uint16_t* act, hipStream_t s);
// The matrix-core kernel fed by direct-to-LDS loads of every operand (5..16 rows; pair
// mode with the identity prologue).
bool plan_ring(int M, int K, int N, Prologue pro, GemvPlan& p);
bool plan_ring_pair(int M, int K, int I, GemvPlan& p);
hipError_t launch_ring(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda, const uint32_t* qw,
                       const uint16_t* sc, int M, int K, int N, const float* out_scale, const uint16_t* residual,
                       uint16_t* y, void* ws, const GemvPlan& p, hipStream_t s);
hipError_t launch_ring_pair(const uint16_t* x, const uint32_t* qw, const uint16_t* sc, int M, int K, int I,
                            uint16_t* act, void* ws, const GemvPlan& p, hipStream_t s);
// Sums the fp32 partials of K slices (slice j of row m at partial + j * split_stride +
// m * row_stride) in slice order and applies the epilogue; launched after the kernel
// that wrote them, on the same stream.
hipError_t launch_splitk_finish(const float* partial, int splits, int64_t split_stride, int64_t row_stride, int M,
                                int N, const float* out_scale, const uint16_t* residual, uint16_t* y, hipStream_t s);
// the larger workspace of the two prologues' built-in plans (no overrides)
size_t gemv_workspace_bytes(int M, int K, int N);

// The plan of a GEMV with prologue pro (kSwiGLU or kIdentity; the matrix-core kernel whose
// waves split K holds fewer groups per wave with the SwiGLU prologue's raw g and u).
GemvPlan plan_gemv(int M, int K, int N, const Overrides& ov, Prologue pro);
hipError_t launch_kmfma(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda, const uint32_t* qw,
                        const uint16_t* sc, int M, int K, int N, const float* out_scale, const uint16_t* residual,
                        uint16_t* y, void* ws, const GemvPlan& p, hipStream_t s);

// Launchers: arguments are validated by the caller; they return the HIP error of the
// launch (hipSuccess on success).
hipError_t launch_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w,
                              float eps, int M, int H, uint16_t* h, uint16_t* y,
                              hipStream_t s);
// The same, also writing y staged for the matrix-core GEMVs (H % 128 == 0): ys [M][H/8]
// 16-byte k-blocks of block-scaled fp16 in pair order, yesc [M][H/128] powers of two.
hipError_t launch_add_rmsnorm_staged(const uint16_t* x, const uint16_t* r, const uint16_t* w, float eps, int M,
                                     int H, uint16_t* h, uint16_t* y, void* ys, float* yesc, hipStream_t s);
// Launches plan p, which the caller made with plan_gemv(M, K, N, ...) and checked ws for.
// xs / xesc: with the identity prologue, a0 already staged (launch_add_rmsnorm_staged's
// layout), which a row-block plan at 5..16 rows copies instead of staging a0 itself;
// other plans ignore them.
hipError_t launch_gemv(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda,
                       const uint32_t* qw, const uint16_t* sc, int M, int K, int N,
                       const float* out_scale, const uint16_t* residual, uint16_t* y,
                       void* ws, const GemvPlan& p, hipStream_t s, const void* xs = nullptr,
                       const float* xesc = nullptr);
// The fused layer's two kernels (column kernel only).
bool norm_gemv_swiglu_supported(int M, int K, int I);
hipError_t launch_norm_gemv_swiglu(const uint16_t* x, const uint16_t* r, const uint16_t* nw, float eps,
                                   const uint32_t* qw, const uint16_t* sc, int M, int K, int I,
                                   uint16_t* h_out, uint16_t* act, hipStream_t s);
bool gemv_column_supported(int M, int K, int N, const Overrides& ov);
hipError_t launch_gemv_copy(Prologue pro, const uint16_t* a0, int64_t lda, const uint32_t* qw, const uint16_t* sc,
                            int M, int K, int N, const float* out_scale, const uint16_t* residual, uint16_t* y,
                            const void* cp_src, void* cp_dst, size_t cp_bytes, const Overrides& ov, hipStream_t s);
hipError_t launch_mfma(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda,
                       const uint32_t* qw, const uint16_t* sc, int M, int K, int N,
                       const float* out_scale, const uint16_t* residual, uint16_t* y,
                       void* ws, const GemvPlan& p, hipStream_t s, const void* xs = nullptr,
                       const float* xesc = nullptr);
// FP4 (E2M1) weights with E4M3 1x16 block scales: M = 1..4 (K % 32 == 0, K <= 16384)
// on the chunk-owning kernel, M = 5..64 (K % 128 == 0) on the matrix-core kernel.  With
// gscale (the activation's per-tensor scale, device fp32) the activation is quantised to
// FP4 as well (both operands FP4); NULL keeps it unquantised.
bool fp4_gemv_supported(int M, int K, int N);
size_t fp4_gemv_workspace_bytes(int M, int K, int N);
hipError_t launch_fp4_gemv(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda, const uint32_t* qw,
                           const uint8_t* sc, int M, int K, int N, const float* out_scale, const uint16_t* residual,
                           uint16_t* y, void* ws, const float* gscale, hipStream_t s);
hipError_t launch_mfma_fp4(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda,
                           const uint32_t* qw, const uint8_t* sc8, int M, int K, int N,
                           const float* out_scale, const uint16_t* residual, uint16_t* y,
                           void* ws, const GemvPlan& p, const float* gscale, hipStream_t s);
// Test hook: FP4 quantisation of a bf16 activation x [M][ldx] (K % 16 == 0): codes
// [M][K/8] packed words, E4M3 scale codes [M][K/16].
hipError_t launch_nvfp4_quantize(const uint16_t* x, int64_t ldx, int M, int K, const float* gscale, uint32_t* codes,
                                 uint8_t* scales, hipStream_t s);
hipError_t launch_fp4_dequant(const uint32_t* qw, const uint8_t* sc, int K, int N, float* w, hipStream_t s);
hipError_t launch_w4_unpack(const uint32_t* qw, int K, int N, int8_t* q, hipStream_t s);
hipError_t launch_w4_dequant(const uint32_t* qw, const uint16_t* sc, int K, int N,
                             float* w, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

// unfused sequences
hipError_t launch_unfused_product(const uint16_t* g, const uint16_t* u, const uint32_t* qw,
                                  const uint16_t* sc, int K, int N, const float* out_scale,
                                  const uint16_t* residual, uint16_t* y, float* P,
                                  hipStream_t s);
hipError_t launch_silu_bf16(const uint16_t* g, int64_t ldg, int M, int K, uint16_t* t,
                            hipStream_t s);
hipError_t launch_mul_bf16(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb,
                           int M, int K, uint16_t* out, hipStream_t s);
hipError_t launch_scale_bf16(uint16_t* y, int64_t n, const float* out_scale, hipStream_t s);
hipError_t launch_add_bf16(uint16_t* y, const uint16_t* r, int64_t n, hipStream_t s);
hipError_t launch_eager_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w,
                                float eps, int M, int H, uint16_t* h, uint16_t* y,
                                float* f32a, float* f32b, float* rowbuf, hipStream_t s);

// Prefill-sized GEMM (any M, bf16 activation as stored) and the fused SwiGLU elementwise
// kernel that precedes it at prefill sizes.
size_t w4_gemm_lds_bytes();
hipError_t launch_w4_gemm(const uint16_t* x, int64_t lda, const uint32_t* qw, const uint16_t* sc, int M, int K, int N,
                          const float* out_scale, const uint16_t* residual, uint16_t* y, hipStream_t s);
hipError_t launch_swiglu_act(const uint16_t* g, const uint16_t* u, int64_t ldgu, int M, int K, uint16_t* act,
                             hipStream_t s);
// measurement probes
hipError_t launch_empty(int wgs, int threads, hipStream_t s);
bool read_ceiling_fits(int per_wg, int bcast16, int rows, int piece_bytes);
hipError_t launch_read_ceiling(const void* stream_buf, int per_wg, const void* b0, const void* b1, int bcast16,
                               const void* pieces, int rows, int row_bytes, int piece_bytes, int wgs,
                               uint32_t* sink, hipStream_t s);

}  // namespace fdec
