// Internal declarations shared by the host library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fdec.h"

namespace fdec {

// Tile geometry of the int4 GEMV: a workgroup of 4 waves covers 64 columns; each
// wave covers whole 128-wide K groups of those columns.
constexpr int kGemvThreads = 256;
constexpr int kGemvCols = 64;
constexpr int kGroup = 128;

struct GemvPlan {
    int tiles;        // ceil(N / 64)
    int groups;       // K / 128
    int gw;           // groups per wave (1, 2 or 4)
    int gps;          // groups per split = 4 * gw
    int splits;       // ceil(groups / gps)
    int mr;           // rows the kernel is compiled for (1, 2, 4, 8, 16)
    size_t partial_bytes;   // splits * M * tiles * 64 * 4 (0 when splits == 1)
    size_t counter_bytes;   // tiles * 4, rounded up to 256 (0 when splits == 1)
    size_t lds_bytes;       // dynamic LDS per workgroup
};

GemvPlan plan_gemv(int M, int K, int N);
size_t gemv_workspace_bytes(int M, int K, int N);

enum Prologue { kIdentity = 0, kSwiGLU = 1 };

// Launchers: arguments are validated by the caller; they return the HIP error of the
// launch (hipSuccess on success).
hipError_t launch_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w,
                              float eps, int M, int H, uint16_t* h, uint16_t* y,
                              hipStream_t s);
hipError_t launch_gemv(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda,
                       const uint32_t* qw, const uint16_t* sc, int M, int K, int N,
                       const float* out_scale, const uint16_t* residual, uint16_t* y,
                       void* ws, hipStream_t s);
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

extern int g_forced_split;   // fdec_set_gemv_split

}  // namespace fdec
