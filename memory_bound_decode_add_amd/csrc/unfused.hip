// The unfused sequences the fused kernels replace (comparison only).
//
// * Materialised product ("PyTorch Community Proposes Fusion Fix as Large
//   Intermediate Buffers May Slow Single-Token Decoding in Quantized LLMs"): for a
//   single-row matmul the broadcast product P[k, n] = act[k] * W[k, n] is written in
//   fp32, then reduced over k; the output scale is a separate launch ("PyTorch folds
//   NVFP4 output scaling into NVGEMM candidates for decode workloads", fallback).
//   The reduction is split in two launches; the first writes each chunk's partial
//   sums over the first row of the chunk it has just read, so no memory beyond the
//   product buffer is needed.
// * Eager SwiGLU as two kernels and the nine-kernel eager RMSNorm ("Kernel Fusion,
//   torch.compile and CUDA Graphs, Measured", Step 1), each kernel reading its inputs
//   from and writing its output to memory, with the same rounding points as the
//   eager sequence.
#include "device_common.h"
#include "fdec_internal.h"

#include <algorithm>

namespace fdec {
namespace {

constexpr int kProdChunk = 256;   // rows of P per first-level reduction workgroup

inline dim3 grid_for(int64_t n, int per_block = 256) {
    return dim3(unsigned((n + per_block - 1) / per_block));
}

// P[8kb + j][n] = act[8kb + j] * q * scale, fp32
__global__ void product_kernel(const uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
                               const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                               int KB, int N, float* __restrict__ P, DecodeMasks dm) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= int64_t(KB) * N) return;
    const int kb = int(i / N), n = int(i % N);
    const uint4 gv = *reinterpret_cast<const uint4*>(g + int64_t(kb) * 8);
    const uint4 uv = *reinterpret_cast<const uint4*>(u + int64_t(kb) * 8);
    const uint32_t ga[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t ua[4] = {uv.x, uv.y, uv.z, uv.w};
    float act[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        act[2 * j] = silu_f32(bf16_lo(ga[j])) * bf16_lo(ua[j]);
        act[2 * j + 1] = silu_f32(bf16_hi(ga[j])) * bf16_hi(ua[j]);
    }
    const Q4x2 d = decode_int4x8(qw[int64_t(n) * KB + kb], dm);      // word (n, kb) of [N][K/8]
    const half2_t p[4] = {d.p04, d.p15, d.p26, d.p37};
    const float s = bf16_to_f32(sc[int64_t(kb / 16) * N + n]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const _Float16 q = (j < 4) ? p[j][0] : p[j - 4][1];
        P[(int64_t(kb) * 8 + j) * N + n] = act[j] * (float(q) * s);
    }
}

// First-level reduction: workgroup (tile of 64 columns, chunk of kProdChunk rows).
__global__ __launch_bounds__(256) void product_reduce1_kernel(float* P, int K, int N) {
    __shared__ float4 red[4][16];
    const int tiles = (N + 63) / 64;
    const int tile = blockIdx.x % tiles, chunk = blockIdx.x / tiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cq = lane & 15, rl = (lane >> 4) + 4 * wave;   // 16 row lanes
    const int col = tile * 64 + cq * 4;
    const int k0 = chunk * kProdChunk;
    const int k1 = min(K, k0 + kProdChunk);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (col < N) {
        for (int k = k0 + rl; k < k1; k += 16) {
            const float4 v = *reinterpret_cast<const float4*>(P + int64_t(k) * N + col);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
        acc.x += __shfl_xor(acc.x, o, kWave);
        acc.y += __shfl_xor(acc.y, o, kWave);
        acc.z += __shfl_xor(acc.z, o, kWave);
        acc.w += __shfl_xor(acc.w, o, kWave);
    }
    if ((lane >> 4) == 0) red[wave][cq] = acc;
    __syncthreads();
    if (threadIdx.x < 16 && tile * 64 + threadIdx.x * 4 < N) {
        float4 t = red[0][threadIdx.x];
        for (int w = 1; w < 4; ++w) {
            const float4 v = red[w][threadIdx.x];
            t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
        }
        *reinterpret_cast<float4*>(P + int64_t(k0) * N + tile * 64 + threadIdx.x * 4) = t;
    }
}

// Second level: z[n] = bf16(sum over chunks of P[chunk * kProdChunk][n]).
__global__ void product_reduce2_kernel(const float* __restrict__ P, int K, int N, uint16_t* __restrict__ z) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float t = 0.f;
    for (int k = 0; k < K; k += kProdChunk) t += P[int64_t(k) * N + n];
    z[n] = f32_to_bf16(t);
}

// t = bf16(silu(g)) over [M][K] (g row stride ldg), 8 elements per thread
__global__ void silu_kernel(const uint16_t* __restrict__ g, int64_t ldg, int M, int K, uint16_t* __restrict__ t) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int cpr = K / 8;
    if (i >= int64_t(M) * cpr) return;
    const int m = int(i / cpr), c = int(i % cpr);
    const uint4 v = *reinterpret_cast<const uint4*>(g + m * ldg + c * 8);
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(silu_f32(bf16_lo(a[j])), silu_f32(bf16_hi(a[j])));
    *reinterpret_cast<uint4*>(t + int64_t(m) * K + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

// out = bf16(a * b) over [M][K]
__global__ void mul_kernel(const uint16_t* __restrict__ a, int64_t lda, const uint16_t* __restrict__ b,
                           int64_t ldb, int M, int K, uint16_t* __restrict__ out) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int cpr = K / 8;
    if (i >= int64_t(M) * cpr) return;
    const int m = int(i / cpr), c = int(i % cpr);
    const uint4 va = *reinterpret_cast<const uint4*>(a + m * lda + c * 8);
    const uint4 vb = *reinterpret_cast<const uint4*>(b + m * ldb + c * 8);
    const uint32_t x[4] = {va.x, va.y, va.z, va.w};
    const uint32_t y[4] = {vb.x, vb.y, vb.z, vb.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(bf16_lo(x[j]) * bf16_lo(y[j]), bf16_hi(x[j]) * bf16_hi(y[j]));
    *reinterpret_cast<uint4*>(out + int64_t(m) * K + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

// y = bf16(s * y) in place (n multiple of 8)
__global__ void scale_kernel(uint16_t* y, int64_t n, const float* out_scale) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n / 8) return;
    const float s = out_scale ? *out_scale : 1.0f;
    uint4 v = reinterpret_cast<uint4*>(y)[i];
    uint32_t a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = pack_bf16x2(s * bf16_lo(a[j]), s * bf16_hi(a[j]));
    reinterpret_cast<uint4*>(y)[i] = make_uint4(a[0], a[1], a[2], a[3]);
}

// y = bf16(y + r) in place
__global__ void add_kernel(uint16_t* y, const uint16_t* __restrict__ r, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n / 8) return;
    uint4 v = reinterpret_cast<uint4*>(y)[i];
    const uint4 w = reinterpret_cast<const uint4*>(r)[i];
    uint32_t a[4] = {v.x, v.y, v.z, v.w};
    const uint32_t b[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = pack_bf16x2(bf16_lo(a[j]) + bf16_lo(b[j]), bf16_hi(a[j]) + bf16_hi(b[j]));
    reinterpret_cast<uint4*>(y)[i] = make_uint4(a[0], a[1], a[2], a[3]);
}

// ---- the nine eager RMSNorm kernels ----
// 1: h = bf16(x + r) (add_kernel pattern, out of place)
__global__ void eager_add_kernel(const uint16_t* __restrict__ x, const uint16_t* r, uint16_t* h, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n / 8) return;
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint4 w = reinterpret_cast<const uint4*>(r)[i];
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};
    const uint32_t b[4] = {w.x, w.y, w.z, w.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(bf16_lo(a[j]) + bf16_lo(b[j]), bf16_hi(a[j]) + bf16_hi(b[j]));
    reinterpret_cast<uint4*>(h)[i] = make_uint4(o[0], o[1], o[2], o[3]);
}
// 2: f = fp32(h)
__global__ void eager_to_f32_kernel(const uint16_t* __restrict__ h, float* __restrict__ f, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n / 8) return;
    const uint4 v = reinterpret_cast<const uint4*>(h)[i];
    float4* o = reinterpret_cast<float4*>(f) + 2 * i;
    o[0] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
    o[1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
}
// 3: sq = f * f
__global__ void eager_square_kernel(const float* __restrict__ f, float* __restrict__ sq, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n / 4) return;
    const float4 v = reinterpret_cast<const float4*>(f)[i];
    reinterpret_cast<float4*>(sq)[i] = make_float4(v.x * v.x, v.y * v.y, v.z * v.z, v.w * v.w);
}
// 4: ms[m] = mean(sq[m, :]) -- one workgroup per row
__global__ __launch_bounds__(256) void eager_mean_kernel(const float* __restrict__ sq, int H, float* __restrict__ ms) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    float t = 0.f;
    for (int c = threadIdx.x; c < H / 4; c += 256) {
        const float4 v = reinterpret_cast<const float4*>(sq + int64_t(m) * H)[c];
        t += (v.x + v.y) + (v.z + v.w);
    }
    t = wave_sum(t);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
    __syncthreads();
    if (threadIdx.x == 0) ms[m] = (red[0] + red[1] + red[2] + red[3]) / float(H);
}
// 5: v = ms + eps ; 6: rstd = rsqrt(v)
__global__ void eager_add_eps_kernel(const float* __restrict__ ms, float eps, float* __restrict__ v, int M) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < M) v[i] = ms[i] + eps;
}
__global__ void eager_rsqrt_kernel(const float* __restrict__ v, float* __restrict__ r, int M) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < M) r[i] = __builtin_amdgcn_rsqf(v[i]);
}
// 7: t = f * rstd[row]
__global__ void eager_mul_row_kernel(const float* __restrict__ f, const float* __restrict__ rstd, int H,
                                     float* __restrict__ t, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n / 4) return;
    const float s = rstd[(i * 4) / H];
    const float4 v = reinterpret_cast<const float4*>(f)[i];
    reinterpret_cast<float4*>(t)[i] = make_float4(v.x * s, v.y * s, v.z * s, v.w * s);
}
// 8: tb = bf16(t)
__global__ void eager_to_bf16_kernel(const float* __restrict__ t, uint16_t* __restrict__ tb, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n / 8) return;
    const float4 a = reinterpret_cast<const float4*>(t)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(t)[2 * i + 1];
    reinterpret_cast<uint4*>(tb)[i] = make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w),
                                                 pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
}
// 9: y = bf16(tb * w[col]) in place
__global__ void eager_mul_weight_kernel(uint16_t* y, const uint16_t* __restrict__ w, int H, int64_t n) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n / 8) return;
    const int c = int((i * 8) % H) / 8;
    uint4 v = reinterpret_cast<uint4*>(y)[i];
    const uint4 wv = reinterpret_cast<const uint4*>(w)[c];
    uint32_t a[4] = {v.x, v.y, v.z, v.w};
    const uint32_t b[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = pack_bf16x2(bf16_lo(a[j]) * bf16_lo(b[j]), bf16_hi(a[j]) * bf16_hi(b[j]));
    reinterpret_cast<uint4*>(y)[i] = make_uint4(a[0], a[1], a[2], a[3]);
}

}  // namespace

hipError_t launch_unfused_product(const uint16_t* g, const uint16_t* u, const uint32_t* qw,
                                  const uint16_t* sc, int K, int N, const float* out_scale,
                                  const uint16_t* residual, uint16_t* y, float* P,
                                  hipStream_t s) {
    const int KB = K / 8;
    product_kernel<<<grid_for(int64_t(KB) * N), 256, 0, s>>>(g, u, qw, sc, KB, N, P,
                                                            DecodeMasks{kDecodeMaskLo, kDecodeMaskHi});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int tiles = (N + 63) / 64, chunks = (K + kProdChunk - 1) / kProdChunk;
    product_reduce1_kernel<<<dim3(tiles * chunks), 256, 0, s>>>(P, K, N);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    product_reduce2_kernel<<<grid_for(N), 256, 0, s>>>(P, K, N, y);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_scale_bf16(y, N, out_scale, s)) != hipSuccess) return e;
    if (residual) return launch_add_bf16(y, residual, N, s);
    return hipSuccess;
}

hipError_t launch_silu_bf16(const uint16_t* g, int64_t ldg, int M, int K, uint16_t* t, hipStream_t s) {
    silu_kernel<<<grid_for(int64_t(M) * (K / 8)), 256, 0, s>>>(g, ldg, M, K, t);
    return hipGetLastError();
}

hipError_t launch_mul_bf16(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, int M, int K,
                           uint16_t* out, hipStream_t s) {
    mul_kernel<<<grid_for(int64_t(M) * (K / 8)), 256, 0, s>>>(a, lda, b, ldb, M, K, out);
    return hipGetLastError();
}

hipError_t launch_scale_bf16(uint16_t* y, int64_t n, const float* out_scale, hipStream_t s) {
    scale_kernel<<<grid_for(n / 8), 256, 0, s>>>(y, n, out_scale);
    return hipGetLastError();
}

hipError_t launch_add_bf16(uint16_t* y, const uint16_t* r, int64_t n, hipStream_t s) {
    add_kernel<<<grid_for(n / 8), 256, 0, s>>>(y, r, n);
    return hipGetLastError();
}

hipError_t launch_eager_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w, float eps,
                                int M, int H, uint16_t* h, uint16_t* y, float* f32a, float* f32b,
                                float* rowbuf, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const int64_t n = int64_t(M) * H;
    float* ms = rowbuf;
    float* v = rowbuf + M;
    float* rstd = rowbuf + 2 * M;
    hipError_t e;
    eager_add_kernel<<<grid_for(n / 8), 256, 0, s>>>(x, r, h, n);                       // 1
    if ((e = hipGetLastError()) != hipSuccess) return e;
    eager_to_f32_kernel<<<grid_for(n / 8), 256, 0, s>>>(h, f32a, n);                   // 2
    if ((e = hipGetLastError()) != hipSuccess) return e;
    eager_square_kernel<<<grid_for(n / 4), 256, 0, s>>>(f32a, f32b, n);                // 3
    if ((e = hipGetLastError()) != hipSuccess) return e;
    eager_mean_kernel<<<dim3(M), 256, 0, s>>>(f32b, H, ms);                            // 4
    if ((e = hipGetLastError()) != hipSuccess) return e;
    eager_add_eps_kernel<<<grid_for(M), 256, 0, s>>>(ms, eps, v, M);                   // 5
    if ((e = hipGetLastError()) != hipSuccess) return e;
    eager_rsqrt_kernel<<<grid_for(M), 256, 0, s>>>(v, rstd, M);                        // 6
    if ((e = hipGetLastError()) != hipSuccess) return e;
    eager_mul_row_kernel<<<grid_for(n / 4), 256, 0, s>>>(f32a, rstd, H, f32b, n);      // 7
    if ((e = hipGetLastError()) != hipSuccess) return e;
    eager_to_bf16_kernel<<<grid_for(n / 8), 256, 0, s>>>(f32b, y, n);                  // 8
    if ((e = hipGetLastError()) != hipSuccess) return e;
    eager_mul_weight_kernel<<<grid_for(n / 8), 256, 0, s>>>(y, w, H, n);               // 9
    return hipGetLastError();
}

}  // namespace fdec
