// Prefill-sized int4 group-quantised GEMM on the matrix cores, gfx950, and the fused
// SwiGLU elementwise kernel that feeds it.
//
// At decode batches the SwiGLU activation is formed inside the GEMV's prologue ("Kernel
// Fusion, torch.compile and CUDA Graphs, Measured", Step 3).  At a prefill of 2,048
// tokens the same MLP half is compute-bound ("Kernel Fusion, torch.compile and CUDA
// Graphs, Measured": the fusion win shrinks there), and a tiled GEMM would recompute the
// prologue once per column tile.  So the prefill path is two kernels:
//     act = bf16(silu(g) * u)                  (one elementwise pass, one rounding; 6 bytes
//                                               per element, as the fused SwiGLU of Step 1)
//     y   = bf16(s * act @ dequant(W) (+ res)) (this GEMM; act is used as stored)
//
// GEMM tiling.  A workgroup of 8 waves (two per SIMD) computes a 128-row x 160-column tile of y (at
// M = 2048, N = 2560: 16 x 16 = 256 workgroups, one per CU), looping over K one 128-wide
// group at a time with two LDS buffers: while the matrix cores work on group g, the
// global loads of group g + 1 are in flight, and their values are then written to the
// other buffer.  Per group the workgroup stages
//   - the 128 x 128 bf16 activation block, each 8-value block stored in the int4 pair
//     order (e0, e4, e1, e5, e2, e6, e3, e7) -- four byte permutes per 16 bytes;
//   - the 160 x 128 weights, each packed word decoded once into eight exact bf16 values
//     136 + q in pair order: a 4-bit field of offset-binary q + 8 in the mantissa of bf16
//     128 (0x4300), field j of the word shifted to bits 0..3 and 16..19 (three shifts and
//     four v_bitop3_b32 per word);
//   - the group's 160 column scales.
// Wave (wr, wc), wr = 0..3, wc = 0..1, owns rows 32 wr .. 32 wr + 31 (2 row tiles of 16)
// and columns 80 wc .. 80 wc + 79 (5 column tiles); per group and k-step it reads its 2
// activation and 5 weight operands from LDS and issues 10 v_mfma_f32_16x16x32_bf16, plus one MFMA per
// row tile with a constant -136 operand that removes the weights' offset (shared by the
// 5 column tiles).  The group's fp32 sums are scaled by the group scale once and added to
// the running tile (fp32).  The epilogue applies the output scale and residual and rounds
// to bf16 once.  The MFMA operand layout is that of the GEMV kernels: lane l supplies
// A[l%16][8(l/16)+e] (weights, row = column n), B[8(l/16)+e][l%16] (activation, column =
// row m), and holds D[4(l/16)+r][l%16].  Two waves per SIMD (210 VGPRs each) hide each
// other's LDS latency: at 2048 x 9216 x 2560 this runs 12 % faster than 4 waves with
// 64 x 80 wave tiles (one wave per SIMD, 384 VGPRs), although it reads more from LDS.
#include "device_common.h"
#include "fdec_internal.h"

#include <algorithm>

namespace fdec {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGBM = 128;               // rows per workgroup
constexpr int kGBN = 160;               // columns per workgroup
constexpr int kGThreads = 512;          // 8 waves, 4 x 2, two per SIMD
constexpr int kGRowTiles = 2;           // per wave (32 rows)
constexpr int kGColTiles = 5;           // per wave (80 columns)
constexpr int kGActChunks = kGBM * 16 / kGThreads;                     // 16-byte pieces per thread: 4
constexpr int kGWChunks = (kGBN * 4 + kGThreads - 1) / kGThreads;      // 16-byte weight chunks: 2
constexpr int kGStride = 128 + 8;       // LDS row stride of a staged block, in bf16
constexpr size_t kGBufBytes = size_t(kGBM + kGBN) * kGStride * 2 + size_t(kGBN) * 4;
constexpr size_t kGLdsBytes = 2 * kGBufBytes;

struct GemmArgs {
    const uint16_t* x;      // bf16 [M][lda]
    int64_t lda;
    const uint4* qw;        // [N][K/32] chunks of 4 words
    const uint16_t* sc;     // bf16 scales [K/128][N]
    int M, N, nch, groups;
    int ntiles;             // column tiles of kGBN
    const float* out_scale;
    const uint16_t* residual;
    uint16_t* y;
    DecodeMasks dm;
};

// bf16 pairs of word w in pair order, 136 + q each: field j (nibbles j and j + 4) is the
// word shifted right by 4 j, masked to bits 0..3 of each half, XOR-ed into 0x4308 (the
// bits of 128 and the flip of the nibble's sign bit).
__device__ __forceinline__ uint4 decode_bf16x8_biased(uint32_t w, uint32_t mask) {
    const uint32_t k = 0x43084308u;
    return make_uint4(k ^ (w & mask), k ^ ((w >> 4) & mask), k ^ ((w >> 8) & mask), k ^ ((w >> 12) & mask));
}

// 8 bf16 in k order (e0 .. e7 in the dwords' halves) -> pair order (e0, e4), (e1, e5), ...
__device__ __forceinline__ uint4 to_pair_order(uint4 v) {
    // v_perm_b32 selector bytes: 0..3 pick from the second operand, 4..7 from the first
    return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),   // e0 = x.lo, e4 = z.lo
                      __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),   // e1 = x.hi, e5 = z.hi
                      __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),   // e2 = y.lo, e6 = w.lo
                      __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));  // e3 = y.hi, e7 = w.hi
}

__global__ __launch_bounds__(kGThreads) void w4_gemm_kernel(GemmArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ls = lane >> 4, lm = lane & 15;
    const int wr = wave >> 1, wc = wave & 1;
    // workgroups of one row block are consecutive on an XCD (they share its activation)
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = lb % a.ntiles, mt = lb / a.ntiles;
    const int m0 = mt * kGBM, n0 = nt * kGBN;

    auto act_s = [&](int b) { return reinterpret_cast<uint16_t*>(smem + b * kGBufBytes); };
    auto w_s = [&](int b) { return act_s(b) + kGBM * kGStride; };
    auto sc_s = [&](int b) { return reinterpret_cast<float*>(w_s(b) + kGBN * kGStride); };

    // ---- staging: global loads of group g into registers, then stores into buffer b ----
    uint4 av[kGActChunks], wv[kGWChunks];
    uint16_t sv = 0;
    auto stage_load = [&](int g) {
#pragma unroll
        for (int i = 0; i < kGActChunks; ++i) {
            const int c = tid + kGThreads * i;                 // 16 chunks of 8 values per row
            const int row = min(m0 + (c >> 4), a.M - 1);
            av[i] = *reinterpret_cast<const uint4*>(a.x + size_t(row) * a.lda + g * 128 + (c & 15) * 8);
        }
#pragma unroll
        for (int i = 0; i < kGWChunks; ++i) {
            const int c = min(tid + kGThreads * i, kGBN * 4 - 1);   // 4 chunks of 32 k per column
            const int n = min(n0 + (c >> 2), a.N - 1);
            wv[i] = nt_load(a.qw + size_t(n) * a.nch + 4 * g + (c & 3));
        }
        if (tid < kGBN) sv = a.sc[size_t(g) * a.N + min(n0 + tid, a.N - 1)];
    };
    auto stage_store = [&](int b) {
        uint16_t* as = act_s(b);
        uint16_t* ws = w_s(b);
#pragma unroll
        for (int i = 0; i < kGActChunks; ++i) {
            const int c = tid + kGThreads * i;
            *reinterpret_cast<uint4*>(as + (c >> 4) * kGStride + (c & 15) * 8) = to_pair_order(av[i]);
        }
#pragma unroll
        for (int i = 0; i < kGWChunks; ++i) {
            const int c = tid + kGThreads * i;
            if (c < kGBN * 4) {
                uint16_t* dst = ws + (c >> 2) * kGStride + (c & 3) * 32;
                const uint32_t wd[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<uint4*>(dst + 8 * j) = decode_bf16x8_biased(wd[j], a.dm.lo);
            }
        }
        if (tid < kGBN) sc_s(b)[tid] = bf16_to_f32(sv);
    };

    const uint32_t m136 = 0xC308C308u;                  // bf16 -136 in each half
    const bf16x8_t negoff = __builtin_bit_cast(bf16x8_t, make_uint4(m136, m136, m136, m136));
    f32x4_t out[kGRowTiles][kGColTiles];
#pragma unroll
    for (int r = 0; r < kGRowTiles; ++r)
#pragma unroll
        for (int c = 0; c < kGColTiles; ++c) out[r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    stage_load(0);
    stage_store(0);
    __syncthreads();
    for (int g = 0; g < a.groups; ++g) {
        const int b = g & 1;
        if (g + 1 < a.groups) stage_load(g + 1);
        const uint16_t* as = act_s(b) + (16 * kGRowTiles * wr + lm) * kGStride + ls * 8;
        const uint16_t* ws = w_s(b) + (80 * wc + lm) * kGStride + ls * 8;
        f32x4_t d[kGRowTiles][kGColTiles], bias[kGRowTiles];
#pragma unroll
        for (int r = 0; r < kGRowTiles; ++r) {
            bias[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < kGColTiles; ++c) d[r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8_t bop[kGRowTiles], aop[kGColTiles];
#pragma unroll
            for (int r = 0; r < kGRowTiles; ++r)
                bop[r] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(as + r * 16 * kGStride + ks * 32));
#pragma unroll
            for (int c = 0; c < kGColTiles; ++c)
                aop[c] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(ws + c * 16 * kGStride + ks * 32));
#pragma unroll
            for (int r = 0; r < kGRowTiles; ++r) {
                bias[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(negoff, bop[r], bias[r], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < kGColTiles; ++c)
                    d[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[c], bop[r], d[r][c], 0, 0, 0);
            }
        }
        const float* ss = sc_s(b) + 80 * wc + 4 * ls;
#pragma unroll
        for (int c = 0; c < kGColTiles; ++c) {
            const float4 s4 = *reinterpret_cast<const float4*>(ss + c * 16);
#pragma unroll
            for (int r = 0; r < kGRowTiles; ++r) {
                out[r][c][0] = fmaf(s4.x, d[r][c][0] + bias[r][0], out[r][c][0]);
                out[r][c][1] = fmaf(s4.y, d[r][c][1] + bias[r][1], out[r][c][1]);
                out[r][c][2] = fmaf(s4.z, d[r][c][2] + bias[r][2], out[r][c][2]);
                out[r][c][3] = fmaf(s4.w, d[r][c][3] + bias[r][3], out[r][c][3]);
            }
        }
        if (g + 1 < a.groups) stage_store(b ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds columns 4 ls .. 4 ls + 3 of row lm of each tile ----
    const float os = a.out_scale ? *a.out_scale : 1.0f;
#pragma unroll
    for (int r = 0; r < kGRowTiles; ++r) {
        const int m = m0 + 16 * kGRowTiles * wr + 16 * r + lm;
        if (m >= a.M) continue;
#pragma unroll
        for (int c = 0; c < kGColTiles; ++c) {
            const int n = n0 + 80 * wc + 16 * c + 4 * ls;
            if (n >= a.N) continue;
            float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
            if (a.residual) {
                const uint2 rr = *reinterpret_cast<const uint2*>(a.residual + size_t(m) * a.N + n);
                r0 = bf16_lo(rr.x);
                r1 = bf16_hi(rr.x);
                r2 = bf16_lo(rr.y);
                r3 = bf16_hi(rr.y);
            }
            uint2 o;
            o.x = pack_bf16x2(fmaf(out[r][c][0], os, r0), fmaf(out[r][c][1], os, r1));
            o.y = pack_bf16x2(fmaf(out[r][c][2], os, r2), fmaf(out[r][c][3], os, r3));
            *reinterpret_cast<uint2*>(a.y + size_t(m) * a.N + n) = o;
        }
    }
}

// act[m][k] = bf16(silu(g[m][k]) * u[m][k]), 8 values per thread (K % 8 == 0).
__global__ __launch_bounds__(256) void swiglu_act_kernel(const uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
                                                        int64_t ldgu, int K, int64_t n8, uint16_t* __restrict__ act) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n8) return;
    const int kb = K / 8;
    const int64_t m = i / kb, k = (i % kb) * 8;
    const uint4 gv = *reinterpret_cast<const uint4*>(g + m * ldgu + k);
    const uint4 uv = *reinterpret_cast<const uint4*>(u + m * ldgu + k);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
        o[h] = pack_bf16x2(silu_f32(bf16_lo(gw[h])) * bf16_lo(uw[h]), silu_f32(bf16_hi(gw[h])) * bf16_hi(uw[h]));
    nt_store(make_uint4(o[0], o[1], o[2], o[3]), reinterpret_cast<uint4*>(act + m * int64_t(K) + k));
}

}  // namespace

size_t w4_gemm_lds_bytes() { return kGLdsBytes; }

hipError_t launch_w4_gemm(const uint16_t* x, int64_t lda, const uint32_t* qw, const uint16_t* sc, int M, int K, int N,
                          const float* out_scale, const uint16_t* residual, uint16_t* y, hipStream_t s) {
    GemmArgs a{};
    a.x = x;
    a.lda = lda;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.N = N;
    a.nch = K / 32;
    a.groups = K / kGroup;
    a.ntiles = (N + kGBN - 1) / kGBN;
    a.out_scale = out_scale;
    a.residual = residual;
    a.y = y;
    a.dm = DecodeMasks{kDecodeMaskLo, kDecodeMaskHi};
    const int64_t wgs = int64_t((M + kGBM - 1) / kGBM) * a.ntiles;
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(w4_gemm_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(kGLdsBytes));
    if (e != hipSuccess) return e;
    w4_gemm_kernel<<<dim3(unsigned(wgs)), kGThreads, kGLdsBytes, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_swiglu_act(const uint16_t* g, const uint16_t* u, int64_t ldgu, int M, int K, uint16_t* act,
                             hipStream_t s) {
    const int64_t n8 = int64_t(M) * (K / 8);
    if (n8 == 0) return hipSuccess;
    swiglu_act_kernel<<<dim3(unsigned((n8 + 255) / 256)), 256, 0, s>>>(g, u, ldgu, K, n8, act);
    return hipGetLastError();
}

}  // namespace fdec
