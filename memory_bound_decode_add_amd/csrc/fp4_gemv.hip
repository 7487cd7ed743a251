// FP4 (E2M1) weight GEMV with E4M3 block scales of 16 along K, a SwiGLU (or identity)
// prologue and an fp32 output-scale + residual epilogue, M = 1..4, gfx950.
//
// What it computes ("PyTorch folds NVFP4 output scaling into NVGEMM candidates for
// decode workloads": packed FP4 weights with E4M3 1x16 block scales and a
// zero-dimensional fp32 output multiplier applied inside the GEMM):
//     y[m, n] = bf16( s * sum_k act[m, k] * e2m1(q[k, n]) * e4m3(scale[n, k/16])  (+ res[m, n]) )
// with act = silu(g) * u or act = x.  The activation exists only in registers.
//
// Weights: qweight uint32 [N][K/8], E2M1 code of k = 8 kb + j in bits [4j, 4j+4) of word
// (n, kb); scales E4M3 bytes [N][K/16], so the two scales of a 32-wide chunk of a column
// are one 16-bit word.
//
// Work assignment.  A workgroup owns C = 2 CH consecutive columns and has ceil(K/1024)
// waves; wave w covers the 32-wide K chunks 32 w .. 32 w + 31.  Lane (h = lane / 32, cl =
// lane % 32) owns chunk c = 32 w + cl and columns h CH .. h CH + CH - 1 of the workgroup:
//  * it loads half of the chunk's activation inputs (k = 32 c + 16 h .. + 15), forms
//    those 16 activation values in fp32, and the two lanes of the chunk (l, l ^ 32)
//    exchange their halves as block-scaled fp16: one power of two per chunk puts the
//    chunk's largest magnitude in [2^14, 2^15), so every value fits fp16 with an 11-bit
//    significand relative to it.  Each activation value is computed once per workgroup.
//  * for each of its CH columns it loads the chunk's 16 bytes of weights (a half-wave
//    reads 512 contiguous bytes of one column) and the chunk's two block scales.  gfx950's
//    v_cvt_scalef32_pk_f16_fp4 turns a byte of two E2M1 codes into two exact fp16 values;
//    it is run with scale 1, because it applies only the exponent of its fp32 scale
//    operand (the power-of-two scales of the MX formats; measured: an E4M3 scale's
//    mantissa is dropped).  Eight v_dot2_f32_f16 sum each 16-wide block in fp32, and the
//    two block sums are multiplied by their E4M3 scales.
// A column's 32-lane sums are reduced with DPP and lane reads, the per-wave results meet
// in LDS, and one lane per output sums them in wave order and applies the epilogue.  No
// workspace, no cross-workgroup step; results do not depend on scheduling.
//
// FP4 activations (A4: both operands FP4, as the page's scaled matmul takes them).  A
// lane's 16 activation values are exactly one block of 16 along K, so it quantises them
// on its own (nvfp4_quantize_block: E4M3 block scale from the block's largest magnitude
// and the per-tensor scale G, E2M1 codes) and exchanges the exact fp16 values q s instead
// of the block-scaled activation; the chunk's power of two is then 1.
#include "device_common.h"
#include "fdec_internal.h"

#include <algorithm>

namespace fdec {

namespace {

constexpr int kFp4MaxWaves = 16;
constexpr int kFp4MaxCh = 8;                                  // columns per lane, at most
constexpr int kFp4ScBytes = 2 * kFp4MaxCh * 32 * kFp4MaxWaves * 2 + 32;   // a workgroup's scales + alignment slack

__device__ __forceinline__ float xchg32(float v) { return __shfl_xor(v, 32, kWave); }
__device__ __forceinline__ uint32_t xchg32u(uint32_t v) {
    return __builtin_bit_cast(uint32_t, __shfl_xor(__builtin_bit_cast(int, v), 32, kWave));
}

struct Fp4Args {
    const uint16_t* a0;     // g (SwiGLU) or x (identity), row stride lda
    const uint16_t* a1;     // u (SwiGLU) or unused
    int64_t lda;
    const uint4* qw;        // [N][K/32] chunks of four words
    const uint8_t* sc;      // [N][K/16] E4M3 block scales
    int M, K, N;
    int nch;                // K / 32
    int cols;               // columns per workgroup (2 CH)
    const float* out_scale;
    const uint16_t* residual;
    uint16_t* y;
    const float* gscale;    // A4: the activation's per-tensor scale G (device fp32)
};

template <int MR, int CH, int PRO, bool A4>
__global__ __launch_bounds__(kFp4MaxWaves * kWave) void fp4_gemv_kernel(Fp4Args a) {
    __shared__ float red[kFp4MaxWaves][MR][2 * CH];
    __shared__ __align__(16) unsigned char sc_s[kFp4ScBytes];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h = lane >> 5, cl = lane & 31;
    const int cbase = xcd_remap(blockIdx.x, gridDim.x) * a.cols;
    const int c = wave * 32 + cl;
    const bool valid = c < a.nch;
    const int cc = min(c, a.nch - 1);          // loads stay inside the tensors

    // ---- every global load first: activation inputs, then weights and scales ----
    uint4 ga[MR][2], ua[MR][2];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const uint16_t* p = a.a0 + size_t(min(m, a.M - 1)) * a.lda + size_t(cc) * 32 + 16 * h;
        ga[m][0] = *reinterpret_cast<const uint4*>(p);
        ga[m][1] = *reinterpret_cast<const uint4*>(p + 8);
        if (PRO == kSwiGLU) {
            const uint16_t* q = a.a1 + size_t(min(m, a.M - 1)) * a.lda + size_t(cc) * 32 + 16 * h;
            ua[m][0] = *reinterpret_cast<const uint4*>(q);
            ua[m][1] = *reinterpret_cast<const uint4*>(q + 8);
        }
    }
    uint4 wv[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const size_t n = size_t(min(cbase + h * CH + j, a.N - 1));
        wv[j] = nt_load(a.qw + n * a.nch + cc);
    }
    // The workgroup's block scales are one contiguous run of cols * K/16 bytes (its
    // columns are consecutive rows of [N][K/16]).  Threads load it in 16-byte pieces from
    // the 16-byte boundary at or below its start; the tensor's size is a multiple of 16
    // (N % 8 == 0, K/16 even), so no piece reads past its end.
    const size_t sb = size_t(a.K) / 16;                      // scale bytes per column
    const int ncols = min(a.cols, a.N - cbase);              // columns that exist
    const size_t s0 = size_t(cbase) * sb, s1 = s0 + size_t(ncols) * sb;
    const size_t a0 = s0 & ~size_t(15);
    const int npieces = int((s1 - a0 + 15) >> 4);
    uint4 spc[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int t = min(tid + r * int(blockDim.x), npieces - 1);
        spc[r] = *reinterpret_cast<const uint4*>(a.sc + a0 + size_t(t) * 16);
    }

    // ---- the chunk's activation, block-scaled fp16, both halves in every lane ----
    uint32_t act[MR][16];                      // the chunk's 32 values as 16 pairs, k order
    float e2[MR];                              // the chunk's power of two
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const bool live = valid && m < a.M;
        const uint32_t gw[8] = {ga[m][0].x, ga[m][0].y, ga[m][0].z, ga[m][0].w,
                                ga[m][1].x, ga[m][1].y, ga[m][1].z, ga[m][1].w};
        uint32_t uw[8] = {};
        if (PRO == kSwiGLU) {
            const uint32_t t[8] = {ua[m][0].x, ua[m][0].y, ua[m][0].z, ua[m][0].w,
                                   ua[m][1].x, ua[m][1].y, ua[m][1].z, ua[m][1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) uw[i] = t[i];
        }
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (PRO == kSwiGLU) {
                v[2 * i] = silu_f32(bf16_lo(gw[i])) * bf16_lo(uw[i]);
                v[2 * i + 1] = silu_f32(bf16_hi(gw[i])) * bf16_hi(uw[i]);
            } else {
                v[2 * i] = bf16_lo(gw[i]);
                v[2 * i + 1] = bf16_hi(gw[i]);
            }
        }
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            v[i] = live ? v[i] : 0.f;
            mx = fmaxf(mx, fabsf(v[i]));
        }
        uint32_t own[8];
        if (A4) {
            // the lane's 16 values are one block: its codes and the exact values q s
            uint32_t words[2];
            (void)nvfp4_quantize_block<16>(v, mx, *a.gscale, words, own);
            e2[m] = 1.0f;
        } else {
            mx = fmaxf(mx, xchg32(mx));            // the chunk's largest magnitude
            int e = 0;
            (void)__builtin_frexpf(mx, &e);
            const int E = min(max(e - 15, -126), 127);
            const float down = __builtin_ldexpf(1.0f, -E);
            e2[m] = __builtin_ldexpf(1.0f, E);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                own[i] = __builtin_bit_cast(uint32_t, pk_f16_rtz(v[2 * i] * down, v[2 * i + 1] * down));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t oth = xchg32u(own[i]);
            act[m][i] = h ? oth : own[i];      // k = 32 c + 0 .. 15 come from half 0
            act[m][8 + i] = h ? own[i] : oth;  // k = 32 c + 16 .. 31 from half 1
        }
    }

    // ---- scales to LDS: piece t at sc_s[16 t], so byte i of the run is at sc_s[s0 - a0 + i]
    // (s0 - a0 is even: cbase and K/16 are) ----
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int t = tid + r * int(blockDim.x);
        if (t < npieces) *reinterpret_cast<uint4*>(sc_s + size_t(t) * 16) = spc[r];
    }
    __syncthreads();

    // ---- the chunk's dot product for each of the lane's columns ----
    float part[MR][CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int col = min(h * CH + j, ncols - 1);
        const uint32_t sp = *reinterpret_cast<const uint16_t*>(sc_s + (s0 - a0) + size_t(col) * sb + 2 * cc);
        const float bs0 = e4m3_to_f32(sp & 0xFFu), bs1 = e4m3_to_f32(sp >> 8);   // block scales
        half2_t q[16];
        fp4x8(wv[j].x, q);
        fp4x8(wv[j].y, q + 4);
        fp4x8(wv[j].z, q + 8);
        fp4x8(wv[j].w, q + 12);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float d0 = 0.f, d1 = 0.f;          // the chunk's two 16-wide blocks
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                d0 = dot2(q[i], __builtin_bit_cast(half2_t, act[m][i]), d0);
                d1 = dot2(q[8 + i], __builtin_bit_cast(half2_t, act[m][8 + i]), d1);
            }
            part[m][j] = valid ? fmaf(d0, bs0, d1 * bs1) * e2[m] : 0.f;
        }
    }

    // ---- per column: the row swap folds the two rows of each half for two columns at
    // once (rows then hold column j0 and j1 of half 0, j0 and j1 of half 1), four DPP steps
    // sum each row, and each row's first lane writes its column's wave sum ----
    const int orow = lane >> 4;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int p = 0; p < (CH + 1) / 2; ++p) {
            const int j0 = 2 * p, j1 = min(2 * p + 1, CH - 1);
            const f32x2_t z = swap16(part[m][j0], part[m][j1]);
            float t = z[0] + z[1];
            t += dpp<kQuadSwap1>(t);
            t += dpp<kQuadSwap2>(t);
            t += dpp<kRowRor4>(t);
            t += dpp<kRowRor8>(t);
            if ((lane & 15) == 0 && 2 * p + (orow & 1) < CH)
                red[wave][m][(orow >> 1) * CH + ((orow & 1) ? j1 : j0)] = t;
        }
    __syncthreads();
    if (wave == 0 && lane < MR * 2 * CH) {
        const int m = lane / (2 * CH), col = lane % (2 * CH), n = cbase + col;
        const int nw = blockDim.x >> 6;
        float t = 0.f;
        for (int w = 0; w < nw; ++w) t += red[w][m][col];
        if (m < a.M && col < a.cols && n < a.N) {
            const float os = a.out_scale ? *a.out_scale : 1.0f;
            const float res = a.residual ? bf16_to_f32(a.residual[size_t(m) * a.N + n]) : 0.f;
            a.y[size_t(m) * a.N + n] = f32_to_bf16(fmaf(t, os, res));
        }
    }
}

// Test hook: the same decode, written out as fp32 w[k][n].
__global__ void fp4_dequant_kernel(const uint32_t* __restrict__ qw, const uint8_t* __restrict__ sc, int KB, int N,
                                   float* __restrict__ w) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;     // word (n, kb)
    if (i >= int64_t(KB) * N) return;
    const int n = int(i / KB), kb = int(i % KB);
    const float s = e4m3_to_f32(sc[int64_t(n) * (KB / 2) + kb / 2]);
    half2_t q[4];
    fp4x8(qw[i], q);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        w[(int64_t(kb) * 8 + 2 * p) * N + n] = float(q[p][0]) * s;
        w[(int64_t(kb) * 8 + 2 * p + 1) * N + n] = float(q[p][1]) * s;
    }
}

// Test hook: FP4 quantisation of a bf16 activation, one thread per block of 16 values:
// codes [M][K/8] packed words (k order), E4M3 scale codes [M][K/16].
__global__ void nvfp4_quantize_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M, int nblk,
                                      const float* __restrict__ gscale, uint32_t* __restrict__ codes,
                                      uint8_t* __restrict__ scales) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;   // block (m, b)
    if (i >= int64_t(M) * nblk) return;
    const int64_t m = i / nblk, b = i % nblk;
    const uint4* src = reinterpret_cast<const uint4*>(x + m * ldx + b * 16);
    const uint4 p0 = src[0], p1 = src[1];
    const uint32_t wd[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float v[16], mx = 0.f;
#pragma unroll
    for (int h = 0; h < 8; ++h) {
        v[2 * h] = bf16_lo(wd[h]);
        v[2 * h + 1] = bf16_hi(wd[h]);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) mx = fmaxf(mx, fabsf(v[k]));
    uint32_t words[2], xq[8];
    const uint32_t sc = nvfp4_quantize_block<16>(v, mx, *gscale, words, xq);
    codes[m * (nblk * 2) + 2 * b] = words[0];
    codes[m * (nblk * 2) + 2 * b + 1] = words[1];
    scales[m * nblk + b] = uint8_t(sc);
}

struct Fp4Plan {
    int mr, ch, cols, waves, wgs;
};

// Columns per lane: about N / 512, so that C = 2 CH columns per workgroup gives one
// workgroup per CU; capped by the registers the rows need (8, 6 and 2 for 1, 2 and 4 rows).
constexpr int kFp4Ch[] = {1, 2, 3, 4, 5, 6, 8};

bool fp4_plan(int M, int K, int N, Fp4Plan& p) {
    if (M < 1 || M > 4 || K <= 0 || K % 32 || K > 32 * 32 * kFp4MaxWaves || N <= 0 || N % 8) return false;
    p.mr = M <= 1 ? 1 : M <= 2 ? 2 : 4;
    const int chmax = p.mr == 1 ? 8 : p.mr == 2 ? 6 : 2;
    const int want = std::min(chmax, std::max(1, (N + 511) / 512));
    p.ch = chmax;
    for (int c : kFp4Ch)
        if (c >= want && c <= chmax) { p.ch = c; break; }
    p.cols = 2 * p.ch;
    p.waves = (K / 32 + 31) / 32;
    p.wgs = (N + p.cols - 1) / p.cols;
    return true;
}

template <int MR, int CH>
hipError_t launch_fp4_2(Prologue pro, const Fp4Args& a, const Fp4Plan& p, hipStream_t s) {
    const dim3 grid(p.wgs), block(p.waves * kWave);
    if (a.gscale) {
        if (pro == kSwiGLU)
            fp4_gemv_kernel<MR, CH, kSwiGLU, true><<<grid, block, 0, s>>>(a);
        else
            fp4_gemv_kernel<MR, CH, kIdentity, true><<<grid, block, 0, s>>>(a);
    } else if (pro == kSwiGLU) {
        fp4_gemv_kernel<MR, CH, kSwiGLU, false><<<grid, block, 0, s>>>(a);
    } else {
        fp4_gemv_kernel<MR, CH, kIdentity, false><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

// Instantiated: CH in {1, 2} for every MR, 3..6 for MR <= 2, 8 for MR == 1 (the
// register budget: no spills); fp4_plan only picks these.
template <int MR>
hipError_t launch_fp4_1(Prologue pro, const Fp4Args& a, const Fp4Plan& p, hipStream_t s) {
    if constexpr (MR == 1)
        if (p.ch == 8) return launch_fp4_2<MR, 8>(pro, a, p, s);
    if constexpr (MR <= 2) {
        switch (p.ch) {
            case 6: return launch_fp4_2<MR, 6>(pro, a, p, s);
            case 5: return launch_fp4_2<MR, 5>(pro, a, p, s);
            case 4: return launch_fp4_2<MR, 4>(pro, a, p, s);
            case 3: return launch_fp4_2<MR, 3>(pro, a, p, s);
            default: break;
        }
    }
    switch (p.ch) {
        case 1: return launch_fp4_2<MR, 1>(pro, a, p, s);
        case 2: return launch_fp4_2<MR, 2>(pro, a, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// One or two rows: the chunk-owning kernel above; also three or four where K % 128 != 0.
// Otherwise the matrix-core kernel with the FP4 weight format (K % 128 == 0; two or four
// 16-row blocks past 16 rows), whose K slices need a workspace.  At three and four rows
// the chunk-owning kernel holds two columns per lane half (its registers), so some 640
// workgroups each recompute the whole activation's SiLU.
bool fp4_on_lanes(int M, int K) { return M <= 2 || (M <= 4 && K % 128 != 0); }

bool fp4_gemv_supported(int M, int K, int N) {
    Fp4Plan p;
    if (fp4_on_lanes(M, K)) return fp4_plan(M, K, N, p);
    GemvPlan g{};
    return M <= kMfmaMaxRows && K > 0 && K % 128 == 0 && N > 0 && N % 8 == 0 && plan_mfma(M, K, N, g, 3);
}

size_t fp4_gemv_workspace_bytes(int M, int K, int N) {
    if (fp4_on_lanes(M, K) || !fp4_gemv_supported(M, K, N)) return 0;
    GemvPlan g{};
    g.groups = K / kGroup;
    plan_mfma(M, K, N, g, 3);
    return g.partial_bytes;
}

hipError_t launch_fp4_gemv(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda, const uint32_t* qw,
                           const uint8_t* sc, int M, int K, int N, const float* out_scale, const uint16_t* residual,
                           uint16_t* y, void* ws, const float* gscale, hipStream_t s) {
    if (!fp4_on_lanes(M, K)) {
        GemvPlan g{};
        g.groups = K / kGroup;
        if (!fp4_gemv_supported(M, K, N) || !plan_mfma(M, K, N, g, 3)) return hipErrorInvalidValue;
        return launch_mfma_fp4(pro, a0, a1, lda, qw, sc, M, K, N, out_scale, residual, y, ws, g, gscale, s);
    }
    Fp4Plan p;
    if (!fp4_plan(M, K, N, p)) return hipErrorInvalidValue;
    Fp4Args a{};
    a.a0 = a0;
    a.a1 = a1;
    a.lda = lda;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.K = K;
    a.N = N;
    a.nch = K / 32;
    a.cols = p.cols;
    a.out_scale = out_scale;
    a.residual = residual;
    a.y = y;
    a.gscale = gscale;
    switch (p.mr) {
        case 1: return launch_fp4_1<1>(pro, a, p, s);
        case 2: return launch_fp4_1<2>(pro, a, p, s);
        default: return launch_fp4_1<4>(pro, a, p, s);
    }
}

hipError_t launch_nvfp4_quantize(const uint16_t* x, int64_t ldx, int M, int K, const float* gscale, uint32_t* codes,
                                 uint8_t* scales, hipStream_t s) {
    const int64_t n = int64_t(M) * (K / 16);
    if (n == 0) return hipSuccess;
    nvfp4_quantize_kernel<<<dim3(unsigned((n + 255) / 256)), 256, 0, s>>>(x, ldx, M, K / 16, gscale, codes, scales);
    return hipGetLastError();
}

hipError_t launch_fp4_dequant(const uint32_t* qw, const uint8_t* sc, int K, int N, float* w, hipStream_t s) {
    const int64_t n = int64_t(K / 8) * N;
    fp4_dequant_kernel<<<dim3((n + 255) / 256), 256, 0, s>>>(qw, sc, K / 8, N, w);
    return hipGetLastError();
}

}  // namespace fdec
