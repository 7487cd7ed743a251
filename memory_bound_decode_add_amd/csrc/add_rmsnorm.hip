// Fused residual add + RMSNorm with two outputs, gfx950.
//
// Semantics ("Kernel Fusion, torch.compile and CUDA Graphs, Measured", Step 2; "09 -
// Operator fusion", section 5): h = bf16(x + r) is the new residual, written once;
// y = bf16(h * w / sqrt(mean(h^2) + eps)) with h taken after its bf16 rounding, the
// mean over the row, eps inside the root, and one final rounding.
//
// Design: the row lives in registers between the add and the scale, so x and r are
// read once and h and y written once (8 bytes per element, the minimum).  A row is
// spread over 1 to 8 waves so that no lane holds more than 4 chunks of 16 bytes (8
// bf16) of each of x, r and w, which keeps registers low enough for 5-8 waves per
// SIMD to hide HBM latency (rows of 449..512 chunks take eight waves of one chunk).  Lane chunks are strided by 64 so every load and store
// instruction of a wave touches 1 KB of contiguous memory.  The sum of squares is
// reduced with cross-lane shuffles, and across the waves of a row through LDS.
// h may alias r (in-place residual update): each lane reads its chunks of r before it
// writes the same chunks of h.
//
// Optionally (ys non-null; H % 128 == 0) the kernel also writes y as the matrix-core
// GEMVs stage their activation: each 16-byte chunk of y as block-scaled fp16 in pair
// order (ys, [M][H/8] chunks) and each 128-wide group's power of two (yesc, [M][H/128]).
// A chunk is one k-block, and the 16 lanes of a DPP row hold a group's 16 chunks, so the
// group scale is the same DPP reduction the GEMVs run; a GEMV that copies this instead of
// staging y itself computes bit-identical products.  Each of the 224 workgroups of the
// 16-row layer's gate_up otherwise converts the same 16 x 4096 activation.
#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {
namespace {

constexpr int kThreads = 256;

// WPR waves share a row (WPR in {1, 2, 4, 8}); a workgroup holds max(4, WPR) waves.
// Lane l of part p owns the 16-byte chunks l + 64 (p + WPR i), i < NC.  With WPR > 1
// the parts' sums of squares meet in LDS and are added in part order.
template <int NC, int WPR>
__global__ __launch_bounds__(WPR > 4 ? 64 * WPR : kThreads) void add_rmsnorm_kernel(
    const uint4* __restrict__ x, const uint4* r, const uint4* __restrict__ w,
    uint4* h, uint4* __restrict__ y, uint4* __restrict__ ys, float* __restrict__ yesc,
    int M, int chunks, float inv_h, float eps) {
    constexpr int kWaves = WPR > 4 ? WPR : kThreads / kWave;
    constexpr int kRows = kWaves / WPR;
    __shared__ float part_ss[kWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int part = wave % WPR;
    const int row = blockIdx.x * kRows + wave / WPR;
    const bool live_row = row < M;
    const size_t base = size_t(min(row, M - 1)) * chunks;

    // every load of the row, the weight included, is issued before the first use, so a
    // row costs one memory round trip; x and r are streamed (non-temporal), w stays cached
    uint4 xv[NC], rv[NC], wv[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = min(lane + kWave * (part + WPR * i), chunks - 1);
        xv[i] = nt_load(x + base + c);
        rv[i] = nt_load(r + base + c);
        wv[i] = w[c];
    }

    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + kWave * (part + WPR * i);
        const uint32_t xa[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        const uint32_t ra[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
        uint32_t ha[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t hw = pack_bf16x2(bf16_lo(xa[j]) + bf16_lo(ra[j]), bf16_hi(xa[j]) + bf16_hi(ra[j]));
            ha[j] = hw;
            const float h0 = bf16_lo(hw), h1 = bf16_hi(hw);
            ss = (c < chunks) ? fmaf(h1, h1, fmaf(h0, h0, ss)) : ss;
        }
        xv[i] = make_uint4(ha[0], ha[1], ha[2], ha[3]);      // xv now holds h
        if (live_row && c < chunks) nt_store(xv[i], h + base + c);
    }
    ss = wave_sum(ss);
    if (WPR > 1) {
        if (lane == 0) part_ss[wave] = ss;
        __syncthreads();
        ss = 0.f;
#pragma unroll
        for (int p = 0; p < WPR; ++p) ss += part_ss[wave - part + p];
    }
    const float rstd = __builtin_amdgcn_rsqf(fmaf(ss, inv_h, eps));

#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + kWave * (part + WPR * i);
        const uint32_t ha[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        const uint32_t wa[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
        uint32_t ya[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ya[j] = pack_bf16x2(bf16_lo(ha[j]) * rstd * bf16_lo(wa[j]), bf16_hi(ha[j]) * rstd * bf16_hi(wa[j]));
        const uint4 yw = make_uint4(ya[0], ya[1], ya[2], ya[3]);
        if (live_row && c < chunks) nt_store(yw, y + base + c);
        if (ys) {       // uniform; the whole wave takes part in the group reduction
            float esc;
            const uint4 st = stage_bf16_kblock(yw, &esc);
            if (live_row && c < chunks) {
                ys[base + c] = st;
                if ((c & 15) == 0) yesc[size_t(row) * (chunks >> 4) + (c >> 4)] = esc;
            }
        }
    }
}

template <int NC, int WPR>
hipError_t launch_nc(const uint16_t* x, const uint16_t* r, const uint16_t* w, float eps,
                     int M, int H, uint16_t* h, uint16_t* y, void* ys, float* yesc, hipStream_t s) {
    constexpr int waves = WPR > 4 ? WPR : kThreads / kWave;
    constexpr int rows = waves / WPR;
    const int chunks = H / 8;
    const int blocks = (M + rows - 1) / rows;
    add_rmsnorm_kernel<NC, WPR><<<blocks, waves * kWave, 0, s>>>(
        reinterpret_cast<const uint4*>(x), reinterpret_cast<const uint4*>(r),
        reinterpret_cast<const uint4*>(w), reinterpret_cast<uint4*>(h),
        reinterpret_cast<uint4*>(y), static_cast<uint4*>(ys), yesc, M, chunks, 1.0f / float(H), eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w,
                              float eps, int M, int H, uint16_t* h, uint16_t* y,
                              hipStream_t s) {
    return launch_add_rmsnorm_staged(x, r, w, eps, M, H, h, y, nullptr, nullptr, s);
}

hipError_t launch_add_rmsnorm_staged(const uint16_t* x, const uint16_t* r, const uint16_t* w, float eps, int M,
                                     int H, uint16_t* h, uint16_t* y, void* ys, float* yesc, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (ys && (H % 128 || !yesc)) return hipErrorInvalidValue;
    // at most 4 chunks per lane (x, r and w in registers), more waves per row beyond that
    const int per_lane = (H / 8 + kWave - 1) / kWave;   // 1..32 for H <= 16384
    if (M <= 64 && per_lane <= 8) {
        // a few rows (decode): one chunk per lane, the row spread over up to eight waves,
        // so that a row's loads are spread over as many waves as possible
        switch (per_lane) {
            case 1: return launch_nc<1, 1>(x, r, w, eps, M, H, h, y, ys, yesc, s);
            case 2: return launch_nc<1, 2>(x, r, w, eps, M, H, h, y, ys, yesc, s);
            case 3: case 4: return launch_nc<1, 4>(x, r, w, eps, M, H, h, y, ys, yesc, s);
            default: return launch_nc<1, 8>(x, r, w, eps, M, H, h, y, ys, yesc, s);
        }
    }
    switch (per_lane) {
        case 1: return launch_nc<1, 1>(x, r, w, eps, M, H, h, y, ys, yesc, s);
        case 2: return launch_nc<2, 1>(x, r, w, eps, M, H, h, y, ys, yesc, s);
        case 3: return launch_nc<3, 1>(x, r, w, eps, M, H, h, y, ys, yesc, s);
        case 4: return launch_nc<4, 1>(x, r, w, eps, M, H, h, y, ys, yesc, s);
        case 5: case 6: return launch_nc<3, 2>(x, r, w, eps, M, H, h, y, ys, yesc, s);
        // 449..512 chunks (H = 4096): eight waves of one chunk per lane measured 3 % faster
        // at 8192 x 4096 than two waves of four
        case 7: case 8: return launch_nc<1, 8>(x, r, w, eps, M, H, h, y, ys, yesc, s);
        case 9: case 10: case 11: case 12: return launch_nc<3, 4>(x, r, w, eps, M, H, h, y, ys, yesc, s);
        case 13: case 14: case 15: case 16: return launch_nc<4, 4>(x, r, w, eps, M, H, h, y, ys, yesc, s);
        default: return launch_nc<4, 8>(x, r, w, eps, M, H, h, y, ys, yesc, s);
    }
}

}  // namespace fdec
