// Fused residual add + RMSNorm with two outputs, gfx950.
//
// Semantics ("Kernel Fusion, torch.compile and CUDA Graphs, Measured", Step 2; "09 -
// Operator fusion", section 5): h = bf16(x + r) is the new residual, written once;
// y = bf16(h * w / sqrt(mean(h^2) + eps)) with h taken after its bf16 rounding, the
// mean over the row, eps inside the root, and one final rounding.
//
// Design: one wave per row; the row lives in registers between the add and the
// scale, so x and r are read once and h and y written once (8 bytes per element,
// the minimum).  Each lane owns NC 16-byte chunks (8 bf16) strided by 64 chunks, so
// every load and store instruction of a wave touches 1 KB of contiguous memory.  The
// sum of squares is reduced with cross-lane shuffles; there is no LDS and no barrier.
// Four rows per 256-thread workgroup.  h may alias r (in-place residual update): each
// lane reads its chunks of r before it writes the same chunks of h.
#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {
namespace {

constexpr int kRowsPerBlock = 4;

template <int NC>
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(
    const uint4* __restrict__ x, const uint4* r, const uint4* __restrict__ w,
    uint4* h, uint4* __restrict__ y, int M, int chunks, float inv_h, float eps) {
    const int lane = threadIdx.x & (kWave - 1);
    const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= M) return;
    const size_t base = size_t(row) * chunks;

    uint4 xv[NC], rv[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + i * kWave;
        if (c < chunks) {
            xv[i] = x[base + c];
            rv[i] = r[base + c];
        }
    }

    uint4 hv[NC];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + i * kWave;
        if (c < chunks) {
            const uint32_t xa[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
            const uint32_t ra[4] = {rv[i].x, rv[i].y, rv[i].z, rv[i].w};
            uint32_t ha[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t hw = pack_bf16x2(bf16_lo(xa[j]) + bf16_lo(ra[j]),
                                                bf16_hi(xa[j]) + bf16_hi(ra[j]));
                ha[j] = hw;
                const float h0 = bf16_lo(hw), h1 = bf16_hi(hw);
                ss = fmaf(h0, h0, ss);
                ss = fmaf(h1, h1, ss);
            }
            hv[i] = make_uint4(ha[0], ha[1], ha[2], ha[3]);
            h[base + c] = hv[i];
        }
    }
    ss = wave_sum(ss);
    const float rstd = __builtin_amdgcn_rsqf(fmaf(ss, inv_h, eps));

#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + i * kWave;
        if (c < chunks) {
            const uint4 wv = w[c];
            const uint32_t ha[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
            const uint32_t wa[4] = {wv.x, wv.y, wv.z, wv.w};
            uint32_t ya[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ya[j] = pack_bf16x2(bf16_lo(ha[j]) * rstd * bf16_lo(wa[j]),
                                    bf16_hi(ha[j]) * rstd * bf16_hi(wa[j]));
            y[base + c] = make_uint4(ya[0], ya[1], ya[2], ya[3]);
        }
    }
}

template <int NC>
hipError_t launch_nc(const uint16_t* x, const uint16_t* r, const uint16_t* w, float eps,
                     int M, int H, uint16_t* h, uint16_t* y, hipStream_t s) {
    const int chunks = H / 8;
    const int blocks = (M + kRowsPerBlock - 1) / kRowsPerBlock;
    add_rmsnorm_kernel<NC><<<blocks, 256, 0, s>>>(
        reinterpret_cast<const uint4*>(x), reinterpret_cast<const uint4*>(r),
        reinterpret_cast<const uint4*>(w), reinterpret_cast<uint4*>(h),
        reinterpret_cast<uint4*>(y), M, chunks, 1.0f / float(H), eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* w,
                              float eps, int M, int H, uint16_t* h, uint16_t* y,
                              hipStream_t s) {
    if (M == 0) return hipSuccess;
    const int per_lane = (H / 8 + kWave - 1) / kWave;   // 1..32 for H <= 16384
    switch (per_lane) {
        case 1: return launch_nc<1>(x, r, w, eps, M, H, h, y, s);
        case 2: return launch_nc<2>(x, r, w, eps, M, H, h, y, s);
        case 3: return launch_nc<3>(x, r, w, eps, M, H, h, y, s);
        case 4: return launch_nc<4>(x, r, w, eps, M, H, h, y, s);
        case 5: case 6: return launch_nc<6>(x, r, w, eps, M, H, h, y, s);
        case 7: case 8: return launch_nc<8>(x, r, w, eps, M, H, h, y, s);
        case 9: case 10: case 11: case 12: return launch_nc<12>(x, r, w, eps, M, H, h, y, s);
        case 13: case 14: case 15: case 16: return launch_nc<16>(x, r, w, eps, M, H, h, y, s);
        default: return launch_nc<32>(x, r, w, eps, M, H, h, y, s);
    }
}

}  // namespace fdec
