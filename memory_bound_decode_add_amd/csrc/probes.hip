// Measurement probes: an empty kernel (the per-launch floor of back-to-back launches)
// and a read-only kernel that reads the column-owning GEMV's bytes in that kernel's
// order (the ceiling of any kernel that must read them).  Neither is part of the method.
#include "device_common.h"
#include "fdec_internal.h"

namespace fdec {
namespace {

__global__ void empty_kernel() {}

constexpr int kProbeThreads = 1024;
// 16-byte loads per thread, at most, for the stream, each broadcast buffer and the pieces
// (few enough that every load of a thread stays in flight in registers at once)
constexpr int kWLoads = 4, kBLoads = 2, kPLoads = 1;

struct ReadArgs {
    const uint4* stream;     // per_wg chunks per workgroup, contiguous
    int per_wg;
    const uint4* b0;         // bcast16 chunks, read by every workgroup
    const uint4* b1;
    int bcast16;
    const unsigned char* pieces;
    int rows, row_bytes, piece_bytes;
    uint32_t* sink;
};

__global__ __launch_bounds__(kProbeThreads) void read_ceiling_kernel(ReadArgs a) {
    const int b = xcd_remap(blockIdx.x, gridDim.x);    // the GEMV's workgroup numbering
    const int t = threadIdx.x;
    // every load is issued before any is used; a load past its region's end is skipped
    // (whole waves skip together except at a region's last partial wave), so the kernel
    // issues the same number of wave-level loads as the GEMV does for these bytes
    // Rounds of loads stop at a region's end (a workgroup-uniform test); inside a round
    // every lane loads, lanes past the end from the region's last chunk, and their values
    // are dropped when the checksum is formed.
    u32x4_t wv[kWLoads], gv[kBLoads], uv[kBLoads], sv[kPLoads];
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const u32x4_t* wbase = reinterpret_cast<const u32x4_t*>(a.stream) + size_t(b) * a.per_wg;
    const u32x4_t* g4 = reinterpret_cast<const u32x4_t*>(a.b0);
    const u32x4_t* u4 = reinterpret_cast<const u32x4_t*>(a.b1);
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) {
        wv[i] = zero;
        if (i * kProbeThreads >= a.per_wg) break;              // uniform
        wv[i] = __builtin_nontemporal_load(wbase + min(t + i * kProbeThreads, a.per_wg - 1));
    }
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
        gv[i] = uv[i] = zero;
        if (i * kProbeThreads >= a.bcast16) break;             // uniform
        const int c = min(t + i * kProbeThreads, a.bcast16 - 1);
        gv[i] = g4[c];
        uv[i] = u4[c];
    }
    // scale pieces: row r, the aligned 16-byte pieces covering [b * pb, (b + 1) * pb)
    const int p0 = (b * a.piece_bytes) >> 4, p1 = ((b + 1) * a.piece_bytes - 1) >> 4;
    const int ppr = p1 - p0 + 1, npieces = a.rows * ppr;
#pragma unroll
    for (int i = 0; i < kPLoads; ++i) {
        sv[i] = zero;
        if (i * kProbeThreads >= npieces) break;               // uniform
        const int j = min(t + i * kProbeThreads, npieces - 1);
        sv[i] = *reinterpret_cast<const u32x4_t*>(a.pieces + size_t(j / ppr) * a.row_bytes + size_t(p0 + j % ppr) * 16);
    }
    u32x4_t x = zero;
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) x ^= t + i * kProbeThreads < a.per_wg ? wv[i] : zero;
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) x ^= t + i * kProbeThreads < a.bcast16 ? gv[i] ^ uv[i] : zero;
#pragma unroll
    for (int i = 0; i < kPLoads; ++i) x ^= t + i * kProbeThreads < npieces ? sv[i] : zero;
    uint32_t acc = x[0] ^ x[1] ^ x[2] ^ x[3];
    // one word per workgroup: the per-wave XOR, summed over the waves in LDS
    __shared__ uint32_t red[kProbeThreads / kWave];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
    if ((t & 63) == 0) red[t >> 6] = acc;
    __syncthreads();
    if (t == 0) {
        uint32_t r = 0;
        for (int w = 0; w < kProbeThreads / kWave; ++w) r ^= red[w];
        a.sink[b] = r;
    }
}

}  // namespace

hipError_t launch_empty(int wgs, int threads, hipStream_t s) {
    empty_kernel<<<dim3(wgs), dim3(threads), 0, s>>>();
    return hipGetLastError();
}

bool read_ceiling_fits(int per_wg, int bcast16, int rows, int piece_bytes) {
    const int ppr = piece_bytes / 16 + 2;
    return per_wg >= 1 && per_wg <= kProbeThreads * kWLoads && bcast16 >= 1 && bcast16 <= kProbeThreads * kBLoads &&
           rows >= 1 && piece_bytes >= 1 && int64_t(rows) * ppr <= kProbeThreads * kPLoads;
}

hipError_t launch_read_ceiling(const void* stream_buf, int per_wg, const void* b0, const void* b1, int bcast16,
                               const void* pieces, int rows, int row_bytes, int piece_bytes, int wgs,
                               uint32_t* sink, hipStream_t s) {
    ReadArgs a{};
    a.stream = static_cast<const uint4*>(stream_buf);
    a.per_wg = per_wg;
    a.b0 = static_cast<const uint4*>(b0);
    a.b1 = static_cast<const uint4*>(b1);
    a.bcast16 = bcast16;
    a.pieces = static_cast<const unsigned char*>(pieces);
    a.rows = rows;
    a.row_bytes = row_bytes;
    a.piece_bytes = piece_bytes;
    a.sink = sink;
    read_ceiling_kernel<<<dim3(wgs), dim3(kProbeThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace fdec
