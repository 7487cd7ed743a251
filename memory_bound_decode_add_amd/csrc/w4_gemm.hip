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
// GEMM tiling.  A workgroup of 8 waves (two per SIMD) computes a 128-row x 160-column
// tile of y (at M = 2048, N = 2560: 16 x 16 = 256 workgroups, one per CU), looping over K
// one 128-wide group at a time.  Each group's raw bytes -- the 128 x 128 bf16 activation
// block in k order, the 160 columns' packed words and their 160 scales -- go straight from
// global memory into one of three LDS slots with global_load_lds_dwordx4 (a lane's 16
// bytes land at the wave load's slot address plus 16 x lane).  No register holds them in
// flight, and the loads of groups g + 1 and g + 2 stay outstanding while group g is
// multiplied.  Rows and columns are padded by one 16-byte chunk (lanes that land on a pad
// re-read a chunk of their row), which keeps the operand reads free of bank conflicts.
// Per group, after one barrier, a wave reads all its operands from the slot in one batch
// and issues the loads of group g + 2 into the slot every wave has finished with.
// Wave (wr, wc), wr = 0..3, wc = 0..1, owns rows 32 wr .. 32 wr + 31 (2 row tiles of 16)
// and columns 80 wc .. 80 wc + 79 (5 column tiles).  Per group and k-step it
//   - permutes its 2 activation operands to the int4 pair order (e0, e4, e1, e5, e2, e6,
//     e3, e7): four byte permutes per 16 bytes;
//   - decodes its 5 weight words into eight exact bf16 values 136 + q each, in pair order:
//     a 4-bit field of offset-binary q + 8 in the mantissa of bf16 128 (0x4300), field j
//     of the word shifted to bits 0..3 and 16..19 (three shifts and four v_bitop3_b32 per
//     word);
//   - issues 10 v_mfma_f32_16x16x32_bf16.
// The offset is removed inside the matrix cores: per row tile, a chain of four MFMAs with
// a constant -136 operand forms -136 * sum_k act, which starts each product chain of the
// group.  The group's fp32 sums are scaled by the group scale once and added to the
// running tile (fp32); the epilogue applies the output scale and residual and rounds to
// bf16 once.  The MFMA k-slots are permuted so that lane (lm, ls) takes word 4 ls + ks of
// its column in k-step ks (one 16-byte chunk per column and group) against activation
// k = 32 ls + 8 ks .. + 7.  The operand layout is that of the GEMV kernels: lane l
// supplies A[l%16][8(l/16)+e] (weights, row = column n), B[8(l/16)+e][l%16] (activation,
// column = row m), and holds D[4(l/16)+r][l%16].
// Measured at 2048 x 9216 x 2560: 147-151 us.  The same tiling staged through registers
// (one group ahead, decoded once per workgroup into LDS) took 162 us, and with 4 waves of
// 64 x 80 (one per SIMD) 184 us; this ring with 4 waves of 64 x 80 took 154 us.
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
constexpr int kRT = 2;                  // row tiles of 16 per wave (32 rows)
constexpr int kGColTiles = 5;           // per wave (80 columns)

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

constexpr int kRActCPR = 17;                          // 16-byte chunks per padded activation row
constexpr int kRActLoads = kGBM * kRActCPR / 64;      // wave loads of a slot's activation: 34
constexpr int kRWCPC = 5;                             // 16-byte chunks per padded weight column
constexpr int kRWLoads = (kGBN * kRWCPC + 63) / 64;   // 13 (the last one partly past the 800 chunks)
constexpr int kRActBytes = kRActLoads * 1024;
constexpr int kRWBytes = kRWLoads * 1024;
constexpr int kRSlotBytes = kRActBytes + kRWBytes + 1024;          // + the scales' wave load
constexpr int kRSlots = 3;
constexpr size_t kRLdsBytes = size_t(kRSlots) * kRSlotBytes;
constexpr int kRLoads = kRActLoads + kRWLoads + 1;    // 48 wave loads per group ...
constexpr int kRLoadsPerWave = kRLoads / 8;           // ... six per wave
static_assert(kRLoads % 8 == 0 && kGBM * kRActCPR % 64 == 0, "every wave issues the same loads per group");
static_assert(kRLdsBytes <= 160 * 1024, "three slots fit LDS");

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only the vector-memory count limited (gfx9 encoding: vmcnt in bits 3..0
// and 15..14, expcnt 6..4 and lgkmcnt 11..8 left at their maxima)
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// The wave loads of a group: wave load q = wave + 8 j; q < 34 the activation, then 13
// of weights, then the scales; lane l covers chunk 64 q' + l of its region (addresses
// clamped inside the tensors; what lands on a pad or past the 160 columns is never read).
// A lane's byte offset from its region's base is the same for every group, so it is
// computed once; the bases are workgroup-uniform and advance by one group per step.
struct RingLoads {
    static constexpr int kPerWave = kRLoadsPerWave;
    uint32_t off[kPerWave];      // the lane's byte offset from its region's base, per load
    __device__ __forceinline__ RingLoads(const GemmArgs& a, int m0, int n0, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int q = wave + 8 * j;
            if (q < kRActLoads) {
                const int p = 64 * q + lane, r = p / kRActCPR, c = min(p % kRActCPR, 15);
                off[j] = uint32_t((min(m0 + r, a.M - 1) - m0) * uint32_t(a.lda) * 2u + uint32_t(c) * 16u);
            } else if (q < kRActLoads + kRWLoads) {
                const int p = 64 * (q - kRActLoads) + lane;
                const int col = min(p / kRWCPC, kGBN - 1), c = min(p % kRWCPC, 3);
                off[j] = uint32_t((min(n0 + col, a.N - 1) - n0) * uint32_t(a.nch) * 16u + uint32_t(c) * 16u);
            } else {
                off[j] = uint32_t((min(n0 + 8 * min(lane, kGBN / 8 - 1), a.N - 8) - n0) * 2);
            }
        }
    }
    __device__ __forceinline__ void issue(const GemmArgs& a, unsigned char* dst_slot, int g, int m0, int n0,
                                          int wave) const {
        const char* xb = reinterpret_cast<const char*>(a.x + size_t(m0) * a.lda) + size_t(g) * 256;
        const char* wb = reinterpret_cast<const char*>(a.qw + size_t(n0) * a.nch) + size_t(g) * 64;
        const char* sb = reinterpret_cast<const char*>(a.sc + size_t(g) * a.N + n0);
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int q = wave + 8 * j;
            const char* base;
            unsigned char* dst;
            if (q < kRActLoads) {
                base = xb;
                dst = dst_slot + q * 1024;
            } else if (q < kRActLoads + kRWLoads) {
                base = wb;
                dst = dst_slot + kRActBytes + (q - kRActLoads) * 1024;
            } else {
                base = sb;
                dst = dst_slot + kRActBytes + kRWBytes;
            }
            __builtin_amdgcn_global_load_lds(base + off[j], (lds_void_t*)dst, 16, 0, 0);
        }
    }
};

// One step of the ring: the loads of group g_next (if >= 0) into nxt, then the products of
// the group in cur.  cur and nxt are distinct slots; declaring them restrict lets the
// compiler see that the reads of cur need not wait for the loads into nxt.
__device__ __forceinline__ void ring_step(const GemmArgs& a, const RingLoads& ld,
                                          const unsigned char* __restrict__ cur, unsigned char* __restrict__ nxt,
                                          int g_next, int m0, int n0, int wave, int lane,
                                          f32x4_t (&out)[kRT][kGColTiles]) {
    const int ls = lane >> 4, lm = lane & 15;
    const int wr = wave >> 1, wc = wave & 1;
    // MFMA k-slot order: lane (lm, ls) takes word 4 ls + ks of its column in k-step ks, so
    // its four weight words are one 16-byte chunk and its activation operands are the 32
    // consecutive values from k = 32 ls
    const uint16_t* as = reinterpret_cast<const uint16_t*>(cur) + (16 * kRT * wr + lm) * (kRActCPR * 8) + 32 * ls;
    const uint4* wsp = reinterpret_cast<const uint4*>(cur + kRActBytes) + (80 * wc + lm) * kRWCPC + ls;
    const uint16_t* ssp = reinterpret_cast<const uint16_t*>(cur + kRActBytes + kRWBytes) + 80 * wc + 4 * ls;
    // every LDS read of the group in one batch, then the next loads, then the arithmetic
    uint4 wq[kGColTiles], araw[4][kRT];
    uint2 sq[kGColTiles];
#pragma unroll
    for (int c = 0; c < kGColTiles; ++c) wq[c] = wsp[c * 16 * kRWCPC];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int r = 0; r < kRT; ++r) araw[ks][r] = *reinterpret_cast<const uint4*>(as + r * 16 * (kRActCPR * 8) + 8 * ks);
#pragma unroll
    for (int c = 0; c < kGColTiles; ++c) sq[c] = *reinterpret_cast<const uint2*>(ssp + 16 * c);
    if (g_next >= 0) ld.issue(a, nxt, g_next, m0, n0, wave);
    __builtin_amdgcn_sched_barrier(0);

    const uint32_t m136 = 0xC308C308u;                  // bf16 -136 in each half
    const bf16x8_t negoff = __builtin_bit_cast(bf16x8_t, make_uint4(m136, m136, m136, m136));
    // the offset sums -136 * sum_k act (one chain per row tile) start the products' chains:
    // no separate add per output element
    bf16x8_t bop[4][kRT];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int r = 0; r < kRT; ++r) bop[ks][r] = __builtin_bit_cast(bf16x8_t, to_pair_order(araw[ks][r]));
    f32x4_t bias[kRT];
#pragma unroll
    for (int r = 0; r < kRT; ++r) {
        bias[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            bias[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(negoff, bop[ks][r], bias[r], 0, 0, 0);
    }
    f32x4_t d[kRT][kGColTiles];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int c = 0; c < kGColTiles; ++c) {
            const uint32_t w = ks == 0 ? wq[c].x : ks == 1 ? wq[c].y : ks == 2 ? wq[c].z : wq[c].w;
            const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, decode_bf16x8_biased(w, a.dm.lo));
#pragma unroll
            for (int r = 0; r < kRT; ++r)
                d[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[ks][r], ks == 0 ? bias[r] : d[r][c], 0, 0, 0);
        }
    }
#pragma unroll
    for (int c = 0; c < kGColTiles; ++c) {
        const float s0 = bf16_lo(sq[c].x), s1 = bf16_hi(sq[c].x), s2 = bf16_lo(sq[c].y), s3 = bf16_hi(sq[c].y);
#pragma unroll
        for (int r = 0; r < kRT; ++r) {
            out[r][c][0] = fmaf(s0, d[r][c][0], out[r][c][0]);
            out[r][c][1] = fmaf(s1, d[r][c][1], out[r][c][1]);
            out[r][c][2] = fmaf(s2, d[r][c][2], out[r][c][2]);
            out[r][c][3] = fmaf(s3, d[r][c][3], out[r][c][3]);
        }
    }
}

__global__ __launch_bounds__(kGThreads) void w4_gemm_kernel(GemmArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    // the wave index as a scalar, so that everything derived from it (which loads a wave
    // issues, where they land) is computed once per wave
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int ls = lane >> 4, lm = lane & 15;
    const int wr = wave >> 1, wc = wave & 1;
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int nt = lb % a.ntiles, mt = lb / a.ntiles;
    const int m0 = mt * kGBM, n0 = nt * kGBN;

    f32x4_t out[kRT][kGColTiles];
#pragma unroll
    for (int r = 0; r < kRT; ++r)
#pragma unroll
        for (int c = 0; c < kGColTiles; ++c) out[r][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const RingLoads ld(a, m0, n0, wave, lane);
    ld.issue(a, smem, 0, m0, n0, wave);
    if (a.groups > 1) ld.issue(a, smem + kRSlotBytes, 1, m0, n0, wave);
    for (int g = 0; g < a.groups; ++g) {
        // this wave's loads of group g have landed (those of g + 1 may still be in flight);
        // the barrier makes every wave's visible, and it follows every wave's reads of the
        // slot that group g + 2 reuses.  A plain s_barrier: a fence here would also wait
        // for the loads still in flight.  The signal fences (compiler-only, no instruction)
        // keep the compiler from moving LDS accesses across it.
        if (g + 1 < a.groups)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(kRLoadsPerWave));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        ring_step(a, ld, smem + (g % kRSlots) * kRSlotBytes, smem + ((g + 2) % kRSlots) * kRSlotBytes,
                  g + 2 < a.groups ? g + 2 : -1, m0, n0, wave, lane, out);
    }

    const float os = a.out_scale ? *a.out_scale : 1.0f;
#pragma unroll
    for (int r = 0; r < kRT; ++r) {
        const int m = m0 + 16 * kRT * wr + 16 * r + lm;
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

size_t w4_gemm_lds_bytes() { return kRLdsBytes; }

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
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(kRLdsBytes));
    if (e != hipSuccess) return e;
    w4_gemm_kernel<<<dim3(unsigned(wgs)), kGThreads, kRLdsBytes, s>>>(a);
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
