// int4 group-quantised GEMV for 5..16 rows on the matrix cores, with every operand
// streamed into LDS by direct-to-LDS loads ahead of its use, gfx950.
//
// Same operation as the other int4 kernels ("PyTorch Community Proposes Fusion Fix as
// Large Intermediate Buffers May Slow Single-Token Decoding in Quantized LLMs"; "Kernel
// Fusion, torch.compile and CUDA Graphs, Measured", Step 3):
//     y[m, n] = bf16( s * sum_k act[m, k] * q[k, n] * scale[k/128, n]  (+ res[m, n]) )
// with act = silu(g) * u (SwiGLU prologue) or act = x (identity prologue); in pair mode
// (the gate_up projection with the SwiGLU epilogue, N = 2 I) the output is
// act[m][i] = bf16(silu(sum of column i) * sum of column I + i).
//
// Why a third matrix-core kernel.  The row-block kernel stages its whole K slice of the
// activation in LDS before it requests a weight, and holds weight loads at most two
// batches deep in registers; at the large projections of a 16-row layer the staging
// alone is 4-7 us in which no weight byte moves.  Here nothing is staged up front: the
// slice is walked in steps of two 128-wide groups, and each step's operands are requested
// D steps before its products.
//
// Work assignment (as the row-block kernel).  A workgroup of 8 waves owns 8 tiles of 16
// columns, one per wave (pair mode: waves 0-3 take the gate tiles of its P = 64 column
// pairs, waves 4-7 the matching up tiles), over a K slice of whole groups.
//
// Per step and wave, into a ring of D slots private to the wave (global_load_lds, a
// lane's 16 bytes land at the slot base + 16 lane; a lane reads back only what it loaded,
// so each wave waits on its own vector-memory count and no barrier guards the ring):
//   - activation: 1 KB of g (and 1 KB of u with SwiGLU): thread t = 64 wave + lane takes
//     row t / 32, k-block t % 32 (8 values) of the step's 16 x 256 values;
//   - weights: its tile's two groups as two 1 KB loads of 8 columns x 128 bytes (one
//     column's two groups are 128 consecutive bytes: a load covers whole 128-byte lines;
//     gathering 16 columns x 64 bytes per load measured 3.9-4.8 TB/s against 5.2-5.3 in a
//     streaming probe at the 16-row projections' shapes).  The 8 lanes of a column take its
//     eight 16-byte pieces rotated by the column index, and the second load lands 128 bytes
//     further, so the MFMA operand reads (16 columns of one piece) hit 16 distinct 16-byte
//     bank groups;
//   - scales: its tile's 16 bf16 scales of both groups (lanes 0-15, 4 bytes each).
// One step before its products, each thread converts its 8 activation values (SiLU in
// fp32) into block-scaled fp16 exactly as the row-block kernel stages them and writes them
// to one of three shared slots; one barrier per step publishes them.  LDS holds D steps
// of operands and three steps of staged activation, not the slice's activation, so a
// 16-row, 4096-wide slice needs no K split.
//
// Products.  v_mfma_f32_16x16x32_f16 with A = the decoded weights (fp16 1032 + q /
// 1152 + 16 q in pair order), B = the staged activation; each group's chain starts from
// the group's offset sum per row (-1032 / -1152 times the staged values, summed when the
// step is converted and published with its power of two), which removes the offsets.
// (That sum is the same for every column: formed once per step instead of by four MFMAs
// of a constant matrix in every wave, which were half of the kernel's MFMAs.)  The group's bf16 scale times the row's
// power of two multiplies the group's result once.
//
// Epilogue.  One K slice: the output (residual and scale) or, in pair mode, the up waves
// hand their sums to the gate waves through LDS.  Several slices: fp32 partial sums
// [slice][16][columns] with plain stores, summed in slice order by the finish kernels.
#include "device_common.h"
#include "fdec_internal.h"

#include <algorithm>

namespace fdec {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kRgWaves = 8;
constexpr int kRgThreads = kRgWaves * kWave;
constexpr int kRgPairs = kRgWaves / 2 * 16;            // column pairs per workgroup, pair mode
constexpr int kRgRowBlocks = 33;                        // 16-byte blocks per staged row: 32 + a pad
constexpr int kRgActBytes = 16 * kRgRowBlocks * 16;     // one staged step: 16 rows
constexpr int kRgActSlot = kRgActBytes + 2 * 16 * 2 * 4;   // + per (row, group): power of two, offset sum
constexpr int kRgActSlots = 3;

// s_waitcnt with only one count limited (gfx9 encoding: vmcnt in bits 3..0 and 15..14,
// expcnt 6..4, lgkmcnt 11..8; the others at their maxima)
constexpr int waitcnt_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

template <int PRO>
struct RgShape {
    static constexpr int kActLoads = PRO == kSwiGLU ? 2 : 1;   // per wave and step
    static constexpr int kOps = kActLoads + 3;                 // + two weight loads + the scales
    static constexpr int kWBytes = 2 * 1024 + 128;              // two weight loads + the pad
    static constexpr int kSlot = kActLoads * 1024 + kWBytes + 256;
    static constexpr int kDepth = PRO == kSwiGLU ? 3 : 4;      // steps in flight (LDS bound)
    static constexpr int kBytes = kRgActSlots * kRgActSlot + kRgWaves * kDepth * kSlot;
};
static_assert(RgShape<kSwiGLU>::kBytes <= 160 * 1024 && RgShape<kIdentity>::kBytes <= 160 * 1024, "fits LDS");

struct RgArgs {
    const uint16_t* a0;     // g (SwiGLU) or x (identity), row stride lda
    const uint16_t* a1;     // u (SwiGLU) or unused
    int64_t lda;
    const uint4* qw;        // [N][K/32] chunks of 4 words
    const uint16_t* sc;     // bf16 scales [K/128][N]
    int M, N;
    int nch;                // K / 32
    int groups;             // K / 128
    int kgroups;            // groups per K slice
    int cgroups;            // column ranges (workgroups per slice)
    int npad;               // columns of a slice's partial sums
    int splits;
    const float* out_scale;
    const uint16_t* residual;
    uint16_t* y;            // [M][N], or act [M][I] in pair mode
    float* partial;         // [splits][16][npad]
    DecodeMasks dm;
    int half_n;             // pair mode: I
};

// Waits until at most k steps of OPS loads each are still in flight (k <= 3).
template <int OPS>
__device__ __forceinline__ void wait_steps(int k) {
    if (k >= 3)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * OPS));
    else if (k == 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * OPS));
    else if (k == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(OPS));
    else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// The workgroup barrier without the vector-memory wait __syncthreads implies (loads of
// later steps stay in flight); LDS writes are complete first.  The signal fences are
// compiler-only: no LDS access moves across them.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 8 consecutive activation values of one row -> fp16 in pair order with the odd
// positions / 16, block-scaled by 2^-E per (row, group); the 16 lanes of a DPP row hold
// the 16 k-blocks of one (row, group).  *esc = 2^E.  Whole wave active.
template <int PRO>
__device__ __forceinline__ uint4 stage8(uint4 gv, uint4 uv, float* esc) {
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
    float v[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        if (PRO == kSwiGLU) {
            v[2 * h] = silu_f32(bf16_lo(gw[h])) * bf16_lo(uw[h]);
            v[2 * h + 1] = silu_f32(bf16_hi(gw[h])) * bf16_hi(uw[h]);
        } else {
            v[2 * h] = bf16_lo(gw[h]);
            v[2 * h + 1] = bf16_hi(gw[h]);
        }
    }
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[j]));
    return stage_pair_order(v, stage_group_scale(mx, esc));
}

// The lane's fixed parts of its loads: byte offsets from per-step bases.
struct RgLane {
    uint32_t aoff;          // activation: row * lda * 2 + k-block * 16 within a group pair
    uint32_t woff[2];       // weight load b: column * nch * 16 + chunk-in-group * 16
    uint32_t soff;          // scales: column * 2
    uint32_t rd[2];         // byte offsets in the slot's weights of the A operands of group h
    bool ah;                // activation of the step's second group
    bool wh;                // weight piece of the step's second group
    bool sh;                // scales of the step's second group
};

// Issues step s's loads (groups gA, gB of the slice, clamped) into ring slot dst.
template <int PRO>
__device__ __forceinline__ void rg_issue(const RgArgs& a, const RgLane& ln, int gA, int gB,
                                         unsigned char* __restrict__ dst) {
    const int ga = ln.ah ? gB : gA;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(a.a0) + size_t(ga) * 256 + ln.aoff,
                                     (lds_void_t*)dst, 16, 0, 0);
    if (PRO == kSwiGLU)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(a.a1) + size_t(ga) * 256 + ln.aoff,
                                         (lds_void_t*)(dst + 1024), 16, 0, 0);
    unsigned char* wd = dst + RgShape<PRO>::kActLoads * 1024;
    const char* wb = reinterpret_cast<const char*>(a.qw) + size_t(ln.wh ? gB : gA) * 64;
    __builtin_amdgcn_global_load_lds(wb + ln.woff[0], (lds_void_t*)wd, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(wb + ln.woff[1], (lds_void_t*)(wd + 1024 + 128), 16, 0, 0);
    const int gs = ln.sh ? gB : gA;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(a.sc) + size_t(gs) * a.N * 2 + ln.soff,
                                     (lds_void_t*)(wd + RgShape<PRO>::kWBytes), 4, 0, 0);
}

// One step: convert the next step's activation (raw in rnext, to anext), read this step's
// weights and scales (wcur), issue the loads of step s + D into the slot just read (nxt
// is the same slot as wcur's; its reads complete first), publish, then the products with
// the staged activation of this step (acur).  Distinct restrict pointers tell the
// compiler that the reads here do not wait for the loads in flight.
template <int PRO>
__device__ __forceinline__ void rg_step(const RgArgs& a, const RgLane& ln, int tid, int lane,
                                        const unsigned char* __restrict__ rnext, unsigned char* __restrict__ anext,
                                        bool convert,
                                        const unsigned char* __restrict__ wcur, unsigned char* __restrict__ nxt,
                                        int issue_gA, int issue_gB, const unsigned char* __restrict__ acur,
                                        float e_valid0, float e_valid1, f32x4_t& out) {
    const int ls = lane >> 4, lm = lane & 15;
    if (convert) {
        const uint4 gv = reinterpret_cast<const uint4*>(rnext)[lane];
        const uint4 uv = PRO == kSwiGLU ? reinterpret_cast<const uint4*>(rnext + 1024)[lane] : make_uint4(0, 0, 0, 0);
        float esc;
        const uint4 h = stage8<PRO>(gv, uv, &esc);
        const float off = staged_offset_sum16(h);
        const int row = tid >> 5, kb = tid & 31;
        reinterpret_cast<uint4*>(anext)[row * kRgRowBlocks + kb] = h;
        if ((kb & 15) == 0) reinterpret_cast<float2*>(anext + kRgActBytes)[row * 2 + (kb >> 4)] = make_float2(esc, off);
    }
    const unsigned char* wq = wcur + RgShape<PRO>::kActLoads * 1024;
    const uint4 w0 = *reinterpret_cast<const uint4*>(wq + ln.rd[0]);
    const uint4 w1 = *reinterpret_cast<const uint4*>(wq + ln.rd[1]);
    const uint2 s0 = reinterpret_cast<const uint2*>(wq + RgShape<PRO>::kWBytes)[ls];        // group 0, columns 4 ls ..
    const uint2 s1 = reinterpret_cast<const uint2*>(wq + RgShape<PRO>::kWBytes + 32)[ls];   // group 1
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (issue_gA >= 0) rg_issue<PRO>(a, ln, issue_gA, issue_gB, nxt);
    lds_barrier();

    const uint4* as = reinterpret_cast<const uint4*>(acur) + lm * kRgRowBlocks + 4 * ls;
    f16x8_t b0[4], b1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        b0[j] = __builtin_bit_cast(f16x8_t, as[j]);
        b1[j] = __builtin_bit_cast(f16x8_t, as[16 + j]);
    }
    const float4 es = reinterpret_cast<const float4*>(acur + kRgActBytes)[lm];   // (esc, off) of groups 0, 1
    const float e0 = es.x * e_valid0, e1 = es.z * e_valid1;
    f32x4_t d0 = {es.y, es.y, es.y, es.y}, d1 = {es.w, es.w, es.w, es.w};
    const uint32_t wa[4] = {w0.x, w0.y, w0.z, w0.w}, wb[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, decode_int4x8_biased(wa[j], a.dm)),
                                                    b0[j], d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, decode_int4x8_biased(wb[j], a.dm)),
                                                    b1[j], d1, 0, 0, 0);
    }
    out[0] = fmaf(bf16_lo(s0.x) * e0, d0[0], out[0]);
    out[1] = fmaf(bf16_hi(s0.x) * e0, d0[1], out[1]);
    out[2] = fmaf(bf16_lo(s0.y) * e0, d0[2], out[2]);
    out[3] = fmaf(bf16_hi(s0.y) * e0, d0[3], out[3]);
    out[0] = fmaf(bf16_lo(s1.x) * e1, d1[0], out[0]);
    out[1] = fmaf(bf16_hi(s1.x) * e1, d1[1], out[1]);
    out[2] = fmaf(bf16_lo(s1.y) * e1, d1[2], out[2]);
    out[3] = fmaf(bf16_hi(s1.y) * e1, d1[3], out[3]);
}

// The first min(D, nsteps) steps' loads, then step 0's activation converted into the
// first shared slot.  Slot 0 and the later slots are distinct restrict pointers, so the
// conversion waits for step 0's loads only.
template <int PRO>
__device__ __forceinline__ void rg_prologue(const RgArgs& a, const RgLane& ln, int tid, int lane, int g0, int ng,
                                            int npre, unsigned char* __restrict__ slot0,
                                            unsigned char* __restrict__ later, unsigned char* __restrict__ act0) {
    rg_issue<PRO>(a, ln, g0, g0 + min(1, ng - 1), slot0);
    for (int s = 1; s < npre; ++s)
        rg_issue<PRO>(a, ln, g0 + min(2 * s, ng - 1), g0 + min(2 * s + 1, ng - 1), later + (s - 1) * RgShape<PRO>::kSlot);
    wait_steps<RgShape<PRO>::kOps>(npre - 1);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint4 gv = reinterpret_cast<const uint4*>(slot0)[lane];
    const uint4 uv = PRO == kSwiGLU ? reinterpret_cast<const uint4*>(slot0 + 1024)[lane] : make_uint4(0, 0, 0, 0);
    float esc;
    const uint4 h = stage8<PRO>(gv, uv, &esc);
    const float off = staged_offset_sum16(h);
    const int row = tid >> 5, kb = tid & 31;
    reinterpret_cast<uint4*>(act0)[row * kRgRowBlocks + kb] = h;
    if ((kb & 15) == 0) reinterpret_cast<float2*>(act0 + kRgActBytes)[row * 2 + (kb >> 4)] = make_float2(esc, off);
}

template <int PRO, bool PAIR>
__global__ __launch_bounds__(kRgThreads) void w4_gemv_ring_kernel(RgArgs a) {
    using S = RgShape<PRO>;
    constexpr int D = S::kDepth;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ls = lane >> 4, lm = lane & 15;
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int cg = lb % a.cgroups, split = lb / a.cgroups;
    const int g0 = split * a.kgroups;
    const int ng = min(a.kgroups, a.groups - g0);      // groups in this slice
    const int nsteps = (ng + 1) >> 1;
    const bool up = PAIR && wave >= kRgWaves / 2;
    const int wl = up ? wave - kRgWaves / 2 : wave;
    // the wave's column offset in the workgroup's range, and its first column
    const int col_local = PAIR ? (up ? kRgPairs : 0) + wl * 16 : wave * 16;
    const int c0 = PAIR ? (up ? a.half_n : 0) + cg * kRgPairs + wl * 16 : cg * (kRgWaves * 16) + col_local;
    unsigned char* ring = smem + kRgActSlots * kRgActSlot + wave * (D * S::kSlot);

    RgLane ln;
    {
        const int row = min(tid >> 5, a.M - 1), kb = tid & 31;
        ln.aoff = uint32_t(row) * uint32_t(a.lda) * 2u + uint32_t(kb & 15) * 16u;
        ln.ah = kb >= 16;
        // weight load b: lane l takes column 8 b + l / 8 of the tile, piece p = (l % 8 - l / 8)
        // mod 8 of its 128 bytes (group p / 4 of the step, chunk p % 4); piece p of column c
        // thus sits at lane 8 (c % 8) + (p + c) % 8 of load c / 8
        {
            const int cc = lane >> 3, pc = ((lane & 7) - cc) & 7;
            for (int b = 0; b < 2; ++b)
                ln.woff[b] = uint32_t(min(c0 + 8 * b + cc, a.N - 1)) * uint32_t(a.nch) * 16u + uint32_t(pc & 3) * 16u;
            ln.wh = pc >= 4;
            for (int h = 0; h < 2; ++h) {
                const int p = 4 * h + ls, cw = lm & 7;
                ln.rd[h] = uint32_t((lm >> 3) * (1024 + 128) + 16 * (8 * cw + ((p + cw) & 7)));
            }
        }
        ln.soff = uint32_t(min(c0 + 2 * (lane & 7), a.N - 2)) * 2u;
        ln.sh = (lane >> 3) & 1;
    }
    auto gsel = [&](int s, int h) { return g0 + min(2 * s + h, ng - 1); };

    // epilogue inputs, requested first (they complete before any step's loads)
    uint2 rraw = make_uint2(0u, 0u);
    if (!PAIR && a.splits == 1 && a.residual)
        rraw = *reinterpret_cast<const uint2*>(a.residual + size_t(min(lm, a.M - 1)) * a.N + min(c0 + 4 * ls, a.N - 4));
    const float os = a.out_scale ? *a.out_scale : 1.0f;

    // prologue: steps 0 .. D - 1 requested, step 0 converted
    rg_prologue<PRO>(a, ln, tid, lane, g0, ng, min(D, nsteps), ring, ring + S::kSlot, smem);
    lds_barrier();

    f32x4_t out = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsteps; ++s) {
        // steps <= s + 1 have landed once no more than `later` steps are in flight
        wait_steps<S::kOps>(max(0, min(s + D - 1, nsteps - 1) - (s + 1)));
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const bool cv = s + 1 < nsteps;
        const int sn = cv ? s + 1 : s;
        const bool iss = s + D < nsteps;
        // a step's second group past the slice's end re-reads its last group and is
        // weighted 0 in the products
        rg_step<PRO>(a, ln, tid, lane, ring + (sn % D) * S::kSlot, smem + (sn % kRgActSlots) * kRgActSlot, cv,
                     ring + (s % D) * S::kSlot, ring + (s % D) * S::kSlot,
                     iss ? gsel(s + D, 0) : -1, iss ? gsel(s + D, 1) : -1, smem + (s % kRgActSlots) * kRgActSlot,
                     1.0f, 2 * s + 1 < ng ? 1.0f : 0.0f, out);
    }

    // ---- epilogue: lane holds D[column 4 ls + q][row lm] of the wave's tile ----
    if (a.splits > 1) {
        float* dst = a.partial + (size_t(split) * 16 + lm) * a.npad + cg * (kRgWaves * 16) + col_local + 4 * ls;
        *reinterpret_cast<float4*>(dst) = make_float4(out[0], out[1], out[2], out[3]);
        return;
    }
    if (PAIR) {
        // the up waves hand their sums to the gate waves through LDS (free once every wave
        // has passed the barrier after its last products)
        float4* xs = reinterpret_cast<float4*>(smem);
        __syncthreads();
        if (up) xs[wl * kWave + lane] = make_float4(out[0], out[1], out[2], out[3]);
        __syncthreads();
        if (!up) {
            const float4 u = xs[wl * kWave + lane];
            const int i = c0 + 4 * ls;                  // four pairs i .. i + 3 (I % 8 == 0)
            if (lm < a.M && i < a.half_n) {
                uint2 o;
                o.x = pack_bf16x2(silu_f32(out[0]) * u.x, silu_f32(out[1]) * u.y);
                o.y = pack_bf16x2(silu_f32(out[2]) * u.z, silu_f32(out[3]) * u.w);
                *reinterpret_cast<uint2*>(a.y + size_t(lm) * a.half_n + i) = o;
            }
        }
        return;
    }
    const int n = c0 + 4 * ls;
    if (lm < a.M && n < a.N) {
        const float r0 = a.residual ? bf16_lo(rraw.x) : 0.f, r1 = a.residual ? bf16_hi(rraw.x) : 0.f;
        const float r2 = a.residual ? bf16_lo(rraw.y) : 0.f, r3 = a.residual ? bf16_hi(rraw.y) : 0.f;
        uint2 o;
        o.x = pack_bf16x2(fmaf(out[0], os, r0), fmaf(out[1], os, r1));
        o.y = pack_bf16x2(fmaf(out[2], os, r2), fmaf(out[3], os, r3));
        *reinterpret_cast<uint2*>(a.y + size_t(lm) * a.N + n) = o;
    }
}

template <typename Kern>
hipError_t launch_rg(Kern k, int wgs, size_t lds, hipStream_t s, const RgArgs& a) {
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(wgs), dim3(kRgThreads), lds, s, a);
    return hipGetLastError();
}

// K slices toward 256 workgroups when the column ranges alone give fewer than 192.
// Slices of an even number of groups, so that every step's two groups of a column are
// one 128-byte-aligned piece when K / 128 is even.
void ring_slices(int groups, int ranges, GemvPlan& p) {
    const int S = ranges >= 192 ? 1 : std::max(1, std::min(groups, 256 / ranges));
    p.gps = (groups + S - 1) / S;
    p.gps += p.gps & 1;
    p.splits = (groups + p.gps - 1) / p.gps;
}

}  // namespace

// 5..16 rows (one block of 16), K % 128 == 0, N % 8 == 0, byte offsets of the weights
// inside 32 bits.
bool plan_ring(int M, int K, int N, Prologue pro, GemvPlan& p) {
    p = GemvPlan{};
    if (M < 1 || M > 16 || K <= 0 || K % kGroup || N < 8 || N % 8 || int64_t(K) * N / 2 >= (int64_t(1) << 32))
        return false;
    if (pro != kIdentity && pro != kSwiGLU) return false;
    p.kind = kRing;
    p.mr = 16;
    p.groups = K / kGroup;
    p.waves = kRgWaves;
    p.cpw = 1;
    p.tiles = (N + kRgWaves * 16 - 1) / (kRgWaves * 16);
    ring_slices(p.groups, p.tiles, p);
    if (p.splits > 1) p.partial_bytes = size_t(p.splits) * 16 * p.tiles * kRgWaves * 16 * 4;
    p.lds_bytes = pro == kSwiGLU ? RgShape<kSwiGLU>::kBytes : RgShape<kIdentity>::kBytes;
    return true;
}

bool plan_ring_pair(int M, int K, int I, GemvPlan& p) {
    p = GemvPlan{};
    if (M < 1 || M > 16 || K <= 0 || K % kGroup || I < 8 || I % 8 || int64_t(K) * I >= (int64_t(1) << 32))
        return false;
    p.kind = kRing;
    p.mr = 16;
    p.groups = K / kGroup;
    p.waves = kRgWaves;
    p.cpw = 1;
    p.tiles = (I + kRgPairs - 1) / kRgPairs;
    ring_slices(p.groups, p.tiles, p);
    if (p.splits > 1) p.partial_bytes = size_t(p.splits) * 16 * p.tiles * 2 * kRgPairs * 4;
    p.lds_bytes = RgShape<kIdentity>::kBytes;
    return true;
}

hipError_t launch_ring(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda, const uint32_t* qw,
                       const uint16_t* sc, int M, int K, int N, const float* out_scale, const uint16_t* residual,
                       uint16_t* y, void* ws, const GemvPlan& p, hipStream_t s) {
    if (p.kind != kRing || M > 16) return hipErrorInvalidValue;
    RgArgs a{};
    a.a0 = a0;
    a.a1 = pro == kSwiGLU ? a1 : a0;
    a.lda = lda;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.N = N;
    a.nch = K / 32;
    a.groups = p.groups;
    a.kgroups = p.gps;
    a.cgroups = p.tiles;
    a.npad = p.tiles * kRgWaves * 16;
    a.splits = p.splits;
    a.out_scale = out_scale;
    a.residual = residual;
    a.y = y;
    a.partial = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    a.dm = DecodeMasks{kDecodeMaskLo, kDecodeMaskHi};
    const int wgs = p.tiles * p.splits;
    const hipError_t e = pro == kSwiGLU ? launch_rg(w4_gemv_ring_kernel<kSwiGLU, false>, wgs, p.lds_bytes, s, a)
                                        : launch_rg(w4_gemv_ring_kernel<kIdentity, false>, wgs, p.lds_bytes, s, a);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_finish(a.partial, p.splits, int64_t(16) * a.npad, a.npad, M, N, out_scale, residual, y, s);
}

hipError_t launch_ring_pair(const uint16_t* x, const uint32_t* qw, const uint16_t* sc, int M, int K, int I,
                            uint16_t* act, void* ws, const GemvPlan& p, hipStream_t s) {
    if (p.kind != kRing || M > 16) return hipErrorInvalidValue;
    RgArgs a{};
    a.a0 = x;
    a.a1 = x;
    a.lda = K;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.N = 2 * I;
    a.nch = K / 32;
    a.groups = p.groups;
    a.kgroups = p.gps;
    a.cgroups = p.tiles;
    a.npad = p.tiles * 2 * kRgPairs;
    a.splits = p.splits;
    a.y = act;
    a.partial = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    a.dm = DecodeMasks{kDecodeMaskLo, kDecodeMaskHi};
    a.half_n = I;
    const hipError_t e = launch_rg(w4_gemv_ring_kernel<kIdentity, true>, p.tiles * p.splits, p.lds_bytes, s, a);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_finish_swiglu(a.partial, p.splits, int64_t(16) * a.npad, a.npad, M, I, kRgPairs, act, s);
}

}  // namespace fdec
