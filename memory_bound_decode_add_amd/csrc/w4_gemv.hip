// int4 group-quantised GEMV for M = 1..16 rows, with a SwiGLU (or identity) prologue
// and an fp32 output-scale + residual epilogue, gfx950.
//
// What it computes ("PyTorch Community Proposes Fusion Fix as Large Intermediate
// Buffers May Slow Single-Token Decoding in Quantized LLMs"; "Kernel Fusion,
// torch.compile and CUDA Graphs, Measured", Step 3; "PyTorch folds NVFP4 output
// scaling into NVGEMM candidates for decode workloads"):
//     y[m, n] = bf16( s * sum_k act[m, k] * q[k, n] * scale[k/128, n]  (+ res[m, n]) )
// with act = silu(g) * u (SwiGLU prologue) or act = x (identity prologue).  The
// activation exists only in LDS and registers; the (M, K, N) product never exists.
//
// Weights: qweight uint32 [N][K/8] (the K values of a column are contiguous, 8 per
// word), scales bf16 [K/128][N].
//
// Both kernels stage the activation in LDS as block-scaled fp16: a block of values is
// multiplied by a power of two 2^-E chosen from its largest magnitude so that this
// magnitude lands in [2^14, 2^15) (any finite fp32 activation then fits fp16 with an
// 11-bit significand relative to its block's maximum), and 2^E is folded back in with
// the group scale.  Values are stored in the pair order of the int4 decode, so four
// v_dot2_f32_f16 consume one packed word with fp32 accumulation.  Every global load is
// issued before any arithmetic, from addresses clamped into the tensors, activation
// inputs first, so the prologue runs while the weights are still in flight.
//
// Column-owning kernel (M <= 4, K <= 16384).  A workgroup of W waves owns C consecutive
// columns; wave w owns columns w, w + W, ... (at most CPW) over the whole K.  Lane l
// loads the 16-byte chunks (32 consecutive k) l, l+64, ... of each of the wave's
// columns, so one load instruction reads 1 KB of contiguous weights, and one read of
// the staged activation of a chunk serves all of the wave's columns.  The workgroup
// stages the activation of the full K (fp16 blocks of 32, offsets folded per chunk,
// see stage_word_col) and the group scales of its columns in LDS once.  A column's
// sum is reduced across the wave with DPP and scalar lane reads, and one lane applies
// the epilogue.  There is no cross-workgroup step and no workspace; results do not
// depend on scheduling.
//
// Split-K kernel (M <= 16, any K).  A 256-thread workgroup owns a 64-column tile and
// a slice of whole 128-wide groups; wave w owns groups w, w+4, ... of the slice; lane
// (kr = lane % 4, cq = lane / 4) owns columns 4cq..4cq+3 and packed words 4kr..4kr+3
// of each group of those columns.  The activation of a group is staged in blocks of
// 128 (2 values per lane) and the weights are decoded to exact fp16 (XOR, shift, four
// AND-OR and four packed fp16 ops per word).  The quad of lanes sharing columns reduces
// with DPP, the waves through LDS.  With several slices each workgroup writes its fp32
// partials to the workspace with plain stores, and splitk_finish_kernel, launched next
// on the same stream, sums them in slice order and applies the epilogue.
#include "device_common.h"
#include "fdec_internal.h"

#include <algorithm>

namespace fdec {

namespace {

__device__ __forceinline__ float epilogue(float v, float s, const uint16_t* res, size_t idx) {
    v *= s;
    if (res) v += bf16_to_f32(res[idx]);
    return v;
}

// Activation of one (row, group) task, 2 values per lane, to LDS as block-scaled fp16.
// Must be called by a full wave (wave-uniform control flow).
template <int PRO>
__device__ __forceinline__ void stage_act(uint32_t ga, uint32_t ua, bool live, int lane, _Float16* dst128,
                                          float* esc) {
    float v0 = 0.f, v1 = 0.f;
    if (live) {
        if (PRO == kSwiGLU) {
            v0 = silu_f32(bf16_lo(ga)) * bf16_lo(ua);
            v1 = silu_f32(bf16_hi(ga)) * bf16_hi(ua);
        } else {
            v0 = bf16_lo(ga);
            v1 = bf16_hi(ga);
        }
    }
    const float mx = wave_max_uniform(fmaxf(fabsf(v0), fabsf(v1)));
    int e = 0;
    (void)__builtin_frexpf(mx, &e);
    const int E = min(max(e - 15, -126), 127);
    const int k0 = 2 * lane;                      // k within the group
    _Float16* dst = dst128 + (k0 >> 3) * 8;
    dst[pair_slot(k0 & 7)] = (_Float16)__builtin_ldexpf(v0, -E);
    dst[pair_slot((k0 & 7) + 1)] = (_Float16)__builtin_ldexpf(v1, -E);
    if (lane == 0) *esc = __builtin_ldexpf(1.0f, E);
}

// sum over 32 k: four packed words against 64 bytes of staged activation
__device__ __forceinline__ float dot32(const uint4 w, const _Float16* act, DecodeMasks dm) {
    const uint4 a0 = *reinterpret_cast<const uint4*>(act);
    const uint4 a1 = *reinterpret_cast<const uint4*>(act + 8);
    const uint4 a2 = *reinterpret_cast<const uint4*>(act + 16);
    const uint4 a3 = *reinterpret_cast<const uint4*>(act + 24);
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    const uint4 av[4] = {a0, a1, a2, a3};
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const Q4x2 q = decode_int4x8(wd[j], dm);
        v = dot2(q.p04, __builtin_bit_cast(half2_t, av[j].x), v);
        v = dot2(q.p15, __builtin_bit_cast(half2_t, av[j].y), v);
        v = dot2(q.p26, __builtin_bit_cast(half2_t, av[j].z), v);
        v = dot2(q.p37, __builtin_bit_cast(half2_t, av[j].w), v);
    }
    return v;
}

// ===========================================================================
// column-owning kernel
// ===========================================================================
struct ColArgs {
    const uint16_t* a0;     // g (SwiGLU) or x (identity), row stride lda
    const uint16_t* a1;     // u (SwiGLU) or unused
    int64_t lda;
    const uint4* qw;        // [N][K/32] chunks of 4 words
    const uint16_t* sc;     // bf16 scales [K/128][N]
    int M, K, N;
    int nch;                // K / 32
    int groups;             // K / 128
    int cols;               // columns per workgroup (column kernel)
    int stagers;            // staging waves per workgroup (column kernel)
    const float* out_scale;
    const uint16_t* residual;
    uint16_t* y;
    // add + RMSNorm prologue with the SwiGLU pair epilogue (prologue kAddRmsNorm)
    const uint16_t* nw;     // RMSNorm weight [K]
    float eps;
    uint16_t* h_out;        // h = bf16(x + r) [M][K], written by workgroup 0
    int pairs;              // gate/up column pairs per workgroup (cols = 2 * pairs)
    int half_n;             // I = N / 2: column i pairs with column I + i; y is [M][I]
    // side copy of cp_n16 16-byte words, spread over the grid's dot waves
    const uint4* cp_src;
    uint4* cp_dst;
    int cp_n16;
    DecodeMasks dm;         // int4 decode field masks (scalar registers)
};

// Staged activation of the column kernel, per row: fp16 in the layout [quarter q][chunk
// c][8] with a quarter stride of 8*nch + 32 halves; quarter q of chunk c holds k = 32c +
// 8q .. 32c + 8q + 7 in the decode's pair order.  A wave reading quarter q of chunks l,
// l+1, ... (one per lane) touches consecutive 16-byte blocks, and the 64-byte pad
// spreads the staging writes of a quad (one chunk, four quarters) over distinct banks.
//
// The weights are decoded without removing their offsets: a nibble at an even position
// j (bits 0..3 of a half) decodes to 1032 + q, at an odd position (bits 4..7) to
// 1152 + 16 q.  Odd-position activations are staged divided by 16, so each product is
// a*q plus a per-k offset 1032*a or 72*a that does not depend on the weight; the
// staging phase sums those offsets per chunk and the dot phase subtracts them.  Every
// staged value and every product is exact; what changes is that the fp32 sums now also
// carry the offset terms, about 1032/|q| times larger than the wanted ones, so a
// chunk's dot keeps roughly 10 fewer significant bits (relative error ~1e-4).
//
// Staging task: one row and 512 consecutive k; lane l takes the 8 values of packed word
// l of the block (16-byte loads of g and u) and writes them as one 16-byte LDS store.
// The four lanes of a quad hold one 32-wide chunk: they share the chunk's power-of-two
// scale 2^E (its largest magnitude lands in [2^14, 2^15), so no value overflows fp16)
// and sum its offsets; lane 0 of the quad stores (2^E, offset sum) for the chunk.
// fp32 -> fp16 rounds toward zero (one packed conversion per pair); the offsets are
// summed from the rounded values, so they cancel exactly whatever the rounding.
__device__ __forceinline__ int col_quarter_stride(int nch) { return nch * 8 + 32; }

// Which waves load the group scales: the dot waves with three or more 64-chunk ranges per
// lane (long K), the staging waves otherwise (see the kernel).
__host__ __device__ constexpr bool col_dot_scales(int ni) { return ni >= 3; }

// Eight activation values k = 8w + j (j = 0..7) of one lane -> LDS (see above).
// Lanes past K (a quad is wholly inside or outside) store nothing; rows past M stage
// copies of row M - 1 (clamped loads), whose sums no lane stores: neither is zeroed.
__device__ __forceinline__ void stage_values_col(float (&v)[8], bool in_k, bool quad_lead,
                                                 _Float16* dst, float2* eb_dst) {
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[j]));
    mx = fmaxf(mx, dpp<kQuadSwap1>(mx));
    mx = fmaxf(mx, dpp<kQuadSwap2>(mx));           // the chunk's largest magnitude
    int e = 0;
    (void)__builtin_frexpf(mx, &e);
    const int E = min(max(e - 15, -126), 127);
    const float down = __builtin_ldexpf(1.0f, -E);
    const float down16 = down * 0.0625f;
    // slot order (j0, j4, j1, j5, j2, j6, j3, j7); odd j stored divided by 16
    const half2_t p0 = pk_f16_rtz(v[0] * down, v[4] * down);
    const half2_t p1 = pk_f16_rtz(v[1] * down16, v[5] * down16);
    const half2_t p2 = pk_f16_rtz(v[2] * down, v[6] * down);
    const half2_t p3 = pk_f16_rtz(v[3] * down16, v[7] * down16);
    if (in_k)
        *reinterpret_cast<uint4*>(dst) = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
    const half2_t even = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t odd = {(_Float16)1152.0f, (_Float16)1152.0f};
    float b = dot2(p0, even, 0.f);
    b = dot2(p2, even, b);
    b = dot2(p1, odd, b);
    b = dot2(p3, odd, b);
    b += dpp<kQuadSwap1>(b);
    b += dpp<kQuadSwap2>(b);
    if (quad_lead && in_k) *eb_dst = make_float2(__builtin_ldexpf(1.0f, E), b);
}

template <int PRO>
__device__ __forceinline__ void stage_word_col(const uint4 gv, const uint4 uv, bool in_k, bool quad_lead,
                                               _Float16* dst, float2* eb_dst) {
    float v[8];                                    // k = 8w + j, j = 0..7
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
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
    stage_values_col(v, in_k, quad_lead, dst, eb_dst);
}

// Sum over a full wave (all 64 lanes active), returned uniform, in a fixed order.
__device__ __forceinline__ float wave_sum_uniform(float v) {
    v += dpp<kQuadSwap1>(v);
    v += dpp<kQuadSwap2>(v);
    v += dpp<kRowRor4>(v);
    v += dpp<kRowRor8>(v);
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// The workgroup has S + W waves in two roles.
//  * Staging waves 0..S-1: they load the activation inputs and the group scales, stage
//    them in LDS and retire at the barrier.  They are the older waves, so their loads
//    are issued ahead of the weight loads.
//  * Dot waves S..S+W-1: dot wave w owns columns w, w + W, ... below C (at most CPW of
//    them).  It issues its weight loads first thing and, after the barrier, runs the dot.
// Measured on MI355X: a wave that issues many loads stalls at issue behind the CU's
// outstanding requests, and one wave per SIMD issues VALU work at about half rate.
// Split roles keep the staging waves' issue free of weight loads, and give every SIMD
// two waves in each phase.
template <int MR, int CPW, int NI, int PRO>
__global__ __launch_bounds__(16 * kWave) void w4_gemv_col_kernel(ColArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    // With the add + RMSNorm prologue the workgroup owns column pairs (i, I + i): gate
    // and up of the same i, so the epilogue can form silu(gate) * up.
    constexpr bool PAIR = PRO == kAddRmsNorm;
    constexpr int TMAX = PAIR ? kColMaxTasksNorm : kColMaxTasks;
    const int S = a.stagers;                       // staging waves
    const int W = (blockDim.x >> 6) - S;           // dot waves
    const int C = a.cols;                          // columns per workgroup (2 * pairs with PAIR)
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: slot tests branch on scalars
    const int lane = tid & 63;
    const int nblk = (a.K + 511) >> 9;             // 512-wide staging blocks
    const int qs = col_quarter_stride(a.nch);      // halves
    const int kw = a.K >> 3;                       // packed words per row
    _Float16* act_s = reinterpret_cast<_Float16*>(smem);                          // [MR][4][qs]
    float2* eb_s = reinterpret_cast<float2*>(smem + size_t(MR) * 4 * qs * 2);     // [MR][nch]
    float* sc_s = reinterpret_cast<float*>(eb_s + MR * a.nch);                     // [groups][C]
    float* ss_s = sc_s + a.groups * C;                                             // [S][MR]

    // first column (pair) of the workgroup; column of local column slot cj in [0, C)
    const int cbase = xcd_remap(blockIdx.x, gridDim.x) * (PAIR ? a.pairs : C);
    auto column = [&](int cj) {
        if (PAIR) return cj < a.pairs ? cbase + cj : a.half_n + cbase + (cj - a.pairs);
        return cbase + cj;
    };

    // ---- group scales of the workgroup's columns, as aligned 8-column pieces of each
    // group's row.  One column range, or two with PAIR (gate i.., up I + i..): range r
    // covers columns [cb_r, cb_r + n_r) and LDS slots [o_r, o_r + n_r).  Loaded into
    // registers by thread tid0 + r nthr, then written to LDS.  With long K (kDotScales)
    // the dot waves load them ahead of their own weights: cold like the weights, they then
    // land while the activation is staged, where behind the staging waves' activation
    // loads they held the barrier (measured on MI355X at K = 9216, N = 2560: landing
    // ≈ 0.9 us after the staged activation).  With short K the staging waves do it, the
    // dot waves having many columns' weights to request. ----
    const int n0 = PAIR ? a.pairs : C;
    const int cb0 = cbase, cb1 = PAIR ? a.half_n + cbase : 0;
    const int p00 = cb0 >> 3, npc0 = ((min(cb0 + n0, a.N) - 1) >> 3) - p00 + 1;
    const int p01 = cb1 >> 3, npc1 = PAIR ? ((min(cb1 + n0, a.N) - 1) >> 3) - p01 + 1 : 0;
    const int nsc0 = a.groups * npc0, nsc = nsc0 + a.groups * npc1;
    constexpr bool kDotScales = col_dot_scales(NI);
    auto load_scales = [&](uint4 (&sraw)[kColScLoads], int tid0, int nthr) {
#pragma unroll
        for (int r = 0; r < kColScLoads; ++r) {
            if (r * nthr >= nsc) break;            // uniform
            const int idx = min(tid0 + r * nthr, nsc - 1);
            const bool hi = idx >= nsc0;
            const int j = hi ? idx - nsc0 : idx, npc = hi ? npc1 : npc0;
            const int g = j / npc, pc = (hi ? p01 : p00) + j % npc;
            sraw[r] = *reinterpret_cast<const uint4*>(a.sc + size_t(g) * a.N + pc * 8);
        }
    };
    auto write_scales = [&](const uint4 (&sraw)[kColScLoads], int tid0, int nthr) {
#pragma unroll
        for (int r = 0; r < kColScLoads; ++r) {
            if (r * nthr >= nsc) break;
            const int idx = tid0 + r * nthr;
            if (idx < nsc) {
                const bool hi = idx >= nsc0;
                const int j = hi ? idx - nsc0 : idx, npc = hi ? npc1 : npc0;
                const int g = j / npc;
                const int cc0 = ((hi ? p01 : p00) + j % npc) * 8 - (hi ? cb1 : cb0), o = hi ? n0 : 0;
                const uint32_t wd[4] = {sraw[r].x, sraw[r].y, sraw[r].z, sraw[r].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int cc = cc0 + e;
                    if (cc >= 0 && cc < n0) sc_s[g * C + o + cc] = (e & 1) ? bf16_hi(wd[e >> 1]) : bf16_lo(wd[e >> 1]);
                }
            }
        }
    };
    if (wave < S) {
        // ================= staging waves =================
        const int sw = wave;
        // ---- activation inputs: task t = sw + S * ti -> (row t % MR, block t / MR) ----
        const int ntask = MR * nblk;
        uint4 ga[TMAX], ua[TMAX], wa[PAIR ? TMAX : 1];
#pragma unroll
        for (int ti = 0; ti < TMAX; ++ti) {
            const int t = sw + S * ti;
            if (t >= ntask) break;                 // uniform across the wave
            const int m = min(t % MR, a.M - 1), b = t / MR;
            const int k = min(b * 64 + lane, kw - 1) * 8;
            ga[ti] = *reinterpret_cast<const uint4*>(a.a0 + size_t(m) * a.lda + k);
            ua[ti] = PRO != kIdentity ? *reinterpret_cast<const uint4*>(a.a1 + size_t(m) * a.lda + k)
                                      : make_uint4(0, 0, 0, 0);
            if (PAIR) wa[ti] = *reinterpret_cast<const uint4*>(a.nw + k);
        }
        uint4 sraw[kColScLoads];
        if (!kDotScales) load_scales(sraw, tid, S * kWave);
        // ---- activations, per-chunk scale and offsets to LDS ----
        // word wi = 64 b + lane: chunk wi / 4, quarter wi % 4
        const int lofs = (lane & 3) * qs + (lane >> 2) * 8;
        if (PAIR) {
            // h = bf16(x + r) (written out by workgroup 0), then the mean of h^2 over the
            // row: per-wave sums meet in LDS, and every staging wave adds them up in the
            // same order.
            float ssr[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) ssr[m] = 0.f;
#pragma unroll
            for (int ti = 0; ti < TMAX; ++ti) {
                const int t = sw + S * ti;
                if (t >= ntask) break;             // uniform
                const int m = t % MR, b = t / MR;
                const bool in_k = b * 64 + lane < kw;
                const bool live = in_k && m < a.M;
                const uint32_t xw[4] = {ga[ti].x, ga[ti].y, ga[ti].z, ga[ti].w};
                const uint32_t rw[4] = {ua[ti].x, ua[ti].y, ua[ti].z, ua[ti].w};
                uint32_t hw[4];
                float ss = 0.f;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    hw[h] = pack_bf16x2(bf16_lo(xw[h]) + bf16_lo(rw[h]), bf16_hi(xw[h]) + bf16_hi(rw[h]));
                    const float lo = bf16_lo(hw[h]), hi = bf16_hi(hw[h]);
                    ss = fmaf(lo, lo, ss);
                    ss = fmaf(hi, hi, ss);
                }
                ga[ti] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
#pragma unroll
                for (int mm = 0; mm < MR; ++mm) ssr[mm] += (mm == m && live) ? ss : 0.f;
                if (blockIdx.x == 0 && live)
                    *reinterpret_cast<uint4*>(a.h_out + size_t(m) * a.K + (b * 64 + lane) * 8) = ga[ti];
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float tot = wave_sum_uniform(ssr[m]);
                if (lane == 0) ss_s[sw * MR + m] = tot;
            }
            __syncthreads();                       // row sums of squares in LDS
            float rstd[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float tot = 0.f;
                for (int w = 0; w < S; ++w) tot += ss_s[w * MR + m];
                rstd[m] = __builtin_amdgcn_rsqf(fmaf(tot, 1.0f / float(a.K), a.eps));
            }
#pragma unroll
            for (int ti = 0; ti < TMAX; ++ti) {
                const int t = sw + S * ti;
                if (t >= ntask) break;             // uniform
                const int m = t % MR, b = t / MR;
                const bool in_k = b * 64 + lane < kw;
                float rs = rstd[0];
#pragma unroll
                for (int mm = 1; mm < MR; ++mm) rs = mm == m ? rstd[mm] : rs;
                const uint32_t hw[4] = {ga[ti].x, ga[ti].y, ga[ti].z, ga[ti].w};
                const uint32_t ww[4] = {wa[ti].x, wa[ti].y, wa[ti].z, wa[ti].w};
                float v[8];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    v[2 * h] = bf16_lo(hw[h]) * rs * bf16_lo(ww[h]);
                    v[2 * h + 1] = bf16_hi(hw[h]) * rs * bf16_hi(ww[h]);
                }
                stage_values_col(v, in_k, (lane & 3) == 0,
                                 act_s + size_t(m) * 4 * qs + lofs + b * 128,
                                 eb_s + m * a.nch + b * 16 + (lane >> 2));
            }
        } else {
#pragma unroll
            for (int ti = 0; ti < TMAX; ++ti) {
                const int t = sw + S * ti;
                if (t >= ntask) break;             // uniform across the wave
                const int m = t % MR, b = t / MR;
                const bool in_k = b * 64 + lane < kw;  // a chunk lies wholly inside or outside K
                stage_word_col<PRO>(ga[ti], ua[ti], in_k, (lane & 3) == 0,
                                    act_s + size_t(m) * 4 * qs + lofs + b * 128,
                                    eb_s + m * a.nch + b * 16 + (lane >> 2));
            }
        }
        if (!kDotScales) write_scales(sraw, tid, S * kWave);
        __syncthreads();
        return;
    }

    // ================= dot waves =================
    const int wave_all = wave;
    {
    const int wave = wave_all - S;
    // The wave's slots j = 0..CPW-1.  Plain: slot j is column slot wave + W j.  PAIR:
    // slots 2p and 2p+1 are the gate and up columns of pair wave + W p.
    auto slot_unit = [&](int j) { return wave + W * (PAIR ? (j >> 1) : j); };
    auto slot_ok = [&](int j) { return slot_unit(j) < (PAIR ? a.pairs : C); };
    auto slot_cj = [&](int j) { return PAIR && (j & 1) ? a.pairs + slot_unit(j) : slot_unit(j); };
    // The wave's outputs n = m * OPW + o: row m, unit o (a column, or with PAIR a pair).
    // kRowSums (two or more plain outputs): they are summed four to a register, output n of
    // group g ends in row r of it, n = 4 g + {0, 2, 1, 3}[r], and lane 16 r stores it.
    // Otherwise lane n stores output n, its sums read as scalars.  (The per-row stores
    // measured faster for plain outputs; for the SwiGLU pairs, where one lane needs both
    // sums of a pair, the scalar reads did.)
    constexpr int OPW = PAIR ? CPW / 2 : CPW;
    constexpr int NO = MR * OPW;
    constexpr bool kRowSums = !PAIR && NO >= 2;
    constexpr int NG = kRowSums ? (NO + 3) / 4 : 1;
    const int ldy = PAIR ? a.half_n : a.N;
    const int orow = lane >> 4;
    const bool lead = !kRowSums || (lane & 15) == 0;
    const uint16_t* rsrc = a.residual ? a.residual : a.y;   // y: a readable stand-in, value unused
    int o_m[NG], o_n[NG];
    bool o_ok[NG];
    uint16_t o_r[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int n = kRowSums ? 4 * g + (((orow & 1) << 1) | (orow >> 1)) : lane;
        const int m = n / OPW, u = wave + W * (n % OPW);
        o_m[g] = m;
        o_n[g] = cbase + u;
        o_ok[g] = lead && n < NO && m < a.M && u < (PAIR ? a.pairs : C) && cbase + u < ldy;
        o_r[g] = rsrc[size_t(min(m, a.M - 1)) * ldy + min(cbase + u, ldy - 1)];
    }
    const float os = a.out_scale ? *a.out_scale : 1.0f;
    // weight chunks: lane l takes chunks l, l+64, ... of each of the wave's columns (a
    // slot the wave does not own re-reads its first column: the loads stay unconditional,
    // so every wait in the dot is exact; skipping them measured slower)
    // the group scales first (long K), ahead of this wave's weights
    uint4 sraw[kColScLoads];
    if (kDotScales) load_scales(sraw, tid - S * kWave, W * kWave);
    uint4 wv[NI][CPW];
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const int cj = slot_ok(j) ? slot_cj(j) : slot_cj(0);
        const uint4* colp = a.qw + size_t(min(column(cj), a.N - 1)) * a.nch;
#pragma unroll
        for (int i = 0; i < NI; ++i) wv[i][j] = nt_load(colp + min(lane + kWave * i, a.nch - 1));
    }
    if (kDotScales) write_scales(sraw, tid - S * kWave, W * kWave);
    if (PAIR) __syncthreads();                     // the staging waves' row sums
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);

    // ---- dot products: one activation read per chunk serves the wave's columns ----
    float acc[MR][CPW];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < CPW; ++j) acc[m][j] = 0.f;
    // One row: the activation of range i + 1 is read from LDS while range i is worked (a
    // second buffer; with more rows its registers would spill).
    constexpr int NB = MR == 1 ? 2 : 1;
    uint4 avb[NB][MR][4];
    float2 ebb[NB][MR];
    auto read_act = [&](int i, int b) {
        // only the last range can pass K: the others need no clamp (constant LDS offsets)
        const int c = i < NI - 1 ? lane + kWave * i : min(lane + kWave * i, a.nch - 1);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const _Float16* arow = act_s + size_t(m) * 4 * qs + c * 8;
#pragma unroll
            for (int h = 0; h < 4; ++h) avb[b][m][h] = *reinterpret_cast<const uint4*>(arow + h * qs);
            ebb[b][m] = eb_s[m * a.nch + c];
        }
    };
    const float* sc_row = sc_s + (lane >> 2) * C;    // chunk lane + 64 i is in group lane / 4 + 16 i
    // The decode masks as vector registers, set once: a VALU instruction takes one scalar
    // operand, so with the masks in scalars every block of the dot re-copied them (an
    // identity DPP move, which the compiler does not re-materialise).
    const DecodeMasks dmv{uint32_t(__builtin_amdgcn_update_dpp(0, int(a.dm.lo), 0xE4, 0xF, 0xF, false)),
                          uint32_t(__builtin_amdgcn_update_dpp(0, int(a.dm.hi), 0xE4, 0xF, 0xF, false))};
    if (NB == 2) read_act(0, 0);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (NB == 2 && i + 1 < NI) read_act(i + 1, (i + 1) % NB);
        const int c = lane + kWave * i;
        if (i < NI - 1 || c < a.nch) {             // only the last range can pass K (NI = ceil(nch / 64))
            if (NB == 1) read_act(i, 0);
            const uint4 (&av)[MR][4] = avb[i % NB];
            const float2 (&eb)[MR] = ebb[i % NB];
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                if (!slot_ok(j)) break;            // uniform
                const float s = sc_row[16 * C * i + slot_cj(j)];
                const uint32_t wd[4] = {wv[i][j].x, wv[i][j].y, wv[i][j].z, wv[i][j].w};
                Q4x2 q[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) q[h] = decode_int4x8_biased(wd[h], dmv);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    float d = -eb[m].y;
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        d = dot2(q[h].p04, __builtin_bit_cast(half2_t, av[m][h].x), d);
                        d = dot2(q[h].p15, __builtin_bit_cast(half2_t, av[m][h].y), d);
                        d = dot2(q[h].p26, __builtin_bit_cast(half2_t, av[m][h].z), d);
                        d = dot2(q[h].p37, __builtin_bit_cast(half2_t, av[m][h].w), d);
                    }
                    acc[m][j] = fmaf(d, s * eb[m].x, acc[m][j]);
                }
            }
        }
    }

    if constexpr (kRowSums) {
    // ---- sum the outputs over the wave, four to a register; the epilogue in every row ----
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        if (MR == 1 && !slot_ok(4 * g)) break;     // uniform: no owned column left
        const int n0 = min(4 * g, NO - 1), n1 = min(4 * g + 1, NO - 1);
        const int n2 = min(4 * g + 2, NO - 1), n3 = min(4 * g + 3, NO - 1);
        const float v = wave_sum4_rows(acc[n0 / CPW][n0 % CPW], acc[n1 / CPW][n1 % CPW],
                                       acc[n2 / CPW][n2 % CPW], acc[n3 / CPW][n3 % CPW]);
        const float res = a.residual ? bf16_to_f32(o_r[g]) : 0.f;
        if (o_ok[g]) a.y[size_t(o_m[g]) * ldy + o_n[g]] = f32_to_bf16(fmaf(v, os, res));
    }
    } else {
    // ---- reduce each column over the wave, read the totals as scalars; the owning lane
    // applies the epilogue.  Two or more slots (the SwiGLU pairs): four slots to a
    // register, then one lane read per slot (C5-shaped layer 11.03 -> 10.76 us, same-run
    // A/B); one slot: DPP within the rows, then the four row sums ----
    float tot[MR][CPW];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j0 = 0; j0 < CPW; j0 += 4) {
#pragma unroll
            for (int j = j0; j < j0 + 4 && j < CPW; ++j) tot[m][j] = 0.f;
            if (!slot_ok(j0)) continue;            // uniform
            if (CPW >= 2) {
                const float t = wave_sum4_rows(acc[m][j0], acc[m][min(j0 + 1, CPW - 1)],
                                               acc[m][min(j0 + 2, CPW - 1)], acc[m][min(j0 + 3, CPW - 1)]);
                const int b = __builtin_bit_cast(int, t);    // rows: slots j0, j0 + 2, j0 + 1, j0 + 3
                tot[m][j0] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
                if (j0 + 1 < CPW) tot[m][j0 + 1] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
                if (j0 + 2 < CPW) tot[m][j0 + 2] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
                if (j0 + 3 < CPW) tot[m][j0 + 3] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
            } else {
                float v = acc[m][j0];
                v += dpp<kQuadSwap1>(v);
                v += dpp<kQuadSwap2>(v);
                v += dpp<kRowRor4>(v);
                v += dpp<kRowRor8>(v);             // every lane holds its row-of-16 sum
                const int b = __builtin_bit_cast(int, v);
                tot[m][j0] = (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
                              __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
                             (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
                              __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
            }
        }
    float mine = 0.f;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int o = 0; o < OPW; ++o) {
            // PAIR: silu(gate) * up of the pair's fp32 sums, rounded once
            const float v = PAIR ? silu_f32(tot[m][2 * o]) * tot[m][2 * o + 1] : tot[m][o];
            mine = lane == m * OPW + o ? v : mine;
        }
    if (PAIR) {
        if (o_ok[0]) a.y[size_t(o_m[0]) * ldy + o_n[0]] = f32_to_bf16(mine);
    } else {
        const float res = a.residual ? bf16_to_f32(o_r[0]) : 0.f;
        if (o_ok[0]) a.y[size_t(o_m[0]) * ldy + o_n[0]] = f32_to_bf16(fmaf(mine, os, res));
    }
    }
    // ---- side copy (the fused layer's residual update), spread over the grid ----
    if (a.cp_n16 > 0) {
        const int nt = W * kWave;
        for (int i = blockIdx.x * nt + (tid - S * kWave); i < a.cp_n16; i += gridDim.x * nt) a.cp_dst[i] = a.cp_src[i];
    }
    }
}

// ===========================================================================
// split-K kernel
// ===========================================================================
struct SplitArgs {
    const uint16_t* a0;
    const uint16_t* a1;
    int64_t lda;
    const uint4* qw;        // [N][K/32] chunks of 4 words
    const uint16_t* sc;
    int M, K, N;
    int nch;
    int groups, gps, splits, tiles;
    const float* out_scale;
    const uint16_t* residual;
    uint16_t* y;
    float* partial;         // [splits][M][tiles*64]
    DecodeMasks dm;         // int4 decode field masks (scalar registers)
};

template <int MR, int GW, int PRO>
__global__ __launch_bounds__(256) void w4_gemv_split_kernel(SplitArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int GPS = 4 * GW;
    _Float16* act_s = reinterpret_cast<_Float16*>(smem);                 // [GPS][MR][128]
    float* esc_s = reinterpret_cast<float*>(smem + GPS * MR * 128 * 2);   // [GPS][MR]
    float* red_s = esc_s + GPS * MR;                                      // [4][MR][64]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int tile = blockIdx.x % a.tiles;
    const int split = blockIdx.x / a.tiles;
    const int g0 = split * a.gps;
    const int ng = min(a.gps, a.groups - g0);
    const int kr = lane & 3;          // the four lanes of a quad share columns
    const int cq = lane >> 2;
    const int col = tile * kGemvCols + cq * 4;
    const bool col_ok = col < a.N;

    // ---- activation inputs: tasks (i, m) = (this wave's i-th group, row m) ----
    constexpr int T = MR * GW;
    constexpr int B = T < 8 ? T : 8;
    uint32_t ga[B], ua[B];
    auto load_batch = [&](int b0) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int t = b0 + b;
            const int i = t / MR, m = min(t % MR, a.M - 1);
            const int lg = min(wave + 4 * i, ng - 1);
            const size_t off = size_t(m) * a.lda + size_t(g0 + lg) * kGroup + 2 * lane;
            ga[b] = *reinterpret_cast<const uint32_t*>(a.a0 + off);
            ua[b] = PRO == kSwiGLU ? *reinterpret_cast<const uint32_t*>(a.a1 + off) : 0u;
        }
    };
    load_batch(0);

    // ---- weights and scales of this wave's groups: per column one 16-byte load of the
    // lane's four words ----
    uint4 wv[GW][4];
    uint2 sv[GW];
    const int colc = col_ok ? col : 0;
#pragma unroll
    for (int i = 0; i < GW; ++i) {
        const int g = g0 + min(wave + 4 * i, ng - 1);
#pragma unroll
        for (int c = 0; c < 4; ++c) wv[i][c] = nt_load(a.qw + size_t(colc + c) * a.nch + g * 4 + kr);
        sv[i] = *reinterpret_cast<const uint2*>(a.sc + size_t(g) * a.N + colc);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- prologue ----
#pragma unroll
    for (int b0 = 0; b0 < T; b0 += B) {
        if (b0 > 0) load_batch(b0);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int t = b0 + b;
            const int i = t / MR, m = t % MR;
            const int lg = wave + 4 * i;
            if (t >= T || lg >= ng) continue;          // uniform across the wave
            stage_act<PRO>(ga[b], ua[b], m < a.M, lane, act_s + (lg * MR + m) * kGroup, esc_s + lg * MR + m);
        }
    }
    // Each wave reads back only the groups it wrote; LDS operations of one wave complete
    // in order, so a wave-level scheduling barrier suffices.
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // ---- dot products ----
    float acc[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[m][c] = 0.f;

#pragma unroll
    for (int i = 0; i < GW; ++i) {
        const int lg = wave + 4 * i;
        if (lg >= ng) break;                              // uniform across the wave
        const float s4[4] = {bf16_lo(sv[i].x), bf16_hi(sv[i].x), bf16_lo(sv[i].y), bf16_hi(sv[i].y)};
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const _Float16* act = act_s + (lg * MR + m) * kGroup + kr * 32;
            const float e = esc_s[lg * MR + m];
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[m][c] = fmaf(dot32(wv[i][c], act, a.dm), s4[c] * e, acc[m][c]);
        }
    }

    // ---- reduce: the quad's lanes (same columns), then the four waves ----
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[m][c] = quad_sum(acc[m][c]);
    if (kr == 0) {
#pragma unroll
        for (int m = 0; m < MR; ++m)
            *reinterpret_cast<float4*>(red_s + (wave * MR + m) * kGemvCols + cq * 4) =
                make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
    }
    __syncthreads();

    const float s = a.out_scale ? *a.out_scale : 1.0f;
    const int npad = a.tiles * kGemvCols;
    for (int idx = tid; idx < MR * kGemvCols; idx += kGemvThreads) {
        const int m = idx / kGemvCols, cc = idx % kGemvCols;
        const int n = tile * kGemvCols + cc;
        if (m >= a.M || n >= a.N) continue;
        const float v = red_s[(0 * MR + m) * kGemvCols + cc] + red_s[(1 * MR + m) * kGemvCols + cc] +
                        red_s[(2 * MR + m) * kGemvCols + cc] + red_s[(3 * MR + m) * kGemvCols + cc];
        if (a.splits == 1) {
            const size_t o = size_t(m) * a.N + n;
            a.y[o] = f32_to_bf16(epilogue(v, s, a.residual, o));
        } else {
            a.partial[(size_t(split) * a.M + m) * npad + n] = v;   // summed by splitk_finish_kernel
        }
    }
}

// y[m, n] = bf16(s * sum over slices, in slice order, of partial[slice][m][n] (+ res)),
// slice j of row m at partial + j * split_stride + m * row_stride.  Runs after the
// kernel that wrote the partials, on the same stream: the kernel boundary makes them
// visible.  (Summing inside that kernel, by the last workgroup to arrive, needs
// device-scope atomic stores and loads and an arrival counter, which go past the XCDs'
// L2s: measured about 5 us slower per call.)
__global__ __launch_bounds__(256) void splitk_finish_kernel(const float* __restrict__ partial, int splits,
                                                           int64_t split_stride, int64_t row_stride, int M, int N,
                                                           const float* out_scale, const uint16_t* residual,
                                                           uint16_t* y) {
    const int o = blockIdx.x * 256 + threadIdx.x;
    if (o >= M * N) return;
    const int m = o / N, n = o % N;
    const float* p = partial + m * row_stride + n;
    // the epilogue's operands and up to kFinishBatch slices are all requested before the
    // first is used: one memory round trip (a loop that waited per batch of 8, then for
    // the residual, measured three for 9 slices)
    const float os = out_scale ? *out_scale : 1.0f;
    const uint16_t rraw = (residual ? residual : y)[o];   // y: a readable stand-in, value unused
    float v = 0.f;
    for (int s0 = 0; s0 < splits; s0 += kFinishBatch) {
        float t[kFinishBatch];
#pragma unroll
        for (int b = 0; b < kFinishBatch; ++b) t[b] = s0 + b < splits ? p[(s0 + b) * split_stride] : 0.f;
#pragma unroll
        for (int b = 0; b < kFinishBatch; ++b) v += t[b];
    }
    const float r = residual ? bf16_to_f32(rraw) : 0.f;
    y[o] = f32_to_bf16(fmaf(v, os, r));
}

// ===========================================================================
// launch plumbing
// ===========================================================================
// Kernels that need more than 64 KB of dynamic LDS must say so before launch.
template <typename Kern>
hipError_t allow_lds(Kern k, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               int(bytes));
}

template <typename Args, typename Kern>
hipError_t launch(Kern k, dim3 grid, int threads, size_t lds, hipStream_t s, const Args& a) {
    hipError_t e = allow_lds(k, lds);
    if (e != hipSuccess) return e;
    k<<<grid, threads, lds, s>>>(a);
    return hipGetLastError();
}

// The kernels take every chunk range but the last as inside K: NI must be ceil(nch / 64).
template <int MR, int CPW, int NI>
hipError_t launch_col3(Prologue pro, const ColArgs& a, const GemvPlan& p, hipStream_t s) {
    if (p.ni != NI) return hipErrorInvalidValue;
    if (pro == kSwiGLU)
        return launch(w4_gemv_col_kernel<MR, CPW, NI, kSwiGLU>, dim3(p.wgs), (p.stagers + p.waves) * kWave, p.lds_bytes,
                      s, a);
    return launch(w4_gemv_col_kernel<MR, CPW, NI, kIdentity>, dim3(p.wgs), (p.stagers + p.waves) * kWave, p.lds_bytes,
                  s, a);
}

// The (CPW, NI) pairs col_cpw_max allows (for some row count) are instantiated.
template <int MR>
hipError_t launch_col(Prologue pro, const ColArgs& a, const GemvPlan& p, hipStream_t s) {
    switch (p.cpw) {
        case 8: return launch_col3<MR, 8, 1>(pro, a, p, s);
        case 6: return launch_col3<MR, 6, 1>(pro, a, p, s);
        case 4:
            switch (p.ni) {
                case 1: return launch_col3<MR, 4, 1>(pro, a, p, s);
                case 2: return launch_col3<MR, 4, 2>(pro, a, p, s);
                default: return launch_col3<MR, 4, 3>(pro, a, p, s);
            }
        case 3:
            switch (p.ni) {
                case 1: return launch_col3<MR, 3, 1>(pro, a, p, s);
                case 2: return launch_col3<MR, 3, 2>(pro, a, p, s);
                case 3: return launch_col3<MR, 3, 3>(pro, a, p, s);
                default: return launch_col3<MR, 3, 4>(pro, a, p, s);
            }
        case 2:
            switch (p.ni) {
                case 1: return launch_col3<MR, 2, 1>(pro, a, p, s);
                case 2: return launch_col3<MR, 2, 2>(pro, a, p, s);
                case 3: return launch_col3<MR, 2, 3>(pro, a, p, s);
                case 4: return launch_col3<MR, 2, 4>(pro, a, p, s);
                case 5: return launch_col3<MR, 2, 5>(pro, a, p, s);
                default: return launch_col3<MR, 2, 6>(pro, a, p, s);
            }
        default:
            switch (p.ni) {
                case 1: return launch_col3<MR, 1, 1>(pro, a, p, s);
                case 2: return launch_col3<MR, 1, 2>(pro, a, p, s);
                case 3: return launch_col3<MR, 1, 3>(pro, a, p, s);
                case 4: return launch_col3<MR, 1, 4>(pro, a, p, s);
                case 5: return launch_col3<MR, 1, 5>(pro, a, p, s);
                case 6: return launch_col3<MR, 1, 6>(pro, a, p, s);
                case 7: return launch_col3<MR, 1, 7>(pro, a, p, s);
                default: return launch_col3<MR, 1, 8>(pro, a, p, s);
            }
    }
}

// Pair mode (add + RMSNorm prologue, SwiGLU pair epilogue): even slot counts only.
template <int MR, int CPW, int NI>
hipError_t launch_pair3(const ColArgs& a, const GemvPlan& p, hipStream_t s) {
    if (p.ni != NI) return hipErrorInvalidValue;
    return launch(w4_gemv_col_kernel<MR, CPW, NI, kAddRmsNorm>, dim3(p.wgs), (p.stagers + p.waves) * kWave,
                  p.lds_bytes, s, a);
}

template <int MR>
hipError_t launch_pair(const ColArgs& a, const GemvPlan& p, hipStream_t s) {
    switch (p.cpw) {
        case 8: return launch_pair3<MR, 8, 1>(a, p, s);
        case 6: return launch_pair3<MR, 6, 1>(a, p, s);
        case 4:
            switch (p.ni) {
                case 1: return launch_pair3<MR, 4, 1>(a, p, s);
                case 2: return launch_pair3<MR, 4, 2>(a, p, s);
                default: return launch_pair3<MR, 4, 3>(a, p, s);
            }
        default:
            switch (p.ni) {
                case 1: return launch_pair3<MR, 2, 1>(a, p, s);
                case 2: return launch_pair3<MR, 2, 2>(a, p, s);
                case 3: return launch_pair3<MR, 2, 3>(a, p, s);
                case 4: return launch_pair3<MR, 2, 4>(a, p, s);
                case 5: return launch_pair3<MR, 2, 5>(a, p, s);
                default: return launch_pair3<MR, 2, 6>(a, p, s);
            }
    }
}

template <int MR, int GW>
hipError_t launch_split2(Prologue pro, const SplitArgs& a, const GemvPlan& p, hipStream_t s) {
    const dim3 grid(p.tiles * p.splits);
    if (pro == kSwiGLU) return launch(w4_gemv_split_kernel<MR, GW, kSwiGLU>, grid, kGemvThreads, p.lds_bytes, s, a);
    return launch(w4_gemv_split_kernel<MR, GW, kIdentity>, grid, kGemvThreads, p.lds_bytes, s, a);
}

template <int MR>
hipError_t launch_split(Prologue pro, const SplitArgs& a, const GemvPlan& p, hipStream_t s) {
    switch (p.gw) {
        case 1: return launch_split2<MR, 1>(pro, a, p, s);
        case 2: return launch_split2<MR, 2>(pro, a, p, s);
        default: return launch_split2<MR, 4>(pro, a, p, s);
    }
}

int round_gw(int gw) { return gw <= 1 ? 1 : (gw <= 2 ? 2 : 4); }

// ---- test hooks: the decode every int4 kernel runs (decode_int4x8_biased), with its
// offsets removed (decode_int4x8), written out ----
__global__ void w4_unpack_kernel(const uint32_t* __restrict__ qw, int KB, int N, int8_t* __restrict__ q,
                                 DecodeMasks dm) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;     // word (n, kb)
    if (i >= int64_t(KB) * N) return;
    const int n = int(i / KB), kb = int(i % KB);
    const Q4x2 d = decode_int4x8(qw[i], dm);
    const half2_t p[4] = {d.p04, d.p15, d.p26, d.p37};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const _Float16 v = (j < 4) ? p[j][0] : p[j - 4][1];
        q[(int64_t(kb) * 8 + j) * N + n] = int8_t(float(v));
    }
}

__global__ void w4_dequant_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                                  int KB, int N, float* __restrict__ w, DecodeMasks dm) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= int64_t(KB) * N) return;
    const int n = int(i / KB), kb = int(i % KB);
    const Q4x2 d = decode_int4x8(qw[i], dm);
    const half2_t p[4] = {d.p04, d.p15, d.p26, d.p37};
    const float s = bf16_to_f32(sc[int64_t(kb / 16) * N + n]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const _Float16 v = (j < 4) ? p[j][0] : p[j - 4][1];
        w[(int64_t(kb) * 8 + j) * N + n] = float(v) * s;
    }
}

__global__ void fill_zero_kernel(uint4* p, int64_t n16, unsigned char* tail, int ntail) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
    if (i < ntail) tail[i] = 0;
}

// Largest columns-per-wave the weight registers allow (CPW * NI chunks of 16 bytes
// per lane, at most 128 VGPRs with 16 waves) without spilling; only these (CPW, NI)
// pairs are instantiated.
int col_cpw_max(int ni, int mr) {
    if (mr >= 4) return ni <= 1 ? 4 : ni <= 3 ? 2 : 1;
    return ni <= 1 ? 8 : ni <= 3 ? 4 : ni <= 4 ? 3 : ni <= 6 ? 2 : 1;
}

// Columns per wave as instantiated: 5 and 7 round up to 6 and 8 (only for one chunk
// per lane); the extra slots are skipped.
int col_cpw_round(int cpw) { return cpw <= 4 ? cpw : cpw <= 6 ? 6 : 8; }

// Dot waves for `units` columns (or column pairs) of a workgroup, unit u on wave u % W,
// at most `per_max` per wave, with S staging waves ahead of them (waves go to the SIMDs
// round robin): the W in [8, 16 - S] whose busiest SIMD holds the fewest units, ties to
// fewer waves.  The dot is VALU work, so the busiest SIMD sets its time; measured on
// MI355X at K = 1536 (one chunk range per lane), 12 dot waves against 9.
int col_dot_waves(int S, int units, int per_max) {
    int best_w = 0, best_load = 1 << 30;
    for (int W = 8; W <= 16 - S; ++W) {
        if ((units + W - 1) / W > per_max) continue;
        int load[4] = {0, 0, 0, 0};
        for (int w = 0; w < W && w < units; ++w) load[(S + w) % 4] += (units - w + W - 1) / W;
        const int mx = std::max(std::max(load[0], load[1]), std::max(load[2], load[3]));
        if (mx < best_load) {
            best_load = mx;
            best_w = W;
        }
    }
    return best_w;
}

bool plan_column(int M, int K, int N, GemvPlan& p, const Overrides& ov) {
    if (M > 4 || K > 32 * kColMaxChunks * kWave) return false;
    const int nch = K / 32;
    const int nblk = (K + 511) / 512;
    p.mr = M <= 1 ? 1 : M <= 2 ? 2 : 4;
    p.ni = (nch + kWave - 1) / kWave;
    const int ntask = p.mr * nblk;
    if (ntask > 8 * kColMaxTasks) return false;             // at most 8 staging waves
    // staging waves: two per SIMD when there is enough staging work, fewer for short K
    p.stagers = std::min(8, std::max(2, ntask));
    const int cmax = col_cpw_max(p.ni, p.mr);
    // Eight dot waves (two per SIMD: one wave per SIMD issues VALU work at about half
    // rate) and about N / 256 columns per workgroup, so that every CU gets one workgroup.
    // When eight waves cannot hold that many columns, the fewest waves (at most
    // 16 - stagers) that reach the smallest columns-per-wave variant.
    const int cwant = std::max(1, (N + 255) / 256);
    p.waves = 8;
    if (cwant > 8 * cmax) {
        // the wave count whose busiest SIMD holds the fewest columns, at most cmax per wave
        // after rounding to an instantiated variant; else the fewest waves that reach cmax
        int w = 0;
        for (int cap = cmax; cap >= 1 && !w; --cap)
            if (col_cpw_round(cap) <= cmax) w = col_dot_waves(p.stagers, cwant, cap);
        if (w) {
            p.waves = w;
        } else {
            const int cpw = std::min(cmax, col_cpw_round((cwant + 15 - p.stagers) / (16 - p.stagers)));
            p.waves = std::max(8, std::min(16 - p.stagers, (cwant + cpw - 1) / cpw));
        }
    }
    int C = std::min(cwant, p.waves * cmax);
    // a forced shape replaces the choice when the kernel has a variant for it; more dot
    // waves than 8 take slots from the staging waves (16 waves in all)
    if (ov.col_waves > 0 && ov.col_cols > 0) {
        const int w = std::min(ov.col_waves, kColMaxWaves);
        const int st = std::min(p.stagers, 16 - w);
        if ((ov.col_cols + w - 1) / w <= cmax && st * kColMaxTasks >= ntask && st >= 1) {
            p.waves = w;
            p.stagers = st;
            C = ov.col_cols;
        }
    }
    p.cols = C;
    p.cpw = col_cpw_round((C + p.waves - 1) / p.waves);
    if (p.cpw < 1 || p.cpw > cmax || p.stagers * kColMaxTasks < ntask) return false;
    const int pieces = (C + 7) / 8 + 1;                       // 8-column scale pieces per group, at most
    if (p.groups * pieces > kColScLoads * (col_dot_scales(p.ni) ? p.waves : p.stagers) * kWave) return false;
    p.wgs = (N + C - 1) / C;
    p.lds_bytes = size_t(p.mr) * 4 * (nch * 8 + 32) * 2 + size_t(p.mr) * nch * 8 + size_t(p.groups) * C * 4;
    if (p.lds_bytes > kMaxLds) return false;
    p.kind = kColumnOwning;
    return true;
}

// The fused layer's gate_up: column kernel in pair mode over K = H, N = 2I.  The
// workgroup owns about I / 256 pairs (so every CU gets one workgroup), with slots
// (two per pair) spread over 8..16 - stagers dot waves.
bool plan_column_pair(int M, int K, int I, GemvPlan& p) {
    p = GemvPlan{};
    p.groups = K / kGroup;
    if (M > 4 || K > 32 * kColMaxChunks * kWave || I < 1) return false;
    const int nch = K / 32;
    const int nblk = (K + 511) / 512;
    p.mr = M <= 1 ? 1 : M <= 2 ? 2 : 4;
    p.ni = (nch + kWave - 1) / kWave;
    if (p.ni > 6) return false;
    const int ntask = p.mr * nblk;
    if (ntask > 8 * kColMaxTasksNorm) return false;
    p.stagers = std::min(8, std::max(2, ntask));
    if (p.stagers * kColMaxTasksNorm < ntask) return false;
    const int cmax = col_cpw_max(p.ni, p.mr) & ~1;            // slots per wave, even
    if (cmax < 2) return false;
    const int ppw = cmax / 2;                                  // pairs per wave, at most
    const int pwant = std::max(1, (I + 255) / 256);
    p.waves = 8;
    if (pwant > 8 * ppw) {
        const int w = col_dot_waves(p.stagers, pwant, ppw);
        p.waves = w ? w : std::min(16 - p.stagers, (pwant + ppw - 1) / ppw);
    }
    const int pairs = std::min(pwant, p.waves * ppw);
    p.cpw = 2 * ((pairs + p.waves - 1) / p.waves);
    if (p.cpw > cmax) return false;
    p.cols = 2 * pairs;
    const int pieces = 2 * ((pairs + 7) / 8 + 1);
    if (p.groups * pieces > kColScLoads * (col_dot_scales(p.ni) ? p.waves : p.stagers) * kWave) return false;
    p.wgs = (I + pairs - 1) / pairs;
    p.lds_bytes = size_t(p.mr) * 4 * (nch * 8 + 32) * 2 + size_t(p.mr) * nch * 8 + size_t(p.groups) * p.cols * 4 +
                  size_t(p.stagers) * p.mr * 4;
    if (p.lds_bytes > kMaxLds) return false;
    p.kind = kColumnOwning;
    return true;
}

}  // namespace

// Matrix-core kernel: 6..8 waves of one 16-column tile each, K split into slices
// until there are about 256 workgroups, one per CU (and each slice's activation fits
// LDS); of the wave counts, the one whose workgroups fill the 256 CUs best (fewest idle
// slots in the last round of workgroups), ties to more waves.
int mfma_splits(int groups, int tiles, int max_slice = kMfmaMaxSliceGroups) {
    const int S = std::max((groups + max_slice - 1) / max_slice,
                           std::min(groups, (256 + tiles - 1) / tiles));
    const int gps = (groups + S - 1) / S;
    return (groups + gps - 1) / gps;
}

bool plan_mfma(int M, int K, int N, GemvPlan& p, int min_rows) {
    if (M < std::max(min_rows, 1) || M > kMfmaMaxRows) return false;
    const int rb = M <= 16 ? 1 : M <= 32 ? 2 : 4;     // row blocks of 16
    const int max_slice = kMfmaMaxSliceGroups / rb;   // LDS holds 16 rb rows of the slice
    p.kind = kMfma;
    p.mr = 16 * rb;
    p.groups = K / kGroup;
    p.cpw = 1;
    p.waves = kMfmaWaves;
    double best = 1e30;
    for (int w = kMfmaWaves; w >= 6; --w) {
        const int tiles = (N + 16 * p.cpw * w - 1) / (16 * p.cpw * w);
        const int wgs = tiles * mfma_splits(p.groups, tiles, max_slice);
        const double fill = double((wgs + 255) / 256 * 256) / wgs;
        if (fill < best - 1e-9) { best = fill; p.waves = w; }
    }
    const int ncol = p.waves * p.cpw * 16;
    p.tiles = (N + ncol - 1) / ncol;
    int S = mfma_splits(p.groups, p.tiles, max_slice);
    p.gps = (p.groups + S - 1) / S;
    p.splits = (p.groups + p.gps - 1) / p.gps;
    if (p.splits > 1) p.partial_bytes = size_t(p.splits) * p.mr * p.tiles * ncol * 4;
    p.lds_bytes = size_t(p.mr) * (size_t(p.gps) * 16 + 1) * 16 + size_t(p.mr) * (p.gps | 1) * 4;
    return true;
}

// The gate_up projection with the SwiGLU epilogue (pair mode of the row-block matrix-core
// kernel, 1..64 rows): even wave counts, P = 8 waves column pairs per workgroup.  The K slices
// are kept whole (one slice, the epilogue in the kernel) when that already gives about
// one workgroup per CU; otherwise split toward 256 workgroups, summed by the pair finish.
bool plan_mfma_pair(int M, int K, int I, GemvPlan& p) {
    p = GemvPlan{};
    if (M < 1 || M > kMfmaMaxRows || K <= 0 || K % kGroup || I < 8 || I % 8) return false;
    const int rb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    const int max_slice = kMfmaMaxSliceGroups / rb;
    p.kind = kMfma;
    p.mr = 16 * rb;
    p.groups = K / kGroup;
    p.cpw = 1;
    auto splits_for = [&](int ranges) {
        const int S = std::max((p.groups + max_slice - 1) / max_slice,
                               ranges >= 192 ? 1 : std::min(p.groups, (256 + ranges - 1) / ranges));
        const int gps = (p.groups + S - 1) / S;
        return (p.groups + gps - 1) / gps;
    };
    double best = 1e30;
    p.waves = kMfmaWaves;
    for (int w = kMfmaWaves; w >= 6; w -= 2) {
        const int ranges = (I + 8 * w - 1) / (8 * w);
        const int wgs = ranges * splits_for(ranges);
        const double fill = double((wgs + 255) / 256 * 256) / wgs;
        if (fill < best - 1e-9) {
            best = fill;
            p.waves = w;
        }
    }
    const int P = 8 * p.waves;
    p.tiles = (I + P - 1) / P;
    const int S = splits_for(p.tiles);
    p.gps = (p.groups + S - 1) / S;
    p.splits = (p.groups + p.gps - 1) / p.gps;
    if (p.splits > 1) p.partial_bytes = size_t(p.splits) * p.mr * p.tiles * 2 * P * 4;
    const size_t stage = size_t(p.mr) * (size_t(p.gps) * 16 + 1) * 16 + size_t(p.mr) * (p.gps | 1) * 4;
    const size_t xchg = size_t(p.waves / 2) * rb * kWave * 16;
    p.lds_bytes = std::max(stage, xchg);
    return p.lds_bytes <= kMaxLds;
}

// The ring kernel's plan where it measured faster than the row-block kernel (5..16 rows,
// identity prologue and pair mode): K slices of at most 16 groups in at most 256
// workgroups.  Longer slices favour the row-block kernel, whose main loop runs without a
// barrier once its activation is staged (16 x 4096 x 28672: 19.0 against 21.8 us), and
// shorter ones the ring, which has no staging pass (16 x 1536 x 17920: 9.1 against
// 14.1 us; 16 x 4096 x 11008: 14.1 against 19.1; 16 x 1024 x 512: 5.5 against 7.5).
bool ring_preferred(const GemvPlan& r) { return r.gps <= 16 && r.tiles * r.splits <= 256; }

bool plan_pair(int M, int K, int I, const Overrides& ov, GemvPlan& p) {
    if ((ov.mfma_kernel == 3 || ov.mfma_kernel == 0) && M > 4 && plan_ring_pair(M, K, I, p) &&
        (ov.mfma_kernel == 3 || ring_preferred(p)))
        return true;
    return plan_mfma_pair(M, K, I, p);
}

GemvPlan plan_gemv(int M, int K, int N, const Overrides& ov, Prologue pro) {
    GemvPlan p{};
    p.groups = K / kGroup;
    if (M > 16) {                 // only the matrix-core kernel takes more than 16 rows
        plan_mfma(M, K, N, p);
        return p;
    }
    if (ov.split == 0 && plan_column(M, K, N, p, ov)) return p;
    p = GemvPlan{};
    // the ring kernel: forced, or built in where it measured faster -- the SwiGLU prologue
    // above about 12 MB of weights (16 x 14336 x 4096: 15.5 against 16.4 us; 16 x 4096 x 11008:
    // 15.7 against 23.9), the identity prologue by ring_preferred where the kernel whose
    // waves split K is not taken (short K or above about 12 MB: 16 x 1536 x 17920 9.8
    // against 18.3 us, 16 x 14336 x 4096 14.9 against 18.0)
    const bool small = int64_t(K) * N / 2 <= (int64_t(12) << 20);
    const bool kmfma_ident = pro == kIdentity && M > 4 && K >= 4096 && small;
    if (ov.split == 0 && (ov.mfma_kernel == 3 || (ov.mfma_kernel == 0 && M > 4)) && plan_ring(M, K, N, pro, p)) {
        if (ov.mfma_kernel == 3 || (pro == kSwiGLU && !small) || (pro == kIdentity && !kmfma_ident && ring_preferred(p)))
            return p;
    }
    p = GemvPlan{};
    // the kernel whose waves split K: the SwiGLU prologue up to about 12 MB of weights, one
    // group per wave (measured faster there, slower elsewhere), also 3..4 rows the column
    // kernel cannot stage (K = 9216: 11.9 -> 11.65 us against split-K); the identity
    // prologue at K >= 4096 up to about 12 MB, groups per wave by its cost (16 x 8960 x 1536:
    // 8.61 -> 7.25 us, 16 x 4096 x 4096: 8.46 -> 7.55 us against the ring); or when forced
    const bool kmfma = ov.mfma_kernel == 2 || (ov.mfma_kernel == 0 && ((pro == kSwiGLU && M > 2 && small) || kmfma_ident));
    Overrides ovk = ov;
    if (ov.mfma_kernel == 0) ovk.mfma_gw = pro == kSwiGLU ? 1 : 0;
    if (ov.split == 0 && kmfma && plan_kmfma(M, K, N, pro == kSwiGLU ? 2 : 4, p, ovk)) return p;
    p = GemvPlan{};
    if (ov.split == 0 && plan_mfma(M, K, N, p)) return p;
    p = GemvPlan{};
    p.kind = kSplitK;
    p.groups = K / kGroup;
    p.tiles = (N + kGemvCols - 1) / kGemvCols;
    p.mr = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    int gw;
    if (ov.split > 0) {
        const int k = std::min(ov.split, p.groups);
        const int gps = (p.groups + k - 1) / k;
        gw = round_gw((gps + 3) / 4);
    } else if (p.tiles >= 192 && p.groups <= 16) {
        gw = round_gw((p.groups + 3) / 4);          // one split: no cross-workgroup step
    } else {
        gw = 1;
        while (gw < 4 && int64_t(p.tiles) * ((p.groups + 4 * gw - 1) / (4 * gw)) > 2048) gw *= 2;
    }
    p.gw = gw;
    p.gps = 4 * gw;
    p.splits = (p.groups + p.gps - 1) / p.gps;
    if (p.splits > 1) p.partial_bytes = size_t(p.splits) * M * p.tiles * kGemvCols * 4;
    p.lds_bytes = size_t(p.gps) * p.mr * kGroup * 2 + size_t(p.gps) * p.mr * 4 +
                  size_t(4) * p.mr * kGemvCols * 4;
    return p;
}

size_t gemv_workspace_bytes(int M, int K, int N) {
    return std::max(plan_gemv(M, K, N, Overrides{}, kSwiGLU).partial_bytes,
                    plan_gemv(M, K, N, Overrides{}, kIdentity).partial_bytes);
}

hipError_t launch_splitk_finish(const float* partial, int splits, int64_t split_stride, int64_t row_stride, int M,
                                int N, const float* out_scale, const uint16_t* residual, uint16_t* y, hipStream_t s) {
    splitk_finish_kernel<<<dim3((M * N + 255) / 256), 256, 0, s>>>(partial, splits, split_stride, row_stride, M, N,
                                                                 out_scale, residual, y);
    return hipGetLastError();
}

hipError_t launch_gemv(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda,
                       const uint32_t* qw, const uint16_t* sc, int M, int K, int N,
                       const float* out_scale, const uint16_t* residual, uint16_t* y,
                       void* ws, const GemvPlan& p, hipStream_t s, const void* xs, const float* xesc) {
    if (p.kind == kColumnOwning) {
        ColArgs a{};
        a.dm = DecodeMasks{kDecodeMaskLo, kDecodeMaskHi};
        a.a0 = a0;
        a.a1 = a1;
        a.lda = lda;
        a.qw = reinterpret_cast<const uint4*>(qw);
        a.sc = sc;
        a.M = M;
        a.K = K;
        a.N = N;
        a.nch = K / 32;
        a.groups = p.groups;
        a.cols = p.cols;
        a.stagers = p.stagers;
        a.out_scale = out_scale;
        a.residual = residual;
        a.y = y;
        switch (p.mr) {
            case 1: return launch_col<1>(pro, a, p, s);
            case 2: return launch_col<2>(pro, a, p, s);
            default: return launch_col<4>(pro, a, p, s);
        }
    }
    if (p.kind == kRing) return launch_ring(pro, a0, a1, lda, qw, sc, M, K, N, out_scale, residual, y, ws, p, s);
    if (p.kind == kKMfma) return launch_kmfma(pro, a0, a1, lda, qw, sc, M, K, N, out_scale, residual, y, ws, p, s);
    if (p.kind == kMfma)
        return launch_mfma(pro, a0, a1, lda, qw, sc, M, K, N, out_scale, residual, y, ws, p, s, xs, xesc);
    SplitArgs a{};
    a.dm = DecodeMasks{kDecodeMaskLo, kDecodeMaskHi};
    a.a0 = a0;
    a.a1 = a1;
    a.lda = lda;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.K = K;
    a.N = N;
    a.nch = K / 32;
    a.groups = p.groups;
    a.gps = p.gps;
    a.splits = p.splits;
    a.tiles = p.tiles;
    a.out_scale = out_scale;
    a.residual = residual;
    a.y = y;
    a.partial = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    hipError_t e;
    switch (p.mr) {
        case 1: e = launch_split<1>(pro, a, p, s); break;
        case 2: e = launch_split<2>(pro, a, p, s); break;
        case 4: e = launch_split<4>(pro, a, p, s); break;
        case 8: e = launch_split<8>(pro, a, p, s); break;
        default: e = launch_split<16>(pro, a, p, s); break;
    }
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t npad = int64_t(p.tiles) * kGemvCols;
    return launch_splitk_finish(a.partial, p.splits, int64_t(M) * npad, npad, M, N, out_scale, residual, y, s);
}

hipError_t launch_w4_unpack(const uint32_t* qw, int K, int N, int8_t* q, hipStream_t s) {
    const int64_t n = int64_t(K / 8) * N;
    w4_unpack_kernel<<<dim3((n + 255) / 256), 256, 0, s>>>(qw, K / 8, N, q, DecodeMasks{kDecodeMaskLo, kDecodeMaskHi});
    return hipGetLastError();
}

hipError_t launch_w4_dequant(const uint32_t* qw, const uint16_t* sc, int K, int N, float* w,
                             hipStream_t s) {
    const int64_t n = int64_t(K / 8) * N;
    w4_dequant_kernel<<<dim3((n + 255) / 256), 256, 0, s>>>(qw, sc, K / 8, N, w,
                                                             DecodeMasks{kDecodeMaskLo, kDecodeMaskHi});
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    const int64_t n16 = int64_t(bytes / 16);
    const int ntail = int(bytes % 16);
    unsigned char* tail = static_cast<unsigned char*>(p) + n16 * 16;
    const int64_t threads = std::max<int64_t>(n16, ntail);
    fill_zero_kernel<<<dim3((threads + 255) / 256), 256, 0, s>>>(static_cast<uint4*>(p), n16, tail, ntail);
    return hipGetLastError();
}

bool norm_gemv_swiglu_supported(int M, int K, int I) {
    GemvPlan p;
    return plan_column_pair(M, K, I, p);
}

hipError_t launch_norm_gemv_swiglu(const uint16_t* x, const uint16_t* r, const uint16_t* nw, float eps,
                                   const uint32_t* qw, const uint16_t* sc, int M, int K, int I,
                                   uint16_t* h_out, uint16_t* act, hipStream_t s) {
    GemvPlan p;
    if (!plan_column_pair(M, K, I, p)) return hipErrorInvalidValue;
    ColArgs a{};
    a.dm = DecodeMasks{kDecodeMaskLo, kDecodeMaskHi};
    a.a0 = x;
    a.a1 = r;
    a.lda = K;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.K = K;
    a.N = 2 * I;
    a.nch = K / 32;
    a.groups = p.groups;
    a.cols = p.cols;
    a.stagers = p.stagers;
    a.y = act;
    a.nw = nw;
    a.eps = eps;
    a.h_out = h_out;
    a.pairs = p.cols / 2;
    a.half_n = I;
    switch (p.mr) {
        case 1: return launch_pair<1>(a, p, s);
        case 2: return launch_pair<2>(a, p, s);
        default: return launch_pair<4>(a, p, s);
    }
}

bool gemv_column_supported(int M, int K, int N, const Overrides& ov) {
    GemvPlan p{};
    p.groups = K / kGroup;
    return plan_column(M, K, N, p, ov);
}

hipError_t launch_gemv_copy(Prologue pro, const uint16_t* a0, int64_t lda, const uint32_t* qw, const uint16_t* sc,
                            int M, int K, int N, const float* out_scale, const uint16_t* residual, uint16_t* y,
                            const void* cp_src, void* cp_dst, size_t cp_bytes, const Overrides& ov, hipStream_t s) {
    GemvPlan p{};
    p.groups = K / kGroup;
    if (pro != kIdentity || !plan_column(M, K, N, p, ov) || cp_bytes % 16) return hipErrorInvalidValue;
    ColArgs a{};
    a.dm = DecodeMasks{kDecodeMaskLo, kDecodeMaskHi};
    a.a0 = a0;
    a.lda = lda;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.K = K;
    a.N = N;
    a.nch = K / 32;
    a.groups = p.groups;
    a.cols = p.cols;
    a.stagers = p.stagers;
    a.out_scale = out_scale;
    a.residual = residual;
    a.y = y;
    a.cp_src = static_cast<const uint4*>(cp_src);
    a.cp_dst = static_cast<uint4*>(cp_dst);
    a.cp_n16 = int(cp_bytes / 16);
    switch (p.mr) {
        case 1: return launch_col<1>(kIdentity, a, p, s);
        case 2: return launch_col<2>(kIdentity, a, p, s);
        default: return launch_col<4>(kIdentity, a, p, s);
    }
}

}  // namespace fdec
