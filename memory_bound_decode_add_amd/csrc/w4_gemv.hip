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
// Work decomposition.  A 256-thread workgroup owns a 64-column tile and a slice of
// whole 128-wide K groups (a "split").  Wave w of the workgroup owns groups
// w, w+4, ... of the slice.  Lane (kr = lane % 4, cq = lane / 4) owns columns
// 4cq..4cq+3 and packed rows 4kr..4kr+3 of each of its wave's groups, loading each
// packed row of its four columns with one 16-byte load: one load instruction of a
// wave covers four 256-byte runs of the weight matrix.  Every weight load of the
// workgroup is issued before any arithmetic, so the whole slice is in flight at once.
//
// Prologue.  Each wave computes the activation of its own groups (2 values per lane
// per group and row) in fp32, then stores it to LDS as fp16 scaled by a power of two
// 2^-E chosen per (row, group) from the group's largest magnitude, so the largest
// value lands in [2^14, 2^15): any finite fp32 activation fits fp16 with an 11-bit
// significand relative to its group's maximum.  The factor 2^E is folded back in
// with the group scale.  Activation values are stored in the pair order of the int4
// decode (see decode_int4x8), so four dot2 instructions consume one packed word.
//
// Dot.  Per packed word: one XOR, one shift, four AND-OR and four packed fp16 ops turn
// eight nibbles into four exact fp16 pairs; four v_dot2_f32_f16 accumulate them
// against the activations in fp32.  The group scale (times 2^E) multiplies the
// lane's 32-element partial sum once per group.
//
// Reduction.  The four lanes sharing columns form a quad and are summed with DPP; the
// four waves through LDS.  With one split the workgroup applies the epilogue directly.  With several,
// each workgroup writes fp32 partial sums for its tile to the workspace with
// device-scope atomic stores, waits for them to complete, then bumps the tile's
// arrival counter; the last workgroup to arrive reads the partials back with
// device-scope atomic loads, sums them in split order (so results do not depend on
// arrival order), applies the epilogue and resets the counter.
#include "device_common.h"
#include "fdec_internal.h"

#include <algorithm>

namespace fdec {

int g_forced_split = 0;

namespace {

struct GemvArgs {
    const uint16_t* a0;     // g (SwiGLU) or x (identity), row stride lda
    const uint16_t* a1;     // u (SwiGLU) or unused
    int64_t lda;
    const uint4* qw;        // packed words viewed as uint4: [K/8][N/4]
    const uint16_t* sc;     // bf16 scales [K/128][N]
    int M, K, N;
    int groups, gps, splits, tiles;
    const float* out_scale;
    const uint16_t* residual;
    uint16_t* y;
    float* partial;         // [splits][M][tiles*64]
    unsigned* counters;     // [tiles]
};

__device__ __forceinline__ float epilogue(float v, float s, const uint16_t* res, size_t idx) {
    v *= s;
    if (res) v += bf16_to_f32(res[idx]);
    return v;
}

template <int MR, int GW, int PRO>
__global__ __launch_bounds__(256) void w4_gemv_kernel(GemvArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int GPS = 4 * GW;
    _Float16* act_s = reinterpret_cast<_Float16*>(smem);                 // [GPS][MR][128]
    float* esc_s = reinterpret_cast<float*>(smem + GPS * MR * 128 * 2);   // [GPS][MR]
    float* red_s = esc_s + GPS * MR;                                      // [4][MR][64]
    __shared__ int last_flag;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int tile = blockIdx.x % a.tiles;
    const int split = blockIdx.x / a.tiles;
    const int g0 = split * a.gps;
    const int ng = min(a.gps, a.groups - g0);
    const int kr = lane & 3;          // the four lanes of a quad share columns
    const int cq = lane >> 2;
    const int col = tile * kGemvCols + cq * 4;
    const bool col_ok = col < a.N;
    const int nq = a.N >> 2;

    // ---- activation inputs: tasks (i, m) = (this wave's i-th group, row m) ----
    constexpr int T = MR * GW;
    constexpr int B = T < 8 ? T : 8;
    uint32_t ga[B], ua[B];
    // Every load below is unconditional, from an address clamped into the tensor: a
    // task or group outside the slice re-reads a valid location and its value is never
    // used.  Without branches around the loads, the compiler's wait counting can let
    // the prologue start as soon as its own (first-issued) loads arrive.
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

    // ---- weights and scales of this wave's groups, all in flight at once ----
    uint4 wv[GW][4];
    uint2 sv[GW];
    const int colc = col_ok ? col : 0;
#pragma unroll
    for (int i = 0; i < GW; ++i) {
        const int g = g0 + min(wave + 4 * i, ng - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const size_t kb = size_t(g) * 16 + kr * 4 + j;
            wv[i][j] = a.qw[kb * nq + (colc >> 2)];
        }
        sv[i] = *reinterpret_cast<const uint2*>(a.sc + size_t(g) * a.N + colc);
    }
    // Keep the weight decode below the prologue: the prologue needs only the (earlier)
    // activation loads, so the weights stay in flight while it runs.
    __builtin_amdgcn_sched_barrier(0);

    // ---- prologue: activations to LDS as block-scaled fp16 ----
#pragma unroll
    for (int b0 = 0; b0 < T; b0 += B) {
        if (b0 > 0) load_batch(b0);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int t = b0 + b;
            const int i = t / MR, m = t % MR;
            const int lg = wave + 4 * i;
            if (t >= T || lg >= ng) continue;          // uniform across the wave
            float v0 = 0.f, v1 = 0.f;
            if (m < a.M) {                                // uniform; rows past M stay zero
                if (PRO == kSwiGLU) {
                    v0 = silu_f32(bf16_lo(ga[b])) * bf16_lo(ua[b]);
                    v1 = silu_f32(bf16_hi(ga[b])) * bf16_hi(ua[b]);
                } else {
                    v0 = bf16_lo(ga[b]);
                    v1 = bf16_hi(ga[b]);
                }
            }
            const float mx = wave_max_uniform(fmaxf(fabsf(v0), fabsf(v1)));
            int e = 0;
            (void)__builtin_frexpf(mx, &e);
            const int E = min(max(e - 15, -126), 127);
            const int k0 = 2 * lane;                      // k within the group
            const int r = k0 >> 3, j0 = k0 & 7;
            _Float16* dst = act_s + (lg * MR + m) * kGroup + r * 8;
            dst[pair_slot(j0)] = (_Float16)__builtin_ldexpf(v0, -E);
            dst[pair_slot(j0 + 1)] = (_Float16)__builtin_ldexpf(v1, -E);
            if (lane == 0) esc_s[lg * MR + m] = __builtin_ldexpf(1.0f, E);
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
        float gs[MR][4];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c) gs[m][c] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = kr * 4 + j;
            const uint32_t wd[4] = {wv[i][j].x, wv[i][j].y, wv[i][j].z, wv[i][j].w};
            Q4x2 q[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) q[c] = decode_int4x8(wd[c]);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const uint4 av = *reinterpret_cast<const uint4*>(act_s + (lg * MR + m) * kGroup + r * 8);
                const half2_t a04 = __builtin_bit_cast(half2_t, av.x);
                const half2_t a15 = __builtin_bit_cast(half2_t, av.y);
                const half2_t a26 = __builtin_bit_cast(half2_t, av.z);
                const half2_t a37 = __builtin_bit_cast(half2_t, av.w);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float v = gs[m][c];
                    v = dot2(q[c].p04, a04, v);
                    v = dot2(q[c].p15, a15, v);
                    v = dot2(q[c].p26, a26, v);
                    v = dot2(q[c].p37, a37, v);
                    gs[m][c] = v;
                }
            }
        }
        const float s4[4] = {bf16_lo(sv[i].x), bf16_hi(sv[i].x), bf16_lo(sv[i].y), bf16_hi(sv[i].y)};
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const float e = esc_s[lg * MR + m];
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[m][c] = fmaf(gs[m][c], s4[c] * e, acc[m][c]);
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
            __hip_atomic_store(a.partial + (size_t(split) * a.M + m) * npad + n, v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (a.splits == 1) return;

    // ---- split-K: the last workgroup of the tile to arrive finishes it ----
    // The partials were written with device-scope atomic stores, which are coherent
    // across the XCDs' L2 caches (they write through).  Waiting for their completion
    // before the arrival counter is bumped orders them before it without a release
    // fence, which on this part would write back the whole L2 once per workgroup.
    // The finishing workgroup reads them back with device-scope atomic loads.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (old == unsigned(a.splits - 1));
    }
    __syncthreads();
    if (!last_flag) return;

    // P threads per output, each summing every P-th split with all its loads issued
    // before the first add; the P sums are then added in a fixed order through LDS.
    constexpr int OUTS = MR * kGemvCols;
    constexpr int P = OUTS >= kGemvThreads ? 1 : kGemvThreads / OUTS;
    constexpr int BATCH = 16;
    for (int o = tid % OUTS; o < OUTS; o += (P == 1 ? kGemvThreads : OUTS)) {
        const int p = P == 1 ? 0 : tid / OUTS;
        const int m = o / kGemvCols, cc = o % kGemvCols;
        const int n = tile * kGemvCols + cc;
        const bool live = m < a.M && n < a.N;
        float v = 0.f;
        for (int s0 = p; s0 < a.splits; s0 += P * BATCH) {
            float t[BATCH];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) {
                const int sp = s0 + b * P;
                t[b] = (live && sp < a.splits)
                           ? __hip_atomic_load(a.partial + (size_t(sp) * a.M + m) * npad + n, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
            }
#pragma unroll
            for (int b = 0; b < BATCH; ++b) v += t[b];
        }
        if (P == 1) {
            if (live) {
                const size_t oo = size_t(m) * a.N + n;
                a.y[oo] = f32_to_bf16(epilogue(v, s, a.residual, oo));
            }
        } else {
            red_s[p * OUTS + o] = v;
        }
    }
    if (P > 1) {
        __syncthreads();
        for (int o = tid; o < OUTS; o += kGemvThreads) {
            const int m = o / kGemvCols, cc = o % kGemvCols;
            const int n = tile * kGemvCols + cc;
            if (m >= a.M || n >= a.N) continue;
            float v = 0.f;
            for (int p = 0; p < P; ++p) v += red_s[p * OUTS + o];
            const size_t oo = size_t(m) * a.N + n;
            a.y[oo] = f32_to_bf16(epilogue(v, s, a.residual, oo));
        }
    }
    if (tid == 0) __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Kernels that need more than 64 KB of dynamic LDS must say so once before launch.
template <typename Kern>
hipError_t allow_lds(Kern k, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               int(bytes));
}

template <int MR, int GW>
hipError_t launch_mr_gw(Prologue pro, const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
    const dim3 grid(p.tiles * p.splits);
    hipError_t e;
    if (pro == kSwiGLU) {
        if ((e = allow_lds(w4_gemv_kernel<MR, GW, kSwiGLU>, p.lds_bytes)) != hipSuccess) return e;
        w4_gemv_kernel<MR, GW, kSwiGLU><<<grid, kGemvThreads, p.lds_bytes, s>>>(a);
    } else {
        if ((e = allow_lds(w4_gemv_kernel<MR, GW, kIdentity>, p.lds_bytes)) != hipSuccess) return e;
        w4_gemv_kernel<MR, GW, kIdentity><<<grid, kGemvThreads, p.lds_bytes, s>>>(a);
    }
    return hipGetLastError();
}

template <int MR>
hipError_t launch_mr(Prologue pro, const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
    switch (p.gw) {
        case 1: return launch_mr_gw<MR, 1>(pro, a, p, s);
        case 2: return launch_mr_gw<MR, 2>(pro, a, p, s);
        default: return launch_mr_gw<MR, 4>(pro, a, p, s);
    }
}

int round_gw(int gw) { return gw <= 1 ? 1 : (gw <= 2 ? 2 : 4); }

// ---- test hooks: the same in-register decode, written out ----
__global__ void w4_unpack_kernel(const uint32_t* __restrict__ qw, int KB, int N, int8_t* __restrict__ q) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= int64_t(KB) * N) return;
    const int kb = int(i / N), n = int(i % N);
    const Q4x2 d = decode_int4x8(qw[i]);
    const half2_t p[4] = {d.p04, d.p15, d.p26, d.p37};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const _Float16 v = (j < 4) ? p[j][0] : p[j - 4][1];
        q[(int64_t(kb) * 8 + j) * N + n] = int8_t(float(v));
    }
}

__global__ void w4_dequant_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                                  int KB, int N, float* __restrict__ w) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= int64_t(KB) * N) return;
    const int kb = int(i / N), n = int(i % N);
    const Q4x2 d = decode_int4x8(qw[i]);
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

}  // namespace

GemvPlan plan_gemv(int M, int K, int N) {
    GemvPlan p{};
    p.tiles = (N + kGemvCols - 1) / kGemvCols;
    p.groups = K / kGroup;
    p.mr = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    int gw;
    if (g_forced_split > 0) {
        const int k = std::min(g_forced_split, p.groups);
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
    if (p.splits > 1) {
        p.counter_bytes = (size_t(p.tiles) * 4 + 255) / 256 * 256;
        p.partial_bytes = size_t(p.splits) * M * p.tiles * kGemvCols * 4;
    }
    p.lds_bytes = size_t(p.gps) * p.mr * kGroup * 2 + size_t(p.gps) * p.mr * 4 +
                  size_t(4) * p.mr * kGemvCols * 4;
    return p;
}

size_t gemv_workspace_bytes(int M, int K, int N) {
    const GemvPlan p = plan_gemv(M, K, N);
    return p.counter_bytes + p.partial_bytes;
}

hipError_t launch_gemv(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda,
                       const uint32_t* qw, const uint16_t* sc, int M, int K, int N,
                       const float* out_scale, const uint16_t* residual, uint16_t* y,
                       void* ws, hipStream_t s) {
    const GemvPlan p = plan_gemv(M, K, N);
    GemvArgs a{};
    a.a0 = a0;
    a.a1 = a1;
    a.lda = lda;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.K = K;
    a.N = N;
    a.groups = p.groups;
    a.gps = p.gps;
    a.splits = p.splits;
    a.tiles = p.tiles;
    a.out_scale = out_scale;
    a.residual = residual;
    a.y = y;
    a.counters = p.splits > 1 ? static_cast<unsigned*>(ws) : nullptr;
    a.partial = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.counter_bytes) : nullptr;
    switch (p.mr) {
        case 1: return launch_mr<1>(pro, a, p, s);
        case 2: return launch_mr<2>(pro, a, p, s);
        case 4: return launch_mr<4>(pro, a, p, s);
        case 8: return launch_mr<8>(pro, a, p, s);
        default: return launch_mr<16>(pro, a, p, s);
    }
}

hipError_t launch_w4_unpack(const uint32_t* qw, int K, int N, int8_t* q, hipStream_t s) {
    const int64_t n = int64_t(K / 8) * N;
    w4_unpack_kernel<<<dim3((n + 255) / 256), 256, 0, s>>>(qw, K / 8, N, q);
    return hipGetLastError();
}

hipError_t launch_w4_dequant(const uint32_t* qw, const uint16_t* sc, int K, int N, float* w,
                             hipStream_t s) {
    const int64_t n = int64_t(K / 8) * N;
    w4_dequant_kernel<<<dim3((n + 255) / 256), 256, 0, s>>>(qw, sc, K / 8, N, w);
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

}  // namespace fdec
