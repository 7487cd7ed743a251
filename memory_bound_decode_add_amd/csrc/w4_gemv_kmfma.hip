// int4 group-quantised GEMV for 5..16 rows on the matrix cores, with the workgroup's
// waves splitting K, gfx950.
//
// Same operation as the other int4 kernels ("PyTorch Community Proposes Fusion Fix as
// Large Intermediate Buffers May Slow Single-Token Decoding in Quantized LLMs"; "Kernel
// Fusion, torch.compile and CUDA Graphs, Measured", Step 3):
//     y[m, n] = bf16( s * sum_k act[m, k] * q[k, n] * scale[k/128, n]  (+ res[m, n]) )
// with act = silu(g) * u (SwiGLU prologue) or act = x (identity prologue).
//
// Work assignment.  A workgroup of W waves (6..8) owns T tiles of 16 columns over a K
// slice of W GW whole 128-wide groups;
// wave w takes GW consecutive groups of the slice for all T tiles.  So a wave needs the
// activation of its own GW groups only (16 rows x 128 GW values), which it loads straight
// into the registers that are its MFMA B operands: there is no activation staging in LDS
// and no barrier before the matrix cores start.  Every activation load and the weights of
// the first two groups are requested at entry, activation first; each group's weights
// (T 16-byte chunks per lane) feed T MFMA chains.  The waves' fp32 sums meet once, in LDS,
// in a fixed order; then either the epilogue runs, or (K split into several slices) the
// workgroup's sums go to the workspace and splitk_finish_kernel adds the slices in order.
//
// Where it runs.  Measured against the row-block kernel (which stages the activation in
// LDS before any weight is requested) at 8 and 16 rows: faster with the SwiGLU prologue
// and one group per wave (every load of the workgroup in flight at once) up to about
// 12 MB of weights -- 16 x 9216 x 2560: 11.0 against 12.2 us; 16 x 4096 x 4096: 8.7
// against 10.6 us -- and slower beyond (16 x 14336 x 4096: 18.4 against 16.4 us), with
// the identity prologue (whose staging is cheap) and with more groups per wave (each
// group then waits for the one before).  plan_gemv takes it for that range only.
//
// MFMA mapping (v_mfma_f32_16x16x32_f16, lane l: A[l%16][8(l/16)+e], B[8(l/16)+e][l%16],
// D[4(l/16)+r][l%16]).  A is a tile's weights (row = column n of the tile), B the
// activation (column = row m), D[n][m].  For group g, lane l loads chunk 4g + l/16 (32
// consecutive k) of column l%16 of each tile, and word j of it is its A operand in MFMA j;
// the matching B operand is the 8 activation values of the same k, row l%16 -- so a lane's
// B operands for the four MFMAs of a group are the 32 consecutive activation values of
// row l%16 at k = 128 g + 32 (l/16): one contiguous 64-byte piece of the row.
//
// Decode and offsets as in the other int4 kernels: decode_int4x8_biased gives fp16
// 1032 + q (even positions) and 1152 + 16 q (odd), the activation is stored with odd
// positions divided by 16 in the pair order (j0, j4, j1, j5, j2, j6, j3, j7), and the
// offsets are removed by starting each group's accumulation from what a constant
// -1032 / -1152 matrix times the group's B operands gives: per row, the offsets summed
// against the row's staged values (16 dot2 per lane and two lane swaps per wave and group,
// shared by all T tiles; four MFMAs of that matrix measured 0.27 us slower at 8 and 16
// rows, K = 9216, N = 2560).  The activation is block-scaled fp16: per (row, group) a
// power of two puts the group's largest magnitude in [2^14, 2^15), folded back in with
// the group scale; fp32 -> fp16 rounds toward zero.
#include "device_common.h"
#include "fdec_internal.h"

#include <algorithm>

namespace fdec {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKWaves = 8;          // waves per workgroup, at most (KArgs::nw)

struct KArgs {
    const uint16_t* a0;     // g (SwiGLU) or x (identity), row stride lda
    const uint16_t* a1;     // u (SwiGLU) or unused
    int64_t lda;
    const uint4* qw;        // [N][K/32] chunks of 4 words
    const uint16_t* sc;     // bf16 scales [K/128][N]
    int M, N;
    int nch;                // K / 32
    int groups;             // K / 128
    int cgroups;            // column ranges (workgroups per K slice)
    int splits;             // K slices of nw GW groups
    int nw;                 // waves per workgroup (the kernel's W)
    int npad;               // cgroups * 16 T: columns of a slice's partial sums
    const float* out_scale;
    const uint16_t* residual;
    uint16_t* y;            // [M][N], or act [M][I] in pair mode
    float* partial;         // [splits][16][npad]
    DecodeMasks dm;
};

template <int PRO, int T, int GW, int W>
__global__ __launch_bounds__(kKWaves * kWave) void w4_gemv_kmfma_kernel(KArgs a) {
    static_assert(W >= 6 && W <= kKWaves, "6..8 waves");
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ls = lane >> 4, lm = lane & 15;
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int cg = lb % a.cgroups, split = lb / a.cgroups;
    const int gw0 = (split * W + wave) * GW;           // this wave's first group
    auto tile_col = [&](int t) { return cg * 16 * T + 16 * t; };   // first column of tile t

    // ---- activation: rows past M read row M - 1 (never stored); groups past K read the
    // last group and get weight 0 ----
    const int row = min(lm, a.M - 1);
    uint4 gr[GW][4], ur[GW][4];
#pragma unroll
    for (int gi = 0; gi < GW; ++gi) {
        const int g = min(gw0 + gi, a.groups - 1);
        const uint16_t* src0 = a.a0 + size_t(row) * a.lda + g * 128 + ls * 32;
        const uint16_t* src1 = a.a1 + size_t(row) * a.lda + g * 128 + ls * 32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            gr[gi][j] = *reinterpret_cast<const uint4*>(src0 + 8 * j);
            ur[gi][j] = PRO == kSwiGLU ? *reinterpret_cast<const uint4*>(src1 + 8 * j) : make_uint4(0, 0, 0, 0);
        }
    }

    // ---- weights and scales of a group, all T tiles (addresses clamped) ----
    uint4 wv[2][T];
    uint2 sv[2][T];
    auto load_group = [&](int gi, uint4 (&w)[T], uint2 (&s)[T]) {
        const int g = min(gw0 + gi, a.groups - 1);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int c0 = tile_col(t);
            const int n = min(c0 + lm, a.N - 1);
            w[t] = nt_load(a.qw + size_t(n) * a.nch + 4 * g + ls);
            s[t] = *reinterpret_cast<const uint2*>(a.sc + size_t(g) * a.N + min(c0 + 4 * ls, a.N - 4));
        }
    };
    load_group(0, wv[0], sv[0]);
    if (GW > 1) load_group(1, wv[1], sv[1]);

    // ---- the B operands: block-scaled fp16 in pair order, odd positions / 16 ----
    f16x8_t bop[GW][4];
    float esc[GW], off[GW];
#pragma unroll
    for (int gi = 0; gi < GW; ++gi) {
        float v[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t gw[4] = {gr[gi][j].x, gr[gi][j].y, gr[gi][j].z, gr[gi][j].w};
            const uint32_t uw[4] = {ur[gi][j].x, ur[gi][j].y, ur[gi][j].z, ur[gi][j].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if (PRO == kSwiGLU) {
                    v[j][2 * h] = silu_f32(bf16_lo(gw[h])) * bf16_lo(uw[h]);
                    v[j][2 * h + 1] = silu_f32(bf16_hi(gw[h])) * bf16_hi(uw[h]);
                } else {
                    v[j][2 * h] = bf16_lo(gw[h]);
                    v[j][2 * h + 1] = bf16_hi(gw[h]);
                }
            }
        }
        float mx = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[j][e]));
        // the group's 128 values of row lm sit in lanes lm, lm + 16, lm + 32, lm + 48;
        // magnitudes order as their bit patterns do
        uint32_t mb = __builtin_bit_cast(uint32_t, mx);
        mb = max(mb, uint32_t(__shfl_xor(int(mb), 16, kWave)));
        mb = max(mb, uint32_t(__shfl_xor(int(mb), 32, kWave)));
        int ex = 0;
        (void)__builtin_frexpf(__builtin_bit_cast(float, mb), &ex);
        const int E = min(max(ex - 15, -126), 127);
        const float down = __builtin_ldexpf(1.0f, -E);
        const float down16 = down * 0.0625f;
        esc[gi] = gw0 + gi < a.groups ? __builtin_ldexpf(1.0f, E) : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bop[gi][j] = __builtin_bit_cast(
                f16x8_t, make_uint4(__builtin_bit_cast(uint32_t, pk_f16_rtz(v[j][0] * down, v[j][4] * down)),
                                    __builtin_bit_cast(uint32_t, pk_f16_rtz(v[j][1] * down16, v[j][5] * down16)),
                                    __builtin_bit_cast(uint32_t, pk_f16_rtz(v[j][2] * down, v[j][6] * down)),
                                    __builtin_bit_cast(uint32_t, pk_f16_rtz(v[j][3] * down16, v[j][7] * down16))));
        // The decode's offsets: -1032 at the even pair slots and -1152 at the odd ones,
        // summed against the group's 128 staged values of row lm (what the constant offset
        // matrix times these B operands gives in every column).  The row's four lanes
        // (lm + 16 ls) meet through the half-wave and row swaps.
        const half2_t ne = {(_Float16)-1032.0f, (_Float16)-1032.0f};
        const half2_t no = {(_Float16)-1152.0f, (_Float16)-1152.0f};
        float ob = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 h = __builtin_bit_cast(uint4, bop[gi][j]);
            ob = dot2(__builtin_bit_cast(half2_t, h.x), ne, ob);
            ob = dot2(__builtin_bit_cast(half2_t, h.z), ne, ob);
            ob = dot2(__builtin_bit_cast(half2_t, h.y), no, ob);
            ob = dot2(__builtin_bit_cast(half2_t, h.w), no, ob);
        }
        const f32x2_t oh = swap32(ob, ob);
        const f32x2_t orw = swap16(oh[0] + oh[1], oh[0] + oh[1]);
        off[gi] = orw[0] + orw[1];
    }

    // ---- main loop over the wave's groups, the next group's loads in flight ----
    f32x4_t out[T];
#pragma unroll
    for (int t = 0; t < T; ++t) out[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < GW; ++gi) {
        const int buf = gi & 1;
        const f32x4_t bias = f32x4_t{off[gi], off[gi], off[gi], off[gi]};
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint32_t wd[4] = {wv[buf][t].x, wv[buf][t].y, wv[buf][t].z, wv[buf][t].w};
            f32x4_t d = bias;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(f16x8_t, decode_int4x8_biased(wd[j], a.dm)), bop[gi][j], d, 0, 0, 0);
            out[t][0] = fmaf(bf16_lo(sv[buf][t].x) * esc[gi], d[0], out[t][0]);
            out[t][1] = fmaf(bf16_hi(sv[buf][t].x) * esc[gi], d[1], out[t][1]);
            out[t][2] = fmaf(bf16_lo(sv[buf][t].y) * esc[gi], d[2], out[t][2]);
            out[t][3] = fmaf(bf16_hi(sv[buf][t].y) * esc[gi], d[3], out[t][3]);
        }
        if (gi + 2 < GW) load_group(gi + 2, wv[buf], sv[buf]);
    }

    // ---- the waves' sums meet in LDS: red[w][t][lane], lane = (ls, lm) holds rows lm,
    // columns 4 ls .. 4 ls + 3 of tile t ----
    float4* red = reinterpret_cast<float4*>(smem);
#pragma unroll
    for (int t = 0; t < T; ++t) red[(wave * T + t) * kWave + lane] = make_float4(out[t][0], out[t][1], out[t][2], out[t][3]);
    __syncthreads();
    // wave w sums the waves' values of tiles w, w + W, ..., lane ln = (ls, lm) its quad,
    // in wave order
    const int ln = lane;
    auto wave_sum = [&](int tt) {
        float4 acc = red[tt * kWave + ln];
#pragma unroll
        for (int w = 1; w < W; ++w) {
            const float4 v = red[(w * T + tt) * kWave + ln];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        return acc;
    };
    const int orow = ln & 15, oc = 4 * (ln >> 4);        // row, column offset in the tile
#pragma unroll
    for (int t0 = 0; t0 < T; t0 += W) {
        const int t = t0 + wave;
        if (t >= T) break;                                 // uniform across the wave
        if (a.splits > 1) {
            const float4 v = wave_sum(t);
            float* dst = a.partial + (size_t(split) * 16 + orow) * a.npad + cg * 16 * T + 16 * t + oc;
            *reinterpret_cast<float4*>(dst) = v;
            continue;
        }
        const int n = tile_col(t) + oc;
        if (orow >= a.M || n >= a.N) continue;
        const float4 v = wave_sum(t);
        const float os = a.out_scale ? *a.out_scale : 1.0f;
        float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
        if (a.residual) {
            const uint2 rr = *reinterpret_cast<const uint2*>(a.residual + size_t(orow) * a.N + n);
            r0 = bf16_lo(rr.x);
            r1 = bf16_hi(rr.x);
            r2 = bf16_lo(rr.y);
            r3 = bf16_hi(rr.y);
        }
        uint2 o;
        o.x = pack_bf16x2(fmaf(v.x, os, r0), fmaf(v.y, os, r1));
        o.y = pack_bf16x2(fmaf(v.z, os, r2), fmaf(v.w, os, r3));
        *reinterpret_cast<uint2*>(a.y + size_t(orow) * a.N + n) = o;
    }
}

template <int PRO, int T, int GW, int W>
hipError_t launch_kmfma5(const KArgs& a, const GemvPlan& p, hipStream_t s) {
    const auto k = w4_gemv_kmfma_kernel<PRO, T, GW, W>;
    const size_t lds = size_t(W) * T * kWave * 16;
    if (lds > 65536) {
        const hipError_t e =
            hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    k<<<dim3(p.tiles * p.splits), dim3(W * kWave), lds, s>>>(a);
    return hipGetLastError();
}

template <int PRO, int T, int GW>
hipError_t launch_kmfma4(const KArgs& a, const GemvPlan& p, hipStream_t s) {
    switch (a.nw) {
        case 6: return launch_kmfma5<PRO, T, GW, 6>(a, p, s);
        case 7: return launch_kmfma5<PRO, T, GW, 7>(a, p, s);
        default: return launch_kmfma5<PRO, T, GW, 8>(a, p, s);
    }
}

template <int PRO, int T>
hipError_t launch_kmfma3(const KArgs& a, const GemvPlan& p, hipStream_t s) {
    switch (p.gw) {
        case 1: return launch_kmfma4<PRO, T, 1>(a, p, s);
        case 2: return launch_kmfma4<PRO, T, 2>(a, p, s);
        case 3: return PRO == kSwiGLU ? hipErrorInvalidValue : launch_kmfma4<PRO, T, 3>(a, p, s);
        default: return PRO == kSwiGLU ? hipErrorInvalidValue : launch_kmfma4<PRO, T, 4>(a, p, s);
    }
}

template <int PRO>
hipError_t launch_kmfma2(const KArgs& a, const GemvPlan& p, hipStream_t s) {
    return p.cpw == 8 ? launch_kmfma3<PRO, 8>(a, p, s) : launch_kmfma3<PRO, 4>(a, p, s);
}

}  // namespace

// T (tiles of 16 columns per workgroup, 8 or 4; p.cpw), GW (groups per wave, 1..max_gw;
// the SwiGLU prologue takes at most 2, its raw g and u needing twice the registers; p.gw)
// and W (waves per workgroup, 8 down to 6; p.waves): the choice with the least estimated
// time, counted in (16-column, 128-k) weight blocks per workgroup times rounds of
// workgroups over 256 CUs, plus about 75 such blocks for the slice-summing kernel when K
// is split; ties go to more waves.  Fewer than 8 waves make thinner K slices, hence more
// workgroups: measured on MI355X at 16 rows, 9216 x 2560 takes 8 tiles and 6 waves (240
// workgroups; 10.7 against 11.0 us with 8 waves), 8960 x 1536 4 tiles and 7 waves (240;
// 8.7 against 9.3 us), while 4096 x 4096 and 8192 x 2048 keep 4 tiles and 8 waves (256).
bool plan_kmfma(int M, int K, int N, int max_gw, GemvPlan& p, const Overrides& ov) {
    p = GemvPlan{};
    if (M < 1 || M > 16 || K <= 0 || K % kGroup || N <= 0 || N % 8) return false;
    p.kind = kKMfma;
    p.mr = 16;
    p.groups = K / kGroup;
    double best = 1e30;
    for (int W = kKWaves; W >= 6; --W) {
        if (ov.mfma_waves && W != ov.mfma_waves) continue;
        for (int T : {8, 4}) {
            if (ov.mfma_tiles && T != ov.mfma_tiles) continue;
            const int ranges = (N + 16 * T - 1) / (16 * T);
            for (int gw = std::min(max_gw, 4); gw >= 1; --gw) {
                if (ov.mfma_gw && gw != ov.mfma_gw) continue;
                const int slice = W * gw;
                const int S = (p.groups + slice - 1) / slice;
                const int wgs = ranges * S;
                const double cost = double((wgs + 255) / 256) * T * std::min(slice, p.groups) + (S > 1 ? 75.0 : 0.0);
                if (cost < best - 1e-9) {
                    best = cost;
                    p.cpw = T;
                    p.gw = gw;
                    p.waves = W;
                    p.tiles = ranges;
                    p.splits = S;
                }
            }
        }
    }
    if (best >= 1e29) return false;
    p.gps = p.waves * p.gw;
    if (p.splits > 1) p.partial_bytes = size_t(p.splits) * 16 * p.tiles * 16 * p.cpw * 4;
    p.lds_bytes = size_t(p.waves) * p.cpw * kWave * 16;
    return true;
}

hipError_t launch_kmfma(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda, const uint32_t* qw,
                        const uint16_t* sc, int M, int K, int N, const float* out_scale, const uint16_t* residual,
                        uint16_t* y, void* ws, const GemvPlan& p, hipStream_t s) {
    KArgs a{};
    a.a0 = a0;
    a.a1 = pro == kSwiGLU ? a1 : a0;
    a.lda = lda;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.N = N;
    a.nch = K / 32;
    a.groups = p.groups;
    a.cgroups = p.tiles;
    a.splits = p.splits;
    a.nw = p.waves;
    a.npad = p.tiles * 16 * p.cpw;
    a.out_scale = out_scale;
    a.residual = residual;
    a.y = y;
    a.partial = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    a.dm = DecodeMasks{kDecodeMaskLo, kDecodeMaskHi};
    if (p.kind != kKMfma || M > 16 || (p.cpw != 4 && p.cpw != 8) || p.gw < 1 || p.gw > 4 || p.waves < 6 ||
        p.waves > kKWaves)
        return hipErrorInvalidValue;
    const hipError_t e = pro == kSwiGLU ? launch_kmfma2<kSwiGLU>(a, p, s) : launch_kmfma2<kIdentity>(a, p, s);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_finish(a.partial, p.splits, int64_t(16) * a.npad, a.npad, M, N, out_scale, residual, y, s);
}

}  // namespace fdec
