// int4 group-quantised GEMV for 5..16 rows on the matrix cores, gfx950.
//
// Same operation as the VALU kernels ("PyTorch Community Proposes Fusion Fix as Large
// Intermediate Buffers May Slow Single-Token Decoding in Quantized LLMs"; "Kernel
// Fusion, torch.compile and CUDA Graphs, Measured", Step 3):
//     y[m, n] = bf16( s * sum_k act[m, k] * q[k, n] * scale[k/128, n]  (+ res[m, n]) )
// with act = silu(g) * u (SwiGLU prologue) or act = x (identity prologue).  At 16 rows
// every weight byte feeds 16 rows of products, which the VALU cannot keep up with at
// HBM speed; v_mfma_f32_16x16x32_f16 does the products, the VALU only decodes.
//
// Row blocks.  A batch of 17..64 rows is RB = 2 or 4 blocks of 16 (either weight format): the
// workgroup stages all 16 RB rows, and each weight word, decoded once per block, feeds
// RB MFMAs, so the weights are read once for the whole batch.  The K slices shrink by RB
// so the staged activation still fits LDS.
//
// Tiling.  A tile is 16 consecutive columns.  A workgroup of W waves owns W * TPW
// tiles (each wave TPW of them) over a slice of whole 128-wide groups of K.  With
// several slices per column range, each workgroup writes its fp32 partial sums to the
// workspace with plain stores, and a second kernel on the same stream sums the slices in
// order and applies the epilogue (splitk_finish_kernel): the kernel boundary makes the
// partials visible.
//
// MFMA mapping (16x16x32, checked on the hardware for the f16 and bf16 forms: lane l
// supplies A[l%16][8(l/16) + e],
// B[8(l/16) + e][l%16] and receives D[4(l/16) + r][l%16]).  A is a tile's weights (row
// = column n of the tile), B the activation (column = row m), D[n][m].  Lane l loads
// the 16-byte chunk (4 packed words, 32 consecutive k) number 4g + l/16 of column
// l%16 of the tile, for group g; word j of it is its A operand in the j-th MFMA of the
// group, so MFMA j of group g covers the k-blocks (8 k each) 16g + 4s + j, s = 0..3.
//
// Decode.  The packed words are decoded as in the VALU column kernel, with their fp16
// offsets left in (1032 + q at even nibble positions, 1152 + 16 q at odd ones, five
// integer ops per word here), in the pair order (j0, j4, j1, j5, j2, j6, j3, j7).  The
// offsets are removed inside the matrix core: each group's accumulation starts from
// the product of a constant matrix of -1032 / -1152 with the same activation operands.
// (A bf16 operand path was measured slower in the main loop, and bf16 loses 3 bits of
// the fp32 SwiGLU activation, which failed the parity bound at K = 14336.)
//
// Activation.  The workgroup stages its slice of act (16 RB rows; rows past M repeat row
// M - 1 and are never stored) in LDS as
// block-scaled fp16 with the odd positions divided by 16 (so each product is a * q plus
// a weight-independent offset): per (row, 128-wide group) a power of two 2^-E puts the
// largest magnitude in [2^14, 2^15); 2^E is folded back in with the group scale.  The
// layout is [row][k-block][8] with a 16-byte pad per row, so the B operands of one MFMA
// (16 rows of one k-block per k-slot) are spread over all LDS banks.  With the SwiGLU
// prologue silu(g) * u is computed in fp32; fp32 -> fp16 rounds toward zero.
//
// FP4 weights (E2M1 codes with E4M3 block scales of 16 along K; template WF = kWFp4).
// The same tiling and staging, with three differences: the activation is staged in k
// order without the 1/16 at odd positions; the A operand of MFMA j is the word's eight
// E2M1 values (v_cvt_scalef32_pk_f16_fp4) times its block scale in fp16 (exact: an E2M1
// value has 2 significant bits, an E4M3 value 4, and every product is a normal fp16
// number), so there are no offsets to remove; and there is no group scale to apply.
#include "device_common.h"
#include "fdec_internal.h"

#include <algorithm>

namespace fdec {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaP = 4;          // groups per batch of weight loads
constexpr int kWInt4 = 0;          // weight formats
constexpr int kWFp4 = 1;
constexpr int kWFp4A4 = 2;         // FP4 weights and FP4 activations (quantised while staged)

struct MfmaArgs {
    const uint16_t* a0;     // g (SwiGLU) or x (identity), row stride lda
    const uint16_t* a1;     // u (SwiGLU) or unused
    int64_t lda;
    const uint4* qw;        // [N][K/32] chunks of 4 words
    const uint16_t* sc;     // bf16 scales [K/128][N] (int4)
    const uint8_t* sc8;     // E4M3 block scales [N][K/16] (FP4)
    const float* gscale;    // FP4 activations: their per-tensor scale G (device fp32)
    int M, K, N;
    int nch;                // K / 32
    int groups;             // K / 128
    int kgroups;            // groups per K slice
    int splits;             // K slices
    int cgroups;            // column ranges (workgroups per slice)
    int npad;               // cgroups * columns per workgroup
    const float* out_scale;
    const uint16_t* residual;
    uint16_t* y;
    float* partial;         // [splits][16 RB][npad]
    uint32_t m_lo, m_hi;    // int4 decode field masks 0x000F000F and 0x00F000F0
    // pair mode (the gate_up projection with the SwiGLU epilogue): N = 2 I, y is act [M][I]
    int half_n;             // I
    int pairs;              // P: gate/up column pairs per workgroup
    // identity prologue, int4 weights, one row block: the activation already staged by its
    // producer ([M][K/8] k-blocks, [M][K/128] powers of two), or null
    const uint4* st;
    const float* stesc;
};

// One packed word -> 8 fp16 values with their offsets, in pair order: the decode every
// int4 kernel runs (decode_int4x8_biased, plain integer code the compiler sees, so it
// spaces an MFMA and a later instruction that writes registers the MFMA still reads).
__device__ __forceinline__ f16x8_t decode_f16x8_biased(uint32_t w, DecodeMasks dm) {
    return __builtin_bit_cast(f16x8_t, decode_int4x8_biased(w, dm));
}

// One staging item: 8 consecutive activation values of one row.  The 16 lanes of a
// DPP row hold the 16 k-blocks of one 128-wide group of that row and share its scale.
// Must be called with the whole wave active.  Returns the fp16 words in pair order;
// *esc = 2^E of the group.  Rows past M need no zeroing: row m of the activation only
// reaches output row m, which is never stored.  With FP4 activations (kWFp4A4) the two
// items of a 16-value block sit in lanes 2i and 2i + 1 (k-blocks 2b and 2b + 1; a row has
// an even number of k-blocks and a workgroup an even number of threads); they take the
// block's largest magnitude from each other and return the exact values q s in k order,
// with *esc = 1.
template <int PRO, int WF>
__device__ __forceinline__ uint4 stage_item_mfma(uint4 gv, uint4 uv, float* esc, float G) {
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
    if (WF == kWFp4A4) {
        mx = fmaxf(mx, dpp<kQuadSwap1>(mx));           // the block's other half (lane ^ 1)
        uint32_t words[1], xq[4];
        (void)nvfp4_quantize_block<8>(v, mx, G, words, xq);
        *esc = 1.0f;
        return make_uint4(xq[0], xq[1], xq[2], xq[3]);
    }
    const float down = stage_group_scale(mx, esc);
    if (WF == kWFp4)   // k order, as v_cvt_scalef32_pk_f16_fp4 produces the weights
        return make_uint4(__builtin_bit_cast(uint32_t, pk_f16_rtz(v[0] * down, v[1] * down)),
                          __builtin_bit_cast(uint32_t, pk_f16_rtz(v[2] * down, v[3] * down)),
                          __builtin_bit_cast(uint32_t, pk_f16_rtz(v[4] * down, v[5] * down)),
                          __builtin_bit_cast(uint32_t, pk_f16_rtz(v[6] * down, v[7] * down)));
    return stage_pair_order(v, down);
}

// The A operand of one MFMA for FP4 weights: the eight values of word w times the
// block scale s (fp16, exact).
__device__ __forceinline__ f16x8_t fp4_operand(uint32_t w, _Float16 s) {
    half2_t q[4];
    fp4x8(w, q);
    const half2_t s2 = {s, s};
    return __builtin_bit_cast(f16x8_t, make_uint4(__builtin_bit_cast(uint32_t, q[0] * s2),
                                                  __builtin_bit_cast(uint32_t, q[1] * s2),
                                                  __builtin_bit_cast(uint32_t, q[2] * s2),
                                                  __builtin_bit_cast(uint32_t, q[3] * s2)));
}

// PAIR: the workgroup owns P = 16 TPW W / 2 column pairs (i, I + i): waves 0 .. W/2 - 1
// take the gate columns cg P + ..., the other half the up columns I + cg P + ...; the
// epilogue writes act[m][i] = bf16(silu(gate) * up) from the two fp32 sums (through LDS
// when the slice is the whole K, else through the partial sums and the pair finish).
template <int TPW, int PRO, int WF, int RB, bool PAIR = false>
__global__ __launch_bounds__(kMfmaWaves * kWave) void w4_gemv_mfma_kernel(MfmaArgs a) {
    constexpr int kRows = 16 * RB;                     // activation rows staged: RB blocks of 16
    // groups per batch of weight loads: several row blocks already give the matrix cores
    // independent chains, and four groups of them would not fit the register file
    constexpr int kP = RB > 1 ? 2 : kMfmaP;
    extern __shared__ __align__(16) unsigned char smem[];
    const int W = blockDim.x >> 6;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ls = lane >> 4, lm = lane & 15;          // k-slot, row / column-in-tile
    const int lb = xcd_remap(blockIdx.x, gridDim.x);
    const int cg = lb % a.cgroups, split = lb / a.cgroups;
    const int g0 = split * a.kgroups;
    const int ng = min(a.kgroups, a.groups - g0);      // groups in this slice
    const int nkb = ng * 16;                           // 8-wide k-blocks in this slice
    const int ncol = W * TPW * 16;                     // columns per workgroup
    const int half = W >> 1;
    const bool up = PAIR && wave >= half;              // pair mode: this wave holds up columns
    const int wl = up ? wave - half : wave;
    // the wave's first column, and its offset inside the workgroup's range of partial sums
    const int col_local = PAIR ? (up ? a.pairs : 0) + wl * TPW * 16 : wave * TPW * 16;
    const int nw0 = PAIR ? (up ? a.half_n : 0) + cg * a.pairs + wl * TPW * 16 : cg * ncol + col_local;
    const int rs = nkb + 1;                            // row stride of act_s, in 16-byte blocks
    uint4* act_s = reinterpret_cast<uint4*>(smem);     // [kRows][rs] of 8 fp16
    // [kRows][es]: an odd row stride puts the 16 rows a wave reads at once in 16 different
    // banks (a stride of 32 groups put them all in one)
    const int es = a.kgroups | 1;
    float* esc_s = reinterpret_cast<float*>(act_s + kRows * rs);

    // the activation already staged by its producer: identity prologue, int4 weights, one
    // row block
    const bool prestaged = PRO == kIdentity && WF == kWInt4 && RB == 1 && a.st != nullptr;

    // ---- weight and scale loads of one batch of groups (addresses clamped) ----
    auto load_batch = [&](int b, uint4 (&w)[kP][TPW], uint2 (&sv)[kP][TPW]) {
#pragma unroll
        for (int p = 0; p < kP; ++p) {
            const int g = g0 + min(b * kP + p, ng - 1);
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int n = min(nw0 + t * 16 + lm, a.N - 1);
                w[p][t] = a.qw[size_t(n) * a.nch + 4 * g + ls];
                if (WF != kWInt4) {
                    // the two E4M3 scales of this lane's chunk (column n, chunk 4g + ls)
                    sv[p][t].x = *reinterpret_cast<const uint16_t*>(a.sc8 + size_t(n) * (a.K / 16) + 2 * (4 * g + ls));
                    sv[p][t].y = 0;
                } else {
                    const int ns = min(nw0 + t * 16 + 4 * ls, a.N - 4);
                    sv[p][t] = *reinterpret_cast<const uint2*>(a.sc + size_t(g) * a.N + ns);
                }
            }
        }
    };

    uint4 wA[kP][TPW], wB[kP][TPW];
    uint2 sA[kP][TPW], sB[kP][TPW];
    // epilogue inputs: 4 consecutive columns of row 16 r + lm per tile
    uint2 rraw[RB][TPW];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            rraw[r][t] = make_uint2(0u, 0u);
            if (PAIR) continue;                                      // no residual (y is [M][I])
            const uint16_t* rsrc = a.residual ? a.residual : a.y;   // y: a readable stand-in, value unused
            rraw[r][t] = *reinterpret_cast<const uint2*>(rsrc + size_t(min(16 * r + lm, a.M - 1)) * a.N +
                                                         min(nw0 + t * 16 + 4 * ls, a.N - 4));
        }
    const float os = a.out_scale ? *a.out_scale : 1.0f;

    // ---- stage the activation slice: item i = (row i / nkb, k-block i % nkb) ----
    // All of a thread's items (up to UMAX of them) are loaded before the first is
    // converted, so the staging waits for one L2 round trip, not one per item.
    const int nitems = nkb * kRows;
    const int kbase = g0 * 128;
    const float G = WF == kWFp4A4 ? *a.gscale : 0.0f;
    constexpr int UMAX = PRO == kSwiGLU ? 12 : 24;
    const int nthr = blockDim.x;
    // Item it has row it / nkb and k-block it % nkb.  A thread's items are nthr apart, so
    // after one division per round the pair is advanced by the (uniform) quotient and
    // remainder of nthr / nkb.
    const int qn = nthr / nkb, rn = nthr - qn * nkb;
    auto advance = [&](int& m, int& kb) {
        kb += rn;
        m += qn;
        if (kb >= nkb) {
            kb -= nkb;
            ++m;
        }
    };
    uint4 gv[UMAX], uv[UMAX];
    auto load_items = [&](int base) {
        int m = (base + tid) / nkb, kb = base + tid - m * nkb;
#pragma unroll
        for (int u = 0; u < UMAX; ++u) {
            if (base + u * nthr >= nitems) break;                   // uniform
            // rows past M (and items past the end) read row M - 1: in bounds, value unused
            const size_t off = size_t(min(m, a.M - 1)) * a.lda + kbase + kb * 8;
            gv[u] = *reinterpret_cast<const uint4*>(a.a0 + off);
            uv[u] = PRO == kSwiGLU ? *reinterpret_cast<const uint4*>(a.a1 + off) : make_uint4(0, 0, 0, 0);
            advance(m, kb);
        }
    };
    auto stage_items = [&](int base) {
        int m = (base + tid) / nkb, kb = base + tid - m * nkb;
#pragma unroll
        for (int u = 0; u < UMAX; ++u) {
            if (base + u * nthr >= nitems) break;                   // uniform: the whole wave stays active
            float esc;
            const uint4 h = stage_item_mfma<PRO, WF>(gv[u], uv[u], &esc, G);
            if (base + u * nthr + tid < nitems) {
                act_s[m * rs + kb] = h;
                if ((kb & 15) == 0) esc_s[m * es + (kb >> 4)] = esc;
            }
            advance(m, kb);
        }
    };
    if (prestaged && nkb % 64 == 0) {
        // a pre-staged slice whose rows are whole 1 KB pieces: the first weights, the
        // slice's powers of two (into registers), then direct-to-LDS loads of the slice (wave
        // load q copies k-blocks 64 q .. 64 q + 63 of the flattened [row][k-block] slice,
        // which stay inside one row): all in flight together, one barrier after them all.
        // (Loading the powers of two with each weight batch instead, straight into
        // registers, measured 8 us slower on the 16-row layer's gate_up.)
        load_batch(0, wA, sA);
        float ev[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) {                // kRows * ng <= 16 * 36 <= 2 * 384
            const int i = tid + it * nthr, m = i / ng, g = i - m * ng;
            ev[it] = i < kRows * ng ? a.stesc[size_t(min(m, a.M - 1)) * (a.K / 128) + g0 + g] : 0.f;
        }
        const int W = blockDim.x >> 6;
        const int rows_per = nkb / 64;                 // 1 KB loads per row
        for (int q = __builtin_amdgcn_readfirstlane(wave); q < kRows * rows_per; q += W) {
            const int m = q / rows_per, kb0 = 64 * (q - m * rows_per);
            __builtin_amdgcn_global_load_lds(a.st + size_t(min(m, a.M - 1)) * (a.K / 8) + g0 * 16 + kb0 + lane,
                                             (__attribute__((address_space(3))) void*)(act_s + m * rs + kb0), 16, 0,
                                             0);
        }
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = tid + it * nthr, m = i / ng, g = i - m * ng;
            if (i < kRows * ng) esc_s[m * es + g] = ev[it];
        }
        __syncthreads();
    } else if (prestaged) {
        // a pre-staged slice of any length: copied through registers
        for (int i = tid; i < nitems; i += nthr) {
            const int m = i / nkb, kb = i - m * nkb;
            act_s[m * rs + kb] = a.st[size_t(min(m, a.M - 1)) * (a.K / 8) + g0 * 16 + kb];
        }
        for (int i = tid; i < kRows * ng; i += nthr) {
            const int m = i / ng, g = i - m * ng;
            esc_s[m * es + g] = a.stesc[size_t(min(m, a.M - 1)) * (a.K / 128) + g0 + g];
        }
        load_batch(0, wA, sA);
        __syncthreads();
    } else {
        for (int base = 0; base < nitems; base += UMAX * nthr) {       // uniform trip count
            load_items(base);
            stage_items(base);
        }
        // the first weights are requested only now: issued earlier, they would sit ahead of
        // the activation loads in the CU's memory queue and every staging wait would cover them
        load_batch(0, wA, sA);
        __syncthreads();
    }

    // ---- main loop: batches of kP groups, next batch's loads in flight ----
    f32x4_t out[RB][TPW];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < TPW; ++t) out[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // -offset of each pair-order slot: (-1032, -1032), (-1152, -1152), ...
    const uint32_t o_even = 0xE408E408u, o_odd = 0xE480E480u;
    const f16x8_t negoff = __builtin_bit_cast(f16x8_t, make_uint4(o_even, o_odd, o_even, o_odd));

    // The kP groups of a batch are independent accumulation chains; their MFMAs are
    // interleaved so that no MFMA waits on the one issued just before it.  A group past
    // the slice's end re-reads the last group and contributes with weight 0.  With
    // several row blocks the same weight registers feed each block's MFMAs in turn.
    auto compute_batch = [&](int b, const uint4 (&w)[kP][TPW], const uint2 (&sv)[kP][TPW]) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int row = 16 * r + lm;
        f16x8_t bop[kP][4];
        float e[kP];
#pragma unroll
        for (int p = 0; p < kP; ++p) {
            const int gl = min(b * kP + p, ng - 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) bop[p][j] = __builtin_bit_cast(f16x8_t, act_s[row * rs + 16 * gl + 4 * ls + j]);
            e[p] = b * kP + p < ng ? esc_s[row * es + gl] : 0.f;
        }
        f32x4_t bias[kP];
#pragma unroll
        for (int p = 0; p < kP; ++p) bias[p] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (WF == kWInt4) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int p = 0; p < kP; ++p)
                    bias[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(negoff, bop[p][j], bias[p], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            f32x4_t d[kP];
#pragma unroll
            for (int p = 0; p < kP; ++p) d[p] = bias[p];
            _Float16 fs[kP][2];
            if (WF != kWInt4) {
#pragma unroll
                for (int p = 0; p < kP; ++p) {
                    fs[p][0] = (_Float16)e4m3_to_f32(sv[p][t].x & 0xFFu);
                    fs[p][1] = (_Float16)e4m3_to_f32(sv[p][t].x >> 8);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int p = 0; p < kP; ++p) {
                    const uint32_t wd = j == 0 ? w[p][t].x : j == 1 ? w[p][t].y : j == 2 ? w[p][t].z : w[p][t].w;
                    const f16x8_t aop = WF != kWInt4 ? fp4_operand(wd, fs[p][j >> 1]) : decode_f16x8_biased(wd, DecodeMasks{a.m_lo, a.m_hi});
                    d[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[p][j], d[p], 0, 0, 0);
                }
#pragma unroll
            for (int p = 0; p < kP; ++p) {
                if (WF != kWInt4) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) out[r][t][q] = fmaf(e[p], d[p][q], out[r][t][q]);
                } else {
                    out[r][t][0] = fmaf(bf16_lo(sv[p][t].x) * e[p], d[p][0], out[r][t][0]);
                    out[r][t][1] = fmaf(bf16_hi(sv[p][t].x) * e[p], d[p][1], out[r][t][1]);
                    out[r][t][2] = fmaf(bf16_lo(sv[p][t].y) * e[p], d[p][2], out[r][t][2]);
                    out[r][t][3] = fmaf(bf16_hi(sv[p][t].y) * e[p], d[p][3], out[r][t][3]);
                }
            }
        }
      }
    };

    const int nbatch = (ng + kP - 1) / kP;
    for (int b = 0; b < nbatch; b += 2) {
        load_batch(b + 1, wB, sB);                     // clamped: harmless past the end
        compute_batch(b, wA, sA);
        load_batch(b + 2, wA, sA);
        compute_batch(b + 1, wB, sB);
    }

    // ---- epilogue: lane holds D[column 4 ls + q][row 16 r + lm] of each tile ----
    if (PAIR && a.splits == 1) {
        // the up waves hand their sums to the gate waves through LDS (act_s is free once
        // every wave has finished its main loop)
        float4* xs = reinterpret_cast<float4*>(smem);      // [W/2][RB][TPW][64]
        __syncthreads();
        if (up) {
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    xs[((wl * RB + r) * TPW + t) * kWave + lane] =
                        make_float4(out[r][t][0], out[r][t][1], out[r][t][2], out[r][t][3]);
        }
        __syncthreads();
        if (!up) {
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const float4 u = xs[((wl * RB + r) * TPW + t) * kWave + lane];
                    const int i = nw0 + t * 16 + 4 * ls;          // four pairs i .. i + 3 (I % 8 == 0)
                    const int row = 16 * r + lm;
                    if (row < a.M && i < a.half_n) {
                        uint2 o;
                        o.x = pack_bf16x2(silu_f32(out[r][t][0]) * u.x, silu_f32(out[r][t][1]) * u.y);
                        o.y = pack_bf16x2(silu_f32(out[r][t][2]) * u.z, silu_f32(out[r][t][3]) * u.w);
                        *reinterpret_cast<uint2*>(a.y + size_t(row) * a.half_n + i) = o;
                    }
                }
        }
        return;
    }
    if (!PAIR && a.splits == 1) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int n = nw0 + t * 16 + 4 * ls;
                const int row = 16 * r + lm;
                if (row < a.M && n < a.N) {
                    const uint2 rr = rraw[r][t];
                    const float r0 = a.residual ? bf16_lo(rr.x) : 0.f, r1 = a.residual ? bf16_hi(rr.x) : 0.f;
                    const float r2 = a.residual ? bf16_lo(rr.y) : 0.f, r3 = a.residual ? bf16_hi(rr.y) : 0.f;
                    uint2 o;
                    o.x = pack_bf16x2(fmaf(out[r][t][0], os, r0), fmaf(out[r][t][1], os, r1));
                    o.y = pack_bf16x2(fmaf(out[r][t][2], os, r2), fmaf(out[r][t][3], os, r3));
                    *reinterpret_cast<uint2*>(a.y + size_t(row) * a.N + n) = o;
                }
            }
        return;
    }

    // ---- several K slices: this slice's partial sums (all kRows rows), plain stores ----
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int nc = col_local + t * 16 + 4 * ls;          // column within the range
            float* dst = a.partial + (size_t(split) * kRows + 16 * r + lm) * a.npad + cg * ncol + nc;
            *reinterpret_cast<float4*>(dst) = make_float4(out[r][t][0], out[r][t][1], out[r][t][2], out[r][t][3]);
        }
}

template <typename Kern>
hipError_t launch_k(Kern k, dim3 grid, int threads, size_t lds, hipStream_t s, const MfmaArgs& a) {
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, grid, dim3(threads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

namespace {

template <int WF>
hipError_t launch_mfma_wf(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda, const uint32_t* qw,
                          const uint16_t* sc, const uint8_t* sc8, int M, int K, int N, const float* out_scale,
                          const uint16_t* residual, uint16_t* y, void* ws, const GemvPlan& p, hipStream_t s,
                          const float* gscale = nullptr, const void* xs = nullptr, const float* xesc = nullptr) {
    MfmaArgs a{};
    a.gscale = gscale;
    // a pre-staged activation: identity prologue, int4 weights, one row block
    a.st = WF == kWInt4 && pro == kIdentity && p.mr == 16 ? static_cast<const uint4*>(xs) : nullptr;
    a.stesc = xesc;
    a.a0 = a0;
    a.a1 = a1;
    a.lda = lda;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.sc8 = sc8;
    a.M = M;
    a.K = K;
    a.N = N;
    a.nch = K / 32;
    a.groups = p.groups;
    a.kgroups = p.gps;
    a.splits = p.splits;
    a.cgroups = p.tiles;
    a.npad = p.tiles * p.waves * p.cpw * 16;
    a.out_scale = out_scale;
    a.residual = residual;
    a.y = y;
    a.partial = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    a.m_lo = kDecodeMaskLo;
    a.m_hi = kDecodeMaskHi;
    const dim3 grid(p.tiles * p.splits);
    const int threads = p.waves * kWave;
    // one 16-column tile per wave (two per wave measured slower: more registers and a
    // K split for the same workgroup count); p.mr / 16 row blocks
    const int rb = p.mr / 16;
    if (M > p.mr || (rb != 1 && rb != 2 && rb != 4)) return hipErrorInvalidValue;
    hipError_t e;
    if (rb == 1)
        e = pro == kSwiGLU ? launch_k(w4_gemv_mfma_kernel<1, kSwiGLU, WF, 1>, grid, threads, p.lds_bytes, s, a)
                           : launch_k(w4_gemv_mfma_kernel<1, kIdentity, WF, 1>, grid, threads, p.lds_bytes, s, a);
    else if (rb == 2)
        e = pro == kSwiGLU ? launch_k(w4_gemv_mfma_kernel<1, kSwiGLU, WF, 2>, grid, threads, p.lds_bytes, s, a)
                           : launch_k(w4_gemv_mfma_kernel<1, kIdentity, WF, 2>, grid, threads, p.lds_bytes, s, a);
    else
        e = pro == kSwiGLU ? launch_k(w4_gemv_mfma_kernel<1, kSwiGLU, WF, 4>, grid, threads, p.lds_bytes, s, a)
                           : launch_k(w4_gemv_mfma_kernel<1, kIdentity, WF, 4>, grid, threads, p.lds_bytes, s, a);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_finish(a.partial, p.splits, int64_t(p.mr) * a.npad, a.npad, M, N, out_scale, residual, y, s);
}

// act[m][i] = bf16(silu(g) * u), with g and u the sums over the K slices (in slice order)
// of the pair's gate and up partials: pair i of column-pair range cg = i / P sits at
// columns cg 2P + i % P (gate) and cg 2P + P + i % P (up) of a slice's [rows][npad]
// partials.  Runs after the kernel that wrote them, on the same stream.
__global__ __launch_bounds__(256) void splitk_finish_swiglu_kernel(const float* __restrict__ partial, int splits,
                                                                  int64_t split_stride, int64_t row_stride, int M,
                                                                  int I, int P, uint16_t* act) {
    const int o = blockIdx.x * 256 + threadIdx.x;
    if (o >= M * I) return;
    const int m = o / I, i = o % I;
    const float* pg = partial + m * row_stride + size_t(i / P) * 2 * P + i % P;
    const float* pu = pg + P;
    // every slice of a batch requested before the first is used (one memory round trip
    // per kFinishBatch slices, not one per slice); sums in slice order
    float g = 0.f, u = 0.f;
    for (int s0 = 0; s0 < splits; s0 += kFinishBatch) {
        float tg[kFinishBatch], tu[kFinishBatch];
#pragma unroll
        for (int b = 0; b < kFinishBatch; ++b) {
            tg[b] = s0 + b < splits ? pg[(s0 + b) * split_stride] : 0.f;
            tu[b] = s0 + b < splits ? pu[(s0 + b) * split_stride] : 0.f;
        }
#pragma unroll
        for (int b = 0; b < kFinishBatch; ++b) {
            g += tg[b];
            u += tu[b];
        }
    }
    act[o] = f32_to_bf16(silu_f32(g) * u);
}

}  // namespace

hipError_t launch_splitk_finish_swiglu(const float* partial, int splits, int64_t split_stride, int64_t row_stride,
                                       int M, int I, int P, uint16_t* act, hipStream_t s) {
    splitk_finish_swiglu_kernel<<<dim3((M * I + 255) / 256), 256, 0, s>>>(partial, splits, split_stride, row_stride, M,
                                                                         I, P, act);
    return hipGetLastError();
}

hipError_t launch_mfma_pair(const uint16_t* x, const uint32_t* qw, const uint16_t* sc, int M, int K, int I,
                            uint16_t* act, void* ws, const GemvPlan& p, hipStream_t s, const void* xs,
                            const float* xesc) {
    if (p.kind == kRing) return launch_ring_pair(x, qw, sc, M, K, I, act, ws, p, s);
    MfmaArgs a{};
    a.st = p.mr == 16 ? static_cast<const uint4*>(xs) : nullptr;
    a.stesc = xesc;
    a.a0 = x;
    a.lda = K;
    a.qw = reinterpret_cast<const uint4*>(qw);
    a.sc = sc;
    a.M = M;
    a.K = K;
    a.N = 2 * I;
    a.nch = K / 32;
    a.groups = p.groups;
    a.kgroups = p.gps;
    a.splits = p.splits;
    a.cgroups = p.tiles;
    a.npad = p.tiles * p.waves * p.cpw * 16;
    a.y = act;
    a.partial = p.splits > 1 ? static_cast<float*>(ws) : nullptr;
    a.m_lo = kDecodeMaskLo;
    a.m_hi = kDecodeMaskHi;
    a.half_n = I;
    a.pairs = p.waves / 2 * p.cpw * 16;
    const dim3 grid(p.tiles * p.splits);
    const int threads = p.waves * kWave;
    const int rb = p.mr / 16;
    if (M > p.mr || (rb != 1 && rb != 2 && rb != 4) || p.cpw != 1 || p.waves % 2) return hipErrorInvalidValue;
    hipError_t e;
    if (rb == 1)
        e = launch_k(w4_gemv_mfma_kernel<1, kIdentity, kWInt4, 1, true>, grid, threads, p.lds_bytes, s, a);
    else if (rb == 2)
        e = launch_k(w4_gemv_mfma_kernel<1, kIdentity, kWInt4, 2, true>, grid, threads, p.lds_bytes, s, a);
    else
        e = launch_k(w4_gemv_mfma_kernel<1, kIdentity, kWInt4, 4, true>, grid, threads, p.lds_bytes, s, a);
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_finish_swiglu(a.partial, p.splits, int64_t(p.mr) * a.npad, a.npad, M, I, a.pairs, act, s);
}

hipError_t launch_mfma(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda,
                       const uint32_t* qw, const uint16_t* sc, int M, int K, int N,
                       const float* out_scale, const uint16_t* residual, uint16_t* y,
                       void* ws, const GemvPlan& p, hipStream_t s, const void* xs, const float* xesc) {
    return launch_mfma_wf<kWInt4>(pro, a0, a1, lda, qw, sc, nullptr, M, K, N, out_scale, residual, y, ws, p, s,
                                  nullptr, xs, xesc);
}

hipError_t launch_mfma_fp4(Prologue pro, const uint16_t* a0, const uint16_t* a1, int64_t lda,
                           const uint32_t* qw, const uint8_t* sc8, int M, int K, int N,
                           const float* out_scale, const uint16_t* residual, uint16_t* y,
                           void* ws, const GemvPlan& p, const float* gscale, hipStream_t s) {
    if (gscale)
        return launch_mfma_wf<kWFp4A4>(pro, a0, a1, lda, qw, nullptr, sc8, M, K, N, out_scale, residual, y, ws, p, s,
                                       gscale);
    return launch_mfma_wf<kWFp4>(pro, a0, a1, lda, qw, nullptr, sc8, M, K, N, out_scale, residual, y, ws, p, s);
}

}  // namespace fdec
