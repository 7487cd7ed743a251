// Device helpers shared by the fdec kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fdec {

constexpr int kWave = 64;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  A bf16 pattern is the top half of an fp32 pattern, so widening
// is a shift; narrowing uses gfx950's v_cvt_pk_bf16_f32 (round to nearest even).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two floats -> one word of two bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// ---------------------------------------------------------------------------
// int4 decode, shared by every int4 kernel (column, split-K, matrix-core) and by the
// unpack/dequant test hooks.  A packed word holds weights j = 0..7 of one column in
// bits [4j, 4j+4) as two's-complement nibbles.  XOR-ing a nibble with 8 turns its code
// into q + 8 (offset binary, 0..15); placing that 4-bit field in the mantissa of the
// fp16 value 1024 (0x6400) gives an exact fp16 number:
//   field in bits 0..3 of a half  -> 1024 + (q + 8)     = 1032 + q
//   field in bits 4..7 of a half  -> 1024 + 16 (q + 8)  = 1152 + 16 q
// One word becomes four half2 pairs ordered (j0, j4), (j1, j5), (j2, j6), (j3, j7)
// ("pair order"); the activations are stored in the same order, so a dot2 (or an MFMA
// k-slot) of matching pairs sums the right products.  The kernels keep the offsets in
// and remove them once per chunk or group; decode_int4x8 removes them per value.
//
// Each field is K ^ (v & m): inside the nibble mask m the XOR flips the code to offset
// binary, outside it are the bits of 1024, which share none with m, so K holds 1024's
// bits and an 8 in each masked nibble (0x64086408 for the low nibbles of both halves,
// 0x64806480 for the high ones).  The XOR commutes with the shift by 8, so the fields of
// w >> 8 use the same constants.  With the masks in scalar registers (kernel arguments:
// a VOP3 instruction takes no literal constant on this target) each field is one
// v_bitop3_b32, five VALU instructions per word, all visible to the compiler, which
// therefore places the wait states an MFMA still reading its operands requires.
// ---------------------------------------------------------------------------
struct Q4x2 { half2_t p04, p15, p26, p37; };

struct DecodeMasks { uint32_t lo, hi; };        // 0x000F000F and 0x00F000F0, from the host
constexpr uint32_t kDecodeMaskLo = 0x000F000Fu;
constexpr uint32_t kDecodeMaskHi = 0x00F000F0u;

__device__ __forceinline__ Q4x2 decode_int4x8_biased(uint32_t w, DecodeMasks dm) {
    const uint32_t t = w >> 8;
    const uint32_t k_lo = 0x64086408u, k_hi = 0x64806480u;
    Q4x2 q;
    q.p04 = __builtin_bit_cast(half2_t, k_lo ^ (w & dm.lo));
    q.p15 = __builtin_bit_cast(half2_t, k_hi ^ (w & dm.hi));
    q.p26 = __builtin_bit_cast(half2_t, k_lo ^ (t & dm.lo));
    q.p37 = __builtin_bit_cast(half2_t, k_hi ^ (t & dm.hi));
    return q;
}

// The same pairs as exact integer weights q (offsets removed: v - 1032 at even
// positions, v / 16 - 72 at odd ones; every step is exact in fp16).
__device__ __forceinline__ Q4x2 decode_int4x8(uint32_t w, DecodeMasks dm) {
    Q4x2 q = decode_int4x8_biased(w, dm);
    const half2_t off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    q.p04 = q.p04 + off_lo;
    q.p15 = q.p15 * sixteenth + off_hi;   // b / 16 is an integer in [64, 79]
    q.p26 = q.p26 + off_lo;
    q.p37 = q.p37 * sixteenth + off_hi;
    return q;
}

// Workgroups are dispatched to the eight XCDs round-robin (workgroup b runs on XCD
// b % 8), and each XCD has its own L2.  Renumbering b so that the workgroups of one XCD
// get consecutive logical indices (XCD x takes a contiguous range) makes neighbouring
// tiles, which share cache lines of the scales and of the activation, meet in one L2
// instead of being fetched from HBM once per XCD.  A bijection on [0, n) for any n.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int x = b % kXcds, q = n / kXcds, r = n % kXcds;
    return x * q + min(x, r) + b / kXcds;
}

// 16-byte loads and stores marked non-temporal (streamed data that is not re-read).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void nt_store(uint4 v, uint4* p) {
    const u32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

// Two fp32 values to one packed fp16 pair, rounding toward zero (one instruction).
__device__ __forceinline__ half2_t pk_f16_rtz(float a, float b) {
    return __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// ---------------------------------------------------------------------------
// FP4 weights: E2M1 codes (bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa)
// with E4M3 block scales.
// ---------------------------------------------------------------------------
// E4M3 ('fn': no infinities) byte -> fp32 from its fields: sign bit 7, exponent bits
// 6..3 (bias 7), mantissa bits 2..0; exponent 0 is subnormal m * 2^-9; S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
    float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;
    v = (e == 15u && m == 7u) ? __builtin_nanf("") : v;
    return (b & 0x80u) ? -v : v;
}

// The two E2M1 codes of byte B of w (the lower-k code in the low nibble) as exact fp16
// values: (w[k = 2B], w[k = 2B + 1]).  gfx950's v_cvt_scalef32_pk_f16_fp4 applies only
// the exponent of its fp32 scale operand (the power-of-two scales of the MX formats), so
// it runs with scale 1 and E4M3 block scales are applied separately.
template <int B>
__device__ __forceinline__ half2_t fp4x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B);
}

// The eight weights of one packed word, in k order.
__device__ __forceinline__ void fp4x8(uint32_t w, half2_t* q) {
    q[0] = fp4x2<0>(w);
    q[1] = fp4x2<1>(w);
    q[2] = fp4x2<2>(w);
    q[3] = fp4x2<3>(w);
}

// ---------------------------------------------------------------------------
// FP4 activations (the scaled matmul with both operands FP4): a block of 16 values along
// K is quantised with the per-tensor scale G, every step an fp32 operation rounding to
// nearest with ties to even:
//     s = e4m3(amax / (6 G)),   q_k = e2m1(x_k / (s G))   (q_k = 0 where s = 0),
// and the exact values q_k s are what the dot products use: an E2M1 value has 2
// significant bits and an E4M3 value 4, so q s is an fp16 number (2^-10 <= |q s| <= 2688).
// ---------------------------------------------------------------------------
// Non-negative fp32 -> E4M3 code: the nearest E4M3 value, ties to the even code, 448
// (code 126) for everything above it.
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
    if (!(t > 0.0f)) return 0u;
    if (t >= 448.0f) return 126u;
    if (t < 0.015625f) return uint32_t(__builtin_rintf(t * 512.0f));   // steps of 2^-9; code 8 is 2^-6
    const uint32_t b = __float_as_uint(t);
    const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);                 // 3 mantissa bits, ties to even
    return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);                 // exponent bias 127 -> 7
}

// fp32 -> E2M1 code: the magnitude to the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (a
// midpoint goes to the even code), 6 for everything above; bit 3 is the sign bit.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
    const float a = fabsf(y);
    const uint32_t c = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                       uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
    return c | ((__float_as_uint(y) >> 28) & 8u);
}

// N (8 or 16) values of one block, given the block's largest magnitude (taken over the
// whole block, which may span two lanes): their codes packed 8 to a word in k order
// (code of value i in bits 4 (i % 8) of word i / 8), and the fp16 pairs q s in k order.
// Returns the block's E4M3 scale code.
template <int N>
__device__ __forceinline__ uint32_t nvfp4_quantize_block(const float (&v)[N], float amax, float G,
                                                         uint32_t (&words)[N / 8], uint32_t (&xq)[N / 2]) {
    const uint32_t sc = e4m3_encode(amax / (6.0f * G));
    const float s = e4m3_to_f32(sc);
    const float d = s * G;
#pragma unroll
    for (int w = 0; w < N / 8; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) word |= (s > 0.0f ? e2m1_encode(v[8 * w + j] / d) : 0u) << (4 * j);
        words[w] = word;
        half2_t q[4];
        fp4x8(word, q);
        const half2_t sh = {(_Float16)s, (_Float16)s};
#pragma unroll
        for (int p = 0; p < 4; ++p) xq[4 * w + p] = __builtin_bit_cast(uint32_t, q[p] * sh);
    }
    return sc;
}

// Position of weight j (0..7) of a word in the pair order above.
__host__ __device__ constexpr int pair_slot(int j) { return 2 * (j & 3) + (j >> 2); }

__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// ---------------------------------------------------------------------------
// wave64 reductions (DPP / permute through the LDS crossbar, no LDS storage)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// DPP lane moves (gfx9 encodings): quad permutations and rotations within a row of 16.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// Sum over the four lanes of each quad; every lane of the quad gets the sum.
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp<kQuadSwap1>(v);
    v += dpp<kQuadSwap2>(v);
    return v;
}

// Maximum over a full wave (all 64 lanes active), returned uniform: DPP within each row
// of 16 lanes, then the four row results read as scalars.
__device__ __forceinline__ float wave_max_uniform(float v) {
    v = fmaxf(v, dpp<kQuadSwap1>(v));
    v = fmaxf(v, dpp<kQuadSwap2>(v));
    v = fmaxf(v, dpp<kRowRor4>(v));
    v = fmaxf(v, dpp<kRowRor8>(v));
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// SiLU in fp32: v / (1 + exp(-v)).  exp overflows to +inf for v < -88, giving -0.
__device__ __forceinline__ float silu_f32(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v));
}

// gfx950 lane swaps (v_permlane32_swap, v_permlane16_swap), both results as floats.
//   swap32(x, y) = {x lanes 0..31 then y lanes 0..31,  x lanes 32..63 then y lanes 32..63};
//   swap16(x, y), in rows of 16 lanes = {x0 y0 x2 y2,  x1 y1 x3 y3}.
// The builtin's two-element result is cast as a whole: with this compiler a cast of one
// element of it on its own read element 0 for both.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2_t swap32(float x, float y) {
    return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                                        __builtin_bit_cast(uint32_t, y), false, false));
}
__device__ __forceinline__ f32x2_t swap16(float x, float y) {
    return __builtin_bit_cast(f32x2_t, __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                                        __builtin_bit_cast(uint32_t, y), false, false));
}

// Sums a, b, c and d over a full wave (all 64 lanes active), four values in one register:
// the half-wave swaps fold lanes 32..63 onto 0..31 for two values each, the row swap folds
// the odd rows onto the even ones, and four DPP steps sum within each row of 16 lanes.
// Every lane of row r then holds the total of {a, c, b, d}[r].
__device__ __forceinline__ float wave_sum4_rows(float a, float b, float c, float d) {
    const f32x2_t x = swap32(a, b), y = swap32(c, d);
    const f32x2_t z = swap16(x[0] + x[1], y[0] + y[1]);   // rows a a b b | c c d d
    float u = z[0] + z[1];                                 // rows a c b d
    u += dpp<kQuadSwap1>(u);
    u += dpp<kQuadSwap2>(u);
    u += dpp<kRowRor4>(u);
    u += dpp<kRowRor8>(u);
    return u;
}

// ---------------------------------------------------------------------------
// Block-scaled fp16 staging of the activation for the matrix-core GEMVs.  A k-block is 8
// consecutive values of one row; the 16 lanes of a DPP row hold the 16 k-blocks of one
// 128-wide group.  The group's largest magnitude mx sets a power of two 2^E that puts it
// in [2^14, 2^15); the values are stored times 2^-E in fp16, rounded toward zero, and 2^E
// is folded back in with the group's weight scale.  Every staging site (the GEMV kernels'
// own, and the norm kernel writing a staged copy of its output) runs these two functions,
// so a pre-staged activation is bit-identical to one staged by the GEMV.
// ---------------------------------------------------------------------------
// The group's power of two from this lane's largest magnitude: *esc = 2^E, returns 2^-E.
// Whole wave active, the 16 lanes of each DPP row one group.
__device__ __forceinline__ float stage_group_scale(float mx, float* esc) {
    // magnitudes order as their bit patterns do, so the group max is an unsigned max
    uint32_t mb = __builtin_bit_cast(uint32_t, mx);
    mb = max(mb, dpp_u32<kQuadSwap1>(mb));
    mb = max(mb, dpp_u32<kQuadSwap2>(mb));
    mb = max(mb, dpp_u32<kRowRor4>(mb));
    mb = max(mb, dpp_u32<kRowRor8>(mb));
    int e = 0;
    (void)__builtin_frexpf(__builtin_bit_cast(float, mb), &e);
    const int E = min(max(e - 15, -126), 127);
    *esc = __builtin_ldexpf(1.0f, E);
    return __builtin_ldexpf(1.0f, -E);
}

// The offset terms of a staged 128-wide group for the int4 matrix-core kernels: a lane
// holds one staged k-block (pair order, odd positions / 16) and the 16 lanes of its DPP
// row the group's 16 k-blocks.  Returns, in every lane of the row, the sum over the group
// of -1032 * (even slot) - 1152 * (odd slot): what the MFMA of the constant offset matrix
// with these values gives in every column, so a product chain can start from it instead.
__device__ __forceinline__ float staged_offset_sum16(uint4 h) {
    const half2_t ne = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t no = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    float b = dot2(__builtin_bit_cast(half2_t, h.x), ne, 0.f);
    b = dot2(__builtin_bit_cast(half2_t, h.z), ne, b);
    b = dot2(__builtin_bit_cast(half2_t, h.y), no, b);
    b = dot2(__builtin_bit_cast(half2_t, h.w), no, b);
    b += dpp<kQuadSwap1>(b);
    b += dpp<kQuadSwap2>(b);
    b += dpp<kRowRor4>(b);
    b += dpp<kRowRor8>(b);
    return b;
}

// One k-block staged for the int4 kernels: pair order (k0, k4), (k1, k5), (k2, k6),
// (k3, k7), the odd positions also divided by 16, matching decode_int4x8_biased.
__device__ __forceinline__ uint4 stage_pair_order(const float (&v)[8], float down) {
    const float down16 = down * 0.0625f;
    return make_uint4(__builtin_bit_cast(uint32_t, pk_f16_rtz(v[0] * down, v[4] * down)),
                      __builtin_bit_cast(uint32_t, pk_f16_rtz(v[1] * down16, v[5] * down16)),
                      __builtin_bit_cast(uint32_t, pk_f16_rtz(v[2] * down, v[6] * down)),
                      __builtin_bit_cast(uint32_t, pk_f16_rtz(v[3] * down16, v[7] * down16)));
}

// A k-block of 8 bf16 values (one 16-byte word) staged for the int4 kernels.
__device__ __forceinline__ uint4 stage_bf16_kblock(uint4 w, float* esc) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
    float v[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        v[2 * h] = bf16_lo(a[h]);
        v[2 * h + 1] = bf16_hi(a[h]);
    }
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[j]));
    return stage_pair_order(v, stage_group_scale(mx, esc));
}

}  // namespace fdec
