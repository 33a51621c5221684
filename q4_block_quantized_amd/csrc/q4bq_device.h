// Device-side helpers shared by the q4bq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4bq_internal.h"

namespace q4bq {

// Internal activation block ("dot order"), written by the activation
// quantizer and read by both product kernels:
//   8 dwords of int8 -- dword t, byte i holds element 8*(t/2) + (t%2) + 2*i,
//   i.e. dword 2k = elements 8k+{0,2,4,6}, dword 2k+1 = elements 8k+{1,3,5,7}.
//   This is the order in which one 32-bit word of Q4_0 nibbles splits into
//   its low nibbles (even elements) and high nibbles (odd elements), so a
//   weight word needs only a mask and a shift before v_dot4.
// plus one 8-byte scale record {float d; int32 bias}, bias = -8 * sum(q).
struct ActScale {
    float d;
    int32_t bias;
};
static_assert(sizeof(ActScale) == kActSBytes, "scale record is 8 bytes");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// fp32 -> binary16 bits, round to nearest even (the hardware conversion in
// the default rounding mode; binary16 subnormals are kept).
__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Largest value over the 32 lanes of an aligned half-wave.
__device__ __forceinline__ float max32(float v) {
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 32));
    return v;
}

__device__ __forceinline__ int sum32(int v) {
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) v += __shfl_xor(v, m, 32);
    return v;
}

__device__ __forceinline__ uint32_t or_lanes(uint32_t v, int m) {
    return v | static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m, 32));
}

// Cross-lane steps inside aligned groups of 8 lanes on the vector ALU (DPP,
// no LDS round trip): lane i reads lane i ^ 1 or i ^ 2 (quad permutations), or
// lane 7 - i of its group (half-row mirror).  After the two quad steps every
// quad holds its own reduction, so the mirror step completes a reduction over
// the 8 lanes.  The whole group must be active.
constexpr int kDppXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppMirror8 = 0x141;  // row_half_mirror
template <int kCtrl>
__device__ __forceinline__ int dpp8_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp8_f(float v) {
    return __builtin_bit_cast(float, dpp8_i<kCtrl>(__builtin_bit_cast(int, v)));
}

// Q8_0 activation rule on four consecutive values of a block: lane m of an
// aligned group of 8 lanes holds elements 4m..4m+3 of the same block.
//   d = binary16(amax / 127) (widened back to fp32), q = round(x / d) half
//   away from zero, clamped to [-127, 127]; q = 0 when d == 0.
// Returns the block's scale record and writes this lane's dword of the block
// in dot order: the lane pair (2k, 2k+1) covers elements 8k..8k+7; lane 2k
// keeps the even ones (8k, 8k+2, 8k+4, 8k+6) and lane 2k+1 the odd ones, so
// lane m owns dword m.
__device__ __forceinline__ int8_t q8_rule(float x, float d) {
    if (d == 0.0f) return 0;
    const int q = static_cast<int>(__builtin_roundf(x / d));
    return static_cast<int8_t>(min(max(q, -127), 127));
}

// The same codes for four values sharing d, with one reciprocal instead of a
// correctly rounded division per value.  r = 1/d from the hardware
// reciprocal refined by one Newton step has a relative error of about 2^-24,
// so y = x r is within 2^-15 of x/d, and the rounded quotient fl(x/d) within
// 2^-17 of it, as long as |x/d| < 256 (d is amax/127 rounded to binary16:
// about amax/127 in the normal range, at least two thirds of it among the
// subnormals, so |x/d| <= 190.5).  When y lies farther than 2^-13 from every half-integer, y and
// fl(x/d) therefore fall strictly inside the same rounding interval, so
// round(fl(x/d)) (half away from zero) is trunc(y + copysign(1/2, y)): that
// sum stays 2^-13 clear of the integers, more than its rounding error.  A
// wave in which any value comes that close takes the division for its four
// values instead, so the codes equal q8_rule's for every input.
__device__ __forceinline__ void q8_rule4(float x0, float x1, float x2, float x3, float d, int8_t q[4]) {
    const bool zero = d == 0.0f;
    const float dd = zero ? 1.0f : d;
    float r = __builtin_amdgcn_rcpf(dd);
    r = fmaf(fmaf(-dd, r, 1.0f), r, r);
    const float x[4] = {x0, x1, x2, x3};
    int k[4];
    bool close = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float y = x[i] * r;
        close |= fabsf(__builtin_amdgcn_fractf(y) - 0.5f) <= 0x1p-13f;
        k[i] = static_cast<int>(fminf(fmaxf(y + copysignf(0.5f, y), -127.0f), 127.0f));
    }
    if (__builtin_amdgcn_ballot_w64(close) != 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = q8_rule(x[i], d);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = static_cast<int8_t>(zero ? 0 : k[i]);
}

// Four int8 values of lane m (elements 4m..4m+3) -> this lane's dot-order
// dword, and the block's -8 * sum(q) (both over the 8-lane group).
__device__ __forceinline__ uint32_t dot_order_word(int8_t q0, int8_t q1, int8_t q2, int8_t q3, int m, int& bias) {
    const uint32_t ev = static_cast<uint8_t>(q0) | (static_cast<uint32_t>(static_cast<uint8_t>(q2)) << 8);
    const uint32_t od = static_cast<uint8_t>(q1) | (static_cast<uint32_t>(static_cast<uint8_t>(q3)) << 8);
    const uint32_t mine = ev | (od << 16);
    const uint32_t other = static_cast<uint32_t>(dpp8_i<kDppXor1>(static_cast<int>(mine)));
    int sum = static_cast<int>(q0) + q1 + q2 + q3;
    sum += dpp8_i<kDppXor1>(sum);
    sum += dpp8_i<kDppXor2>(sum);
    sum += dpp8_i<kDppMirror8>(sum);
    bias = -8 * sum;
    return (m & 1) ? ((other >> 16) | (od << 16)) : (ev | (other << 16));
}

// The Q8_0 rule for one block held by an aligned group of 8 lanes (lane m:
// elements 4m..4m+3; the whole group active): the block's binary16 scale
// (bits and value) and this lane's four codes.  amax is taken over the
// group with integer maxima (non-negative floats order as their bit
// patterns).
__device__ __forceinline__ float q8_block_quad(float x0, float x1, float x2, float x3, uint32_t& dbits,
                                               int8_t q[4]) {
    const float a4 = fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3)));
    uint32_t ab = __builtin_bit_cast(uint32_t, a4);
    ab = max(ab, static_cast<uint32_t>(dpp8_i<kDppXor1>(static_cast<int>(ab))));
    ab = max(ab, static_cast<uint32_t>(dpp8_i<kDppXor2>(static_cast<int>(ab))));
    ab = max(ab, static_cast<uint32_t>(dpp8_i<kDppMirror8>(static_cast<int>(ab))));
    dbits = float_to_half_bits(__builtin_bit_cast(float, ab) / 127.0f);
    const float d = half_bits_to_float(dbits);
    q8_rule4(x0, x1, x2, x3, d, q);
    return d;
}

// The same codes as one dword in element order (byte i: element 4m + i).
__device__ __forceinline__ uint32_t q8_natural_word(const int8_t q[4]) {
    return static_cast<uint32_t>(static_cast<uint8_t>(q[0])) | (static_cast<uint32_t>(static_cast<uint8_t>(q[1])) << 8) |
           (static_cast<uint32_t>(static_cast<uint8_t>(q[2])) << 16) |
           (static_cast<uint32_t>(static_cast<uint8_t>(q[3])) << 24);
}

__device__ __forceinline__ ActScale quant_act_quad(float x0, float x1, float x2, float x3, int m, uint32_t& word,
                                                   uint32_t& dbits) {
    int8_t q[4];
    const float d = q8_block_quad(x0, x1, x2, x3, dbits, q);
    int bias;
    word = dot_order_word(q[0], q[1], q[2], q[3], m, bias);
    return ActScale{d, bias};
}

__device__ __forceinline__ ActScale quant_act_quad(float x0, float x1, float x2, float x3, int m, uint32_t& word) {
    uint32_t dbits;
    return quant_act_quad(x0, x1, x2, x3, m, word, dbits);
}

// One 32-bit word of Q4_0 nibbles (bytes 4k..4k+3 of qs, elements 8k..8k+7)
// split into the even elements (low nibbles) and odd elements (high nibbles),
// each as four unsigned bytes 0..15.
__device__ __forceinline__ uint32_t nib_lo(uint32_t w) { return w & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t w) { return (w >> 4) & 0x0F0F0F0Fu; }

// ---------------------------------------------------------------------------
// fp6 (e2m3) operand codes for the prefill kernel.
//
// The block dot s = sum_j (nibble_j - 8) * q_j is evaluated exactly on the
// fp6 matrix cores: with y = 16h + l (h = y >> 4 in [-8, 7], l = y & 15),
//   s = sum_j [(nibble_j - 8)/8 * 8] * ([h_j/2 * 32] + [l_j/2 * 2]),
// where (nibble - 8)/8, h/2 and l/2 are all exact e2m3 values and the powers
// of two are the operands' E8M0 block scales.  Every product and partial sum
// is an integer below 2^24, so the fp32 result equals the int32 dot.
//
// e2m3: sign bit, 2 exponent bits (bias 1), 3 mantissa bits.  Codes of k/2:
//   k = 0..8  -> 00 04 08 0C 10 12 14 16 18,  k = 9..15 -> 19 1A 1B 1C 1D 1E 1F.
// The byte-wise selects below pick, per byte, table entry `idx` from one of
// two 8-entry tables according to bit 3 of the source nibble (v_perm_b32
// with selector i or i + 4).
// ---------------------------------------------------------------------------

// Four bytes n (0..15) -> e2m3 codes of (n - 8) / 2, one per byte.
__device__ __forceinline__ uint32_t e2m3_half_offset(uint32_t n) {
    const uint32_t idx = n & 0x07070707u;
    // n = 0..7: -8/2 .. -1/2 (sign bit set); n = 8..15: 0 .. 7/2
    const uint32_t neg = __builtin_amdgcn_perm(0x24282C30u, 0x32343638u, idx);
    const uint32_t pos = __builtin_amdgcn_perm(0x16141210u, 0x0C080400u, idx);
    return __builtin_amdgcn_perm(pos, neg, ((n >> 1) & 0x04040404u) | 0x03020100u);
}

// Four bytes l (0..15) -> e2m3 codes of l / 2.
__device__ __forceinline__ uint32_t e2m3_half(uint32_t l) {
    const uint32_t idx = l & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(0x16141210u, 0x0C080400u, idx);
    const uint32_t hi = __builtin_amdgcn_perm(0x1F1E1D1Cu, 0x1B1A1918u, idx);
    return __builtin_amdgcn_perm(hi, lo, ((l >> 1) & 0x04040404u) | 0x03020100u);
}

// Four 6-bit codes (one per byte) -> 24 bits, code i at bits 6i..6i+5.
__device__ __forceinline__ uint32_t pack4x6(uint32_t c) {
    const uint32_t t = (c & 0x003F003Fu) | ((c >> 2) & 0x0FC00FC0u);
    return (t & 0xFFFu) | ((t >> 4) & ~0xFFFu);  // t bits 28..31 are zero
}

// Eight 24-bit chunks -> the six dwords of a 32-value fp6 operand.
__device__ __forceinline__ void assemble6(const uint32_t P[8], uint32_t d[6]) {
    d[0] = P[0] | (P[1] << 24);
    d[1] = (P[1] >> 8) | (P[2] << 16);
    d[2] = (P[2] >> 16) | (P[3] << 8);
    d[3] = P[4] | (P[5] << 24);
    d[4] = (P[5] >> 8) | (P[6] << 16);
    d[5] = (P[6] >> 16) | (P[7] << 8);
}

// Four nibble bytes n -> e2m3 codes of (n - 8) / 8, given idx = n & 7 in each
// byte and sel4 = 4 in the bytes where n >= 8.  Below 1.0 the e2m3 codes are
// linear (value code/8), and 1.0 = code 8, so k/8 for |k| <= 8 has the code
// |k| plus the sign bit 0x20: n >= 8 gives k = idx, n < 8 gives
// 0x20 | (8 - n) = 0x28 - idx (an 8-entry byte table).
__device__ __forceinline__ uint32_t e2m3_eighth_offset(uint32_t idx, uint32_t sel4) {
    const uint32_t neg = __builtin_amdgcn_perm(0x21222324u, 0x25262728u, idx);
    return __builtin_amdgcn_perm(idx, neg, sel4 | 0x03020100u);
}

// A Q4_0 block's nibbles -> fp6 operand of (nibble - 8)/8 in dot order: chunk
// 2k holds the even elements of nibble word k, chunk 2k+1 the odd ones (the
// same element order as the activation records).
__device__ __forceinline__ void weight_fp6(const uint32_t qs[4], uint32_t d[6]) {
    uint32_t P[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t q = qs[k];
        P[2 * k] = pack4x6(e2m3_eighth_offset(q & 0x07070707u, (q >> 1) & 0x04040404u));
        P[2 * k + 1] = pack4x6(e2m3_eighth_offset((q >> 4) & 0x07070707u, (q >> 5) & 0x04040404u));
    }
    assemble6(P, d);
}

// Prefill activation record of one block, written by its 8-lane group (lane m
// holds dot-order dword m, i.e. chunk m, of int8 values): 64 bytes per
// (token, block), stored block-major at record index o = block * N + token.
// Dwords 0..5: fp6 operand of h/2; dword 6: the block's binary16 scale bits;
// dword 7: zero; dwords 8..15: the same for l/2.
constexpr int kAct6Bytes = 64;

__device__ __forceinline__ void store_act6(int m, uint32_t word, uint32_t dbits, bool valid, int64_t o,
                                           uint32_t* __restrict__ rec) {
    const uint32_t ph = pack4x6(e2m3_half_offset(((word >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u));  // h + 8
    const uint32_t pl = pack4x6(e2m3_half(word & 0x0F0F0F0Fu));                                 // l
    // output dword d (lanes 0..5) = chunk c1 shifted down | chunk c1+1 shifted up
    const int d = m < 6 ? m : 0;
    const int c1 = d + d / 3;
    const int s1 = 32 * d - 24 * c1;
    const int s2 = 24 * (c1 + 1) - 32 * d;
    const uint32_t h1 = static_cast<uint32_t>(__shfl(static_cast<int>(ph), c1, 8));
    const uint32_t h2 = static_cast<uint32_t>(__shfl(static_cast<int>(ph), c1 + 1, 8));
    const uint32_t l1 = static_cast<uint32_t>(__shfl(static_cast<int>(pl), c1, 8));
    const uint32_t l2 = static_cast<uint32_t>(__shfl(static_cast<int>(pl), c1 + 1, 8));
    if (valid) {
        const uint32_t tail = m == 6 ? (dbits & 0xFFFFu) : 0u;
        rec[o * 16 + m] = m < 6 ? (h1 >> s1) | (h2 << s2) : tail;
        rec[o * 16 + 8 + m] = m < 6 ? (l1 >> s1) | (l2 << s2) : tail;
    }
}

// 36 bytes starting at p (two consecutive Q4_0 blocks), any 2-byte alignment:
// gfx950 serves unaligned global loads, so this is three plain loads.
struct Pair36 {
    uint32_t w[9];
};

__device__ __forceinline__ Pair36 load_pair(const uint8_t* p) {
    Pair36 r;
    u32x4 a, b;
    uint32_t c;
    __builtin_memcpy(&a, p, 16);
    __builtin_memcpy(&b, p + 16, 16);
    __builtin_memcpy(&c, p + 32, 4);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
    r.w[8] = c;
    return r;
}

// Decoded view of a Q4_0 block: scale bits and the four words of nibbles.
struct Block4 {
    uint32_t dbits;
    uint32_t qs[4];
};

// First block of a pair: d = bytes 0-1, nibbles = bytes 2-17.
__device__ __forceinline__ Block4 pair_first(const Pair36& p) {
    Block4 b;
    b.dbits = p.w[0] & 0xFFFFu;
#pragma unroll
    for (int k = 0; k < 4; ++k) b.qs[k] = __builtin_amdgcn_alignbit(p.w[k + 1], p.w[k], 16);
    return b;
}

// Second block of a pair: d = bytes 18-19, nibbles = bytes 20-35.
__device__ __forceinline__ Block4 pair_second(const Pair36& p) {
    Block4 b;
    b.dbits = p.w[4] >> 16;
#pragma unroll
    for (int k = 0; k < 4; ++k) b.qs[k] = p.w[5 + k];
    return b;
}

// A single block at p (18 bytes, 2-byte aligned).
__device__ __forceinline__ Block4 load_block(const uint8_t* p) {
    Block4 b;
    uint16_t d;
    u32x4 q;
    __builtin_memcpy(&d, p, 2);
    __builtin_memcpy(&q, p + 2, 16);
    b.dbits = d;
    b.qs[0] = q.x; b.qs[1] = q.y; b.qs[2] = q.z; b.qs[3] = q.w;
    return b;
}

// Repacked weights (q4_0_repack): a nibble stream of 16 bytes per block, then a
// stream of the binary16 scales, both in (row, block) order.  Two consecutive
// blocks: 32 aligned nibble bytes and 4 scale bytes, kept in the same nine
// dwords as a raw pair (nibbles of the first block in w[0..3], of the second
// in w[4..7], both scales in w[8]).
__device__ __forceinline__ Pair36 load_pair_rp(const uint8_t* nib, const uint8_t* sc) {
    Pair36 r;
    u32x4 a, b;
    uint32_t c;
    __builtin_memcpy(&a, nib, 16);
    __builtin_memcpy(&b, nib + 16, 16);
    __builtin_memcpy(&c, sc, 4);
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
    r.w[4] = b.x; r.w[5] = b.y; r.w[6] = b.z; r.w[7] = b.w;
    r.w[8] = c;
    return r;
}

__device__ __forceinline__ Block4 pair_first_rp(const Pair36& p) {
    Block4 b;
    b.dbits = p.w[8] & 0xFFFFu;
#pragma unroll
    for (int k = 0; k < 4; ++k) b.qs[k] = p.w[k];
    return b;
}

__device__ __forceinline__ Block4 pair_second_rp(const Pair36& p) {
    Block4 b;
    b.dbits = p.w[8] >> 16;
#pragma unroll
    for (int k = 0; k < 4; ++k) b.qs[k] = p.w[4 + k];
    return b;
}

__device__ __forceinline__ Block4 load_block_rp(const uint8_t* nib, const uint8_t* sc) {
    Block4 b;
    uint16_t d;
    u32x4 q;
    __builtin_memcpy(&d, sc, 2);
    __builtin_memcpy(&q, nib, 16);
    b.dbits = d;
    b.qs[0] = q.x; b.qs[1] = q.y; b.qs[2] = q.z; b.qs[3] = q.w;
    return b;
}

// The block's integer dot with one activation block in dot order:
//   s = sum_j (nibble_j - 8) * q_j = sum_j nibble_j * q_j + bias,
// bias = -8 * sum_j q_j.  Nibbles 0..15 are valid positive int8, so the signed
// 4-way byte dot applies directly; every partial sum is exact in int32.
__device__ __forceinline__ int32_t block_dot(const Block4& w, const uint32_t* a, int32_t bias) {
    int32_t s = bias;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        s = __builtin_amdgcn_sdot4(static_cast<int>(nib_lo(w.qs[k])), static_cast<int>(a[2 * k]), s, false);
        s = __builtin_amdgcn_sdot4(static_cast<int>(nib_hi(w.qs[k])), static_cast<int>(a[2 * k + 1]), s, false);
    }
    return s;
}

// The epilogue of a product output y for token n, row r (rows per token:
// rows): y + bias[r], then GELU (GPT-2's tanh form) or SiLU (x * sigmoid(x)),
// then times mul[n][r].
// ---------------------------------------------------------------------------
// LayerNorm before the product (the ggml GPT-2 walkthrough, section 3.1:
// gamma * (x - mu) / sqrt(sigma^2 + eps) + beta over each token's K values).
// The statistics are taken in fp64 and the normalized value is evaluated in
// fp64 and rounded once to fp32: the fp32 value that decides the Q8_0 codes
// then does not depend on the summation order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ln_value(float x, double mu, double rstd, float g, float b) {
#pragma clang fp contract(off)
    return static_cast<float>(static_cast<double>(g) * ((static_cast<double>(x) - mu) * rstd) +
                              static_cast<double>(b));
}

// Sum of one fp64 value per thread over a workgroup of THREADS threads; red:
// THREADS / 64 doubles of LDS.  Every thread of the workgroup calls it (one
// workgroup barrier) and gets the total, added in wave order.  A later call
// must use other LDS (or come after another barrier): slow waves may still be
// reading red.
// One DPP move of an fp64 value (both 32-bit halves); lanes outside kRowMask
// read 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), kCtrl, kRowMask, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(u >> 32), kCtrl, kRowMask, 0xF, false));
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Sum over the 64 lanes of a wave, returned in every lane: DPP adds inside
// rows of 16 lanes, two row broadcasts into lane 63, then lane 63's value.
__device__ __forceinline__ double wave_total_f64(double v) {
    v += dpp_f64<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v += dpp_f64<0x141, 0xF>(v);  // row_half_mirror
    v += dpp_f64<0x140, 0xF>(v);  // row_mirror: each row of 16 holds its sum
    v += dpp_f64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_f64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(u), 63);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(u >> 32), 63);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

template <int THREADS>
__device__ __forceinline__ double wg_sum_f64(double v, double* red) {
    v = wave_total_f64(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < THREADS / 64; ++i) t += red[i];
    return t;
}

__device__ __forceinline__ double quad_sum_f64(float4 v) {
    return (static_cast<double>(v.x) + static_cast<double>(v.y)) + (static_cast<double>(v.z) + static_cast<double>(v.w));
}
__device__ __forceinline__ double quad_sqdev_f64(float4 v, double mu) {
    const double a = static_cast<double>(v.x) - mu, b = static_cast<double>(v.y) - mu;
    const double c = static_cast<double>(v.z) - mu, d = static_cast<double>(v.w) - mu;
    return (a * a + b * b) + (c * c + d * d);
}
__device__ __forceinline__ float4 ln_quad(float4 v, double mu, double rstd, float4 g, float4 b) {
    return make_float4(ln_value(v.x, mu, rstd, g.x, b.x), ln_value(v.y, mu, rstd, g.y, b.y),
                       ln_value(v.z, mu, rstd, g.z, b.z), ln_value(v.w, mu, rstd, g.w, b.w));
}

// The epilogue with its operands already loaded: b = bias[r], m = mul[n][r]
// (either ignored when its pointer is null), so that a kernel can fetch them
// with the row's weights instead of at the store.
__device__ __forceinline__ float epilogue_with(float y, float b, float m, const Epilogue& e) {
    if (e.bias) y += b;
    if (e.act == kEpiGelu) {
        y = 0.5f * y * (1.0f + tanhf(0.7978845608028654f * (y + 0.044715f * y * y * y)));
    } else if (e.act == kEpiSilu) {
        y = y / (1.0f + expf(-y));
    }
    if (e.mul) y *= m;
    return y;
}
__device__ __forceinline__ float epi_bias(const Epilogue& e, int64_t r) { return e.bias ? e.bias[r] : 0.0f; }
__device__ __forceinline__ float epi_mul(const Epilogue& e, int64_t n, int64_t r, int64_t rows) {
    return e.mul ? e.mul[n * rows + r] : 1.0f;
}

__device__ __forceinline__ float apply_epilogue(float y, int64_t n, int64_t r, int64_t rows, const Epilogue& e) {
    return epilogue_with(y, epi_bias(e, r), epi_mul(e, n, r, rows), e);
}

}  // namespace q4bq
