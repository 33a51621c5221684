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

__device__ __forceinline__ ActScale quant_act_quad(float x0, float x1, float x2, float x3, int m, uint32_t& word) {
    float a = fmaxf(fmaxf(fabsf(x0), fabsf(x1)), fmaxf(fabsf(x2), fabsf(x3)));
    a = fmaxf(a, __shfl_xor(a, 1, 8));
    a = fmaxf(a, __shfl_xor(a, 2, 8));
    a = fmaxf(a, __shfl_xor(a, 4, 8));
    const uint32_t dbits = float_to_half_bits(a / 127.0f);
    const float d = half_bits_to_float(dbits);
    const int8_t q0 = q8_rule(x0, d), q1 = q8_rule(x1, d), q2 = q8_rule(x2, d), q3 = q8_rule(x3, d);
    const uint32_t ev = static_cast<uint8_t>(q0) | (static_cast<uint32_t>(static_cast<uint8_t>(q2)) << 8);
    const uint32_t od = static_cast<uint8_t>(q1) | (static_cast<uint32_t>(static_cast<uint8_t>(q3)) << 8);
    const uint32_t mine = ev | (od << 16);
    const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(mine), 1, 8));
    word = (m & 1) ? ((other >> 16) | (od << 16)) : (ev | (other << 16));
    int sum = static_cast<int>(q0) + q1 + q2 + q3;
    sum += __shfl_xor(sum, 1, 8);
    sum += __shfl_xor(sum, 2, 8);
    sum += __shfl_xor(sum, 4, 8);
    return ActScale{d, -8 * sum};
}

// One 32-bit word of Q4_0 nibbles (bytes 4k..4k+3 of qs, elements 8k..8k+7)
// split into the even elements (low nibbles) and odd elements (high nibbles),
// each as four unsigned bytes 0..15.
__device__ __forceinline__ uint32_t nib_lo(uint32_t w) { return w & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t w) { return (w >> 4) & 0x0F0F0F0Fu; }

// Four unsigned nibble bytes (0..15) -> four signed bytes (nibble - 8).
// Adding 0x78 to a byte <= 0x0F cannot carry into the next byte; flipping the
// top bit then maps 0x78..0x87 to -8..7.
__device__ __forceinline__ uint32_t nib_to_s8(uint32_t v) {
    return (v + 0x78787878u) ^ 0x80808080u;
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

}  // namespace q4bq
