// Block quantizers.
//
// Q4_0 encode follows "llama.cpp 深度解读" (luoboask.github.io) section 2
// "量化数据结构 — Q4_0 格式详解": per 32 weights take the largest magnitude, the
// scale is that over 8, each weight becomes round(w / scale) + 8 and two 4-bit
// values share a byte (even element low).  The scale is stored as binary16 and
// the division uses the stored value; round() is half away from zero; values
// are clamped to the nibble range [0, 15]; an all-zero block stores d = 0 and
// nibble 8.  The Q8_0 activation rule is the same with 127 levels and a
// symmetric clamp to [-127, 127].
//
// One half-wave (32 lanes) owns one block: lane e holds element e, the
// largest magnitude is a 5-step butterfly, and lanes OR their small fields
// together before a few 16/32-bit stores.
#include "q4bq_device.h"
#include "q4bq_internal.h"

namespace q4bq {

namespace {

constexpr int kThreads = 256;  // 4 waves = 8 blocks per workgroup iteration

__device__ __forceinline__ int quant4(float w, float d) {
    if (d == 0.0f) return 8;
    int q = static_cast<int>(__builtin_roundf(w / d)) + 8;
    return min(max(q, 0), 15);
}

__device__ __forceinline__ int quant8(float x, float d) {
    if (d == 0.0f) return 0;
    int q = static_cast<int>(__builtin_roundf(x / d));
    return min(max(q, -127), 127);
}

__global__ void __launch_bounds__(kThreads)
k_q4_0_quantize(const float* __restrict__ W, int64_t nblocks, uint8_t* __restrict__ Wq) {
    const int e = threadIdx.x & 31;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 5;
    const int64_t step = static_cast<int64_t>(gridDim.x) * (kThreads / 32);
    // The trip count is uniform over the wave: both halves iterate together.
    const int64_t wave_first = first & ~static_cast<int64_t>(1);
    for (int64_t g0 = wave_first; g0 < nblocks; g0 += step) {
        const int64_t g = g0 + (first & 1);
        const bool valid = g < nblocks;
        const float w = valid ? W[g * kQK + e] : 0.0f;
        const float amax = max32(fabsf(w));
        const uint32_t dbits = float_to_half_bits(amax / 8.0f);
        const float d = half_bits_to_float(dbits);
        const uint32_t q = static_cast<uint32_t>(quant4(w, d));
        // 16-bit word j of the nibble bytes holds elements 4j..4j+3.
        uint32_t v = q << (4 * (e & 3));
        v = or_lanes(v, 1);
        v = or_lanes(v, 2);
        if (valid) {
            uint16_t* out = reinterpret_cast<uint16_t*>(Wq + g * kQ4Bytes);
            if ((e & 3) == 0) out[1 + (e >> 2)] = static_cast<uint16_t>(v);
            if (e == 0) out[0] = static_cast<uint16_t>(dbits);
        }
    }
}

__global__ void __launch_bounds__(kThreads)
k_q8_0_quantize(const float* __restrict__ X, int64_t nblocks, uint8_t* __restrict__ Xq) {
    const int e = threadIdx.x & 31;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 5;
    const int64_t step = static_cast<int64_t>(gridDim.x) * (kThreads / 32);
    const int64_t wave_first = first & ~static_cast<int64_t>(1);
    for (int64_t g0 = wave_first; g0 < nblocks; g0 += step) {
        const int64_t g = g0 + (first & 1);
        const bool valid = g < nblocks;
        const float x = valid ? X[g * kQK + e] : 0.0f;
        const float amax = max32(fabsf(x));
        const uint32_t dbits = float_to_half_bits(amax / 127.0f);
        const float d = half_bits_to_float(dbits);
        const uint32_t q = static_cast<uint32_t>(quant8(x, d)) & 0xFFu;
        uint32_t v = q << (8 * (e & 1));
        v = or_lanes(v, 1);
        if (valid) {
            uint16_t* out = reinterpret_cast<uint16_t*>(Xq + g * kQ8Bytes);
            if ((e & 1) == 0) out[1 + (e >> 1)] = static_cast<uint16_t>(v);
            if (e == 0) out[0] = static_cast<uint16_t>(dbits);
        }
    }
}

// One workgroup per token: the statistics (fp64, two passes), then the token's
// blocks normalized and quantized, into the decode layout (token-major blocks
// g = n nb + b, PREFILL false) or the prefill records (o = b N + n).  Thread t
// holds quads t, t + T, ... (QPT of them, four values each, loaded in one
// round); T is a multiple of 8, so the 8 lanes of a block are neighbours, as
// the quantizer wants.  QPT = 0: rows too long for registers, re-read per pass.

template <bool PREFILL, int QPT>
__global__ void __launch_bounds__(kLnActThreads)
k_ln_act(const float* __restrict__ X, int64_t N, int64_t nb, const float* __restrict__ gamma,
         const float* __restrict__ beta, float eps, uint32_t* __restrict__ act_q, ActScale* __restrict__ act_s) {
    __shared__ double red[2][kLnActThreads / 64];
    const int64_t n = blockIdx.x;
    const int64_t nq = nb * 8;  // quads of the token
    const float* x = X + n * nb * kQK;
    constexpr int kReg = QPT > 0 ? QPT : 1;
    float4 xr[kReg];
    double s = 0.0;
    if constexpr (QPT > 0) {
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
            const int64_t q = threadIdx.x + static_cast<int64_t>(kLnActThreads) * i;
            xr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (q < nq) __builtin_memcpy(&xr[i], x + 4 * q, 16);
        }
#pragma unroll
        for (int i = 0; i < QPT; ++i)
            s += (static_cast<double>(xr[i].x) + static_cast<double>(xr[i].y)) +
                 (static_cast<double>(xr[i].z) + static_cast<double>(xr[i].w));
    } else {
        for (int64_t q = threadIdx.x; q < nq; q += kLnActThreads) {
            float4 v;
            __builtin_memcpy(&v, x + 4 * q, 16);
            s += (static_cast<double>(v.x) + static_cast<double>(v.y)) + (static_cast<double>(v.z) + static_cast<double>(v.w));
        }
    }
    const double K = static_cast<double>(nb * kQK);
    const double mu = wg_sum_f64<kLnActThreads>(s, red[0]) / K;
    auto sq = [&](const float4& v) __attribute__((always_inline)) {
        const double a = static_cast<double>(v.x) - mu, b = static_cast<double>(v.y) - mu;
        const double c = static_cast<double>(v.z) - mu, d = static_cast<double>(v.w) - mu;
        return (a * a + b * b) + (c * c + d * d);
    };
    double v2 = 0.0;
    if constexpr (QPT > 0) {
#pragma unroll
        for (int i = 0; i < QPT; ++i)
            if (threadIdx.x + static_cast<int64_t>(kLnActThreads) * i < nq) v2 += sq(xr[i]);
    } else {
        for (int64_t q = threadIdx.x; q < nq; q += kLnActThreads) {
            float4 v;
            __builtin_memcpy(&v, x + 4 * q, 16);
            v2 += sq(v);
        }
    }
    const double rstd = 1.0 / sqrt(wg_sum_f64<kLnActThreads>(v2, red[1]) / K + static_cast<double>(eps));
    const int m = threadIdx.x & 7;
    auto emit = [&](float4 v, int64_t q) __attribute__((always_inline)) {
        const int64_t k = 4 * q;
        v.x = ln_value(v.x, mu, rstd, gamma[k], beta[k]);
        v.y = ln_value(v.y, mu, rstd, gamma[k + 1], beta[k + 1]);
        v.z = ln_value(v.z, mu, rstd, gamma[k + 2], beta[k + 2]);
        v.w = ln_value(v.w, mu, rstd, gamma[k + 3], beta[k + 3]);
        uint32_t word, dbits;
        const ActScale sc = quant_act_quad(v.x, v.y, v.z, v.w, m, word, dbits);
        const int64_t b = q >> 3;
        if constexpr (PREFILL) {
            store_act6(m, word, dbits, true, b * N + n, act_q);
        } else {
            act_q[(n * nb + b) * 8 + m] = word;
            if (m == 0) act_s[n * nb + b] = sc;
        }
    };
    // a block's 8 quads sit in 8 neighbouring lanes, all valid or all past the end
    if constexpr (QPT > 0) {
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
            const int64_t q = threadIdx.x + static_cast<int64_t>(kLnActThreads) * i;
            if (q < nq) emit(xr[i], q);
        }
    } else {
        for (int64_t q = threadIdx.x; q < nq; q += kLnActThreads) {
            float4 v;
            __builtin_memcpy(&v, x + 4 * q, 16);
            emit(v, q);
        }
    }
}

// fp32 activations -> internal dot-order blocks: 8 lanes per block, four
// consecutive values per lane (one 16-byte load).
__global__ void __launch_bounds__(kThreads)
k_act_from_f32(const float* __restrict__ X, int64_t nblocks, uint32_t* __restrict__ act_q,
               ActScale* __restrict__ act_s) {
    const int m = threadIdx.x & 7;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 3;
    const int64_t step = static_cast<int64_t>(gridDim.x) * (kThreads / 8);
    // uniform trip count over the wave (8 blocks per wave)
    const int64_t wave_first = first & ~static_cast<int64_t>(7);
    for (int64_t g0 = wave_first; g0 < nblocks; g0 += step) {
        const int64_t g = g0 + (first & 7);
        const bool valid = g < nblocks;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) __builtin_memcpy(&x, X + g * kQK + 4 * m, 16);
        uint32_t word;
        const ActScale sc = quant_act_quad(x.x, x.y, x.z, x.w, m, word);
        if (valid) {
            act_q[g * 8 + m] = word;
            if (m == 0) act_s[g] = sc;
        }
    }
}

// The optional one-time repack, three streams:
//  * 16-byte nibble blocks in (row, block) order (aligned, for plain 16-byte
//    loads in the decode kernels);
//  * the binary16 scales in (row, block) order;
//  * at rec_off, the matrix-core weight records of the prefill kernel, block
//    major ([block][row], 32 bytes: 6 dwords of fp6 codes of (nibble - 8)/8,
//    the scale bits, a zero dword; the two 16-byte halves swapped in rows where
//    bit 2 xor bit 3 is set, the LDS order), followed by one plane of zero records that
//    stands for blocks past the end.
// The bytes between the scale stream and the records are zero.  No value
// changes; the records are the kernel's own conversion, done once.
__global__ void __launch_bounds__(kThreads)
k_q4_0_repack(const uint8_t* __restrict__ Wq, int64_t rows, int64_t nb, int64_t rec_off, uint8_t* __restrict__ Wr) {
    const int64_t nblocks = rows * nb;
    uint16_t* sc = reinterpret_cast<uint16_t*>(Wr + nblocks * 16);
    uint8_t* rec = Wr + rec_off;
    const int64_t pad = rec_off - nblocks * kQ4Bytes;  // zero bytes before the records
    for (int64_t g = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; g < nblocks + rows + pad;
         g += static_cast<int64_t>(gridDim.x) * kThreads) {
        if (g >= nblocks + rows) {
            Wr[nblocks * kQ4Bytes + (g - nblocks - rows)] = 0;
            continue;
        }
        uint32_t d6[6] = {0u, 0u, 0u, 0u, 0u, 0u};
        uint32_t dbits = 0u;
        int64_t r, b;
        if (g < nblocks) {
            const Block4 blk = load_block(Wq + g * kQ4Bytes);
            *reinterpret_cast<u32x4*>(Wr + g * 16) = u32x4{blk.qs[0], blk.qs[1], blk.qs[2], blk.qs[3]};
            sc[g] = static_cast<uint16_t>(blk.dbits);
            weight_fp6(blk.qs, d6);
            dbits = blk.dbits;
            r = g / nb;
            b = g - r * nb;
        } else {
            r = g - nblocks;  // the zero plane
            b = nb;
        }
        const int swap = static_cast<int>(((r >> 2) ^ (r >> 3)) & 1);
        uint8_t* p = rec + (b * rows + r) * 32;
        *reinterpret_cast<u32x4*>(p + 16 * swap) = u32x4{d6[0], d6[1], d6[2], d6[3]};
        *reinterpret_cast<u32x4*>(p + 16 * (swap ^ 1)) = u32x4{d6[4], d6[5], dbits, 0u};
    }
}

// Rows `ids` of a Q4_0 table, decoded to fp32: ggml_get_rows on Q4_0, the
// token-embedding lookup ("llama.cpp 深度解读" section 4, and the GPT-2
// walkthrough's wte/wpe), each element (nibble - 8) * d by section 2's decode
// (exact in fp32).  8 lanes per block, 4 consecutive values (16 bytes) per
// lane, so a wave writes 8 blocks = 1 KB contiguously; the output stream is 7x
// the input.  An id outside [0, rows) gives a row of NaN.
__global__ void __launch_bounds__(kThreads)
k_q4_0_get_rows(const uint8_t* __restrict__ Wq, int64_t rows, int64_t nb, const int32_t* __restrict__ ids,
                int64_t n, float* __restrict__ out) {
    const int64_t total = n * nb;
    const int m = threadIdx.x & 7;
    const int64_t step = static_cast<int64_t>(gridDim.x) * (kThreads / 8);
    for (int64_t o = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 3; o < total; o += step) {
        const int64_t i = o / nb;
        const int64_t b = o - i * nb;
        const int64_t id = ids[i];
        float4 v;
        if (id >= 0 && id < rows) {
            const uint8_t* blk = Wq + (id * nb + b) * kQ4Bytes;
            uint16_t dbits, q2;
            __builtin_memcpy(&dbits, blk, 2);
            __builtin_memcpy(&q2, blk + 2 + 2 * m, 2);  // elements 4m .. 4m+3
            const float d = half_bits_to_float(dbits);
            v = make_float4(static_cast<float>(static_cast<int>(q2 & 15u) - 8) * d,
                            static_cast<float>(static_cast<int>((q2 >> 4) & 15u) - 8) * d,
                            static_cast<float>(static_cast<int>((q2 >> 8) & 15u) - 8) * d,
                            static_cast<float>(static_cast<int>(q2 >> 12) - 8) * d);
        } else {
            const float nan = __builtin_nanf("");
            v = make_float4(nan, nan, nan, nan);
        }
        *reinterpret_cast<float4*>(out + o * kQK + 4 * m) = v;
    }
}

// Prefill records are written block-major (record o = block * N + token).
// Grid: y walks the blocks, x the tokens 32 at a time (an 8-lane group per
// token; both loop bounds are uniform over each wave), so no index is
// divided.
constexpr int kAct6Tokens = kThreads / 8;  // tokens per workgroup iteration

// fp32 activations -> prefill records (fp6 operands + binary16 scale bits).
__global__ void __launch_bounds__(kThreads)
k_act6_from_f32(const float* __restrict__ X, int64_t N, int64_t nb, uint32_t* __restrict__ rec) {
    const int m = threadIdx.x & 7;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kAct6Tokens;
    const int64_t wave_first = static_cast<int64_t>(blockIdx.x) * kAct6Tokens + ((threadIdx.x >> 3) & ~7);
    for (int64_t b = blockIdx.y; b < nb; b += gridDim.y)
    for (int64_t n0 = wave_first; n0 < N; n0 += step) {
        const int64_t n = n0 + ((threadIdx.x >> 3) & 7);
        const bool valid = n < N;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (valid) __builtin_memcpy(&x, X + (n * nb + b) * kQK + 4 * m, 16);
        uint32_t word, dbits;
        quant_act_quad(x.x, x.y, x.z, x.w, m, word, dbits);
        store_act6(m, word, dbits, valid, b * N + n, rec);
    }
}

// Q8_0 blocks -> prefill records.
__global__ void __launch_bounds__(kThreads)
k_act6_from_q8(const uint8_t* __restrict__ Xq, int64_t N, int64_t nb, uint32_t* __restrict__ rec) {
    const int m = threadIdx.x & 7;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kAct6Tokens;
    const int64_t wave_first = static_cast<int64_t>(blockIdx.x) * kAct6Tokens + ((threadIdx.x >> 3) & ~7);
    for (int64_t b = blockIdx.y; b < nb; b += gridDim.y)
    for (int64_t n0 = wave_first; n0 < N; n0 += step) {
        const int64_t n = n0 + ((threadIdx.x >> 3) & 7);
        const bool valid = n < N;
        int8_t q[4] = {0, 0, 0, 0};
        uint16_t h = 0;
        if (valid) {
            const uint8_t* blk = Xq + (n * nb + b) * kQ8Bytes;
            __builtin_memcpy(q, blk + 2 + 4 * m, 4);
            __builtin_memcpy(&h, blk, 2);
        }
        int bias;
        const uint32_t word = dot_order_word(q[0], q[1], q[2], q[3], m, bias);
        store_act6(m, word, h, valid, b * N + n, rec);
    }
}

// Pack one block's int8 values (lane e of a half-wave holds q_e) into the
// internal dot order and store it with its scale record.
__device__ __forceinline__ void store_act(int e, int q, float d, bool valid, int64_t g,
                                          uint32_t* __restrict__ act_q, ActScale* __restrict__ act_s) {
    // element e -> dword 2*(e/8) + (e%2), byte (e/2)%4
    uint32_t v = (static_cast<uint32_t>(q) & 0xFFu) << (8 * ((e >> 1) & 3));
    v = or_lanes(v, 2);
    v = or_lanes(v, 4);
    const int bias = -8 * sum32(q);
    if (valid) {
        if ((e & 6) == 0) act_q[g * 8 + 2 * (e >> 3) + (e & 1)] = v;
        if (e == 0) act_s[g] = ActScale{d, bias};
    }
}

__global__ void __launch_bounds__(kThreads)
k_act_from_q8(const uint8_t* __restrict__ Xq, int64_t nblocks, uint32_t* __restrict__ act_q,
              ActScale* __restrict__ act_s) {
    const int e = threadIdx.x & 31;
    const int64_t first = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 5;
    const int64_t step = static_cast<int64_t>(gridDim.x) * (kThreads / 32);
    const int64_t wave_first = first & ~static_cast<int64_t>(1);
    for (int64_t g0 = wave_first; g0 < nblocks; g0 += step) {
        const int64_t g = g0 + (first & 1);
        const bool valid = g < nblocks;
        int q = 0;
        uint32_t dbits = 0;
        if (valid) {
            const uint8_t* blk = Xq + g * kQ8Bytes;
            q = static_cast<int>(static_cast<int8_t>(blk[2 + e]));
            uint16_t h;
            __builtin_memcpy(&h, blk, 2);
            dbits = h;
        }
        store_act(e, q, half_bits_to_float(dbits), valid, g, act_q, act_s);
    }
}

int quant_grid(int64_t nblocks) {
    int64_t wgs = (nblocks + (kThreads / 32) - 1) / (kThreads / 32);
    const int64_t cap = 8192;
    if (wgs > cap) wgs = cap;
    if (wgs < 1) wgs = 1;
    return static_cast<int>(wgs);
}

}  // namespace

size_t act_bytes(int64_t N, int64_t nb) {
    if (N <= kGemvMaxN) return static_cast<size_t>(N * nb) * (kActQBytes + kActSBytes);
    return static_cast<size_t>(N * nb) * kAct6Bytes;
}

hipError_t launch_q4_0_quantize(const float* W, int64_t nblocks, uint8_t* Wq, hipStream_t s) {
    hipLaunchKernelGGL(k_q4_0_quantize, dim3(quant_grid(nblocks)), dim3(kThreads), 0, s, W, nblocks, Wq);
    return hipGetLastError();
}

int64_t repack_records_offset(int64_t rows, int64_t nb) { return (rows * nb * kQ4Bytes + 255) & ~int64_t(255); }

size_t repack_bytes(int64_t rows, int64_t nb) {
    return static_cast<size_t>(repack_records_offset(rows, nb) + (nb + 1) * rows * 32);
}

hipError_t launch_q4_0_repack(const uint8_t* Wq, int64_t rows, int64_t nb, uint8_t* Wr, hipStream_t s) {
    hipLaunchKernelGGL(k_q4_0_repack, dim3(quant_grid(rows * nb + rows + 256)), dim3(kThreads), 0, s, Wq, rows, nb,
                       repack_records_offset(rows, nb), Wr);
    return hipGetLastError();
}

hipError_t launch_q4_0_get_rows(const uint8_t* Wq, int64_t rows, int64_t nb, const int32_t* ids, int64_t n,
                                float* out, hipStream_t s) {
    int64_t wgs = (n * nb + (kThreads / 8) - 1) / (kThreads / 8);
    if (wgs > 16384) wgs = 16384;
    hipLaunchKernelGGL(k_q4_0_get_rows, dim3(static_cast<uint32_t>(wgs < 1 ? 1 : wgs)), dim3(kThreads), 0, s, Wq, rows,
                       nb, ids, n, out);
    return hipGetLastError();
}

hipError_t launch_q8_0_quantize(const float* X, int64_t nblocks, uint8_t* Xq, hipStream_t s) {
    hipLaunchKernelGGL(k_q8_0_quantize, dim3(quant_grid(nblocks)), dim3(kThreads), 0, s, X, nblocks, Xq);
    return hipGetLastError();
}

namespace {
// Prefill records: y = blocks (at most 8192), x = token groups of kAct6Tokens,
// at most 8192 workgroups in all.
dim3 act6_grid(int64_t N, int64_t nb) {
    const int64_t y = nb < 8192 ? nb : 8192;
    int64_t x = (N + kAct6Tokens - 1) / kAct6Tokens;
    const int64_t xmax = 8192 / y > 0 ? 8192 / y : 1;
    if (x > xmax) x = xmax;
    return dim3(static_cast<uint32_t>(x < 1 ? 1 : x), static_cast<uint32_t>(y < 1 ? 1 : y));
}
}  // namespace

hipError_t launch_act_from_f32(const float* X, int64_t N, int64_t nb, void* act, hipStream_t s) {
    const int64_t nblocks = N * nb;
    if (N > kGemvMaxN) {
        uint32_t* rec = static_cast<uint32_t*>(act);
        hipLaunchKernelGGL(k_act6_from_f32, act6_grid(N, nb), dim3(kThreads), 0, s, X, N, nb, rec);
        return hipGetLastError();
    }
    uint32_t* q = static_cast<uint32_t*>(act);
    ActScale* sc = reinterpret_cast<ActScale*>(static_cast<uint8_t*>(act) + nblocks * kActQBytes);
    int64_t wgs = (nblocks + (kThreads / 8) - 1) / (kThreads / 8);
    if (wgs > 8192) wgs = 8192;
    hipLaunchKernelGGL(k_act_from_f32, dim3(static_cast<uint32_t>(wgs)), dim3(kThreads), 0, s, X, nblocks, q, sc);
    return hipGetLastError();
}

namespace {

template <bool PREFILL, int QPT>
hipError_t ln_act_k(const float* X, int64_t N, int64_t nb, const float* gamma, const float* beta, float eps,
                    uint32_t* q, ActScale* sc, hipStream_t s) {
    hipLaunchKernelGGL((k_ln_act<PREFILL, QPT>), dim3(static_cast<uint32_t>(N)), dim3(kLnActThreads), 0, s, X, N, nb,
                       gamma, beta, eps, q, sc);
    return hipGetLastError();
}

template <bool PREFILL>
hipError_t ln_act_p(const float* X, int64_t N, int64_t nb, const float* gamma, const float* beta, float eps,
                    uint32_t* q, ActScale* sc, hipStream_t s) {
    const int64_t qpt = (nb * 8 + kLnActThreads - 1) / kLnActThreads;
    if (qpt <= 1) return ln_act_k<PREFILL, 1>(X, N, nb, gamma, beta, eps, q, sc, s);
    if (qpt <= 2) return ln_act_k<PREFILL, 2>(X, N, nb, gamma, beta, eps, q, sc, s);
    if (qpt <= 4) return ln_act_k<PREFILL, 4>(X, N, nb, gamma, beta, eps, q, sc, s);
    if (qpt <= 8) return ln_act_k<PREFILL, 8>(X, N, nb, gamma, beta, eps, q, sc, s);
    return ln_act_k<PREFILL, 0>(X, N, nb, gamma, beta, eps, q, sc, s);
}

}  // namespace

hipError_t launch_ln_act(const float* X, int64_t N, int64_t nb, const float* gamma, const float* beta, float eps,
                         void* act, hipStream_t s) {
    uint32_t* q = static_cast<uint32_t*>(act);
    if (N > kGemvMaxN) return ln_act_p<true>(X, N, nb, gamma, beta, eps, q, nullptr, s);
    ActScale* sc = reinterpret_cast<ActScale*>(static_cast<uint8_t*>(act) + N * nb * kActQBytes);
    return ln_act_p<false>(X, N, nb, gamma, beta, eps, q, sc, s);
}

hipError_t launch_act_from_q8(const uint8_t* Xq, int64_t N, int64_t nb, void* act, hipStream_t s) {
    const int64_t nblocks = N * nb;
    if (N > kGemvMaxN) {
        uint32_t* rec = static_cast<uint32_t*>(act);
        hipLaunchKernelGGL(k_act6_from_q8, act6_grid(N, nb), dim3(kThreads), 0, s, Xq, N, nb, rec);
        return hipGetLastError();
    }
    uint32_t* q = static_cast<uint32_t*>(act);
    ActScale* sc = reinterpret_cast<ActScale*>(static_cast<uint8_t*>(act) + nblocks * kActQBytes);
    hipLaunchKernelGGL(k_act_from_q8, dim3(quant_grid(nblocks)), dim3(kThreads), 0, s, Xq, nblocks, q, sc);
    return hipGetLastError();
}

}  // namespace q4bq
