// Decode product on the matrix cores, up to 8 tokens (`k_gemv_mma`).
//
// The arithmetic of ggml_vec_dot_q4_0_q8_0 as "llama.cpp 深度解读"
// (luoboask.github.io) section 3 "量化矩阵乘法 — 核心算子" describes it, with
// the nibble offset of 8 from section 2's decode: per 32-value block the
// integer dot s = sum_j (nibble_j - 8) * q_j, then fp32 acc += s * (d_w * d_x).
//
// With several tokens the row-streaming kernel spends most of its vector
// instructions on the byte dots (eight v_dot4 per block and token).  Here one
// v_mfma_i32_32x32x32_i8 takes the integer dots of a tile of 32 rows x one
// block for all tokens at once: the activations are the M side (32 token
// slots, 8 of them used: lane l's outputs 0..3 are tokens 4 (l / 32) + 0..3),
// the weights the N side (lane l holds row l % 32).  The operands need no
// conversion: a Q4_0 nibble word splits into unsigned bytes 0..15 with a mask
// and a shift, in the activation blocks' dot order, and the matrix core's
// accumulator input is seeded with the activation block's -8 * sum(q), so the
// result is s exactly.  The vector ALU keeps, per lane and block, the split of
// two nibble words and four (convert, scale product, FMA) for its four
// outputs.
//
// Loads: workgroup g takes the tiles of 32 rows (32 * K/32 * 18 contiguous
// bytes) g, g + G, ... one at a time, so that the grid streams one band of the
// matrix; its waves split the tile's K: wave w takes chunks w, w + W,
// ... of 4 blocks; lane (j, h) of a wave reads the block pair 2c + h of row j
// (36 bytes), and one v_permlane32_swap per nibble word gives lane (j, 0) the
// first half and lane (j, 1) the second half of all four blocks, as the matrix
// instruction wants them.  Each wave keeps D chunks' loads in flight across
// tiles.  At the end of a tile the waves' partial sums meet in LDS and 256
// threads add them in wave order (a fixed order: repeated calls give the same
// bits) and store Y.
//
// LDS: the activations of the N tokens (token n's blocks at n * S, 32
// dot-order bytes per block; S = 32 mod 256 bytes so that the 16-byte operand
// reads of 16 lanes hit 16 distinct bank groups), their scale records as two
// [block][8 tokens] planes (bias, d), and two buffers of partial sums.
//
// One matrix may carry the fused forms' epilogue (md.epi: bias, activation,
// factor), applied at the store.
#include "q4bq_device.h"
#include "q4bq_internal.h"

namespace q4bq {

namespace {

typedef int32_t i32x4v __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kMmaSlots = 8;  // token slots of the scale planes
constexpr int kRsrcFlags = 0x00020000;  // buffer resource word 3: raw 32-bit data
constexpr int kMmaMaxLds = 160 * 1024;

// Blocks per token in LDS: the row's blocks and two more (the last chunk of
// a row reads up to two blocks past its end; their scales are zero).
__host__ __device__ inline int64_t mma_blocks(int64_t nb) { return nb + 2; }
// Byte stride of one token's activation blocks in LDS.
__host__ __device__ inline int64_t mma_token_stride(int64_t nb) {
    return (mma_blocks(nb) * kActQBytes + 255) / 256 * 256 + 32;
}

template <int THREADS>
inline int64_t mma_lds_bytes(int64_t N, int64_t nb) {
    return N * mma_token_stride(nb) + mma_blocks(nb) * kMmaSlots * 12 + 2 * (THREADS / 64) * 4 * 64 * 4;
}

// The matrix core's accumulator is seeded with the activation block's
// -8 * sum(q) plus 0x4B400000, so its int32 result, read as fp32, is exactly
// 12582912 + s (|s| < 2^22: the fp32 spacing there is 1); one FMA against the
// plane of -12582912 * d_x then gives fl(s * d_x) with a single rounding.
constexpr int32_t kMagicBits = 0x4B400000;
constexpr float kMagic = 12582912.0f;

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Swaps a's upper 32 lanes with b's lower 32 lanes.
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = static_cast<uint32_t>(r[0]);
    b = static_cast<uint32_t>(r[1]);
}

template <int THREADS, int D, int SRC, int LAY>
__global__ void __launch_bounds__(THREADS)
k_gemv_mma(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const void* __restrict__ src, int N,
           float* __restrict__ Y, const MultiDesc md) {
    static_assert(SRC == kXF32 || SRC == kActGlobal, "activation source");
    constexpr bool RP = LAY == kLayRepacked;
    constexpr bool MULTI = LAY == kLayMulti;
    constexpr int kWaves = THREADS / 64;
    extern __shared__ __align__(16) uint8_t smem[];
    const int64_t S = mma_token_stride(nb);
    uint8_t* sA = smem;
    // scale planes [block][slot]: seed (bias + kMagicBits), d_x, -kMagic * d_x
    const int nbp = static_cast<int>(mma_blocks(nb));
    int32_t* sBias = reinterpret_cast<int32_t*>(smem + N * S);
    float* sDx = reinterpret_cast<float*>(sBias + nbp * kMmaSlots);
    float* sDxm = sDx + nbp * kMmaSlots;
    float* sPart = sDxm + nbp * kMmaSlots;  // [2][kWaves][4][64]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int P = nb >> 1;                          // block pairs per row
    const int nc = (P + 1) >> 1;                    // chunks of two pairs
    const int cpw = (nc + kWaves - 1) / kWaves;     // chunks per wave and tile
    // this workgroup's 32-row tiles: blockIdx.x, blockIdx.x + G, ... (so the
    // grid streams one band of the matrix at a time; measured faster on the
    // vocabulary head than contiguous shares of the rows)
    const int64_t G = gridDim.x;
    const int64_t ntiles = (rows + 31) >> 5;
    const int64_t ntq = blockIdx.x < ntiles ? (ntiles - 1 - blockIdx.x) / G + 1 : 0;
    const int64_t nitems = ntq * cpw;               // the same for every wave
    const int nblk = N * nb;

    // 1. the activations' first loads: X's first 16-byte quads (kXF32), or the
    // quantizer's first 16-byte pieces and scale records
    constexpr int kJpre = 8;               // quads per thread
    constexpr int kPpre = 4, kRpre = 2;    // pieces and records per thread
    float4 xv[SRC == kXF32 ? kJpre : 1];
    u32x4 av[SRC == kActGlobal ? kPpre : 1];
    ActScale rv[SRC == kActGlobal ? kRpre : 1];
    const u32x4* act_q = static_cast<const u32x4*>(src);
    const ActScale* act_s =
        reinterpret_cast<const ActScale*>(static_cast<const uint8_t*>(src) + static_cast<size_t>(nblk) * kActQBytes);
    if constexpr (SRC == kXF32) {
        const float* X = static_cast<const float*>(src);
#pragma unroll
        for (int j = 0; j < kJpre; ++j) {
            const int g = min(static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j, nblk - 1);
            __builtin_memcpy(&xv[j], X + static_cast<int64_t>(g) * kQK + 4 * (threadIdx.x & 7), 16);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPpre; ++j) av[j] = act_q[min(static_cast<int>(threadIdx.x) + THREADS * j, 2 * nblk - 1)];
#pragma unroll
        for (int j = 0; j < kRpre; ++j) rv[j] = act_s[min(static_cast<int>(threadIdx.x) + THREADS * j, nblk - 1)];
    }

    // the activations land before any weight load goes out: once the weight
    // streams of the whole grid fill the memory pipelines, a load waits behind
    // them (2-10 us measured, against 1-2 us without them)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // 2. the first D chunks of this wave.  Item k: tile q = k / cpw of this
    // workgroup, chunk c = wave + kWaves (k % cpw); lane (j, h) reads pair
    // 2c + h of row j of the tile.  The loads go through a buffer resource
    // that spans the item's tile (wave-uniform: a tile of the multi-matrix
    // form lies in one matrix), so that the loads stay unconditional -- the
    // compiler's in-order load counter then waits for exactly one item -- and
    // still cost nothing where there is nothing to read: past the wave's last
    // item the resource has zero bytes and its loads return zeros without a
    // memory access.  Inside a tile, rows past the matrix end and pairs past
    // the row end re-read valid ones (their scales are zeroed below).  A
    // tile's bytes stay below 2^32: 32 rows of at most 1280 blocks (the LDS
    // bound on K with four or more tokens).
    auto load_item = [&](Pair36& dst, int64_t k) __attribute__((always_inline)) {
        const bool live = k < nitems;
        if (k > nitems - 1) k = nitems - 1;
        if (k < 0) k = 0;
        const int64_t q = k / cpw;
        const int c = wave + kWaves * static_cast<int>(k - q * cpw);
        const int p = min(2 * c + h, P - 1);
        const int64_t r0 = (blockIdx.x + q * G) * 32;
        const int64_t nr = live ? min(static_cast<int64_t>(32), rows - r0) : 0;  // rows of the tile to read
        const uint32_t lr = static_cast<uint32_t>(min(static_cast<int64_t>(l32), nr > 0 ? nr - 1 : 0));
        if constexpr (RP) {
            const uint8_t* nib = Wq + (nr > 0 ? r0 : 0) * nb * 16;
            const uint8_t* sc = Wq + rows * nb * 16 + (nr > 0 ? r0 : 0) * nb * 2;
            const auto rn = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(nib), static_cast<short>(0),
                                                               static_cast<int>(nr > 0 ? nr * nb * 16 : 0), kRsrcFlags);
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sc), static_cast<short>(0),
                                                               static_cast<int>(nr > 0 ? nr * nb * 2 : 0), kRsrcFlags);
            const uint32_t o = (lr * nb + 2 * p) * 16;
            const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rn, o, 0, 0));
            const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rn, o + 16, 0, 0));
            const uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(rs, (lr * nb + 2 * p) * 2, 0, 0);
            dst.w[0] = a.x; dst.w[1] = a.y; dst.w[2] = a.z; dst.w[3] = a.w;
            dst.w[4] = b.x; dst.w[5] = b.y; dst.w[6] = b.z; dst.w[7] = b.w;
            dst.w[8] = e;
        } else {
            const uint8_t* wb = Wq;
            int64_t f = 0;
            if constexpr (MULTI) {
                wb = md.w[0];
#pragma unroll
                for (int m = 1; m < kMaxMulti; ++m)
                    if (m < md.count && r0 >= md.first[m]) {
                        wb = md.w[m];
                        f = md.first[m];
                    }
            }
            const uint8_t* base = wb + (nr > 0 ? r0 - f : 0) * nb * kQ4Bytes;
            const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0),
                                                               static_cast<int>(nr > 0 ? nr * nb * kQ4Bytes : 0),
                                                               kRsrcFlags);
            const uint32_t o = (lr * nb + 2 * p) * kQ4Bytes;
            const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, o, 0, 0));
            const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, o + 16, 0, 0));
            const uint32_t e = __builtin_amdgcn_raw_buffer_load_b32(rw, o + 32, 0, 0);
            dst.w[0] = a.x; dst.w[1] = a.y; dst.w[2] = a.z; dst.w[3] = a.w;
            dst.w[4] = b.x; dst.w[5] = b.y; dst.w[6] = b.z; dst.w[7] = b.w;
            dst.w[8] = e;
        }
    };
    // the first D items: for fp32 X in flight while the workgroup quantizes
    // it; the quantizer's buffer only needs copying, and its copy is shortest
    // with no weight loads of this workgroup in flight (measured), so there
    // they follow the copy
    Pair36 raw[D];
    auto prefetch = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_item(raw[d], d);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (SRC == kXF32) prefetch();

    // 3. activations into LDS: blocks at n * S + 32 b, scale records into the
    // [block][slot] planes; slots n >= N hold zeros
    if constexpr (SRC == kXF32) {
        const float* X = static_cast<const float*>(src);
        const int m = threadIdx.x & 7;
        auto quantize = [&](float4 x, int j) __attribute__((always_inline)) {
            const int g = static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j;
            const bool valid = g < nblk;
            if (!valid) x = make_float4(0.f, 0.f, 0.f, 0.f);
            uint32_t word;
            const ActScale sc = quant_act_quad(x.x, x.y, x.z, x.w, m, word);
            if (valid) {
                const int n = g / nb, b = g - n * nb;
                *reinterpret_cast<uint32_t*>(sA + n * S + b * kActQBytes + 4 * m) = word;
                if (m == 0) {
                    sBias[b * kMmaSlots + n] = sc.bias + kMagicBits;
                    sDx[b * kMmaSlots + n] = sc.d;
                    sDxm[b * kMmaSlots + n] = -kMagic * sc.d;
                }
            }
        };
        // quads past the N tokens' blocks are skipped (a whole 8-lane group
        // at a time, which is what the quantizer's lane exchanges span)
#pragma unroll
        for (int j = 0; j < kJpre; ++j)
            if (static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j < nblk) quantize(xv[j], j);
        const int jend = (nblk + THREADS / 8 - 1) / (THREADS / 8);
        for (int j = kJpre; j < jend; ++j) {
            const int g = min(static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j, nblk - 1);
            float4 x;
            __builtin_memcpy(&x, X + static_cast<int64_t>(g) * kQK + 4 * m, 16);
            quantize(x, j);
        }
    } else {
        auto put_piece = [&](int i, const u32x4& v) __attribute__((always_inline)) {
            const int n = i / (2 * nb), pc = i - n * 2 * nb;
            *reinterpret_cast<u32x4*>(sA + n * S + pc * 16) = v;
        };
        auto put_record = [&](int g, const ActScale& r) __attribute__((always_inline)) {
            const int n = g / nb, b = g - n * nb;
            sBias[b * kMmaSlots + n] = r.bias + kMagicBits;
            sDx[b * kMmaSlots + n] = r.d;
            sDxm[b * kMmaSlots + n] = -kMagic * r.d;
        };
#pragma unroll
        for (int j = 0; j < kPpre; ++j)
            if (static_cast<int>(threadIdx.x) + THREADS * j < 2 * nblk) put_piece(threadIdx.x + THREADS * j, av[j]);
#pragma unroll
        for (int j = 0; j < kRpre; ++j)
            if (static_cast<int>(threadIdx.x) + THREADS * j < nblk) put_record(threadIdx.x + THREADS * j, rv[j]);
        // the rest of long activations (loaded after the weights: these wait for them)
        for (int i = threadIdx.x + THREADS * kPpre; i < 2 * nblk; i += THREADS) put_piece(i, act_q[i]);
        for (int g = threadIdx.x + THREADS * kRpre; g < nblk; g += THREADS) put_record(g, act_s[g]);
    }
    // slots past the N tokens and the two blocks past the row: scale 0 (and a
    // seed that keeps the matrix core's result a finite fp32 value)
    for (int i = threadIdx.x; i < nbp * kMmaSlots; i += THREADS)
        if ((i & (kMmaSlots - 1)) >= N || i >= nb * kMmaSlots) {
            sBias[i] = kMagicBits;
            sDx[i] = 0.0f;
            sDxm[i] = 0.0f;
        }
    lds_barrier();
    if (nitems == 0) return;  // the whole workgroup: no rows
    if constexpr (SRC == kActGlobal) prefetch();

    // this lane's activation operand: token slot l & 7 (clamped to the N
    // tokens), 16-byte half h; lanes 8..15 of each 16-lane group read the
    // other half (their outputs are never used) so that 16 lanes touch 16
    // distinct bank groups
    const int a_tok = min(lane & 7, N - 1);
    const int a_half = h ^ ((lane >> 3) & 1);
    const uint8_t* a_base = sA + a_tok * S + 16 * a_half;

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int buf = 0;
    int ci = 0;        // chunk index within the tile
    int64_t q = 0;     // tile of this workgroup
    for (int64_t k = 0; k < nitems; k += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (k + d < nitems) {
                // (a wave without a chunk in this tile takes the last one, its scales zeroed)
                const int c = min(wave + kWaves * ci, nc - 1);
                const bool pv = wave + kWaves * ci < nc && 2 * c + h < P;
                Block4 f, s;
                if constexpr (RP) {
                    f = pair_first_rp(raw[d]);
                    s = pair_second_rp(raw[d]);
                } else {
                    f = pair_first(raw[d]);
                    s = pair_second(raw[d]);
                }
                // blocks 4c, 4c+1 sit in lanes h = 0, blocks 4c+2, 4c+3 in h = 1;
                // afterwards word pair (x0, x1) of block i is half h of block 4c + i
                uint32_t fa0 = f.qs[0], fa1 = f.qs[1], fb0 = f.qs[2], fb1 = f.qs[3];
                uint32_t sa0 = s.qs[0], sa1 = s.qs[1], sb0 = s.qs[2], sb1 = s.qs[3];
                swap_halves(fa0, fb0);
                swap_halves(fa1, fb1);
                swap_halves(sa0, sb0);
                swap_halves(sa1, sb1);
                uint32_t d01 = pv ? (f.dbits | (s.dbits << 16)) : 0u;
                uint32_t d23 = d01;
                swap_halves(d01, d23);
                const uint32_t x0[4] = {fa0, sa0, fb0, sb0};
                const uint32_t x1[4] = {fa1, sa1, fb1, sb1};
                const uint32_t db[4] = {d01 & 0xFFFFu, d01 >> 16, d23 & 0xFFFFu, d23 >> 16};
                // the chunk's blocks 4c .. 4c + 3 (at most nb + 1: the LDS rows are padded)
                const uint8_t* ab = a_base + 4 * c * kActQBytes;
                const int pb = 4 * c * kMmaSlots + 4 * h;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const i32x4v wop = {static_cast<int>(nib_lo(x0[i])), static_cast<int>(nib_hi(x0[i])),
                                        static_cast<int>(nib_lo(x1[i])), static_cast<int>(nib_hi(x1[i]))};
                    const i32x4v aop = *reinterpret_cast<const i32x4v*>(ab + i * kActQBytes);
                    const i32x4v seed = *reinterpret_cast<const i32x4v*>(sBias + pb + i * kMmaSlots);
                    const f32x4v dx = *reinterpret_cast<const f32x4v*>(sDx + pb + i * kMmaSlots);
                    const f32x4v dxm = *reinterpret_cast<const f32x4v*>(sDxm + pb + i * kMmaSlots);
                    const i32x16 cin = __builtin_shufflevector(seed, seed, 0, 1, 2, 3, -1, -1, -1, -1, -1, -1, -1,
                                                               -1, -1, -1, -1, -1);
                    const i32x16 sdot = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, wop, cin, 0, 0, 0);
                    const float dw = half_bits_to_float(db[i]);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int32_t bits = sdot[v];  // (a vector element is not an object to bit-cast)
                        const float t = fmaf(__builtin_bit_cast(float, bits), dx[v], dxm[v]);  // fl(s * d_x)
                        acc[v] = fmaf(t, dw, acc[v]);
                    }
                }
                if (++ci == cpw) {
                    // the tile's partial sums: [buf][wave][output v][lane]
                    float* pw = sPart + ((buf * kWaves + wave) * 4) * 64 + lane;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        pw[v * 64] = acc[v];
                        acc[v] = 0.0f;
                    }
                    lds_barrier();
                    if (threadIdx.x < 256) {
                        // output (row j, token n): lane 32 (n >> 2) + j, value n & 3
                        const int j = threadIdx.x & 31, n = threadIdx.x >> 5;
                        const float* pr = sPart + (buf * kWaves * 4 + (n & 3)) * 64 + 32 * (n >> 2) + j;
                        float y = pr[0];
#pragma unroll
                        for (int w = 1; w < kWaves; ++w) y += pr[w * 4 * 64];
                        const int64_t r = (blockIdx.x + q * G) * 32 + j;
                        if (n < N && r < rows) {
                            if constexpr (MULTI) {
                                float* yb = md.y[0];
                                int64_t f0 = 0, f1 = md.first[1];
#pragma unroll
                                for (int m = 1; m < kMaxMulti; ++m)
                                    if (m < md.count && r >= md.first[m]) {
                                        yb = md.y[m];
                                        f0 = md.first[m];
                                        f1 = md.first[m + 1];
                                    }
                                yb[n * (f1 - f0) + (r - f0)] = y;
                            } else {
                                Y[n * rows + r] = apply_epilogue(y, n, r, rows, md.epi);
                            }
                        }
                    }
                    buf ^= 1;
                    ci = 0;
                    ++q;
                }
            }
            load_item(raw[d], k + d + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

}  // namespace

bool mma_apply(int64_t N, int64_t nb, int64_t rows, const MultiDesc* md) {
    if (md)
        for (int m = 1; m < md->count; ++m)
            if (md->first[m] % 32 != 0) return false;  // every 32-row tile within one matrix
    // measured against the row-streaming and task kernels (graph-timed, the
    // Llama-3-8B, GPT-2 and vocabulary-head shapes): the matrix cores win from
    // five tokens on matrices of at least 2048 rows and K <= 8192; on the
    // longest matrices the row kernel streams at nearly full rate up to six
    // tokens; fewer rows leave CUs idle (one workgroup per 32 rows), longer
    // rows put most of the time into the per-workgroup activation copy
    if (N < kMmaMinN || N > kGemvMaxN || nb % 2 != 0 || nb > kMmaMaxBlocks || rows < kMmaMinRows) return false;
    if (rows >= kMmaLongRows && N < kMmaLongMinN) return false;
    return mma_lds_bytes<kMmaThreads>(N, nb) <= kMmaMaxLds;
}

namespace {

template <int SRC, int LAY>
hipError_t launch_mma_k(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                        int64_t N, float* Y, const MultiDesc& md, hipStream_t s) {
    const int64_t ntiles = (rows + 31) / 32;
    const int64_t grid = ntiles < dev->num_cu ? ntiles : dev->num_cu;
    // items in flight per wave: four where every workgroup has 16 tiles or
    // more (the vocabulary head), else two (measured: 14336 x 4096 at N = 8,
    // 13.7 -> 11.9 us)
    const auto kernel = ntiles >= 16 * grid ? k_gemv_mma<kMmaThreads, 4, SRC, LAY> : k_gemv_mma<kMmaThreads, 2, SRC, LAY>;
    const size_t lds = static_cast<size_t>(mma_lds_bytes<kMmaThreads>(N, nb));
    if (lds > 64 * 1024) {
        const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, kMmaMaxLds);
        if (raised != hipSuccess) return raised;
    }
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(grid)), dim3(kMmaThreads), lds, s, Wq, rows,
                       static_cast<int>(nb), src, static_cast<int>(N), Y, md);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mma(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                           const void* src, bool src_f32, int64_t N, float* Y, const MultiDesc& md, hipStream_t s) {
    if (!mma_apply(N, nb, rows, lay == kLayMulti ? &md : nullptr)) return hipErrorInvalidValue;
    if (src_f32) {
        switch (lay) {
            case kLayRepacked: return launch_mma_k<kXF32, kLayRepacked>(dev, Wq, rows, nb, src, N, Y, md, s);
            case kLayMulti: return launch_mma_k<kXF32, kLayMulti>(dev, Wq, rows, nb, src, N, Y, md, s);
            default: return launch_mma_k<kXF32, kLayAoS>(dev, Wq, rows, nb, src, N, Y, md, s);
        }
    }
    switch (lay) {
        case kLayRepacked: return launch_mma_k<kActGlobal, kLayRepacked>(dev, Wq, rows, nb, src, N, Y, md, s);
        case kLayMulti: return launch_mma_k<kActGlobal, kLayMulti>(dev, Wq, rows, nb, src, N, Y, md, s);
        default: return launch_mma_k<kActGlobal, kLayAoS>(dev, Wq, rows, nb, src, N, Y, md, s);
    }
}

}  // namespace q4bq
