// Decode product on the matrix cores, up to 8 tokens (`k_gemv_mma_tr`, and
// `k_gemv_mma` for the rows it does not take).
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
// matrix; its waves split the tile's K: wave w takes chunks w, w + W, ...
// `k_gemv_mma_tr` (chunks of 8 blocks): each wave loads its chunk of the 32
// rows as consecutive 16-byte pieces and reorders it through its own LDS
// area (below).  `k_gemv_mma` (chunks of 4 blocks): lane (j, h) of a wave
// reads the block pair 2c + h of row j (36 bytes), and one v_permlane32_swap
// per nibble word gives lane (j, 0) the first half and lane (j, 1) the second
// half of all four blocks, as the matrix instruction wants them.  Each wave
// keeps D chunks' loads in flight across tiles.  At the end of a tile the
// waves' partial sums meet in LDS and 256 threads add them in wave order (a
// fixed order: repeated calls give the same bits) and store Y.
//
// LDS: the activations of the N tokens (token n's blocks at n * S, 32
// dot-order bytes per block; S = 32 mod 256 bytes so that the 16-byte operand
// reads of 16 lanes hit 16 distinct bank groups), their scale records as
// [block][8 tokens] planes, two buffers of partial sums, and for
// `k_gemv_mma_tr` one item area per wave.
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

// LDS of both kernels: the activations (token n's blocks at n * S), the
// [block][slot] scale planes (seed = bias + kMagicBits, d_x, -kMagic * d_x)
// and the partial sums, in that order; the item areas of `k_gemv_mma_tr`
// follow.
struct MmaLds {
    uint8_t* a;
    int32_t* seed;
    float* dx;
    float* dxm;
    float* part;
    int64_t S;
};

template <int THREADS>
__device__ __forceinline__ MmaLds mma_lds(uint8_t* smem, int N, int nb) {
    MmaLds L;
    L.S = mma_token_stride(nb);
    const int nbp = static_cast<int>(mma_blocks(nb));
    L.a = smem;
    L.seed = reinterpret_cast<int32_t*>(smem + N * L.S);
    L.dx = reinterpret_cast<float*>(L.seed + nbp * kMmaSlots);
    L.dxm = L.dx + nbp * kMmaSlots;
    L.part = L.dxm + nbp * kMmaSlots;
    return L;
}

// The activations into LDS: fp32 X quantized by the workgroup (kXF32) or the
// quantizer's buffer copied (kActGlobal).  Their first loads go out before
// anything else; `weights` (the first weight loads) runs right behind them,
// for fp32 X once they have landed (the weight loads are in flight while the
// workgroup quantizes).  Once the weight streams of the whole grid fill the
// memory pipelines, a load issued later waits behind them (2-10 us measured,
// against 1-2 us without them).  Ends with a workgroup barrier.
template <int THREADS, int SRC, typename F>
__device__ __forceinline__ void mma_stage_activations(const void* __restrict__ src, int N, int nb, const MmaLds& L,
                                                      F&& weights) {
    const int nblk = N * nb;
    const int nbp = static_cast<int>(mma_blocks(nb));
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
    // fp32 X: everything landed before the first weight loads go out; the
    // quantizer's buffer: the first weight loads go out behind the copy's
    // loads (the compiler waits for the copy alone)
    if constexpr (SRC == kXF32) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    else weights();

    if constexpr (SRC == kXF32) {
        weights();
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
                *reinterpret_cast<uint32_t*>(L.a + n * L.S + b * kActQBytes + 4 * m) = word;
                if (m == 0) {
                    L.seed[b * kMmaSlots + n] = sc.bias + kMagicBits;
                    L.dx[b * kMmaSlots + n] = sc.d;
                    L.dxm[b * kMmaSlots + n] = -kMagic * sc.d;
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
            *reinterpret_cast<u32x4*>(L.a + n * L.S + pc * 16) = v;
        };
        auto put_record = [&](int g, const ActScale& r) __attribute__((always_inline)) {
            const int n = g / nb, b = g - n * nb;
            L.seed[b * kMmaSlots + n] = r.bias + kMagicBits;
            L.dx[b * kMmaSlots + n] = r.d;
            L.dxm[b * kMmaSlots + n] = -kMagic * r.d;
        };
#pragma unroll
        for (int j = 0; j < kPpre; ++j)
            if (static_cast<int>(threadIdx.x) + THREADS * j < 2 * nblk) put_piece(threadIdx.x + THREADS * j, av[j]);
#pragma unroll
        for (int j = 0; j < kRpre; ++j)
            if (static_cast<int>(threadIdx.x) + THREADS * j < nblk) put_record(threadIdx.x + THREADS * j, rv[j]);
        // the rest of long activations
        for (int i = threadIdx.x + THREADS * kPpre; i < 2 * nblk; i += THREADS) put_piece(i, act_q[i]);
        for (int g = threadIdx.x + THREADS * kRpre; g < nblk; g += THREADS) put_record(g, act_s[g]);
    }
    // slots past the N tokens and the two blocks past the row: scale 0 (and a
    // seed that keeps the matrix core's result a finite fp32 value)
    for (int i = threadIdx.x; i < nbp * kMmaSlots; i += THREADS)
        if ((i & (kMmaSlots - 1)) >= N || i >= nb * kMmaSlots) {
            L.seed[i] = kMagicBits;
            L.dx[i] = 0.0f;
            L.dxm[i] = 0.0f;
        }
    lds_barrier();
}

// One block on the matrix cores for a lane's four outputs: a = the lane's
// activation operand, (w0, w1) = its half of the block's nibble words, pb =
// the block's entry in the scale planes for this lane's tokens, dbits = d_w.
__device__ __forceinline__ void mma_block(const MmaLds& L, const uint8_t* a, int pb, uint32_t w0, uint32_t w1,
                                          uint32_t dbits, float (&acc)[4]) {
    const i32x4v wop = {static_cast<int>(nib_lo(w0)), static_cast<int>(nib_hi(w0)), static_cast<int>(nib_lo(w1)),
                        static_cast<int>(nib_hi(w1))};
    const i32x4v aop = *reinterpret_cast<const i32x4v*>(a);
    const i32x4v seed = *reinterpret_cast<const i32x4v*>(L.seed + pb);
    const f32x4v dx = *reinterpret_cast<const f32x4v*>(L.dx + pb);
    const f32x4v dxm = *reinterpret_cast<const f32x4v*>(L.dxm + pb);
    const i32x16 cin = __builtin_shufflevector(seed, seed, 0, 1, 2, 3, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1);
    const i32x16 sdot = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, wop, cin, 0, 0, 0);
    const float dw = half_bits_to_float(dbits);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int32_t bits = sdot[v];  // (a vector element is not an object to bit-cast)
        const float t = fmaf(__builtin_bit_cast(float, bits), dx[v], dxm[v]);  // fl(s * d_x)
        acc[v] = fmaf(t, dw, acc[v]);
    }
}

// A tile's partial sums: each wave's four outputs per lane into buffer `buf`
// ([buf][wave][output v][lane]), accumulators cleared.
template <int kWaves>
__device__ __forceinline__ void mma_put_partials(const MmaLds& L, int buf, int wave, int lane, float (&acc)[4]) {
    float* pw = L.part + ((buf * kWaves + wave) * 4) * 64 + lane;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        pw[v * 64] = acc[v];
        acc[v] = 0.0f;
    }
}

// After a barrier: threads 0..255 add the waves' partial sums of buffer `buf`
// in wave order and store output (row r0 + j, token n): lane 32 (n >> 2) + j,
// value n & 3.  EPI: the epilogue reads bias or multiplier vectors.  Without
// them the store issues no load, so the compiler puts no wait for all loads in
// flight (the next items' weights) before it.
template <int kWaves, bool MULTI, bool EPI>
__device__ __forceinline__ void mma_store_tile(const MmaLds& L, int buf, int64_t r0, int64_t rows, int N, float* Y,
                                               const MultiDesc& md) {
    if (threadIdx.x >= 256) return;
    const int j = threadIdx.x & 31, n = threadIdx.x >> 5;
    const float* pr = L.part + (buf * kWaves * 4 + (n & 3)) * 64 + 32 * (n >> 2) + j;
    float y = pr[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) y += pr[w * 4 * 64];
    const int64_t r = r0 + j;
    if (n >= N || r >= rows) return;
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
        Y[n * rows + r] = EPI ? apply_epilogue(y, n, r, rows, md.epi) : epilogue_with(y, 0.0f, 1.0f, md.epi);
    }
}

template <int THREADS, int D, int SRC, int LAY, bool EPI>
__global__ void __launch_bounds__(THREADS)
k_gemv_mma(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const void* __restrict__ src, int N,
           float* __restrict__ Y, const MultiDesc md) {
    static_assert(SRC == kXF32 || SRC == kActGlobal, "activation source");
    constexpr bool RP = LAY == kLayRepacked;
    constexpr bool MULTI = LAY == kLayMulti;
    constexpr int kWaves = THREADS / 64;
    extern __shared__ __align__(16) uint8_t smem[];
    const MmaLds L = mma_lds<THREADS>(smem, N, nb);

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
    // The items are loaded in order, so their tile and chunk are counters (lr0:
    // the tile's first row, lc: the chunk index in the tile), not divisions (a
    // 64-bit division is some hundred scalar instructions, and the waves of a
    // SIMD share its scalar issue).
    int64_t lr0 = static_cast<int64_t>(blockIdx.x) * 32;
    int lc = 0;
    auto load_item = [&](Pair36& dst, int64_t k) __attribute__((always_inline)) {
        const bool live = k < nitems;
        const int c = wave + kWaves * lc;
        const int p = min(2 * c + h, P - 1);
        const int64_t r0 = lr0;
        if (++lc == cpw) {
            lc = 0;
            lr0 += G * 32;
        }
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
    // the first D items, issued right behind the activations' loads
    Pair36 raw[D];
    auto prefetch = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_item(raw[d], d);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    mma_stage_activations<THREADS, SRC>(src, N, nb, L, prefetch);

    if (nitems == 0) return;  // the whole workgroup: no rows

    // this lane's activation operand: token slot l & 7 (clamped to the N
    // tokens), 16-byte half h; lanes 8..15 of each 16-lane group read the
    // other half (their outputs are never used) so that 16 lanes touch 16
    // distinct bank groups
    const int a_tok = min(lane & 7, N - 1);
    const int a_half = h ^ ((lane >> 3) & 1);
    const uint8_t* a_base = L.a + a_tok * L.S + 16 * a_half;

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
                for (int i = 0; i < 4; ++i) mma_block(L, ab + i * kActQBytes, pb + i * kMmaSlots, x0[i], x1[i], db[i], acc);
                if (++ci == cpw) {
                    mma_put_partials<kWaves>(L, buf, wave, lane, acc);
                    lds_barrier();
                    mma_store_tile<kWaves, MULTI, EPI>(L, buf, (blockIdx.x + q * G) * 32, rows, N, Y, md);
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


// ---------------------------------------------------------------------------
// The same product with contiguous weight loads (block counts that are
// multiples of 8; every weight layout).  Measured
// on the vocabulary head (loads alone): load instructions whose 64 lanes take
// 16-byte pieces of 32 different rows (the kernel above) stream at ~3.9 TB/s;
// lanes that take consecutive 16-byte pieces of a 32-row x 144-byte item
// stream at ~5.4 TB/s, and ~5.3 TB/s with the reordering below.
//
// Item: 32 rows of a tile x one chunk of 8 blocks (144 bytes a row, nine
// 16-byte pieces), loaded by five instructions.  The pages' blocks: piece
// i * 64 + lane is piece p % 9 of row p / 9 (lanes 32..63 of the fifth have
// none).  Repacked: the first four take the 128 nibble bytes of each row
// (piece p % 8 of row p / 8), lanes 0..31 of the fifth its 16 scale bytes.
// Each wave writes its item into its own LDS area (rows 144 bytes apart: the
// pages' bytes, or the nibbles then the scales) and reads the matrix core's
// operands back (lane (j, h): row j, half h of each block) as whole 16-byte
// pieces, the same ones in both halves of the wave (measured: 4-byte reads
// at lane-dependent offsets meet 4- to 8-way bank conflicts that cost more
// than the loads save; 16-byte pieces of rows 36 dwords apart are free of
// them), each lane selecting its half's words.  One wave's LDS instructions
// run in order, so no barrier is needed.
//
// Chunk c = wave + W t of a tile (W waves) belongs to wave c mod W, its fp32
// sums chained through its chunks; after a barrier the waves' sums meet in
// LDS, added in wave order.  Both layouts take the same steps in the same
// order.
constexpr int kTrBlocks = 8;                       // blocks per item row
constexpr int kTrRowBytes = kTrBlocks * kQ4Bytes;  // 144
constexpr int kTrPieces = kTrRowBytes / 16;        // 9
constexpr int kTrLoads = (32 * kTrPieces + 63) / 64;  // 5
constexpr int kTrStride = kTrRowBytes;             // 144
constexpr int kTrWaveBytes = 32 * kTrStride;
static_assert(kTrRowBytes % 16 == 0, "an item row is whole 16-byte pieces");

// LDS: the activations and planes, the partial sums, one item area per wave.
template <int THREADS>
inline int64_t mma_tr_lds_bytes(int64_t N, int64_t nb) {
    return mma_lds_bytes<THREADS>(N, nb) + (THREADS / 64) * kTrWaveBytes;
}

// The contiguous-load kernel takes rows of 64 blocks or more in whole chunks
// of 8 (shorter rows leave most waves without a chunk) whose LDS fits.
constexpr int kTrThreads = 1024;
inline bool mma_tr_takes(int64_t N, int64_t nb) {
    return nb % kTrBlocks == 0 && nb >= 8 * kTrBlocks && mma_tr_lds_bytes<kTrThreads>(N, nb) <= kMmaMaxLds;
}

template <int THREADS, int D, int SRC, int LAY, bool EPI>
__global__ void __launch_bounds__(THREADS)
k_gemv_mma_tr(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const void* __restrict__ src, int N,
              float* __restrict__ Y, const MultiDesc md) {
    static_assert(SRC == kXF32 || SRC == kActGlobal, "activation source");
    constexpr bool RP = LAY == kLayRepacked;
    constexpr bool MULTI = LAY == kLayMulti;
    constexpr int kWaves = THREADS / 64;
    extern __shared__ __align__(16) uint8_t smem[];
    const MmaLds L = mma_lds<THREADS>(smem, N, nb);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    uint8_t* const wl = reinterpret_cast<uint8_t*>(L.part + 2 * kWaves * 4 * 64) + wave * kTrWaveBytes;
    const int nc = nb / kTrBlocks;                  // chunks per row
    const int cpw = (nc + kWaves - 1) / kWaves;     // chunks per wave and tile
    // this workgroup's 32-row tiles: blockIdx.x, blockIdx.x + G, ...
    const int64_t G = gridDim.x;
    const int64_t ntiles = (rows + 31) >> 5;
    const int64_t ntq = blockIdx.x < ntiles ? (ntiles - 1 - blockIdx.x) / G + 1 : 0;
    const int64_t nitems = ntq * cpw;               // the same for every wave
    const int64_t rowbytes = static_cast<int64_t>(nb) * kQ4Bytes;

    // this lane's pieces: byte offsets from the item's first byte in its
    // resource (past the item for the lanes with none: beyond any resource,
    // so their loads read nothing) and in the wave's LDS area
    uint32_t goff[kTrLoads];
    uint32_t loff[kTrLoads];
#pragma unroll
    for (int i = 0; i < kTrLoads; ++i) {
        const int p = i * 64 + lane;
        if constexpr (RP) {
            const int row = i + 1 < kTrLoads ? p >> 3 : lane, pc = i + 1 < kTrLoads ? p & 7 : 8;
            goff[i] = i + 1 < kTrLoads ? static_cast<uint32_t>(row * nb * 16 + pc * 16)
                                       : (lane < 32 ? static_cast<uint32_t>(row * nb * 2) : 0xFFFFFF00u);
            loff[i] = static_cast<uint32_t>(row * kTrStride + pc * 16);
        } else {
            const int row = p / kTrPieces, pc = p - row * kTrPieces;
            goff[i] = p < 32 * kTrPieces ? static_cast<uint32_t>(row * rowbytes + pc * 16) : 0xFFFFFF00u;
            loff[i] = static_cast<uint32_t>(row * kTrStride + pc * 16);
        }
    }

    // Item k: tile lr0 (its first row), chunk wave + W * lc, loaded in order
    // (counters, not divisions: a 64-bit division is some hundred scalar
    // instructions, and the waves of a SIMD share its scalar issue).
    // The loads go through a buffer resource spanning the tile's rows (zero
    // bytes past the wave's last item or for a chunk past the row), so they
    // stay unconditional and read nothing where there is nothing to read.  A
    // tile's bytes stay below 2^32.
    int64_t lr0 = static_cast<int64_t>(blockIdx.x) * 32;
    int lc = 0;
    auto load_item = [&](u32x4 (&dst)[kTrLoads], int64_t k) __attribute__((always_inline)) {
        const int c = wave + kWaves * lc;
        const int64_t r0 = lr0;
        if (++lc == cpw) {
            lc = 0;
            lr0 += G * 32;
        }
        const bool live = k < nitems && c < nc;
        const int64_t nr = live ? min(static_cast<int64_t>(32), rows - r0) : 0;  // rows of the tile to read
        if constexpr (RP) {
            // nibble plane: rows x nb x 16 bytes, then the scale plane: rows x nb x 2
            const uint8_t* nib = Wq + (nr > 0 ? r0 * nb * 16 + c * 128 : 0);
            const uint8_t* sc = Wq + rows * nb * 16 + (nr > 0 ? r0 * nb * 2 + c * 16 : 0);
            const auto rn = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(nib), static_cast<short>(0),
                                                               static_cast<int>(nr > 0 ? (nr - 1) * nb * 16 + 128 : 0),
                                                               kRsrcFlags);
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sc), static_cast<short>(0),
                                                               static_cast<int>(nr > 0 ? (nr - 1) * nb * 2 + 16 : 0),
                                                               kRsrcFlags);
#pragma unroll
            for (int i = 0; i + 1 < kTrLoads; ++i)
                dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rn, goff[i], 0, 0));
            dst[kTrLoads - 1] =
                __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, goff[kTrLoads - 1], 0, 0));
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
            const uint8_t* base = wb + (nr > 0 ? (r0 - f) * rowbytes + c * kTrRowBytes : 0);
            const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0),
                                                               static_cast<int>(nr > 0 ? (nr - 1) * rowbytes + kTrRowBytes : 0),
                                                               kRsrcFlags);
#pragma unroll
            for (int i = 0; i < kTrLoads; ++i)
                dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, goff[i], 0, 0));
        }
    };
    // the first D items, issued right behind the activations' loads
    u32x4 raw[D][kTrLoads];
    auto prefetch = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_item(raw[d], d);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    mma_stage_activations<THREADS, SRC>(src, N, nb, L, prefetch);

    if (nitems == 0) return;  // the whole workgroup: no rows

    // this lane's activation operand: token slot l & 7 (clamped to the N
    // tokens), 16-byte half h; lanes 8..15 of each 16-lane group read the
    // other half (their outputs are never used) so that 16 lanes touch 16
    // distinct bank groups
    const int a_tok = min(lane & 7, N - 1);
    const int a_half = h ^ ((lane >> 3) & 1);
    const uint8_t* a_base = L.a + a_tok * L.S + 16 * a_half;
    // this lane's row in the wave's LDS area
    const u32x4* rp = reinterpret_cast<const u32x4*>(wl + l32 * kTrStride);

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int buf = 0;
    int ci = 0;                                                    // chunk index within the tile
    int64_t r0 = static_cast<int64_t>(blockIdx.x) * 32;           // the tile's first row
    for (int64_t k = 0; k < nitems; k += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            // item k + d into the wave's LDS area, then its registers take the
            // load of item k + d + D at once (D items stay in flight while
            // this one is computed)
            const int c = wave + kWaves * ci;
            const bool work = k + d < nitems && c < nc;
            if (work) {
#pragma unroll
                for (int i = 0; i < kTrLoads; ++i)
                    if (i + 1 < kTrLoads || lane < 32 * kTrPieces - 64 * (kTrLoads - 1))
                        *reinterpret_cast<u32x4*>(wl + loff[i]) = raw[d][i];
            }
            load_item(raw[d], k + d + D);
            __builtin_amdgcn_sched_barrier(0);
            if (k + d < nitems) {
                if (work) {
                    __builtin_amdgcn_wave_barrier();
                    u32x4 scp = {0u, 0u, 0u, 0u};
                    if constexpr (RP) scp = rp[8];  // the eight scales
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        uint32_t w0[4], w1[4], dd[4];
                        // win: 20 dwords of the row (pieces 4g .. 4g + 4 of the
                        // pages' bytes, pieces 4g .. 4g + 3 of the nibbles); sel(k):
                        // dword k, or k + 2 in half h = 1 (8 bytes on)
                        uint32_t win[20];
#pragma unroll
                        for (int m = 0; m < (RP ? 4 : 5); ++m) {
                            const u32x4 v = rp[4 * g + m];
                            win[4 * m] = v.x; win[4 * m + 1] = v.y; win[4 * m + 2] = v.z; win[4 * m + 3] = v.w;
                        }
                        auto sel = [&](int k) __attribute__((always_inline)) { return h ? win[k + 2] : win[k]; };
                        if constexpr (RP) {
                            // block 4g + i: nibbles at dwords 4i .. 4i + 3 of win
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                w0[i] = sel(4 * i);
                                w1[i] = sel(4 * i + 1);
                            }
                            const uint32_t s01 = g ? scp.z : scp.x, s23 = g ? scp.w : scp.y;
                            dd[0] = s01 & 0xFFFFu; dd[1] = s01 >> 16; dd[2] = s23 & 0xFFFFu; dd[3] = s23 >> 16;
                        } else {
                            // block 4g + i at byte 72 g + 18 i of the row, dword
                            // 2g + 4.5 i of win (it starts at dword 16 g): scale
                            // first, nibbles 2 bytes on
                            const int o = 2 * g;
                            w0[0] = __builtin_amdgcn_alignbit(sel(o + 1), sel(o), 16);
                            w1[0] = __builtin_amdgcn_alignbit(sel(o + 2), sel(o + 1), 16);
                            w0[1] = sel(o + 5);
                            w1[1] = sel(o + 6);
                            w0[2] = __builtin_amdgcn_alignbit(sel(o + 10), sel(o + 9), 16);
                            w1[2] = __builtin_amdgcn_alignbit(sel(o + 11), sel(o + 10), 16);
                            w0[3] = sel(o + 14);
                            w1[3] = sel(o + 15);
                            dd[0] = win[o] & 0xFFFFu; dd[1] = win[o + 4] >> 16;
                            dd[2] = win[o + 9] & 0xFFFFu; dd[3] = win[o + 13] >> 16;
                        }
                        const int b0 = kTrBlocks * c + 4 * g;
                        const uint8_t* ab = a_base + b0 * kActQBytes;
                        const int pb = b0 * kMmaSlots + 4 * h;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            mma_block(L, ab + i * kActQBytes, pb + i * kMmaSlots, w0[i], w1[i], dd[i], acc);
                    }
                    __builtin_amdgcn_wave_barrier();
                }
                if (++ci == cpw) {
                    mma_put_partials<kWaves>(L, buf, wave, lane, acc);
                    lds_barrier();
                    mma_store_tile<kWaves, MULTI, EPI>(L, buf, r0, rows, N, Y, md);
                    buf ^= 1;
                    ci = 0;
                    r0 += G * 32;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The same product with whole tiles loaded contiguously (`k_gemv_mma_tile`:
// the pages' blocks, 64..128 blocks a row in whole chunks of 8, many tiles
// per workgroup).  A tile's 32 rows are one contiguous run of 32 * 18 nb
// bytes: thread t of the workgroup loads its 16-byte pieces t, t + 1024, ...
// with non-temporal loads (each instruction of a wave one contiguous 1 KB,
// every cache line whole),
// and the workgroup writes them into one LDS tile whose rows are TS bytes
// apart (TS / 16 odd: the 16-byte reads of 16 consecutive rows hit 16
// distinct bank groups).  After a barrier every wave reads its chunks
// (32 rows x 144 bytes) from there, as `k_gemv_mma_tr` reads its own item,
// while the next tiles' loads are in flight (D tiles per workgroup); a
// second barrier, after the partial sums, frees the tile for the next one.
// Same chunks per wave, same steps in the same order: the same bits as
// `k_gemv_mma_tr`.  Measured (graph-timed, workspace form): the vocabulary
// head at N = 5 / 8 61.8 / 63.5 -> 61.2 / 62.6 us with plain loads, another
// 5 % off with non-temporal ones (59.9 / 61.4 -> 57.0 / 57.9 us in one run);
// 66000 x 3072 at N = 8 31.6 -> 27.5 us.  Without the matrix-core work the
// head takes 52 us, with or without the barriers: the loads set the floor.
constexpr int kNonTemporal = 2;  // buffer load cache policy: nt (whole lines streamed once)
constexpr int kTlThreads = 1024;
constexpr int kTlMaxBlocks = 128;
constexpr int kTlLoads = (36 * kTlMaxBlocks + kTlThreads - 1) / kTlThreads;  // 5: a tile is 36 nb pieces
__host__ __device__ inline int64_t mma_tile_stride(int64_t nb) {
    const int64_t p = nb * kQ4Bytes / 16;  // pieces a row
    return 16 * (p + 1 + (p & 1));
}
template <int THREADS>
inline int64_t mma_tile_lds_bytes(int64_t N, int64_t nb) {
    return mma_lds_bytes<THREADS>(N, nb) + 32 * mma_tile_stride(nb);
}
// Many tiles per workgroup (the pipeline fills), rows of 64..128 blocks.
inline bool mma_tile_takes(int64_t N, int64_t nb, int64_t ntiles, int64_t grid) {
    return nb % kTrBlocks == 0 && nb >= 8 * kTrBlocks && nb <= kTlMaxBlocks && ntiles >= 8 * grid &&
           mma_tile_lds_bytes<kTlThreads>(N, nb) <= kMmaMaxLds;
}

template <int THREADS, int D, int SRC, int LAY, bool EPI>
__global__ void __launch_bounds__(THREADS)
k_gemv_mma_tile(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const void* __restrict__ src, int N,
                float* __restrict__ Y, const MultiDesc md) {
    static_assert(SRC == kXF32 || SRC == kActGlobal, "activation source");
    static_assert(LAY == kLayAoS || LAY == kLayMulti, "the pages' blocks");
    static_assert(THREADS == kTlThreads, "a tile's pieces per thread");
    constexpr bool MULTI = LAY == kLayMulti;
    constexpr int kWaves = THREADS / 64;
    extern __shared__ __align__(16) uint8_t smem[];
    const MmaLds L = mma_lds<THREADS>(smem, N, nb);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int TS = static_cast<int>(mma_tile_stride(nb));
    uint8_t* const tile = reinterpret_cast<uint8_t*>(L.part + 2 * kWaves * 4 * 64);
    const int nc = nb / kTrBlocks;  // chunks per row
    const int64_t G = gridDim.x;
    const int64_t ntiles = (rows + 31) >> 5;
    const int64_t ntq = blockIdx.x < ntiles ? (ntiles - 1 - blockIdx.x) / G + 1 : 0;
    const int rowbytes = nb * kQ4Bytes;
    const int tpieces = 2 * rowbytes;  // 32 rows of rowbytes / 16 pieces

    // this thread's pieces of a tile: byte offset in the tile's run (loads
    // past the tile read nothing) and in the LDS tile
    uint32_t loff[kTlLoads];
#pragma unroll
    for (int i = 0; i < kTlLoads; ++i) {
        const int p = static_cast<int>(threadIdx.x) + THREADS * i;
        const int row = p / (rowbytes / 16), pc = p - row * (rowbytes / 16);
        loff[i] = static_cast<uint32_t>(row * TS + pc * 16);
    }
    // tile k of this workgroup into dst (a buffer resource over the tile's
    // rows: zero bytes past the last row, or for k >= ntq)
    auto load_tile = [&](u32x4 (&dst)[kTlLoads], int64_t k) __attribute__((always_inline)) {
        const int64_t r0 = (static_cast<int64_t>(blockIdx.x) + k * G) * 32;
        const int64_t nr = k < ntq ? min(static_cast<int64_t>(32), rows - r0) : 0;
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
        const uint8_t* base = wb + (nr > 0 ? (r0 - f) * rowbytes : 0);
        const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0),
                                                           static_cast<int>(nr * rowbytes), kRsrcFlags);
#pragma unroll
        for (int i = 0; i < kTlLoads; ++i)
            dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rw, 16 * (static_cast<int>(threadIdx.x) + THREADS * i), 0,
                                                   kNonTemporal));
    };
    u32x4 raw[D][kTlLoads];
    auto prefetch = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_tile(raw[d], d);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    mma_stage_activations<THREADS, SRC>(src, N, nb, L, prefetch);

    if (ntq == 0) return;  // the whole workgroup: no rows

    const int a_tok = min(lane & 7, N - 1);
    const int a_half = h ^ ((lane >> 3) & 1);
    const uint8_t* a_base = L.a + a_tok * L.S + 16 * a_half;

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int buf = 0;
    for (int64_t k = 0; k < ntq; k += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (k + d >= ntq) break;  // (uniform)
            // tile k + d into LDS, then its registers take tile k + d + D
#pragma unroll
            for (int i = 0; i < kTlLoads; ++i)
                if (static_cast<int>(threadIdx.x) + THREADS * i < tpieces)
                    *reinterpret_cast<u32x4*>(tile + loff[i]) = raw[d][i];
            lds_barrier();
            load_tile(raw[d], k + d + D);
            __builtin_amdgcn_sched_barrier(0);
            for (int c = wave; c < nc; c += kWaves) {
                const u32x4* rp = reinterpret_cast<const u32x4*>(tile + l32 * TS + c * kTrRowBytes);
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    uint32_t w0[4], w1[4], dd[4];
                    uint32_t win[20];
#pragma unroll
                    for (int m = 0; m < 5; ++m) {
                        const u32x4 v = rp[4 * g + m];
                        win[4 * m] = v.x; win[4 * m + 1] = v.y; win[4 * m + 2] = v.z; win[4 * m + 3] = v.w;
                    }
                    auto sel = [&](int q) __attribute__((always_inline)) { return h ? win[q + 2] : win[q]; };
                    const int o = 2 * g;
                    w0[0] = __builtin_amdgcn_alignbit(sel(o + 1), sel(o), 16);
                    w1[0] = __builtin_amdgcn_alignbit(sel(o + 2), sel(o + 1), 16);
                    w0[1] = sel(o + 5);
                    w1[1] = sel(o + 6);
                    w0[2] = __builtin_amdgcn_alignbit(sel(o + 10), sel(o + 9), 16);
                    w1[2] = __builtin_amdgcn_alignbit(sel(o + 11), sel(o + 10), 16);
                    w0[3] = sel(o + 14);
                    w1[3] = sel(o + 15);
                    dd[0] = win[o] & 0xFFFFu; dd[1] = win[o + 4] >> 16;
                    dd[2] = win[o + 9] & 0xFFFFu; dd[3] = win[o + 13] >> 16;
                    const int b0 = kTrBlocks * c + 4 * g;
                    const uint8_t* ab = a_base + b0 * kActQBytes;
                    const int pb = b0 * kMmaSlots + 4 * h;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        mma_block(L, ab + i * kActQBytes, pb + i * kMmaSlots, w0[i], w1[i], dd[i], acc);
                }
            }
            mma_put_partials<kWaves>(L, buf, wave, lane, acc);
            lds_barrier();
            mma_store_tile<kWaves, MULTI, EPI>(L, buf, (static_cast<int64_t>(blockIdx.x) + (k + d) * G) * 32, rows,
                                               N, Y, md);
            buf ^= 1;
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
    // longest matrices the row kernel streams at nearly full rate up to three
    // tokens, up to six against the lane-load kernel, and up to four where it
    // loads whole rows contiguously (one pair per lane, 16 rows per wave on a
    // full chip: the vocabulary head at N = 4 58.5 us against 61.2 on the
    // contiguous-load matrix-core kernel, 66000 x 3072 30.4 against 31.1);
    // fewer rows leave CUs idle (one workgroup per 32 rows), longer rows put
    // most of the time into the per-workgroup activation copy
    if (N > kGemvMaxN || nb % 2 != 0 || nb > kMmaMaxBlocks || rows < kMmaMinRows) return false;
    if (mma_lds_bytes<kMmaThreads>(N, nb) > kMmaMaxLds) return false;
    const bool rows_contiguous = rows >= kMmaRowsContiguousRows && rows_fuse_prologue(nb, rows) && (nb / 2) % 4 == 0;
    const int64_t min_n = rows < kMmaLongRows ? kMmaMinN
                          : mma_tr_takes(N, nb) ? (rows_contiguous ? kMmaMinN : kMmaLongMinN)
                                                : kMmaLongMinNPairs;
    return N >= min_n;
}

namespace {

template <int SRC, int LAY, bool EPI>
hipError_t launch_mma_k(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                        int64_t N, float* Y, const MultiDesc& md, hipStream_t s) {
    const int64_t ntiles = (rows + 31) / 32;
    const int64_t grid = ntiles < dev->num_cu ? ntiles : dev->num_cu;
    {
        if constexpr (LAY != kLayRepacked) {
            if (mma_tile_takes(N, nb, ntiles, grid)) {
                constexpr int kTlD = 1;  // tiles in flight per workgroup (two: 1-3 % slower)
                const size_t lds = static_cast<size_t>(mma_tile_lds_bytes<kTlThreads>(N, nb));
                const auto kernel = k_gemv_mma_tile<kTlThreads, kTlD, SRC, LAY, EPI>;
                const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                              hipFuncAttributeMaxDynamicSharedMemorySize, kMmaMaxLds);
                if (raised != hipSuccess) return raised;
                hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(grid)), dim3(kTlThreads), lds, s, Wq, rows,
                                   static_cast<int>(nb), src, static_cast<int>(N), Y, md);
                return hipGetLastError();
            }
        }
        if (mma_tr_takes(N, nb)) {
            constexpr int kTrD = 2;  // items in flight per wave
            const size_t lds = static_cast<size_t>(mma_tr_lds_bytes<kTrThreads>(N, nb));
            const auto kernel = k_gemv_mma_tr<kTrThreads, kTrD, SRC, LAY, EPI>;
            const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                          hipFuncAttributeMaxDynamicSharedMemorySize, kMmaMaxLds);
            if (raised != hipSuccess) return raised;
            hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(grid)), dim3(kTrThreads), lds, s, Wq, rows,
                               static_cast<int>(nb), src, static_cast<int>(N), Y, md);
            return hipGetLastError();
        }
    }
    // items in flight per wave: four where every workgroup has 16 tiles or
    // more (the vocabulary head), else two (measured: 14336 x 4096 at N = 8,
    // 13.7 -> 11.9 us)
    const auto kernel = ntiles >= 16 * grid ? k_gemv_mma<kMmaThreads, 4, SRC, LAY, EPI>
                                            : k_gemv_mma<kMmaThreads, 2, SRC, LAY, EPI>;
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
    // the multi-matrix form stores plain products (no epilogue)
    const bool epi = lay != kLayMulti && (md.epi.bias != nullptr || md.epi.mul != nullptr);
    if (src_f32) {
        switch (lay) {
            case kLayRepacked:
                return epi ? launch_mma_k<kXF32, kLayRepacked, true>(dev, Wq, rows, nb, src, N, Y, md, s)
                           : launch_mma_k<kXF32, kLayRepacked, false>(dev, Wq, rows, nb, src, N, Y, md, s);
            case kLayMulti: return launch_mma_k<kXF32, kLayMulti, false>(dev, Wq, rows, nb, src, N, Y, md, s);
            default:
                return epi ? launch_mma_k<kXF32, kLayAoS, true>(dev, Wq, rows, nb, src, N, Y, md, s)
                           : launch_mma_k<kXF32, kLayAoS, false>(dev, Wq, rows, nb, src, N, Y, md, s);
        }
    }
    switch (lay) {
        case kLayRepacked:
            return epi ? launch_mma_k<kActGlobal, kLayRepacked, true>(dev, Wq, rows, nb, src, N, Y, md, s)
                       : launch_mma_k<kActGlobal, kLayRepacked, false>(dev, Wq, rows, nb, src, N, Y, md, s);
        case kLayMulti: return launch_mma_k<kActGlobal, kLayMulti, false>(dev, Wq, rows, nb, src, N, Y, md, s);
        default:
            return epi ? launch_mma_k<kActGlobal, kLayAoS, true>(dev, Wq, rows, nb, src, N, Y, md, s)
                       : launch_mma_k<kActGlobal, kLayAoS, false>(dev, Wq, rows, nb, src, N, Y, md, s);
    }
}

}  // namespace q4bq
