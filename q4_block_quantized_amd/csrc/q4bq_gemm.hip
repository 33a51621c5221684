// Prefill product on the matrix cores, N > 8 tokens.
//
// Same arithmetic as the decode kernel ("llama.cpp 深度解读", luoboask.github.io,
// section 3 "量化矩阵乘法 — 核心算子": per 32-value block the integer dot of
// (nibble - 8) with the int8 activations, then the fp32 scale d_w * d_x, the
// scaled block terms summed in fp32), organised as a tiled GEMM:
//  * the block dot runs on the fp6 matrix cores, exactly: the weights enter as
//    e2m3 codes of (nibble - 8)/8, the activations as e2m3 codes of h/2 and l/2
//    (y = 16h + l), with E8M0 block scales x8, x32 and x2; one
//    v_mfma_scale_f32_32x32x64_f8f6f4 yields s for a 32-token x 32-row tile
//    as an exact fp32 integer, with no int->float conversion;
//  * the 1024 scale products d_x * d_w of a tile come from one
//    v_mfma_f32_32x32x8_f16 outer product (binary16 x binary16 is exact in
//    fp32), so each (token, row, block) costs a single FMA on the vector ALU;
//  * an fp6 operand occupies 6 of the 8 dwords that two 16-byte LDS reads
//    fetch; the 7th carries the block's binary16 scale bits and the 8th is
//    zero, so the same two reads also deliver the scale-product operand;
//  * the activation records go from global memory straight into LDS
//    (global_load_lds, no registers); the weights are read as raw 18-byte
//    blocks (or, after q4_0_repack, as aligned nibble blocks plus a scale
//    stream) and turned into fp6 codes while they are staged into LDS;
//  * LDS is double-buffered: while one stage (4 blocks of K) is computed, the
//    next stage's activations stream in and its weights are converted, with
//    one barrier per stage.
// Workgroup tile 256 tokens x 128 rows, 8 waves of 64 x 64 (2 x 2 MFMA tiles).
// LDS: 2 x (64 KB activations + 16 KB weights) = 160 KB.
#include <type_traits>

#include "q4bq_device.h"
#include "q4bq_internal.h"

namespace q4bq {

namespace {

constexpr int kWavesT = 4;                 // waves along tokens
constexpr int kWavesR = 2;                 // waves along rows
constexpr int kThreads = 64 * kWavesT * kWavesR;
constexpr int kBT = 64 * kWavesT;          // tokens per workgroup tile
constexpr int kBR = 64 * kWavesR;          // rows per workgroup tile
constexpr int kKB = 4;                     // blocks per stage
constexpr int kRecB = 32;                  // LDS bytes per (row, block): 24 bytes of codes, scale, zero
constexpr int kPlaneA = kBT * kAct6Bytes;  // one block of the token tile
constexpr int kPlaneB = kBR * kRecB;       // one block of the row tile
constexpr int kBufA = kKB * kPlaneA;
constexpr int kBufB = kKB * kPlaneB;
// global_load_lds moves 16 bytes per lane: one instruction fills 16 tokens of
// one block plane, so each wave issues kDma of them per stage.
constexpr int kDma = kKB * kBT * (kAct6Bytes / 16) / kThreads;
static_assert(kDma == 8, "activation staging: 2 instructions per block plane per wave");
static_assert(kBR * kKB == kThreads, "one weight block per thread per stage");
static_assert(2 * kBufA + 2 * kBufB <= 160 * 1024, "LDS budget");

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// E8M0 block scales: 127 is x1.
constexpr int kScaleW = 130;       // weights hold (nibble - 8) / 8
constexpr int kScaleHi = 127 + 5;  // activation high part holds h / 2, weight 16 h
constexpr int kScaleLo = 128;      // activation low part holds l / 2
// Both K halves of the scale-product MFMA hold d in their first slot, so it
// returns 2 * d_x * d_w; the block dot is taken 2 times smaller to match
// (exact: a power of two on an integer well inside the fp32 range).
constexpr int kScaleDown = 1;

// One operand record in registers: fp6 codes in dwords 0..5, {scale bits, 0}
// in dwords 6..7, read as two 16-byte halves that are only joined at use.
struct Operand {
    u32x4 lo;
    u32x4 hi;
};

__device__ __forceinline__ Operand lds_operand(const uint8_t* p0, const uint8_t* p1) {
    Operand o;
    o.lo = *reinterpret_cast<const u32x4*>(p0);
    o.hi = *reinterpret_cast<const u32x4*>(p1);
    return o;
}

__device__ __forceinline__ i32x8 fp6_operand(const Operand& o) {
    return i32x8{static_cast<int>(o.lo.x), static_cast<int>(o.lo.y), static_cast<int>(o.lo.z),
                 static_cast<int>(o.lo.w), static_cast<int>(o.hi.x), static_cast<int>(o.hi.y),
                 static_cast<int>(o.hi.z), static_cast<int>(o.hi.w)};
}

__device__ __forceinline__ f16x4 scale_operand(const Operand& o) {
    return __builtin_bit_cast(f16x4, u32x2{o.hi.z, o.hi.w});
}

// global_load_lds_dwordx4: 16 bytes per lane from src into LDS at dst + 16 *
// lane (dst wave-uniform, through M0).  Written as inline assembly so that
// the compiler does not track it: it would otherwise wait for these loads
// before unrelated LDS reads.  The caller waits for them explicitly
// (s_waitcnt vmcnt) before the data is read; loads complete in order, and
// every load the compiler does track that is issued later is waited for with
// a count that then also covers these.
__device__ __forceinline__ void dma16(const uint8_t* src, const uint8_t* dst) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)dst)));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds), "v"(src) : "memory", "m0");
}

template <bool DOTS, bool RP>
__global__ void __launch_bounds__(kThreads)
k_gemm(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const uint8_t* __restrict__ act, int64_t N,
       float* __restrict__ Y, int32_t* __restrict__ D) {
    __shared__ __align__(16) uint8_t sA0[kBufA];
    __shared__ __align__(16) uint8_t sA1[kBufA];
    __shared__ __align__(16) uint8_t sB0[kBufB];
    __shared__ __align__(16) uint8_t sB1[kBufB];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave / kWavesR;  // token slice of the tile
    const int wn = wave % kWavesR;  // row slice of the tile
    const int l32 = lane & 31;
    const int half = lane >> 5;
    // Token tile fastest: workgroups are dealt to the 8 XCDs round-robin, so
    // with 2, 4 or 8 token tiles each XCD only ever sees 1/2, 1/4 or 1/8 of
    // the activations, which then stay in its L2 while the weights stream.
    const int64_t ntt = (N + kBT - 1) / kBT;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x / ntt) * kBR;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x % ntt) * kBT;
    const int nst = (nb + kKB - 1) / kKB;

    // --- activation staging -------------------------------------------------
    // Records are [block][token][64 bytes]; in LDS, 16-byte quarter q of
    // token t sits at position q ^ ((t >> 2) & 3) of its record: a 16-byte
    // LDS read serves 16 lanes per cycle from 64 banks, and with this swizzle
    // the 16 tokens of such a group hit 16 disjoint 4-bank groups.
    // Instruction e of a block plane covers tokens wave*32 + 16e + lane/4;
    // lane position lane%4 holds quarter (lane%4) ^ ((lane/16)%4).
    const int dq = (lane & 3) ^ ((lane >> 4) & 3);
    int64_t dma_off[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        int64_t tok = n0 + wave * 32 + e * 16 + (lane >> 2);
        if (tok > N - 1) tok = N - 1;  // padding tokens: any valid record, never stored
        dma_off[e] = tok * kAct6Bytes + dq * 16;
    }
    auto issue_dma = [&](int b0, uint8_t* sA) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kDma; ++i) {
            const int blk = i >> 1, e = i & 1;
            int b = b0 + blk;
            if (b > nb - 1) b = nb - 1;  // past the end: neutralised by zero weight scales
            const uint8_t* src = act + static_cast<int64_t>(b) * N * kAct6Bytes + dma_off[e];
            const uint8_t* dst = sA + blk * kPlaneA + (wave * 32 + e * 16) * kAct6Bytes;
            dma16(src, dst);
        }
    };

    // --- weight staging: one block per thread, row w_row, block w_blk ---------
    // LDS record (32 bytes): 6 dwords of fp6 codes, binary16 d bits, zero; the
    // two 16-byte halves swap places in rows with bit 3 set, so that 16
    // consecutive rows (one LDS cycle of reads or writes) hit 16 disjoint
    // 4-bank groups.  A wave stages 16 rows x 4 blocks; each 16-lane group
    // holds one block of the 16 rows.
    const int w_row = (t & 15) | ((t >> 6) << 4);
    const int w_blk = (t >> 4) & 3;
    const bool w_row_ok = r0 + w_row < rows;
    // RP: Wq holds the repacked streams (16 nibble bytes per block, then the scales)
    const int64_t w_row_first = (r0 + (w_row_ok ? w_row : 0)) * nb;  // block index of the row's first block
    const uint8_t* w_src = Wq + w_row_first * (RP ? 16 : kQ4Bytes);
    const uint8_t* w_sc = Wq + (RP ? rows * nb * 16 + w_row_first * 2 : 0);
    const int w_swap = (w_row >> 3) & 1;
    const int w_dst = w_blk * kPlaneB + w_row * kRecB;
    // Raw blocks are loaded two stages ahead into one of two register sets:
    // set t % 2 holds stage t (the global loads hide behind two stages of
    // matrix work).
    Block4 rw[2];
    bool rw_ok[2] = {false, false};
    // The loads are issued unconditionally (from a valid block when the wanted
    // one is past the end) so that the code around them stays branch-free and
    // the compiler can count outstanding loads exactly.
    auto load_w = [&](int st, auto set) __attribute__((always_inline)) {
        constexpr int S = decltype(set)::value;
        const int b0 = st * kKB;
        rw_ok[S] = w_row_ok && st < nst && (b0 + w_blk < nb);
        const int64_t bo = rw_ok[S] ? b0 + w_blk : 0;  // else block 0 of a valid row
        rw[S] = RP ? load_block_rp(w_src + bo * 16, w_sc + bo * 2) : load_block(w_src + bo * kQ4Bytes);
    };
    auto store_w = [&](uint8_t* sB, auto set) __attribute__((always_inline)) {
        constexpr int S = decltype(set)::value;
        uint32_t d6[6] = {0u, 0u, 0u, 0u, 0u, 0u};
        uint32_t dbits = 0u;  // zero scale: the block contributes nothing
        if (rw_ok[S]) {
            weight_fp6(rw[S].qs, d6);
            dbits = rw[S].dbits;
        }
        uint8_t* p = sB + w_dst;
        *reinterpret_cast<u32x4*>(p + 16 * w_swap) = u32x4{d6[0], d6[1], d6[2], d6[3]};
        *reinterpret_cast<u32x4*>(p + 16 * (w_swap ^ 1)) = u32x4{d6[4], d6[5], dbits, 0u};
    };

    // --- operand reads --------------------------------------------------------
    const int a_sw = (l32 >> 2) & 3;
    const int a_row = (wm * 64 + l32) * kAct6Bytes;
    const int a_p0 = a_row + 16 * ((2 * half) ^ a_sw);
    const int a_p1 = a_row + 16 * ((2 * half + 1) ^ a_sw);
    const int b_sw = (l32 >> 3) & 1;
    const int b_row = (wn * 64 + l32) * kRecB;
    const int b_p0 = b_row + 16 * b_sw;
    const int b_p1 = b_row + 16 * (b_sw ^ 1);

    f32x16 acc[4];  // tile k = (token half i = k / 2, row half j = k % 2)
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[k][v] = 0.0f;
    const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // software pipeline: each tile's scaled fold waits one tile, so it runs
    // while the next tile's two matrix instructions execute (a first fold of
    // 0 * 0 into acc[3] is harmless)
    f32x16 s_prev = zero, p_prev = zero;
    const int scale_a = (half ? kScaleLo : kScaleHi) - (DOTS ? 0 : kScaleDown);

    // Operands of block plane `blk` (wrapping, so that a read past the last
    // plane is a harmless re-read of plane 0).  The two 16-byte halves are
    // kept apart until use, so that no register copy forces an early wait.
    auto read_ops = [&](const uint8_t* sA, const uint8_t* sB, int blk, Operand* a, Operand* w)
                        __attribute__((always_inline)) {
        const uint8_t* pa = sA + (blk & (kKB - 1)) * kPlaneA;
        const uint8_t* pb = sB + (blk & (kKB - 1)) * kPlaneB;
#pragma unroll
        for (int i = 0; i < 2; ++i) a[i] = lds_operand(pa + a_p0 + i * 32 * kAct6Bytes, pa + a_p1 + i * 32 * kAct6Bytes);
#pragma unroll
        for (int j = 0; j < 2; ++j) w[j] = lds_operand(pb + b_p0 + j * 32 * kRecB, pb + b_p1 + j * 32 * kRecB);
    };
    // The four 32 x 32 tiles of one block.
    auto tiles = [&](const Operand* a, const Operand* w, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = k >> 1, j = k & 1;
            const f32x16 sk = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fp6_operand(a[i]), fp6_operand(w[j]), zero, 2, 2, 0, scale_a, 0, kScaleW);
            if constexpr (DOTS) {
                const int64_t r = r0 + wn * 64 + j * 32 + l32;
                if (b < nb && r < rows) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int64_t n = n0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                        if (n < N) D[(n * rows + r) * nb + b] = static_cast<int32_t>(sk[v]);
                    }
                }
            } else {
                const f32x16 pk =
                    __builtin_amdgcn_mfma_f32_32x32x8f16(scale_operand(a[i]), scale_operand(w[j]), zero, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[(k + 3) & 3][v] = fmaf(s_prev[v], p_prev[v], acc[(k + 3) & 3][v]);
                s_prev = sk;
                p_prev = pk;
            }
        }
    };
    // One stage of kKB blocks; the next block's operands are read while the
    // current block computes (two register sets, ping-pong).
    auto compute = [&](const uint8_t* sA, const uint8_t* sB, int b0) __attribute__((always_inline)) {
        Operand a0[2], w0[2], a1[2], w1[2];
        read_ops(sA, sB, 0, a0, w0);
#pragma unroll 1
        for (int blk = 0; blk < kKB; blk += 2) {
            read_ops(sA, sB, blk + 1, a1, w1);
            tiles(a0, w0, b0 + blk);
            read_ops(sA, sB, blk + 2, a0, w0);
            tiles(a1, w1, b0 + blk + 1);
        }
    };

    // Weight conversion is split between the two waves that share a SIMD
    // (waves w and w + 4): waves 4-7 convert the next stage's weights when a
    // stage starts, waves 0-3 when it ends.  One wave of each pair then keeps
    // the matrix core busy while the other spends its vector ALU on the
    // conversion.
    const bool late = (wave >> 2) == 0;

    // One stage: prefetch stage s + 1 into the other buffers, compute stage s.
    auto stage = [&](auto bufsel, int s) __attribute__((always_inline)) {
        constexpr int X = decltype(bufsel)::value;
        constexpr std::integral_constant<int, X> cur{};
        constexpr std::integral_constant<int, X ^ 1> nxt{};
        uint8_t* sA = X ? sA1 : sA0;
        uint8_t* sB = X ? sB1 : sB0;
        uint8_t* sA_next = X ? sA0 : sA1;
        uint8_t* sB_next = X ? sB0 : sB1;
        const bool more = s + 1 < nst;
        if (!late && more) store_w(sB_next, nxt);  // stage s + 1
        issue_dma((s + 1) * kKB, sA_next);        // past the end: harmless, never read
        // The raw weights of stage s + 2 go out after the activation loads
        // (loads complete in order): the barrier below then waits for the
        // activations only and leaves these two loads in flight.
        __builtin_amdgcn_sched_barrier(0);
        load_w(s + 2, cur);  // set X held stage s, already converted
        __builtin_amdgcn_sched_barrier(0);
        compute(sA, sB, s * kKB);
        if (late && more) store_w(sB_next, nxt);
        // vmcnt <= 2 (activation DMA landed in LDS), lgkmcnt = 0 (weight
        // records written), expcnt unconstrained
        __builtin_amdgcn_s_waitcnt(0x0072);
        __builtin_amdgcn_s_barrier();
    };

    load_w(0, std::integral_constant<int, 0>{});
    load_w(1, std::integral_constant<int, 1>{});
    issue_dma(0, sA0);
    store_w(sB0, std::integral_constant<int, 0>{});
    __syncthreads();
    for (int s = 0; s < nst; s += 2) {
        stage(std::integral_constant<int, 0>{}, s);
        if (s + 1 < nst) stage(std::integral_constant<int, 1>{}, s + 1);
    }

    if constexpr (!DOTS) {
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[3][v] = fmaf(s_prev[v], p_prev[v], acc[3][v]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = k >> 1, j = k & 1;
            const int64_t r = r0 + wn * 64 + j * 32 + l32;
            if (r >= rows) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t n = n0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                if (n < N) Y[n * rows + r] = acc[k][v];
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                       const void* act, int64_t N, float* Y, int32_t* D, hipStream_t s) {
    (void)dev;
    const uint8_t* rec = static_cast<const uint8_t*>(act);
    const dim3 grid(static_cast<uint32_t>(((rows + kBR - 1) / kBR) * ((N + kBT - 1) / kBT)));
    const int nbi = static_cast<int>(nb);
    if (D)
        hipLaunchKernelGGL((k_gemm<true, false>), grid, dim3(kThreads), 0, s, Wq, rows, nbi, rec, N, Y, D);
    else if (lay == kRepacked)
        hipLaunchKernelGGL((k_gemm<false, true>), grid, dim3(kThreads), 0, s, Wq, rows, nbi, rec, N, Y, D);
    else
        hipLaunchKernelGGL((k_gemm<false, false>), grid, dim3(kThreads), 0, s, Wq, rows, nbi, rec, N, Y, D);
    return hipGetLastError();
}

}  // namespace q4bq
