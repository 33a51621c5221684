// Prefill product on the matrix cores, N > 8 tokens: compute waves and staging
// waves.
//
// Same arithmetic as the decode kernels ("llama.cpp 深度解读", luoboask.github.io,
// section 3 "量化矩阵乘法 — 核心算子": per 32-value block the integer dot of
// (nibble - 8) with the int8 activations, then the fp32 scale d_w * d_x, the
// scaled block terms summed in fp32), organised as a tiled GEMM:
//  * the block dot runs on the fp6 matrix cores, exactly: the weights enter as
//    e2m3 codes of (nibble - 8)/8, the activations as e2m3 codes of h/2 and l/2
//    (y = 16h + l), with E8M0 block scales; one
//    v_mfma_scale_f32_32x32x64_f8f6f4 yields s for a 32-token x 32-row tile as
//    an exact fp32 integer;
//  * the 1024 scale products d_x * d_w of a tile come from one
//    v_mfma_f32_32x32x8_f16 outer product (binary16 x binary16 is exact in
//    fp32), so each (token, row, block) costs one FMA on the vector ALU;
//  * an fp6 operand occupies 6 of the 8 dwords that two 16-byte LDS reads
//    fetch; the 7th carries the block's binary16 scale bits and the 8th is
//    zero, so the same two reads also deliver the scale-product operand;
//  * LDS layouts are swizzled so that a 16-byte read or write serves 16 lanes
//    per cycle from 64 banks without conflicts: activation records
//    ([block][token][64 bytes], from the quantizer) keep 16-byte quarter q of
//    token t at position q ^ ((t >> 2) & 3); weight records (32 bytes per
//    (row, block): 6 dwords of codes, d bits, zero) swap their two halves in
//    rows where bit 2 xor bit 3 is set, which keeps both the 16-lane reads
//    and the staging waves' 16-byte writes (8 lanes per cycle over 32 banks)
//    free of conflicts.
//
// Shape: a workgroup computes 128 tokens x 224 rows.  224 = 7 x 32 makes
// 14336-row matrices split into 64 row tiles, so the 512-token prefill is 256
// workgroups: every CU gets one.  Eight waves, two per SIMD:
//  * waves 0-3 compute: each owns seven of the 28 tiles of 32 tokens x 32
//    rows -- two token tiles against three row tiles, plus one more tile --
//    so that every weight operand read from LDS serves two tiles (fewer
//    reads to issue and to wait for); a wave holds its 7
//    accumulator tiles (112 registers) and runs a software pipeline over its
//    tile steps -- the two matrix instructions of step k are issued around the
//    16 FMAs that drain step k - 1, so the matrix core and the vector ALU work
//    side by side;
//  * waves 4-7 stage: activation records go from global memory straight into
//    LDS (global_load_lds), Q4_0 blocks are loaded into registers and
//    converted into fp6 weight records, ahead of the compute.
// LDS: a ring of 4 stages x (16 KB activations + 14 KB weights) of 2 blocks;
// one workgroup barrier per stage hands a stage from the staging waves to the
// compute waves.
#include "q4bq_device.h"
#include "q4bq_internal.h"

namespace q4bq {

namespace {

constexpr int kCW = 4;                     // compute waves (one per SIMD)
constexpr int kT = 64 * 2 * kCW;           // threads: compute + staging waves
constexpr int kTT = 32 * kCW;              // tokens per workgroup tile
constexpr int kRT = 7;                     // 32-row tiles per workgroup tile
constexpr int kTR = 32 * kRT;              // rows per workgroup tile
constexpr int kKB = 2;                     // blocks per stage
constexpr int kNS = 4;                     // stages in the LDS ring
constexpr int kRecW = 32;                  // LDS bytes per (row, block)
constexpr int kPlaneA = kTT * kAct6Bytes;  // one block of the token tile (8 KB)
constexpr int kPlaneB = kTR * kRecW;       // one block of the row tile (7 KB)
constexpr int kBufA = kKB * kPlaneA;
constexpr int kBufB = kKB * kPlaneB;
constexpr int kStage = kBufA + kBufB;
constexpr int kST = kT / 2;  // staging threads
// global_load_lds moves 16 bytes per lane: one instruction fills 16 tokens of
// one block plane; staging wave sw moves tokens 32sw..32sw+31 of each plane.
constexpr int kDma = kKB * 2;
static_assert(kNS * kStage <= 160 * 1024, "LDS budget");
static_assert(kDma * kCW * 16 == kKB * kTT, "activation staging covers the planes");
static_assert(kTR <= kST, "one weight row per staging thread");
static_assert(kT == kPrefillThreads && kTT == kPrefillTokens && kTR == kPrefillRows,
              "launch geometry the argument checks bound");

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// E8M0 block scales: 127 is x1.
constexpr int kScaleW = 130;       // weights hold (nibble - 8) / 8
constexpr int kScaleHi = 127 + 5;  // activation high part holds h / 2, weight 16 h
constexpr int kScaleLo = 128;      // activation low part holds l / 2
// Both K halves of the scale-product instruction hold d in their first slot,
// so it returns 2 * d_x * d_w; the block dot is taken 2 times smaller to match.
constexpr int kScaleDown = 1;

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
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds), "v"(src) : "memory", "m0");
}

// LDS writes done, at most `vm` global loads still in flight (vmcnt(vm),
// lgkmcnt(0)), then the workgroup barrier.
template <int vm>
__device__ __forceinline__ void stage_barrier() {
    static_assert(vm >= 0 && vm < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((vm & 0xF) | ((vm >> 4) << 14) | 0x0070);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroups are dealt to the 8 XCDs round-robin (workgroup x runs on XCD
// x % 8), and each XCD has its own L2.  Tile order puts the token tiles of one
// row tile next to each other; this map gives every XCD a contiguous range of
// tiles, so the token tiles that read the same weights share one L2.
__device__ __forceinline__ int64_t xcd_tile(uint32_t x, uint32_t grid) {
    constexpr uint32_t kXcd = 8;
    const uint32_t q = grid / kXcd, rem = grid % kXcd, j = x % kXcd;
    return static_cast<int64_t>(j * q + (j < rem ? j : rem) + x / kXcd);
}

// One tile step of the product: the block dot and the scale products of the
// current tile go into result set (sr_cur, pr_cur), and 16 FMAs fold the
// previous tile's set, issued a whole step earlier, into its accumulator.
// SPLIT places the scale products first and the FMAs around the block dot, so
// the vector ALU works while the matrix core does: the better order when the
// compute waves have their SIMDs to themselves (records staged by DMA).  With
// the staging waves converting weights on the same SIMDs, the plain order
// (both matrix instructions, then the FMAs) is the faster one.
template <bool SPLIT>
__device__ __forceinline__ void tile_step(const Operand& ak, const Operand& wk, int scale_a, f32x16& sr_cur,
                                          f32x16& pr_cur, const f32x16& sr_prev, const f32x16& pr_prev,
                                          f32x16& acc_prev) {
    const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (!SPLIT) {
        sr_cur = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp6_operand(ak), fp6_operand(wk), zero, 2, 2, 0,
                                                                 scale_a, 0, kScaleW);
        pr_cur = __builtin_amdgcn_mfma_f32_32x32x8f16(scale_operand(ak), scale_operand(wk), zero, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_prev[v] = fmaf(sr_prev[v], pr_prev[v], acc_prev[v]);
        return;
    }
    pr_cur = __builtin_amdgcn_mfma_f32_32x32x8f16(scale_operand(ak), scale_operand(wk), zero, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 8; ++v) acc_prev[v] = fmaf(sr_prev[v], pr_prev[v], acc_prev[v]);
    sr_cur = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp6_operand(ak), fp6_operand(wk), zero, 2, 2, 0, scale_a,
                                                             0, kScaleW);
#pragma unroll
    for (int v = 8; v < 16; ++v) acc_prev[v] = fmaf(sr_prev[v], pr_prev[v], acc_prev[v]);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // LDS reads ahead
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // scale-product MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // FMAs
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // block-dot MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // FMAs, operand moves
}

// Weight records of one stage: kKB planes of kPlaneB bytes, each a contiguous
// run of the repacked record stream, moved by kRecDma wave instructions of 1 KB
// dealt round-robin to the staging waves.
constexpr int kRecDma = kBufB / 1024;
static_assert(kBufB % 1024 == 0 && kPlaneB % 16 == 0, "record staging in 1 KB wave moves");
static_assert(kTR % 16 == 0, "row tiles keep the record swizzle (bits 2 and 3 of the row)");

template <bool DOTS, bool RP, bool EPI>
__global__ void __launch_bounds__(kT)
k_prefill(const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ Wrec, int64_t rows, int nb,
          const uint8_t* __restrict__ act, int64_t N, float* __restrict__ Y, int32_t* __restrict__ D,
          const Epilogue epi, int kbs, int splits) {
    __shared__ __align__(16) uint8_t smem[kNS * kStage];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    // workgroup tile: token tile (fastest), then split, then row tile; split s
    // takes blocks [kb0, kb1) of every row and writes its sums to slice s of Y
    const int64_t ntt = (N + kTT - 1) / kTT;
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t n0 = (tile % ntt) * kTT;
    const int64_t rs = tile / ntt;
    const int split = __builtin_amdgcn_readfirstlane(static_cast<int>(rs % splits));
    const int64_t r0 = (rs / splits) * kTR;
    const int kb0 = __builtin_amdgcn_readfirstlane(split * kbs);
    const int kb1 = __builtin_amdgcn_readfirstlane(min(nb, kb0 + kbs));
    const int nst = (kb1 - kb0 + kKB - 1) / kKB;

    if (wave >= kCW) {
        // ====================== staging waves ====================================
        const int sw = wave - kCW;
        const int u = t - kST;  // staging thread 0..255
        // activations; in LDS, 16-byte quarter q of token t sits at position
        // q ^ ((t >> 2) & 3) of its record
        const int dq = (lane & 3) ^ ((lane >> 4) & 3);
        int64_t dma_off[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            int64_t tok = n0 + sw * 32 + e * 16 + (lane >> 2);
            if (tok > N - 1) tok = N - 1;  // padding tokens: any valid record, never stored
            dma_off[e] = tok * kAct6Bytes + dq * 16;
        }
        auto issue_dma = [&](int st) __attribute__((always_inline)) {
            uint8_t* sA = smem + (st % kNS) * kStage;
#pragma unroll
            for (int i = 0; i < kDma; ++i) {
                const int blk = i >> 1, e = i & 1;
                int b = kb0 + st * kKB + blk;
                if (b > kb1 - 1) b = kb1 - 1;  // past the range: neutralised by zero weight scales
                const uint8_t* src = act + static_cast<int64_t>(b) * N * kAct6Bytes + dma_off[e];
                dma16(src, sA + blk * kPlaneA + (sw * 32 + e * 16) * kAct6Bytes);
            }
        };
        if constexpr (RP) {
            // Pre-converted records: the weights go straight into LDS as well,
            // three stages ahead (the ring slot of stage i + 3 is the one
            // stage i - 1 used).  Staging wave sw issues instructions g = sw,
            // sw + 4, ... < kRecDma; lane l of instruction g moves 16-byte
            // piece q = (g % 7) * 64 + l of plane g / 7: half q & 1 of row q / 2
            // (rows past the end read the last row: their outputs are never
            // stored).  Blocks past the end read the zero plane (block nb).
            constexpr int kPer = (kRecDma + kCW - 1) / kCW;
            const int nrec = (kRecDma - sw + kCW - 1) / kCW;  // 4 or 3
            int64_t rec_off[kPer];
            int rec_blk[kPer];
#pragma unroll
            for (int m = 0; m < kPer; ++m) {
                const int g = sw + kCW * m < kRecDma ? sw + kCW * m : sw;
                const int q = (g % (kPlaneB / 1024)) * 64 + lane;
                int64_t r = r0 + (q >> 1);
                if (r > rows - 1) r = rows - 1;
                rec_off[m] = r * kRecW + (q & 1) * 16;
                rec_blk[m] = g / (kPlaneB / 1024);
            }
            auto issue_rec = [&](int st) __attribute__((always_inline)) {
                uint8_t* sB = smem + (st % kNS) * kStage + kBufA;
#pragma unroll
                for (int m = 0; m < kPer; ++m) {
                    if (m < nrec) {  // wave-uniform
                        int b = kb0 + st * kKB + rec_blk[m];
                        if (b >= kb1) b = nb;  // past the range: the zero plane
                        const int g = sw + kCW * m;
                        dma16(Wrec + static_cast<int64_t>(b) * rows * kRecW + rec_off[m], sB + g * 1024);
                    }
                }
            };
            auto run = [&](auto per) __attribute__((always_inline)) {
                constexpr int L = kDma + decltype(per)::value;  // loads per stage for this wave
                issue_rec(0);
                issue_dma(0);
                issue_rec(1);
                issue_dma(1);
                issue_rec(2);
                issue_dma(2);
                stage_barrier<2 * L>();  // stage 0 landed
                for (int i = 0; i < nst; ++i) {
                    issue_rec(i + 3);
                    issue_dma(i + 3);
                    stage_barrier<2 * L>();  // stage i + 1 landed
                }
            };
            static_assert(kNS >= 4, "three stages ahead need four ring slots");
            static_assert(2 * (kDma + kPer) < 64, "vmcnt range");
            if (nrec == kPer)
                run(std::integral_constant<int, kPer>{});
            else
                run(std::integral_constant<int, kPer - 1>{});
            __builtin_amdgcn_s_waitcnt(0);  // no LDS writes in flight when the wave ends
            return;
        }
        // weights: staging thread u < 224 converts row u's blocks of a stage.
        // LDS record: 6 dwords of fp6 codes, binary16 d bits, zero; the two
        // 16-byte halves swap places in rows where bit 2 xor bit 3 is set.
        const bool w_thread = u < kTR;
        const int w_row = w_thread ? u : 0;
        const bool w_row_ok = w_thread && r0 + w_row < rows;
        const int64_t w_row_first = (r0 + (w_row_ok ? w_row : 0)) * nb;
        const uint8_t* w_src = Wq + w_row_first * kQ4Bytes;
        const int w_swap = ((w_row >> 2) ^ (w_row >> 3)) & 1;
        Block4 rw[2][kKB];
        bool rw_ok[2][kKB];
        // loads are unconditional (block 0 of a valid row when the wanted block
        // does not exist) so that the wait counts below stay exact
        auto load_w = [&](int st, auto set) __attribute__((always_inline)) {
            constexpr int S = decltype(set)::value;
#pragma unroll
            for (int k = 0; k < kKB; ++k) {
                const int b = kb0 + st * kKB + k;
                rw_ok[S][k] = w_row_ok && b < kb1;
                const int64_t bo = rw_ok[S][k] ? b : 0;
                rw[S][k] = load_block(w_src + bo * kQ4Bytes);
            }
        };
        auto store_w = [&](int st, auto set) __attribute__((always_inline)) {
            constexpr int S = decltype(set)::value;
            if (!w_thread) return;
            uint8_t* sB = smem + (st % kNS) * kStage + kBufA;
#pragma unroll
            for (int k = 0; k < kKB; ++k) {
                uint32_t d6[6] = {0u, 0u, 0u, 0u, 0u, 0u};
                uint32_t dbits = 0u;  // zero scale: the block contributes nothing
                if (rw_ok[S][k]) {
                    weight_fp6(rw[S][k].qs, d6);
                    dbits = rw[S][k].dbits;
                }
                uint8_t* p = sB + k * kPlaneB + w_row * kRecW;
                *reinterpret_cast<u32x4*>(p + 16 * w_swap) = u32x4{d6[0], d6[1], d6[2], d6[3]};
                *reinterpret_cast<u32x4*>(p + 16 * (w_swap ^ 1)) = u32x4{d6[4], d6[5], dbits, 0u};
            }
        };
        // per stage a staging thread issues kDma activation loads and two loads
        // per weight block
        constexpr int kLoads = kDma + 2 * kKB;
        static_assert(2 * kLoads < 64, "vmcnt range");

        // stages 0 and 1 ready before the loop
        load_w(0, std::integral_constant<int, 0>{});
        load_w(1, std::integral_constant<int, 1>{});
        issue_dma(0);
        issue_dma(1);
        store_w(0, std::integral_constant<int, 0>{});
        stage_barrier<0>();
        // iteration i (while stage i is computed): stage i + 2's raw weights
        // and activations go out; stage i + 1's weights, loaded during
        // iteration i - 1, are converted into its records
        auto step = [&](int i, auto set) __attribute__((always_inline)) {
            constexpr int S = decltype(set)::value;  // i % 2: held stage i, already converted
            constexpr std::integral_constant<int, S ^ 1> other{};
            load_w(i + 2, set);
            store_w(i + 1, other);  // waits for stage i + 1's weight loads and all before them
            issue_dma(i + 2);
            // everything up to stage i + 1 has landed; only this iteration's
            // loads may still be in flight
            stage_barrier<kLoads>();
        };
        for (int i = 0; i < nst; i += 2) {
            step(i, std::integral_constant<int, 0>{});
            if (i + 1 < nst) step(i + 1, std::integral_constant<int, 1>{});
        }
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // ======================== compute waves ======================================
    // Wave w takes token tiles A = 2 (w >> 1) and B = A + 1 and, by rh = w & 1,
    // row tiles 4 rh, 4 rh + 1, 4 rh + 2 for both of them plus row tile 3 for
    // one of them (A when rh = 0, B when rh = 1): seven 32 x 32 tiles, visited
    // as (A, R0) (B, R0) (A, R1) (B, R1) (A, R2) (B, R2) (X, 3), so that one
    // weight operand read from LDS serves two tiles.
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int tp = wave >> 1;
    const int a_sw = (l32 >> 2) & 3;
    int a_p0[2], a_p1[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int a_row = ((2 * tp + u) * 32 + l32) * kAct6Bytes;
        a_p0[u] = a_row + 16 * ((2 * half) ^ a_sw);
        a_p1[u] = a_row + 16 * ((2 * half + 1) ^ a_sw);
    }
    const int b_sw = ((l32 >> 2) ^ (l32 >> 3)) & 1;
    const int b_row = l32 * kRecW;
    const int b_p0 = b_row + 16 * b_sw;
    const int b_p1 = b_row + 16 * (b_sw ^ 1);
    const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int scale_a = (half ? kScaleLo : kScaleHi) - (DOTS ? 0 : kScaleDown);

    auto run = [&](auto rh_c) __attribute__((always_inline)) {
        constexpr int RH = decltype(rh_c)::value;
        constexpr int kPos = 7;                                                     // tiles per block
        constexpr int kSeqT[kPos] = {0, 1, 0, 1, 0, 1, RH};                          // A = 0, B = 1
        constexpr int kSeqR[kPos] = {4 * RH, 4 * RH, 4 * RH + 1, 4 * RH + 1, 4 * RH + 2, 4 * RH + 2, 3};
        constexpr int kSeqW[kPos] = {0, 0, 1, 1, 2, 2, 3};                          // weight read of the block
        static_assert(kPos == kRT, "seven tiles per wave");

        f32x16 acc[kPos];
#pragma unroll
        for (int j = 0; j < kPos; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
        // two result sets: step k's matrix instructions fill set k & 1 while
        // the FMAs of step k - 1 drain the other (a first drain of 0 * 0 is
        // harmless)
        f32x16 sr[2] = {zero, zero}, pr[2] = {zero, zero};

        // One stage: kKB blocks x 7 tiles, unrolled.  Operands are read one
        // step before their first use: the weights in a ring of two (four reads
        // per block), the next block's token operands while the current block
        // runs.  Step k issues its two matrix instructions into result set
        // k & 1 and drains set (k - 1) & 1, the previous step's tile, with 16
        // FMAs.  The step count per stage is even, so the parity carries over.
        auto compute = [&](int st) __attribute__((always_inline)) {
            constexpr int kSteps = kKB * kPos;
            static_assert(kSteps % 2 == 0, "result-set parity across stages");
            const uint8_t* sA = smem + (st % kNS) * kStage;
            const uint8_t* sB = sA + kBufA;
            auto w_at = [&](int blk, int p) __attribute__((always_inline)) {
                const uint8_t* pb = sB + blk * kPlaneB + kSeqR[p] * 32 * kRecW;
                return lds_operand(pb + b_p0, pb + b_p1);
            };
            auto a_at = [&](int blk, int u) __attribute__((always_inline)) {
                const uint8_t* pa = sA + blk * kPlaneA;
                return lds_operand(pa + a_p0[u], pa + a_p1[u]);
            };
            Operand a[2][2], w[2];
            a[0][0] = a_at(0, 0);
            a[0][1] = a_at(0, 1);
            w[0] = w_at(0, 0);
#pragma unroll
            for (int k = 0; k < kSteps; ++k) {
                const int blk = k / kPos, p = k % kPos;
                const int g = blk * 4 + kSeqW[p];  // weight read index within the stage
                // next step's weights, when it starts a new weight pair
                if (k + 1 < kSteps) {
                    const int nblk = (k + 1) / kPos, np = (k + 1) % kPos;
                    if (np == 0 || kSeqW[np] != kSeqW[p]) w[(g + 1) & 1] = w_at(nblk, np);
                }
                // next block's token operands, early in this block
                if (blk + 1 < kKB && (p == 2 || p == 3)) a[(blk + 1) & 1][p - 2] = a_at(blk + 1, p - 2);
                const Operand& ak = a[blk & 1][kSeqT[p]];
                const Operand& wk = w[g & 1];
                const int cur = k & 1;
                if constexpr (!DOTS) {
                    const int pj = p == 0 ? kPos - 1 : p - 1;  // the previous step's tile
                    tile_step<RP>(ak, wk, scale_a, sr[cur], pr[cur], sr[cur ^ 1], pr[cur ^ 1], acc[pj]);
                } else {
                    sr[cur] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fp6_operand(ak), fp6_operand(wk), zero,
                                                                              2, 2, 0, scale_a, 0, kScaleW);
                    const int b = kb0 + st * kKB + blk;
                    const int64_t r = r0 + kSeqR[p] * 32 + l32;
                    if (b < kb1 && r < rows) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int64_t n = n0 + (2 * tp + kSeqT[p]) * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                            if (n < N) D[(n * rows + r) * nb + b] = static_cast<int32_t>(sr[cur][v]);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        stage_barrier<0>();  // the first stages staged
        for (int i = 0; i < nst; ++i) {
            compute(i);
            stage_barrier<0>();
        }

        if constexpr (!DOTS) {
            // drain the last step: tile 6 of the last block, in set 1 (the
            // step count is even)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[kPos - 1][v] = fmaf(sr[1][v], pr[1][v], acc[kPos - 1][v]);
            float* const Yo = Y + static_cast<int64_t>(split) * N * rows;  // this split's slice
#pragma unroll
            for (int j = 0; j < kPos; ++j) {
                const int64_t r = r0 + kSeqR[j] * 32 + l32;
                if (r >= rows) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t n = n0 + (2 * tp + kSeqT[j]) * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                    if (n < N) Yo[n * rows + r] = EPI ? apply_epilogue(acc[j][v], n, r, rows, epi) : acc[j][v];
                }
            }
        }
    };
    if (wave & 1)
        run(std::integral_constant<int, 1>{});
    else
        run(std::integral_constant<int, 0>{});
}


// Y = the splits' slices of P added in split order (then the epilogue).
template <bool EPI>
__global__ void __launch_bounds__(256)
k_prefill_sum(const float* __restrict__ P, int splits, int64_t N, int64_t rows, float* __restrict__ Y,
              const Epilogue epi) {
    const int64_t total = N * rows;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        float y = P[i];
        for (int k = 1; k < splits; ++k) y += P[k * total + i];
        const int64_t n = i / rows, r = i - n * rows;
        Y[i] = EPI ? apply_epilogue(y, n, r, rows, epi) : y;
    }
}

}  // namespace

int prefill_splits(int64_t rows, int64_t nb, int64_t N, int num_cu, int* kbs) {
    const int64_t tiles = ((rows + kTR - 1) / kTR) * ((N + kTT - 1) / kTT);
    *kbs = static_cast<int>(nb);
    if (tiles >= kPrefillSplitTiles) return 1;
    int64_t S = num_cu / tiles;
    if (S > kPrefillMaxSplits) S = kPrefillMaxSplits;
    if (S > nb / kPrefillMinSplitBlocks) S = nb / kPrefillMinSplitBlocks;
    if (S < 2) return 1;
    int64_t kb = (nb + S - 1) / S;
    kb += kb & 1;  // whole stages of two blocks
    S = (nb + kb - 1) / kb;
    if (S < 2) return 1;
    *kbs = static_cast<int>(kb);
    return static_cast<int>(S);
}

size_t prefill_partial_bytes(int64_t rows, int64_t nb, int64_t N) {
    const int64_t tiles = ((rows + kTR - 1) / kTR) * ((N + kTT - 1) / kTT);
    if (tiles >= kPrefillSplitTiles || nb < 2 * kPrefillMinSplitBlocks) return 0;
    return static_cast<size_t>(kPrefillMaxSplits) * static_cast<size_t>(N * rows) * sizeof(float);
}

hipError_t launch_prefill(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                          const void* act, int64_t N, float* Y, int32_t* D, hipStream_t s, const Epilogue& epi,
                          float* partial, size_t partial_bytes) {
    const uint8_t* rec = static_cast<const uint8_t*>(act);
    const int nbi = static_cast<int>(nb);
    const bool fused = epi.bias || epi.mul || epi.act != kEpiNone;
    if (fused && lay == kRepacked) return hipErrorInvalidValue;  // the fused forms take the pages' blocks
    // few workgroup tiles: split K (each split's sums into its slice of the
    // partial buffer, added in split order by k_prefill_sum).  The split
    // depends on the shape alone, so every entry point gives the same bits;
    // without room in `partial` the buffer is taken stream-ordered.
    int kbs = nbi, splits = 1;
    if (!D) splits = prefill_splits(rows, nb, N, dev->num_cu, &kbs);
    const size_t need = splits > 1 ? static_cast<size_t>(splits) * static_cast<size_t>(N * rows) * sizeof(float) : 0;
    bool owned = false;
    if (splits > 1 && (!partial || partial_bytes < need)) {
        void* p = nullptr;
        if (hipMallocAsync(&p, need, s) != hipSuccess || p == nullptr) return hipErrorOutOfMemory;
        partial = static_cast<float*>(p);
        owned = true;
    }
    const dim3 grid(static_cast<uint32_t>(((rows + kTR - 1) / kTR) * ((N + kTT - 1) / kTT) * splits));
    float* out = splits > 1 ? partial : Y;
    const bool epi_here = fused && splits == 1;
    if (D)
        hipLaunchKernelGGL((k_prefill<true, false, false>), grid, dim3(kT), 0, s, Wq, nullptr, rows, nbi, rec, N, out,
                           D, epi, kbs, splits);
    else if (epi_here)
        hipLaunchKernelGGL((k_prefill<false, false, true>), grid, dim3(kT), 0, s, Wq, nullptr, rows, nbi, rec, N, out,
                           D, epi, kbs, splits);
    else if (lay == kRepacked)
        hipLaunchKernelGGL((k_prefill<false, true, false>), grid, dim3(kT), 0, s, Wq,
                           Wq + repack_records_offset(rows, nb), rows, nbi, rec, N, out, D, epi, kbs, splits);
    else
        hipLaunchKernelGGL((k_prefill<false, false, false>), grid, dim3(kT), 0, s, Wq, nullptr, rows, nbi, rec, N,
                           out, D, epi, kbs, splits);
    hipError_t err = hipGetLastError();
    if (splits == 1) return err;
    if (err != hipSuccess) {
        if (owned) (void)hipFreeAsync(partial, s);
        return err;
    }
    const int64_t total = N * rows;
    int64_t blocks = (total + 255) / 256;
    const int64_t cap = static_cast<int64_t>(dev->num_cu) * 8;
    if (blocks > cap) blocks = cap;
    if (fused)
        hipLaunchKernelGGL((k_prefill_sum<true>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, partial, splits,
                           N, rows, Y, epi);
    else
        hipLaunchKernelGGL((k_prefill_sum<false>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, partial,
                           splits, N, rows, Y, epi);
    err = hipGetLastError();
    if (owned) {
        const hipError_t ferr = hipFreeAsync(partial, s);
        if (err == hipSuccess) err = ferr;
    }
    return err;
}

size_t prefill_split_bytes(const DeviceInfo* dev, int64_t rows, int64_t nb, int64_t N) {
    int kbs = 0;
    const int splits = prefill_splits(rows, nb, N, dev->num_cu, &kbs);
    return splits > 1 ? static_cast<size_t>(splits) * static_cast<size_t>(N * rows) * sizeof(float) : 0;
}

}  // namespace q4bq
