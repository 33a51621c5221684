// Decode product on long rows, 1..8 tokens (`k_gemv_rows`): the kernel and
// its launch templates.  Included by q4bq_rows_x.hip (fp32 X quantized in the
// kernel) and q4bq_rows_act.hip (the quantizer's buffer), which instantiate it
// for one activation source each.
//
// Arithmetic: the per-block integer dot of ggml_vec_dot_q4_0_q8_0 as described
// in "llama.cpp 深度解读" (luoboask.github.io) section 3 "量化矩阵乘法 — 核心算子",
// the nibble offset of 8 from section 2's decode; the same device functions as
// the task kernel in q4bq_gemv.hip.
#pragma once

#include <algorithm>

#include "q4bq_device.h"
#include "q4bq_internal.h"

namespace q4bq {

namespace {

// ---------------------------------------------------------------------------
// Long rows, 1..8 tokens: rows streamed by whole waves.
//
// The 64 lanes of a wave share one row: lane p owns pairs p, p + 64, ...
// (PPL of them).  With one pair per lane its activation blocks never change,
// so the NT tokens' blocks stay in registers; with longer rows they are read
// from LDS.  Wave w walks rows w, w + S, w + 2S, ... (S = waves in the grid,
// so at any moment the grid reads one contiguous band of rows) and keeps D
// rows' loads in flight: it waits only for the oldest row, folds it, and
// issues the row D ahead.  The loads are unconditional -- past its last row a
// wave re-reads that row, and a lane past the last pair re-reads that pair --
// so the compiler's in-order load counters wait for exactly one row; the
// scheduling barriers keep the issue order fixed.  A row's nibbles are split
// once and meet every token's activations.
//
// Row sums: with several tokens the lanes first trade halves of their
// per-token partial sums (v_permlane32_swap, v_permlane16_swap, then a DPP
// rotate), so each step halves both the lanes to combine and the values per
// lane; the rest is DPP adds inside rows of 16 lanes.  One token: four DPP
// adds and two row broadcasts, lane 63 holds the sum.
//
// Activations: fp32 X quantized by the workgroup into LDS (kXF32) or the
// quantizer's buffer (kActGlobal).  Up to eight of X's 16-byte loads per
// thread are issued before the first weight loads, so that waiting for them
// does not wait for the weights.
//
// Few long rows (chunked form, C > 1): with more pairs than lanes and too few
// rows to give each wave several, a row is cut into C chunks of 48..64
// consecutive pairs and the grid walks "chunk rows" v = C r + c, one pair per
// lane.  Wave w always meets chunk w mod C, so its activations stay in
// registers; the grid still streams one contiguous band of the matrix at a
// time, and each wave has several chunk rows to pipeline.  The C chunks of a
// row belong to C neighbouring waves of one workgroup: each wave keeps its
// per-round partial sums in registers, and at the end the workgroup adds a
// row's C partials in chunk order through LDS and stores Y.
//
// Gate and up of a feed-forward (DUAL, C = 2): the two chunk rows of row r are
// row r of the gate matrix (md.w[0]) and row r of the up matrix (md.w[1]),
// each whole; the workgroup stores SiLU(gate) * up.  One launch reads both
// matrices, quantizing (and normalizing) the token once per workgroup.
// ---------------------------------------------------------------------------
constexpr int kRowsMaxPPL = 4;
constexpr size_t kRowsMaxLds = 128 * 1024;  // quantized activations in LDS (one workgroup per CU)
constexpr int kSplitRounds = 8;              // chunk rows per wave, at most, in the chunked form

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, kRowMask, 0xF,
                                                                 false));
}

__device__ __forceinline__ void swap32(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                    false, false);
    a = __builtin_bit_cast(float, static_cast<uint32_t>(r[0]));
    b = __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
}

__device__ __forceinline__ void swap16(float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                                    false, false);
    a = __builtin_bit_cast(float, static_cast<uint32_t>(r[0]));
    b = __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
}

constexpr int pow2_at_least(int n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8; }

// Sums each of the NT values over the 64 lanes.  Token t's total ends in lane
// sum_lane<NT>(t) (and possibly others).
template <int NT>
__device__ __forceinline__ float wave_sums(const float (&part)[NT], int lane) {
    constexpr int NTP = pow2_at_least(NT);
    float v[NTP];
#pragma unroll
    for (int t = 0; t < NTP; ++t) v[t] = t < NT ? part[t] : 0.0f;
    if constexpr (NTP >= 2) {
        // lanes 0-31 keep token i, lanes 32-63 token i + NTP/2
#pragma unroll
        for (int i = 0; i < NTP / 2; ++i) {
            swap32(v[i], v[i + NTP / 2]);
            v[i] += v[i + NTP / 2];
        }
    }
    if constexpr (NTP >= 4) {
        // rows 0 and 2 keep token i, rows 1 and 3 token i + NTP/4
#pragma unroll
        for (int i = 0; i < NTP / 4; ++i) {
            swap16(v[i], v[i + NTP / 4]);
            v[i] += v[i + NTP / 4];
        }
    }
    if constexpr (NTP >= 8) {
        // lanes with bit 3 clear keep token i, set: token i + 1
        const bool up = lane & 8;
        const float mine = up ? v[1] : v[0];
        const float other = up ? v[0] : v[1];
        v[0] = mine + dpp_f<0x128, 0xF>(other);  // row_ror:8, the lane 8 apart in the row
    }
    float x = v[0];
    x += dpp_f<0xB1, 0xF>(x);       // quad_perm [1,0,3,2]
    x += dpp_f<0x4E, 0xF>(x);       // quad_perm [2,3,0,1]
    x += dpp_f<0x141, 0xF>(x);      // row_half_mirror
    if constexpr (NTP <= 4) x += dpp_f<0x140, 0xF>(x);   // row_mirror: each row holds its sum
    if constexpr (NTP <= 2) x += dpp_f<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    if constexpr (NTP == 1) x += dpp_f<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

template <int NT>
__device__ __forceinline__ int sum_lane(int t) {
    constexpr int NTP = pow2_at_least(NT);
    return NTP == 1 ? 63 : NTP == 2 ? 32 * t + 31 : NTP == 4 ? 16 * t : 8 * t;
}
template <int NT>
__device__ __forceinline__ int lane_token(int lane) {
    constexpr int NTP = pow2_at_least(NT);
    return NTP == 1 ? (lane == 63 ? 0 : -1)
         : NTP == 2 ? ((lane & 31) == 31 ? lane >> 5 : -1)
         : NTP == 4 ? ((lane & 15) == 0 ? lane >> 4 : -1)
                    : ((lane & 7) == 0 ? lane >> 3 : -1);
}

// A 64-bit value the whole wave agrees on, in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// NTL (one pair per lane, the pages' blocks, rows or chunks of a multiple of
// 4 pairs): a wave loads its row (chunk) as consecutive 16-byte pieces with
// non-temporal loads -- each instruction one contiguous 1 KB -- writes them to
// its own LDS area in order and reads its lane's 36-byte pair back (rows 9
// dwords apart per lane: no bank conflicts).  Measured on the vocabulary head
// (loads alone): 36-byte pairs loaded by the lanes directly stream at ~5.8
// TB/s, the contiguous non-temporal pieces with the reordering at ~6.6 TB/s
// (non-temporal loads of the pairs themselves are slower: several load
// instructions touch each line).  The block dots see the same bytes.
constexpr int kNtlRowBytes = 64 * 36;  // a row or chunk of at most 64 pairs
__host__ __device__ inline size_t rows_ntl_offset(int nt, int64_t nb, int C, int waves, bool act_lds) {
    size_t a = act_lds ? static_cast<size_t>(nt) * nb * (kActQBytes + kActSBytes) : 0;
    const size_t p = C > 1 ? static_cast<size_t>(kSplitRounds) * waves * nt * sizeof(float) : 0;
    if (p > a) a = p;
    return (a + 15) / 16 * 16;
}

// DOTS: instead of Y, every per-block integer dot goes to
// Dots[(n * rows + r) * nb + b] (the test export; one matrix of Q4_0 blocks,
// activations from the quantizer's buffer).
template <int THREADS, int NT, int PPL, int D, int SRC, int LAY, bool EPI, bool DOTS = false, int C = 1,
          bool DUAL = false, bool NTL = false>
__global__ void __launch_bounds__(THREADS)
k_gemv_rows(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const void* __restrict__ src,
            float* __restrict__ Y, int32_t* __restrict__ Dots, const MultiDesc md) {
    static_assert(SRC == kXF32 || SRC == kActGlobal, "activation source");
    static_assert(!DOTS || (SRC == kActGlobal && LAY == kLayAoS && !EPI), "block-dot export form");
    constexpr bool RP = LAY == kLayRepacked;
    constexpr bool MULTI = LAY == kLayMulti;  // rows of md's matrices, concatenated (rows = their total)
    constexpr bool kActReg = PPL == 1;         // activations in registers, else read from LDS per row
    constexpr bool kUseLds = SRC == kXF32 || !kActReg;
    constexpr int kWaves = THREADS / 64;
    static_assert(C == 1 || (PPL == 1 && !MULTI && !DOTS && kWaves % C == 0), "chunked form");
    static_assert(!DUAL || (C == 2 && EPI && SRC == kXF32 && NT == 1 && LAY == kLayAoS), "gate and up form");
    static_assert(!NTL || (PPL == 1 && !RP && !DOTS), "contiguous row loads");
    // LayerNorm of the one token in the prologue (md.epi.ln_gamma set): the
    // fused instantiation with one pair per lane, where each thread holds its
    // quads of X in registers
    constexpr bool kLn = EPI && SRC == kXF32 && NT == 1 && PPL == 1 && (C == 1 || DUAL);
    constexpr int kCK = DUAL ? 1 : C;  // K-chunks per row
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t* sq = reinterpret_cast<uint32_t*>(smem);
    ActScale* ss = reinterpret_cast<ActScale*>(smem + static_cast<size_t>(NT) * nb * kActQBytes);
    const uint8_t* __restrict__ Wsc = Wq + (RP ? rows * nb * 16 : 0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar row arithmetic
    const int P = nb >> 1;
    const int Pc = P / kCK;                          // pairs per chunk (kCK divides P)
    const int pbase = kCK > 1 ? (wave % C) * Pc : 0;  // this wave's chunk, as a pair offset in the row
    const int nblk = NT * nb;  // activation blocks, token-major

    // 1. activation loads (before any weight load)
    //    kXF32: thread t quantizes quad (t & 7) of blocks t / 8 + (THREADS / 8) j
    //    kActGlobal into LDS: thread t copies 16-byte piece t + THREADS j of
    //    the int8 blocks and scale record t + THREADS j
    constexpr int kJ = (1024 * NT * PPL * kCK + THREADS - 1) / THREADS;  // nb <= 128 * PPL * kCK
    constexpr int kJpreMax = PPL * kCK == 1 ? 8 : 4;
    constexpr int kJpre = kJ < kJpreMax ? kJ : kJpreMax;
    float4 xv[SRC == kXF32 ? kJpre : 1];
    static_assert(!kLn || kJ == kJpre, "LayerNorm needs every quad of X in registers");
    float4 gv[kLn ? kJpre : 1], bv[kLn ? kJpre : 1];
    const bool do_ln = kLn && md.epi.ln_gamma != nullptr;
    if constexpr (SRC == kXF32) {
        const float* X = static_cast<const float*>(src);
#pragma unroll
        for (int j = 0; j < kJpre; ++j) {
            const int g = min(static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j, nblk - 1);
            __builtin_memcpy(&xv[j], X + static_cast<int64_t>(g) * kQK + 4 * (threadIdx.x & 7), 16);
        }
        if constexpr (kLn) {
            // unconditional (X itself stands in without LayerNorm): a branch
            // here made the compiler wait for these loads before the weights'
            const float* gp = do_ln ? md.epi.ln_gamma : X;
            const float* bp = do_ln ? md.epi.ln_beta : X;
#pragma unroll
            for (int j = 0; j < kJpre; ++j) {
                const int g = min(static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j, nblk - 1);
                const int64_t k = static_cast<int64_t>(g) * kQK + 4 * (threadIdx.x & 7);
                __builtin_memcpy(&gv[j], gp + k, 16);
                __builtin_memcpy(&bv[j], bp + k, 16);
            }
        }
    }
    uint32_t areg[kActReg ? NT : 1][2][8];
    ActScale sreg[kActReg ? NT : 1][2];
    if constexpr (SRC == kActGlobal && kActReg) {
        const int p = pbase + min(lane, Pc - 1);
        const u32x4* q = static_cast<const u32x4*>(src);
        const ActScale* sc = reinterpret_cast<const ActScale*>(static_cast<const uint8_t*>(src) +
                                                               static_cast<size_t>(nblk) * kActQBytes);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int g = n * nb + 2 * p + h;
                const u32x4 a0 = q[2 * g], a1 = q[2 * g + 1];
                areg[n][h][0] = a0.x; areg[n][h][1] = a0.y; areg[n][h][2] = a0.z; areg[n][h][3] = a0.w;
                areg[n][h][4] = a1.x; areg[n][h][5] = a1.y; areg[n][h][6] = a1.z; areg[n][h][7] = a1.w;
                sreg[n][h] = sc[g];
            }
    }

    // 2. the first D rows of this wave
    //    (rows of the chunked form are chunk rows v = C r + c)
    const int64_t V = rows * C;
    const int64_t S = static_cast<int64_t>(gridDim.x) * kWaves;
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
    const int64_t nk = w0 < V ? (V - 1 - w0) / S + 1 : 0;
    // a wave without rows (small matrices) still issues its loads, on the last
    // row, so that no branch leaves the load counters uncertain
    const int64_t rlast = nk > 0 ? w0 + (nk - 1) * S : V - 1;
    int pp[PPL];
    bool pv[PPL];
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
        pv[i] = lane + 64 * i < Pc;
        pp[i] = pbase + min(lane + 64 * i, Pc - 1);
    }
    // where a row's blocks and its output live; every value is wave-uniform
    // (scalar registers) and lanes add a 32-bit offset
    struct RowAt {
        const uint8_t* w;
        const uint8_t* sc;
        float* y;
        int64_t ystride;
    };
    auto row_at = [&](int64_t r) __attribute__((always_inline)) {
        RowAt a;
        if constexpr (MULTI) {
            const uint8_t* wb = md.w[0];
            float* yb = md.y[0];
            int64_t f = 0, f1 = md.first[1];
#pragma unroll
            for (int m = 1; m < kMaxMulti; ++m) {
                if (m < md.count && r >= md.first[m]) {
                    wb = md.w[m];
                    yb = md.y[m];
                    f = md.first[m];
                    f1 = md.first[m + 1];
                }
            }
            a.w = wb + uniform64((r - f) * nb) * kQ4Bytes;
            a.sc = nullptr;
            a.y = yb + (r - f);
            a.ystride = f1 - f;
        } else {
            const int64_t rb = uniform64(static_cast<int64_t>(static_cast<uint64_t>(r) / C) * nb);
            const uint8_t* wb = DUAL && (static_cast<uint64_t>(r) & 1) ? md.w[1] : Wq;
            a.w = wb + rb * (RP ? 16 : kQ4Bytes);
            a.sc = Wsc + rb * 2;
            a.y = Y + static_cast<int64_t>(static_cast<uint64_t>(r) / C);
            a.ystride = rows;
        }
        return a;
    };
    auto load_row = [&](Pair36 (&dst)[PPL], int64_t k) __attribute__((always_inline)) {
        const RowAt a = row_at(min(w0 + k * S, rlast));
#pragma unroll
        for (int i = 0; i < PPL; ++i) {
            const uint32_t p = static_cast<uint32_t>(pp[i]);
            dst[i] = RP ? load_pair_rp(a.w + 32 * p, a.sc + 4 * p) : load_pair(a.w + 36 * p);
        }
    };
    // NTL: the row's (chunk's) 9 Pc / 4 pieces; the lanes past them re-read
    // its last piece (unconditional loads), and only pieces inside are written
    const int npc = 9 * Pc / 4;
    uint8_t* const wrow =
        smem + rows_ntl_offset(NT, nb, C, kWaves, kUseLds) + static_cast<size_t>(wave) * kNtlRowBytes;
    auto load_row_ntl = [&](u32x4 (&dst)[3], int64_t k) __attribute__((always_inline)) {
        typedef u32x4 u32x4_a2 __attribute__((aligned(2)));
        const RowAt a = row_at(min(w0 + k * S, rlast));
        const uint8_t* base = a.w + 36 * pbase;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int pc = min(lane + 64 * i, npc - 1);
            dst[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_a2*>(base + 16 * pc));
        }
    };
    auto unpack_row = [&](const u32x4 (&src)[3], Pair36 (&q)[PPL]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 3; ++i)
            if (lane + 64 * i < npc) reinterpret_cast<u32x4*>(wrow)[lane + 64 * i] = src[i];
        __builtin_amdgcn_wave_barrier();
        const uint32_t* p = reinterpret_cast<const uint32_t*>(wrow + 36 * (pp[0] - pbase));
#pragma unroll
        for (int j = 0; j < 9; ++j) q[0].w[j] = p[j];
        __builtin_amdgcn_wave_barrier();
    };
    Pair36 raw[D][PPL];
    u32x4 rawn[NTL ? D : 1][3];
    auto load_next = [&](int d, int64_t k) __attribute__((always_inline)) {
        if constexpr (NTL) load_row_ntl(rawn[d], k);
        else load_row(raw[d], k);
    };
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_next(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 3. activations into LDS, then (one pair per lane) into registers
    if constexpr (kUseLds) {
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
                    sq[g * 8 + m] = word;
                    if (m == 0) ss[g] = sc;
                }
            };
            if constexpr (kLn) {
                if (do_ln) {
                    // fp64 mean and population variance of the token over the
                    // workgroup, then the normalized values (fp64, rounded
                    // once to fp32)
                    __shared__ double red[2][THREADS / 64];
                    double s1 = 0.0;
#pragma unroll
                    for (int j = 0; j < kJpre; ++j)
                        if (static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j < nblk) s1 += quad_sum_f64(xv[j]);
                    const double kk = static_cast<double>(nb) * kQK;
                    const double mu = wg_sum_f64<THREADS>(s1, red[0]) / kk;
                    double s2 = 0.0;
#pragma unroll
                    for (int j = 0; j < kJpre; ++j)
                        if (static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j < nblk)
                            s2 += quad_sqdev_f64(xv[j], mu);
                    const double rstd =
                        1.0 / sqrt(wg_sum_f64<THREADS>(s2, red[1]) / kk + static_cast<double>(md.epi.ln_eps));
#pragma unroll
                    for (int j = 0; j < kJpre; ++j) xv[j] = ln_quad(xv[j], mu, rstd, gv[j], bv[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < kJpre; ++j) quantize(xv[j], j);
            // the rest of a long X (loaded after the weights: these wait for them)
            const int jend = min(kJ, (nblk + THREADS / 8 - 1) / (THREADS / 8));
#pragma unroll 2
            for (int j = kJpre; j < jend; ++j) {
                const int g = min(static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j, nblk - 1);
                float4 x;
                __builtin_memcpy(&x, X + static_cast<int64_t>(g) * kQK + 4 * m, 16);
                quantize(x, j);
            }
        } else {
            const u32x4* q = static_cast<const u32x4*>(src);
            const ActScale* sc = reinterpret_cast<const ActScale*>(static_cast<const uint8_t*>(src) +
                                                                   static_cast<size_t>(nblk) * kActQBytes);
            for (int t = threadIdx.x; t < 2 * nblk; t += THREADS) reinterpret_cast<u32x4*>(sq)[t] = q[t];
            for (int t = threadIdx.x; t < nblk; t += THREADS) ss[t] = sc[t];
        }
        // LDS writes done, then the workgroup barrier; no wait on the weight loads
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if constexpr (kActReg) {
            const int p = pbase + min(lane, Pc - 1);
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int g = n * nb + 2 * p + h;
                    const u32x4 a0 = reinterpret_cast<const u32x4*>(sq)[g * 2];
                    const u32x4 a1 = reinterpret_cast<const u32x4*>(sq)[g * 2 + 1];
                    areg[n][h][0] = a0.x; areg[n][h][1] = a0.y; areg[n][h][2] = a0.z; areg[n][h][3] = a0.w;
                    areg[n][h][4] = a1.x; areg[n][h][5] = a1.y; areg[n][h][6] = a1.z; areg[n][h][7] = a1.w;
                    sreg[n][h] = ss[g];
                }
        }
    }
    if (C == 1 && nk == 0) return;  // the chunked form's waves all meet the final barriers

    if constexpr (DOTS) {
        // the same loads and block dots as the product, each dot stored
        for (int64_t k = 0; k < nk; k += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (k + d < nk) {
                    const int64_t r = w0 + (k + d) * S;
#pragma unroll
                    for (int i = 0; i < PPL; ++i) {
                        if (!pv[i]) continue;
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const Block4 blk = h ? pair_second(raw[d][i]) : pair_first(raw[d][i]);
#pragma unroll
                            for (int n = 0; n < NT; ++n) {
                                int32_t sdot;
                                if constexpr (kActReg) {
                                    sdot = block_dot(blk, areg[n][h], sreg[n][h].bias);
                                } else {
                                    const int g = n * nb + 2 * pp[i] + h;
                                    const u32x4 a0 = reinterpret_cast<const u32x4*>(sq)[g * 2];
                                    const u32x4 a1 = reinterpret_cast<const u32x4*>(sq)[g * 2 + 1];
                                    const uint32_t a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                                    sdot = block_dot(blk, a, ss[g].bias);
                                }
                                Dots[(static_cast<int64_t>(n) * rows + r) * nb + 2 * pp[i] + h] = sdot;
                            }
                        }
                    }
                }
                load_row(raw[d], k + d + D);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        return;
    }

    // 4. the rolling loop
    auto fold = [&](const Pair36 (&q)[PPL], float (&part)[NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NT; ++n) part[n] = 0.0f;
#pragma unroll
        for (int i = 0; i < PPL; ++i) {
            float v[NT][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const Block4 blk = RP ? (h ? pair_second_rp(q[i]) : pair_first_rp(q[i]))
                                      : (h ? pair_second(q[i]) : pair_first(q[i]));
                const float dw = half_bits_to_float(blk.dbits);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    int32_t s;
                    float dx;
                    if constexpr (kActReg) {
                        s = block_dot(blk, areg[n][h], sreg[n][h].bias);
                        dx = sreg[n][h].d;
                    } else {
                        const int g = n * nb + 2 * pp[i] + h;
                        const u32x4 a0 = reinterpret_cast<const u32x4*>(sq)[g * 2];
                        const u32x4 a1 = reinterpret_cast<const u32x4*>(sq)[g * 2 + 1];
                        const uint32_t a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                        const ActScale sc = ss[g];
                        s = block_dot(blk, a, sc.bias);
                        dx = sc.d;
                    }
                    v[n][h] = static_cast<float>(s) * (dw * dx);
                    // LDS operands: at most four tokens' reads in flight, so
                    // the operands of a long row stay within the register budget
                    if constexpr (!kActReg) {
                        if ((n & 3) == 3) __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const float pair = v[n][0] + v[n][1];
                part[n] = i == 0 ? (pv[0] ? pair : 0.0f) : part[n] + (pv[i] ? pair : 0.0f);
            }
        }
    };
    const int my_token = lane_token<NT>(lane);
    if constexpr (C > 1) {
        // per-round partial sums in registers (round k: chunk row w0 + k S)
        float keep[kSplitRounds];
#pragma unroll
        for (int k = 0; k < kSplitRounds; k += D) {
            if (k >= nk) break;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                float part[NT];
                if constexpr (NTL) unpack_row(rawn[d], raw[d]);
                fold(raw[d], part);
                keep[k + d] = wave_sums<NT>(part, lane);
                load_next(d, k + d + D);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // this workgroup's outputs: round k, row q of the round (kWaves / C
        // rows, from waves C q .. C q + C - 1), token n; at most one per thread
        constexpr int kRowsPerRound = kWaves / C;
        constexpr int kOuts = kSplitRounds * kRowsPerRound * NT;
        static_assert(kOuts <= THREADS, "one output per thread");
        const int on = threadIdx.x % NT, oq = (threadIdx.x / NT) % kRowsPerRound, ok = threadIdx.x / (NT * kRowsPerRound);
        const int64_t ov = static_cast<int64_t>(blockIdx.x) * kWaves + ok * S + oq * C;
        const bool has_out = threadIdx.x < kOuts && ov < V;
        const int64_t orow = has_out ? ov / C : 0;
        float eb = 0.0f, em = 1.0f;
        if constexpr (EPI && !DUAL) {
            if (has_out) {
                eb = epi_bias(md.epi, orow);
                em = epi_mul(md.epi, on, orow, rows);
            }
        }
        // every wave is past its last LDS activation read: the partials take
        // LDS, slot (k * kWaves + wave) * NT + token
        float* pl = reinterpret_cast<float*>(smem);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < kSplitRounds; ++k)
            if (k < nk && my_token >= 0 && my_token < NT) pl[(k * kWaves + wave) * NT + my_token] = keep[k];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (has_out) {
            const float* src_p = pl + (ok * kWaves + oq * C) * NT + on;
            float y = src_p[0];
            if constexpr (DUAL) {
                // SiLU(gate), then times up: the two fused stores' arithmetic
                y = y / (1.0f + expf(-y));
                y *= src_p[NT];
            } else {
#pragma unroll
                for (int c = 1; c < C; ++c) y += src_p[c * NT];
                if constexpr (EPI) y = epilogue_with(y, eb, em, md.epi);
            }
            Y[static_cast<int64_t>(on) * rows + orow] = y;
        }
        return;
    }
    // fused forms: each row's epilogue operands (bias, factor of this lane's
    // token) are loaded with the row's weights, not at its store
    float eb[EPI ? D : 1], em[EPI ? D : 1];
    const int etok = my_token >= 0 && my_token < NT ? my_token : 0;
    auto load_epi = [&](int d, int64_t k) __attribute__((always_inline)) {
        if constexpr (EPI) {
            const int64_t r = min(w0 + k * S, rlast);
            eb[d] = epi_bias(md.epi, r);
            em[d] = epi_mul(md.epi, etok, r, rows);
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) load_epi(d, d);
    for (int64_t k = 0; k < nk; k += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            float part[NT];
            if constexpr (NTL) unpack_row(rawn[d], raw[d]);
            fold(raw[d], part);
            const float t = wave_sums<NT>(part, lane);
            if (k + d < nk && my_token >= 0 && my_token < NT) {
                const int64_t r = w0 + (k + d) * S;
                const RowAt a = row_at(r);
                a.y[static_cast<int64_t>(my_token) * a.ystride] = EPI ? epilogue_with(t, eb[d], em[d], md.epi) : t;
            }
            load_next(d, k + d + D);
            load_epi(d, k + d + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Pairs per lane for the row-streaming kernel, or 0 where it does not apply:
// an even block count, and rows whose pairs fill at least three quarters of
// the lanes; or, for matrices of at most kShortRowsMax rows, one pair per
// lane on rows of 8..47 pairs (most lanes idle, but a whole wave per row
// hides the latency of the small launches that such shapes make: GPT-2's
// K = 768 matrices, 4.4 -> 3.4 us graph-timed).  Other shapes keep the task
// kernel.
constexpr int64_t kShortRowsMax = 16384;
inline int rows_ppl(int64_t nb, int64_t rows) {
    if (nb & 1) return 0;
    const int64_t P = nb >> 1;
    if (P >= 8 && P < 48 && rows <= kShortRowsMax) return 1;
    for (int ppl = 1; ppl <= kRowsMaxPPL; ppl *= 2)
        if (P <= 64 * ppl) return 4 * P >= 3 * 64 * ppl ? ppl : 0;
    return 0;
}

// Chunks per row for the chunked form, or 1: rows of 96..512 pairs (an even
// block count) that split into C = 2, 4 or 8 chunks of 48..64 pairs, when
// the grid gives no wave more than kSplitRounds chunk rows.  waves: per
// workgroup of the one-pair-per-lane kernel for these tokens.
inline int rows_split(int64_t rows, int64_t nb, int waves, int num_cu) {
    if (nb & 1) return 1;
    const int64_t P = nb >> 1;
    if (P <= 64) return 1;
    for (int C = 2; C <= 8; C *= 2) {
        if (C > waves || P % C != 0 || P / C > 64 || P / C < 48) continue;
        const int64_t V = rows * C;
        int64_t wgs = (V + waves - 1) / waves;
        const int64_t cap = static_cast<int64_t>(num_cu) * (16 / waves);
        if (wgs > cap) wgs = cap;
        return (V + wgs * waves - 1) / (wgs * waves) <= kSplitRounds ? C : 1;
    }
    return 1;
}

// Workgroup size: 16 waves per CU (at most 128 registers per lane), or 8 where
// more tokens need more registers (token activations with one pair per lane;
// per-token partial sums and LDS operands on longer rows).  Depth: rows in
// flight per wave.
template <int NT, int PPL>
constexpr int rows_threads() { return NT > (PPL == 1 ? 4 : PPL == 2 ? 6 : 4) ? 512 : 1024; }
template <int NT, int PPL>
constexpr int rows_depth() { return PPL == 1 && NT > 4 ? 2 : 1; }

template <int SRC, int LAY, bool EPI, bool DOTS, int NT, int PPL, int C = 1, bool DUAL = false>
hipError_t launch_rows_k(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                         float* Y, int32_t* dots, const MultiDesc& md, hipStream_t s) {
    constexpr int kThreads = rows_threads<NT, PPL>();
    // one token in the chunked form: two chunk rows in flight per wave (each
    // wave has only a few: 4096 x 14336 at N = 1 10.0 -> 9.5 us; whole rows
    // keep one: 4096 x 4096 4.1 -> 5.2 us with two)
    constexpr int kDepth = NT == 1 && C > 1 && !DUAL ? 2 : rows_depth<NT, PPL>();
    int64_t wgs = (rows * C + kThreads / 64 - 1) / (kThreads / 64);
    const int64_t cap = static_cast<int64_t>(dev->num_cu) * (1024 / kThreads);
    if (wgs > cap) wgs = cap;
    // many tokens with one pair per lane (two waves per SIMD): four rows in
    // flight per wave where every wave has at least 16 rows (the vocabulary
    // head at N = 8: 88 -> 83 us); shorter matrices keep two, since a wave
    // re-reads its last row for each extra slot
    constexpr bool kDeep = kDepth == 2 && C == 1 && !DOTS;
    const bool deep = kDeep && rows >= 16 * wgs * (kThreads / 64);
    // contiguous non-temporal row loads through LDS where a row (chunk) is
    // whole 16-byte pieces and every wave has 16 rows or more (measured: the
    // vocabulary head at N = 1 / 2, 52.0 -> 46.7 / 55.3 -> 50.0 us; with a few
    // rows per wave the extra LDS round trip per row costs more than the
    // loads save: 14336 x 4096 at N = 1 8.1 -> 8.3 us, 4096 x 4096 at N = 2
    // 5.4 -> 6.0 us)
    constexpr bool kNtlForm = PPL == 1 && LAY != kLayRepacked && !DOTS;
    const bool ntl = kNtlForm && ((nb / 2) / C) % 4 == 0 && rows * C >= 16 * wgs * (kThreads / 64) &&
                     rows_ntl_offset(NT, nb, C, kThreads / 64, SRC == kXF32 || PPL > 1) +
                             static_cast<size_t>(kThreads / 64) * kNtlRowBytes <=
                         kRowsMaxLds;
    const auto kernel =
        ntl ? (deep ? k_gemv_rows<kThreads, NT, PPL, kDeep ? 4 : kDepth, SRC, LAY, EPI, DOTS, C, DUAL, kNtlForm>
                    : k_gemv_rows<kThreads, NT, PPL, kDepth, SRC, LAY, EPI, DOTS, C, DUAL, kNtlForm>)
            : (deep ? k_gemv_rows<kThreads, NT, PPL, kDeep ? 4 : kDepth, SRC, LAY, EPI, DOTS, C, DUAL>
                    : k_gemv_rows<kThreads, NT, PPL, kDepth, SRC, LAY, EPI, DOTS, C, DUAL>);
    size_t lds = (SRC == kXF32 || PPL > 1) ? static_cast<size_t>(NT) * nb * (kActQBytes + kActSBytes) : 0;
    if (C > 1) lds = std::max(lds, static_cast<size_t>(kSplitRounds) * (kThreads / 64) * NT * sizeof(float));
    if (ntl)
        lds = rows_ntl_offset(NT, nb, C, kThreads / 64, SRC == kXF32 || PPL > 1) +
              static_cast<size_t>(kThreads / 64) * kNtlRowBytes;
    if (lds > 64 * 1024) {
        // beyond the default dynamic LDS limit: raise it once for this kernel
        const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                                      static_cast<int>(kRowsMaxLds));
        if (raised != hipSuccess) return raised;
    }
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(wgs)), dim3(kThreads), lds, s, Wq, rows,
                       static_cast<int>(nb), src, Y, dots, md);
    return hipGetLastError();
}

template <int SRC, int LAY, bool EPI, bool DOTS, int NT>
hipError_t launch_rows_nt(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                          float* Y, int32_t* dots, const MultiDesc& md, hipStream_t s) {
    if constexpr (LAY != kLayMulti && !DOTS) {
        switch (rows_split(rows, nb, rows_threads<NT, 1>() / 64, dev->num_cu)) {
            case 2: return launch_rows_k<SRC, LAY, EPI, DOTS, NT, 1, 2>(dev, Wq, rows, nb, src, Y, dots, md, s);
            case 4: return launch_rows_k<SRC, LAY, EPI, DOTS, NT, 1, 4>(dev, Wq, rows, nb, src, Y, dots, md, s);
            case 8: return launch_rows_k<SRC, LAY, EPI, DOTS, NT, 1, 8>(dev, Wq, rows, nb, src, Y, dots, md, s);
            default: break;
        }
    }
    switch (rows_ppl(nb, rows)) {
        case 1: return launch_rows_k<SRC, LAY, EPI, DOTS, NT, 1>(dev, Wq, rows, nb, src, Y, dots, md, s);
        case 2: return launch_rows_k<SRC, LAY, EPI, DOTS, NT, 2>(dev, Wq, rows, nb, src, Y, dots, md, s);
        case 4: return launch_rows_k<SRC, LAY, EPI, DOTS, NT, 4>(dev, Wq, rows, nb, src, Y, dots, md, s);
        default: return hipErrorInvalidValue;
    }
}

template <int SRC, int LAY, bool EPI = false, bool DOTS = false>
hipError_t launch_rows_t(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                         int64_t N, float* Y, const MultiDesc& md, hipStream_t s, int32_t* dots = nullptr) {
    switch (N) {
        case 1: return launch_rows_nt<SRC, LAY, EPI, DOTS, 1>(dev, Wq, rows, nb, src, Y, dots, md, s);
        case 2: return launch_rows_nt<SRC, LAY, EPI, DOTS, 2>(dev, Wq, rows, nb, src, Y, dots, md, s);
        case 3: return launch_rows_nt<SRC, LAY, EPI, DOTS, 3>(dev, Wq, rows, nb, src, Y, dots, md, s);
        case 4: return launch_rows_nt<SRC, LAY, EPI, DOTS, 4>(dev, Wq, rows, nb, src, Y, dots, md, s);
        case 5: return launch_rows_nt<SRC, LAY, EPI, DOTS, 5>(dev, Wq, rows, nb, src, Y, dots, md, s);
        case 6: return launch_rows_nt<SRC, LAY, EPI, DOTS, 6>(dev, Wq, rows, nb, src, Y, dots, md, s);
        case 7: return launch_rows_nt<SRC, LAY, EPI, DOTS, 7>(dev, Wq, rows, nb, src, Y, dots, md, s);
        case 8: return launch_rows_nt<SRC, LAY, EPI, DOTS, 8>(dev, Wq, rows, nb, src, Y, dots, md, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

}  // namespace q4bq
