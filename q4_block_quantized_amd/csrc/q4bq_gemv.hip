// Decode product, N = 1..8 tokens: Y[n][r] = sum_b d_w(r,b) * d_x(n,b) * s(r,n,b).
//
// The per-block integer dot s follows ggml_vec_dot_q4_0_q8_0 as described in
// "llama.cpp 深度解读" (luoboask.github.io) section 3 "量化矩阵乘法 — 核心算子":
// unpack the two nibbles of each byte, multiply by the int8 activations,
// accumulate in int32, then scale by the fp32 product of the two fp16 block
// scales; the nibble offset of 8 comes from section 2's decode.
//
// The kernel is bound by streaming the Q4_0 weights from HBM once:
//  * each lane owns whole pairs of consecutive blocks of a row (36 bytes,
//    three loads) -- G lanes share a row, 64/G rows per wave per row slot,
//    and a lane carries up to kRmax rows at a time so that several pairs are
//    in flight and each activation read serves several rows;
//  * a nibble word splits into low/high nibbles with one AND and one
//    shift+AND and meets the activations (stored in the matching order by the
//    quantizer) in v_dot4_i32_i8, seeded with -8 * sum(q) so the offset costs
//    nothing per element;
//  * per block one convert and one FMA fold the int32 dot into fp32;
//  * lanes of a row combine with a butterfly over G lanes.
// The weights are read either as the pages' 18-byte blocks or, after
// q4_0_repack, as 16-byte-aligned nibble blocks plus a separate scale stream
// (same bytes, same arithmetic, same bits).
// Activations come from the quantizer's buffer (read in place, or copied to
// LDS when they fit) or, for one or two tokens, are quantized from fp32 by the
// kernel itself into LDS before it streams the weights; the Q8_0 arithmetic is
// the same device function either way, so both give the same bits.
#include "q4bq_device.h"
#include "q4bq_internal.h"

namespace q4bq {

namespace {

constexpr int kRmax = 4;          // rows per lane per task
constexpr int kU = 2;             // pair slots per load batch
constexpr size_t kMaxActLds = 64 * 1024;

enum Src { kActGlobal = 0, kActLds = 1, kXF32 = 2 };

enum Lay { kLayAoS = 0, kLayRepacked = 1, kLayMulti = 2 };

template <int NT, int THREADS, int SRC, bool DOTS, int LAY>
__global__ void __launch_bounds__(THREADS)
k_gemv(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const void* __restrict__ src,
       float* __restrict__ Y, int32_t* __restrict__ D, int log2G, int rpi, const MultiDesc md) {
    constexpr int kWaves = THREADS / 64;
    constexpr bool RP = LAY == kLayRepacked;
    constexpr bool MULTI = LAY == kLayMulti;  // rows of md's matrices, concatenated (rows = their total)
    // RP: Wq holds the repacked streams (nibbles, then scales)
    const uint8_t* __restrict__ Wsc = Wq + (RP ? rows * nb * 16 : 0);
    extern __shared__ __align__(16) uint8_t smem[];
    const uint32_t* act_q;
    const ActScale* act_s;
    if constexpr (SRC == kActGlobal) {
        act_q = static_cast<const uint32_t*>(src);
        act_s = reinterpret_cast<const ActScale*>(static_cast<const uint8_t*>(src) +
                                                  static_cast<size_t>(NT) * nb * kActQBytes);
    } else {
        uint32_t* sq = reinterpret_cast<uint32_t*>(smem);
        ActScale* ss = reinterpret_cast<ActScale*>(smem + static_cast<size_t>(NT) * nb * kActQBytes);
        if constexpr (SRC == kActLds) {
            const u32x4* gq = static_cast<const u32x4*>(src);
            const ActScale* gs = reinterpret_cast<const ActScale*>(static_cast<const uint8_t*>(src) +
                                                                   static_cast<size_t>(NT) * nb * kActQBytes);
            for (int c = threadIdx.x; c < NT * nb * 2; c += THREADS) reinterpret_cast<u32x4*>(sq)[c] = gq[c];
            for (int c = threadIdx.x; c < NT * nb; c += THREADS) ss[c] = gs[c];
        } else {
            // quantize X (NT x K fp32) here: 8 lanes per block, 4 values per lane
            const float* X = static_cast<const float*>(src);
            const int m = threadIdx.x & 7;
            const int nblk = NT * nb;
            for (int g0 = (threadIdx.x >> 3) & ~7; g0 < nblk; g0 += THREADS / 8) {
                const int g = g0 + ((threadIdx.x >> 3) & 7);
                const bool valid = g < nblk;
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
                if (valid) __builtin_memcpy(&x, X + static_cast<int64_t>(g) * kQK + 4 * m, 16);
                uint32_t word;
                const ActScale sc = quant_act_quad(x.x, x.y, x.z, x.w, m, word);
                if (valid) {
                    sq[g * 8 + m] = word;
                    if (m == 0) ss[g] = sc;
                }
            }
        }
        __syncthreads();
        act_q = sq;
        act_s = ss;
    }

    const int G = 1 << log2G;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> log2G;
    const int pos = lane & (G - 1);
    const int RW = 64 >> log2G;                 // rows per wave per row slot
    const int P = nb >> 1;                      // whole pairs per row
    const int PPL = (P + G - 1) >> log2G;       // pair slots per lane
    const int64_t rows_per_task = static_cast<int64_t>(RW) * rpi;
    const int64_t ntasks = (rows + rows_per_task - 1) / rows_per_task;

    for (int64_t task = static_cast<int64_t>(blockIdx.x) * kWaves + wave; task < ntasks;
         task += static_cast<int64_t>(gridDim.x) * kWaves) {
        int64_t r[kRmax];
        bool rv[kRmax];
#pragma unroll
        for (int j = 0; j < kRmax; ++j) {
            r[j] = task * rows_per_task + static_cast<int64_t>(j) * RW + grp;
            rv[j] = (j < rpi) && (r[j] < rows);
        }
        // per row: its blocks and its output column (one matrix, or the matrix
        // of md that owns the global row)
        const uint8_t* wrow[kRmax];
        float* yrow[kRmax];
        int64_t ystride[kRmax];
#pragma unroll
        for (int j = 0; j < kRmax; ++j) {
            if constexpr (MULTI) {
                int m = 0;
#pragma unroll
                for (int k = 1; k < kMaxMulti; ++k)
                    if (k < md.count && r[j] >= md.first[k]) m = k;
                const int64_t loc = r[j] - md.first[m];
                wrow[j] = md.w[m] + loc * nb * kQ4Bytes;
                yrow[j] = md.y[m] + loc;
                ystride[j] = md.first[m + 1] - md.first[m];
            } else {
                wrow[j] = Wq + r[j] * nb * kQ4Bytes;
                yrow[j] = Y + r[j];
                ystride[j] = rows;
            }
        }
        float acc[kRmax][NT];
#pragma unroll
        for (int j = 0; j < kRmax; ++j)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[j][n] = 0.0f;

        for (int i0 = 0; i0 < PPL; i0 += kU) {
            Pair36 raw[kRmax][kU];
            bool pv[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) pv[u] = (pos + ((i0 + u) << log2G)) < P;
            // issue every load of the batch before using any
#pragma unroll
            for (int j = 0; j < kRmax; ++j)
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int p = pos + ((i0 + u) << log2G);
                    if (rv[j] && pv[u]) {
                        const int64_t blk0 = r[j] * nb + 2 * p;
                        raw[j][u] = RP ? load_pair_rp(Wq + blk0 * 16, Wsc + blk0 * 2)
                                       : load_pair(wrow[j] + 2 * p * kQ4Bytes);
                    }
                }
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (!pv[u]) continue;
                const int p = pos + ((i0 + u) << log2G);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int b = 2 * p + h;
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        const int64_t ab = static_cast<int64_t>(n) * nb + b;
                        const u32x4 a0 = reinterpret_cast<const u32x4*>(act_q + ab * 8)[0];
                        const u32x4 a1 = reinterpret_cast<const u32x4*>(act_q + ab * 8)[1];
                        const ActScale sc = act_s[ab];
                        const uint32_t a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                        for (int j = 0; j < kRmax; ++j) {
                            if (!rv[j]) continue;
                            const Block4 blk = RP ? (h ? pair_second_rp(raw[j][u]) : pair_first_rp(raw[j][u]))
                                                  : (h ? pair_second(raw[j][u]) : pair_first(raw[j][u]));
                            const int32_t s = block_dot(blk, a, sc.bias);
                            if constexpr (DOTS) {
                                D[(static_cast<int64_t>(n) * rows + r[j]) * nb + b] = s;
                            } else {
                                acc[j][n] = fmaf(static_cast<float>(s), half_bits_to_float(blk.dbits) * sc.d,
                                                 acc[j][n]);
                            }
                        }
                    }
                }
            }
        }
        if ((nb & 1) && pos == 0) {  // a row with an odd block count ends in one lone block
            const int b = nb - 1;
#pragma unroll
            for (int j = 0; j < kRmax; ++j) {
                if (!rv[j]) continue;
                const int64_t bi = r[j] * nb + b;
                const Block4 blk = RP ? load_block_rp(Wq + bi * 16, Wsc + bi * 2) : load_block(wrow[j] + b * kQ4Bytes);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const int64_t ab = static_cast<int64_t>(n) * nb + b;
                    const u32x4 a0 = reinterpret_cast<const u32x4*>(act_q + ab * 8)[0];
                    const u32x4 a1 = reinterpret_cast<const u32x4*>(act_q + ab * 8)[1];
                    const ActScale sc = act_s[ab];
                    const uint32_t a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                    const int32_t s = block_dot(blk, a, sc.bias);
                    if constexpr (DOTS) {
                        D[(static_cast<int64_t>(n) * rows + r[j]) * nb + b] = s;
                    } else {
                        acc[j][n] = fmaf(static_cast<float>(s), half_bits_to_float(blk.dbits) * sc.d, acc[j][n]);
                    }
                }
            }
        }
        if constexpr (!DOTS) {
            for (int m = G >> 1; m >= 1; m >>= 1) {
#pragma unroll
                for (int j = 0; j < kRmax; ++j)
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[j][n] += __shfl_xor(acc[j][n], m, 64);
            }
            if (pos == 0) {
#pragma unroll
                for (int j = 0; j < kRmax; ++j) {
                    if (!rv[j]) continue;
#pragma unroll
                    for (int n = 0; n < NT; ++n) yrow[j][static_cast<int64_t>(n) * ystride[j]] = acc[j][n];
                }
            }
        }
    }
}

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
// ---------------------------------------------------------------------------
constexpr int kRowsMaxPPL = 4;
constexpr int kRowsMaxNtPpl = 8;   // NT * PPL: activation registers, or LDS reads per row
constexpr size_t kRowsMaxLds = 64 * 1024;

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

template <int THREADS, int NT, int PPL, int D, int SRC, int LAY>
__global__ void __launch_bounds__(THREADS)
k_gemv_rows(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const void* __restrict__ src,
            float* __restrict__ Y, const MultiDesc md) {
    static_assert(SRC == kXF32 || SRC == kActGlobal, "activation source");
    static_assert(NT * PPL <= kRowsMaxNtPpl, "activation registers");
    constexpr bool RP = LAY == kLayRepacked;
    constexpr bool MULTI = LAY == kLayMulti;  // rows of md's matrices, concatenated (rows = their total)
    constexpr bool kActReg = PPL == 1;         // activations in registers, else read from LDS per row
    constexpr bool kUseLds = SRC == kXF32 || !kActReg;
    constexpr int kWaves = THREADS / 64;
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t* sq = reinterpret_cast<uint32_t*>(smem);
    ActScale* ss = reinterpret_cast<ActScale*>(smem + static_cast<size_t>(NT) * nb * kActQBytes);
    const uint8_t* __restrict__ Wsc = Wq + (RP ? rows * nb * 16 : 0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar row arithmetic
    const int P = nb >> 1;
    const int nblk = NT * nb;  // activation blocks, token-major

    // 1. activation loads (before any weight load)
    //    kXF32: thread t quantizes quad (t & 7) of blocks t / 8 + (THREADS / 8) j
    //    kActGlobal into LDS: thread t copies 16-byte piece t + THREADS j of
    //    the int8 blocks and scale record t + THREADS j
    constexpr int kJ = (1024 * NT * PPL + THREADS - 1) / THREADS;  // nb <= 128 * PPL
    constexpr int kJpre = kJ < 8 ? kJ : 8;
    float4 xv[SRC == kXF32 ? kJpre : 1];
    if constexpr (SRC == kXF32) {
        const float* X = static_cast<const float*>(src);
#pragma unroll
        for (int j = 0; j < kJpre; ++j) {
            const int g = min(static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j, nblk - 1);
            __builtin_memcpy(&xv[j], X + static_cast<int64_t>(g) * kQK + 4 * (threadIdx.x & 7), 16);
        }
    }
    uint32_t areg[kActReg ? NT : 1][2][8];
    ActScale sreg[kActReg ? NT : 1][2];
    if constexpr (SRC == kActGlobal && kActReg) {
        const int p = min(lane, P - 1);
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
    const int64_t S = static_cast<int64_t>(gridDim.x) * kWaves;
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
    const int64_t nk = w0 < rows ? (rows - 1 - w0) / S + 1 : 0;
    // a wave without rows (small matrices) still issues its loads, on the last
    // row, so that no branch leaves the load counters uncertain
    const int64_t rlast = nk > 0 ? w0 + (nk - 1) * S : rows - 1;
    int pp[PPL];
    bool pv[PPL];
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
        pv[i] = lane + 64 * i < P;
        pp[i] = min(lane + 64 * i, P - 1);
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
            const int64_t rb = uniform64(r * nb);
            a.w = Wq + rb * (RP ? 16 : kQ4Bytes);
            a.sc = Wsc + rb * 2;
            a.y = Y + r;
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
    Pair36 raw[D][PPL];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_row(raw[d], d);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 3. activations into LDS, then (one pair per lane) into registers
    if constexpr (kUseLds) {
        if constexpr (SRC == kXF32) {
            const float* X = static_cast<const float*>(src);
            const int m = threadIdx.x & 7;
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                const int g = static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * j;
                const bool valid = g < nblk;
                float4 x;
                if (j < kJpre) {
                    x = xv[j < kJpre ? j : 0];
                } else {
                    __builtin_memcpy(&x, X + static_cast<int64_t>(min(g, nblk - 1)) * kQK + 4 * m, 16);
                }
                if (!valid) x = make_float4(0.f, 0.f, 0.f, 0.f);
                uint32_t word;
                const ActScale sc = quant_act_quad(x.x, x.y, x.z, x.w, m, word);
                if (valid) {
                    sq[g * 8 + m] = word;
                    if (m == 0) ss[g] = sc;
                }
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
            const int p = min(lane, P - 1);
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
    if (nk == 0) return;

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
    for (int64_t k = 0; k < nk; k += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            float part[NT];
            fold(raw[d], part);
            const float t = wave_sums<NT>(part, lane);
            if (k + d < nk && my_token >= 0 && my_token < NT) {
                const RowAt a = row_at(w0 + (k + d) * S);
                a.y[static_cast<int64_t>(my_token) * a.ystride] = t;
            }
            load_row(raw[d], k + d + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

struct Shape {
    int log2G, rpi;
    uint32_t wgs;
    int64_t ntasks;
};

// Launch shape.  A task is RW = 64 / G rows times rpi row slots of one wave;
// waves stride over the tasks.  Each candidate (G lanes per row, rpi rows per
// lane) is scored by
//   util -- the share of a row's pair slots that hold a pair, and
//   fill -- tasks / (rounds x waves), the share of the grid's wave slots that
//           do work over the whole launch (rounds = ceil(tasks / waves)),
// and the best wins; near-ties (within 2 %) go to wider G and more rows per
// lane (more contiguous bytes per row, more loads in flight per lane).
// Several tokens on tall matrices: 16 lanes per row with 4 rows per lane (16
// rows per task) beat 64 when they fill the grid as well -- each lane then
// serves 16 rows per activation read and the per-row butterfly is shorter
// (measured: 128256 x 4096 at N = 8, 126 us against 165 us; on 14336 x 4096,
// where only one row per lane fits, 64 lanes stay better).
Shape pick_shape(const DeviceInfo* dev, int64_t rows, int64_t nb, int threads, int wg_per_cu, int nt) {
    const int waves_per_wg = threads / 64;
    const int64_t cap_wgs = static_cast<int64_t>(dev->num_cu) * wg_per_cu;
    const int64_t max_waves = cap_wgs * waves_per_wg;
    const int64_t P = nb >> 1;
    Shape best{6, 1, 1, 1};
    double best_score = -1.0, g16_score = -1.0;
    Shape g16 = best;
    for (int lg = 6; lg >= 2; --lg) {
        const int64_t G = int64_t(1) << lg;
        const double util = P > 0 ? static_cast<double>(P) / static_cast<double>(((P + G - 1) / G) * G) : 1.0;
        const int64_t RW = 64 >> lg;
        for (int rpi = kRmax; rpi >= 1; rpi >>= 1) {
            const int64_t ntasks = (rows + RW * rpi - 1) / (RW * rpi);
            const int64_t rounds = (ntasks + max_waves - 1) / max_waves;
            const double fill = static_cast<double>(ntasks) / static_cast<double>(rounds * max_waves);
            const double score = util * fill;
            const Shape sh{lg, rpi, 0, ntasks};
            if (score > best_score * 1.02) {
                best_score = score;
                best = sh;
            }
            if (lg == 4 && score > g16_score * 1.02) {
                g16_score = score;
                g16 = sh;
            }
        }
    }
    if (nt >= 2 && best.log2G > 4 && g16.rpi == kRmax && g16_score >= 0.95 * best_score) best = g16;
    int64_t wgs = (best.ntasks + waves_per_wg - 1) / waves_per_wg;
    if (wgs > cap_wgs) wgs = cap_wgs;
    best.wgs = static_cast<uint32_t>(wgs < 1 ? 1 : wgs);
    return best;
}

template <int NT, int THREADS, int SRC, bool DOTS>
hipError_t launch_v(const Shape& sh, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                    float* Y, int32_t* D, const MultiDesc& md, hipStream_t s) {
    const size_t lds = SRC == kActGlobal ? 0 : static_cast<size_t>(NT) * nb * (kActQBytes + kActSBytes);
    const int nbi = static_cast<int>(nb);
    if (lay == kLayRepacked) {
        hipLaunchKernelGGL((k_gemv<NT, THREADS, SRC, DOTS, kLayRepacked>), dim3(sh.wgs), dim3(THREADS), lds, s, Wq,
                           rows, nbi, src, Y, D, sh.log2G, sh.rpi, md);
    } else if (lay == kLayMulti) {
        if constexpr (DOTS) {
            return hipErrorInvalidValue;  // block dots are exported for one matrix only
        } else {
            hipLaunchKernelGGL((k_gemv<NT, THREADS, SRC, false, kLayMulti>), dim3(sh.wgs), dim3(THREADS), lds, s, Wq,
                               rows, nbi, src, Y, D, sh.log2G, sh.rpi, md);
        }
    } else {
        hipLaunchKernelGGL((k_gemv<NT, THREADS, SRC, DOTS, kLayAoS>), dim3(sh.wgs), dim3(THREADS), lds, s, Wq, rows,
                           nbi, src, Y, D, sh.log2G, sh.rpi, md);
    }
    return hipGetLastError();
}

template <int NT>
hipError_t launch_n(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const void* act,
                    float* Y, int32_t* D, const MultiDesc& md, hipStream_t s) {
    const bool lds = static_cast<size_t>(NT) * nb * (kActQBytes + kActSBytes) <= kMaxActLds;
    const Shape sh = pick_shape(dev, rows, nb, 256, 4, NT);
    if (D) {
        return lds ? launch_v<NT, 256, kActLds, true>(sh, lay, Wq, rows, nb, act, Y, D, md, s)
                   : launch_v<NT, 256, kActGlobal, true>(sh, lay, Wq, rows, nb, act, Y, D, md, s);
    }
    return lds ? launch_v<NT, 256, kActLds, false>(sh, lay, Wq, rows, nb, act, Y, D, md, s)
               : launch_v<NT, 256, kActGlobal, false>(sh, lay, Wq, rows, nb, act, Y, D, md, s);
}

// Pairs per lane for the row-streaming kernel, or 0 where it does not apply:
// an even block count, and rows whose pairs fill at least three quarters of
// the lanes (other shapes keep the task kernel above).
int rows_ppl(int64_t nb) {
    if (nb & 1) return 0;
    const int64_t P = nb >> 1;
    for (int ppl = 1; ppl <= kRowsMaxPPL; ppl *= 2)
        if (P <= 64 * ppl) return 4 * P >= 3 * 64 * ppl ? ppl : 0;
    return 0;
}

bool rows_apply(int64_t N, int64_t nb) {
    const int ppl = rows_ppl(nb);
    return ppl > 0 && N >= 1 && N * ppl <= kRowsMaxNtPpl &&
           static_cast<size_t>(N) * nb * (kActQBytes + kActSBytes) <= kRowsMaxLds;
}

// Workgroup size: 16 waves per CU while the token registers leave room for
// four waves per SIMD, 8 waves per CU above that.
template <int NT, int PPL>
constexpr int rows_threads() { return PPL == 1 && NT > 4 ? 512 : 1024; }

template <int SRC, int LAY, int NT, int PPL>
hipError_t launch_rows_k(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                         float* Y, const MultiDesc& md, hipStream_t s) {
    if constexpr (NT * PPL > kRowsMaxNtPpl) {
        return hipErrorInvalidValue;
    } else {
        constexpr int kThreads = rows_threads<NT, PPL>();
        int64_t wgs = (rows + kThreads / 64 - 1) / (kThreads / 64);
        const int64_t cap = static_cast<int64_t>(dev->num_cu) * (1024 / kThreads);
        if (wgs > cap) wgs = cap;
        const size_t lds =
            (SRC == kXF32 || PPL > 1) ? static_cast<size_t>(NT) * nb * (kActQBytes + kActSBytes) : 0;
        hipLaunchKernelGGL((k_gemv_rows<kThreads, NT, PPL, 1, SRC, LAY>), dim3(static_cast<uint32_t>(wgs)),
                           dim3(kThreads), lds, s, Wq, rows, static_cast<int>(nb), src, Y, md);
        return hipGetLastError();
    }
}

template <int SRC, int LAY, int NT>
hipError_t launch_rows_nt(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                          float* Y, const MultiDesc& md, hipStream_t s) {
    switch (rows_ppl(nb)) {
        case 1: return launch_rows_k<SRC, LAY, NT, 1>(dev, Wq, rows, nb, src, Y, md, s);
        case 2: return launch_rows_k<SRC, LAY, NT, 2>(dev, Wq, rows, nb, src, Y, md, s);
        case 4: return launch_rows_k<SRC, LAY, NT, 4>(dev, Wq, rows, nb, src, Y, md, s);
        default: return hipErrorInvalidValue;
    }
}

template <int SRC, int LAY>
hipError_t launch_rows_t(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                         int64_t N, float* Y, const MultiDesc& md, hipStream_t s) {
    switch (N) {
        case 1: return launch_rows_nt<SRC, LAY, 1>(dev, Wq, rows, nb, src, Y, md, s);
        case 2: return launch_rows_nt<SRC, LAY, 2>(dev, Wq, rows, nb, src, Y, md, s);
        case 3: return launch_rows_nt<SRC, LAY, 3>(dev, Wq, rows, nb, src, Y, md, s);
        case 4: return launch_rows_nt<SRC, LAY, 4>(dev, Wq, rows, nb, src, Y, md, s);
        case 5: return launch_rows_nt<SRC, LAY, 5>(dev, Wq, rows, nb, src, Y, md, s);
        case 6: return launch_rows_nt<SRC, LAY, 6>(dev, Wq, rows, nb, src, Y, md, s);
        case 7: return launch_rows_nt<SRC, LAY, 7>(dev, Wq, rows, nb, src, Y, md, s);
        case 8: return launch_rows_nt<SRC, LAY, 8>(dev, Wq, rows, nb, src, Y, md, s);
        default: return hipErrorInvalidValue;
    }
}

template <int SRC>
hipError_t launch_rows(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                       int64_t N, float* Y, const MultiDesc& md, hipStream_t s) {
    switch (lay) {
        case kLayRepacked: return launch_rows_t<SRC, kLayRepacked>(dev, Wq, rows, nb, src, N, Y, md, s);
        case kLayMulti: return launch_rows_t<SRC, kLayMulti>(dev, Wq, rows, nb, src, N, Y, md, s);
        default: return launch_rows_t<SRC, kLayAoS>(dev, Wq, rows, nb, src, N, Y, md, s);
    }
}

int lay_of(WLayout lay) { return lay == kRepacked ? kLayRepacked : kLayAoS; }

// Fused decode (the kernel quantizes X itself): the row-streaming kernel where
// it applies (1..8 tokens); otherwise, for one token, the task kernel in one
// 1024-thread workgroup per CU, so the quantization is repeated once per CU; a
// matrix with fewer tasks than 16 per CU runs in 256-thread workgroups
// instead, spread over more CUs.
hipError_t fused_n(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const float* X,
                   int64_t N, float* Y, const MultiDesc& md, hipStream_t s) {
    if (rows_apply(N, nb)) return launch_rows<kXF32>(dev, lay, Wq, rows, nb, X, N, Y, md, s);
    if (N != 1) return hipErrorInvalidValue;
    const Shape big = pick_shape(dev, rows, nb, 1024, 1, 1);
    if (big.ntasks >= static_cast<int64_t>(dev->num_cu) * 16)
        return launch_v<1, 1024, kXF32, false>(big, lay, Wq, rows, nb, X, Y, nullptr, md, s);
    const Shape small = pick_shape(dev, rows, nb, 256, 4, 1);
    return launch_v<1, 256, kXF32, false>(small, lay, Wq, rows, nb, X, Y, nullptr, md, s);
}

hipError_t gemv_n(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const void* act,
                  int64_t N, float* Y, int32_t* D, const MultiDesc& md, hipStream_t s) {
    if (!D && rows_apply(N, nb)) return launch_rows<kActGlobal>(dev, lay, Wq, rows, nb, act, N, Y, md, s);
    switch (N) {
        case 1: return launch_n<1>(dev, lay, Wq, rows, nb, act, Y, D, md, s);
        case 2: return launch_n<2>(dev, lay, Wq, rows, nb, act, Y, D, md, s);
        case 3: return launch_n<3>(dev, lay, Wq, rows, nb, act, Y, D, md, s);
        case 4: return launch_n<4>(dev, lay, Wq, rows, nb, act, Y, D, md, s);
        case 5: return launch_n<5>(dev, lay, Wq, rows, nb, act, Y, D, md, s);
        case 6: return launch_n<6>(dev, lay, Wq, rows, nb, act, Y, D, md, s);
        case 7: return launch_n<7>(dev, lay, Wq, rows, nb, act, Y, D, md, s);
        case 8: return launch_n<8>(dev, lay, Wq, rows, nb, act, Y, D, md, s);
        default: return hipErrorInvalidValue;
    }
}

const MultiDesc kNoMulti{};

}  // namespace

bool gemv_fuses(int64_t N, int64_t nb) {
    return rows_apply(N, nb) ||
           (N <= kGemvFusedMaxN && static_cast<size_t>(N) * nb * (kActQBytes + kActSBytes) <= kMaxActLds);
}

hipError_t launch_gemv_fused(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                             const float* X, int64_t N, float* Y, hipStream_t s) {
    return fused_n(dev, lay_of(lay), Wq, rows, nb, X, N, Y, kNoMulti, s);
}

hipError_t launch_gemv(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                       const void* act, int64_t N, float* Y, int32_t* D, hipStream_t s) {
    return gemv_n(dev, lay_of(lay), Wq, rows, nb, act, N, Y, D, kNoMulti, s);
}

hipError_t launch_gemv_multi(const DeviceInfo* dev, const MultiDesc& md, int64_t nb, const float* X, const void* act,
                             int64_t N, hipStream_t s) {
    const int64_t rows = md.first[md.count];
    if (X && gemv_fuses(N, nb)) return fused_n(dev, kLayMulti, nullptr, rows, nb, X, N, nullptr, md, s);
    return gemv_n(dev, kLayMulti, nullptr, rows, nb, act, N, nullptr, nullptr, md, s);
}

}  // namespace q4bq
