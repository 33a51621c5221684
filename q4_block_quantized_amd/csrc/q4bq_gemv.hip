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

template <int NT, int THREADS, int SRC, bool DOTS, bool RP>
__global__ void __launch_bounds__(THREADS)
k_gemv(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const void* __restrict__ src,
       float* __restrict__ Y, int32_t* __restrict__ D, int log2G, int rpi) {
    constexpr int kWaves = THREADS / 64;
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
                        raw[j][u] = RP ? load_pair_rp(Wq + blk0 * 16, Wsc + blk0 * 2) : load_pair(Wq + blk0 * kQ4Bytes);
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
                const Block4 blk = RP ? load_block_rp(Wq + bi * 16, Wsc + bi * 2) : load_block(Wq + bi * kQ4Bytes);
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
                    for (int n = 0; n < NT; ++n) Y[static_cast<int64_t>(n) * rows + r[j]] = acc[j][n];
                }
            }
        }
    }
}

// Lanes per row: the power of two in [4, 64] that leaves the fewest idle
// pair slots, the widest among equals (wider = more contiguous bytes per row).
int pick_log2g(int64_t P) {
    int best = 6;
    double best_util = -1.0;
    for (int lg = 6; lg >= 2; --lg) {
        const int64_t G = int64_t(1) << lg;
        const int64_t slots = ((P + G - 1) / G) * G;
        const double util = slots > 0 ? static_cast<double>(P) / static_cast<double>(slots) : 1.0;
        if (util > best_util + 1e-9) {
            best_util = util;
            best = lg;
        }
    }
    return best;
}

struct Shape {
    int log2G, rpi;
    uint32_t wgs;
};

// Launch shape: rows per lane = as many (up to 4) as still leave `want_waves`
// tasks; workgroups capped at `wg_per_cu` per CU (the grid strides over tasks).
// Several tokens: with enough rows, 16 lanes per row (4 rows per wave and row
// slot) beat 64 -- each lane then serves 4 x rpi rows per activation read and
// the per-row butterfly is shorter (measured: 128256 x 4096 at N = 8, 126 us
// against 165 us); with few rows the wider groups keep more waves busy.
Shape pick_shape(const DeviceInfo* dev, int64_t rows, int64_t nb, int threads, int wg_per_cu, int want_waves_per_cu,
                 int nt) {
    Shape sh;
    sh.log2G = pick_log2g(nb >> 1);
    const int64_t want_tasks = static_cast<int64_t>(dev->num_cu) * want_waves_per_cu;
    if (nt >= 2 && sh.log2G > 4 && (rows + 16 * kRmax - 1) / (16 * kRmax) >= want_tasks) sh.log2G = 4;
    const int RW = 64 >> sh.log2G;
    sh.rpi = 1;
    for (int c = kRmax; c >= 1; c >>= 1) {
        if ((rows + int64_t(RW) * c - 1) / (int64_t(RW) * c) >= want_tasks) {
            sh.rpi = c;
            break;
        }
    }
    const int waves = threads / 64;
    const int64_t ntasks = (rows + int64_t(RW) * sh.rpi - 1) / (int64_t(RW) * sh.rpi);
    int64_t wgs = (ntasks + waves - 1) / waves;
    const int64_t cap = static_cast<int64_t>(dev->num_cu) * wg_per_cu;
    if (wgs > cap) wgs = cap;
    sh.wgs = static_cast<uint32_t>(wgs < 1 ? 1 : wgs);
    return sh;
}

template <int NT, int THREADS, int SRC, bool DOTS>
hipError_t launch_v(const Shape& sh, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb, const void* src,
                    float* Y, int32_t* D, hipStream_t s) {
    const size_t lds = SRC == kActGlobal ? 0 : static_cast<size_t>(NT) * nb * (kActQBytes + kActSBytes);
    if (lay == kRepacked)
        hipLaunchKernelGGL((k_gemv<NT, THREADS, SRC, DOTS, true>), dim3(sh.wgs), dim3(THREADS), lds, s, Wq, rows,
                           static_cast<int>(nb), src, Y, D, sh.log2G, sh.rpi);
    else
        hipLaunchKernelGGL((k_gemv<NT, THREADS, SRC, DOTS, false>), dim3(sh.wgs), dim3(THREADS), lds, s, Wq, rows,
                           static_cast<int>(nb), src, Y, D, sh.log2G, sh.rpi);
    return hipGetLastError();
}

template <int NT>
hipError_t launch_n(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb, const void* act,
                    float* Y, int32_t* D, hipStream_t s) {
    const bool lds = static_cast<size_t>(NT) * nb * (kActQBytes + kActSBytes) <= kMaxActLds;
    const Shape sh = pick_shape(dev, rows, nb, 256, 4, 16, NT);
    if (D) {
        return lds ? launch_v<NT, 256, kActLds, true>(sh, lay, Wq, rows, nb, act, Y, D, s)
                   : launch_v<NT, 256, kActGlobal, true>(sh, lay, Wq, rows, nb, act, Y, D, s);
    }
    return lds ? launch_v<NT, 256, kActLds, false>(sh, lay, Wq, rows, nb, act, Y, D, s)
               : launch_v<NT, 256, kActGlobal, false>(sh, lay, Wq, rows, nb, act, Y, D, s);
}

}  // namespace

bool gemv_fuses(int64_t N, int64_t nb) {
    return N <= kGemvFusedMaxN && static_cast<size_t>(N) * nb * (kActQBytes + kActSBytes) <= kMaxActLds;
}

hipError_t launch_gemv_fused(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                             const float* X, int64_t N, float* Y, hipStream_t s) {
    const Shape sh = pick_shape(dev, rows, nb, 1024, 1, 16, static_cast<int>(N));
    switch (N) {
        case 1: return launch_v<1, 1024, kXF32, false>(sh, lay, Wq, rows, nb, X, Y, nullptr, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                       const void* act, int64_t N, float* Y, int32_t* D, hipStream_t s) {
    switch (N) {
        case 1: return launch_n<1>(dev, lay, Wq, rows, nb, act, Y, D, s);
        case 2: return launch_n<2>(dev, lay, Wq, rows, nb, act, Y, D, s);
        case 3: return launch_n<3>(dev, lay, Wq, rows, nb, act, Y, D, s);
        case 4: return launch_n<4>(dev, lay, Wq, rows, nb, act, Y, D, s);
        case 5: return launch_n<5>(dev, lay, Wq, rows, nb, act, Y, D, s);
        case 6: return launch_n<6>(dev, lay, Wq, rows, nb, act, Y, D, s);
        case 7: return launch_n<7>(dev, lay, Wq, rows, nb, act, Y, D, s);
        case 8: return launch_n<8>(dev, lay, Wq, rows, nb, act, Y, D, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace q4bq
