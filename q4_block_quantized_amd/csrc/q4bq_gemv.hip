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


template <int NT, int THREADS, int SRC, bool DOTS, int LAY, bool EPI>
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
            // the fused form may LayerNorm the one token first: fp64 mean and
            // population variance over the workgroup, then each value
            // normalized in fp64 and rounded once to fp32
            constexpr bool kLn = EPI && NT == 1;
            const bool do_ln = kLn && md.epi.ln_gamma != nullptr;
            double mu = 0.0, rstd = 0.0;
            // a token of at most kLnRegQ quads per thread is read once, into
            // registers, with its gamma and beta; longer ones in three passes
            constexpr int kLnRegQ = 4;
            bool ln_done = false;
            if constexpr (kLn) {
                if (do_ln && nblk <= kLnRegQ * (THREADS / 8)) {
                    __shared__ double redr[2][THREADS / 64];
                    const int qn = (nblk + THREADS / 8 - 1) / (THREADS / 8);  // quad rounds, <= kLnRegQ
                    float4 xr[kLnRegQ], gr[kLnRegQ], br[kLnRegQ];
#pragma unroll
                    for (int i = 0; i < kLnRegQ; ++i) {
                        if (i >= qn) break;
                        const int g = min(static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * i, nblk - 1);
                        const int64_t k = static_cast<int64_t>(g) * kQK + 4 * m;
                        __builtin_memcpy(&xr[i], X + k, 16);
                        __builtin_memcpy(&gr[i], md.epi.ln_gamma + k, 16);
                        __builtin_memcpy(&br[i], md.epi.ln_beta + k, 16);
                    }
                    const double kk = static_cast<double>(nb) * kQK;
                    double s1 = 0.0;
#pragma unroll
                    for (int i = 0; i < kLnRegQ; ++i) {
                        if (i >= qn) break;
                        if (static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * i < nblk) s1 += quad_sum_f64(xr[i]);
                    }
                    mu = wg_sum_f64<THREADS>(s1, redr[0]) / kk;
                    double s2 = 0.0;
#pragma unroll
                    for (int i = 0; i < kLnRegQ; ++i) {
                        if (i >= qn) break;
                        if (static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * i < nblk)
                            s2 += quad_sqdev_f64(xr[i], mu);
                    }
                    rstd = 1.0 / sqrt(wg_sum_f64<THREADS>(s2, redr[1]) / kk + static_cast<double>(md.epi.ln_eps));
#pragma unroll
                    for (int i = 0; i < kLnRegQ; ++i) {
                        if (i >= qn) break;
                        const int g = static_cast<int>(threadIdx.x >> 3) + (THREADS / 8) * i;
                        const float4 x = ln_quad(xr[i], mu, rstd, gr[i], br[i]);
                        uint32_t word;
                        const ActScale sc = quant_act_quad(x.x, x.y, x.z, x.w, m, word);
                        if (g < nblk) {
                            sq[g * 8 + m] = word;
                            if (m == 0) ss[g] = sc;
                        }
                    }
                    ln_done = true;
                } else if (do_ln) {
                    __shared__ double red[2][THREADS / 64];
                    const double kk = static_cast<double>(nb) * kQK;
                    double s1 = 0.0;
                    for (int g = threadIdx.x >> 3; g < nblk; g += THREADS / 8) {
                        float4 x;
                        __builtin_memcpy(&x, X + static_cast<int64_t>(g) * kQK + 4 * m, 16);
                        s1 += quad_sum_f64(x);
                    }
                    mu = wg_sum_f64<THREADS>(s1, red[0]) / kk;
                    double s2 = 0.0;
                    for (int g = threadIdx.x >> 3; g < nblk; g += THREADS / 8) {
                        float4 x;
                        __builtin_memcpy(&x, X + static_cast<int64_t>(g) * kQK + 4 * m, 16);
                        s2 += quad_sqdev_f64(x, mu);
                    }
                    rstd = 1.0 / sqrt(wg_sum_f64<THREADS>(s2, red[1]) / kk + static_cast<double>(md.epi.ln_eps));
                }
            }
            for (int g0 = (threadIdx.x >> 3) & ~7; !ln_done && g0 < nblk; g0 += THREADS / 8) {
                const int g = g0 + ((threadIdx.x >> 3) & 7);
                const bool valid = g < nblk;
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
                if (valid) __builtin_memcpy(&x, X + static_cast<int64_t>(g) * kQK + 4 * m, 16);
                if constexpr (kLn) {
                    if (do_ln && valid) {
                        float4 gq, bq;
                        __builtin_memcpy(&gq, md.epi.ln_gamma + static_cast<int64_t>(g) * kQK + 4 * m, 16);
                        __builtin_memcpy(&bq, md.epi.ln_beta + static_cast<int64_t>(g) * kQK + 4 * m, 16);
                        x = ln_quad(x, mu, rstd, gq, bq);
                    }
                }
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
        // fused forms: the rows' epilogue operands, fetched before the weights
        float eb[EPI ? kRmax : 1], em[EPI ? kRmax : 1][EPI ? NT : 1];
        if constexpr (EPI) {
#pragma unroll
            for (int j = 0; j < kRmax; ++j) {
                const int64_t rr = rv[j] ? r[j] : 0;
                eb[j] = epi_bias(md.epi, rr);
#pragma unroll
                for (int n = 0; n < NT; ++n) em[j][n] = epi_mul(md.epi, n, rr, rows);
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
                    for (int n = 0; n < NT; ++n)
                        yrow[j][static_cast<int64_t>(n) * ystride[j]] =
                            EPI ? epilogue_with(acc[j][n], eb[j], em[j][n], md.epi) : acc[j][n];
                }
            }
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
    const bool fused = md.epi.bias || md.epi.mul || md.epi.act != kEpiNone || md.epi.ln_gamma;
    if (lay == kLayRepacked) {
        if (fused) return hipErrorInvalidValue;  // the fused forms take the pages' blocks
        hipLaunchKernelGGL((k_gemv<NT, THREADS, SRC, DOTS, kLayRepacked, false>), dim3(sh.wgs), dim3(THREADS), lds, s,
                           Wq, rows, nbi, src, Y, D, sh.log2G, sh.rpi, md);
    } else if (lay == kLayMulti) {
        if constexpr (DOTS) {
            return hipErrorInvalidValue;  // block dots are exported for one matrix only
        } else {
            hipLaunchKernelGGL((k_gemv<NT, THREADS, SRC, false, kLayMulti, false>), dim3(sh.wgs), dim3(THREADS), lds,
                               s, Wq, rows, nbi, src, Y, D, sh.log2G, sh.rpi, md);
        }
    } else if (fused && !DOTS && (SRC != kXF32 || NT == 1)) {
        if constexpr (!DOTS && (SRC != kXF32 || NT == 1)) {
            if (md.epi.ln_gamma && SRC != kXF32) return hipErrorInvalidValue;  // LayerNorm: fp32 X only
            hipLaunchKernelGGL((k_gemv<NT, THREADS, SRC, false, kLayAoS, true>), dim3(sh.wgs), dim3(THREADS), lds, s,
                               Wq, rows, nbi, src, Y, D, sh.log2G, sh.rpi, md);
        }
    } else {
        if (fused) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_gemv<NT, THREADS, SRC, DOTS, kLayAoS, false>), dim3(sh.wgs), dim3(THREADS), lds, s, Wq,
                           rows, nbi, src, Y, D, sh.log2G, sh.rpi, md);
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

int lay_of(WLayout lay) { return lay == kRepacked ? kLayRepacked : kLayAoS; }

// Fused decode (the kernel quantizes X itself): the row-streaming kernel where
// it applies (1..8 tokens); otherwise, for one token, the task kernel in one
// 1024-thread workgroup per CU, so the quantization is repeated once per CU; a
// matrix with fewer tasks than 16 per CU runs in 256-thread workgroups
// instead, spread over more CUs.
hipError_t fused_n(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const float* X,
                   int64_t N, float* Y, const MultiDesc& md, hipStream_t s) {
    const MultiDesc* mdp = lay == kLayMulti ? &md : nullptr;
    if (mma_apply(N, nb, rows, mdp)) return launch_gemv_mma(dev, lay, Wq, rows, nb, X, true, N, Y, md, s);
    if (rows_apply(N, nb, rows)) return launch_rows_x(dev, lay, Wq, rows, nb, X, N, Y, md, s);
    if (N != 1) return hipErrorInvalidValue;
    const Shape big = pick_shape(dev, rows, nb, 1024, 1, 1);
    if (big.ntasks >= static_cast<int64_t>(dev->num_cu) * 16)
        return launch_v<1, 1024, kXF32, false>(big, lay, Wq, rows, nb, X, Y, nullptr, md, s);
    const Shape small = pick_shape(dev, rows, nb, 256, 4, 1);
    return launch_v<1, 256, kXF32, false>(small, lay, Wq, rows, nb, X, Y, nullptr, md, s);
}

hipError_t gemv_n(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const void* act,
                  int64_t N, float* Y, int32_t* D, const MultiDesc& md, hipStream_t s) {
    if (!D && mma_apply(N, nb, rows, lay == kLayMulti ? &md : nullptr))
        return launch_gemv_mma(dev, lay, Wq, rows, nb, act, false, N, Y, md, s);
    if (rows_apply(N, nb, rows)) return launch_rows_act(dev, lay, Wq, rows, nb, act, N, Y, md, s, D);
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

bool gemv_fuses(int64_t N, int64_t nb, int64_t rows, const MultiDesc* md) {
    return mma_apply(N, nb, rows, md) || rows_apply(N, nb, rows) ||
           (N <= kGemvFusedMaxN && static_cast<size_t>(N) * nb * (kActQBytes + kActSBytes) <= kMaxActLds);
}

// With several tokens, every workgroup of the fused kernel quantizes all of X
// itself, and past N * K = 16384 values that prologue costs more than one
// separate quantizer launch into a caller's workspace (measured on 4096 x
// 14336 at N = 2, 4, 8 and on 14336 x 4096 and 128256 x 4096 at N = 8; below
// it, e.g. 4096- and 14336-row matrices with K = 4096 at N = 4, the fused
// kernel is faster).
constexpr int64_t kFusedMaxValues = 16384;

bool gemv_prefers_fused(int64_t N, int64_t nb, int64_t rows, const MultiDesc* md) {
    return gemv_fuses(N, nb, rows, md) && (N == 1 || N * nb * kQK <= kFusedMaxValues);
}

hipError_t launch_gemv_fused(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                             const float* X, int64_t N, float* Y, hipStream_t s) {
    return fused_n(dev, lay_of(lay), Wq, rows, nb, X, N, Y, kNoMulti, s);
}

bool gemv_fuses_epi(int64_t nb, int64_t rows) {
    return rows_apply(1, nb, rows) ? rows_fuse_prologue(nb, rows) : gemv_fuses(1, nb, rows);
}

hipError_t launch_gemv_fused_epi(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const float* X,
                                 float* Y, const Epilogue& epi, hipStream_t s) {
    if (!gemv_fuses_epi(nb, rows)) return hipErrorInvalidValue;
    MultiDesc md = kNoMulti;
    md.epi = epi;
    return fused_n(dev, kLayAoS, Wq, rows, nb, X, 1, Y, md, s);
}

hipError_t launch_gemv(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                       const void* act, int64_t N, float* Y, int32_t* D, hipStream_t s, const Epilogue& epi) {
    MultiDesc md = kNoMulti;
    md.epi = epi;
    return gemv_n(dev, lay_of(lay), Wq, rows, nb, act, N, Y, D, md, s);
}

hipError_t launch_gemv_multi(const DeviceInfo* dev, const MultiDesc& md, int64_t nb, const float* X, const void* act,
                             int64_t N, hipStream_t s) {
    const int64_t rows = md.first[md.count];
    if (X && gemv_fuses(N, nb, rows, &md)) return fused_n(dev, kLayMulti, nullptr, rows, nb, X, N, nullptr, md, s);
    return gemv_n(dev, kLayMulti, nullptr, rows, nb, act, N, nullptr, nullptr, md, s);
}

}  // namespace q4bq
