// Prefill product on the int8 matrix cores, any N.
//
// Same arithmetic as the decode kernel ("llama.cpp 深度解读", section 3: per
// 32-block integer dot of (nibble - 8) with the int8 activations, in int32,
// then the fp32 scale d_w * d_x, summed in fp32), organised as a tiled GEMM:
//  * one v_mfma_i32_32x32x32_i8 covers exactly one 32-value block for a
//    32-token x 32-row tile, so its int32 result is the block dot s for 1024
//    (token, row) pairs at once -- MFMA operand A = activations (tokens),
//    operand B = weights (rows), so each lane's results share one row and the
//    output rows are contiguous for the Y store;
//  * weights are loaded as raw 36-byte block pairs, their nibbles turned into
//    signed int8 (nibble - 8) once per stage and kept in LDS in the same
//    element order as the activations (the contraction order inside a block
//    only has to agree between A and B);
//  * per block each (token, row) result gets one convert, one multiply for
//    the scale product and one FMA into the fp32 accumulator.
// Workgroup tile 128 tokens x 128 rows, 4 waves of 64 x 64 (2 x 2 MFMA tiles),
// 4 blocks (K = 128) per LDS stage.
#include "q4bq_device.h"
#include "q4bq_internal.h"

namespace q4bq {

namespace {

constexpr int kThreads = 256;
constexpr int kBT = 128;  // tokens per workgroup tile
constexpr int kBR = 128;  // rows per workgroup tile
constexpr int kKB = 4;    // blocks per stage

template <bool DOTS>
__global__ void __launch_bounds__(kThreads)
k_gemm(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const uint32_t* __restrict__ act_q,
       const ActScale* __restrict__ act_s, int64_t N, float* __restrict__ Y, int32_t* __restrict__ D) {
    __shared__ __align__(16) uint32_t sA[kKB * kBT * 8];  // activations, dot order
    __shared__ __align__(16) float sAd[kKB * kBT];
    __shared__ __align__(16) uint32_t sB[kKB * kBR * 8];  // weights as signed int8, dot order
    __shared__ __align__(16) float sBd[kKB * kBR];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1;   // token half of the tile
    const int wn = wave & 1;    // row half of the tile
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kBR;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kBT;

    float acc[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    for (int b0 = 0; b0 < nb; b0 += kKB) {
        // activations: 128 tokens x 4 blocks x 32 bytes, 16 bytes per thread-load
#pragma unroll
        for (int it = 0; it < (kBT * kKB * 2) / kThreads; ++it) {
            const int c = it * kThreads + t;
            const int tok = c >> 3;
            const int blk = (c >> 1) & 3;
            const int half = c & 1;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (n0 + tok < N && b0 + blk < nb)
                v = reinterpret_cast<const u32x4*>(act_q + ((n0 + tok) * nb + b0 + blk) * 8)[half];
            reinterpret_cast<u32x4*>(sA)[(blk * kBT + tok) * 2 + half] = v;
        }
#pragma unroll
        for (int it = 0; it < (kBT * kKB) / kThreads; ++it) {
            const int c = it * kThreads + t;
            const int tok = c >> 2;
            const int blk = c & 3;
            float d = 0.0f;
            if (n0 + tok < N && b0 + blk < nb) d = act_s[(n0 + tok) * nb + b0 + blk].d;
            sAd[blk * kBT + tok] = d;
        }
        // weights: 128 rows x 2 block pairs, one pair per thread
        {
            const int row = t >> 1;
            const int pr = t & 1;
            const int b = b0 + 2 * pr;
            const int64_t r = r0 + row;
            Block4 blk[2];
            bool ok[2] = {false, false};
            if (r < rows && b < nb) {
                const uint8_t* p = Wq + (r * nb + b) * kQ4Bytes;
                if (b + 1 < nb) {
                    const Pair36 raw = load_pair(p);
                    blk[0] = pair_first(raw);
                    blk[1] = pair_second(raw);
                    ok[0] = ok[1] = true;
                } else {
                    blk[0] = load_block(p);
                    ok[0] = true;
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 lo = {0u, 0u, 0u, 0u}, hi4 = {0u, 0u, 0u, 0u};
                float d = 0.0f;
                if (ok[h]) {
                    lo = u32x4{nib_to_s8(nib_lo(blk[h].qs[0])), nib_to_s8(nib_hi(blk[h].qs[0])),
                               nib_to_s8(nib_lo(blk[h].qs[1])), nib_to_s8(nib_hi(blk[h].qs[1]))};
                    hi4 = u32x4{nib_to_s8(nib_lo(blk[h].qs[2])), nib_to_s8(nib_hi(blk[h].qs[2])),
                                nib_to_s8(nib_lo(blk[h].qs[3])), nib_to_s8(nib_hi(blk[h].qs[3]))};
                    d = half_bits_to_float(blk[h].dbits);
                }
                const int bb = 2 * pr + h;
                reinterpret_cast<u32x4*>(sB)[(bb * kBR + row) * 2 + 0] = lo;
                reinterpret_cast<u32x4*>(sB)[(bb * kBR + row) * 2 + 1] = hi4;
                sBd[bb * kBR + row] = d;
            }
        }
        __syncthreads();

#pragma unroll
        for (int blk = 0; blk < kKB; ++blk) {
            i32x4 a[2], w[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = reinterpret_cast<const i32x4*>(sA)[(blk * kBT + wm * 64 + i * 32 + l32) * 2 + hi];
#pragma unroll
            for (int j = 0; j < 2; ++j)
                w[j] = reinterpret_cast<const i32x4*>(sB)[(blk * kBR + wn * 64 + j * 32 + l32) * 2 + hi];
            i32x16 s[2][2];
            const i32x16 zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) s[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], w[j], zero, 0, 0, 0);

            if constexpr (DOTS) {
                const int b = b0 + blk;
                if (b < nb) {
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const int64_t r = r0 + wn * 64 + j * 32 + l32;
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const int64_t n = n0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
                                if (n < N && r < rows) D[(n * rows + r) * nb + b] = s[i][j][v];
                            }
                        }
                }
            } else {
                float dw[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) dw[j] = sBd[blk * kBR + wn * 64 + j * 32 + l32];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    float dx[16];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float4 q = reinterpret_cast<const float4*>(sAd)[(blk * kBT + wm * 64 + i * 32 + 8 * m + 4 * hi) >> 2];
                        dx[4 * m + 0] = q.x;
                        dx[4 * m + 1] = q.y;
                        dx[4 * m + 2] = q.z;
                        dx[4 * m + 3] = q.w;
                    }
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            acc[i][j][v] = fmaf(static_cast<float>(s[i][j][v]), dx[v] * dw[j], acc[i][j][v]);
                }
            }
        }
        __syncthreads();
    }

    if constexpr (!DOTS) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t r = r0 + wn * 64 + j * 32 + l32;
                if (r >= rows) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t n = n0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
                    if (n < N) Y[n * rows + r] = acc[i][j][v];
                }
            }
    }
}

}  // namespace

hipError_t launch_gemm(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* act,
                       int64_t N, float* Y, int32_t* D, hipStream_t s) {
    (void)dev;
    const uint32_t* aq = static_cast<const uint32_t*>(act);
    const ActScale* as = reinterpret_cast<const ActScale*>(static_cast<const uint8_t*>(act) + N * nb * kActQBytes);
    const dim3 grid(static_cast<uint32_t>((rows + kBR - 1) / kBR), static_cast<uint32_t>((N + kBT - 1) / kBT));
    if (D)
        hipLaunchKernelGGL(k_gemm<true>, grid, dim3(kThreads), 0, s, Wq, rows, static_cast<int>(nb), aq, as, N, Y, D);
    else
        hipLaunchKernelGGL(k_gemm<false>, grid, dim3(kThreads), 0, s, Wq, rows, static_cast<int>(nb), aq, as, N, Y, D);
    return hipGetLastError();
}

}  // namespace q4bq
