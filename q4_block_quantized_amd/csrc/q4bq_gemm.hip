// Prefill product on the matrix cores, N > 8 tokens.
//
// Same arithmetic as the decode kernel ("llama.cpp 深度解读", luoboask.github.io,
// section 3 "量化矩阵乘法 — 核心算子": per 32-value block the integer dot of
// (nibble - 8) with the int8 activations, then the fp32 scale d_w * d_x, the
// scaled block terms summed in fp32), organised as a tiled GEMM:
//  * the block dot runs on the fp6 matrix cores, exactly: the weights enter as
//    e2m3 codes of (nibble - 8)/2, the activations as e2m3 codes of h/2 and l/2
//    (y = 16h + l), with E8M0 block scales x2, x32 and x2; one
//    v_mfma_scale_f32_32x32x64_f8f6f4 yields s for a 32-token x 32-row tile
//    as an exact fp32 integer, with no int->float conversion;
//  * the 1024 scale products d_x * d_w of a tile come from one
//    v_mfma_f32_32x32x16_f16 outer product (binary16 x binary16 is exact in
//    fp32), so each (token, row, block) costs a single FMA on the vector ALU;
//  * operand A = activations (tokens), B = weights (rows): each lane's
//    results share one row, so the fp32 Y stores are contiguous;
//  * weights are read as raw 36-byte block pairs and turned into fp6 codes
//    while they are staged into LDS; the next stage's global loads are in
//    flight while the current stage computes.
// Workgroup tile 128 tokens x 128 rows, 4 waves of 64 x 64 (2 x 2 MFMA tiles),
// 4 blocks (K = 128) per stage.
#include "q4bq_device.h"
#include "q4bq_internal.h"

namespace q4bq {

namespace {

constexpr int kThreads = 256;
constexpr int kBT = 128;  // tokens per workgroup tile
constexpr int kBR = 128;  // rows per workgroup tile
constexpr int kKB = 4;    // blocks per stage

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// LDS strides (in dwords).  An activation record (64 bytes) sits in 80 bytes
// and a weight slot (24 bytes) in 48, so the 16 lanes that one 16-byte LDS read
// serves at a time hit 16 disjoint groups of 4 banks; each block plane is
// skewed by 16 dwords so the staging writes of one token (or row) spread too.
constexpr int kRecA = 20;
constexpr int kRecB = 12;
constexpr int kPlaneA = kBT * kRecA + 16;
constexpr int kPlaneB = kBR * kRecB + 16;

// E8M0 block scales: 127 is x1.
constexpr int kScaleW = 128;       // weights hold (nibble - 8) / 2
constexpr int kScaleHi = 127 + 5;  // activation high part holds h / 2, weight 16 h
constexpr int kScaleLo = 128;      // activation low part holds l / 2

template <bool DOTS>
__global__ void __launch_bounds__(kThreads)
k_gemm(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const uint32_t* __restrict__ act_rec,
       const uint16_t* __restrict__ act_dx, int64_t N, float* __restrict__ Y, int32_t* __restrict__ D) {
    __shared__ __align__(16) uint32_t sA[kKB * kPlaneA];  // activation records, 80-byte stride
    __shared__ __align__(16) uint32_t sB[kKB * kPlaneB];  // 24 bytes of weight codes, 48-byte stride
    __shared__ __align__(16) uint16_t sAd[kKB * kBT];      // activation scale bits
    __shared__ __align__(16) uint16_t sBd[kKB * kBR];      // weight scale bits

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1;  // token half of the tile
    const int wn = wave & 1;   // row half of the tile
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kBR;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * kBT;

    // staging registers for one stage
    u32x4 ra[8];
    uint16_t rdx[2];
    Pair36 rw;
    bool rw_ok[2];

    auto load_stage = [&](int b0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = i * kThreads + t;
            const int tok = c >> 4;
            const int blk = (c >> 2) & 3;
            const int q = c & 3;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (n0 + tok < N && b0 + blk < nb)
                v = reinterpret_cast<const u32x4*>(act_rec)[((n0 + tok) * nb + b0 + blk) * 4 + q];
            ra[i] = v;
        }
        {
            const int tok = t >> 1;
            const int pr = t & 1;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int b = b0 + 2 * pr + h;
                rdx[h] = (n0 + tok < N && b < nb) ? act_dx[(n0 + tok) * nb + b] : static_cast<uint16_t>(0);
            }
        }
        {
            const int row = t >> 1;
            const int b = b0 + 2 * (t & 1);
            const int64_t r = r0 + row;
            rw_ok[0] = rw_ok[1] = false;
            if (r < rows && b < nb) {
                const uint8_t* p = Wq + (r * nb + b) * kQ4Bytes;
                if (b + 1 < nb) {
                    rw = load_pair(p);
                    rw_ok[0] = rw_ok[1] = true;
                } else {
                    // a lone last block: load only its 18 bytes
                    const Block4 one = load_block(p);
                    rw.w[0] = one.dbits;
#pragma unroll
                    for (int k = 0; k < 4; ++k) rw.w[5 + k] = one.qs[k];
                    rw_ok[0] = true;
                }
            }
        }
    };

    auto store_stage = [&](int b0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = i * kThreads + t;
            const int tok = c >> 4;
            const int blk = (c >> 2) & 3;
            const int q = c & 3;
            *reinterpret_cast<u32x4*>(sA + blk * kPlaneA + tok * kRecA + q * 4) = ra[i];
        }
        {
            const int tok = t >> 1;
            const int pr = t & 1;
            sAd[(2 * pr) * kBT + tok] = rdx[0];
            sAd[(2 * pr + 1) * kBT + tok] = rdx[1];
        }
        {
            const int row = t >> 1;
            const int pr = t & 1;
            const bool lone = rw_ok[0] && !rw_ok[1] && (b0 + 2 * pr + 1 >= nb);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t d6[6] = {0u, 0u, 0u, 0u, 0u, 0u};
                uint32_t dbits = 0u;
                if (rw_ok[h]) {
                    Block4 blk;
                    if (lone) {
                        blk.dbits = rw.w[0];
#pragma unroll
                        for (int k = 0; k < 4; ++k) blk.qs[k] = rw.w[5 + k];
                    } else {
                        blk = h ? pair_second(rw) : pair_first(rw);
                    }
                    weight_fp6(blk.qs, d6);
                    dbits = blk.dbits;
                }
                const int bb = 2 * pr + h;
                uint32_t* dst = sB + bb * kPlaneB + row * kRecB;
                reinterpret_cast<u32x4*>(dst)[0] = u32x4{d6[0], d6[1], d6[2], d6[3]};
                reinterpret_cast<u32x2*>(dst)[2] = u32x2{d6[4], d6[5]};
                sBd[bb * kBR + row] = static_cast<uint16_t>(dbits);
            }
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int scale_a = half ? kScaleLo : kScaleHi;

    load_stage(0);
    for (int b0 = 0; b0 < nb; b0 += kKB) {
        store_stage(b0);
        __syncthreads();
        if (b0 + kKB < nb) load_stage(b0 + kKB);

#pragma unroll 1
        for (int blk = 0; blk < kKB; ++blk) {
            i32x8 a[2], w[2];
            f16x8 ap[2], wp[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t* src = sA + blk * kPlaneA + (wm * 64 + i * 32 + l32) * kRecA + half * 8;
                const u32x4 x = reinterpret_cast<const u32x4*>(src)[0];
                const u32x2 y = reinterpret_cast<const u32x2*>(src)[2];
                a[i] = i32x8{static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z),
                             static_cast<int>(x.w), static_cast<int>(y.x), static_cast<int>(y.y), 0, 0};
                const uint16_t db = half ? static_cast<uint16_t>(0) : sAd[blk * kBT + wm * 64 + i * 32 + l32];
                ap[i] = f16x8{__builtin_bit_cast(_Float16, db), 0, 0, 0, 0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t* src = sB + blk * kPlaneB + (wn * 64 + j * 32 + l32) * kRecB;
                const u32x4 x = reinterpret_cast<const u32x4*>(src)[0];
                const u32x2 y = reinterpret_cast<const u32x2*>(src)[2];
                w[j] = i32x8{static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z),
                             static_cast<int>(x.w), static_cast<int>(y.x), static_cast<int>(y.y), 0, 0};
                const uint16_t db = half ? static_cast<uint16_t>(0) : sBd[blk * kBR + wn * 64 + j * 32 + l32];
                wp[j] = f16x8{__builtin_bit_cast(_Float16, db), 0, 0, 0, 0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const f32x16 s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        a[i], w[j], zero, 2, 2, 0, scale_a, 0, kScaleW);
                    if constexpr (DOTS) {
                        const int b = b0 + blk;
                        const int64_t r = r0 + wn * 64 + j * 32 + l32;
                        if (b < nb && r < rows) {
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const int64_t n = n0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                                if (n < N) D[(n * rows + r) * nb + b] = static_cast<int32_t>(s[v]);
                            }
                        }
                    } else {
                        const f32x16 p = __builtin_amdgcn_mfma_f32_32x32x16_f16(ap[i], wp[j], zero, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(s[v], p[v], acc[i][j][v]);
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
                    const int64_t n = n0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                    if (n < N) Y[n * rows + r] = acc[i][j][v];
                }
            }
    }
}

}  // namespace

hipError_t launch_gemm(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* act,
                       int64_t N, float* Y, int32_t* D, hipStream_t s) {
    (void)dev;
    const uint32_t* rec = static_cast<const uint32_t*>(act);
    const uint16_t* dxb = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(act) + N * nb * kAct6Bytes);
    const dim3 grid(static_cast<uint32_t>((rows + kBR - 1) / kBR), static_cast<uint32_t>((N + kBT - 1) / kBT));
    if (D)
        hipLaunchKernelGGL(k_gemm<true>, grid, dim3(kThreads), 0, s, Wq, rows, static_cast<int>(nb), rec, dxb, N, Y,
                           D);
    else
        hipLaunchKernelGGL(k_gemm<false>, grid, dim3(kThreads), 0, s, Wq, rows, static_cast<int>(nb), rec, dxb, N, Y,
                           D);
    return hipGetLastError();
}

}  // namespace q4bq
