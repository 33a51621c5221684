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
//    v_mfma_f32_32x32x8_f16 outer product (binary16 x binary16 is exact in
//    fp32), so each (token, row, block) costs a single FMA on the vector ALU;
//  * every operand is two or one plain LDS reads: the records carry their
//    zero padding and the scales come pre-replicated;
//  * operand A = activations (tokens), B = weights (rows): each lane's
//    results share one row, so the fp32 Y stores are contiguous;
//  * weights are read as raw 18-byte blocks and turned into fp6 codes
//    while they are staged into LDS; the next stage's global loads are in
//    flight while the current stage computes.
// Workgroup tile 256 tokens x 128 rows, 8 waves of 64 x 64 (2 x 2 MFMA tiles),
// 4 blocks (K = 128) per stage; each thread converts one weight block per stage.
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
constexpr int kActChunks = kBT * kKB * 4 / kThreads;  // 16-byte activation chunks per thread per stage
static_assert(kBR * kKB == kThreads, "one weight block per thread per stage");
static_assert(kBT * kKB <= 2 * kThreads, "activation scales: at most two per thread");

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
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
// The scale-product MFMA (32x32x8 f16) reads 4 copies of d in each K half, so
// it returns 8 * d_x * d_w; the block dot is taken 8 times smaller to match
// (exact: a power of two on an integer well inside the fp32 range).
constexpr int kScaleDown = 3;

template <bool DOTS>
__global__ void __launch_bounds__(kThreads)
k_gemm(const uint8_t* __restrict__ Wq, int64_t rows, int nb, const uint32_t* __restrict__ act_rec,
       const uint16_t* __restrict__ act_dx, int64_t N, float* __restrict__ Y, int32_t* __restrict__ D) {
    __shared__ __align__(16) uint32_t sA[kKB * kPlaneA];  // activation records, 80-byte stride
    __shared__ __align__(16) uint32_t sB[kKB * kPlaneB];  // 24 bytes of weight codes, 48-byte stride
    __shared__ __align__(16) u32x2 sAd[kKB * kBT];        // activation scale bits, 4 copies
    __shared__ __align__(16) u32x2 sBd[kKB * kBR];        // weight scale bits, 4 copies

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

    // --- per-thread staging roles, fixed for the whole K loop ---------------
    // activations: chunk i of this thread = token a_tok + 32 i (of the tile),
    // block a_blk of the stage, 16-byte quarter a_q of the 64-byte record
    const int a_tok = t >> 4;
    const int a_blk = (t >> 2) & 3;
    const int a_q = t & 3;
    const u32x4* a_src = reinterpret_cast<const u32x4*>(act_rec) + ((n0 + a_tok) * nb + a_blk) * 4 + a_q;
    const int64_t a_step = static_cast<int64_t>(32) * nb * 4;  // 32 tokens further, in 16-byte units
    uint32_t a_tok_ok = 0;
#pragma unroll
    for (int i = 0; i < kActChunks; ++i)
        if (n0 + a_tok + 32 * i < N) a_tok_ok |= 1u << i;
    uint32_t* a_dst = sA + a_blk * kPlaneA + a_tok * kRecA + a_q * 4;
    // activation scale bits: thread t < kBT handles token t, all kKB blocks
    const bool d_role = t < kBT;
    const bool d_ok = d_role && (n0 + t < N);
    const uint16_t* d_src = act_dx + (n0 + (d_role ? t : 0)) * nb;
    // weights: one block per thread, row w_row, block w_blk of the stage
    const int w_row = t >> 2;
    const int w_blk = t & 3;
    const bool w_row_ok = r0 + w_row < rows;
    const uint8_t* w_src = Wq + ((r0 + (w_row_ok ? w_row : 0)) * nb + w_blk) * kQ4Bytes;
    uint32_t* w_dst = sB + w_blk * kPlaneB + w_row * kRecB;

    u32x4 ra[kActChunks];
    uint16_t rdx[kKB];
    Block4 rw;
    bool rw_ok;

    auto load_stage = [&](int b0) {
        const bool a_blk_ok = b0 + a_blk < nb;
#pragma unroll
        for (int i = 0; i < kActChunks; ++i) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (a_blk_ok && ((a_tok_ok >> i) & 1u)) v = a_src[static_cast<int64_t>(b0) * 4 + i * a_step];
            ra[i] = v;
        }
        if (d_role) {
#pragma unroll
            for (int k = 0; k < kKB; ++k) rdx[k] = (d_ok && b0 + k < nb) ? d_src[b0 + k] : static_cast<uint16_t>(0);
        }
        rw_ok = w_row_ok && (b0 + w_blk < nb);
        if (rw_ok) rw = load_block(w_src + static_cast<int64_t>(b0) * kQ4Bytes);
    };

    auto store_stage = [&]() {
#pragma unroll
        for (int i = 0; i < kActChunks; ++i) *reinterpret_cast<u32x4*>(a_dst + 32 * kRecA * i) = ra[i];
        if (d_role) {
#pragma unroll
            for (int k = 0; k < kKB; ++k) {
                const uint32_t x = static_cast<uint32_t>(rdx[k]) * 0x10001u;
                sAd[k * kBT + t] = u32x2{x, x};
            }
        }
        uint32_t d6[6] = {0u, 0u, 0u, 0u, 0u, 0u};
        uint32_t dbits = 0u;
        if (rw_ok) {
            weight_fp6(rw.qs, d6);
            dbits = rw.dbits;
        }
        reinterpret_cast<u32x4*>(w_dst)[0] = u32x4{d6[0], d6[1], d6[2], d6[3]};
        reinterpret_cast<u32x4*>(w_dst)[1] = u32x4{d6[4], d6[5], 0u, 0u};
        const uint32_t wx = dbits * 0x10001u;
        sBd[w_blk * kBR + w_row] = u32x2{wx, wx};
    };

    f32x16 acc[4];  // tile k = (token half i = k / 2, row half j = k % 2)
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[k][v] = 0.0f;
    f32x16 s_prev, p_prev;
    bool have_prev = false;

    const f32x16 zero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int scale_a = (half ? kScaleLo : kScaleHi) - (DOTS ? 0 : kScaleDown);
    const uint32_t* a_rd = sA + (wm * 64 + l32) * kRecA + half * 8;
    const uint32_t* b_rd = sB + (wn * 64 + l32) * kRecB;
    const u32x2* ad_rd = sAd + wm * 64 + l32;
    const u32x2* bd_rd = sBd + wn * 64 + l32;

    load_stage(0);
    for (int b0 = 0; b0 < nb; b0 += kKB) {
        store_stage();
        __syncthreads();
        if (b0 + kKB < nb) load_stage(b0 + kKB);

#pragma unroll 1
        for (int blk = 0; blk < kKB; ++blk) {
            i32x8 a[2], w[2];
            f16x4 ap[2], wp[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const u32x4* src = reinterpret_cast<const u32x4*>(a_rd + blk * kPlaneA + i * 32 * kRecA);
                const u32x4 x0 = src[0], x1 = src[1];
                a[i] = i32x8{static_cast<int>(x0.x), static_cast<int>(x0.y), static_cast<int>(x0.z),
                             static_cast<int>(x0.w), static_cast<int>(x1.x), static_cast<int>(x1.y),
                             static_cast<int>(x1.z), static_cast<int>(x1.w)};
                ap[i] = __builtin_bit_cast(f16x4, ad_rd[blk * kBT + i * 32]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const u32x4* src = reinterpret_cast<const u32x4*>(b_rd + blk * kPlaneB + j * 32 * kRecB);
                const u32x4 x0 = src[0], x1 = src[1];
                w[j] = i32x8{static_cast<int>(x0.x), static_cast<int>(x0.y), static_cast<int>(x0.z),
                             static_cast<int>(x0.w), static_cast<int>(x1.x), static_cast<int>(x1.y),
                             static_cast<int>(x1.z), static_cast<int>(x1.w)};
                wp[j] = __builtin_bit_cast(f16x4, bd_rd[blk * kBR + j * 32]);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = k >> 1, j = k & 1;
                const f32x16 sk = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    a[i], w[j], zero, 2, 2, 0, scale_a, 0, kScaleW);
                if constexpr (DOTS) {
                    const int b = b0 + blk;
                    const int64_t r = r0 + wn * 64 + j * 32 + l32;
                    if (b < nb && r < rows) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int64_t n = n0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                            if (n < N) D[(n * rows + r) * nb + b] = static_cast<int32_t>(sk[v]);
                        }
                    }
                } else {
                    const f32x16 pk = __builtin_amdgcn_mfma_f32_32x32x8f16(ap[i], wp[j], zero, 0, 0, 0);
                    // software pipeline: fold the previous tile while this tile's
                    // two matrix instructions run
                    // (the previous tile is always tile (k + 3) % 4: the last one of
                    // the previous block when k == 0)
                    if (have_prev) {
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            acc[(k + 3) & 3][v] = fmaf(s_prev[v], p_prev[v], acc[(k + 3) & 3][v]);
                    }
                    s_prev = sk;
                    p_prev = pk;
                    have_prev = true;
                }
            }
        }
        __syncthreads();
    }

    if constexpr (!DOTS) {
        if (have_prev) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[3][v] = fmaf(s_prev[v], p_prev[v], acc[3][v]);
        }
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

hipError_t launch_gemm(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const void* act,
                       int64_t N, float* Y, int32_t* D, hipStream_t s) {
    (void)dev;
    const uint32_t* rec = static_cast<const uint32_t*>(act);
    const uint16_t* dxb = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(act) + N * nb * kAct6Bytes);
    const dim3 grid(static_cast<uint32_t>(((rows + kBR - 1) / kBR) * ((N + kBT - 1) / kBT)));
    if (D)
        hipLaunchKernelGGL(k_gemm<true>, grid, dim3(kThreads), 0, s, Wq, rows, static_cast<int>(nb), rec, dxb, N, Y,
                           D);
    else
        hipLaunchKernelGGL(k_gemm<false>, grid, dim3(kThreads), 0, s, Wq, rows, static_cast<int>(nb), rec, dxb, N, Y,
                           D);
    return hipGetLastError();
}

}  // namespace q4bq
