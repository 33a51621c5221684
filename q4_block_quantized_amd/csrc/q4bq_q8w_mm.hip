// Q8_0 weights x Q8_0 activations on the matrix cores, more than 8 tokens
// (`k_q8w_mm`).
//
// The product of "llama.cpp 深度解读" (luoboask.github.io) section 3 with the
// Q8_0 weight block of section 1's type table (binary16 d, 32 int8 q;
// element j = q_j * d): per 32-value block the integer dot s = sum_j qw_j * qx_j,
// scaled by d_w * d_x in fp32 and summed over the blocks.
//
// The int8 values of both operands are exactly what the int8 matrix cores
// take, so the weights need no conversion: one v_mfma_i32_32x32x32_i8 (K = 32,
// one block) gives the exact int32 dots of a 32-token x 32-row tile, one
// v_mfma_f32_32x32x8_f16 outer product of the two binary16 scale vectors gives
// the tile's 1024 scale products (exact in fp32), and the vector ALU folds
// them in: acc = fma(float(s), d_x * d_w, acc), in increasing block order.
//
// Workgroup: 256 threads (4 waves), a tile of 128 tokens x 128 rows, each wave
// 2 x 2 tiles of 32 x 32 (64 tokens x 64 rows).  The K loop stages 4 blocks at
// a time through a double-buffered LDS ring (one barrier per stage): the
// activation records of the stage's blocks ([block][token] 32 bytes of int8,
// and the binary16 scales) and the weight blocks' values and scales, loaded
// into registers one stage ahead.  A token's (or row's) 32 bytes sit in LDS
// with their 16-byte halves swapped when bit 3 of the token (row) is set, so
// the 16-byte operand reads of 16 lanes touch 64 distinct banks.  Two
// workgroups fit a CU (68 KB of LDS each): two waves per SIMD.
#include "q4bq_device.h"
#include "q4bq_internal.h"

namespace q4bq {

namespace {

constexpr int kMmThreads = 256;
constexpr int kMmTok = 128;    // tokens per workgroup tile
constexpr int kMmRows = 128;   // rows per workgroup tile
constexpr int kMmKB = 4;       // blocks per stage
constexpr int kMmPlaneA = kMmTok * 32;
constexpr int kMmPlaneB = kMmRows * 32;
constexpr int kMmCodes = kMmKB * (kMmPlaneA + kMmPlaneB);             // 32 KB
constexpr int kMmStage = kMmCodes + kMmKB * (kMmTok + kMmRows) * 2;   // + 2 KB of scales
static_assert(kMmTok * kMmKB * 32 == 4 * kMmThreads * 16, "activation staging: 4 16-byte loads per thread");
static_assert(kMmRows * kMmKB == 2 * kMmThreads, "weight staging: 2 blocks per thread");
static_assert(kMmThreads == kQ8wMmThreads && kMmRows == kQ8wMmRows && kMmTok == kQ8wMmTokens,
              "launch geometry the argument checks bound");

typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// LDS byte offset of 16-byte half h of item t's 32-byte record in a plane.
__device__ __forceinline__ int rec16(int t, int h) { return t * 32 + 16 * (h ^ ((t >> 3) & 1)); }

// Workgroup tiles in an order that gives each XCD (workgroup x runs on XCD
// x % 8) a contiguous range, so the token tiles that read the same weight
// rows share one L2.
__device__ __forceinline__ int64_t mm_tile(uint32_t x, uint32_t grid) {
    constexpr uint32_t kXcd = 8;
    const uint32_t q = grid / kXcd, rem = grid % kXcd, j = x % kXcd;
    return static_cast<int64_t>(j * q + (j < rem ? j : rem) + x / kXcd);
}

// acts: N x nb activation records, [block][token] 32 bytes of int8 codes in
// element order, followed by the [block][token] binary16 scale bits.
template <bool DOTS>
__global__ void __launch_bounds__(kMmThreads)
k_q8w_mm(const uint8_t* __restrict__ W, int64_t rows, int nb, const uint8_t* __restrict__ acts, int64_t N,
         float* __restrict__ Y, int32_t* __restrict__ D, int kbs, int splits) {
    __shared__ __align__(16) uint8_t smem[2 * kMmStage];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    // workgroup tile: token tile (fastest), then split, then row tile; split s
    // takes blocks [kb0, kb1) of every row and writes its sums to slice s of Y
    const int64_t ntt = (N + kMmTok - 1) / kMmTok;
    const int64_t tile = mm_tile(blockIdx.x, gridDim.x);
    const int64_t n0 = (tile % ntt) * kMmTok;
    const int64_t rs = tile / ntt;
    const int split = __builtin_amdgcn_readfirstlane(static_cast<int>(rs % splits));
    const int64_t r0 = (rs / splits) * kMmRows;
    const int kb0 = __builtin_amdgcn_readfirstlane(split * kbs);
    const int kb1 = __builtin_amdgcn_readfirstlane(min(nb, kb0 + kbs));
    const int nst = (kb1 - kb0 + kMmKB - 1) / kMmKB;
    const uint8_t* __restrict__ act_codes = acts;
    const uint16_t* __restrict__ act_scales =
        reinterpret_cast<const uint16_t*>(acts + static_cast<int64_t>(nb) * N * 32);

    // ---- staging: what this thread moves each stage ---------------------------
    // activations: 16-byte piece c = t + 256 i (i < 4) of the stage's 4 planes:
    // plane c / 256, token (c % 256) / 2, half c % 2.  Tokens past N read the
    // last token (never stored); blocks past the range read its last block with a zero
    // scale (see below).
    int a_tok[4], a_half[4], a_blk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = t + kMmThreads * i;
        a_blk[i] = c >> 8;
        a_tok[i] = (c & 255) >> 1;
        a_half[i] = c & 1;
    }
    // activation scales: plane t / 64, tokens 2 (t % 64) and 2 (t % 64) + 1
    const int as_blk = t >> 6, as_tok = 2 * (t & 63);
    // weights: row t / 2 of the tile, blocks 2 (t % 2) and 2 (t % 2) + 1
    const int w_row = t >> 1, w_blk0 = 2 * (t & 1);
    const int64_t w_r = r0 + w_row < rows ? r0 + w_row : rows - 1;

    // per-thread bases; a stage adds its blocks' offsets (blocks past the end
    // are clamped to the last block)
    const int64_t planeA = N * 32;  // bytes per block of activation records
    const uint8_t* a_base[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + a_tok[i] < N ? n0 + a_tok[i] : N - 1;
        a_base[i] = act_codes + n * 32 + 16 * a_half[i];
    }
    const int64_t s_n = n0 + as_tok;
    const uint16_t* s_base = act_scales + (s_n < N ? s_n : N - 1);
    const bool s_ok0 = s_n < N, s_ok1 = s_n + 1 < N;
    const uint8_t* w_base = W + w_r * nb * kQ8Bytes;

    u32x4 ra[4];
    uint32_t ras;
    uint32_t rwd[2];
    u32x4 rwq[2][2];
    auto load_stage = [&](int st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = min(kb0 + st * kMmKB + a_blk[i], kb1 - 1);
            __builtin_memcpy(&ra[i], a_base[i] + static_cast<int64_t>(b) * planeA, 16);
        }
        {
            // two scales (tokens n, n + 1) as one dword; past N or past the
            // last block: zero scale
            const int b = kb0 + st * kMmKB + as_blk;
            const uint16_t* p = s_base + static_cast<int64_t>(min(b, kb1 - 1)) * N;
            const uint32_t s0 = s_ok0 ? p[0] : 0u;
            const uint32_t s1 = s_ok1 ? p[1] : 0u;
            ras = b < kb1 ? (s0 | (s1 << 16)) : 0u;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int b = kb0 + st * kMmKB + w_blk0 + k;
            const uint8_t* p = w_base + min(b, kb1 - 1) * kQ8Bytes;
            uint16_t d;
            __builtin_memcpy(&d, p, 2);
            __builtin_memcpy(&rwq[k][0], p + 2, 16);
            __builtin_memcpy(&rwq[k][1], p + 18, 16);
            rwd[k] = b < kb1 ? d : 0u;
        }
    };
    auto store_stage = [&](int buf) __attribute__((always_inline)) {
        uint8_t* s = smem + buf * kMmStage;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<u32x4*>(s + a_blk[i] * kMmPlaneA + rec16(a_tok[i], a_half[i])) = ra[i];
        uint16_t* sas = reinterpret_cast<uint16_t*>(s + kMmCodes);
        *reinterpret_cast<uint32_t*>(sas + as_blk * kMmTok + as_tok) = ras;
        uint8_t* sb = s + kMmKB * kMmPlaneA;
        uint16_t* sbs = sas + kMmKB * kMmTok;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int pb = w_blk0 + k;
            *reinterpret_cast<u32x4*>(sb + pb * kMmPlaneB + rec16(w_row, 0)) = rwq[k][0];
            *reinterpret_cast<u32x4*>(sb + pb * kMmPlaneB + rec16(w_row, 1)) = rwq[k][1];
            sbs[pb * kMmRows + w_row] = static_cast<uint16_t>(rwd[k]);
        }
    };

    // ---- compute: wave w owns token tiles 2 (w & 1) + {0, 1} and row tiles
    // 2 (w >> 1) + {0, 1} of the workgroup tile
    const int l32 = lane & 31, half = lane >> 5;
    const int tt0 = 2 * (wave & 1), rt0 = 2 * (wave >> 1);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    const i32x16 izero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const f32x16 fzero = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf, int st) __attribute__((always_inline)) {
        const uint8_t* s = smem + buf * kMmStage;
        const uint16_t* sas = reinterpret_cast<const uint16_t*>(s + kMmCodes);
        const uint8_t* sb = s + kMmKB * kMmPlaneA;
        const uint16_t* sbs = sas + kMmKB * kMmTok;
#pragma unroll
        for (int kb = 0; kb < kMmKB; ++kb) {
            i32x4 a[2], b[2];
            f16x4 as[2], bs[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tok = 32 * (tt0 + i) + l32;
                a[i] = *reinterpret_cast<const i32x4*>(s + kb * kMmPlaneA + rec16(tok, half));
                // K slot 0 of the first half carries the scale, every other slot 0
                const uint32_t dx = sas[kb * kMmTok + tok];
                as[i] = __builtin_bit_cast(f16x4, u32x2v{half ? 0u : dx, 0u});
                const int row = 32 * (rt0 + i) + l32;
                b[i] = *reinterpret_cast<const i32x4*>(sb + kb * kMmPlaneB + rec16(row, half));
                const uint32_t dw = sbs[kb * kMmRows + row];
                bs[i] = __builtin_bit_cast(f16x4, u32x2v{half ? 0u : dw, 0u});
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const i32x16 sdot = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], izero, 0, 0, 0);
                    if constexpr (DOTS) {
                        const int blk = kb0 + st * kMmKB + kb;
                        const int64_t r = r0 + 32 * (rt0 + j) + l32;
                        if (blk < kb1 && r < rows) {
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const int64_t n = n0 + 32 * (tt0 + i) + 8 * (v >> 2) + 4 * half + (v & 3);
                                if (n < N) D[(n * rows + r) * nb + blk] = sdot[v];
                            }
                        }
                    } else {
                        const f32x16 p = __builtin_amdgcn_mfma_f32_32x32x8f16(as[i], bs[j], fzero, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            acc[i][j][v] = fmaf(static_cast<float>(sdot[v]), p[v], acc[i][j][v]);
                    }
                }
            // one block's matrix instructions in flight at a time (bounded
            // registers): the accumulators are final for this block before the
            // next block's operands are read
            if constexpr (!DOTS)
                asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[1][0]), "+v"(acc[1][1])::"memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        if (st + 1 < nst) load_stage(st + 1);
        compute(st & 1, st);
        if (st + 1 < nst) store_stage((st + 1) & 1);
        __syncthreads();
    }

    if constexpr (!DOTS) {
        float* const Yo = Y + static_cast<int64_t>(split) * N * rows;  // this split's slice
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t r = r0 + 32 * (rt0 + j) + l32;
                if (r >= rows) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t n = n0 + 32 * (tt0 + i) + 8 * (v >> 2) + 4 * half + (v & 3);
                    if (n < N) Yo[n * rows + r] = acc[i][j][v];
                }
            }
    }
}

// Y = the splits' slices of P added in split order.
__global__ void __launch_bounds__(256)
k_q8w_mm_sum(const float* __restrict__ P, int splits, int64_t total, float* __restrict__ Y) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        float y = P[i];
        for (int k = 1; k < splits; ++k) y += P[k * total + i];
        Y[i] = y;
    }
}

// fp32 activations -> the records above: one 8-lane group per (token, block),
// lane m quantizing elements 4m..4m+3 by the Q8_0 rule (the q8_0_quantize
// arithmetic).  Grid: y walks the blocks, x the tokens 32 at a time.
__global__ void __launch_bounds__(256)
k_act8_from_f32(const float* __restrict__ X, int64_t N, int64_t nb, uint8_t* __restrict__ acts) {
    const int m = threadIdx.x & 7;
    uint32_t* codes = reinterpret_cast<uint32_t*>(acts);
    uint16_t* scales = reinterpret_cast<uint16_t*>(acts + nb * N * 32);
    const int64_t step = static_cast<int64_t>(gridDim.x) * 32;
    const int64_t wave_first = static_cast<int64_t>(blockIdx.x) * 32 + ((threadIdx.x >> 3) & ~7);
    for (int64_t b = blockIdx.y; b < nb; b += gridDim.y)
        for (int64_t n1 = wave_first; n1 < N; n1 += step) {
            const int64_t n = n1 + ((threadIdx.x >> 3) & 7);
            const bool valid = n < N;
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (valid) __builtin_memcpy(&x, X + (n * nb + b) * kQK + 4 * m, 16);
            uint32_t dbits;
            int8_t qq[4];
            q8_block_quad(x.x, x.y, x.z, x.w, dbits, qq);
            const uint32_t q = q8_natural_word(qq);
            if (valid) {
                codes[(b * N + n) * 8 + m] = q;
                if (m == 0) scales[b * N + n] = static_cast<uint16_t>(dbits);
            }
        }
}

// Q8_0 blocks (the pages' 34-byte layout) -> the same records.
__global__ void __launch_bounds__(256)
k_act8_from_q8(const uint8_t* __restrict__ Xq, int64_t N, int64_t nb, uint8_t* __restrict__ acts) {
    const int m = threadIdx.x & 7;
    uint32_t* codes = reinterpret_cast<uint32_t*>(acts);
    uint16_t* scales = reinterpret_cast<uint16_t*>(acts + nb * N * 32);
    const int64_t step = static_cast<int64_t>(gridDim.x) * 32;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * 32 + (threadIdx.x >> 3);
    for (int64_t b = blockIdx.y; b < nb; b += gridDim.y)
        for (int64_t n = first; n < N; n += step) {
            const uint8_t* blk = Xq + (n * nb + b) * kQ8Bytes;
            uint32_t q;
            __builtin_memcpy(&q, blk + 2 + 4 * m, 4);
            codes[(b * N + n) * 8 + m] = q;
            if (m == 0) {
                uint16_t d;
                __builtin_memcpy(&d, blk, 2);
                scales[b * N + n] = d;
            }
        }
}

dim3 act8_grid(int64_t N, int64_t nb) {
    const int64_t y = nb < 8192 ? nb : 8192;
    int64_t x = (N + 31) / 32;
    const int64_t xmax = 8192 / y > 0 ? 8192 / y : 1;
    if (x > xmax) x = xmax;
    return dim3(static_cast<uint32_t>(x < 1 ? 1 : x), static_cast<uint32_t>(y < 1 ? 1 : y));
}

}  // namespace

size_t q8w_mm_act_bytes(int64_t N, int64_t nb) {
    return (static_cast<size_t>(N * nb) * (32 + 2) + 255) & ~static_cast<size_t>(255);
}

int q8w_mm_splits(int64_t rows, int64_t nb, int64_t N, int num_cu, int* kbs) {
    const int64_t tiles = ((rows + kMmRows - 1) / kMmRows) * ((N + kMmTok - 1) / kMmTok);
    *kbs = static_cast<int>(nb);
    int64_t S = 2 * static_cast<int64_t>(num_cu) / tiles;  // two workgroups per CU
    if (S > kQ8wMmMaxSplits) S = kQ8wMmMaxSplits;
    if (S > nb / 16) S = nb / 16;
    if (S < 2) return 1;
    int64_t kb = (nb + S - 1) / S;
    kb = (kb + kMmKB - 1) / kMmKB * kMmKB;  // whole stages
    S = (nb + kb - 1) / kb;
    if (S < 2) return 1;
    *kbs = static_cast<int>(kb);
    return static_cast<int>(S);
}

size_t q8w_mm_scratch_bytes(int64_t rows, int64_t nb, int64_t N, int num_cu) {
    int kbs = 0;
    const int S = q8w_mm_splits(rows, nb, N, num_cu, &kbs);
    return q8w_mm_act_bytes(N, nb) + (S > 1 ? static_cast<size_t>(S) * static_cast<size_t>(N * rows) * 4 : 0);
}

hipError_t launch_q8w_mm(const DeviceInfo* dev, const uint8_t* W, int64_t rows, int64_t nb, const float* X,
                         const uint8_t* Xq, int64_t N, float* Y, int32_t* D, void* ws, hipStream_t s) {
    uint8_t* acts = static_cast<uint8_t*>(ws);
    if (X)
        hipLaunchKernelGGL(k_act8_from_f32, act8_grid(N, nb), dim3(256), 0, s, X, N, nb, acts);
    else
        hipLaunchKernelGGL(k_act8_from_q8, act8_grid(N, nb), dim3(256), 0, s, Xq, N, nb, acts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // few workgroup tiles: K split into ranges, each range's sums into its
    // slice of the buffer behind the activation records (q8w_mm_scratch_bytes),
    // added in range order by k_q8w_mm_sum; the block-dot export never splits
    int kbs = static_cast<int>(nb), splits = 1;
    if (!D) splits = q8w_mm_splits(rows, nb, N, dev->num_cu, &kbs);
    float* partial = reinterpret_cast<float*>(acts + q8w_mm_act_bytes(N, nb));
    const dim3 grid(
        static_cast<uint32_t>(((rows + kMmRows - 1) / kMmRows) * ((N + kMmTok - 1) / kMmTok) * splits));
    if (D)
        hipLaunchKernelGGL(k_q8w_mm<true>, grid, dim3(kMmThreads), 0, s, W, rows, static_cast<int>(nb), acts, N, Y,
                           D, kbs, splits);
    else
        hipLaunchKernelGGL(k_q8w_mm<false>, grid, dim3(kMmThreads), 0, s, W, rows, static_cast<int>(nb), acts, N,
                           splits > 1 ? partial : Y, D, kbs, splits);
    e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t total = N * rows;
    int64_t blocks = (total + 255) / 256;
    const int64_t cap = static_cast<int64_t>(dev->num_cu) * 8;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(k_q8w_mm_sum, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, partial, splits, total, Y);
    return hipGetLastError();
}

}  // namespace q4bq
