// Q8_0 weights x Q8_0 activations (`k_q8w_rows`, `k_q8w_block_dots`).
//
// "llama.cpp 深度解读" (luoboask.github.io) section 1 lists Q8_0 (8 bits per
// weight) beside Q4_0 in its table of ggml quantization types; its block is
// the block_q8_0 that section 3's product takes as activations: a binary16
// scale and 32 int8 values, element j = q_j * d.  The product is section 3's
// with that weight decode: per block the integer dot s = sum_j qw_j * qx_j
// (no offset), scaled by d_w * d_x in fp32 and summed over the blocks.
//
// Decode-shaped work, bound by HBM: rows are streamed by whole waves as in the
// Q4_0 row kernel.  The 64 lanes of a wave share one row; with an even block
// count lane l owns block pairs l, l + 64, ... (68 bytes from a 4-byte aligned
// address: four 16-byte loads and one 4-byte load), otherwise single blocks
// (a 2-byte scale load and two 16-byte loads from a 2-byte aligned address;
// gfx950 serves unaligned global loads).  The workgroup quantizes the NT tokens into
// LDS with the Q8_0 rule in natural element order, so a weight dword and an
// activation dword hold the same four elements and meet in v_dot4_i32_i8.
#include "q4bq_rows.h"

namespace q4bq {

namespace {

constexpr int kQ8wMaxBpl = 16;  // 64 * 16 blocks: K <= 32768

// The integer dot of one Q8_0 weight block with one activation block, both as
// eight dwords of four int8 in element order.  Every partial sum is exact in
// int32 (|s| <= 32 * 127 * 127).
__device__ __forceinline__ int32_t q8w_block_dot(const uint32_t (&w)[8], const uint32_t* a) {
    int32_t s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_sdot4(static_cast<int>(w[k]), static_cast<int>(a[k]), s, false);
    return s;
}

struct Q8Block {
    uint32_t dbits;
    uint32_t q[8];
};

// A Q8_0 block at p (34 bytes, 2-byte aligned).
__device__ __forceinline__ Q8Block load_q8_block(const uint8_t* p) {
    Q8Block b;
    uint16_t d;
    u32x4 lo, hi;
    __builtin_memcpy(&d, p, 2);
    __builtin_memcpy(&lo, p + 2, 16);
    __builtin_memcpy(&hi, p + 18, 16);
    b.dbits = d;
    b.q[0] = lo.x; b.q[1] = lo.y; b.q[2] = lo.z; b.q[3] = lo.w;
    b.q[4] = hi.x; b.q[5] = hi.y; b.q[6] = hi.z; b.q[7] = hi.w;
    return b;
}

// Q8_0 of one block by its 8-lane group: lane m holds elements 4m..4m+3 and
// gets their four int8 as one dword (element order), plus the block's scale.
__device__ __forceinline__ uint32_t quant_q8_natural(float x0, float x1, float x2, float x3, float& d) {
    uint32_t dbits;
    int8_t q[4];
    d = q8_block_quad(x0, x1, x2, x3, dbits, q);
    return q8_natural_word(q);
}

// LDS: NT x nb blocks of 8 dwords of codes (token-major), then NT x nb fp32
// scales.  With an even block count each pair of blocks takes 80 bytes (64 of
// codes, 16 unused): lane l reads blocks 2l and 2l + 1, and at a 64-byte lane
// stride every fourth lane's 16-byte read would meet the same four banks; at
// 80 bytes the 16 lanes of one LDS cycle cover all 64 banks (this matters to
// the 5..8-token kernels, which read the codes for every row: 128256 x 4096
// at N = 8 149.8 -> 135.7 us, graph-timed).
__host__ __device__ inline int q8w_code_dword(int g, bool padded) {
    return padded ? (g >> 1) * 20 + (g & 1) * 8 : g * 8;
}
__host__ __device__ inline size_t q8w_code_bytes(int64_t nblk, bool padded) {
    return static_cast<size_t>(nblk) * (padded ? 40 : 32);
}
__host__ __device__ inline size_t q8w_act_lds(int64_t nt, int64_t nb) {
    return q8w_code_bytes(nt * nb, nb % 2 == 0) + static_cast<size_t>(nt) * nb * 4;
}

// Two consecutive blocks (68 bytes) from a 4-byte aligned address: four
// 16-byte loads and one 4-byte load.  Block 0: scale in bytes 0-1, values in
// bytes 2-33 (realigned by 16 bits); block 1: scale in bytes 34-35, values in
// bytes 36-67 (dword aligned).
struct Q8Pair {
    uint32_t w[17];
};

__device__ __forceinline__ Q8Pair load_q8_pair(const uint8_t* p) {
    Q8Pair r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        u32x4 v;
        __builtin_memcpy(&v, p + 16 * k, 16);
        r.w[4 * k] = v.x; r.w[4 * k + 1] = v.y; r.w[4 * k + 2] = v.z; r.w[4 * k + 3] = v.w;
    }
    __builtin_memcpy(&r.w[16], p + 64, 4);
    return r;
}

__device__ __forceinline__ Q8Block pair_block(const Q8Pair& p, int h) {
    Q8Block b;
    if (h == 0) {
        b.dbits = p.w[0] & 0xFFFFu;
#pragma unroll
        for (int k = 0; k < 8; ++k) b.q[k] = __builtin_amdgcn_alignbit(p.w[k + 1], p.w[k], 16);
    } else {
        b.dbits = p.w[8] >> 16;
#pragma unroll
        for (int k = 0; k < 8; ++k) b.q[k] = p.w[9 + k];
    }
    return b;
}

// Slot: one block (odd block counts) or a pair of blocks (PAIRED, even block
// counts: dword-aligned loads).  Lane l owns slots l, l + 64, ... (SPL of them).
template <bool PAIRED>
struct Q8Slot;
template <>
struct Q8Slot<false> {
    Q8Block b;
};
template <>
struct Q8Slot<true> {
    Q8Pair p;
};

// NTL (pairs, one per lane: rows of at most 128 blocks, a multiple of 8):
// a wave loads its row as 17 nb / 8 consecutive 16-byte pieces with
// non-temporal loads -- each instruction one contiguous 1 KB, the lanes past
// the row re-reading its last piece -- writes them to its own LDS area in
// order and reads its lane's 68-byte pair back (17 dwords apart per lane: no
// bank conflicts).  The folds see the same bytes.
constexpr int kQ8wNtlLoads = 5;  // 17 * 128 / 8 = 272 pieces at most
__host__ __device__ inline size_t q8w_ntl_offset(int nt, int64_t nb) {
    return (q8w_act_lds(nt, nb) + 15) / 16 * 16;
}

// 5..8 tokens on one block pair per lane: the tokens' 16 activation blocks
// stay in registers and the 512-thread workgroups run one per CU (measured,
// graph-timed: 14336 x 4096 at N = 8 27.0 -> 23.3 us, the 128256 x 4096 head
// 136.1 -> 131.0 us, against two workgroups per CU reading the blocks from
// LDS for every row)
template <int THREADS, int BPL>
constexpr bool kRegPairs = THREADS == 512 && BPL == 2;

template <int THREADS, int NT, int SPL, int D, bool PAIRED, bool NTL = false>
__global__ void __launch_bounds__(THREADS)
k_q8w_rows(const uint8_t* __restrict__ W, int64_t rows, int nb, const float* __restrict__ X, float* __restrict__ Y) {
    static_assert(!NTL || (PAIRED && SPL == 1), "contiguous row loads: one pair per lane");
    constexpr int kWaves = THREADS / 64;
    constexpr int kBps = PAIRED ? 2 : 1;              // blocks per slot
    constexpr int BPL = SPL * kBps;
    // activations in registers (up to 16 blocks in the one-pair 512-thread
    // form, which then runs one workgroup per CU: two waves per SIMD have the
    // registers), else read from LDS per row
    constexpr bool kActReg = NT * BPL <= (kRegPairs<THREADS, BPL> ? 16 : 8);
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t* sq = reinterpret_cast<uint32_t*>(smem);
    float* sd = reinterpret_cast<float*>(smem + q8w_code_bytes(static_cast<int64_t>(NT) * nb, PAIRED));
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nblk = NT * nb;

    // rows of this wave: w0, w0 + S, ...; loads past the last row re-read it,
    // so the load counters always wait for exactly the oldest row
    const int64_t S = static_cast<int64_t>(gridDim.x) * kWaves;
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
    const int64_t nk = w0 < rows ? (rows - 1 - w0) / S + 1 : 0;
    const int64_t rlast = nk > 0 ? w0 + (nk - 1) * S : rows - 1;
    // block i of the lane: slot i / kBps, half i % kBps
    const int nslot = nb / kBps;
    int ss[SPL];
    bool sv[SPL];
    int bb[BPL];
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
        sv[i] = lane + 64 * i < nslot;
        ss[i] = min(lane + 64 * i, nslot - 1);
#pragma unroll
        for (int h = 0; h < kBps; ++h) bb[i * kBps + h] = ss[i] * kBps + h;
    }
    auto load_row = [&](Q8Slot<PAIRED> (&dst)[SPL], int64_t k) __attribute__((always_inline)) {
        const int64_t r = min(w0 + k * S, rlast);
        const uint8_t* base = W + uniform64(r * nb) * kQ8Bytes;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            const uint8_t* p = base + static_cast<uint32_t>(ss[i]) * (kBps * kQ8Bytes);
            if constexpr (PAIRED)
                dst[i].p = load_q8_pair(p);
            else
                dst[i].b = load_q8_block(p);
        }
    };
    const int npc = 17 * nb / 8;
    uint8_t* const wrow = smem + q8w_ntl_offset(NT, nb) + static_cast<size_t>(wave) * nb * kQ8Bytes;
    auto load_row_ntl = [&](u32x4 (&dst)[kQ8wNtlLoads], int64_t k) __attribute__((always_inline)) {
        typedef u32x4 u32x4_a2 __attribute__((aligned(2)));
        const int64_t r = min(w0 + k * S, rlast);
        const uint8_t* base = W + uniform64(r * nb) * kQ8Bytes;
#pragma unroll
        for (int i = 0; i < kQ8wNtlLoads; ++i) {
            const int pc = min(lane + 64 * i, npc - 1);
            dst[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_a2*>(base + 16 * pc));
        }
    };
    auto unpack_row = [&](const u32x4 (&src)[kQ8wNtlLoads], Q8Slot<PAIRED> (&q)[SPL]) __attribute__((always_inline)) {
        if constexpr (NTL) {
#pragma unroll
            for (int i = 0; i < kQ8wNtlLoads; ++i)
                if (lane + 64 * i < npc) reinterpret_cast<u32x4*>(wrow)[lane + 64 * i] = src[i];
            __builtin_amdgcn_wave_barrier();
            const uint32_t* p = reinterpret_cast<const uint32_t*>(wrow + 2 * kQ8Bytes * ss[0]);
#pragma unroll
            for (int j = 0; j < 17; ++j) q[0].p.w[j] = p[j];
            __builtin_amdgcn_wave_barrier();
        }
    };
    Q8Slot<PAIRED> raw[D][SPL];
    u32x4 rawn[NTL ? D : 1][kQ8wNtlLoads];
    auto load_next = [&](int d, int64_t k) __attribute__((always_inline)) {
        if constexpr (NTL) load_row_ntl(rawn[d], k);
        else load_row(raw[d], k);
    };
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_next(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }

    // the tokens, quantized into LDS (8 lanes per block; the loop bound is the
    // same for the 8 lanes of a group)
    {
        const int m = threadIdx.x & 7;
        for (int g = threadIdx.x >> 3; g < nblk; g += THREADS / 8) {
            float4 x;
            __builtin_memcpy(&x, X + static_cast<int64_t>(g) * kQK + 4 * m, 16);
            float d;
            const uint32_t word = quant_q8_natural(x.x, x.y, x.z, x.w, d);
            sq[q8w_code_dword(g, PAIRED) + m] = word;
            if (m == 0) sd[g] = d;
        }
        // LDS writes done, then the workgroup barrier; no wait on the weight loads
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    uint32_t areg[kActReg ? NT : 1][kActReg ? BPL : 1][8];
    float dreg[kActReg ? NT : 1][kActReg ? BPL : 1];
    if constexpr (kActReg) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int i = 0; i < BPL; ++i) {
                const int g = n * nb + bb[i];
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(sq + q8w_code_dword(g, PAIRED));
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(sq + q8w_code_dword(g, PAIRED) + 4);
                areg[n][i][0] = a0.x; areg[n][i][1] = a0.y; areg[n][i][2] = a0.z; areg[n][i][3] = a0.w;
                areg[n][i][4] = a1.x; areg[n][i][5] = a1.y; areg[n][i][6] = a1.z; areg[n][i][7] = a1.w;
                dreg[n][i] = sd[g];
            }
    }
    if (nk == 0) return;

    auto fold = [&](const Q8Slot<PAIRED> (&q)[SPL], float (&part)[NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NT; ++n) part[n] = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            Q8Block blk;
            if constexpr (PAIRED)
                blk = pair_block(q[i / 2].p, i % 2);
            else
                blk = q[i].b;
            const float dw = half_bits_to_float(blk.dbits);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                int32_t s;
                float dx;
                if constexpr (kActReg) {
                    s = q8w_block_dot(blk.q, areg[n][i]);
                    dx = dreg[n][i];
                } else {
                    const int g = n * nb + bb[i];
                    const u32x4 a0 = *reinterpret_cast<const u32x4*>(sq + q8w_code_dword(g, PAIRED));
                    const u32x4 a1 = *reinterpret_cast<const u32x4*>(sq + q8w_code_dword(g, PAIRED) + 4);
                    const uint32_t a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                    s = q8w_block_dot(blk.q, a);
                    dx = sd[g];
                    if ((n & 3) == 3) __builtin_amdgcn_sched_barrier(0);
                }
                const float v = static_cast<float>(s) * (dw * dx);
                part[n] += sv[i / kBps] ? v : 0.0f;
            }
        }
    };
    const int my_token = lane_token<NT>(lane);
    for (int64_t k = 0; k < nk; k += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            float part[NT];
            if constexpr (NTL) unpack_row(rawn[d], raw[d]);
            fold(raw[d], part);
            const float t = wave_sums<NT>(part, lane);
            if (k + d < nk && my_token >= 0 && my_token < NT)
                Y[static_cast<int64_t>(my_token) * rows + w0 + (k + d) * S] = t;
            load_next(d, k + d + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// D[(n * rows + r) * nb + b] = the integer dot of weight block (r, b) with
// activation block (n, b) of the pages' Q8_0 layout; the product kernel's
// dot function.  One thread per dot.
__global__ void __launch_bounds__(256)
k_q8w_block_dots(const uint8_t* __restrict__ W, int64_t rows, int64_t nb, const uint8_t* __restrict__ Xq, int64_t N,
                 int32_t* __restrict__ D) {
    const int64_t total = N * rows * nb;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t b = i % nb;
        const int64_t r = (i / nb) % rows;
        const int64_t n = i / (nb * rows);
        const Q8Block w = load_q8_block(W + (r * nb + b) * kQ8Bytes);
        const Q8Block x = load_q8_block(Xq + (n * nb + b) * kQ8Bytes);
        D[i] = q8w_block_dot(w.q, x.q);
    }
}

template <int BPL>
constexpr int q8w_threads(int nt) { return (BPL >= 8 || nt * BPL > 8) ? 512 : 1024; }

template <int NT, int SPL, bool PAIRED>
hipError_t launch_q8w_k(const DeviceInfo* dev, const uint8_t* W, int64_t rows, int64_t nb, const float* X, float* Y,
                        hipStream_t s) {
    constexpr int BPL = SPL * (PAIRED ? 2 : 1);
    constexpr int kThreads = q8w_threads<BPL>(NT);
    constexpr int kDepth = BPL <= 2 ? 2 : 1;
    int64_t wgs = (rows + kThreads / 64 - 1) / (kThreads / 64);
    const int64_t cap = static_cast<int64_t>(dev->num_cu) * (kRegPairs<kThreads, BPL> ? 1 : 1024 / kThreads);
    if (wgs > cap) wgs = cap;
    // contiguous non-temporal row loads where rows are whole 16-byte pieces
    // and every wave has 16 rows or more (as for the Q4_0 row kernel), up to
    // four tokens (measured, graph-timed, 128256 x 4096: N = 1 99.6 -> 88.8
    // us, N = 4 113.5 -> 98.3 us; at N = 8, where the vector ALU bounds the
    // 512-thread kernel, the LDS pass costs more than it saves: 153.6 ->
    // 165.9 us)
    constexpr bool kNtlForm = PAIRED && SPL == 1 && kThreads == 1024;
    const size_t ntl_lds = q8w_ntl_offset(NT, nb) + static_cast<size_t>(kThreads / 64) * nb * kQ8Bytes;
    const bool ntl = kNtlForm && nb % 8 == 0 && rows >= 16 * wgs * (kThreads / 64) && ntl_lds <= kRowsMaxLds;
    const auto plain = k_q8w_rows<kThreads, NT, SPL, kDepth, PAIRED>;
    const auto contiguous = k_q8w_rows<kThreads, NT, SPL, kDepth, PAIRED, kNtlForm>;
    const auto kernel = ntl ? contiguous : plain;
    const size_t lds = ntl ? ntl_lds : q8w_act_lds(NT, nb);
    if (lds > 64 * 1024) {
        static const hipError_t raised = [&] {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(plain),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kRowsMaxLds));
            if (e == hipSuccess)
                e = hipFuncSetAttribute(reinterpret_cast<const void*>(contiguous),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kRowsMaxLds));
            return e;
        }();
        if (raised != hipSuccess) return raised;
    }
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(wgs)), dim3(kThreads), lds, s, W, rows,
                       static_cast<int>(nb), X, Y);
    return hipGetLastError();
}

// Even block counts: pairs (dword-aligned loads); odd: single blocks.  Slots
// per lane: the smallest power of two that covers the row.
template <int NT>
hipError_t launch_q8w_nt(const DeviceInfo* dev, const uint8_t* W, int64_t rows, int64_t nb, const float* X, float* Y,
                         hipStream_t s) {
    if ((nb & 1) == 0) {
        const int64_t spl = (nb / 2 + 63) / 64;
        if (spl <= 1) return launch_q8w_k<NT, 1, true>(dev, W, rows, nb, X, Y, s);
        if (spl <= 2) return launch_q8w_k<NT, 2, true>(dev, W, rows, nb, X, Y, s);
        if (spl <= 4) return launch_q8w_k<NT, 4, true>(dev, W, rows, nb, X, Y, s);
        if constexpr (NT <= 2) return launch_q8w_k<NT, 8, true>(dev, W, rows, nb, X, Y, s);
        return hipErrorInvalidValue;  // q8w_tokens_per_launch keeps long rows at two tokens
    }
    const int64_t bpl = (nb + 63) / 64;
    if (bpl <= 1) return launch_q8w_k<NT, 1, false>(dev, W, rows, nb, X, Y, s);
    if (bpl <= 2) return launch_q8w_k<NT, 2, false>(dev, W, rows, nb, X, Y, s);
    if (bpl <= 4) return launch_q8w_k<NT, 4, false>(dev, W, rows, nb, X, Y, s);
    if (bpl <= 8) return launch_q8w_k<NT, 8, false>(dev, W, rows, nb, X, Y, s);
    if constexpr (NT <= 2) return launch_q8w_k<NT, 16, false>(dev, W, rows, nb, X, Y, s);
    return hipErrorInvalidValue;  // q8w_tokens_per_launch keeps long rows at two tokens
}

}  // namespace

// Tokens per launch: their quantized blocks fit the LDS budget; rows longer
// than 512 blocks (16 per lane) take at most two (register budget).
int64_t q8w_tokens_per_launch(int64_t nb) {
    int64_t t = static_cast<int64_t>(kRowsMaxLds / q8w_act_lds(1, nb));
    if (t > 8) t = 8;
    if (nb > 512 && t > 2) t = 2;
    return t;
}

bool q8w_supported_k(int64_t nb) { return nb <= 64 * kQ8wMaxBpl && q8w_tokens_per_launch(nb) >= 1; }

hipError_t launch_q8w_product(const DeviceInfo* dev, const uint8_t* W, int64_t rows, int64_t nb, const float* X,
                              int64_t N, float* Y, hipStream_t s) {
    const int64_t per = q8w_tokens_per_launch(nb);
    for (int64_t n0 = 0; n0 < N; n0 += per) {
        const int64_t nt = N - n0 < per ? N - n0 : per;
        const float* Xg = X + n0 * nb * kQK;
        float* Yg = Y + n0 * rows;
        hipError_t e;
        switch (nt) {
            case 1: e = launch_q8w_nt<1>(dev, W, rows, nb, Xg, Yg, s); break;
            case 2: e = launch_q8w_nt<2>(dev, W, rows, nb, Xg, Yg, s); break;
            case 3: e = launch_q8w_nt<3>(dev, W, rows, nb, Xg, Yg, s); break;
            case 4: e = launch_q8w_nt<4>(dev, W, rows, nb, Xg, Yg, s); break;
            case 5: e = launch_q8w_nt<5>(dev, W, rows, nb, Xg, Yg, s); break;
            case 6: e = launch_q8w_nt<6>(dev, W, rows, nb, Xg, Yg, s); break;
            case 7: e = launch_q8w_nt<7>(dev, W, rows, nb, Xg, Yg, s); break;
            default: e = launch_q8w_nt<8>(dev, W, rows, nb, Xg, Yg, s); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_q8w_block_dots(const uint8_t* W, int64_t rows, int64_t nb, const uint8_t* Xq, int64_t N, int32_t* D,
                                 hipStream_t s) {
    const int64_t total = N * rows * nb;
    int64_t wgs = (total + 255) / 256;
    if (wgs > 16384) wgs = 16384;
    hipLaunchKernelGGL(k_q8w_block_dots, dim3(static_cast<uint32_t>(wgs)), dim3(256), 0, s, W, rows, nb, Xq, N, D);
    return hipGetLastError();
}

}  // namespace q4bq
