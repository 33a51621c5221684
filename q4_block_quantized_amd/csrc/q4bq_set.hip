// Several independent one-token products in one launch (`k_gemv_set`).
//
// Each product is the pages' operator, "llama.cpp 深度解读" (luoboask.github.io)
// section 3 "量化矩阵乘法 — 核心算子": y_m[r] = sum over blocks of
// d_w * d_x * (integer dot of the block), with section 2's nibble offset of 8;
// section 4 ("计算图构建 — 以 Llama 模型为例") runs a layer as a sequence of such
// products (Q, K, V, output, gate, up, down), each with its own input here.
//
// Separate launches of small matrices spend most of their time outside the
// weight stream: launch ramp, each workgroup quantizing its X, the tail.  One
// launch streams the weights of all products back to back:
//  - every workgroup quantizes every product's X into LDS once (the row
//    kernel's quantizer, the same bytes);
//  - a row with P block pairs is cut into C chunks of Pc = P / C pairs (C the
//    smallest power of two with Pc <= 64 that divides P, the chunked row
//    kernel's cut), one pair per lane;
//  - a round is 16 chunk rows of one product, one per wave of the
//    workgroup: 16 / C rows, wave w taking chunk w mod C of row w / C; the
//    rounds of all products are numbered one after the other and workgroup g
//    takes rounds g, g + G, ...;
//  - each wave folds its chunk row exactly as the row kernel does (block dot,
//    s * (d_w * d_x) per block, the pair's two terms added, the wave's lanes
//    added by DPP) and writes the sum to LDS; after one barrier the C chunks
//    of each row are added in chunk order and stored.
// Rows thus get the same fp32 operations in the same order as from the row
// kernel on that product alone (one pair per lane, chunked where C > 1).
#include "q4bq_rows.h"

namespace q4bq {

namespace {

constexpr int kSetThreads = 1024;
constexpr int kSetWaves = kSetThreads / 64;
constexpr int kSetD = 2;  // rounds in flight per wave

template <int D>
__global__ void __launch_bounds__(kSetThreads) k_gemv_set(const SetDesc sd) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int nblk = sd.nblk;
    uint32_t* sq = reinterpret_cast<uint32_t*>(smem);
    ActScale* ss = reinterpret_cast<ActScale*>(smem + static_cast<size_t>(nblk) * kActQBytes);
    float* pl = reinterpret_cast<float*>(smem + static_cast<size_t>(nblk) * (kActQBytes + kActSBytes));
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t G = gridDim.x;
    const int64_t R = sd.round0[sd.count];
    const int64_t nk = blockIdx.x < R ? (R - 1 - blockIdx.x) / G + 1 : 0;  // this workgroup's rounds
    if (nk == 0) return;  // the whole workgroup

    // 1. X loads: thread t takes quad t & 7 of blocks t / 8 + 128 j (block g
    //    of the concatenation: product m's block g - boff[m]).  The product's
    //    fields are picked by selects over constant indices (a lane-dependent
    //    index into the argument block would read it from memory).
    constexpr int kJ = kSetMaxBlocks / (kSetThreads / 8);
    int bo[kMaxMulti];
    uint64_t xa[kMaxMulti];
#pragma unroll
    for (int i = 0; i < kMaxMulti; ++i) {
        bo[i] = i < sd.count ? sd.boff[i] : kSetMaxBlocks;
        xa[i] = reinterpret_cast<uint64_t>(sd.x[i]);
    }
    float4 xv[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
        const int g = static_cast<int>(threadIdx.x >> 3) + (kSetThreads / 8) * j;
        uint64_t xp = xa[0];
        int b0 = 0;
#pragma unroll
        for (int i = 1; i < kMaxMulti; ++i) {
            const bool in = g >= bo[i];
            xp = in ? xa[i] : xp;
            b0 = in ? bo[i] : b0;
        }
        xv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (g < nblk)
            __builtin_memcpy(&xv[j], reinterpret_cast<const float*>(xp) + static_cast<int64_t>(g - b0) * kQK +
                                         4 * (threadIdx.x & 7), 16);
    }

    // 2. the first D rounds' weights.  Round r: product m (round0[m] <= r <
    //    round0[m + 1]), its rows (r - round0[m]) * 16 / C + w / C, chunk
    //    w mod C; lanes past the chunk and rows past the product re-read its
    //    last pair or row (their terms are dropped), so every wave issues the
    //    same loads
    // A wave's rounds r = blockIdx.x + k G only move forward through the
    // products, so each of the two streams (the loads, D rounds ahead, and the
    // folds) keeps its current product's fields in scalar registers and
    // reloads them only when it passes into the next product (a scalar load
    // per round would wait for the LDS reads in flight as well).
    struct Cursor {
        int m;
        int64_t r0, r1;  // the product's rounds [r0, r1)
        const uint8_t* w;
        int64_t rows;
        int nb, Pc, C, boff;
    };
    auto cursor_set = [&](Cursor& q, int m) __attribute__((always_inline)) {
        q.m = m;
        q.r0 = sd.round0[m];
        q.r1 = sd.round0[m + 1];
        q.w = sd.w[m];
        q.rows = sd.rows[m];
        q.nb = sd.nb[m];
        q.Pc = sd.Pc[m];
        q.C = sd.C[m];
        q.boff = sd.boff[m];
    };
    auto cursor_seek = [&](Cursor& q, int64_t r) __attribute__((always_inline)) {
        while (r >= q.r1 && q.m + 1 < sd.count) cursor_set(q, q.m + 1);
    };
    Cursor lcur, fcur;
    cursor_set(lcur, 0);
    cursor_set(fcur, 0);
    struct RoundAt {
        int64_t row;  // this wave's row (unclamped)
        int c;        // its chunk
    };
    auto round_at = [&](Cursor& q, int64_t k) __attribute__((always_inline)) {
        const int64_t r = blockIdx.x + min(k, nk - 1) * G;
        cursor_seek(q, r);
        RoundAt a;
        a.row = (r - q.r0) * (kSetWaves / q.C) + wave / q.C;
        a.c = wave % q.C;
        return a;
    };
    auto load_round = [&](Pair36& dst, int64_t k) __attribute__((always_inline)) {
        const RoundAt a = round_at(lcur, k);
        const int64_t row = min(a.row, lcur.rows - 1);
        const int p = a.c * lcur.Pc + min(lane, lcur.Pc - 1);
        const uint8_t* wr = lcur.w + uniform64(row * lcur.nb) * kQ4Bytes;
        dst = load_pair(wr + 36 * p);
    };
    Pair36 raw[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_round(raw[d], d);
        __builtin_amdgcn_sched_barrier(0);
    }

    // 3. X into LDS as the quantizer's blocks and records (measured: spreading
    //    these passes over the rounds, or running each product's just before
    //    its first round, does not shorten the launch)
    {
        const int qd = threadIdx.x & 7;
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int g = static_cast<int>(threadIdx.x >> 3) + (kSetThreads / 8) * j;
            if (j * (kSetThreads / 8) >= nblk) break;  // (uniform) no block of this pass
            uint32_t word;
            const ActScale sc = quant_act_quad(xv[j].x, xv[j].y, xv[j].z, xv[j].w, qd, word);
            if (g < nblk) {
                sq[g * 8 + qd] = word;
                if (qd == 0) ss[g] = sc;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // 4. the rounds: fold, wave sum (lane 63), partial to LDS slot k * 16 + w
    for (int64_t k = 0; k < nk; k += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (k + d < nk) {
                const RoundAt a = round_at(fcur, k + d);
                const bool valid = lane < fcur.Pc;
                const int p = a.c * fcur.Pc + min(lane, fcur.Pc - 1);
                float v[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const Block4 blk = h ? pair_second(raw[d]) : pair_first(raw[d]);
                    const float dw = half_bits_to_float(blk.dbits);
                    const int g = fcur.boff + 2 * p + h;
                    const u32x4 a0 = reinterpret_cast<const u32x4*>(sq)[g * 2];
                    const u32x4 a1 = reinterpret_cast<const u32x4*>(sq)[g * 2 + 1];
                    const uint32_t act[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                    const ActScale sc = ss[g];
                    const int32_t s = block_dot(blk, act, sc.bias);
                    v[h] = static_cast<float>(s) * (dw * sc.d);
                }
                const float part[1] = {valid ? v[0] + v[1] : 0.0f};
                const float t = wave_sums<1>(part, lane);
                if (lane == 63) pl[(k + d) * kSetWaves + wave] = t;
            }
            load_round(raw[d], k + d + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // 5. every partial is in LDS: wave w stores rounds w, w + 16, ... (lane q:
    //    row q of the round, its C chunks added in chunk order)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    for (int64_t k = wave; k < nk; k += kSetWaves) {
        const int64_t r = blockIdx.x + k * G;
        int m = 0;
#pragma unroll
        for (int i = 1; i < kMaxMulti; ++i)
            if (i < sd.count && r >= sd.round0[i]) m = i;
        m = __builtin_amdgcn_readfirstlane(m);
        const int C = sd.C[m];
        const int rpr = kSetWaves / C;
        const int64_t row = (r - sd.round0[m]) * rpr + lane;
        if (lane < rpr && row < sd.rows[m]) {
            const float* src = pl + k * kSetWaves + lane * C;
            float y = src[0];
            for (int c = 1; c < C; ++c) y += src[c];
            sd.y[m][row] = y;
        }
    }
}

}  // namespace

bool set_plan(SetDesc& sd, int64_t num_cu) {
    int64_t round = 0;
    int boff = 0;
    sd.round0[0] = 0;
    for (int m = 0; m < sd.count; ++m) {
        const int nb = sd.nb[m];
        if (nb & 1) return false;
        const int P = nb >> 1;
        int C = 1;
        while (C <= kSetWaves && (P % C != 0 || P / C > 64)) C *= 2;
        if (C > kSetWaves) return false;
        sd.C[m] = C;
        sd.Pc[m] = P / C;
        sd.boff[m] = boff;
        boff += nb;
        if (boff > kSetMaxBlocks) return false;
        round += (sd.rows[m] * C + kSetWaves - 1) / kSetWaves;
        sd.round0[m + 1] = round;
    }
    sd.nblk = boff;
    const int64_t grid = round < num_cu ? round : num_cu;
    return (round + grid - 1) / grid <= kSetMaxRounds;
}

size_t set_lds_bytes(const SetDesc& sd) {
    return static_cast<size_t>(sd.nblk) * (kActQBytes + kActSBytes) +
           static_cast<size_t>(kSetMaxRounds) * kSetWaves * sizeof(float);
}

hipError_t launch_gemv_set(const DeviceInfo* dev, const SetDesc& sd, hipStream_t s) {
    const int64_t R = sd.round0[sd.count];
    const int64_t grid = R < dev->num_cu ? R : dev->num_cu;
    const size_t lds = set_lds_bytes(sd);
    const auto kernel = k_gemv_set<kSetD>;
    if (lds > 64 * 1024) {
        const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                                      static_cast<int>(lds));
        if (raised != hipSuccess) return raised;
    }
    hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(grid)), dim3(kSetThreads), lds, s, sd);
    return hipGetLastError();
}

}  // namespace q4bq
