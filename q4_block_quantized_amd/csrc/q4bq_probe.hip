// Peak-rate probes for the benchmark's roofline figures (libq4bq_probe.so; not
// part of the product library): how fast this MI355X actually runs the
// instructions the product kernels are built from, measured the same way the
// kernels are (HIP events on the caller's stream).
//
//   q4bq_probe_mfma(kind, iters, out, stream):
//     kind 0  v_mfma_i32_32x32x32_i8            (int8, 65536 ops per instruction)
//     kind 1  v_mfma_scale_f32_32x32x64_f8f6f4  with fp6 e2m3 operands (131072)
//     kind 2  v_mfma_f32_32x32x8_f16            (16384: the prefill's scale products)
//     kind 3  v_fma_f32 on the vector ALU       (2 flops per lane)
//   Every wave runs `iters` rounds of four independent instructions (no
//   dependence between rounds other than through the accumulators, which the
//   matrix core chains without stalls); 1024 workgroups of 256 threads, i.e.
//   16 waves per CU.  Ops per launch: q4bq_probe_ops(kind, iters).  `out`
//   receives one value per thread (so nothing is optimised away): a device
//   buffer of q4bq_probe_threads() floats.
//
//   q4bq_probe_read(src, bytes, out, stream): streams `bytes` (a multiple of
//   16, src 16-byte aligned) with 16-byte non-temporal loads, each wave
//   instruction reading 1 KB contiguous, grid-stride, and writes one xor per
//   thread to `out` (q4bq_probe_threads() floats): the streaming-read
//   bandwidth the decode kernels are measured against.
//
// Returns 0, -1 (bad argument) or -2 (HIP error).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 1024;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kThreads) k_probe_i8(int64_t iters, float* __restrict__ out) {
    const int l = threadIdx.x;
    const i32x4 a = {l, l * 3, l * 5, l * 7};
    const i32x4 b = {l * 11, l * 13, l * 17, l * 19};
    i32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += c0[v] ^ c1[v] ^ c2[v] ^ c3[v];
    out[blockIdx.x * kThreads + threadIdx.x] = static_cast<float>(s);
}

__global__ void __launch_bounds__(kThreads) k_probe_fp6(int64_t iters, float* __restrict__ out) {
    const int l = threadIdx.x;
    // fp6 operands: 6 of the 8 dwords carry the 32 codes (any bit pattern is
    // a finite e2m3 value)
    const i32x8 a = {l, l * 3, l * 5, l * 7, l * 9, l * 11, 0, 0};
    const i32x8 b = {l * 13, l * 17, l * 19, l * 23, l * 29, l * 31, 0, 0};
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 2, 2, 0, 120, 0, 120);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 2, 2, 0, 120, 0, 120);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 2, 2, 0, 120, 0, 120);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 2, 2, 0, 120, 0, 120);
    }
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

__global__ void __launch_bounds__(kThreads) k_probe_f16(int64_t iters, float* __restrict__ out) {
    const _Float16 x = static_cast<_Float16>((threadIdx.x & 7) * 0.125f);
    const f16x4 a = {x, x, x, x};
    const f16x4 b = {x, static_cast<_Float16>(0.5f), x, static_cast<_Float16>(0.25f)};
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x8f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x8f16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x8f16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x8f16(b, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// 16 independent fp32 FMA chains per lane (enough to cover the ALU latency);
// 16 FMAs per round.
__global__ void __launch_bounds__(kThreads) k_probe_valu(int64_t iters, float* __restrict__ out) {
    float x[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = static_cast<float>(threadIdx.x + k) * 1e-3f;
    const float m = 0.999f + static_cast<float>(blockIdx.x & 1) * 1e-7f;
    const float c = 1e-4f;
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < 16; ++k) x[k] = fmaf(x[k], m, c);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) s += x[k];
    out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// 1024 threads a workgroup, 256 workgroups (the same thread count as the
// other probes): chunks of 4 x 1024 consecutive 16-byte pieces, lane t taking
// pieces t, t + 1024, t + 2048, t + 3072 of a chunk (each load instruction one
// contiguous 1 KB per wave), non-temporal, grid-stride over the chunks.
// Measured on this GPU: ~6.9 TB/s over 1 GiB, against ~5.7 TB/s with the four
// loads of a lane a grid stride apart and ~6.2 TB/s with plain loads.
constexpr int kReadThreads = 1024;
constexpr int kReadBlocks = kBlocks * kThreads / kReadThreads;
__global__ void __launch_bounds__(kReadThreads)
k_probe_read(const u32x4* __restrict__ src, int64_t n16, float* __restrict__ out) {
    uint32_t acc = 0;
    constexpr int kU = 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kReadThreads * kU;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kReadThreads * kU + threadIdx.x; base < n16;
         base += stride) {
        u32x4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kReadThreads;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[blockIdx.x * kReadThreads + threadIdx.x] = static_cast<float>(acc);
}

}  // namespace

extern "C" {

int q4bq_probe_threads(void) { return kBlocks * kThreads; }

double q4bq_probe_ops(int kind, int64_t iters) {
    const double per_wave_round = kind == 0 ? 4.0 * 65536 : kind == 1 ? 4.0 * 131072
                                : kind == 2 ? 4.0 * 16384 : 16.0 * 2 * 64;
    return per_wave_round * static_cast<double>(iters) * (kBlocks * kThreads / 64);
}

int q4bq_probe_mfma(int kind, int64_t iters, float* out, void* stream) {
    if (!out || iters < 1 || kind < 0 || kind > 3) return -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    switch (kind) {
        case 0: hipLaunchKernelGGL(k_probe_i8, dim3(kBlocks), dim3(kThreads), 0, s, iters, out); break;
        case 1: hipLaunchKernelGGL(k_probe_fp6, dim3(kBlocks), dim3(kThreads), 0, s, iters, out); break;
        case 2: hipLaunchKernelGGL(k_probe_f16, dim3(kBlocks), dim3(kThreads), 0, s, iters, out); break;
        default: hipLaunchKernelGGL(k_probe_valu, dim3(kBlocks), dim3(kThreads), 0, s, iters, out); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int q4bq_probe_read(const void* src, int64_t bytes, float* out, void* stream) {
    if (!src || !out || bytes < 16 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15)) return -1;
    hipLaunchKernelGGL(k_probe_read, dim3(kReadBlocks), dim3(kReadThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
