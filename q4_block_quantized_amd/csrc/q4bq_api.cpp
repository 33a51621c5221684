// C ABI of libq4bq.so: argument checks, dispatch, scratch handling.
// See include/q4bq.h for the contract of each entry point.
#include "q4bq.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "q4bq_internal.h"

namespace q4bq {

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];
hipError_t g_dev_err[kMaxDevices];

// Largest sizes accepted: keep every byte offset far inside int64 and every
// per-row block index inside int32.
constexpr int64_t kMaxDim = int64_t(1) << 40;
constexpr int64_t kMaxBlocksPerRow = int64_t(1) << 30;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bn && y < x + an;
}

bool bad_k(int64_t K) { return K < kQK || K % kQK != 0 || K / kQK > kMaxBlocksPerRow; }
bool bad_dim(int64_t n) { return n < 1 || n > kMaxDim; }

int status_of(hipError_t e) { return e == hipSuccess ? Q4BQ_OK : Q4BQ_EHIP; }

// Sizes whose products could overflow the byte arithmetic are rejected.
bool too_big(int64_t a, int64_t b, int64_t bytes_per) {
    // a * b * bytes_per < 2^62
    const double v = static_cast<double>(a) * static_cast<double>(b) * static_cast<double>(bytes_per);
    return v >= 4.0e18;
}

// A few more tokens than the decode kernels take at once run as groups of up
// to kGemvMaxN through the decode path, where the row-streaming or the
// matrix-core decode kernel takes the shape: the prefill kernel's workgroup
// always computes 224 rows x 128 tokens, so below a few dozen tokens most of
// its work is padding.  Up to 16 tokens, and up to 32 where the prefill
// kernel would not split K.  Measured (graph-timed, workspace form), prefill -> groups: 14336 x
// 4096 at N = 9 / 32 86.4 / 87.6 -> 22.1 / 50.8 us; 4096 x 14336 278 / 279 ->
// 65 / 215 us; the 128256 x 4096 head 255 / 259 -> 105 / 233 us; 2304 x 768
// 23.8 / 24.7 -> 9.8 / 24.5 us.
// (Where the prefill kernel splits K, from 17 tokens on it is the faster one:
// 14336 x 4096 at N = 32 ~40 against 51 us as groups, 4096 x 14336 at N = 16
// 85 against 110 us.)
constexpr int64_t kDecodeGroupsMaxN = 32;
constexpr int64_t kDecodeGroupsSplitMaxN = 16;
constexpr int64_t kQ8wGroupsMaxN = 32;
constexpr int64_t kQ8wGroupsSplitMaxN = 16;
constexpr int64_t kQ8wGroupsLongRows = 65536;
bool decode_groups_pay(const DeviceInfo* dev, int64_t N, int64_t nb, int64_t rows) {
    if (N > kDecodeGroupsMaxN || !(rows_apply(kGemvMaxN, nb, rows) || mma_apply(kGemvMaxN, nb, rows))) return false;
    int kbs = 0;
    return N <= kDecodeGroupsSplitMaxN || prefill_splits(rows, nb, N, dev->num_cu, &kbs) == 1;
}

// Workspace layout: the activations (act_bytes, rounded up to 256 bytes), then
// room for the prefill kernel's split sums.
size_t act_ws_bytes(int64_t N, int64_t nb) { return (act_bytes(N, nb) + 255) & ~static_cast<size_t>(255); }

// ws_bytes: the workspace's size (the prefill kernel splits K only where its
// partial sums fit behind the activations).
int run_product(WLayout lay, const uint8_t* Wq, int64_t rows, int64_t K, const float* X, const uint8_t* Xq,
                int64_t N, float* Y, int32_t* D, void* ws, size_t ws_bytes, hipStream_t s) {
    hipError_t err = hipSuccess;
    const DeviceInfo* dev = current_device(&err);
    if (!dev) return Q4BQ_EHIP;
    const int64_t nb = K / kQK;
    // without a workspace the fused kernel runs whenever it fits (run_with_scratch
    // passes none in exactly that case)
    if (X && !D && (ws ? gemv_prefers_fused(N, nb, rows) : gemv_fuses(N, nb, rows)))
        return status_of(launch_gemv_fused(dev, lay, Wq, rows, nb, X, N, Y, s));
    if (N > kGemvMaxN && !D && decode_groups_pay(dev, N, nb, rows)) {
        // up to kGemvMaxN tokens at a time through the decode path: token n0's
        // inputs and outputs start n0 rows into X (Xq) and Y
        for (int64_t n0 = 0; n0 < N; n0 += kGemvMaxN) {
            const int64_t g = N - n0 < kGemvMaxN ? N - n0 : kGemvMaxN;
            const int rc = run_product(lay, Wq, rows, K, X ? X + n0 * K : nullptr,
                                       Xq ? Xq + n0 * nb * kQ8Bytes : nullptr, g, Y + n0 * rows, nullptr, ws,
                                       ws_bytes, s);
            if (rc != Q4BQ_OK) return rc;
        }
        return Q4BQ_OK;
    }
    err = X ? launch_act_from_f32(X, N, nb, ws, s) : launch_act_from_q8(Xq, N, nb, ws, s);
    if (err != hipSuccess) return Q4BQ_EHIP;
    if (N <= kGemvMaxN) {
        err = launch_gemv(dev, lay, Wq, rows, nb, ws, N, Y, D, s);
    } else {
        const size_t off = act_ws_bytes(N, nb);
        float* partial = ws_bytes > off ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + off) : nullptr;
        err = launch_prefill(dev, lay, Wq, rows, nb, ws, N, Y, D, s, Epilogue{nullptr, nullptr, kEpiNone}, partial,
                             partial ? ws_bytes - off : 0);
    }
    return status_of(err);
}

// Runs the product with stream-ordered scratch taken from the device pool.
int run_with_scratch(WLayout lay, const uint8_t* Wq, int64_t rows, int64_t K, const float* X, const uint8_t* Xq,
                     int64_t N, float* Y, int32_t* D, hipStream_t s) {
    hipError_t err = hipSuccess;
    if (!current_device(&err)) return Q4BQ_EHIP;
    if (X && !D && gemv_fuses(N, K / kQK, rows)) return run_product(lay, Wq, rows, K, X, Xq, N, Y, D, nullptr, 0, s);
    const size_t bytes = q4bq_workspace_size(rows, K, N);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, bytes, s) != hipSuccess || ws == nullptr) {
        (void)hipGetLastError();
        return Q4BQ_ENOMEM;
    }
    const int rc = run_product(lay, Wq, rows, K, X, Xq, N, Y, D, ws, bytes, s);
    if (hipFreeAsync(ws, s) != hipSuccess) return Q4BQ_EHIP;
    return rc;
}

}  // namespace

const DeviceInfo* current_device(hipError_t* err) {
    int id = 0;
    hipError_t e = hipGetDevice(&id);
    if (e != hipSuccess || id < 0 || id >= kMaxDevices) {
        *err = e != hipSuccess ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_once[id], [id] {
        DeviceInfo d{id, 0, 1};
        hipError_t r = hipDeviceGetAttribute(&d.num_cu, hipDeviceAttributeMultiprocessorCount, id);
        if (r == hipSuccess && d.num_cu <= 0) r = hipErrorInvalidDevice;
        d.num_xcd = 8;
        g_dev[id] = d;
        g_dev_err[id] = r;
    });
    if (g_dev_err[id] != hipSuccess) {
        *err = g_dev_err[id];
        return nullptr;
    }
    return &g_dev[id];
}

}  // namespace q4bq

using namespace q4bq;

extern "C" {

int q4_0_quantize(const float* W, int64_t rows, int64_t K, void* Wq, void* stream) {
    if (!W || !Wq || bad_dim(rows) || bad_k(K) || too_big(rows, K, 4)) return Q4BQ_EINVAL;
    if (!aligned(W, 4) || !aligned(Wq, 2)) return Q4BQ_EINVAL;
    const int64_t nblocks = rows * (K / kQK);
    if (overlap(W, static_cast<size_t>(rows * K) * 4, Wq, static_cast<size_t>(nblocks) * kQ4Bytes))
        return Q4BQ_EINVAL;
    return status_of(launch_q4_0_quantize(W, nblocks, static_cast<uint8_t*>(Wq), static_cast<hipStream_t>(stream)));
}

int q8_0_quantize(const float* X, int64_t N, int64_t K, void* Xq, void* stream) {
    if (!X || !Xq || bad_dim(N) || bad_k(K) || too_big(N, K, 4)) return Q4BQ_EINVAL;
    if (!aligned(X, 4) || !aligned(Xq, 2)) return Q4BQ_EINVAL;
    const int64_t nblocks = N * (K / kQK);
    if (overlap(X, static_cast<size_t>(N * K) * 4, Xq, static_cast<size_t>(nblocks) * kQ8Bytes))
        return Q4BQ_EINVAL;
    return status_of(launch_q8_0_quantize(X, nblocks, static_cast<uint8_t*>(Xq), static_cast<hipStream_t>(stream)));
}

size_t q4bq_repack_size(int64_t rows, int64_t K) {
    if (bad_dim(rows) || bad_k(K) || too_big(rows, K + kQK, 2)) return 0;
    return repack_bytes(rows, K / kQK);
}

int q4_0_repack(const void* Wq, int64_t rows, int64_t K, void* Wr, void* stream) {
    if (!Wq || !Wr || bad_dim(rows) || bad_k(K) || too_big(rows, K + kQK, 2)) return Q4BQ_EINVAL;
    if (!aligned(Wq, 2) || !aligned(Wr, 16)) return Q4BQ_EINVAL;
    const int64_t nb = K / kQK;
    if (overlap(Wq, static_cast<size_t>(rows * nb) * kQ4Bytes, Wr, repack_bytes(rows, nb))) return Q4BQ_EINVAL;
    hipError_t err = hipSuccess;
    if (!current_device(&err)) return Q4BQ_EHIP;
    return status_of(launch_q4_0_repack(static_cast<const uint8_t*>(Wq), rows, nb, static_cast<uint8_t*>(Wr),
                                        static_cast<hipStream_t>(stream)));
}

int q4_0_get_rows(const void* Wq, int64_t rows, int64_t K, const int32_t* ids, int64_t n, float* out, void* stream) {
    if (!Wq || !ids || !out || bad_dim(rows) || bad_dim(n) || bad_k(K) || too_big(rows, K, 1) || too_big(n, K, 4))
        return Q4BQ_EINVAL;
    if (!aligned(Wq, 2) || !aligned(ids, 4) || !aligned(out, 16)) return Q4BQ_EINVAL;
    const int64_t nb = K / kQK;
    const size_t o_bytes = static_cast<size_t>(n * K) * 4;
    if (overlap(out, o_bytes, Wq, static_cast<size_t>(rows * nb) * kQ4Bytes) ||
        overlap(out, o_bytes, ids, static_cast<size_t>(n) * 4))
        return Q4BQ_EINVAL;
    hipError_t err = hipSuccess;
    if (!current_device(&err)) return Q4BQ_EHIP;
    return status_of(launch_q4_0_get_rows(static_cast<const uint8_t*>(Wq), rows, nb, ids, n, out,
                                          static_cast<hipStream_t>(stream)));
}

size_t q4bq_workspace_size(int64_t rows, int64_t K, int64_t N) {
    if (bad_dim(rows) || bad_dim(N) || bad_k(K) || too_big(N, K, 4)) return 0;
    const int64_t nb = K / kQK;
    size_t b = act_ws_bytes(N, nb);
    if (N > kGemvMaxN && !too_big(N, rows, 4 * kPrefillMaxSplits)) b += prefill_partial_bytes(rows, nb, N);
    return b;
}

}  // extern "C"

namespace {

// Common checks of the product entry points.  The activation operand is one
// of: fp32 X (kF32, 4-byte aligned), Q8_0 blocks (kQ8, 2-byte aligned) or the
// library's prepared workspace (kPrepared, 16-byte aligned).  dots: the output
// is the int32 block-dot array (N * rows * K/32) instead of Y (N * rows).
enum ActKind { kF32, kQ8, kPrepared };

int check_product(const void* Wq, int64_t rows, int64_t K, const void* Xany, ActKind kind, int64_t N,
                  const void* out, bool dots, WLayout lay = kAoS) {
    if (!Wq || !Xany || !out || bad_dim(rows) || bad_dim(N) || bad_k(K)) return Q4BQ_EINVAL;
    const int64_t nb = K / kQK;
    if (too_big(rows, K, 1) || too_big(N, K, 4) || too_big(N, rows, 4)) return Q4BQ_EINVAL;
    if (dots && too_big(N * rows, nb, 4)) return Q4BQ_EINVAL;
    // the matrix-core kernel's grid must stay within HIP's work-item limit
    if (N > kGemvMaxN &&
        ((rows + kPrefillRows - 1) / kPrefillRows) * ((N + kPrefillTokens - 1) / kPrefillTokens) >
            kMaxWorkItems / kPrefillThreads)
        return Q4BQ_EINVAL;
    const uintptr_t x_align = kind == kF32 ? 4 : kind == kQ8 ? 2 : 16;
    if (!aligned(Wq, lay == kRepacked ? 16 : 2) || !aligned(Xany, x_align) || !aligned(out, 4)) return Q4BQ_EINVAL;
    if (lay == kRepacked && too_big(rows, K + kQK, 2)) return Q4BQ_EINVAL;
    const size_t w_bytes = lay == kRepacked ? repack_bytes(rows, nb) : static_cast<size_t>(rows * nb) * kQ4Bytes;
    const size_t x_bytes = kind == kF32 ? static_cast<size_t>(N * K) * 4
                           : kind == kQ8 ? static_cast<size_t>(N * nb) * kQ8Bytes
                                         : act_bytes(N, nb);
    const size_t o_bytes = static_cast<size_t>(N * rows) * 4 * static_cast<size_t>(dots ? nb : 1);
    if (overlap(out, o_bytes, Wq, w_bytes) || overlap(out, o_bytes, Xany, x_bytes)) return Q4BQ_EINVAL;
    return Q4BQ_OK;
}

}  // namespace

extern "C" {

int mul_mat_q4_0_q8_0(const void* Wq, int64_t rows, int64_t K, const float* X, int64_t N, float* Y, void* stream) {
    const int rc = check_product(Wq, rows, K, X, kF32, N, Y, false);
    if (rc != Q4BQ_OK) return rc;
    return run_with_scratch(kAoS, static_cast<const uint8_t*>(Wq), rows, K, X, nullptr, N, Y, nullptr,
                            static_cast<hipStream_t>(stream));
}

int mul_mat_q4_0_q8_0_ex(const void* Wq, int64_t rows, int64_t K, const float* X, int64_t N, float* Y,
                         void* workspace, size_t ws_bytes, void* stream) {
    const int rc = check_product(Wq, rows, K, X, kF32, N, Y, false);
    if (rc != Q4BQ_OK) return rc;
    if (!workspace || !aligned(workspace, 16)) return Q4BQ_EINVAL;
    const size_t need = q4bq_workspace_size(rows, K, N);
    if (ws_bytes < need) return Q4BQ_ENOMEM;
    const int64_t nb = K / kQK;
    if (overlap(workspace, need, Y, static_cast<size_t>(N * rows) * 4) ||
        overlap(workspace, need, X, static_cast<size_t>(N * K) * 4) ||
        overlap(workspace, need, Wq, static_cast<size_t>(rows * nb) * kQ4Bytes))
        return Q4BQ_EINVAL;
    // (only the checked `need` bytes are used)
    return run_product(kAoS, static_cast<const uint8_t*>(Wq), rows, K, X, nullptr, N, Y, nullptr, workspace, need,
                       static_cast<hipStream_t>(stream));
}

int mul_mat_q4_0r_q8_0(const void* Wr, int64_t rows, int64_t K, const float* X, int64_t N, float* Y, void* stream) {
    const int rc = check_product(Wr, rows, K, X, kF32, N, Y, false, kRepacked);
    if (rc != Q4BQ_OK) return rc;
    return run_with_scratch(kRepacked, static_cast<const uint8_t*>(Wr), rows, K, X, nullptr, N, Y, nullptr,
                            static_cast<hipStream_t>(stream));
}

int mul_mat_q4_0r_q8_0_ex(const void* Wr, int64_t rows, int64_t K, const float* X, int64_t N, float* Y,
                          void* workspace, size_t ws_bytes, void* stream) {
    const int rc = check_product(Wr, rows, K, X, kF32, N, Y, false, kRepacked);
    if (rc != Q4BQ_OK) return rc;
    if (!workspace || !aligned(workspace, 16)) return Q4BQ_EINVAL;
    const size_t need = q4bq_workspace_size(rows, K, N);
    if (ws_bytes < need) return Q4BQ_ENOMEM;
    const int64_t nb = K / kQK;
    if (overlap(workspace, need, Y, static_cast<size_t>(N * rows) * 4) ||
        overlap(workspace, need, X, static_cast<size_t>(N * K) * 4) ||
        overlap(workspace, need, Wr, repack_bytes(rows, nb)))
        return Q4BQ_EINVAL;
    return run_product(kRepacked, static_cast<const uint8_t*>(Wr), rows, K, X, nullptr, N, Y, nullptr, workspace,
                       need, static_cast<hipStream_t>(stream));
}

int mul_mat_q4_0_q8_0_multi(int count, const void* const* Wq, const int64_t* rows, int64_t K, const float* X,
                            int64_t N, float* const* Y, void* workspace, size_t ws_bytes, void* stream) {
    if (count < 1 || count > kMaxMulti || !Wq || !rows || !Y) return Q4BQ_EINVAL;
    const int64_t nb = bad_k(K) ? 0 : K / kQK;
    MultiDesc md{};
    md.count = count;
    md.first[0] = 0;
    for (int i = 0; i < count; ++i) {
        const int rc = check_product(Wq[i], rows[i], K, X, kF32, N, Y[i], false);
        if (rc != Q4BQ_OK) return rc;
        md.w[i] = static_cast<const uint8_t*>(Wq[i]);
        md.y[i] = Y[i];
        md.first[i + 1] = md.first[i] + rows[i];
    }
    if (bad_dim(md.first[count]) || too_big(md.first[count], K, 1)) return Q4BQ_EINVAL;
    for (int i = 0; i < count; ++i)
        for (int j = 0; j < count; ++j) {
            const size_t yb = static_cast<size_t>(N * rows[i]) * 4;
            if (overlap(Y[i], yb, Wq[j], static_cast<size_t>(rows[j] * nb) * kQ4Bytes)) return Q4BQ_EINVAL;
            if (i != j && overlap(Y[i], yb, Y[j], static_cast<size_t>(N * rows[j]) * 4)) return Q4BQ_EINVAL;
        }
    const size_t need = act_ws_bytes(N, K / kQK);  // the activations alone (no rows: no split sums here)
    if (workspace) {
        if (!aligned(workspace, 16)) return Q4BQ_EINVAL;
        if (ws_bytes < need) return Q4BQ_ENOMEM;
        if (overlap(workspace, need, X, static_cast<size_t>(N * K) * 4)) return Q4BQ_EINVAL;
        for (int i = 0; i < count; ++i)
            if (overlap(workspace, need, Y[i], static_cast<size_t>(N * rows[i]) * 4) ||
                overlap(workspace, need, Wq[i], static_cast<size_t>(rows[i] * nb) * kQ4Bytes))
                return Q4BQ_EINVAL;
    }
    hipError_t err = hipSuccess;
    const DeviceInfo* dev = current_device(&err);
    if (!dev) return Q4BQ_EHIP;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t total = md.first[count];
    auto fuses = [&](int64_t n, const MultiDesc& m) {
        return n <= kGemvMaxN && (workspace ? gemv_prefers_fused(n, nb, total, &m) : gemv_fuses(n, nb, total, &m));
    };
    // more tokens than one decode launch takes: groups of up to kGemvMaxN
    // (as in run_product), each on its rows of X and of every Y
    const bool groups = N > kGemvMaxN && decode_groups_pay(dev, N, nb, total);
    const int64_t step = groups ? kGemvMaxN : N;
    bool need_ws = false;
    for (int64_t n0 = 0; n0 < N; n0 += step) need_ws = need_ws || !fuses(N - n0 < step ? N - n0 : step, md);
    void* ws = workspace;
    if (need_ws && !ws && (hipMallocAsync(&ws, need, s) != hipSuccess || ws == nullptr)) {
        (void)hipGetLastError();
        return Q4BQ_ENOMEM;
    }
    for (int64_t n0 = 0; n0 < N && err == hipSuccess; n0 += step) {
        const int64_t g = N - n0 < step ? N - n0 : step;
        MultiDesc mg = md;
        for (int i = 0; i < count; ++i) mg.y[i] = Y[i] + n0 * rows[i];
        const float* Xg = X + n0 * K;
        if (fuses(g, mg)) {
            err = launch_gemv_multi(dev, mg, nb, Xg, nullptr, g, s);
            continue;
        }
        err = launch_act_from_f32(Xg, g, nb, ws, s);
        if (err != hipSuccess) break;
        if (g <= kGemvMaxN) {
            err = launch_gemv_multi(dev, mg, nb, nullptr, ws, g, s);
        } else {
            for (int i = 0; i < count && err == hipSuccess; ++i)
                err = launch_prefill(dev, kAoS, mg.w[i], rows[i], nb, ws, g, mg.y[i], nullptr, s);
        }
    }
    if (need_ws && !workspace && hipFreeAsync(ws, s) != hipSuccess) return Q4BQ_EHIP;
    return status_of(err);
}

int mul_mat_q4_0_q8_0_set(int count, const void* const* Wq, const int64_t* rows, const int64_t* K,
                          const float* const* X, float* const* Y, void* stream) {
    if (count < 1 || count > kMaxMulti || !Wq || !rows || !K || !X || !Y) return Q4BQ_EINVAL;
    SetDesc sd{};
    sd.count = count;
    for (int i = 0; i < count; ++i) {
        const int rc = check_product(Wq[i], rows[i], K[i], X[i], kF32, 1, Y[i], false);
        if (rc != Q4BQ_OK) return rc;
        sd.w[i] = static_cast<const uint8_t*>(Wq[i]);
        sd.x[i] = X[i];
        sd.y[i] = Y[i];
        sd.rows[i] = rows[i];
        sd.nb[i] = static_cast<int>(K[i] / kQK);
    }
    // no output may overlap another product's weights, activations or output
    for (int i = 0; i < count; ++i)
        for (int j = 0; j < count; ++j) {
            if (i == j) continue;
            const size_t yb = static_cast<size_t>(rows[i]) * 4;
            if (overlap(Y[i], yb, Wq[j], static_cast<size_t>(rows[j] * (K[j] / kQK)) * kQ4Bytes) ||
                overlap(Y[i], yb, X[j], static_cast<size_t>(K[j]) * 4) ||
                overlap(Y[i], yb, Y[j], static_cast<size_t>(rows[j]) * 4))
                return Q4BQ_EINVAL;
        }
    hipError_t err = hipSuccess;
    const DeviceInfo* dev = current_device(&err);
    if (!dev) return Q4BQ_EHIP;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (set_plan(sd, dev->num_cu)) return status_of(launch_gemv_set(dev, sd, s));
    // shapes the one launch does not take: the products one by one
    for (int i = 0; i < count; ++i) {
        const int rc = run_with_scratch(kAoS, sd.w[i], rows[i], K[i], X[i], nullptr, 1, Y[i], nullptr, s);
        if (rc != Q4BQ_OK) return rc;
    }
    return Q4BQ_OK;
}

int mul_mat_q4_0_q8_0_pq(const void* Wq, int64_t rows, int64_t K, const void* Xq, int64_t N, float* Y,
                         void* stream) {
    const int rc = check_product(Wq, rows, K, Xq, kQ8, N, Y, false);
    if (rc != Q4BQ_OK) return rc;
    return run_with_scratch(kAoS, static_cast<const uint8_t*>(Wq), rows, K, nullptr, static_cast<const uint8_t*>(Xq),
                            N, Y, nullptr, static_cast<hipStream_t>(stream));
}

int mul_mat_q4_0_q8_0_noalloc(const void* Wq, int64_t rows, int64_t K, const float* X, int64_t N, float* Y,
                              void* stream) {
    const int rc = check_product(Wq, rows, K, X, kF32, N, Y, false);
    if (rc != Q4BQ_OK) return rc;
    hipError_t err = hipSuccess;
    const DeviceInfo* dev = current_device(&err);
    if (!dev) return Q4BQ_EHIP;
    // the activations and, where the prefill kernel splits K, its partial sums
    const int64_t nb = K / kQK;
    size_t need = act_ws_bytes(N, nb);
    if (N > kGemvMaxN && !decode_groups_pay(dev, N, nb, rows)) need += prefill_split_bytes(dev, rows, nb, N);
    if (need > Q4BQ_NOALLOC_SCRATCH_BYTES) return Q4BQ_ESCRATCH;
    void* ws = noalloc_scratch(dev->id, &err);
    if (!ws) return Q4BQ_EHIP;
    // the scratch is device memory of its own, apart from every caller buffer
    return run_product(kAoS, static_cast<const uint8_t*>(Wq), rows, K, X, nullptr, N, Y, nullptr, ws,
                       Q4BQ_NOALLOC_SCRATCH_BYTES, static_cast<hipStream_t>(stream));
}

int q4_0_q8_0_block_dots(const void* Wq, int64_t rows, int64_t K, const void* Xq, int64_t N, int32_t* D,
                         void* stream) {
    const int rc = check_product(Wq, rows, K, Xq, kQ8, N, D, true);
    if (rc != Q4BQ_OK) return rc;
    return run_with_scratch(kAoS, static_cast<const uint8_t*>(Wq), rows, K, nullptr, static_cast<const uint8_t*>(Xq),
                            N, nullptr, D, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Checks shared by the fused forms: the LayerNorm parameters (both or
// neither), the epilogue's bias and factor, their alignment and overlaps.
int check_fusion(int64_t K, int64_t rows, int64_t N, const float* ln_gamma, const float* ln_beta, float ln_eps,
                 const float* bias, int act, const float* mul, const float* Y) {
    if ((ln_gamma == nullptr) != (ln_beta == nullptr)) return Q4BQ_EINVAL;
    if (ln_gamma && (!(ln_eps >= 0.0f) || ln_eps > 3.0e38f || N > kMaxWorkItems / kLnActThreads)) return Q4BQ_EINVAL;
    if (act != kEpiNone && act != kEpiGelu && act != kEpiSilu) return Q4BQ_EINVAL;
    if (!aligned(ln_gamma, 4) || !aligned(ln_beta, 4) || !aligned(bias, 4) || !aligned(mul, 4)) return Q4BQ_EINVAL;
    const size_t y_bytes = static_cast<size_t>(N * rows) * 4;
    if ((ln_gamma && overlap(Y, y_bytes, ln_gamma, static_cast<size_t>(K) * 4)) ||
        (ln_beta && overlap(Y, y_bytes, ln_beta, static_cast<size_t>(K) * 4)) ||
        (bias && overlap(Y, y_bytes, bias, static_cast<size_t>(rows) * 4)))
        return Q4BQ_EINVAL;
    if (mul && mul != Y && overlap(Y, y_bytes, mul, y_bytes)) return Q4BQ_EINVAL;  // in place, or apart
    return Q4BQ_OK;
}

// LayerNorm (optional) + Q8_0 of X into stream-ordered scratch, then the
// products of `count` matrices on it, each with its epilogue.
size_t fused_act_bytes(int64_t N, int64_t nb) { return (act_bytes(N, nb) + 255) & ~static_cast<size_t>(255); }
// ... and room for the matrix-core kernel's range sums where it may split K
size_t fused_ws_bytes(int64_t rows, int64_t N, int64_t nb) {
    return fused_act_bytes(N, nb) + (N > kGemvMaxN ? prefill_partial_bytes(rows, nb, N) : 0);
}

int run_fused(int count, const uint8_t* const* Wq, int64_t rows, int64_t K, const float* X, int64_t N,
              const float* ln_gamma, const float* ln_beta, float ln_eps, const Epilogue* epi, float* const* Y,
              void* workspace, size_t ws_bytes, hipStream_t s) {
    hipError_t err = hipSuccess;
    const DeviceInfo* dev = current_device(&err);
    if (!dev) return Q4BQ_EHIP;
    const int64_t nb = K / kQK;
    if (N == 1 && gemv_fuses_epi(nb, rows)) {
        // one launch per matrix: the decode kernel normalizes and quantizes
        // the token in its prologue (no scratch)
        for (int i = 0; i < count && err == hipSuccess; ++i) {
            Epilogue e = epi[i];
            e.ln_gamma = ln_gamma;
            e.ln_beta = ln_beta;
            e.ln_eps = ln_eps;
            err = launch_gemv_fused_epi(dev, Wq[i], rows, nb, X, Y[i], e, s);
        }
        return err == hipSuccess ? Q4BQ_OK : Q4BQ_EHIP;
    }
    const size_t bytes = fused_ws_bytes(rows, N, nb);
    const size_t act_b = fused_act_bytes(N, nb);
    void* ws = workspace;
    if (ws) {
        if (ws_bytes < bytes) return Q4BQ_ENOMEM;
    } else if (hipMallocAsync(&ws, bytes, s) != hipSuccess || ws == nullptr) {
        (void)hipGetLastError();
        return Q4BQ_ENOMEM;
    }
    // more tokens than one decode launch takes: groups of up to kGemvMaxN
    // (as in run_product), each on its rows of X, Y and the factor
    const int64_t step = N > kGemvMaxN && decode_groups_pay(dev, N, nb, rows) ? kGemvMaxN : N;
    for (int64_t n0 = 0; n0 < N && err == hipSuccess; n0 += step) {
        const int64_t g = N - n0 < step ? N - n0 : step;
        const float* Xg = X + n0 * K;
        if (ln_gamma) {
            err = launch_ln_act(Xg, g, nb, ln_gamma, ln_beta, ln_eps, ws, s);
        } else {
            err = launch_act_from_f32(Xg, g, nb, ws, s);
        }
        for (int i = 0; i < count && err == hipSuccess; ++i) {
            Epilogue e = epi[i];
            if (e.mul) e.mul += n0 * rows;
            float* Yg = Y[i] + n0 * rows;
            // (the range sums, where K is split, behind the activations)
            err = g <= kGemvMaxN ? launch_gemv(dev, kAoS, Wq[i], rows, nb, ws, g, Yg, nullptr, s, e)
                                 : launch_prefill(dev, kAoS, Wq[i], rows, nb, ws, g, Yg, nullptr, s, e,
                                                  reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + act_b),
                                                  bytes - act_b);
        }
    }
    const hipError_t ferr = workspace ? hipSuccess : hipFreeAsync(ws, s);
    if (err != hipSuccess) return Q4BQ_EHIP;
    return ferr == hipSuccess ? Q4BQ_OK : Q4BQ_EHIP;
}

// A caller's workspace: 16-byte aligned, apart from every other buffer.
int check_workspace(const void* ws, int64_t rows, int64_t K, int64_t N, const void* const* bufs, const size_t* sizes,
                    int nbufs) {
    if (!ws) return Q4BQ_OK;
    if (!aligned(ws, 16)) return Q4BQ_EINVAL;
    const size_t need = fused_ws_bytes(rows, N, K / kQK);
    for (int i = 0; i < nbufs; ++i)
        if (bufs[i] && overlap(ws, need, bufs[i], sizes[i])) return Q4BQ_EINVAL;
    return Q4BQ_OK;
}

}  // namespace

extern "C" {

size_t q4bq_fused_workspace_size(int64_t rows, int64_t K, int64_t N) {
    if (bad_dim(rows) || bad_dim(N) || bad_k(K) || too_big(N, K, 4) || too_big(N, rows, 4 * kPrefillMaxSplits))
        return 0;
    return fused_ws_bytes(rows, N, K / kQK);
}

int mul_mat_q4_0_q8_0_fused(const void* Wq, int64_t rows, int64_t K, const float* X, int64_t N,
                            const float* ln_gamma, const float* ln_beta, float ln_eps, const float* bias, int act,
                            const float* mul, float* Y, void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_product(Wq, rows, K, X, kF32, N, Y, false);
    if (rc != Q4BQ_OK) return rc;
    rc = check_fusion(K, rows, N, ln_gamma, ln_beta, ln_eps, bias, act, mul, Y);
    if (rc != Q4BQ_OK) return rc;
    const void* bufs[] = {Wq, X, Y, ln_gamma, ln_beta, bias, mul};
    const size_t sizes[] = {static_cast<size_t>(rows * (K / kQK)) * kQ4Bytes, static_cast<size_t>(N * K) * 4,
                            static_cast<size_t>(N * rows) * 4, static_cast<size_t>(K) * 4, static_cast<size_t>(K) * 4,
                            static_cast<size_t>(rows) * 4, static_cast<size_t>(N * rows) * 4};
    rc = check_workspace(workspace, rows, K, N, bufs, sizes, 7);
    if (rc != Q4BQ_OK) return rc;
    const uint8_t* w = static_cast<const uint8_t*>(Wq);
    const Epilogue epi{bias, mul, act};
    return run_fused(1, &w, rows, K, X, N, ln_gamma, ln_beta, ln_eps, &epi, &Y, workspace, ws_bytes,
                     static_cast<hipStream_t>(stream));
}

int mul_mat_q4_0_q8_0_swiglu(const void* Wgate, const void* Wup, int64_t rows, int64_t K, const float* X, int64_t N,
                             const float* ln_gamma, const float* ln_beta, float ln_eps, float* H, void* workspace,
                             size_t ws_bytes, void* stream) {
    int rc = check_product(Wgate, rows, K, X, kF32, N, H, false);
    if (rc != Q4BQ_OK) return rc;
    rc = check_product(Wup, rows, K, X, kF32, N, H, false);
    if (rc != Q4BQ_OK) return rc;
    rc = check_fusion(K, rows, N, ln_gamma, ln_beta, ln_eps, nullptr, kEpiNone, nullptr, H);
    if (rc != Q4BQ_OK) return rc;
    const size_t w_bytes = static_cast<size_t>(rows * (K / kQK)) * kQ4Bytes;
    const void* bufs[] = {Wgate, Wup, X, H, ln_gamma, ln_beta};
    const size_t sizes[] = {w_bytes, w_bytes, static_cast<size_t>(N * K) * 4, static_cast<size_t>(N * rows) * 4,
                            static_cast<size_t>(K) * 4, static_cast<size_t>(K) * 4};
    rc = check_workspace(workspace, rows, K, N, bufs, sizes, 6);
    if (rc != Q4BQ_OK) return rc;
    if (N == 1) {
        hipError_t err = hipSuccess;
        const DeviceInfo* dev = current_device(&err);
        if (!dev) return Q4BQ_EHIP;
        if (rows_dual_apply(dev, rows, K / kQK)) {
            // one launch: gate and up rows side by side, LayerNorm and
            // quantization of the token in its prologue
            Epilogue ln{nullptr, nullptr, kEpiNone};
            ln.ln_gamma = ln_gamma;
            ln.ln_beta = ln_beta;
            ln.ln_eps = ln_eps;
            return status_of(launch_rows_dual(dev, static_cast<const uint8_t*>(Wgate), static_cast<const uint8_t*>(Wup),
                                              rows, K / kQK, X, H, ln, static_cast<hipStream_t>(stream)));
        }
    }
    // H = SiLU(gate) first, then H = up * H in place
    const uint8_t* w[2] = {static_cast<const uint8_t*>(Wgate), static_cast<const uint8_t*>(Wup)};
    const Epilogue epi[2] = {Epilogue{nullptr, nullptr, kEpiSilu}, Epilogue{nullptr, H, kEpiNone}};
    float* const y[2] = {H, H};
    return run_fused(2, w, rows, K, X, N, ln_gamma, ln_beta, ln_eps, epi, y, workspace, ws_bytes,
                     static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// The matrix-core grid for Q8_0 weights stays within HIP's work-item limit.
bool q8w_mm_grid_ok(int64_t rows, int64_t N) {
    return ((rows + kQ8wMmRows - 1) / kQ8wMmRows) * ((N + kQ8wMmTokens - 1) / kQ8wMmTokens) <=
           kMaxWorkItems / kQ8wMmThreads;
}

// Runs the matrix-core Q8_0-weight product with stream-ordered scratch.
int run_q8w_mm(const uint8_t* W, int64_t rows, int64_t nb, const float* X, const uint8_t* Xq, int64_t N, float* Y,
               int32_t* D, hipStream_t s) {
    hipError_t derr = hipSuccess;
    const DeviceInfo* dev = current_device(&derr);
    if (!dev) return Q4BQ_EHIP;
    void* ws = nullptr;
    const size_t bytes = D ? q8w_mm_act_bytes(N, nb) : q8w_mm_scratch_bytes(rows, nb, N, dev->num_cu);
    if (hipMallocAsync(&ws, bytes, s) != hipSuccess || ws == nullptr) {
        (void)hipGetLastError();
        return Q4BQ_ENOMEM;
    }
    const hipError_t err = launch_q8w_mm(dev, W, rows, nb, X, Xq, N, Y, D, ws, s);
    if (hipFreeAsync(ws, s) != hipSuccess) return Q4BQ_EHIP;
    return status_of(err);
}

}  // namespace

extern "C" {

int mul_mat_q8_0_q8_0(const void* Wq8, int64_t rows, int64_t K, const float* X, int64_t N, float* Y, void* stream) {
    if (!Wq8 || !X || !Y || bad_dim(rows) || bad_dim(N) || bad_k(K)) return Q4BQ_EINVAL;
    const int64_t nb = K / kQK;
    if (!q8w_supported_k(nb) || too_big(rows, K, 2) || too_big(N, K, 4) || too_big(N, rows, 4)) return Q4BQ_EINVAL;
    // a few more tokens than one decode launch takes: groups of up to 8 on the
    // row kernel rather than the matrix-core kernel, whose workgroups cover 128
    // tokens -- up to 16 tokens where that kernel splits K, up to 32 elsewhere
    // (measured, graph-timed, groups against the matrix cores: 14336 x 4096 at
    // N = 16 / 24 43.9 / 65.1 against 51.5 / 52.3 us, 3072 x 768 at N = 32 24.6
    // against 34.7 us); on the 128256 x 4096 head only at 9 tokens (8 tokens
    // take 127-149 us there)
    const bool may_group = N > kGemvMaxN && N <= kQ8wGroupsMaxN && q8w_tokens_per_launch(nb) == kGemvMaxN &&
                           (rows < kQ8wGroupsLongRows || N <= kGemvMaxN + 1);
    if (N > kGemvMaxN && !may_group && !q8w_mm_grid_ok(rows, N)) return Q4BQ_EINVAL;
    if (!aligned(Wq8, 2) || !aligned(X, 4) || !aligned(Y, 4)) return Q4BQ_EINVAL;
    const size_t y_bytes = static_cast<size_t>(N * rows) * 4;
    if (overlap(Y, y_bytes, Wq8, static_cast<size_t>(rows * nb) * kQ8Bytes) ||
        overlap(Y, y_bytes, X, static_cast<size_t>(N * K) * 4))
        return Q4BQ_EINVAL;
    hipError_t err = hipSuccess;
    const DeviceInfo* dev = current_device(&err);
    if (!dev) return Q4BQ_EHIP;
    int kbs = 0;
    const bool groups =
        may_group && (N <= kQ8wGroupsSplitMaxN || q8w_mm_splits(rows, nb, N, dev->num_cu, &kbs) == 1);
    if (N > kGemvMaxN && !groups)
        return run_q8w_mm(static_cast<const uint8_t*>(Wq8), rows, nb, X, nullptr, N, Y, nullptr,
                          static_cast<hipStream_t>(stream));
    return status_of(launch_q8w_product(dev, static_cast<const uint8_t*>(Wq8), rows, nb, X, N, Y,
                                        static_cast<hipStream_t>(stream)));
}

int q8_0_q8_0_block_dots(const void* Wq8, int64_t rows, int64_t K, const void* Xq, int64_t N, int32_t* D,
                         void* stream) {
    if (!Wq8 || !Xq || !D || bad_dim(rows) || bad_dim(N) || bad_k(K)) return Q4BQ_EINVAL;
    const int64_t nb = K / kQK;
    if (too_big(rows, K, 2) || too_big(N, K, 2) || too_big(N * rows, nb, 4)) return Q4BQ_EINVAL;
    if (!aligned(Wq8, 2) || !aligned(Xq, 2) || !aligned(D, 4)) return Q4BQ_EINVAL;
    const size_t d_bytes = static_cast<size_t>(N * rows * nb) * 4;
    if (overlap(D, d_bytes, Wq8, static_cast<size_t>(rows * nb) * kQ8Bytes) ||
        overlap(D, d_bytes, Xq, static_cast<size_t>(N * nb) * kQ8Bytes))
        return Q4BQ_EINVAL;
    if (N > kGemvMaxN && !q8w_mm_grid_ok(rows, N)) return Q4BQ_EINVAL;
    hipError_t err = hipSuccess;
    if (!current_device(&err)) return Q4BQ_EHIP;
    if (N > kGemvMaxN)
        return run_q8w_mm(static_cast<const uint8_t*>(Wq8), rows, nb, nullptr, static_cast<const uint8_t*>(Xq), N,
                          nullptr, D, static_cast<hipStream_t>(stream));
    return status_of(launch_q8w_block_dots(static_cast<const uint8_t*>(Wq8), rows, nb,
                                           static_cast<const uint8_t*>(Xq), N, D, static_cast<hipStream_t>(stream)));
}

int q4bq_quantize_activations(const float* X, int64_t N, int64_t K, void* workspace, size_t ws_bytes,
                              void* stream) {
    if (!X || !workspace || bad_dim(N) || bad_k(K) || too_big(N, K, 4)) return Q4BQ_EINVAL;
    if (!aligned(X, 4) || !aligned(workspace, 16)) return Q4BQ_EINVAL;
    const size_t need = act_ws_bytes(N, K / kQK);  // the activations alone (no rows: no split sums here)
    if (ws_bytes < need) return Q4BQ_ENOMEM;
    if (overlap(workspace, need, X, static_cast<size_t>(N * K) * 4)) return Q4BQ_EINVAL;
    hipError_t err = hipSuccess;
    if (!current_device(&err)) return Q4BQ_EHIP;
    return status_of(launch_act_from_f32(X, N, K / kQK, workspace, static_cast<hipStream_t>(stream)));
}

int mul_mat_q4_0_q8_0_prepared(const void* Wq, int64_t rows, int64_t K, const void* workspace, int64_t N, float* Y,
                               void* stream) {
    const int rc = check_product(Wq, rows, K, workspace, kPrepared, N, Y, false);
    if (rc != Q4BQ_OK) return rc;
    hipError_t err = hipSuccess;
    const DeviceInfo* dev = current_device(&err);
    if (!dev) return Q4BQ_EHIP;
    const int64_t nb = K / kQK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* w = static_cast<const uint8_t*>(Wq);
    err = N <= kGemvMaxN ? launch_gemv(dev, kAoS, w, rows, nb, workspace, N, Y, nullptr, s)
                         : launch_prefill(dev, kAoS, w, rows, nb, workspace, N, Y, nullptr, s);
    return status_of(err);
}

const char* q4bq_status_string(int status) {
    switch (status) {
        case Q4BQ_OK: return "ok";
        case Q4BQ_EINVAL: return "invalid argument (null pointer, size < 1, K not a positive multiple of 32, "
                                 "misaligned pointer or overlapping buffers)";
        case Q4BQ_EHIP: return "HIP runtime or kernel launch failure";
        case Q4BQ_ENOMEM: return "scratch allocation failed or workspace too small";
        case Q4BQ_ESCRATCH: return "sizes need more scratch than the no-allocation entry point holds "
                                   "(Q4BQ_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int q4bq_version(void) { return 400; }

}  // extern "C"
