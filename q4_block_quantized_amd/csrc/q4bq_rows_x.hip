// Row-streaming decode, activations quantized from fp32 X inside the kernel.
#include "q4bq_rows.h"

namespace q4bq {

bool rows_apply(int64_t N, int64_t nb, int64_t rows) {
    return rows_ppl(nb, rows) > 0 && N >= 1 && N <= 8 &&
           static_cast<size_t>(N) * nb * (kActQBytes + kActSBytes) <= kRowsMaxLds;
}

bool rows_fuse_prologue(int64_t nb, int64_t rows) { return rows_ppl(nb, rows) == 1; }

bool rows_dual_apply(const DeviceInfo* dev, int64_t rows, int64_t nb) {
    if (!rows_fuse_prologue(nb, rows)) return false;
    constexpr int kWaves = rows_threads<1, 1>() / 64;
    int64_t wgs = (2 * rows + kWaves - 1) / kWaves;
    if (wgs > dev->num_cu) wgs = dev->num_cu;
    return (2 * rows + wgs * kWaves - 1) / (wgs * kWaves) <= kSplitRounds;
}

hipError_t launch_rows_dual(const DeviceInfo* dev, const uint8_t* Wgate, const uint8_t* Wup, int64_t rows, int64_t nb,
                            const float* X, float* H, const Epilogue& ln, hipStream_t s) {
    if (!rows_dual_apply(dev, rows, nb)) return hipErrorInvalidValue;
    MultiDesc md{};
    md.w[0] = Wgate;
    md.w[1] = Wup;
    md.epi = ln;
    return launch_rows_k<kXF32, kLayAoS, true, false, 1, 1, 2, true>(dev, Wgate, rows, nb, X, H, nullptr, md, s);
}

hipError_t launch_rows_x(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const float* src,
                         int64_t N, float* Y, const MultiDesc& md, hipStream_t s) {
    const Epilogue& e = md.epi;
    if (e.bias || e.mul || e.act != kEpiNone || e.ln_gamma) {
        // the fused forms: one token, the pages' blocks, one pair per lane
        if (lay != kLayAoS || N != 1 || !rows_fuse_prologue(nb, rows)) return hipErrorInvalidValue;
        return launch_rows_nt<kXF32, kLayAoS, true, false, 1>(dev, Wq, rows, nb, src, Y, nullptr, md, s);
    }
    switch (lay) {
        case kLayRepacked: return launch_rows_t<kXF32, kLayRepacked>(dev, Wq, rows, nb, src, N, Y, md, s);
        case kLayMulti: return launch_rows_t<kXF32, kLayMulti>(dev, Wq, rows, nb, src, N, Y, md, s);
        default: return launch_rows_t<kXF32, kLayAoS>(dev, Wq, rows, nb, src, N, Y, md, s);
    }
}

}  // namespace q4bq
