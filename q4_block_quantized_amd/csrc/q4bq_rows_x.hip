// Row-streaming decode, activations quantized from fp32 X inside the kernel.
#include "q4bq_rows.h"

namespace q4bq {

bool rows_apply(int64_t N, int64_t nb) {
    return rows_ppl(nb) > 0 && N >= 1 && N <= 8 &&
           static_cast<size_t>(N) * nb * (kActQBytes + kActSBytes) <= kRowsMaxLds;
}

hipError_t launch_rows_x(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const float* src,
                         int64_t N, float* Y, const MultiDesc& md, hipStream_t s) {
    switch (lay) {
        case kLayRepacked: return launch_rows_t<kXF32, kLayRepacked>(dev, Wq, rows, nb, src, N, Y, md, s);
        case kLayMulti: return launch_rows_t<kXF32, kLayMulti>(dev, Wq, rows, nb, src, N, Y, md, s);
        default: return launch_rows_t<kXF32, kLayAoS>(dev, Wq, rows, nb, src, N, Y, md, s);
    }
}

}  // namespace q4bq
