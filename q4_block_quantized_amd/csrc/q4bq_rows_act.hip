// Row-streaming decode on the activation quantizer's buffer.
#include "q4bq_rows.h"

namespace q4bq {

hipError_t launch_rows_act(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                           const void* src, int64_t N, float* Y, const MultiDesc& md, hipStream_t s, int32_t* D) {
    if (D) {
        if (lay != kLayAoS) return hipErrorInvalidValue;  // block dots are exported for Q4_0 blocks only
        return launch_rows_t<kActGlobal, kLayAoS, false, true>(dev, Wq, rows, nb, src, N, Y, md, s, D);
    }
    switch (lay) {
        case kLayRepacked: return launch_rows_t<kActGlobal, kLayRepacked>(dev, Wq, rows, nb, src, N, Y, md, s);
        case kLayMulti: return launch_rows_t<kActGlobal, kLayMulti>(dev, Wq, rows, nb, src, N, Y, md, s);
        default:
            if (md.epi.bias || md.epi.mul || md.epi.act != kEpiNone)
                return launch_rows_t<kActGlobal, kLayAoS, true>(dev, Wq, rows, nb, src, N, Y, md, s);
            return launch_rows_t<kActGlobal, kLayAoS>(dev, Wq, rows, nb, src, N, Y, md, s);
    }
}

}  // namespace q4bq
