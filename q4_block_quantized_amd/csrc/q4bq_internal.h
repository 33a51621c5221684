// Host-side launchers shared between the C-ABI layer and the kernel files.
// Arguments are validated by the caller (q4bq_api.cpp); launchers only
// enqueue work on `stream` and return hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4bq {

constexpr int kQK = 32;         // values per block
constexpr int kQ4Bytes = 18;    // Q4_0 block: binary16 d + 16 nibble bytes
constexpr int kQ8Bytes = 34;    // Q8_0 block: binary16 d + 32 int8
constexpr int kActQBytes = 32;  // internal activation block (int8, dot order)
constexpr int kActSBytes = 8;   // internal scale record {float d; int32 bias}

// Weight layouts: the pages' 18-byte blocks, or the repacked streams of
// q4_0_repack (16 nibble bytes per block, then one binary16 scale per block).
enum WLayout { kAoS = 0, kRepacked = 1 };

// Several matrices with the same K that read the same activations, handled as
// one concatenation of their rows (decode kernel): matrix m owns global rows
// [first[m], first[m + 1]), its blocks at w[m], its output (N x rows_m) at y[m].
constexpr int kMaxMulti = 8;

// What a product kernel applies to each output before it stores it: the bias
// add and activation after GPT-2's c_mlp_fc, or the element-wise factor of
// SiLU(gate) * up: y = act(y + bias[r]) * mul[n][r], every part optional
// (null pointers, kEpiNone).  Single-matrix launches only.  ln_gamma set: the
// decode kernels that quantize one fp32 token themselves first LayerNorm it
// with ln_gamma, ln_beta, ln_eps (the host routes only those launches here).
enum EpiAct { kEpiNone = 0, kEpiGelu = 1, kEpiSilu = 2 };
struct Epilogue {
    const float* bias;
    const float* mul;
    int act;
    const float* ln_gamma = nullptr;
    const float* ln_beta = nullptr;
    float ln_eps = 0.0f;
};

struct MultiDesc {
    const uint8_t* w[kMaxMulti];
    float* y[kMaxMulti];
    int64_t first[kMaxMulti + 1];
    int count;
    Epilogue epi;  // decode kernels on one matrix
};

struct DeviceInfo {
    int id;
    int num_cu;
    int num_xcd;
};

// Launch parameters of the device current on this thread (cached).
const DeviceInfo* current_device(hipError_t* err);

// Device address of the no-allocation entry point's fixed scratch
// (Q4BQ_NOALLOC_SCRATCH_BYTES) on `device`, which must be the current device;
// looked up once per device.  nullptr and *err set on failure.
void* noalloc_scratch(int device, hipError_t* err);

// Internal activation buffer ([n][b], b fastest):
//  N <= kGemvMaxN (decode kernel): N*nb blocks of 32 int8 bytes in dot order,
//    then N*nb scale records of 8 bytes {float d; int32 -8*sum(q)};
//  larger N (prefill kernel): N*nb records of 64 bytes, block-major
//    ([b][n]): fp6 operands of the high and low parts of q, each followed by
//    the block's binary16 scale bits and a zero dword.
size_t act_bytes(int64_t N, int64_t nb);

hipError_t launch_q4_0_quantize(const float* W, int64_t nblocks, uint8_t* Wq, hipStream_t s);
hipError_t launch_q8_0_quantize(const float* X, int64_t nblocks, uint8_t* Xq, hipStream_t s);
// Repacked weights: nibble stream, scale stream, then (from
// repack_records_offset) the prefill kernel's weight records, block-major,
// with one trailing plane of zero records; repack_bytes in all.
int64_t repack_records_offset(int64_t rows, int64_t nb);
size_t repack_bytes(int64_t rows, int64_t nb);
hipError_t launch_q4_0_repack(const uint8_t* Wq, int64_t rows, int64_t nb, uint8_t* Wr, hipStream_t s);
// Q8_0 weights (34-byte blocks) x Q8_0 activations: row-streaming decode in
// groups of up to q8w_tokens_per_launch tokens (whose quantized blocks fit the
// kernel's LDS); block dots with the same dot function.
int64_t q8w_tokens_per_launch(int64_t nb);
bool q8w_supported_k(int64_t nb);
hipError_t launch_q8w_product(const DeviceInfo* dev, const uint8_t* W, int64_t rows, int64_t nb, const float* X,
                              int64_t N, float* Y, hipStream_t s);
hipError_t launch_q8w_block_dots(const uint8_t* W, int64_t rows, int64_t nb, const uint8_t* Xq, int64_t N, int32_t* D,
                                 hipStream_t s);
// Q8_0 weights x Q8_0 activations on the matrix cores (N > kGemvMaxN): the
// activations (fp32 X, or Q8_0 blocks Xq) are first laid out in `ws`
// (q8w_mm_act_bytes), then one launch of ceil(rows / kQ8wMmRows) *
// ceil(N / kQ8wMmTokens) workgroups of kQ8wMmThreads, times the K ranges
// (q8w_mm_splits: up to kQ8wMmMaxSplits, so that there are about two
// workgroups per CU) whose sums a second kernel adds in range order from
// the rest of `ws` (q8w_mm_scratch_bytes in all).  D != nullptr: the
// block-dot export instead of Y (no split).
constexpr int kQ8wMmThreads = 256;
constexpr int kQ8wMmRows = 128;
constexpr int kQ8wMmTokens = 128;
constexpr int64_t kQ8wMmMaxSplits = 4;
size_t q8w_mm_act_bytes(int64_t N, int64_t nb);
int q8w_mm_splits(int64_t rows, int64_t nb, int64_t N, int num_cu, int* kbs);
size_t q8w_mm_scratch_bytes(int64_t rows, int64_t nb, int64_t N, int num_cu);
hipError_t launch_q8w_mm(const DeviceInfo* dev, const uint8_t* W, int64_t rows, int64_t nb, const float* X,
                         const uint8_t* Xq, int64_t N, float* Y, int32_t* D, void* ws, hipStream_t s);
hipError_t launch_q4_0_get_rows(const uint8_t* Wq, int64_t rows, int64_t nb, const int32_t* ids, int64_t n,
                                float* out, hipStream_t s);

// fp32 X (N x K) -> internal activations, or Q8_0 blocks -> internal.
hipError_t launch_act_from_f32(const float* X, int64_t N, int64_t nb, void* act, hipStream_t s);
// LayerNorm + the same quantization, one workgroup per token (N < 2^31): fp64
// mean and population variance, then gamma * (x - mu) / sqrt(var + eps) +
// beta evaluated in fp64, rounded to fp32 and quantized.
hipError_t launch_ln_act(const float* X, int64_t N, int64_t nb, const float* gamma, const float* beta, float eps,
                         void* act, hipStream_t s);
hipError_t launch_act_from_q8(const uint8_t* Xq, int64_t N, int64_t nb, void* act, hipStream_t s);

// Streaming decode kernel, N in 1..8.  D != nullptr selects the block-dot
// export (D written, Y untouched).
hipError_t launch_gemv(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                       const void* act, int64_t N, float* Y, int32_t* D, hipStream_t s,
                       const Epilogue& epi = Epilogue{nullptr, nullptr, kEpiNone});

// Decode kernel that quantizes fp32 X itself (no scratch, one launch), for
// N <= kGemvFusedMaxN when the quantized activations fit in LDS.  Same bits
// as launch_act_from_f32 followed by launch_gemv.
constexpr int64_t kGemvFusedMaxN = 1;
// md: the multi-matrix form's table, else nullptr.
bool gemv_fuses(int64_t N, int64_t nb, int64_t rows, const MultiDesc* md = nullptr);
// Whether the fused kernel is also the faster choice when the caller has a
// workspace for a separate quantizer launch.
bool gemv_prefers_fused(int64_t N, int64_t nb, int64_t rows, const MultiDesc* md = nullptr);
hipError_t launch_gemv_fused(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                             const float* X, int64_t N, float* Y, hipStream_t s);
// One token, the pages' blocks, with an epilogue and optionally LayerNorm:
// the decode kernel normalizes (epi.ln_gamma set) and quantizes the fp32 token
// in its prologue and applies the epilogue at its stores, in one launch, for
// shapes where gemv_fuses_epi(nb, rows).
bool gemv_fuses_epi(int64_t nb, int64_t rows);
hipError_t launch_gemv_fused_epi(const DeviceInfo* dev, const uint8_t* Wq, int64_t rows, int64_t nb, const float* X,
                                 float* Y, const Epilogue& epi, hipStream_t s);

// The decode kernel over the rows of several matrices (N <= kGemvMaxN; AoS
// blocks).  X fp32 is quantized in the kernel when gemv_fuses(N, nb), else
// `act` holds the quantizer's output.
hipError_t launch_gemv_multi(const DeviceInfo* dev, const MultiDesc& md, int64_t nb, const float* X, const void* act,
                             int64_t N, hipStream_t s);

// Several independent one-token products in one launch (`k_gemv_set`):
// product m multiplies its Q4_0 blocks w[m] (rows[m] x nb[m]) with its own
// fp32 token x[m] (nb[m] * 32 values) into y[m] (rows[m]).  set_plan fills
// C, Pc, boff, round0 and nblk from count, w, x, y, rows, nb and returns
// false where the launch does not apply (an odd block count, a row of more
// than 16 chunks of 64 pairs, more than kSetMaxBlocks activation blocks in
// all, or more than kSetMaxRounds rounds for a workgroup).
constexpr int kSetMaxBlocks = 1024;  // activation blocks of all products (LDS)
constexpr int kSetMaxRounds = 64;    // rounds of 16 chunk rows per workgroup
struct SetDesc {
    const uint8_t* w[kMaxMulti];
    const float* x[kMaxMulti];
    float* y[kMaxMulti];
    int64_t rows[kMaxMulti];
    int nb[kMaxMulti];
    int C[kMaxMulti];      // chunks per row (a power of two, at most 16)
    int Pc[kMaxMulti];     // block pairs per chunk (at most 64)
    int boff[kMaxMulti];   // first activation block of the product in LDS
    int64_t round0[kMaxMulti + 1];  // first round of each product; round0[count]: all rounds
    int count;
    int nblk;              // activation blocks of all products
};
bool set_plan(SetDesc& sd, int64_t num_cu);
hipError_t launch_gemv_set(const DeviceInfo* dev, const SetDesc& sd, hipStream_t s);

// Decode kernels: activation sources and weight layouts (the rows of several
// matrices, MultiDesc, count as one more layout).
enum DecodeSrc { kActGlobal = 0, kActLds = 1, kXF32 = 2 };
enum DecodeLayout { kLayAoS = 0, kLayRepacked = 1, kLayMulti = 2 };

// Row-streaming decode (whole waves per row), for N tokens when
// rows_apply(N, nb): from fp32 X quantized in the kernel, or from the
// quantizer's buffer.  `lay` is a DecodeLayout; Wq/Y unused for kLayMulti.
bool rows_apply(int64_t N, int64_t nb, int64_t rows);
// Whether the row kernel's fused form (epilogue, LayerNorm of the one token in
// its prologue) covers this block count: one pair per lane.
bool rows_fuse_prologue(int64_t nb, int64_t rows);
// SiLU(LN(x) Wgate^T) * (LN(x) Wup^T) for one token in one launch (the row
// kernel's gate-and-up form), where rows_dual_apply; ln: LayerNorm operands
// (ln.ln_gamma null: none), its other fields unused.
bool rows_dual_apply(const DeviceInfo* dev, int64_t rows, int64_t nb);
hipError_t launch_rows_dual(const DeviceInfo* dev, const uint8_t* Wgate, const uint8_t* Wup, int64_t rows, int64_t nb,
                            const float* X, float* H, const Epilogue& ln, hipStream_t s);
hipError_t launch_rows_x(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb, const float* X,
                         int64_t N, float* Y, const MultiDesc& md, hipStream_t s);
// D != nullptr: the block-dot export (Q4_0 blocks, one matrix) instead of Y.
hipError_t launch_rows_act(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                           const void* act, int64_t N, float* Y, const MultiDesc& md, hipStream_t s,
                           int32_t* D = nullptr);

// Decode on the matrix cores (`k_gemv_mma_tr` with contiguous weight loads
// where a row is whole chunks of 8 blocks, at least 64 blocks, and its LDS
// fits; `k_gemv_mma` with 36-byte lane loads otherwise): one
// v_mfma_i32_32x32x32_i8 per 32-row tile and block, for the shapes where
// mma_apply (up to kGemvMaxN tokens, at least kMmaMinRows rows, even block
// counts up to kMmaMaxBlocks; from kMmaMinN tokens, or on matrices of
// kMmaLongRows rows and more from kMmaLongMinN tokens with contiguous loads
// -- kMmaMinN where the row kernel loads rows whole --, kMmaLongMinNPairs
// with lane loads).  src is fp32 X (src_f32) or the
// quantizer's buffer; `lay` a DecodeLayout; md.epi applies at the store
// (single matrix).
constexpr int kMmaThreads = 1024;
constexpr int64_t kMmaMinN = 5;
constexpr int64_t kMmaMinRows = 2048;
constexpr int64_t kMmaMaxBlocks = 256;
constexpr int64_t kMmaLongRows = 32768;
constexpr int64_t kMmaLongMinN = 4;
constexpr int64_t kMmaLongMinNPairs = 7;
constexpr int64_t kMmaRowsContiguousRows = 65536;  // below: kMmaLongMinN even where the row kernel loads rows whole
// md: the multi-matrix form's table (its matrices must start on 32-row
// boundaries), else nullptr.
bool mma_apply(int64_t N, int64_t nb, int64_t rows, const MultiDesc* md = nullptr);
hipError_t launch_gemv_mma(const DeviceInfo* dev, int lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                           const void* src, bool src_f32, int64_t N, float* Y, const MultiDesc& md, hipStream_t s);

// Matrix-core kernel geometry: a workgroup of kPrefillThreads threads computes
// kPrefillTokens tokens x kPrefillRows rows, so a launch has
// ceil(rows / kPrefillRows) * ceil(N / kPrefillTokens) workgroups.
constexpr int kPrefillThreads = 512;
constexpr int kPrefillTokens = 128;
constexpr int kPrefillRows = 224;
// LayerNorm + quantization kernel: one workgroup of kLnActThreads per token.
constexpr int kLnActThreads = 1024;
// HIP launches fewer than 2^32 work-items per grid dimension.
constexpr int64_t kMaxWorkItems = (int64_t(1) << 32) - 1;

// Matrix-core kernel, any N; the one the library runs above kGemvMaxN.  D as
// above.  With fewer than kPrefillSplitTiles workgroup tiles, K is split in up
// to kPrefillMaxSplits ranges of at least kPrefillMinSplitBlocks blocks (one
// workgroup per tile and range, as many as the CUs take; the shape alone
// decides); the ranges' sums go to a buffer of splits * N * rows floats --
// `partial` where partial_bytes holds them, else one taken stream-ordered --
// and a second kernel adds them in range order and applies the epilogue.
constexpr int64_t kPrefillSplitTiles = 256;
constexpr int64_t kPrefillMaxSplits = 4;
constexpr int64_t kPrefillMinSplitBlocks = 16;
int prefill_splits(int64_t rows, int64_t nb, int64_t N, int num_cu, int* kbs);
// Room for the largest split of these sizes on any device (0 where none can
// happen), and the bytes this device's split takes.
size_t prefill_partial_bytes(int64_t rows, int64_t nb, int64_t N);
size_t prefill_split_bytes(const DeviceInfo* dev, int64_t rows, int64_t nb, int64_t N);
hipError_t launch_prefill(const DeviceInfo* dev, WLayout lay, const uint8_t* Wq, int64_t rows, int64_t nb,
                          const void* act, int64_t N, float* Y, int32_t* D, hipStream_t s,
                          const Epilogue& epi = Epilogue{nullptr, nullptr, kEpiNone}, float* partial = nullptr,
                          size_t partial_bytes = 0);

constexpr int64_t kGemvMaxN = 8;

}  // namespace q4bq
