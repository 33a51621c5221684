/*
 * q4bq -- Q4_0-weight x Q8_0-activation quantized matrix product on MI355X.
 *
 * C ABI of libq4bq.so.  Every pointer argument is a DEVICE pointer (memory the
 * caller allocated on the current HIP device), every size is an element count,
 * and `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 * calls are asynchronous on `stream`: they validate their arguments on the host,
 * enqueue kernels and return; buffers must stay alive until the stream has
 * passed them.  The library keeps no pointer after a call returns and holds no
 * state other than per-device launch parameters, so calls are reentrant.
 *
 * Formats (as defined in "llama.cpp 深度解读", luoboask.github.io):
 *   Q4_0 block, section 2 "量化数据结构 — Q4_0 格式详解": 18 bytes for 32
 *     consecutive weights -- bytes 0-1 the scale d (IEEE binary16,
 *     little-endian), bytes 2-17 the nibbles; byte 2+j holds element 2j in its
 *     low 4 bits and element 2j+1 in its high 4 bits; element value
 *     (nibble - 8) * d.
 *   Q8_0 block, the activation operand of ggml_vec_dot_q4_0_q8_0 in section 3
 *     "量化矩阵乘法 — 核心算子": 34 bytes -- bytes 0-1 the scale d (binary16),
 *     bytes 2-33 the 32 int8 values in element order; element value q * d.
 *
 * Matrix layouts (row-major, innermost dimension contiguous, as in ggml where
 * mul_mat contracts the innermost dimension -- "解锁模型适配能力：Llama.cpp 框架下
 * 新架构开发全流程指南", tahou.com, "GGML 的特性与注意事项" item 2):
 *   W  fp32 rows x K            Wq  rows x (K/32) Q4_0 blocks; block (r, b) at
 *                                   byte offset (r * K/32 + b) * 18
 *   X  fp32 N x K               Xq  N x (K/32) Q8_0 blocks; block (n, b) at
 *                                   byte offset (n * K/32 + b) * 34
 *   Y  fp32 N x rows            Y[n * rows + r] = sum over k of
 *                                   W~[r][k] * X~[n][k] (~ = quantized values)
 *
 * Errors: every entry point returns Q4BQ_OK (0) or a negative status and never
 * aborts.  Arguments are checked before anything is enqueued; on Q4BQ_EINVAL
 * nothing was launched and no output was touched.  Q4BQ_EHIP reports a HIP
 * runtime or launch failure (outputs then undefined).  Inputs are assumed
 * finite, with |W| / 8 and |X| / 127 below 65504 (the binary16 range); outside
 * that the results are unspecified but the call still returns normally.
 */
#ifndef Q4BQ_H
#define Q4BQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4BQ_OK 0
#define Q4BQ_EINVAL (-1) /* bad argument: null, size < 1, K % 32 != 0, misaligned, overlap */
#define Q4BQ_EHIP (-2)   /* HIP runtime / launch failure */
#define Q4BQ_ENOMEM (-3) /* scratch allocation failed, or workspace too small */
#define Q4BQ_ESCRATCH (-4) /* sizes beyond the no-allocation entry point's fixed scratch */

#define Q4BQ_QK 32
#define Q4BQ_Q4_0_BYTES 18
#define Q4BQ_Q8_0_BYTES 34

/*
 * Q4_0 encode, "llama.cpp 深度解读" section 2 (the block encode): per block of
 * 32 weights, amax = max |w|; the scale amax / 8 is stored as binary16
 * (round to nearest even, subnormals kept); q = round(w / d) + 8 with d the
 * stored scale widened to fp32, round() half away from zero, clamped to
 * [0, 15]; an all-zero block stores d = 0 and nibbles 8.
 *   W   fp32 rows x K, 4-byte aligned.        Wq  rows*(K/32)*18 bytes, 2-byte aligned.
 * Requires rows >= 1, K >= 32, K % 32 == 0.  Bit-exact; deterministic.
 */
int q4_0_quantize(const float *W, int64_t rows, int64_t K, void *Wq, void *stream);

/*
 * Q8_0 encode of activations (the rule the pages leave implicit, read as the
 * Q4_0 rule with 127 levels): per block, d = binary16(amax / 127),
 * q = round(x / d) clamped to [-127, 127], q = 0 when d == 0.
 *   X   fp32 N x K, 4-byte aligned.           Xq  N*(K/32)*34 bytes, 2-byte aligned.
 * Requires N >= 1, K >= 32, K % 32 == 0.  Bit-exact; deterministic.
 */
int q8_0_quantize(const float *X, int64_t N, int64_t K, void *Xq, void *stream);

/*
 * The operator: Y = mul_mat(Wq, X), "llama.cpp 深度解读" section 3 (Q4_0
 * weights times Q8_0 activations, one fp32 scale d_w * d_x per 32-block, the
 * block's integer dot of (nibble - 8) with the int8 activations accumulated in
 * int32, the scaled block terms summed in fp32).  X is fp32; it is quantized
 * to Q8_0 by exactly the rule of q8_0_quantize inside the call.
 *   Wq  rows x (K/32) Q4_0 blocks, 2-byte aligned.
 *   X   fp32 N x K, 4-byte aligned.
 *   Y   fp32 N x rows, 4-byte aligned, overwritten; must not overlap Wq or X.
 * N <= 8 runs the streaming decode kernel (9..32 tokens run as groups of up
 * to 8 through it where it takes the shape); larger N the matrix-core kernel,
 * in ceil(rows / 224) * ceil(N / 128) workgroups of 512 threads: shapes whose
 * grid would exceed HIP's 2^32 - 1 work-items return Q4BQ_EINVAL.  When that
 * is fewer than 256 workgroups, K is split into up to 4 ranges (as many
 * workgroups more) whose fp32 sums a second kernel adds in range order.
 * Needs stream-ordered scratch of q4bq_workspace_size(rows, K, N) bytes (the
 * activations and room for those sums), taken with hipMallocAsync on
 * `stream` (Q4BQ_ENOMEM if that fails).
 * The summation order is fixed for a given (rows, K, N, device), so repeated
 * calls give bitwise-identical Y.
 */
int mul_mat_q4_0_q8_0(const void *Wq, int64_t rows, int64_t K, const float *X,
                      int64_t N, float *Y, void *stream);

/* Scratch bytes the operator needs for these sizes (0 on invalid sizes). */
size_t q4bq_workspace_size(int64_t rows, int64_t K, int64_t N);

/*
 * mul_mat_q4_0_q8_0 with caller-owned scratch: `workspace` is a device buffer
 * of ws_bytes >= q4bq_workspace_size(rows, K, N), 16-byte aligned, not
 * overlapping the other arguments (Q4BQ_ENOMEM if too small).  No allocation
 * happens inside.  Same results as mul_mat_q4_0_q8_0, bit for bit.
 */
int mul_mat_q4_0_q8_0_ex(const void *Wq, int64_t rows, int64_t K, const float *X,
                         int64_t N, float *Y, void *workspace, size_t ws_bytes,
                         void *stream);

/*
 * Two-phase form of mul_mat_q4_0_q8_0_ex, for several products that share one
 * activation matrix (for example the projections that read the same token
 * vector).  q4bq_quantize_activations runs the Q8_0 rule of q8_0_quantize on
 * X (fp32 N x K, 4-byte aligned) and leaves the result in `workspace` (16-byte
 * aligned, ws_bytes >= q4bq_workspace_size(1, K, N); its contents are private
 * to the library).  mul_mat_q4_0_q8_0_prepared then computes Y from Wq and
 * that workspace; it may be called any number of times, for different Wq with
 * the same K, while the workspace is left untouched.  Running the two in
 * sequence gives exactly the Y of mul_mat_q4_0_q8_0 (where that splits K,
 * mul_mat_q4_0_q8_0_prepared takes the buffer for the range sums
 * stream-ordered on `stream`).
 */
int q4bq_quantize_activations(const float *X, int64_t N, int64_t K, void *workspace,
                              size_t ws_bytes, void *stream);
int mul_mat_q4_0_q8_0_prepared(const void *Wq, int64_t rows, int64_t K,
                               const void *workspace, int64_t N, float *Y, void *stream);

/*
 * Optional one-time weight repack for the product below.  The Q4_0 blocks of
 * "llama.cpp 深度解读" section 2 ("量化数据结构 — Q4_0 格式详解") are laid out
 * again as three streams (nblk = rows * K/32, nb = K/32):
 *   bytes [0, 16*nblk)            nibble stream: the 16 nibble bytes of block
 *                                 (r, b) at (r * nb + b) * 16, unchanged;
 *   bytes [16*nblk, 18*nblk)      scale stream: the binary16 scale of block
 *                                 (r, b) at 16*nblk + (r * nb + b) * 2;
 *   bytes [R, R + (nb+1)*rows*32) record stream, R = 18*nblk rounded up to a
 *                                 multiple of 256: a 32-byte record for block
 *                                 (r, b) at R + (b * rows + r) * 32 (block
 *                                 major), then one plane (b = nb) of zero
 *                                 records.  A record is 24 bytes of 6-bit
 *                                 codes, code c at bits 6c..6c+5 (little
 *                                 endian), then the 2 scale bytes, then 6 zero
 *                                 bytes; code c = 4*m + i stands for element
 *                                 8*(m/2) + 2*i + (m%2) of the block and is
 *                                 the FP6 E2M3 encoding of (nibble - 8)/8
 *                                 (exact: |nibble - 8| <= 8).  In rows r
 *                                 where bit 2 xor bit 3 of r is set the
 *                                 record's two 16-byte halves are stored
 *                                 swapped.
 * The bytes in [18*nblk, R) are zero.  q4bq_repack_size(rows, K) gives the
 * total (0 for invalid sizes).  Every
 * 16-byte nibble block is aligned, so the decode kernels read it with single
 * 16-byte loads; the records are the matrix-core operands of the many-token
 * kernel, converted once instead of at every use.  No value changes.
 *   Wq  rows x (K/32) Q4_0 blocks, 2-byte aligned.
 *   Wr  q4bq_repack_size(rows, K) bytes, 16-byte aligned, must not overlap Wq.
 * Requires rows >= 1, K >= 32, K % 32 == 0.
 */
size_t q4bq_repack_size(int64_t rows, int64_t K);
int q4_0_repack(const void *Wq, int64_t rows, int64_t K, void *Wr, void *stream);

/*
 * Rows of a Q4_0 table, decoded: ggml_get_rows on Q4_0, the token-embedding
 * lookup that starts the Llama graph in "llama.cpp 深度解读" section 4
 * ("计算图构建 — 以 Llama 模型为例", inpL = ggml_get_rows(tok_embeddings,
 * inp_tokens)) and GPT-2's wte/wpe lookups in the ggml GPT-2 walkthrough
 * (section 3.5); the decode is section 2's: element j of a block is
 * (nibble_j - 8) * d, exact in fp32.
 *   Wq    device, rows x K/32 Q4_0 blocks (the pages' layout), 2-byte aligned.
 *   ids   device, n int32 row indices, 4-byte aligned.
 *   out   device, fp32 n x K (row i = row ids[i]), 16-byte aligned,
 *         overwritten; may not overlap Wq or ids.
 * An id outside [0, rows) gives a row of NaN (no out-of-range read; the
 * pages do not define this case).  Errors as for q4_0_quantize; n >= 1.
 */
int q4_0_get_rows(const void *Wq, int64_t rows, int64_t K, const int32_t *ids,
                  int64_t n, float *out, void *stream);

/*
 * mul_mat_q4_0_q8_0 and mul_mat_q4_0_q8_0_ex on repacked weights (Wr from
 * q4_0_repack, 16-byte aligned); every other argument and the result are as
 * for the forms on Q4_0 blocks, bit for bit.
 */
int mul_mat_q4_0r_q8_0(const void *Wr, int64_t rows, int64_t K, const float *X,
                       int64_t N, float *Y, void *stream);
int mul_mat_q4_0r_q8_0_ex(const void *Wr, int64_t rows, int64_t K, const float *X,
                          int64_t N, float *Y, void *workspace, size_t ws_bytes,
                          void *stream);

/*
 * Several products that read the same activations, in one launch for N <= 8:
 * Y[i] = mul_mat(Wq[i], X) for i < count, all with the same K -- the
 * projections of one token in "llama.cpp 深度解读" section 4 ("计算图构建 —
 * 以 Llama 模型为例": step B's Q, K and V projections of the same normalised
 * input; step I's up and gate projections).  X is quantized once.
 *   count         1 <= count <= 8.
 *   Wq, rows, Y   HOST arrays of count entries: device pointers to each
 *                 matrix's Q4_0 blocks (rows[i] x K/32, 2-byte aligned) and to
 *                 its output (fp32 N x rows[i], 4-byte aligned, overwritten);
 *                 no output may overlap any input or another output.
 *   X             fp32 N x K, 4-byte aligned.
 *   workspace     NULL, or a device buffer of ws_bytes >=
 *                 q4bq_workspace_size(1, K, N), 16-byte aligned; with NULL the
 *                 scratch (not needed for N = 1) is taken with hipMallocAsync.
 *                 Above 8 tokens, where the matrix-core kernel splits K (few
 *                 row tiles), its range sums take stream-ordered scratch too.
 * For N <= 8 the decode kernel runs once over the concatenated rows; larger N
 * runs the matrix-core kernel per matrix on the shared quantized X.  Each
 * Y[i] equals mul_mat_q4_0_q8_0(Wq[i], X) within the operator's tolerance
 * (the same block terms; the fp32 sum of a row may be split across lanes
 * differently when the concatenated shape picks another launch shape).
 */
int mul_mat_q4_0_q8_0_multi(int count, const void *const *Wq, const int64_t *rows,
                            int64_t K, const float *X, int64_t N, float *const *Y,
                            void *workspace, size_t ws_bytes, void *stream);

/*
 * Several independent one-token products in one launch: Y[i] = mul_mat(Wq[i],
 * X[i]) with N = 1 for i < count, each with its own K and its own token --
 * a decode step's products as "llama.cpp 深度解读" section 4 ("计算图构建 — 以
 * Llama 模型为例") lists them (Q, K, V, output, gate, up and down
 * projections), with the operator of section 3 ("量化矩阵乘法 — 核心算子").
 *   count          1 <= count <= 8.
 *   Wq, rows, K,   HOST arrays of count entries: device pointers to each
 *   X, Y           product's Q4_0 blocks (rows[i] x K[i]/32, 2-byte aligned),
 *                  its fp32 token (K[i] values, 4-byte aligned) and its fp32
 *                  output (rows[i] values, 4-byte aligned, overwritten);
 *                  K[i] a positive multiple of 32; no output may overlap any
 *                  input or another output.
 * The workgroups quantize every token once and stream the products' weights
 * in one pass, where every block count is even, a row is at most 16 chunks of
 * 64 block pairs (K <= 65536), the tokens hold at most 1024 blocks in all
 * (32768 values) and the rows at most 64 rounds of 16 chunk rows per
 * workgroup (the one launch allocates nothing); other sets run as count
 * separate products.  Each Y[i] equals mul_mat_q4_0_q8_0(Wq[i], rows[i], K[i],
 * X[i], 1, Y[i]) within the operator's tolerance (the same block terms), and
 * bitwise where that call runs the row kernel with one block pair per lane and
 * the same chunks (the GPT-2- and Llama-3-8B-shaped matrices).  Errors as
 * mul_mat_q4_0_q8_0: nothing is launched for an invalid argument; products
 * enqueued before a failed launch may have run.
 */
int mul_mat_q4_0_q8_0_set(int count, const void *const *Wq, const int64_t *rows,
                          const int64_t *K, const float *const *X, float *const *Y,
                          void *stream);

/*
 * The operator with pre-quantized activations: Xq holds N x (K/32) Q8_0 blocks
 * (2-byte aligned), otherwise as mul_mat_q4_0_q8_0.  Feeding it the output of
 * q8_0_quantize(X) gives exactly the Y of mul_mat_q4_0_q8_0(X).
 */
int mul_mat_q4_0_q8_0_pq(const void *Wq, int64_t rows, int64_t K, const void *Xq,
                         int64_t N, float *Y, void *stream);

/*
 * Test export: every per-block integer dot, "llama.cpp 深度解读" section 3
 * step 4 with the (nibble - 8) offset of section 2's decode:
 *   D[(n * rows + r) * (K/32) + b] = sum_j (nibble_j(r, b) - 8) * q_j(n, b)
 * (int32, exact).  Computed by the same block-dot code as the operator's
 * kernel for this N (the decode kernel for N <= 8, the matrix-core kernel
 * otherwise).  D: N*rows*(K/32) int32, 4-byte aligned, must not overlap the
 * inputs.  Xq as in mul_mat_q4_0_q8_0_pq.
 */
int q4_0_q8_0_block_dots(const void *Wq, int64_t rows, int64_t K, const void *Xq,
                         int64_t N, int32_t *D, void *stream);

/*
 * The product with the steps around it fused: LayerNorm of X before it (the
 * ggml GPT-2 walkthrough, section 3.1: gamma * (x - mu) / sqrt(sigma^2 + eps)
 * + beta over each token's K values), and after it the bias add and
 * activation of section 3.5 (GELU after c_mlp_fc) or SiLU ("llama.cpp 深度解读"
 * section 4), and an element-wise factor:
 *   Y[n][r] = act(sum_k LN(X)[n][k] W[r][k] + bias[r]) * mul[n][r]
 * with the Q4_0 x Q8_0 product of mul_mat_q4_0_q8_0 (LN(X) is what gets
 * quantized).  LayerNorm: mean and population variance in fp64, the normalized
 * value evaluated in fp64 and rounded to fp32.  GELU: GPT-2's tanh form
 * 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))); SiLU: y / (1 + exp(-y)).
 *   ln_gamma, ln_beta  device fp32[K] each, or both NULL (no LayerNorm);
 *                      ln_eps >= 0.
 *   bias               device fp32[rows] or NULL.
 *   act                Q4BQ_ACT_NONE, Q4BQ_ACT_GELU or Q4BQ_ACT_SILU.
 *   mul                device fp32 N x rows or NULL; may be Y itself (read
 *                      before Y is written), otherwise must not overlap it.
 *   workspace          NULL (the library takes stream-ordered scratch) or a
 *                      16-byte aligned device buffer of ws_bytes >=
 *                      q4bq_fused_workspace_size(rows, K, N), apart from every
 *                      other buffer (the form for graph capture).
 * Other arguments and errors as for mul_mat_q4_0_q8_0 (a short workspace:
 * Q4BQ_ENOMEM); N < 2^22 with LayerNorm (one 1024-thread workgroup per
 * token).  Launches: with one token (N = 1) and rows of at most 128 blocks or
 * a block count the task kernel takes (every K of the GPT-2 and Llama shapes),
 * one launch per product: the decode kernel normalizes and quantizes the
 * token in its prologue (each workgroup takes the statistics over the whole
 * token itself) and applies the epilogue in its store, and the workspace is
 * not touched.  Otherwise one kernel that normalizes X (if asked) and
 * quantizes it into the workspace, then the product with the epilogue in its
 * store.
 */
#define Q4BQ_ACT_NONE 0
#define Q4BQ_ACT_GELU 1
#define Q4BQ_ACT_SILU 2
size_t q4bq_fused_workspace_size(int64_t rows, int64_t K, int64_t N);
int mul_mat_q4_0_q8_0_fused(const void *Wq, int64_t rows, int64_t K, const float *X,
                            int64_t N, const float *ln_gamma, const float *ln_beta,
                            float ln_eps, const float *bias, int act, const float *mul,
                            float *Y, void *workspace, size_t ws_bytes, void *stream);

/*
 * The Llama feed-forward's first half ("llama.cpp 深度解读" section 4, step I:
 * up and gate projections of the same normalized input, then
 * SiLU(gate) * up):
 *   H = SiLU(LN(X) Wgate^T) * (LN(X) Wup^T)
 * X is normalized (optional, as above) and quantized, once (or, in the one-
 * token form of mul_mat_q4_0_q8_0_fused, in the prologue of each of the two
 * product launches); the gate product writes SiLU(gate) into H and the up
 * product multiplies it in its store.
 *   Wgate, Wup  rows x (K/32) Q4_0 blocks each; H device fp32 N x rows.
 * Workspace and errors as for mul_mat_q4_0_q8_0_fused.
 */
int mul_mat_q4_0_q8_0_swiglu(const void *Wgate, const void *Wup, int64_t rows, int64_t K,
                             const float *X, int64_t N, const float *ln_gamma,
                             const float *ln_beta, float ln_eps, float *H, void *workspace,
                             size_t ws_bytes, void *stream);

/*
 * Q8_0 weights: Y = mul_mat with weight blocks in the Q8_0 format.  Section 1
 * of "llama.cpp 深度解读" lists Q8_0 (8 bits per weight) beside Q4_0 in its
 * table of quantization types; its block is the block_q8_0 of the
 * activations (binary16 d, then 32 int8 q; element j = q_j * d), so the
 * weights come from q8_0_quantize(W, rows, K, Wq8).  Per block the integer
 * dot s = sum_j qw_j * qx_j (no offset) is scaled by d_w * d_x in fp32, as in
 * section 3's product.
 *   Wq8  device, rows x (K/32) blocks of 34 bytes, 2-byte aligned.
 *   X, N, Y, stream  as for mul_mat_q4_0_q8_0 (X is quantized inside).
 * Requires K/32 <= 1024 (K <= 32768); other errors as for mul_mat_q4_0_q8_0.
 * N <= 8: one row-streaming launch per group of tokens (fewer than 8 above
 * K = 14336), no scratch memory.  N > 8: the activations are quantized into
 * stream-ordered scratch of N * K/32 * 34 bytes (hipMallocAsync on `stream`,
 * Q4BQ_ENOMEM if that fails), then the int8 matrix-core kernel reads Wq8 once
 * per 128-token tile, in ceil(rows / 128) * ceil(N / 128) workgroups of 256
 * threads (shapes past HIP's grid limit: Q4BQ_EINVAL).
 */
int mul_mat_q8_0_q8_0(const void *Wq8, int64_t rows, int64_t K, const float *X,
                      int64_t N, float *Y, void *stream);

/*
 * Test export for Q8_0 weights: D[(n * rows + r) * (K/32) + b] = the integer
 * dot of weight block (r, b) with activation block (n, b) of Xq (pages' Q8_0
 * layout): for N <= 8 by the decode kernel's dot function, above 8 by the
 * matrix-core kernel's int8 MFMA (stream-ordered scratch as for the product).
 * D: N*rows*(K/32) int32, 4-byte aligned, must not overlap the inputs.
 */
int q8_0_q8_0_block_dots(const void *Wq8, int64_t rows, int64_t K, const void *Xq,
                         int64_t N, int32_t *D, void *stream);

/*
 * For callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): mul_mat_q4_0_q8_0 with its
 * scratch in a fixed device array that the library holds on each GPU it runs
 * on until the process ends (Q4BQ_NOALLOC_SCRATCH_BYTES = 16 MiB per GPU).
 * Arguments, checks and results are those of mul_mat_q4_0_q8_0 (the same
 * kernels; Y bit for bit that of mul_mat_q4_0_q8_0_ex); no hipMalloc,
 * hipMallocAsync or hipFree is called.  Sizes whose scratch exceeds the
 * array return Q4BQ_ESCRATCH before anything is launched: above 8 tokens the
 * activations take N * K/32 * 64 bytes (up to 512 tokens at K = 16384), and
 * where the matrix-core kernel splits K (fewer than 256 workgroup tiles) its
 * range sums splits * N * rows * 4 bytes more.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap in time on one GPU (two
 * streams, or two host threads) race and must be serialized by the caller.
 */
#define Q4BQ_NOALLOC_SCRATCH_BYTES (16u * 1024u * 1024u)
int mul_mat_q4_0_q8_0_noalloc(const void *Wq, int64_t rows, int64_t K, const float *X,
                              int64_t N, float *Y, void *stream);

/* Static text for a status code. */
const char *q4bq_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int q4bq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4BQ_H */
