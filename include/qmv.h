/*
 * qmv.h — block-quantized weight mat-vec on AMD Instinct MI355X (gfx950).
 *
 * y = W x for weights stored as GGML-style 32-element blocks (Q4_0, Q8_0)
 * or 256-element super-blocks (Q6_K, Q5_K) against fp32 activations, for 1 to 16
 * activation rows, plus the expert-indexed variant over a stack of
 * per-expert weight matrices and the MoE steps around it.
 *
 * Source of the operations: the hf2q 0.1.1 pages.
 *  - Dense call: `dispatch_qmatmul(session, registry, device, x, &MlxQWeight,
 *    y, m, hint)` as used for the Q/K/V, O, FFN gate/up/down and router
 *    projections in `MlxModelWeights::encode_one_layer`
 *    (src/inference/models/gemma4/gpu_full_attn.rs). The weight handle
 *    `MlxQWeight { buffer, info: QuantWeightInfo { ggml_dtype, rows, cols } }`
 *    (src/inference/models/gemma4/model.rs, `lm_head_q8` block in
 *    `load_from_gguf`) holds `rows` = output features N and `cols` = K,
 *    in a byte buffer of shape [rows, blocks_per_row * block_bytes].
 *  - Expert-indexed call: `quantized_matmul_id_ggml(...)` with parameter
 *    block `GgmlQuantizedMatmulIdParams { n_tokens, top_k, n, k, n_experts,
 *    expert_stride, ggml_type }` (gpu_full_attn.rs, MoE blocks B11 gate_up and
 *    B13 down); stacked weights `[n_experts, N, packed_K]` with a byte stride
 *    per expert (model.rs, `MlxMoeWeights`).
 *  - The MoE steps on either side of the down call in the same function:
 *    SwiGLU of the gate_up rows (B12, `moe_swiglu_batch_encode`) and the
 *    routing-weighted sum over slots (B14, `moe_weighted_sum_encode`).
 *
 * Block formats (32 weights per block):
 *   Q4_0, 18 bytes: binary16 scale d (little-endian), then 16 bytes where
 *         byte j holds element j in its low nibble and element j+16 in its
 *         high nibble; w = (code - 8) * d. (The pages only name the format;
 *         this is the GGML Q4_0 layout.)
 *   Q8_0, 34 bytes: binary16 scale d, then 32 int8 codes; w = code * d
 *         (the inverse of the lm_head Q8_0 encoder in `load_from_gguf`).
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers, owned by the caller. The
 *    library never synchronizes and never allocates or frees memory: each
 *    call only enqueues kernels on `stream` (a hipStream_t; NULL = the null
 *    stream) that read the inputs and write the outputs, and returns. Every
 *    call can therefore be captured into a HIP graph as it is.
 *  - Arguments are validated on the host before any HIP call. A rejected call
 *    launches nothing, returns a negative status and sets a thread-local
 *    message readable with qmv_last_error().
 *  - Y is overwritten (not accumulated into) and must not overlap W, X, the
 *    ids or the scales.
 *  - Results: each output element is an fp32 sum whose error against the
 *    exact value is below 1e-4 * sum_k |w_k x_k| + 1e-6. With M >= 2 the
 *    Q4_0 / Q8_0 products run on the matrix cores with each activation
 *    split into two bf16 (x = hi + lo, relative error at most 2^-16, the
 *    fp32 exponent range kept), so that bound holds for every finite input
 *    whose block sums stay within the fp32 range: the code sum of a block,
 *    sum_k c_k x_k (c = code - 8 or the int8 code), is formed before the
 *    block scale is applied, which is always in range for |x| < 2^116.
 *    Non-finite activations propagate as in exact arithmetic (inf * 0 = NaN). Runs on the same
 *    inputs and the same device give bitwise-identical outputs (no atomics).
 *  - Calls are reentrant; concurrent calls on different streams are safe as
 *    long as their outputs do not overlap.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QMV_OK 0
#define QMV_EINVAL (-1)       /* bad shape, stride, pointer or overlap */
#define QMV_EALIGN (-2)       /* misaligned pointer or stride */
#define QMV_EUNSUPPORTED (-3) /* unsupported qtype or shape (M outside 0..16, limits stated per call) */
#define QMV_EHIP (-4)         /* the HIP runtime reported a launch error */

/* Weight types (GGML type numbers). */
#define QMV_Q4_0 2
#define QMV_Q8_0 8
#define QMV_Q5_K 13
#define QMV_Q6_K 14

#define QMV_MAX_M 16

/*
 * qmv_q4_0 — Y[m, n] = sum_{k<K} w[n, k] * X[m, k], for m < M, n < N, with
 * w the Q4_0-decoded weights.
 *
 *  W          device, N rows of K/32 Q4_0 blocks; row n starts at byte
 *             n * ldw_bytes. Must be 2-byte aligned.
 *  ldw_bytes  row stride in bytes, >= K/32 * 18, even.
 *  X          device fp32, M rows of K values; row m starts at X + m*ldx.
 *             4-byte aligned.
 *  ldx        row stride of X in elements, >= K (ignored when M <= 1).
 *  Y          device fp32, M rows of N values; row m at Y + m*ldy.
 *  ldy        row stride of Y in elements, >= N (ignored when M <= 1).
 *  M          number of activation rows, 0..16 (0: nothing to do).
 *  N          output features, >= 0 (0: nothing to do).
 *  K          input features, >= 0 and a multiple of 32 (0: Y is zeroed).
 *  stream     hipStream_t to enqueue on.
 * Returns QMV_OK or a negative status (see above).
 */
int qmv_q4_0(const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy,
             int M, int N, int K, void* stream);

/*
 * qmv_q8_0 — as qmv_q4_0 with Q8_0 blocks (34 bytes): ldw_bytes >= K/32*34.
 */
int qmv_q8_0(const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy,
             int M, int N, int K, void* stream);

/*
 * qmv_ws — the qmv_q4_0 / qmv_q8_0 product (qtype QMV_Q4_0 or QMV_Q8_0) with
 * a caller-provided workspace, for the batched-verify calls of few output
 * rows (M >= 2, N below about 16K). The pages allocate every activation and
 * scratch buffer once at load and only encode work into them (model.rs,
 * `alloc_activation_buffers`; gpu_full_attn.rs, `encode_one_layer`); a
 * workspace of qmv_ws_bytes() bytes taken the same way lets such a call cut
 * K into segments over more compute units: each segment writes fp32 partial
 * sums into the workspace and a second launch adds them in segment order
 * (bitwise reproducible). Without it every workgroup must read and convert
 * all of X.
 *
 *  workspace        device, 256-byte aligned, owned by the caller, not
 *                   overlapping W, X or Y; NULL = none (the call is then
 *                   qmv_q4_0 / qmv_q8_0).
 *  workspace_bytes  its size; at least qmv_ws_bytes(qtype, M, N, K) when
 *                   workspace is not NULL (QMV_EINVAL otherwise).
 *  Other arguments and rules as qmv_q4_0. The workspace needs no
 *  initialisation; calls that use the same workspace must be ordered (one
 *  stream, or events), as its contents are overwritten by every call.
 */
int qmv_ws(int qtype, const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy,
           int M, int N, int K, void* workspace, size_t workspace_bytes, void* stream);

/*
 * qmv_ws_bytes — the workspace qmv_ws uses for these arguments: 0 when it
 * would not split K (M = 1, many output rows, K % 64 != 0, other qtypes),
 * else S * M * N * 4 bytes for S segments.
 */
size_t qmv_ws_bytes(int qtype, int M, int N, int K);

/*
 * qmv_ws_static — qmv_ws for callers that cannot allocate memory (code under
 * HIP graph capture that must not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation): the K-segment partial sums go to a
 * scratch array in the library's own device memory, QMV_STATIC_SCRATCH_BYTES
 * per GPU, held until the process ends; the call itself allocates nothing.
 *
 *  Arguments as qmv_ws without the workspace. A call whose
 *  qmv_ws_bytes(qtype, M, N, K) exceeds QMV_STATIC_SCRATCH_BYTES is rejected
 *  (QMV_EINVAL) before anything is launched. The device is the current one
 *  (the array's address is looked up on the first call on each device; that
 *  lookup failing gives QMV_EHIP).
 *  Every call on one GPU shares that GPU's array: calls that may overlap in
 *  time on one GPU (different streams, or graphs replayed concurrently) race
 *  and give wrong results; order them. Nothing in the array needs to start
 *  at zero (each call writes the partial sums it reads).
 */
#define QMV_STATIC_SCRATCH_BYTES (4 << 20)
int qmv_ws_static(int qtype, const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy,
                  int M, int N, int K, void* stream);

/*
 * qmv_q6_k — as qmv_q4_0 with Q6_K super-blocks: 256 weights in 210 bytes.
 *
 * The pages load the lm_head natively in this format (`lm_head_q6k` of
 * `MlxModelWeights` in model.rs: gemma4's token_embd.weight as Q6_K
 * [2816, 262144] = 605 MB, dispatched through `dispatch_qmatmul`). They name
 * the format but do not lay it out; the layout taken is the GGML k-quant
 * Q6_K super-block:
 *   bytes   0..127  ql, low 4 bits of the 6-bit codes
 *   bytes 128..191  qh, high 2 bits
 *   bytes 192..207  16 int8 scales, scale j for weights 16j..16j+15
 *   bytes 208..209  binary16 d
 * Weight i: h = i/128, r = i%128, g = r/32, l = r%32; low bits = nibble g/2
 * (0 = low) of ql[64h + 32(g%2) + l]; high bits = bits 2g, 2g+1 of
 * qh[32h + l]; code q = low | high << 4; w = d * scale[i/16] * (q - 32).
 *
 *  K          a non-negative multiple of 256, at most 16384.
 *  ldw_bytes  >= K/256 * 210, even; W 2-byte aligned (rows of an odd number
 *             of super-blocks are 2-byte aligned, and are read as such).
 *  Other arguments as qmv_q4_0 (M 0..16; activation rows are processed in
 *  launches of up to 4, each reading the weights once).
 */
int qmv_q6_k(const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy,
             int M, int N, int K, void* stream);

/*
 * qmv_q5_k — as qmv_q6_k with Q5_K super-blocks: 256 weights in 176 bytes.
 *
 * The pages' production model keeps its dense FFN gate, up and router
 * projections in this format (the comment on the B9 dispatch group of
 * `encode_one_layer`: Q5_K projections from 2816 to 5760, twice, plus a 2816 to 128 router). Named only; the
 * layout taken is the GGML k-quant Q5_K super-block:
 *   bytes   0..1    binary16 d        bytes 2..3  binary16 dmin
 *   bytes   4..15   eight 6-bit sub-block scales and minimums, packed: for
 *                   sub-block j < 4 scale = s[j] & 63, min = s[j+4] & 63; for
 *                   j >= 4 scale = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
 *                   min = (s[j+4] >> 4) | (s[j] >> 6) << 4   (s = bytes 4..15)
 *   bytes  16..47   qh: bit j of qh[l] is bit 4 of the code of weight 32j + l
 *   bytes  48..175  qs: the low 4 bits; sub-blocks 2i and 2i+1 in the low and
 *                   high nibbles of qs[32i + l]
 * w = d * scale_j * q - dmin * min_j for weight 32j + l.
 *  K          a non-negative multiple of 256, at most 16384.
 *  ldw_bytes  >= K/256 * 176, even; W 2-byte aligned.
 *  Other arguments as qmv_q4_0 (M 0..16, launches of up to 4 rows).
 */
int qmv_q5_k(const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy,
             int M, int N, int K, void* stream);

/*
 * qmv_gemm — Y = deq(W) X^T for any number of activation rows M (prefill):
 * the product of qmv_q4_0 / qmv_q8_0 / qmv_q5_k / qmv_q6_k without the
 * M <= 16 limit.
 *
 * The pages route m > 8 through an F16 shadow of the weights (the F16 shadow
 * population pass of the gemma4 model page: every attention and dense-MLP
 * quantized weight pre-dequantized to F16 after load, so that
 * `dispatch_qmatmul` takes an F16-input matmul for m > 8; about 1 GB extra,
 * +16% prefill at 2K tokens). Here the weights
 * stay block-quantized and no shadow is kept. Q4_0 and Q8_0 with M >= 64,
 * K a multiple of 64, X 16-byte aligned with ldx % 4 == 0 and W, ldw_bytes
 * 4-byte aligned (ldw_bytes < 2^32) go through one tiled matrix-core launch:
 * tiles of 64 activation rows x 256 weight rows, each weight decoded once
 * per 64 activation rows and each activation converted once per 256 weight
 * rows. Other Q4_0 / Q8_0 calls take the rows of X in blocks of 16 through
 * the matrix-core product (one launch, blocks that read a weight tile side
 * by side), and Q5_K / Q6_K through their own product, up to 16 rows a
 * launch.
 *
 *  qtype   QMV_Q4_0, QMV_Q8_0, QMV_Q5_K or QMV_Q6_K.
 *  M       >= 0 (0: nothing to do); other arguments and rules as qmv_q4_0
 *          (qmv_q6_k / qmv_q5_k for the super-block types).
 */
int qmv_gemm(int qtype, const void* W, size_t ldw_bytes, const float* X, size_t ldx, float* Y, size_t ldy,
             int M, int N, int K, void* stream);

/*
 * qmv_affine4 — Y = deq(W) X^T for MLX affine 4-bit weights, groups of 32.
 *
 * The gemma4 model page builds its DWQ MoE stacks this way: each row's codes
 * packed eight to a 32-bit word, code j of a word in bits 4j..4j+3, and one
 * bf16 scale and one bf16 bias per group of 32 weights in arrays of their
 * own (the `MlxAffineMoeStack` weight, scales and biases buffers, bits = 4,
 * group_size = 32). The pages call the format affine and store a bias per
 * group; the dequantization taken is w = scale * q + bias, q = 0..15.
 *
 *  Wq       device uint32, row n at Wq + n*ldw (ldw in words, >= K/8),
 *           4-byte aligned.
 *  scales, biases  device bf16 bit patterns, row n at + n*lds (lds >= K/32),
 *           2-byte aligned.
 *  K        a positive multiple of 32, at most 16384 (rows need not hold a
 *           multiple of 128 weights).
 *  Other arguments as qmv_q4_0 (M 0..16).
 */
int qmv_affine4(const uint32_t* Wq, size_t ldw, const uint16_t* scales, const uint16_t* biases, size_t lds,
                const float* X, size_t ldx, float* Y, size_t ldy, int M, int N, int K, void* stream);

/*
 * qmv_affine4_id — the expert-indexed product (qmv_id's mapping and error
 * behaviour) over stacked affine 4-bit experts: expert e's words start at
 * Wq + e*expert_stride_words, its scales and biases at
 * + e*expert_stride_groups. Each (token, slot) pair reads its expert's rows.
 */
int qmv_affine4_id(const uint32_t* Wq, size_t expert_stride_words, size_t ldw, const uint16_t* scales,
                   const uint16_t* biases, size_t expert_stride_groups, size_t lds, int n_experts,
                   const float* X, size_t ldx, const uint32_t* ids, int n_tokens, int top_k,
                   float* Y, size_t ldy, int N, int K, const float* expert_scale, int* err_flag,
                   void* stream);

/*
 * qmv_id — expert-indexed product over a stack of weight matrices.
 *
 * For t < n_tokens and s < top_k, with p = t*top_k + s and e = ids[p]:
 *   Y[p, n] = sc_e * sum_{k<K} w_e[n, k] * X[t, k],   n < N,
 * where w_e is the N x K matrix of type `qtype` starting at byte
 * e * expert_stride_bytes of W (rows ldw_bytes apart), and sc_e =
 * expert_scale[e] when expert_scale is non-NULL, else 1.
 *
 * The gate_up form of the pages is (n_tokens = T, top_k = k) with one X row
 * per token; the down form flattens the slots: (n_tokens = T*k, top_k = 1)
 * with one X row per slot.
 *
 *  qtype                QMV_Q4_0, QMV_Q8_0, QMV_Q6_K or QMV_Q5_K (the pages'
 *                       production MoE stores the gate_up experts as Q6_K; for the
 *                       super-block types K is a multiple of 256, at most 16384,
 *                       and each (token, slot) pair reads its expert's rows, with
 *                       no grouping of pairs by expert).
 *  W                    device, stacked weights, 2-byte aligned.
 *  expert_stride_bytes  >= N * ldw_bytes, even.
 *  ldw_bytes            row stride within an expert, >= K/32 * block bytes, even.
 *  n_experts            > 0.
 *  X, ldx               device fp32 [n_tokens, K] with row stride ldx >= K.
 *  ids                  device uint32 [n_tokens * top_k].
 *  n_tokens             >= 0 (0: nothing to do).
 *  top_k                > 0.
 *  Y, ldy               device fp32 [n_tokens * top_k, N], row stride ldy >= N.
 *  N, K                 as for qmv_q4_0.
 *  expert_scale         device fp32 [n_experts] or NULL.
 *  err_flag             device int or NULL. An id >= n_experts is invalid
 *                       input: its output row is filled with NaN and, when
 *                       err_flag is given, 1 is stored to *err_flag (the
 *                       library never clears it; the caller zeroes it).
 * Reads (Q4_0, Q8_0): with more than 64 (token, slot) pairs, each selected
 * expert's weights are read from memory once per call, however many pairs
 * select it; with up to 64 pairs (decode-sized calls) every pair reads its
 * expert's rows, which is faster at that size although an expert selected by
 * several pairs is then read once per pair.
 * Returns QMV_OK or a negative status.
 */
int qmv_id(int qtype, const void* W, size_t expert_stride_bytes, size_t ldw_bytes, int n_experts,
           const float* X, size_t ldx, const uint32_t* ids, int n_tokens, int top_k,
           float* Y, size_t ldy, int N, int K, const float* expert_scale, int* err_flag,
           void* stream);

/*
 * qmv_id_swiglu — the MoE down projection fed by SwiGLU: qmv_id with
 *   X[t, k] = silu(G[t, k]) * G[t, K + k],   silu(z) = z / (1 + e^-z),
 * so that the SwiGLU step between the gate_up and down calls (block B12,
 * `moe_swiglu_batch_encode`, of `encode_one_layer`) runs inside the down call
 * (block B13) and its result never goes to memory. Row t of G is a gate_up
 * output row: 2K values, the gate half first (the pages do not order the
 * halves; gate first follows the buffer name `gate_up`).
 *
 *  G, ldg   device fp32 [n_tokens, 2K], row stride ldg >= 2K, 4-byte aligned.
 *  qtype    QMV_Q4_0 or QMV_Q8_0 (the super-block types return QMV_EUNSUPPORTED).
 *  Every other argument, the result layout, NaN rows for bad ids and the
 *  error behaviour are those of qmv_id. For the pages' down form pass the
 *  gate_up output rows with (n_tokens = T*k, top_k = 1).
 * In fp32, silu(z) for z < -88.7 is -0 (e^-z overflows), against a true
 * value below 1e-36 in size.
 */
int qmv_id_swiglu(int qtype, const void* W, size_t expert_stride_bytes, size_t ldw_bytes, int n_experts,
                  const float* G, size_t ldg, const uint32_t* ids, int n_tokens, int top_k,
                  float* Y, size_t ldy, int N, int K, const float* expert_scale, int* err_flag,
                  void* stream);

/*
 * qmv_moe_wsum — routing-weighted sum over each token's slots (block B14,
 * `moe_weighted_sum_encode`, of `encode_one_layer`):
 *   out[t, n] = sum_{s<top_k} weights[t*top_k + s] * Y[t*top_k + s, n],
 * accumulated in slot order (s = 0 first) with one fp32 fma per slot.
 * The pages pass routing weights already multiplied by the per-expert scale;
 * pass those, or plain weights with the scale applied by qmv_id's
 * expert_scale (the sum is linear, so both give the same value).
 *
 *  Y, ldy     device fp32 [n_tokens*top_k, N], row stride ldy >= N.
 *  weights    device fp32 [n_tokens*top_k].
 *  n_tokens   >= 0 (0: nothing to do).   top_k > 0.   N >= 0.
 *  out, ldo   device fp32 [n_tokens, N], row stride ldo >= N; overwritten,
 *             must not overlap Y or weights.
 * All pointers 4-byte aligned. Returns QMV_OK or a negative status.
 */
int qmv_moe_wsum(const float* Y, size_t ldy, const float* weights, int n_tokens, int top_k, int N,
                 float* out, size_t ldo, void* stream);

/*
 * qmv_moe_down — the down half of the MoE block in one launch: SwiGLU of each
 * slot's gate_up row (B12), the expert-indexed down product (B13) and the
 * routing-weighted sum (B14):
 *   out[t, n] = sum_{s<top_k} weights[p] * sc_e * sum_{k<K} w_e[n, k] *
 *               silu(G[p, k]) * G[p, K + k],      p = t*top_k + s, e = ids[p],
 * with w_e and sc_e as in qmv_id, and the slot sum in slot order.
 *
 *  G, ldg     device fp32 [n_tokens*top_k, 2K]: the gate_up id output, row p
 *             for slot s of token t; ldg >= 2K.
 *  ids        device uint32 [n_tokens*top_k].
 *  weights    device fp32 [n_tokens*top_k] routing weights.
 *  out, ldo   device fp32 [n_tokens, N], ldo >= N; overwritten, must not
 *             overlap any input.
 *  W, expert_stride_bytes, ldw_bytes, n_experts, N, K, expert_scale: as qmv_id.
 *  err_flag   as qmv_id: a bad id makes the token's outputs NaN.
 * Each token reads the rows of its own top_k experts, so tokens that share
 * an expert read it again: this is the form for decode, one or a few tokens
 * with distinct experts. With many tokens, qmv_id_swiglu (each selected
 * expert read once per call) followed by qmv_moe_wsum reads less.
 * Supported: K a positive multiple of 64, top_k <= 64, top_k * K within
 * 64 KiB of staged rows (top_k * K <= 15360), W, ldw_bytes and
 * expert_stride_bytes 4-byte aligned; other shapes return QMV_EUNSUPPORTED
 * (qmv_id_swiglu + qmv_moe_wsum compute them). Returns QMV_OK or a negative
 * status.
 */
int qmv_moe_down(int qtype, const void* W, size_t expert_stride_bytes, size_t ldw_bytes, int n_experts,
                 const float* G, size_t ldg, const uint32_t* ids, const float* weights, int n_tokens,
                 int top_k, float* out, size_t ldo, int N, int K, const float* expert_scale,
                 int* err_flag, void* stream);

/*
 * qmv_batch — several independent M = 1 products in one launch:
 *   problems[i].y = deq(problems[i].W) x problems[i].x,  i < n_problems.
 *
 * This is the grouped launch of projections that run together: the pages
 * encode Q, K and V (which share one input) as one concurrent group, and
 * the FFN gate, up and router as another (`encode_one_layer`, the barrier
 * groups before the first and the ninth block of dispatches). Problems may
 * share x; their outputs must not overlap each other or any W or x. When
 * every problem reads the same x pointer with the same K, their rows are
 * streamed as one matrix (Q4_0 and Q8_0: the results equal the single calls'
 * bit for bit; Q5_K and Q6_K: the launch picks its lane-group width for all
 * the rows together, so a result may differ from the single call's in the
 * order of its fp32 sums, both within the tolerance). For the super-block
 * types the problems on the first problem's x and K go out as one launch,
 * any others one call each.
 *
 *  qtype        QMV_Q4_0, QMV_Q8_0, QMV_Q5_K or QMV_Q6_K (all problems of a
 *               batch have one type).
 *  problems     HOST array of n_problems descriptors, read during the call.
 *  n_problems   0..QMV_MAX_BATCH (0: nothing to do).
 * Each descriptor follows the single call's rules for M = 1 (W 2-byte
 * aligned, ldw_bytes even and >= the row's blocks in bytes, x and y 4-byte
 * aligned; K a non-negative multiple of 32, and for Q5_K / Q6_K of 256 and
 * at most 16384: QMV_EUNSUPPORTED above). Every problem is validated before anything
 * is launched; one bad descriptor rejects the whole call.
 */
#define QMV_MAX_BATCH 16

typedef struct {
    const void* W;    /* device: N rows of K/32 blocks */
    size_t ldw_bytes; /* row stride in bytes */
    const float* x;   /* device: K activations */
    float* y;         /* device: N outputs (overwritten) */
    int N;            /* output features, >= 0 */
    int K;            /* input features, multiple of 32, >= 0 */
} qmv_problem;

int qmv_batch(int qtype, const qmv_problem* problems, int n_problems, void* stream);

/* Message for the last non-zero status returned on the calling thread. */
const char* qmv_last_error(void);

/*
 * qmv_stream_read — the memory-roofline reference for measurements, not part
 * of the product: reads every byte of [src, src + bytes) once from device
 * memory with 16-byte non-temporal loads and discards the data. A
 * benchmark times it next to the qmv calls so that their bandwidth can be
 * read against what a plain streaming read reaches on the same GPU.
 *
 *  src     device, 16-byte aligned; bytes a multiple of 16 (0: no-op).
 *  sink    device, one uint32 the kernel may overwrite (4-byte aligned).
 *  stream  hipStream_t, asynchronous. Errors as for the other calls
 *          (QMV_EINVAL for NULL pointers, QMV_EALIGN for alignment).
 */
int qmv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMV_H */
