/*
 * CPU oracle for block-quantized weight mat-vec (test infrastructure only).
 *
 * This file is TEST INFRASTRUCTURE. Only the test suite, the package's smoke
 * check and the benchmark's CPU-baseline leg may load or call it. The HIP
 * library never links, includes or calls anything here, and nothing here
 * includes anything of the HIP library.
 *
 * What it computes is the plain definition, in fp64, with no blocking,
 * fusion or reordering:
 *
 *   1. decode every 32-element block of a weight row into fp64 values
 *      (a binary16 scale times an integer code), giving the dense row w[0..K);
 *   2. y[m][n] = sum_{k<K} w[n][k] * x[m][k], summed in index order in fp64;
 *      a[m][n] = sum_{k<K} |w[n][k] * x[m][k]|, the magnitude the acceptance
 *      tolerance is scaled by.
 *
 * Block formats (32 weights per block, rows of K/32 blocks, row stride ldw
 * bytes):
 *
 *   Q8_0 (34 B): bytes 0,1 = scale bits, low byte first; bytes 2..33 = int8
 *   codes, element j in byte 2+j; w = code * d. This is the inverse of the
 *   lm_head Q8_0 encoder on the hf2q page `src/inference/models/gemma4/
 *   model.rs` (`load_from_gguf`, the block that builds `lm_head_q8`: it
 *   writes `d_bits & 0xFF`, then `d_bits >> 8`, then each code as a byte).
 *   Any int8 decodes as-is, -128 included.
 *
 *   Q4_0 (18 B): the pages name the format (the `MlxMoeWeights` doc calls
 *   the weights as kept in the GGML block layout; a `qwen3-vl-2b-q4_0.gguf` model is
 *   named in `MlxMoeWeights::dense_placeholder`) but never lay it out. The
 *   reading taken here is the GGML Q4_0 block: bytes 0,1 = binary16 scale
 *   (low byte first); byte 2+j (j < 16) holds element j in its low nibble and
 *   element j+16 in its high nibble; w = (code - 8) * d.
 *
 *   The scale is decoded exactly from its IEEE 754 binary16 bit pattern:
 *   subnormals kept, signed zero kept, Inf/NaN propagate.
 *
 *   Q6_K (210 B per 256 weights): the format of the lm_head the pages load
 *   natively (`lm_head_q6k` in `MlxModelWeights`, model.rs: gemma4's
 *   token_embd.weight as Q6_K [2816, 262144] = 605 MB, which fixes 210 bytes
 *   per 256 weights). The pages name the format only; the layout read here is
 *   the GGML k-quant Q6_K super-block, written out at decode_superblock_q6_k.
 *
 *   Q5_K (176 B per 256 weights): the format of the dense FFN gate, up and
 *   router projections of the pages' production model (the B9 comment in
 *   `encode_one_layer`: Q5_K projections from 2816 to 5760, twice, plus a 2816 to 128 router). Named only; the
 *   layout read here is the GGML k-quant Q5_K super-block, written out at
 *   decode_superblock_q5_k.
 *
 * Expert-indexed variant (the `quantized_matmul_id_ggml` calls in
 * `MlxModelWeights::encode_one_layer` on the hf2q page
 * `src/inference/models/gemma4/gpu_full_attn.rs`, MoE blocks B11 and B13,
 * with the parameter block n_tokens, top_k, n, k, n_experts, expert_stride):
 * for token t < n_tokens and slot s < top_k, e = ids[t*top_k + s]; expert
 * e's weights start at byte e*expert_stride of the stacked buffer; the
 * output row is t*top_k + s and the input row is t. An optional per-expert
 * scale multiplies the row (the pages fold `per_expert_scale` into the
 * routing weights of the weighted sum that follows; since that sum is linear,
 * scaling the id output row is the same product).
 *
 * MoE steps around the expert-indexed product (same page, blocks B12 and
 * B14): SwiGLU of the gate_up rows, silu(gate) * up, which becomes the down
 * projection's activation rows, and the routing-weighted sum of the down
 * rows over each token's top_k slots. Composed in that order (gate_up id,
 * SwiGLU, down id, weighted sum) they are the MoE feed-forward of one layer.
 *
 * Every function returns 0 on success and a negative value on bad arguments
 * (oracle_silu returns its value).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_QK 32
#define ORACLE_QK_K 256
#define ORACLE_Q4_0 2
#define ORACLE_Q8_0 8
#define ORACLE_Q5_K 13
#define ORACLE_Q6_K 14

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal or zero: f * 2^-14 * 2^-10 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

static int block_bytes(int qtype) {
    if (qtype == ORACLE_Q4_0) return 18;
    if (qtype == ORACLE_Q8_0) return 34;
    if (qtype == ORACLE_Q6_K) return 210;
    if (qtype == ORACLE_Q5_K) return 176;
    return -1;
}

/* Weights per block: 32, or 256 for the super-block formats. */
static int block_elems(int qtype) {
    return (qtype == ORACLE_Q6_K || qtype == ORACLE_Q5_K) ? ORACLE_QK_K : ORACLE_QK;
}

/*
 * Q5_K super-block (176 bytes, 256 weights), the GGML k-quant 5-bit format:
 *   bytes   0..1    binary16 d (scale of the sub-block scales)
 *   bytes   2..3    binary16 dmin (scale of the sub-block minimums)
 *   bytes   4..15   eight 6-bit sub-block scales and eight 6-bit minimums
 *   bytes  16..47   qh: bit j of qh[l] is the high bit of weight 32j + l
 *   bytes  48..175  qs: low 4 bits; sub-blocks 2i and 2i+1 share
 *                   qs[32i .. 32i+31], 2i in the low nibbles, 2i+1 in the high
 * Sub-block j (weights 32j .. 32j+31), with s = bytes 4..15:
 *   j < 4:  scale = s[j] & 63,                     min = s[j+4] & 63
 *   j >= 4: scale = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
 *           min   = (s[j+4] >> 4) | (s[j] >> 6) << 4
 * Weight 32j + l: q = nibble of qs[32(j/2) + l] (low if j even) + 16 * bit j
 * of qh[l]; w = d * scale * q - dmin * min.
 */
static void decode_superblock_q5_k(const uint8_t* b, double* out) {
    double d = oracle_f16_to_f64((uint16_t)(b[0] | (b[1] << 8)));
    double dmin = oracle_f16_to_f64((uint16_t)(b[2] | (b[3] << 8)));
    const uint8_t* s = b + 4;
    const uint8_t* qh = b + 16;
    const uint8_t* qs = b + 48;
    for (int j = 0; j < 8; ++j) {
        int sc, mn;
        if (j < 4) {
            sc = s[j] & 63;
            mn = s[j + 4] & 63;
        } else {
            sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
        for (int l = 0; l < 32; ++l) {
            int byte = qs[32 * (j / 2) + l];
            int low = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
            int q = low + 16 * ((qh[l] >> j) & 1);
            out[32 * j + l] = d * (double)sc * (double)q - dmin * (double)mn;
        }
    }
}

/*
 * Q6_K super-block (210 bytes, 256 weights), the GGML k-quant 6-bit format:
 *   bytes   0..127  ql: low 4 bits of the codes
 *   bytes 128..191  qh: high 2 bits of the codes
 *   bytes 192..207  16 int8 sub-block scales, one per 16 weights
 *   bytes 208..209  binary16 super-block scale d (low byte first)
 * Weight i (0..255): half h = i / 128 and r = i % 128, quarter g = r / 32,
 * l = r % 32. Its low 4 bits are the low (g < 2) or high (g >= 2) nibble of
 * ql[64h + 32(g % 2) + l]; its high 2 bits are bits 2g, 2g + 1 of
 * qh[32h + l]; code q = low + 16 * high (0..63); its scale is
 * scales[8h + 2g + l / 16]; w = d * scale * (q - 32).
 */
static void decode_superblock_q6_k(const uint8_t* b, double* out) {
    const uint8_t* ql = b;
    const uint8_t* qh = b + 128;
    const int8_t* sc = (const int8_t*)(b + 192);
    double d = oracle_f16_to_f64((uint16_t)(b[208] | (b[209] << 8)));
    for (int i = 0; i < ORACLE_QK_K; ++i) {
        int h = i / 128, r = i % 128, g = r / 32, l = r % 32;
        int byte = ql[64 * h + 32 * (g % 2) + l];
        int low = g < 2 ? (byte & 0x0F) : (byte >> 4);
        int high = (qh[32 * h + l] >> (2 * g)) & 3;
        int q = low + 16 * high;
        out[i] = d * (double)sc[8 * h + 2 * g + l / 16] * (double)(q - 32);
    }
}

/* Decode one 32-element block into out[0..32). */
static void decode_block(int qtype, const uint8_t* b, double* out) {
    uint16_t bits = (uint16_t)(b[0] | (b[1] << 8));
    double d = oracle_f16_to_f64(bits);
    if (qtype == ORACLE_Q4_0) {
        for (int j = 0; j < 16; ++j) {
            int lo = b[2 + j] & 0x0F;
            int hi = b[2 + j] >> 4;
            out[j] = (double)(lo - 8) * d;
            out[j + 16] = (double)(hi - 8) * d;
        }
    } else {
        for (int j = 0; j < 32; ++j) {
            int8_t q = (int8_t)b[2 + j];
            out[j] = (double)q * d;
        }
    }
}

/* Dequantize one row of K weights (K a multiple of the block size) into w[0..K). */
int oracle_dequant_row(int qtype, const uint8_t* row, int K, double* w) {
    int bb = block_bytes(qtype), qk = block_elems(qtype);
    if (bb < 0 || K <= 0 || K % qk) return -1;
    for (int b = 0; b < K / qk; ++b) {
        if (qtype == ORACLE_Q6_K)
            decode_superblock_q6_k(row + (size_t)b * bb, w + (size_t)b * qk);
        else if (qtype == ORACLE_Q5_K)
            decode_superblock_q5_k(row + (size_t)b * bb, w + (size_t)b * qk);
        else
            decode_block(qtype, row + (size_t)b * bb, w + (size_t)b * qk);
    }
    return 0;
}

static void dot_row(const double* w, const float* x, int K, double* y, double* a) {
    double s = 0.0, m = 0.0;
    for (int k = 0; k < K; ++k) {
        double p = w[k] * (double)x[k];
        s += p;
        m += fabs(p);
    }
    *y = s;
    if (a) *a = m;
}

/* The same sum for an fp64 activation row. */
static void dot_row_f64(const double* w, const double* x, int K, double* y, double* a) {
    double s = 0.0, m = 0.0;
    for (int k = 0; k < K; ++k) {
        double p = w[k] * x[k];
        s += p;
        m += fabs(p);
    }
    *y = s;
    if (a) *a = m;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/*
 * Dense product: Y[m*ldy + n] = sum_k w[n][k] * X[m*ldx + k] for m < M, n < N.
 * W: N rows of K/32 blocks, row n at W + n*ldw. A (nullable) receives the
 * absolute-product sums in the same layout as Y. nthreads <= 0 keeps the
 * OpenMP default.
 */
int oracle_qmv(int qtype, const uint8_t* W, size_t ldw, const float* X, size_t ldx,
               int M, int N, int K, double* Y, double* A, size_t ldy, int nthreads) {
    int bb = block_bytes(qtype), qk = block_elems(qtype);
    if (bb < 0 || M < 0 || N < 0 || K <= 0 || K % qk) return -1;
    if (ldw < (size_t)(K / qk) * bb || ldx < (size_t)K || ldy < (size_t)N) return -1;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
        if (!w) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(static)
            for (int n = 0; n < N; ++n) {
                oracle_dequant_row(qtype, W + (size_t)n * ldw, K, w);
                for (int m = 0; m < M; ++m)
                    dot_row(w, X + (size_t)m * ldx, K, &Y[(size_t)m * ldy + n],
                            A ? &A[(size_t)m * ldy + n] : NULL);
            }
            free(w);
        }
    }
    return err;
}

/*
 * Expert-indexed product. For t < n_tokens, s < top_k:
 *   e = ids[t*top_k + s]  (must be < n_experts, else the call fails with -3)
 *   Y[(t*top_k + s)*ldy + n] = sc * sum_k w_e[n][k] * X[t*ldx + k]
 * with w_e the N x K matrix at W + e*expert_stride (row stride ldw) and
 * sc = expert_scale[e] when expert_scale is given, else 1.
 * A receives |sc| * sum_k |w_e[n][k] * X[t*ldx + k]|.
 */
static int qmv_id_core(int qtype, const uint8_t* W, size_t expert_stride, size_t ldw, int n_experts,
                       const float* X, const double* Xd, size_t ldx, const uint32_t* ids, int n_tokens,
                       int top_k, const float* expert_scale, int N, int K, double* Y, double* A, size_t ldy,
                       int nthreads) {
    int bb = block_bytes(qtype), qk = block_elems(qtype);
    if (bb < 0 || n_experts <= 0 || n_tokens < 0 || top_k <= 0 || N < 0 || K <= 0 || K % qk) return -1;
    if (ldw < (size_t)(K / qk) * bb || ldx < (size_t)K || ldy < (size_t)N) return -1;
    if (expert_stride < (size_t)N * ldw) return -1;
    int P = n_tokens * top_k;
    for (int p = 0; p < P; ++p)
        if (ids[p] >= (uint32_t)n_experts) return -3;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
        if (!w) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(static) collapse(2)
            for (int p = 0; p < P; ++p) {
                for (int n = 0; n < N; ++n) {
                    uint32_t e = ids[p];
                    int t = p / top_k;
                    double sc = expert_scale ? (double)expert_scale[e] : 1.0;
                    const uint8_t* row = W + (size_t)e * expert_stride + (size_t)n * ldw;
                    double y, a;
                    oracle_dequant_row(qtype, row, K, w);
                    if (Xd)
                        dot_row_f64(w, Xd + (size_t)t * ldx, K, &y, &a);
                    else
                        dot_row(w, X + (size_t)t * ldx, K, &y, &a);
                    Y[(size_t)p * ldy + n] = sc * y;
                    if (A) A[(size_t)p * ldy + n] = fabs(sc) * a;
                }
            }
            free(w);
        }
    }
    return err;
}

int oracle_qmv_id(int qtype, const uint8_t* W, size_t expert_stride, size_t ldw, int n_experts,
                  const float* X, size_t ldx, const uint32_t* ids, int n_tokens, int top_k,
                  const float* expert_scale, int N, int K, double* Y, double* A, size_t ldy,
                  int nthreads) {
    if (!X) return -1;
    return qmv_id_core(qtype, W, expert_stride, ldw, n_experts, X, NULL, ldx, ids, n_tokens, top_k,
                       expert_scale, N, K, Y, A, ldy, nthreads);
}

/*
 * SiLU, the sigmoid-weighted linear unit: silu(z) = z * sigmoid(z)
 * = z / (1 + e^(-z)). For z below about -709, e^(-z) overflows to +Inf and
 * the quotient is -0, the limit; NaN propagates.
 */
double oracle_silu(double z) {
    return z / (1.0 + exp(-z));
}

/*
 * SwiGLU over rows of a gate_up product (the `moe_swiglu_batch_encode` step,
 * block B12 of `MlxModelWeights::encode_one_layer` on the hf2q page
 * `src/inference/models/gemma4/gpu_full_attn.rs`; the same page set writes the
 * dense form as down(silu(gate(x)) * up(x)) in the doc of its drafter MLP).
 * Row r of G holds 2*I values: the gate half in [0, I), the up half in
 * [I, 2I). The pages never say which half comes first; gate first is the
 * order the buffer name `gate_up` gives.
 *   H[r*ldh + i] = silu(G[r*ldg + i]) * G[r*ldg + I + i],  i < I,
 * all in fp64 from the fp32 inputs.
 */
int oracle_swiglu(const float* G, size_t ldg, int rows, int I, double* H, size_t ldh) {
    if (rows < 0 || I < 0 || ldg < (size_t)2 * I || ldh < (size_t)I) return -1;
    for (int r = 0; r < rows; ++r)
        for (int i = 0; i < I; ++i) {
            const float* g = G + (size_t)r * ldg;
            H[(size_t)r * ldh + i] = oracle_silu((double)g[i]) * (double)g[I + i];
        }
    return 0;
}

/*
 * Expert-indexed product whose activation rows are the SwiGLU of gate_up
 * rows (the down projection of the MoE block, B13 after B12): the
 * expert-indexed product above with X[t] = H[t], H = oracle_swiglu(G) over
 * n_tokens rows of 2*K values (row stride ldg).
 */
int oracle_qmv_id_swiglu(int qtype, const uint8_t* W, size_t expert_stride, size_t ldw, int n_experts,
                         const float* G, size_t ldg, const uint32_t* ids, int n_tokens, int top_k,
                         const float* expert_scale, int N, int K, double* Y, double* A, size_t ldy,
                         int nthreads) {
    if (!G || n_tokens < 0 || K <= 0 || ldg < (size_t)2 * K) return -1;
    double* H = (double*)malloc(sizeof(double) * (size_t)K * (size_t)(n_tokens > 0 ? n_tokens : 1));
    if (!H) return -2;
    int rc = oracle_swiglu(G, ldg, n_tokens, K, H, (size_t)K);
    if (rc == 0)
        rc = qmv_id_core(qtype, W, expert_stride, ldw, n_experts, NULL, H, (size_t)K, ids, n_tokens, top_k,
                         expert_scale, N, K, Y, A, ldy, nthreads);
    free(H);
    return rc;
}

/*
 * Routing-weighted sum over the top_k slots of each token (the
 * `moe_weighted_sum_encode` step, block B14 of `encode_one_layer` on the same
 * page; its weights are the routing weights that the routing step has
 * already multiplied by the per-expert scale):
 *   out[t*ldo + n] = sum_{s < top_k} w[t*top_k + s] * Y[(t*top_k + s)*ldy + n],
 * summed in slot order in fp64. A (nullable) receives
 * sum_s |w[t*top_k + s]| * YA[(t*top_k + s)*ldy + n] when YA is given (the
 * magnitudes of the rows' own sums), else sum_s |w * Y|.
 */
int oracle_moe_wsum(const double* Y, const double* YA, size_t ldy, const float* w, int n_tokens, int top_k,
                    int N, double* out, double* A, size_t ldo) {
    if (n_tokens < 0 || top_k <= 0 || N < 0 || ldy < (size_t)N || ldo < (size_t)N) return -1;
    for (int t = 0; t < n_tokens; ++t)
        for (int n = 0; n < N; ++n) {
            double s = 0.0, m = 0.0;
            for (int k = 0; k < top_k; ++k) {
                size_t p = (size_t)t * top_k + k;
                double wk = (double)w[p];
                double y = Y[p * ldy + n];
                s += wk * y;
                m += YA ? fabs(wk) * YA[p * ldy + n] : fabs(wk * y);
            }
            out[(size_t)t * ldo + n] = s;
            if (A) A[(size_t)t * ldo + n] = m;
        }
    return 0;
}

/*
 * MLX affine 4-bit weights with groups of 32 (the DWQ MoE stacks of the
 * gemma4 model page: each row's codes packed eight to a 32-bit word, code j
 * of a word in bits 4j..4j+3, and one bf16 scale and one bf16 bias per group
 * of 32 weights, in arrays of their own). The pages name the format affine
 * and store a bias beside each scale; the reading taken is the affine
 * dequantization w = scale * q + bias, q = 0..15.
 *   Wq     row n at Wq + n*ldw (ldw in 32-bit words, >= K/8)
 *   S, B   row n's scales and biases at S + n*lds, B + n*lds (>= K/32), bf16
 * bf16 is the upper half of an IEEE binary32; it is decoded exactly.
 */
double oracle_bf16_to_f64(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_dequant_affine4_row(const uint32_t* wq, const uint16_t* sc, const uint16_t* bi, int K, double* w) {
    if (K <= 0 || K % 32) return -1;
    for (int k = 0; k < K; ++k) {
        int q = (int)((wq[k / 8] >> (4 * (k % 8))) & 15);
        w[k] = oracle_bf16_to_f64(sc[k / 32]) * (double)q + oracle_bf16_to_f64(bi[k / 32]);
    }
    return 0;
}

/*
 * Y[m*ldy + n] = sum_k w[n][k] * X[m*ldx + k] for affine 4-bit rows; A
 * (nullable) receives sum_k |w x|. Same index order and fp64 as oracle_qmv.
 */
int oracle_qmv_affine4(const uint32_t* Wq, size_t ldw, const uint16_t* S, const uint16_t* B, size_t lds,
                       const float* X, size_t ldx, int M, int N, int K, double* Y, double* A, size_t ldy,
                       int nthreads) {
    if (M < 0 || N < 0 || K <= 0 || K % 32) return -1;
    if (ldw < (size_t)K / 8 || lds < (size_t)K / 32 || ldx < (size_t)K || ldy < (size_t)N) return -1;
    set_threads(nthreads);
    int err = 0;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
        if (!w) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(static)
            for (int n = 0; n < N; ++n) {
                oracle_dequant_affine4_row(Wq + (size_t)n * ldw, S + (size_t)n * lds, B + (size_t)n * lds, K, w);
                for (int m = 0; m < M; ++m)
                    dot_row(w, X + (size_t)m * ldx, K, &Y[(size_t)m * ldy + n], A ? &A[(size_t)m * ldy + n] : NULL);
            }
            free(w);
        }
    }
    return err;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
