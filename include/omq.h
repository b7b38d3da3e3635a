/*
 * omq.h -- C ABI of the OmniQuant block-calibration hot path on MI355X (gfx950).
 *
 * The method (paper reading "OmniQuant: Omnidirectionally Calibrated Quantization
 * for Large Language Models", onecrewdev.com/posts/omniquant-paper-reading):
 * weights are frozen; per LLaMA-shaped decoder block the learnable clipping
 * strengths gamma/beta of Learnable Weight Clipping (section "LWC", the LWC
 * equation) and the Learnable Equivalent Transformation parameters s, delta and
 * s_a (section "LET", the linear-layer and attention-affinity equations) are
 * trained against the full-precision block output (section "框架", the block-wise
 * objective) with AdamW (section "实验证据").
 *
 * Conventions (every entry point):
 *  - Tensor pointers are DEVICE pointers unless stated.  The caller owns every
 *    buffer; the library allocates nothing and keeps no global mutable state.
 *  - Weights are stored like nn.Linear: W is [c_out x c_in] row-major, Y = X W^T + B.
 *    The page's s (.) W therefore scales W's input channels (columns).
 *  - Activations are [T x C] row-major (T tokens).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; a kernel fault surfaces at the caller's next synchronisation.
 *  - Outputs never alias inputs unless stated.
 *  - Every function validates its arguments before launching anything and returns
 *    OMQ_OK (0) or a negative OMQ_E_* status; on error nothing is launched.
 *  - Row lengths must be multiples of 4 elements (OMQ_E_ALIGN), and of 8 for the
 *    bf16 operands of omq_gemm; pointers must be 16-byte aligned (OMQ_E_ALIGN).
 *  - Empty outputs: omq_lwc_fakequant with c_out = 0, omq_act_quant with T = 0, and
 *    omq_gemm / omq_code_gemm with M = 0 or N = 0 return OMQ_OK at once, reading
 *    and writing nothing (their pointers may then be NULL).
 *  - Bit widths: 2..8, or 16 meaning "this quantizer is off".
 *  - Quantizer arithmetic is IEEE float32, one rounding per operation, no fused
 *    multiply-add, rint = round half to even, gamma = sigmoid(a) computed in
 *    double and rounded to float; integer codes are therefore reproducible.
 */
#ifndef OMQ_H_
#define OMQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OMQ_ABI_VERSION 4

/* status codes */
#define OMQ_OK 0
#define OMQ_E_INVALID_ARG -1   /* NULL where required, bit width out of range, bad enum */
#define OMQ_E_SHAPE -2         /* inconsistent or unsupported sizes */
#define OMQ_E_DTYPE -3         /* unsupported dtype combination */
#define OMQ_E_ALIGN -4         /* row length or pointer alignment not supported */
#define OMQ_E_WORKSPACE -5     /* workspace NULL or smaller than the query says */
#define OMQ_E_HIP -6           /* a HIP call or kernel launch failed */
#define OMQ_E_UNIMPLEMENTED -7

/* element types */
#define OMQ_F32 0
#define OMQ_BF16 1

/* LET applied to the quantizer input x (section "LET" of the paper reading) */
#define OMQ_LET_NONE 0  /* x~ = x */
#define OMQ_LET_DIV 1   /* x~ = (x - delta) / s   (activation side; delta may be NULL = 0) */
#define OMQ_LET_MUL 2   /* x~ = s * x             (weight side, and K~ = s_a * K) */

/* optimizers */
#define OMQ_OPT_ADAMW 0
#define OMQ_OPT_SGD 1

/* compute path of a quantized linear layer */
#define OMQ_PATH_FP32 0  /* fp32 storage, fp32 GEMM */
#define OMQ_PATH_BF16 1  /* bf16 weights/activations, dequantized operands in bf16, fp32 accumulate */

/* Human-readable name of a status code (static string, never NULL). */
const char* omq_status_str(int status);
int omq_abi_version(void);

/*
 * omq_lwc_fakequant -- weight side of one linear layer (LWC + LET-W + bias fold).
 * Paper reading, section "LWC" (the LWC equation) and section "LET" (W~ = s (.) W,
 * B~ = B + delta W).  Per output channel o (row of W):
 *   W~_o = s (.) W_o                       (s NULL: W~ = W)
 *   M, m = max / min of W~_o (first index on ties) -> arg_max[o], arg_min[o]
 *   gamma = sigmoid(a_gamma[o]), beta = sigmoid(a_beta[o])
 *   h[o] = max((gamma M - beta m) / (2^N - 1), 1e-8);  z[o] = -rint(beta m / h)
 *   codes = clamp(rint(W~ / h) + z, 0, 2^N - 1);  W_hat = (codes - z) h
 *   B_tilde[o] = B[o] + sum_i delta_i W_oi  (original W; B, delta may be NULL = 0)
 * Group-wise LWC (the pages' g128 setting): with group = 128 each run of 128 input
 * channels of an output channel is its own quantizer row, with its own logits,
 * max/min, h and z; those arrays then hold c_out * c_in / 128 entries, index
 * o * (c_in / 128) + g, and arg_max / arg_min give the column within row o.
 * group 0 (or c_in) is per output channel; other values return OMQ_E_SHAPE, as
 * does group 128 when c_in is not a multiple of 128.
 * W: [c_out x c_in] of w_dt.  W_hat: [c_out x c_in] of what_dt (required).
 * h, z: float[rows] (required).  arg_max, arg_min: int32[rows] (required), rows
 * = c_out or c_out * c_in / 128.  a_gamma, a_beta: float[rows].
 * B_tilde: float[c_out] or NULL.  codes: uint8[c_out x c_in] or NULL.
 * n_bits 2..8.
 * nonfinite: int32 device flag or NULL; set to 1 when any element of W~ is NaN or
 * infinite (never cleared: the caller zeroes it).  A non-finite element never
 * wins the max / min comparisons, so such a row's h, z and codes are meaningless
 * (its arg_max / arg_min still name columns of the row); the other rows are
 * unaffected.
 */
int omq_lwc_fakequant(const void* W, int w_dt, int64_t c_out, int64_t c_in, int64_t group,
                      int n_bits,
                      const float* a_gamma, const float* a_beta, const float* s,
                      const float* delta, const float* B, void* W_hat, int what_dt, float* h,
                      float* z, int32_t* arg_max, int32_t* arg_min, float* B_tilde,
                      uint8_t* codes, int32_t* nonfinite, void* stream);

/*
 * omq_let_apply -- the LET transforms alone (paper reading, section "LET",
 * linear-layer equation), each group optional:
 *   activation side (X != NULL): X_tilde = (X - delta) / s, X [T x c_in] of x_dt,
 *     X_tilde [T x c_in] of xt_dt (delta NULL = 0);
 *   weight side (W != NULL): W_tilde = s (.) W, [c_out x c_in] of w_dt / wt_dt, and
 *     B_tilde = B + delta W (float[c_out], NULL to skip; B NULL = 0).
 * s: float[c_in] (required), delta: float[c_in] or NULL.
 */
int omq_let_apply(const void* X, int x_dt, int64_t T, int64_t c_in, const float* s,
                  const float* delta, void* X_tilde, int xt_dt, const void* W, int w_dt,
                  int64_t c_out, const float* B, void* W_tilde, int wt_dt, float* B_tilde,
                  void* stream);

/*
 * omq_act_quant -- per-token asymmetric MinMax fake quantization (gamma = beta = 1)
 * with an optional fused LET on its input.  Paper reading, section "实验证据"
 * (per-token activations) with the LWC equation's quantizer.  Per token t:
 *   x~ = LET(X_t) per let_mode (s, delta: float[C]);  M, m = max / min of x~
 *   h[t] = max((M - m) / (2^N - 1), 1e-8); z[t] = -rint(m / h)
 *   X_hat = (clamp(rint(x~ / h) + z, 0, 2^N - 1) - z) h
 * n_bits 2..8, or 16: X_hat = x~ and h, z, arg_max, arg_min are not written.
 * X: [T x C] of x_dt; X_hat: [T x C] of xh_dt; h, z: float[T]; arg_max,
 * arg_min: int32[T]; codes: uint8[T x C] or NULL.
 * nonfinite: int32 device flag or NULL; set to 1 when any element of x~ is NaN or
 * infinite (n_bits < 16 only; never cleared), as for omq_lwc_fakequant.
 */
int omq_act_quant(const void* X, int x_dt, int64_t T, int64_t C, int n_bits, int let_mode,
                  const float* s, const float* delta, void* X_hat, int xh_dt, float* h, float* z,
                  int32_t* arg_max, int32_t* arg_min, uint8_t* codes, int32_t* nonfinite,
                  void* stream);

/*
 * omq_gemm -- the quantized layer's contraction (paper reading, section "LET":
 * Y = Q_a(X~) Q_w(W~) + B~, and the two products of its backward):
 *   C[M x N] (float32) = alpha * op(A) * op(B)^T + bias[N]  (bias NULL = 0)
 * op(A) is [M x K]: A stored [M x K] row-major (trans_a = 0) or [K x M] (trans_a = 1);
 * op(B) is [N x K]: B stored [N x K] (trans_b = 0) or [K x N] (trans_b = 1).
 * A and B are both dt (OMQ_BF16 on the matrix cores with float32 accumulation,
 * or OMQ_F32); lda, ldb, ldc are leading dimensions in elements.
 * accumulate != 0 adds the result to C's current contents.
 * bf16: the contiguous extent of each operand and lda, ldb must be multiples of 8.
 */
int omq_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int trans_a,
             const void* B, int64_t ldb, int trans_b, int dt, const float* bias, float alpha,
             float* C, int64_t ldc, int accumulate, void* stream);

/*
 * omq_code_gemm -- the weight-activation quantized product on integer codes (paper
 * reading, section "LWC": a quantized value is (q - z) h with integer code q, step
 * h and zero point z per quantizer row; section "LET": Y = Q_a(X~) Q_w(W~)^T + B~):
 *   C[m, n] = h_a[m] h_b[n] sum_k (qa[m,k] - z_a[m]) (qb[n,k] - z_b[n]) + bias[n]
 * the same product as omq_gemm on the fake-quantized operands, computed exactly:
 * the matrix cores sum the int8 code products in int32, the zero points enter
 * through the rows' code sums, sum_k (qa - z_a)(qb - z_b) = S - z_b sum_a - z_a
 * sum_b + K z_a z_b, formed in double without rounding, and the result is rounded
 * once to float (before bias).
 * qa: uint8 [M x K], row stride lda; qb: uint8 [N x K], row stride ldb (codes below
 * 128, i.e. n_bits up to 7, as the codes output of omq_act_quant and
 * omq_lwc_fakequant with group 0).  h_a, z_a: float[M]; h_b, z_b: float[N] (z
 * integer-valued); sum_a: int32[M], sum_b: int32[N], the rows' code sums (see
 * omq_code_rowsum).  bias: float[N] or NULL.  C: float [M x N], row stride ldc,
 * overwritten.  K, lda, ldb multiples of 16, qa and qb 16-byte aligned
 * (OMQ_E_ALIGN), K at most 131072 (OMQ_E_SHAPE).
 */
int omq_code_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* qa, int64_t lda,
                  const float* h_a, const float* z_a, const int32_t* sum_a, const uint8_t* qb,
                  int64_t ldb, const float* h_b, const float* z_b, const int32_t* sum_b,
                  const float* bias, float* C, int64_t ldc, void* stream);

/*
 * omq_code_gemm4 -- omq_code_gemm on 4-bit codes (n_bits up to 4) stored two to a
 * byte, the packed form of omq_pack_codes with n_bits = 4: code k of a row in byte
 * k / 2, the low nibble for even k.  lda, ldb: row strides in bytes (at least K / 2,
 * multiples of 16); sum_a, sum_b as for omq_code_gemm (sums of the code values).
 * The same exact product and rounding; half the operand bytes through memory and
 * the local data share.  M, N and K multiples of 128 (OMQ_E_SHAPE), qa, qb 16-byte
 * aligned (OMQ_E_ALIGN).
 */
int omq_code_gemm4(int64_t M, int64_t N, int64_t K, const uint8_t* qa, int64_t lda,
                   const float* h_a, const float* z_a, const int32_t* sum_a, const uint8_t* qb,
                   int64_t ldb, const float* h_b, const float* z_b, const int32_t* sum_b,
                   const float* bias, float* C, int64_t ldc, void* stream);

/*
 * omq_attention_fwd -- the block's causal attention on its quantized operands
 * (paper reading, section "LET": the affinity of Q~ = Q / s_a and K~ = s_a K, and
 * the softmax output kept in full precision).  Per query head h, with KV head
 * g = h / (n_q / n_kv) (grouped-query attention):
 *   S = Q_h K_g^T / sqrt(head_dim) with the causal mask (key position <= query),
 *   P = softmax(S) in float32, O_h = P V_g with P rounded to bf16 as the matrix-core
 *   operand (the probabilities themselves are never quantized).
 * Q: bf16 [T x n_q*128], row stride ldq; K, V: bf16 [T x n_kv*128], row stride ldk
 * (e.g. the X_hat outputs of omq_act_quant for Q~, K~, V).  O: float [T x n_q*128],
 * row stride ldo.  lse2: float [n_q x T], the base-2 log-sum-exp of each query's
 * scaled scores, which omq_attention_bwd takes.  head_dim must be 128 (OMQ_E_SHAPE);
 * ldq, ldk multiples of 8 and ldo of 4, pointers 16-byte aligned (OMQ_E_ALIGN);
 * n_q a multiple of n_kv; T up to 2^30; T = 0 returns OMQ_OK at once.
 */
int omq_attention_fwd(const void* Q, int64_t ldq, const void* K, const void* V, int64_t ldk,
                      int64_t T, int64_t n_q, int64_t n_kv, int64_t head_dim, float* O,
                      int64_t ldo, float* lse2, void* stream);

/*
 * omq_attention_bwd -- backward of omq_attention_fwd given dO = dL/dO:
 *   dV_g = sum over the group's heads of P^T dO_h;  dP = dO_h V_g^T;
 *   dS = P (dP - rowsum(dO_h O_h)) / sqrt(head_dim);  dQ_h = dS K_g;
 *   dK_g = sum over the group's heads of dS^T Q_h
 * with the scores recomputed from lse2; dO, P and dS enter the matrix cores in
 * bf16, every sum is float32.  The dK/dV pass writes the bf16 dS it forms to the
 * workspace and dQ is formed from that same dS (the probabilities are never stored).
 * O, dO: float [T x n_q*128], row stride ldo; lse2 as the forward wrote it.
 * dQ: float [T x n_q*128], row stride lddq; dK, dV: float [T x n_kv*128], row
 * stride lddk (multiples of 4); all overwritten.  ws: device workspace of at least
 * omq_attention_bwd_workspace_size(T, n_q, ldq) bytes: dO in bf16, rowsum(dO O);
 * where the K/V heads are too few to occupy the device, float32 partial dK, dV of
 * query-head subsets, added in a fixed order (the size covers any n_kv dividing
 * n_q); and dS, n_q * Tp * Tp bf16 with Tp = T rounded up to 128 (268 MB at T 2048
 * with 32 heads).  The size is 0, and the call returns OMQ_E_SHAPE, when that dS
 * would exceed 2^50 elements.  The result is bitwise repeatable: no float atomics.
 */
size_t omq_attention_bwd_workspace_size(int64_t T, int64_t n_q, int64_t ldq);
int omq_attention_bwd(const void* Q, int64_t ldq, const void* K, const void* V, int64_t ldk,
                      int64_t T, int64_t n_q, int64_t n_kv, int64_t head_dim, const float* O,
                      const float* dO, int64_t ldo, const float* lse2, float* dQ, int64_t lddq,
                      float* dK, float* dV, int64_t lddk, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * omq_code_rowsum -- sums[r] = sum over c < cols of codes[r * ld + c] (int32), the
 * code sums omq_code_gemm takes.  codes: uint8, rows x cols with row stride ld.
 */
int omq_code_rowsum(const uint8_t* codes, int64_t rows, int64_t cols, int64_t ld, int32_t* sums,
                    void* stream);

/*
 * Deployment form of a calibrated layer (paper reading, section "LWC": the deployed
 * weight is the integer code q with step h and zero point z, W_hat = (q - z) h;
 * section "LET": after calibration the transformation is folded into the
 * neighbouring parameters, so the deployed block keeps its original operators).
 *
 * Packed codes: along each row, floor(32 / n_bits) codes per 32-bit word, code j
 * of a word in bits [j n_bits, (j+1) n_bits), lowest column first, unused high bits
 * zero; ceil(cols / per_word) words per row.
 *
 * omq_pack_codes -- codes: uint8 [rows x cols] (values < 2^n_bits, e.g. the codes
 * output of omq_lwc_fakequant); words: uint32 [rows x ceil(cols / per_word)].
 * n_bits 2..8.
 */
int omq_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int n_bits,
                   uint32_t* words, void* stream);

/*
 * omq_fold_linear -- weight-only (A16) fold of a calibrated linear's LET sites:
 *   bias_out[n] = B[n] - sum_k W_hat[n,k] delta[k] / s[k]      (input site: the
 *     layer then takes X / s, i.e. the normalization in front gets gain 1 / s)
 *   then, with s_o (the attention-output site folded into the value projection,
 *   per output row n of W_v): bias_out[n] = (bias_out[n] - delta_o[n]) / s_o[n] and
 *   h_out[n, g] = h[n, g] / s_o[n].
 * words: packed codes [N x K]; h, z: float[N] or float[N x K/128] (group 0 or 128);
 * B (the layer's B~ = B + delta W), s, delta, s_o, delta_o: float, each may be NULL
 * (B NULL = 0; delta NULL: no input-site term; s_o NULL: no value fold).
 * bias_out: float[N] (required); h_out: float like h (required when s_o is set);
 * gain_out: float[K] or NULL, receives the input site's gain 1 / s (needs s).
 */
int omq_fold_linear(const uint32_t* words, int n_bits, int64_t N, int64_t K, const float* h,
                    const float* z, int64_t group, const float* B, const float* s,
                    const float* delta, const float* s_o, const float* delta_o,
                    float* bias_out, float* h_out, float* gain_out, void* stream);

/*
 * omq_w4a16_gemm -- weight-only product on packed 4-bit codes:
 *   Y[T x N] = X[T x K] W_hat^T + bias,  W_hat[n, k] = bf16((q[n,k] - z) h)
 * with (h, z) per output row (group 0) or per 128-column group (group 128, index
 * n * K/128 + k/128); the dequantized value is the calibration's fake-quant weight.
 * X: bf16 [T x K] contiguous; words: uint32 [N x K/8]; bias: float[N] or NULL;
 * Y: float [T x N], overwritten.  K a multiple of 64 (and of 128 for group 128).
 * Built for small T: up to 8 tokens on the vector units (one wave per output row,
 * bf16-pair dot products), more on the matrix cores (the weight codes are re-read
 * for every 32 tokens).  Launches only kernels, so it can be captured in a graph.
 */
int omq_w4a16_gemm(const void* X, int64_t T, int64_t K, const uint32_t* words, int64_t N,
                   const float* h, const float* z, int64_t group, const float* bias, float* Y,
                   void* stream);

/*
 * omq_lwc_backward -- straight-through backward of omq_lwc_fakequant.
 * Only rint is straight-through (the LWC blog, section 2.2: the gradient bypasses
 * the rounding); clamp, max/min, h and z are differentiated exactly.  Per row o,
 * with g = gW_hat[o, :], u = W~/h, in = [0 <= rint(u) + z <= 2^N - 1]:
 *   g_h = sum g ((q - z) - in u),  g_z = -h sum g (1 - in)
 *   G = g_h + g_z beta m / h^2 (0 when the h floor is active)
 *   g_gamma = G M / Q,  g_beta = -(G / Q + g_z / h) m
 *   g_a_gamma = g_gamma gamma (1 - gamma), likewise beta
 *   gW~ = g in, plus G gamma / Q at arg_max and -(G / Q + g_z / h) beta at arg_min
 *   g_s[i] = sum_o gW~_oi W_oi      (if g_s != NULL; s may be NULL = 1)
 *   g_delta[i] = sum_o dy_colsum[o] W_oi   (the bias fold; if g_delta != NULL,
 *     dy_colsum: float[c_out] = sum over tokens of dL/dY)
 * group: as in omq_lwc_fakequant; with group 128 the sums above run over each
 * (row, group) and g_a_gamma, g_a_beta have one entry per (row, group).
 * gW_hat: float[c_out x c_in] (dL/dW_hat).  h, z, arg_max, arg_min: the forward's.
 * g_a_gamma, g_a_beta: float[rows] (required).  g_s, g_delta: float[c_in] or NULL.
 * ws: device workspace of at least omq_lwc_backward_workspace_size(c_out, c_in) bytes.
 */
size_t omq_lwc_backward_workspace_size(int64_t c_out, int64_t c_in);
int omq_lwc_backward(const float* gW_hat, const void* W, int w_dt, int64_t c_out, int64_t c_in,
                     int64_t group, int n_bits, const float* a_gamma, const float* a_beta, const float* s,
                     const float* h, const float* z, const int32_t* arg_max,
                     const int32_t* arg_min, const float* dy_colsum, float* g_a_gamma,
                     float* g_a_beta, float* g_s, float* g_delta, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * omq_act_quant_backward -- straight-through backward of omq_act_quant (the same
 * rule as omq_lwc_backward with gamma = beta = 1) chained through the fused LET:
 *   gx~ = g in + scatter at arg_max / arg_min
 *   OMQ_LET_DIV: gX = gx~ / s;  g_s += sum_t gx~ (-x~ / s);  g_delta = sum_t gx~ (-1 / s)
 *   OMQ_LET_MUL: gX = gx~ s;    g_s = sum_t gx~ X
 *   OMQ_LET_NONE: gX = gx~
 * gX_hat: float[T x C]; X, s, delta, let_mode, n_bits and h, z, arg_max, arg_min as
 * given to / returned by omq_act_quant (n_bits 16: gx~ = gX_hat).
 * gX: float[T x C] or NULL; g_s, g_delta: float[C] or NULL (written, not accumulated).
 * ws: at least omq_act_quant_backward_workspace_size(T, C) bytes.
 */
/*
 * omq_lwc_backward_noalloc -- omq_lwc_backward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without ws / ws_bytes, the same results.
 * The partial buffers live in a fixed device array of omq_noalloc_scratch_bytes()
 * (64 MiB) that each GPU the library runs on holds until the process ends; the
 * call allocates and frees nothing.  Shapes whose workspace query
 * (omq_lwc_backward_workspace_size) exceeds that size return OMQ_E_WORKSPACE
 * before any launch (every 7B-shaped weight, and the 70B-shaped q, k, v, o
 * weights, fit).  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (two streams, two threads) race and must be serialized by
 * the caller.  Nothing in the array needs clearing between calls.  The first call
 * on a device looks up the array's device address (an exception to "no global
 * mutable state": the per-device address is cached, under a lock).
 */
size_t omq_noalloc_scratch_bytes(void);
int omq_lwc_backward_noalloc(const float* gW_hat, const void* W, int w_dt, int64_t c_out,
                             int64_t c_in, int64_t group, int n_bits, const float* a_gamma,
                             const float* a_beta, const float* s, const float* h, const float* z,
                             const int32_t* arg_max, const int32_t* arg_min,
                             const float* dy_colsum, float* g_a_gamma, float* g_a_beta,
                             float* g_s, float* g_delta, void* stream);

size_t omq_act_quant_backward_workspace_size(int64_t T, int64_t C);
int omq_act_quant_backward(const float* gX_hat, int64_t T, int64_t C, const void* X, int x_dt,
                           int n_bits, int let_mode, const float* s, const float* delta,
                           const float* h, const float* z, const int32_t* arg_max,
                           const int32_t* arg_min, float* gX, float* g_s, float* g_delta,
                           void* ws, size_t ws_bytes, void* stream);

/* A quantized linear layer Y = Q_a(X~) Q_w(W~)^T + B~ (paper reading, section "LET"). */
typedef struct omq_qlinear_desc {
  size_t struct_size; /* sizeof(omq_qlinear_desc) */
  int64_t T, c_in, c_out;
  int wbits;   /* 2..8, or 16 = weight quantizer off */
  int abits;   /* 2..8, or 16 = activation quantizer off */
  int use_let; /* 1: theta carries s, delta (LET on this layer) */
  int path;    /* OMQ_PATH_FP32: X, W float32;  OMQ_PATH_BF16: X, W bf16 */
  int64_t group; /* LWC group along c_in: 0 = per output channel, or 128 */
} omq_qlinear_desc;

/*
 * theta / dtheta layout (float): a_gamma[rows], a_beta[rows] (rows = c_out, or
 * c_out * c_in / 128 with group 128, output-channel major), then when use_let
 * s[c_in], delta[c_in].  omq_qlinear_theta_size gives the element count.
 */
int64_t omq_qlinear_theta_size(const omq_qlinear_desc* d);
size_t omq_qlinear_workspace_size(const omq_qlinear_desc* d);

/*
 * omq_qlinear_fwd -- Y[T x c_out] (float32) = Q_a(X~) Q_w(W~)^T + B~.
 * X: [T x c_in], W: [c_out x c_in] (path dtype), B: float[c_out] or NULL.
 * The state the backward needs (dequantized operands, step sizes, indices) is
 * kept in ws, which must be passed unchanged to omq_qlinear_bwd.
 * c_in must be a multiple of 4, and on the bf16 path T, c_in and c_out multiples of
 * 8 (OMQ_E_ALIGN: the 16-byte operand rows of the matrix-core products); with
 * group 128, c_in a multiple of 128 (OMQ_E_SHAPE).
 */
int omq_qlinear_fwd(const omq_qlinear_desc* d, const void* X, const void* W, const float* B,
                    const float* theta, float* Y, void* ws, size_t ws_bytes, void* stream);

/*
 * omq_qlinear_bwd -- given dY = dL/dY (float[T x c_out]) after omq_qlinear_fwd with
 * the same arguments and ws: dtheta (theta layout) and dX = dL/dX (float[T x c_in],
 * NULL to skip).
 */
int omq_qlinear_bwd(const omq_qlinear_desc* d, const void* X, const void* W, const float* theta,
                    const float* dY, float* dX, float* dtheta, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * omq_sgd / omq_adamw -- parameter update over a packed float vector (paper reading,
 * section "实验证据": AdamW, zero weight decay, lr 5e-3 for LWC logits and 1e-2 for
 * LET parameters).  Elements [0, n_lwc) use lr_lwc, [n_lwc, n) use lr_let.
 * adamw: m, v float[n] moments (zero before step 1); step counts from 1;
 * theta -= lr * (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps) after
 * theta *= (1 - lr * weight_decay).
 */
int omq_sgd(float* theta, const float* grad, int64_t n, int64_t n_lwc, float lr_lwc,
            float lr_let, void* stream);
int omq_adamw(float* theta, const float* grad, float* m, float* v, int64_t n, int64_t n_lwc,
              float lr_lwc, float lr_let, float beta1, float beta2, float eps,
              float weight_decay, int64_t step, void* stream);

/*
 * Optional timing of a block step's launches (benchmarks).  The caller creates
 * 2 * capacity hipEvent_t handles in `events`; while count < capacity the library
 * records events[2*count] before and events[2*count+1] after each timed launch it
 * issues on the call's stream and increments count.  Timed launches: every GEMM
 * (its algorithmic FLOPs, 2 M N K per batch entry, are added to flops), and the
 * quantized forward's fake quantizers (weights and activations).
 * kinds (int[capacity] or NULL) receives each launch's kind (OMQ_TIMED_*), work
 * (double[capacity] or NULL) its algorithmic work: FLOPs for the GEMMs, HBM bytes
 * for the quantizers (read x, write x_hat, and the codes when written).
 * flops_codes sums the int8 code products' share of flops.
 */
#define OMQ_TIMED_GEMM 0          /* bf16 (or float32) operands */
#define OMQ_TIMED_GEMM_I8 1       /* int8 codes (the forward's products, omq_code_gemm) */
#define OMQ_TIMED_WEIGHT_QUANT 2  /* LWC fake quantizer of a weight */
#define OMQ_TIMED_ACT_QUANT 3     /* per-token activation quantizer */
typedef struct omq_timer {
  void** events;
  int capacity;
  int count;
  double flops;
  int* kinds;
  double flops_codes;
  double* work;
} omq_timer;

/*
 * A LLaMA-shaped decoder block (or its FFN alone): RMSNorm (unit gain) -> q/k/v ->
 * RoPE (rotate-half) -> s_a on Q/K -> causal scaled attention with float32
 * softmax -> o -> residual -> RMSNorm -> SiLU(gate) * up -> down -> residual.
 * LET sites (paper reading, section "LET"): (s_qkv, delta_qkv) on the q/k/v input,
 * (s_o, delta_o) on the o input (per KV channel, broadcast over the query heads of
 * a group), (s_ffn, delta_ffn) on the gate/up input, none on down; s_a per KV
 * channel on the post-RoPE Q (divided) and K (multiplied), learned only when
 * abits < 16.  Q~, K~, V and every linear input are quantized per token at abits;
 * softmax is never quantized.  ffn_only: y = down(SiLU(gate(x~)) * up(x~)) with the
 * ffn LET site, no norm and no residual.
 * With both quantizers on, the forward's four quantized products are formed exactly
 * on the integer codes (h_x h_w sum (q_x - z_x)(q_w - z_w), rounded once to float).
 * Limits (checked by every block entry point; omq_block_workspace_size returns 0):
 * head_dim must be 128 and n_q a multiple of n_kv (OMQ_E_SHAPE), and the attention
 * backward's dS (n_q * Tp * Tp bf16, Tp = T rounded up to 128) at most 2^50 elements
 * (OMQ_E_SHAPE); T, d, F multiples of 8 (OMQ_E_ALIGN); group 128 needs d and F multiples of 128 (OMQ_E_SHAPE); group
 * 128 with abits < 16 and wbits < 16 (group-wise clipping with quantized
 * activations) is not implemented (OMQ_E_UNIMPLEMENTED).
 */
typedef struct omq_block_desc {
  size_t struct_size; /* sizeof(omq_block_desc) */
  int64_t T, d, n_q, n_kv, head_dim, F;
  int wbits, abits;   /* 2..8 / 16 */
  int ffn_only;
  float eps;          /* RMSNorm epsilon */
  float rope_theta;
  int optimizer;      /* OMQ_OPT_ADAMW or OMQ_OPT_SGD */
  float lr_lwc, lr_let;
  float beta1, beta2, adam_eps, weight_decay;
  omq_timer* timer;   /* NULL, or per-launch GEMM timing (host struct, caller-owned) */
  int64_t group;      /* LWC group along C_in: 0 = per output channel, or 128 (every
                         C_in of the block a multiple of 128) */
  int32_t* nonfinite; /* NULL, or an int32 device flag that every quantizer of the
                         quantized forward sets to 1 when its input holds a NaN or an
                         infinity (never cleared by the library) */
} omq_block_desc;

/*
 * Packed theta order: for each linear of (q, k, v, o, gate, up, down) (ffn_only:
 * gate, up, down) a_gamma[R] then a_beta[R] with R = C_out, or C_out * C_in / 128
 * for group 128 (output-channel major); then for each LET site of
 * (qkv, o, ffn) (ffn_only: ffn) s[C] then delta[C] (C = d, n_kv*head_dim, d);
 * then s_a[n_kv*head_dim] when abits < 16 and not ffn_only.
 * offsets: int64[2*n_linears + 2*n_sites + 1] host array or NULL; *total: count.
 * *n_lwc: number of leading LWC logits (or NULL).
 */
int omq_block_theta_layout(const omq_block_desc* d, int64_t* offsets, int64_t* n_entries,
                           int64_t* n_lwc, int64_t* total);
size_t omq_block_workspace_size(const omq_block_desc* d);

/*
 * omq_block_forward -- y[T x d] (float32) of the block.  x: bf16 [T x d];
 * weights: host array of 7 device pointers (q, k, v, o, gate, up, down; bf16,
 * [C_out x C_in]; ffn_only: the first four may be NULL).  theta == NULL runs the
 * full-precision block (no quantizers, no LET): the calibration target.
 */
int omq_block_forward(const omq_block_desc* d, const void* x, const void* const* weights,
                      const float* theta, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * omq_block_step -- one calibration step (paper reading, section "框架"): quantized
 * forward, L = mean((y - y_target)^2) over T x d, straight-through backward into
 * dtheta (theta layout), and the optimizer update of theta (and m, v for AdamW,
 * float[total], zero before step 1; step counts from 1).  loss: float device
 * scalar (the loss before the update), or NULL.  y_target: float32 [T x d].
 */
int omq_block_step(const omq_block_desc* d, const void* x, const float* y_target,
                   const void* const* weights, float* theta, float* dtheta, float* adam_m,
                   float* adam_v, int64_t step, float* loss, void* ws, size_t ws_bytes,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OMQ_H_ */
