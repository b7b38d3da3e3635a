// C ABI of the OmniQuant calibration hot path: argument validation, workspace
// layout, and the composition of kernels into the layer-level operations.
#include "api_util.h"

#include <math.h>

using namespace omq;

extern "C" {

const char* omq_status_str(int status) {
  switch (status) {
    case OMQ_OK: return "ok";
    case OMQ_E_INVALID_ARG: return "invalid argument";
    case OMQ_E_SHAPE: return "inconsistent or unsupported shape";
    case OMQ_E_DTYPE: return "unsupported dtype";
    case OMQ_E_ALIGN: return "unsupported row length or pointer alignment";
    case OMQ_E_WORKSPACE: return "workspace missing or too small";
    case OMQ_E_HIP: return "HIP launch failed";
    case OMQ_E_UNIMPLEMENTED: return "not implemented";
    default: return "unknown status";
  }
}

int omq_abi_version(void) { return OMQ_ABI_VERSION; }

}  // extern "C"

namespace {
// LWC grouping: 0 or c_in -> 0 (per output channel); 128 with c_in % 128 == 0 -> 128;
// anything else -> -1 (unsupported)
int64_t lwc_group(int64_t group, int64_t c_in) {
  if (group == 0 || group == c_in) return 0;
  if (group == 128 && c_in % 128 == 0) return 128;
  return -1;
}
// LWC quantizer rows of a qlinear layer: output channels, or (channel, group) pairs
int64_t qlin_rows(const omq_qlinear_desc* d) {
  return lwc_group(d->group, d->c_in) > 0 ? d->c_out * (d->c_in / 128) : d->c_out;
}
}  // namespace

extern "C" {


int omq_lwc_fakequant(const void* W, int w_dt, int64_t c_out, int64_t c_in, int64_t group,
                      int n_bits, const float* a_gamma, const float* a_beta, const float* s,
                      const float* delta, const float* B, void* W_hat, int what_dt, float* h,
                      float* z, int32_t* arg_max, int32_t* arg_min, float* B_tilde,
                      uint8_t* codes, int32_t* nonfinite, void* stream) {
  if (c_out == 0) return OMQ_OK;                   // no rows: nothing read or written
  if (!W || !a_gamma || !a_beta || !W_hat || !h || !z || !arg_max || !arg_min)
    return OMQ_E_INVALID_ARG;
  if (n_bits < 2 || n_bits > 8) return OMQ_E_INVALID_ARG;
  if (!dt_ok(w_dt) || !dt_ok(what_dt)) return OMQ_E_DTYPE;
  if (c_out < 0 || c_in <= 0) return OMQ_E_SHAPE;
  if (c_in % 4) return OMQ_E_ALIGN;
  const int64_t grp = lwc_group(group, c_in);
  if (grp < 0) return OMQ_E_SHAPE;
  if (!al16(W) || !al16(W_hat) || !al16(s) || !al16(delta) || !al4(codes) || !al4(nonfinite))
    return OMQ_E_ALIGN;
  RowQuantFwd a;
  a.x = W; a.x_dt = w_dt; a.rows = c_out; a.cols = c_in; a.ldx = c_in;
  a.let_mode = s ? OMQ_LET_MUL : OMQ_LET_NONE; a.s = s;
  a.nbits = n_bits; a.a_gamma = a_gamma; a.a_beta = a_beta;
  a.out = W_hat; a.out_dt = what_dt; a.ldo = c_in;
  a.h = h; a.z = z; a.amax = arg_max; a.amin = arg_min; a.codes = codes;
  a.fold_delta = delta; a.bias = B; a.bias_out = B_tilde;
  a.group = grp; a.nonfinite = nonfinite;
  if (B_tilde && !delta) {
    // no shift: B~ = B
    if (B) OMQ_HIP_CHECK(hipMemcpyAsync(B_tilde, B, c_out * 4, hipMemcpyDeviceToDevice, S(stream)));
    else OMQ_HIP_CHECK(launch_fill_f32(B_tilde, c_out, 0.f, S(stream)));
    a.bias_out = nullptr;
  }
  if (grp) {
    // grouped rows: the bias fold runs over whole output channels on its own
    a.fold_delta = nullptr; a.bias_out = nullptr;
    if (B_tilde && delta)
      OMQ_HIP_CHECK(launch_bias_fold(W, w_dt, c_out, c_in, delta, B, B_tilde, S(stream)));
  }
  OMQ_HIP_CHECK(launch_rowquant_fwd(a, S(stream)));
  return OMQ_OK;
}

int omq_let_apply(const void* X, int x_dt, int64_t T, int64_t c_in, const float* s,
                  const float* delta, void* X_tilde, int xt_dt, const void* W, int w_dt,
                  int64_t c_out, const float* B, void* W_tilde, int wt_dt, float* B_tilde,
                  void* stream) {
  if (!s) return OMQ_E_INVALID_ARG;
  if (c_in <= 0) return OMQ_E_SHAPE;
  if (c_in % 4) return OMQ_E_ALIGN;
  if (X) {
    if (!X_tilde) return OMQ_E_INVALID_ARG;
    if (!dt_ok(x_dt) || !dt_ok(xt_dt)) return OMQ_E_DTYPE;
    if (T < 0) return OMQ_E_SHAPE;
    if (!al16(X) || !al16(X_tilde)) return OMQ_E_ALIGN;
  }
  if (W) {
    if (!W_tilde && !B_tilde) return OMQ_E_INVALID_ARG;
    if (!dt_ok(w_dt) || (W_tilde && !dt_ok(wt_dt))) return OMQ_E_DTYPE;
    if (c_out < 0) return OMQ_E_SHAPE;
    if (!al16(W) || !al16(W_tilde)) return OMQ_E_ALIGN;
  }
  if (X)
    OMQ_HIP_CHECK(launch_let_elementwise(X, x_dt, T, c_in, OMQ_LET_DIV, s, delta, X_tilde, xt_dt,
                                         S(stream)));
  if (W && W_tilde)
    OMQ_HIP_CHECK(launch_let_elementwise(W, w_dt, c_out, c_in, OMQ_LET_MUL, s, nullptr, W_tilde,
                                         wt_dt, S(stream)));
  if (W && B_tilde) {
    if (delta)
      OMQ_HIP_CHECK(launch_bias_fold(W, w_dt, c_out, c_in, delta, B, B_tilde, S(stream)));
    else if (B)
      OMQ_HIP_CHECK(hipMemcpyAsync(B_tilde, B, c_out * 4, hipMemcpyDeviceToDevice, S(stream)));
    else
      OMQ_HIP_CHECK(launch_fill_f32(B_tilde, c_out, 0.f, S(stream)));
  }
  return OMQ_OK;
}

int omq_act_quant(const void* X, int x_dt, int64_t T, int64_t C, int n_bits, int let_mode,
                  const float* s, const float* delta, void* X_hat, int xh_dt, float* h, float* z,
                  int32_t* arg_max, int32_t* arg_min, uint8_t* codes, int32_t* nonfinite,
                  void* stream) {
  if (T == 0) return OMQ_OK;                       // no rows: nothing read or written
  if (!X || !X_hat) return OMQ_E_INVALID_ARG;
  if (!bits_ok(n_bits)) return OMQ_E_INVALID_ARG;
  if (n_bits < 16 && (!h || !z || !arg_max || !arg_min)) return OMQ_E_INVALID_ARG;
  if (let_mode < 0 || let_mode > 2 || (let_mode != OMQ_LET_NONE && !s)) return OMQ_E_INVALID_ARG;
  if (!dt_ok(x_dt) || !dt_ok(xh_dt)) return OMQ_E_DTYPE;
  if (T < 0 || C <= 0) return OMQ_E_SHAPE;
  if (C % 4) return OMQ_E_ALIGN;
  if (!al16(X) || !al16(X_hat) || !al4(codes) || !al16(s) || !al16(delta) || !al4(nonfinite))
    return OMQ_E_ALIGN;
  RowQuantFwd a;
  a.x = X; a.x_dt = x_dt; a.rows = T; a.cols = C; a.ldx = C;
  a.let_mode = let_mode; a.s = s; a.delta = delta; a.nbits = n_bits;
  a.out = X_hat; a.out_dt = xh_dt; a.ldo = C;
  a.h = h; a.z = z; a.amax = arg_max; a.amin = arg_min; a.codes = codes;
  a.nonfinite = nonfinite;
  OMQ_HIP_CHECK(launch_rowquant_fwd(a, S(stream)));
  return OMQ_OK;
}

int omq_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int trans_a,
             const void* B, int64_t ldb, int trans_b, int dt, const float* bias, float alpha,
             float* C, int64_t ldc, int accumulate, void* stream) {
  if (M == 0 || N == 0) return OMQ_OK;             // empty C: nothing read or written
  if (!A || !B || !C) return OMQ_E_INVALID_ARG;
  if (!dt_ok(dt)) return OMQ_E_DTYPE;
  if (M < 0 || N < 0 || K < 0 || ldc < N) return OMQ_E_SHAPE;
  if (lda < (trans_a ? M : K) || ldb < (trans_b ? N : K)) return OMQ_E_SHAPE;
  if (dt == OMQ_BF16 && ((trans_a ? M : K) % 8 || (trans_b ? N : K) % 8 || lda % 8 ||
                         ldb % 8 || !al16(A) || !al16(B)))
    return OMQ_E_ALIGN;
  Gemm g;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc; g.bias = bias;
  g.M = M; g.N = N; g.K = K; g.alpha = alpha; g.accumulate = accumulate; g.dt = dt;
  g.ta = trans_a != 0; g.tb = trans_b != 0;
  OMQ_HIP_CHECK(launch_gemm(g, S(stream)));
  return OMQ_OK;
}

int omq_code_rowsum(const uint8_t* codes, int64_t rows, int64_t cols, int64_t ld, int32_t* sums,
                    void* stream) {
  if (!codes || !sums) return OMQ_E_INVALID_ARG;
  if (rows < 0 || cols < 0 || ld < cols) return OMQ_E_SHAPE;
  OMQ_HIP_CHECK(launch_code_rowsum(codes, rows, cols, ld, sums, S(stream)));
  return OMQ_OK;
}

int omq_code_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* qa, int64_t lda,
                  const float* h_a, const float* z_a, const int32_t* sum_a, const uint8_t* qb,
                  int64_t ldb, const float* h_b, const float* z_b, const int32_t* sum_b,
                  const float* bias, float* C, int64_t ldc, void* stream) {
  if (M == 0 || N == 0) return OMQ_OK;             // empty C: nothing read or written
  if (!qa || !qb || !C || !h_a || !z_a || !sum_a || !h_b || !z_b || !sum_b)
    return OMQ_E_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0 || ldc < N || lda < K || ldb < K || K > (1 << 17))
    return OMQ_E_SHAPE;
  if (K % 16 || lda % 16 || ldb % 16 || !al16(qa) || !al16(qb)) return OMQ_E_ALIGN;
  if (M == 0 || N == 0) return OMQ_OK;
  Gemm g;
  g.codes = 1;
  g.A = qa; g.lda = lda; g.B = qb; g.ldb = ldb; g.C = C; g.ldc = ldc; g.bias = bias;
  g.M = M; g.N = N; g.K = K;
  g.ha = h_a; g.za = z_a; g.sa = sum_a; g.hb = h_b; g.zb = z_b; g.sb = sum_b;
  OMQ_HIP_CHECK(launch_gemm(g, S(stream)));
  return OMQ_OK;
}

int omq_code_gemm4(int64_t M, int64_t N, int64_t K, const uint8_t* qa, int64_t lda,
                   const float* h_a, const float* z_a, const int32_t* sum_a, const uint8_t* qb,
                   int64_t ldb, const float* h_b, const float* z_b, const int32_t* sum_b,
                   const float* bias, float* C, int64_t ldc, void* stream) {
  if (M == 0 || N == 0) return OMQ_OK;             // empty C: nothing read or written
  if (!qa || !qb || !C || !h_a || !z_a || !sum_a || !h_b || !z_b || !sum_b)
    return OMQ_E_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0 || ldc < N || 2 * lda < K || 2 * ldb < K || K > (1 << 17) ||
      M % 128 || N % 128 || K % 128)
    return OMQ_E_SHAPE;
  if (lda % 16 || ldb % 16 || !al16(qa) || !al16(qb)) return OMQ_E_ALIGN;
  Gemm g;
  g.codes = 1;
  g.pack4 = 1;
  g.A = qa; g.lda = lda; g.B = qb; g.ldb = ldb; g.C = C; g.ldc = ldc; g.bias = bias;
  g.M = M; g.N = N; g.K = K;
  g.ha = h_a; g.za = z_a; g.sa = sum_a; g.hb = h_b; g.zb = z_b; g.sb = sum_b;
  OMQ_HIP_CHECK(launch_gemm(g, S(stream)));
  return OMQ_OK;
}

// ---------------------------------------------------------------------------
// causal attention of the block on its quantized operands
// ---------------------------------------------------------------------------

namespace {
int attn_check(const void* Q, int64_t ldq, const void* K, const void* V, int64_t ldk, int64_t T,
               int64_t n_q, int64_t n_kv, int64_t head_dim, const void* O, int64_t ldo) {
  if (!Q || !K || !V || !O) return OMQ_E_INVALID_ARG;
  if (T < 0 || T > ((int64_t)1 << 30) || n_q <= 0 || n_kv <= 0 || n_q % n_kv) return OMQ_E_SHAPE;
  if (head_dim != 128) return OMQ_E_SHAPE;
  if (ldq < n_q * 128 || ldk < n_kv * 128 || ldo < n_q * 128) return OMQ_E_SHAPE;
  if (ldq % 8 || ldk % 8 || ldo % 4 || !al16(Q) || !al16(K) || !al16(V) || !al16(O))
    return OMQ_E_ALIGN;
  return OMQ_OK;
}
}  // namespace

int omq_attention_fwd(const void* Q, int64_t ldq, const void* K, const void* V, int64_t ldk,
                      int64_t T, int64_t n_q, int64_t n_kv, int64_t head_dim, float* O,
                      int64_t ldo, float* lse2, void* stream) {
  int rc = attn_check(Q, ldq, K, V, ldk, T, n_q, n_kv, head_dim, O, ldo);
  if (rc) return rc;
  if (!lse2) return OMQ_E_INVALID_ARG;
  if (T == 0) return OMQ_OK;
  FlashFwd f;
  f.Q = reinterpret_cast<const uint16_t*>(Q);
  f.K = reinterpret_cast<const uint16_t*>(K);
  f.V = reinterpret_cast<const uint16_t*>(V);
  f.ldq = ldq; f.ldk = ldk; f.T = T; f.n_q = (int)n_q; f.grp = (int)(n_q / n_kv);
  f.scale2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  f.O = O; f.ldo = ldo; f.lse2 = lse2;
  OMQ_HIP_CHECK(launch_flash_fwd(f, S(stream)));
  return OMQ_OK;
}

size_t omq_attention_bwd_workspace_size(int64_t T, int64_t n_q, int64_t ldq) {
  if (T < 0 || n_q < 0 || ldq < 0) return 0;
  Bump b(nullptr);
  b.take<float>(n_q * T);       // D = rowsum(dO * O) per (head, query)
  b.take<uint16_t>(T * ldq);    // dO in bf16, rows like Q's
  // partial dK, dV of the query-head splits, for the largest need of any n_kv
  // dividing n_q (the divisors in pairs i, n_q / i)
  if (n_q > (int64_t)1 << 30) return 0;
  int64_t part = 0;
  for (int64_t i = 1; i * i <= n_q; ++i)
    if (n_q % i == 0) {
      part = std::max(part, flash_bwd_part_floats(T, (int)n_q, (int)i));
      part = std::max(part, flash_bwd_part_floats(T, (int)n_q, (int)(n_q / i)));
    }
  b.take<float>(part);
  // bf16 dS of every head, [Tp][Tp] each (Tp = T rounded up to 128)
  const int64_t ds = flash_bwd_ds_elems(T, n_q);
  if (ds < 0) return 0;
  b.take<uint16_t>(ds);
  return b.off;
}

int omq_attention_bwd(const void* Q, int64_t ldq, const void* K, const void* V, int64_t ldk,
                      int64_t T, int64_t n_q, int64_t n_kv, int64_t head_dim, const float* O,
                      const float* dO, int64_t ldo, const float* lse2, float* dQ, int64_t lddq,
                      float* dK, float* dV, int64_t lddk, void* ws, size_t ws_bytes,
                      void* stream) {
  int rc = attn_check(Q, ldq, K, V, ldk, T, n_q, n_kv, head_dim, O, ldo);
  if (rc) return rc;
  if (!dO || !lse2 || !dQ || !dK || !dV) return OMQ_E_INVALID_ARG;
  if (lddq < n_q * 128 || lddk < n_kv * 128) return OMQ_E_SHAPE;
  if (lddq % 4 || lddk % 4 || !al16(dO) || !al16(dQ) || !al16(dK) || !al16(dV))
    return OMQ_E_ALIGN;
  if (T == 0) return OMQ_OK;
  const size_t need = omq_attention_bwd_workspace_size(T, n_q, ldq);
  if (need == 0) return OMQ_E_SHAPE;
  if (!ws || ws_bytes < need) return OMQ_E_WORKSPACE;
  Bump b(ws);
  float* D = b.take<float>(n_q * T);
  uint16_t* dOb = b.take<uint16_t>(T * ldq);
  float* part = b.take<float>(flash_bwd_part_floats(T, (int)n_q, (int)n_kv));
  uint16_t* ds = b.take<uint16_t>(flash_bwd_ds_elems(T, n_q));
  const hipStream_t st = S(stream);
  OMQ_HIP_CHECK(launch_attn_bwd_prep(dO, O, ldo, T, (int)n_q, D, dOb, ldq, st));
  FlashBwd f;
  f.Q = reinterpret_cast<const uint16_t*>(Q);
  f.K = reinterpret_cast<const uint16_t*>(K);
  f.V = reinterpret_cast<const uint16_t*>(V);
  f.dO = dOb; f.ldq = ldq; f.ldk = ldk; f.T = T; f.n_q = (int)n_q; f.grp = (int)(n_q / n_kv);
  f.scale = (float)(1.0 / sqrt((double)head_dim));
  f.scale2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
  f.lse2 = lse2; f.D = D;
  f.dQ = dQ; f.lddq = lddq; f.dK = dK; f.dV = dV; f.lddk = lddk; f.part = part; f.ds = ds;
  OMQ_HIP_CHECK(launch_flash_bwd(f, st));
  return OMQ_OK;
}

size_t omq_lwc_backward_workspace_size(int64_t c_out, int64_t c_in) {
  return rowquant_bwd_ws_bytes(c_out, c_in);
}

int omq_lwc_backward(const float* gW_hat, const void* W, int w_dt, int64_t c_out, int64_t c_in,
                     int64_t group, int n_bits, const float* a_gamma, const float* a_beta,
                     const float* s,
                     const float* h, const float* z, const int32_t* arg_max,
                     const int32_t* arg_min, const float* dy_colsum, float* g_a_gamma,
                     float* g_a_beta, float* g_s, float* g_delta, void* ws, size_t ws_bytes,
                     void* stream) {
  if (!gW_hat || !W || !a_gamma || !a_beta || !h || !z || !arg_max || !arg_min || !g_a_gamma ||
      !g_a_beta)
    return OMQ_E_INVALID_ARG;
  if (g_delta && !dy_colsum) return OMQ_E_INVALID_ARG;
  if (n_bits < 2 || n_bits > 8) return OMQ_E_INVALID_ARG;
  if (!dt_ok(w_dt)) return OMQ_E_DTYPE;
  if (c_out < 0 || c_in <= 0) return OMQ_E_SHAPE;
  if (c_in % 4) return OMQ_E_ALIGN;
  const int64_t grp = lwc_group(group, c_in);
  if (grp < 0) return OMQ_E_SHAPE;
  if (!al16(gW_hat) || !al16(W) || !al16(s) || !al16(dy_colsum)) return OMQ_E_ALIGN;
  if (!ws || ws_bytes < omq_lwc_backward_workspace_size(c_out, c_in)) return OMQ_E_WORKSPACE;
  RowQuantBwd a;
  a.g = gW_hat; a.ldg = c_in; a.x = W; a.x_dt = w_dt; a.rows = c_out; a.cols = c_in;
  a.ldx = c_in; a.let_mode = s ? OMQ_LET_MUL : OMQ_LET_NONE; a.s = s; a.nbits = n_bits;
  a.h = h; a.z = z; a.amax = arg_max; a.amin = arg_min; a.a_gamma = a_gamma; a.a_beta = a_beta;
  a.col_mode = (g_s || g_delta) ? COL_WEIGHT : COL_NONE;
  a.rowvec = dy_colsum; a.g_agamma = g_a_gamma; a.g_abeta = g_a_beta;
  a.out0 = g_s; a.out1 = g_delta; a.ws = reinterpret_cast<float*>(ws);
  a.group = grp;
  OMQ_HIP_CHECK(launch_rowquant_bwd(a, S(stream)));
  return OMQ_OK;
}

size_t omq_act_quant_backward_workspace_size(int64_t T, int64_t C) {
  return rowquant_bwd_ws_bytes(T, C);
}

int omq_act_quant_backward(const float* gX_hat, int64_t T, int64_t C, const void* X, int x_dt,
                           int n_bits, int let_mode, const float* s, const float* delta,
                           const float* h, const float* z, const int32_t* arg_max,
                           const int32_t* arg_min, float* gX, float* g_s, float* g_delta,
                           void* ws, size_t ws_bytes, void* stream) {
  if (!gX_hat || !X) return OMQ_E_INVALID_ARG;
  if (!bits_ok(n_bits)) return OMQ_E_INVALID_ARG;
  if (n_bits < 16 && (!h || !z || !arg_max || !arg_min)) return OMQ_E_INVALID_ARG;
  if (let_mode < 0 || let_mode > 2 || (let_mode != OMQ_LET_NONE && !s)) return OMQ_E_INVALID_ARG;
  if ((g_s || g_delta) && let_mode == OMQ_LET_NONE) return OMQ_E_INVALID_ARG;
  if (g_delta && let_mode != OMQ_LET_DIV) return OMQ_E_INVALID_ARG;
  if (!dt_ok(x_dt)) return OMQ_E_DTYPE;
  if (T < 0 || C <= 0) return OMQ_E_SHAPE;
  if (C % 4) return OMQ_E_ALIGN;
  if (!al16(gX_hat) || !al16(X) || !al16(gX) || !al16(s) || !al16(delta)) return OMQ_E_ALIGN;
  if (!ws || ws_bytes < omq_act_quant_backward_workspace_size(T, C)) return OMQ_E_WORKSPACE;
  RowQuantBwd a;
  a.g = gX_hat; a.ldg = C; a.x = X; a.x_dt = x_dt; a.rows = T; a.cols = C; a.ldx = C;
  a.let_mode = let_mode; a.s = s; a.delta = delta; a.nbits = n_bits;
  a.h = h; a.z = z; a.amax = arg_max; a.amin = arg_min;
  a.col_mode = (g_s || g_delta) ? (let_mode == OMQ_LET_DIV ? COL_ACT_DIV : COL_ACT_MUL) : COL_NONE;
  a.gx = gX; a.ldgx = C; a.out0 = g_s; a.out1 = g_delta;
  a.ws = reinterpret_cast<float*>(ws);
  OMQ_HIP_CHECK(launch_rowquant_bwd(a, S(stream)));
  return OMQ_OK;
}

// ---------------------------------------------------------------------------
// quantized linear layer
// ---------------------------------------------------------------------------

int64_t omq_qlinear_theta_size(const omq_qlinear_desc* d) {
  if (!d || lwc_group(d->group, d->c_in) < 0) return -1;
  return 2 * qlin_rows(d) + (d->use_let ? 2 * d->c_in : 0);
}

namespace {

struct QLinWs {
  void* What; float *wh, *wz; int32_t *wamax, *wamin; float* Bt;
  void* Xhat; float *ah, *az; int32_t *aamax, *aamin;
  // the forward product on integer codes (bf16 path, both sides quantized per row):
  // code rows padded with zero codes to cip columns, and the rows' code sums
  uint8_t *Wq, *Xq; int32_t *wqs, *aqs; int64_t cip;
  float *gW, *gXh, *colsum;
  uint16_t* dYb;
  float *rq, *cs;
  size_t total;
};

// whether the forward product runs exactly on the integer codes: the bf16 path with
// both quantizers on, per output channel (8-bit codes stored shifted by 128)
bool qlin_codes(const omq_qlinear_desc* d) {
  return d->path == OMQ_PATH_BF16 && d->wbits <= 8 && d->abits <= 8 &&
         lwc_group(d->group, d->c_in) == 0;
}

QLinWs qlin_layout(const omq_qlinear_desc* d, void* base) {
  Bump b(base);
  QLinWs w;
  const bool bf = d->path == OMQ_PATH_BF16;
  const size_t es = bf ? 2 : 4;
  const int64_t T = d->T, ci = d->c_in, co = d->c_out;
  w.What = b.take<char>(co * ci * es);
  const int64_t rq = qlin_rows(d);
  w.wh = b.take<float>(rq); w.wz = b.take<float>(rq);
  w.wamax = b.take<int32_t>(rq); w.wamin = b.take<int32_t>(rq);
  w.Bt = b.take<float>(co);
  w.Xhat = b.take<char>(T * ci * es);
  w.ah = b.take<float>(T); w.az = b.take<float>(T);
  w.aamax = b.take<int32_t>(T); w.aamin = b.take<int32_t>(T);
  w.gW = b.take<float>(co * ci);
  w.gXh = b.take<float>(T * ci);
  w.colsum = b.take<float>(co);
  w.dYb = bf ? b.take<uint16_t>(T * co) : nullptr;
  w.cip = (ci + 15) / 16 * 16;
  w.Wq = w.Xq = nullptr; w.wqs = w.aqs = nullptr;
  if (qlin_codes(d)) {
    w.Wq = b.take<uint8_t>(co * w.cip); w.Xq = b.take<uint8_t>(T * w.cip);
    w.wqs = b.take<int32_t>(co); w.aqs = b.take<int32_t>(T);
  }
  int64_t n1, t1, n2, t2;
  gemm_ste_extents(co, ci, &n1, &t1);
  gemm_ste_extents(T, ci, &n2, &t2);
  w.rq = b.take<float>(std::max({rowquant_bwd_ws_bytes(co, ci) / 4, rowquant_bwd_ws_bytes(T, ci) / 4,
                                 ste_partials_floats(co, ci, n1, t1),
                                 ste_partials_floats(T, ci, n2, t2)}));
  w.cs = b.take<float>(colsum_ws_bytes(T, co) / 4);
  w.total = b.off;
  return w;
}

int qlin_check(const omq_qlinear_desc* d) {
  if (!d || d->struct_size < sizeof(omq_qlinear_desc)) return OMQ_E_INVALID_ARG;
  if (!bits_ok(d->wbits) || !bits_ok(d->abits)) return OMQ_E_INVALID_ARG;
  if (d->path != OMQ_PATH_FP32 && d->path != OMQ_PATH_BF16) return OMQ_E_INVALID_ARG;
  if (d->T < 0 || d->c_in <= 0 || d->c_out <= 0) return OMQ_E_SHAPE;
  if (d->c_in % 4) return OMQ_E_ALIGN;
  if (d->path == OMQ_PATH_BF16 && (d->T % 8 || d->c_in % 8 || d->c_out % 8)) return OMQ_E_ALIGN;
  if (lwc_group(d->group, d->c_in) < 0) return OMQ_E_SHAPE;
  return OMQ_OK;
}

}  // namespace

size_t omq_qlinear_workspace_size(const omq_qlinear_desc* d) {
  if (qlin_check(d) != OMQ_OK) return 0;
  return qlin_layout(d, nullptr).total;
}

int omq_qlinear_fwd(const omq_qlinear_desc* d, const void* X, const void* W, const float* B,
                    const float* theta, float* Y, void* ws, size_t ws_bytes, void* stream) {
  int rc = qlin_check(d);
  if (rc) return rc;
  if (!X || !W || !theta || !Y) return OMQ_E_INVALID_ARG;
  if (!al16(X) || !al16(W) || !al16(Y)) return OMQ_E_ALIGN;
  if (!ws || ws_bytes < omq_qlinear_workspace_size(d)) return OMQ_E_WORKSPACE;
  const QLinWs w = qlin_layout(d, ws);
  const hipStream_t st = S(stream);
  const int dt = d->path == OMQ_PATH_BF16 ? OMQ_BF16 : OMQ_F32;
  const int64_t T = d->T, ci = d->c_in, co = d->c_out, rq = qlin_rows(d);
  const int64_t grp = lwc_group(d->group, ci);
  const float* ag = theta;
  const float* ab = theta + rq;
  const float* s = d->use_let ? theta + 2 * rq : nullptr;
  const float* dl = d->use_let ? theta + 2 * rq + ci : nullptr;
  // weight side: LET-W, LWC, bias fold
  RowQuantFwd a;
  a.x = W; a.x_dt = dt; a.rows = co; a.cols = ci; a.ldx = ci;
  a.let_mode = s ? OMQ_LET_MUL : OMQ_LET_NONE; a.s = s;
  a.nbits = d->wbits; a.a_gamma = ag; a.a_beta = ab;
  a.out = w.What; a.out_dt = dt; a.ldo = ci;
  a.h = w.wh; a.z = w.wz; a.amax = w.wamax; a.amin = w.wamin;
  a.fold_delta = dl; a.bias = B; a.bias_out = dl ? w.Bt : nullptr;
  if (grp && d->wbits < 16) {     // grouped rows: the bias fold runs on its own
    a.group = grp; a.fold_delta = nullptr; a.bias_out = nullptr;
  }
  const bool cq = qlin_codes(d);
  const int woff = d->wbits == 8 ? 128 : 0, aoff = d->abits == 8 ? 128 : 0;
  if (cq) {
    if (w.cip != ci) {           // padded code rows: zero codes past the row end
      OMQ_HIP_CHECK(launch_fill_f32(reinterpret_cast<float*>(w.Wq), co * w.cip / 4, 0.f, st));
      OMQ_HIP_CHECK(launch_fill_f32(reinterpret_cast<float*>(w.Xq), T * w.cip / 4, 0.f, st));
    }
    a.codes = w.Wq; a.ldq = w.cip; a.code_off = woff; a.qsum = w.wqs;
  }
  OMQ_HIP_CHECK(launch_rowquant_fwd(a, st));
  if (dl && (d->wbits >= 16 || grp))
    OMQ_HIP_CHECK(launch_bias_fold(W, dt, co, ci, dl, B, w.Bt, st));
  const float* bias = dl ? w.Bt : B;
  // activation side: LET-X, per-token quantizer
  RowQuantFwd x;
  x.x = X; x.x_dt = dt; x.rows = T; x.cols = ci; x.ldx = ci;
  x.let_mode = s ? OMQ_LET_DIV : OMQ_LET_NONE; x.s = s; x.delta = dl;
  x.nbits = d->abits; x.out = w.Xhat; x.out_dt = dt; x.ldo = ci;
  x.h = w.ah; x.z = w.az; x.amax = w.aamax; x.amin = w.aamin;
  if (cq) { x.codes = w.Xq; x.ldq = w.cip; x.code_off = aoff; x.qsum = w.aqs; }
  OMQ_HIP_CHECK(launch_rowquant_fwd(x, st));
  Gemm g;
  if (cq) {
    // Q_a(X~) Q_w(W~)^T exactly: h_x h_w sum (q_x - z_x)(q_w - z_w), rounded once
    g.codes = 1;
    g.A = w.Xq; g.lda = w.cip; g.B = w.Wq; g.ldb = w.cip; g.K = w.cip; g.kz = ci;
    g.ha = w.ah; g.za = w.az; g.sa = w.aqs; g.hb = w.wh; g.zb = w.wz; g.sb = w.wqs;
    g.zoa = (float)aoff; g.zob = (float)woff;
  } else {
    g.A = w.Xhat; g.lda = ci; g.B = w.What; g.ldb = ci; g.K = ci; g.dt = dt;
  }
  g.C = Y; g.ldc = co; g.bias = bias; g.M = T; g.N = co;
  OMQ_HIP_CHECK(launch_gemm(g, st));
  return OMQ_OK;
}

int omq_qlinear_bwd(const omq_qlinear_desc* d, const void* X, const void* W, const float* theta,
                    const float* dY, float* dX, float* dtheta, void* ws, size_t ws_bytes,
                    void* stream) {
  int rc = qlin_check(d);
  if (rc) return rc;
  if (!X || !W || !theta || !dY || !dtheta) return OMQ_E_INVALID_ARG;
  if (!al16(X) || !al16(W) || !al16(dY) || !al16(dX)) return OMQ_E_ALIGN;
  if (!ws || ws_bytes < omq_qlinear_workspace_size(d)) return OMQ_E_WORKSPACE;
  const QLinWs w = qlin_layout(d, ws);
  const hipStream_t st = S(stream);
  const bool bf = d->path == OMQ_PATH_BF16;
  const int dt = bf ? OMQ_BF16 : OMQ_F32;
  const int64_t T = d->T, ci = d->c_in, co = d->c_out, rq = qlin_rows(d);
  const int64_t grp = lwc_group(d->group, ci);
  const float* s = d->use_let ? theta + 2 * rq : nullptr;
  const float* dl = d->use_let ? theta + 2 * rq + ci : nullptr;
  float* g_ag = dtheta;
  float* g_ab = dtheta + rq;
  float* g_s = d->use_let ? dtheta + 2 * rq : nullptr;
  float* g_d = d->use_let ? dtheta + 2 * rq + ci : nullptr;
  // dW = dY^T X_hat and dX_hat = dY W_hat, with dY^T, X_hat and W_hat read K-major
  if (dl && !bf) OMQ_HIP_CHECK(launch_colsum(dY, T, co, co, w.colsum, w.cs, st));
  if (d->wbits >= 16) OMQ_HIP_CHECK(launch_fill_f32(dtheta, 2 * rq, 0.f, st));
  if (bf) {
    // bf16 path: dY's bf16 copy and column sums in one pass; both straight-through
    // passes run in the GEMM epilogues
    OMQ_HIP_CHECK(launch_cvt_bf16_colsum(dY, T, co, w.dYb, dl ? w.colsum : nullptr, w.cs, st));
    int64_t nsl, ntl;
    if (d->wbits < 16 || s) {
      gemm_ste_extents(co, ci, &nsl, &ntl);
      float* rowpart = w.rq;
      float* colpart = w.rq + nsl * co * 2;
      Gemm g;
      g.A = w.dYb; g.lda = co; g.ta = 1; g.B = w.Xhat; g.ldb = ci; g.tb = 1;
      g.ldc = ci; g.M = co; g.N = ci; g.K = T;
      SteEpi& se = g.ste;
      se.mode = 1; se.nseg = 1; se.seg_end[0] = co; se.xseg[0] = W;
      se.x_dt = OMQ_BF16; se.ldx = ci; se.let_mode = s ? OMQ_LET_MUL : OMQ_LET_NONE; se.s = s;
      se.h = w.wh; se.z = w.wz; se.nbits = d->wbits; se.rowvec = dl ? w.colsum : nullptr;
      se.col_mode = s ? COL_WEIGHT : COL_NONE; se.rowpart = rowpart; se.colpart = colpart;
      se.grouped = grp > 0;      // one 128-column tile = one group
      OMQ_HIP_CHECK(launch_gemm(g, st));
      RowQuantBwd a;
      a.x = W; a.x_dt = OMQ_BF16; a.rows = co; a.cols = ci; a.ldx = ci;
      a.let_mode = se.let_mode; a.s = s; a.nbits = d->wbits;
      a.h = w.wh; a.z = w.wz; a.amax = w.wamax; a.amin = w.wamin;
      a.a_gamma = theta; a.a_beta = theta + rq; a.g_agamma = g_ag; a.g_abeta = g_ab;
      a.col_mode = se.col_mode; a.out0 = g_s; a.out1 = g_d; a.group = grp;
      OMQ_HIP_CHECK(launch_ste_finish(a, (int)ntl, colpart, a, grp ? 1 : (int)nsl, rowpart,
                                      kSteTileRows, st));
    }
    if (dX || s) {
      gemm_ste_extents(T, ci, &nsl, &ntl);
      float* rowpart = w.rq;
      float* colpart = w.rq + nsl * T * 2;
      Gemm g;
      g.A = w.dYb; g.lda = co; g.B = w.What; g.ldb = ci; g.tb = 1;
      g.C = dX ? dX : w.gXh; g.ldc = ci; g.M = T; g.N = ci; g.K = co;
      SteEpi& se = g.ste;
      se.mode = 2; se.nseg = 1; se.seg_end[0] = T; se.xseg[0] = X;
      se.x_dt = OMQ_BF16; se.ldx = ci; se.let_mode = s ? OMQ_LET_DIV : OMQ_LET_NONE;
      se.s = s; se.delta = dl; se.h = w.ah; se.z = w.az; se.nbits = d->abits;
      se.col_mode = s ? COL_ACT_DIV : COL_NONE; se.rowpart = rowpart; se.colpart = colpart;
      OMQ_HIP_CHECK(launch_gemm(g, st));
      RowQuantBwd x;
      x.x = X; x.x_dt = OMQ_BF16; x.rows = T; x.cols = ci; x.ldx = ci;
      x.let_mode = se.let_mode; x.s = s; x.delta = dl; x.nbits = d->abits;
      x.h = w.ah; x.z = w.az; x.amax = w.aamax; x.amin = w.aamin;
      x.col_mode = se.col_mode; x.gx = g.C; x.ldgx = ci; x.out0 = g_s; x.out1 = g_d;
      x.accumulate = 1;
      OMQ_HIP_CHECK(launch_ste_finish(x, (int)ntl, colpart, x, (int)nsl, rowpart,
                                      kSteTileRows, st));
    }
    return OMQ_OK;
  }
  // fp32 path: the products, then the tile passes
  Gemm gw, gx;
  gw.A = dY; gw.lda = co; gw.ta = 1; gw.B = w.Xhat; gw.ldb = ci; gw.tb = 1;
  gx.A = dY; gx.lda = co; gx.B = w.What; gx.ldb = ci; gx.tb = 1;
  gw.C = w.gW; gw.ldc = ci; gw.M = co; gw.N = ci; gw.K = T; gw.dt = dt;
  OMQ_HIP_CHECK(launch_gemm(gw, st));
  gx.C = w.gXh; gx.ldc = ci; gx.M = T; gx.N = ci; gx.K = co; gx.dt = dt;
  OMQ_HIP_CHECK(launch_gemm(gx, st));
  RowQuantBwd a;
  a.g = w.gW; a.ldg = ci; a.x = W; a.x_dt = dt; a.rows = co; a.cols = ci; a.ldx = ci;
  a.let_mode = s ? OMQ_LET_MUL : OMQ_LET_NONE; a.s = s; a.nbits = d->wbits;
  a.h = w.wh; a.z = w.wz; a.amax = w.wamax; a.amin = w.wamin;
  a.a_gamma = theta; a.a_beta = theta + rq;
  a.col_mode = s ? COL_WEIGHT : COL_NONE; a.rowvec = dl ? w.colsum : nullptr;
  a.g_agamma = g_ag; a.g_abeta = g_ab; a.out0 = g_s; a.out1 = g_d; a.ws = w.rq;
  a.group = grp;
  OMQ_HIP_CHECK(launch_rowquant_bwd(a, st));
  if (dX || s) {
    RowQuantBwd x;
    x.g = w.gXh; x.ldg = ci; x.x = X; x.x_dt = dt; x.rows = T; x.cols = ci; x.ldx = ci;
    x.let_mode = s ? OMQ_LET_DIV : OMQ_LET_NONE; x.s = s; x.delta = dl; x.nbits = d->abits;
    x.h = w.ah; x.z = w.az; x.amax = w.aamax; x.amin = w.aamin;
    x.col_mode = s ? COL_ACT_DIV : COL_NONE; x.gx = dX; x.ldgx = ci;
    x.out0 = g_s; x.out1 = g_d; x.accumulate = 1; x.ws = w.rq;
    OMQ_HIP_CHECK(launch_rowquant_bwd(x, st));
  }
  return OMQ_OK;
}

int omq_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int n_bits,
                   uint32_t* words, void* stream) {
  if (!codes || !words) return OMQ_E_INVALID_ARG;
  if (n_bits < 2 || n_bits > 8) return OMQ_E_INVALID_ARG;
  if (rows < 0 || cols < 0) return OMQ_E_SHAPE;
  if (!al4(words)) return OMQ_E_ALIGN;
  OMQ_HIP_CHECK(launch_pack_codes(codes, rows, cols, n_bits, words, S(stream)));
  return OMQ_OK;
}

int omq_fold_linear(const uint32_t* words, int n_bits, int64_t N, int64_t K, const float* h,
                    const float* z, int64_t group, const float* B, const float* s,
                    const float* delta, const float* s_o, const float* delta_o,
                    float* bias_out, float* h_out, float* gain_out, void* stream) {
  if (!words || !h || !z || !bias_out) return OMQ_E_INVALID_ARG;
  if ((delta && !s) || (s_o && !h_out) || (gain_out && !s)) return OMQ_E_INVALID_ARG;
  if (n_bits < 2 || n_bits > 8) return OMQ_E_INVALID_ARG;
  if (N < 0 || K <= 0) return OMQ_E_SHAPE;
  const int64_t grp = lwc_group(group, K);
  if (grp < 0) return OMQ_E_SHAPE;
  DeployFold a;
  a.words = words; a.nbits = n_bits; a.N = N; a.K = K; a.h = h; a.z = z; a.group = grp;
  a.B = B; a.s = s; a.delta = delta; a.s_o = s_o; a.delta_o = delta_o;
  a.bias_out = bias_out; a.h_out = h_out; a.gain_out = gain_out;
  OMQ_HIP_CHECK(launch_fold_linear(a, S(stream)));
  return OMQ_OK;
}

int omq_w4a16_gemm(const void* X, int64_t T, int64_t K, const uint32_t* words, int64_t N,
                   const float* h, const float* z, int64_t group, const float* bias, float* Y,
                   void* stream) {
  if (!X || !words || !h || !z || !Y) return OMQ_E_INVALID_ARG;
  if (T < 0 || N < 0 || K <= 0) return OMQ_E_SHAPE;
  if (K % 64) return OMQ_E_ALIGN;
  const int64_t grp = lwc_group(group, K);
  if (grp < 0) return OMQ_E_SHAPE;
  if (!al16(X) || !al16(words)) return OMQ_E_ALIGN;
  DeployGemm a;
  a.X = X; a.T = T; a.K = K; a.words = words; a.N = N; a.h = h; a.z = z; a.group = grp;
  a.bias = bias; a.Y = Y;
  OMQ_HIP_CHECK(launch_w4a16_gemm(a, S(stream)));
  return OMQ_OK;
}

int omq_sgd(float* theta, const float* grad, int64_t n, int64_t n_lwc, float lr_lwc,
            float lr_let, void* stream) {
  if (!theta || !grad) return OMQ_E_INVALID_ARG;
  if (n < 0 || n_lwc < 0 || n_lwc > n) return OMQ_E_SHAPE;
  OMQ_HIP_CHECK(launch_sgd(theta, grad, n, n_lwc, lr_lwc, lr_let, S(stream)));
  return OMQ_OK;
}

int omq_adamw(float* theta, const float* grad, float* m, float* v, int64_t n, int64_t n_lwc,
              float lr_lwc, float lr_let, float beta1, float beta2, float eps,
              float weight_decay, int64_t step, void* stream) {
  if (!theta || !grad || !m || !v) return OMQ_E_INVALID_ARG;
  if (step < 1) return OMQ_E_INVALID_ARG;
  if (n < 0 || n_lwc < 0 || n_lwc > n) return OMQ_E_SHAPE;
  OMQ_HIP_CHECK(launch_adamw(theta, grad, m, v, n, n_lwc, lr_lwc, lr_let, beta1, beta2, eps,
                             weight_decay, step, S(stream)));
  return OMQ_OK;
}

}  // extern "C"
