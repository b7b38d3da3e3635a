// One OmniQuant block-reconstruction step on a LLaMA-shaped decoder block
// (paper reading, section "框架": frozen weights, learn Theta1 = {gamma, beta} and
// Theta2 = {s, delta, s_a} against the full-precision block output; section "LET":
// LET on every linear except the second FFN linear, s_a on the attention affinity,
// Q/K/V quantized, softmax kept in full precision).
//
// Everything runs as a fixed sequence of launches on the caller's stream; nothing
// is copied to the host.  Weight rows of q/k/v and of gate/up are dequantized into
// concatenated buffers so each pair/triple runs as one GEMM (N = dq + 2 dk and 2F).
#include "api_util.h"

#include <math.h>

using namespace omq;

namespace {

enum { LQ = 0, LK, LV, LO, LG, LU, LD, NLIN };

struct Dims {
  int64_t T, d, nq, nkv, hd, F, dq, dk, nqkv;
  int grp;
  bool ffn_only, use_sa;
};

Dims dims_of(const omq_block_desc* b) {
  Dims m;
  m.T = b->T; m.d = b->d; m.nq = b->n_q; m.nkv = b->n_kv; m.hd = b->head_dim; m.F = b->F;
  m.dq = m.nq * m.hd; m.dk = m.nkv * m.hd; m.nqkv = m.dq + 2 * m.dk;
  m.grp = (int)(m.nkv ? m.nq / m.nkv : 1);
  m.ffn_only = b->ffn_only != 0;
  m.use_sa = !m.ffn_only && b->abits < 16;
  return m;
}

struct Theta {  // offsets (elements) into the packed parameter vector
  int64_t ag[NLIN], ab[NLIN];
  int64_t s_qkv, d_qkv, s_o, d_o, s_ffn, d_ffn, s_a;
  int64_t n_lwc, total;
  int64_t offs[2 * NLIN + 7];
  int64_t n_entries;
};

Theta theta_of(const Dims& m) {
  Theta t;
  const int64_t cout[NLIN] = {m.dq, m.dk, m.dk, m.d, m.F, m.F, m.d};
  int64_t o = 0;
  int e = 0;
  for (int l = 0; l < NLIN; ++l) {
    t.ag[l] = t.ab[l] = -1;
    if (m.ffn_only && l < LG) continue;
    t.ag[l] = o; t.offs[e++] = o; o += cout[l];
    t.ab[l] = o; t.offs[e++] = o; o += cout[l];
  }
  t.n_lwc = o;
  t.s_qkv = t.d_qkv = t.s_o = t.d_o = t.s_a = -1;
  if (!m.ffn_only) {
    t.s_qkv = o; t.offs[e++] = o; o += m.d;
    t.d_qkv = o; t.offs[e++] = o; o += m.d;
    t.s_o = o; t.offs[e++] = o; o += m.dk;
    t.d_o = o; t.offs[e++] = o; o += m.dk;
  }
  t.s_ffn = o; t.offs[e++] = o; o += m.d;
  t.d_ffn = o; t.offs[e++] = o; o += m.d;
  if (m.use_sa) { t.s_a = o; t.offs[e++] = o; o += m.dk; }
  t.total = o;
  t.n_entries = e;
  return t;
}

struct Stats {  // per-row quantizer state
  float *h, *z;
  int32_t *amax, *amin;
};

Stats take_stats(Bump& b, int64_t n) {
  Stats s;
  s.h = b.take<float>(n); s.z = b.take<float>(n);
  s.amax = b.take<int32_t>(n); s.amin = b.take<int32_t>(n);
  return s;
}

struct Ws {
  // parameters broadcast over query heads
  float *s_o_x, *d_o_x, *sa_q;
  // dequantized weights (concatenated) and their per-row state
  uint16_t *Wqkv, *Wo, *Wgu, *Wd;
  Stats wq_qkv, wq_o, wq_gu, wq_d;
  float *Bt_qkv, *Bt_o, *Bt_gu;
  // forward activations
  float *cos_t, *sin_t, *xn, *r1, *Yqkv, *Qr, *Kr, *S, *O, *h1, *r2, *xn2, *GU, *A, *y;
  uint16_t *Xqkv, *Qh, *Kh, *Vh, *Vt, *P, *Xo, *Xf, *Xd;
  Stats a_qkv, a_q, a_k, a_v, a_o, a_f, a_d;
  // backward
  float *dy, *gW, *gX, *gA, *gGU, *gxn2, *dh1, *gO, *gQh, *gKh, *gVh, *gQr, *gKr, *gY, *dP;
  uint16_t *dyb, *dyt, *Wt, *Xt, *gGUb, *gGUt, *dh1b, *dh1t, *gOb, *gOt, *Pt, *dS, *dSt, *Qt,
      *Kt, *gYb, *gYt;
  float *cs, *gs_full, *gd_full, *gsa_full;
  float *rq, *csws, *msews;
  size_t total;
};

Ws layout(const Dims& m, void* base) {
  Bump b(base);
  Ws w{};
  const int64_t T = m.T, d = m.d, F = m.F, dq = m.dq, dk = m.dk, nqkv = m.nqkv;
  const bool att = !m.ffn_only;
  const int64_t maxw = std::max({att ? nqkv * d : 0, att ? d * dq : 0, 2 * F * d, d * F});
  const int64_t maxc = std::max({d, att ? dq : 0, F});
  if (att) {
    w.s_o_x = b.take<float>(dq); w.d_o_x = b.take<float>(dq); w.sa_q = b.take<float>(dq);
    w.Wqkv = b.take<uint16_t>(nqkv * d); w.Wo = b.take<uint16_t>(d * dq);
    w.wq_qkv = take_stats(b, nqkv); w.wq_o = take_stats(b, d);
    w.Bt_qkv = b.take<float>(nqkv); w.Bt_o = b.take<float>(d);
    w.cos_t = b.take<float>(T * m.hd / 2); w.sin_t = b.take<float>(T * m.hd / 2);
    w.xn = b.take<float>(T * d); w.r1 = b.take<float>(T);
    w.Yqkv = b.take<float>(T * nqkv); w.Qr = b.take<float>(T * dq); w.Kr = b.take<float>(T * dk);
    w.S = b.take<float>(m.nq * T * T); w.O = b.take<float>(T * dq);
    w.h1 = b.take<float>(T * d); w.r2 = b.take<float>(T); w.xn2 = b.take<float>(T * d);
    w.Xqkv = b.take<uint16_t>(T * d); w.Qh = b.take<uint16_t>(T * dq);
    w.Kh = b.take<uint16_t>(T * dk); w.Vh = b.take<uint16_t>(T * dk);
    w.Vt = b.take<uint16_t>(dk * T); w.P = b.take<uint16_t>(m.nq * T * T);
    w.Xo = b.take<uint16_t>(T * dq);
    w.a_qkv = take_stats(b, T); w.a_q = take_stats(b, T); w.a_k = take_stats(b, T);
    w.a_v = take_stats(b, T); w.a_o = take_stats(b, T);
  }
  w.Wgu = b.take<uint16_t>(2 * F * d); w.Wd = b.take<uint16_t>(d * F);
  w.wq_gu = take_stats(b, 2 * F); w.wq_d = take_stats(b, d);
  w.Bt_gu = b.take<float>(2 * F);
  w.GU = b.take<float>(T * 2 * F); w.A = b.take<float>(T * F); w.y = b.take<float>(T * d);
  w.Xf = b.take<uint16_t>(T * d); w.Xd = b.take<uint16_t>(T * F);
  w.a_f = take_stats(b, T); w.a_d = take_stats(b, T);
  // backward
  w.dy = b.take<float>(T * d);
  w.gW = b.take<float>(maxw); w.Wt = b.take<uint16_t>(maxw);
  w.gX = b.take<float>(T * maxc); w.Xt = b.take<uint16_t>(maxc * T);
  w.gA = b.take<float>(T * F); w.gGU = b.take<float>(T * 2 * F);
  w.dyb = b.take<uint16_t>(T * d); w.dyt = b.take<uint16_t>(d * T);
  w.gGUb = b.take<uint16_t>(T * 2 * F); w.gGUt = b.take<uint16_t>(2 * F * T);
  if (att) {
    w.gxn2 = b.take<float>(T * d); w.dh1 = b.take<float>(T * d);
    w.dh1b = b.take<uint16_t>(T * d); w.dh1t = b.take<uint16_t>(d * T);
    w.gO = b.take<float>(T * dq); w.gOb = b.take<uint16_t>(T * dq);
    w.gOt = b.take<uint16_t>(dq * T);
    w.gQh = b.take<float>(T * dq); w.gKh = b.take<float>(T * dk); w.gVh = b.take<float>(T * dk);
    w.gQr = b.take<float>(T * dq); w.gKr = b.take<float>(T * dk);
    w.gY = b.take<float>(T * nqkv);
    w.gYb = b.take<uint16_t>(T * nqkv); w.gYt = b.take<uint16_t>(nqkv * T);
    w.dP = b.take<float>(m.nq * T * T);
    w.Pt = b.take<uint16_t>(m.nq * T * T); w.dS = b.take<uint16_t>(m.nq * T * T);
    w.dSt = b.take<uint16_t>(m.nq * T * T);
    w.Qt = b.take<uint16_t>(dq * T); w.Kt = b.take<uint16_t>(dk * T);
    w.gs_full = b.take<float>(dq); w.gd_full = b.take<float>(dq); w.gsa_full = b.take<float>(dq);
  }
  w.cs = b.take<float>(std::max(nqkv, 2 * F));
  size_t rq = 0;
  const int64_t rshapes[][2] = {{nqkv, d}, {d, dq}, {2 * F, d}, {d, F}, {T, d}, {T, dq}, {T, F}};
  for (auto& r : rshapes) rq = std::max(rq, rowquant_bwd_ws_bytes(r[0], r[1]));
  w.rq = b.take<float>(rq / 4);
  w.csws = b.take<float>(colsum_ws_bytes(T, std::max(nqkv, 2 * F)) / 4);
  w.msews = b.take<float>(2048);
  w.total = b.off;
  return w;
}

int check(const omq_block_desc* b) {
  if (!b || b->struct_size < sizeof(omq_block_desc)) return OMQ_E_INVALID_ARG;
  if (!bits_ok(b->wbits) || !bits_ok(b->abits)) return OMQ_E_INVALID_ARG;
  if (b->optimizer != OMQ_OPT_ADAMW && b->optimizer != OMQ_OPT_SGD) return OMQ_E_INVALID_ARG;
  if (b->T <= 0 || b->d <= 0 || b->F <= 0) return OMQ_E_SHAPE;
  if (!b->ffn_only) {
    if (b->n_q <= 0 || b->n_kv <= 0 || b->head_dim <= 0 || b->n_q % b->n_kv) return OMQ_E_SHAPE;
    if (b->head_dim % 8) return OMQ_E_ALIGN;
  }
  if (b->T % 8 || b->d % 8 || b->F % 8) return OMQ_E_ALIGN;
  return OMQ_OK;
}

// one linear's weight side: LET-W (s), LWC (theta logits), bias fold (delta)
hipError_t wfq(const void* W, int64_t rows, int64_t cols, const float* s, const float* delta,
               const float* th, const Theta& t, int l, int wbits, bool fp, uint16_t* out,
               const Stats& st, int64_t row0, float* Bt, hipStream_t stream) {
  RowQuantFwd a;
  a.x = W; a.x_dt = OMQ_BF16; a.rows = rows; a.cols = cols; a.ldx = cols;
  a.let_mode = (s && !fp) ? OMQ_LET_MUL : OMQ_LET_NONE; a.s = s;
  a.nbits = fp ? 16 : wbits;
  a.a_gamma = fp ? nullptr : th + t.ag[l]; a.a_beta = fp ? nullptr : th + t.ab[l];
  a.out = out + row0 * cols; a.out_dt = OMQ_BF16; a.ldo = cols;
  a.h = st.h + row0; a.z = st.z + row0; a.amax = st.amax + row0; a.amin = st.amin + row0;
  if (!fp && delta) { a.fold_delta = delta; a.bias_out = Bt + row0; }
  hipError_t e = launch_rowquant_fwd(a, stream);
  if (e == hipSuccess && !fp && delta && a.nbits >= 16)
    e = launch_bias_fold(W, OMQ_BF16, rows, cols, delta, nullptr, Bt + row0, stream);
  return e;
}

// per-token quantizer with fused LET on its input
hipError_t aq(const void* X, int x_dt, int64_t T, int64_t C, int64_t ldx, int mode,
              const float* s, const float* delta, int abits, uint16_t* out, const Stats& st,
              hipStream_t stream) {
  RowQuantFwd a;
  a.x = X; a.x_dt = x_dt; a.rows = T; a.cols = C; a.ldx = ldx;
  a.let_mode = mode; a.s = s; a.delta = delta; a.nbits = abits;
  a.out = out; a.out_dt = OMQ_BF16; a.ldo = C;
  a.h = st.h; a.z = st.z; a.amax = st.amax; a.amin = st.amin;
  return launch_rowquant_fwd(a, stream);
}

hipError_t gemm(const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc,
                int64_t M, int64_t N, int64_t K, const float* bias, const void* resid,
                int resid_dt, int64_t ldr, hipStream_t st) {
  Gemm g;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K; g.bias = bias; g.resid = resid; g.resid_dt = resid_dt; g.ldr = ldr;
  return launch_gemm(g, st);
}

#define CK(x)                               \
  do {                                      \
    hipError_t e__ = (x);                   \
    if (e__ != hipSuccess) return OMQ_E_HIP; \
  } while (0)

// Forward.  fp: the full-precision target (no quantizers, no LET).
int forward(const omq_block_desc* bd, const Dims& m, const Theta& t, const Ws& w, const void* x,
            const void* const* W, const float* th, bool fp, hipStream_t st) {
  const int64_t T = m.T, d = m.d, F = m.F, dq = m.dq, dk = m.dk, nqkv = m.nqkv;
  const int wb = fp ? 16 : bd->wbits, ab = fp ? 16 : bd->abits;
  const float* s_ffn = fp ? nullptr : th + t.s_ffn;
  const float* d_ffn = fp ? nullptr : th + t.d_ffn;
  const int mode_let = fp ? OMQ_LET_NONE : OMQ_LET_DIV;
  const float* xf = nullptr;  // FFN input
  int xf_dt = OMQ_F32;
  if (!m.ffn_only) {
    const float* s_qkv = fp ? nullptr : th + t.s_qkv;
    const float* d_qkv = fp ? nullptr : th + t.d_qkv;
    if (!fp) {
      CK(launch_kv_expand(th + t.s_o, m.nq, m.nkv, m.hd, w.s_o_x, st));
      CK(launch_kv_expand(th + t.d_o, m.nq, m.nkv, m.hd, w.d_o_x, st));
      if (m.use_sa) CK(launch_kv_expand(th + t.s_a, m.nq, m.nkv, m.hd, w.sa_q, st));
    }
    const float* s_o = fp ? nullptr : w.s_o_x;
    const float* d_o = fp ? nullptr : w.d_o_x;
    CK(launch_rope_tables(T, m.hd, bd->rope_theta, w.cos_t, w.sin_t, st));
    // weight side of q, k, v, o
    CK(wfq(W[LQ], dq, d, s_qkv, d_qkv, th, t, LQ, wb, fp, w.Wqkv, w.wq_qkv, 0, w.Bt_qkv, st));
    CK(wfq(W[LK], dk, d, s_qkv, d_qkv, th, t, LK, wb, fp, w.Wqkv, w.wq_qkv, dq, w.Bt_qkv, st));
    CK(wfq(W[LV], dk, d, s_qkv, d_qkv, th, t, LV, wb, fp, w.Wqkv, w.wq_qkv, dq + dk, w.Bt_qkv, st));
    CK(wfq(W[LO], d, dq, s_o, d_o, th, t, LO, wb, fp, w.Wo, w.wq_o, 0, w.Bt_o, st));
    // attention input
    CK(launch_rmsnorm(x, OMQ_BF16, T, d, bd->eps, w.xn, w.r1, st));
    CK(aq(w.xn, OMQ_F32, T, d, d, mode_let, s_qkv, d_qkv, ab, w.Xqkv, w.a_qkv, st));
    CK(gemm(w.Xqkv, d, w.Wqkv, d, w.Yqkv, nqkv, T, nqkv, d, fp ? nullptr : w.Bt_qkv, nullptr, 0,
            0, st));
    CK(launch_rope(w.Yqkv, nqkv, T, m.nq, m.hd, w.cos_t, w.sin_t, 0, w.Qr, dq, st));
    CK(launch_rope(w.Yqkv + dq, nqkv, T, m.nkv, m.hd, w.cos_t, w.sin_t, 0, w.Kr, dk, st));
    // s_a on the affinity, then Q/K/V quantized per token
    const bool sa = m.use_sa && !fp;
    CK(aq(w.Qr, OMQ_F32, T, dq, dq, sa ? OMQ_LET_DIV : OMQ_LET_NONE, w.sa_q, nullptr, ab, w.Qh,
          w.a_q, st));
    CK(aq(w.Kr, OMQ_F32, T, dk, dk, sa ? OMQ_LET_MUL : OMQ_LET_NONE, th + (sa ? t.s_a : 0),
          nullptr, ab, w.Kh, w.a_k, st));
    CK(aq(w.Yqkv + dq + dk, OMQ_F32, T, dk, nqkv, OMQ_LET_NONE, nullptr, nullptr, ab, w.Vh, w.a_v,
          st));
    // causal attention, float32 softmax
    {
      Gemm g;
      g.A = w.Qh; g.lda = dq; g.strideA = m.hd;
      g.B = w.Kh; g.ldb = dk; g.strideB = m.hd; g.b_group = m.grp;
      g.C = w.S; g.ldc = T; g.strideC = T * T;
      g.M = T; g.N = T; g.K = m.hd; g.batch = (int)m.nq;
      g.alpha = 1.f / sqrtf((float)m.hd); g.causal = CAUSAL_SKIP_UPPER;
      CK(launch_gemm(g, st));
    }
    CK(launch_softmax_causal(w.S, T, (int)m.nq, w.P, nullptr, st));
    CK(launch_transpose_bf16(w.Vh, T, dk, dk, w.Vt, T, 1, 0, 0, st));
    {
      Gemm g;
      g.A = w.P; g.lda = T; g.strideA = T * T;
      g.B = w.Vt; g.ldb = T; g.strideB = m.hd * T; g.b_group = m.grp;
      g.C = w.O; g.ldc = dq; g.strideC = m.hd;
      g.M = T; g.N = m.hd; g.K = T; g.batch = (int)m.nq; g.causal = CAUSAL_K_UPPER;
      CK(launch_gemm(g, st));
    }
    // o_proj with its LET site, residual
    CK(aq(w.O, OMQ_F32, T, dq, dq, mode_let, s_o, d_o, ab, w.Xo, w.a_o, st));
    CK(gemm(w.Xo, dq, w.Wo, dq, w.h1, d, T, d, dq, fp ? nullptr : w.Bt_o, x, OMQ_BF16, d, st));
    CK(launch_rmsnorm(w.h1, OMQ_F32, T, d, bd->eps, w.xn2, w.r2, st));
    xf = w.xn2;
    xf_dt = OMQ_F32;
  } else {
    xf = reinterpret_cast<const float*>(x);
    xf_dt = OMQ_BF16;
  }
  // FFN
  CK(wfq(W[LG], F, d, s_ffn, d_ffn, th, t, LG, wb, fp, w.Wgu, w.wq_gu, 0, w.Bt_gu, st));
  CK(wfq(W[LU], F, d, s_ffn, d_ffn, th, t, LU, wb, fp, w.Wgu, w.wq_gu, F, w.Bt_gu, st));
  CK(wfq(W[LD], d, F, nullptr, nullptr, th, t, LD, wb, fp, w.Wd, w.wq_d, 0, nullptr, st));
  CK(aq(xf, xf_dt, T, d, d, mode_let, s_ffn, d_ffn, ab, w.Xf, w.a_f, st));
  CK(gemm(w.Xf, d, w.Wgu, d, w.GU, 2 * F, T, 2 * F, d, fp ? nullptr : w.Bt_gu, nullptr, 0, 0, st));
  CK(launch_silu_gate(w.GU, T, F, w.A, st));
  CK(aq(w.A, OMQ_F32, T, F, F, OMQ_LET_NONE, nullptr, nullptr, ab, w.Xd, w.a_d, st));
  CK(gemm(w.Xd, F, w.Wd, F, w.y, d, T, d, F, nullptr, m.ffn_only ? nullptr : w.h1, OMQ_F32, d,
          st));
  return OMQ_OK;
}

// weight-side straight-through backward of one linear (rows [row0, row0 + rows) of gW)
hipError_t wbwd(const Ws& w, const void* W, int64_t rows, int64_t cols, const float* s,
                const float* th, const Theta& t, int l, int wbits, const Stats& st, int64_t row0,
                const float* gW, const float* cs, float* gs, float* gd, int accumulate,
                float* dth, hipStream_t stream) {
  if (wbits >= 16 && !s) return hipSuccess;  // no parameter depends on this weight
  RowQuantBwd a;
  a.g = gW + row0 * cols; a.ldg = cols;
  a.x = W; a.x_dt = OMQ_BF16; a.rows = rows; a.cols = cols; a.ldx = cols;
  a.let_mode = s ? OMQ_LET_MUL : OMQ_LET_NONE; a.s = s; a.nbits = wbits;
  a.h = st.h + row0; a.z = st.z + row0; a.amax = st.amax + row0; a.amin = st.amin + row0;
  a.a_gamma = th + t.ag[l]; a.a_beta = th + t.ab[l];
  a.col_mode = s ? COL_WEIGHT : COL_NONE;
  a.rowvec = cs ? cs + row0 : nullptr;
  a.g_agamma = dth + t.ag[l]; a.g_abeta = dth + t.ab[l];
  a.out0 = gs; a.out1 = gd; a.accumulate = accumulate; a.ws = w.rq;
  return launch_rowquant_bwd(a, stream);
}

// activation-side backward through the per-token quantizer and the fused LET
hipError_t abwd(const Ws& w, const float* g, int64_t T, int64_t C, const void* X, int x_dt,
                int64_t ldx, int mode, const float* s, const float* delta, int abits,
                const Stats& st, float* gx, int64_t ldgx, int col_mode, float* out0, float* out1,
                int accumulate, hipStream_t stream) {
  RowQuantBwd a;
  a.g = g; a.ldg = C; a.x = X; a.x_dt = x_dt; a.rows = T; a.cols = C; a.ldx = ldx;
  a.let_mode = mode; a.s = s; a.delta = delta; a.nbits = abits;
  a.h = st.h; a.z = st.z; a.amax = st.amax; a.amin = st.amin;
  a.col_mode = col_mode; a.gx = gx; a.ldgx = ldgx;
  a.out0 = out0; a.out1 = out1; a.accumulate = accumulate; a.ws = w.rq;
  return launch_rowquant_bwd(a, stream);
}

// dX = dY_b Wt^T and dW = dY_t X_t^T for one (possibly concatenated) linear.
// gY: float [T x N]; Xh: bf16 [T x K]; Wh: bf16 [N x K].
hipError_t lin_bwd_gemms(const Ws& w, const float* gY, int64_t T, int64_t N, int64_t K,
                         const uint16_t* Xh, const uint16_t* Wh, uint16_t* gYb, uint16_t* gYt,
                         float* cs, hipStream_t st) {
  hipError_t e;
  if ((e = launch_f32_to_bf16(gY, T, N, N, gYb, N, gYt, T, st)) != hipSuccess) return e;
  if ((e = launch_transpose_bf16(Xh, T, K, K, w.Xt, T, 1, 0, 0, st)) != hipSuccess) return e;
  if ((e = launch_transpose_bf16(Wh, N, K, K, w.Wt, N, 1, 0, 0, st)) != hipSuccess) return e;
  if ((e = gemm(gYt, T, w.Xt, T, w.gW, K, N, K, T, nullptr, nullptr, 0, 0, st)) != hipSuccess)
    return e;
  if ((e = gemm(gYb, N, w.Wt, N, w.gX, K, T, K, N, nullptr, nullptr, 0, 0, st)) != hipSuccess)
    return e;
  if (cs) e = launch_colsum(gY, T, N, N, cs, w.csws, st);
  return e;
}

int backward(const omq_block_desc* bd, const Dims& m, const Theta& t, const Ws& w,
             const void* x, const void* const* W, const float* th, float* dth, hipStream_t st) {
  const int64_t T = m.T, d = m.d, F = m.F, dq = m.dq, dk = m.dk, nqkv = m.nqkv;
  const int wb = bd->wbits, ab = bd->abits;
  CK(hipMemsetAsync(dth, 0, t.total * sizeof(float), st));
  // FFN second linear (no LET)
  CK(lin_bwd_gemms(w, w.dy, T, d, F, w.Xd, w.Wd, w.dyb, w.dyt, nullptr, st));
  CK(wbwd(w, W[LD], d, F, nullptr, th, t, LD, wb, w.wq_d, 0, w.gW, nullptr, nullptr, nullptr, 0,
          dth, st));
  CK(abwd(w, w.gX, T, F, w.A, OMQ_F32, F, OMQ_LET_NONE, nullptr, nullptr, ab, w.a_d, w.gA, F,
          COL_NONE, nullptr, nullptr, 0, st));
  CK(launch_silu_gate_bwd(w.GU, w.gA, T, F, w.gGU, st));
  // gate / up with the shared ffn LET site
  const float* s_f = th + t.s_ffn;
  const float* d_f = th + t.d_ffn;
  float* gs_f = dth + t.s_ffn;
  float* gd_f = dth + t.d_ffn;
  CK(lin_bwd_gemms(w, w.gGU, T, 2 * F, d, w.Xf, w.Wgu, w.gGUb, w.gGUt, w.cs, st));
  CK(wbwd(w, W[LG], F, d, s_f, th, t, LG, wb, w.wq_gu, 0, w.gW, w.cs, gs_f, gd_f, 1, dth, st));
  CK(wbwd(w, W[LU], F, d, s_f, th, t, LU, wb, w.wq_gu, F, w.gW, w.cs, gs_f, gd_f, 1, dth, st));
  const void* xf = m.ffn_only ? x : (const void*)w.xn2;
  const int xf_dt = m.ffn_only ? OMQ_BF16 : OMQ_F32;
  CK(abwd(w, w.gX, T, d, xf, xf_dt, d, OMQ_LET_DIV, s_f, d_f, ab, w.a_f,
          m.ffn_only ? nullptr : w.gxn2, d, COL_ACT_DIV, gs_f, gd_f, 1, st));
  if (m.ffn_only) return OMQ_OK;

  // RMSNorm before the FFN, residual
  CK(launch_rmsnorm_bwd(w.gxn2, w.h1, w.r2, T, d, w.dy, w.dh1, st));
  // o_proj with its LET site (per KV channel, broadcast over the query heads)
  CK(lin_bwd_gemms(w, w.dh1, T, d, dq, w.Xo, w.Wo, w.dh1b, w.dh1t, w.cs, st));
  CK(wbwd(w, W[LO], d, dq, w.s_o_x, th, t, LO, wb, w.wq_o, 0, w.gW, w.cs, w.gs_full, w.gd_full,
          0, dth, st));
  CK(abwd(w, w.gX, T, dq, w.O, OMQ_F32, dq, OMQ_LET_DIV, w.s_o_x, w.d_o_x, ab, w.a_o, w.gO, dq,
          COL_ACT_DIV, w.gs_full, w.gd_full, 1, st));
  CK(launch_kv_reduce_add(w.gs_full, m.nq, m.nkv, m.hd, dth + t.s_o, st));
  CK(launch_kv_reduce_add(w.gd_full, m.nq, m.nkv, m.hd, dth + t.d_o, st));
  // attention backward (softmax in float32, recomputed from S)
  CK(launch_f32_to_bf16(w.gO, T, dq, dq, w.gOb, dq, w.gOt, T, st));
  {
    Gemm g;  // dP = dO V^T
    g.A = w.gOb; g.lda = dq; g.strideA = m.hd;
    g.B = w.Vh; g.ldb = dk; g.strideB = m.hd; g.b_group = m.grp;
    g.C = w.dP; g.ldc = T; g.strideC = T * T;
    g.M = T; g.N = T; g.K = m.hd; g.batch = (int)m.nq; g.causal = CAUSAL_SKIP_UPPER;
    CK(launch_gemm(g, st));
  }
  const float scale = 1.f / sqrtf((float)m.hd);
  CK(launch_softmax_bwd_causal(w.S, w.dP, w.O, w.gO, T, (int)m.nq, m.hd, dq, scale, w.dS, w.dSt,
                               st));
  CK(launch_transpose_bf16(w.P, T, T, T, w.Pt, T, (int)m.nq, T * T, T * T, st));
  CK(launch_transpose_bf16(w.Kh, T, dk, dk, w.Kt, T, 1, 0, 0, st));
  CK(launch_transpose_bf16(w.Qh, T, dq, dq, w.Qt, T, 1, 0, 0, st));
  {
    Gemm g;  // dQ = dS K
    g.A = w.dS; g.lda = T; g.strideA = T * T;
    g.B = w.Kt; g.ldb = T; g.strideB = m.hd * T; g.b_group = m.grp;
    g.C = w.gQh; g.ldc = dq; g.strideC = m.hd;
    g.M = T; g.N = m.hd; g.K = T; g.batch = (int)m.nq; g.causal = CAUSAL_K_UPPER;
    CK(launch_gemm(g, st));
  }
  for (int r = 0; r < m.grp; ++r) {
    Gemm g;  // dK_g = sum_h dS_h^T Q_h ;  dV_g = sum_h P_h^T dO_h
    g.A = w.dSt + (int64_t)r * T * T; g.lda = T; g.strideA = (int64_t)m.grp * T * T;
    g.B = w.Qt + (int64_t)r * m.hd * T; g.ldb = T; g.strideB = (int64_t)m.grp * m.hd * T;
    g.C = w.gKh; g.ldc = dk; g.strideC = m.hd;
    g.M = T; g.N = m.hd; g.K = T; g.batch = (int)m.nkv; g.causal = CAUSAL_K_LOWER;
    g.accumulate = r > 0;
    CK(launch_gemm(g, st));
    g.A = w.Pt + (int64_t)r * T * T;
    g.B = w.gOt + (int64_t)r * m.hd * T;
    g.C = w.gVh;
    CK(launch_gemm(g, st));
  }
  // Q~ / K~ / V quantizers and s_a
  const bool sa = m.use_sa;
  CK(abwd(w, w.gQh, T, dq, w.Qr, OMQ_F32, dq, sa ? OMQ_LET_DIV : OMQ_LET_NONE, w.sa_q, nullptr,
          ab, w.a_q, w.gQr, dq, sa ? COL_ACT_DIV : COL_NONE, sa ? w.gsa_full : nullptr, nullptr, 0,
          st));
  CK(abwd(w, w.gKh, T, dk, w.Kr, OMQ_F32, dk, sa ? OMQ_LET_MUL : OMQ_LET_NONE,
          sa ? th + t.s_a : nullptr, nullptr, ab, w.a_k, w.gKr, dk, sa ? COL_ACT_MUL : COL_NONE,
          sa ? dth + t.s_a : nullptr, nullptr, 1, st));
  CK(abwd(w, w.gVh, T, dk, w.Yqkv + dq + dk, OMQ_F32, nqkv, OMQ_LET_NONE, nullptr, nullptr, ab,
          w.a_v, w.gY + dq + dk, nqkv, COL_NONE, nullptr, nullptr, 0, st));
  if (sa) CK(launch_kv_reduce_add(w.gsa_full, m.nq, m.nkv, m.hd, dth + t.s_a, st));
  CK(launch_rope(w.gQr, dq, T, m.nq, m.hd, w.cos_t, w.sin_t, 1, w.gY, nqkv, st));
  CK(launch_rope(w.gKr, dk, T, m.nkv, m.hd, w.cos_t, w.sin_t, 1, w.gY + dq, nqkv, st));
  // q / k / v with the shared qkv LET site
  const float* s_q = th + t.s_qkv;
  const float* d_q = th + t.d_qkv;
  float* gs_q = dth + t.s_qkv;
  float* gd_q = dth + t.d_qkv;
  CK(lin_bwd_gemms(w, w.gY, T, nqkv, d, w.Xqkv, w.Wqkv, w.gYb, w.gYt, w.cs, st));
  CK(wbwd(w, W[LQ], dq, d, s_q, th, t, LQ, wb, w.wq_qkv, 0, w.gW, w.cs, gs_q, gd_q, 1, dth, st));
  CK(wbwd(w, W[LK], dk, d, s_q, th, t, LK, wb, w.wq_qkv, dq, w.gW, w.cs, gs_q, gd_q, 1, dth, st));
  CK(wbwd(w, W[LV], dk, d, s_q, th, t, LV, wb, w.wq_qkv, dq + dk, w.gW, w.cs, gs_q, gd_q, 1, dth,
          st));
  CK(abwd(w, w.gX, T, d, w.xn, OMQ_F32, d, OMQ_LET_DIV, s_q, d_q, ab, w.a_qkv, nullptr, d,
          COL_ACT_DIV, gs_q, gd_q, 1, st));
  return OMQ_OK;
}

int check_ptrs(const Dims& m, const void* x, const void* const* weights) {
  if (!x || !weights) return OMQ_E_INVALID_ARG;
  for (int l = 0; l < NLIN; ++l) {
    if (m.ffn_only && l < LG) continue;
    if (!weights[l]) return OMQ_E_INVALID_ARG;
    if (!al16(weights[l])) return OMQ_E_ALIGN;
  }
  if (!al16(x)) return OMQ_E_ALIGN;
  return OMQ_OK;
}

}  // namespace

extern "C" {

int omq_block_theta_layout(const omq_block_desc* d, int64_t* offsets, int64_t* n_entries,
                           int64_t* n_lwc, int64_t* total) {
  int rc = check(d);
  if (rc) return rc;
  const Dims m = dims_of(d);
  const Theta t = theta_of(m);
  if (offsets)
    for (int64_t i = 0; i < t.n_entries; ++i) offsets[i] = t.offs[i];
  if (n_entries) *n_entries = t.n_entries;
  if (n_lwc) *n_lwc = t.n_lwc;
  if (total) *total = t.total;
  return OMQ_OK;
}

size_t omq_block_workspace_size(const omq_block_desc* d) {
  if (check(d)) return 0;
  return layout(dims_of(d), nullptr).total;
}

int omq_block_forward(const omq_block_desc* d, const void* x, const void* const* weights,
                      const float* theta, float* y, void* ws, size_t ws_bytes, void* stream) {
  int rc = check(d);
  if (rc) return rc;
  const Dims m = dims_of(d);
  if ((rc = check_ptrs(m, x, weights))) return rc;
  if (!y) return OMQ_E_INVALID_ARG;
  if (!ws || ws_bytes < omq_block_workspace_size(d)) return OMQ_E_WORKSPACE;
  const Theta t = theta_of(m);
  const Ws w = layout(m, ws);
  const hipStream_t st = S(stream);
  rc = forward(d, m, t, w, x, weights, theta, theta == nullptr, st);
  if (rc) return rc;
  OMQ_HIP_CHECK(hipMemcpyAsync(y, w.y, m.T * m.d * sizeof(float), hipMemcpyDeviceToDevice, st));
  return OMQ_OK;
}

int omq_block_step(const omq_block_desc* d, const void* x, const float* y_target,
                   const void* const* weights, float* theta, float* dtheta, float* adam_m,
                   float* adam_v, int64_t step, float* loss, void* ws, size_t ws_bytes,
                   void* stream) {
  int rc = check(d);
  if (rc) return rc;
  const Dims m = dims_of(d);
  if ((rc = check_ptrs(m, x, weights))) return rc;
  if (!y_target || !theta || !dtheta) return OMQ_E_INVALID_ARG;
  if (d->optimizer == OMQ_OPT_ADAMW && (!adam_m || !adam_v || step < 1)) return OMQ_E_INVALID_ARG;
  if (!ws || ws_bytes < omq_block_workspace_size(d)) return OMQ_E_WORKSPACE;
  const Theta t = theta_of(m);
  const Ws w = layout(m, ws);
  const hipStream_t st = S(stream);
  rc = forward(d, m, t, w, x, weights, theta, false, st);
  if (rc) return rc;
  OMQ_HIP_CHECK(launch_mse(w.y, y_target, m.T * m.d, loss, w.dy, w.msews, st));
  rc = backward(d, m, t, w, x, weights, theta, dtheta, st);
  if (rc) return rc;
  if (d->optimizer == OMQ_OPT_ADAMW)
    OMQ_HIP_CHECK(launch_adamw(theta, dtheta, adam_m, adam_v, t.total, t.n_lwc, d->lr_lwc,
                               d->lr_let, d->beta1, d->beta2, d->adam_eps, d->weight_decay, step,
                               st));
  else
    OMQ_HIP_CHECK(launch_sgd(theta, dtheta, t.total, t.n_lwc, d->lr_lwc, d->lr_let, st));
  return OMQ_OK;
}

}  // extern "C"
