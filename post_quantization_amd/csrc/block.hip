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
  int64_t group;   // LWC group along C_in: 0 (per output channel) or 128
  int grp;
  bool ffn_only, use_sa;
  // the forward's four products on integer codes (int8 matrix cores): weights and
  // activations both quantized, per row (8-bit codes stored shifted by 128 into
  // signed bytes); code rows padded with zero codes to a multiple of 16 columns
  bool codes;
  // ... and with 4-bit codes on both sides and whole 128 x 128 tiles, the codes two to
  // a byte (half the bytes the quantizers write and the products read)
  bool pk;
  int64_t dp, dqp, Fp;     // code-row strides (bytes) of the d-, dq- and F-wide inputs
  int woff, aoff;          // stored code offsets (128 for 8-bit codes)
  // LWC quantizer rows per output channel of a weight with C_in = cin
  int64_t g_of(int64_t cin) const { return group ? cin / group : 1; }
};

Dims dims_of(const omq_block_desc* b) {
  Dims m;
  m.T = b->T; m.d = b->d; m.nq = b->n_q; m.nkv = b->n_kv; m.hd = b->head_dim; m.F = b->F;
  m.dq = m.nq * m.hd; m.dk = m.nkv * m.hd; m.nqkv = m.dq + 2 * m.dk;
  m.grp = (int)(m.nkv ? m.nq / m.nkv : 1);
  m.ffn_only = b->ffn_only != 0;
  m.use_sa = !m.ffn_only && b->abits < 16;
  m.group = b->group;
  m.codes = b->wbits <= 8 && b->abits <= 8 && m.group == 0;
  auto up16 = [](int64_t v) { return (v + 15) / 16 * 16; };
  m.pk = m.codes && b->wbits <= 4 && b->abits <= 4 && m.T % 128 == 0 && m.d % 128 == 0 &&
         m.F % 128 == 0 && (m.ffn_only || (m.dq % 128 == 0 && m.nqkv % 128 == 0));
  if (m.pk) {
    m.dp = m.d / 2; m.dqp = m.dq / 2; m.Fp = m.F / 2;
  } else {
    m.dp = up16(m.d); m.dqp = up16(m.dq); m.Fp = up16(m.F);
  }
  m.woff = b->wbits == 8 ? 128 : 0;
  m.aoff = b->abits == 8 ? 128 : 0;
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
  const int64_t cin[NLIN] = {m.d, m.d, m.d, m.dq, m.d, m.d, m.F};
  int64_t o = 0;
  int e = 0;
  for (int l = 0; l < NLIN; ++l) {
    t.ag[l] = t.ab[l] = -1;
    if (m.ffn_only && l < LG) continue;
    const int64_t rows = cout[l] * m.g_of(cin[l]);
    t.ag[l] = o; t.offs[e++] = o; o += rows;
    t.ab[l] = o; t.offs[e++] = o; o += rows;
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
  int32_t* qsum;   // code sums (integer-code products)
};

Stats take_stats(Bump& b, int64_t n) {
  Stats s;
  s.h = b.take<float>(n); s.z = b.take<float>(n);
  s.amax = b.take<int32_t>(n); s.amin = b.take<int32_t>(n);
  s.qsum = b.take<int32_t>(n);
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
  float *cos_t, *sin_t, *xn, *r1, *Yqkv, *Qr, *Kr, *O, *lse2, *h1, *r2, *xn2, *GU, *A, *y;
  uint16_t *Xqkv, *Qh, *Kh, *Vh, *Xo, *Xf, *Xd;
  Stats a_qkv, a_q, a_k, a_v, a_o, a_f, a_d;
  // backward
  float *dy, *gA, *gGU, *gxn2, *dh1, *gO, *Datt, *gQh, *gKh, *gVh, *gQr, *gKr, *gY;
  float* attn_part;   // partial dK, dV of the attention backward's query-head splits
  uint16_t* attn_ds;  // the attention backward's bf16 dS, [n_q][Tp][Tp]
  uint16_t *dyb, *gGUb, *dh1b, *gOb, *gYb;
  float *cs, *gs_full, *gd_full, *gsa_full;
  float *rq, *csws, *msews;
  // the weight side's straight-through partials of q|k|v, o, gate|up, down (kept until
  // their finalizers run together at the end of the backward)
  float* wpart[4];
  // the Q~, K~, V quantizers' straight-through partials (their finalizers run together)
  float* apart[3];
  // the activation side's partials of gate|up, o and q|k|v (column passes at the end)
  float* xpart[3];
  // integer codes of the forward's product operands (weights, activations)
  uint8_t *Cqkv, *Co, *Cgu, *Cd, *Cxqkv, *Cxo, *Cxf, *Cxd;
  size_t total;
};

Ws layout(const Dims& m, void* base) {
  Bump b(base);
  Ws w{};
  const int64_t T = m.T, d = m.d, F = m.F, dq = m.dq, dk = m.dk, nqkv = m.nqkv;
  const bool att = !m.ffn_only;
  if (att) {
    w.s_o_x = b.take<float>(dq); w.d_o_x = b.take<float>(dq); w.sa_q = b.take<float>(dq);
    w.Wqkv = b.take<uint16_t>(nqkv * d); w.Wo = b.take<uint16_t>(d * dq);
    w.wq_qkv = take_stats(b, nqkv * m.g_of(d)); w.wq_o = take_stats(b, d * m.g_of(dq));
    w.Bt_qkv = b.take<float>(nqkv); w.Bt_o = b.take<float>(d);
    w.cos_t = b.take<float>(T * m.hd / 2); w.sin_t = b.take<float>(T * m.hd / 2);
    w.xn = b.take<float>(T * d); w.r1 = b.take<float>(T);
    w.Yqkv = b.take<float>(T * nqkv); w.Qr = b.take<float>(T * dq); w.Kr = b.take<float>(T * dk);
    w.O = b.take<float>(T * dq); w.lse2 = b.take<float>(m.nq * T);
    w.h1 = b.take<float>(T * d); w.r2 = b.take<float>(T); w.xn2 = b.take<float>(T * d);
    w.Xqkv = b.take<uint16_t>(T * d); w.Qh = b.take<uint16_t>(T * dq);
    w.Kh = b.take<uint16_t>(T * dk); w.Vh = b.take<uint16_t>(T * dk);
    w.Xo = b.take<uint16_t>(T * dq);
    w.a_qkv = take_stats(b, T); w.a_q = take_stats(b, T); w.a_k = take_stats(b, T);
    w.a_v = take_stats(b, T); w.a_o = take_stats(b, T);
  }
  w.Wgu = b.take<uint16_t>(2 * F * d); w.Wd = b.take<uint16_t>(d * F);
  w.wq_gu = take_stats(b, 2 * F * m.g_of(d)); w.wq_d = take_stats(b, d * m.g_of(F));
  w.Bt_gu = b.take<float>(2 * F);
  w.GU = b.take<float>(T * 2 * F); w.A = b.take<float>(T * F); w.y = b.take<float>(T * d);
  w.Xf = b.take<uint16_t>(T * d); w.Xd = b.take<uint16_t>(T * F);
  w.a_f = take_stats(b, T); w.a_d = take_stats(b, T);
  // backward
  w.dy = b.take<float>(T * d);
  w.gA = b.take<float>(T * F); w.gGU = b.take<float>(T * 2 * F);
  w.dyb = b.take<uint16_t>(T * d);
  w.gGUb = b.take<uint16_t>(T * 2 * F);
  if (att) {
    w.gxn2 = b.take<float>(T * d); w.dh1 = b.take<float>(T * d);
    w.dh1b = b.take<uint16_t>(T * d);
    w.gO = b.take<float>(T * dq); w.gOb = b.take<uint16_t>(T * dq);
    w.Datt = b.take<float>(m.nq * T);
    w.gQh = b.take<float>(T * dq); w.gKh = b.take<float>(T * dk); w.gVh = b.take<float>(T * dk);
    w.attn_part = b.take<float>(flash_bwd_part_floats(T, (int)m.nq, (int)m.nkv));
    w.attn_ds = b.take<uint16_t>(flash_bwd_ds_elems(T, m.nq));
    w.gQr = b.take<float>(T * dq); w.gKr = b.take<float>(T * dk);
    w.gY = b.take<float>(T * nqkv);
    w.gYb = b.take<uint16_t>(T * nqkv);
    w.gs_full = b.take<float>(dq); w.gd_full = b.take<float>(dq); w.gsa_full = b.take<float>(dq);
  }
  w.cs = b.take<float>(std::max(nqkv, 2 * F));
  size_t rq = 0;
  const int64_t rshapes[][2] = {{nqkv, d}, {d, dq}, {2 * F, d}, {d, F}, {T, d}, {T, dq}, {T, F}};
  for (auto& r : rshapes) {
    rq = std::max(rq, rowquant_bwd_ws_bytes(r[0], r[1]));
    int64_t nsl, ntl;
    gemm_ste_extents(r[0], r[1], &nsl, &ntl);
    rq = std::max(rq, ste_partials_floats(r[0], r[1], nsl, ntl) * sizeof(float));
  }
  w.rq = b.take<float>(rq / 4);
  {
    const int64_t wsh[4][2] = {{nqkv, d}, {d, dq}, {2 * F, d}, {d, F}};
    for (int i = 0; i < 4; ++i) {
      if (!att && i < 2) continue;
      int64_t nsl, ntl;
      gemm_ste_extents(wsh[i][0], wsh[i][1], &nsl, &ntl);
      w.wpart[i] = b.take<float>((int64_t)ste_partials_floats(wsh[i][0], wsh[i][1], nsl, ntl));
    }
    const int64_t xk[3] = {d, dq, d};
    for (int i = 0; i < 3; ++i) {
      if (!att && i > 0) continue;
      int64_t nsl, ntl;
      gemm_ste_extents(T, xk[i], &nsl, &ntl);
      w.xpart[i] = b.take<float>((int64_t)ste_partials_floats(T, xk[i], nsl, ntl));
    }
    if (att) {
      w.apart[0] = b.take<float>((int64_t)(rowquant_bwd_ws_bytes(T, dq) / 4));
      w.apart[1] = b.take<float>((int64_t)(rowquant_bwd_ws_bytes(T, dk) / 4));
      w.apart[2] = b.take<float>((int64_t)(rowquant_bwd_ws_bytes(T, dk) / 4));
    }
  }
  w.csws = b.take<float>(colsum_ws_bytes(T, std::max(nqkv, 2 * F)) / 4);
  w.msews = b.take<float>(2048);
  if (m.codes) {
    if (att) {
      w.Cqkv = b.take<uint8_t>(nqkv * m.dp); w.Co = b.take<uint8_t>(d * m.dqp);
      w.Cxqkv = b.take<uint8_t>(T * m.dp); w.Cxo = b.take<uint8_t>(T * m.dqp);
    }
    w.Cgu = b.take<uint8_t>(2 * F * m.dp); w.Cd = b.take<uint8_t>(d * m.Fp);
    w.Cxf = b.take<uint8_t>(T * m.dp); w.Cxd = b.take<uint8_t>(T * m.Fp);
  }
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
    if (b->head_dim != 128) return OMQ_E_SHAPE;   // the fused attention kernels
    if (flash_bwd_ds_elems(b->T, b->n_q) < 0) return OMQ_E_SHAPE;   // dS scratch size
  }
  if (b->T % 8 || b->d % 8 || b->F % 8) return OMQ_E_ALIGN;
  // group-wise LWC in groups of 128 input channels: every C_in (d, F, and the
  // attention width) a multiple of 128
  if (b->group != 0 && (b->group != 128 || b->d % 128 || b->F % 128)) return OMQ_E_SHAPE;
  // weight-activation quantization runs its forward products exactly on integer codes
  // of per-row quantizers: group-wise clipping with quantized activations has no such
  // product here
  if (b->group != 0 && b->wbits < 16 && b->abits < 16) return OMQ_E_UNIMPLEMENTED;
  return OMQ_OK;
}

// Optional event timing of one launch (benchmarks): kind and work (FLOPs, or
// algorithmic HBM bytes for the quantizers) are recorded beside the event pair.
template <typename F>
hipError_t timed(omq_timer* tm, int kind, double work, hipStream_t st, F&& launch) {
  const bool rec = tm && tm->events && tm->count < tm->capacity;
  if (rec) {
    hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(tm->events[2 * tm->count]), st);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (rec && e == hipSuccess) {
    e = hipEventRecord(reinterpret_cast<hipEvent_t>(tm->events[2 * tm->count + 1]), st);
    if (kind <= OMQ_TIMED_GEMM_I8) tm->flops += work;
    if (kind == OMQ_TIMED_GEMM_I8) tm->flops_codes += work;
    if (tm->kinds) tm->kinds[tm->count] = kind;
    if (tm->work) tm->work[tm->count] = work;
    tm->count += 1;
  }
  return e;
}

// one linear's weight side: LET-W (s), LWC (theta logits), bias fold (delta)
hipError_t wfq(const void* W, int64_t rows, int64_t cols, const float* s, const float* delta,
               const float* th, const Theta& t, int l, int wbits, bool fp, uint16_t* out,
               const Stats& st, int64_t row0, float* Bt, int64_t group, uint8_t* codes,
               int64_t ldq, int code_off, int code_pack, hipStream_t stream, omq_timer* tm,
               int32_t* nf) {
  RowQuantFwd a;
  a.x = W; a.x_dt = OMQ_BF16; a.rows = rows; a.cols = cols; a.ldx = cols;
  a.let_mode = (s && !fp) ? OMQ_LET_MUL : OMQ_LET_NONE; a.s = s;
  a.nbits = fp ? 16 : wbits;
  a.a_gamma = fp ? nullptr : th + t.ag[l]; a.a_beta = fp ? nullptr : th + t.ab[l];
  a.out = out + row0 * cols; a.out_dt = OMQ_BF16; a.ldo = cols;
  // quantizer state of these rows: per output channel, or per (channel, group)
  const int64_t q0 = row0 * (group && a.nbits < 16 ? cols / group : 1);
  a.h = st.h + q0; a.z = st.z + q0; a.amax = st.amax + q0; a.amin = st.amin + q0;
  const bool grouped = group && a.nbits < 16;
  if (grouped) a.group = group;
  if (!fp && delta && !grouped) { a.fold_delta = delta; a.bias_out = Bt + row0; }
  if (codes && !fp) {
    a.codes = codes + row0 * ldq; a.ldq = ldq; a.code_off = code_off; a.qsum = st.qsum + row0;
    a.code_pack = code_pack;
  }
  if (!fp) a.nonfinite = nf;
  // algorithmic bytes: read W, write W_hat (and the codes)
  const double bytes =
      (double)rows * (double)cols * (4.0 + (a.codes ? (code_pack ? 0.5 : 1.0) : 0.0));
  hipError_t e = timed(fp ? nullptr : tm, OMQ_TIMED_WEIGHT_QUANT, bytes, stream,
                       [&] { return launch_rowquant_fwd(a, stream); });
  if (e == hipSuccess && !fp && delta && (a.nbits >= 16 || grouped))
    e = launch_bias_fold(W, OMQ_BF16, rows, cols, delta, nullptr, Bt + row0, stream);
  return e;
}

// the weight side of linears that share an input (q|k|v, gate|up): one launch over the
// concatenated rows where the whole-row quantizer applies, else one wfq per linear
hipError_t wfq_cat(int n, const void* const* Ws, const int64_t* rows, const int* ls,
                   int64_t cols, const float* s, const float* delta, const float* th, const Theta& t,
                   int wbits, bool fp, uint16_t* out, const Stats& st, float* Bt, int64_t group,
                   uint8_t* codes, int64_t ldq, int code_off, int code_pack, hipStream_t stream,
                   omq_timer* tm, int32_t* nf) {
  RowQuantFwd a;
  a.x = Ws[0]; a.x_dt = OMQ_BF16; a.cols = cols; a.ldx = cols; a.nbits = wbits;
  a.group = fp ? 0 : group;
  if (fp || !rowquant_fwd_segments_ok(a)) {
    int64_t r0 = 0;
    for (int k = 0; k < n; ++k) {
      hipError_t e = wfq(Ws[k], rows[k], cols, s, delta, th, t, ls[k], wbits, fp, out, st, r0,
                         Bt, group, codes, ldq, code_off, code_pack, stream, tm, nf);
      if (e != hipSuccess) return e;
      r0 += rows[k];
    }
    return hipSuccess;
  }
  a.nseg = n;
  int64_t r0 = 0;
  for (int k = 0; k < n; ++k) {
    a.xseg[k] = Ws[k];
    a.agseg[k] = th + t.ag[ls[k]];
    a.abseg[k] = th + t.ab[ls[k]];
    r0 += rows[k];
    a.seg_end[k] = r0;
  }
  a.rows = r0;
  a.let_mode = s ? OMQ_LET_MUL : OMQ_LET_NONE; a.s = s;
  a.out = out; a.out_dt = OMQ_BF16; a.ldo = cols;
  a.h = st.h; a.z = st.z; a.amax = st.amax; a.amin = st.amin;
  if (delta) { a.fold_delta = delta; a.bias_out = Bt; }
  if (codes) {
    a.codes = codes; a.ldq = ldq; a.code_off = code_off; a.qsum = st.qsum;
    a.code_pack = code_pack;
  }
  a.nonfinite = nf;
  // algorithmic bytes: read W, write W_hat (and the codes)
  const double bytes =
      (double)r0 * (double)cols * (4.0 + (a.codes ? (code_pack ? 0.5 : 1.0) : 0.0));
  return timed(tm, OMQ_TIMED_WEIGHT_QUANT, bytes, stream,
               [&] { return launch_rowquant_fwd(a, stream); });
}

// whether the per-token quantizer of a d-wide input can take its RMSNorm along
bool rms_fused(int x_dt, int64_t d, int abits, int mode) {
  RowQuantFwd p;
  p.x_dt = x_dt; p.cols = d; p.ldx = d; p.nbits = abits; p.let_mode = mode;
  return rowquant_fwd_rms_ok(p);
}

// per-token quantizer with fused LET on its input
hipError_t aq(const void* X, int x_dt, int64_t T, int64_t C, int64_t ldx, int mode,
              const float* s, const float* delta, int abits, uint16_t* out, const Stats& st,
              hipStream_t stream, omq_timer* tm, int32_t* nf, uint8_t* codes = nullptr,
              int64_t ldq = 0,
              int code_off = 0, int code_pack = 0, float* rms_out = nullptr,
              float* rstd = nullptr,
              float eps = 0.f, const float* rope_cos = nullptr, const float* rope_sin = nullptr,
              float* rope_out = nullptr) {
  RowQuantFwd a;
  a.x = X; a.x_dt = x_dt; a.rows = T; a.cols = C; a.ldx = ldx;
  a.rms_out = rms_out; a.rstd = rstd; a.eps = eps;
  a.rope_cos = rope_cos; a.rope_sin = rope_sin; a.rope_out = rope_out;
  a.let_mode = mode; a.s = s; a.delta = delta; a.nbits = abits;
  a.out = out; a.out_dt = OMQ_BF16; a.ldo = C;
  a.h = st.h; a.z = st.z; a.amax = st.amax; a.amin = st.amin;
  if (codes && abits < 16) {
    a.codes = codes; a.ldq = ldq; a.code_off = code_off; a.qsum = st.qsum; a.code_pack = code_pack;
  }
  if (abits < 16) a.nonfinite = nf;
  // algorithmic bytes: read X, write X_hat (and the codes, and the normalized or
  // rotated rows)
  const double bytes = (double)T * (double)C *
                       ((x_dt == OMQ_F32 ? 4.0 : 2.0) + 2.0 +
                        (a.codes ? (code_pack ? 0.5 : 1.0) : 0.0) +
                        (rms_out || rope_out ? 4.0 : 0.0));
  return timed(abits < 16 ? tm : nullptr, OMQ_TIMED_ACT_QUANT, bytes, stream,
               [&] { return launch_rowquant_fwd(a, stream); });
}

// whether aq can rotate float32 rows of C columns (row stride ldx) itself (RoPE)
bool aq_rope_ok(int64_t T, int64_t C, int64_t ldx, int abits) {
  RowQuantFwd a;
  a.x_dt = OMQ_F32; a.rows = T; a.cols = C; a.ldx = ldx; a.nbits = abits;
  a.out_dt = OMQ_BF16; a.ldo = C;
  static const float one = 1.f;
  a.rope_cos = a.rope_sin = &one;            // presence only
  return rowquant_fwd_rope_ok(a);
}

// n bytes (a multiple of 4, 4-byte aligned) set to zero by a fill kernel
hipError_t zero_bytes(void* p, int64_t n, hipStream_t st) {
  return launch_fill_f32(reinterpret_cast<float*>(p), n / 4, 0.f, st);
}

// every matrix-core launch of the step goes through here (optional event timing)
hipError_t run_gemm(const Gemm& g, hipStream_t st, omq_timer* tm) {
  const double f = 2.0 * (double)g.M * (double)g.N * (double)g.K * (double)g.batch;
  return timed(tm, g.codes ? OMQ_TIMED_GEMM_I8 : OMQ_TIMED_GEMM, f, st,
               [&] { return launch_gemm(g, st); });
}

hipError_t gemm(const void* A, int64_t lda, const void* B, int64_t ldb, float* C, int64_t ldc,
                int64_t M, int64_t N, int64_t K, const float* bias, const void* resid,
                int resid_dt, int64_t ldr, hipStream_t st, omq_timer* tm) {
  Gemm g;
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.M = M; g.N = N; g.K = K; g.bias = bias; g.resid = resid; g.resid_dt = resid_dt; g.ldr = ldr;
  return run_gemm(g, st, tm);
}

// the forward product Y = X_hat W_hat^T (+ bias) (+ resid) on the operands' integer
// codes: X [T x K] per-token, W [N x K] per-output-channel quantizer rows
// (code rows Kp long: K codes, then zero codes; stored codes shifted by the offsets)
hipError_t code_gemm(const uint8_t* qx, const Stats& sx, const uint8_t* qw, const Stats& sw,
                     float* C, int64_t ldc, int64_t T, int64_t N, int64_t K, int64_t Kp,
                     const Dims& m, const float* bias, const void* resid, int resid_dt,
                     int64_t ldr, hipStream_t st, omq_timer* tm) {
  Gemm g;
  g.codes = 1;
  // byte codes: rows of Kp (padded) codes; packed: rows of K / 2 bytes (Kp)
  g.pack4 = m.pk;
  g.A = qx; g.lda = Kp; g.B = qw; g.ldb = Kp; g.C = C; g.ldc = ldc;
  g.M = T; g.N = N; g.K = m.pk ? K : Kp; g.kz = K; g.bias = bias; g.resid = resid;
  g.resid_dt = resid_dt;
  g.ldr = ldr;
  g.ha = sx.h; g.za = sx.z; g.sa = sx.qsum; g.hb = sw.h; g.zb = sw.z; g.sb = sw.qsum;
  g.zoa = (float)m.aoff; g.zob = (float)m.woff;
  // timed with the algorithmic K
  const double f = 2.0 * (double)T * (double)N * (double)K;
  return timed(tm, OMQ_TIMED_GEMM_I8, f, st, [&] { return launch_gemm(g, st); });
}

#define CK(x)                               \
  do {                                      \
    hipError_t e__ = (x);                   \
    if (e__ != hipSuccess) return OMQ_E_HIP; \
  } while (0)

// The o-input LET pair and s_a live on the KV channels; with grouped-query
// attention they are broadcast over each group's query heads into workspace
// copies (and their gradients reduced back), with one query head per KV head the
// parameter vector itself serves (and the gradients go straight into dtheta,
// which the backward clears first).
struct KvSites {
  const float *s_o, *d_o, *sa_q;
  float *gs_o, *gd_o, *gsa_q;
};
KvSites kv_sites(const Dims& m, const Theta& t, const Ws& w, const float* th, float* dth) {
  KvSites k{};
  const bool bc = m.grp > 1;
  k.s_o = bc ? w.s_o_x : th + t.s_o;
  k.d_o = bc ? w.d_o_x : th + t.d_o;
  k.sa_q = bc || t.s_a < 0 ? w.sa_q : th + t.s_a;
  if (dth) {
    k.gs_o = bc ? w.gs_full : dth + t.s_o;
    k.gd_o = bc ? w.gd_full : dth + t.d_o;
    k.gsa_q = bc || t.s_a < 0 ? w.gsa_full : dth + t.s_a;
  }
  return k;
}

// Forward.  fp: the full-precision target (no quantizers, no LET).
int forward(const omq_block_desc* bd, const Dims& m, const Theta& t, const Ws& w, const void* x,
            const void* const* W, const float* th, bool fp, hipStream_t st) {
  omq_timer* tm = bd->timer;
  int32_t* const nf = fp ? nullptr : bd->nonfinite;   // the input-health flag
  const int64_t T = m.T, d = m.d, F = m.F, dq = m.dq, dk = m.dk, nqkv = m.nqkv;
  const int wb = fp ? 16 : bd->wbits, ab = fp ? 16 : bd->abits;
  const float* s_ffn = fp ? nullptr : th + t.s_ffn;
  const float* d_ffn = fp ? nullptr : th + t.d_ffn;
  const int mode_let = fp ? OMQ_LET_NONE : OMQ_LET_DIV;
  const float* xf = nullptr;  // FFN input
  int xf_dt = OMQ_F32;
  const bool cq = m.codes && !fp;  // forward products on integer codes
  if (!m.ffn_only) {
    const float* s_qkv = fp ? nullptr : th + t.s_qkv;
    const float* d_qkv = fp ? nullptr : th + t.d_qkv;
    if (!fp) {
      if (m.grp > 1) {
        CK(launch_kv_expand(th + t.s_o, m.nq, m.nkv, m.hd, w.s_o_x, st));
        CK(launch_kv_expand(th + t.d_o, m.nq, m.nkv, m.hd, w.d_o_x, st));
        if (m.use_sa) CK(launch_kv_expand(th + t.s_a, m.nq, m.nkv, m.hd, w.sa_q, st));
      }
    }
    const KvSites kv = kv_sites(m, t, w, th, nullptr);
    const float* s_o = fp ? nullptr : kv.s_o;
    if (cq && !m.pk && (m.dp != d || m.dqp != dq)) {
      // padded code rows: the columns past the row end must hold zero codes
      CK(zero_bytes(w.Cqkv, nqkv * m.dp, st));
      CK(zero_bytes(w.Co, d * m.dqp, st));
      CK(zero_bytes(w.Cxqkv, T * m.dp, st));
      CK(zero_bytes(w.Cxo, T * m.dqp, st));
    }
    const float* d_o = fp ? nullptr : kv.d_o;
    CK(launch_rope_tables(T, m.hd, bd->rope_theta, w.cos_t, w.sin_t, st));
    // weight side of q, k, v, o
    {
      const void* Wc[3] = {W[LQ], W[LK], W[LV]};
      const int64_t rc[3] = {dq, dk, dk};
      const int lc[3] = {LQ, LK, LV};
      CK(wfq_cat(3, Wc, rc, lc, d, s_qkv, d_qkv, th, t, wb, fp, w.Wqkv, w.wq_qkv, w.Bt_qkv,
                 m.group, cq ? w.Cqkv : nullptr, m.dp, m.woff, m.pk, st, tm, nf));
    }
    CK(wfq(W[LO], d, dq, s_o, d_o, th, t, LO, wb, fp, w.Wo, w.wq_o, 0, w.Bt_o, m.group,
           cq ? w.Co : nullptr, m.dqp, m.woff, m.pk, st, tm, nf));
    // attention input: the RMSNorm runs inside the quantizer where that applies
    if (rms_fused(OMQ_BF16, d, ab, mode_let)) {
      CK(aq(x, OMQ_BF16, T, d, d, mode_let, s_qkv, d_qkv, ab, w.Xqkv, w.a_qkv, st, tm, nf,
            cq ? w.Cxqkv : nullptr, m.dp, m.aoff, m.pk, w.xn, w.r1, bd->eps));
    } else {
      CK(launch_rmsnorm(x, OMQ_BF16, T, d, bd->eps, w.xn, w.r1, st));
      CK(aq(w.xn, OMQ_F32, T, d, d, mode_let, s_qkv, d_qkv, ab, w.Xqkv, w.a_qkv, st, tm, nf,
            cq ? w.Cxqkv : nullptr, m.dp, m.aoff, m.pk));
    }
    if (cq)
      CK(code_gemm(w.Cxqkv, w.a_qkv, w.Cqkv, w.wq_qkv, w.Yqkv, nqkv, T, nqkv, d, m.dp, m,
                   w.Bt_qkv, nullptr, 0, 0, st, tm));
    else
      CK(gemm(w.Xqkv, d, w.Wqkv, d, w.Yqkv, nqkv, T, nqkv, d, fp ? nullptr : w.Bt_qkv, nullptr,
              0, 0, st, tm));
    // RoPE, s_a on the affinity, then Q/K/V quantized per token; the per-token
    // quantizers of Q and K rotate their rows themselves where they can
    const bool sa = m.use_sa && !fp;
    if (aq_rope_ok(T, dq, nqkv, ab) && aq_rope_ok(T, dk, nqkv, ab)) {
      CK(aq(w.Yqkv, OMQ_F32, T, dq, nqkv, sa ? OMQ_LET_DIV : OMQ_LET_NONE, kv.sa_q, nullptr, ab,
            w.Qh, w.a_q, st, tm, nf, nullptr, 0, 0, 0, nullptr, nullptr, 0.f, w.cos_t, w.sin_t,
            w.Qr));
      CK(aq(w.Yqkv + dq, OMQ_F32, T, dk, nqkv, sa ? OMQ_LET_MUL : OMQ_LET_NONE,
            th + (sa ? t.s_a : 0), nullptr, ab, w.Kh, w.a_k, st, tm, nf, nullptr, 0, 0, 0, nullptr,
            nullptr, 0.f, w.cos_t, w.sin_t, w.Kr));
    } else {
      CK(launch_rope2(w.Yqkv, nqkv, w.Qr, dq, m.nq, w.Yqkv + dq, nqkv, w.Kr, dk, m.nkv, T, m.hd,
                      w.cos_t, w.sin_t, 0, st));
      CK(aq(w.Qr, OMQ_F32, T, dq, dq, sa ? OMQ_LET_DIV : OMQ_LET_NONE, kv.sa_q, nullptr, ab, w.Qh,
            w.a_q, st, tm, nf));
      CK(aq(w.Kr, OMQ_F32, T, dk, dk, sa ? OMQ_LET_MUL : OMQ_LET_NONE, th + (sa ? t.s_a : 0),
            nullptr, ab, w.Kh, w.a_k, st, tm, nf));
    }
    CK(aq(w.Yqkv + dq + dk, OMQ_F32, T, dk, nqkv, OMQ_LET_NONE, nullptr, nullptr, ab, w.Vh, w.a_v,
          st, tm, nf));
    // causal attention, float32 softmax, fused
    {
      FlashFwd f;
      f.Q = w.Qh; f.K = w.Kh; f.V = w.Vh; f.ldq = dq; f.ldk = dk; f.T = T;
      f.n_q = (int)m.nq; f.grp = (int)m.grp;
      f.scale2 = (float)(1.4426950408889634 / sqrt((double)m.hd));
      f.O = w.O; f.ldo = dq; f.lse2 = w.lse2;
      CK(launch_flash_fwd(f, st));
    }
    // o_proj with its LET site, residual
    CK(aq(w.O, OMQ_F32, T, dq, dq, mode_let, s_o, d_o, ab, w.Xo, w.a_o, st, tm, nf,
          cq ? w.Cxo : nullptr, m.dqp, m.aoff, m.pk));
    if (cq)
      CK(code_gemm(w.Cxo, w.a_o, w.Co, w.wq_o, w.h1, d, T, d, dq, m.dqp, m, w.Bt_o, x, OMQ_BF16,
                   d, st, tm));
    else
      CK(gemm(w.Xo, dq, w.Wo, dq, w.h1, d, T, d, dq, fp ? nullptr : w.Bt_o, x, OMQ_BF16, d, st,
              tm));
    // the FFN input's RMSNorm runs inside its quantizer where that applies
    if (!rms_fused(OMQ_F32, d, ab, mode_let))
      CK(launch_rmsnorm(w.h1, OMQ_F32, T, d, bd->eps, w.xn2, w.r2, st));
    xf = w.xn2;
    xf_dt = OMQ_F32;
  } else {
    xf = reinterpret_cast<const float*>(x);
    xf_dt = OMQ_BF16;
  }
  // FFN
  if (cq && !m.pk && (m.dp != d || m.Fp != F)) {
    CK(zero_bytes(w.Cgu, 2 * F * m.dp, st));
    CK(zero_bytes(w.Cd, d * m.Fp, st));
    CK(zero_bytes(w.Cxf, T * m.dp, st));
    CK(zero_bytes(w.Cxd, T * m.Fp, st));
  }
  {
    const void* Wc[2] = {W[LG], W[LU]};
    const int64_t rc[2] = {F, F};
    const int lc[2] = {LG, LU};
    CK(wfq_cat(2, Wc, rc, lc, d, s_ffn, d_ffn, th, t, wb, fp, w.Wgu, w.wq_gu, w.Bt_gu, m.group,
               cq ? w.Cgu : nullptr, m.dp, m.woff, m.pk, st, tm, nf));
  }
  CK(wfq(W[LD], d, F, nullptr, nullptr, th, t, LD, wb, fp, w.Wd, w.wq_d, 0, nullptr, m.group,
         cq ? w.Cd : nullptr, m.Fp, m.woff, m.pk, st, tm, nf));
  if (!m.ffn_only && rms_fused(OMQ_F32, d, ab, mode_let))
    CK(aq(w.h1, OMQ_F32, T, d, d, mode_let, s_ffn, d_ffn, ab, w.Xf, w.a_f, st, tm, nf,
          cq ? w.Cxf : nullptr, m.dp, m.aoff, m.pk, w.xn2, w.r2, bd->eps));
  else
    CK(aq(xf, xf_dt, T, d, d, mode_let, s_ffn, d_ffn, ab, w.Xf, w.a_f, st, tm, nf,
          cq ? w.Cxf : nullptr, m.dp, m.aoff, m.pk));
  if (cq)
    CK(code_gemm(w.Cxf, w.a_f, w.Cgu, w.wq_gu, w.GU, 2 * F, T, 2 * F, d, m.dp, m, w.Bt_gu,
                 nullptr, 0, 0, st, tm));
  else
    CK(gemm(w.Xf, d, w.Wgu, d, w.GU, 2 * F, T, 2 * F, d, fp ? nullptr : w.Bt_gu, nullptr, 0, 0,
            st, tm));
  CK(launch_silu_gate(w.GU, T, F, w.A, st));
  CK(aq(w.A, OMQ_F32, T, F, F, OMQ_LET_NONE, nullptr, nullptr, ab, w.Xd, w.a_d, st, tm, nf,
        cq ? w.Cxd : nullptr, m.Fp, m.aoff, m.pk));
  if (cq)
    CK(code_gemm(w.Cxd, w.a_d, w.Cd, w.wq_d, w.y, d, T, d, F, m.Fp, m, nullptr,
                 m.ffn_only ? nullptr : w.h1, OMQ_F32, d, st, tm));
  else
    CK(gemm(w.Xd, F, w.Wd, F, w.y, d, T, d, F, nullptr, m.ffn_only ? nullptr : w.h1, OMQ_F32, d,
            st, tm));
  return OMQ_OK;
}

// activation-side backward through the per-token quantizer and the fused LET
hipError_t abwd(const Ws& w, const float* g, int64_t T, int64_t C, const void* X, int x_dt,
                int64_t ldx, int mode, const float* s, const float* delta, int abits,
                const Stats& st, float* gx, int64_t ldgx, int col_mode, float* out0, float* out1,
                int accumulate, hipStream_t stream, float* part = nullptr,
                SteFinJob* job = nullptr) {
  RowQuantBwd a;
  a.g = g; a.ldg = C; a.x = X; a.x_dt = x_dt; a.rows = T; a.cols = C; a.ldx = ldx;
  a.let_mode = mode; a.s = s; a.delta = delta; a.nbits = abits;
  a.h = st.h; a.z = st.z; a.amax = st.amax; a.amin = st.amin;
  a.col_mode = col_mode; a.gx = gx; a.ldgx = ldgx;
  a.out0 = out0; a.out1 = out1; a.accumulate = accumulate; a.ws = part ? part : w.rq;
  return launch_rowquant_bwd_tiles(a, stream, job);
}

// The backward of one (possibly concatenated) quantized linear with both
// straight-through passes fused into its GEMM epilogues:
//   dW = dY^T X_hat with the LWC / LET-W backward of every weight row in the
//   epilogue (no fp32 dW in HBM), then per-segment row finalizers;
//   dX_hat = dY W_hat with the per-token quantizer / LET-X backward in the
//   epilogue, which writes dL/dX (gx_out) directly.
struct WSeg {
  const void* W;
  int64_t rows;
  int l;
};

struct LinBwd {
  // the linear: gY [T x N] float, X_hat [T x K] bf16, W_hat [N x K] bf16
  const float* gY;
  int64_t N, K;
  const uint16_t* Xh;
  const uint16_t* Wh;
  uint16_t* gYb;
  bool have_gYb;         // gYb (and, with fold, its column sums) already formed
  // weight side
  const WSeg* segs;
  int nseg;
  Stats wst;
  const float* s_w;      // LET scale on W (NULL: none)
  bool fold;             // bias fold with delta (needs column sums of dY)
  float* gs_w;           // gradients of the LET pair: added to (running totals)
  float* gd_w;
  int64_t group;         // LWC group along K (0 or 128)
  // activation side
  const void* X;
  int x_dt;
  int a_mode;
  const float* s_x;
  const float* d_x;
  Stats ast;
  float* gx_out;         // dL/dX [T x K]
  float* gs_x;
  float* gd_x;
  // q|k|v: the Q and K columns of gY come from their rotated gradients (inverse RoPE
  // on the way to the bf16 copy); NULL otherwise
  const RopeIn* rope;
  // the weight side's partials in a buffer of their own (else the shared w.rq), and
  // its finalizers queued there instead of launched (else launched at once)
  float* wpart;
  struct FinQueue* defer;
  // the activation side's partials in a buffer of their own (else w.rq): its column
  // pass queued (its row finalizers too when dL/dX is not written)
  float* xpart;
};

// Straight-through work queued by the layers' backward passes: the weight sides'
// finalizers, the q|k|v input's (no dL/dx written there) and every column pass.
// Nothing reads their outputs (the logit gradients, the LET and s_a column totals)
// before the update, so they run together once every GEMM is done: one row-finalizer
// launch per kernel instance and two rounds of column passes for the whole block.
struct FinQueue {
  SteFinJob job[kMaxFinJobs];
  int n = 0;
  bool room() const { return n < kMaxFinJobs; }
  void push(const SteFinJob& j) { job[n++] = j; }
  hipError_t flush(hipStream_t st) {
    const hipError_t e = launch_ste_finish_multi(job, n, st);
    n = 0;
    return e;
  }
};

hipError_t lin_bwd_fused(const Ws& w, const LinBwd& L, int64_t T, int wbits, int abits,
                         const float* th, const Theta& t, float* dth, hipStream_t st,
                         omq_timer* tm) {
  hipError_t e;
  const int64_t N = L.N, K = L.K;
  if (!L.have_gYb) {
    e = L.rope ? launch_cvt_bf16_colsum_rope(L.gY, T, N, *L.rope, L.gYb,
                                             L.fold ? w.cs : nullptr, w.csws, st)
               : launch_cvt_bf16_colsum(L.gY, T, N, L.gYb, L.fold ? w.cs : nullptr, w.csws, st);
    if (e != hipSuccess) return e;
  }
  int64_t nsl, ntl;
  // weight side (skipped when no learnable parameter depends on these weights)
  if (wbits < 16 || L.s_w) {
    gemm_ste_extents(N, K, &nsl, &ntl);
    float* const base = L.wpart ? L.wpart : w.rq;
    float* rowpart = base;
    float* colpart = base + nsl * N * 2;
    Gemm g;
    g.A = L.gYb; g.lda = N; g.ta = 1; g.B = L.Xh; g.ldb = K; g.tb = 1;
    g.C = nullptr; g.ldc = K; g.M = N; g.N = K; g.K = T;
    SteEpi& se = g.ste;
    se.mode = 1; se.nseg = L.nseg;
    int64_t r0 = 0;
    for (int k = 0; k < L.nseg; ++k) {
      r0 += L.segs[k].rows;
      se.seg_end[k] = r0;
      se.xseg[k] = L.segs[k].W;
    }
    se.x_dt = OMQ_BF16; se.ldx = K;
    se.let_mode = L.s_w ? OMQ_LET_MUL : OMQ_LET_NONE; se.s = L.s_w;
    se.h = L.wst.h; se.z = L.wst.z; se.nbits = wbits;
    se.rowvec = L.fold ? w.cs : nullptr;
    se.col_mode = L.s_w ? COL_WEIGHT : COL_NONE;
    se.rowpart = rowpart; se.colpart = colpart;
    const bool grouped = L.group > 0 && wbits < 16;
    se.grouped = grouped;        // one 128-column tile of a row = one group
    if ((e = run_gemm(g, st, tm)) != hipSuccess) return e;
    RowQuantBwd a;
    a.cols = K; a.col_mode = se.col_mode; a.out0 = L.gs_w; a.out1 = L.fold ? L.gd_w : nullptr;
    a.accumulate = 1;     // running totals of the LET pair's gradients
    // one finalizer launch over the concatenated rows, each segment with its own
    // weight rows and logits
    RowQuantBwd b;
    b.x = L.segs[0].W; b.x_dt = OMQ_BF16; b.rows = r0; b.cols = K; b.ldx = K;
    b.let_mode = se.let_mode; b.s = L.s_w; b.nbits = wbits;
    b.h = L.wst.h; b.z = L.wst.z; b.amax = L.wst.amax; b.amin = L.wst.amin;
    b.a_gamma = th + t.ag[L.segs[0].l]; b.a_beta = th + t.ab[L.segs[0].l];
    b.g_agamma = dth + t.ag[L.segs[0].l]; b.g_abeta = dth + t.ab[L.segs[0].l];
    b.nseg = L.nseg;
    for (int k = 0; k < L.nseg; ++k) {
      const WSeg& sg = L.segs[k];
      b.seg_end[k] = se.seg_end[k];
      b.xseg[k] = sg.W;
      b.agseg[k] = th + t.ag[sg.l]; b.abseg[k] = th + t.ab[sg.l];
      b.gagseg[k] = dth + t.ag[sg.l]; b.gabseg[k] = dth + t.ab[sg.l];
    }
    b.col_mode = se.col_mode; b.out0 = L.gs_w;
    if (grouped) b.group = L.group;
    // the row finalizers, then the column sums with their scatter terms (both into gs_w)
    if (L.defer && L.wpart && L.defer->room()) {
      SteFinJob j;
      j.rf = b; j.nslabs = grouped ? 1 : (int)nsl; j.tile_rows = kSteTileRows;
      j.ntiles = (int)ntl; j.rowpart = rowpart; j.colpart = colpart;
      j.cols = a.cols; j.col_mode = a.col_mode; j.out0 = a.out0; j.out1 = a.out1;
      j.accumulate = a.accumulate;
      L.defer->push(j);
    } else if ((e = launch_ste_finish(a, (int)ntl, colpart, b, grouped ? 1 : (int)nsl, rowpart,
                                      kSteTileRows, st)) != hipSuccess) {
      return e;
    }
  }
  // activation side
  gemm_ste_extents(T, K, &nsl, &ntl);
  float* const xbase = L.xpart ? L.xpart : w.rq;
  float* rowpart = xbase;
  float* colpart = xbase + nsl * T * 2;
  Gemm g;
  g.A = L.gYb; g.lda = N; g.B = L.Wh; g.ldb = K; g.tb = 1;
  g.C = L.gx_out; g.ldc = K; g.M = T; g.N = K; g.K = N;
  SteEpi& se = g.ste;
  const int acol = L.a_mode == OMQ_LET_DIV ? COL_ACT_DIV : COL_NONE;
  se.mode = 2; se.nseg = 1; se.seg_end[0] = T; se.xseg[0] = L.X;
  se.x_dt = L.x_dt; se.ldx = K;
  se.let_mode = L.a_mode; se.s = L.s_x; se.delta = L.d_x;
  se.h = L.ast.h; se.z = L.ast.z; se.nbits = abits;
  se.col_mode = acol; se.rowpart = rowpart; se.colpart = colpart;
  if ((e = run_gemm(g, st, tm)) != hipSuccess) return e;
  RowQuantBwd a;
  a.x = L.X; a.x_dt = L.x_dt; a.rows = T; a.cols = K; a.ldx = K;
  a.let_mode = L.a_mode; a.s = L.s_x; a.delta = L.d_x; a.nbits = abits;
  a.h = L.ast.h; a.z = L.ast.z; a.amax = L.ast.amax; a.amin = L.ast.amin;
  a.col_mode = acol; a.gx = L.gx_out; a.ldgx = K;
  a.out0 = L.gs_x; a.out1 = L.gd_x; a.accumulate = 1;
  const bool cols_out = acol != COL_NONE && (a.out0 || a.out1) && K > 0;
  if (L.defer && L.xpart && cols_out && L.defer->room()) {
    SteFinJob j;
    j.rf = a; j.nslabs = (int)nsl; j.tile_rows = kSteTileRows; j.ntiles = (int)ntl;
    j.rowpart = rowpart; j.colpart = colpart;
    j.cols = K; j.col_mode = acol; j.out0 = a.out0; j.out1 = a.out1; j.accumulate = 1;
    if (L.gx_out) {
      // the row finalizers now (their scatter completes dL/dX for the next stage),
      // merging into this layer's own column partials; the column pass queued
      if ((e = launch_ste_finish_rows(a, colpart, a, (int)nsl, rowpart, kSteTileRows, st)) !=
          hipSuccess)
        return e;
      j.rf.rows = 0;
    }
    L.defer->push(j);
    return hipSuccess;
  }
  return launch_ste_finish(a, (int)ntl, colpart, a, (int)nsl, rowpart, kSteTileRows, st);
}

int backward(const omq_block_desc* bd, const Dims& m, const Theta& t, const Ws& w,
             const void* x, const void* const* W, const float* th, float* dth, hipStream_t st,
             bool dyb_ready) {
  omq_timer* tm = bd->timer;
  const int64_t T = m.T, d = m.d, F = m.F, dq = m.dq, dk = m.dk, nqkv = m.nqkv;
  const int wb = bd->wbits, ab = bd->abits;
  CK(launch_fill_f32(dth, t.total, 0.f, st));
  FinQueue fq;          // the weight side's finalizers, run after the last GEMM
  // the column sums add into their destinations: the o-site LET gradients of grouped
  // heads are formed per query channel first
  if (!m.ffn_only && m.grp > 1) {
    CK(launch_fill_f32(w.gs_full, m.dq, 0.f, st));
    CK(launch_fill_f32(w.gd_full, m.dq, 0.f, st));
  }
  // FFN second linear (no LET): its input is A = SiLU(G) * U
  {
    const WSeg segs[1] = {{W[LD], d, LD}};
    LinBwd L{};
    L.group = m.group;
    L.gY = w.dy; L.N = d; L.K = F; L.Xh = w.Xd; L.Wh = w.Wd; L.gYb = w.dyb;
    L.have_gYb = dyb_ready;            // no LET on down: no column sums needed
    L.segs = segs; L.nseg = 1; L.wst = w.wq_d;
    L.X = w.A; L.x_dt = OMQ_F32; L.a_mode = OMQ_LET_NONE; L.ast = w.a_d; L.gx_out = w.gA;
    L.wpart = w.wpart[3]; L.defer = &fq;
    CK(lin_bwd_fused(w, L, T, wb, ab, th, t, dth, st, tm));
  }
  // dL/d(gate|up) goes straight to its bf16 operand form with its column sums
  const bool gu_bf16 = silu_gate_bwd_bf16_fits(w.GU, w.gA, T, F, w.gGUb);
  if (gu_bf16)
    CK(launch_silu_gate_bwd_bf16(w.GU, w.gA, T, F, w.gGUb, w.cs, w.csws, st));
  else
    CK(launch_silu_gate_bwd(w.GU, w.gA, T, F, w.gGU, st));
  // gate / up with the shared ffn LET site
  {
    const WSeg segs[2] = {{W[LG], F, LG}, {W[LU], F, LU}};
    LinBwd L{};
    L.group = m.group;
    L.gY = w.gGU; L.N = 2 * F; L.K = d; L.Xh = w.Xf; L.Wh = w.Wgu; L.gYb = w.gGUb;
    L.have_gYb = gu_bf16;
    L.segs = segs; L.nseg = 2; L.wst = w.wq_gu; L.s_w = th + t.s_ffn; L.fold = true;
    L.gs_w = dth + t.s_ffn; L.gd_w = dth + t.d_ffn;
    L.X = m.ffn_only ? x : (const void*)w.xn2; L.x_dt = m.ffn_only ? OMQ_BF16 : OMQ_F32;
    L.a_mode = OMQ_LET_DIV; L.s_x = th + t.s_ffn; L.d_x = th + t.d_ffn; L.ast = w.a_f;
    L.gx_out = m.ffn_only ? nullptr : w.gxn2; L.gs_x = dth + t.s_ffn; L.gd_x = dth + t.d_ffn;
    L.wpart = w.wpart[2]; L.xpart = w.xpart[0]; L.defer = &fq;
    CK(lin_bwd_fused(w, L, T, wb, ab, th, t, dth, st, tm));
  }
  if (m.ffn_only) {
    CK(fq.flush(st));
    return OMQ_OK;
  }
  const KvSites kv = kv_sites(m, t, w, th, dth);

  // RMSNorm before the FFN, residual
  CK(launch_rmsnorm_bwd(w.gxn2, w.h1, w.r2, T, d, w.dy, w.dh1, st));
  // o_proj with its LET site (per KV channel, broadcast over the query heads)
  {
    const WSeg segs[1] = {{W[LO], d, LO}};
    LinBwd L{};
    L.group = m.group;
    L.gY = w.dh1; L.N = d; L.K = dq; L.Xh = w.Xo; L.Wh = w.Wo; L.gYb = w.dh1b;
    L.segs = segs; L.nseg = 1; L.wst = w.wq_o; L.s_w = kv.s_o; L.fold = true;
    L.gs_w = kv.gs_o; L.gd_w = kv.gd_o;
    L.X = w.O; L.x_dt = OMQ_F32; L.a_mode = OMQ_LET_DIV; L.s_x = kv.s_o; L.d_x = kv.d_o;
    L.ast = w.a_o; L.gx_out = w.gO; L.gs_x = kv.gs_o; L.gd_x = kv.gd_o;
    L.wpart = w.wpart[1]; L.xpart = w.xpart[1]; L.defer = &fq;
    CK(lin_bwd_fused(w, L, T, wb, ab, th, t, dth, st, tm));
  }
  // attention backward (scores recomputed from the forward's log-sum-exp; dQ from the
  // dS the dK/dV pass writes)
  CK(launch_attn_bwd_prep(w.gO, w.O, dq, T, (int)m.nq, w.Datt, w.gOb, dq, st));
  {
    FlashBwd f;
    f.Q = w.Qh; f.K = w.Kh; f.V = w.Vh; f.dO = w.gOb; f.ldq = dq; f.ldk = dk; f.T = T;
    f.n_q = (int)m.nq; f.grp = (int)m.grp;
    f.scale = (float)(1.0 / sqrt((double)m.hd));
    f.scale2 = (float)(1.4426950408889634 / sqrt((double)m.hd));
    f.lse2 = w.lse2; f.D = w.Datt;
    f.dQ = w.gQh; f.lddq = dq; f.dK = w.gKh; f.dV = w.gVh; f.lddk = dk;
    f.part = w.attn_part; f.ds = w.attn_ds;
    CK(launch_flash_bwd(f, st));
  }
  // Q~ / K~ / V quantizers and s_a
  // (the three tile passes, then their finalizers together: each has partial buffers
  // of its own; the Q and K column passes, both into s_a without grouped heads, keep
  // their order)
  const bool sa = m.use_sa;
  SteFinJob qkvj[3];
  CK(abwd(w, w.gQh, T, dq, w.Qr, OMQ_F32, dq, sa ? OMQ_LET_DIV : OMQ_LET_NONE, kv.sa_q, nullptr,
          ab, w.a_q, w.gQr, dq, sa ? COL_ACT_DIV : COL_NONE, sa ? kv.gsa_q : nullptr, nullptr,
          m.grp > 1 ? 0 : 1,
          st, w.apart[0], &qkvj[0]));
  CK(abwd(w, w.gKh, T, dk, w.Kr, OMQ_F32, dk, sa ? OMQ_LET_MUL : OMQ_LET_NONE,
          sa ? th + t.s_a : nullptr, nullptr, ab, w.a_k, w.gKr, dk, sa ? COL_ACT_MUL : COL_NONE,
          sa ? dth + t.s_a : nullptr, nullptr, 1, st, w.apart[1], &qkvj[1]));
  CK(abwd(w, w.gVh, T, dk, w.Yqkv + dq + dk, OMQ_F32, nqkv, OMQ_LET_NONE, nullptr, nullptr, ab,
          w.a_v, w.gY + dq + dk, nqkv, COL_NONE, nullptr, nullptr, 0, st, w.apart[2], &qkvj[2]));
  // their row finalizers now (the scatter completes the gradients the q|k|v backward
  // reads), their column passes (s_a) queued
  for (SteFinJob& j : qkvj) j.skip_cols = true;
  CK(launch_ste_finish_multi(qkvj, 3, st));
  for (SteFinJob& j : qkvj) {
    if (j.col_mode == COL_NONE || !(j.out0 || j.out1) || j.cols == 0) continue;
    SteFinJob c = j;
    c.rf.rows = 0;
    c.skip_cols = false;
    if (fq.room()) {
      fq.push(c);
    } else {
      CK(launch_ste_finish_multi(&c, 1, st));
    }
  }
  // q / k / v with the shared qkv LET site; the inverse RoPE of the Q and K gradients
  // runs inside the bf16 conversion of dL/dY
  {
    const RopeIn rp{w.gQr, dq, dq, w.gKr, dk, dk, w.cos_t, w.sin_t};
    const WSeg segs[3] = {{W[LQ], dq, LQ}, {W[LK], dk, LK}, {W[LV], dk, LV}};
    LinBwd L{};
    L.group = m.group;
    L.gY = w.gY; L.N = nqkv; L.K = d; L.Xh = w.Xqkv; L.Wh = w.Wqkv; L.gYb = w.gYb;
    L.segs = segs; L.nseg = 3; L.wst = w.wq_qkv; L.s_w = th + t.s_qkv; L.fold = true;
    L.gs_w = dth + t.s_qkv; L.gd_w = dth + t.d_qkv;
    L.X = w.xn; L.x_dt = OMQ_F32; L.a_mode = OMQ_LET_DIV; L.s_x = th + t.s_qkv;
    // dL/dx of the block input is not needed (x is no parameter): not written
    L.d_x = th + t.d_qkv; L.ast = w.a_qkv; L.gx_out = nullptr;
    L.gs_x = dth + t.s_qkv; L.gd_x = dth + t.d_qkv;
    L.rope = &rp;
    L.wpart = w.wpart[0]; L.xpart = w.xpart[2]; L.defer = &fq;
    CK(lin_bwd_fused(w, L, T, wb, ab, th, t, dth, st, tm));
  }
  CK(fq.flush(st));
  // the o-site LET and s_a gradients of grouped heads, per query channel until here,
  // summed over each group
  if (m.grp > 1) {
    CK(launch_kv_reduce_add(w.gs_full, m.nq, m.nkv, m.hd, dth + t.s_o, st));
    CK(launch_kv_reduce_add(w.gd_full, m.nq, m.nkv, m.hd, dth + t.d_o, st));
    if (sa) CK(launch_kv_reduce_add(w.gsa_full, m.nq, m.nkv, m.hd, dth + t.s_a, st));
  }
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
  // dL/dy also in bf16 (the down product's operand) when the target is 16-byte aligned
  const bool dyb = al16(y_target);
  OMQ_HIP_CHECK(
      launch_mse(w.y, y_target, m.T * m.d, loss, w.dy, w.msews, st, dyb ? w.dyb : nullptr));
  rc = backward(d, m, t, w, x, weights, theta, dtheta, st, dyb);
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
