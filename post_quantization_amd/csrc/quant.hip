// Row quantizer kernels for OmniQuant calibration on gfx950.
//
// Forward: the LWC equation of the paper reading (section "LWC") applied per row,
// with the LET transform of the row's input fused in (section "LET").  Rows are
// weight output channels (LWC, gamma/beta from sigmoid logits) or tokens (per-token
// activation quantizer, gamma = beta = 1).
//
// Backward: the straight-through rule (rint is the identity; clamp, max/min, h and
// z differentiated exactly) as a 2-D tile pass plus two small finalizers, the same
// decomposition a GEMM epilogue can produce.
#include "common.h"
#include "kernels.h"

#include <algorithm>

#include <float.h>

namespace omq {

namespace {

constexpr int kThreads = 256;
constexpr int kSlab = 1024;   // columns per thread block in the tile pass (256 x 4)

OMQ_DEV float let_x(float x, int mode, const float* s, const float* delta, int64_t c) {
  if (mode == OMQ_LET_DIV) {
    float dl = delta ? delta[c] : 0.f;
    return (x - dl) / s[c];
  }
  if (mode == OMQ_LET_MUL) return s[c] * x;
  return x;
}

// row stride of the codes output, in bytes
OMQ_DEV int64_t code_ld(const RowQuantFwd& a) {
  return a.ldq ? a.ldq : a.code_pack ? a.cols / 2 : a.cols;
}

// Code stores: 4 or 8 consecutive codes (one per byte of cw) of row r from column c,
// as bytes, or two to a byte when code_pack is set (byte c / 2 holds codes c, c + 1 in
// its low and high nibble).
OMQ_DEV uint32_t nibble_pack4(uint32_t w) {   // bytes b0..b3 (each < 16) -> b0|b1<<4|b2<<8|b3<<12
  const uint32_t t = w | (w >> 4);
  return (t & 0xffu) | ((t >> 8) & 0xff00u);
}
OMQ_DEV void store_codes4(const RowQuantFwd& a, int64_t r, int64_t c, uint32_t cw) {
  if (a.code_pack)
    *reinterpret_cast<uint16_t*>(a.codes + r * code_ld(a) + (c >> 1)) = (uint16_t)nibble_pack4(cw);
  else
    *reinterpret_cast<uint32_t*>(a.codes + r * code_ld(a) + c) = cw;
}
OMQ_DEV void store_codes8(const RowQuantFwd& a, int64_t r, int64_t c, uint32_t lo, uint32_t hi) {
  if (a.code_pack)
    *reinterpret_cast<uint32_t*>(a.codes + r * code_ld(a) + (c >> 1)) =
        nibble_pack4(lo) | (nibble_pack4(hi) << 16);
  else
    *reinterpret_cast<uint2*>(a.codes + r * code_ld(a) + c) = make_uint2(lo, hi);
}

// a row's extreme-value column, kept inside the row: with a NaN in the row the
// comparisons of the reductions never pick it, and lanes that held no column could
// leave their sentinel index
OMQ_DEV int col_in(int i, int64_t cols) { return (i >= 0 && (int64_t)i < cols) ? i : 0; }

// the input flag: set when any lane of the wave saw a NaN or infinite x~ (every
// lane of the wave calls it; the flag is only ever set, never cleared)
OMQ_DEV void flag_nonfinite(int32_t* flag, bool nf) {
  if (__builtin_amdgcn_ballot_w64(nf) != 0 && (threadIdx.x & 63) == 0) *flag = 1;
}

// the block's code sum into *out (every thread of the 4-wave block calls it)
OMQ_DEV void block_qsum(int qs, int32_t* out) {
  __shared__ int s_qs[4];
  qs = wave_sum(qs);
  if ((threadIdx.x & 63) == 0) s_qs[wave_id()] = qs;
  __syncthreads();
  if (threadIdx.x == 0) *out = s_qs[0] + s_qs[1] + s_qs[2] + s_qs[3];
}

// ---------------------------------------------------------------------------
// chunk helpers of the whole-row forward kernels: a lane holds 8 consecutive
// elements of x~ at a time
// ---------------------------------------------------------------------------
// largest and smallest of 8 values (three-operand max / min; a NaN operand is
// passed over, as the comparisons of an element-wise scan pass it over)
OMQ_DEV float max8(const float (&v)[8]) {
  return fmaxf(fmaxf(fmaxf(fmaxf(v[0], v[1]), v[2]), fmaxf(fmaxf(v[3], v[4]), v[5])),
               fmaxf(v[6], v[7]));
}
OMQ_DEV float min8(const float (&v)[8]) {
  return fminf(fminf(fminf(fminf(v[0], v[1]), v[2]), fminf(fminf(v[3], v[4]), v[5])),
               fminf(v[6], v[7]));
}
OMQ_DEV float wave_maxf(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
OMQ_DEV float wave_minf(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}
// the first of 8 values equal to v (float comparison, so -0 == +0): its position
// in j (8 when none is) and its own value in x
OMQ_DEV void first_eq8(const float (&t)[8], float v, int& j, float& x) {
  j = 8;
#pragma unroll
  for (int q = 7; q >= 0; --q)
    if (t[q] == v) { j = q; x = t[q]; }
}
// finiteness accumulator: x * 0 is 0 for a finite x and NaN for an infinite or NaN
// one, so acc stays finite exactly while every element is finite
OMQ_DEV float nf_acc8(const float (&v)[8], float acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = fmaf(v[j], 0.f, acc);
  return acc;
}
// the codes of 8 elements: q (integer-valued floats in [0, 255]) as the bytes
// q - off (off 0 or 128: then the byte is q xor 0x80), their sum of q added to qsum
OMQ_DEV uint2 codes8(const float (&q)[8], bool off128, uint32_t& qsum) {
  uint32_t lo = 0u, hi = 0u;
  lo = __builtin_amdgcn_cvt_pk_u8_f32(q[0], 0, lo);
  lo = __builtin_amdgcn_cvt_pk_u8_f32(q[1], 1, lo);
  lo = __builtin_amdgcn_cvt_pk_u8_f32(q[2], 2, lo);
  lo = __builtin_amdgcn_cvt_pk_u8_f32(q[3], 3, lo);
  hi = __builtin_amdgcn_cvt_pk_u8_f32(q[4], 0, hi);
  hi = __builtin_amdgcn_cvt_pk_u8_f32(q[5], 1, hi);
  hi = __builtin_amdgcn_cvt_pk_u8_f32(q[6], 2, hi);
  hi = __builtin_amdgcn_cvt_pk_u8_f32(q[7], 3, hi);
  qsum = __builtin_amdgcn_udot4(lo, 0x01010101u, qsum, false);
  qsum = __builtin_amdgcn_udot4(hi, 0x01010101u, qsum, false);
  if (off128) {
    lo ^= 0x80808080u;
    hi ^= 0x80808080u;
  }
  return make_uint2(lo, hi);
}
// rint(x~ / h) of a chunk by the reciprocal product u = x~ rh, which lies within 3
// ulp of the exact quotient: the two can round apart only within |u| 2^-20 of a
// half-integer, and thr (the row's bound max|x~| rh 2^-20) covers every element, so a
// chunk whose smallest distance | |u - rint u| - 1/2 | is not above thr takes the
// exact quotient, behind a wave-uniform branch (a divergent one would be flattened
// into a division for every element).  f = u - rint u is exact and |f| <= 1/2, so
// that smallest distance is 1/2 - max |f| (rounding is monotone: the same float as
// the smallest of the rounded distances).  A NaN f (u infinite or NaN) is passed
// over: both quotients then clamp to the same code.
OMQ_DEV void rint_quot8(const float (&xt)[8], float h, float rh, float thr, bool in,
                        float (&rr)[8]) {
  float fm = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float u = xt[j] * rh;
    rr[j] = rintf(u);
    fm = fmaxf(fm, fabsf(u - rr[j]));
  }
  const bool near = in && !(0.5f - fm > thr);
  if (__builtin_amdgcn_ballot_w64(near) != 0) {
    if (near) {
#pragma unroll
      for (int j = 0; j < 8; ++j) rr[j] = rintf(xt[j] / h);
    }
  }
}
// code and dequantized value of a chunk: q = clamp(r + z, 0, Q), (q - z) h
OMQ_DEV void dequant8(const float (&rr)[8], const RowQ& q, float (&qq)[8], float (&o)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    qq[j] = __builtin_amdgcn_fmed3f(rr[j] + q.z, 0.f, q.Q);
    o[j] = (qq[j] - q.z) * q.h;
  }
}

// ---------------------------------------------------------------------------
// forward, pass-through (16 bits and more: x~ only, no rounding): 8 consecutive
// columns per thread and step, 16-byte accesses, the LET mode fixed at compile time;
// the same arithmetic as the per-row kernel's pass-through below
// ---------------------------------------------------------------------------
OMQ_DEV void load8x(const char* xr, int dt, int64_t c, float (&v)[8]);
template <int XDT, int LET>
__global__ __launch_bounds__(kThreads) void k_rowquant_pass8(RowQuantFwd a) {
  const int64_t per_row = a.cols / 8, n = a.rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / per_row, c = (i - r * per_row) * 8;
    const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
    float v[8];
    load8x(xr, XDT, c, v);
    if constexpr (LET == OMQ_LET_DIV) {
      float sv[8], dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const float4 s0 = *reinterpret_cast<const float4*>(a.s + c);
      const float4 s1 = *reinterpret_cast<const float4*>(a.s + c + 4);
      sv[0] = s0.x; sv[1] = s0.y; sv[2] = s0.z; sv[3] = s0.w;
      sv[4] = s1.x; sv[5] = s1.y; sv[6] = s1.z; sv[7] = s1.w;
      if (a.delta) {
        const float4 d0 = *reinterpret_cast<const float4*>(a.delta + c);
        const float4 d1 = *reinterpret_cast<const float4*>(a.delta + c + 4);
        dv[0] = d0.x; dv[1] = d0.y; dv[2] = d0.z; dv[3] = d0.w;
        dv[4] = d1.x; dv[5] = d1.y; dv[6] = d1.z; dv[7] = d1.w;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (v[j] - dv[j]) / sv[j];
    } else if constexpr (LET == OMQ_LET_MUL) {
      const float4 s0 = *reinterpret_cast<const float4*>(a.s + c);
      const float4 s1 = *reinterpret_cast<const float4*>(a.s + c + 4);
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = sv[j] * v[j];
    }
    store8(a.out, a.out_dt, r * a.ldo + c, v);
  }
}

// ---------------------------------------------------------------------------
// forward: one 256-thread block per row
// ---------------------------------------------------------------------------
template <int XDT>
__global__ __launch_bounds__(kThreads) void k_rowquant_fwd(RowQuantFwd a) {
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = wave_id();
  const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
  const int64_t cols = a.cols;

  if (a.nbits >= 16) {  // pass-through: x~ only
    for (int64_t c = (int64_t)tid * 4; c < cols; c += 4 * kThreads) {
      float v[4];
      load4(xr, XDT, c, v);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = let_x(v[j], a.let_mode, a.s, a.delta, c + j);
      store4(a.out, a.out_dt, r * a.ldo + c, v);
    }
    return;
  }

  float vmax = -FLT_MAX, vmin = FLT_MAX, dot = 0.f;
  int imax = 0x7fffffff, imin = 0x7fffffff;
  bool nf = false;
  for (int64_t c = (int64_t)tid * 4; c < cols; c += 4 * kThreads) {
    float v[4];
    load4(xr, XDT, c, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float xt = let_x(v[j], a.let_mode, a.s, a.delta, c + j);
      if (xt > vmax || imax == 0x7fffffff) { vmax = xt; imax = (int)(c + j); }
      if (xt < vmin || imin == 0x7fffffff) { vmin = xt; imin = (int)(c + j); }
      nf |= !__builtin_isfinite(xt);
      if (a.fold_delta) dot = fmaf(a.fold_delta[c + j], v[j], dot);
    }
  }
  if (a.nonfinite) flag_nonfinite(a.nonfinite, nf);
  wave_argmax(vmax, imax);
  wave_argmin(vmin, imin);
  dot = wave_sum(dot);
  __shared__ float s_max[4], s_min[4], s_dot[4];
  __shared__ int s_imax[4], s_imin[4];
  if (lane == 0) {
    s_max[wid] = vmax; s_imax[wid] = imax;
    s_min[wid] = vmin; s_imin[wid] = imin;
    s_dot[wid] = dot;
  }
  __syncthreads();
  float M = s_max[0], m = s_min[0], D = s_dot[0];
  int iM = s_imax[0], im = s_imin[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    argmax_merge(M, iM, s_max[w], s_imax[w]);
    argmin_merge(m, im, s_min[w], s_imin[w]);
    D += s_dot[w];
  }
  const float gamma = a.a_gamma ? sigmoid_f32(a.a_gamma[r]) : 1.f;
  const float beta = a.a_beta ? sigmoid_f32(a.a_beta[r]) : 1.f;
  const RowQ q = row_step(M, m, gamma, beta, a.nbits);
  if (tid == 0) {
    if (a.h) a.h[r] = q.h;
    if (a.z) a.z[r] = q.z;
    if (a.amax) a.amax[r] = col_in(iM, cols);
    if (a.amin) a.amin[r] = col_in(im, cols);
    if (a.bias_out) a.bias_out[r] = (a.bias ? a.bias[r] : 0.f) + D;
  }
  const float rh = 1.f / q.h;
  int qs = 0;
  for (int64_t c = (int64_t)tid * 4; c < cols; c += 4 * kThreads) {
    float v[4], o[4];
    load4(xr, XDT, c, v);
    uint32_t cw = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float xt = let_x(v[j], a.let_mode, a.s, a.delta, c + j);
      float u;
      float rr = rint_quot(xt, q.h, rh, u) + q.z;
      float qq = fminf(fmaxf(rr, 0.f), q.Q);
      o[j] = (qq - q.z) * q.h;
      const int qi = (int)qq - a.code_off;
      cw |= ((uint32_t)qi & 0xffu) << (8 * j);
      qs += qi;
    }
    store4(a.out, a.out_dt, r * a.ldo + c, o);
    if (a.codes) store_codes4(a, r, c, cw);
  }
  if (a.qsum) block_qsum(qs, a.qsum + r);
}

// Single-pass variant: the row (up to NCH * 1024 elements) stays in registers
// between the min/max reduction and the quantization, so HBM sees one read of x
// and one write of x_hat.
template <int XDT, int NCH>
__global__ __launch_bounds__(kThreads) void k_rowquant_fwd_reg(RowQuantFwd a) {
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = wave_id();
  const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
  const int64_t cols = a.cols;
  float xt[NCH][4];
  float vmax = -FLT_MAX, vmin = FLT_MAX, dot = 0.f;
  int imax = 0x7fffffff, imin = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int64_t c = ((int64_t)k * kThreads + tid) * 4;
    if (c < cols) {
      float v[4];
      load4(xr, XDT, c, v);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xt[k][j] = let_x(v[j], a.let_mode, a.s, a.delta, c + j);
        if (a.fold_delta) dot = fmaf(a.fold_delta[c + j], v[j], dot);
      }
    }
  }
  // per-thread scan in increasing column order keeps the first index on ties
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int64_t c = ((int64_t)k * kThreads + tid) * 4;
    if (c < cols) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (xt[k][j] > vmax || imax == 0x7fffffff) { vmax = xt[k][j]; imax = (int)(c + j); }
        if (xt[k][j] < vmin || imin == 0x7fffffff) { vmin = xt[k][j]; imin = (int)(c + j); }
      }
    }
  }
  if (a.nonfinite) {
    bool nf = false;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int64_t c = ((int64_t)k * kThreads + tid) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c + j < cols) nf |= !__builtin_isfinite(xt[k][j]);
    }
    flag_nonfinite(a.nonfinite, nf);
  }
  wave_argmax(vmax, imax);
  wave_argmin(vmin, imin);
  dot = wave_sum(dot);
  __shared__ float s_max[4], s_min[4], s_dot[4];
  __shared__ int s_imax[4], s_imin[4];
  if (lane == 0) {
    s_max[wid] = vmax; s_imax[wid] = imax;
    s_min[wid] = vmin; s_imin[wid] = imin;
    s_dot[wid] = dot;
  }
  __syncthreads();
  float M = s_max[0], m = s_min[0], D = s_dot[0];
  int iM = s_imax[0], im = s_imin[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    argmax_merge(M, iM, s_max[w], s_imax[w]);
    argmin_merge(m, im, s_min[w], s_imin[w]);
    D += s_dot[w];
  }
  const float gamma = a.a_gamma ? sigmoid_f32(a.a_gamma[r]) : 1.f;
  const float beta = a.a_beta ? sigmoid_f32(a.a_beta[r]) : 1.f;
  const RowQ q = row_step(M, m, gamma, beta, a.nbits);
  if (tid == 0) {
    if (a.h) a.h[r] = q.h;
    if (a.z) a.z[r] = q.z;
    if (a.amax) a.amax[r] = col_in(iM, cols);
    if (a.amin) a.amin[r] = col_in(im, cols);
    if (a.bias_out) a.bias_out[r] = (a.bias ? a.bias[r] : 0.f) + D;
  }
  const float rh = 1.f / q.h;
  int qs = 0;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int64_t c = ((int64_t)k * kThreads + tid) * 4;
    if (c < cols) {
      float o[4];
      uint32_t cw = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float u;
        const float rr = rint_quot(xt[k][j], q.h, rh, u) + q.z;
        const float qq = fminf(fmaxf(rr, 0.f), q.Q);
        o[j] = (qq - q.z) * q.h;
        const int qi = (int)qq - a.code_off;
        cw |= ((uint32_t)qi & 0xffu) << (8 * j);
        qs += qi;
      }
      store4(a.out, a.out_dt, r * a.ldo + c, o);
      if (a.codes) store_codes4(a, r, c, cw);
    }
  }
  if (a.qsum) block_qsum(qs, a.qsum + r);
}

// One wave per row (rows up to NC * 512 elements): each lane keeps NC chunks of
// 8 consecutive elements (16-byte bf16 loads, 2 x 16-byte float32 loads) in
// registers; the row reductions are wave shuffles only, with no barrier.
OMQ_DEV void load8(const char* xr, int dt, int64_t c, float v[8]) {
  if (dt == OMQ_F32) {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(xr) + c);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(xr) + c + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 t = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(xr) + c);
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
  }
}

OMQ_DEV void load8x(const char* xr, int dt, int64_t c, float (&v)[8]) { load8(xr, dt, c, v); }

// 8 consecutive float32 parameters (s, delta) starting at c; n = 8 or 4 valid
OMQ_DEV void load8f(const float* p, int64_t c, int n, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p + c);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  if (n == 8) {
    const float4 b = *reinterpret_cast<const float4*>(p + c + 4);
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    v[4] = v[5] = v[6] = v[7] = 1.f;
  }
}

// RoPE of the 8 consecutive columns c .. c+7 of row r, in heads of 128 columns with
// the row as the position: column k < 64 of a head becomes x_k cos - x_(k+64) sin and
// column k + 64 becomes x_(k+64) cos + x_k sin (cos, sin of table column k; products
// rounded before the sum).  In the block-per-row kernel the partner columns are 64
// columns, 8 lanes, away in the same wave, and a head's 16 lanes are all in range
// or all out.  The rotated values are also written to rope_out.
OMQ_DEV void rope8(const RowQuantFwd& a, int64_t r, int64_t c, float (&v)[8]) {
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = __shfl_xor(v[j], 8);
  const int kh = (int)(c & 127);
  float cs[8], sn[8];
  load8f(a.rope_cos + r * 64, kh & 63, 8, cs);
  load8f(a.rope_sin + r * 64, kh & 63, 8, sn);
  if (kh < 64) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * cs[j] - p[j] * sn[j];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * cs[j] + p[j] * sn[j];
  }
  store8(a.rope_out, OMQ_F32, r * a.cols + c, v);
}

// Long rows (up to NC * 2048 elements, columns a multiple of 8), one 4-wave block per
// row: each thread keeps NC chunks of 8 consecutive elements in registers (16-byte
// bf16 loads, 2 x 16-byte float32 loads), so HBM sees one read of x and one write of
// x_hat; the LET mode is fixed at compile time and the quotient takes the reciprocal
// product with the exact quotient behind a wave-uniform branch, as in the
// whole-row LDS kernel.  Same results as k_rowquant_fwd_reg.
// RMS: the row is first divided by its root mean square (as the whole-row LDS kernel).
// ROPE: the row is first rotated (rope8; float32 rows, heads of 128 columns).
template <int XDT, int NC, int LET, bool RMS = false, bool ROPE = false>
__global__ __launch_bounds__(kThreads) void k_rowquant_fwd_blk8(RowQuantFwd a) {
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
  const int64_t cols = a.cols;
  float xt[NC][8];
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * kThreads + tid) * 8;
    if (c < cols) {
      float v[8];
      load8(xr, XDT, c, v);
      if constexpr (ROPE) rope8(a, r, c, v);
      if constexpr (RMS) {                         // LET after the normalization below
#pragma unroll
        for (int j = 0; j < 8; ++j) xt[k][j] = v[j];
      } else if constexpr (LET == OMQ_LET_DIV) {
        float sv[8], dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        load8f(a.s, c, 8, sv);
        if (a.delta) load8f(a.delta, c, 8, dv);
#pragma unroll
        for (int j = 0; j < 8; ++j) xt[k][j] = (v[j] - dv[j]) / sv[j];
      } else if constexpr (LET == OMQ_LET_MUL) {
        float sv[8];
        load8f(a.s, c, 8, sv);
#pragma unroll
        for (int j = 0; j < 8; ++j) xt[k][j] = sv[j] * v[j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xt[k][j] = v[j];
      }
      if (!RMS && a.fold_delta) {
        float fv[8];
        load8f(a.fold_delta, c, 8, fv);
#pragma unroll
        for (int j = 0; j < 8; ++j) dot = fmaf(fv[j], v[j], dot);
      }
    }
  }
  if constexpr (RMS) {
    // 1 / rms of the row (block sum of squares in double), the normalized row stored,
    // then LET
    __shared__ double s_ss[4];
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int64_t c = ((int64_t)k * kThreads + tid) * 8;
      if (c < cols) {
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fma((double)xt[k][j], (double)xt[k][j], ss);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) s_ss[wid] = ss;
    __syncthreads();
    ss = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
    const float rs = rms_scale(ss, cols, a.eps);
    if (tid == 0 && a.rstd) a.rstd[r] = rs;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int64_t c = ((int64_t)k * kThreads + tid) * 8;
      if (c < cols) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = xt[k][j] * rs;
        store8(a.rms_out, OMQ_F32, r * cols + c, v);
        if constexpr (LET == OMQ_LET_DIV) {
          float sv[8], dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          load8f(a.s, c, 8, sv);
          if (a.delta) load8f(a.delta, c, 8, dv);
#pragma unroll
          for (int j = 0; j < 8; ++j) xt[k][j] = (v[j] - dv[j]) / sv[j];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) xt[k][j] = v[j];
        }
      }
    }
  }
  // per chunk its max / min; the thread keeps the first chunk holding its extreme
  // (chunks run in increasing column order)
  float lmax = -FLT_MAX, lmin = FLT_MAX, nfa = 0.f;
  int kmx = -1, kmn = -1;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * kThreads + tid) * 8;
    if (c < cols) {
      const float cM = max8(xt[k]), cm = min8(xt[k]);
      if (kmx < 0 || cM > lmax) { lmax = cM; kmx = k; }
      if (kmn < 0 || cm < lmin) { lmin = cm; kmn = k; }
      if (a.nonfinite) nfa = nf_acc8(xt[k], nfa);
    }
  }
  if (a.nonfinite) flag_nonfinite(a.nonfinite, nfa != nfa);
  // the row's extreme values over the block
  __shared__ float s_ext[2][4];
  {
    const float wM = wave_maxf(lmax), wm = wave_minf(lmin);
    if (lane == 0) { s_ext[0][wid] = wM; s_ext[1][wid] = wm; }
  }
  dot = wave_sum(dot);
  __syncthreads();
  float M = fmaxf(fmaxf(s_ext[0][0], s_ext[0][1]), fmaxf(s_ext[0][2], s_ext[0][3]));
  float m = fminf(fminf(s_ext[1][0], s_ext[1][1]), fminf(s_ext[1][2], s_ext[1][3]));
  // their first columns: the threads holding an extreme take the first equal element
  // of their chunk (only waves with such a thread search); the others offer (the
  // extreme, no column), so the lowest column wins and its value is kept
  int imax = 0x7fffffff, imin = 0x7fffffff;
  const bool hM = kmx >= 0 && lmax == M, hm = kmn >= 0 && lmin == m;
  if (__builtin_amdgcn_ballot_w64(hM) != 0) {
    if (hM) {
      float t[8];
#pragma unroll
      for (int k = 0; k < NC; ++k)
        if (k == kmx) {
#pragma unroll
          for (int j = 0; j < 8; ++j) t[j] = xt[k][j];
        }
      int j;
      first_eq8(t, M, j, M);
      if (j < 8) imax = (int)(((int64_t)kmx * kThreads + tid) * 8 + j);
    }
  }
  if (__builtin_amdgcn_ballot_w64(hm) != 0) {
    if (hm) {
      float t[8];
#pragma unroll
      for (int k = 0; k < NC; ++k)
        if (k == kmn) {
#pragma unroll
          for (int j = 0; j < 8; ++j) t[j] = xt[k][j];
        }
      int j;
      first_eq8(t, m, j, m);
      if (j < 8) imin = (int)(((int64_t)kmn * kThreads + tid) * 8 + j);
    }
  }
  wave_argmax(M, imax);
  wave_argmin(m, imin);
  __shared__ float s_max[4], s_min[4], s_dot[4];
  __shared__ int s_imax[4], s_imin[4];
  if (lane == 0) {
    s_max[wid] = M; s_imax[wid] = imax;
    s_min[wid] = m; s_imin[wid] = imin;
    s_dot[wid] = dot;
  }
  __syncthreads();
  M = s_max[0]; m = s_min[0];
  float D = s_dot[0];
  int iM = s_imax[0], im = s_imin[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    argmax_merge(M, iM, s_max[w], s_imax[w]);
    argmin_merge(m, im, s_min[w], s_imin[w]);
    D += s_dot[w];
  }
  const float gamma = a.a_gamma ? sigmoid_f32(a.a_gamma[r]) : 1.f;
  const float beta = a.a_beta ? sigmoid_f32(a.a_beta[r]) : 1.f;
  const RowQ q = row_step(M, m, gamma, beta, a.nbits);
  if (tid == 0) {
    if (a.h) a.h[r] = q.h;
    if (a.z) a.z[r] = q.z;
    if (a.amax) a.amax[r] = col_in(iM, cols);
    if (a.amin) a.amin[r] = col_in(im, cols);
    if (a.bias_out) a.bias_out[r] = (a.bias ? a.bias[r] : 0.f) + D;
  }
  // round, clamp, dequantize and store from the registers
  const float rh = 1.f / q.h;
  const float thr = fmaxf(fabsf(M), fabsf(m)) * rh * 0x1p-20f;
  const bool off128 = a.code_off != 0;
  uint32_t qsum = 0u;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * kThreads + tid) * 8;
    const bool in = c < cols;
    float rr[8];
    rint_quot8(xt[k], q.h, rh, thr, in, rr);
    if (in) {
      float o[8], qq[8];
      dequant8(rr, q, qq, o);
      store8(a.out, a.out_dt, r * a.ldo + c, o);
      if (a.codes) {
        const uint2 cw = codes8(qq, off128, qsum);
        store_codes8(a, r, c, cw.x, cw.y);
      }
    }
  }
  // sum of the stored codes q - off over the row's columns
  if (a.qsum) block_qsum((int)qsum - (tid == 0 ? a.code_off * (int)cols : 0), a.qsum + r);
}

// FULL: every 512-column chunk of the row is whole (cols is a multiple of 512), so
// no column bounds are checked.
template <int XDT, int NC, int LET, bool FULL>
__global__ __launch_bounds__(kThreads) void k_rowquant_fwd_wave(RowQuantFwd a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave_id();
  if (r >= a.rows) return;
  const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
  const int64_t cols = a.cols;
  float xt[NC][8];
  float vmax = -FLT_MAX, vmin = FLT_MAX, dot = 0.f;
  int imax = 0x7fffffff, imin = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * 64 + lane) * 8;
    if (FULL || c < cols) {
      const int n = FULL || c + 8 <= cols ? 8 : 4;  // rows are multiples of 4 long
      float v[8];
      if (n == 8) {
        load8(xr, XDT, c, v);
      } else {
        load4(xr, XDT, c, v);
        v[4] = v[5] = v[6] = v[7] = 0.f;
      }
      if constexpr (LET == OMQ_LET_DIV) {
        float sv[8], dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        load8f(a.s, c, n, sv);
        if (a.delta) load8f(a.delta, c, n, dv);
#pragma unroll
        for (int j = 0; j < 8; ++j) xt[k][j] = (v[j] - dv[j]) / sv[j];
      } else if constexpr (LET == OMQ_LET_MUL) {
        float sv[8];
        load8f(a.s, c, n, sv);
#pragma unroll
        for (int j = 0; j < 8; ++j) xt[k][j] = sv[j] * v[j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xt[k][j] = v[j];
      }
      if (a.fold_delta) {
        float fv[8];
        load8f(a.fold_delta, c, n, fv);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < n) dot = fmaf(fv[j], v[j], dot);
      }
    }
  }
  // the lane's max / min with the lowest column among equal values (columns are
  // visited in increasing order)
  if constexpr (FULL) {
    vmax = vmin = xt[0][0];
    imax = imin = lane * 8;
  }
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * 64 + lane) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (FULL) {
        if (k == 0 && j == 0) continue;
        if (xt[k][j] > vmax) { vmax = xt[k][j]; imax = (int)(c + j); }
        if (xt[k][j] < vmin) { vmin = xt[k][j]; imin = (int)(c + j); }
      } else if (c + j < cols) {
        if (xt[k][j] > vmax || imax == 0x7fffffff) { vmax = xt[k][j]; imax = (int)(c + j); }
        if (xt[k][j] < vmin || imin == 0x7fffffff) { vmin = xt[k][j]; imin = (int)(c + j); }
      }
    }
  }
  if (a.nonfinite) {
    bool nf = false;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int64_t c = ((int64_t)k * 64 + lane) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (FULL || c + j < cols) nf |= !__builtin_isfinite(xt[k][j]);
    }
    flag_nonfinite(a.nonfinite, nf);
  }
  wave_argmax(vmax, imax);
  wave_argmin(vmin, imin);
  dot = wave_sum(dot);
  const float gamma = a.a_gamma ? sigmoid_f32(a.a_gamma[r]) : 1.f;
  const float beta = a.a_beta ? sigmoid_f32(a.a_beta[r]) : 1.f;
  const RowQ q = row_step(vmax, vmin, gamma, beta, a.nbits);
  if (lane == 0) {
    if (a.h) a.h[r] = q.h;
    if (a.z) a.z[r] = q.z;
    if (a.amax) a.amax[r] = col_in(imax, a.cols);
    if (a.amin) a.amin[r] = col_in(imin, a.cols);
    if (a.bias_out) a.bias_out[r] = (a.bias ? a.bias[r] : 0.f) + dot;
  }
  // rint(x~ / h) for every element by the reciprocal product, then the exact
  // quotient for the (rare) elements whose product lies within |u| 2^-20 of a
  // half-integer or is not finite, behind wave-uniform branches (divergent ones
  // would be flattened into a division for every element)
  const float rh = 1.f / q.h;
  bool near = false;
#pragma unroll
  for (int k = 0; k < NC; ++k)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = xt[k][j] * rh;
      const float rr = rintf(u);
      near |= !(fabsf(fabsf(u - rr) - 0.5f) > fabsf(u) * 0x1p-20f);
      xt[k][j] = rr;                                // xt now holds rint(x~ / h)
    }
  if (__builtin_amdgcn_ballot_w64(near) != 0) {
    // recompute the chunk's x~ exactly where needed
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int64_t c = ((int64_t)k * 64 + lane) * 8;
      bool nk = false;
      float v[8];
      if (FULL || c < cols) {
        const int n = FULL || c + 8 <= cols ? 8 : 4;
        if (n == 8) {
          load8(xr, XDT, c, v);
        } else {
          load4(xr, XDT, c, v);
          v[4] = v[5] = v[6] = v[7] = 0.f;
        }
        float sv[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
        float dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if constexpr (LET != OMQ_LET_NONE) load8f(a.s, c, n, sv);
        if constexpr (LET == OMQ_LET_DIV) {
          if (a.delta) load8f(a.delta, c, n, dv);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x1 = LET == OMQ_LET_DIV ? (v[j] - dv[j]) / sv[j]
                           : LET == OMQ_LET_MUL ? sv[j] * v[j] : v[j];
          v[j] = x1;
          const float u = x1 * rh;
          const float rr = rintf(u);
          nk |= !(fabsf(fabsf(u - rr) - 0.5f) > fabsf(u) * 0x1p-20f);
        }
      }
      if (__builtin_amdgcn_ballot_w64(nk) != 0) {
        if (nk) {
#pragma unroll
          for (int j = 0; j < 8; ++j) xt[k][j] = rintf(v[j] / q.h);
        }
      }
    }
  }
  int qs = 0;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * 64 + lane) * 8;
    if (FULL || c < cols) {
      float o[8];
      uint32_t cw[2] = {0u, 0u};
      const int n = FULL || c + 8 <= cols ? 8 : 4;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float rr = xt[k][j] + q.z;
        const float qq = fminf(fmaxf(rr, 0.f), q.Q);
        o[j] = (qq - q.z) * q.h;
        const int qi = (int)qq - a.code_off;
        cw[j >> 2] |= ((uint32_t)qi & 0xffu) << (8 * (j & 3));
        if (j < n) qs += qi;
      }
      store4(a.out, a.out_dt, r * a.ldo + c, o);
      if (a.codes) store_codes4(a, r, c, cw[0]);
      if (FULL || c + 8 <= cols) {
        store4(a.out, a.out_dt, r * a.ldo + c + 4, o + 4);
        if (a.codes) store_codes4(a, r, c + 4, cw[1]);
      }
    }
  }
  if (a.qsum) {
    qs = wave_sum(qs);
    if (lane == 0) a.qsum[r] = qs;
  }
}

// Whole rows (cols = 512 NC), one wave per row, the row staged in LDS: the wave
// copies its row straight from HBM into its own LDS slot, then forms x~ chunk by
// chunk into registers (pass 1: the chunk's max / min, the bias fold, finiteness),
// and rounds and stores from those registers (pass 2).  The extreme values take the
// three-operand max / min per chunk and the lane remembers the first chunk holding
// its extreme; only the lanes holding the row's extreme look for its first column
// inside that chunk (re-forming it from LDS), so the column is the lowest one among
// equal values, as an element-wise scan in column order gives.  Same results as
// k_rowquant_fwd_wave.  (One row per wave: a wave that kept taking rows would have to
// wait for its previous row's stores before reading the next copy from LDS, where a
// finished wave lets them drain.)
// RMS: x is first normalized by its row's root mean square (the RMSNorm before the
// linear, unit gain), the normalized row written to rms_out and 1/rms to rstd.
template <int XDT, int NC, int LET, bool RMS = false>
__global__ __launch_bounds__(kThreads) void k_rowquant_fwd_lds(RowQuantFwd a) {
  constexpr int ESZ = XDT == OMQ_F32 ? 4 : 2;
  constexpr int NH = ESZ / 2;                      // 1 KB copies per 8-element chunk
  __shared__ uint4 slot[4][NC * NH * 64];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int64_t r = (int64_t)blockIdx.x * 4 + w;
  if (r >= a.rows) return;
  // the row's segment (concatenated weights): its x rows and logits
  const void* xb = a.x;
  const float *lg_g = a.a_gamma, *lg_b = a.a_beta;
  int64_t rl = r;
  if (a.nseg > 1) {
    // selects, not a run-time index into the argument arrays (that would copy the
    // argument block to scratch memory)
    const bool s1 = r >= a.seg_end[0], s2 = a.nseg > 2 && r >= a.seg_end[1];
    xb = s2 ? a.xseg[2] : s1 ? a.xseg[1] : a.xseg[0];
    lg_g = s2 ? a.agseg[2] : s1 ? a.agseg[1] : a.agseg[0];
    lg_b = s2 ? a.abseg[2] : s1 ? a.abseg[1] : a.abseg[0];
    rl = r - (s2 ? a.seg_end[1] : s1 ? a.seg_end[0] : 0);
  }
  uint4* my = slot[w];
  {
    // lane l's 16-byte piece h of chunk k lands at my[(k NH + h) 64 + l]
    const char* xr = reinterpret_cast<const char*>(xb) + rl * a.ldx * ESZ;
#pragma unroll
    for (int k = 0; k < NC; ++k)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        __builtin_amdgcn_global_load_lds(
            (const void*)(xr + ((int64_t)k * 64 + lane) * 8 * ESZ + 16 * h),
            (__attribute__((address_space(3))) void*)(my + (k * NH + h) * 64), 16, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  // the raw elements of chunk k
  auto raw = [&](int k, float (&v)[8]) {
    if constexpr (XDT == OMQ_F32) {
      const uint4 t0 = my[(2 * k) * 64 + lane], t1 = my[(2 * k + 1) * 64 + lane];
      const uint32_t wv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(wv[j]);
    } else {
      const uint4 t0 = my[k * 64 + lane];
      const uint32_t wv[4] = {t0.x, t0.y, t0.z, t0.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(wv[q] << 16);
        v[2 * q + 1] = __uint_as_float(wv[q] & 0xffff0000u);
      }
    }
  };
  // the row's 1 / rms: sum of squares over the staged row
  float rs = 1.f;
  if constexpr (RMS) {
    double ss = 0.0;
#pragma unroll 2
    for (int k = 0; k < NC; ++k) {
      float v[8];
      raw(k, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fma((double)v[j], (double)v[j], ss);
    }
    ss = wave_sum(ss);
    rs = rms_scale(ss, a.cols, a.eps);
    if (lane == 0 && a.rstd) a.rstd[r] = rs;
  }
  // x~ of chunk k (columns c .. c+7, c = (64 k + lane) 8) from the raw elements v
  // (normalized when RMS)
  auto let = [&](int k, const float (&v)[8], float (&xt)[8]) {
    const int64_t c = ((int64_t)k * 64 + lane) * 8;
    if constexpr (LET == OMQ_LET_DIV) {
      float sv[8], dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      load8f(a.s, c, 8, sv);
      if (a.delta) load8f(a.delta, c, 8, dv);
#pragma unroll
      for (int j = 0; j < 8; ++j) xt[j] = (v[j] - dv[j]) / sv[j];
    } else if constexpr (LET == OMQ_LET_MUL) {
      float sv[8];
      load8f(a.s, c, 8, sv);
#pragma unroll
      for (int j = 0; j < 8; ++j) xt[j] = sv[j] * v[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) xt[j] = v[j];
    }
  };
  auto xtilde = [&](int k, float (&xt)[8]) {
    float v[8];
    raw(k, v);
    if constexpr (RMS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * rs;
    }
    let(k, v, xt);
  };
  // pass 1: x~ into registers; per chunk its max / min (the lane keeps the first
  // chunk holding its extreme), the bias fold and the finiteness accumulator
  float xs[NC][8];
  float lmax = 0.f, lmin = 0.f, dot = 0.f, nfa = 0.f;
  int kmx = 0, kmn = 0;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * 64 + lane) * 8;
    float v[8];
    raw(k, v);
    if constexpr (RMS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * rs;
      store8(a.rms_out, OMQ_F32, r * a.cols + c, v);
    }
    if (a.fold_delta) {
      float fv[8];
      load8f(a.fold_delta, c, 8, fv);
#pragma unroll
      for (int j = 0; j < 8; ++j) dot = fmaf(fv[j], v[j], dot);
    }
    let(k, v, xs[k]);
    const float cM = max8(xs[k]), cm = min8(xs[k]);
    if (k == 0) {
      lmax = cM;
      lmin = cm;
    } else {
      if (cM > lmax) { lmax = cM; kmx = k; }
      if (cm < lmin) { lmin = cm; kmn = k; }
    }
    if (a.nonfinite) nfa = nf_acc8(xs[k], nfa);
  }
  if (a.nonfinite) flag_nonfinite(a.nonfinite, nfa != nfa);
  // the row's extremes, then their first columns: the lanes holding an extreme
  // re-form their chunk from LDS and take its first equal element; the others offer
  // (the extreme, no column), so the lowest column wins and its value is kept
  float M = wave_maxf(lmax), m = wave_minf(lmin);
  int imax = 0x7fffffff, imin = 0x7fffffff;
  {
    float t[8];
    int j;
    if (lmax == M) {
      xtilde(kmx, t);
      first_eq8(t, M, j, M);
      if (j < 8) imax = (kmx * 64 + lane) * 8 + j;
    }
    if (lmin == m) {
      xtilde(kmn, t);
      first_eq8(t, m, j, m);
      if (j < 8) imin = (kmn * 64 + lane) * 8 + j;
    }
  }
  wave_argmax(M, imax);
  wave_argmin(m, imin);
  dot = wave_sum(dot);
  const float gamma = lg_g ? sigmoid_f32(lg_g[rl]) : 1.f;
  const float beta = lg_b ? sigmoid_f32(lg_b[rl]) : 1.f;
  const RowQ q = row_step(M, m, gamma, beta, a.nbits);
  if (lane == 0) {
    if (a.h) a.h[r] = q.h;
    if (a.z) a.z[r] = q.z;
    if (a.amax) a.amax[r] = col_in(imax, a.cols);
    if (a.amin) a.amin[r] = col_in(imin, a.cols);
    if (a.bias_out) a.bias_out[r] = (a.bias ? a.bias[r] : 0.f) + dot;
  }
  // pass 2: round, clamp, dequantize and store from the registers
  const float rh = 1.f / q.h;
  const float thr = fmaxf(fabsf(M), fabsf(m)) * rh * 0x1p-20f;
  const bool off128 = a.code_off != 0;
  uint32_t qsum = 0u;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * 64 + lane) * 8;
    float rr[8], o[8], qq[8];
    rint_quot8(xs[k], q.h, rh, thr, true, rr);
    dequant8(rr, q, qq, o);
    store8(a.out, a.out_dt, r * a.ldo + c, o);
    if (a.codes) {
      const uint2 cw = codes8(qq, off128, qsum);
      store_codes8(a, r, c, cw.x, cw.y);
    }
  }
  if (a.qsum) {
    const int qs = (int)wave_sum(qsum) - a.code_off * (int)a.cols;
    if (lane == 0) a.qsum[r] = qs;
  }
}

// Group-wise forward (groups of 128 columns): 16 lanes per group with 8 columns
// each, 4 groups per wave, 16 per block; reductions stay inside each 16-lane group.
template <int XDT>
__global__ __launch_bounds__(kThreads) void k_rowquant_fwd_g128(RowQuantFwd a) {
  const int lane = threadIdx.x & 63;
  const int64_t G = a.cols / 128;
  const int64_t p = (int64_t)blockIdx.x * 16 + wave_id() * 4 + (lane >> 4);
  const bool pv = p < a.rows * G;             // every lane takes part in the shuffles
  const int64_t r = pv ? p / G : 0, k = pv ? p % G : 0;
  const int64_t c = k * 128 + (lane & 15) * 8;
  const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
  float xt[8];
  float vmax = -FLT_MAX, vmin = FLT_MAX;
  int imax = 0x7fffffff, imin = 0x7fffffff;
  bool nf = false;
  if (pv) {
    float v[8];
    load8(xr, XDT, c, v);
    if (a.let_mode == OMQ_LET_DIV) {
      float sv[8], dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      load8f(a.s, c, 8, sv);
      if (a.delta) load8f(a.delta, c, 8, dv);
#pragma unroll
      for (int j = 0; j < 8; ++j) xt[j] = (v[j] - dv[j]) / sv[j];
    } else if (a.let_mode == OMQ_LET_MUL) {
      float sv[8];
      load8f(a.s, c, 8, sv);
#pragma unroll
      for (int j = 0; j < 8; ++j) xt[j] = sv[j] * v[j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) xt[j] = v[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (xt[j] > vmax || imax == 0x7fffffff) { vmax = xt[j]; imax = (int)(c + j); }
      if (xt[j] < vmin || imin == 0x7fffffff) { vmin = xt[j]; imin = (int)(c + j); }
      nf |= !__builtin_isfinite(xt[j]);
    }
  }
  if (a.nonfinite) flag_nonfinite(a.nonfinite, nf);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(vmax, o, kWave);
    const int i2 = __shfl_xor(imax, o, kWave);
    argmax_merge(vmax, imax, v2, i2);
    const float w2 = __shfl_xor(vmin, o, kWave);
    const int j2 = __shfl_xor(imin, o, kWave);
    argmin_merge(vmin, imin, w2, j2);
  }
  if (!pv) return;
  const float gamma = a.a_gamma ? sigmoid_f32(a.a_gamma[p]) : 1.f;
  const float beta = a.a_beta ? sigmoid_f32(a.a_beta[p]) : 1.f;
  const RowQ q = row_step(vmax, vmin, gamma, beta, a.nbits);
  if ((lane & 15) == 0) {
    if (a.h) a.h[p] = q.h;
    if (a.z) a.z[p] = q.z;
    if (a.amax) a.amax[p] = col_in(imax, a.cols);
    if (a.amin) a.amin[p] = col_in(imin, a.cols);
  }
  const float rh = 1.f / q.h;
  float o[8];
  uint32_t cw[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float u;
    const float rr = rint_quot(xt[j], q.h, rh, u) + q.z;
    const float qq = fminf(fmaxf(rr, 0.f), q.Q);
    o[j] = (qq - q.z) * q.h;
    cw[j >> 2] |= ((uint32_t)((int)qq - a.code_off) & 0xffu) << (8 * (j & 3));
  }
  store4(a.out, a.out_dt, r * a.ldo + c, o);
  store4(a.out, a.out_dt, r * a.ldo + c + 4, o + 4);
  if (a.codes) store_codes8(a, r, c, cw[0], cw[1]);
}

// ---------------------------------------------------------------------------
// backward tile pass: grid (col slabs, row tiles); wave w takes rows w, w+4, ...
// ---------------------------------------------------------------------------
// LET and COL (the column-partial kind) are fixed at compile time, so the
// per-element arithmetic is straight-line code.
template <int XDT, int LET, int COL>
__global__ __launch_bounds__(kThreads) void k_rowquant_bwd_tile(RowQuantBwd a, int rows_per_tile,
                                                                float* rowpart, float* colpart) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = wave_id();
  const int64_t c0 = (int64_t)blockIdx.x * kSlab;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_tile;
  const int64_t cols = a.cols, rows = a.rows;
  const bool pass = a.nbits >= 16;
  const float Q = pass ? 0.f : (float)((1 << a.nbits) - 1);
  float acc0[16], acc1[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) { acc0[i] = 0.f; acc1[i] = 0.f; }
  // this lane's 16 columns: LET scale, shift and reciprocal scale, for every row
  float sc[16], dc[16], rc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t c = c0 + lane * 4 + 256 * (i >> 2) + (i & 3);
    const bool cv = c < cols && LET != OMQ_LET_NONE;
    sc[i] = cv ? a.s[c] : 1.f;
    dc[i] = (cv && LET == OMQ_LET_DIV && a.delta) ? a.delta[c] : 0.f;
    rc[i] = 1.f / sc[i];
  }

  // grouped rows: the 32 lanes of a half-wave cover one 128-column group per k
  const bool grouped = a.group > 0;
  const int64_t G = grouped ? cols / 128 : 1;
  for (int rr_ = wid; rr_ < rows_per_tile; rr_ += 4) {
    const int64_t r = r0 + rr_;
    if (r >= rows) break;
    const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
    const float* gr = a.g + r * a.ldg;
    float hk[4], zk[4], rhk[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t gi = grouped ? min(r * G + (c0 + 256 * k) / 128 + (lane >> 5), rows * G - 1)
                                 : r;
      hk[k] = pass ? 1.f : a.h[gi];
      zk[k] = pass ? 0.f : a.z[gi];
      rhk[k] = 1.f / hk[k];
    }
    const float vrow = a.rowvec ? a.rowvec[r] : 0.f;
    float shk[4] = {0.f, 0.f, 0.f, 0.f}, szk[4] = {0.f, 0.f, 0.f, 0.f};
    // the row's 16 elements of this lane: x~, then rint(x~ / h) by the reciprocal
    // product; elements within |u| 2^-20 of a half-integer (or not finite) take the
    // exact quotient behind wave-uniform branches (a divergent branch per element
    // would be flattened into a division for every element)
    float v[16], gg[16], xd[16], xt[16], u[16], rq[16];
    bool near = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t c = c0 + lane * 4 + 256 * k;
      const bool ok = c < cols;
      float vv[4] = {0.f, 0.f, 0.f, 0.f};
      float4 g4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok) {
        load4(xr, XDT, c, vv);
        g4 = *reinterpret_cast<const float4*>(gr + c);
      }
      const float g1[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ai = k * 4 + j;
        v[ai] = vv[j];
        gg[ai] = g1[j];
        // x~ (exact for MUL / NONE; within 2 ulp for DIV, used only in sums)
        xd[ai] = v[ai] - dc[ai];
        xt[ai] = LET == OMQ_LET_DIV ? xd[ai] * rc[ai]
                 : LET == OMQ_LET_MUL ? sc[ai] * v[ai] : v[ai];
        u[ai] = xt[ai] * rhk[k];
        rq[ai] = rintf(u[ai]);
        near |= ok && !(fabsf(fabsf(u[ai] - rq[ai]) - 0.5f) > fabsf(u[ai]) * 0x1p-20f);
      }
    }
    if (!pass && __builtin_amdgcn_ballot_w64(near) != 0) {
#pragma unroll
      for (int ai = 0; ai < 16; ++ai) {
        const bool ne = !(fabsf(fabsf(u[ai] - rq[ai]) - 0.5f) > fabsf(u[ai]) * 0x1p-20f);
        if (__builtin_amdgcn_ballot_w64(ne) != 0) {
          if (ne) {
            u[ai] = LET == OMQ_LET_DIV ? (xd[ai] / sc[ai]) / hk[ai >> 2] : xt[ai] / hk[ai >> 2];
            rq[ai] = rintf(u[ai]);
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t c = c0 + lane * 4 + 256 * k;
      const float z = zk[k];
      float sh = 0.f, sz = 0.f;
      float up[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ai = k * 4 + j;
        float gns;
        if (pass) {
          gns = gg[ai];
        } else {
          const float rr = rq[ai] + z;
          const bool in = (rr >= 0.f) && (rr <= Q);
          const float qmz = fminf(fmaxf(rr, 0.f), Q) - z;
          sh += gg[ai] * (qmz - (in ? u[ai] : 0.f));
          sz += in ? 0.f : gg[ai];
          gns = in ? gg[ai] : 0.f;
        }
        if constexpr (COL == COL_WEIGHT) {
          acc0[ai] += gns * v[ai];
          acc1[ai] += vrow * v[ai];
        } else if constexpr (COL == COL_ACT_DIV) {
          acc0[ai] += gns * (-xt[ai] * rc[ai]);
          acc1[ai] += gns * (-rc[ai]);
        } else if constexpr (COL == COL_ACT_MUL) {
          acc0[ai] += gns * v[ai];
        }
        up[j] = LET == OMQ_LET_DIV ? gns * rc[ai] : LET == OMQ_LET_MUL ? gns * sc[ai] : gns;
      }
      if (a.gx && c < cols)
        *reinterpret_cast<float4*>(a.gx + r * a.ldgx + c) = make_float4(up[0], up[1], up[2], up[3]);
      shk[k] = sh;
      szk[k] = sz;
    }
    if (!pass) {
      if (grouped) {
        // one partial per (row, group): sum over the half-wave
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float sh = shk[k], sz = szk[k];
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) {
            sh += __shfl_xor(sh, o, kWave);
            sz += __shfl_xor(sz, o, kWave);
          }
          const int64_t cg = c0 + 256 * k + 128 * (lane >> 5);
          if ((lane & 31) == 0 && cg < cols) {
            rowpart[(r * G + cg / 128) * 2 + 0] = sh;
            rowpart[(r * G + cg / 128) * 2 + 1] = sz;
          }
        }
      } else {
        float sh = shk[0] + shk[1] + shk[2] + shk[3];
        float sz = szk[0] + szk[1] + szk[2] + szk[3];
        sh = wave_sum(sh);
        sz = wave_sum(sz);
        if (lane == 0) {
          rowpart[(r * gridDim.x + blockIdx.x) * 2 + 0] = sh;
          rowpart[(r * gridDim.x + blockIdx.x) * 2 + 1] = sz;
        }
      }
    }
  }
  if constexpr (COL == COL_NONE) return;
  __shared__ float red[4][2][kSlab];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      red[wid][0][lane * 4 + 256 * k + j] = acc0[k * 4 + j];
      red[wid][1][lane * 4 + 256 * k + j] = acc1[k * 4 + j];
    }
  __syncthreads();
  for (int cl = tid; cl < kSlab; cl += kThreads) {
    const int64_t c = c0 + cl;
    if (c >= cols) continue;
    float s0 = red[0][0][cl] + red[1][0][cl] + red[2][0][cl] + red[3][0][cl];
    float s1 = red[0][1][cl] + red[1][1][cl] + red[2][1][cl] + red[3][1][cl];
    colpart[((int64_t)blockIdx.y * 2 + 0) * cols + c] = s0;
    colpart[((int64_t)blockIdx.y * 2 + 1) * cols + c] = s1;
  }
}

// One quantizer row's finalizer, in two parts.  row_fetch: the row's segment
// (concatenated weights: its x rows and logits), its extreme columns, and every
// value that depends on them alone (x and x~ there, the LET scale and shift there,
// the upstream gradient there, the tile's column partials there when the terms
// are merged) and the clipping strengths, all issued in one round once the extreme
// columns have arrived and before the row's partial sums are read, so the
// dependent loads overlap them.  row_finish: the LWC-logit gradients, the max / min
// scatter into the upstream gradient (one writer per row), and the row's two
// scatter terms of the column outputs (column, term for out0, term for out1:
// argmax first, then argmin).  gh, gzs: the row's summed partials.
struct RowFetch {
  int64_t r, pl;
  float *gg_g, *gg_b;
  int iM, im;
  float xM, xm, M, m, gamma, beta;
  float sv[2];          // LET scale at arg_max, arg_min (1 without LET)
  float gxo[2];         // upstream gradient there before the scatter (with gx)
  float cp0[2], cp1[2]; // the tile's two column partials there (merged terms)
};

template <int XDT>
OMQ_DEV RowFetch row_fetch(const RowQuantBwd& a, int64_t p, const float* colpart, int64_t t,
                           bool merge) {
  RowFetch f;
  const int64_t ng = a.group > 0 ? a.cols / 128 : 1;
  f.r = p / ng;
  const void* xb = a.x;
  const float *lg_g = a.a_gamma, *lg_b = a.a_beta;
  f.gg_g = a.g_agamma;
  f.gg_b = a.g_abeta;
  int64_t rl = f.r;
  f.pl = p;
  if (a.nseg > 1) {
    const int sg = (f.r >= a.seg_end[0]) + (a.nseg > 2 && f.r >= a.seg_end[1]);
    const int64_t r0 = sg == 0 ? 0 : a.seg_end[sg - 1];
    xb = a.xseg[sg];
    lg_g = a.agseg[sg]; lg_b = a.abseg[sg]; f.gg_g = a.gagseg[sg]; f.gg_b = a.gabseg[sg];
    rl = f.r - r0;
    f.pl = p - r0 * ng;
  }
  const char* xr = reinterpret_cast<const char*>(xb) + rl * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
  auto xval = [&](int64_t c) -> float {
    return XDT == OMQ_F32 ? reinterpret_cast<const float*>(xr)[c]
                          : bf16_to_f32(reinterpret_cast<const uint16_t*>(xr)[c]);
  };
  f.iM = a.amax[p];
  f.im = a.amin[p];
  const int idx[2] = {f.iM, f.im};
  float xo[2], dl[2] = {0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int c = idx[e];
    xo[e] = xval(c);
    f.sv[e] = a.let_mode != OMQ_LET_NONE ? a.s[c] : 1.f;
    if (a.let_mode == OMQ_LET_DIV && a.delta) dl[e] = a.delta[c];
    f.gxo[e] = a.gx ? a.gx[f.r * a.ldgx + c] : 0.f;
    f.cp0[e] = merge ? colpart[(t * 2 + 0) * a.cols + c] : 0.f;
    f.cp1[e] = merge ? colpart[(t * 2 + 1) * a.cols + c] : 0.f;
  }
  f.xM = xo[0];
  f.xm = xo[1];
  // x~ exactly as the forward formed it (the LET of the quantizer's input)
  auto let = [&](float x, int e) {
    if (a.let_mode == OMQ_LET_DIV) return (x - dl[e]) / f.sv[e];
    if (a.let_mode == OMQ_LET_MUL) return f.sv[e] * x;
    return x;
  };
  f.M = let(f.xM, 0);
  f.m = let(f.xm, 1);
  f.gamma = lg_g ? sigmoid_f32(lg_g[f.pl]) : 1.f;
  f.beta = lg_b ? sigmoid_f32(lg_b[f.pl]) : 1.f;
  return f;
}

OMQ_DEV void row_finish(const RowQuantBwd& a, const RowFetch& f, float gh, float gzs,
                        int (&cs)[2], float (&v0)[2], float (&v1)[2]) {
  const float M = f.M, m = f.m, gamma = f.gamma, beta = f.beta;
  const RowQ q = row_step(M, m, gamma, beta, a.nbits);
  const float h = q.h;
  const float gz = -h * gzs;
  const float G = q.floor ? 0.f : gh + gz * q.t2 / (h * h);
  const float gt1 = G / q.Q;
  const float gt2 = -G / q.Q - gz / h;
  const float gM = gt1 * gamma, gm = gt2 * beta;
  if (f.gg_g) f.gg_g[f.pl] = (gt1 * M) * gamma * (1.f - gamma);
  if (f.gg_b) f.gg_b[f.pl] = (gt2 * m) * beta * (1.f - beta);
  // scatter of dL/dmax and dL/dmin into the gradient of x~ at arg_max / arg_min
  const int idx[2] = {f.iM, f.im};
  const float gv[2] = {gM, gm};
  const float xo[2] = {f.xM, f.xm};
  const float xtl[2] = {M, m};
  float up[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int c = idx[e];
    const float gsc = gv[e];
    up[e] = gsc;
    if (a.let_mode == OMQ_LET_DIV) up[e] = gsc / f.sv[e];
    else if (a.let_mode == OMQ_LET_MUL) up[e] = gsc * f.sv[e];
    cs[e] = c;
    const bool div = a.col_mode == COL_ACT_DIV;
    const bool mul = a.col_mode == COL_WEIGHT || a.col_mode == COL_ACT_MUL;
    v0[e] = div ? gsc * (-xtl[e] / f.sv[e]) : mul ? gsc * xo[e] : 0.f;
    v1[e] = div ? gsc * (-1.f / f.sv[e]) : 0.f;
  }
  // the argmax term first, then the argmin term, on the value read before either
  if (a.gx) {
    float* gr = a.gx + f.r * a.ldgx;
    if (f.iM == f.im) {
      gr[f.iM] = (f.gxo[0] + up[0]) + up[1];
    } else {
      gr[f.iM] = f.gxo[0] + up[0];
      gr[f.im] = f.gxo[1] + up[1];
    }
  }
}

// Row finalizers, one workgroup per (column-partial tile, column group): the tile's
// tile_rows rows (for group-wise rows, their quantizer rows of one 128-column group)
// in one pass, LPR lanes per row summing its per-slab partials; then the rows'
// scatter terms of the column outputs are merged by the first wave alone and added
// to the tile's column partials in row order: the first of the tile's terms on a
// column adds, in row order, every term on that column.  The tile's partials of
// those columns have this workgroup as their only writer, so the column pass that
// follows sums everything in a fixed order.
constexpr int kFinThreads = 1024;

// The finalizers of one unit (bid: the workgroup's index within its job).
template <int XDT, int LPR>
OMQ_DEV void ste_rows_unit(const RowQuantBwd& a, int nslabs, const float* rowpart,
                           int tile_rows, float* colpart, int merge, int64_t bid) {
  __shared__ int e_col[256];
  __shared__ float e_v0[256], e_v1[256], e_c0[256], e_c1[256];
  const int64_t ng = a.group > 0 ? a.cols / 128 : 1;
  const int64_t t = bid / ng, g = bid % ng;
  const int64_t r0 = t * tile_rows;
  const int nr = (int)min((int64_t)tile_rows, a.rows - r0);
  const int sub = (int)(threadIdx.x % LPR);
  const int i = (int)(threadIdx.x / LPR);               // row of the tile
  const bool valid = i < nr;
  const int64_t p = (r0 + i) * ng + g;                  // its quantizer row
  RowFetch rf;
  if (valid && sub == 0) rf = row_fetch<XDT>(a, p, colpart, t, merge != 0);
  float gh = 0.f, gzs = 0.f;
  if (valid) {
    for (int s = sub; s < nslabs; s += LPR) {
      const float2 v = *reinterpret_cast<const float2*>(&rowpart[(p * nslabs + s) * 2]);
      gh += v.x;
      gzs += v.y;
    }
  }
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) {
    gh += __shfl_xor(gh, o);
    gzs += __shfl_xor(gzs, o);
  }
  if (valid && sub == 0) {
    int cs[2];
    float v0[2], v1[2];
    row_finish(a, rf, gh, gzs, cs, v0, v1);
    if (merge) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        e_col[2 * i + e] = cs[e];
        e_v0[2 * i + e] = v0[e];
        e_v1[2 * i + e] = v1[e];
        e_c0[2 * i + e] = rf.cp0[e];
        e_c1[2 * i + e] = rf.cp1[e];
      }
    }
  }
  if (!merge) return;                                   // uniform over the workgroup
  // every row's terms are in LDS before the first wave reads them
  __syncthreads();
  if (threadIdx.x >= 64) return;
  // The first wave merges the (at most 256) terms in registers, 4 per lane: term
  // slot e = 4 lane + k.  Sort by (column, term index), a bitonic network whose
  // partners are in the lane (distance 1, 2) or 4 slots per lane apart (a lane
  // exchange); the unused slots are keyed past every column.
  const int ln = (int)threadIdx.x;
  const int ne = 2 * nr;
  int key[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = 4 * ln + k;
    key[k] = e < ne ? (e_col[e] << 8) | e : 0x7fffffff;
  }
#pragma unroll
  for (int kb = 2; kb <= 256; kb <<= 1) {
#pragma unroll
    for (int j = kb >> 1; j > 0; j >>= 1) {
      int pk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pk[k] = j >= 4 ? __shfl_xor(key[k], j >> 2, 64) : key[k ^ j];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = 4 * ln + k, o = e ^ j;
        const bool asc = (e & kb) == 0;
        key[k] = (asc == (e < o)) ? min(key[k], pk[k]) : max(key[k], pk[k]);
      }
    }
  }
  // a segmented inclusive scan of each column's run (the tree of offsets 1, 2, 4,
  // ..., 128), then the last term of each run adds the run's total to the tile's
  // partial of that column (read before any term was added)
  int col[4], hd[4];
  float s0[4], s1[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = 4 * ln + k;
    col[k] = key[k] >> 8;
    s0[k] = e < ne ? e_v0[key[k] & 255] : 0.f;
    s1[k] = e < ne ? e_v1[key[k] & 255] : 0.f;
  }
  {
    const int pc = __shfl_up(col[3], 1, 64);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 4 * ln + k;
      hd[k] = e == 0 || (k > 0 ? col[k - 1] : pc) != col[k];
    }
  }
#pragma unroll
  for (int off = 1; off < 256; off <<= 1) {
    float a0[4], a1[4];
    int ah[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (off >= 4) {
        a0[k] = __shfl_up(s0[k], off >> 2, 64);
        a1[k] = __shfl_up(s1[k], off >> 2, 64);
        ah[k] = __shfl_up(hd[k], off >> 2, 64);
      } else if (k >= off) {
        a0[k] = s0[k - off];
        a1[k] = s1[k - off];
        ah[k] = hd[k - off];
      } else {
        a0[k] = __shfl_up(s0[(k - off + 4) & 3], 1, 64);
        a1[k] = __shfl_up(s1[(k - off + 4) & 3], 1, 64);
        ah[k] = __shfl_up(hd[(k - off + 4) & 3], 1, 64);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 4 * ln + k;
      if (!hd[k] && e >= off) {
        s0[k] += a0[k];
        s1[k] += a1[k];
        hd[k] = ah[k];
      }
    }
  }
  const int nc = __shfl_down(col[0], 1, 64);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = 4 * ln + k;
    const int cn = k < 3 ? col[k + 1] : nc;
    if (e < ne && (e == ne - 1 || cn != col[k])) {
      const int te = key[k] & 255;
      colpart[(t * 2 + 0) * a.cols + col[k]] = e_c0[te] + s0[k];
      colpart[(t * 2 + 1) * a.cols + col[k]] = e_c1[te] + s1[k];
    }
  }
}

template <int XDT, int LPR>
__global__ __launch_bounds__(kFinThreads) void k_ste_rows(RowQuantBwd a, int nslabs,
                                                          const float* rowpart, int tile_rows,
                                                          float* colpart, int merge) {
  ste_rows_unit<XDT, LPR>(a, nslabs, rowpart, tile_rows, colpart, merge, blockIdx.x);
}

// Up to kMaxRowJobs independent finalizer jobs in one launch: job j takes the
// workgroups [sum of the earlier jobs' units, + its own units).  Each job is read
// through a constant index (a run-time index into the argument block would copy it
// to scratch memory).
struct SteRowsJob {
  RowQuantBwd a;
  const float* rowpart;
  float* colpart;
  int nslabs, tile_rows, merge, units;
};
struct SteRowsJobs {
  SteRowsJob j[kMaxRowJobs];
  int n;
};

// (at most 64 registers, so two workgroups of 16 waves fit on a compute unit)
template <int XDT, int LPR>
__global__ __launch_bounds__(kFinThreads) __attribute__((amdgpu_waves_per_eu(8)))
void k_ste_rows_multi(SteRowsJobs m) {
  int64_t bid = blockIdx.x;
#pragma unroll
  for (int q = 0; q < kMaxRowJobs; ++q) {
    if (q < m.n) {
      const SteRowsJob& jb = m.j[q];
      if (bid < jb.units) {
        ste_rows_unit<XDT, LPR>(jb.a, jb.nslabs, jb.rowpart, jb.tile_rows, jb.colpart,
                                jb.merge, bid);
        return;
      }
      bid -= jb.units;
    }
  }
}

// Column pass of a straight-through backward, after the row finalizers: per column c
// (64 per workgroup, 4 waves)
//   out_k[c] = (accumulate ? out_k[c] : 0) + sum_t colpart_k[t][c]
// the waves taking the partial rows t = w, w + 4, ..., their sums added in LDS in
// wave order.  Deterministic: no atomics anywhere.
OMQ_DEV void ste_cols_unit(const float* colpart, int ntiles, int64_t cols, float* out0,
                           float* out1, int accumulate, int64_t bid) {
  __shared__ float red[2][4][64];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int64_t c = bid * 64 + lane;
  float s0 = 0.f, s1 = 0.f;
  if (c < cols) {
#pragma unroll 4
    for (int t = w; t < ntiles; t += 4) {
      s0 += colpart[((int64_t)t * 2 + 0) * cols + c];
      s1 += colpart[((int64_t)t * 2 + 1) * cols + c];
    }
  }
  red[0][w][lane] = s0;
  red[1][w][lane] = s1;
  __syncthreads();
  if (w < 2 && c < cols) {
    float* o = w == 0 ? out0 : out1;
    if (o) {
      const float cs = ((red[w][0][lane] + red[w][1][lane]) + red[w][2][lane]) + red[w][3][lane];
      o[c] = (accumulate ? o[c] : 0.f) + cs;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_ste_cols(const float* colpart, int ntiles,
                                                       int64_t cols, float* out0, float* out1,
                                                       int accumulate) {
  ste_cols_unit(colpart, ntiles, cols, out0, out1, accumulate, blockIdx.x);
}

struct SteColsJob {
  const float* colpart;
  float *out0, *out1;
  int64_t cols;
  int ntiles, accumulate, units;
};
struct SteColsJobs {
  SteColsJob j[kMaxFinJobs];
  int n;
};

__global__ __launch_bounds__(kThreads) void k_ste_cols_multi(SteColsJobs m) {
  int64_t bid = blockIdx.x;
#pragma unroll
  for (int q = 0; q < kMaxFinJobs; ++q) {
    if (q < m.n) {
      const SteColsJob& jb = m.j[q];
      if (bid < jb.units) {
        ste_cols_unit(jb.colpart, jb.ntiles, jb.cols, jb.out0, jb.out1, jb.accumulate, bid);
        return;
      }
      bid -= jb.units;
    }
  }
}

// ---------------------------------------------------------------------------
// LET alone, bias fold, column sums
// ---------------------------------------------------------------------------
template <int XDT>
__global__ __launch_bounds__(kThreads) void k_let(const void* x, int64_t rows, int64_t cols,
                                                  int mode, const float* s, const float* delta,
                                                  void* y, int y_dt) {
  const int64_t n4 = rows * cols / 4;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t e = i * 4;
    const int64_t c = e % cols;
    float v[4];
    load4(x, XDT, e, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = let_x(v[j], mode, s, delta, c + j);
    store4(y, y_dt, e, v);
  }
}

template <int XDT>
__global__ __launch_bounds__(kThreads) void k_bias_fold(const void* W, int64_t rows, int64_t cols,
                                                        const float* delta, const float* B,
                                                        float* out) {
  const int64_t r = blockIdx.x;
  const char* wr = reinterpret_cast<const char*>(W) + r * cols * (XDT == OMQ_F32 ? 4 : 2);
  float dot = 0.f;
  for (int64_t c = (int64_t)threadIdx.x * 4; c < cols; c += 4 * kThreads) {
    float v[4];
    load4(wr, XDT, c, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) dot = fmaf(delta[c + j], v[j], dot);
  }
  dot = wave_sum(dot);
  __shared__ float sd[4];
  if ((threadIdx.x & 63) == 0) sd[threadIdx.x >> 6] = dot;
  __syncthreads();
  if (threadIdx.x == 0) out[r] = (B ? B[r] : 0.f) + ((sd[0] + sd[1]) + (sd[2] + sd[3]));
}

__global__ __launch_bounds__(kThreads) void k_colsum_part(const float* in, int64_t rows,
                                                          int64_t cols, int64_t ld, float* part) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * kColsumRows;
  float s = 0.f;
  for (int64_t r = r0; r < r0 + kColsumRows && r < rows; ++r) s += in[r * ld + c];
  part[(int64_t)blockIdx.y * cols + c] = s;
}

// dY in float32 -> its bf16 copy (the matrix-core operand) and, when `part` is
// set, the column sums of each kColsumRows-row chunk, in one pass over dY.
// VEC 8 (cols % 8 == 0): a workgroup takes 512 columns (8 per lane) of one chunk,
// its 4 waves take the chunk's rows in turn, and their sums are added in LDS in a
// fixed order.  VEC 1: one column per thread over the chunk.  ROPE (VEC 8 only):
// the columns of the Q and K heads come from rp.q / rp.k through the inverse RoPE,
// x c + x' s in the first half of a head and x c - x' s in the second, x' the
// element 64 positions away and c, s the row's table entries (products rounded
// before the sum, as in the rotation kernel).
template <int VEC, bool ROPE = false>
__global__ __launch_bounds__(kThreads) void k_cvt_bf16_colpart(const float* __restrict__ in,
                                                               int64_t rows, int64_t cols,
                                                               uint16_t* __restrict__ out,
                                                               float* __restrict__ part,
                                                               RopeIn rp = {}) {
  const int64_t r0 = (int64_t)blockIdx.y * kColsumRows;
  const int64_t r1 = min(r0 + kColsumRows, rows);
  if constexpr (VEC == 8) {
    __shared__ float4 red[4][2][64];
    const int lane = threadIdx.x & 63, w = wave_id();
    const int64_t c = ((int64_t)blockIdx.x * 64 + lane) * 8;
    const bool ok = c < cols;
    // (ROPE) this thread's 8 columns: their source, the partner offset, the sign
    const bool rot = ROPE && c < rp.qcols + rp.kcols;
    const bool isq = c < rp.qcols;
    const float* src = !rot ? nullptr : isq ? rp.q + c : rp.k + (c - rp.qcols);
    const int64_t lds = isq ? rp.ldq : rp.ldk;
    const int kh = (int)(c & 127);                 // position in the head (qcols % 128 == 0)
    const int pofs = kh < 64 ? 64 : -64;
    const float sg = kh < 64 ? 1.f : -1.f;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ok) {
#pragma unroll 4
      for (int64_t r = r0 + w; r < r1; r += 4) {
        float4 a, b;
        if (rot) {
          const float* x = src + r * lds;
          const float* cs = rp.cos_t + r * 64 + (kh & 63);
          const float* sn = rp.sin_t + r * 64 + (kh & 63);
          const float4 x0 = *reinterpret_cast<const float4*>(x);
          const float4 x1 = *reinterpret_cast<const float4*>(x + 4);
          const float4 p0 = *reinterpret_cast<const float4*>(x + pofs);
          const float4 p1 = *reinterpret_cast<const float4*>(x + pofs + 4);
          const float4 c0 = *reinterpret_cast<const float4*>(cs);
          const float4 c1 = *reinterpret_cast<const float4*>(cs + 4);
          const float4 s0 = *reinterpret_cast<const float4*>(sn);
          const float4 s1 = *reinterpret_cast<const float4*>(sn + 4);
          // sg * (p s) is exact: the sum is the rotation kernel's a c + b s or b c - a s
          a = make_float4(x0.x * c0.x + sg * (p0.x * s0.x), x0.y * c0.y + sg * (p0.y * s0.y),
                          x0.z * c0.z + sg * (p0.z * s0.z), x0.w * c0.w + sg * (p0.w * s0.w));
          b = make_float4(x1.x * c1.x + sg * (p1.x * s1.x), x1.y * c1.y + sg * (p1.y * s1.y),
                          x1.z * c1.z + sg * (p1.z * s1.z), x1.w * c1.w + sg * (p1.w * s1.w));
        } else {
          const float* p = in + r * cols + c;
          a = *reinterpret_cast<const float4*>(p);
          b = *reinterpret_cast<const float4*>(p + 4);
        }
        s[0] += a.x; s[1] += a.y; s[2] += a.z; s[3] += a.w;
        s[4] += b.x; s[5] += b.y; s[6] += b.z; s[7] += b.w;
        *reinterpret_cast<uint4*>(out + r * cols + c) =
            make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y),
                       pack_bf16(b.z, b.w));
      }
    }
    if (!part) return;                               // uniform over the workgroup
    red[w][0][lane] = make_float4(s[0], s[1], s[2], s[3]);
    red[w][1][lane] = make_float4(s[4], s[5], s[6], s[7]);
    __syncthreads();
    if (w < 2 && ok) {
      float4 acc = red[0][w][lane];
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const float4 v = red[q][w][lane];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
      *reinterpret_cast<float4*>(part + (int64_t)blockIdx.y * cols + c + 4 * w) = acc;
    }
  } else {
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= cols) return;
    float s0 = 0.f;
    for (int64_t r = r0; r < r1; ++r) {
      const float v = in[r * cols + c];
      s0 += v;
      out[r * cols + c] = f32_to_bf16(v);
    }
    if (part) part[(int64_t)blockIdx.y * cols + c] = s0;
  }
}


// Column sums of partial rows: out_k[c] (+)= sum_t part[(t * nk + k) * cols + c] for
// the nk (1 or 2) kinds.  A workgroup takes 64 columns; its 16 waves take the
// partial rows t = w, w + 16, ... (one coalesced 256-byte segment per row), and the
// 16 wave sums are added in LDS in a fixed order, so the result is deterministic.
constexpr int kSumWaves = 16;

__global__ __launch_bounds__(kSumWaves * 64) void k_part_colsum(const float* part, int nparts,
                                                                int nk, int64_t cols,
                                                                float* out0, float* out1,
                                                                int accumulate) {
  __shared__ float red[2][kSumWaves][64];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  float s[2] = {0.f, 0.f};
  if (c < cols) {
#pragma unroll 4
    for (int t = w; t < nparts; t += kSumWaves)
      for (int k = 0; k < nk; ++k) s[k] += part[((int64_t)t * nk + k) * cols + c];
  }
  red[0][w][lane] = s[0];
  red[1][w][lane] = s[1];
  __syncthreads();
  if (w < nk && c < cols) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < kSumWaves; ++q) t += red[w][q][lane];
    float* o = w == 0 ? out0 : out1;
    if (o) o[c] = (accumulate ? o[c] : 0.f) + t;
  }
}

int bwd_rows_per_tile(int64_t rows) { return rows >= 8192 ? 32 : 16; }

}  // namespace

hipError_t launch_part_colsum(const float* part, int nparts, int nk, int64_t cols, float* out0,
                              float* out1, int accumulate, hipStream_t st) {
  if (cols == 0 || (!out0 && !out1)) return hipSuccess;
  hipLaunchKernelGGL(k_part_colsum, dim3((unsigned)((cols + 63) / 64)), dim3(kSumWaves * 64), 0,
                     st, part, nparts, nk, cols, out0, out1, accumulate);
  return hipGetLastError();
}

template <int XDT>
bool launch_fwd_wave(const RowQuantFwd& a, hipStream_t st) {
  // 16-byte row loads: bf16 rows must start on 8-element boundaries
  if (XDT == OMQ_BF16 && (a.ldx % 8)) return false;
  const int64_t nc = (a.cols + 511) / 512;
  dim3 grid((unsigned)((a.rows + 3) / 4));
#define OMQ_FWD_WAVE_L(N, F)                                                                  \
  if (a.let_mode == OMQ_LET_DIV)                                                              \
    hipLaunchKernelGGL((k_rowquant_fwd_wave<XDT, N, OMQ_LET_DIV, F>), grid, dim3(kThreads), 0, \
                       st, a);                                                                \
  else if (a.let_mode == OMQ_LET_MUL)                                                         \
    hipLaunchKernelGGL((k_rowquant_fwd_wave<XDT, N, OMQ_LET_MUL, F>), grid, dim3(kThreads), 0, \
                       st, a);                                                                \
  else                                                                                        \
    hipLaunchKernelGGL((k_rowquant_fwd_wave<XDT, N, OMQ_LET_NONE, F>), grid, dim3(kThreads), 0,\
                       st, a);
#define OMQ_FWD_LDS(N)                                                                      \
  if (a.let_mode == OMQ_LET_DIV)                                                            \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_DIV>), grid, dim3(kThreads), 0,   \
                       st, a);                                                              \
  else if (a.let_mode == OMQ_LET_MUL)                                                       \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_MUL>), grid, dim3(kThreads), 0,   \
                       st, a);                                                              \
  else                                                                                      \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_NONE>), grid, dim3(kThreads), 0,  \
                       st, a);
#define OMQ_FWD_RMS(N)                                                                      \
  if (a.let_mode == OMQ_LET_DIV)                                                            \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_DIV, true>), grid,               \
                       dim3(kThreads), 0, st, a);                                           \
  else                                                                                      \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_NONE, true>), grid,              \
                       dim3(kThreads), 0, st, a);
#define OMQ_FWD_WAVE(N)                                                                       \
  if (nc <= N) {                                                                              \
    if (a.rms_out && a.cols == N * 512) {                                                     \
      OMQ_FWD_RMS(N)                                                                          \
    } else if (a.cols == N * 512) {                                                           \
      OMQ_FWD_LDS(N)                                                                          \
    } else {                                                                                  \
      OMQ_FWD_WAVE_L(N, false)                                                                \
    }                                                                                         \
    return true;                                                                              \
  }
  OMQ_FWD_WAVE(1) OMQ_FWD_WAVE(2) OMQ_FWD_WAVE(4) OMQ_FWD_WAVE(8)
#undef OMQ_FWD_LDS
#undef OMQ_FWD_RMS
#undef OMQ_FWD_WAVE_L
#undef OMQ_FWD_WAVE
  return false;
}

// rows of 4097 .. 32768 columns, a multiple of 8, with 16-byte aligned rows and
// outputs (the 16-byte loads and stores)
template <int XDT>
bool launch_fwd_blk8(const RowQuantFwd& a, hipStream_t st) {
  if (a.cols % 8 || a.ldx % (XDT == OMQ_F32 ? 4 : 8) || a.ldo % (a.out_dt == OMQ_F32 ? 4 : 8))
    return false;
  const int64_t nch = (a.cols + 8 * kThreads - 1) / (8 * kThreads);
  if (nch > 16) return false;
  dim3 grid((unsigned)a.rows);
#define OMQ_FWD_BLK8(N)                                                                     \
  if (nch <= N) {                                                                           \
    if (a.let_mode == OMQ_LET_DIV)                                                          \
      hipLaunchKernelGGL((k_rowquant_fwd_blk8<XDT, N, OMQ_LET_DIV>), grid, dim3(kThreads), 0, \
                         st, a);                                                            \
    else if (a.let_mode == OMQ_LET_MUL)                                                     \
      hipLaunchKernelGGL((k_rowquant_fwd_blk8<XDT, N, OMQ_LET_MUL>), grid, dim3(kThreads), 0, \
                         st, a);                                                            \
    else                                                                                    \
      hipLaunchKernelGGL((k_rowquant_fwd_blk8<XDT, N, OMQ_LET_NONE>), grid, dim3(kThreads), 0,\
                         st, a);                                                            \
    return true;                                                                            \
  }
  if (a.rope_out) {
    if constexpr (XDT == OMQ_F32) {
#define OMQ_FWD_BLK8P(N)                                                                    \
  if (nch <= N) {                                                                           \
    if (a.let_mode == OMQ_LET_DIV)                                                          \
      hipLaunchKernelGGL((k_rowquant_fwd_blk8<XDT, N, OMQ_LET_DIV, false, true>), grid,     \
                         dim3(kThreads), 0, st, a);                                         \
    else if (a.let_mode == OMQ_LET_MUL)                                                     \
      hipLaunchKernelGGL((k_rowquant_fwd_blk8<XDT, N, OMQ_LET_MUL, false, true>), grid,     \
                         dim3(kThreads), 0, st, a);                                         \
    else                                                                                    \
      hipLaunchKernelGGL((k_rowquant_fwd_blk8<XDT, N, OMQ_LET_NONE, false, true>), grid,    \
                         dim3(kThreads), 0, st, a);                                         \
    return true;                                                                            \
  }
      OMQ_FWD_BLK8P(1) OMQ_FWD_BLK8P(2) OMQ_FWD_BLK8P(4) OMQ_FWD_BLK8P(8) OMQ_FWD_BLK8P(16)
#undef OMQ_FWD_BLK8P
    }
    return false;
  }
  if (a.rms_out) {
#define OMQ_FWD_BLK8R(N)                                                                    \
  if (nch <= N) {                                                                           \
    if (a.let_mode == OMQ_LET_DIV)                                                          \
      hipLaunchKernelGGL((k_rowquant_fwd_blk8<XDT, N, OMQ_LET_DIV, true>), grid,            \
                         dim3(kThreads), 0, st, a);                                         \
    else                                                                                    \
      hipLaunchKernelGGL((k_rowquant_fwd_blk8<XDT, N, OMQ_LET_NONE, true>), grid,           \
                         dim3(kThreads), 0, st, a);                                         \
    return true;                                                                            \
  }
    OMQ_FWD_BLK8R(1) OMQ_FWD_BLK8R(2) OMQ_FWD_BLK8R(4) OMQ_FWD_BLK8R(8) OMQ_FWD_BLK8R(16)
#undef OMQ_FWD_BLK8R
    return false;
  }
  OMQ_FWD_BLK8(1) OMQ_FWD_BLK8(2) OMQ_FWD_BLK8(4) OMQ_FWD_BLK8(6) OMQ_FWD_BLK8(8)
  OMQ_FWD_BLK8(12) OMQ_FWD_BLK8(16)
#undef OMQ_FWD_BLK8
  return false;
}

template <int XDT>
bool launch_fwd_reg(const RowQuantFwd& a, hipStream_t st) {
  const int64_t nch = (a.cols + 4 * kThreads - 1) / (4 * kThreads);
  dim3 grid((unsigned)a.rows);
#define OMQ_FWD_REG(N)                                                                   \
  if (nch <= N) {                                                                        \
    hipLaunchKernelGGL((k_rowquant_fwd_reg<XDT, N>), grid, dim3(kThreads), 0, st, a);  \
    return true;                                                                         \
  }
  OMQ_FWD_REG(1) OMQ_FWD_REG(2) OMQ_FWD_REG(4) OMQ_FWD_REG(8) OMQ_FWD_REG(12)
  OMQ_FWD_REG(16) OMQ_FWD_REG(24) OMQ_FWD_REG(32)
#undef OMQ_FWD_REG
  return false;
}

bool rowquant_fwd_rms_ok(const RowQuantFwd& a) {
  // activations (no logits, no fold), LET divide or none: the whole-row LDS kernel
  // (512 or 1024 columns) or the block-per-row kernel (2048 .. 32768, multiples of 8)
  return a.group == 0 && a.nbits < 16 && a.nseg == 1 && !a.fold_delta && !a.a_gamma &&
         (a.let_mode == OMQ_LET_DIV || a.let_mode == OMQ_LET_NONE) && a.ldx == a.cols &&
         (a.cols == 512 || a.cols == 1024 || (a.cols >= 2048 && a.cols <= 32768 && a.cols % 8 == 0)) &&
         (a.x_dt == OMQ_F32 || a.ldx % 8 == 0);
}

bool rowquant_fwd_rope_ok(const RowQuantFwd& a) {
  // float32 activations in heads of 128 columns (no logits, fold or normalization):
  // the block-per-row kernel, rows of 2048 .. 32768 columns
  return a.group == 0 && a.nbits < 16 && a.nseg == 1 && !a.fold_delta && !a.a_gamma &&
         !a.rms_out && a.x_dt == OMQ_F32 && a.cols % 128 == 0 && a.cols >= 2048 &&
         a.cols <= 32768 && a.ldx % 4 == 0 && a.ldo % (a.out_dt == OMQ_F32 ? 4 : 8) == 0 &&
         a.rope_cos && a.rope_sin;
}

bool rowquant_fwd_segments_ok(const RowQuantFwd& a) {
  // the whole-row LDS kernel: rows of 512 n columns (n <= 8), 16-byte rows
  return a.group == 0 && a.nbits < 16 &&
         (a.cols == 512 || a.cols == 1024 || a.cols == 2048 || a.cols == 4096) &&
         (a.x_dt == OMQ_F32 || a.ldx % 8 == 0);
}

hipError_t launch_rowquant_fwd(const RowQuantFwd& a, hipStream_t st) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  if (a.nseg > 1 && (!rowquant_fwd_segments_ok(a) || a.nseg > 3)) return hipErrorInvalidValue;
  if (a.rms_out && !rowquant_fwd_rms_ok(a)) return hipErrorInvalidValue;
  // two 4-bit codes to a byte: 4-bit codes at most, stored as q, whole 8-column chunks
  if (a.codes && a.code_pack &&
      (a.nbits > 4 || a.code_off != 0 || a.cols % 8 || (a.ldq && a.ldq % 4)))
    return hipErrorInvalidValue;
  if (a.rope_out) {
    if (!rowquant_fwd_rope_ok(a) || (a.qsum && !a.codes)) return hipErrorInvalidValue;
    if (a.codes && a.code_off != 0 && a.code_off != 128) return hipErrorInvalidValue;
    if (!launch_fwd_blk8<OMQ_F32>(a, st)) return hipErrorInvalidValue;
    return hipGetLastError();
  }
  // code sums come with the codes, per whole row
  if (a.qsum && (!a.codes || a.group > 0 || a.nbits >= 16)) return hipErrorInvalidValue;
  // stored codes are q itself or q - 128 (8-bit codes as signed bytes)
  if (a.codes && a.code_off != 0 && a.code_off != 128) return hipErrorInvalidValue;
  if (a.group > 0) {           // groups of 128 (the caller checked cols % 128 == 0)
    if (a.group != 128 || a.cols % 128 || a.nbits >= 16 || a.fold_delta)
      return hipErrorInvalidValue;
    const int64_t n = a.rows * (a.cols / 128);
    dim3 gg((unsigned)((n + 15) / 16));
    if (a.x_dt == OMQ_F32)
      hipLaunchKernelGGL(k_rowquant_fwd_g128<OMQ_F32>, gg, dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL(k_rowquant_fwd_g128<OMQ_BF16>, gg, dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  dim3 grid((unsigned)a.rows);
  if (a.nbits >= 16 && a.cols % 8 == 0 && a.ldx % 8 == 0 && a.ldo % 8 == 0 &&
      (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0 &&
      (a.let_mode == OMQ_LET_NONE ||
       ((reinterpret_cast<uintptr_t>(a.s) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(a.delta) & 15) == 0))) {
    const int64_t n8 = a.rows * (a.cols / 8);
    const unsigned nb = (unsigned)std::min<int64_t>((n8 + kThreads - 1) / kThreads, 8192);
#define OMQ_PASS8(XD)                                                                        \
  if (a.let_mode == OMQ_LET_DIV)                                                             \
    hipLaunchKernelGGL((k_rowquant_pass8<XD, OMQ_LET_DIV>), dim3(nb), dim3(kThreads), 0, st, a); \
  else if (a.let_mode == OMQ_LET_MUL)                                                        \
    hipLaunchKernelGGL((k_rowquant_pass8<XD, OMQ_LET_MUL>), dim3(nb), dim3(kThreads), 0, st, a); \
  else                                                                                       \
    hipLaunchKernelGGL((k_rowquant_pass8<XD, OMQ_LET_NONE>), dim3(nb), dim3(kThreads), 0, st, a);
    if (a.x_dt == OMQ_F32) {
      OMQ_PASS8(OMQ_F32)
    } else {
      OMQ_PASS8(OMQ_BF16)
    }
#undef OMQ_PASS8
    return hipGetLastError();
  }
  if (a.nbits < 16) {
    // float32 rows of 2048 .. 4096 columns (activations): a block per row in registers
    // keeps more rows in flight than staging each in LDS (16 KB a row)
    bool done = (a.x_dt == OMQ_F32 || a.rms_out) && a.nseg == 1 && a.cols >= 2048 &&
                (a.cols <= 4096 || a.rms_out) &&
                (a.x_dt == OMQ_F32 ? launch_fwd_blk8<OMQ_F32>(a, st)
                                   : launch_fwd_blk8<OMQ_BF16>(a, st));
    if (!done)
      done = a.x_dt == OMQ_F32 ? launch_fwd_wave<OMQ_F32>(a, st)
                               : launch_fwd_wave<OMQ_BF16>(a, st);
    if (!done)
      done = a.x_dt == OMQ_F32 ? launch_fwd_blk8<OMQ_F32>(a, st) : launch_fwd_blk8<OMQ_BF16>(a, st);
    if (!done)
      done = a.x_dt == OMQ_F32 ? launch_fwd_reg<OMQ_F32>(a, st) : launch_fwd_reg<OMQ_BF16>(a, st);
    if (done) return hipGetLastError();
  }
  if (a.x_dt == OMQ_F32)
    hipLaunchKernelGGL(k_rowquant_fwd<OMQ_F32>, grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_rowquant_fwd<OMQ_BF16>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// sums of uint8 codes per row: one wave per row (off the calibration path, where the
// quantizer forms the sums while it writes the codes)
__global__ __launch_bounds__(kThreads) void k_code_rowsum(const uint8_t* codes, int64_t rows,
                                                          int64_t cols, int64_t ld, int32_t* sums) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave_id();
  if (r >= rows) return;
  const uint8_t* p = codes + r * ld;
  int s = 0;
  for (int64_t c = lane; c < cols; c += 64) s += p[c];
  s = wave_sum(s);
  if (lane == 0) sums[r] = s;
}

hipError_t launch_code_rowsum(const uint8_t* codes, int64_t rows, int64_t cols, int64_t ld,
                              int32_t* sums, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_code_rowsum, dim3((unsigned)((rows + 3) / 4)), dim3(kThreads), 0, st, codes,
                     rows, cols, ld, sums);
  return hipGetLastError();
}

size_t rowquant_bwd_ws_bytes(int64_t rows, int64_t cols) {
  // row partials per column slab, or per 128-column group for grouped rows
  const int64_t nslabs = (cols + 127) / 128;
  const int R = bwd_rows_per_tile(rows);
  const int64_t ntiles = (rows + R - 1) / R;
  return ste_partials_floats(rows, cols, nslabs, ntiles) * sizeof(float);
}

hipError_t launch_rowquant_bwd(const RowQuantBwd& a, hipStream_t st) {
  return launch_rowquant_bwd_tiles(a, st, nullptr);
}

hipError_t launch_rowquant_bwd_tiles(const RowQuantBwd& a, hipStream_t st, SteFinJob* job) {
  if (job) *job = SteFinJob{};        // nothing to finish unless filled in below
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  if (a.group > 0 && (a.group != 128 || a.cols % 128)) return hipErrorInvalidValue;
  const int64_t nslabs = (a.cols + kSlab - 1) / kSlab;
  const int R = bwd_rows_per_tile(a.rows);
  const int64_t ntiles = (a.rows + R - 1) / R;
  float* rowpart = a.ws;
  float* colpart = a.ws + ((a.cols + 127) / 128) * a.rows * 2;
  dim3 grid((unsigned)nslabs, (unsigned)ntiles);
  if (a.let_mode < OMQ_LET_NONE || a.let_mode > OMQ_LET_MUL || a.col_mode < COL_NONE ||
      a.col_mode > COL_ACT_MUL)
    return hipErrorInvalidValue;
  // every (x dtype, LET mode, column kind) instance
#define OMQ_TILE(XD, L, C)                                                                   \
  if (a.x_dt == XD && a.let_mode == L && a.col_mode == C)                                    \
    hipLaunchKernelGGL((k_rowquant_bwd_tile<XD, L, C>), grid, dim3(kThreads), 0, st, a, R,   \
                       rowpart, colpart);
#define OMQ_TILE_L(XD, L)                                                                    \
  OMQ_TILE(XD, L, COL_NONE) OMQ_TILE(XD, L, COL_WEIGHT) OMQ_TILE(XD, L, COL_ACT_DIV)         \
  OMQ_TILE(XD, L, COL_ACT_MUL)
  OMQ_TILE_L(OMQ_F32, OMQ_LET_NONE) OMQ_TILE_L(OMQ_F32, OMQ_LET_DIV)
  OMQ_TILE_L(OMQ_F32, OMQ_LET_MUL) OMQ_TILE_L(OMQ_BF16, OMQ_LET_NONE)
  OMQ_TILE_L(OMQ_BF16, OMQ_LET_DIV) OMQ_TILE_L(OMQ_BF16, OMQ_LET_MUL)
#undef OMQ_TILE_L
#undef OMQ_TILE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rs = a.group > 0 ? 1 : (int)nslabs;
  if (job) {
    job->rf = a; job->nslabs = rs; job->tile_rows = R; job->ntiles = (int)ntiles;
    job->rowpart = rowpart; job->colpart = colpart;
    job->cols = a.cols; job->col_mode = a.col_mode; job->out0 = a.out0; job->out1 = a.out1;
    job->accumulate = a.accumulate;
    return hipSuccess;
  }
  return launch_ste_finish(a, (int)ntiles, colpart, a, rs, rowpart, R, st);
}

size_t ste_partials_floats(int64_t rows, int64_t cols, int64_t nslabs, int64_t ntiles) {
  return (size_t)(nslabs * rows * 2 + ntiles * 2 * cols) + 64;
}

hipError_t launch_ste_finish(const RowQuantBwd& cf, int ntiles, float* colpart,
                             const RowQuantBwd& rf, int nslabs, const float* rowpart,
                             int tile_rows, hipStream_t st) {
  const hipError_t e = launch_ste_finish_rows(cf, colpart, rf, nslabs, rowpart, tile_rows, st);
  if (e != hipSuccess) return e;
  const bool cols_out = cf.col_mode != COL_NONE && (cf.out0 || cf.out1) && cf.cols > 0;
  if (!cols_out) return hipSuccess;
  hipLaunchKernelGGL(k_ste_cols, dim3((unsigned)((cf.cols + 63) / 64)), dim3(kThreads), 0, st,
                     colpart, ntiles, cf.cols, cf.out0, cf.out1, cf.accumulate);
  return hipGetLastError();
}

hipError_t launch_ste_finish_rows(const RowQuantBwd& cf, float* colpart, const RowQuantBwd& rf,
                                  int nslabs, const float* rowpart, int tile_rows,
                                  hipStream_t st) {
  const bool cols_out = cf.col_mode != COL_NONE && (cf.out0 || cf.out1) && cf.cols > 0;
  const int64_t ng = rf.group > 0 ? rf.cols / 128 : 1;
  const bool rows = rf.nbits < 16 && rf.rows > 0;
  if (tile_rows < 1 || tile_rows > 128) return hipErrorInvalidValue;   // 256 LDS terms
  if (rows) {
    const int merge = cols_out && rf.col_mode != COL_NONE;
    // the tile's rows in one pass: one lane per row when it has one slab, else 8 lanes
    // per row for 128-row tiles, 16 for shorter ones
    const int lpr = nslabs == 1 ? 1 : tile_rows > 64 ? 8 : 16;
    const int nt = std::max(256, (tile_rows * lpr + 63) / 64 * 64);
    const int64_t units = ((rf.rows + tile_rows - 1) / tile_rows) * ng;
    const dim3 grid((unsigned)units), block((unsigned)nt);
    const bool f32 = rf.x_dt == OMQ_F32;
#define OMQ_ROWS(L)                                                                          \
  if (lpr == L) {                                                                            \
    if (f32)                                                                                 \
      hipLaunchKernelGGL((k_ste_rows<OMQ_F32, L>), grid, block, 0, st, rf, nslabs, rowpart,  \
                         tile_rows, colpart, merge);                                         \
    else                                                                                     \
      hipLaunchKernelGGL((k_ste_rows<OMQ_BF16, L>), grid, block, 0, st, rf, nslabs, rowpart, \
                         tile_rows, colpart, merge);                                         \
  }
    OMQ_ROWS(1) OMQ_ROWS(8) OMQ_ROWS(16)
#undef OMQ_ROWS
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_ste_finish_multi(const SteFinJob* jobs, int n, hipStream_t st) {
  if (n < 0 || n > kMaxFinJobs) return hipErrorInvalidValue;
  // row finalizers: the jobs that take one kernel instance (x type, lanes per row)
  // share a launch, up to kMaxRowJobs at a time; jobs are independent, so the
  // launches' order does not matter
  bool done[kMaxFinJobs] = {};
  for (int i = 0; i < n; ++i) {
    const SteFinJob& J = jobs[i];
    if (J.tile_rows < 0 || J.tile_rows > 128) return hipErrorInvalidValue;
    if (!(J.rf.nbits < 16 && J.rf.rows > 0)) done[i] = true;
    else if (J.tile_rows < 1) return hipErrorInvalidValue;
  }
  auto lpr_of = [](const SteFinJob& J) {
    return J.nslabs == 1 ? 1 : J.tile_rows > 64 ? 8 : 16;
  };
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    const int lpr = lpr_of(jobs[i]), xdt = jobs[i].rf.x_dt;
    const int nt = std::max(256, (jobs[i].tile_rows * lpr + 63) / 64 * 64);
    SteRowsJobs rj{};
    int64_t units = 0;
    for (int k = i; k < n && rj.n < kMaxRowJobs; ++k) {
      const SteFinJob& J = jobs[k];
      if (done[k] || lpr_of(J) != lpr || J.rf.x_dt != xdt ||
          std::max(256, (J.tile_rows * lpr + 63) / 64 * 64) != nt)
        continue;
      done[k] = true;
      const RowQuantBwd& rf = J.rf;
      const bool cols_out = J.col_mode != COL_NONE && (J.out0 || J.out1) && J.cols > 0;
      const int64_t ng = rf.group > 0 ? rf.cols / 128 : 1;
      SteRowsJob& r = rj.j[rj.n++];
      r.a = rf; r.rowpart = J.rowpart; r.colpart = J.colpart; r.nslabs = J.nslabs;
      r.tile_rows = J.tile_rows; r.merge = cols_out && rf.col_mode != COL_NONE;
      r.units = (int)(((rf.rows + J.tile_rows - 1) / J.tile_rows) * ng);
      units += r.units;
    }
    const dim3 grid((unsigned)units), block((unsigned)nt);
    const bool f32 = xdt == OMQ_F32;
#define OMQ_ROWS_M(L)                                                                        \
  if (lpr == L) {                                                                            \
    if (f32) hipLaunchKernelGGL((k_ste_rows_multi<OMQ_F32, L>), grid, block, 0, st, rj);     \
    else hipLaunchKernelGGL((k_ste_rows_multi<OMQ_BF16, L>), grid, block, 0, st, rj);        \
  }
    OMQ_ROWS_M(1) OMQ_ROWS_M(8) OMQ_ROWS_M(16)
#undef OMQ_ROWS_M
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // column passes, in rounds: a pass goes to the round after the last earlier pass
  // that shares one of its outputs
  int round[kMaxFinJobs];
  int nround = 0;
  for (int i = 0; i < n; ++i) {
    const SteFinJob& J = jobs[i];
    round[i] = -1;
    const bool cols_out = J.col_mode != COL_NONE && (J.out0 || J.out1) && J.cols > 0;
    if (!cols_out || J.skip_cols) continue;
    int rd = 0;
    for (int k = 0; k < i; ++k) {
      if (round[k] < 0) continue;
      const float* oa[2] = {jobs[k].out0, jobs[k].out1};
      const float* ob[2] = {J.out0, J.out1};
      bool share = false;
      for (const float* x : oa)
        for (const float* y : ob) share = share || (x && x == y);
      if (share) rd = std::max(rd, round[k] + 1);
    }
    round[i] = rd;
    nround = std::max(nround, rd + 1);
  }
  for (int rd = 0; rd < nround; ++rd) {
    SteColsJobs cj{};
    int64_t units = 0;
    for (int i = 0; i < n; ++i) {
      if (round[i] != rd) continue;
      const SteFinJob& J = jobs[i];
      SteColsJob& c = cj.j[cj.n++];
      c.colpart = J.colpart; c.out0 = J.out0; c.out1 = J.out1; c.cols = J.cols;
      c.ntiles = J.ntiles; c.accumulate = J.accumulate; c.units = (int)((J.cols + 63) / 64);
      units += c.units;
    }
    hipLaunchKernelGGL(k_ste_cols_multi, dim3((unsigned)units), dim3(kThreads), 0, st, cj);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_let_elementwise(const void* x, int x_dt, int64_t rows, int64_t cols, int mode,
                                  const float* s, const float* delta, void* y, int y_dt,
                                  hipStream_t st) {
  const int64_t n4 = rows * cols / 4;
  if (n4 == 0) return hipSuccess;
  unsigned blocks = (unsigned)((n4 + kThreads - 1) / kThreads);
  if (blocks > 65536u) blocks = 65536u;
  if (x_dt == OMQ_F32)
    hipLaunchKernelGGL(k_let<OMQ_F32>, dim3(blocks), dim3(kThreads), 0, st, x, rows, cols, mode,
                       s, delta, y, y_dt);
  else
    hipLaunchKernelGGL(k_let<OMQ_BF16>, dim3(blocks), dim3(kThreads), 0, st, x, rows, cols, mode,
                       s, delta, y, y_dt);
  return hipGetLastError();
}

hipError_t launch_bias_fold(const void* W, int w_dt, int64_t rows, int64_t cols,
                            const float* delta, const float* B, float* out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (w_dt == OMQ_F32)
    hipLaunchKernelGGL(k_bias_fold<OMQ_F32>, dim3((unsigned)rows), dim3(kThreads), 0, st, W, rows,
                       cols, delta, B, out);
  else
    hipLaunchKernelGGL(k_bias_fold<OMQ_BF16>, dim3((unsigned)rows), dim3(kThreads), 0, st, W,
                       rows, cols, delta, B, out);
  return hipGetLastError();
}

size_t colsum_ws_bytes(int64_t rows, int64_t cols) {
  return (size_t)(((rows + kColsumRows - 1) / kColsumRows) * cols) * sizeof(float) + 256;
}

hipError_t launch_cvt_bf16_colsum_rope(const float* in, int64_t rows, int64_t cols,
                                       const RopeIn& rp, uint16_t* out, float* colsum, float* ws,
                                       hipStream_t st) {
  if (cols % 8 || rp.qcols % 128 || rp.kcols % 128 || rp.qcols + rp.kcols > cols ||
      rp.ldq % 4 || rp.ldk % 4 || !rp.q || !rp.k || !rp.cos_t || !rp.sin_t)
    return hipErrorInvalidValue;
  if (cols == 0) return hipSuccess;
  const int64_t np = (rows + kColsumRows - 1) / kColsumRows;
  if (np == 0) return colsum ? launch_fill_f32(colsum, cols, 0.f, st) : hipSuccess;
  float* part = colsum ? ws : nullptr;
  const unsigned cb = (unsigned)((cols / 8 + 63) / 64);
  hipLaunchKernelGGL((k_cvt_bf16_colpart<8, true>), dim3(cb, (unsigned)np), dim3(kThreads), 0, st,
                     in, rows, cols, out, part, rp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !colsum) return e;
  return launch_part_colsum(ws, (int)np, 1, cols, colsum, nullptr, 0, st);
}

hipError_t launch_cvt_bf16_colsum(const float* in, int64_t rows, int64_t cols, uint16_t* out,
                                  float* colsum, float* ws, hipStream_t st) {
  if (cols == 0) return hipSuccess;
  const int64_t np = (rows + kColsumRows - 1) / kColsumRows;
  if (np == 0) return colsum ? launch_fill_f32(colsum, cols, 0.f, st) : hipSuccess;
  float* part = colsum ? ws : nullptr;
  if (cols % 8 == 0) {
    const unsigned cb = (unsigned)((cols / 8 + 63) / 64);
    hipLaunchKernelGGL(k_cvt_bf16_colpart<8>, dim3(cb, (unsigned)np), dim3(kThreads), 0, st, in,
                       rows, cols, out, part);
  } else {
    const unsigned cb = (unsigned)((cols + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(k_cvt_bf16_colpart<1>, dim3(cb, (unsigned)np), dim3(kThreads), 0, st, in,
                       rows, cols, out, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !colsum) return e;
  return launch_part_colsum(ws, (int)np, 1, cols, colsum, nullptr, 0, st);
}

hipError_t launch_colsum(const float* in, int64_t rows, int64_t cols, int64_t ld, float* out,
                         float* ws, hipStream_t st) {
  if (cols == 0) return hipSuccess;
  const int64_t np = (rows + kColsumRows - 1) / kColsumRows;
  const unsigned cb = (unsigned)((cols + kThreads - 1) / kThreads);
  if (np == 0) {
    return launch_fill_f32(out, cols, 0.f, st);
  }
  hipLaunchKernelGGL(k_colsum_part, dim3(cb, (unsigned)np), dim3(kThreads), 0, st, in, rows, cols,
                     ld, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_part_colsum(ws, (int)np, 1, cols, out, nullptr, 0, st);
}

}  // namespace omq
