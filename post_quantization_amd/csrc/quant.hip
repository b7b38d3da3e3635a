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

// the block's code sum into *out (every thread of the 4-wave block calls it)
OMQ_DEV void block_qsum(int qs, int32_t* out) {
  __shared__ int s_qs[4];
  qs = wave_sum(qs);
  if ((threadIdx.x & 63) == 0) s_qs[wave_id()] = qs;
  __syncthreads();
  if (threadIdx.x == 0) *out = s_qs[0] + s_qs[1] + s_qs[2] + s_qs[3];
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
  for (int64_t c = (int64_t)tid * 4; c < cols; c += 4 * kThreads) {
    float v[4];
    load4(xr, XDT, c, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float xt = let_x(v[j], a.let_mode, a.s, a.delta, c + j);
      if (xt > vmax || imax == 0x7fffffff) { vmax = xt; imax = (int)(c + j); }
      if (xt < vmin || imin == 0x7fffffff) { vmin = xt; imin = (int)(c + j); }
      if (a.fold_delta) dot = fmaf(a.fold_delta[c + j], v[j], dot);
    }
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
    if (a.amax) a.amax[r] = iM;
    if (a.amin) a.amin[r] = im;
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
      cw |= ((uint32_t)qq) << (8 * j);
      qs += (int)qq;
    }
    store4(a.out, a.out_dt, r * a.ldo + c, o);
    if (a.codes) *reinterpret_cast<uint32_t*>(a.codes + r * cols + c) = cw;
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
    if (a.amax) a.amax[r] = iM;
    if (a.amin) a.amin[r] = im;
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
        cw |= ((uint32_t)qq) << (8 * j);
        qs += (int)qq;
      }
      store4(a.out, a.out_dt, r * a.ldo + c, o);
      if (a.codes) *reinterpret_cast<uint32_t*>(a.codes + r * cols + c) = cw;
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

// Long rows (up to NC * 2048 elements, columns a multiple of 8), one 4-wave block per
// row: each thread keeps NC chunks of 8 consecutive elements in registers (16-byte
// bf16 loads, 2 x 16-byte float32 loads), so HBM sees one read of x and one write of
// x_hat; the LET mode is fixed at compile time and the quotient takes the reciprocal
// product with the exact quotient behind a wave-uniform branch, as in the
// whole-row LDS kernel.  Same results as k_rowquant_fwd_reg.
// RMS: the row is first divided by its root mean square (as the whole-row LDS kernel).
template <int XDT, int NC, int LET, bool RMS = false>
__global__ __launch_bounds__(kThreads) void k_rowquant_fwd_blk8(RowQuantFwd a) {
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  const char* xr = reinterpret_cast<const char*>(a.x) + r * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
  const int64_t cols = a.cols;
  float xt[NC][8];
  float vmax = -FLT_MAX, vmin = FLT_MAX, dot = 0.f;
  int imax = 0x7fffffff, imin = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * kThreads + tid) * 8;
    if (c < cols) {
      float v[8];
      load8(xr, XDT, c, v);
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
    // 1 / rms of the row (block sum of squares), the normalized row stored, then LET
    __shared__ float s_ss[4];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int64_t c = ((int64_t)k * kThreads + tid) * 8;
      if (c < cols) {
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(xt[k][j], xt[k][j], ss);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) s_ss[wid] = ss;
    __syncthreads();
    ss = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
    const float rs = 1.f / sqrtf(ss / (float)cols + a.eps);
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
  // per-thread scan in increasing column order keeps the first index on ties
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * kThreads + tid) * 8;
    if (c < cols) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (xt[k][j] > vmax || imax == 0x7fffffff) { vmax = xt[k][j]; imax = (int)(c + j); }
        if (xt[k][j] < vmin || imin == 0x7fffffff) { vmin = xt[k][j]; imin = (int)(c + j); }
      }
    }
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
    if (a.amax) a.amax[r] = iM;
    if (a.amin) a.amin[r] = im;
    if (a.bias_out) a.bias_out[r] = (a.bias ? a.bias[r] : 0.f) + D;
  }
  // rint(x~ / h) as in the whole-row LDS kernel: reciprocal product, exact quotient
  // for the chunks with an element within the row's bound of a half-integer
  const float rh = 1.f / q.h;
  const float thr = fmaxf(fabsf(M), fabsf(m)) * rh * 0x1p-20f;
  int qs = 0;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * kThreads + tid) * 8;
    const bool in = c < cols;
    float rr[8];
    bool near = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = xt[k][j] * rh;
      rr[j] = rintf(u);
      near |= in && !(fabsf(fabsf(u - rr[j]) - 0.5f) > thr);
    }
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
      if (near) {
#pragma unroll
        for (int j = 0; j < 8; ++j) rr[j] = rintf(xt[k][j] / q.h);
      }
    }
    if (in) {
      float o[8], qq[8];
      uint32_t cw[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qq[j] = __builtin_amdgcn_fmed3f(rr[j] + q.z, 0.f, q.Q);
        o[j] = (qq[j] - q.z) * q.h;
        cw[j >> 2] |= ((uint32_t)qq[j]) << (8 * (j & 3));
        qs += (int)qq[j];
      }
      store8(a.out, a.out_dt, r * a.ldo + c, o);
      if (a.codes) *reinterpret_cast<uint2*>(a.codes + r * cols + c) = make_uint2(cw[0], cw[1]);
    }
  }
  if (a.qsum) block_qsum(qs, a.qsum + r);
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
  wave_argmax(vmax, imax);
  wave_argmin(vmin, imin);
  dot = wave_sum(dot);
  const float gamma = a.a_gamma ? sigmoid_f32(a.a_gamma[r]) : 1.f;
  const float beta = a.a_beta ? sigmoid_f32(a.a_beta[r]) : 1.f;
  const RowQ q = row_step(vmax, vmin, gamma, beta, a.nbits);
  if (lane == 0) {
    if (a.h) a.h[r] = q.h;
    if (a.z) a.z[r] = q.z;
    if (a.amax) a.amax[r] = imax;
    if (a.amin) a.amin[r] = imin;
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
        cw[j >> 2] |= ((uint32_t)qq) << (8 * (j & 3));
        if (j < n) qs += (int)qq;
      }
      store4(a.out, a.out_dt, r * a.ldo + c, o);
      if (a.codes) *reinterpret_cast<uint32_t*>(a.codes + r * cols + c) = cw[0];
      if (FULL || c + 8 <= cols) {
        store4(a.out, a.out_dt, r * a.ldo + c + 4, o + 4);
        if (a.codes) *reinterpret_cast<uint32_t*>(a.codes + r * cols + c + 4) = cw[1];
      }
    }
  }
  if (a.qsum) {
    qs = wave_sum(qs);
    if (lane == 0) a.qsum[r] = qs;
  }
}

// Whole rows (cols = 512 NC), one wave per row, the row staged in LDS: the wave
// copies its row straight from HBM into its own LDS slot, then reads it twice:
// pass 1 forms x~ and its max / min (lowest column among equal values), pass 2
// rounds and stores.  Registers hold one 8-element chunk at a time, so many rows'
// copies are in flight per compute unit.  For fp32 input pass 1 writes x~ back
// over the raw value (the LET division happens once per element).  Same results as
// k_rowquant_fwd_wave.
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
  // the row's 1 / rms: sum of squares over the staged row
  float rs = 1.f;
  if constexpr (RMS) {
    float ss = 0.f;
#pragma unroll 2
    for (int k = 0; k < NC; ++k) {
      if constexpr (XDT == OMQ_F32) {
        const uint4 t0 = my[(2 * k) * 64 + lane], t1 = my[(2 * k + 1) * 64 + lane];
        const uint32_t wv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) ss = fmaf(__uint_as_float(wv[j]), __uint_as_float(wv[j]), ss);
      } else {
        const uint4 t0 = my[k * 64 + lane];
        const uint32_t wv[4] = {t0.x, t0.y, t0.z, t0.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(wv[q] << 16), hi = __uint_as_float(wv[q] & 0xffff0000u);
          ss = fmaf(lo, lo, ss);
          ss = fmaf(hi, hi, ss);
        }
      }
    }
    ss = wave_sum(ss);
    rs = 1.f / sqrtf(ss / (float)a.cols + a.eps);
    if (lane == 0 && a.rstd) a.rstd[r] = rs;
  }
  // x~ of chunk k for this lane (8 consecutive columns c .. c+7)
  auto chunk = [&](int k, float (&xt)[8], float& dot, bool first) {
    const int64_t c = ((int64_t)k * 64 + lane) * 8;
    float v[8];
    if constexpr (XDT == OMQ_F32) {
      const uint4 t0 = my[(2 * k) * 64 + lane], t1 = my[(2 * k + 1) * 64 + lane];
      const uint32_t wv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(wv[j]);
      if (!first) {                                // pass 1 stored x~ itself
#pragma unroll
        for (int j = 0; j < 8; ++j) xt[j] = v[j];
        return;
      }
    } else {
      const uint4 t0 = my[k * 64 + lane];
      const uint32_t wv[4] = {t0.x, t0.y, t0.z, t0.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(wv[q] << 16);
        v[2 * q + 1] = __uint_as_float(wv[q] & 0xffff0000u);
      }
    }
    if constexpr (RMS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * rs;
      if (first) store8(a.rms_out, OMQ_F32, r * a.cols + c, v);
    }
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
    if (first && a.fold_delta) {
      float fv[8];
      load8f(a.fold_delta, c, 8, fv);
#pragma unroll
      for (int j = 0; j < 8; ++j) dot = fmaf(fv[j], v[j], dot);
    }
    if constexpr (XDT == OMQ_F32) {
      if (first) {
        my[(2 * k) * 64 + lane] =
            make_uint4(__float_as_uint(xt[0]), __float_as_uint(xt[1]), __float_as_uint(xt[2]),
                       __float_as_uint(xt[3]));
        my[(2 * k + 1) * 64 + lane] =
            make_uint4(__float_as_uint(xt[4]), __float_as_uint(xt[5]), __float_as_uint(xt[6]),
                       __float_as_uint(xt[7]));
      }
    }
  };
  // pass 1: max / min with the lowest column among equal values (columns are
  // visited in increasing order; chunk 0 seeds the lane's values)
  float vmax, vmin, dot = 0.f;
  int imax, imin;
  {
    float xt[8];
    chunk(0, xt, dot, true);
    vmax = vmin = xt[0];
    imax = imin = lane * 8;
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      if (xt[j] > vmax) { vmax = xt[j]; imax = lane * 8 + j; }
      if (xt[j] < vmin) { vmin = xt[j]; imin = lane * 8 + j; }
    }
  }
  // (two chunks per iteration: unrolling all of them would hoist every chunk's loads
  // and take the registers the occupancy needs)
#pragma unroll 2
  for (int k = 1; k < NC; ++k) {
    float xt[8];
    chunk(k, xt, dot, true);
    const int c = (k * 64 + lane) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (xt[j] > vmax) { vmax = xt[j]; imax = c + j; }
      if (xt[j] < vmin) { vmin = xt[j]; imin = c + j; }
    }
  }
  wave_argmax(vmax, imax);
  wave_argmin(vmin, imin);
  dot = wave_sum(dot);
  const float gamma = lg_g ? sigmoid_f32(lg_g[rl]) : 1.f;
  const float beta = lg_b ? sigmoid_f32(lg_b[rl]) : 1.f;
  const RowQ q = row_step(vmax, vmin, gamma, beta, a.nbits);
  if (lane == 0) {
    if (a.h) a.h[r] = q.h;
    if (a.z) a.z[r] = q.z;
    if (a.amax) a.amax[r] = imax;
    if (a.amin) a.amin[r] = imin;
    if (a.bias_out) a.bias_out[r] = (a.bias ? a.bias[r] : 0.f) + dot;
  }
  // pass 2: rint(x~ / h) by the reciprocal product.  u = x~ rh lies within 3 ulp of
  // the exact quotient, so they can round apart only within |u| 2^-20 of a
  // half-integer; the test uses the row's bound max|x~| rh 2^-20 >= |u| 2^-20 (a few
  // more elements take the exact path, none fewer).  A chunk with such an element (or
  // a non-finite u) takes the exact quotient behind a wave-uniform branch (a
  // divergent one would be flattened into a division for every element).
  const float rh = 1.f / q.h;
  const float thr = fmaxf(fabsf(vmax), fabsf(vmin)) * rh * 0x1p-20f;
  const bool want_codes = a.codes != nullptr;
  int qs = 0;
#pragma unroll 2
  for (int k = 0; k < NC; ++k) {
    const int64_t c = ((int64_t)k * 64 + lane) * 8;
    float xt[8], rr[8];
    chunk(k, xt, dot, false);
    bool near = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float u = xt[j] * rh;
      rr[j] = rintf(u);
      near |= !(fabsf(fabsf(u - rr[j]) - 0.5f) > thr);
    }
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
      if (near) {
#pragma unroll
        for (int j = 0; j < 8; ++j) rr[j] = rintf(xt[j] / q.h);
      }
    }
    float o[8], qq[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qq[j] = __builtin_amdgcn_fmed3f(rr[j] + q.z, 0.f, q.Q);
      o[j] = (qq[j] - q.z) * q.h;
    }
    store8(a.out, a.out_dt, r * a.ldo + c, o);
    if (want_codes) {
      uint32_t cw[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        cw[j >> 2] |= ((uint32_t)qq[j]) << (8 * (j & 3));
        qs += (int)qq[j];
      }
      *reinterpret_cast<uint2*>(a.codes + r * a.cols + c) = make_uint2(cw[0], cw[1]);
    }
  }
  if (a.qsum) {
    qs = wave_sum(qs);
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
    }
  }
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
    if (a.amax) a.amax[p] = imax;
    if (a.amin) a.amin[p] = imin;
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
    cw[j >> 2] |= ((uint32_t)qq) << (8 * (j & 3));
  }
  store4(a.out, a.out_dt, r * a.ldo + c, o);
  store4(a.out, a.out_dt, r * a.ldo + c + 4, o + 4);
  if (a.codes) {
    *reinterpret_cast<uint32_t*>(a.codes + r * a.cols + c) = cw[0];
    *reinterpret_cast<uint32_t*>(a.codes + r * a.cols + c + 4) = cw[1];
  }
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

// row finalize: LPR lanes per quantizer row sum its per-slab partials (coalesced
// reads, then a shuffle reduction), one of them finishes the row: LWC-logit
// gradients and the max/min scatter.
template <int XDT, int LPR>
OMQ_DEV void rows_final(const RowQuantBwd& a, int nslabs, const float* rowpart, int64_t blk) {
  // quantizer rows: rows, or (row, group) pairs p = row * ng + group
  const int64_t ng = a.group > 0 ? a.cols / 128 : 1;
  const int64_t p = (blk * kThreads + threadIdx.x) / LPR;
  const int sub = (int)(threadIdx.x % LPR);
  const bool valid = p < a.rows * ng;
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
  if (!valid || sub != 0) return;
  const int64_t r = p / ng;
  // the row's segment (concatenated weights): its x rows and logits
  const void* xb = a.x;
  const float *lg_g = a.a_gamma, *lg_b = a.a_beta;
  float *gg_g = a.g_agamma, *gg_b = a.g_abeta;
  int64_t rl = r, pl = p;
  if (a.nseg > 1) {
    const int sg = (r >= a.seg_end[0]) + (a.nseg > 2 && r >= a.seg_end[1]);
    const int64_t r0 = sg == 0 ? 0 : a.seg_end[sg - 1];
    xb = a.xseg[sg];
    lg_g = a.agseg[sg]; lg_b = a.abseg[sg]; gg_g = a.gagseg[sg]; gg_b = a.gabseg[sg];
    rl = r - r0;
    pl = p - r0 * ng;
  }
  const char* xr = reinterpret_cast<const char*>(xb) + rl * a.ldx * (XDT == OMQ_F32 ? 4 : 2);
  auto xval = [&](int64_t c) -> float {
    return XDT == OMQ_F32 ? reinterpret_cast<const float*>(xr)[c]
                          : bf16_to_f32(reinterpret_cast<const uint16_t*>(xr)[c]);
  };
  const int iM = a.amax[p], im = a.amin[p];
  const float xM = xval(iM), xm = xval(im);
  const float M = let_x(xM, a.let_mode, a.s, a.delta, iM);
  const float m = let_x(xm, a.let_mode, a.s, a.delta, im);
  const float gamma = lg_g ? sigmoid_f32(lg_g[pl]) : 1.f;
  const float beta = lg_b ? sigmoid_f32(lg_b[pl]) : 1.f;
  const RowQ q = row_step(M, m, gamma, beta, a.nbits);
  const float h = q.h;
  const float gz = -h * gzs;
  const float G = q.floor ? 0.f : gh + gz * q.t2 / (h * h);
  const float gt1 = G / q.Q;
  const float gt2 = -G / q.Q - gz / h;
  const float gM = gt1 * gamma, gm = gt2 * beta;
  if (gg_g) gg_g[pl] = (gt1 * M) * gamma * (1.f - gamma);
  if (gg_b) gg_b[pl] = (gt2 * m) * beta * (1.f - beta);
  // scatter of dL/dmax and dL/dmin into the gradient of x~ at arg_max / arg_min
  const int idx[2] = {iM, im};
  const float gv[2] = {gM, gm};
  const float xo[2] = {xM, xm};
  const float xtl[2] = {M, m};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int c = idx[e];
    const float gsc = gv[e];
    if (a.gx) {
      float up = gsc;
      if (a.let_mode == OMQ_LET_DIV) up = gsc / a.s[c];
      else if (a.let_mode == OMQ_LET_MUL) up = gsc * a.s[c];
      a.gx[r * a.ldgx + c] += up;
    }
    switch (a.col_mode) {
      case COL_WEIGHT:
        if (a.out0) atomicAdd(a.out0 + c, gsc * xo[e]);
        break;
      case COL_ACT_DIV:
        if (a.out0) atomicAdd(a.out0 + c, gsc * (-xtl[e] / a.s[c]));
        if (a.out1) atomicAdd(a.out1 + c, gsc * (-1.f / a.s[c]));
        break;
      case COL_ACT_MUL:
        if (a.out0) atomicAdd(a.out0 + c, gsc * xo[e]);
        break;
      default:
        break;
    }
  }
}

template <int XDT, int LPR>
__global__ __launch_bounds__(kThreads) void k_rowquant_bwd_rows(RowQuantBwd a, int nslabs,
                                                                const float* rowpart) {
  rows_final<XDT, LPR>(a, nslabs, rowpart, blockIdx.x);
}

// Both second stages of a straight-through GEMM epilogue in one launch: workgroups
// [0, ncb) sum the column partials of 64 columns each (4 waves over the partial
// rows, the wave sums added in LDS in a fixed order) and add the totals to out0 /
// out1 atomically, since the row finalizers of the other workgroups scatter into the
// same vectors meanwhile; the rest finish the quantizer rows as k_rowquant_bwd_rows.
template <int XDT, int LPR>
__global__ __launch_bounds__(kThreads) void k_ste_final(RowQuantBwd cf, int ntiles,
                                                        const float* colpart, int ncb,
                                                        RowQuantBwd rf, int nslabs,
                                                        const float* rowpart) {
  __shared__ float red[2][4][64];
  if ((int)blockIdx.x >= ncb) {
    rows_final<XDT, LPR>(rf, nslabs, rowpart, (int64_t)blockIdx.x - ncb);
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id();
  const int64_t cols = cf.cols, c = (int64_t)blockIdx.x * 64 + lane;
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
    float* o = w == 0 ? cf.out0 : cf.out1;
    if (o) atomicAdd(o + c, ((red[w][0][lane] + red[w][1][lane]) + red[w][2][lane]) + red[w][3][lane]);
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
// fixed order.  VEC 1: one column per thread over the chunk.
template <int VEC>
__global__ __launch_bounds__(kThreads) void k_cvt_bf16_colpart(const float* __restrict__ in,
                                                               int64_t rows, int64_t cols,
                                                               uint16_t* __restrict__ out,
                                                               float* __restrict__ part) {
  const int64_t r0 = (int64_t)blockIdx.y * kColsumRows;
  const int64_t r1 = min(r0 + kColsumRows, rows);
  if constexpr (VEC == 8) {
    __shared__ float4 red[4][2][64];
    const int lane = threadIdx.x & 63, w = wave_id();
    const int64_t c = ((int64_t)blockIdx.x * 64 + lane) * 8;
    const bool ok = c < cols;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ok) {
#pragma unroll 4
      for (int64_t r = r0 + w; r < r1; r += 4) {
        const float* p = in + r * cols + c;
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
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
#define OMQ_FWD_LDS(N)                                                                        \
  if (a.let_mode == OMQ_LET_DIV)                                                              \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_DIV>), grid, dim3(kThreads), 0, st, \
                       a);                                                                    \
  else if (a.let_mode == OMQ_LET_MUL)                                                         \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_MUL>), grid, dim3(kThreads), 0, st, \
                       a);                                                                    \
  else                                                                                        \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_NONE>), grid, dim3(kThreads), 0, st,\
                       a);
#define OMQ_FWD_RMS(N)                                                                        \
  if (a.let_mode == OMQ_LET_DIV)                                                              \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_DIV, true>), grid, dim3(kThreads), \
                       0, st, a);                                                             \
  else                                                                                        \
    hipLaunchKernelGGL((k_rowquant_fwd_lds<XDT, N, OMQ_LET_NONE, true>), grid, dim3(kThreads),\
                       0, st, a);
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
  // code sums come with the codes, per whole row
  if (a.qsum && (!a.codes || a.group > 0 || a.nbits >= 16)) return hipErrorInvalidValue;
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
  // column sums added to running totals: one launch with the row finalizers
  if (a.accumulate) return launch_ste_final(a, (int)ntiles, colpart, a, rs, rowpart, st);
  e = launch_ste_colfinal(a, (int)ntiles, colpart, st);
  if (e != hipSuccess) return e;
  return launch_ste_rowfinal(a, rs, rowpart, st);
}

size_t ste_partials_floats(int64_t rows, int64_t cols, int64_t nslabs, int64_t ntiles) {
  return (size_t)(nslabs * rows * 2 + ntiles * 2 * cols) + 64;
}

hipError_t launch_ste_colfinal(const RowQuantBwd& a, int ntiles, float* colpart,
                               hipStream_t st) {
  if (a.col_mode == COL_NONE || !(a.out0 || a.out1)) return hipSuccess;
  return launch_part_colsum(colpart, ntiles, 2, a.cols, a.out0, a.out1, a.accumulate, st);
}

hipError_t launch_ste_final(const RowQuantBwd& cf, int ntiles, const float* colpart,
                           const RowQuantBwd& rf, int nslabs, const float* rowpart,
                           hipStream_t st) {
  const int ncb = (cf.col_mode != COL_NONE && (cf.out0 || cf.out1) && cf.cols > 0)
                      ? (int)((cf.cols + 63) / 64) : 0;
  const int lpr = nslabs == 1 ? 1 : 16;
  const int64_t n = (rf.nbits < 16 && rf.rows > 0) ? rf.rows * (rf.group > 0 ? rf.cols / 128 : 1)
                                                   : 0;
  const int64_t nrb = (n * lpr + kThreads - 1) / kThreads;
  if (ncb + nrb == 0) return hipSuccess;
  const dim3 grid((unsigned)(ncb + nrb));
  const bool f32 = rf.x_dt == OMQ_F32;
  if (lpr == 1) {
    if (f32)
      hipLaunchKernelGGL((k_ste_final<OMQ_F32, 1>), grid, dim3(kThreads), 0, st, cf, ntiles,
                         colpart, ncb, rf, nslabs, rowpart);
    else
      hipLaunchKernelGGL((k_ste_final<OMQ_BF16, 1>), grid, dim3(kThreads), 0, st, cf, ntiles,
                         colpart, ncb, rf, nslabs, rowpart);
  } else {
    if (f32)
      hipLaunchKernelGGL((k_ste_final<OMQ_F32, 16>), grid, dim3(kThreads), 0, st, cf, ntiles,
                         colpart, ncb, rf, nslabs, rowpart);
    else
      hipLaunchKernelGGL((k_ste_final<OMQ_BF16, 16>), grid, dim3(kThreads), 0, st, cf, ntiles,
                         colpart, ncb, rf, nslabs, rowpart);
  }
  return hipGetLastError();
}

hipError_t launch_ste_rowfinal(const RowQuantBwd& a, int nslabs, const float* rowpart,
                               hipStream_t st) {
  hipError_t e = hipSuccess;
  if (a.nbits < 16 && a.rows > 0) {
    const int64_t n = a.rows * (a.group > 0 ? a.cols / 128 : 1);
    // one slab per row: a lane per row; else 16 lanes share a row's slabs
    if (nslabs == 1) {
      dim3 g2((unsigned)((n + kThreads - 1) / kThreads));
      if (a.x_dt == OMQ_F32)
        hipLaunchKernelGGL((k_rowquant_bwd_rows<OMQ_F32, 1>), g2, dim3(kThreads), 0, st, a,
                           (int)nslabs, rowpart);
      else
        hipLaunchKernelGGL((k_rowquant_bwd_rows<OMQ_BF16, 1>), g2, dim3(kThreads), 0, st, a,
                           (int)nslabs, rowpart);
    } else {
      dim3 g2((unsigned)((n * 16 + kThreads - 1) / kThreads));
      if (a.x_dt == OMQ_F32)
        hipLaunchKernelGGL((k_rowquant_bwd_rows<OMQ_F32, 16>), g2, dim3(kThreads), 0, st, a,
                           (int)nslabs, rowpart);
      else
        hipLaunchKernelGGL((k_rowquant_bwd_rows<OMQ_BF16, 16>), g2, dim3(kThreads), 0, st, a,
                           (int)nslabs, rowpart);
    }
    e = hipGetLastError();
  }
  return e;
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
