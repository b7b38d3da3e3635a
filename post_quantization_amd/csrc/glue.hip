// Block glue around the quantized linears: RMSNorm, RoPE, SiLU gating, the MSE
// objective (paper reading, section "框架": block output reconstruction), the
// grouped-head broadcasts of the LET parameters, and the parameter updates
// (section "实验证据": AdamW, zero weight decay).
#include "common.h"
#include "kernels.h"

#include <float.h>
#include <math.h>

namespace omq {

namespace {

constexpr int kThreads = 256;

template <typename T>
OMQ_DEV T block_sum(T v, T* sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = wave_id();
  __syncthreads();
  if (lane == 0) sh[wid] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

template <int XDT>
__global__ __launch_bounds__(kThreads) void k_rmsnorm(const void* x, int64_t d, float eps,
                                                      float* y, float* rstd) {
  const int64_t r = blockIdx.x;
  const char* xr = reinterpret_cast<const char*>(x) + r * d * (XDT == OMQ_F32 ? 4 : 2);
  __shared__ double sh[4];
  double ss = 0.0;
  for (int64_t c = (int64_t)threadIdx.x * 4; c < d; c += 4 * kThreads) {
    float v[4];
    load4(xr, XDT, c, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) ss = fma((double)v[j], (double)v[j], ss);
  }
  ss = block_sum(ss, sh);
  const float rs = rms_scale(ss, d, eps);
  if (threadIdx.x == 0 && rstd) rstd[r] = rs;
  for (int64_t c = (int64_t)threadIdx.x * 4; c < d; c += 4 * kThreads) {
    float v[4];
    load4(xr, XDT, c, v);
    *reinterpret_cast<float4*>(y + r * d + c) =
        make_float4(v[0] * rs, v[1] * rs, v[2] * rs, v[3] * rs);
  }
}

// gx = rstd * gy - x * (rstd^3 * sum(gy * x) / d)  (+ add)
__global__ __launch_bounds__(kThreads) void k_rmsnorm_bwd(const float* gy, const float* x,
                                                          const float* rstd, int64_t d,
                                                          const float* add, float* gx) {
  const int64_t r = blockIdx.x;
  __shared__ float sh[4];
  float dot = 0.f;
  for (int64_t c = (int64_t)threadIdx.x * 4; c < d; c += 4 * kThreads) {
    const float4 a = *reinterpret_cast<const float4*>(gy + r * d + c);
    const float4 b = *reinterpret_cast<const float4*>(x + r * d + c);
    dot = fmaf(a.x, b.x, dot); dot = fmaf(a.y, b.y, dot);
    dot = fmaf(a.z, b.z, dot); dot = fmaf(a.w, b.w, dot);
  }
  dot = block_sum(dot, sh);
  const float rs = rstd[r];
  const float k = rs * rs * rs * dot / (float)d;
  for (int64_t c = (int64_t)threadIdx.x * 4; c < d; c += 4 * kThreads) {
    const float4 a = *reinterpret_cast<const float4*>(gy + r * d + c);
    const float4 b = *reinterpret_cast<const float4*>(x + r * d + c);
    float4 o = make_float4(rs * a.x - b.x * k, rs * a.y - b.y * k, rs * a.z - b.z * k,
                           rs * a.w - b.w * k);
    if (add) {
      const float4 e = *reinterpret_cast<const float4*>(add + r * d + c);
      o.x += e.x; o.y += e.y; o.z += e.z; o.w += e.w;
    }
    *reinterpret_cast<float4*>(gx + r * d + c) = o;
  }
}

__global__ void k_rope_tables(int64_t T, int64_t hd, float theta, float* cos_t, float* sin_t) {
  const int64_t half = hd / 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * half) return;
  const int64_t t = i / half, k = i % half;
  const double inv = pow((double)theta, -2.0 * (double)k / (double)hd);
  const double ang = (double)t * inv;
  cos_t[i] = (float)cos(ang);
  sin_t[i] = (float)sin(ang);
}

// rotate-half RoPE per head; inverse applies the transposed rotation
__global__ __launch_bounds__(kThreads) void k_rope(const float* x, int64_t ldx, int64_t T,
                                                   int64_t n_heads, int64_t hd,
                                                   const float* cos_t, const float* sin_t,
                                                   int inverse, float* y, int64_t ldy) {
  const int64_t half = hd / 2;
  const int64_t n = T * n_heads * half;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t k = i % half;
    const int64_t hh = (i / half) % n_heads;
    const int64_t t = i / (half * n_heads);
    const float c = cos_t[t * half + k], s = sin_t[t * half + k];
    const float a = x[t * ldx + hh * hd + k], b = x[t * ldx + hh * hd + k + half];
    float ya, yb;
    if (!inverse) { ya = a * c - b * s; yb = b * c + a * s; }
    else { ya = a * c + b * s; yb = b * c - a * s; }
    y[t * ldy + hh * hd + k] = ya;
    y[t * ldy + hh * hd + k + half] = yb;
  }
}

OMQ_DEV float sigmoidf_(float x) { return 1.f / (1.f + expf(-x)); }

// Row-parallel forms of the elementwise kernels below: blockIdx.y is the token,
// each thread takes 4 consecutive columns with 16-byte accesses (the launchers use
// them when the widths and strides are multiples of 4 and the pointers 16-byte
// aligned); the per-element arithmetic is the same.
__global__ __launch_bounds__(kThreads) void k_rope4(const float* __restrict__ x, int64_t ldx,
                                                    int n_heads, int hd,
                                                    const float* __restrict__ cos_t,
                                                    const float* __restrict__ sin_t, int inverse,
                                                    float* __restrict__ y, int64_t ldy) {
  const int half = hd / 2;
  const int j = (blockIdx.x * kThreads + threadIdx.x) * 4;   // over n_heads * half
  if (j >= n_heads * half) return;
  const int64_t t = blockIdx.y;
  const int hh = j / half, k = j % half;
  const float4 c = *reinterpret_cast<const float4*>(cos_t + t * half + k);
  const float4 s = *reinterpret_cast<const float4*>(sin_t + t * half + k);
  const float* xr = x + t * ldx + (int64_t)hh * hd + k;
  const float4 a = *reinterpret_cast<const float4*>(xr);
  const float4 b = *reinterpret_cast<const float4*>(xr + half);
  float4 ya, yb;
  if (!inverse) {
    ya = make_float4(a.x * c.x - b.x * s.x, a.y * c.y - b.y * s.y, a.z * c.z - b.z * s.z,
                     a.w * c.w - b.w * s.w);
    yb = make_float4(b.x * c.x + a.x * s.x, b.y * c.y + a.y * s.y, b.z * c.z + a.z * s.z,
                     b.w * c.w + a.w * s.w);
  } else {
    ya = make_float4(a.x * c.x + b.x * s.x, a.y * c.y + b.y * s.y, a.z * c.z + b.z * s.z,
                     a.w * c.w + b.w * s.w);
    yb = make_float4(b.x * c.x - a.x * s.x, b.y * c.y - a.y * s.y, b.z * c.z - a.z * s.z,
                     b.w * c.w - a.w * s.w);
  }
  float* yr = y + t * ldy + (int64_t)hh * hd + k;
  *reinterpret_cast<float4*>(yr) = ya;
  *reinterpret_cast<float4*>(yr + half) = yb;
}

// Two RoPE operands in one launch (Q and K heads of one token row): heads [0, n0) of
// the first, then n1 heads of the second; the per-element arithmetic is k_rope4's.
struct RopeSeg {
  const float* x; int64_t ldx; float* y; int64_t ldy; int n;
};
__global__ __launch_bounds__(kThreads) void k_rope4x2(RopeSeg s0, RopeSeg s1, int hd,
                                                      const float* __restrict__ cos_t,
                                                      const float* __restrict__ sin_t,
                                                      int inverse) {
  const int half = hd / 2;
  const int j = (blockIdx.x * kThreads + threadIdx.x) * 4;   // over (n0 + n1) * half
  if (j >= (s0.n + s1.n) * half) return;
  const int64_t t = blockIdx.y;
  const int hg = j / half, k = j % half;
  const bool second = hg >= s0.n;
  const int hh = second ? hg - s0.n : hg;
  const float* x = second ? s1.x : s0.x;
  const int64_t ldx = second ? s1.ldx : s0.ldx;
  float* y = second ? s1.y : s0.y;
  const int64_t ldy = second ? s1.ldy : s0.ldy;
  const float4 c = *reinterpret_cast<const float4*>(cos_t + t * half + k);
  const float4 s = *reinterpret_cast<const float4*>(sin_t + t * half + k);
  const float* xr = x + t * ldx + (int64_t)hh * hd + k;
  const float4 a = *reinterpret_cast<const float4*>(xr);
  const float4 b = *reinterpret_cast<const float4*>(xr + half);
  float4 ya, yb;
  if (!inverse) {
    ya = make_float4(a.x * c.x - b.x * s.x, a.y * c.y - b.y * s.y, a.z * c.z - b.z * s.z,
                     a.w * c.w - b.w * s.w);
    yb = make_float4(b.x * c.x + a.x * s.x, b.y * c.y + a.y * s.y, b.z * c.z + a.z * s.z,
                     b.w * c.w + a.w * s.w);
  } else {
    ya = make_float4(a.x * c.x + b.x * s.x, a.y * c.y + b.y * s.y, a.z * c.z + b.z * s.z,
                     a.w * c.w + b.w * s.w);
    yb = make_float4(b.x * c.x - a.x * s.x, b.y * c.y - a.y * s.y, b.z * c.z - a.z * s.z,
                     b.w * c.w - a.w * s.w);
  }
  float* yr = y + t * ldy + (int64_t)hh * hd + k;
  *reinterpret_cast<float4*>(yr) = ya;
  *reinterpret_cast<float4*>(yr + half) = yb;
}

__global__ __launch_bounds__(kThreads) void k_silu_gate4(const float* __restrict__ gu, int64_t F,
                                                         float* __restrict__ a) {
  const int64_t f = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (f >= F) return;
  const int64_t t = blockIdx.y;
  const float4 g = *reinterpret_cast<const float4*>(gu + t * 2 * F + f);
  const float4 u = *reinterpret_cast<const float4*>(gu + t * 2 * F + F + f);
  *reinterpret_cast<float4*>(a + t * F + f) =
      make_float4(g.x * sigmoidf_(g.x) * u.x, g.y * sigmoidf_(g.y) * u.y,
                  g.z * sigmoidf_(g.z) * u.z, g.w * sigmoidf_(g.w) * u.w);
}

__global__ __launch_bounds__(kThreads) void k_silu_gate_bwd4(const float* __restrict__ gu,
                                                             const float* __restrict__ ga,
                                                             int64_t F, float* __restrict__ ggu) {
  const int64_t f = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4;
  if (f >= F) return;
  const int64_t t = blockIdx.y;
  const float4 g4 = *reinterpret_cast<const float4*>(gu + t * 2 * F + f);
  const float4 u4 = *reinterpret_cast<const float4*>(gu + t * 2 * F + F + f);
  const float4 d4 = *reinterpret_cast<const float4*>(ga + t * F + f);
  const float g[4] = {g4.x, g4.y, g4.z, g4.w}, u[4] = {u4.x, u4.y, u4.z, u4.w};
  const float d[4] = {d4.x, d4.y, d4.z, d4.w};
  float og[4], ou[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float sg = sigmoidf_(g[e]);
    og[e] = d[e] * u[e] * sg * (1.f + g[e] * (1.f - sg));
    ou[e] = d[e] * g[e] * sg;
  }
  *reinterpret_cast<float4*>(ggu + t * 2 * F + f) = make_float4(og[0], og[1], og[2], og[3]);
  *reinterpret_cast<float4*>(ggu + t * 2 * F + F + f) = make_float4(ou[0], ou[1], ou[2], ou[3]);
}

// The gate/up gradient as the bf16 operand of the backward products, with the
// column sums of each kColsumRows-row chunk (the bias-fold gradient needs the
// column sums of dL/d(gate|up)).  A workgroup takes 256 columns of each half (4
// per lane: the same 4 of the gate and of the up half) over one chunk; its 4 waves
// take the chunk's rows in turn and their sums are added in LDS in a fixed order.
__global__ __launch_bounds__(kThreads) void k_silu_gate_bwd_bf16(const float* __restrict__ gu,
                                                                 const float* __restrict__ ga,
                                                                 int64_t T, int64_t F,
                                                                 uint16_t* __restrict__ ggub,
                                                                 float* __restrict__ part) {
  __shared__ float4 red[4][2][64];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int64_t f = ((int64_t)blockIdx.x * 64 + lane) * 4;
  const bool ok = f < F;
  const int64_t r0 = (int64_t)blockIdx.y * kColsumRows;
  const int64_t r1 = min(r0 + kColsumRows, T);
  float sg_[4] = {0.f, 0.f, 0.f, 0.f}, su_[4] = {0.f, 0.f, 0.f, 0.f};
  if (ok) {
#pragma unroll 2
    for (int64_t t = r0 + w; t < r1; t += 4) {
      const float4 g4 = *reinterpret_cast<const float4*>(gu + t * 2 * F + f);
      const float4 u4 = *reinterpret_cast<const float4*>(gu + t * 2 * F + F + f);
      const float4 d4 = *reinterpret_cast<const float4*>(ga + t * F + f);
      const float g[4] = {g4.x, g4.y, g4.z, g4.w}, u[4] = {u4.x, u4.y, u4.z, u4.w};
      const float d[4] = {d4.x, d4.y, d4.z, d4.w};
      float og[4], ou[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sg = sigmoidf_(g[e]);
        og[e] = d[e] * u[e] * sg * (1.f + g[e] * (1.f - sg));
        ou[e] = d[e] * g[e] * sg;
        sg_[e] += og[e];
        su_[e] += ou[e];
      }
      *reinterpret_cast<uint2*>(ggub + t * 2 * F + f) =
          make_uint2(pack_bf16(og[0], og[1]), pack_bf16(og[2], og[3]));
      *reinterpret_cast<uint2*>(ggub + t * 2 * F + F + f) =
          make_uint2(pack_bf16(ou[0], ou[1]), pack_bf16(ou[2], ou[3]));
    }
  }
  red[w][0][lane] = make_float4(sg_[0], sg_[1], sg_[2], sg_[3]);
  red[w][1][lane] = make_float4(su_[0], su_[1], su_[2], su_[3]);
  __syncthreads();
  if (w < 2 && ok) {
    float4 acc = red[0][w][lane];
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      const float4 v = red[q][w][lane];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4*>(part + (int64_t)blockIdx.y * 2 * F + w * F + f) = acc;
  }
}

__global__ __launch_bounds__(kThreads) void k_silu_gate(const float* gu, int64_t T, int64_t F,
                                                        float* a) {
  const int64_t n = T * F;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t t = i / F, f = i % F;
    const float g = gu[t * 2 * F + f], u = gu[t * 2 * F + F + f];
    a[i] = g * sigmoidf_(g) * u;
  }
}

__global__ __launch_bounds__(kThreads) void k_silu_gate_bwd(const float* gu, const float* ga,
                                                            int64_t T, int64_t F, float* ggu) {
  const int64_t n = T * F;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t t = i / F, f = i % F;
    const float g = gu[t * 2 * F + f], u = gu[t * 2 * F + F + f];
    const float sg = sigmoidf_(g);
    const float d = ga[i];
    ggu[t * 2 * F + f] = d * u * sg * (1.f + g * (1.f - sg));
    ggu[t * 2 * F + F + f] = d * g * sg;
  }
}

constexpr int kMseBlocks = 1024;

__global__ __launch_bounds__(kThreads) void k_mse_part(const float* y, const float* t, int64_t n,
                                                       float* dy, float* part) {
  __shared__ float sh[4];
  float s = 0.f;
  const float sc = 2.f / (float)n;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const float d = y[i] - t[i];
    s = fmaf(d, d, s);
    if (dy) dy[i] = sc * d;
  }
  s = block_sum(s, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// four elements per thread (16-byte loads and stores); dyb, when set, receives dy
// in bf16 as well (the next product's operand)
__global__ __launch_bounds__(kThreads) void k_mse_part4(const float* __restrict__ y,
                                                        const float* __restrict__ t, int64_t n,
                                                        float* __restrict__ dy,
                                                        uint16_t* __restrict__ dyb,
                                                        float* __restrict__ part) {
  __shared__ float sh[4];
  float s = 0.f;
  const float sc = 2.f / (float)n;
  for (int64_t i = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 4; i < n;
       i += (int64_t)gridDim.x * kThreads * 4) {
    const float4 a = *reinterpret_cast<const float4*>(y + i);
    const float4 b = *reinterpret_cast<const float4*>(t + i);
    const float d[4] = {a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) s = fmaf(d[j], d[j], s);
    const float g[4] = {sc * d[0], sc * d[1], sc * d[2], sc * d[3]};
    if (dy) *reinterpret_cast<float4*>(dy + i) = make_float4(g[0], g[1], g[2], g[3]);
    if (dyb)
      *reinterpret_cast<uint2*>(dyb + i) = make_uint2(pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3]));
  }
  s = block_sum(s, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void k_mse_final(const float* part, int np, int64_t n,
                                                        float* loss) {
  __shared__ float sh[4];
  float s = 0.f;
  for (int i = threadIdx.x; i < np; i += kThreads) s += part[i];
  s = block_sum(s, sh);
  if (threadIdx.x == 0) *loss = s / (float)n;
}

__global__ void k_kv_expand(const float* v, int64_t n_q, int64_t n_kv, int64_t hd, float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_q * hd) return;
  const int64_t grp = n_q / n_kv;
  const int64_t h = i / hd, k = i % hd;
  out[i] = v[(h / grp) * hd + k];
}

__global__ void k_kv_reduce_add(const float* v, int64_t n_q, int64_t n_kv, int64_t hd,
                                float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_kv * hd) return;
  const int64_t grp = n_q / n_kv;
  const int64_t g = i / hd, k = i % hd;
  float s = 0.f;
  for (int64_t r = 0; r < grp; ++r) s += v[(g * grp + r) * hd + k];
  out[i] += s;
}

__global__ __launch_bounds__(kThreads) void k_adamw(float* th, const float* g, float* m, float* v,
                                                    int64_t n, int64_t n_lwc, float lr_lwc,
                                                    float lr_let, float b1, float b2, float eps,
                                                    float wd, float c1, float c2) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const float lr = i < n_lwc ? lr_lwc : lr_let;
  const float gi = g[i];
  const float mi = b1 * m[i] + (1.f - b1) * gi;
  const float vi = b2 * v[i] + (1.f - b2) * gi * gi;
  m[i] = mi;
  v[i] = vi;
  const float mh = mi / c1, vh = vi / c2;
  th[i] = th[i] * (1.f - lr * wd) - lr * mh / (sqrtf(vh) + eps);
}

__global__ __launch_bounds__(kThreads) void k_sgd(float* th, const float* g, int64_t n,
                                                  int64_t n_lwc, float lr_lwc, float lr_let) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  th[i] -= (i < n_lwc ? lr_lwc : lr_let) * g[i];
}

__global__ __launch_bounds__(kThreads) void k_axpy(float* y, const float* x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) y[i] += x[i];
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + kThreads - 1) / kThreads;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, int x_dt, int64_t T, int64_t d, float eps, float* y,
                          float* rstd, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (x_dt == OMQ_F32)
    hipLaunchKernelGGL(k_rmsnorm<OMQ_F32>, dim3((unsigned)T), dim3(kThreads), 0, st, x, d, eps, y,
                       rstd);
  else
    hipLaunchKernelGGL(k_rmsnorm<OMQ_BF16>, dim3((unsigned)T), dim3(kThreads), 0, st, x, d, eps,
                       y, rstd);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const float* gy, const float* x, const float* rstd, int64_t T,
                              int64_t d, const float* add, float* gx, hipStream_t st) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm_bwd, dim3((unsigned)T), dim3(kThreads), 0, st, gy, x, rstd, d, add,
                     gx);
  return hipGetLastError();
}

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

hipError_t launch_rope_tables(int64_t T, int64_t hd, float theta, float* cos_t, float* sin_t,
                              hipStream_t st) {
  const int64_t n = T * (hd / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_tables, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, T, hd,
                     theta, cos_t, sin_t);
  return hipGetLastError();
}

hipError_t launch_rope(const float* x, int64_t ldx, int64_t T, int64_t n_heads, int64_t hd,
                       const float* cos_t, const float* sin_t, int inverse, float* y, int64_t ldy,
                       hipStream_t st) {
  const int64_t n = T * n_heads * (hd / 2);
  if (n == 0) return hipSuccess;
  if ((hd / 2) % 4 == 0 && ldx % 4 == 0 && ldy % 4 == 0 && al16(x) && al16(y) && al16(cos_t) &&
      al16(sin_t) && T < 65536) {
    const int64_t w = n_heads * (hd / 2) / 4;
    hipLaunchKernelGGL(k_rope4, dim3((unsigned)((w + kThreads - 1) / kThreads), (unsigned)T),
                       dim3(kThreads), 0, st, x, ldx, (int)n_heads, (int)hd, cos_t, sin_t, inverse,
                       y, ldy);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_rope, dim3(grid_for(n)), dim3(kThreads), 0, st, x, ldx, T, n_heads, hd,
                     cos_t, sin_t, inverse, y, ldy);
  return hipGetLastError();
}

// a float32 buffer set to one value: a kernel rather than a memset, so the
// calls stay valid inside a captured graph
__global__ __launch_bounds__(kThreads) void k_fill_f32(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = v;
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)blocks), dim3(kThreads), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_rope2(const float* x0, int64_t ldx0, float* y0, int64_t ldy0, int64_t n0,
                        const float* x1, int64_t ldx1, float* y1, int64_t ldy1, int64_t n1,
                        int64_t T, int64_t hd, const float* cos_t, const float* sin_t,
                        int inverse, hipStream_t st) {
  const bool vec = (hd / 2) % 4 == 0 && ldx0 % 4 == 0 && ldy0 % 4 == 0 && ldx1 % 4 == 0 &&
                   ldy1 % 4 == 0 && al16(x0) && al16(y0) && al16(x1) && al16(y1) &&
                   al16(cos_t) && al16(sin_t) && T < 65536 && (n0 + n1) * hd < (1 << 30);
  if (!vec) {
    hipError_t e = launch_rope(x0, ldx0, T, n0, hd, cos_t, sin_t, inverse, y0, ldy0, st);
    if (e != hipSuccess) return e;
    return launch_rope(x1, ldx1, T, n1, hd, cos_t, sin_t, inverse, y1, ldy1, st);
  }
  if (T == 0 || n0 + n1 == 0) return hipSuccess;
  const RopeSeg s0{x0, ldx0, y0, ldy0, (int)n0}, s1{x1, ldx1, y1, ldy1, (int)n1};
  const int64_t w = (n0 + n1) * (hd / 2) / 4;
  hipLaunchKernelGGL(k_rope4x2, dim3((unsigned)((w + kThreads - 1) / kThreads), (unsigned)T),
                     dim3(kThreads), 0, st, s0, s1, (int)hd, cos_t, sin_t, inverse);
  return hipGetLastError();
}

hipError_t launch_silu_gate(const float* gu, int64_t T, int64_t F, float* a, hipStream_t st) {
  if (T * F == 0) return hipSuccess;
  if (F % 4 == 0 && al16(gu) && al16(a) && T < 65536) {
    hipLaunchKernelGGL(k_silu_gate4, dim3((unsigned)((F / 4 + kThreads - 1) / kThreads), (unsigned)T),
                       dim3(kThreads), 0, st, gu, F, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_silu_gate, dim3(grid_for(T * F)), dim3(kThreads), 0, st, gu, T, F, a);
  return hipGetLastError();
}

hipError_t launch_silu_gate_bwd(const float* gu, const float* ga, int64_t T, int64_t F,
                                float* ggu, hipStream_t st) {
  if (T * F == 0) return hipSuccess;
  if (F % 4 == 0 && al16(gu) && al16(ga) && al16(ggu) && T < 65536) {
    hipLaunchKernelGGL(k_silu_gate_bwd4,
                       dim3((unsigned)((F / 4 + kThreads - 1) / kThreads), (unsigned)T),
                       dim3(kThreads), 0, st, gu, ga, F, ggu);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_silu_gate_bwd, dim3(grid_for(T * F)), dim3(kThreads), 0, st, gu, ga, T, F,
                     ggu);
  return hipGetLastError();
}

bool silu_gate_bwd_bf16_fits(const float* gu, const float* ga, int64_t T, int64_t F,
                             const uint16_t* ggub) {
  return F % 4 == 0 && al16(gu) && al16(ga) && (reinterpret_cast<uintptr_t>(ggub) & 7) == 0 &&
         T > 0 && (T + kColsumRows - 1) / kColsumRows < 65536;
}

hipError_t launch_silu_gate_bwd_bf16(const float* gu, const float* ga, int64_t T, int64_t F,
                                     uint16_t* ggub, float* colsum, float* ws, hipStream_t st) {
  if (!silu_gate_bwd_bf16_fits(gu, ga, T, F, ggub)) return hipErrorInvalidValue;
  const int64_t np = (T + kColsumRows - 1) / kColsumRows;
  hipLaunchKernelGGL(k_silu_gate_bwd_bf16, dim3((unsigned)((F / 4 + 63) / 64), (unsigned)np),
                     dim3(kThreads), 0, st, gu, ga, T, F, ggub, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_part_colsum(ws, (int)np, 1, 2 * F, colsum, nullptr, 0, st);
}

hipError_t launch_mse(const float* y, const float* target, int64_t n, float* loss, float* dy,
                      float* ws, hipStream_t st, uint16_t* dyb) {
  const bool v4 = n % 4 == 0 && al16(y) && al16(target) && (!dy || al16(dy)) &&
                  (reinterpret_cast<uintptr_t>(dyb) & 7) == 0;
  if (dyb && !v4) return hipErrorInvalidValue;
  const int nb = (int)std::min<int64_t>(kMseBlocks, (n + kThreads * (v4 ? 4 : 1) - 1) /
                                                        (kThreads * (v4 ? 4 : 1)));
  if (nb == 0) return hipSuccess;
  if (v4)
    hipLaunchKernelGGL(k_mse_part4, dim3(nb), dim3(kThreads), 0, st, y, target, n, dy, dyb, ws);
  else
    hipLaunchKernelGGL(k_mse_part, dim3(nb), dim3(kThreads), 0, st, y, target, n, dy, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !loss) return e;
  hipLaunchKernelGGL(k_mse_final, dim3(1), dim3(kThreads), 0, st, ws, nb, n, loss);
  return hipGetLastError();
}

hipError_t launch_kv_expand(const float* v, int64_t n_q, int64_t n_kv, int64_t hd, float* out,
                            hipStream_t st) {
  const int64_t n = n_q * hd;
  hipLaunchKernelGGL(k_kv_expand, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, v, n_q,
                     n_kv, hd, out);
  return hipGetLastError();
}

hipError_t launch_kv_reduce_add(const float* v, int64_t n_q, int64_t n_kv, int64_t hd,
                                float* out, hipStream_t st) {
  const int64_t n = n_kv * hd;
  hipLaunchKernelGGL(k_kv_reduce_add, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, v, n_q,
                     n_kv, hd, out);
  return hipGetLastError();
}

hipError_t launch_adamw(float* theta, const float* grad, float* m, float* v, int64_t n,
                        int64_t n_lwc, float lr_lwc, float lr_let, float b1, float b2, float eps,
                        float wd, int64_t step, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const float c1 = (float)(1.0 - pow((double)b1, (double)step));
  const float c2 = (float)(1.0 - pow((double)b2, (double)step));
  hipLaunchKernelGGL(k_adamw, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     st, theta, grad, m, v, n, n_lwc, lr_lwc, lr_let, b1, b2, eps, wd, c1, c2);
  return hipGetLastError();
}

hipError_t launch_sgd(float* theta, const float* grad, int64_t n, int64_t n_lwc, float lr_lwc,
                      float lr_let, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_sgd, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     st, theta, grad, n, n_lwc, lr_lwc, lr_let);
  return hipGetLastError();
}

hipError_t launch_axpy_bcast(float* y, const float* x, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_axpy, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     st, y, x, n);
  return hipGetLastError();
}

}  // namespace omq
