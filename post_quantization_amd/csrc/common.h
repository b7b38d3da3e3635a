// Shared device helpers for the OmniQuant calibration kernels (gfx950).
//
// Every translation unit is compiled with -ffp-contract=off, so no multiply-add
// is fused unless written as an explicit fmaf(); float division is IEEE
// correctly rounded (-fhip-fp32-correctly-rounded-divide-sqrt) and rintf maps to
// round-half-to-even.  These three properties make the quantizer's integer codes
// reproducible bit for bit against a float32 reference.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/omq.h"

#define OMQ_DEV __device__ __forceinline__

namespace omq {

constexpr int kWave = 64;

OMQ_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float32 -> bf16, round to nearest even (the gfx950 conversion instruction;
// NaN stays NaN).  Two at a time: a in the low half, b in the high half.
typedef __attribute__((ext_vector_type(2))) float omq_f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 omq_bf16x2;
OMQ_DEV uint32_t pack_bf16(float a, float b) {
  const omq_f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, omq_bf16x2));
}
OMQ_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Four consecutive elements of a float32 or bf16 row, widened to float32.
OMQ_DEV void load4(const void* base, int dt, int64_t idx, float v[4]) {
  if (dt == OMQ_F32) {
    float4 t = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
    uint2 t = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
    v[0] = __uint_as_float(t.x << 16);
    v[1] = __uint_as_float(t.x & 0xffff0000u);
    v[2] = __uint_as_float(t.y << 16);
    v[3] = __uint_as_float(t.y & 0xffff0000u);
  }
}

OMQ_DEV void store4(void* base, int dt, int64_t idx, const float v[4]) {
  if (dt == OMQ_F32) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx) =
        make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 t;
    t.x = pack_bf16(v[0], v[1]);
    t.y = pack_bf16(v[2], v[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + idx) = t;
  }
}

// 8 consecutive values as one 16-byte (bf16) or two 16-byte (fp32) stores: whole
// cache lines per wave instruction
OMQ_DEV void store8(void* base, int dt, int64_t idx, const float v[8]) {
  if (dt == OMQ_F32) {
    float* p = reinterpret_cast<float*>(base) + idx;
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 t;
    t.x = pack_bf16(v[0], v[1]);
    t.y = pack_bf16(v[2], v[3]);
    t.z = pack_bf16(v[4], v[5]);
    t.w = pack_bf16(v[6], v[7]);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + idx) = t;
  }
}

// gamma = sigmoid(a) evaluated in double and rounded once to float.
OMQ_DEV float sigmoid_f32(float a) { return (float)(1.0 / (1.0 + exp(-(double)a))); }

template <typename T>
OMQ_DEV T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// The RMSNorm scale of a row from its sum of squares (accumulated in double):
// 1 / sqrt(ss / n + eps) in double, rounded once to float; the normalized row is
// then x * scale in float (one rounding per element).
OMQ_DEV float rms_scale(double ss, int64_t n, float eps) {
  return (float)(1.0 / sqrt(ss / (double)n + (double)eps));
}

// (value, index) reductions; ties go to the lower index.
OMQ_DEV void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}
OMQ_DEV void argmin_merge(float& v, int& i, float v2, int i2) {
  if (v2 < v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

OMQ_DEV void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v2 = __shfl_xor(v, o, kWave);
    int i2 = __shfl_xor(i, o, kWave);
    argmax_merge(v, i, v2, i2);
  }
}
OMQ_DEV void wave_argmin(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v2 = __shfl_xor(v, o, kWave);
    int i2 = __shfl_xor(i, o, kWave);
    argmin_merge(v, i, v2, i2);
  }
}

// The quantization step of one row (the LWC equation), float32 one op at a time:
// h = (gamma*max - beta*min) / (2^N - 1), floored at 1e-8; z = -rint(beta*min / h).
struct RowQ {
  float h, z, Q, t2;
  bool floor;
};

// rint(fl32(x / h)) without a division on the common path.  With rh = fl32(1/h),
// u = fl32(x * rh) lies within 3 ulp of fl32(x / h) (one rounding each in the
// reciprocal, the product and the true quotient), so the two can round to
// different integers only when a half-integer lies between them.  Whenever u is
// within |u| * 2^-20 (8 ulp) of a half-integer, or is not finite, the exact quotient
// decides.  As |u - rint(u)| <= 1/2, every |u| >= 2^19 takes the exact path.  u
// returns the quotient used, for sums where a few ulp do not matter.
OMQ_DEV float rint_quot(float x, float h, float rh, float& u) {
  u = x * rh;
  const float r = rintf(u);
  if (!(fabsf(fabsf(u - r) - 0.5f) > fabsf(u) * 0x1p-20f)) {
    u = x / h;
    return rintf(u);
  }
  return r;
}

// The same for a LET-divided input: rint(fl32(fl32(xd / s) / h)) with xd = x - delta
// already rounded; the product form fl32(fl32(xd * rs) * rh) with rs = fl32(1/s)
// carries at most 6 ulp against it, inside the same 8-ulp guard.
OMQ_DEV float rint_quot2(float xd, float s, float rs, float h, float rh, float& u) {
  u = (xd * rs) * rh;
  const float r = rintf(u);
  if (!(fabsf(fabsf(u - r) - 0.5f) > fabsf(u) * 0x1p-20f)) {
    u = (xd / s) / h;
    return rintf(u);
  }
  return r;
}

// index of the calling wave in its block, in a scalar register (it is uniform
// within the wave, which the compiler cannot tell from threadIdx.x >> 6): rows,
// offsets and addresses derived from it then stay scalar
OMQ_DEV int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

OMQ_DEV RowQ row_step(float M, float m, float gamma, float beta, int nbits) {
  RowQ r;
  r.Q = (float)((1 << nbits) - 1);
  float t1 = gamma * M;
  r.t2 = beta * m;
  float h = (t1 - r.t2) / r.Q;
  r.floor = h < 1e-8f;
  r.h = r.floor ? 1e-8f : h;
  r.z = -rintf(r.t2 / r.h);
  return r;
}

}  // namespace omq

#define OMQ_HIP_CHECK(expr)                                   \
  do {                                                        \
    hipError_t e_ = (expr);                                   \
    if (e_ != hipSuccess) return OMQ_E_HIP;                   \
  } while (0)
