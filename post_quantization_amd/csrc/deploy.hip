// Deployment form of a calibrated layer (paper reading, section "LWC": the
// deployed weight is the integer code with its step h and zero point z, and
// section "LET": the equivalent transformation is folded into neighbouring
// parameters after calibration): packing of N-bit codes into 32-bit words, the
// weight-only LET fold of a layer's bias (and of the attention-output pair into
// the value projection), and the weight-only product on packed 4-bit codes.
//
// Packed layout: along a row, floor(32 / N) codes per 32-bit word, code j of a word
// in bits [jN, (j+1)N), lowest column first; ceil(cols / per_word) words per row.
#include "common.h"
#include "kernels.h"

namespace omq {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__global__ __launch_bounds__(256) void k_pack_codes(const uint8_t* codes, int64_t rows,
                                                    int64_t cols, int nbits, uint32_t* words) {
  const int P = 32 / nbits;
  const int64_t nw = (cols + P - 1) / P;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * nw) return;
  const int64_t r = i / nw, j = i % nw;
  const uint8_t* cr = codes + r * cols + j * P;
  const int n = (int)min((int64_t)P, cols - j * P);
  uint32_t w = 0;
  for (int p = 0; p < n; ++p) w |= (uint32_t)cr[p] << (p * nbits);
  words[i] = w;
}

// The 4-bit codes of one word as two words of bytes: the even columns' codes in
// lo, the odd columns' in hi.  Formed in one ALU block the compiler cannot see
// into, so that each byte of lo / hi then converts with one v_cvt_f32_ubyteN (it
// would otherwise fold the masks into a bit-field extract per code, two
// instructions per column).
OMQ_DEV void nibble_bytes(uint32_t w, uint32_t& lo, uint32_t& hi) {
  asm("v_and_b32 %0, 0x0f0f0f0f, %2\n\tv_lshrrev_b32 %1, 4, %2\n\t"
      "v_and_b32 %1, 0x0f0f0f0f, %1"
      : "=&v"(lo), "=&v"(hi)
      : "v"(w));
}

// W_hat of 8 consecutive columns from one word of 4-bit codes: (q - z) h rounded
// once to float32, the same values the calibration's fake quantizer produced
OMQ_DEV void dequant8(uint32_t w, float h, float z, float out[8]) {
  uint32_t lo, hi;
  nibble_bytes(w, lo, hi);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    out[2 * b] = ((float)((lo >> (8 * b)) & 0xffu) - z) * h;
    out[2 * b + 1] = ((float)((hi >> (8 * b)) & 0xffu) - z) * h;
  }
}

// One wave per output row n: bias_out[n] = (B~[n] - sum_k W_hat[n,k] delta[k] / s[k]
// - delta_o[n]) / s_o[n]; with s_o, also h_out = h / s_o for the row's steps.
__global__ __launch_bounds__(256) void k_fold_linear(DeployFold a) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave_id();
  if (n >= a.N) return;
  const int P = 32 / a.nbits;
  const int64_t nw = (a.K + P - 1) / P;
  const int64_t G = a.group ? a.K / a.group : 1;
  const uint32_t mask = (1u << a.nbits) - 1u;
  float acc = 0.f;
  if (a.delta) {
    for (int64_t j = lane; j < nw; j += 64) {
      const uint32_t w = a.words[n * nw + j];
#pragma unroll 4
      for (int p = 0; p < P; ++p) {
        const int64_t k = j * P + p;
        if (k >= a.K) break;
        const int64_t gi = a.group ? n * G + (k >> 7) : n;   // group 128 or the row
        const float wh = ((float)((w >> (p * a.nbits)) & mask) - a.z[gi]) * a.h[gi];
        acc += wh * (a.delta[k] / a.s[k]);
      }
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    float b = (a.B ? a.B[n] : 0.f) - acc;
    if (a.s_o) b = (b - (a.delta_o ? a.delta_o[n] : 0.f)) / a.s_o[n];
    a.bias_out[n] = b;
  }
  if (a.s_o && a.h_out) {
    for (int64_t g = lane; g < G; g += 64) a.h_out[n * G + g] = a.h[n * G + g] / a.s_o[n];
  }
  // the input site's gain, written by the waves of the first output rows
  if (a.gain_out)
    for (int64_t k = n * 64 + lane; k < a.K && n * 64 < a.K; k += a.N * 64)
      a.gain_out[k] = 1.f / a.s[k];
}

// Y[T x N] = X[T x K] W_hat^T (+ bias), W_hat from 4-bit packed codes with (h, z)
// per row or per 128-column group, on the matrix cores (more than 8 tokens).
// Block: 32 output rows x 32 tokens over all of
// K, 16 waves taking the 64-column blocks of K in turn, 4 blocks at a time with
// all their code loads issued before the arithmetic (memory-level parallelism is
// what a bandwidth-bound small-T product needs).  In a 64-column block, lane half
// hf supplies columns 32 hf + 8 s + 0..7 for k slice s (one 32-bit word of codes),
// and the token operand is read in the same order, so each MFMA contracts 16
// matching columns.  The 16 partial tiles are summed through LDS.
constexpr int kWaves = 16;
constexpr int kBatch = 4;

__global__ __launch_bounds__(kWaves * 64) void k_w4a16_gemm(DeployGemm a) {
  __shared__ float red[kWaves][32][33];
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), hf = lane >> 5, l32 = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * 32, t0 = (int64_t)blockIdx.y * 32;
  const int64_t n = n0 + l32, t = t0 + l32;
  const bool nv = n < a.N, tv = t < a.T;
  const int64_t nw = a.K / 8;                      // words per row
  const int64_t G = a.group ? a.K / a.group : 1;
  const int64_t nkb = a.K / 64;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.X);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int64_t base = w; base < nkb; base += kWaves * kBatch) {
    u32x4 cw[kBatch];
    float hh[kBatch], zz[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t kb = base + kWaves * j;
      const int64_t k0 = kb * 64 + 32 * hf;
      cw[j] = u32x4{0u, 0u, 0u, 0u};
      hh[j] = 0.f;
      zz[j] = 0.f;
      if (nv && kb < nkb) {
        cw[j] = *reinterpret_cast<const u32x4*>(a.words + n * nw + k0 / 8);
        const int64_t gi = a.group ? n * G + (k0 >> 7) : n;  // group 128 or the row
        hh[j] = a.h[gi];
        zz[j] = a.z[gi];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t kb = base + kWaves * j;
      if (kb >= nkb) break;                        // wave-uniform
      const int64_t k0 = kb * 64 + 32 * hf;
      const uint32_t wv[4] = {cw[j].x, cw[j].y, cw[j].z, cw[j].w};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float f[8];
        dequant8(wv[s], hh[j], zz[j], f);
        const u32x4 av = {pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
                          pack_bf16(f[6], f[7])};
        u32x4 bv = {0u, 0u, 0u, 0u};
        if (tv) bv = *reinterpret_cast<const u32x4*>(X + t * a.K + k0 + 8 * s);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, bv), acc, 0, 0,
                                                      0);
      }
    }
  }
  // C: column = token (lane & 31), rows = output channels 8 (r/4) + 4 hf + (r%4)
#pragma unroll
  for (int r = 0; r < 16; ++r) red[w][8 * (r >> 2) + 4 * hf + (r & 3)][l32] = acc[r];
  __syncthreads();
  const int i = tid >> 5, jt = tid & 31;           // i: output channel, jt: token
  const int64_t nn = n0 + i, tt = t0 + jt;
  if (nn < a.N && tt < a.T) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) v += red[q][i][jt];
    if (a.bias) v += a.bias[nn];
    a.Y[tt * a.N + nn] = v;
  }
}

// Y[T x N] for a few tokens (T <= TM) on the vector units: one wave per output row
// streams the row's packed codes with 16-byte loads (32 columns per lane and load,
// always inside one 128-column group), dequantizes each pair of columns to bf16
// exactly as the matrix-core kernel forms its operand, and accumulates bf16-pair
// dot products with the tokens' bf16 pairs in fp32; one wave reduction per token.
// A bandwidth-bound product: each code is read once per TM tokens, x comes from the
// caches.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

template <int TM>
__global__ __launch_bounds__(256) void k_w4a16_gemv(DeployGemm a) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave_id();
  if (n >= a.N) return;
  const int64_t nw = a.K / 8;                      // words per row
  const int64_t G = a.group ? a.K / a.group : 1;
  const uint32_t* wr = a.words + n * nw;
  const uint32_t* X = reinterpret_cast<const uint32_t*>(a.X);   // bf16 pairs
  const int64_t xw = a.K / 2;                      // pairs per token
  float acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = 0.f;
  // one 16-byte chunk (32 columns) of codes into the accumulators
  auto chunk = [&](const u32x4 cw, int64_t j) {
    const int64_t col0 = j * 8;
    const int64_t gi = a.group ? n * G + (col0 >> 7) : n;  // group 128 or the row
    const float hh = a.h[gi], zz = a.z[gi];
    // W_hat pairs (columns col0 + 2p, col0 + 2p + 1), p = 0..15
    uint32_t wp[16];
    const uint32_t ws[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t lo, hi;
      nibble_bytes(ws[s], lo, hi);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float f0 = ((float)((lo >> (8 * b)) & 0xffu) - zz) * hh;
        const float f1 = ((float)((hi >> (8 * b)) & 0xffu) - zz) * hh;
        wp[4 * s + b] = pack_bf16(f0, f1);
      }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < a.T) {                               // uniform
        const u32x4* xr = reinterpret_cast<const u32x4*>(X + t * xw + col0 / 2);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 xv = xr[v];
          const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wp[4 * v + e]),
                                                      __builtin_bit_cast(bf16x2, xs[e]), acc[t],
                                                      false);
        }
      }
    }
  };
  // two chunks' code loads in flight before their arithmetic
  int64_t j = (int64_t)lane * 4;
  for (; j + 256 < nw; j += 512) {
    const u32x4 c0 = *reinterpret_cast<const u32x4*>(wr + j);
    const u32x4 c1 = *reinterpret_cast<const u32x4*>(wr + j + 256);
    chunk(c0, j);
    chunk(c1, j + 256);
  }
  if (j < nw) chunk(*reinterpret_cast<const u32x4*>(wr + j), j);
  const float b = a.bias ? a.bias[n] : 0.f;
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < a.T) {
      const float v = wave_sum(acc[t]);
      if (lane == 0) a.Y[t * a.N + n] = v + b;
    }
  }
}

}  // namespace

hipError_t launch_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int nbits,
                             uint32_t* words, hipStream_t st) {
  const int P = 32 / nbits;
  const int64_t n = rows * ((cols + P - 1) / P);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_codes, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, codes,
                     rows, cols, nbits, words);
  return hipGetLastError();
}

hipError_t launch_fold_linear(const DeployFold& a, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fold_linear, dim3((unsigned)((a.N + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_w4a16_gemm(const DeployGemm& a, hipStream_t st) {
  if (a.N == 0 || a.T == 0) return hipSuccess;
  // a few tokens: the vector-unit product, one wave per output row (at 16 tokens
  // the matrix-core kernel is 3x faster: every wave would re-read all the tokens)
  if (a.T <= 8) {
    const dim3 g((unsigned)((a.N + 3) / 4));
    if (a.T == 1) hipLaunchKernelGGL(k_w4a16_gemv<1>, g, dim3(256), 0, st, a);
    else if (a.T == 2) hipLaunchKernelGGL(k_w4a16_gemv<2>, g, dim3(256), 0, st, a);
    else if (a.T <= 4) hipLaunchKernelGGL(k_w4a16_gemv<4>, g, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(k_w4a16_gemv<8>, g, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((a.N + 31) / 32), (unsigned)((a.T + 31) / 32));
  hipLaunchKernelGGL(k_w4a16_gemm, grid, dim3(kWaves * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace omq
