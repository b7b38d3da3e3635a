// Dense contractions of the quantized layer (paper reading, section "LET":
// Y = Q_a(X~) Q_w(W~) + B~, and the two products of its backward) on gfx950.
//
// C[M x N] = alpha * A[M x K] * B[N x K]^T (+ bias[N]) (+ residual) (+ C)
// Both operands are K-contiguous ("NT"), the layout the matrix cores read without
// any transposition: a lane of v_mfma_f32_32x32x16_bf16 holds 8 consecutive k of
// one row of A and 8 consecutive k of one column of B^T.
//
// Tile 128 x 128 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave 64 x 64 as
// 2 x 2 MFMA 32x32x16 blocks (64 float accumulators per lane).  Global loads are
// 16-byte vectors staged in registers while the matrix cores consume the other
// LDS buffer (double buffered, one barrier per K step).  LDS rows are padded by
// 16 bytes so the 16-byte fragment reads of 8 consecutive rows hit distinct banks.
// Tiles are visited in groups of 8 row-tiles and dealt to the 8 XCDs in
// contiguous runs, so tiles sharing A rows / B columns share an L2.
#include "common.h"
#include "kernels.h"

namespace omq {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = 128, BN = 128, BK = 64, LDP = BK + 8;
constexpr int kGroupM = 8;

OMQ_DEV void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = tiles_m * tiles_n;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int gsize = kGroupM * tiles_n;
  const int gid = pid / gsize;
  const int first_m = gid * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int in_g = pid - gid * gsize;
  tm = first_m + in_g % gsz;
  tn = in_g / gsz;
}

__global__ __launch_bounds__(256, 2) void k_gemm_bf16(Gemm g, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDP];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int bz = blockIdx.y;
  if (g.causal == CAUSAL_SKIP_UPPER && n0 > m0 + BM - 1) return;
  int64_t kb = 0, ke = g.K;
  if (g.causal == CAUSAL_K_UPPER) ke = min(g.K, m0 + BM);
  if (g.causal == CAUSAL_K_LOWER) kb = (m0 / BK) * BK;

  const uint16_t* A = reinterpret_cast<const uint16_t*>(g.A) + bz * g.strideA;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(g.B) + (bz / g.b_group) * g.strideB;
  const int64_t M = g.M, N = g.N;

  uint4 ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 3;
      const int kc = (id & 7) * 8;
      const int64_t gk = k0 + kc;
      const int64_t gm = m0 + row, gn = n0 + row;
      ra[i] = (gm < M && gk < ke) ? *reinterpret_cast<const uint4*>(A + gm * g.lda + gk)
                                  : make_uint4(0, 0, 0, 0);
      rb[i] = (gn < N && gk < ke) ? *reinterpret_cast<const uint4*>(B + gn * g.ldb + gk)
                                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 3;
      const int kc = (id & 7) * 8;
      *reinterpret_cast<uint4*>(&As[buf][row][kc]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[buf][row][kc]) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (int)((ke - kb + BK - 1) / BK);
  if (nk > 0) {
    gload(kb);
    sstore(0);
  }
  __syncthreads();
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kb + (int64_t)(kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][wm * 64 + i * 32 + fr][kk + fk]);
        bf[i] = *reinterpret_cast<const bf16x8*>(&Bs[buf][wn * 64 + i * 32 + fr][kk + fk]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
  float* C = g.C ? g.C + bz * g.strideC : nullptr;
  uint16_t* Cb = g.Cb ? g.Cb + bz * g.strideC : nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t gn = n0 + wn * 64 + j * 32 + (lane & 31);
      if (gn >= N) continue;
      const float bias = g.bias ? g.bias[gn] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gm = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (gm >= M) continue;
        float v = g.alpha * acc[i][j][r] + bias;
        if (g.resid) {
          v += g.resid_dt == OMQ_F32
                   ? reinterpret_cast<const float*>(g.resid)[gm * g.ldr + gn]
                   : bf16_to_f32(reinterpret_cast<const uint16_t*>(g.resid)[gm * g.ldr + gn]);
        }
        if (Cb) {
          Cb[gm * g.ldc + gn] = f32_to_bf16(v);
        } else {
          if (g.accumulate) v += C[gm * g.ldc + gn];
          C[gm * g.ldc + gn] = v;
        }
      }
    }
}

// float32 operands (the fp32 path): 64 x 64 tiles, 4 x 4 outputs per thread.
__global__ __launch_bounds__(256) void k_gemm_f32(Gemm g) {
  constexpr int T = 64, KB = 16;
  __shared__ float As[KB][T + 4];
  __shared__ float Bs[KB][T + 4];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * T, n0 = (int64_t)blockIdx.x * T;
  const int bz = blockIdx.z;
  const float* A = reinterpret_cast<const float*>(g.A) + bz * g.strideA;
  const float* B = reinterpret_cast<const float*>(g.B) + (bz / g.b_group) * g.strideB;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < g.K; k0 += KB) {
    for (int i = threadIdx.x; i < T * KB; i += 256) {
      const int r = i / KB, kk = i % KB;
      const int64_t gk = k0 + kk;
      const bool ina = m0 + r < g.M && gk < g.K, inb = n0 + r < g.N && gk < g.K;
      As[kk][r] = ina ? (g.ta ? A[gk * g.lda + m0 + r] : A[(m0 + r) * g.lda + gk]) : 0.f;
      Bs[kk][r] = inb ? (g.tb ? B[gk * g.ldb + n0 + r] : B[(n0 + r) * g.ldb + gk]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][ty * 4 + i]; b[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* C = g.C ? g.C + bz * g.strideC : nullptr;
  uint16_t* Cb = g.Cb ? g.Cb + bz * g.strideC : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gm = m0 + ty * 4 + i, gn = n0 + tx * 4 + j;
      if (gm >= g.M || gn >= g.N) continue;
      float v = g.alpha * acc[i][j] + (g.bias ? g.bias[gn] : 0.f);
      if (g.resid)
        v += g.resid_dt == OMQ_F32
                 ? reinterpret_cast<const float*>(g.resid)[gm * g.ldr + gn]
                 : bf16_to_f32(reinterpret_cast<const uint16_t*>(g.resid)[gm * g.ldr + gn]);
      if (Cb) {
        Cb[gm * g.ldc + gn] = f32_to_bf16(v);
      } else {
        if (g.accumulate) v += C[gm * g.ldc + gn];
        C[gm * g.ldc + gn] = v;
      }
    }
}

// 64 x 64 tile transposes through LDS
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* in, int64_t rows,
                                                        int64_t cols, int64_t ldi, uint16_t* out,
                                                        int64_t ldo, int64_t sin, int64_t sout) {
  __shared__ uint16_t t[64][66];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  in += blockIdx.z * sin;
  out += blockIdx.z * sout;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < rows && c < cols) ? in[r * ldi + c] : (uint16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) out[c * ldo + r] = t[tx][i];
  }
}

__global__ __launch_bounds__(256) void k_f32_to_bf16(const float* in, int64_t rows, int64_t cols,
                                                     int64_t ldi, uint16_t* out, int64_t ldo,
                                                     uint16_t* out_t, int64_t ldt) {
  __shared__ uint16_t t[64][66];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    uint16_t b = 0;
    if (r < rows && c < cols) {
      b = f32_to_bf16(in[r * ldi + c]);
      if (out) out[r * ldo + c] = b;
    }
    t[i][tx] = b;
  }
  if (!out_t) return;
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) out_t[c * ldt + r] = t[tx][i];
  }
}

}  // namespace

hipError_t launch_gemm(const Gemm& g, hipStream_t st) {
  if (g.M == 0 || g.N == 0 || g.batch == 0) return hipSuccess;
  if (g.dt == OMQ_BF16) {
    const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
    hipLaunchKernelGGL(k_gemm_bf16, dim3((unsigned)(tiles_m * tiles_n), (unsigned)g.batch),
                       dim3(256), 0, st, g, tiles_m, tiles_n);
  } else {
    dim3 grid((unsigned)((g.N + 63) / 64), (unsigned)((g.M + 63) / 64), (unsigned)g.batch);
    hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, int64_t ldi,
                                 uint16_t* out, int64_t ldo, int batch, int64_t stride_in,
                                 int64_t stride_out, hipStream_t st) {
  if (rows == 0 || cols == 0 || batch == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64), (unsigned)batch);
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, st, in, rows, cols, ldi, out, ldo,
                     stride_in, stride_out);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* in, int64_t rows, int64_t cols, int64_t ldi,
                              uint16_t* out, int64_t ldo, uint16_t* out_t, int64_t ldt,
                              hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
  hipLaunchKernelGGL(k_f32_to_bf16, grid, dim3(256), 0, st, in, rows, cols, ldi, out, ldo, out_t,
                     ldt);
  return hipGetLastError();
}

}  // namespace omq
