// Dense contractions of the quantized layer (paper reading, section "LET":
// Y = Q_a(X~) Q_w(W~) + B~, and the two products of its backward) on gfx950.
//
// C[M x N] = alpha * op(A)[M x K] * op(B)[N x K]^T (+ bias[N]) (+ residual) (+ C)
// In LDS both operands are held K-contiguous, the layout the matrix cores read:
// a lane of v_mfma_f32_32x32x16_bf16 holds 8 consecutive k of one row of A and 8
// consecutive k of one column of B^T.  An operand stored K-major in HBM ("T",
// [K x M] with M contiguous) is copied into LDS in that layout and transposed by
// the LDS read itself (ds_read_b64_tr_b16) when every tile is whole, or loaded as
// 4 k-rows x 8 contiguous elements per thread and transposed in registers with
// byte permutes on its way into LDS otherwise, so no product of the backward needs
// a transposed copy in HBM.
//
// Tile 128 x 128 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave 64 x 64 as
// 2 x 2 MFMA 32x32x16 blocks (64 float accumulators per lane).  Global loads are
// 16-byte vectors staged in registers while the matrix cores consume the other
// LDS buffer (double buffered, one barrier per K step).
// Tiles are visited in groups of 8 row-tiles and dealt to the 8 XCDs in
// contiguous runs, so tiles sharing A rows / B columns share an L2.
// LDS rows are unpadded and XOR-swizzled (see lds_idx).
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace omq {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) int i32x16;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int BK = 64, LDP = BK;

// LDS tiles are [rows][64] bf16 with the 16-byte k-chunk index XOR-swizzled by
// (row & 7) ^ ((row >> 3) & 7): the matrix-core fragment reads (8 consecutive rows,
// one chunk) and the transposed-operand stores (rows 8 apart, one k-quad) both
// spread over distinct banks.
// 32-wide k steps: [rows][32] with the chunk index XOR-swizzled by (row >> 1) & 3, so
// the 8 rows one 8-lane group of a fragment read touches cover 8 distinct 16-byte
// slots of a 256-byte bank window.
template <int KB = 64>
OMQ_DEV int lds_idx(int row, int k) {
  if constexpr (KB == 32) return row * 32 + ((((k >> 3) ^ (row >> 1)) & 3) << 3) + (k & 7);
  else return row * LDP + ((((k >> 3) ^ row ^ (row >> 3)) & 7) << 3) + (k & 7);
}
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

// One operand tile (R rows x 64 k) staged through registers by NT threads.
//  N layout ([rows x K], K contiguous): 16-byte chunks, 8 per row.
//  T layout ([K x rows], rows contiguous): 4 k-rows x 8 rows per thread, transposed
//  in registers (byte permutes) into 8-byte LDS writes of 4 consecutive k.
template <int TRANS, int R, int NT>
struct Stage {
  static constexpr int kUnits = TRANS ? R * 2 : R * 8;          // sub-blocks / chunks
  static constexpr int kN = (kUnits + NT - 1) / NT;              // per thread
  uint4 r[TRANS ? 4 * kN : kN];

  // interior tiles (all rows and the whole k-step in range) skip the bounds checks
  OMQ_DEV void load_full(const uint16_t* P, int64_t ld, int64_t row0, int64_t k0, int tid) {
    if (!TRANS) {
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        const int id = tid + NT * i;
        if (kUnits % NT == 0 || id < kUnits)
          r[i] = *reinterpret_cast<const uint4*>(P + (row0 + (id >> 3)) * ld + k0 + (id & 7) * 8);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kN; ++u) {
        const int id = tid + NT * u;
        if (kUnits % NT == 0 || id < kUnits) {
          const int64_t gr = row0 + (id % (R / 8)) * 8;
          const int kq = id / (R / 8);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            r[4 * u + i] = *reinterpret_cast<const uint4*>(P + (k0 + kq * 4 + i) * ld + gr);
        }
      }
    }
  }

  OMQ_DEV void load(const uint16_t* P, int64_t ld, int64_t rows, int64_t row0, int64_t k0,
                    int64_t ke, int tid) {
    if (row0 + R <= rows && k0 + BK <= ke) {
      load_full(P, ld, row0, k0, tid);
      return;
    }
    if (!TRANS) {
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        const int id = tid + NT * i;
        const int64_t gr = row0 + (id >> 3), gk = k0 + (id & 7) * 8;
        r[i] = (id < kUnits && gr < rows && gk < ke)
                   ? *reinterpret_cast<const uint4*>(P + gr * ld + gk)
                   : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kN; ++u) {
        const int id = tid + NT * u;             // sub-block: (R/8) row blocks x 16 k-quads
        const int64_t gr = row0 + (id % (R / 8)) * 8;
        const int kq = id / (R / 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t gk = k0 + kq * 4 + i;
          r[4 * u + i] = (id < kUnits && gr < rows && gk < ke)
                             ? *reinterpret_cast<const uint4*>(P + gk * ld + gr)
                             : make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  OMQ_DEV void store(uint16_t* S, int tid) const {
    if (!TRANS) {
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        const int id = tid + NT * i;
        if (kUnits % NT == 0 || id < kUnits)
          *reinterpret_cast<uint4*>(S + lds_idx(id >> 3, (id & 7) * 8)) = r[i];
      }
    } else {
#pragma unroll
      for (int u = 0; u < kN; ++u) {
        const int id = tid + NT * u;
        if (kUnits % NT != 0 && id >= kUnits) continue;
        const int rb = (id % (R / 8)) * 8, kc = (id / (R / 8)) * 4;
        const uint32_t w[4][4] = {{r[4 * u].x, r[4 * u].y, r[4 * u].z, r[4 * u].w},
                                  {r[4 * u + 1].x, r[4 * u + 1].y, r[4 * u + 1].z, r[4 * u + 1].w},
                                  {r[4 * u + 2].x, r[4 * u + 2].y, r[4 * u + 2].z, r[4 * u + 2].w},
                                  {r[4 * u + 3].x, r[4 * u + 3].y, r[4 * u + 3].z, r[4 * u + 3].w}};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int q = j >> 1;
          const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
          uint2 v;
          v.x = __builtin_amdgcn_perm(w[1][q], w[0][q], sel);
          v.y = __builtin_amdgcn_perm(w[3][q], w[2][q], sel);
          *reinterpret_cast<uint2*>(S + lds_idx(rb + j, kc)) = v;
        }
      }
    }
  }
};

// Direct global -> LDS copy of a full R x 64 tile of a K-contiguous operand:
// one wave instruction fills 8 swizzled LDS rows (1 KB, lane l at byte 16 l), so
// lane l fetches the k-chunk that the swizzle places at its slot.  Completion is
// tracked by vmcnt like any vector load.
template <int R, int NW, int KB = 64>
OMQ_DEV void dma_tile(const uint16_t* P, int64_t ld, int64_t row0, int64_t k0, uint16_t* S,
                      int wid, int lane) {
  constexpr int RPI = 512 / KB;                    // rows per 1 KB wave instruction
  constexpr int CPR = KB / 8;                      // 16-byte chunks per row
  constexpr int NB = R / RPI;
  static_assert(NB % NW == 0, "row blocks must divide over the waves");
#pragma unroll
  for (int i = 0; i < NB / NW; ++i) {
    const int b = wid + NW * i;
    const int r = b * RPI + lane / CPR;
    const int c = KB == 32 ? (((lane & 3) ^ (r >> 1)) & 3) : (((lane & 7) ^ r ^ (r >> 3)) & 7);
    __builtin_amdgcn_global_load_lds(
        (const void*)(P + (row0 + r) * ld + k0 + c * 8),
        (__attribute__((address_space(3))) void*)(S + b * RPI * KB), 16, 0, 0);
  }
}

// K-major tiles in LDS are [64 k-rows][R] bf16, the tile as it lies in HBM, with the
// 16-byte chunk index of k-row kr XOR-swizzled by ((kr & 3) << 1) | ((kr & 1) << 3):
// a transposing read of one 16-lane group touches 4 consecutive k-rows x 32 bytes,
// which then fall on distinct banks, and so do the 16-lane group reading the other
// 32 bytes of the same rows.
template <int R>
OMQ_DEV int ldsT_idx(int kr, int col) {
  static_assert(R >= 128, "the swizzle spans 16 chunks");
  return kr * R + ((((col >> 3) ^ (((kr & 3) << 1) | ((kr & 1) << 3)))) << 3) + (col & 7);
}

// Direct global -> LDS copy of a full 64 x R tile of a K-major operand ([K x rows],
// rows contiguous): one wave instruction fills 1 KB = 1024 / (2R) k-rows, lane l at
// byte 16 l, so lane l fetches the chunk the swizzle places at its slot.
template <int R, int NW, int KB = 64>
OMQ_DEV void dma_tile_t(const uint16_t* P, int64_t ld, int64_t col0, int64_t k0, uint16_t* S,
                        int wid, int lane) {
  constexpr int CPR = R / 8;                       // 16-byte chunks per k-row
  constexpr int RPI = 64 / CPR;                    // k-rows per wave instruction
  constexpr int NI = KB / RPI;                     // instructions per tile
  static_assert(NI % NW == 0, "k-row blocks must divide over the waves");
#pragma unroll
  for (int i = 0; i < NI / NW; ++i) {
    const int b = wid + NW * i;
    const int kr = b * RPI + lane / CPR;
    const int c = (lane % CPR) ^ (((kr & 3) << 1) | ((kr & 1) << 3));
    __builtin_amdgcn_global_load_lds(
        (const void*)(P + (k0 + kr) * ld + col0 + c * 8),
        (__attribute__((address_space(3))) void*)(S + b * RPI * R), 16, 0, 0);
  }
}

// direct copy of one operand tile: K-contiguous (R rows x KB) or K-major (KB x R)
template <int TR, int R, int NW, int KB = 64>
OMQ_DEV void dma_copy(const uint16_t* P, int64_t ld, int64_t r0, int64_t k0, uint16_t* S, int wid,
                      int lane) {
  if constexpr (TR) dma_tile_t<R, NW, KB>(P, ld, r0, k0, S, wid, lane);
  else dma_tile<R, NW, KB>(P, ld, r0, k0, S, wid, lane);
}

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;

// Matrix-core fragment (8 consecutive k of one row, in the lane order of
// v_mfma_f32_32x32x16_bf16: row rb + (lane & 31), k kb + 8 (lane >> 5) + 0..7) of a
// K-major LDS tile, from two transposing reads.  In each 16-lane group the read
// hands lane i element j of the 4-element chunk that lane 4j + i/4 addressed, at
// position i % 4; so lane 4j + q of the group addresses k-row j, columns 4q..4q+3
// of its 16 rows, and lane i receives 4 consecutive k of row i.
template <int R>
OMQ_DEV bf16x8 tr_frag(const uint16_t* S, int rb, int kb, int lane) {
  const int G = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
  const int kr = kb + 8 * (G >> 1) + j;
  const int col = rb + 16 * (G & 1) + 4 * q;
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(S + ldsT_idx<R>(kr, col)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(S + ldsT_idx<R>(kr + 4, col)));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
OMQ_DEV void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Straight-through epilogue variants, fixed at compile time so the per-element
// arithmetic is straight-line code: EPI = mode | let << 2 | xf << 4, with mode 1 the
// weight side (rows = output channels, x = the weights, column partials of the LET
// scale) and mode 2 the activation side (rows = tokens, x = the activations, dL/dx
// written, column partials of the LET pair); let 0 none, 1 divide (activations),
// 2 multiply (weights); xf: x stored in fp32 (else bf16).  0 = no epilogue.
constexpr int kLetNone = 0, kLetDiv = 1, kLetMul = 2;
constexpr int epi_code(int mode, int let, int xf) { return mode | (let << 2) | (xf << 4); }

// BM x BN tile, WM x WN waves, each wave (BM/WM) x (BN/WN) as 32x32 MFMA blocks.
// DMA: both operands are copied straight into LDS (the launcher only sets it when
// every tile is full and the operands are 16-byte aligned), K-major ones read back
// through the transposing LDS read; otherwise both are staged through registers.
// I8: the operands are int8 codes, K contiguous, moved through exactly the same
// tiles as bf16 pairs (a 64-wide bf16 k-step is 128 codes), and the matrix cores
// run v_mfma_i32_32x32x32_i8, whose lane holds 16 consecutive codes where the bf16
// form holds 8 elements: the same 16 bytes.  The epilogue dequantizes.
// KB: the k-step, 64, or 32 with direct copies (half the LDS per stage, so wider
// wave tiles still fit two workgroups per compute unit).
// PK (with I8, direct copies and KB = 32): 4-bit codes two to a byte; a k-step of 64
// bytes is 128 codes, and each fragment read of 8 bytes is unpacked into the 16
// bytes of the int8 operand (the low nibbles of a word, then its high nibbles: codes
// 0 2 4 6 1 3 5 7 of each 8).  Both operands take the same order, so the sum over k
// is the same.
template <int BM, int BN, int WM, int WN, int TA, int TB, int EPI, int DMA, int I8 = 0,
          int KB = 64, int PK = 0>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void k_gemm_bf16(Gemm g, int tiles_m, int tiles_n) {
  constexpr int NT = WM * WN * 64, NW = WM * WN;
  constexpr int FM = BM / WM / 32, FN = BN / WN / 32;   // MFMA blocks per wave
  constexpr bool kDmaA = DMA, kDmaB = DMA;
  static_assert(EPI == 0 ||
                    (BN == 128 && ((BM == 128 && WM == 2 && WN == 2) ||
                                   (BM == 256 && WM == 4 && WN == 1 && (EPI & 3) == 1))),
                "straight-through epilogue tile");
  static_assert(!I8 || (EPI == 0 && TA == 0 && TB == 0), "integer codes: plain K-contiguous");
  static_assert(KB == 64 || (KB == 32 && DMA), "32-wide k steps take direct copies");
  static_assert(!PK || (I8 && DMA && KB == 32 && BM == 128 && BN == 128), "packed codes");
  // operand ring, and the epilogue's [128][128] float32 parking area
  constexpr int kRing = 2 * (BM + BN) * KB, kPark = EPI ? 128 * 128 * 2 : 0;
  __shared__ __attribute__((aligned(16))) uint16_t smem[kRing > kPark ? kRing : kPark];
  uint16_t (*As)[BM * KB] = reinterpret_cast<uint16_t (*)[BM * KB]>(smem);
  uint16_t (*Bs)[BN * KB] = reinterpret_cast<uint16_t (*)[BN * KB]>(smem + 2 * BM * KB);

  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  const int wm = wid / WN, wn = wid % WN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int bz = blockIdx.y;
  // K extent and leading dimensions in 16-bit units (codes: pairs of bytes)
  const int64_t kb = 0, ke = I8 ? (PK ? g.K >> 2 : g.K >> 1) : g.K;
  const int64_t lda = I8 ? g.lda >> 1 : g.lda, ldb = I8 ? g.ldb >> 1 : g.ldb;

  const uint16_t* A =
      reinterpret_cast<const uint16_t*>(g.A) + bz * (I8 ? g.strideA >> 1 : g.strideA);
  const uint16_t* B = reinterpret_cast<const uint16_t*>(g.B) +
                      (bz / g.b_group) * (I8 ? g.strideB >> 1 : g.strideB);
  const int64_t M = g.M, N = g.N;

  Stage<TA, BM, NT> sa;
  Stage<TB, BN, NT> sb;
  typedef std::conditional_t<I8 != 0, i32x16, f32x16> AccT;
  AccT acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  // The straight-through epilogue reads x for
  // each of the RW rows a wave finishes, 2 columns per lane, in batches of RB rows
  // fetched two batches ahead of their use.
  constexpr int kMode = EPI & 3, kLet = (EPI >> 2) & 3;
  constexpr bool kXF = (EPI >> 4) & 1;
  static_assert(EPI == 0 || (kMode == 1 && kLet != kLetDiv && !kXF) ||
                    (kMode == 2 && kLet != kLetMul), "epilogue variant");
  // Rows per wave and pass: 32.  With 2 x 2 waves (a wave holds 64 x 64) the tile is
  // parked whole and each wave takes 32 rows; with 4 x 1 waves (a wave holds 64 whole
  // rows of 128 columns) each wave parks and finishes its own rows, 32 at a time.
  constexpr bool kOwnRows = WN == 1;
  constexpr int NPASS = kOwnRows ? BM / WM / 32 : 1;
  constexpr int RW = 32;
  constexpr int RB = kOwnRows ? 4 : 8;            // rows per batch (4: registers for the
                                                  // accumulators of the pass still to come)
  constexpr int XR = kXF ? 2 : 1;                 // 32-bit words of x per lane and row
  const int64_t gn = n0 + 2 * lane;               // the epilogue lane's two columns
  int64_t wr0 = m0 + wid * RW;                    // first epilogue row of this wave
  // direct copies imply whole tiles: no row or column bounds in the epilogue
  constexpr bool kFull = DMA;
  auto fetch_x = [&](int b, uint32_t (&xb)[RB][XR]) {
    if constexpr (EPI != 0) {
      const SteEpi& e = g.ste;
      const bool colv = kFull || gn < N;          // N is a multiple of 8
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const int64_t gm = wr0 + b * RB + q;      // wave-uniform
#pragma unroll
        for (int w = 0; w < XR; ++w) xb[q][w] = 0u;
        if (kFull || gm < M) {
          const int sg = (e.nseg > 1 && gm >= e.seg_end[0]) + (e.nseg > 2 && gm >= e.seg_end[1]);
          const int64_t lr = gm - (sg == 0 ? 0 : e.seg_end[sg - 1]);
          // the row's 2-column words start at column n0; lane l reads word l
          const uint32_t* xr = reinterpret_cast<const uint32_t*>(
              reinterpret_cast<const char*>(e.xseg[sg]) + (lr * e.ldx + n0) * (kXF ? 4 : 2));
          if (colv) {
            if constexpr (kXF) {
              const uint2 t = reinterpret_cast<const uint2*>(xr)[lane];
              xb[q][0] = t.x;
              xb[q][1] = t.y;
            } else {
              xb[q][0] = xr[lane];
            }
          }
        }
      }
    }
  };

  // Pipeline per K step.  Direct copies: the next tile is copied into the other LDS
  // buffer while this one is consumed.  Register staging: the next tile (loaded one
  // step earlier) is stored into the other buffer and the tile after it is loaded.
  // 128 x 128 tiles read every fragment of the buffer first and then run the MFMAs;
  // 256 x 256 tiles (twice the fragments per wave) read each 16-k slice one slice
  // ahead of its MFMAs.  One barrier per step.
  const int nk = (int)((ke - kb + KB - 1) / KB);
  if (nk > 0) {
    if (kDmaA) dma_copy<TA, BM, NW, KB>(A, lda, m0, kb, As[0], wid, lane);
    else { sa.load(A, lda, M, m0, kb, ke, tid); sa.store(As[0], tid); }
    if (kDmaB) dma_copy<TB, BN, NW, KB>(B, ldb, n0, kb, Bs[0], wid, lane);
    else { sb.load(B, ldb, N, n0, kb, ke, tid); sb.store(Bs[0], tid); }
    if (nk > 1) {
      if (!kDmaA) sa.load(A, lda, M, m0, kb + BK, ke, tid);
      if (!kDmaB) sb.load(B, ldb, N, n0, kb + BK, ke, tid);
    }
  }
  if constexpr (DMA) wait_vmem<0>();
  __syncthreads();
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  auto mfma = [](AccT& c, bf16x8 a, bf16x8 b) {
    if constexpr (I8)
      c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
    else
      c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  };
  const int ar = wm * (BM / WM) + fr, br = wn * (BN / WN) + fr;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const uint16_t* Ab = As[buf];
    const uint16_t* Bb = Bs[buf];
    // next tile into the other buffer (staged: the tile after it into registers)
    auto issue_next = [&]() {
      if (kt + 1 < nk) {
        const int64_t k1 = kb + (int64_t)(kt + 1) * KB;
        if (kDmaA) dma_copy<TA, BM, NW, KB>(A, lda, m0, k1, As[buf ^ 1], wid, lane);
        if (kDmaB) dma_copy<TB, BN, NW, KB>(B, ldb, n0, k1, Bs[buf ^ 1], wid, lane);
        if (!kDmaA) sa.store(As[buf ^ 1], tid);
        if (!kDmaB) sb.store(Bs[buf ^ 1], tid);
        if (kt + 2 < nk) {
          const int64_t k2 = kb + (int64_t)(kt + 2) * BK;
          if (!kDmaA) sa.load(A, lda, M, m0, k2, ke, tid);
          if (!kDmaB) sb.load(B, ldb, N, n0, k2, ke, tid);
        }
      }
    };
    // fragment i of A / j of B for the 16-k slice kk
    auto fa = [&](int i, int kk) -> bf16x8 {
      if constexpr (DMA && TA) return tr_frag<BM>(Ab, wm * (BM / WM) + i * 32, kk * 16, lane);
      else return *reinterpret_cast<const bf16x8*>(&Ab[lds_idx<KB>(ar + i * 32, kk * 16 + fk)]);
    };
    auto fb = [&](int j, int kk) -> bf16x8 {
      if constexpr (DMA && TB) return tr_frag<BN>(Bb, wn * (BN / WN) + j * 32, kk * 16, lane);
      else return *reinterpret_cast<const bf16x8*>(&Bb[lds_idx<KB>(br + j * 32, kk * 16 + fk)]);
    };
    if constexpr (DMA && BM > 128 && KB == 64) {
      issue_next();
      bf16x8 af[2][FM], bf[2][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[0][i] = fa(i, 0);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[0][j] = fb(j, 0);
#pragma unroll
      for (int kk = 0; kk < KB / 16; ++kk) {
        const int cu = kk & 1;
        if (kk + 1 < KB / 16) {
#pragma unroll
          for (int i = 0; i < FM; ++i) af[cu ^ 1][i] = fa(i, kk + 1);
#pragma unroll
          for (int j = 0; j < FN; ++j) bf[cu ^ 1][j] = fb(j, kk + 1);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            mfma(acc[i][j], af[cu][i], bf[cu][j]);
      }
    } else if constexpr (PK) {
      // 4 slices of 32 codes per k-step; lane half h reads the slice's 8 bytes of
      // codes 16h .. 16h+15
      const int f4 = (lane >> 5) * 4;
      auto unpack = [](const uint16_t* p) -> bf16x8 {
        const u32x2 w = *reinterpret_cast<const u32x2*>(p);
        const u32x4 v = {w.x & 0x0f0f0f0fu, (w.x >> 4) & 0x0f0f0f0fu, w.y & 0x0f0f0f0fu,
                         (w.y >> 4) & 0x0f0f0f0fu};
        return __builtin_bit_cast(bf16x8, v);
      };
      bf16x8 af[4][FM], bf[4][FN];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[kk][i] = unpack(&Ab[lds_idx<32>(ar + i * 32, kk * 8 + f4)]);
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[kk][j] = unpack(&Bb[lds_idx<32>(br + j * 32, kk * 8 + f4)]);
      }
      issue_next();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            mfma(acc[i][j], af[kk][i], bf[kk][j]);
    } else {
      bf16x8 af[KB / 16][FM], bf[KB / 16][FN];
#pragma unroll
      for (int kk = 0; kk < KB / 16; ++kk) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[kk][i] = fa(i, kk);
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[kk][j] = fb(j, kk);
      }
      issue_next();
#pragma unroll
      for (int kk = 0; kk < KB / 16; ++kk)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            mfma(acc[i][j], af[kk][i], bf[kk][j]);
    }
    // the direct copies into the other buffer must land before the barrier
    if constexpr (DMA) {
      if (kt + 1 < nk) wait_vmem<0>();
    }
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
  if constexpr (EPI != 0) {
    // Straight-through backward of the row quantizer on the dL/dx_hat tile: the
    // accumulators are parked in LDS (the K loop ended on a barrier, so the operand
    // buffers are free), then each wave takes whole rows: it recomputes x~ and the
    // forward's in-range decision from x and the row's (h, z), reduces the per-row
    // partials (g_h, sum g (1 - in)) over the tile's 128 columns, accumulates the
    // per-column partials over its rows, and for token rows writes dL/dx (through
    // the LET) into C.  Rows go in batches of 8: the batch's gradients are read
    // from LDS first, its 8 rows are then independent chains of arithmetic, and
    // their partials are written last.
    float* T = reinterpret_cast<float*>(smem);     // [128][128] fp32
    const SteEpi& e = g.ste;
    const bool pass = e.nbits >= 16;
    const float Q = pass ? 0.f : (float)((1 << e.nbits) - 1);
    const bool colv = gn < N;
    // the T rows of this wave's pass
    const int tb0 = wid * RW;
    float ca0[2] = {0.f, 0.f}, ca1[2] = {0.f, 0.f};
#pragma unroll 1
    for (int hf = 0; hf < NPASS; ++hf) {
      wr0 = kOwnRows ? m0 + wid * (BM / WM) + hf * RW : m0 + wid * RW;
      // x of the first two batches, in flight while the accumulators are parked
      uint32_t x0[RB][XR], x1[RB][XR], x2[RB][XR];
      fetch_x(0, x0);
      fetch_x(1, x1);
      const int64_t rme = wr0 + (lane & (RW - 1));
      const bool rmv = rme < M;
      const int64_t hz = e.grouped ? rme * tiles_n + tn : rme;
      const float h_l = (!pass && rmv) ? e.h[hz] : 1.f;
      const float z_l = (!pass && rmv) ? e.z[hz] : 0.f;
      const float v_l = (e.rowvec && rmv) ? e.rowvec[rme] : 0.f;
      float s_c[2] = {1.f, 1.f}, d_c[2] = {0.f, 0.f};
      if (colv && kLet != kLetNone) { s_c[0] = e.s[gn]; s_c[1] = e.s[gn + 1]; }
      if (colv && kLet == kLetDiv && e.delta) {
        d_c[0] = e.delta[gn];
        d_c[1] = e.delta[gn + 1];
      }
      if constexpr (kOwnRows) {
        // this wave's 32 rows of the pass into its own T rows (read back only by
        // itself: LDS operations of one wave complete in order)
#pragma unroll
        for (int i = 0; i < FM; ++i)
          if (i == hf) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = tb0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                T[row * BN + j * 32 + (lane & 31)] = g.alpha * acc[i][j][r];
              }
          }
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = wm * (BM / WM) + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              const int col = wn * (BN / WN) + j * 32 + (lane & 31);
              T[row * BN + col] = g.alpha * acc[i][j][r];
            }
        __syncthreads();
      }
      const float r_c[2] = {1.f / s_c[0], 1.f / s_c[1]};
      const float rh_l = 1.f / h_l;
      // activation side: dL/dx is written unless the caller has no use for it (C null)
      float* Cp = g.C ? g.C + bz * g.strideC : nullptr;
#pragma unroll 1
      for (int b = 0; b < RW / RB; ++b) {
        if (wr0 + b * RB >= M) break;                // wave-uniform
        if (b + 2 < RW / RB) fetch_x(b + 2, x2);
        float gv[RB][2], xv[RB][2], xt[RB][2], xd[RB][2], u[RB][2], rr[RB][2];
        float hh[RB], zz[RB], vr[RB];
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          const float2 t =
              *reinterpret_cast<const float2*>(&T[(tb0 + b * RB + q) * BN + 2 * lane]);
          const bool ok = kFull || (colv && wr0 + b * RB + q < M);
          gv[q][0] = ok ? t.x : 0.f;
          gv[q][1] = ok ? t.y : 0.f;
        }
        // x~ and the rounding of x~ / h by the reciprocal product for every element
        // of the batch; an element whose product lies within |u| 2^-20 of a
        // half-integer takes the exact quotient below.  The batch test uses the
        // batch's bound: with f = u - rint u (exact, |f| <= 1/2), an element that
        // needs the exact quotient has 1/2 - |f| <= |u| 2^-20, so 1/2 - max|f| <=
        // max|u| 2^-20 too; the flagged batches then test each element.  (An
        // infinite u flags its batch through max|u|; a NaN u is passed over, its
        // exact quotient being NaN as well.)
        float fmx = 0.f, umx = 0.f;
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          const int rw = b * RB + q;
          hh[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h_l), rw));
          const float rhh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rh_l), rw));
          zz[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z_l), rw));
          vr[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v_l), rw));
          if constexpr (kXF) {
            xv[q][0] = __uint_as_float(x0[q][0]);
            xv[q][1] = __uint_as_float(x0[q][1]);
          } else {
            xv[q][0] = __uint_as_float(x0[q][0] << 16);
            xv[q][1] = __uint_as_float(x0[q][0] & 0xffff0000u);
          }
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            // x~: exact for MUL / NONE; for DIV within 2 ulp (it enters sums only; the
            // decisions follow the exact quotient)
            xd[q][c2] = xv[q][c2] - d_c[c2];
            if constexpr (kLet == kLetDiv) xt[q][c2] = xd[q][c2] * r_c[c2];
            else if constexpr (kLet == kLetMul) xt[q][c2] = s_c[c2] * xv[q][c2];
            else xt[q][c2] = xv[q][c2];
            u[q][c2] = xt[q][c2] * rhh;
            rr[q][c2] = rintf(u[q][c2]);
            fmx = fmaxf(fmx, fabsf(u[q][c2] - rr[q][c2]));
            umx = fmaxf(umx, fabsf(u[q][c2]));
          }
        }
        const bool near = !(0.5f - fmx > umx * 0x1p-20f);
        // (wave-uniform branches: divergent ones would be flattened into a division
        // for every element)
        if (!pass && __builtin_amdgcn_ballot_w64(near) != 0) {
#pragma unroll
          for (int q = 0; q < RB; ++q)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
              const bool ne =
                  !(fabsf(fabsf(u[q][c2] - rr[q][c2]) - 0.5f) > fabsf(u[q][c2]) * 0x1p-20f);
              if (__builtin_amdgcn_ballot_w64(ne) != 0) {
                if (ne) {
                  u[q][c2] = kLet == kLetDiv ? (xd[q][c2] / s_c[c2]) / hh[q] : xt[q][c2] / hh[q];
                  rr[q][c2] = rintf(u[q][c2]);
                }
              }
            }
        }
        float ph[RB], pz[RB];
#pragma unroll
        for (int q = 0; q < RB; ++q) {
          ph[q] = 0.f;
          pz[q] = 0.f;
          float up[2];
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2) {
            const float g1 = gv[q][c2];
            float gns = g1;
            if (!pass) {
              const float rq = rr[q][c2] + zz[q];
              const bool in = (rq >= 0.f) && (rq <= Q);
              const float qmz = fminf(fmaxf(rq, 0.f), Q) - zz[q];
              ph[q] += g1 * (qmz - (in ? u[q][c2] : 0.f));
              pz[q] += in ? 0.f : g1;
              gns = in ? g1 : 0.f;
            }
            if constexpr (kMode == 1 && kLet == kLetMul) {
              ca0[c2] += gns * xv[q][c2];
              ca1[c2] += vr[q] * xv[q][c2];
            } else if constexpr (kMode == 2 && kLet == kLetDiv) {
              ca0[c2] += gns * (-xt[q][c2] * r_c[c2]);
              ca1[c2] += gns * (-r_c[c2]);
            }
            up[c2] = kLet == kLetDiv ? gns * r_c[c2] : kLet == kLetMul ? gns * s_c[c2] : gns;
          }
          if constexpr (kMode == 2) {
            const int64_t gm = wr0 + b * RB + q;
            if (Cp && (kFull || (gm < M && colv)))
              *reinterpret_cast<float2*>(&Cp[gm * g.ldc + gn]) = make_float2(up[0], up[1]);
          }
        }
        if (!pass) {
          // the batch's gradients are consumed: its LDS rows now hold the lanes'
          // partials (g_h in columns 0..63, out-of-range sum in 64..127)
#pragma unroll
          for (int q = 0; q < RB; ++q) {
            float* tr = &T[(tb0 + b * RB + q) * BN];
            tr[lane] = ph[q];
            tr[64 + lane] = pz[q];
          }
        }
#pragma unroll
        for (int q = 0; q < RB; ++q)
#pragma unroll
          for (int w = 0; w < XR; ++w) {
            x0[q][w] = x1[q][w];
            x1[q][w] = x2[q][w];
          }
      }
      if (!pass) {
        // lane l sums row (l & 31)'s 64 partials of kind (l >> 5), starting at a
        // lane-dependent offset so the 64 lanes read 64 different banks
        const int rw = lane & 31, half = lane >> 5;
        const int64_t gm = wr0 + rw;
        if (gm < M) {
          const float* src = &T[(tb0 + rw) * BN + half * 64];
          float sum = 0.f;
#pragma unroll 16
          for (int j = 0; j < 64; ++j) sum += src[(j + lane) & 63];
          e.rowpart[(gm * tiles_n + tn) * 2 + half] = sum;
        }
      }
    }
    // column partials of each 128-row block: the four waves' sums (2 x 2 waves: one
    // block, all four; 4 x 1 waves: waves 2b and 2b+1 make block b), added in LDS in a
    // fixed order
    if constexpr ((kMode == 1 && kLet == kLetMul) || (kMode == 2 && kLet == kLetDiv)) {
      __syncthreads();                               // every wave is done reading T
      T[(wid * 2 + 0) * BN + 2 * lane] = ca0[0];
      T[(wid * 2 + 0) * BN + 2 * lane + 1] = ca0[1];
      T[(wid * 2 + 1) * BN + 2 * lane] = ca1[0];
      T[(wid * 2 + 1) * BN + 2 * lane + 1] = ca1[1];
      __syncthreads();
      constexpr int NB = BM / 128, WPB = 4 / NB;     // 128-row blocks, waves per block
      if (tid < BN * NB) {
        const int cc = tid % BN, bb = tid / BN;
        const int64_t c = n0 + cc;
        if (c < N) {
          float a0 = 0.f, a1 = 0.f;
#pragma unroll
          for (int w = 0; w < WPB; ++w) {
            a0 += T[((bb * WPB + w) * 2 + 0) * BN + cc];
            a1 += T[((bb * WPB + w) * 2 + 1) * BN + cc];
          }
          const int64_t tb = (int64_t)tm * NB + bb;
          e.colpart[(tb * 2 + 0) * N + c] = a0;
          e.colpart[(tb * 2 + 1) * N + c] = a1;
        }
      }
    }
    return;
  }
  float* C = g.C ? g.C + bz * g.strideC : nullptr;
  uint16_t* Cb = g.Cb ? g.Cb + bz * g.strideC : nullptr;
  // the lane's columns (one per 32-column block) and the first of its rows; a
  // lane holds rows row0 + 32 i + 8 (r / 4) + r % 4 of accumulator (i, j, r)
  int64_t gnj[FN];
  float bias[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    gnj[j] = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
    bias[j] = (g.bias && gnj[j] < N) ? g.bias[gnj[j]] : 0.f;
  }
  const int lr0 = wm * (BM / WM) + 4 * (lane >> 5);
  const int64_t row0 = m0 + lr0;
  // Integer codes: C = ha hb (S - zb Ra - za (Rb - K zb)) with S the integer sum of
  // code products and Ra, Rb the rows' code sums, i.e. sum_k (qa - za)(qb - zb)
  // (codes and zero points both shifted by the stored offsets; zero-code padding
  // adds nothing to S, Ra, Rb, and K is the unpadded length)
  // without rounding (every term an integer below 2^53), then one rounding to
  // float.  The rows' and columns' (h, z, code sum) go through LDS (the K loop
  // ended on a barrier, so the operand buffers are free).
  float* qs = reinterpret_cast<float*>(smem);      // [3][BM] rows, then [3][BN] columns
  double hb[FN], zb[FN], cb[FN];
  if constexpr (I8) {
    for (int t = tid; t < BM; t += NT) {
      const int64_t gm = m0 + t;
      const bool ok = gm < M;
      qs[t] = ok ? g.ha[gm] : 0.f;
      qs[BM + t] = ok ? g.za[gm] - g.zoa : 0.f;
      qs[2 * BM + t] = ok ? (float)g.sa[gm] : 0.f;
    }
    for (int t = tid; t < BN; t += NT) {
      const int64_t gn = n0 + t;
      const bool ok = gn < N;
      qs[3 * BM + t] = ok ? g.hb[gn] : 0.f;
      qs[3 * BM + BN + t] = ok ? g.zb[gn] - g.zob : 0.f;
      qs[3 * BM + 2 * BN + t] = ok ? (float)g.sb[gn] : 0.f;
    }
    __syncthreads();
    const double Kd = (double)(g.kz ? g.kz : g.K);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = wn * (BN / WN) + j * 32 + (lane & 31);
      hb[j] = (double)qs[3 * BM + col];
      zb[j] = (double)qs[3 * BM + BN + col];
      cb[j] = (double)qs[3 * BM + 2 * BN + col] - Kd * zb[j];
    }
  }
  // Whole tiles take every load and store of a 32-row slice without per-element
  // conditions, so each slice's residual (and accumulated C) reads are in flight
  // together; partial tiles check every element.
  const bool whole = m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    float v[FN][16];
    if constexpr (I8) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rb = lr0 + i * 32 + 8 * r4;
        const float4 h4 = *reinterpret_cast<const float4*>(&qs[rb]);
        const float4 z4 = *reinterpret_cast<const float4*>(&qs[BM + rb]);
        const float4 s4 = *reinterpret_cast<const float4*>(&qs[2 * BM + rb]);
        const float hr[4] = {h4.x, h4.y, h4.z, h4.w}, zr[4] = {z4.x, z4.y, z4.z, z4.w};
        const float sr[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const double S = (double)acc[i][j][4 * r4 + q];
            const double D = fma(-(double)zr[q], cb[j], fma(-zb[j], (double)sr[q], S));
            v[j][4 * r4 + q] = (float)(((double)hr[q] * hb[j]) * D) + bias[j];
          }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[j][r] = g.alpha * acc[i][j][r] + bias[j];
    }
    const int64_t ri = row0 + i * 32;
    auto roff = [](int r) { return 8 * (r >> 2) + (r & 3); };
    if (whole) {
      if (g.resid) {
        float rv[FN][16];
        if (g.resid_dt == OMQ_F32) {
          const float* R = reinterpret_cast<const float*>(g.resid) + ri * g.ldr;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) rv[j][r] = R[roff(r) * g.ldr + gnj[j]];
        } else {
          const uint16_t* R = reinterpret_cast<const uint16_t*>(g.resid) + ri * g.ldr;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) rv[j][r] = bf16_to_f32(R[roff(r) * g.ldr + gnj[j]]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) v[j][r] += rv[j][r];
      }
      if (Cb) {
        uint16_t* Cr = Cb + ri * g.ldc;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) Cr[roff(r) * g.ldc + gnj[j]] = f32_to_bf16(v[j][r]);
      } else {
        float* Cr = C + ri * g.ldc;
        if (g.accumulate) {
          float cv[FN][16];
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) cv[j][r] = Cr[roff(r) * g.ldc + gnj[j]];
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) v[j][r] += cv[j][r];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) Cr[roff(r) * g.ldc + gnj[j]] = v[j][r];
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t gn = gnj[j];
        if (gn >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t gm = ri + roff(r);
          if (gm >= M) continue;
          float x = v[j][r];
          if (g.resid) {
            x += g.resid_dt == OMQ_F32
                     ? reinterpret_cast<const float*>(g.resid)[gm * g.ldr + gn]
                     : bf16_to_f32(reinterpret_cast<const uint16_t*>(g.resid)[gm * g.ldr + gn]);
          }
          if (Cb) {
            Cb[gm * g.ldc + gn] = f32_to_bf16(x);
          } else {
            if (g.accumulate) x += C[gm * g.ldc + gn];
            C[gm * g.ldc + gn] = x;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
void launch_cfg(const Gemm& g, hipStream_t st) {
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)g.batch), block(WM * WN * 64);
  if (!g.ta && !g.tb)
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, 0, 0, 0, 0>), grid, block, 0, st, g, tiles_m,
                       tiles_n);
  else if (!g.ta && g.tb)
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, 0, 1, 0, 0>), grid, block, 0, st, g, tiles_m,
                       tiles_n);
  else if (g.ta && !g.tb)
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, 1, 0, 0, 0>), grid, block, 0, st, g, tiles_m,
                       tiles_n);
  else
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, 1, 1, 0, 0>), grid, block, 0, st, g, tiles_m,
                       tiles_n);
}

// every tile full: direct-to-LDS operand copies, for any operand layouts
template <int BM, int BN, int WM, int WN>
void launch_dma(const Gemm& g, hipStream_t st) {
  const int tiles_m = (int)(g.M / BM), tiles_n = (int)(g.N / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)g.batch), block(WM * WN * 64);
  if (!g.ta && !g.tb)
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, 0, 0, 0, 1>), grid, block, 0, st, g, tiles_m,
                       tiles_n);
  else if (!g.ta && g.tb)
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, 0, 1, 0, 1>), grid, block, 0, st, g, tiles_m,
                       tiles_n);
  else if (g.ta && !g.tb)
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, 1, 0, 0, 1>), grid, block, 0, st, g, tiles_m,
                       tiles_n);
  else
    hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, 1, 1, 0, 1>), grid, block, 0, st, g, tiles_m,
                       tiles_n);
}

// integer-code operands (K contiguous): direct copies when every tile is whole
template <int BM, int BN, int WM, int WN, int DMA>
void launch_codes(const Gemm& g, hipStream_t st) {
  const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)g.batch), block(WM * WN * 64);
  hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, 0, 0, 0, DMA, 1>), grid, block, 0, st, g,
                     tiles_m, tiles_n);
}

// Direct LDS copies need whole tiles (no bounds checks), whole K steps and 16-byte
// aligned rows.
bool dma_fits(const Gemm& g, int BM, int BN, int KB = BK) {
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  return g.M % BM == 0 && g.N % BN == 0 && g.K % KB == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 &&
         g.strideA % 8 == 0 && g.strideB % 8 == 0 && al16(g.A) && al16(g.B);
}

// the straight-through epilogue runs on 128 x 128 tiles of 4 waves (64-row blocks,
// 64-column slabs), for the two layouts the backward uses
constexpr int kSteBM = kSteTileRows, kSteBN = 128, kSteWM = 2, kSteWN = 2;

template <int EPI>
void launch_ste_x(const Gemm& g, hipStream_t st) {
  constexpr int TA = (EPI & 3) == 1;             // weight side: dY^T is the K-major A
  if constexpr (TA) {
    // weight rows (output channels) come in the thousands: 256 x 128 tiles of 4 waves
    // (each 64 whole rows) on 32-wide k steps read fewer LDS fragments per product
    // (both operands take the transposing read) and keep two workgroups per CU
    if (dma_fits(g, 256, 128, 32)) {
      const int tm = (int)(g.M / 256), tn = (int)(g.N / 128);
      hipLaunchKernelGGL((k_gemm_bf16<256, 128, 4, 1, 1, 1, EPI, 1, 0, 32>),
                         dim3((unsigned)(tm * tn), (unsigned)g.batch), dim3(256), 0, st, g, tm,
                         tn);
      return;
    }
  }
  const int tiles_m = (int)((g.M + kSteBM - 1) / kSteBM);
  const int tiles_n = (int)((g.N + kSteBN - 1) / kSteBN);
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)g.batch), block(kSteWM * kSteWN * 64);
  if (dma_fits(g, kSteBM, kSteBN))
    hipLaunchKernelGGL((k_gemm_bf16<kSteBM, kSteBN, kSteWM, kSteWN, TA, 1, EPI, 1>), grid, block, 0,
                       st, g, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((k_gemm_bf16<kSteBM, kSteBN, kSteWM, kSteWN, TA, 1, EPI, 0>), grid, block, 0,
                       st, g, tiles_m, tiles_n);
}

// The backward's two layouts: the weight side (dW = dY^T X^, both K-major, x = the
// bf16 weights, LET multiply with the scale's column partials, or no LET) and the
// activation side (dX = dY W^, W^ K-major, x = the activations, LET divide with the
// pair's column partials, or no LET).
hipError_t launch_ste(const Gemm& g, hipStream_t st) {
  const SteEpi& e = g.ste;
  const bool xf = e.x_dt == OMQ_F32;
  if (e.mode == 1 && g.ta && g.tb && !xf) {
    if (e.let_mode == OMQ_LET_MUL && e.col_mode == COL_WEIGHT)
      launch_ste_x<epi_code(1, kLetMul, 0)>(g, st);
    else if (e.let_mode == OMQ_LET_NONE && e.col_mode == COL_NONE)
      launch_ste_x<epi_code(1, kLetNone, 0)>(g, st);
    else
      return hipErrorInvalidValue;
  } else if (e.mode == 2 && !g.ta && g.tb) {
    if (e.let_mode == OMQ_LET_DIV && e.col_mode == COL_ACT_DIV) {
      if (xf) launch_ste_x<epi_code(2, kLetDiv, 1)>(g, st);
      else launch_ste_x<epi_code(2, kLetDiv, 0)>(g, st);
    } else if (e.let_mode == OMQ_LET_NONE && e.col_mode == COL_NONE) {
      if (xf) launch_ste_x<epi_code(2, kLetNone, 1)>(g, st);
      else launch_ste_x<epi_code(2, kLetNone, 0)>(g, st);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
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


}  // namespace

void gemm_ste_extents(int64_t rows, int64_t cols, int64_t* nslabs, int64_t* ntiles) {
  *nslabs = (cols + kSteBN - 1) / kSteBN;
  *ntiles = (rows + kSteBM - 1) / kSteBM;
}

// Integer codes: K and the leading dimensions in bytes, multiples of 16 (whole
// 16-byte chunks), rows 16-byte aligned; K up to 2^17 keeps every sum of code
// products in int32 and every code sum exact in float.  Tiles as for bf16, on the
// operands' 16-bit view.
hipError_t launch_gemm_codes(const Gemm& g, hipStream_t st) {
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (g.ta || g.tb || g.ste.mode || g.batch != 1) return hipErrorInvalidValue;
  if (g.K % 16 || g.lda % 16 || g.ldb % 16 || g.K > (1 << 17) || !al16(g.A) || !al16(g.B))
    return hipErrorInvalidValue;
  if (!g.ha || !g.za || !g.sa || !g.hb || !g.zb || !g.sb) return hipErrorInvalidValue;
  Gemm v = g;                                     // the 16-bit view
  v.K = g.K / 2;
  v.lda = g.lda / 2;
  v.ldb = g.ldb / 2;
  if (g.pack4) {
    // two codes to a byte: whole 128 x 128 tiles and 128-code k-steps, direct copies
    v.K = g.K / 4;
    if (g.K % 128 || g.M % 128 || g.N % 128 || g.zoa != 0.f || g.zob != 0.f ||
        g.lda * 2 < g.K || g.ldb * 2 < g.K || !dma_fits(v, 128, 128, 32))
      return hipErrorInvalidValue;
    const int tiles_m = (int)(g.M / 128), tiles_n = (int)(g.N / 128);
    hipLaunchKernelGGL((k_gemm_bf16<128, 128, 2, 2, 0, 0, 0, 1, 1, 32, 1>),
                       dim3((unsigned)(tiles_m * tiles_n), (unsigned)g.batch), dim3(256), 0, st, g,
                       tiles_m, tiles_n);
    return hipGetLastError();
  }
  const int64_t big_tiles = (g.M / 256) * (g.N / 256);
  if (big_tiles >= 512 && dma_fits(v, 256, 256))
    launch_codes<256, 256, 2, 4, 1>(g, st);
  else if (dma_fits(v, 128, 128))
    launch_codes<128, 128, 2, 2, 1>(g, st);
  else
    launch_codes<128, 128, 2, 2, 0>(g, st);
  return hipGetLastError();
}

hipError_t launch_gemm(const Gemm& g, hipStream_t st) {
  if (g.M == 0 || g.N == 0 || g.batch == 0) return hipSuccess;
  if (g.codes) return launch_gemm_codes(g, st);
  if (g.dt == OMQ_BF16 && g.ste.mode != 0) return launch_ste(g, st);
  if (g.dt == OMQ_BF16) {
    // 256 x 256 tiles halve the operand traffic per flop; they pay once there are
    // enough of them to keep every CU busy for two rounds
    const int64_t big_tiles = (g.M / 256) * (g.N / 256) * g.batch;
    if (big_tiles >= 512 && dma_fits(g, 256, 256))
      launch_dma<256, 256, 2, 4>(g, st);
    else if (dma_fits(g, 128, 128))
      launch_dma<128, 128, 2, 2>(g, st);
    else
      launch_cfg<128, 128, 2, 2>(g, st);
  } else {
    dim3 grid((unsigned)((g.N + 63) / 64), (unsigned)((g.M + 63) / 64), (unsigned)g.batch);
    hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace omq
