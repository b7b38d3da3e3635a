// Causal attention of the quantized block, fused on gfx950 (paper reading,
// section "LET": the affinity Q~ K~^T with s_a folded into the quantized Q^ and K^
// that arrive here; the softmax output is never quantized and stays float32 up to
// its bf16 rounding as a matrix-core operand).
//
// Head dimension 128, causal mask, grouped K/V heads (query head h reads K/V head
// h / grp).  Scores and probabilities never reach HBM: the forward keeps a running
// max and sum per query (exp2 domain) and writes O and the row's log-sum-exp; the
// backward's dK/dV pass recomputes the scores from that log-sum-exp and writes the
// bf16 dS it forms, which the dQ pass reads back.
//
// MFMA 32x32x16 bf16 layouts.  A lane of the instruction supplies 8 consecutive k
// of one row (A) or one column (B) and receives a column of C: col = lane & 31,
// rows 8*(r/4) + 4*(lane/32) + (r%4), r = 0..15.  Every product here is arranged
// so that the C tile of one step is the B operand of the next without moving data
// between lanes: a C tile whose columns are indexed by lane is re-read as B with
// its rows as k.  Those rows come in the order 16s + {0..3, 8..11} + 4*(lane/32)
// within a 16-wide k slice s, so the A operand of that product is read from LDS in
// the same order: from a transposed copy (tt_frag, the forward's V) or by transposing
// reads of the row tile itself (rt_tr_frag, the backward's Q, dO and K, whose row
// tiles the backward reads as well).
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace omq {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
// native vectors (HIP's uint4 is a struct whose copies can keep a stack object alive)
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int HD = 128;             // head dimension
constexpr int kT = 256;             // threads per block (4 waves)

OMQ_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row tile [R][128] bf16 with rows padded to 136 elements (272 bytes): 8 lanes
// reading the same 16-byte chunk of 8 consecutive rows land 16 bytes apart modulo
// 128, i.e. in 8 distinct bank groups, and a fragment's address is the row base
// plus an immediate offset.
constexpr int RS = HD + 8;
OMQ_DEV int rt_idx(int r, int c) { return r * RS + (c << 3); }

// Transposed tile [128][64] bf16 (64 positions per row): the 8-byte chunk q (4
// positions) of row r sits at q ^ ((r & 15) ^ (r >> 4)); 16 lanes reading chunk q of
// 16 consecutive rows, and the staging writes (rows 8c + j for c = 0..15), both
// spread over 16 distinct chunks.
OMQ_DEV int tt_idx(int r, int q) { return r * 64 + ((q ^ ((r & 15) ^ (r >> 4))) << 2); }

// A-operand fragment of a row tile: row r, k slice s (16 wide), lane half h.
OMQ_DEV bf16x8 rt_frag(const uint16_t* t, int r, int s, int h) {
  return *reinterpret_cast<const bf16x8*>(&t[rt_idx(r, 2 * s + h)]);
}

// A-operand fragment of a transposed tile in C-row order: positions
// 16s + 4h + {0..3} and 16s + 8 + 4h + {0..3} of row r.
OMQ_DEV bf16x8 tt_frag(const uint16_t* t, int r, int s, int h) {
  const u32x2 lo = *reinterpret_cast<const u32x2*>(&t[tt_idx(r, 4 * s + h)]);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(&t[tt_idx(r, 4 * s + 2 + h)]);
  const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(bf16x8, v);
}

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// A-operand fragment of the transposed view of a row tile, in C-row order: fragment
// row rb + (lane & 31) is tile column rb + (lane & 31), its k positions are tile rows
// 16s + 4h + {0..3} and 16s + 8 + 4h + {0..3}.  Two transposing LDS reads
// (ds_read_b64_tr_b16): in each 16-lane group, lane 4j + q addresses tile row
// k + j, columns 4q .. 4q+3 of the group's 16 columns, and lane i receives the 4
// rows k .. k+3 of column i.  (The 272-byte rows put the 4 rows of one read 16 bytes
// apart modulo 256, a 2-way bank overlap the fragment reads along rows avoid.)
// The same read with the lane's 4-column group given by its LDS column `col` (a tile
// whose groups of 4 columns are stored in another order).
template <int STRIDE = RS>
OMQ_DEV bf16x8 rt_tr_frag_at(const uint16_t* t, int col, int s, int lane) {
  const int G = lane >> 4, j = (lane >> 2) & 3;
  const int k = 16 * s + 4 * (G >> 1) + j;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + k * STRIDE + col));
  const i16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + (k + 8) * STRIDE + col));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <int STRIDE = RS>
OMQ_DEV bf16x8 rt_tr_frag(const uint16_t* t, int rb, int s, int lane) {
  const int G = lane >> 4, q = lane & 3;
  return rt_tr_frag_at<STRIDE>(t, rb + 16 * (G & 1) + 4 * q, s, lane);
}

// Stored dS rows (one key, the queries of 64-query blocks): query 16s + 8b + 4h + i of
// a block sits at 32h + 8s + 4b + i, so that the dK/dV pass's lane (key, h) writes its
// 32 values (C-row order) as 64 contiguous bytes.  Position of the 4-query group
// starting at query n (a multiple of 4) of a row:
OMQ_DEV int ds_pos(int n) {
  const int m = n & 63;
  return (n & ~63) + 32 * ((m >> 2) & 1) + 8 * (m >> 4) + 4 * ((m >> 3) & 1);
}

// 8 consecutive C values r0..r0+7 of one tile as a B-operand fragment
OMQ_DEV bf16x8 c_frag(const f32x16& c, int r0) {
  const u32x4 v = {pack_bf16(c[r0 + 0], c[r0 + 1]), pack_bf16(c[r0 + 2], c[r0 + 3]),
                   pack_bf16(c[r0 + 4], c[r0 + 5]), pack_bf16(c[r0 + 6], c[r0 + 7])};
  return __builtin_bit_cast(bf16x8, v);
}

// One thread's staging unit of a 64-row block of a [rows x ld] bf16 matrix: rows
// 4kq .. 4kq+3 (kq = tid >> 4) at 16-byte column chunk c = tid & 15.  Rows past
// `rows` are clamped to the last one (in bounds; the callers mask their results).
struct Unit {
  u32x4 v0, v1, v2, v3;     // rows 4kq + 0..3
  OMQ_DEV void load(const uint16_t* P, int64_t ld, int64_t col0, int64_t row0, int64_t rows,
                    int tid) {
    const int kq = tid >> 4, c = tid & 15;
    const int64_t r = row0 + 4 * kq;
    const uint16_t* b = P + col0 + 8 * c;
    v0 = *reinterpret_cast<const u32x4*>(b + min(r + 0, rows - 1) * ld);
    v1 = *reinterpret_cast<const u32x4*>(b + min(r + 1, rows - 1) * ld);
    v2 = *reinterpret_cast<const u32x4*>(b + min(r + 2, rows - 1) * ld);
    v3 = *reinterpret_cast<const u32x4*>(b + min(r + 3, rows - 1) * ld);
  }
  template <int STRIDE = RS>
  OMQ_DEV void store_rows(uint16_t* t, int tid) const {
    const int kq = tid >> 4, c = tid & 15;
    *reinterpret_cast<u32x4*>(&t[(4 * kq + 0) * STRIDE + 8 * c]) = v0;
    *reinterpret_cast<u32x4*>(&t[(4 * kq + 1) * STRIDE + 8 * c]) = v1;
    *reinterpret_cast<u32x4*>(&t[(4 * kq + 2) * STRIDE + 8 * c]) = v2;
    *reinterpret_cast<u32x4*>(&t[(4 * kq + 3) * STRIDE + 8 * c]) = v3;
  }
  // the same 4 x 8 block written transposed: 8 rows (columns 8c + j) of 4 positions
  OMQ_DEV void store_transposed(uint16_t* t, int tid) const {
    const int kq = tid >> 4, c = tid & 15;
    tr2(t, 8 * c + 0, kq, v0.x, v1.x, v2.x, v3.x, 0x05040100u);
    tr2(t, 8 * c + 1, kq, v0.x, v1.x, v2.x, v3.x, 0x07060302u);
    tr2(t, 8 * c + 2, kq, v0.y, v1.y, v2.y, v3.y, 0x05040100u);
    tr2(t, 8 * c + 3, kq, v0.y, v1.y, v2.y, v3.y, 0x07060302u);
    tr2(t, 8 * c + 4, kq, v0.z, v1.z, v2.z, v3.z, 0x05040100u);
    tr2(t, 8 * c + 5, kq, v0.z, v1.z, v2.z, v3.z, 0x07060302u);
    tr2(t, 8 * c + 6, kq, v0.w, v1.w, v2.w, v3.w, 0x05040100u);
    tr2(t, 8 * c + 7, kq, v0.w, v1.w, v2.w, v3.w, 0x07060302u);
  }
  // one bf16 of each of the 4 rows (low or high half of the words, per sel) as the
  // 4 consecutive positions of transposed row r
  static OMQ_DEV void tr2(uint16_t* t, int r, int kq, uint32_t a0, uint32_t a1, uint32_t a2,
                          uint32_t a3, uint32_t sel) {
    const u32x2 o = {__builtin_amdgcn_perm(a1, a0, sel), __builtin_amdgcn_perm(a3, a2, sel)};
    *reinterpret_cast<u32x2*>(&t[tt_idx(r, kq)]) = o;
  }
};

constexpr float kNegInf = -__builtin_huge_valf();

// paired causal blocks (a long and a short key block per workgroup, dK/dV) are
// used when that still leaves at least one workgroup per compute unit
constexpr int64_t kPairMinBlocks = 256;

// The query-stationary kernels (forward, dQ) take one 128-query unit per workgroup
// and fit two waves per SIMD (two workgroups per compute unit).  Under the causal
// mask a unit's work grows with its position, so the grid is ordered by unit size:
// workgroup b < half takes query block nqb-1-v (v = b / heads) and workgroup
// b + half takes block v of the same head, where half = ceil(nqb/2) * heads.  The
// dispatcher fills the second slot of each compute unit in the same order as the
// first, so a long and a short unit share a compute unit (equal work per unit in
// one round on the 7B and 70B shapes); with more rounds the longest run first.
OMQ_DEV void query_unit(int heads, int nqb, int& hq, int& qb) {
  const int v = blockIdx.x / heads, half = (nqb + 1) / 2;
  hq = blockIdx.x % heads;
  qb = v < half ? nqb - 1 - v : v - half;
}

// 2^x on the transcendental unit (no denormal rescaling: results below 2^-126 are
// probabilities that vanish against the row sum anyway)
OMQ_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// forward: block = (query head, 128 queries); wave w owns queries q0 + 32w + 0..31,
// one per lane (both lane halves hold the same query).  Two passes over the keys
// in 64-key blocks, S^T = K Q^T each time (A = K rows from LDS, B = Q from
// registers):
//   1. running max and sum of exp2 per query -> the log-sum-exp lse2;
//   2. P = exp2(S c - lse2), already normalized, rounded to bf16 as the P V
//      operand (the same rounding of the same normalized probabilities as a
//      two-step softmax, and as the backward's recomputation), O^T += V^T P^T
//      (A = V^T from LDS, B = P from registers).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(2)))
void k_flash_fwd(FlashFwd a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][HD * 64];
  const int64_t T = a.T;
  const int nqb = (int)((T + 127) / 128);
  int hq, qb;
  query_unit(a.n_q, nqb, hq, qb);
  const int hk = hq / a.grp;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), h = lane >> 5, l32 = lane & 31;
  {
    const int64_t q0 = (int64_t)qb * 128;
    const int64_t q = q0 + 32 * w + l32;
    const int64_t qc = min(q, T - 1);

    bf16x8 qf[8];
  #pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(a.Q + qc * a.ldq + hq * HD + 16 * s + 8 * h);

    const int64_t kend = min(q0 + 128, T);
    const int nkb = (int)((kend + 63) / 64);
    // unscaled scores of key block kb for this lane's query, masked to -inf (the
    // mask runs only on the blocks that cross the diagonal or the end, one
    // wave-uniform branch per block)
    auto scores = [&](const uint16_t* Kb, int kb, f32x16 (&sc)[2]) {
  #pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
  #pragma unroll
        for (int r = 0; r < 16; ++r) sc[kk][r] = 0.f;
  #pragma unroll
        for (int s = 0; s < 8; ++s) sc[kk] = mfma(rt_frag(Kb, 32 * kk + l32, s, h), qf[s], sc[kk]);
      }
      const int k0 = kb * 64;
      if (k0 + 63 > (int)q0 + 32 * w || k0 + 64 > (int)T) {   // wave-uniform
        const int qi = (int)q, Ti = (int)T;
  #pragma unroll
        for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kk + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key > qi || key >= Ti) sc[kk][r] = kNegInf;
          }
      }
    };

    // pass 1: log-sum-exp
    Unit uk, uv;
    uk.load(a.K, a.ldk, hk * HD, 0, T, tid);
    uk.store_rows(Ks[0], tid);
    if (nkb > 1) uk.load(a.K, a.ldk, hk * HD, 64, T, tid);
    __syncthreads();
    float m2 = kNegInf, l = 0.f;
    for (int kb = 0; kb < nkb; ++kb) {
      const int buf = kb & 1;
      f32x16 sc[2];
      scores(Ks[buf], kb, sc);
      if (kb + 1 < nkb) {
        uk.store_rows(Ks[buf ^ 1], tid);
        if (kb + 2 < nkb) uk.load(a.K, a.ldk, hk * HD, (int64_t)(kb + 2) * 64, T, tid);
      }
      // the running max in the scaled (exp2) domain: the largest scaled score is the
      // largest unscaled one times c (rounding is monotonic)
      float mx = kNegInf;
  #pragma unroll
      for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kk][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.scale2;
      const float mn = fmaxf(m2, mx);
      const float ms = mn == kNegInf ? 0.f : mn;
      float add = 0.f;
  #pragma unroll
      for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
        for (int r = 0; r < 16; ++r) add += fast_exp2(fmaf(sc[kk][r], a.scale2, -ms));
      l = l * fast_exp2(m2 - ms) + add;
      m2 = mn;
      __syncthreads();
    }
    l += __shfl_xor(l, 32, 64);
    const float lse2 = m2 + log2f(l);

    // pass 2: normalized probabilities into O^T += V^T P^T
    uk.load(a.K, a.ldk, hk * HD, 0, T, tid);
    uv.load(a.V, a.ldk, hk * HD, 0, T, tid);
    uk.store_rows(Ks[0], tid);
    uv.store_transposed(Vt[0], tid);
    if (nkb > 1) {
      uk.load(a.K, a.ldk, hk * HD, 64, T, tid);
      uv.load(a.V, a.ldk, hk * HD, 64, T, tid);
    }
    __syncthreads();
    f32x16 o[4];
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
    for (int kb = 0; kb < nkb; ++kb) {
      const int buf = kb & 1;
      f32x16 sc[2];
      scores(Ks[buf], kb, sc);
      if (kb + 1 < nkb) {
        uk.store_rows(Ks[buf ^ 1], tid);
        uv.store_transposed(Vt[buf ^ 1], tid);
        if (kb + 2 < nkb) {
          uk.load(a.K, a.ldk, hk * HD, (int64_t)(kb + 2) * 64, T, tid);
          uv.load(a.V, a.ldk, hk * HD, (int64_t)(kb + 2) * 64, T, tid);
        }
      }
  #pragma unroll
      for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
        for (int r = 0; r < 16; ++r) sc[kk][r] = fast_exp2(fmaf(sc[kk][r], a.scale2, -lse2));
      bf16x8 pf[4];
  #pragma unroll
      for (int s = 0; s < 4; ++s) pf[s] = c_frag(sc[s >> 1], 8 * (s & 1));
  #pragma unroll
      for (int hb = 0; hb < 4; ++hb)
  #pragma unroll
        for (int s = 0; s < 4; ++s) o[hb] = mfma(tt_frag(Vt[buf], 32 * hb + l32, s, h), pf[s], o[hb]);
      __syncthreads();
    }
    if (q < T) {
      float* orow = a.O + q * a.ldo + hq * HD;
  #pragma unroll
      for (int hb = 0; hb < 4; ++hb)
  #pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(orow + 32 * hb + 8 * g + 4 * h) =
              make_float4(o[hb][4 * g], o[hb][4 * g + 1], o[hb][4 * g + 2], o[hb][4 * g + 3]);
      if (h == 0) a.lse2[(int64_t)hq * T + q] = lse2;
    }
  }
}

// ---------------------------------------------------------------------------
// backward prologue: D = rowsum(dO * O) per (head, query) and dO in bf16
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void k_attn_bwd_prep(const float* gO, const float* O, int64_t ld,
                                                      int64_t T, int n_q, float* D, uint16_t* gOb,
                                                      int64_t ldb) {
  const int64_t q = blockIdx.x;
  const int n4 = n_q * (HD / 4);
  for (int base = 0; base < n4; base += kT) {
    const int idx = base + threadIdx.x;        // n4 is a multiple of 32: whole half-waves
    float dot = 0.f;
    if (idx < n4) {
      const float4 g = *reinterpret_cast<const float4*>(gO + q * ld + 4 * idx);
      const float4 o = *reinterpret_cast<const float4*>(O + q * ld + 4 * idx);
      dot = g.x * o.x + g.y * o.y + g.z * o.z + g.w * o.w;
      *reinterpret_cast<uint2*>(gOb + q * ldb + 4 * idx) =
          make_uint2(pack_bf16(g.x, g.y), pack_bf16(g.z, g.w));
    }
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (idx < n4 && (idx & 31) == 0) D[(int64_t)(idx >> 5) * T + q] = dot;
  }
}

// ---------------------------------------------------------------------------
// backward, keys stationary: block = (K/V head, 128 keys); wave w owns keys
// k0 + 32w + 0..31, one per lane.  Over every query head of the group and every
// 64-query block at or after the keys: S = Q K^T and dP = dO V^T (A = Q / dO rows
// from LDS, B = K / V from registers), P = exp2(S c - lse2), dS = P (dP - D) / sqrt(hd),
// dV^T += dO^T P and dK^T += Q^T dS (A = transposed Q / dO from LDS, B = P / dS).
// The bf16 dS of every (query, key) it forms goes to a.ds for the dQ pass.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void k_flash_bwd_dkdv(FlashBwd a, int pair, int nsplit) {
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[2][64 * RS];
  __shared__ __attribute__((aligned(16))) float Ls[2][64];
  __shared__ __attribute__((aligned(16))) float Ds[2][64];
  const int64_t T = a.T, Tp = (T + 127) / 128 * 128;
  const int nkb = (int)((T + 127) / 128);
  // pair: key blocks p and then nkb-1-p (equal causal work per block); else key
  // block p alone (kb = 0, the longest, first).  Workgroup (g, sp, p) covers query
  // heads sp*gh .. sp*gh + gh-1 of K/V head g's group; split 0 writes dK, dV, the
  // others their own partial slices, added in split order afterwards.
  const int npb = pair ? (nkb + 1) / 2 : nkb;
  const int p = (int)(blockIdx.x % npb);
  const int g = (int)(blockIdx.x / npb) / nsplit;
  const int sp = (int)(blockIdx.x / npb) % nsplit;
  const int gh = a.grp / nsplit;
  const int64_t ldp = (int64_t)(a.n_q / a.grp) * HD;
  float* const oK = sp == 0 ? a.dK : a.part + (int64_t)(sp - 1) * 2 * T * ldp;
  float* const oV = sp == 0 ? a.dV : oK + T * ldp;
  const int64_t ldo = sp == 0 ? a.lddk : ldp;
  const int nunits = (pair && p != nkb - 1 - p) ? 2 : 1;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), h = lane >> 5, l32 = lane & 31;
  for (int u = 0; u < nunits; ++u) {
    const int kb = u == 0 ? p : nkb - 1 - p;
    if (u > 0) __syncthreads();                          // LDS of the previous unit
    const int64_t k0 = (int64_t)kb * 128;
    const int64_t key = k0 + 32 * w + l32;
    const int64_t kc = min(key, T - 1);

    bf16x8 kf[8], vf[8];
  #pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = *reinterpret_cast<const bf16x8*>(a.K + kc * a.ldk + g * HD + 16 * s + 8 * h);
      vf[s] = *reinterpret_cast<const bf16x8*>(a.V + kc * a.ldk + g * HD + 16 * s + 8 * h);
    }
    const int nqb = (int)((T + 63) / 64);
    const int qb0 = (int)(k0 / 64);
    const int per = nqb - qb0;                              // query blocks per head
    const int nit = per * gh;
    auto qbase = [&](int it, int& hq) -> int64_t {
      hq = g * a.grp + sp * gh + it / per;
      return (int64_t)(qb0 + it % per) * 64;
    };

    Unit uq, ug;
    float lv = 0.f, dv = 0.f;
    auto load = [&](int it) {
      int hq;
      const int64_t q0 = qbase(it, hq);
      uq.load(a.Q, a.ldq, hq * HD, q0, T, tid);
      ug.load(a.dO, a.ldq, hq * HD, q0, T, tid);
      if (tid < 64) {
        const int64_t qq = min(q0 + tid, T - 1);
        lv = a.lse2[(int64_t)hq * T + qq];
        dv = a.D[(int64_t)hq * T + qq];
      }
    };
    auto store = [&](int buf) {
      uq.store_rows(Qs[buf], tid);
      ug.store_rows(Gs[buf], tid);
      if (tid < 64) {
        Ls[buf][tid] = lv;
        Ds[buf][tid] = dv;
      }
    };
    if (nit > 0) {
      load(0);
      store(0);
      if (nit > 1) load(1);
    }
    __syncthreads();

    f32x16 dk[4], dvt[4];
  #pragma unroll
    for (int i = 0; i < 4; ++i)
  #pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[i][r] = 0.f;
        dvt[i][r] = 0.f;
      }
    for (int it = 0; it < nit; ++it) {
      const int buf = it & 1;
      int hq;
      const int64_t q0 = qbase(it, hq);
      f32x16 sc[2], dp[2];
  #pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[mb][r] = 0.f;
          dp[mb][r] = 0.f;
        }
  #pragma unroll
        for (int s = 0; s < 8; ++s) {
          sc[mb] = mfma(rt_frag(Qs[buf], 32 * mb + l32, s, h), kf[s], sc[mb]);
          dp[mb] = mfma(rt_frag(Gs[buf], 32 * mb + l32, s, h), vf[s], dp[mb]);
        }
      }
      if (it + 1 < nit) {
        store(buf ^ 1);
        if (it + 2 < nit) load(it + 2);
      }
      // P from the forward's log-sum-exp (the forward's own formula), masked on the
      // blocks that cross the diagonal or the end (one block-uniform branch)
  #pragma unroll
      for (int mb = 0; mb < 2; ++mb)
  #pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int row0 = 32 * mb + 8 * gg + 4 * h;
          const float4 L4 = *reinterpret_cast<const float4*>(&Ls[buf][row0]);
          const float Lr[4] = {L4.x, L4.y, L4.z, L4.w};
  #pragma unroll
          for (int c = 0; c < 4; ++c)
            sc[mb][4 * gg + c] = fast_exp2(fmaf(sc[mb][4 * gg + c], a.scale2, -Lr[c]));
        }
      if ((int)q0 < (int)k0 + 127 || (int)q0 + 64 > (int)T) {
        const int ki = (int)key, Ti = (int)T;
  #pragma unroll
        for (int mb = 0; mb < 2; ++mb)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qr = (int)q0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
            if (ki > qr || qr >= Ti) sc[mb][r] = 0.f;
          }
      }
  #pragma unroll
      for (int mb = 0; mb < 2; ++mb)
  #pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int row0 = 32 * mb + 8 * gg + 4 * h;
          const float4 D4 = *reinterpret_cast<const float4*>(&Ds[buf][row0]);
          const float Dr[4] = {D4.x, D4.y, D4.z, D4.w};
  #pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = 4 * gg + c;
            dp[mb][r] = sc[mb][r] * (dp[mb][r] - Dr[c]) * a.scale;
          }
        }
      bf16x8 pf[4], sf[4];
  #pragma unroll
      for (int s = 0; s < 4; ++s) {
        pf[s] = c_frag(sc[s >> 1], 8 * (s & 1));
        sf[s] = c_frag(dp[s >> 1], 8 * (s & 1));
      }
      // dS as rounded here, kept for the dQ pass: the lane's key row, queries
      // q0 + 16s + 4h + {0..3} and q0 + 16s + 8 + 4h + {0..3} (zero where masked), at
      // q0 + 32h + 8s + {0..7} (ds_pos)
      {
        uint16_t* drow = a.ds + ((int64_t)hq * Tp + key) * Tp + q0 + 32 * h;
  #pragma unroll
        for (int s = 0; s < 4; ++s)
          *reinterpret_cast<u32x4*>(drow + 8 * s) = __builtin_bit_cast(u32x4, sf[s]);
      }
  #pragma unroll
      for (int hb = 0; hb < 4; ++hb)
  #pragma unroll
        for (int s = 0; s < 4; ++s) {
          dvt[hb] = mfma(rt_tr_frag(Gs[buf], 32 * hb, s, lane), pf[s], dvt[hb]);
          dk[hb] = mfma(rt_tr_frag(Qs[buf], 32 * hb, s, lane), sf[s], dk[hb]);
        }
      __syncthreads();
    }
    if (key < T) {
      float* krow = oK + key * ldo + g * HD;
      float* vrow = oV + key * ldo + g * HD;
  #pragma unroll
      for (int hb = 0; hb < 4; ++hb)
  #pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int c = 32 * hb + 8 * gg + 4 * h;
          *reinterpret_cast<float4*>(krow + c) =
              make_float4(dk[hb][4 * gg], dk[hb][4 * gg + 1], dk[hb][4 * gg + 2], dk[hb][4 * gg + 3]);
          *reinterpret_cast<float4*>(vrow + c) = make_float4(dvt[hb][4 * gg], dvt[hb][4 * gg + 1],
                                                             dvt[hb][4 * gg + 2], dvt[hb][4 * gg + 3]);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// backward, queries stationary: block = (query head, 128 queries); per 64-key block
// dQ^T += K^T dS^T (A = transposed K rows from LDS, B = the stored dS read
// transposed from LDS, each lane at its query group's stored position: lane = query,
// k = keys), so the scores are not formed again.
// The dS tile [64 keys][128 queries] of every key block at or before the queries was
// written by the dK/dV pass (zeros where the mask applies); its columns past T, and
// K rows clamped to T - 1, meet only zeros or outputs that are not stored.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(2)))
void k_flash_bwd_dq(FlashBwd a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t Ss[2][64 * RS];
  const int64_t T = a.T, Tp = (T + 127) / 128 * 128;
  const int nqb = (int)((T + 127) / 128);
  int hq, qb;
  query_unit(a.n_q, nqb, hq, qb);
  const int hk = hq / a.grp;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), h = lane >> 5, l32 = lane & 31;
  const int64_t q0 = (int64_t)qb * 128;
  const int64_t q = q0 + 32 * w + l32;
  const uint16_t* Sh = a.ds + (int64_t)hq * Tp * Tp;
  const int nkb = (int)((min(q0 + 128, T) + 63) / 64);
  // the lane's 4-query group of the stored dS rows (B operand: lane = query)
  const int pc = ds_pos(32 * w + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  Unit uk, us;
  uk.load(a.K, a.ldk, hk * HD, 0, T, tid);
  us.load(Sh, Tp, q0, 0, Tp, tid);
  uk.store_rows(Ks[0], tid);
  us.store_rows(Ss[0], tid);
  if (nkb > 1) {
    uk.load(a.K, a.ldk, hk * HD, 64, T, tid);
    us.load(Sh, Tp, q0, 64, Tp, tid);
  }
  __syncthreads();

  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.f;
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    bf16x8 sf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) sf[s] = rt_tr_frag_at(Ss[buf], pc, s, lane);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int s = 0; s < 4; ++s) dq[hb] = mfma(rt_tr_frag(Ks[buf], 32 * hb, s, lane), sf[s], dq[hb]);
    if (kb + 1 < nkb) {
      uk.store_rows(Ks[buf ^ 1], tid);
      us.store_rows(Ss[buf ^ 1], tid);
      if (kb + 2 < nkb) {
        uk.load(a.K, a.ldk, hk * HD, (int64_t)(kb + 2) * 64, T, tid);
        us.load(Sh, Tp, q0, (int64_t)(kb + 2) * 64, Tp, tid);
      }
    }
    __syncthreads();
  }
  if (q < T) {
    float* qrow = a.dQ + q * a.lddq + hq * HD;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        *reinterpret_cast<float4*>(qrow + 32 * hb + 8 * gg + 4 * h) =
            make_float4(dq[hb][4 * gg], dq[hb][4 * gg + 1], dq[hb][4 * gg + 2], dq[hb][4 * gg + 3]);
  }
}

// dK, dV += the partial slices of splits 1 .. nsplit-1, added in that order (float4
// units; ldp, a multiple of 128, is the row length of every slice)
__global__ __launch_bounds__(kT) void k_kv_part_add(float* dK, float* dV, int64_t lddk,
                                                    const float* part, int64_t T, int64_t ldp,
                                                    int nsplit) {
  const int64_t n4 = T * ldp / 4;
  for (int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x; i < 2 * n4;
       i += (int64_t)gridDim.x * kT) {
    const int which = i >= n4;                   // 0: dK, 1: dV
    const int64_t j = i - which * n4, t = j / (ldp / 4), c = 4 * (j % (ldp / 4));
    float* o = (which ? dV : dK) + t * lddk + c;
    float4 acc = *reinterpret_cast<const float4*>(o);
    for (int sp = 1; sp < nsplit; ++sp) {
      const float4 v = *reinterpret_cast<const float4*>(
          part + ((int64_t)(sp - 1) * 2 + which) * T * ldp + t * ldp + c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4*>(o) = acc;
  }
}

}  // namespace

// The dK/dV grid has npb workgroups per K/V head (paired key blocks).  When the K/V
// heads alone leave compute units without a workgroup, each group's query heads
// are split over the smallest divisor of the group size that fills the device.
int flash_bwd_splits(int64_t T, int n_q, int n_kv) {
  if (T <= 0 || n_q <= 0 || n_kv <= 0 || n_q % n_kv) return 1;
  const int64_t npb = ((T + 127) / 128 + 1) / 2;
  const int grp = n_q / n_kv;
  for (int s = 1; s < grp; ++s)
    if (grp % s == 0 && npb * n_kv * s >= kPairMinBlocks) return s;
  return grp;
}

int64_t flash_bwd_part_floats(int64_t T, int n_q, int n_kv) {
  return (int64_t)(flash_bwd_splits(T, n_q, n_kv) - 1) * 2 * T * n_kv * HD;
}

int64_t flash_bwd_ds_elems(int64_t T, int64_t n_q) {
  if (T < 0 || n_q < 0) return -1;
  const int64_t Tp = (T + 127) / 128 * 128;
  if (Tp > ((int64_t)1 << 25) || (Tp && n_q > ((int64_t)1 << 50) / Tp / Tp)) return -1;
  return n_q * Tp * Tp;
}

hipError_t launch_flash_fwd(const FlashFwd& a, hipStream_t st) {
  if (a.T == 0 || a.n_q == 0) return hipSuccess;
  if (a.T > (int64_t)1 << 30) return hipErrorInvalidValue;    // positions are 32-bit
  const int nqb = (int)((a.T + 127) / 128);
  hipLaunchKernelGGL(k_flash_fwd, dim3((unsigned)(nqb * a.n_q)), dim3(kT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_prep(const float* gO, const float* O, int64_t ld, int64_t T, int n_q,
                                float* D, uint16_t* gOb, int64_t ldb, hipStream_t st) {
  if (T == 0 || n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(k_attn_bwd_prep, dim3((unsigned)T), dim3(kT), 0, st, gO, O, ld, T, n_q, D,
                     gOb, ldb);
  return hipGetLastError();
}

hipError_t launch_flash_bwd(const FlashBwd& a, hipStream_t st) {
  if (a.T == 0 || a.n_q == 0) return hipSuccess;
  if (a.T > (int64_t)1 << 30) return hipErrorInvalidValue;    // positions are 32-bit
  const int nkb = (int)((a.T + 127) / 128);
  const int npb = (nkb + 1) / 2;
  const int n_kv = a.n_q / a.grp;
  const int ns = flash_bwd_splits(a.T, a.n_q, n_kv);
  if ((ns > 1 && !a.part) || !a.ds) return hipErrorInvalidValue;
  const int pair_kv = (int64_t)npb * n_kv * ns >= kPairMinBlocks;
  hipLaunchKernelGGL(k_flash_bwd_dkdv, dim3((unsigned)((pair_kv ? npb : nkb) * n_kv * ns)),
                     dim3(kT), 0, st, a, pair_kv, ns);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ns > 1) {
    const int64_t ldp = (int64_t)n_kv * HD;
    const int64_t n4 = 2 * a.T * ldp / 4;
    const unsigned nb = (unsigned)std::min<int64_t>((n4 + kT - 1) / kT, 2048);
    hipLaunchKernelGGL(k_kv_part_add, dim3(nb), dim3(kT), 0, st, a.dK, a.dV, a.lddk, a.part, a.T,
                       ldp, ns);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_flash_bwd_dq, dim3((unsigned)(nkb * a.n_q)), dim3(kT), 0, st, a);
  return hipGetLastError();
}

}  // namespace omq
