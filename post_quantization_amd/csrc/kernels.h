// Internal launchers of the OmniQuant calibration kernels (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace omq {

// ---------------------------------------------------------------------------
// Row quantizer (LWC equation; rows are weight output channels or tokens)
// ---------------------------------------------------------------------------
struct RowQuantFwd {
  const void* x = nullptr;  int x_dt = 0;  int64_t rows = 0, cols = 0, ldx = 0;
  int let_mode = 0;  const float* s = nullptr;  const float* delta = nullptr;
  int nbits = 16;                                   // >= 16: pass-through (x~ only)
  const float* a_gamma = nullptr;  const float* a_beta = nullptr;  // NULL: 1
  void* out = nullptr;  int out_dt = 0;  int64_t ldo = 0;
  float* h = nullptr;  float* z = nullptr;  int32_t* amax = nullptr;  int32_t* amin = nullptr;
  uint8_t* codes = nullptr;                         // [rows x cols], row stride ldq
  int64_t ldq = 0;                                  // 0: cols (multiple of 4 otherwise)
  int code_off = 0;                                 // codes stored as q - code_off (a byte);
                                                    // 0 or 128
  int code_pack = 0;                                // 1: 4-bit codes two to a byte (code c in
                                                    // byte c / 2, low nibble for even c;
                                                    // ldq in bytes), n_bits <= 4, cols % 8 == 0
  int32_t* qsum = nullptr;                          // per-row sum of the stored codes (group 0)
  int32_t* nonfinite = nullptr;                     // set to 1 when any x~ is NaN or infinite
  const float* fold_delta = nullptr;                // bias fold: sum_i fold_delta_i x_ri
  const float* bias = nullptr;  float* bias_out = nullptr;
  // 128: each run of 128 columns of a row is its own quantizer (group-wise LWC);
  // h, z, arg_max/arg_min (column within the row), logits are then per
  // (row, group), index row * cols/128 + group.  0: one quantizer per row.
  // Grouped rows take no fold_delta (the bias fold runs on its own).
  int64_t group = 0;
  // nseg > 1 (whole rows of 512 n columns, group 0): concatenated weights (up to 3)
  // sharing s and fold_delta, segment k holding rows [seg_end[k-1], seg_end[k]) with
  // its own x rows and logits (indexed by the segment's own row); every output runs
  // over the concatenated rows.
  int nseg = 1;
  int64_t seg_end[3] = {0, 0, 0};
  const void* xseg[3] = {nullptr, nullptr, nullptr};
  const float* agseg[3] = {nullptr, nullptr, nullptr};
  const float* abseg[3] = {nullptr, nullptr, nullptr};
  // rms_out set (whole-row LDS kernel, activations): x is first divided by its row's
  // root mean square, sqrt(mean(x^2) + eps); the normalized rows go to rms_out
  // ([rows x cols] float32) and 1/rms to rstd[rows]
  float* rms_out = nullptr;
  float* rstd = nullptr;
  float eps = 0.f;
  // rope_out set (float32 activations in heads of 128 columns, rowquant_fwd_rope_ok):
  // each row is first rotated, RoPE with position = the row and tables rope_cos,
  // rope_sin [rows x 64] (rotate-half: column k of a head pairs with k + 64); the
  // rotated rows go to rope_out ([rows x cols] float32) and are then quantized
  const float* rope_cos = nullptr;
  const float* rope_sin = nullptr;
  float* rope_out = nullptr;
};
hipError_t launch_rowquant_fwd(const RowQuantFwd& a, hipStream_t st);
// whether launch_rowquant_fwd takes a.nseg > 1 (the whole-row LDS kernel applies)
bool rowquant_fwd_segments_ok(const RowQuantFwd& a);
// whether launch_rowquant_fwd takes a.rms_out
bool rowquant_fwd_rms_ok(const RowQuantFwd& a);
// whether launch_rowquant_fwd takes a.rope_out
bool rowquant_fwd_rope_ok(const RowQuantFwd& a);

enum ColMode { COL_NONE = 0, COL_WEIGHT = 1, COL_ACT_DIV = 2, COL_ACT_MUL = 3 };

// Straight-through backward, pass 1: a 2-D tile pass over (g, x) producing per-row
// partial sums (g_h, sum g (1 - in)) per column slab, per-column partial sums per
// row block, and (activations) the non-scatter part of the upstream gradient.
struct RowQuantBwd {
  const float* g = nullptr;  int64_t ldg = 0;       // dL/dx_hat
  const void* x = nullptr;  int x_dt = 0;  int64_t rows = 0, cols = 0, ldx = 0;
  int let_mode = 0;  const float* s = nullptr;  const float* delta = nullptr;
  int nbits = 16;
  const float* h = nullptr;  const float* z = nullptr;
  const int32_t* amax = nullptr;  const int32_t* amin = nullptr;
  const float* a_gamma = nullptr;  const float* a_beta = nullptr;
  int col_mode = COL_NONE;
  const float* rowvec = nullptr;                    // COL_WEIGHT: per-row v for sum_o v_o W_oi
  float* gx = nullptr;  int64_t ldgx = 0;           // upstream gradient (activations)
  float* g_agamma = nullptr;  float* g_abeta = nullptr;  // per row (weights)
  float* out0 = nullptr;  float* out1 = nullptr;    // column results (g_s, g_delta)
  int accumulate = 0;                               // add into out0/out1
  float* ws = nullptr;                              // partial buffers
  int64_t group = 0;                                // as in RowQuantFwd (128 or 0)
  // Row finalizer only: nseg > 1 concatenated weights (up to 3), segment k holding
  // rows [seg_end[k-1], seg_end[k]) with its own x rows and logits (indexed by the
  // segment's own quantizer row); h, z, arg_max/arg_min and the row partials run
  // over the concatenated rows.
  int nseg = 1;
  int64_t seg_end[3] = {0, 0, 0};
  const void* xseg[3] = {nullptr, nullptr, nullptr};
  const float* agseg[3] = {nullptr, nullptr, nullptr};
  const float* abseg[3] = {nullptr, nullptr, nullptr};
  float* gagseg[3] = {nullptr, nullptr, nullptr};
  float* gabseg[3] = {nullptr, nullptr, nullptr};
};
size_t rowquant_bwd_ws_bytes(int64_t rows, int64_t cols);
hipError_t launch_rowquant_bwd(const RowQuantBwd& a, hipStream_t st);
// Finalizers of the straight-through backward, shared by the tile pass and the
// GEMM-epilogue form.  Partials: rowpart [rows][nslabs][2] (g_h, sum g (1 - in)),
// colpart [ntiles][2][cols], one column-partial row per tile of tile_rows rows.
// launch_ste_finish runs the row finalizers of rf (LWC-logit gradients, the max/min
// scatter into rf.gx, and the scatter terms of the column outputs, which each tile
// adds to its own column partials in row order) and then the column pass of cf:
// out0 / out1 = (cf.accumulate ? their contents : 0) + the column partials, every
// sum in a fixed order (no atomics: a step is bitwise reproducible).
constexpr int kSteTileRows = 128;   // rows per column-partial tile of the GEMM epilogues
size_t ste_partials_floats(int64_t rows, int64_t cols, int64_t nslabs, int64_t ntiles);
hipError_t launch_ste_finish(const RowQuantBwd& cf, int ntiles, float* colpart,
                             const RowQuantBwd& rf, int nslabs, const float* rowpart,
                             int tile_rows, hipStream_t st);
// Finalizer jobs (each one launch_ste_finish's arguments, with cf's column-pass
// fields inline) in few launches: every job's row finalizers in one (up to
// kMaxRowJobs jobs of one kernel instance; otherwise one per job), then the column
// passes in rounds of one launch each, a pass going to the round after the last
// earlier job that adds into one of its outputs, so each output receives its jobs'
// sums in job order.  A job with rf.rows 0 has no row finalizers; skip_cols: the
// row finalizers still merge their scatter terms into the column partials, but the
// column pass is left to a later column-only job.
constexpr int kMaxFinJobs = 10, kMaxRowJobs = 4;
struct SteFinJob {
  RowQuantBwd rf;
  int nslabs = 0, tile_rows = 0, ntiles = 0;
  const float* rowpart = nullptr;
  float* colpart = nullptr;
  int64_t cols = 0;
  int col_mode = COL_NONE;
  float *out0 = nullptr, *out1 = nullptr;
  int accumulate = 0;
  bool skip_cols = false;
};
hipError_t launch_ste_finish_multi(const SteFinJob* jobs, int n, hipStream_t st);
// the row finalizers of launch_ste_finish alone (merging into colpart when cf names
// column outputs); its column pass is left to the caller
hipError_t launch_ste_finish_rows(const RowQuantBwd& cf, float* colpart, const RowQuantBwd& rf,
                                  int nslabs, const float* rowpart, int tile_rows,
                                  hipStream_t st);
// launch_rowquant_bwd's tile pass alone, its finalizers left in *job for
// launch_ste_finish_multi (job->rf.rows 0: nothing to finish)
hipError_t launch_rowquant_bwd_tiles(const RowQuantBwd& a, hipStream_t st, SteFinJob* job);

// LET alone: y = (x - delta) / s  or  y = s * x, elementwise over [rows x cols].
hipError_t launch_let_elementwise(const void* x, int x_dt, int64_t rows, int64_t cols,
                                  int mode, const float* s, const float* delta, void* y,
                                  int y_dt, hipStream_t st);
// B~ = B + W delta (float accumulate) for W [rows x cols].
hipError_t launch_bias_fold(const void* W, int w_dt, int64_t rows, int64_t cols,
                            const float* delta, const float* B, float* out, hipStream_t st);

// ---------------------------------------------------------------------------
// GEMM  C = alpha A B^T (+ bias) (+ C) ; A [M x K], B [N x K]
// ---------------------------------------------------------------------------

// Straight-through backward fused into a GEMM epilogue (the GEMM's C is dL/dx_hat
// for rows x cols of x).  Rows may come from up to 3 buffers (concatenated linears).
struct SteEpi {
  int mode = 0;                                     // 0 off, 1 weight rows, 2 token rows
  int nseg = 1;
  int64_t seg_end[3] = {0, 0, 0};                   // row ends of the segments
  const void* xseg[3] = {nullptr, nullptr, nullptr};
  int x_dt = 0;  int64_t ldx = 0;
  int let_mode = 0;  const float* s = nullptr;  const float* delta = nullptr;
  const float* h = nullptr;  const float* z = nullptr;  int nbits = 16;
  const float* rowvec = nullptr;
  int col_mode = 0;
  float* rowpart = nullptr;                         // [rows][tiles_n][2]
  float* colpart = nullptr;                         // [tiles_m][2][cols]
  // weight rows with group-wise LWC in groups of 128 columns: h, z are per (row,
  // 128-column tile), index row * tiles_n + tile; the row partials of a tile are
  // then exactly those of one (row, group)
  int grouped = 0;
};

struct Gemm {
  const void* A = nullptr;  int64_t lda = 0, strideA = 0;
  const void* B = nullptr;  int64_t ldb = 0, strideB = 0;  int b_group = 1;
  float* C = nullptr;  int64_t ldc = 0, strideC = 0;
  uint16_t* Cb = nullptr;                           // bf16 output instead of C
  const float* bias = nullptr;
  const void* resid = nullptr;  int resid_dt = 0;  int64_t ldr = 0;
  int64_t M = 0, N = 0, K = 0;  int batch = 1;
  float alpha = 1.f;
  int accumulate = 0;
  int dt = 1;                                       // OMQ_BF16 or OMQ_F32 operands
  // Integer-code product (dt ignored): A, B are uint8 codes [M x K], [N x K] (K
  // contiguous, ta = tb = 0, lda/ldb in bytes, values < 128) of row quantizers
  // with steps ha/hb, zero points za/zb and code sums sa/sb per row; C =
  // ha hb sum_k (qa - za)(qb - zb) (+ bias) (+ resid) (+ C), alpha unused.
  int codes = 0;
  const float *ha = nullptr, *za = nullptr, *hb = nullptr, *zb = nullptr;
  const int32_t *sa = nullptr, *sb = nullptr;
  // codes stored as q - zoa / q - zob (signed bytes: 8-bit codes shift by 128), so the
  // zero points enter as za - zoa, zb - zob; kz: the K of the zero-point term when
  // the code rows are padded with zero codes up to K (0: K)
  float zoa = 0.f, zob = 0.f;
  int64_t kz = 0;
  // 4-bit codes two to a byte (code k of a row in byte k / 2, the low nibble for even
  // k; lda/ldb in bytes): M, N and K multiples of 128, zoa = zob = 0
  int pack4 = 0;
  int ta = 0, tb = 0;                               // A is [K x M] / B is [K x N]
  SteEpi ste;                                       // bf16 only; mode 2 writes dL/dx into C
};
hipError_t launch_gemm(const Gemm& g, hipStream_t st);
// sums[r] = sum_c codes[r * ld + c]
hipError_t launch_code_rowsum(const uint8_t* codes, int64_t rows, int64_t cols, int64_t ld,
                              int32_t* sums, hipStream_t st);
// The fused form's partial-buffer extents for a C of rows x cols.
void gemm_ste_extents(int64_t rows, int64_t cols, int64_t* nslabs, int64_t* ntiles);

// Transposes: out[c][r] = in[r][c]  (bf16 -> bf16, or float -> bf16 with an
// optional straight bf16 copy written beside it).
// dY (float32, contiguous rows) -> bf16 copy, plus its column sums when colsum is
// set (ws: colsum_ws_bytes(rows, cols))
hipError_t launch_cvt_bf16_colsum(const float* in, int64_t rows, int64_t cols, uint16_t* out,
                                  float* colsum, float* ws, hipStream_t st);
// The same for a q|k|v gradient whose Q and K heads (head dimension 128) arrive as
// gradients of the rotated values: columns [0, qcols) are read from q and
// [qcols, qcols + kcols) from k, each through the inverse RoPE (cos/sin tables
// [rows x 64]) with the rotation kernel's arithmetic; the other columns from `in`.
struct RopeIn {
  const float* q; int64_t ldq, qcols;
  const float* k; int64_t ldk, kcols;
  const float *cos_t, *sin_t;
};
hipError_t launch_cvt_bf16_colsum_rope(const float* in, int64_t rows, int64_t cols,
                                       const RopeIn& rp, uint16_t* out, float* colsum, float* ws,
                                       hipStream_t st);
// Column sums in two deterministic stages: partial sums over chunks of kColsumRows
// rows ([nparts][cols] per kind), then out_k[c] (+)= sum of the nparts partials.
constexpr int kColsumRows = 64;
hipError_t launch_part_colsum(const float* part, int nparts, int nk, int64_t cols, float* out0,
                              float* out1, int accumulate, hipStream_t st);
// out[c] = sum_r in[r][c]   (deterministic two-stage)
hipError_t launch_colsum(const float* in, int64_t rows, int64_t cols, int64_t ld, float* out,
                         float* ws, hipStream_t st);
size_t colsum_ws_bytes(int64_t rows, int64_t cols);

// ---------------------------------------------------------------------------
// Block glue
// ---------------------------------------------------------------------------
hipError_t launch_rmsnorm(const void* x, int x_dt, int64_t T, int64_t d, float eps, float* y,
                          float* rstd, hipStream_t st);
hipError_t launch_rmsnorm_bwd(const float* gy, const float* x, const float* rstd, int64_t T,
                              int64_t d, const float* add, float* gx, hipStream_t st);
hipError_t launch_rope_tables(int64_t T, int64_t hd, float theta, float* cos_t, float* sin_t,
                              hipStream_t st);
hipError_t launch_rope(const float* x, int64_t ldx, int64_t T, int64_t n_heads, int64_t hd,
                       const float* cos_t, const float* sin_t, int inverse, float* y,
                       int64_t ldy, hipStream_t st);
// p[0 .. n) = v (a kernel, also inside captured graphs)
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st);
// RoPE of two operands (the Q and K heads) in one launch
hipError_t launch_rope2(const float* x0, int64_t ldx0, float* y0, int64_t ldy0, int64_t n0,
                        const float* x1, int64_t ldx1, float* y1, int64_t ldy1, int64_t n1,
                        int64_t T, int64_t hd, const float* cos_t, const float* sin_t,
                        int inverse, hipStream_t st);
hipError_t launch_silu_gate(const float* gu, int64_t T, int64_t F, float* a, hipStream_t st);
hipError_t launch_silu_gate_bwd(const float* gu, const float* ga, int64_t T, int64_t F,
                                float* ggu, hipStream_t st);
// The same gradient written only as the bf16 matrix-core operand [T x 2F], with its
// column sums (colsum: float[2F]; ws: colsum_ws_bytes(T, 2F)) formed in the same
// pass; false when the shape does not suit (F % 4, alignment): then use the above.
bool silu_gate_bwd_bf16_fits(const float* gu, const float* ga, int64_t T, int64_t F,
                             const uint16_t* ggub);
hipError_t launch_silu_gate_bwd_bf16(const float* gu, const float* ga, int64_t T, int64_t F,
                                     uint16_t* ggub, float* colsum, float* ws, hipStream_t st);
// loss = mean((y - target)^2), dy = 2 (y - target) / n (NULL: not written); dyb, when
// set, receives dy in bf16 too (needs n % 4 == 0 and 16-byte aligned y, target, dy)
hipError_t launch_mse(const float* y, const float* target, int64_t n, float* loss, float* dy,
                      float* ws, hipStream_t st, uint16_t* dyb = nullptr);
// fused causal attention, head dimension 128 (csrc/attn.hip).  lse2 is the
// per-(head, query) log-sum-exp of the scaled scores in the exp2 domain.
struct FlashFwd {
  const uint16_t* Q;        // [T x n_q*128] bf16, row stride ldq
  const uint16_t* K;        // [T x n_kv*128] bf16, row stride ldk
  const uint16_t* V;        // [T x n_kv*128] bf16, row stride ldk
  int64_t ldq, ldk, T;
  int n_q, grp;             // grp = n_q / n_kv
  float scale2;             // log2(e) / sqrt(128)
  float* O;                 // [T x n_q*128] fp32, row stride ldo
  int64_t ldo;
  float* lse2;              // [n_q x T]
};
struct FlashBwd {
  const uint16_t *Q, *K, *V;
  const uint16_t* dO;       // bf16, row stride ldq
  int64_t ldq, ldk, T;
  int n_q, grp;
  float scale, scale2;      // 1 / sqrt(128) and log2(e) / sqrt(128)
  const float* lse2;        // from the forward
  const float* D;           // [n_q x T] rowsum(dO * O)
  float* dQ;                // [T x n_q*128] fp32, row stride lddq
  int64_t lddq;
  float *dK, *dV;           // [T x n_kv*128] fp32, row stride lddk
  int64_t lddk;
  // flash_bwd_part_floats(T, n_q, n_kv) floats of scratch for the partial dK, dV of
  // the query-head splits beyond the first (nullptr when that count is 0)
  float* part;
  // flash_bwd_ds_elems(T, n_q) bf16 of scratch: dS as the dK/dV pass rounds it, per
  // query head [Tp keys][Tp queries] (Tp = T rounded up to 128), read back by dQ
  uint16_t* ds;
};
// Query-head splits of the dK/dV pass: a grouped K/V head's query heads are shared
// over this many workgroups when the K/V heads alone leave compute units idle.
int flash_bwd_splits(int64_t T, int n_q, int n_kv);
int64_t flash_bwd_part_floats(int64_t T, int n_q, int n_kv);
// n_q * Tp * Tp, or -1 when that exceeds 2^50 elements
int64_t flash_bwd_ds_elems(int64_t T, int64_t n_q);
hipError_t launch_flash_fwd(const FlashFwd& a, hipStream_t st);
hipError_t launch_attn_bwd_prep(const float* gO, const float* O, int64_t ld, int64_t T, int n_q,
                                float* D, uint16_t* gOb, int64_t ldb, hipStream_t st);
hipError_t launch_flash_bwd(const FlashBwd& a, hipStream_t st);
// deployment form (csrc/deploy.hip)
struct DeployFold {
  const uint32_t* words = nullptr;  int nbits = 4;  int64_t N = 0, K = 0;
  const float* h = nullptr;  const float* z = nullptr;  int64_t group = 0;
  const float* B = nullptr;  const float* s = nullptr;  const float* delta = nullptr;
  const float* s_o = nullptr;  const float* delta_o = nullptr;
  float* bias_out = nullptr;  float* h_out = nullptr;  float* gain_out = nullptr;
};
struct DeployGemm {
  const void* X = nullptr;  int64_t T = 0, K = 0;
  const uint32_t* words = nullptr;  int64_t N = 0;
  const float* h = nullptr;  const float* z = nullptr;  int64_t group = 0;
  const float* bias = nullptr;  float* Y = nullptr;
};
hipError_t launch_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int nbits,
                             uint32_t* words, hipStream_t st);
hipError_t launch_fold_linear(const DeployFold& a, hipStream_t st);
hipError_t launch_w4a16_gemm(const DeployGemm& a, hipStream_t st);
hipError_t launch_axpy_bcast(float* y, const float* x, int64_t n, hipStream_t st);
hipError_t launch_kv_expand(const float* v, int64_t n_q, int64_t n_kv, int64_t hd, float* out,
                            hipStream_t st);
hipError_t launch_kv_reduce_add(const float* v, int64_t n_q, int64_t n_kv, int64_t hd,
                                float* out, hipStream_t st);
hipError_t launch_adamw(float* theta, const float* grad, float* m, float* v, int64_t n,
                        int64_t n_lwc, float lr_lwc, float lr_let, float b1, float b2,
                        float eps, float wd, int64_t step, hipStream_t st);
hipError_t launch_sgd(float* theta, const float* grad, int64_t n, int64_t n_lwc, float lr_lwc,
                      float lr_let, hipStream_t st);

}  // namespace omq
