// Internal launch interface between the C-ABI layer (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nm.h"

namespace nml {

// The caller's route hints (NM_ROUTE_* bits and tuning values, nm.h) travel with every
// call's arguments; `taken` (a host pointer or null) collects NM_TAKEN_* bits of the
// kernels the call enqueues.  Nothing is read from the process environment.
struct Route {
  uint32_t flags;
  int few_wpb, few_splits, tile_wg;
  uint32_t* taken;
  bool has(uint32_t bit) const { return (flags & bit) != 0; }
  void note(uint32_t bits) const {
    if (taken != nullptr) *taken |= bits;
  }
};

// Output epilogue of the dense-operand products, applied to each finished sum:
//   y[t][o] (=|+=) row_scale[t] * (w_scale[o] * acc) + beta_t * col_shift[o]
// with beta_t = row_shift[t], or 1 when row_shift is null.  Null pointers drop their
// factor or term.  Besides the fp8 weights' per-row scale it carries the activation
// mitigations: the variance correction's per-token scale and the term that undoes a shift
// of the activations (mu_t * (W . 1)_o, or (W . c)_o for a static shift).
struct Epi {
  const float* w_scale;
  const float* row_scale;
  const float* row_shift;
  const float* col_shift;
  __host__ __device__ bool extra() const { return row_scale != nullptr || col_shift != nullptr; }
};

__host__ __device__ inline float epi_apply(const Epi& e, float acc, int64_t t, int64_t o) {
  float v = e.w_scale != nullptr ? acc * e.w_scale[o] : acc;
  if (e.row_scale != nullptr) v *= e.row_scale[t];
  if (e.col_shift != nullptr) v += (e.row_shift != nullptr ? e.row_shift[t] : 1.f) * e.col_shift[o];
  return v;
}

// scored top-n (m in {4, 8, 16, 32}): score = fp32(|x|) * col_score[k] (use_x) or
// col_score[k] alone; outputs S(X) and/or the bitmask
hipError_t launch_select_scored(int m, const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, int n,
                                const float* col_score, int use_x, uint16_t* y, int64_t ldy, uint32_t* mask,
                                hipStream_t s);
// yblk: S(X) written in blocks of 16 token rows, [rows / 16][k / 32][16][32] (ldy unused;
// m in {4, 8, 16, 32}, k % 32 == 0) for the few-token streaming kernel's XL_BLK loader
hipError_t launch_select(int m, const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, int n,
                         uint16_t* y, int64_t ldy, uint32_t* mask, uint16_t* values,
                         uint8_t* meta, int meta_2bit, hipStream_t s, int yblk = 0);
hipError_t launch_decompress(int m, const uint16_t* values, const uint8_t* meta, int meta_2bit,
                             int64_t rows, int64_t k, int n, uint16_t* y, int64_t ldy, hipStream_t s);
hipError_t launch_lower_slide(int ns, const uint16_t* values, const uint8_t* idx, int64_t rows,
                              int64_t k, uint16_t* vout, uint8_t* mout, int meta_2bit, hipStream_t s);
// per-token fp8 quantization fused with the lift (ns = 2: no lift): codes xq [t][ldq]
// (lifted length K (2ns-2)/ns, zero up to ldq; ldq % 4 == 0), scales xs [t]
hipError_t launch_quant_lift(int ns, const uint16_t* x, int64_t t, int64_t k, int64_t ldx, uint8_t* xq,
                             int64_t ldq, float* xs, hipStream_t s);
hipError_t launch_lift(int ns, const uint16_t* x, int64_t t, int64_t k, int64_t ldx, uint16_t* xo,
                       int64_t ldo, hipStream_t s);
// shifted selection (dynamic: row mean; cshift: static per-channel shift; neither: none),
// S(x~) into y, optional mask, mu_out [rows] (dynamic), alpha_out [rows] (var)
hipError_t launch_select_pts(int m, const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, int n, int dynamic,
                             const float* cshift, int var, uint16_t* y, int64_t ldy, uint32_t* mask, float* mu_out,
                             float* alpha_out, hipStream_t s);
// out[o] = fp32(s_o * sum_k dec(W[o][k]) * (shift ? shift[k] : 1)), fp64 sum
hipError_t launch_weight_sums(const void* w, int64_t o, int64_t k, int64_t ldw, int fp8, const float* w_scale,
                              const float* shift, float* out, hipStream_t s);

// Activation-side prologue applied to X tiles inside the dense-MFMA GEMM.
enum Prologue { PRO_NONE = 0, PRO_SELECT = 1, PRO_MASK = 2 };

struct GemmArgs {
  const void* w;          // [O][ldw] bf16 or fp8 bytes
  int64_t ldw;
  int w_fp8;
  const float* w_scale;   // [O] or null
  const uint16_t* x;      // [T][ldx] bf16
  int64_t ldx;
  const uint32_t* x_mask; // PRO_MASK: [T][ceil(K/32)]
  int prologue, n, m;
  int64_t t, o, k;
  float* y;
  int64_t ldy;
  int accumulate;
  uint32_t* mask_out;     // PRO_SELECT: optional mask export
  Route route;
  // optional epilogue terms (Epi): per-token scale, per-token shift coefficient, per-row term
  const float* row_scale;
  const float* row_shift;
  const float* col_shift;
  Epi epi() const { return Epi{w_scale, row_scale, row_shift, col_shift}; }
};
hipError_t launch_gemm_dense(const GemmArgs& a, hipStream_t s);
// direct-to-LDS variant for large PRO_NONE / PRO_MASK problems with K % 64 == 0
bool gemm_lds_eligible(const GemmArgs& a, bool any_size);
hipError_t launch_gemm_lds(const GemmArgs& a, hipStream_t s);
// 256 x 256 tiles with the reduction split in `splits` K ranges (PRO_NONE): with part
// (scratch of at least splits * t * o floats) the ranges write fp32 partial tiles that a
// second kernel sums in range order; without it, one range.
hipError_t launch_gemm_lds_split(const GemmArgs& a, int64_t splits, float* part, int64_t part_bytes, hipStream_t s);
// fp8 e4m3fn weights [o][ldw] bytes -> bf16 [o][k] (exact), k % 8 == 0
hipError_t launch_widen_fp8(const uint8_t* w8, int64_t ldw, int64_t o, int64_t k, uint16_t* wb, hipStream_t s);
// split-K variant with 128-row tiles (PRO_NONE; few tokens, and token counts whose
// 256 x 256 tiles would not fill the chip): with part (scratch of at least
// gemm_lds_small_part_bytes(a) bytes) the K slices write fp32 partial tiles that a second
// kernel sums in slice order; without it, one slice.
bool gemm_lds_small_eligible(const GemmArgs& a);
int64_t gemm_lds_small_part_bytes(const GemmArgs& a);
hipError_t launch_gemm_lds_small(const GemmArgs& a, float* part, int64_t part_bytes, hipStream_t s);

// 2:4 sparse-operand GEMM on the gfx950 sparse matrix instructions.  The sparse
// operand is W (values [O][kc/2], 2-bit meta [O][ceil(kc/8)]) over a (possibly lowered)
// reduction length kc; the dense operand is X, read plainly or lifted.
// XL_F8: the X rows are e4m3 codes, one byte per position (x as bytes, ldx in bytes),
// widened to bf16 (exactly) as they are loaded.
// XL_BLK (few-token streaming kernel only): X rows in blocks of 16 tokens,
// [t / 16][k / 32][t % 16][32], block stride ldx elements (16 k).
enum XLoader { XL_PLAIN = 0, XL_LIFT = 1, XL_F8 = 2, XL_BLK = 3 };
struct SparseArgs {
  const uint16_t* w_vals;
  const uint8_t* w_meta;  // 2-bit
  int64_t kc;             // reduction length of the 2:4 operand (K or K')
  const uint16_t* x;
  int64_t ldx;
  int loader, ns;
  int64_t t, o;
  // optional dense second phase (hybrid): Y += Xd . Wd^T
  const uint16_t* wd;
  int64_t ldwd, kd;
  int64_t dbase;          // x column of the first dense reduction index (multiple of 8)
  float* y;
  int64_t ldy;
  int accumulate;
  int trans_out;          // 0: Y[t][o] with o = sparse-side row; 1: Y[s][d] (X sparse)
  // optional K-blocked copy of w_meta, [kc/64][o][8 bytes] (launch_meta_block), read by
  // the direct-to-LDS kernel in place of w_meta; the other kernels ignore it
  const uint8_t* w_meta_blk;
  // fp8 x fp8 (direct-to-LDS kernel only): w_vals are e4m3 codes [o][kc/2], x holds e4m3
  // codes [t][ldx bytes] (quantized per token, lifted), y = x_scale[t] * w_scale[o] * sum;
  // K-steps of 128 positions (kc % 128 == 0), blocked positions [kc/128][o][16 bytes]
  int f8;
  const float* x_scale;
  const float* w_scale;
  // lowered weights (loader XL_LIFT, no dense phase, bf16): the direct-to-LDS kernels build
  // the lifted X rows from the raw x in their loads (no lifted copy)
  int lift_dma;
  Route route;
};
hipError_t launch_gemm_sparse(const SparseArgs& a, hipStream_t s);
// whether launch_gemm_sparse hands this call to the direct-to-LDS kernel
bool gemm_sparse_uses_lds(const SparseArgs& a);
// 2-bit positions [o][kc/8] -> K-blocked [kc/64][o][8 bytes] (kc % 64 == 0): one K-step's
// positions for consecutive rows are contiguous, so a tile loads them as whole lines
// (unit = bytes of positions per row per K-step: 8 for bf16 steps of 64, 16 for fp8 steps of 128)
int64_t meta_block_bytes(int64_t o, int64_t kc);
hipError_t launch_meta_block(const uint8_t* meta, int64_t o, int64_t kc, int unit, uint8_t* out, hipStream_t s);

// Ranking and packing pieces of the hybrid packer, shared with the Spense GLU packer:
// flag[i] = 1 for the n_top largest scores (ties to the lower index; NaN scores must be
// mapped below every real score by the caller); the unflagged / flagged index lists in
// ascending order (one workgroup); 2:4 compression of the columns `cols` of each row; and
// the gather of the columns `cols`.  Column indices are clamped into [0, ncols).
hipError_t launch_rank_flags(const double* scores, int64_t n, int64_t n_top, int32_t* flag, hipStream_t s);
hipError_t launch_flag_lists(const int32_t* flag, int64_t n, int64_t n_flagged, int32_t* unflagged,
                             int32_t* flagged, hipStream_t s);
hipError_t launch_pack_cols(const uint16_t* w, int64_t o, int64_t ldw, int64_t ncols, const int32_t* cols,
                            int64_t ks, uint16_t* vals, uint8_t* meta, int meta_2bit, hipStream_t s);
hipError_t launch_gather_cols(const uint16_t* w, int64_t o, int64_t ldw, int64_t ncols, const int32_t* cols,
                              int64_t kd, uint16_t* wd, int64_t ldwd, hipStream_t s);

// Spense GLU: per-intermediate-index scores, tail flags, and a row gather
hipError_t launch_glu_scores(const uint16_t* wg, const uint16_t* wu, int64_t ld_gu, const uint16_t* wdn,
                             int64_t ld_d, int64_t hidden, int64_t inter, const double* hs_in,
                             const double* hs_mid, double* scores, hipStream_t s);
hipError_t launch_tail_flags(int64_t n, int64_t n_tail, int32_t* flag, hipStream_t s);
hipError_t launch_gather_rows(const uint16_t* w, int64_t ldw, int64_t o, int64_t k, const int32_t* rows,
                              int64_t count, uint16_t* out, int64_t ldo, hipStream_t s);
// direct-to-LDS variant for large problems (plain loader, kc % 64 == 0, kd % 64 == 0)
bool gemm_lds_sp_eligible(const SparseArgs& a, bool any_size);
hipError_t launch_gemm_lds_sp(const SparseArgs& a, hipStream_t s);
// its 256 x 256 tiles with the reduction split in `splits` step ranges (gemm_lds_sp_eligible
// with any_size): with part (scratch of at least splits * t * o floats) the ranges write
// fp32 partial tiles that a second kernel sums in range order; without it, one range.
hipError_t launch_gemm_lds_sp_split(const SparseArgs& a, int64_t splits, float* part, int64_t part_bytes,
                                    hipStream_t s);
// split variant with 128-row tiles (same eligibility with any_size; few tokens, and
// token counts whose 256 x 256 tiles would not fill the chip): with part (scratch of at least
// gemm_lds_sp_small_part_bytes(a) bytes) the splits write fp32 partial tiles that a second
// kernel sums in split order; without it, one split.
int64_t gemm_lds_sp_small_part_bytes(const SparseArgs& a);
hipError_t launch_gemm_lds_sp_small(const SparseArgs& a, float* part, int64_t part_bytes, hipStream_t s);

// Few-token streaming product (T <= 128): one or two weight segments summed into one
// accumulator, then scaled (w_scale, per output row) and written or added to y.
enum WKind { WK_BF16 = 0, WK_FP8 = 1, WK_SP24 = 2, WK_SP24F8 = 3 };
struct FewSeg {
  const void* w;          // WK_BF16 [o][ldw] bf16, WK_FP8 [o][ldw] bytes, WK_SP24 values [o][k/2],
                          // WK_SP24F8 e4m3 codes of the values [o][k/2] bytes
  int64_t ldw;
  const uint8_t* w_meta;  // WK_SP24, WK_SP24F8: 2-bit metadata [o][ceil(k/8)]
  int w_kind;
  const uint16_t* x;      // X rows of this segment (first column of the segment)
  int64_t ldx;
  int loader, ns;         // XL_PLAIN or XL_LIFT (lowered (2ns-2):2ns weights)
  int64_t k;              // reduction length in X~ coordinates (lifted for XL_LIFT)
};
struct FewArgs {
  FewSeg seg[2];
  int nseg;
  const float* w_scale;   // [o] or null
  int64_t t, o;
  float* y;
  int64_t ldy;
  int accumulate;
  int sel_m;              // > 0: seg[0].x is X itself; keep the m/2 largest of every m (see below)
  int q_ns;               // > 0 (one token, seg[0] e4m3 2:4 with the XL_F8 loader): seg[0].x is the
                          // bf16 X row itself; the kernel quantizes it to e4m3 per token and lifts it
                          // (NS = q_ns) in LDS, applies the token scale, and writes it to row_scale[0]
  Route route;
  const float* row_scale; // optional epilogue terms (Epi)
  const float* row_shift;
  const float* col_shift;
  Epi epi() const { return Epi{w_scale, row_scale, row_shift, col_shift}; }
};
// One token, one plain dense segment (bf16 or fp8 W), m in {4, 8, 16, 32}: whether
// launch_few applies the n = m/2 selection to the X row inside the product (the row
// staged in LDS), so that no separate select pass is needed (never under the
// NM_ROUTE_NO_FEW_SELECT or NM_ROUTE_NO_XLDS hints).
bool few_select_in_kernel(const FewArgs& a);
// One token, one e4m3 2:4 segment (XL_F8): whether launch_few can quantize and lift the
// bf16 X row inside the product (q_ns > 0; the raw row and its codes staged in LDS).
bool few_quant_in_kernel(const FewArgs& a);
// Scratch bytes of fp32 partial sums the preferred launch uses (0: single pass).
int64_t few_partial_bytes(const FewArgs& a);
// part: scratch of part_bytes bytes or null; with less than few_partial_bytes(a) the
// product runs as a single pass (fewer workgroups when o is small).
hipError_t launch_few(const FewArgs& a, float* part, int64_t part_bytes, hipStream_t s);
// Single token, K-major weights wk [k][o] (row stride o, o % 8 == 0): y[0][o] (=|+=)
// sum over the n:m-selected k of x[k] * wk[k][o]; part: scratch of gather1_part_bytes.
int64_t gather1_part_bytes(int64_t k, int64_t o, int m);
hipError_t launch_gather1(int m, const uint16_t* x, int64_t k, int n, const uint16_t* wk, int64_t o, float* y,
                          int accumulate, uint32_t* mask_out, float* part, int64_t part_bytes, const Route& r,
                          hipStream_t s);
// y[t][o] (=|+=) epi(sum_{s < splits} part[s][t][o])   (part rows have stride o)
hipError_t launch_reduce_parts(const float* part, int64_t splits, const Epi& epi, int64_t t, int64_t o,
                               float* y, int64_t ldy, int accumulate, const Route& r, hipStream_t s);
// xo[t][j] = x[t][c0[j]] (j < k0), xo[t][off1 + j] = x[t][c1[j]] (j < k1); indices
// clamped to [0, kx)
hipError_t launch_permute_cols(const uint16_t* x, int64_t t, int64_t ldx, int64_t kx, const int32_t* c0, int64_t k0,
                               const int32_t* c1, int64_t k1, int64_t off1, uint16_t* xo, int64_t ldo,
                               hipStream_t s);

hipError_t launch_hybrid_pack(const uint16_t* w, int64_t o, int64_t k, int64_t ldw, int64_t k_dense,
                              int32_t* sparse_cols, int32_t* dense_cols, uint16_t* ws_values,
                              uint8_t* ws_meta, int meta_2bit, uint16_t* wd, int64_t ldwd,
                              void* scratch, hipStream_t s);

}  // namespace nml
