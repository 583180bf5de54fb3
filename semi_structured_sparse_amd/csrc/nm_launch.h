// Internal launch interface between the C-ABI layer (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nml {

hipError_t launch_select(int m, const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, int n,
                         uint16_t* y, int64_t ldy, uint32_t* mask, uint16_t* values,
                         uint8_t* meta, int meta_2bit, hipStream_t s);
hipError_t launch_decompress(int m, const uint16_t* values, const uint8_t* meta, int meta_2bit,
                             int64_t rows, int64_t k, int n, uint16_t* y, int64_t ldy, hipStream_t s);
hipError_t launch_lower_slide(int ns, const uint16_t* values, const uint8_t* idx, int64_t rows,
                              int64_t k, uint16_t* vout, uint8_t* mout, int meta_2bit, hipStream_t s);
hipError_t launch_lift(int ns, const uint16_t* x, int64_t t, int64_t k, int64_t ldx, uint16_t* xo,
                       int64_t ldo, hipStream_t s);

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
};
hipError_t launch_gemm_dense(const GemmArgs& a, hipStream_t s);
// direct-to-LDS variant for large PRO_NONE / PRO_MASK problems with K % 64 == 0
bool gemm_lds_eligible(const GemmArgs& a, bool any_size);
hipError_t launch_gemm_lds(const GemmArgs& a, hipStream_t s);
// few-token split-K variant (T <= 128, PRO_NONE, bf16); adds atomically when splits > 1
bool gemm_lds_small_eligible(const GemmArgs& a);
int64_t gemm_lds_small_splits(const GemmArgs& a);
hipError_t launch_gemm_lds_small(const GemmArgs& a, hipStream_t s);

// 2:4 sparse-operand GEMM on the gfx950 sparse matrix instructions.  The sparse
// operand is W (values [O][kc/2], 2-bit meta [O][ceil(kc/8)]) over a (possibly lowered)
// reduction length kc; the dense operand is X, read through one of three loaders.
enum XLoader { XL_PLAIN = 0, XL_LIFT = 1, XL_GATHER = 2 };
struct SparseArgs {
  const uint16_t* w_vals;
  const uint8_t* w_meta;  // 2-bit
  int64_t kc;             // reduction length of the 2:4 operand (K or K')
  const uint16_t* x;
  int64_t ldx;
  int loader, ns;
  const int32_t* cols;    // XL_GATHER: x column of each reduction index
  int64_t t, o;
  // optional dense second phase (hybrid): Y += Xd . Wd^T
  const uint16_t* wd;
  int64_t ldwd, kd;
  const int32_t* dcols;   // x column of each dense reduction index (null: kc + j)
  float* y;
  int64_t ldy;
  int accumulate;
  int trans_out;          // 0: Y[t][o] with o = sparse-side row; 1: Y[s][d] (X sparse)
};
hipError_t launch_gemm_sparse(const SparseArgs& a, hipStream_t s);

// Few-token streaming product (T <= 128).  w_kind: 0 bf16 [o][ldw], 1 fp8 [o][ldw] bytes
// (+ w_scale), 2 2:4 compressed over k (values [o][k/2], 2-bit meta [o][ceil(k/8)]).
// Adds into y with atomics when K is split; the caller clears y first when
// skinny_needs_zero() says so.
struct SkinnyArgs {
  const void* w;
  int64_t ldw;
  const uint8_t* w_meta;
  const float* w_scale;
  int w_kind;
  const uint16_t* x;
  int64_t ldx;
  int loader, ns;
  const int32_t* cols;
  int64_t col_base;
  int64_t t, o, k;
  float* y;
  int64_t ldy;
  int accumulate;
};
bool skinny_needs_zero(const SkinnyArgs& a);
hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t s);

hipError_t launch_hybrid_pack(const uint16_t* w, int64_t o, int64_t k, int64_t ldw, int64_t k_dense,
                              int32_t* sparse_cols, int32_t* dense_cols, uint16_t* ws_values,
                              uint8_t* ws_meta, int meta_2bit, uint16_t* wd, int64_t ldwd,
                              void* scratch, hipStream_t s);

}  // namespace nml
