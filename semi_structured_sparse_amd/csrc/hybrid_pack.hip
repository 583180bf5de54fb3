// Offline packing of the hybrid dense + 2:4 weight format (SpenseGPT page, technical
// summary 2.A: one dense region and one 2:4 region per weight matrix; 2.B: the dense
// indices are chosen by an importance score and permuted into one contiguous block).
// The dense columns are the k_dense columns of largest L2 norm over the output
// dimension.  Every step is deterministic:
//   1. c_k = sum_o W[o][k]^2 in fp64, o ascending, one thread per column (the squares
//      of bf16 values are exact in fp64, so only the fixed-order additions round);
//   2. rank_k = #{j : c_j > c_k or (c_j == c_k and j < k)}; dense iff rank_k < k_dense;
//   3. sparse / dense column lists in ascending column order (one workgroup, scan);
//   4. W_s = W[:, sparse_cols] pruned 2:4 by magnitude and compressed; W_d = W[:, dense_cols].
#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;

__global__ __launch_bounds__(256) void k_col_norms(const uint16_t* __restrict__ w, int64_t o, int64_t k,
                                                   int64_t ldw, double* __restrict__ norms) {
  const int64_t col = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (col >= k) return;
  double c = 0.0;
  for (int64_t r = 0; r < o; ++r) {
    const float v = __uint_as_float((uint32_t)w[r * ldw + col] << 16);
    const double d = (double)v;
    c = __dadd_rn(c, __dmul_rn(d, d));
  }
  // a NaN weight makes the norm unordered; rank it below every real norm so that the
  // ranks stay a permutation of 0..k-1 (non-finite weights are a caller error)
  norms[col] = (c != c) ? -1.0 : c;
}

__global__ __launch_bounds__(256) void k_col_rank(const double* __restrict__ norms, int64_t k,
                                                  int64_t k_dense, int32_t* __restrict__ flag) {
  __shared__ double s[1024];
  const int64_t col = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const double ck = col < k ? norms[col] : 0.0;
  int64_t rank = 0;
  for (int64_t base = 0; base < k; base += 1024) {
    __syncthreads();
    for (int i = threadIdx.x; i < 1024; i += blockDim.x) s[i] = (base + i < k) ? norms[base + i] : 0.0;
    __syncthreads();
    const int lim = (int)((k - base) < 1024 ? (k - base) : 1024);
    for (int i = 0; i < lim; ++i) {
      const double cj = s[i];
      const int64_t j = base + i;
      rank += (cj > ck || (cj == ck && j < col)) ? 1 : 0;
    }
  }
  if (col < k) flag[col] = rank < k_dense ? 1 : 0;
}

// One workgroup of 1024 threads; thread i scans a contiguous chunk of columns.
__global__ __launch_bounds__(1024) void k_col_lists(const int32_t* __restrict__ flag, int64_t k,
                                                    int64_t k_dense, int32_t* __restrict__ sparse_cols,
                                                    int32_t* __restrict__ dense_cols) {
  __shared__ int32_t s[1024];
  const int tid = threadIdx.x;
  const int64_t chunk = (k + 1023) / 1024;
  const int64_t c0 = tid * chunk, c1 = min(k, c0 + chunk);
  int32_t cnt = 0;
  for (int64_t c = c0; c < c1; ++c) cnt += flag[c];
  s[tid] = cnt;
  __syncthreads();
  // inclusive Hillis-Steele scan
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = (tid >= off) ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += v;
    __syncthreads();
  }
  int32_t dpos = s[tid] - cnt;                         // dense columns before my chunk
  int32_t spos = (int32_t)(c0 < k ? c0 : k) - dpos;   // sparse columns before my chunk
  for (int64_t c = c0; c < c1; ++c) {
    if (flag[c]) {
      if (dpos < k_dense) dense_cols[dpos] = (int32_t)c;
      ++dpos;
    } else {
      if (spos < k - k_dense) sparse_cols[spos] = (int32_t)c;
      ++spos;
    }
  }
}

// Column index from a list, clamped into [0, ncols) (lists may come from the caller).
__device__ __forceinline__ int64_t col_at(const int32_t* cols, int64_t j, int64_t ncols) {
  const int64_t c = cols[j];
  return c < 0 ? 0 : (c >= ncols ? ncols - 1 : c);
}

// One thread packs two consecutive 4-groups of the sparse region of one row.
__global__ __launch_bounds__(256) void k_pack_ws(const uint16_t* __restrict__ w, int64_t o, int64_t ldw,
                                                 int64_t ncols, const int32_t* __restrict__ sparse_cols, int64_t ks,
                                                 uint16_t* __restrict__ vals, uint8_t* __restrict__ meta,
                                                 int meta_2bit) {
  const int64_t G = ks / 4, pairs = (G + 1) / 2;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= o * pairs) return;
  const int64_t row = tid / pairs, gp = tid - row * pairs;
  const uint16_t* rp = w + row * ldw;
  uint32_t byte = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t g = 2 * gp + h;
    if (g >= G) break;
    uint32_t d[2];
    const uint32_t e0 = rp[col_at(sparse_cols, 4 * g, ncols)], e1 = rp[col_at(sparse_cols, 4 * g + 1, ncols)];
    const uint32_t e2 = rp[col_at(sparse_cols, 4 * g + 2, ncols)], e3 = rp[col_at(sparse_cols, 4 * g + 3, ncols)];
    d[0] = e0 | (e1 << 16);
    d[1] = e2 | (e3 << 16);
    const uint32_t keep = topn_bits<4>(d, 2);
    const uint32_t p0 = (uint32_t)__builtin_ctz(keep | 0x10u);
    const uint32_t p1 = 31u - (uint32_t)__builtin_clz(keep | 1u);
    const uint32_t v0 = (d[p0 >> 1] >> (16 * (p0 & 1))) & 0xFFFFu;
    const uint32_t v1 = (d[p1 >> 1] >> (16 * (p1 & 1))) & 0xFFFFu;
    const int64_t slot = row * (ks / 2) + 2 * g;
    vals[slot] = (uint16_t)v0;
    vals[slot + 1] = (uint16_t)v1;
    if (!meta_2bit) {
      meta[slot] = (uint8_t)p0;
      meta[slot + 1] = (uint8_t)p1;
    } else {
      byte |= ((p0 & 3u) | ((p1 & 3u) << 2)) << (4 * h);
    }
  }
  if (meta_2bit) meta[row * ((ks + 7) / 8) + gp] = (uint8_t)byte;
}

__global__ __launch_bounds__(256) void k_gather_wd(const uint16_t* __restrict__ w, int64_t o, int64_t ldw,
                                                   int64_t ncols, const int32_t* __restrict__ dense_cols, int64_t kd,
                                                   uint16_t* __restrict__ wd, int64_t ldwd) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= o * kd) return;
  const int64_t row = tid / kd, j = tid - row * kd;
  wd[row * ldwd + j] = w[row * ldw + col_at(dense_cols, j, ncols)];
}

inline unsigned blocks_for(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

}  // namespace

namespace nml {

hipError_t launch_rank_flags(const double* scores, int64_t n, int64_t n_top, int32_t* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_col_rank<<<blocks_for(n, 256), 256, 0, s>>>(scores, n, n_top, flag);
  return hipGetLastError();
}

hipError_t launch_flag_lists(const int32_t* flag, int64_t n, int64_t n_flagged, int32_t* unflagged,
                             int32_t* flagged, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_col_lists<<<1, 1024, 0, s>>>(flag, n, n_flagged, unflagged, flagged);
  return hipGetLastError();
}

hipError_t launch_pack_cols(const uint16_t* w, int64_t o, int64_t ldw, int64_t ncols, const int32_t* cols,
                            int64_t ks, uint16_t* vals, uint8_t* meta, int meta_2bit, hipStream_t s) {
  if (ks <= 0 || o <= 0 || ncols <= 0) return hipSuccess;
  k_pack_ws<<<blocks_for(o * ((ks / 4 + 1) / 2), 256), 256, 0, s>>>(w, o, ldw, ncols, cols, ks, vals, meta,
                                                                      meta_2bit);
  return hipGetLastError();
}

hipError_t launch_gather_cols(const uint16_t* w, int64_t o, int64_t ldw, int64_t ncols, const int32_t* cols,
                              int64_t kd, uint16_t* wd, int64_t ldwd, hipStream_t s) {
  if (kd <= 0 || o <= 0 || ncols <= 0) return hipSuccess;
  k_gather_wd<<<blocks_for(o * kd, 256), 256, 0, s>>>(w, o, ldw, ncols, cols, kd, wd, ldwd);
  return hipGetLastError();
}

hipError_t launch_hybrid_pack(const uint16_t* w, int64_t o, int64_t k, int64_t ldw, int64_t k_dense,
                              int32_t* sparse_cols, int32_t* dense_cols, uint16_t* ws_values,
                              uint8_t* ws_meta, int meta_2bit, uint16_t* wd, int64_t ldwd,
                              void* scratch, hipStream_t s) {
  if (k == 0) return hipSuccess;
  double* norms = reinterpret_cast<double*>(scratch);
  int32_t* flag = reinterpret_cast<int32_t*>(norms + k);
  k_col_norms<<<blocks_for(k, 256), 256, 0, s>>>(w, o, k, ldw, norms);
  k_col_rank<<<blocks_for(k, 256), 256, 0, s>>>(norms, k, k_dense, flag);
  k_col_lists<<<1, 1024, 0, s>>>(flag, k, k_dense, sparse_cols, dense_cols);
  const int64_t ks = k - k_dense;
  if (ks > 0 && o > 0)
    k_pack_ws<<<blocks_for(o * ((ks / 4 + 1) / 2), 256), 256, 0, s>>>(w, o, ldw, k, sparse_cols, ks,
                                                                        ws_values, ws_meta, meta_2bit);
  if (k_dense > 0 && o > 0)
    k_gather_wd<<<blocks_for(o * k_dense, 256), 256, 0, s>>>(w, o, ldw, k, dense_cols, k_dense, wd, ldwd);
  return hipGetLastError();
}

}  // namespace nml
