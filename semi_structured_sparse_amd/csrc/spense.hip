// Spense layout of a GLU MLP (SpenseGPT page, technical summary 2.A and 2.B): the scores
// that pick which intermediate indices stay dense, and the row gather of the output-split
// packer.  Offline steps, run once per weight set; deterministic.
//
// Score of intermediate index i (the loss-aware strategy): the per-weight score
// |W_ij| * sqrt(H_jj) summed over the three projections that touch i,
//   g_i = sum_j |Wg[i][j]| hs_in[j],  u_i = sum_j |Wu[i][j]| hs_in[j]   (j ascending)
//   d_i = sum_o |Wd[o][i]|                                              (o ascending)
//   S_i = (g_i + u_i) + hs_mid[i] * d_i
// in fp64 with every product and sum rounded once in that order: contraction into fused
// multiply-adds is switched off in the kernel body (the compiler fuses a * b + c by default,
// and the __dmul_rn / __dadd_rn helpers do not prevent it).  One thread per index: the gate and up
// rows are read along j by one thread each (offline, so the strided reads are accepted);
// the down column reads are coalesced across threads.
#include "nm_device.h"
#include "nm_launch.h"

namespace {

__device__ __forceinline__ double abs_bf16(uint16_t b) {
  return (double)__uint_as_float((uint32_t)(b & 0x7FFFu) << 16);
}

__global__ __launch_bounds__(256) void k_glu_scores(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                                    int64_t ld_gu, const uint16_t* __restrict__ wdn, int64_t ld_d,
                                                    int64_t hidden, int64_t inter, const double* __restrict__ hs_in,
                                                    const double* __restrict__ hs_mid, double* __restrict__ scores) {
#pragma clang fp contract(off)
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= inter) return;
  double g = 0.0, u = 0.0, d = 0.0;
  const uint16_t* gr = wg + i * ld_gu;
  const uint16_t* ur = wu + i * ld_gu;
  for (int64_t j = 0; j < hidden; ++j) g = g + abs_bf16(gr[j]) * hs_in[j];
  for (int64_t j = 0; j < hidden; ++j) u = u + abs_bf16(ur[j]) * hs_in[j];
  for (int64_t o = 0; o < hidden; ++o) d = d + abs_bf16(wdn[o * ld_d + i]);
  const double sc = (g + u) + hs_mid[i] * d;
  // a NaN score is unordered: rank it below every real score (non-finite input is a
  // caller error; the ranks must stay a permutation)
  scores[i] = (sc != sc) ? -1.0 : sc;
}

__global__ __launch_bounds__(256) void k_tail_flags(int64_t n, int64_t n_tail, int32_t* __restrict__ flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) flag[i] = i >= n - n_tail ? 1 : 0;
}

// out[r][c] = w[rows[r]][c], rows clamped into [0, o)
__global__ __launch_bounds__(256) void k_gather_rows(const uint16_t* __restrict__ w, int64_t ldw, int64_t o,
                                                     int64_t k, const int32_t* __restrict__ rows, int64_t count,
                                                     uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= count * k) return;
  const int64_t r = tid / k, c = tid - r * k;
  int64_t src = rows[r];
  src = src < 0 ? 0 : (src >= o ? o - 1 : src);
  out[r * ldo + c] = w[src * ldw + c];
}

inline unsigned blocks_for(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

}  // namespace

namespace nml {

hipError_t launch_glu_scores(const uint16_t* wg, const uint16_t* wu, int64_t ld_gu, const uint16_t* wdn,
                             int64_t ld_d, int64_t hidden, int64_t inter, const double* hs_in,
                             const double* hs_mid, double* scores, hipStream_t s) {
  if (inter <= 0) return hipSuccess;
  k_glu_scores<<<blocks_for(inter, 256), 256, 0, s>>>(wg, wu, ld_gu, wdn, ld_d, hidden, inter, hs_in, hs_mid,
                                                      scores);
  return hipGetLastError();
}

hipError_t launch_tail_flags(int64_t n, int64_t n_tail, int32_t* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_tail_flags<<<blocks_for(n, 256), 256, 0, s>>>(n, n_tail, flag);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* w, int64_t ldw, int64_t o, int64_t k, const int32_t* rows,
                              int64_t count, uint16_t* out, int64_t ldo, hipStream_t s) {
  if (count <= 0 || k <= 0) return hipSuccess;
  k_gather_rows<<<blocks_for(count * k, 256), 256, 0, s>>>(w, ldw, o, k, rows, count, out, ldo);
  return hipGetLastError();
}

}  // namespace nml
