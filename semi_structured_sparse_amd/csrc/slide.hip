// (2N-2):2N -> overlapping 2:4 windows (offline packer) and activation lifting.
//
// SlideSparse page, technical summary section 2.A: a group of 2N positions holding 2N-2
// kept values is covered by N-1 windows of width 4 and stride 2 (window w covers
// positions 2w..2w+3), each holding at most two; values that overflow a window go to
// the next one.  Kept positions are placed in ascending order into the lowest covering
// window with room.  Window w of group g becomes lowered positions g*4(N-1)+4w+s, and
// section 2.B's lifting duplicates the activations accordingly:
//   X'[t][g*4(N-1) + 4w + s] = X[t][g*2N + 2w + s].
#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;

// One thread lowers two consecutive groups of one row, so that its 2-bit metadata
// output (4(N-1) slots = N-1 bytes) never shares a byte with another thread.
template <int NS>
__global__ __launch_bounds__(256) void k_lower_slide(const uint16_t* __restrict__ values,
                                                     const uint8_t* __restrict__ idx,
                                                     int64_t rows, int64_t k,
                                                     uint16_t* __restrict__ vout,
                                                     uint8_t* __restrict__ mout, int meta_2bit) {
  constexpr int N = 2 * NS - 2;   // kept per group
  constexpr int W = NS - 1;       // windows per group
  const int64_t G = k / (2 * NS);
  const int64_t pairs = (G + 1) / 2;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= rows * pairs) return;
  const int64_t row = tid / pairs;
  const int64_t gp = (tid - row * pairs) * 2;
  const int64_t kin = G * N;          // input compressed row length
  const int64_t kout = G * 2 * W;     // output compressed row length (K'/2)
  uint32_t meta_bits[2] = {0u, 0u};   // per group: 2W slots x 2 bits <= 28 bits
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t g = gp + h;
    if (g >= G) break;
    uint16_t wv0[W], wv1[W];
    uint8_t ws0[W], ws1[W];
    int cnt[W];
#pragma unroll
    for (int w = 0; w < W; ++w) { wv0[w] = 0; wv1[w] = 0; ws0[w] = 0; ws1[w] = 1; cnt[w] = 0; }
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const uint16_t v = values[row * kin + g * N + j];
      const int p = idx[row * kin + g * N + j];
      bool placed = false;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const bool fits = !placed && p >= 2 * w && p <= 2 * w + 3 && cnt[w] < 2;
        if (fits) {
          if (cnt[w] == 0) { wv0[w] = v; ws0[w] = (uint8_t)(p - 2 * w); }
          else { wv1[w] = v; ws1[w] = (uint8_t)(p - 2 * w); }
          cnt[w] += 1;
          placed = true;
        }
      }
    }
    const int64_t ob = row * kout + g * 2 * W;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      vout[ob + 2 * w] = wv0[w];
      vout[ob + 2 * w + 1] = wv1[w];
      if (!meta_2bit) {
        mout[ob + 2 * w] = ws0[w];
        mout[ob + 2 * w + 1] = ws1[w];
      } else {
        meta_bits[h] |= ((uint32_t)(ws0[w] & 3) | ((uint32_t)(ws1[w] & 3) << 2)) << (4 * w);
      }
    }
  }
  if (meta_2bit) {
    // slots of group pair gp..gp+1 start at slot gp*2W, a multiple of 4W -> byte aligned
    const int64_t mstride = (2 * kout + 7) / 8;        // ceil(K'/8)
    const int64_t byte0 = row * mstride + (gp * 2 * W) / 4;
    const uint64_t all = (uint64_t)meta_bits[0] | ((uint64_t)meta_bits[1] << (4 * W));
    const int nslots = (gp + 1 < G) ? 4 * W : 2 * W;
    const int nbytes = (nslots * 2 + 7) / 8;
    for (int b = 0; b < nbytes; ++b) mout[byte0 + b] = (uint8_t)(all >> (8 * b));
  }
}

template <int NS>
__global__ __launch_bounds__(256) void k_lift(const uint16_t* __restrict__ x, int64_t t, int64_t k,
                                              int64_t ldx, uint16_t* __restrict__ xo, int64_t ldo) {
  constexpr int W = NS - 1;
  const int64_t G = k / (2 * NS);
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= t * G) return;
  const int64_t row = tid / G, g = tid - row * G;
  const uint16_t* src = x + row * ldx + g * 2 * NS;
  uint16_t* dst = xo + row * ldo + g * 4 * W;
#pragma unroll
  for (int w = 0; w < W; ++w)
#pragma unroll
    for (int s = 0; s < 4; ++s) dst[4 * w + s] = src[2 * w + s];
}

// Per-token fp8 quantization fused with the lift (SlideSparse page, technical summary
// 2.B: the online step quantizes the activations and expands them for the lowered
// weights in one pass).  One workgroup per token row: the row's magnitude maximum (on
// the 15-bit patterns, which order like |x|), then r = fp32(448 / amax) and
// s = fp32(amax / 448) (1 for an all-zero row), then every value x -> e4m3(clamp(x * r)),
// written in lifted order: out[g 4(NS-1) + 4w + s] = q[g 2NS + 2w + s] (NS = 2: no lift).
// Codes past the lifted length, up to ldq, are written as zero.
template <int NS, bool VEC>
__global__ __launch_bounds__(256) void k_quant_lift(const uint16_t* __restrict__ x, int64_t k, int64_t ldx,
                                                    uint8_t* __restrict__ xq, int64_t ldq, float* __restrict__ xs) {
  // VEC (k % 8 == 0, 16-byte aligned rows): the maximum pass reads 8 values per load and
  // NS = 4 groups (8 values) are single 16-byte loads; otherwise values move one by one
  constexpr int W = NS - 1;
  __shared__ uint32_t red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* xr = x + row * ldx;
  uint8_t* qr = xq + row * ldq;
  const int tid = threadIdx.x;
  uint32_t mk = 0;
  if constexpr (VEC) {
    for (int64_t i = (int64_t)tid * 8; i < k; i += 256 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(xr + i);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = d[j] & 0x7FFFu, hi = (d[j] >> 16) & 0x7FFFu;
        mk = lo > mk ? lo : mk;
        mk = hi > mk ? hi : mk;
      }
    }
  } else {
    for (int64_t i = tid; i < k; i += 256) {
      const uint32_t key = xr[i] & 0x7FFFu;
      mk = key > mk ? key : mk;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)mk, off, 64);
    mk = o > mk ? o : mk;
  }
  if ((tid & 63) == 0) red[tid >> 6] = mk;
  __syncthreads();
  mk = red[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) mk = red[w] > mk ? red[w] : mk;
  float r, st;
  token_scales(mk, r, st);
  if (tid == 0) xs[row] = st;
  const int64_t G = k / (2 * NS);
  for (int64_t g = tid; g < G; g += 256) {
    uint32_t v16[2 * NS];
    if constexpr (VEC && NS == 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(xr + g * 8);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) { v16[2 * j] = d[j] & 0xFFFFu; v16[2 * j + 1] = d[j] >> 16; }
    } else {
#pragma unroll
      for (int i = 0; i < 2 * NS; ++i) v16[i] = xr[g * 2 * NS + i];
    }
    uint32_t win[W];
    quant_lift_group<NS>(v16, r, win);
    uint32_t* dst = reinterpret_cast<uint32_t*>(qr + g * 4 * W);
#pragma unroll
    for (int w = 0; w < W; ++w) dst[w] = win[w];
  }
  for (int64_t i = G * 4 * W + tid; i < ldq; i += 256) qr[i] = 0;
}

}  // namespace

namespace nml {

hipError_t launch_quant_lift(int ns, const uint16_t* x, int64_t t, int64_t k, int64_t ldx, uint8_t* xq,
                             int64_t ldq, float* xs, hipStream_t s) {
  if (t <= 0) return hipSuccess;
  if (t > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)t), block(256);
  const bool vec = (k % 8) == 0 && (ldx % 8) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  switch (ns) {
#define NM_CASE(NSV)                                                                           \
  case NSV:                                                                                    \
    if (vec) k_quant_lift<NSV, true><<<grid, block, 0, s>>>(x, k, ldx, xq, ldq, xs);           \
    else k_quant_lift<NSV, false><<<grid, block, 0, s>>>(x, k, ldx, xq, ldq, xs);              \
    break;
    NM_CASE(2) NM_CASE(3) NM_CASE(4) NM_CASE(5) NM_CASE(6) NM_CASE(7) NM_CASE(8)
#undef NM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lower_slide(int ns, const uint16_t* values, const uint8_t* idx, int64_t rows,
                              int64_t k, uint16_t* vout, uint8_t* mout, int meta_2bit, hipStream_t s) {
  const int64_t G = k / (2 * ns);
  const int64_t threads = rows * ((G + 1) / 2);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(256);
  switch (ns) {
#define NM_CASE(NSV) case NSV: k_lower_slide<NSV><<<grid, block, 0, s>>>(values, idx, rows, k, vout, mout, meta_2bit); break;
    NM_CASE(2) NM_CASE(3) NM_CASE(4) NM_CASE(5) NM_CASE(6) NM_CASE(7) NM_CASE(8)
#undef NM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lift(int ns, const uint16_t* x, int64_t t, int64_t k, int64_t ldx, uint16_t* xo,
                       int64_t ldo, hipStream_t s) {
  const int64_t threads = t * (k / (2 * ns));
  const int64_t blocks = (threads + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(256);
  switch (ns) {
#define NM_CASE(NSV) case NSV: k_lift<NSV><<<grid, block, 0, s>>>(x, t, k, ldx, xo, ldo); break;
    NM_CASE(2) NM_CASE(3) NM_CASE(4) NM_CASE(5) NM_CASE(6) NM_CASE(7) NM_CASE(8)
#undef NM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nml
