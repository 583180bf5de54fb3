// Device-side helpers shared by the libnmsparse kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nmk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------------
// Magnitude top-n of one group of M bf16 values.
//
// Order: larger magnitude first (the 15 bits below the sign), ties to the lower index.
// Each element gets a unique 32-bit composite key  (magnitude << 16) | (0xFFFF - i),
// so "rank < n" becomes "key >= the n-th largest key".  The n-th largest key comes
// from a bitonic sorting network on the composites (branch-free, register resident).
// ---------------------------------------------------------------------------------

template <int M>
__device__ __forceinline__ void sort_desc(uint32_t (&c)[M]) {
#pragma unroll
  for (int size = 2; size <= M; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const uint32_t a = c[i], b = c[j];
          const uint32_t hi = a > b ? a : b, lo = a > b ? b : a;
          if ((i & size) == 0) { c[i] = hi; c[j] = lo; } else { c[i] = lo; c[j] = hi; }
        }
      }
    }
  }
}

// Descending sort by Batcher's odd-even merge network (5 / 19 / 63 / 191 comparators for
// M = 4 / 8 / 16 / 32, against 6 / 24 / 80 / 240 for the bitonic network above).  When
// only one output is used the compiler drops the comparators it does not depend on.
template <int M, typename T>
__device__ __forceinline__ void sort_desc_oem(T (&c)[M]) {
#pragma unroll
  for (int p = 1; p < M; p <<= 1) {
#pragma unroll
    for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
      for (int j = k % p; j + k < M; j += 2 * k) {
#pragma unroll
        for (int i = 0; i < k; ++i) {
          const int a = i + j, b = i + j + k;
          if (b < M && a / (2 * p) == b / (2 * p)) {
            const T x = c[a], y = c[b];
            c[a] = x > y ? x : y;
            c[b] = x > y ? y : x;
          }
        }
      }
    }
  }
}

// Keep bits for a compile-time n: only the n-th largest key is needed.
template <int M, int N>
__device__ __forceinline__ uint32_t topn_bits_n(const uint32_t (&d)[M / 2]) {
  static_assert(N >= 1 && N <= M, "1 <= n <= m");
  uint32_t c[M], s[M];
#pragma unroll
  for (int q = 0; q < M / 2; ++q) {
    c[2 * q] = ((d[q] << 16) & 0x7FFF0000u) | (0xFFFFu - 2 * q);
    c[2 * q + 1] = (d[q] & 0x7FFF0000u) | (0xFFFFu - 2 * q - 1);
  }
#pragma unroll
  for (int i = 0; i < M; ++i) s[i] = c[i];
  sort_desc_oem<M>(s);
  const uint32_t tau = s[N - 1];
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) bits |= (c[i] >= tau ? 1u : 0u) << i;
  return bits;
}

// Groups whose width is not a power of two (m = 6, 10, 12, 14: the (2N-2):2N family):
// the keys are padded with zeros to P = the next power of two.  Every real key is at
// least 0xFFFF - i > 0, so the pads sort last and the n-th largest key is unchanged.
template <int M, int P>
__device__ __forceinline__ uint32_t topn_bits_pad(const uint32_t (&d)[M / 2], int n) {
  static_assert(M % 2 == 0 && M <= P && (P & (P - 1)) == 0, "even width, power-of-two pad");
  uint32_t c[M], s[P];
#pragma unroll
  for (int q = 0; q < M / 2; ++q) {
    c[2 * q] = ((d[q] << 16) & 0x7FFF0000u) | (0xFFFFu - 2 * q);
    c[2 * q + 1] = (d[q] & 0x7FFF0000u) | (0xFFFFu - 2 * q - 1);
  }
#pragma unroll
  for (int i = 0; i < P; ++i) s[i] = i < M ? c[i] : 0u;
  sort_desc_oem<P>(s);
  uint32_t tau = s[0];
#pragma unroll
  for (int j = 1; j < M; ++j) tau = (j == n - 1) ? s[j] : tau;
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) bits |= (c[i] >= tau ? 1u : 0u) << i;
  return bits;
}

// d: the group as packed dwords (element 2q in the low half of d[q]).  Returns the keep
// bits (bit i set iff element i is kept), exactly n bits set for 1 <= n <= M.
template <int M>
__device__ __forceinline__ uint32_t topn_bits(const uint32_t (&d)[M / 2], int n) {
  uint32_t c[M], s[M];
#pragma unroll
  for (int q = 0; q < M / 2; ++q) {
    c[2 * q] = ((d[q] << 16) & 0x7FFF0000u) | (0xFFFFu - 2 * q);
    c[2 * q + 1] = (d[q] & 0x7FFF0000u) | (0xFFFFu - 2 * q - 1);
  }
#pragma unroll
  for (int i = 0; i < M; ++i) s[i] = c[i];
  sort_desc<M>(s);
  uint32_t tau = s[0];
#pragma unroll
  for (int j = 1; j < M; ++j) tau = (j == n - 1) ? s[j] : tau;
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) bits |= (c[i] >= tau ? 1u : 0u) << i;
  return bits;
}

// Scored top-n (the weight-magnitude and activation-times-weight-magnitude scores):
// score_i = fp32(|x_i|) * c_i (one multiply, round to nearest even) or c_i alone, with
// c_i >= 0 finite and x finite, so scores are non-negative floats whose bit patterns
// order like their values.  The odd-even merge network on the 32-bit patterns gives the
// n-th largest score tau; then every score above tau is kept, and of the scores equal to
// tau the lowest-index ones, as many as n minus the count above tau (ties to the lower
// index).  NT > 0: n = NT known at compile time (only the comparators that tau depends
// on survive); NT = 0: n at run time.
template <int M, int NT>
__device__ __forceinline__ uint32_t topn_bits_scored(const uint32_t (&d)[M / 2], const float (&c)[M], int n,
                                                     bool use_x) {
  uint32_t sc[M], s[M];
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const uint32_t h = (i & 1) ? (d[i >> 1] >> 16) : (d[i >> 1] & 0xFFFFu);
    const float mag = __uint_as_float((h & 0x7FFFu) << 16);
    sc[i] = __float_as_uint(use_x ? mag * c[i] : c[i]);
    s[i] = sc[i];
  }
  sort_desc_oem<M>(s);
  uint32_t tau;
  if constexpr (NT > 0) {
    tau = s[NT - 1];
    n = NT;
  } else {
    tau = s[0];
#pragma unroll
    for (int j = 1; j < M; ++j) tau = (j == n - 1) ? s[j] : tau;
  }
  int above = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) above += sc[i] > tau ? 1 : 0;
  int ties_left = n - above;   // >= 1: tau is the n-th largest
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const bool eq = sc[i] == tau;
    const bool keep = sc[i] > tau || (eq && ties_left > 0);
    ties_left -= eq ? 1 : 0;
    bits |= (keep ? 1u : 0u) << i;
  }
  return bits;
}

// Zero the pruned halves of a packed dword pair-of-bf16 given 2 keep bits.
__device__ __forceinline__ uint32_t mask_pair(uint32_t d, uint32_t two_bits) {
  const uint32_t lo = (two_bits & 1u) ? 0x0000FFFFu : 0u;
  const uint32_t hi = (two_bits & 2u) ? 0xFFFF0000u : 0u;
  return d & (lo | hi);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Four OCP e4m3fn codes (one per byte of q) -> four bf16, exactly (every e4m3 value is a
// bf16 value): hardware decode to fp32, then the high halves.  lo = codes 0,1; hi = 2,3.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t q, uint32_t& lo, uint32_t& hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, false);
  const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, true);
  lo = __builtin_amdgcn_perm(__float_as_uint(a.y), __float_as_uint(a.x), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(b.y), __float_as_uint(b.x), 0x07060302u);
}

}  // namespace nmk
