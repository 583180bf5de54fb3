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

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8): lgkmcnt(0) alone, and vmcnt(n) alone, the other counters at their maxima
constexpr int kWaitLgkm0 = 0xC07F;
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

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

// ---------------------------------------------------------------------------------
// Per-token e4m3 quantization (the fp8 x fp8 lowered product; shared by the quantizing
// pass and the one-token weight-streaming kernel, so both produce the same codes).
// ---------------------------------------------------------------------------------

// e4m3fn code of v (|v| <= 448, finite), round to nearest, ties to even: in the normal
// range the 23 fraction bits are rounded to 3 (a carry moves to the next exponent), below
// 2^-6 the value is rounded to a multiple of the subnormal step 2^-9 (q = 8 is code 0x08,
// the smallest normal).
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7FFFFFFFu;
  if (__uint_as_float(a) >= 0x1p-6f) {
    int e = (int)(a >> 23) - 127;
    uint32_t m3 = (a >> 20) & 7u;
    const uint32_t rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) { m3 = 0u; ++e; }
    return sign | ((uint32_t)(e + 7) << 3) | m3;
  }
  return sign | (uint32_t)rintf(__uint_as_float(a) * 512.0f);
}

// From the row's largest 15-bit magnitude pattern mk: r = fp32(448 / amax) scales the
// values to codes, s = fp32(amax / 448) is the token scale (both 1 for an all-zero row).
__device__ __forceinline__ void token_scales(uint32_t mk, float& r, float& s) {
  const float amax = __uint_as_float(mk << 16);
  r = mk == 0 ? 1.0f : 448.0f / amax;
  s = mk == 0 ? 1.0f : amax / 448.0f;
}

// One group of 2 NS bf16 values (low 16 bits of v16) -> e4m3(clamp(x r, +-448)), lifted:
// window w (one dword) holds the codes of values 2w .. 2w + 3 (NS = 2: the group itself).
template <int NS>
__device__ __forceinline__ void quant_lift_group(const uint32_t (&v16)[2 * NS], float r, uint32_t (&win)[NS - 1]) {
  uint32_t q[2 * NS];
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i) {
    const float v = __uint_as_float(v16[i] << 16) * r;
    q[i] = e4m3_rne(fminf(fmaxf(v, -448.0f), 448.0f));
  }
#pragma unroll
  for (int w = 0; w < NS - 1; ++w) win[w] = q[2 * w] | (q[2 * w + 1] << 8) | (q[2 * w + 2] << 16) | (q[2 * w + 3] << 24);
}

// K-loop over n >= 1 steps through NST >= 3 LDS stages (distinct static arrays A[j], B[j],
// j < NST, named by constant indices so the compiler tracks the direct-to-LDS loads into
// each one).  issue(a, b, s) enqueues at least L direct-to-LDS requests per wave for step s
// into stage (a, b), the same number for every s; compute(a, b) multiplies a staged step.  Step q issues step q + NST - 1 into the
// stage step q - 1 used, multiplies step q, waits until this wave's requests of step q + 1
// have landed (the (NST - 2) L requests of the later steps may remain) and ends on a bare
// barrier, which makes every wave's step q + 1 visible and retires every read of step q.
// Past the last step the issue re-requests step n - 1 (into a stage no step reads again),
// so every step runs the same request-and-wait sequence: the compiler's wait analysis,
// which does not follow which branch issued what, then adds no drain of its own.  The
// loop ends with every request landed, so the stages are free for the caller.
template <int NST, int L, typename Issue, typename Compute>
__device__ __forceinline__ void lds_ring(int n, unsigned char* const* A, unsigned char* const* B, Issue&& issue,
                                         Compute&& compute) {
  static_assert(NST >= 3 && L >= 1 && L * (NST - 2) <= 63, "stages and requests per step");
  auto bar = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
#pragma unroll
  for (int j = 0; j + 1 < NST; ++j) issue(A[j], B[j], j < n ? j : n - 1);
  __builtin_amdgcn_s_waitcnt(vm_wait(L * (NST - 2)));
  bar();
  auto step = [&](int j, int q) {   // j = q % NST, a constant after unrolling
    const int ahead = q + NST - 1;
    issue(A[(j + NST - 1) % NST], B[(j + NST - 1) % NST], ahead < n ? ahead : n - 1);
    compute(A[j], B[j]);
    __builtin_amdgcn_s_waitcnt(vm_wait(L * (NST - 2)));
    bar();
  };
  // whole trips of NST steps: one block with no branch (the compiler's analysis added a
  // drain to loops whose trip had exits)
  int s = 0;
  for (; s + NST <= n; s += NST) {
#pragma unroll
    for (int j = 0; j < NST; ++j) step(j, s + j);
  }
  // the last n % NST steps
#pragma unroll
  for (int j = 0; j + 1 < NST; ++j) {
    if (s + j >= n) break;
    step(j, s + j);
  }
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  bar();
}

// Final fp32 stores of a wave's FI x FJ blocks of 16 x 16 results, v_mfma_f32_16x16 layout:
// block (i, j) holds, in lane (fr, fq) = (lane & 15, lane >> 4), outputs o = ob0 + 16 i + 4 fq
// + [0, 4) of token row t = tb0 + 16 j + fr.  y[t][o] (=|+=) the block values; rows t >= T
// are skipped.  With `whole` (every o of the wave inside O, ldy % 4 == 0, 16-byte aligned y)
// and FI even, a block pair (i, i + 1) goes out as two stores of whole 128-byte row pieces:
// lanes fr and fr ^ 8 swap one block, so the first store writes rows 0-7 (lanes fr < 8 block
// i, lanes fr >= 8 block i + 1 of row fr - 8) and the second rows 8-15.  A store per block
// would write 64-byte halves of 16 rows, which the memory system wrote back as separate
// pieces (1.46x the output bytes, measured).  Otherwise element by element, bounds-checked.
template <int FI, int FJ>
__device__ __forceinline__ void store_blocks(const f32x4 (&acc)[FI][FJ], float* __restrict__ y, int64_t ldy,
                                             int64_t T, int64_t O, int64_t ob0, int64_t tb0, int fr, int fq,
                                             bool whole, int accumulate) {
  if (FI % 2 == 0 && whole) {
    const bool up = fr < 8;
#pragma unroll
    for (int i = 0; i + 1 < FI; i += 2) {
      const int64_t ob = ob0 + i * 16 + 4 * fq + (up ? 0 : 16);
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int64_t tb = tb0 + j * 16 + (fr & 7);
        const f32x4 lo = acc[i][j], hi = acc[i + 1][j];
        const f32x4 send = up ? hi : lo;
        f32x4 got;
#pragma unroll
        for (int r = 0; r < 4; ++r) got[r] = __shfl_xor(send[r], 8);
        const f32x4 v0 = up ? lo : got, v1 = up ? got : hi;
        if (tb < T) {
          float4* yp = reinterpret_cast<float4*>(y + tb * ldy + ob);
          const float4 cur = accumulate ? *yp : make_float4(0.f, 0.f, 0.f, 0.f);
          *yp = make_float4(cur.x + v0[0], cur.y + v0[1], cur.z + v0[2], cur.w + v0[3]);
        }
        if (tb + 8 < T) {
          float4* yp = reinterpret_cast<float4*>(y + (tb + 8) * ldy + ob);
          const float4 cur = accumulate ? *yp : make_float4(0.f, 0.f, 0.f, 0.f);
          *yp = make_float4(cur.x + v1[0], cur.y + v1[1], cur.z + v1[2], cur.w + v1[3]);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const int64_t ob = ob0 + i * 16 + 4 * fq;
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int64_t t = tb0 + j * 16 + fr;
      if (t >= T) continue;
      float* yp = y + t * ldy + ob;
      // highest o first: a store sequence the compiler does not merge with the whole-line
      // path's last float4 store
#pragma unroll
      for (int r = 3; r >= 0; --r)
        if (ob + r < O) yp[r] = accumulate ? yp[r] + acc[i][j][r] : acc[i][j][r];
    }
  }
}

}  // namespace nmk
