// Error mitigation of activation sparsity: the per-token shift (dynamic: the row mean, or a
// static per-channel shift) applied before the selection, and the per-token variance
// correction after it.  The activation-sparsity page's technical summary 2.B names both
// (D-PTS / S-PTS, VAR) as light-weight corrections needing little or no calibration data;
// 4.C ranks them among the most effective.  The page gives no formulas; the readings:
//   x~ = bf16(fp32(x - shift)),  shift = mu_t (row mean) or c_k (caller's static shift)
//   S(x~): the magnitude top-n of every group of m, ties to the lower index
//   alpha_t = sqrt(Var(x~_t) / Var(S(x~_t)))  (1 when the pruned row has no variance)
// and the product adds back the shift through a per-output term (see Epi in nm_launch.h).
//
// k_select_pts: one workgroup per token row.  The row is staged in LDS (one HBM read), its
// largest magnitude found, and -- for the dynamic shift -- its mean computed so that every
// implementation reaches the same bits whatever its summation order: each value is rounded
// to a multiple of q = 2^(E - 162) (E = exponent field of the largest magnitude, so every
// |x|/q < 2^36), the integers are summed exactly (in fp64: every partial sum is an integer
// below 2^52), and mu = fp32(fp64(S q) / K).
// Then each thread shifts, ranks and writes whole groups (the select kernel's ranking), the
// keep bits go into mask words by lane shuffles, and the VAR sums are accumulated in fp64.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;

typedef __attribute__((address_space(3))) void lds_void;

constexpr int PTS_THREADS = 256;
constexpr int PTS_WAVES = PTS_THREADS / 64;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

// fp32 -> bf16 bits, round to nearest even (finite or infinite input)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// x (a bf16 in the low 16 bits of h) minus shift, rounded to fp32 and then to bf16
__device__ __forceinline__ uint32_t shift_bf16(uint32_t h, float shift) {
  const float f = __uint_as_float(h << 16);
  return bf16_rne(__fsub_rn(f, shift));
}

// SH: 0 no shift, 1 the row mean (dynamic), 2 the caller's per-channel shift (static);
// VAR: accumulate the variance sums.  Both are template parameters so the per-element
// work has no branch.
template <int M, int SH, bool VAR>
__global__ __launch_bounds__(PTS_THREADS) void k_select_pts(const uint16_t* __restrict__ x, int64_t K, int64_t ldx,
                                                            int n, const float* __restrict__ cshift,
                                                            uint16_t* __restrict__ y, int64_t ldy,
                                                            uint32_t* __restrict__ mask, float* __restrict__ mu_out,
                                                            float* __restrict__ alpha_out) {
  constexpr bool dynamic = SH == 1;
  extern __shared__ __align__(16) uint16_t row[];     // the token row, K bf16
  __shared__ int red_i[PTS_WAVES];
  __shared__ double red_d[4][PTS_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r = blockIdx.x;
  const uint16_t* xr = x + r * ldx;
  const int64_t nch = K / 8;                         // 16-byte pieces (K % 8 == 0)

  // 1. stage the row: whole KiB with direct-to-LDS loads (every request of the row in
  // flight at once), the ragged tail through registers; then the largest magnitude key
  const int64_t nkb = nch / 64;
  for (int64_t kb = wave; kb < nkb; kb += PTS_WAVES)
    __builtin_amdgcn_global_load_lds(xr + 8 * (kb * 64 + lane), (lds_void*)(row + 8 * kb * 64), 16, 0, 0);
  for (int64_t c = nkb * 64 + tid; c < nch; c += PTS_THREADS)
    *reinterpret_cast<u32x4*>(row + 8 * c) = *reinterpret_cast<const u32x4*>(xr + 8 * c);
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  __syncthreads();
  int mx = 0;
  for (int64_t c = tid; c < nch; c += PTS_THREADS) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int a = (int)(v[q] & 0x7FFFu), b = (int)((v[q] >> 16) & 0x7FFFu);
      mx = a > mx ? a : mx;
      mx = b > mx ? b : mx;
    }
  }
  mx = wave_max_i32(mx);
  if (lane == 0) red_i[wave] = mx;
  __syncthreads();
  mx = red_i[0];
#pragma unroll
  for (int w = 1; w < PTS_WAVES; ++w) mx = red_i[w] > mx ? red_i[w] : mx;

  // 2. the dynamic shift: exact sum of the values rounded to multiples of q.  Every
  // rounded term x / q is an integer below 2^36 in magnitude and every partial sum one
  // below 2^52, so fp64 adds them exactly (the same integer in any order).
  float shift = 0.f;
  if constexpr (dynamic) {
    const int e = (mx >> 7) > 1 ? (mx >> 7) : 1;
    const double scale = __builtin_ldexp(1.0, 162 - e);   // 1 / q, a power of two
    double acc = 0.0, acc1 = 0.0;   // two chains of dependent adds
    if (mx != 0) {
      for (int64_t c = tid; c < nch; c += PTS_THREADS) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc += __builtin_rint((double)__uint_as_float(v[q] << 16) * scale);
          acc1 += __builtin_rint((double)__uint_as_float(v[q] & 0xFFFF0000u) * scale);
        }
      }
    }
    acc = wave_sum_f64(acc + acc1);
    if (lane == 0) red_d[0][wave] = acc;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < PTS_WAVES; ++w) tot += red_d[0][w];
    shift = mx == 0 ? 0.f : (float)(__builtin_ldexp(tot, e - 162) / (double)K);
    if (tid == 0 && mu_out != nullptr) mu_out[r] = shift;
  }

  // 3. shift, select, write S(x~) and the mask; VAR sums
  double sa = 0.0, sa2 = 0.0, sb = 0.0, sb2 = 0.0;
  const int64_t G = K / M;
  constexpr int GPW = 32 / M;                         // groups per mask word
  uint16_t* yr = y + r * ldy;
  for (int64_t g0 = 0; g0 < G; g0 += PTS_THREADS) {
    const int64_t g = g0 + tid;
    uint32_t bits = 0;
    if (g < G) {
      // the group in whole pieces (8 bytes for m = 4, else 16-byte pieces)
      uint32_t d[M / 2];
      if constexpr (M == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(row + g * M);
        d[0] = v.x;
        d[1] = v.y;
      } else {
#pragma unroll
        for (int p = 0; p < M / 8; ++p) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(row + g * M + 8 * p);
#pragma unroll
          for (int q = 0; q < 4; ++q) d[4 * p + q] = v[q];
        }
      }
      if constexpr (SH != 0) {
        float c[M];
        if constexpr (SH == 1) {
#pragma unroll
          for (int i = 0; i < M; ++i) c[i] = shift;
        } else {
#pragma unroll
          for (int p = 0; p < M / 4; ++p) {
            const float4 v = *reinterpret_cast<const float4*>(cshift + g * M + 4 * p);
            c[4 * p] = v.x;
            c[4 * p + 1] = v.y;
            c[4 * p + 2] = v.z;
            c[4 * p + 3] = v.w;
          }
        }
#pragma unroll
        for (int q = 0; q < M / 2; ++q)
          d[q] = shift_bf16(d[q] & 0xFFFFu, c[2 * q]) | (shift_bf16(d[q] >> 16, c[2 * q + 1]) << 16);
      }
      bits = (2 * n == M) ? topn_bits_n<M, M / 2>(d) : topn_bits<M>(d, n);
      uint32_t o[M / 2];
#pragma unroll
      for (int q = 0; q < M / 2; ++q) {
        o[q] = mask_pair(d[q], (bits >> (2 * q)) & 3u);
        if constexpr (VAR) {
          const double a0 = (double)__uint_as_float(d[q] << 16), a1 = (double)__uint_as_float(d[q] & 0xFFFF0000u);
          const double b0 = (bits >> (2 * q)) & 1u ? a0 : 0.0, b1 = (bits >> (2 * q + 1)) & 1u ? a1 : 0.0;
          sa += a0;
          sa += a1;
          sa2 = __builtin_fma(a0, a0, sa2);
          sa2 = __builtin_fma(a1, a1, sa2);
          sb += b0;
          sb += b1;
          sb2 = __builtin_fma(b0, b0, sb2);
          sb2 = __builtin_fma(b1, b1, sb2);
        }
      }
      if constexpr (M == 4) {
        *reinterpret_cast<uint2*>(yr + g * M) = make_uint2(o[0], o[1]);
      } else {
#pragma unroll
        for (int q = 0; q < M / 8; ++q)
          *reinterpret_cast<u32x4*>(yr + g * M + 8 * q) = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
      }
    }
    if (mask != nullptr) {
      // the lanes of one word hold consecutive groups (g0 is a multiple of 64)
      uint32_t wbits = bits << ((lane % GPW) * M);
#pragma unroll
      for (int off = 1; off < GPW; off <<= 1) wbits |= (uint32_t)__shfl_xor((int)wbits, off);
      if (g < G && (lane % GPW) == 0) mask[r * ((K + 31) / 32) + g / GPW] = wbits;
    }
  }

  // 4. VAR: alpha = sqrt(Var(x~) / Var(S(x~))), population variances over the K entries
  if constexpr (VAR) {
    sa = wave_sum_f64(sa);
    sa2 = wave_sum_f64(sa2);
    sb = wave_sum_f64(sb);
    sb2 = wave_sum_f64(sb2);
    __syncthreads();
    if (lane == 0) {
      red_d[0][wave] = sa;
      red_d[1][wave] = sa2;
      red_d[2][wave] = sb;
      red_d[3][wave] = sb2;
    }
    __syncthreads();
    if (tid == 0) {
      double ta = 0, ta2 = 0, tb = 0, tb2 = 0;
#pragma unroll
      for (int w = 0; w < PTS_WAVES; ++w) {
        ta += red_d[0][w];
        ta2 += red_d[1][w];
        tb += red_d[2][w];
        tb2 += red_d[3][w];
      }
      const double kk = (double)K;
      const double va = ta2 / kk - (ta / kk) * (ta / kk);
      const double vb = tb2 / kk - (tb / kk) * (tb / kk);
      alpha_out[r] = vb > 0.0 ? (float)__builtin_sqrt((va > 0.0 ? va : 0.0) / vb) : 1.f;
    }
  }
}

// v[o] = fp32( s_o * sum_k dec(W[o][k]) * c_k ) with c = shift or 1, s = w_scale or 1, the
// sum in fp64.  One workgroup per output row.
template <bool FP8>
__global__ __launch_bounds__(PTS_THREADS) void k_weight_sums(const void* __restrict__ w, int64_t K, int64_t ldw,
                                                             const float* __restrict__ w_scale,
                                                             const float* __restrict__ shift, float* __restrict__ out) {
  __shared__ double red[PTS_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t o = blockIdx.x;
  double acc = 0.0;
  for (int64_t k = tid; k < K; k += PTS_THREADS) {
    float v;
    if constexpr (FP8) {
      const uint8_t q = reinterpret_cast<const uint8_t*>(w)[o * ldw + k];
      typedef float f2 __attribute__((ext_vector_type(2)));
      const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, false);
      v = a.x;
    } else {
      v = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(w)[o * ldw + k] << 16);
    }
    acc += (double)v * (shift != nullptr ? (double)shift[k] : 1.0);
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < PTS_WAVES; ++i) t += red[i];
    if (w_scale != nullptr) t *= (double)w_scale[o];
    out[o] = (float)t;
  }
}

}  // namespace

namespace nml {

hipError_t launch_select_pts(int m, const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, int n, int dynamic,
                             const float* cshift, int var, uint16_t* y, int64_t ldy, uint32_t* mask, float* mu_out,
                             float* alpha_out, hipStream_t s) {
  if (rows <= 0 || k <= 0) return hipSuccess;
  if (rows > 0x7FFFFFFF || k % 8 != 0 || k > 65536) return hipErrorInvalidValue;
  const size_t lds = (size_t)k * 2;
  const dim3 g((unsigned)rows), b(PTS_THREADS);
#define NM_PTS_K(MV, SHV, VARV)                                                                             \
  {                                                                                                         \
    auto kern = k_select_pts<MV, SHV, VARV>;                                                               \
    if (lds > 65536) {                                                                                      \
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,     \
                                         (int)lds);                                                        \
      if (e != hipSuccess) return e;                                                                        \
    }                                                                                                       \
    kern<<<g, b, lds, s>>>(x, k, ldx, n, cshift, y, ldy, mask, mu_out, alpha_out);                          \
    return hipGetLastError();                                                                               \
  }
#define NM_PTS_V(MV, SHV) \
  if (var) NM_PTS_K(MV, SHV, true) else NM_PTS_K(MV, SHV, false)
#define NM_PTS(MV)                                  \
  {                                                 \
    if (dynamic) NM_PTS_V(MV, 1)                    \
    else if (cshift != nullptr) NM_PTS_V(MV, 2)     \
    else NM_PTS_V(MV, 0)                            \
  }
  switch (m) {
    case 4: NM_PTS(4)
    case 8: NM_PTS(8)
    case 16: NM_PTS(16)
    case 32: NM_PTS(32)
    default: return hipErrorInvalidValue;
  }
#undef NM_PTS
#undef NM_PTS_V
#undef NM_PTS_K
  return hipErrorInvalidValue;
}

hipError_t launch_weight_sums(const void* w, int64_t o, int64_t k, int64_t ldw, int fp8, const float* w_scale,
                              const float* shift, float* out, hipStream_t s) {
  if (o <= 0) return hipSuccess;
  if (o > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (fp8) k_weight_sums<true><<<dim3((unsigned)o), dim3(PTS_THREADS), 0, s>>>(w, k, ldw, w_scale, shift, out);
  else k_weight_sums<false><<<dim3((unsigned)o), dim3(PTS_THREADS), 0, s>>>(w, k, ldw, w_scale, shift, out);
  return hipGetLastError();
}

}  // namespace nml
