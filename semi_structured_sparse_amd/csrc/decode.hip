// Few-token ("decode") products, T <= 128: HBM-bound streaming of the weights.
//
//   Y[t][o] (+)= scale[o] * ( sum_k X0[t][k] * W0[o][k]  +  sum_k X1[t][k] * W1[o][k] )
//
// Each segment W_i is one of: dense bf16 rows, dense fp8-e4m3 rows (widened to bf16 in
// registers, exact; the per-row scale is applied once to the finished sum), or a 2:4
// compressed matrix (values + 2-bit positions) fed to v_smfmac_f32_16x16x64_bf16.  X_i is
// X or lift_N(X) (lowered (2N-2):2N weights; SlideSparse page, technical summary 2.A/2.B).
// Two segments express the hybrid format's input split with one accumulator (SpenseGPT
// page, technical summary 2.A): the 2:4 region first, the dense region second.
//
// With few tokens the weights dominate the bytes, so the kernel is built to stream them
// at full HBM bandwidth and to leave no reduction work to atomics:
//  * a workgroup owns 16 output rows; its waves (4-16) split the reduction range of every
//    segment into contiguous parts, one per wave, and stream their part;
//  * each lane loads its 16-byte weight fragment straight from global memory into the
//    matrix-instruction operand layout (no LDS), several chunks per batch, with the next
//    batch requested before the current one is multiplied (software pipeline);
//  * the small X tile is read per chunk through L1/L2;
//  * the waves' 16 x T partial tiles are summed through LDS in wave order and written
//    with plain stores.  When there are too few row blocks to fill the GPU (small O), the
//    reduction range is also split across workgroups; those write fp32 partial tiles to a
//    scratch buffer and a second kernel sums them in split order.  Either way the
//    summation order is fixed, so results are bit-for-bit reproducible.
#include <cstdlib>

#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;
using namespace nml;

constexpr int WK_NONE = -1;

__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t q, uint32_t& lo, uint32_t& hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, false);
  const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, true);
  lo = __builtin_amdgcn_perm(__float_as_uint(a.y), __float_as_uint(a.x), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(b.y), __float_as_uint(b.x), 0x07060302u);
}

// 8 consecutive reduction positions [k, k+8) of an X~ row (rp = start of the row), zero
// beyond kend.  k is in X~ coordinates (lifted index space for XL_LIFT).
template <int XL>
__device__ __forceinline__ u32x4 load_x8(const uint16_t* __restrict__ rp, int64_t k, int64_t kend, int ns,
                                         bool row_ok) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if (!row_ok) return r;
  if constexpr (XL == XL_PLAIN) {
    if (k + 8 <= kend) return *reinterpret_cast<const u32x4*>(rp + k);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k + e < kend) r[e >> 1] |= (uint32_t)rp[k + e] << (16 * (e & 1));
    return r;
  } else {
    // two windows of 4 lifted positions, each 4 consecutive original positions
    const int wpg = ns - 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t kp = k + 4 * h;
      if (kp < kend) {
        const int64_t win = kp >> 2;
        const int64_t g = win / wpg;
        const int64_t w = win - g * wpg;
        // 4-byte aligned only: two dword loads
        const uint32_t* src = reinterpret_cast<const uint32_t*>(rp + g * 2 * ns + 2 * w);
        r[2 * h] = src[0];
        r[2 * h + 1] = src[1];
      }
    }
    return r;
  }
}

// reduction positions covered by one matrix instruction: 32 (dense) or 64 (2:4 sparse,
// dense-equivalent)
template <int WK> struct Chunk { static constexpr int K = (WK == WK_SP24) ? 64 : 32; };

// chunks per pipelined batch: two batches of weight + X fragments live in registers,
// within 128 VGPRs for 1-2 token blocks (up to 16 waves per workgroup) and 256 above
constexpr int unroll_for(int tb, int wk) {
  return wk == WK_SP24 ? (tb == 1 ? 2 : 1) : (tb == 1 ? 4 : tb <= 4 ? 2 : 1);
}

// Stream reduction positions [k0, k1) of one segment for the lane's weight row o_ld into
// acc (lane holds Y^T rows 4*fq + r of the 16-row block for tokens 16*j + fr).
template <int TB, int WK, int XL>
__device__ __forceinline__ void stream_seg(f32x4 (&acc)[TB], const FewSeg& sg, int64_t o_ld, int64_t T,
                                           int64_t k0, int64_t k1, int lane) {
  constexpr int CK = Chunk<WK>::K;
  constexpr int UNROLL = unroll_for(TB, WK);
  const int fr = lane & 15, fq = lane >> 4;

  const uint16_t* xrow[TB];
  bool xok[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int64_t t = 16 * j + fr;
    xok[j] = t < T;
    xrow[j] = sg.x + (xok[j] ? t : 0) * sg.ldx;
  }
  const int64_t kcv = sg.k / 2;               // compressed row length (2:4)
  const int64_t mstride = (sg.k + 7) >> 3;    // 2-bit metadata bytes per row
  const bool vec_sp = (kcv & 7) == 0;         // 16-byte aligned compressed rows

  struct Batch {
    u32x4 w[UNROLL];
    uint32_t m[UNROLL];
    u32x4 xl[UNROLL][TB];
    u32x4 xh[UNROLL][TB];
  };
  auto fetch = [&](Batch& bt, int64_t kc) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t k = kc + (int64_t)u * CK;
      bt.m[u] = 0;
      if constexpr (WK == WK_BF16) {
        const int64_t kk = k + 8 * fq;
        const uint16_t* rp = reinterpret_cast<const uint16_t*>(sg.w) + o_ld * sg.ldw;
        if (kk + 8 <= k1) {
          bt.w[u] = *reinterpret_cast<const u32x4*>(rp + kk);
        } else {
          u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (kk + e < k1) v[e >> 1] |= (uint32_t)rp[kk + e] << (16 * (e & 1));
          bt.w[u] = v;
        }
      } else if constexpr (WK == WK_FP8) {
        const int64_t kk = k + 8 * fq;
        const uint8_t* rp = reinterpret_cast<const uint8_t*>(sg.w) + o_ld * sg.ldw;
        uint2 q;
        if (kk + 8 <= k1) {
          q = *reinterpret_cast<const uint2*>(rp + kk);
        } else {
          uint32_t qq[2] = {0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (kk + e < k1) qq[e >> 2] |= (uint32_t)rp[kk + e] << (8 * (e & 3));
          q = make_uint2(qq[0], qq[1]);
        }
        bt.w[u] = u32x4{q.x, q.y, 0u, 0u};   // widened to bf16 at use
      } else {
        // 2:4 compressed: 8 values covering dense positions [k + 16 fq, +16)
        const int64_t v0 = k / 2 + 8 * fq;
        const uint16_t* vp = reinterpret_cast<const uint16_t*>(sg.w) + o_ld * kcv + v0;
        const uint8_t* mp = sg.w_meta + o_ld * mstride + (v0 >> 2);
        if (vec_sp && v0 + 8 <= kcv && k + 16 * fq + 16 <= k1) {
          bt.w[u] = *reinterpret_cast<const u32x4*>(vp);
          bt.m[u] = (uint32_t)mp[0] | ((uint32_t)mp[1] << 8);
        } else {
          u32x4 v = {0u, 0u, 0u, 0u};
          uint32_t m = 0;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k + 16 * fq + 2 * e < k1 && v0 + e < kcv) v[e >> 1] |= (uint32_t)vp[e] << (16 * (e & 1));
#pragma unroll
          for (int bq = 0; bq < 2; ++bq)
            if ((v0 >> 2) + bq < mstride) m |= (uint32_t)mp[bq] << (8 * bq);
          bt.w[u] = v;
          bt.m[u] = m;
        }
      }
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        bt.xl[u][j] = load_x8<XL>(xrow[j], k + 8 * fq, k1, sg.ns, xok[j]);
        if constexpr (WK == WK_SP24) bt.xh[u][j] = load_x8<XL>(xrow[j], k + 32 + 8 * fq, k1, sg.ns, xok[j]);
      }
    }
  };
  auto consume = [&](const Batch& bt, int64_t kc) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t k = kc + (int64_t)u * CK;
      if (k >= k1) break;
      u32x4 wv = bt.w[u];
      if constexpr (WK == WK_FP8) {
        uint32_t c0, c1, c2, c3;
        fp8x4_to_bf16x4(wv[0], c0, c1);
        fp8x4_to_bf16x4(wv[1], c2, c3);
        wv = u32x4{c0, c1, c2, c3};
      }
      const bf16x8 af = __builtin_bit_cast(bf16x8, wv);
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        if constexpr (WK == WK_SP24) {
          const u32x4 lo = bt.xl[u][j], hi = bt.xh[u][j];
          const u32x8 bb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af, __builtin_bit_cast(bf16x16, bb), acc[j],
                                                             (int)bt.m[u], 0, 0);
        } else {
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, bt.xl[u][j]), acc[j], 0, 0, 0);
        }
      }
    }
  };

  constexpr int64_t STEP = (int64_t)CK * UNROLL;
  Batch b0, b1;
  int64_t kc = k0;
  fetch(b0, kc);
  while (true) {
    const int64_t kn = kc + STEP;
    if (kn < k1) fetch(b1, kn);
    consume(b0, kc);
    if (kn >= k1) break;
    const int64_t kn2 = kn + STEP;
    if (kn2 < k1) fetch(b0, kn2);
    consume(b1, kn);
    if (kn2 >= k1) break;
    kc = kn2;
  }
}

// the part [k0, k1) of a segment of length k handled by wave part p of P (chunk aligned)
template <int WK>
__device__ __forceinline__ void part_range(int64_t k, int64_t p, int64_t P, int64_t& k0, int64_t& k1) {
  constexpr int CK = Chunk<WK>::K;
  const int64_t c = (k + CK - 1) / CK;
  k0 = (p * c / P) * CK;
  k1 = ((p + 1) * c / P) * CK;
  if (k1 > k) k1 = k;
}

template <int TB> struct MaxThreads { static constexpr int V = TB >= 4 ? 512 : 1024; };

template <int TB, int WK0, int XL0, int WK1>
__global__ __launch_bounds__(MaxThreads<TB>::V) void k_few(FewSeg s0, FewSeg s1, const float* __restrict__ wscale,
                                                          int64_t T, int64_t O, float* __restrict__ y, int64_t ldy,
                                                          int accumulate, float* __restrict__ part, int splits) {
  extern __shared__ __align__(16) float red[];   // [waves][16 * TB * 16]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wpb = blockDim.x >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int64_t nob = (O + 15) / 16;
  const int64_t ob = blockIdx.x % nob;
  const int split = (int)(blockIdx.x / nob);
  const int64_t o_row = ob * 16 + fr;            // the weight row this lane loads
  const int64_t o_ld = o_row < O ? o_row : O - 1;
  const int64_t P = (int64_t)splits * wpb, p = (int64_t)split * wpb + wave;

  f32x4 acc[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    int64_t k0, k1;
    part_range<WK0>(s0.k, p, P, k0, k1);
    if (k0 < k1) stream_seg<TB, WK0, XL0>(acc, s0, o_ld, T, k0, k1, lane);
  }
  if constexpr (WK1 != WK_NONE) {
    int64_t k0, k1;
    part_range<WK1>(s1.k, p, P, k0, k1);
    if (k0 < k1) stream_seg<TB, WK1, XL_PLAIN>(acc, s1, o_ld, T, k0, k1, lane);
  }

  // sum the waves' tiles in wave order; element e = t * 16 + (o - 16 ob)
  constexpr int PER = TB * 256;
  float* mine = red + wave * PER;
#pragma unroll
  for (int j = 0; j < TB; ++j) *reinterpret_cast<f32x4*>(mine + (16 * j + fr) * 16 + 4 * fq) = acc[j];
  __syncthreads();
  for (int e = threadIdx.x; e < PER; e += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < wpb; ++w) sum += red[w * PER + e];
    const int64_t t = e >> 4, o = ob * 16 + (e & 15);
    if (t >= T || o >= O) continue;
    if (part != nullptr) {
      part[((int64_t)split * T + t) * O + o] = sum;
    } else {
      float v = wscale != nullptr ? sum * wscale[o] : sum;
      if (accumulate) v += y[t * ldy + o];
      y[t * ldy + o] = v;
    }
  }
}

__global__ void k_reduce_parts(const float* __restrict__ part, int64_t splits, const float* __restrict__ wscale,
                               int64_t T, int64_t O, float* __restrict__ y, int64_t ldy, int accumulate) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * O) return;
  const int64_t t = i / O, o = i - t * O;
  float sum = 0.f;
  for (int64_t sp = 0; sp < splits; ++sp) sum += part[sp * T * O + i];
  float v = wscale != nullptr ? sum * wscale[o] : sum;
  if (accumulate) v += y[t * ldy + o];
  y[t * ldy + o] = v;
}

// X[:, c0] then X[:, c1] side by side: xo[t][j] = x[t][c0[j]] (j < k0),
// xo[t][off1 + j] = x[t][c1[j]] (j < k1).  Column indices are clamped to [0, kx).
__global__ void k_permute_cols(const uint16_t* __restrict__ x, int64_t T, int64_t ldx, int64_t kx,
                               const int32_t* __restrict__ c0, int64_t k0, const int32_t* __restrict__ c1,
                               int64_t k1, int64_t off1, uint16_t* __restrict__ xo, int64_t ldo) {
  const int64_t n = k0 + k1;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * n) return;
  const int64_t t = i / n, j = i - t * n;
  int64_t c, dst;
  if (j < k0) {
    c = c0[j];
    dst = j;
  } else {
    c = c1[j - k0];
    dst = off1 + (j - k0);
  }
  c = c < 0 ? 0 : (c >= kx ? kx - 1 : c);
  xo[t * ldo + dst] = x[t * ldx + c];
}

struct Plan {
  int tb, wpb;
  int64_t splits;
};

int env_int(const char* name) {   // A/B measurement overrides
  const char* e = std::getenv(name);
  return e ? std::atoi(e) : 0;
}

Plan make_plan(const FewArgs& a, bool allow_split) {
  Plan p;
  p.tb = a.t <= 16 ? 1 : a.t <= 32 ? 2 : a.t <= 64 ? 4 : 8;
  const int max_wpb = p.tb >= 4 ? 8 : 16;
  const int64_t nob = (a.o + 15) / 16;
  int64_t chunks = 0;   // chunks of the longest segment
  for (int i = 0; i < a.nseg; ++i) {
    const int ck = a.seg[i].w_kind == WK_SP24 ? 64 : 32;
    const int64_t c = (a.seg[i].k + ck - 1) / ck;
    chunks = c > chunks ? c : chunks;
  }
  // about one workgroup of max_wpb waves per CU (256 CUs); many row blocks -> fewer waves
  // per block, few row blocks -> the reduction is also split across workgroups
  int wpb = max_wpb;
  int64_t splits = 1;
  if (nob >= 256) {
    while (wpb > 4 && nob * wpb > 256 * max_wpb) wpb /= 2;
  } else if (allow_split) {
    splits = (256 + nob - 1) / nob;
  }
  // keep at least two chunks per wave part
  if (splits > 1 && splits * wpb * 2 > chunks) splits = chunks / (2 * wpb) > 1 ? chunks / (2 * wpb) : 1;
  while (wpb > 4 && splits * wpb * 2 > chunks) wpb /= 2;
  const int ew = env_int("NM_FEW_WPB"), es = env_int("NM_FEW_SPLITS");
  if (ew == 4 || ew == 8 || (ew == 16 && max_wpb == 16)) wpb = ew;
  if (es > 0 && allow_split) splits = es;
  p.wpb = wpb;
  p.splits = splits;
  return p;
}

template <int TB, int WK0, int XL0, int WK1>
hipError_t launch_k(const FewArgs& a, const Plan& p, float* part, hipStream_t s) {
  auto kern = k_few<TB, WK0, XL0, WK1>;
  const int64_t nob = (a.o + 15) / 16;
  const int64_t blocks = nob * p.splits;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const size_t lds = (size_t)p.wpb * TB * 1024;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const FewSeg s1 = a.nseg > 1 ? a.seg[1] : FewSeg{};
  kern<<<dim3((unsigned)blocks), dim3(64 * p.wpb), lds, s>>>(a.seg[0], s1, a.w_scale, a.t, a.o, a.y, a.ldy,
                                                             a.accumulate, p.splits > 1 ? part : nullptr,
                                                             (int)p.splits);
  return hipGetLastError();
}

template <int WK0, int XL0, int WK1>
hipError_t launch_tb(const FewArgs& a, const Plan& p, float* part, hipStream_t s) {
  switch (p.tb) {
    case 1: return launch_k<1, WK0, XL0, WK1>(a, p, part, s);
    case 2: return launch_k<2, WK0, XL0, WK1>(a, p, part, s);
    case 4: return launch_k<4, WK0, XL0, WK1>(a, p, part, s);
    default: return launch_k<8, WK0, XL0, WK1>(a, p, part, s);
  }
}

}  // namespace

namespace nml {

int64_t few_partial_bytes(const FewArgs& a) {
  if (a.t <= 0 || a.o <= 0) return 0;
  const Plan p = make_plan(a, true);
  return p.splits > 1 ? p.splits * a.t * a.o * 4 : 0;
}

hipError_t launch_few(const FewArgs& a, float* part, int64_t part_bytes, hipStream_t s) {
  if (a.t > 128 || a.nseg < 1 || a.nseg > 2) return hipErrorInvalidValue;
  if (a.t == 0 || a.o == 0) return hipSuccess;
  Plan p = make_plan(a, part != nullptr);
  if (p.splits > 1 && part_bytes < p.splits * a.t * a.o * 4) p = make_plan(a, false);
  const FewSeg& s0 = a.seg[0];
  hipError_t e = hipErrorInvalidValue;
  if (a.nseg == 2) {
    if (s0.w_kind == WK_SP24 && s0.loader == XL_PLAIN && a.seg[1].w_kind == WK_BF16 && a.seg[1].loader == XL_PLAIN)
      e = launch_tb<WK_SP24, XL_PLAIN, WK_BF16>(a, p, part, s);
  } else if (s0.w_kind == WK_BF16 && s0.loader == XL_PLAIN) {
    e = launch_tb<WK_BF16, XL_PLAIN, WK_NONE>(a, p, part, s);
  } else if (s0.w_kind == WK_FP8 && s0.loader == XL_PLAIN) {
    e = launch_tb<WK_FP8, XL_PLAIN, WK_NONE>(a, p, part, s);
  } else if (s0.w_kind == WK_SP24 && s0.loader == XL_PLAIN) {
    e = launch_tb<WK_SP24, XL_PLAIN, WK_NONE>(a, p, part, s);
  } else if (s0.w_kind == WK_SP24 && s0.loader == XL_LIFT) {
    e = launch_tb<WK_SP24, XL_LIFT, WK_NONE>(a, p, part, s);
  }
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_reduce_parts(part, p.splits, a.w_scale, a.t, a.o, a.y, a.ldy, a.accumulate, s);
}

hipError_t launch_reduce_parts(const float* part, int64_t splits, const float* w_scale, int64_t t, int64_t o,
                               float* y, int64_t ldy, int accumulate, hipStream_t s) {
  const int64_t n = t * o;
  if (n == 0) return hipSuccess;
  k_reduce_parts<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(part, splits, w_scale, t, o, y, ldy,
                                                                        accumulate);
  return hipGetLastError();
}

hipError_t launch_permute_cols(const uint16_t* x, int64_t t, int64_t ldx, int64_t kx, const int32_t* c0, int64_t k0,
                               const int32_t* c1, int64_t k1, int64_t off1, uint16_t* xo, int64_t ldo,
                               hipStream_t s) {
  const int64_t n = t * (k0 + k1);
  if (n == 0) return hipSuccess;
  k_permute_cols<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(x, t, ldx, kx, c0, k0, c1, k1, off1, xo,
                                                                         ldo);
  return hipGetLastError();
}

}  // namespace nml
