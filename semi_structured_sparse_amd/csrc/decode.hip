// Few-token ("decode") products, T <= 128: HBM-bound streaming of the weights.
//
//   Y[t][o] (+)= scale[o] * sum_k X~[t][k] * W~[o][k]
//
// W~ is one of: dense bf16 rows, dense fp8-e4m3 rows (widened to bf16 in registers,
// exact; per-row scale applied to the partial sums), or a 2:4 compressed matrix (values
// + 2-bit positions) fed to v_smfmac_f32_16x16x64_bf16.  X~ is X, lift_N(X) (lowered
// (2N-2):2N weights; SlideSparse page, technical summary 2.A/2.B) or X[:, cols] (hybrid
// regions; SpenseGPT page, technical summary 2.A/2.B).
//
// With few tokens the weights dominate the bytes, so the kernel is built to stream them
// at full HBM bandwidth:
//  * a workgroup of 4 waves owns 64 output rows and one slice of K (split-K so that
//    there are ~4 workgroups per CU); each wave owns 16 rows;
//  * each lane loads its 16-byte weight fragment straight from global memory into the
//    matrix-instruction operand layout (no LDS), UNROLL reduction chunks at a time so
//    that several KiB per wave are in flight;
//  * the small X tile is read per chunk through L1/L2 (shared by the 4 waves);
//  * split-K partial sums are added into Y with hardware fp32 atomics (the caller's Y is
//    zeroed first unless accumulating), so the summation order between K slices is not
//    fixed: results are reproducible to fp32 rounding, not bit for bit.
#include <cstdlib>

#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;
using namespace nml;

enum WKind { WK_BF16 = 0, WK_FP8 = 1, WK_SP24 = 2 };

__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t q, uint32_t& lo, uint32_t& hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, false);
  const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, true);
  lo = __builtin_amdgcn_perm(__float_as_uint(a.y), __float_as_uint(a.x), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(b.y), __float_as_uint(b.x), 0x07060302u);
}

// 8 consecutive reduction positions [k, k+8) of X~ row (already offset to the row), zero
// beyond kend.  kk is the position in the X~ coordinate (lifted / gathered index space).
template <int XL>
__device__ __forceinline__ u32x4 load_x8(const uint16_t* __restrict__ rp, int64_t k, int64_t kend, int ns,
                                         const int32_t* __restrict__ cols, bool row_ok) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if (!row_ok) return r;
  if constexpr (XL == XL_PLAIN) {
    if (k + 8 <= kend) return *reinterpret_cast<const u32x4*>(rp + k);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k + e < kend) r[e >> 1] |= (uint32_t)rp[k + e] << (16 * (e & 1));
    return r;
  } else if constexpr (XL == XL_LIFT) {
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
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k + e < kend) r[e >> 1] |= (uint32_t)rp[cols[k + e]] << (16 * (e & 1));
    return r;
  }
}

// K-chunk handled by one matrix instruction: 32 (dense) or 64 (2:4 sparse, dense-equivalent)
template <int WK> struct Chunk { static constexpr int K = (WK == WK_SP24) ? 64 : 32; };

template <int TB, int WK, int XL, int UNROLL>
__global__ __launch_bounds__(256) void k_skinny(
    const void* __restrict__ wptr, int64_t ldw, const uint8_t* __restrict__ wmeta, const float* __restrict__ wscale,
    const uint16_t* __restrict__ x, int64_t ldx, const int32_t* __restrict__ cols, int ns, int64_t col_base,
    int64_t T, int64_t O, int64_t K, int64_t kslice, float* __restrict__ y, int64_t ldy, int atomic) {
  constexpr int CK = Chunk<WK>::K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int64_t nob = (O + 63) / 64;
  const int64_t ob = blockIdx.x % nob, ks = blockIdx.x / nob;
  const int64_t o_row = ob * 64 + wave * 16 + fr;            // the weight row this lane loads
  const int64_t o_ld = o_row < O ? o_row : O - 1;
  const int64_t k0 = ks * kslice;
  const int64_t k1 = (k0 + kslice < K) ? k0 + kslice : K;
  if (k0 >= k1) return;

  f32x4 acc[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // X rows of this lane's t-blocks
  const uint16_t* xrow[TB];
  bool xok[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int64_t t = 16 * j + fr;
    xok[j] = t < T;
    xrow[j] = x + (xok[j] ? t : 0) * ldx + col_base;
  }

  const int64_t kcv = K / 2;                // compressed row length (2:4)
  const int64_t mstride = (K + 7) >> 3;
  const bool vec_sp = (kcv & 7) == 0;       // 16-byte aligned compressed rows

  // Software pipeline over batches of UNROLL chunks: the weight and X fragments of batch
  // b+1 are requested before batch b is multiplied, so the (in-order) load counter lets
  // the compiler wait only for batch b while b+1 streams in.
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
        const uint16_t* rp = reinterpret_cast<const uint16_t*>(wptr) + o_ld * ldw;
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
        const uint8_t* rp = reinterpret_cast<const uint8_t*>(wptr) + o_ld * ldw;
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
        const uint16_t* vp = reinterpret_cast<const uint16_t*>(wptr) + o_ld * kcv + v0;
        const uint8_t* mp = wmeta + o_ld * mstride + (v0 >> 2);
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
        bt.xl[u][j] = load_x8<XL>(xrow[j], k + 8 * fq, k1, ns, cols, xok[j]);
        if constexpr (WK == WK_SP24) bt.xh[u][j] = load_x8<XL>(xrow[j], k + 32 + 8 * fq, k1, ns, cols, xok[j]);
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

  // lane holds Y^T rows o = 4*fq + r (of this wave's 16) for token t = 16*j + fr
  const int64_t obase = ob * 64 + wave * 16 + 4 * fq;
  float sc[4] = {1.f, 1.f, 1.f, 1.f};
  if (wscale != nullptr) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (obase + r < O) ? wscale[obase + r] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int64_t t = 16 * j + fr;
    if (t >= T) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (obase + r >= O) continue;
      float* yp = y + t * ldy + obase + r;
      const float v = acc[j][r] * sc[r];
      if (atomic) unsafeAtomicAdd(yp, v);
      else *yp = v;
    }
  }
}

// chunks per pipelined batch: two batches of weight + X fragments live in registers
constexpr int unroll_for(int64_t t, int wk) {
  return wk == WK_SP24 ? (t <= 16 ? 4 : t <= 32 ? 2 : 1) : (t <= 16 ? 4 : t <= 32 ? 4 : t <= 64 ? 2 : 1);
}

// Split-K plan: ~1024 workgroups (4 per CU), slices a multiple of the chunk and at least
// one unrolled step long.
int64_t skinny_target_blocks() {
  const char* e = std::getenv("NM_SKINNY_BLOCKS");   // A/B measurement override
  const int64_t v = e ? std::atoll(e) : 0;
  return v > 0 ? v : 1024;
}

void skinny_plan(const SkinnyArgs& a, int64_t* splits_out, int64_t* kslice_out) {
  const int ck = a.w_kind == WK_SP24 ? 64 : 32;
  const int64_t nob = (a.o + 63) / 64;
  const int64_t target = skinny_target_blocks();
  int64_t splits = (target + nob - 1) / nob;
  const int64_t step = (int64_t)ck * unroll_for(a.t, a.w_kind);
  const int64_t max_splits = (a.k + step - 1) / step;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t kslice = (a.k + splits - 1) / splits;
  kslice = ((kslice + ck - 1) / ck) * ck;
  *splits_out = (a.k + kslice - 1) / kslice;
  *kslice_out = kslice;
}

template <int TB, int WK, int XL>
hipError_t launch_tb(const SkinnyArgs& a, hipStream_t s) {
  constexpr int UNROLL = unroll_for(16 * TB, WK);
  const int64_t nob = (a.o + 63) / 64;
  int64_t splits, kslice;
  skinny_plan(a, &splits, &kslice);
  const int64_t blocks = nob * splits;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const int atomic = (splits > 1 || a.accumulate) ? 1 : 0;
  k_skinny<TB, WK, XL, UNROLL><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
      a.w, a.ldw, a.w_meta, a.w_scale, a.x, a.ldx, a.cols, a.ns, a.col_base, a.t, a.o, a.k, kslice, a.y, a.ldy,
      atomic);
  return hipGetLastError();
}

template <int WK, int XL>
hipError_t launch_wx(const SkinnyArgs& a, hipStream_t s) {
  if (a.t <= 16) return launch_tb<1, WK, XL>(a, s);
  if (a.t <= 32) return launch_tb<2, WK, XL>(a, s);
  if (a.t <= 64) return launch_tb<4, WK, XL>(a, s);
  return launch_tb<8, WK, XL>(a, s);
}

}  // namespace

namespace nml {

// Whether Y must be cleared before the skinny kernel adds into it (split-K atomics).
bool skinny_needs_zero(const SkinnyArgs& a) {
  int64_t splits, kslice;
  skinny_plan(a, &splits, &kslice);
  return splits > 1 && !a.accumulate;
}

hipError_t launch_skinny(const SkinnyArgs& a, hipStream_t s) {
  if (a.t > 128) return hipErrorInvalidValue;
  switch (a.w_kind) {
    case 0:
      if (a.loader == XL_PLAIN) return launch_wx<WK_BF16, XL_PLAIN>(a, s);
      if (a.loader == XL_GATHER) return launch_wx<WK_BF16, XL_GATHER>(a, s);
      break;
    case 1:
      if (a.loader == XL_PLAIN) return launch_wx<WK_FP8, XL_PLAIN>(a, s);
      break;
    case 2:
      if (a.loader == XL_PLAIN) return launch_wx<WK_SP24, XL_PLAIN>(a, s);
      if (a.loader == XL_LIFT) return launch_wx<WK_SP24, XL_LIFT>(a, s);
      if (a.loader == XL_GATHER) return launch_wx<WK_SP24, XL_GATHER>(a, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace nml
