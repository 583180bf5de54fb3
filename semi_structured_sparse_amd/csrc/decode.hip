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
#include <cstring>
#include <type_traits>

#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;
using namespace nml;

constexpr int WK_NONE = -1;

// 8 consecutive reduction positions [k, k+8) of an X~ row (rp = start of the row), zero
// beyond kend.  k is in X~ coordinates (lifted index space for XL_LIFT, where window
// w of group g -- 4 lifted positions -- holds original positions g*2NS + 2w + [0, 4)).
// CHECKED = false: the caller guarantees [k, k+8) < kend (no bounds tests, no branches).
template <int XL, int NS, bool CHECKED>
__device__ __forceinline__ u32x4 load_x8(const uint16_t* __restrict__ rp, int k, int kend) {
  u32x4 r = {0u, 0u, 0u, 0u};
  if constexpr (XL == XL_F8) {
    // e4m3 codes, one byte per position (rp addresses bytes), widened to bf16
    const uint8_t* bp = reinterpret_cast<const uint8_t*>(rp);
    uint32_t q[2] = {0u, 0u};
    if (!CHECKED || k + 8 <= kend) {
      const uint2 v = *reinterpret_cast<const uint2*>(bp + k);
      q[0] = v.x;
      q[1] = v.y;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k + e < kend) q[e >> 2] |= (uint32_t)bp[k + e] << (8 * (e & 3));
    }
    uint32_t c0, c1, c2, c3;
    fp8x4_to_bf16x4(q[0], c0, c1);
    fp8x4_to_bf16x4(q[1], c2, c3);
    return u32x4{c0, c1, c2, c3};
  } else if constexpr (XL == XL_BLK) {
    // rp: the token's row inside its 16-token block; positions [k, k + 8) lie in one
    // 32-position piece (k % 8 == 0)
    const uint16_t* pp = rp + ((k >> 5) << 9) + (k & 31);
    if (!CHECKED || k + 8 <= kend) return *reinterpret_cast<const u32x4*>(pp);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k + e < kend) r[e >> 1] |= (uint32_t)pp[e] << (16 * (e & 1));
    return r;
  } else if constexpr (XL == XL_PLAIN) {
    if (!CHECKED || k + 8 <= kend) return *reinterpret_cast<const u32x4*>(rp + k);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (k + e < kend) r[e >> 1] |= (uint32_t)rp[k + e] << (16 * (e & 1));
    return r;
  } else {
    constexpr uint32_t WPG = NS - 1;   // windows per group (compile-time divisor)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kp = k + 4 * h;
      if (!CHECKED || kp < kend) {
        const uint32_t win = (uint32_t)kp >> 2;
        const uint32_t g = win / WPG;
        const uint32_t w = win - g * WPG;
        // 4-byte aligned only: two dword loads
        const uint32_t* src = reinterpret_cast<const uint32_t*>(rp + g * (2 * NS) + 2 * w);
        r[2 * h] = src[0];
        r[2 * h + 1] = src[1];
      }
    }
    return r;
  }
}

// The window pair (k/4, k/4 + 1) of a lifted X row in global memory (k % 8 == 0, both
// windows inside the row, raw row length kraw >= 64) with one 16-byte load instead of two
// 8-byte ones.  The first window starts at raw position a (dword aligned; global memory
// takes dword-aligned multi-dword accesses).  The second starts one dword later when both
// lie in one group, two dwords later when the first closes its group; in the first case
// the load starts a dword early where a + 8 would pass the row end, so it never reads
// outside [a, end of the second window] except inside the row.  Same values as load_x8.
template <int NS>
__device__ __forceinline__ u32x4 load_x8_lift_pair(const uint16_t* __restrict__ rp, int k, int kraw) {
  constexpr uint32_t WPG = NS - 1;   // windows per group (compile-time divisor)
  const uint32_t win = (uint32_t)k >> 2;
  const uint32_t g = win / WPG;
  const uint32_t w = win - g * WPG;
  const int a = (int)(g * (2 * NS) + 2 * w);
  const bool same = w + 1 < WPG;
  const bool back = same && a + 8 > kraw;   // only with both windows in one group
  u32x4 v;
  __builtin_memcpy(&v, rp + (back ? a - 2 : a), 16);
  if (back) return u32x4{v[1], v[2], v[2], v[3]};
  return same ? u32x4{v[0], v[1], v[1], v[2]} : u32x4{v[0], v[1], v[2], v[3]};
}

// 2:4 weights on the sparse matrix instruction: bf16 values, or e4m3 codes of them
constexpr bool sp_kind(int wk) { return wk == WK_SP24 || wk == WK_SP24F8; }

// the row of token t of an X segment (XL_F8 rows are bytes, ldx in bytes)
template <int XL>
__device__ __forceinline__ const uint16_t* x_row(const FewSeg& sg, int64_t t) {
  if constexpr (XL == XL_F8) return reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(sg.x) + t * sg.ldx);
  else if constexpr (XL == XL_BLK) return sg.x + (t >> 4) * sg.ldx + (t & 15) * 32;   // ldx: block stride
  else return sg.x + t * sg.ldx;
}

// reduction positions covered by one matrix instruction: 32 (dense) or 64 (2:4 sparse,
// dense-equivalent)
template <int WK> struct Chunk { static constexpr int K = sp_kind(WK) ? 64 : 32; };

// 16-row weight tiles per wave: each X fragment feeds RW matrix instructions, so the X
// bytes a wave pulls through L1 per weight byte drop from TB to TB/RW (2 TB/RW for 2:4).
constexpr int rw_for(int tb, int wk) { return tb == 1 ? 1 : tb == 2 ? 2 : tb == 4 ? 4 : 2; }

// chunks per pipelined batch: two batches of weight + X fragments live in registers
// next to the accumulators, within 128 VGPRs for 1-2 token blocks (up to 16 waves per
// workgroup) and 256 above
constexpr int unroll_for(int tb, int rw, int wk) {
  const int per_chunk = rw * (sp_kind(wk) ? 5 : 4) + tb * (sp_kind(wk) ? 8 : 4);
  const int budget = (tb <= 2 ? 128 : 256) - 48 - 4 * rw * tb - 2 * tb;
  const int u = budget / (2 * per_chunk);
  return u < 1 ? 1 : (u > 4 ? 4 : u);
}

// Stream reduction positions [k0, k1) of one segment for the lane's weight rows into acc
// (lane holds Y^T rows 16*i + 4*fq + r of the block for tokens 16*j + fr).
//
// Whole chunks go through a branch-free software pipeline: every load is issued
// unconditionally (token rows past T read row T-1; their outputs are never stored, and a
// matrix instruction's output column depends only on its own input column), so the
// compiler can count outstanding loads exactly and wait only for the batch it is about
// to multiply.  The ragged end of the part is handled chunk by chunk with checked loads.
template <int TB, int RW, int WK, int XL, int NS>
__device__ __forceinline__ void stream_seg(f32x4 (&acc)[RW][TB], const FewSeg& sg, const int64_t (&orow)[RW],
                                           int64_t T, int k0, int k1, int lane) {
  constexpr int CK = Chunk<WK>::K;
  constexpr int UNROLL = unroll_for(TB, RW, WK);
  const int fr = lane & 15, fq = lane >> 4;

  const uint16_t* xrow[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int64_t t = 16 * j + fr;
    xrow[j] = x_row<XL>(sg, t < T ? t : T - 1);
  }
  const int kcv = (int)(sg.k / 2);            // compressed row length (2:4)
  const int mstride = (int)((sg.k + 7) >> 3); // 2-bit metadata bytes per row
  const uint8_t* wrow[RW];                    // start of each weight row (bytes)
  const uint8_t* mrow[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    if constexpr (WK == WK_BF16) wrow[i] = reinterpret_cast<const uint8_t*>(sg.w) + orow[i] * sg.ldw * 2;
    else if constexpr (WK == WK_FP8) wrow[i] = reinterpret_cast<const uint8_t*>(sg.w) + orow[i] * sg.ldw;
    else if constexpr (WK == WK_SP24F8) wrow[i] = reinterpret_cast<const uint8_t*>(sg.w) + orow[i] * (int64_t)kcv;
    else wrow[i] = reinterpret_cast<const uint8_t*>(sg.w) + orow[i] * (int64_t)kcv * 2;
    mrow[i] = sp_kind(WK) ? sg.w_meta + orow[i] * (int64_t)mstride : nullptr;
  }

  struct Batch {
    u32x4 w[UNROLL][RW];
    uint32_t m[UNROLL][RW];
    u32x4 xl[UNROLL][TB];
    u32x4 xh[UNROLL][TB];
  };
  // unchecked loads of chunk k (the whole chunk lies inside the part)
  auto load_chunk = [&](Batch& bt, int u, int k) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if constexpr (WK == WK_BF16) {
        bt.w[u][i] = *reinterpret_cast<const u32x4*>(wrow[i] + 2 * (k + 8 * fq));
      } else if constexpr (WK == WK_FP8) {
        const uint2 q = *reinterpret_cast<const uint2*>(wrow[i] + k + 8 * fq);
        bt.w[u][i] = u32x4{q.x, q.y, 0u, 0u};   // widened to bf16 at use
      } else if constexpr (WK == WK_SP24F8) {
        const int v0 = k / 2 + 8 * fq;
        const uint2 q = *reinterpret_cast<const uint2*>(wrow[i] + v0);
        bt.w[u][i] = u32x4{q.x, q.y, 0u, 0u};   // widened to bf16 at use
        bt.m[u][i] = *reinterpret_cast<const uint16_t*>(mrow[i] + (v0 >> 2));   // v0 % 8 == 0
      } else {
        const int v0 = k / 2 + 8 * fq;
        bt.w[u][i] = *reinterpret_cast<const u32x4*>(wrow[i] + 2 * v0);
        bt.m[u][i] = *reinterpret_cast<const uint16_t*>(mrow[i] + (v0 >> 2));   // v0 % 8 == 0
      }
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      bt.xl[u][j] = load_x8<XL, NS, false>(xrow[j], k + 8 * fq, k + CK);
      if constexpr (sp_kind(WK)) bt.xh[u][j] = load_x8<XL, NS, false>(xrow[j], k + 32 + 8 * fq, k + CK);
    }
  };
  // checked loads of chunk k (any part of it may lie beyond k1)
  auto load_chunk_checked = [&](Batch& bt, int u, int k) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      bt.m[u][i] = 0;
      if constexpr (WK == WK_BF16) {
        const int kk = k + 8 * fq;
        const uint16_t* rp = reinterpret_cast<const uint16_t*>(wrow[i]);
        u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kk + e < k1) v[e >> 1] |= (uint32_t)rp[kk + e] << (16 * (e & 1));
        bt.w[u][i] = v;
      } else if constexpr (WK == WK_FP8) {
        const int kk = k + 8 * fq;
        const uint8_t* rp = wrow[i];
        uint32_t qq[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kk + e < k1) qq[e >> 2] |= (uint32_t)rp[kk + e] << (8 * (e & 3));
        bt.w[u][i] = u32x4{qq[0], qq[1], 0u, 0u};
      } else if constexpr (WK == WK_SP24F8) {
        const int v0 = k / 2 + 8 * fq;
        const uint8_t* vp = wrow[i] + v0;
        const uint8_t* mp = mrow[i] + (v0 >> 2);
        uint32_t qq[2] = {0u, 0u}, m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k + 16 * fq + 2 * e < k1 && v0 + e < kcv) qq[e >> 2] |= (uint32_t)vp[e] << (8 * (e & 3));
#pragma unroll
        for (int bq = 0; bq < 2; ++bq)
          if ((v0 >> 2) + bq < mstride) m |= (uint32_t)mp[bq] << (8 * bq);
        bt.w[u][i] = u32x4{qq[0], qq[1], 0u, 0u};
        bt.m[u][i] = m;
      } else {
        const int v0 = k / 2 + 8 * fq;
        const uint16_t* vp = reinterpret_cast<const uint16_t*>(wrow[i]) + v0;
        const uint8_t* mp = mrow[i] + (v0 >> 2);
        u32x4 v = {0u, 0u, 0u, 0u};
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k + 16 * fq + 2 * e < k1 && v0 + e < kcv) v[e >> 1] |= (uint32_t)vp[e] << (16 * (e & 1));
#pragma unroll
        for (int bq = 0; bq < 2; ++bq)
          if ((v0 >> 2) + bq < mstride) m |= (uint32_t)mp[bq] << (8 * bq);
        bt.w[u][i] = v;
        bt.m[u][i] = m;
      }
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      bt.xl[u][j] = load_x8<XL, NS, true>(xrow[j], k + 8 * fq, k1);
      if constexpr (sp_kind(WK)) bt.xh[u][j] = load_x8<XL, NS, true>(xrow[j], k + 32 + 8 * fq, k1);
    }
  };
  auto mma = [&](const Batch& bt, int u) {
    bf16x8 af[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      u32x4 wv = bt.w[u][i];
      if constexpr (WK == WK_FP8 || WK == WK_SP24F8) {
        uint32_t c0, c1, c2, c3;
        fp8x4_to_bf16x4(wv[0], c0, c1);
        fp8x4_to_bf16x4(wv[1], c2, c3);
        wv = u32x4{c0, c1, c2, c3};
      }
      af[i] = __builtin_bit_cast(bf16x8, wv);
    }
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if constexpr (sp_kind(WK)) {
        const u32x4 lo = bt.xl[u][j], hi = bt.xh[u][j];
        const u32x8 bb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x16 bv = __builtin_bit_cast(bf16x16, bb);
#pragma unroll
        for (int i = 0; i < RW; ++i)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[i], bv, acc[i][j], (int)bt.m[u][i], 0, 0);
      } else {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, bt.xl[u][j]);
#pragma unroll
        for (int i = 0; i < RW; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bv, acc[i][j], 0, 0, 0);
      }
    }
  };
  // the scheduling barrier keeps the next batch's loads ahead of this batch's matrix
  // instructions (under register pressure the scheduler would otherwise sink them)
  auto fetch = [&](Batch& bt, int kc) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) load_chunk(bt, u, kc + u * CK);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto consume = [&](const Batch& bt) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) mma(bt, u);
  };

  // whole-chunk loads need 16-byte aligned compressed rows for 2:4 weights (8-byte for
  // their e4m3 codes)
  const bool aligned = !sp_kind(WK) || (kcv & 7) == 0;
  constexpr int STEP = CK * UNROLL;
  const int nb = aligned ? (k1 - k0) / STEP : 0;   // batches of whole chunks
  if (nb > 0) {
    Batch b0, b1;
    int b = 0;
    fetch(b0, k0);
    while (b + 2 < nb) {
      fetch(b1, k0 + (b + 1) * STEP);
      consume(b0);
      fetch(b0, k0 + (b + 2) * STEP);
      consume(b1);
      b += 2;
    }
    if (b + 2 == nb) {
      fetch(b1, k0 + (b + 1) * STEP);
      consume(b0);
      consume(b1);
    } else {
      consume(b0);
    }
  }
  for (int k = k0 + nb * STEP; k < k1; k += CK) {   // ragged end, one chunk at a time
    Batch bt;
    load_chunk_checked(bt, 0, k);
    mma(bt, 0);
  }
}

// the part [k0, k1) of a segment of length k handled by wave part p of P (chunk aligned)
template <int WK>
__device__ __forceinline__ void part_range(int64_t k, int64_t p, int64_t P, int& k0, int& k1) {
  constexpr int CK = Chunk<WK>::K;
  const int64_t c = (k + CK - 1) / CK;
  const int64_t a = (p * c / P) * CK;
  int64_t b = ((p + 1) * c / P) * CK;
  if (b > k) b = k;
  k0 = (int)a;
  k1 = (int)b;
}

template <int TB> struct MaxThreads { static constexpr int V = TB >= 4 ? 512 : 1024; };

template <int TB, int RW, int WK0, int XL0, int NS, int WK1>
__global__ __launch_bounds__(MaxThreads<TB>::V) void k_few(FewSeg s0, FewSeg s1, Epi epi,
                                                          int64_t T, int64_t O, float* __restrict__ y, int64_t ldy,
                                                          int accumulate, float* __restrict__ part, int splits) {
  extern __shared__ __align__(16) float red[];   // [waves][16 * TB * 16]
  constexpr int RB = 16 * RW;                    // output rows per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wpb = blockDim.x >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int64_t nob = (O + RB - 1) / RB;
  const int64_t ob = blockIdx.x % nob;
  const int split = (int)(blockIdx.x / nob);
  int64_t orow[RW];                               // the weight rows this lane loads
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int64_t o = ob * RB + 16 * i + fr;
    orow[i] = o < O ? o : O - 1;
  }
  const int64_t P = (int64_t)splits * wpb, p = (int64_t)split * wpb + wave;

  f32x4 acc[RW][TB];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    int k0, k1;
    part_range<WK0>(s0.k, p, P, k0, k1);
    if (k0 < k1) stream_seg<TB, RW, WK0, XL0, NS>(acc, s0, orow, T, k0, k1, lane);
  }
  if constexpr (WK1 != WK_NONE) {
    int k0, k1;
    part_range<WK1>(s1.k, p, P, k0, k1);
    if (k0 < k1) stream_seg<TB, RW, WK1, XL_PLAIN, 0>(acc, s1, orow, T, k0, k1, lane);
  }

  // sum the waves' tiles in wave order, one 16-row tile at a time; element
  // e = t * 16 + (o - RB ob - 16 i)
  constexpr int PER = TB * 256;
  float* mine = red + wave * PER;
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    if (i > 0) __syncthreads();   // the previous tile's sums have been read
#pragma unroll
    for (int j = 0; j < TB; ++j) *reinterpret_cast<f32x4*>(mine + (16 * j + fr) * 16 + 4 * fq) = acc[i][j];
    __syncthreads();
    for (int e = threadIdx.x; e < PER; e += blockDim.x) {
      float sum = 0.f;
      for (int w = 0; w < wpb; ++w) sum += red[w * PER + e];
      const int64_t t = e >> 4, o = ob * RB + 16 * i + (e & 15);
      if (t >= T || o >= O) continue;
      if (part != nullptr) {
        part[((int64_t)split * T + t) * O + o] = sum;
      } else {
        float v = epi_apply(epi, sum, t, o);
        if (accumulate) v += y[t * ldy + o];
        y[t * ldy + o] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Direct-to-LDS variant for 1-2 token blocks (T <= 32).  Loading 16-byte weight
// fragments into registers makes every load instruction touch 16 rows (64 bytes each),
// and together with the X fragments that saturates the L1 address path; measured on
// gfx950, streaming the weights with global_load_lds instead (8 lanes per 128-byte row
// segment, 8 rows per instruction) recovers most of the HBM bandwidth.  Each wave owns a
// private ring of four LDS stages, each one 128-byte segment of its 16-row tiles (+ the
// 2:4 metadata); stage s+3 is requested while stage s is multiplied.  Pieces are stored
// XOR-swizzled (piece j of row r at j ^ ((r>>1)&7)) so the reads back into the matrix
// operand layout are conflict-free.  X fragments stay in registers, one stage ahead.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void g2lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}
__device__ __forceinline__ int dswz(int r) { return (r >> 1) & 7; }

template <int TB, int WK = WK_BF16> struct Dma {
  // waves per workgroup (LDS budget: four ring stages per wave; e4m3 2:4 stages are larger)
  static constexpr int WPB = TB == 1 ? (WK == WK_SP24F8 ? 12 : 16) : 8;
  static constexpr int RW = TB == 1 ? 1 : 2;     // 16-row tiles per wave (= rw_for)
};
template <int WK> struct DmaFmt {
  // chunks per stage: one 128-byte segment of every weight row
  static constexpr int U = (WK == WK_FP8 || WK == WK_SP24F8) ? 4 : 2;
  // weight bytes of reduction positions [0, kpos) of a row
  static __device__ __forceinline__ int64_t off(int kpos) {
    return WK == WK_BF16 ? 2 * (int64_t)kpos : WK == WK_SP24F8 ? (int64_t)kpos / 2 : (int64_t)kpos;
  }
};
// a wave's ring stage: RW tiles of 16 rows x 128 bytes, then the 2-bit positions of the
// stage (16 bytes per row for bf16 2:4 values, 32 for their e4m3 codes)
constexpr int dma_stage_bytes(int rw, int wk) {
  return rw * (2048 + (wk == WK_SP24 ? 256 : wk == WK_SP24F8 ? 512 : 0));
}

// XS: the segment's X row (T == 1) is staged in LDS at xs.  `pre` runs before the first
// weight stages are requested and `mid(n)` after them, n = the requests this wave issued
// in between (every wave calls this, also with an empty part, so that `mid` may hold a
// workgroup barrier).
template <int TB, int RW, int WK, int XL, int NS, bool XS, typename Pre, typename Mid>
__device__ __forceinline__ void stream_dma(f32x4 (&acc)[RW][TB], const FewSeg& sg, int64_t rbase, int64_t O,
                                           int64_t T, int k0, int k1, int lane, unsigned char* R0,
                                           unsigned char* R1, unsigned char* R2, unsigned char* R3,
                                           const uint16_t* xs, Pre&& pre, Mid&& mid) {
  constexpr int CK = Chunk<WK>::K;
  constexpr int U = DmaFmt<WK>::U;
  constexpr int SK = U * CK;   // reduction positions per stage (128 bytes of every weight row)
  constexpr int MB = WK == WK_SP24F8 ? 512 : 256;   // position bytes per tile per stage
  const int fr = lane & 15, fq = lane >> 4;
  const int kcv = (int)(sg.k / 2);
  const int mstride = (int)((sg.k + 7) >> 3);
  auto row_ptr = [&](int64_t o) -> const uint8_t* {
    o = o < O ? o : O - 1;
    if constexpr (WK == WK_BF16) return reinterpret_cast<const uint8_t*>(sg.w) + o * sg.ldw * 2;
    else if constexpr (WK == WK_FP8) return reinterpret_cast<const uint8_t*>(sg.w) + o * sg.ldw;
    else if constexpr (WK == WK_SP24F8) return reinterpret_cast<const uint8_t*>(sg.w) + o * (int64_t)kcv;
    else return reinterpret_cast<const uint8_t*>(sg.w) + o * (int64_t)kcv * 2;
  };
  // DMA sources: tile i, half h -> row 8h + lane/8, logical piece (lane&7) ^ swizzle
  const uint8_t* dsrc[RW][2];
  const uint8_t* msrc[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * h + (lane >> 3);
      dsrc[i][h] = row_ptr(rbase + 16 * i + r) + 16 * ((lane & 7) ^ dswz(r));
    }
    if constexpr (sp_kind(WK)) {
      int64_t o = rbase + 16 * i + (lane >> 2);
      o = o < O ? o : O - 1;
      msrc[i] = sg.w_meta + o * (int64_t)mstride + 4 * (lane & 3);
    }
  }
  const uint16_t* xrow[TB];
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int64_t t = 16 * j + fr;
    xrow[j] = XS ? xs : x_row<XL>(sg, t < T ? t : T - 1);
  }

  auto issue_w = [&](unsigned char* R, int st) {
    const int kpos = k0 + st * SK;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      g2lds16(dsrc[i][0] + DmaFmt<WK>::off(kpos), R + i * 2048);
      g2lds16(dsrc[i][1] + DmaFmt<WK>::off(kpos), R + i * 2048 + 1024);
      // positions: 16 rows x 16 bytes per request (lane -> row lane / 4, bytes 4 (lane % 4))
      if constexpr (sp_kind(WK)) g2lds4(msrc[i] + (kpos >> 3), R + RW * 2048 + i * MB);
      if constexpr (WK == WK_SP24F8) g2lds4(msrc[i] + (kpos >> 3) + 16, R + RW * 2048 + i * MB + 256);
    }
  };
  struct XB {
    u32x4 xl[U][TB];
    u32x4 xh[U][TB];
  };
  // lifted rows in global memory: a window pair per 16-byte load (raw row length kraw)
  constexpr bool PAIR = XL == XL_LIFT && !XS;
  const int kraw = PAIR ? (int)(sg.k / (4 * (NS - 1)) * (2 * NS)) : 0;
  auto load_x = [&](XB& xb, int st) {
    const int kpos = k0 + st * SK;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        if constexpr (PAIR) {
          xb.xl[u][j] = load_x8_lift_pair<NS>(xrow[j], kpos + u * CK + 8 * fq, kraw);
          if constexpr (sp_kind(WK)) xb.xh[u][j] = load_x8_lift_pair<NS>(xrow[j], kpos + u * CK + 32 + 8 * fq, kraw);
        } else {
          xb.xl[u][j] = load_x8<XL, NS, false>(xrow[j], kpos + u * CK + 8 * fq, 0);
          if constexpr (sp_kind(WK)) xb.xh[u][j] = load_x8<XL, NS, false>(xrow[j], kpos + u * CK + 32 + 8 * fq, 0);
        }
      }
  };
  // XS: the stage about to be read has landed once at most `later` stages' requests
  // (issued after it) are still in flight.  Without XS the waits for the X registers,
  // which are requested after their stage's weights, order the LDS reads; with X in LDS
  // nothing would, and the compiler does not order LDS reads after direct-to-LDS loads
  // on every path, so the waits are explicit.
  constexpr int OPS = 2 * RW + (WK == WK_SP24 ? RW : WK == WK_SP24F8 ? 2 * RW : 0);   // requests per stage
  auto stage_ready = [&](auto later) {
    if constexpr (XS) {
      constexpr int n = decltype(later)::value * OPS;
      __builtin_amdgcn_s_waitcnt(vm_wait(n));
    }
  };
  using L3 = std::integral_constant<int, 3>;
  using L0 = std::integral_constant<int, 0>;
  // the scheduling barriers keep each stage's LDS reads after its own wait (the
  // scheduler would otherwise hoist later stages' reads and force a full drain)
  auto compute = [&](const unsigned char* R, const XB& xb) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bf16x8 af[RW];
      int meta[RW];
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const unsigned char* tile = R + i * 2048 + (fr >> 3) * 1024 + (fr & 7) * 128;
        if constexpr (WK == WK_FP8 || WK == WK_SP24F8) {
          // 8 codes (fp8 dense: positions 8 fq of chunk u; e4m3 2:4: values 8 fq of chunk u)
          const int pc = 2 * u + (fq >> 1);
          const uint2 q = *reinterpret_cast<const uint2*>(tile + 16 * (pc ^ dswz(fr)) + 8 * (fq & 1));
          uint32_t c0, c1, c2, c3;
          fp8x4_to_bf16x4(q.x, c0, c1);
          fp8x4_to_bf16x4(q.y, c2, c3);
          af[i] = __builtin_bit_cast(bf16x8, u32x4{c0, c1, c2, c3});
        } else {
          const int pc = 4 * u + fq;
          af[i] = *reinterpret_cast<const bf16x8*>(tile + 16 * (pc ^ dswz(fr)));
        }
        if constexpr (WK == WK_SP24)
          meta[i] = *reinterpret_cast<const uint16_t*>(R + RW * 2048 + i * 256 + fr * 16 + 8 * u + 2 * fq);
        if constexpr (WK == WK_SP24F8)   // chunks 0-1 in the first 256 bytes, 2-3 in the second
          meta[i] = *reinterpret_cast<const uint16_t*>(R + RW * 2048 + i * MB + (u >> 1) * 256 + fr * 16 +
                                                       8 * (u & 1) + 2 * fq);
      }
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        if constexpr (sp_kind(WK)) {
          const u32x4 lo = xb.xl[u][j], hi = xb.xh[u][j];
          const u32x8 bb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const bf16x16 bv = __builtin_bit_cast(bf16x16, bb);
#pragma unroll
          for (int i = 0; i < RW; ++i)
            acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[i], bv, acc[i][j], meta[i], 0, 0);
        } else {
          const bf16x8 bv = __builtin_bit_cast(bf16x8, xb.xl[u][j]);
#pragma unroll
          for (int i = 0; i < RW; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bv, acc[i][j], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // whole stages need 16-byte aligned compressed rows and 4-byte aligned metadata rows
  const bool aligned = !sp_kind(WK) || (((WK == WK_SP24F8 ? kcv : 2 * kcv) & 15) == 0 && (mstride & 3) == 0);
  const int ns = (aligned && k0 < k1) ? (k1 - k0) / SK : 0;
  pre();
  if (ns > 0) {
    issue_w(R0, 0);
    if (ns > 1) issue_w(R1, 1);
    if (ns > 2) issue_w(R2, 2);
  }
  mid((ns < 3 ? ns : 3) * OPS);
  if (ns > 0) {
    XB xa, xb;
    load_x(xa, 0);
    int st = 0;
    // steady state: every step has a stage to prefetch (straight-line, so the compiler
    // waits exactly for the stage it reads)
    for (; st + 7 <= ns; st += 4) {
      issue_w(R3, st + 3);
      load_x(xb, st + 1);
      stage_ready(L3{});
      compute(R0, xa);
      issue_w(R0, st + 4);
      load_x(xa, st + 2);
      stage_ready(L3{});
      compute(R1, xb);
      issue_w(R1, st + 5);
      load_x(xb, st + 3);
      stage_ready(L3{});
      compute(R2, xa);
      issue_w(R2, st + 6);
      load_x(xa, st + 4);
      stage_ready(L3{});
      compute(R3, xb);
    }
    // the last stages (fewer than seven), prefetching only what exists
    for (; st < ns; st += 4) {
      if (st + 3 < ns) issue_w(R3, st + 3);
      if (st + 1 < ns) load_x(xb, st + 1);
      stage_ready(L0{});
      compute(R0, xa);
      if (st + 1 >= ns) break;
      if (st + 4 < ns) issue_w(R0, st + 4);
      if (st + 2 < ns) load_x(xa, st + 2);
      stage_ready(L0{});
      compute(R1, xb);
      if (st + 2 >= ns) break;
      if (st + 5 < ns) issue_w(R1, st + 5);
      if (st + 3 < ns) load_x(xb, st + 3);
      stage_ready(L0{});
      compute(R2, xa);
      if (st + 3 >= ns) break;
      if (st + 6 < ns) issue_w(R2, st + 6);
      if (st + 4 < ns) load_x(xa, st + 4);
      stage_ready(L0{});
      compute(R3, xb);
    }
  }
  // ragged end (and unaligned compressed rows): register loads, chunk by chunk
  const int kt = k0 + ns * SK;
  if (k0 < k1 && kt < k1) {
    int64_t orow[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int64_t o = rbase + 16 * i + fr;
      orow[i] = o < O ? o : O - 1;
    }
    if constexpr (XS) {
      // the staged row (selected in place when the kernel selects): one token, row 0
      FewSeg sl = sg;
      sl.x = xs;
      stream_seg<TB, RW, WK, XL, NS>(acc, sl, orow, T, kt, k1, lane);
    } else {
      stream_seg<TB, RW, WK, XL, NS>(acc, sg, orow, T, kt, k1, lane);
    }
  }
}

// Request an X row of n elements (n % 8 == 0, 16-byte aligned) into LDS by direct-to-LDS
// loads, 1 KiB (512 elements) per request, requests spread over the waves; lanes past the
// row end re-read its last 16 bytes into the tail of the last KiB (LDS holds whole KiB).
__device__ __forceinline__ void stage_row_dma(const uint16_t* __restrict__ src, int n, uint16_t* dst, int wave,
                                              int wpb, int lane) {
  const int nch = (n + 511) >> 9;
  for (int c = wave; c < nch; c += wpb) {
    int e = c * 512 + lane * 8;
    e = e <= n - 8 ? e : n - 8;
    g2lds16(src + e, dst + c * 512);
  }
}

// XS (one token): each segment's X row -- xn0 and xn1 elements, the second at the next
// KiB -- is requested into dynamic LDS before the first weight stages, so its (mostly L2)
// latency overlaps theirs, and the fragments are read from there.  Register loads of X
// between the direct-to-LDS weight loads made the compiler drain every request in flight
// before each use; LDS reads need only the explicit per-stage waits.  Same values, same
// arithmetic: bit-identical results.
// SELM > 0 (with XS, one plain segment): the staged row is X itself; after it lands every
// workgroup keeps the SELM/2 largest magnitudes of each SELM-group in place (the select
// pass's ranking, ties to the lower index) before the first multiply.
// RWV: the waves the LDS rings are sized for (the launch may not exceed it).  Rings for
// half the waves let two workgroups share a CU's LDS.
template <int TB, int WK0, int XL0, int NS, int WK1, bool XS, int SELM = 0, int QNS = 0, int RWV = Dma<TB, WK0>::WPB>
__global__ __launch_bounds__((64 * Dma<TB, WK0>::WPB)) void k_fewd(FewSeg s0, FewSeg s1, Epi epi,
                                                           int64_t T, int64_t O, float* __restrict__ y, int64_t ldy,
                                                           int accumulate, float* __restrict__ part, int splits,
                                                           int xn0, int xn1, float* __restrict__ q_out) {
  constexpr int RW = Dma<TB, WK0>::RW, WPB = RWV;
  static_assert(RWV >= 1 && RWV <= Dma<TB, WK0>::WPB, "ring waves");
  constexpr int STAGE = dma_stage_bytes(RW, WK0);   // the first segment's kind is the larger one
  static_assert(WK1 == WK_NONE || dma_stage_bytes(RW, WK1) <= STAGE, "stage size");
  static_assert(STAGE >= TB * 1024, "reduction buffer reuses stage 0");
  __shared__ __align__(16) unsigned char r0[WPB * STAGE], r1[WPB * STAGE], r2[WPB * STAGE], r3[WPB * STAGE];
  constexpr int RB = 16 * RW;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wpb = blockDim.x >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int64_t nob = (O + RB - 1) / RB;
  const int64_t ob = blockIdx.x % nob;
  const int split = (int)(blockIdx.x / nob);
  const int64_t P = (int64_t)splits * wpb, p = (int64_t)split * wpb + wave;
  f32x4 acc[RW][TB];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  unsigned char* w0 = r0 + wave * STAGE;
  unsigned char* w1 = r1 + wave * STAGE;
  unsigned char* w2 = r2 + wave * STAGE;
  unsigned char* w3 = r3 + wave * STAGE;
  extern __shared__ __align__(16) uint16_t xs_lds[];
  const int off1 = ((xn0 + 511) >> 9) << 9;   // whole KiB per staged row
  // QNS: the staged bf16 row (xn0 elements), then its lifted e4m3 codes (s0.k bytes, read
  // by the stream), then 1 KiB for the maximum's reduction
  static_assert(QNS == 0 || (XS && TB == 1 && WK0 == WK_SP24F8 && XL0 == XL_F8 && WK1 == WK_NONE), "quantize in LDS");
  uint16_t* const xs_read = QNS > 0 ? xs_lds + off1 : xs_lds;
  float qs = 1.f;   // QNS: the token scale
  {
    int k0, k1;
    part_range<WK0>(s0.k, p, P, k0, k1);
    auto pre = [&]() {
      if constexpr (XS) {
        stage_row_dma(s0.x, xn0, xs_lds, wave, wpb, lane);
        if constexpr (WK1 != WK_NONE) stage_row_dma(s1.x, xn1, xs_lds + off1, wave, wpb, lane);
      }
    };
    // this wave's X requests have landed once only the n weight requests issued after
    // them are in flight; then the barrier makes every wave's X visible
    auto mid = [&](int n) {
      if constexpr (XS) {
        switch (n) {   // 0 to 3 stages of 2, 3 or 4 requests
          case 12: __builtin_amdgcn_s_waitcnt(vm_wait(12)); break;
          case 9: __builtin_amdgcn_s_waitcnt(vm_wait(9)); break;
          case 8: __builtin_amdgcn_s_waitcnt(vm_wait(8)); break;
          case 6: __builtin_amdgcn_s_waitcnt(vm_wait(6)); break;
          case 4: __builtin_amdgcn_s_waitcnt(vm_wait(4)); break;
          case 3: __builtin_amdgcn_s_waitcnt(vm_wait(3)); break;
          case 2: __builtin_amdgcn_s_waitcnt(vm_wait(2)); break;
          default: __builtin_amdgcn_s_waitcnt(vm_wait(0)); break;
        }
        __builtin_amdgcn_s_barrier();
        if constexpr (SELM > 0) {
          // the groups are whole (xn0 % SELM == 0); LDS writes done before the barrier,
          // weight requests left in flight
          for (int g = threadIdx.x; g < xn0 / SELM; g += blockDim.x) {
            uint32_t* gp = reinterpret_cast<uint32_t*>(xs_lds + g * SELM);
            uint32_t d[SELM / 2];
#pragma unroll
            for (int q = 0; q < SELM / 2; ++q) d[q] = gp[q];
            const uint32_t keep = topn_bits_n<SELM, SELM / 2>(d);
#pragma unroll
            for (int q = 0; q < SELM / 2; ++q) {
              const uint32_t lo = ((keep >> (2 * q)) & 1u) ? 0x0000FFFFu : 0u;
              const uint32_t hi = ((keep >> (2 * q + 1)) & 1u) ? 0xFFFF0000u : 0u;
              gp[q] = d[q] & (lo | hi);
            }
          }
          __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes done
          __builtin_amdgcn_s_barrier();
        }
        if constexpr (QNS > 0) {
          // the row's largest magnitude pattern, the token's scales, then the codes (the
          // quantizing pass's arithmetic), with the weight requests still in flight
          uint32_t* red = reinterpret_cast<uint32_t*>(xs_lds + off1 + (((s0.k >> 1) + 511) >> 9 << 9));
          uint32_t mk = 0;
          for (int c = threadIdx.x; c < xn0 / 8; c += blockDim.x) {
            const uint4 v = *reinterpret_cast<const uint4*>(xs_lds + 8 * c);
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t lo = d[q] & 0x7FFFu, hi = (d[q] >> 16) & 0x7FFFu;
              mk = lo > mk ? lo : mk;
              mk = hi > mk ? hi : mk;
            }
          }
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)mk, off, 64);
            mk = o > mk ? o : mk;
          }
          if (lane == 0) red[wave] = mk;
          __builtin_amdgcn_s_waitcnt(0xC07F);
          __builtin_amdgcn_s_barrier();
          mk = red[0];
          for (int w = 1; w < wpb; ++w) mk = red[w] > mk ? red[w] : mk;
          float r;
          token_scales(mk, r, qs);
          if (blockIdx.x == 0 && threadIdx.x == 0 && q_out != nullptr) q_out[0] = qs;
          constexpr int W = QNS - 1;
          uint32_t* codes = reinterpret_cast<uint32_t*>(xs_read);
          for (int g = threadIdx.x; g < xn0 / (2 * QNS); g += blockDim.x) {
            uint32_t v16[2 * QNS];
#pragma unroll
            for (int i = 0; i < 2 * QNS; ++i) v16[i] = xs_lds[g * 2 * QNS + i];
            uint32_t win[W];
            quant_lift_group<QNS>(v16, r, win);
#pragma unroll
            for (int w = 0; w < W; ++w) codes[g * W + w] = win[w];
          }
          __builtin_amdgcn_s_waitcnt(0xC07F);
          __builtin_amdgcn_s_barrier();
        }
      }
    };
    stream_dma<TB, RW, WK0, XL0, NS, XS>(acc, s0, ob * RB, O, T, k0, k1, lane, w0, w1, w2, w3, xs_read, pre, mid);
  }
  if constexpr (WK1 != WK_NONE) {
    int k0, k1;
    part_range<WK1>(s1.k, p, P, k0, k1);
    if (k0 < k1)
      stream_dma<TB, RW, WK1, XL_PLAIN, 0, XS>(acc, s1, ob * RB, O, T, k0, k1, lane, w0, w1, w2, w3, xs_lds + off1,
                                               []() {}, [](int) {});
  }
  // sum the waves' tiles in wave order through stage 0's memory (one 16 x 16 token block
  // at a time); element e = t_local * 16 + (o - RB ob - 16 i)
  __syncthreads();
  float* red = reinterpret_cast<float*>(r0);
#pragma unroll
  for (int i = 0; i < RW; ++i) {
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if (i + j > 0) __syncthreads();
      *reinterpret_cast<f32x4*>(red + wave * 256 + fr * 16 + 4 * fq) = acc[i][j];
      __syncthreads();
      for (int e = threadIdx.x; e < 256; e += blockDim.x) {
        float sum = 0.f;
        for (int w = 0; w < wpb; ++w) sum += red[w * 256 + e];
        const int64_t t = 16 * j + (e >> 4), o = ob * RB + 16 * i + (e & 15);
        if (t >= T || o >= O) continue;
        if (part != nullptr) {
          part[((int64_t)split * T + t) * O + o] = sum;
        } else if constexpr (QNS > 0) {
          // the token scale from LDS (row_scale[0] is written by workgroup 0 for the reduction)
          Epi e = epi;
          e.row_scale = nullptr;
          float v = qs * epi_apply(e, sum, t, o);
          if (accumulate) v += y[t * ldy + o];
          y[t * ldy + o] = v;
        } else {
          float v = epi_apply(epi, sum, t, o);
          if (accumulate) v += y[t * ldy + o];
          y[t * ldy + o] = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Single token with K-major weights Wk [K][O]:  y[o] = sum_{k kept} x[k] * Wk[k][o].
// With one token the selection keeps n of every m inputs, so only those K-rows of the
// weights are read (n/m of the bytes) -- each a contiguous run of the output dimension.
// Workgroup (k-span, o-chunk): select the span's groups of x in registers (top-n by
// magnitude, ties to the lower index: the same rule as the select kernel), list the kept
// (k, x[k]) in LDS in ascending k (exactly n per group, so every slot is known), then
// stream those rows' o-chunk with 16-byte loads, 8 rows in flight per thread, and write
// the span's fp32 partial sums; a second kernel adds the spans in order.
constexpr int G1_THREADS = 512;
constexpr int G1_MAX_SPAN = 2048;

template <int M>
__global__ __launch_bounds__(G1_THREADS) void k_gather1(const uint16_t* __restrict__ x, int64_t K, int n,
                                                       const uint16_t* __restrict__ wk, int64_t O, int kspan,
                                                       int ochunk, int nochunk, float* __restrict__ part,
                                                       uint32_t* __restrict__ mask_out) {
  __shared__ int sk[G1_MAX_SPAN];
  __shared__ float sv[G1_MAX_SPAN];
  __shared__ uint32_t mw[G1_MAX_SPAN / 32];
  __shared__ __align__(16) float red[G1_THREADS * 8];
  const int tid = threadIdx.x;
  const int oc = (int)(blockIdx.x % nochunk);
  const int ks = (int)(blockIdx.x / nochunk);
  const int64_t k0 = (int64_t)ks * kspan;
  const int span = (int)((k0 + kspan <= K) ? kspan : K - k0);
  const int groups = span / M;
  const bool want_mask = mask_out != nullptr && oc == 0;
  if (want_mask)
    for (int w = tid; w < (span + 31) / 32; w += G1_THREADS) mw[w] = 0u;
  __syncthreads();
  for (int g = tid; g < groups; g += G1_THREADS) {
    uint32_t d[M / 2];
    const uint32_t* src = reinterpret_cast<const uint32_t*>(x + k0 + (int64_t)g * M);
#pragma unroll
    for (int q = 0; q < M / 2; ++q) d[q] = src[q];
    const uint32_t bits = topn_bits<M>(d, n);
    int slot = g * n;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if ((bits >> i) & 1u) {
        const uint32_t b = (d[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        sk[slot] = (int)(k0 + (int64_t)g * M + i);
        sv[slot] = __uint_as_float(b << 16);
        ++slot;
      }
    }
    if (want_mask) atomicOr(&mw[(g * M) >> 5], (M == 32 ? bits : bits << ((g * M) & 31)));
  }
  __syncthreads();
  if (want_mask)
    for (int w = tid; w < (span + 31) / 32; w += G1_THREADS) mask_out[(k0 >> 5) + w] = mw[w];

  const int lanes_o = ochunk / 8;                 // threads across the o-chunk
  const int nkl = G1_THREADS / lanes_o;           // threads along the kept list
  const int kl = tid / lanes_o, lo = tid % lanes_o;
  const int64_t o0 = (int64_t)oc * ochunk + 8 * lo;
  const int nsel = groups * n;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (o0 < O) {
    // software pipeline: batch b+1 (8 kept rows) is requested before batch b is used
    const uint16_t* wcol = wk + o0;
    struct B8 {
      u32x4 w[8];
      float v[8];
    };
    auto fetch = [&](B8& bt, int e) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int ee = e + q * nkl;
        bt.w[q] = *reinterpret_cast<const u32x4*>(wcol + (int64_t)sk[ee] * O);
        bt.v[q] = sv[ee];
      }
    };
    auto use = [&](const B8& bt) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[2 * c] += bt.v[q] * __uint_as_float(bt.w[q][c] << 16);
          acc[2 * c + 1] += bt.v[q] * __uint_as_float(bt.w[q][c] & 0xFFFF0000u);
        }
    };
    const int stride = 8 * nkl;
    const int nb = (nsel - kl + stride - 1) / stride > 0 ? (nsel - kl) / stride : 0;   // whole batches
    int e = kl;
    if (nb > 0) {
      B8 b0, b1;
      int b = 0;
      fetch(b0, e);
      while (b + 2 < nb) {
        fetch(b1, e + stride);
        use(b0);
        fetch(b0, e + 2 * stride);
        use(b1);
        b += 2;
        e += 2 * stride;
      }
      if (b + 2 == nb) {
        fetch(b1, e + stride);
        use(b0);
        use(b1);
        e += 2 * stride;
      } else {
        use(b0);
        e += stride;
      }
    }
    // the ragged end (fewer than 8 rows per thread: nsel - e < stride): requested together,
    // rows past the list re-read the first one and are not added; same order as a batch
    if (e < nsel) {
      B8 bt;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int ee = e + q * nkl;
        const int es = ee < nsel ? ee : e;
        bt.w[q] = *reinterpret_cast<const u32x4*>(wcol + (int64_t)sk[es] * O);
        bt.v[q] = sv[es];
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (e + q * nkl < nsel) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            acc[2 * c] += bt.v[q] * __uint_as_float(bt.w[q][c] << 16);
            acc[2 * c + 1] += bt.v[q] * __uint_as_float(bt.w[q][c] & 0xFFFF0000u);
          }
        }
      }
    }
  }
  // add the list lanes in order, write the span's partial sums
#pragma unroll
  for (int q = 0; q < 8; ++q) red[kl * ochunk + 8 * lo + q] = acc[q];
  __syncthreads();
  for (int i = tid; i < ochunk; i += G1_THREADS) {
    const int64_t o = (int64_t)oc * ochunk + i;
    if (o >= O) continue;
    float sum = 0.f;
    for (int l = 0; l < nkl; ++l) sum += red[l * ochunk + i];
    part[(int64_t)ks * O + o] = sum;
  }
}

struct G1Plan {
  int kspan, ochunk, nochunk;
  int64_t nks;
};

G1Plan g1_plan(int64_t k, int64_t o, int m) {
  G1Plan p;
  int oc = 64;
  while (oc < 1024 && oc < o) oc *= 2;
  p.ochunk = oc;
  p.nochunk = (int)((o + oc - 1) / oc);
  const int64_t target = (256 + p.nochunk - 1) / p.nochunk;   // about one workgroup per CU
  int64_t span = (k + target - 1) / target;
  const int unit = m > 32 ? m : 32;                           // whole mask words and groups
  span = (span + unit - 1) / unit * unit;
  if (span > G1_MAX_SPAN) span = G1_MAX_SPAN;
  if (span < unit) span = unit;
  p.kspan = (int)span;
  p.nks = (k + span - 1) / span;
  return p;
}

// y = w_scale * sum of the partial tiles, accumulated or stored.  A workgroup owns 64
// consecutive outputs; its 4 thread lanes per output take every 4th partial (unrolled,
// so many loads are in flight) and the 4 lane sums are added in lane order.  Fixed
// order throughout: results do not depend on timing.
constexpr int RP_OUT = 64, RP_LANES = 4;

__global__ __launch_bounds__(RP_OUT * RP_LANES) void k_reduce_parts(const float* __restrict__ part, int64_t splits,
                                                                   Epi epi, int64_t T,
                                                                   int64_t O, float* __restrict__ y, int64_t ldy,
                                                                   int accumulate) {
  __shared__ float sums[RP_LANES][RP_OUT];
  const int lo = threadIdx.x % RP_OUT, sl = threadIdx.x / RP_OUT;
  const int64_t n = T * O;
  const int64_t i = (int64_t)blockIdx.x * RP_OUT + lo;
  float acc = 0.f;
  if (i < n) {
    const float* p = part + i;
    int64_t sp = sl;
    for (; sp + 7 * RP_LANES < splits; sp += 8 * RP_LANES) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = p[(sp + q * RP_LANES) * n];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc += v[q];
    }
    for (; sp < splits; sp += RP_LANES) acc += p[sp * n];
  }
  sums[sl][lo] = acc;
  __syncthreads();
  if (sl != 0 || i >= n) return;
  float sum = sums[0][lo];
#pragma unroll
  for (int l = 1; l < RP_LANES; ++l) sum += sums[l][lo];
  const int64_t t = i / O, o = i - t * O;
  float v = epi_apply(epi, sum, t, o);
  if (accumulate) v += y[t * ldy + o];
  y[t * ldy + o] = v;
}

// Few splits over many outputs (the split-K tile kernels): each thread owns 4 consecutive
// outputs and adds the splits' float4 partials in split order.  The partials of up to
// RP4_BATCH splits are requested together before the first add (one memory round trip
// per batch, not one per split past the first four).
constexpr int RP4_THREADS = 256;
constexpr int RP4_BATCH = 16;

__global__ __launch_bounds__(RP4_THREADS) void k_reduce_parts4(const float* __restrict__ part, int64_t splits,
                                                               Epi epi, int64_t T,
                                                               int64_t O, float* __restrict__ y, int64_t ldy,
                                                               int accumulate) {
  const int64_t n = T * O;
  const int64_t i = ((int64_t)blockIdx.x * RP4_THREADS + threadIdx.x) * 4;
  if (i >= n) return;
  const float* p = part + i;
  float4 acc = *reinterpret_cast<const float4*>(p);   // split 0 (its bits kept, -0 included)
  for (int64_t s0 = 1; s0 < splits; s0 += RP4_BATCH) {
    float4 v[RP4_BATCH];
#pragma unroll
    for (int q = 0; q < RP4_BATCH; ++q)
      if (s0 + q < splits) v[q] = *reinterpret_cast<const float4*>(p + (s0 + q) * n);
#pragma unroll
    for (int q = 0; q < RP4_BATCH; ++q) {
      if (s0 + q < splits) {
        acc.x += v[q].x;
        acc.y += v[q].y;
        acc.z += v[q].z;
        acc.w += v[q].w;
      }
    }
  }
  const int64_t t = i / O, o = i - t * O;   // O % 4 == 0: the 4 outputs share a row
  if (epi.w_scale != nullptr) {
    acc.x *= epi.w_scale[o];
    acc.y *= epi.w_scale[o + 1];
    acc.z *= epi.w_scale[o + 2];
    acc.w *= epi.w_scale[o + 3];
  }
  if (epi.extra()) {
    const float rs = epi.row_scale != nullptr ? epi.row_scale[t] : 1.f;
    const float rb = epi.col_shift != nullptr ? (epi.row_shift != nullptr ? epi.row_shift[t] : 1.f) : 0.f;
    const float4 cs = epi.col_shift != nullptr ? *reinterpret_cast<const float4*>(epi.col_shift + o)
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
    acc.x = acc.x * rs + rb * cs.x;
    acc.y = acc.y * rs + rb * cs.y;
    acc.z = acc.z * rs + rb * cs.z;
    acc.w = acc.w * rs + rb * cs.w;
  }
  float4* yp = reinterpret_cast<float4*>(y + t * ldy + o);
  if (accumulate) {
    const float4 c = *yp;
    acc.x += c.x;
    acc.y += c.y;
    acc.z += c.z;
    acc.w += c.w;
  }
  *yp = acc;
}

// X[:, c0] then X[:, c1] side by side: xo[t][j] = x[t][c0[j]] (j < k0),
// xo[t][off1 + j] = x[t][c1[j]] (j < k1).  Column indices are clamped to [0, kx).
// Element by element: the form for layouts the row kernel below does not take.
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

// The same gather a token row per workgroup: the row is read into LDS with 16-byte loads,
// then each thread gathers 8 consecutive outputs from LDS (column indices read as two
// 16-byte pieces) and writes them as one 16-byte piece.  The first pieces' indices are
// requested before the row, so the two reads overlap instead of following each other.
// Needs kx, ldx, k0, k1, off1 and ldo multiples of 8 and 16-byte aligned x and xo; the row
// takes kx * 2 bytes of LDS.
constexpr int PERM_THREADS = 256;
constexpr int PERM_BATCH = 4;   // 8-output pieces per thread whose indices are in flight together
__global__ __launch_bounds__(PERM_THREADS) void k_permute_rows(const uint16_t* __restrict__ x, int64_t ldx, int kx,
                                                               const int32_t* __restrict__ c0, int k0,
                                                               const int32_t* __restrict__ c1, int k1, int64_t off1,
                                                               uint16_t* __restrict__ xo, int64_t ldo) {
  extern __shared__ __align__(16) uint16_t xrow[];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const uint16_t* src = x + t * ldx;
  uint16_t* dst = xo + t * ldo;
  const int n8 = (k0 + k1) / 8;
  int4 ia[PERM_BATCH], ib[PERM_BATCH];
  auto load_idx = [&](int p0) {
#pragma unroll
    for (int q = 0; q < PERM_BATCH; ++q) {
      const int p = p0 + q * PERM_THREADS + tid;
      if (p < n8) {
        const int j = 8 * p;
        const int32_t* cl = j < k0 ? c0 + j : c1 + (j - k0);
        ia[q] = *reinterpret_cast<const int4*>(cl);
        ib[q] = *reinterpret_cast<const int4*>(cl + 4);
      }
    }
  };
  load_idx(0);
  for (int c = tid; c < kx / 8; c += PERM_THREADS)
    *reinterpret_cast<uint4*>(xrow + 8 * c) = *reinterpret_cast<const uint4*>(src + 8 * c);
  __syncthreads();
  for (int p0 = 0; p0 < n8; p0 += PERM_BATCH * PERM_THREADS) {
    if (p0 > 0) load_idx(p0);
#pragma unroll
    for (int q = 0; q < PERM_BATCH; ++q) {
      const int p = p0 + q * PERM_THREADS + tid;
      if (p >= n8) continue;
      const int j = 8 * p;
      const int idx[8] = {ia[q].x, ia[q].y, ia[q].z, ia[q].w, ib[q].x, ib[q].y, ib[q].z, ib[q].w};
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int a = idx[2 * e], b = idx[2 * e + 1];
        a = a < 0 ? 0 : (a >= kx ? kx - 1 : a);
        b = b < 0 ? 0 : (b >= kx ? kx - 1 : b);
        w[e] = (uint32_t)xrow[a] | ((uint32_t)xrow[b] << 16);
      }
      *reinterpret_cast<uint4*>(dst + (j < k0 ? j : off1 + (j - k0))) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

struct Plan {
  int tb, rw, wpb;
  int64_t splits;
};

Plan make_plan(const FewArgs& a, bool allow_split) {
  Plan p;
  p.tb = a.t <= 16 ? 1 : a.t <= 32 ? 2 : a.t <= 64 ? 4 : 8;
  p.rw = rw_for(p.tb, a.seg[0].w_kind);
  // waves per workgroup: LDS rings bound the direct-to-LDS kernels (16 waves for one token
  // block, 8 for two); 4 measured best for the register kernel at four token blocks
  const int max_wpb = p.tb == 1 ? (a.seg[0].w_kind == WK_SP24F8 ? Dma<1, WK_SP24F8>::WPB : 16) : p.tb == 4 ? 4 : 8;
  int64_t chunks = 0;   // chunks of the longest segment
  for (int i = 0; i < a.nseg; ++i) {
    const int ck = sp_kind(a.seg[i].w_kind) ? 64 : 32;
    const int64_t c = (a.seg[i].k + ck - 1) / ck;
    chunks = c > chunks ? c : chunks;
  }
  const int ew = a.route.few_wpb, es = a.route.few_splits;   // caller's partition (0: chosen here)
  const int64_t nob = (a.o + 16 * p.rw - 1) / (16 * p.rw);
  // about one workgroup of max_wpb waves per CU (256 CUs); many row blocks -> fewer waves
  // per block, few row blocks -> the reduction is also split across workgroups
  int wpb = max_wpb;
  int64_t splits = 1;
  if (nob >= 256) {
    // past one workgroup per CU: the direct-to-LDS kernels take half the waves on rings
    // sized for them, two workgroups per CU (measured at 14336 and 21504 rows, 1 and 8
    // tokens: 16-27% faster than whole rings with 16 waves, 5-11% faster than with 4 waves
    // on half rings); the register kernel keeps 4 (two segments: 8, since each wave's parts
    // are short and more waves keep more of them in flight)
    const int floor_wpb = p.tb <= 2 ? max_wpb / 2 : (a.nseg == 2 && max_wpb >= 8) ? 8 : 4;
    while (wpb > floor_wpb && nob * wpb > 256 * max_wpb) wpb /= 2;
  } else if (allow_split) {
    splits = (256 + nob - 1) / nob;
  }
  // keep at least two chunks per wave part
  if (splits > 1 && splits * wpb * 2 > chunks) splits = chunks / (2 * wpb) > 1 ? chunks / (2 * wpb) : 1;
  while (wpb > 4 && splits * wpb * 2 > chunks) wpb /= 2;
  if (ew == 4 || ew == 8 || (ew == 16 && max_wpb == 16)) wpb = ew;
  if (es > 0 && allow_split) splits = es;
  p.wpb = wpb;
  p.splits = splits;
  return p;
}

template <int TB, int WK0, int XL0, int NS, int WK1>
hipError_t launch_k(const FewArgs& a, const Plan& p, float* part, hipStream_t s) {
  constexpr int RW = rw_for(TB, WK0);
  const int64_t nob = (a.o + 16 * RW - 1) / (16 * RW);
  const int64_t blocks = nob * p.splits;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const FewSeg s1 = a.nseg > 1 ? a.seg[1] : FewSeg{};
  float* pp = p.splits > 1 ? part : nullptr;
  if constexpr (TB <= 2) {
    static_assert(RW == Dma<TB, WK0>::RW, "row tiles");
    if (p.wpb > Dma<TB, WK0>::WPB) return hipErrorInvalidConfiguration;
    // at most half the waves the rings are sized for: rings for half of them, so that two
    // workgroups share a CU's LDS (the plain kernels; selection and quantization keep
    // whole rings)
    constexpr int HALFW = Dma<TB, WK0>::WPB / 2;
    const bool half = p.wpb <= HALFW && a.sel_m == 0 && a.q_ns == 0;
    if constexpr (TB == 1 && XL0 != XL_BLK) {
      // one token: stage the X rows in LDS next to the weight rings when they fit
      // (the NM_ROUTE_NO_XLDS hint keeps the register loads)
      // rows of whole 16-byte pieces from 16-byte aligned starts, staged in whole KiB
      // (in 2-byte units: an e4m3 row of k codes is k / 2 of them; quantized in the kernel:
      // the bf16 row, then its codes and 1 KiB for the maximum)
      const int qn = XL0 == XL_F8 ? a.q_ns : 0;
      const int64_t xn0 = XL0 == XL_LIFT ? a.seg[0].k / (4 * (NS - 1)) * (2 * NS)
                          : qn > 0       ? a.seg[0].k / (4 * (qn - 1)) * (2 * qn)
                          : XL0 == XL_F8 ? a.seg[0].k / 2
                                         : a.seg[0].k;
      const int64_t xn1 = a.nseg > 1 ? a.seg[1].k : 0;
      const int64_t xbytes = (((xn0 + 511) >> 9) + ((xn1 + 511) >> 9) + (qn > 0 ? ((a.seg[0].k / 2 + 511) >> 9) + 1 : 0)) * 1024;
      const int64_t full_ring = 4LL * Dma<TB, WK0>::WPB * dma_stage_bytes(RW, WK0);
      const int64_t half_ring = 4LL * HALFW * dma_stage_bytes(RW, WK0);
      auto piece_ok = [](const uint16_t* x, int64_t n) {
        return n == 0 || (n >= 8 && (n % 8) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0);
      };
      const bool rows_ok = piece_ok(a.seg[0].x, xn0) && (a.nseg < 2 || piece_ok(a.seg[1].x, xn1)) && xn0 > 0;
      // half rings only while two workgroups with their staged rows still share a CU;
      // otherwise one workgroup per CU, with every wave the whole rings serve.  Two-segment
      // (hybrid) rows too long to fit beside whole rings get rings for three quarters of
      // the waves (measured, 4096 x 14336 hybrid at one token: 19.2 us against 25.0 us
      // with X read from global memory; one-segment 2:4 weights were faster with X from
      // global memory and all 16 waves, 16.6 against 18.5 us, so they keep that)
      const bool half_x = half && 2 * (half_ring + xbytes) <= 163840;
      constexpr int TQW = 3 * Dma<TB, WK0>::WPB / 4;
      const bool tq_x = !half && WK1 != WK_NONE && a.nseg == 2 && a.sel_m == 0 && a.q_ns == 0 &&
                        full_ring + xbytes > 163840 && 4LL * TQW * dma_stage_bytes(RW, WK0) + xbytes <= 163840;
      const int wpb_x = tq_x ? TQW : half && !half_x ? Dma<TB, WK0>::WPB : p.wpb;
      const int64_t ring_x = half_x ? half_ring : tq_x ? 4LL * TQW * dma_stage_bytes(RW, WK0) : full_ring;
      if (a.t == 1 && rows_ok && ring_x + xbytes <= 163840 && !a.route.has(NM_ROUTE_NO_XLDS)) {
        auto kern = k_fewd<TB, WK0, XL0, NS, WK1, true>;
        if (half_x) kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 0, 0, HALFW>;
        if constexpr (WK1 != WK_NONE) {
          if (tq_x) kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 0, 0, TQW>;
        }
        if constexpr (WK0 == WK_SP24F8 && XL0 == XL_F8 && WK1 == WK_NONE) {
          switch (qn) {
            case 0: break;
            case 2: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 0, 2>; break;
            case 3: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 0, 3>; break;
            case 4: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 0, 4>; break;
            case 5: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 0, 5>; break;
            case 6: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 0, 6>; break;
            case 7: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 0, 7>; break;
            case 8: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 0, 8>; break;
            default: return hipErrorInvalidValue;
          }
        }
        if constexpr (XL0 == XL_PLAIN && WK1 == WK_NONE && (WK0 == WK_BF16 || WK0 == WK_FP8)) {
          switch (a.sel_m) {
            case 0: break;
            case 4: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 4>; break;
            case 8: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 8>; break;
            case 16: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 16>; break;
            case 32: kern = k_fewd<TB, WK0, XL0, NS, WK1, true, 32>; break;
            default: return hipErrorInvalidValue;
          }
        } else if (a.sel_m != 0) {
          return hipErrorInvalidValue;
        }
        hipError_t ae = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)xbytes);
        if (ae != hipSuccess) return ae;
        a.route.note(NM_TAKEN_FEW_STREAM | NM_TAKEN_FEW_XLDS | (a.sel_m != 0 ? NM_TAKEN_FEW_SELECT : 0u) |
                     (sp_kind(WK0) ? NM_TAKEN_SPARSE_MMA : 0u) | (qn > 0 ? NM_TAKEN_QUANT : 0u));
        kern<<<dim3((unsigned)blocks), dim3(64 * wpb_x), (size_t)xbytes, s>>>(
            a.seg[0], s1, a.epi(), a.t, a.o, a.y, a.ldy, a.accumulate, pp, (int)p.splits, (int)xn0, (int)xn1,
            qn > 0 ? const_cast<float*>(a.row_scale) : nullptr);
        return hipGetLastError();
      }
    }
    if (a.sel_m != 0 || a.q_ns != 0) return hipErrorInvalidValue;   // these need the staged row
    a.route.note(NM_TAKEN_FEW_STREAM | (sp_kind(WK0) ? NM_TAKEN_SPARSE_MMA : 0u));
    auto kern = k_fewd<TB, WK0, XL0, NS, WK1, false>;
    if (half) kern = k_fewd<TB, WK0, XL0, NS, WK1, false, 0, 0, HALFW>;
    kern<<<dim3((unsigned)blocks), dim3(64 * p.wpb), 0, s>>>(a.seg[0], s1, a.epi(), a.t, a.o, a.y, a.ldy,
                                                            a.accumulate, pp, (int)p.splits, 0, 0, nullptr);
  } else {
    auto kern = k_few<TB, RW, WK0, XL0, NS, WK1>;
    const size_t lds = (size_t)p.wpb * TB * 1024;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    if (a.sel_m != 0 || a.q_ns != 0) return hipErrorInvalidValue;
    a.route.note(NM_TAKEN_FEW_STREAM | (sp_kind(WK0) ? NM_TAKEN_SPARSE_MMA : 0u));
    kern<<<dim3((unsigned)blocks), dim3(64 * p.wpb), lds, s>>>(a.seg[0], s1, a.epi(), a.t, a.o, a.y, a.ldy,
                                                               a.accumulate, pp, (int)p.splits);
  }
  return hipGetLastError();
}

template <int WK0, int XL0, int NS, int WK1>
hipError_t launch_tb(const FewArgs& a, const Plan& p, float* part, hipStream_t s) {
  switch (p.tb) {
    case 1: return launch_k<1, WK0, XL0, NS, WK1>(a, p, part, s);
    case 2: return launch_k<2, WK0, XL0, NS, WK1>(a, p, part, s);
    case 4: return launch_k<4, WK0, XL0, NS, WK1>(a, p, part, s);
    default: return launch_k<8, WK0, XL0, NS, WK1>(a, p, part, s);
  }
}

hipError_t launch_lift(const FewArgs& a, const Plan& p, float* part, hipStream_t s) {
  switch (a.seg[0].ns) {
    case 2: return launch_tb<WK_SP24, XL_LIFT, 2, WK_NONE>(a, p, part, s);
    case 3: return launch_tb<WK_SP24, XL_LIFT, 3, WK_NONE>(a, p, part, s);
    case 4: return launch_tb<WK_SP24, XL_LIFT, 4, WK_NONE>(a, p, part, s);
    case 5: return launch_tb<WK_SP24, XL_LIFT, 5, WK_NONE>(a, p, part, s);
    case 6: return launch_tb<WK_SP24, XL_LIFT, 6, WK_NONE>(a, p, part, s);
    case 7: return launch_tb<WK_SP24, XL_LIFT, 7, WK_NONE>(a, p, part, s);
    case 8: return launch_tb<WK_SP24, XL_LIFT, 8, WK_NONE>(a, p, part, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

namespace nml {

int64_t few_partial_bytes(const FewArgs& a) {
  if (a.t <= 0 || a.o <= 0) return 0;
  const Plan p = make_plan(a, true);
  return p.splits > 1 ? p.splits * a.t * a.o * 4 : 0;
}

bool few_select_in_kernel(const FewArgs& a) {
  if (a.route.has(NM_ROUTE_NO_FEW_SELECT) || a.route.has(NM_ROUTE_NO_XLDS)) return false;
  if (a.t != 1 || a.nseg != 1 || a.o <= 0) return false;
  const int m = a.sel_m;
  if (m != 4 && m != 8 && m != 16 && m != 32) return false;
  const FewSeg& sg = a.seg[0];
  if (sg.loader != XL_PLAIN || (sg.w_kind != WK_BF16 && sg.w_kind != WK_FP8)) return false;
  const int64_t n = sg.k;
  if (n < 8 || n % 8 != 0 || n % m != 0 || (reinterpret_cast<uintptr_t>(sg.x) & 15) != 0) return false;
  // the staged row beside the weight ring (one token block: dense stages of 2 KiB)
  const int64_t ring = 4LL * Dma<1>::WPB * dma_stage_bytes(1, sg.w_kind);
  if (ring + ((n + 511) >> 9) * 1024 > 163840) return false;
  return make_plan(a, true).tb == 1;
}

bool few_quant_in_kernel(const FewArgs& a) {
  if (a.route.has(NM_ROUTE_NO_XLDS)) return false;
  if (a.t != 1 || a.nseg != 1 || a.o <= 0 || a.sel_m != 0) return false;
  const FewSeg& sg = a.seg[0];
  const int q = a.q_ns;
  if (sg.w_kind != WK_SP24F8 || sg.loader != XL_F8 || q < 2 || q > 8 || a.row_scale == nullptr) return false;
  if (sg.k <= 0 || sg.k % (4 * (q - 1)) != 0) return false;
  const int64_t kx = sg.k / (4 * (q - 1)) * (2 * q);   // the bf16 row's length
  if (kx < 8 || kx % 8 != 0 || (reinterpret_cast<uintptr_t>(sg.x) & 15) != 0) return false;
  const int64_t xbytes = (((kx + 511) >> 9) + ((sg.k / 2 + 511) >> 9) + 1) * 1024;
  const int64_t ring = 4LL * Dma<1, WK_SP24F8>::WPB * dma_stage_bytes(1, WK_SP24F8);
  if (ring + xbytes > 163840) return false;
  return make_plan(a, true).tb == 1;
}

hipError_t launch_few(const FewArgs& a, float* part, int64_t part_bytes, hipStream_t s) {
  if (a.t > 128 || a.nseg < 1 || a.nseg > 2) return hipErrorInvalidValue;
  for (int i = 0; i < a.nseg; ++i)   // reduction indices are 32-bit inside the kernel
    if (a.seg[i].k > 0x3FFFFFFF) return hipErrorInvalidValue;
  if (a.t == 0 || a.o == 0) return hipSuccess;
  if (a.sel_m != 0 && !few_select_in_kernel(a)) return hipErrorInvalidValue;
  if (a.q_ns != 0 && !few_quant_in_kernel(a)) return hipErrorInvalidValue;
  Plan p = make_plan(a, part != nullptr);
  if (p.splits > 1 && part_bytes < p.splits * a.t * a.o * 4) p = make_plan(a, false);
  const FewSeg& s0 = a.seg[0];
  hipError_t e = hipErrorInvalidValue;
  if (a.nseg == 2) {
    if (s0.w_kind == WK_SP24 && s0.loader == XL_PLAIN && a.seg[1].w_kind == WK_BF16 && a.seg[1].loader == XL_PLAIN)
      e = launch_tb<WK_SP24, XL_PLAIN, 0, WK_BF16>(a, p, part, s);
  } else if (s0.w_kind == WK_BF16 && s0.loader == XL_PLAIN) {
    e = launch_tb<WK_BF16, XL_PLAIN, 0, WK_NONE>(a, p, part, s);
  } else if (s0.w_kind == WK_FP8 && s0.loader == XL_PLAIN) {
    e = launch_tb<WK_FP8, XL_PLAIN, 0, WK_NONE>(a, p, part, s);
  } else if (s0.w_kind == WK_SP24 && s0.loader == XL_PLAIN) {
    e = launch_tb<WK_SP24, XL_PLAIN, 0, WK_NONE>(a, p, part, s);
  } else if (s0.w_kind == WK_SP24 && s0.loader == XL_LIFT) {
    e = launch_lift(a, p, part, s);
  } else if (s0.w_kind == WK_SP24F8 && s0.loader == XL_F8 && p.tb == 1) {
    e = launch_k<1, WK_SP24F8, XL_F8, 0, WK_NONE>(a, p, part, s);
  } else if (s0.loader == XL_BLK && a.t >= 2 && (s0.w_kind == WK_BF16 || s0.w_kind == WK_FP8) && p.tb <= 2) {
    // token-blocked S(X) (2-32 tokens, weight-streaming kernel only)
    if (s0.w_kind == WK_BF16)
      e = p.tb == 1 ? launch_k<1, WK_BF16, XL_BLK, 0, WK_NONE>(a, p, part, s)
                    : launch_k<2, WK_BF16, XL_BLK, 0, WK_NONE>(a, p, part, s);
    else
      e = p.tb == 1 ? launch_k<1, WK_FP8, XL_BLK, 0, WK_NONE>(a, p, part, s)
                    : launch_k<2, WK_FP8, XL_BLK, 0, WK_NONE>(a, p, part, s);
  }
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_reduce_parts(part, p.splits, a.epi(), a.t, a.o, a.y, a.ldy, a.accumulate, a.route, s);
}

int64_t gather1_part_bytes(int64_t k, int64_t o, int m) {
  if (k <= 0 || o <= 0) return 0;
  return g1_plan(k, o, m).nks * o * 4;
}

hipError_t launch_gather1(int m, const uint16_t* x, int64_t k, int n, const uint16_t* wk, int64_t o, float* y,
                          int accumulate, uint32_t* mask_out, float* part, int64_t part_bytes, const Route& r,
                          hipStream_t s) {
  const G1Plan p = g1_plan(k, o, m);
  if (part == nullptr || part_bytes < p.nks * o * 4 || (o % 8) != 0) return hipErrorInvalidValue;
  const int64_t blocks = p.nks * p.nochunk;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)blocks), b(G1_THREADS);
  switch (m) {
    case 4: k_gather1<4><<<g, b, 0, s>>>(x, k, n, wk, o, p.kspan, p.ochunk, p.nochunk, part, mask_out); break;
    case 8: k_gather1<8><<<g, b, 0, s>>>(x, k, n, wk, o, p.kspan, p.ochunk, p.nochunk, part, mask_out); break;
    case 16: k_gather1<16><<<g, b, 0, s>>>(x, k, n, wk, o, p.kspan, p.ochunk, p.nochunk, part, mask_out); break;
    case 32: k_gather1<32><<<g, b, 0, s>>>(x, k, n, wk, o, p.kspan, p.ochunk, p.nochunk, part, mask_out); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  r.note(NM_TAKEN_GATHER1);
  return launch_reduce_parts(part, p.nks, Epi{}, 1, o, y, o, accumulate, r, s);   // one row: ldy unused
}

hipError_t launch_reduce_parts(const float* part, int64_t splits, const Epi& epi, int64_t t, int64_t o,
                               float* y, int64_t ldy, int accumulate, const Route& r, hipStream_t s) {
  const int64_t n = t * o;
  if (n == 0) return hipSuccess;
  r.note(NM_TAKEN_REDUCE);
  // y is 16-byte aligned (checked at the boundary); float4 rows need o and ldy % 4 == 0
  if (splits >= 1 && splits <= 16 && o % 4 == 0 && ldy % 4 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(part) & 15) == 0 && (reinterpret_cast<uintptr_t>(epi.col_shift) & 15) == 0) {
    k_reduce_parts4<<<dim3((unsigned)((n / 4 + RP4_THREADS - 1) / RP4_THREADS)), dim3(RP4_THREADS), 0, s>>>(
        part, splits, epi, t, o, y, ldy, accumulate);
    return hipGetLastError();
  }
  k_reduce_parts<<<dim3((unsigned)((n + RP_OUT - 1) / RP_OUT)), dim3(RP_OUT * RP_LANES), 0, s>>>(
      part, splits, epi, t, o, y, ldy, accumulate);
  return hipGetLastError();
}

hipError_t launch_permute_cols(const uint16_t* x, int64_t t, int64_t ldx, int64_t kx, const int32_t* c0, int64_t k0,
                               const int32_t* c1, int64_t k1, int64_t off1, uint16_t* xo, int64_t ldo,
                               hipStream_t s) {
  const int64_t n = t * (k0 + k1);
  if (n == 0) return hipSuccess;
  const bool rows = kx % 8 == 0 && ldx % 8 == 0 && k0 % 8 == 0 && k1 % 8 == 0 && off1 % 8 == 0 && ldo % 8 == 0 &&
                    ((uintptr_t)x & 15) == 0 && ((uintptr_t)xo & 15) == 0 && ((uintptr_t)c0 & 15) == 0 &&
                    ((uintptr_t)c1 & 15) == 0 && kx <= 65536 && k0 + k1 <= 0x7FFFFFFF && t <= 0x7FFFFFFF;
  if (rows) {
    const size_t lds = (size_t)kx * 2;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)k_permute_rows, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)lds);
      if (e != hipSuccess) return e;
    }
    k_permute_rows<<<dim3((unsigned)t), dim3(PERM_THREADS), lds, s>>>(x, ldx, (int)kx, c0, (int)k0, c1, (int)k1,
                                                                       off1, xo, ldo);
    return hipGetLastError();
  }
  k_permute_cols<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(x, t, ldx, kx, c0, k0, c1, k1, off1, xo,
                                                                         ldo);
  return hipGetLastError();
}

}  // namespace nml
