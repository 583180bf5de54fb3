// Dense-MFMA product for activation N:M sparsity:  Y[t][o] = sum_k S(X)[t][k] * W[o][k].
//
// gfx950 has no matrix instruction for 8:16 or 16:32 patterns, so the selected
// activation tile is zero-filled and contracted with v_mfma_f32_16x16x32_bf16 (the
// Flexible (N:M) Activation Sparsity page, technical summary section 4.E, notes that
// such patterns have only been emulated; sections 2.A/2.C define the selection).  The
// selection happens in the X-tile loader ("prologue"), between the global load and the
// LDS store:
//   PRO_SELECT: top-n of each m-group computed in registers (fused sparsify);
//   PRO_MASK:   a keep bitmask produced by a separate select pass is applied;
//   PRO_NONE:   X is used as given (already sparsified, or a dense layer).
// The fp8 (OCP E4M3FN) weight variant is widened to bf16 in the W-tile loader (exact)
// and its per-row scale is applied once in the epilogue.
//
// Tiling: a workgroup computes a BO x BT tile of Y^T (o x t) with NW = WO*WT waves, each
// owning a (BO/WO) x (BT/WT) sub-tile of 16x16 accumulators.  K advances in steps of 64
// through double-buffered LDS tiles (row pitch 72 bf16 = 144 bytes: conflict-free
// 16-byte fragment reads).  Workgroups are remapped so that each of the 8 XCDs (own L2)
// works on a contiguous band of output tiles.
#include <cstdlib>
#include <cstring>

#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;
using namespace nml;

constexpr int BK = 64;
constexpr int PITCH = BK + 8;   // LDS row pitch in bf16

// Load 8 bf16 (one 16-byte chunk) of a row at column kk, zero beyond K.
__device__ __forceinline__ uint4 load_chunk_bf16(const uint16_t* rowp, int64_t kk, int64_t K) {
  if (kk + 8 <= K) return *reinterpret_cast<const uint4*>(rowp + kk);
  uint32_t v[4] = {0, 0, 0, 0};
  for (int e = 0; e < 8; ++e)
    if (kk + e < K) v[e >> 1] |= (uint32_t)rowp[kk + e] << (16 * (e & 1));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Load 16 fp8 bytes of a row at column kk, zero beyond K.
__device__ __forceinline__ uint4 load_chunk_fp8(const uint8_t* rowp, int64_t kk, int64_t K) {
  if (kk + 16 <= K) return *reinterpret_cast<const uint4*>(rowp + kk);
  uint32_t v[4] = {0, 0, 0, 0};
  for (int e = 0; e < 16; ++e)
    if (kk + e < K) v[e >> 2] |= (uint32_t)rowp[kk + e] << (8 * (e & 3));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int M>
__device__ __forceinline__ uint32_t select32(const uint32_t (&d)[16], int n) {
  // keep bits of 32 consecutive elements, groups of M
  uint32_t bits = 0;
#pragma unroll
  for (int gq = 0; gq < 32 / M; ++gq) {
    uint32_t gd[M / 2];
#pragma unroll
    for (int q = 0; q < M / 2; ++q) gd[q] = d[gq * (M / 2) + q];
    bits |= topn_bits<M>(gd, n) << (gq * M);
  }
  return bits;
}

template <int BO, int BT, int WO, int WT, int PRO, int M, bool FP8>
__global__ __launch_bounds__(64 * WO * WT) void k_gemm_dense(
    const void* __restrict__ wptr, int64_t ldw, Epi epi,
    const uint16_t* __restrict__ x, int64_t ldx, const uint32_t* __restrict__ xmask, int n,
    int64_t T, int64_t O, int64_t K, float* __restrict__ y, int64_t ldy, int accumulate,
    uint32_t* __restrict__ mask_out, int tiles_o, int tiles_t) {
  constexpr int NTH = 64 * WO * WT;
  constexpr int ROWS_PER_PASS = NTH / 2;      // each thread stages 32 k of one row
  constexpr int PASS_A = BO / ROWS_PER_PASS;
  constexpr int PASS_B = BT / ROWS_PER_PASS;
  static_assert(BO % ROWS_PER_PASS == 0 && BT % ROWS_PER_PASS == 0, "tile/threads");
  constexpr int SO = BO / WO, ST = BT / WT;  // wave sub-tile
  constexpr int FI = SO / 16, FJ = ST / 16;

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sA = smem;                         // [2][BO][PITCH]
  uint16_t* sB = smem + 2 * BO * PITCH;        // [2][BT][PITCH]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wo = wave % WO, wt = wave / WO;

  // XCD-aware remap: hardware places workgroup b on XCD b % 8; give each XCD a
  // contiguous range of tiles, walked t-major within bands of 8 o-tiles.
  const int ntiles = tiles_o * tiles_t;
  const int b = blockIdx.x;
  int lin;
  {
    const int per = (ntiles + 7) / 8;
    const int xcd = b % 8, slot = b / 8;
    lin = xcd * per + slot;
    if ((ntiles % 8) != 0) lin = b;          // simple order when not evenly divisible
  }
  if (lin >= ntiles) return;
  constexpr int GROUP = 8;
  const int band = lin / (GROUP * tiles_t);
  const int band_w = min(GROUP, tiles_o - band * GROUP);
  const int inband = lin - band * GROUP * tiles_t;
  const int tile_o = band * GROUP + inband % band_w;
  const int tile_t = inband / band_w;
  const int64_t o0 = (int64_t)tile_o * BO, t0 = (int64_t)tile_t * BT;

  const int lrow = tid >> 1, lhalf = tid & 1;

  uint32_t ra[PASS_A][16];   // staged A (W) as bf16
  uint32_t rb[PASS_B][16];   // staged B (X) as bf16

  auto load_tiles = [&](int64_t k0) {
#pragma unroll
    for (int p = 0; p < PASS_A; ++p) {
      const int64_t o = o0 + lrow + p * ROWS_PER_PASS;
      const int64_t kk = k0 + 32 * lhalf;
      if (o < O && kk < K) {
        if constexpr (FP8) {
          const uint8_t* rp = reinterpret_cast<const uint8_t*>(wptr) + o * ldw;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint4 q = load_chunk_fp8(rp, kk + 16 * c, K);
            fp8x4_to_bf16x4(q.x, ra[p][8 * c + 0], ra[p][8 * c + 1]);
            fp8x4_to_bf16x4(q.y, ra[p][8 * c + 2], ra[p][8 * c + 3]);
            fp8x4_to_bf16x4(q.z, ra[p][8 * c + 4], ra[p][8 * c + 5]);
            fp8x4_to_bf16x4(q.w, ra[p][8 * c + 6], ra[p][8 * c + 7]);
          }
        } else {
          const uint16_t* rp = reinterpret_cast<const uint16_t*>(wptr) + o * ldw;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint4 v = load_chunk_bf16(rp, kk + 8 * c, K);
            ra[p][4 * c] = v.x; ra[p][4 * c + 1] = v.y; ra[p][4 * c + 2] = v.z; ra[p][4 * c + 3] = v.w;
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) ra[p][q] = 0;
      }
    }
#pragma unroll
    for (int p = 0; p < PASS_B; ++p) {
      const int64_t t = t0 + lrow + p * ROWS_PER_PASS;
      const int64_t kk = k0 + 32 * lhalf;
      if (t < T && kk < K) {
        const uint16_t* rp = x + t * ldx;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint4 v = load_chunk_bf16(rp, kk + 8 * c, K);
          rb[p][4 * c] = v.x; rb[p][4 * c + 1] = v.y; rb[p][4 * c + 2] = v.z; rb[p][4 * c + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) rb[p][q] = 0;
      }
    }
  };

  auto prologue = [&](int64_t k0) {
    if constexpr (PRO == PRO_SELECT) {
#pragma unroll
      for (int p = 0; p < PASS_B; ++p) {
        const int64_t t = t0 + lrow + p * ROWS_PER_PASS;
        const int64_t kk = k0 + 32 * lhalf;
        const uint32_t bits = select32<M>(rb[p], n);
#pragma unroll
        for (int q = 0; q < 16; ++q) rb[p][q] = mask_pair(rb[p][q], bits >> (2 * q));
        if (mask_out != nullptr && tile_o == 0 && t < T && kk < K)
          mask_out[t * ((K + 31) >> 5) + (kk >> 5)] = (kk + 32 <= K) ? bits : (bits & ((1u << (K - kk)) - 1u));
      }
    } else if constexpr (PRO == PRO_MASK) {
#pragma unroll
      for (int p = 0; p < PASS_B; ++p) {
        const int64_t t = t0 + lrow + p * ROWS_PER_PASS;
        const int64_t kk = k0 + 32 * lhalf;
        const uint32_t bits = (t < T && kk < K) ? xmask[t * ((K + 31) >> 5) + (kk >> 5)] : 0u;
#pragma unroll
        for (int q = 0; q < 16; ++q) rb[p][q] = mask_pair(rb[p][q], bits >> (2 * q));
      }
    }
  };

  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PASS_A; ++p) {
      uint16_t* dst = sA + (buf * BO + lrow + p * ROWS_PER_PASS) * PITCH + 32 * lhalf;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        reinterpret_cast<uint4*>(dst)[c] = make_uint4(ra[p][4 * c], ra[p][4 * c + 1], ra[p][4 * c + 2], ra[p][4 * c + 3]);
    }
#pragma unroll
    for (int p = 0; p < PASS_B; ++p) {
      uint16_t* dst = sB + (buf * BT + lrow + p * ROWS_PER_PASS) * PITCH + 32 * lhalf;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        reinterpret_cast<uint4*>(dst)[c] = make_uint4(rb[p][4 * c], rb[p][4 * c + 1], rb[p][4 * c + 2], rb[p][4 * c + 3]);
    }
  };

  f32x4 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)((K + BK - 1) / BK);
  if (nk > 0) {
    load_tiles(0);
    prologue(0);
    store_tiles(0);
  }
  __syncthreads();
  const int fr = lane & 15, fk = 8 * (lane >> 4);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tiles((int64_t)(kt + 1) * BK);
    const uint16_t* a_base = sA + (buf * BO + wo * SO + fr) * PITCH + fk;
    const uint16_t* b_base = sB + (buf * BT + wt * ST + fr) * PITCH + fk;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[FI], bfr[FJ];
#pragma unroll
      for (int i = 0; i < FI; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(a_base + i * 16 * PITCH + ks * 32);
#pragma unroll
      for (int j = 0; j < FJ; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(b_base + j * 16 * PITCH + ks * 32);
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      prologue((int64_t)(kt + 1) * BK);
      store_tiles(buf ^ 1);
    }
    __syncthreads();
  }

  // epilogue: lane holds 4 consecutive o for one t in each 16x16 block
  const bool vec_ok = ((ldy & 3) == 0);
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const int64_t ob = o0 + wo * SO + i * 16 + 4 * (lane >> 4);
    float sc[4] = {1.f, 1.f, 1.f, 1.f}, cs[4] = {0.f, 0.f, 0.f, 0.f};
    if (epi.w_scale != nullptr) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = (ob + r < O) ? epi.w_scale[ob + r] : 0.f;
    }
    if (epi.col_shift != nullptr) {
#pragma unroll
      for (int r = 0; r < 4; ++r) cs[r] = (ob + r < O) ? epi.col_shift[ob + r] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int64_t t = t0 + wt * ST + j * 16 + (lane & 15);
      if (t >= T) continue;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r] * sc[r];
      if (epi.extra()) {
        const float rs = epi.row_scale != nullptr ? epi.row_scale[t] : 1.f;
        const float rb = epi.row_shift != nullptr ? epi.row_shift[t] : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = v[r] * rs + rb * cs[r];
      }
      float* yp = y + t * ldy + ob;
      if (vec_ok && ob + 4 <= O) {
        float4 cur = accumulate ? *reinterpret_cast<float4*>(yp) : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(yp) = make_float4(cur.x + v[0], cur.y + v[1], cur.z + v[2], cur.w + v[3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (ob + r < O) yp[r] = accumulate ? yp[r] + v[r] : v[r];
      }
    }
  }
}

template <int BO, int BT, int WO, int WT, int PRO, int M, bool FP8>
hipError_t launch_cfg(const nml::GemmArgs& a, hipStream_t s) {
  const int tiles_o = (int)((a.o + BO - 1) / BO), tiles_t = (int)((a.t + BT - 1) / BT);
  const int64_t ntiles = (int64_t)tiles_o * tiles_t;
  if (ntiles == 0) return hipSuccess;
  const size_t lds = (size_t)2 * (BO + BT) * PITCH * sizeof(uint16_t);
  auto kern = k_gemm_dense<BO, BT, WO, WT, PRO, M, FP8>;
  static bool attr_set = false;   // benign race: idempotent attribute write
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  kern<<<dim3((unsigned)ntiles), dim3(64 * WO * WT), lds, s>>>(
      a.w, a.ldw, a.epi(), a.x, a.ldx, a.x_mask, a.n, a.t, a.o, a.k, a.y, a.ldy, a.accumulate,
      a.mask_out, tiles_o, tiles_t);
  return hipGetLastError();
}

template <int PRO, int M, bool FP8>
hipError_t launch_pick(const nml::GemmArgs& a, hipStream_t s) {
  // large problems: 256x256 tiles with 8 waves; small ones: 128x128 with 4 waves
  const int64_t big_tiles = ((a.o + 255) / 256) * ((a.t + 255) / 256);
  if (big_tiles >= 256) return launch_cfg<256, 256, 2, 4, PRO, M, FP8>(a, s);
  return launch_cfg<128, 128, 2, 2, PRO, M, FP8>(a, s);
}

template <int PRO, bool FP8>
hipError_t launch_m(const nml::GemmArgs& a, hipStream_t s) {
  if constexpr (PRO == PRO_SELECT) {
    switch (a.m) {
      case 4: return launch_pick<PRO, 4, FP8>(a, s);
      case 8: return launch_pick<PRO, 8, FP8>(a, s);
      case 16: return launch_pick<PRO, 16, FP8>(a, s);
      case 32: return launch_pick<PRO, 32, FP8>(a, s);
      default: return hipErrorInvalidValue;
    }
  } else {
    return launch_pick<PRO, 4, FP8>(a, s);
  }
}

}  // namespace

namespace nml {

hipError_t launch_gemm_dense(const GemmArgs& a, hipStream_t s) {
  // the NM_ROUTE_TILE_REGS / NM_ROUTE_TILE_LDS hints override the kernel choice
  const bool regs_only = a.route.has(NM_ROUTE_TILE_REGS);
  const bool lds_any = a.route.has(NM_ROUTE_TILE_LDS);
  if (!regs_only && gemm_lds_eligible(a, lds_any)) return launch_gemm_lds(a, s);
  a.route.note(NM_TAKEN_TILE_REGS | (a.prologue == PRO_SELECT ? NM_TAKEN_FUSED_SELECT : 0u) |
               (a.prologue == PRO_MASK ? NM_TAKEN_MASK : 0u));
  if (a.w_fp8) {
    switch (a.prologue) {
      case PRO_NONE: return launch_m<PRO_NONE, true>(a, s);
      case PRO_SELECT: return launch_m<PRO_SELECT, true>(a, s);
      case PRO_MASK: return launch_m<PRO_MASK, true>(a, s);
    }
  } else {
    switch (a.prologue) {
      case PRO_NONE: return launch_m<PRO_NONE, false>(a, s);
      case PRO_SELECT: return launch_m<PRO_SELECT, false>(a, s);
      case PRO_MASK: return launch_m<PRO_MASK, false>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace nml
