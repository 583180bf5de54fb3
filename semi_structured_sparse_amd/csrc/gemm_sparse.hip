// 2:4 sparse-operand product on the gfx950 sparse matrix instruction
// v_smfmac_f32_16x16x64_bf16:   Y[t][o] (=|+=) sum_k X~[t][k] * W24[o][k]
//
// W24 is a 2:4 matrix over a reduction length kc, stored compressed (values [O][kc/2],
// 2-bit positions [O][ceil(kc/8)]).  It is the sparse (first) operand of the
// instruction; X~ is the dense operand, produced by the X-tile loader:
//   XL_PLAIN : X~ = X                              (2:4 weights)
//   XL_LIFT  : X~ = lift_N(X), never materialised  (SlideSparse page, technical summary
//              2.B: lowered (2N-2):2N weights need the activations lifted; section 2.A
//              gives the window geometry: X'[g*4(N-1)+4w+s] = X[g*2N+2w+s])
// An optional second phase contracts a dense region with v_mfma_f32_16x16x32_bf16 into
// the same accumulators (SpenseGPT page, technical summary 2.A: input split with
// accumulation): Y += X[:, dbase:dbase+kd] . Wd^T, X holding the permuted columns
// (sparse region first, dense region at column dbase).
//
// Operand layouts (verified on gfx950): for the sparse instruction, lane l holds row
// l%16 of the sparse operand for dense reduction positions [16*(l/16), +16) as 8
// compressed values plus a 16-bit index word (2 bits per value, one nibble per group
// of 4); the dense operand's lane l holds column l%16 at reduction positions
// 8*(l/16)+[0,8) and 32+8*(l/16)+[0,8).  The accumulator layout equals the dense
// 16x16 instruction's, so both phases share it.
#include <cstdlib>
#include <cstring>

#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;
using namespace nml;

constexpr int BKS = 64;             // dense-equivalent reduction per sparse stage
constexpr int PV = BKS / 2 + 8;     // LDS pitch of compressed values (40 bf16 = 80 B)
constexpr int PB = BKS + 8;         // LDS pitch of dense tiles (72 bf16 = 144 B)

template <int BO, int BT, int WO, int WT>
struct Lds {
  static constexpr int sparse_a = BO * PV;          // values
  static constexpr int sparse_m = BO * 4;           // meta as u16 words (8 bytes/row)
  static constexpr int dense_a = BO * PB;
  static constexpr int a_elems = (sparse_a + sparse_m) > dense_a ? (sparse_a + sparse_m) : dense_a;
  static constexpr int b_elems = BT * PB;
  static constexpr int stage = a_elems + b_elems;  // u16 elements per stage
};

__device__ __forceinline__ uint32_t ld_u16(const uint16_t* p) { return *p; }

// 32 consecutive reduction positions [kk, kk+32) of X~ row t into 16 dwords.
template <int LOADER>
__device__ __forceinline__ void load_x32(const uint16_t* __restrict__ x, int64_t ldx, int64_t t,
                                         int64_t kk, int64_t kc, int ns, int64_t col_base,
                                         uint32_t (&r)[16]) {
  const uint16_t* rp = x + t * ldx;
  if constexpr (LOADER == XL_PLAIN) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t k = kk + 8 * c;
      if (k + 8 <= kc) {
        const uint4 v = *reinterpret_cast<const uint4*>(rp + col_base + k);
        r[4 * c] = v.x; r[4 * c + 1] = v.y; r[4 * c + 2] = v.z; r[4 * c + 3] = v.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t lo = (k + 2 * q < kc) ? ld_u16(rp + col_base + k + 2 * q) : 0u;
          uint32_t hi = (k + 2 * q + 1 < kc) ? ld_u16(rp + col_base + k + 2 * q + 1) : 0u;
          r[4 * c + q] = lo | (hi << 16);
        }
      }
    }
  } else if constexpr (LOADER == XL_LIFT) {
    // windows of 4 lifted positions = 4 consecutive original positions g*2N + 2w
    const int wpg = ns - 1;
#pragma unroll
    for (int wq = 0; wq < 8; ++wq) {
      const int64_t kp = kk + 4 * wq;
      if (kp < kc) {
        const int64_t win = kp >> 2;
        const int64_t g = win / wpg;
        const int64_t w = win - g * wpg;
        const uint32_t* src = reinterpret_cast<const uint32_t*>(rp + g * 2 * ns + 2 * w);
        r[2 * wq] = src[0];
        r[2 * wq + 1] = src[1];
      } else {
        r[2 * wq] = 0; r[2 * wq + 1] = 0;
      }
    }
  }
}

template <int BO, int BT, int WO, int WT, int LOADER>
__global__ __launch_bounds__(64 * WO * WT) void k_gemm_sparse(
    const uint16_t* __restrict__ wv, const uint8_t* __restrict__ wm, int64_t kc,
    const uint16_t* __restrict__ x, int64_t ldx, int ns,
    int64_t T, int64_t O, const uint16_t* __restrict__ wd, int64_t ldwd, int64_t kd,
    int64_t dbase, float* __restrict__ y, int64_t ldy, int accumulate,
    int trans_out, int tiles_o, int tiles_t) {
  constexpr int NTH = 64 * WO * WT;
  constexpr int RPP = NTH / 2;
  constexpr int PASS_A = BO / RPP, PASS_B = BT / RPP;
  static_assert(BO % RPP == 0 && BT % RPP == 0, "tile/threads");
  constexpr int SO = BO / WO, ST = BT / WT;
  constexpr int FI = SO / 16, FJ = ST / 16;
  using L = Lds<BO, BT, WO, WT>;

  extern __shared__ __align__(16) uint16_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wo = wave % WO, wt = wave / WO;
  const int ntiles = tiles_o * tiles_t;
  int lin = blockIdx.x;
  if ((ntiles % 8) == 0) lin = (blockIdx.x % 8) * (ntiles / 8) + blockIdx.x / 8;
  constexpr int GROUP = 8;
  const int band = lin / (GROUP * tiles_t);
  const int band_w = min(GROUP, tiles_o - band * GROUP);
  const int inband = lin - band * GROUP * tiles_t;
  const int tile_o = band * GROUP + inband % band_w;
  const int tile_t = inband / band_w;
  const int64_t o0 = (int64_t)tile_o * BO, t0 = (int64_t)tile_t * BT;
  const int lrow = tid >> 1, lhalf = tid & 1;
  const int fr = lane & 15, fg = lane >> 4;

  f32x4 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ------------------------------------------------------------ sparse phase ---
  {
    const int64_t kcv = kc / 2;                 // compressed values per row
    const int64_t mstride = (kc + 7) >> 3;      // meta bytes per row
    const bool vec_a = ((kcv & 7) == 0);
    uint32_t rav[PASS_A][8];                    // 16 values
    uint32_t ram[PASS_A];                       // 4 meta bytes (16 values)
    uint32_t rb[PASS_B][16];

    auto load = [&](int64_t k0) {
#pragma unroll
      for (int p = 0; p < PASS_A; ++p) {
        const int64_t o = o0 + lrow + p * RPP;
        const int64_t v0 = k0 / 2 + 16 * lhalf;   // first compressed value
        if (o < O && v0 < kcv) {
          const uint16_t* vp = wv + o * kcv + v0;
          if (vec_a && v0 + 16 <= kcv) {
            const uint4 a = reinterpret_cast<const uint4*>(vp)[0];
            const uint4 b = reinterpret_cast<const uint4*>(vp)[1];
            rav[p][0] = a.x; rav[p][1] = a.y; rav[p][2] = a.z; rav[p][3] = a.w;
            rav[p][4] = b.x; rav[p][5] = b.y; rav[p][6] = b.z; rav[p][7] = b.w;
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const uint32_t lo = (v0 + 2 * q < kcv) ? (uint32_t)vp[2 * q] : 0u;
              const uint32_t hi = (v0 + 2 * q + 1 < kcv) ? (uint32_t)vp[2 * q + 1] : 0u;
              rav[p][q] = lo | (hi << 16);
            }
          }
          const uint8_t* mp = wm + o * mstride + (v0 >> 2);
          uint32_t mw = 0;
#pragma unroll
          for (int bq = 0; bq < 4; ++bq)
            if ((v0 >> 2) + bq < mstride) mw |= (uint32_t)mp[bq] << (8 * bq);
          ram[p] = mw;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) rav[p][q] = 0;
          ram[p] = 0;
        }
      }
#pragma unroll
      for (int p = 0; p < PASS_B; ++p) {
        const int64_t t = t0 + lrow + p * RPP;
        const int64_t kk = k0 + 32 * lhalf;
        if (t < T && kk < kc) {
          load_x32<LOADER>(x, ldx, t, kk, kc, ns, 0, rb[p]);
        } else {
#pragma unroll
          for (int q = 0; q < 16; ++q) rb[p][q] = 0;
        }
      }
    };
    auto store = [&](int buf) {
      uint16_t* st = smem + buf * L::stage;
      uint16_t* sav = st;
      uint16_t* sam = st + L::sparse_a;
      uint16_t* sb = st + L::a_elems;
#pragma unroll
      for (int p = 0; p < PASS_A; ++p) {
        const int row = lrow + p * RPP;
        uint4* dst = reinterpret_cast<uint4*>(sav + row * PV + 16 * lhalf);
        dst[0] = make_uint4(rav[p][0], rav[p][1], rav[p][2], rav[p][3]);
        dst[1] = make_uint4(rav[p][4], rav[p][5], rav[p][6], rav[p][7]);
        reinterpret_cast<uint32_t*>(sam + row * 4)[lhalf] = ram[p];
      }
#pragma unroll
      for (int p = 0; p < PASS_B; ++p) {
        uint4* dst = reinterpret_cast<uint4*>(sb + (lrow + p * RPP) * PB + 32 * lhalf);
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = make_uint4(rb[p][4 * c], rb[p][4 * c + 1], rb[p][4 * c + 2], rb[p][4 * c + 3]);
      }
    };

    const int nk = (int)((kc + BKS - 1) / BKS);
    if (nk > 0) { load(0); store(0); }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) load((int64_t)(kt + 1) * BKS);
      const uint16_t* st = smem + buf * L::stage;
      const uint16_t* sav = st;
      const uint16_t* sam = st + L::sparse_a;
      const uint16_t* sb = st + L::a_elems;
      bf16x8 af[FI];
      int idx[FI];
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const int row = wo * SO + i * 16 + fr;
        af[i] = *reinterpret_cast<const bf16x8*>(sav + row * PV + 8 * fg);
        idx[i] = (int)sam[row * 4 + fg];
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const uint16_t* bp = sb + (wt * ST + j * 16 + fr) * PB + 8 * fg;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(bp);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(bp + 32);
        const u32x8 bb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x16 bv = __builtin_bit_cast(bf16x16, bb);
#pragma unroll
        for (int i = 0; i < FI; ++i)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[i], bv, acc[i][j], idx[i], 0, 0);
      }
      if (kt + 1 < nk) store(buf ^ 1);
      __syncthreads();
    }
  }

  // ------------------------------------------------------------- dense phase ---
  if (kd > 0) {
    uint32_t ra[PASS_A][16], rb[PASS_B][16];
    auto load = [&](int64_t k0) {
#pragma unroll
      for (int p = 0; p < PASS_A; ++p) {
        const int64_t o = o0 + lrow + p * RPP;
        const int64_t kk = k0 + 32 * lhalf;
        if (o < O && kk < kd) {
          const uint16_t* rp = wd + o * ldwd;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int64_t k = kk + 8 * c;
            if (k + 8 <= kd) {
              const uint4 v = *reinterpret_cast<const uint4*>(rp + k);
              ra[p][4 * c] = v.x; ra[p][4 * c + 1] = v.y; ra[p][4 * c + 2] = v.z; ra[p][4 * c + 3] = v.w;
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint32_t lo = (k + 2 * q < kd) ? (uint32_t)rp[k + 2 * q] : 0u;
                const uint32_t hi = (k + 2 * q + 1 < kd) ? (uint32_t)rp[k + 2 * q + 1] : 0u;
                ra[p][4 * c + q] = lo | (hi << 16);
              }
            }
          }
        } else {
#pragma unroll
          for (int q = 0; q < 16; ++q) ra[p][q] = 0;
        }
      }
#pragma unroll
      for (int p = 0; p < PASS_B; ++p) {
        const int64_t t = t0 + lrow + p * RPP;
        const int64_t kk = k0 + 32 * lhalf;
        if (t < T && kk < kd) {
          load_x32<XL_PLAIN>(x, ldx, t, kk, kd, ns, dbase, rb[p]);
        } else {
#pragma unroll
          for (int q = 0; q < 16; ++q) rb[p][q] = 0;
        }
      }
    };
    auto store = [&](int buf) {
      uint16_t* st = smem + buf * L::stage;
      uint16_t* sa = st;
      uint16_t* sb = st + L::a_elems;
#pragma unroll
      for (int p = 0; p < PASS_A; ++p) {
        uint4* dst = reinterpret_cast<uint4*>(sa + (lrow + p * RPP) * PB + 32 * lhalf);
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = make_uint4(ra[p][4 * c], ra[p][4 * c + 1], ra[p][4 * c + 2], ra[p][4 * c + 3]);
      }
#pragma unroll
      for (int p = 0; p < PASS_B; ++p) {
        uint4* dst = reinterpret_cast<uint4*>(sb + (lrow + p * RPP) * PB + 32 * lhalf);
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = make_uint4(rb[p][4 * c], rb[p][4 * c + 1], rb[p][4 * c + 2], rb[p][4 * c + 3]);
      }
    };
    const int nk = (int)((kd + BKS - 1) / BKS);
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) load((int64_t)(kt + 1) * BKS);
      const uint16_t* st = smem + buf * L::stage;
      const uint16_t* a_base = st + (wo * SO + fr) * PB + 8 * fg;
      const uint16_t* b_base = st + L::a_elems + (wt * ST + fr) * PB + 8 * fg;
#pragma unroll
      for (int ks = 0; ks < BKS / 32; ++ks) {
        bf16x8 af[FI], bfr[FJ];
#pragma unroll
        for (int i = 0; i < FI; ++i) af[i] = *reinterpret_cast<const bf16x8*>(a_base + i * 16 * PB + ks * 32);
#pragma unroll
        for (int j = 0; j < FJ; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(b_base + j * 16 * PB + ks * 32);
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
          for (int j = 0; j < FJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < nk) store(buf ^ 1);
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------- epilogue ---
  // lane holds 4 consecutive sparse-side rows (ob..ob+3) of one dense-side row t.
  // trans_out == 0: Y[t][ob + r] (W is the sparse operand, a 16-byte store);
  // trans_out == 1: Y[ob + r][t] (X is the sparse operand).
  const bool vec_ok = ((ldy & 3) == 0) && !trans_out;
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const int64_t ob = o0 + wo * SO + i * 16 + 4 * fg;
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int64_t t = t0 + wt * ST + j * 16 + fr;
      if (t >= T) continue;
      if (vec_ok && ob + 4 <= O) {
        float* yp = y + t * ldy + ob;
        float4 cur = accumulate ? *reinterpret_cast<float4*>(yp) : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(yp) =
            make_float4(cur.x + acc[i][j][0], cur.y + acc[i][j][1], cur.z + acc[i][j][2], cur.w + acc[i][j][3]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (ob + r >= O) continue;
          float* yp = trans_out ? (y + (ob + r) * ldy + t) : (y + t * ldy + ob + r);
          *yp = accumulate ? *yp + acc[i][j][r] : acc[i][j][r];
        }
      }
    }
  }
}

template <int BO, int BT, int WO, int WT, int LOADER>
hipError_t launch_cfg(const nml::SparseArgs& a, hipStream_t s) {
  const int tiles_o = (int)((a.o + BO - 1) / BO), tiles_t = (int)((a.t + BT - 1) / BT);
  const int64_t ntiles = (int64_t)tiles_o * tiles_t;
  if (ntiles == 0) return hipSuccess;
  using L = Lds<BO, BT, WO, WT>;
  const size_t lds = (size_t)2 * L::stage * sizeof(uint16_t);
  auto kern = k_gemm_sparse<BO, BT, WO, WT, LOADER>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  kern<<<dim3((unsigned)ntiles), dim3(64 * WO * WT), lds, s>>>(
      a.w_vals, a.w_meta, a.kc, a.x, a.ldx, a.ns, a.t, a.o, a.wd, a.ldwd, a.kd, a.dbase,
      a.y, a.ldy, a.accumulate, a.trans_out, tiles_o, tiles_t);
  return hipGetLastError();
}

template <int LOADER>
hipError_t launch_pick(const nml::SparseArgs& a, hipStream_t s) {
  const int64_t big_tiles = ((a.o + 255) / 256) * ((a.t + 255) / 256);
  if (big_tiles >= 256) return launch_cfg<256, 256, 2, 4, LOADER>(a, s);
  return launch_cfg<128, 128, 2, 2, LOADER>(a, s);
}

}  // namespace

namespace nml {

bool gemm_sparse_uses_lds(const SparseArgs& a) {
  // the NM_ROUTE_TILE_REGS / NM_ROUTE_TILE_LDS hints override the kernel choice
  return !a.route.has(NM_ROUTE_TILE_REGS) && gemm_lds_sp_eligible(a, a.route.has(NM_ROUTE_TILE_LDS));
}

hipError_t launch_gemm_sparse(const SparseArgs& a, hipStream_t s) {
  if (gemm_sparse_uses_lds(a)) return launch_gemm_lds_sp(a, s);
  a.route.note(NM_TAKEN_TILE_REGS | NM_TAKEN_SPARSE_MMA);
  switch (a.loader) {
    case XL_PLAIN: return launch_pick<XL_PLAIN>(a, s);
    case XL_LIFT: return launch_pick<XL_LIFT>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace nml
