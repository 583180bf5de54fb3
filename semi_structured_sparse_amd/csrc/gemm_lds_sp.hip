// Large-token product with a 2:4 sparse weight operand, staged direct-to-LDS:
//   Y[t][o] (=|+=) sum_k X[t][k] * W24[o][k]  (+ sum_j X[t][dbase + j] * Wd[o][j])
//
// W24 is 2:4 along the reduction (values [O][kc/2], 2-bit positions [O][kc/8]) -- plain
// 2:4 weights, or (2N-2):2N weights lowered to overlapping 2:4 windows with lifted
// activations (SlideSparse page, technical summary 2.A/2.B): X lifted beforehand, or (LX)
// the raw X, whose lifted rows the stage loads build with one dword per lane (every lifted
// dword is one raw dword: a window is 4 bf16 starting at an even raw position).  The optional
// dense second phase is the hybrid format's dense region, accumulated into the same
// accumulators (SpenseGPT page, technical summary 2.A).
//
// gfx950 design, after the dense direct-to-LDS kernel:
//  * 256 x 256 output tile, 8 waves of 64 (o) x 128 (t); two LDS stages, each a distinct
//    static array (so the compiler tracks the DMA into each one separately); the
//    few-token tiles use three (lds_ring, two K-steps in flight).
//  * Few tokens (33-128): 128 x 64 or 128 x 128 tiles and a reduction split across
//    workgroups (one per CU); each split writes its fp32 partial tile, and a second
//    kernel sums the splits in a fixed order.  The sparse and dense steps form one
//    reduction sequence that the splits cut into contiguous ranges.
//  * One sparse K-step covers 64 reduction positions: per weight row 64 bytes of
//    compressed values (global_load_lds_dwordx4, 4 lanes per row) and 8 bytes of 2-bit
//    positions (global_load_lds_dword, 2 lanes per row); per token row 128 bytes of X
//    (8 lanes per row).  Pieces are XOR-swizzled per row so the fragment reads are
//    conflict-free.
//  * Positions K-blocked (MB): the loads of a step read [step][row][8 bytes], so 32 rows'
//    positions are one 256-byte run instead of 32 separate 8-byte pieces.  The tile loads
//    are bound by requests in flight per CU (L1 stalls on pending L2 data most cycles),
//    and row-major positions were a third of all requests: measured on gfx950, the
//    product takes 12-14% less time at the cfg3 / cfg4 shapes and 25% at 8192 tokens.
//    launch_meta_block makes the blocked copy (o * kc / 8 bytes) in the caller's
//    workspace; row-major positions remain the fallback.
//  * v_smfmac_f32_16x16x64_bf16: lane l holds weight row l%16 as 8 compressed values for
//    positions [16(l/16), +16) plus its 16-bit index word, and token l%16 at positions
//    8(l/16)+[0,8) and 32+8(l/16)+[0,8).
//  * Dense phase: 128 bytes per weight row per K-step, two v_mfma_f32_16x16x32_bf16.
// Requirements (checked by the caller): kc % 64 == 0 and kd % 64 == 0, 16-byte aligned
// rows (kc % 32 == 0 makes the value and position rows aligned), X and Wd ld % 8 == 0.
#include <cstdlib>
#include <cstring>

#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;
using namespace nml;

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void g2lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}


// The two-stage K-loop (one step in flight): each step issues the next step's loads,
// multiplies, then waits for all loads and synchronises.  Deeper pipelines use lds_ring.
template <typename Issue, typename Compute>
__device__ __forceinline__ void k_loop2(int n, unsigned char* a0, unsigned char* b0, unsigned char* a1,
                                        unsigned char* b1, Issue&& issue, Compute&& compute) {
  issue(a0, b0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // two steps per trip (stage 0, then stage 1); the next step's loads go out first
  for (int s = 0; s < n; s += 2) {
    if (s + 1 < n) issue(a1, b1, s + 1);
    compute(a0, b0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (s + 1 < n) {
      if (s + 2 < n) issue(a0, b0, s + 2);
      compute(a1, b1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }   // 8 pieces per row
__device__ __forceinline__ int swz4(int r, int c) { return c ^ ((r >> 2) & 3); }   // 4 pieces per row

// LX > 0: the weights are (2 LX - 2):2 LX rows lowered to 2:4 windows and x is the raw
// activation: the loads of each step build the lifted X rows in LDS themselves (no
// lifted copy of X; the sparse phase only).
template <int BM, int BN, int WM, int WN, bool MB, bool F8, int NST = 2, int LX = 0>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_lds_sp(
    const uint16_t* __restrict__ wv, const uint8_t* __restrict__ wm, int64_t kc, const uint16_t* __restrict__ x,
    int64_t ldx, const uint16_t* __restrict__ wd, int64_t ldwd, int64_t kd, int64_t dbase, int64_t T, int64_t O,
    float* __restrict__ y, int64_t ldy, int accumulate, int tiles_m, int tiles_n, int steps_per_split,
    float* __restrict__ part, int group, const float* __restrict__ xscale, const float* __restrict__ wscale) {
  // F8: e4m3 codes for both operands, K-steps of 128 positions: the value and X bytes per
  // row per step stay 64 and 128, the positions grow to 16 bytes per row per step, and the
  // matrix instruction is v_smfmac_f32_16x16x128_fp8_fp8 (same operand placement by byte)
  constexpr int STEPK = F8 ? 128 : 64;       // reduction positions per sparse step
  constexpr int MU = F8 ? 16 : 8;            // position bytes per row per sparse step
  constexpr int NW = WM * WN;
  constexpr int SM = BM / WM, SN = BN / WN, FI = SM / 16, FJ = SN / 16;
  constexpr int A_BYTES = BM * 128;          // dense W rows (sparse phase: values + positions)
  constexpr int SV_BYTES = BM * 64;          // compressed values per sparse step
  constexpr int B_BYTES = BN * 128;          // X rows
  constexpr int NV = BM / 16 / NW;           // value load groups (16 rows) per wave
  constexpr int NX = BN / 8 / NW;            // X load groups (8 rows) per wave
  constexpr int ND = BM / 8 / NW;            // dense weight load groups (8 rows) per wave
  // lifted X: each request fills 256 bytes of the stage (two token rows' 128-byte step
  // pieces) with one dword per lane, gathered from the raw row
  static_assert(LX == 0 || (!F8 && LX >= 2 && LX <= 8 && BN % (2 * NW) == 0), "lifted X: bf16, 2 <= N <= 8");
  constexpr int NXL = LX > 0 ? BN / 2 / NW : NX;   // X requests per wave per sparse step
  static_assert(NV >= 1 && NX >= 1 && ND >= 1 && BM % (16 * NW) == 0 && BN % (8 * NW) == 0,
                "load groups per wave");
  static_assert(NST >= 2 && NST <= 4, "two to four stages");
  constexpr int A2B = NST >= 3 ? A_BYTES : 16, B2B = NST >= 3 ? B_BYTES : 16;
  constexpr int A3B = NST >= 4 ? A_BYTES : 16, B3B = NST >= 4 ? B_BYTES : 16;
  __shared__ __align__(16) unsigned char sA0[A_BYTES], sB0[B_BYTES];
  __shared__ __align__(16) unsigned char sA1[A_BYTES], sB1[B_BYTES];
  __shared__ __align__(16) unsigned char sA2[A2B], sB2[B2B];
  __shared__ __align__(16) unsigned char sA3[A3B], sB3[B3B];
  unsigned char* const SA[4] = {sA0, sA1, sA2, sA3};
  unsigned char* const SB[4] = {sB0, sB1, sB2, sB3};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wmi = wave % WM, wni = wave / WM;

  // XCD-aware tile order (workgroup b runs on XCD b % 8), bands of `group` o-tiles; with a
  // split reduction, block b takes split b / ntiles of tile b % ntiles
  const int ntiles = tiles_m * tiles_n;
  const int kpart = blockIdx.x / ntiles;
  int lin = blockIdx.x - kpart * ntiles;
  if ((ntiles & 7) == 0 && gridDim.x == (unsigned)ntiles) lin = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int band = lin / (group * tiles_n);
  const int band_w = min(group, tiles_m - band * group);
  const int inband = lin - band * group * tiles_n;
  const int tile_m = band * group + inband % band_w, tile_n = inband / band_w;
  const int64_t o0 = (int64_t)tile_m * BM, t0 = (int64_t)tile_n * BN;

  const int64_t vrow = F8 ? kc / 2 : kc, mstride = kc / 8;   // value / position bytes per row
  // this split's range [sb, se) of the step sequence (sparse steps, then dense steps)
  const int nks_all = (int)(kc / STEPK), nk_all = nks_all + (int)(kd / 64);
  const int sb = kpart * steps_per_split;
  const int se = min(nk_all, sb + steps_per_split);
  const int ks0 = min(sb, nks_all), ks1 = min(se, nks_all);          // sparse steps [ks0, ks1)
  const int kd0 = max(sb, nks_all) - nks_all, kd1 = max(se, nks_all) - nks_all;   // dense [kd0, kd1)
  const int nks = ks1 - ks0, nkd = kd1 - kd0;

  f32x4 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fg = lane >> 4;

  // X rows: groups of 8 rows (8 lanes x 16 bytes per row), NX per wave; 128 bytes per
  // step (64 bf16 or 128 fp8 codes); ldx in elements (bytes for fp8)
  const unsigned char* xsrc[NX];
  const int64_t ldxb = F8 ? ldx : 2 * ldx;
#pragma unroll
  for (int q = 0; q < NX; ++q) {
    const int r = (wave + q * NW) * 8 + (lane >> 3);
    int64_t t = t0 + r;
    t = t < T ? t : T - 1;
    xsrc[q] = reinterpret_cast<const unsigned char*>(x) + t * ldxb + 16 * swz8(r, lane & 7);
  }

  // ----------------------------------------------------------- sparse phase ---
  if (nks > 0) {
    // compressed values: groups of 16 rows (4 lanes x 16 bytes per row), NV per wave;
    // positions: 32 rows per loading wave (2 lanes x 4 bytes per row)
    const uint8_t* vsrc[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const int r = (wave + q * NW) * 16 + (lane >> 2);
      int64_t o = o0 + r;
      o = o < O ? o : O - 1;
      vsrc[q] = reinterpret_cast<const uint8_t*>(wv) + o * vrow + 16 * swz4(r, lane & 3);
    }
    // positions of step s for row o: wm + o * mstride + MU s (row-major) or
    // wm + (s * O + o) * MU (K-blocked); bf16: 2 lanes of 4 bytes per row (32 rows per
    // loading wave), fp8: one lane of 16 bytes per row (64 rows per loading wave)
    constexpr int MROWS = F8 ? 64 : 32, NMWAVES = BM / MROWS;
    static_assert(NMWAVES <= NW, "position load waves");
    const uint8_t* msrc;
    const int64_t mstep = MB ? O * MU : MU;
    {
      const int r = (wave < NMWAVES ? wave : 0) * MROWS + (F8 ? lane : (lane >> 1));
      int64_t o = o0 + r;
      o = o < O ? o : O - 1;
      msrc = wm + o * (MB ? MU : mstride) + (F8 ? 0 : 4 * (lane & 1));
    }
    // LX: request q of a wave fills rows 2 (wave + q NW) + {0, 1}; lane -> row + lane / 32,
    // physical 16-byte slot (lane / 4) % 8 (holding logical piece swz8(row, slot)), dword
    // lane % 4.  Its lifted dword of step s is D = 32 s + xd[q] of the row: lifted group
    // g = D / (2 (LX - 1)) (4 (LX - 1) positions, 2 LX raw positions), window w and dword
    // e within it, raw dword LX g + w + e.
    const unsigned char* xraw[LX > 0 ? NXL : 1];
    int xd[LX > 0 ? NXL : 1];
    if constexpr (LX > 0) {
#pragma unroll
      for (int q = 0; q < NXL; ++q) {
        const int r = (wave + q * NW) * 2 + (lane >> 5);
        int64_t t = t0 + r;
        t = t < T ? t : T - 1;
        xraw[q] = reinterpret_cast<const unsigned char*>(x) + t * ldxb;
        xd[q] = 4 * swz8(r, (lane >> 2) & 7) + (lane & 3);
      }
    }
    auto issue = [&](unsigned char* a, unsigned char* b, int s) {
      const int64_t v0 = (int64_t)(ks0 + s) * 64;   // value bytes per row per step: 64
#pragma unroll
      for (int q = 0; q < NV; ++q) g2lds16(vsrc[q] + v0, a + (wave + q * NW) * 1024);
      if (wave < NMWAVES) {
        if constexpr (F8) g2lds16(msrc + (ks0 + s) * mstep, a + SV_BYTES + wave * 1024);
        else g2lds4(msrc + (ks0 + s) * mstep, a + SV_BYTES + wave * 256);
      }
      if constexpr (LX > 0) {
        constexpr uint32_t P = 2 * (LX - 1);   // lifted dwords per group
#pragma unroll
        for (int q = 0; q < NXL; ++q) {
          const uint32_t D = (uint32_t)(ks0 + s) * 32u + (uint32_t)xd[q];
          const uint32_t g = D / P, rr = D - g * P;
          const int64_t raw = (int64_t)g * LX + (rr >> 1) + (rr & 1);
          g2lds4(xraw[q] + 4 * raw, b + (wave + q * NW) * 256);
        }
      } else {
#pragma unroll
        for (int q = 0; q < NX; ++q) g2lds16(xsrc[q] + (int64_t)(ks0 + s) * 128, b + (wave + q * NW) * 1024);
      }
    };
    // The B fragment of column block j + 1 is read while block j is multiplied; the wait
    // for it sits before the next reads (while a direct-to-LDS load is in flight the
    // compiler can only wait for all LDS reads, so a wait after them would stall on them).
    auto read_bv = [&](const unsigned char* b, int j) {
      const int c = wni * SN + j * 16 + fr;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(b + c * 128 + 16 * swz8(c, fg));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(b + c * 128 + 16 * swz8(c, 4 + fg));
      return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto compute = [&](const unsigned char* a, const unsigned char* b) {
      bf16x8 af[FI];
      int idx[FI];
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        const int r = wmi * SM + i * 16 + fr;
        af[i] = *reinterpret_cast<const bf16x8*>(a + r * 64 + 16 * swz4(r, fg));
        if constexpr (F8) idx[i] = *reinterpret_cast<const int*>(a + SV_BYTES + r * 16 + 4 * fg);
        else idx[i] = *reinterpret_cast<const uint16_t*>(a + SV_BYTES + r * 8 + 2 * fg);
      }
      u32x8 bcur = read_bv(b, 0), bnxt;
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < FJ) bnxt = read_bv(b, j + 1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        if constexpr (F8) {
          const i32x8 bv = __builtin_bit_cast(i32x8, bcur);
#pragma unroll
          for (int i = 0; i < FI; ++i)
            acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(__builtin_bit_cast(i32x4, af[i]), bv,
                                                                       acc[i][j], idx[i], 0, 0);
        } else {
          const bf16x16 bv = __builtin_bit_cast(bf16x16, bcur);
#pragma unroll
          for (int i = 0; i < FI; ++i)
            acc[i][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(af[i], bv, acc[i][j], idx[i], 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        bcur = bnxt;
      }
    };
    // direct-to-LDS requests per wave per sparse step: values and X (positions: some waves)
    if constexpr (NST == 2) k_loop2(nks, sA0, sB0, sA1, sB1, issue, compute);
    else lds_ring<NST, NV + NXL>(nks, SA, SB, issue, compute);
  }

  // ------------------------------------------------------------ dense phase ---
  if (nkd > 0) {
    // dense weight rows: groups of 8 rows (8 lanes x 16 bytes per row), ND per wave
    const uint16_t* dsrc[ND];
#pragma unroll
    for (int q = 0; q < ND; ++q) {
      const int r = (wave + q * NW) * 8 + (lane >> 3);
      int64_t o = o0 + r;
      o = o < O ? o : O - 1;
      dsrc[q] = wd + o * ldwd + 8 * swz8(r, lane & 7);
    }
    auto issue = [&](unsigned char* a, unsigned char* b, int s) {
      const int64_t j0 = (int64_t)(kd0 + s) * 64;
#pragma unroll
      for (int q = 0; q < ND; ++q) g2lds16(dsrc[q] + j0, a + (wave + q * NW) * 1024);
#pragma unroll
      for (int q = 0; q < NX; ++q) g2lds16(xsrc[q] + 2 * (dbase + j0), b + (wave + q * NW) * 1024);
    };
    // A fragments one row step ahead, waits before the next reads (as in the sparse phase)
    auto read_ad = [&](const unsigned char* a, int ks, int i) {
      const int r = wmi * SM + i * 16 + fr;
      return *reinterpret_cast<const bf16x8*>(a + r * 128 + 16 * swz8(r, 4 * ks + fg));
    };
    auto compute = [&](const unsigned char* a, const unsigned char* b) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 bfr[FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          const int c = wni * SN + j * 16 + fr;
          bfr[j] = *reinterpret_cast<const bf16x8*>(b + c * 128 + 16 * swz8(c, 4 * ks + fg));
        }
        bf16x8 acur = read_ad(a, ks, 0), anxt;
#pragma unroll
        for (int i = 0; i < FI; ++i) {
          __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
          __builtin_amdgcn_sched_barrier(0);
          if (i + 1 < FI) anxt = read_ad(a, ks, i + 1);
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int j = 0; j < FJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur, bfr[j], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_s_setprio(0);
          __builtin_amdgcn_sched_barrier(0);
          acur = anxt;
        }
      }
    };
    if constexpr (NST == 2) k_loop2(nkd, sA0, sB0, sA1, sB1, issue, compute);
    else lds_ring<NST, ND + NX>(nkd, SA, SB, issue, compute);
  }

  // epilogue: lane holds 4 consecutive o for one t in each 16x16 block; fp8 sums take
  // the token scale, then the row scale: y = (sum * s_t) * s_o
  const bool vec_ok = ((ldy & 3) == 0);
  if constexpr (F8) {
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int64_t ob = o0 + wmi * SM + i * 16 + 4 * fg;
      float wsr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) wsr[r] = wscale[ob + r < O ? ob + r : O - 1];
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int64_t t = t0 + wni * SN + j * 16 + fr;
        const float st = xscale[t < T ? t : T - 1];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = (acc[i][j][r] * st) * wsr[r];
      }
    }
  }
  if (part != nullptr) {
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int64_t ob = o0 + wmi * SM + i * 16 + 4 * fg;
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int64_t t = t0 + wni * SN + j * 16 + fr;
        if (t >= T) continue;
        float* pp = part + ((int64_t)kpart * T + t) * O + ob;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (ob + r < O) pp[r] = acc[i][j][r];
      }
    }
    return;
  }
  store_blocks<FI, FJ>(acc, y, ldy, T, O, o0 + wmi * SM, t0 + wni * SN, fr, fg, vec_ok && o0 + BM <= O, accumulate);
}

// o-tiles per band of the XCD-aware tile order: an XCD runs 32 tiles at a time, and a
// band g o-tiles wide keeps their K-step footprint g*BM + (32/g)*BN rows near its minimum
// (as for the dense direct-to-LDS kernel).
static int group_for(int tiles_m, int bm, int bn) {
  const int g = bn >= bm ? 8 : 4;
  return g < tiles_m ? g : tiles_m;
}

// K-blocked positions ([steps][rows][unit], unit = 8 or 16 bytes per row and step): a
// workgroup moves a block of 32 rows x 16 steps through LDS (small blocks: the copy is a
// few MB and needs many workgroups in flight to run at memory speed).
template <typename U>
__global__ __launch_bounds__(256) void k_meta_block(const uint8_t* __restrict__ meta, int64_t o, int64_t nsteps,
                                                    uint8_t* __restrict__ out) {
  // a block of 32 rows x 16 steps: each row's 16 units are read as one run, each step's
  // 32 rows written as one run
  __shared__ U tile[16][32 + 1];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 32, s0 = (int64_t)blockIdx.y * 16;
  const int64_t rowb = nsteps * (int64_t)sizeof(U);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rr = p * 16 + (tid >> 4), c = tid & 15;
    const int64_t row = r0 + rr, st = s0 + c;
    if (row < o && st < nsteps) tile[c][rr] = *reinterpret_cast<const U*>(meta + row * rowb + st * (int64_t)sizeof(U));
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c = p * 8 + (tid >> 5), rr = tid & 31;
    const int64_t row = r0 + rr, st = s0 + c;
    if (row < o && st < nsteps) *reinterpret_cast<U*>(out + (st * o + row) * (int64_t)sizeof(U)) = tile[c][rr];
  }
}

template <int BM, int BN, int WM, int WN, int NST = 2, int LX = 0>
hipError_t launch_sp_cfg(const SparseArgs& a, hipStream_t s, int64_t splits, float* part) {
  const int tiles_m = (int)((a.o + BM - 1) / BM), tiles_n = (int)((a.t + BN - 1) / BN);
  const int64_t ntiles = (int64_t)tiles_m * tiles_n;
  if (ntiles == 0) return hipSuccess;
  const int64_t nk = a.kc / (a.f8 ? 128 : 64) + a.kd / 64;
  if (splits < 1 || part == nullptr) splits = 1;
  const int64_t per = (nk + splits - 1) / splits;
  splits = per > 0 ? (nk + per - 1) / per : 1;
  if (ntiles * splits > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(ntiles * splits)), block(64 * WM * WN);
  const int steps = (int)(per > 0 ? per : 1), group = group_for(tiles_m, BM, BN);
  float* pp = splits > 1 ? part : nullptr;
#define NM_SP_LAUNCH(MBV, F8V, META)                                                                    \
  k_gemm_lds_sp<BM, BN, WM, WN, MBV, F8V, NST, LX><<<grid, block, 0, s>>>(                              \
      a.w_vals, META, a.kc, a.x, a.ldx, a.wd, a.ldwd, a.kd, a.dbase, a.t, a.o, a.y, a.ldy, a.accumulate, \
      tiles_m, tiles_n, steps, pp, group, a.x_scale, a.w_scale)
  if constexpr (LX > 0) {
    if (a.f8 || a.kd != 0) return hipErrorInvalidValue;
    if (a.w_meta_blk != nullptr) NM_SP_LAUNCH(true, false, a.w_meta_blk);
    else NM_SP_LAUNCH(false, false, a.w_meta);
  } else if (a.f8) {
    if (a.w_meta_blk != nullptr) NM_SP_LAUNCH(true, true, a.w_meta_blk);
    else NM_SP_LAUNCH(false, true, a.w_meta);
  } else {
    if (a.w_meta_blk != nullptr) NM_SP_LAUNCH(true, false, a.w_meta_blk);
    else NM_SP_LAUNCH(false, false, a.w_meta);
  }
#undef NM_SP_LAUNCH
  hipError_t e = hipGetLastError();
  a.route.note(NM_TAKEN_TILE_LDS | NM_TAKEN_SPARSE_MMA | (splits > 1 ? NM_TAKEN_TILE_SPLIT : 0u));
  if (e != hipSuccess || splits == 1) return e;
  return launch_reduce_parts(part, splits, Epi{}, a.t, a.o, a.y, a.ldy, a.accumulate, a.route, s);
}

// the configuration for lowered weights whose lifted X rows the loads build (N = a.ns)
template <int BM, int BN, int WM, int WN, int NST>
hipError_t launch_sp_lx(const SparseArgs& a, hipStream_t s, int64_t splits, float* part) {
  switch (a.ns) {
    case 2: return launch_sp_cfg<BM, BN, WM, WN, NST, 2>(a, s, splits, part);
    case 3: return launch_sp_cfg<BM, BN, WM, WN, NST, 3>(a, s, splits, part);
    case 4: return launch_sp_cfg<BM, BN, WM, WN, NST, 4>(a, s, splits, part);
    case 5: return launch_sp_cfg<BM, BN, WM, WN, NST, 5>(a, s, splits, part);
    case 6: return launch_sp_cfg<BM, BN, WM, WN, NST, 6>(a, s, splits, part);
    case 7: return launch_sp_cfg<BM, BN, WM, WN, NST, 7>(a, s, splits, part);
    case 8: return launch_sp_cfg<BM, BN, WM, WN, NST, 8>(a, s, splits, part);
  }
  return hipErrorInvalidValue;
}

// Few-token split: 128-row tiles, as many workgroups as fit one per CU.
int64_t sp_small_splits(const SparseArgs& a) {
  const int bn = a.t <= 64 ? 64 : 128;
  const int64_t tiles = ((a.o + 127) / 128) * ((a.t + bn - 1) / bn);
  const int64_t nk = a.kc / (a.f8 ? 128 : 64) + a.kd / 64;
  int64_t splits = (a.route.tile_wg > 0 ? a.route.tile_wg : 256) / tiles;
  if (splits > nk / 2) splits = nk / 2;
  return splits < 1 ? 1 : splits;
}

}  // namespace

namespace nml {

bool gemm_lds_sp_eligible(const SparseArgs& a, bool any_size) {
  const bool lifted = a.loader == XL_LIFT && a.lift_dma && a.kd == 0 && !a.f8 && a.ns >= 2 && a.ns <= 8;
  if ((a.loader != XL_PLAIN && !lifted) || a.trans_out) return false;
  if (a.kc % 64 != 0 || a.kd % 64 != 0 || (a.kc == 0 && a.kd == 0)) return false;
  if (a.f8 && (a.kc % 128 != 0 || a.kd != 0 || (a.ldx % 16) != 0 || a.x_scale == nullptr || a.w_scale == nullptr))
    return false;
  if ((a.ldx % 8) != 0 || (a.kd > 0 && ((a.ldwd % 8) != 0 || (a.dbase % 8) != 0))) return false;
  // enough 256 x 256 tiles to fill the machine
  return any_size || ((a.o + 255) / 256) * ((a.t + 255) / 256) >= 128;
}

int64_t meta_block_bytes(int64_t o, int64_t kc) { return o * (kc / 8); }

hipError_t launch_meta_block(const uint8_t* meta, int64_t o, int64_t kc, int unit, uint8_t* out, hipStream_t s) {
  if (unit != 8 && unit != 16) return hipErrorInvalidValue;
  const int64_t nsteps = kc / (8 * unit);
  if (o <= 0 || nsteps <= 0) return hipSuccess;
  const int64_t gx = (o + 31) / 32, gy = (nsteps + 15) / 16;
  if (gx > 0x7FFFFFFF || gy > 65535) return hipErrorInvalidConfiguration;
  if (unit == 8) k_meta_block<uint2><<<dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s>>>(meta, o, nsteps, out);
  else k_meta_block<uint4><<<dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s>>>(meta, o, nsteps, out);
  return hipGetLastError();
}

hipError_t launch_gemm_lds_sp(const SparseArgs& a, hipStream_t s) {
  // waves of 128 (o) x 64 (t): the dense X operand, read by WM waves, is the larger LDS
  // read stream, so WM = 2 beats 4 (measured 1-4% on gfx950)
  if (a.lift_dma && a.loader == XL_LIFT) return launch_sp_lx<256, 256, 2, 4, 2>(a, s, 1, nullptr);
  return launch_sp_cfg<256, 256, 2, 4>(a, s, 1, nullptr);
}

hipError_t launch_gemm_lds_sp_split(const SparseArgs& a, int64_t splits, float* part, int64_t part_bytes,
                                    hipStream_t s) {
  if (splits < 1 || part == nullptr || part_bytes < splits * a.t * a.o * 4) splits = 1;
  if (a.lift_dma && a.loader == XL_LIFT) return launch_sp_lx<256, 256, 2, 4, 2>(a, s, splits, part);
  return launch_sp_cfg<256, 256, 2, 4>(a, s, splits, part);
}

int64_t gemm_lds_sp_small_part_bytes(const SparseArgs& a) {
  const int64_t splits = sp_small_splits(a);
  return splits > 1 ? splits * a.t * a.o * 4 : 0;
}

hipError_t launch_gemm_lds_sp_small(const SparseArgs& a, float* part, int64_t part_bytes, hipStream_t s) {
  int64_t splits = sp_small_splits(a);
  if (part == nullptr || part_bytes < splits * a.t * a.o * 4) splits = 1;
  // three LDS stages (72 / 96 KiB): two K-steps in flight (four measured level)
  if (a.lift_dma && a.loader == XL_LIFT) {
    if (a.t <= 64) return launch_sp_lx<128, 64, 4, 2, 3>(a, s, splits, part);
    return launch_sp_lx<128, 128, 4, 2, 3>(a, s, splits, part);
  }
  if (a.t <= 64) return launch_sp_cfg<128, 64, 4, 2, 3>(a, s, splits, part);
  return launch_sp_cfg<128, 128, 4, 2, 3>(a, s, splits, part);
}

}  // namespace nml
