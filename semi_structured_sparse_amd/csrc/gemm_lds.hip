// Large-token dense-MFMA product with direct global->LDS staging:
//   Y[t][o] = sum_k A~[t][k] * W[o][k]
// where A~ is X itself (PRO_NONE: X already sparsified, or a dense layer) or X with the
// positions whose keep bit is clear zeroed (PRO_MASK: the bitmask of the per-group top-n
// selection -- Flexible (N:M) Activation Sparsity page, technical summary 2.A/2.C --
// produced by a separate select pass).
//
// gfx950 design:
//  * Both operands are K-contiguous rows.  A K-step moves 64 bf16 (128 bytes) of every
//    tile row straight from global memory into LDS with global_load_lds_dwordx4: one
//    wave instruction fills 8 whole rows (1 KiB, contiguous in LDS), so no VGPRs are
//    spent on staging and every global access is a full 128-byte line.  fp8 weights
//    move 64-byte rows of codes and are widened per fragment.
//  * LDS rows are unpadded; the 16-byte chunk c of row r lives at chunk c ^ ((r>>1)&7)
//    (c ^ ((r>>2)&3) for 64-byte rows), which keeps the 16-lane groups of a ds_read_b128
//    fragment read on distinct banks.
//  * Two LDS stages (64 KiB each for a 256x256 tile): each K-step first issues the loads
//    of the next step into the other stage, then multiplies; one barrier per K-step.
//    Fragments are read one matrix step ahead.  Measured on gfx950 (8192 x 14336 x 4096):
//    without the per-step loads the same loop runs at 2.1 PFLOP/s; 32-wide K-steps with
//    four stages (three steps in flight, branch-free steady state, no compiler-added
//    drains) were 13% slower than this (twice the barriers): 890 against 789 us.
//  * The keep mask travels with the X tile (two 32-bit words per row per K-step) and is
//    applied to each 8-element X fragment right after its LDS read.
//  * 8 waves (2 per SIMD), each owning a 64 (o) x 128 (t) block of 16x16 accumulators
//    (v_mfma_f32_16x16x32_bf16); 4 waves of 128 x 128 (one per SIMD) were 15% slower.
//    Workgroups are remapped so each XCD (own L2) runs a near-square block of tiles.
//  * The few-token shapes (128-row tiles, split K) reuse the kernel with three stages.
// Requirements (checked by the dispatcher): K % 64 == 0, 16-byte aligned rows.  Rows
// beyond T or O are read from the last valid row and their outputs are not stored.
#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;
using namespace nml;

constexpr int BK = 64;                 // bf16 per K-step

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }    // 8 pieces per row
__device__ __forceinline__ int swz4(int r, int c) { return c ^ ((r >> 2) & 3); }   // 4 pieces per row
template <int PC>
__device__ __forceinline__ int pswz(int r, int c) { return PC == 8 ? swz(r, c) : swz4(r, c); }

// global -> LDS copy of `bytes` (4 or 16) per lane: lane i writes lds + i * bytes.  The
// LDS address must be wave-uniform (it is passed in M0).
__device__ __forceinline__ void g2lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void g2lds4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}

// zero the halves of dword d whose bits (2q, 2q+1) of `bits` are clear
__device__ __forceinline__ uint32_t keep_pair(uint32_t d, uint32_t bits, int q) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_sbfe((int)bits, 2 * q, 1);      // 0 or ~0
  const uint32_t hi = (uint32_t)__builtin_amdgcn_sbfe((int)bits, 2 * q + 1, 1);
  return d & ((hi & 0xFFFF0000u) | (lo & 0x0000FFFFu));
}

template <int BM, int BN, int WM, int WN, int PRO, bool W8, int KH, int NST>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm_lds(
    const unsigned char* __restrict__ w, int64_t ldw, const uint16_t* __restrict__ x, int64_t ldx,
    const uint32_t* __restrict__ xmask, int64_t T, int64_t O, int64_t K, float* __restrict__ y,
    int64_t ldy, int accumulate, int tiles_m, int tiles_n, int64_t kslice, float* __restrict__ part,
    Epi epi, int group) {
  constexpr int NW = WM * WN;
  constexpr int SM = BM / WM, SN = BN / WN;       // wave sub-tile (o x t)
  constexpr int FI = SM / 16, FJ = SN / 16;
  // A K-step is KH halves of 32 positions.  Rows per step: X 64*KH bytes (8 or 4 pieces of
  // 16 bytes); W the same in bf16, or 32*KH bytes of fp8 codes.  A load group is 1 KiB.
  static_assert(KH == 2 || (KH == 1 && !W8 && PRO == PRO_NONE), "32-position steps: bf16, plain prologue");
  constexpr int SBK = 32 * KH;
  constexpr int XROWB = 2 * SBK, XPC = XROWB / 16, X_RPG = 64 / XPC;
  constexpr int AROWB = W8 ? SBK : XROWB, APC = AROWB / 16, A_RPG = 64 / APC;
  constexpr int A_BYTES = BM * AROWB, B_BYTES = BN * XROWB;
  constexpr int MASK_BYTES = (PRO == PRO_MASK) ? BN * 8 : 16;
  constexpr int A_GROUPS = BM / A_RPG, B_GROUPS = BN / X_RPG;
  constexpr int NGA = A_GROUPS / NW, NGB = B_GROUPS / NW;
  static_assert(A_GROUPS % NW == 0 && B_GROUPS % NW == 0, "load groups per wave");
  constexpr int MASK_GROUPS = (PRO == PRO_MASK) ? BN / 32 : 0;   // 32 rows x 2 words per inst

  // two to four stages as distinct arrays: every LDS access names its stage statically, so
  // the compiler tracks the loads into each stage separately
  static_assert(NST == 2 || (NST >= 3 && NST <= 4 && PRO == PRO_NONE), "deeper pipelines: plain prologue");
  constexpr int A2B = NST >= 3 ? A_BYTES : 16, B2B = NST >= 3 ? B_BYTES : 16;
  constexpr int A3B = NST >= 4 ? A_BYTES : 16, B3B = NST >= 4 ? B_BYTES : 16;
  __shared__ __align__(16) unsigned char sA0[A_BYTES], sB0[B_BYTES], sM0[MASK_BYTES];
  __shared__ __align__(16) unsigned char sA1[A_BYTES], sB1[B_BYTES], sM1[MASK_BYTES];
  __shared__ __align__(16) unsigned char sA2[A2B], sB2[B2B];
  __shared__ __align__(16) unsigned char sA3[A3B], sB3[B3B];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (LDS base goes to M0)
  const int wm = wave % WM, wn = wave / WM;

  // XCD-aware tile order: hardware places workgroup b on XCD b % 8; each XCD takes a
  // contiguous range of tiles, walked t-major inside bands of `group` o-tiles.
  // optional split-K: block b handles reduction slice b / ntiles and writes its fp32
  // partial tile to part[slice][t][o] (summed in slice order by a second kernel)
  const int ntiles = tiles_m * tiles_n;
  const int kpart = blockIdx.x / ntiles;
  int lin = blockIdx.x - kpart * ntiles;
  if ((ntiles & 7) == 0 && gridDim.x == (unsigned)ntiles) lin = (blockIdx.x & 7) * (ntiles >> 3) + (blockIdx.x >> 3);
  const int64_t kbeg = (int64_t)kpart * kslice;
  const int64_t kend = (kbeg + kslice < K) ? kbeg + kslice : K;
  const int band = lin / (group * tiles_n);
  const int band_w = min(group, tiles_m - band * group);
  const int inband = lin - band * group * tiles_n;
  const int tile_m = band * group + inband % band_w;
  const int tile_n = inband / band_w;
  const int64_t o0 = (int64_t)tile_m * BM, t0 = (int64_t)tile_n * BN;

  // per-lane global source addresses of this wave's load groups (K offset added per step)
  const unsigned char* asrc[NGA];
  const uint16_t* bsrc[NGB];
  constexpr int WBYTES = W8 ? 1 : 2;   // bytes per weight element
#pragma unroll
  for (int g = 0; g < NGA; ++g) {
    const int r = (wave + g * NW) * A_RPG + lane / APC;
    int64_t o = o0 + r;
    if (o >= O) o = O - 1;
    asrc[g] = w + (o * ldw) * WBYTES + 16 * pswz<APC>(r, lane % APC);
  }
#pragma unroll
  for (int g = 0; g < NGB; ++g) {
    const int r = (wave + g * NW) * X_RPG + lane / XPC;
    int64_t t = t0 + r;
    if (t >= T) t = T - 1;
    bsrc[g] = x + t * ldx + 8 * pswz<XPC>(r, lane % XPC);
  }
  const int64_t mwords = K >> 5;
  const uint32_t* msrc = nullptr;
  if constexpr (PRO == PRO_MASK) {
    if (wave < MASK_GROUPS) {
      int64_t t = t0 + wave * 32 + (lane >> 1);
      if (t >= T) t = T - 1;
      msrc = xmask + t * mwords + (lane & 1);
    }
  }
  // the slice's K offset is folded into the source addresses
#pragma unroll
  for (int g = 0; g < NGA; ++g) asrc[g] += kbeg * WBYTES;
#pragma unroll
  for (int g = 0; g < NGB; ++g) bsrc[g] += kbeg;
  if constexpr (PRO == PRO_MASK) {
    if (msrc != nullptr) msrc += kbeg >> 5;
  }

  auto issue_all = [&](unsigned char* a, unsigned char* b, unsigned char* mk, int64_t k0) {
#pragma unroll
    for (int g = 0; g < NGA; ++g) g2lds16(asrc[g] + k0 * WBYTES, a + (wave + g * NW) * 1024);
#pragma unroll
    for (int g = 0; g < NGB; ++g) g2lds16(bsrc[g] + k0, b + (wave + g * NW) * 1024);
    if constexpr (PRO == PRO_MASK) {
      if (wave < MASK_GROUPS) g2lds4(msrc + (k0 >> 5), mk + wave * 256);
    }
  };

  f32x4 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fq = lane >> 4;
  const int nk = (int)((kend - kbeg) / SBK);

  // Multiply one staged K-step (two 32-wide halves, FI row steps each).  Fragments are
  // read one step ahead: the A fragment of the next row step, and during the first half
  // the B fragments of the second, so no matrix instruction waits on the LDS read issued
  // just before it.  Scheduling barriers keep the compiler from sinking the early reads
  // below the matrix instructions.
  // A fragment: 8 bf16 (16 bytes), or 8 fp8 codes (8 bytes, widened when used)
  auto read_a = [&](const unsigned char* abase, int ks, int i) {
    const int r = wm * SM + i * 16 + fr;
    if constexpr (W8) {
      const uint2 q = *reinterpret_cast<const uint2*>(abase + r * 64 + 16 * swz4(r, 2 * ks + (fq >> 1)) + 8 * (fq & 1));
      return u32x4{q.x, q.y, 0u, 0u};
    } else {
      return *reinterpret_cast<const u32x4*>(abase + r * AROWB + 16 * pswz<APC>(r, 4 * ks + fq));
    }
  };
  auto a_frag = [&](u32x4 v) {
    if constexpr (W8) {
      uint32_t c0, c1, c2, c3;
      fp8x4_to_bf16x4(v[0], c0, c1);
      fp8x4_to_bf16x4(v[1], c2, c3);
      return __builtin_bit_cast(bf16x8, u32x4{c0, c1, c2, c3});
    } else {
      return __builtin_bit_cast(bf16x8, v);
    }
  };
  auto read_b = [&](const unsigned char* bbase, int ks, int j) {
    const int r = wn * SN + j * 16 + fr;
    return *reinterpret_cast<const u32x4*>(bbase + r * XROWB + 16 * pswz<XPC>(r, 4 * ks + fq));
  };
  auto compute = [&](const unsigned char* abase, const unsigned char* bbase, const unsigned char* mbase) {
    uint2 mw[FJ];
    if constexpr (PRO == PRO_MASK) {
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int r = wn * SN + j * 16 + fr;
        mw[j] = *reinterpret_cast<const uint2*>(mbase + r * 8);
      }
    }
    u32x4 b0[FJ], b1[FJ];
#pragma unroll
    for (int j = 0; j < FJ; ++j) b0[j] = read_b(bbase, 0, j);
    u32x4 acur = read_a(abase, 0, 0), anxt;
    constexpr int BPS = (FJ + FI - 1) / FI;   // second-half B fragments read per row step
#pragma unroll
    for (int ks = 0; ks < KH; ++ks) {
      bf16x8 bfr[FJ];
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        u32x4 v = ks ? b1[j] : b0[j];
        if constexpr (PRO == PRO_MASK) {
          const uint32_t word = ks ? mw[j].y : mw[j].x;
          const uint32_t bits = word >> (8 * fq);
          v[0] = keep_pair(v[0], bits, 0);
          v[1] = keep_pair(v[1], bits, 1);
          v[2] = keep_pair(v[2], bits, 2);
          v[3] = keep_pair(v[3], bits, 3);
        }
        bfr[j] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int i = 0; i < FI; ++i) {
        // Wait for the reads issued one step ago before issuing this step's: while a
        // direct-to-LDS load is in flight the compiler can only wait for all LDS reads,
        // so a wait placed after the new reads would also wait for them.
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < FI) anxt = read_a(abase, ks, i + 1);
        else if (ks + 1 < KH) anxt = read_a(abase, ks + 1, 0);
        if (ks + 1 < KH) {
#pragma unroll
          for (int q = 0; q < BPS; ++q)
            if (i * BPS + q < FJ) b1[i * BPS + q] = read_b(bbase, 1, i * BPS + q);
        }
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 af = a_frag(acur);
        __builtin_amdgcn_s_setprio(1);   // keep the matrix pipe fed ahead of the other wave's memory work
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        acur = anxt;
      }
    }
  };

  if constexpr (NST == 2) {
    issue_all(sA0, sB0, sM0, 0);
    __builtin_amdgcn_s_waitcnt(0);   // the staged tiles have landed in LDS
    __syncthreads();
    // Two K-steps per trip (stage 0, then stage 1).  Each step first issues the loads of
    // the step after it into the other stage (the first matrix step waits for every LDS
    // read anyway, so no later LDS read waits behind them); the last step reloads step 0
    // into the idle stage instead (never read), so every step runs the same code.
    for (int kt = 0; kt < nk; kt += 2) {
      issue_all(sA1, sB1, sM1, kt + 1 < nk ? (int64_t)(kt + 1) * SBK : 0);
      compute(sA0, sB0, sM0);
      __builtin_amdgcn_s_waitcnt(0);   // next stage landed in LDS
      __syncthreads();
      if (kt + 1 < nk) {
        issue_all(sA0, sB0, sM0, kt + 2 < nk ? (int64_t)(kt + 2) * SBK : 0);
        compute(sA1, sB1, sM1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    }
  } else {
    // NST stages, NST - 1 K-steps in flight (lds_ring)
    unsigned char* const SA[4] = {sA0, sA1, sA2, sA3};
    unsigned char* const SB[4] = {sB0, sB1, sB2, sB3};
    lds_ring<NST, NGA + NGB>(
        nk, SA, SB, [&](unsigned char* a, unsigned char* b, int ks) { issue_all(a, b, sM0, (int64_t)ks * SBK); },
        [&](const unsigned char* a, const unsigned char* b) { compute(a, b, sM0); });
  }

  // epilogue: lane holds 4 consecutive o for one t in each 16x16 block (the Epi terms --
  // per-row weight scale, per-token scale and shift term -- applied to the finished sums;
  // split-K partials get them in the reduction)
  const bool vec_ok = ((ldy & 3) == 0);
  const float* wscale = epi.w_scale;
#pragma unroll
  for (int i = 0; i < FI; ++i) {
    const int64_t ob = o0 + wm * SM + i * 16 + 4 * fq;
    if (wscale != nullptr && part == nullptr) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sc = (ob + r < O) ? wscale[ob + r] : 0.f;
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j][r] *= sc;
      }
    }
    if (epi.extra() && part == nullptr) {
      float cs[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) cs[r] = (epi.col_shift != nullptr && ob + r < O) ? epi.col_shift[ob + r] : 0.f;
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int64_t t = t0 + wn * SN + j * 16 + fr;
        const bool tin = t < T;
        const float rs = (epi.row_scale != nullptr && tin) ? epi.row_scale[t] : 1.f;
        const float rb = epi.row_shift != nullptr ? (tin ? epi.row_shift[t] : 0.f) : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = acc[i][j][r] * rs + rb * cs[r];
      }
    }
    if (part != nullptr) {
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int64_t t = t0 + wn * SN + j * 16 + fr;
        if (t >= T) continue;
        float* pp = part + ((int64_t)kpart * T + t) * O + ob;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (ob + r < O) pp[r] = acc[i][j][r];
      }
    }
  }
  if (part != nullptr) return;
  store_blocks<FI, FJ>(acc, y, ldy, T, O, o0 + wm * SM, t0 + wn * SN, fr, fq, vec_ok && o0 + BM <= O, accumulate);
}

// o-tiles per band of the XCD-aware tile order.  An XCD runs 32 tiles at a time (one per
// CU); a band g o-tiles wide makes that set g o-tiles x 32/g t-tiles, whose K-step
// footprint g*BM + (32/g)*BN rows is smallest near g = sqrt(32 BN / BM).  Measured on
// gfx950 at 8192 x 14336 x 4096: bands of 8 (or 4) o-tiles 711 us, of 16 736-820 us
// (every XCD then streamed all of W twice: 2.1 GB of L2 fills per launch).
static int group_for(int tiles_m, int bm, int bn) {
  const int g = bn >= bm ? 8 : 4;
  return g < tiles_m ? g : tiles_m;
}

template <int BM, int BN, int WM, int WN, int PRO, bool W8 = false, int KH = 2, int NST = 2>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s, int64_t splits, float* part) {
  const int tiles_m = (int)((a.o + BM - 1) / BM), tiles_n = (int)((a.t + BN - 1) / BN);
  const int64_t ntiles = (int64_t)tiles_m * tiles_n;
  if (ntiles == 0) return hipSuccess;
  int64_t kslice = ((a.k / BK + splits - 1) / splits) * BK;
  splits = (a.k + kslice - 1) / kslice;
  if (ntiles * splits > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  auto kern = k_gemm_lds<BM, BN, WM, WN, PRO, W8, KH, NST>;
  kern<<<dim3((unsigned)(ntiles * splits)), dim3(64 * WM * WN), 0, s>>>(
      (const unsigned char*)a.w, a.ldw, a.x, a.ldx, a.x_mask, a.t, a.o, a.k, a.y, a.ldy, a.accumulate, tiles_m, tiles_n,
      kslice, splits > 1 ? part : nullptr, a.epi(), group_for(tiles_m, BM, BN));
  hipError_t e = hipGetLastError();
  a.route.note(NM_TAKEN_TILE_LDS | (PRO == PRO_MASK ? NM_TAKEN_MASK : 0u) | (splits > 1 ? NM_TAKEN_TILE_SPLIT : 0u));
  if (e != hipSuccess || splits == 1) return e;
  return launch_reduce_parts(part, splits, a.epi(), a.t, a.o, a.y, a.ldy, a.accumulate, a.route, s);
}

}  // namespace

namespace nml {


// fp8 weights: rows of codes straight into LDS (ldw a multiple of 16 bytes), widened to
// bf16 per fragment; with the plain prologue only.
static bool w_rows_ok(const GemmArgs& a) {
  if (a.w_fp8) return a.prologue == PRO_NONE && (a.ldw % 16) == 0;
  return (a.ldw % 8) == 0;
}

bool gemm_lds_eligible(const GemmArgs& a, bool any_size) {
  if (a.prologue != PRO_NONE && a.prologue != PRO_MASK) return false;
  if (a.k % BK != 0 || a.k == 0) return false;
  if (!w_rows_ok(a) || (a.ldx % 8)) return false;
  // enough tiles to fill the machine with 256x256 tiles
  return any_size || ((a.o + 255) / 256) * ((a.t + 255) / 256) >= 128;
}

hipError_t launch_gemm_lds(const GemmArgs& a, hipStream_t s) {
  // 256 x 128 tiles (twice as many workgroups) when they finish in fewer rounds of one
  // workgroup per CU: a half tile stages 3/4 of a whole tile's bytes per K-step, and the
  // loads bound the kernel, so it takes about 3/4 of the time.  (128 whole tiles: one round
  // of 256 half tiles; 224 whole tiles: one round, against two rounds of half tiles.)
  const int64_t whole = ((a.o + 255) / 256) * ((a.t + 255) / 256), halves = ((a.o + 255) / 256) * ((a.t + 127) / 128);
  const bool half = ((halves + 255) / 256) * 3 < ((whole + 255) / 256) * 4;
  if (a.prologue == PRO_MASK) {
    if (half) return launch_cfg<256, 128, 4, 2, PRO_MASK>(a, s, 1, nullptr);
    return launch_cfg<256, 256, 4, 2, PRO_MASK>(a, s, 1, nullptr);
  }
  if (a.w_fp8) {
    if (half) return launch_cfg<256, 128, 4, 2, PRO_NONE, true>(a, s, 1, nullptr);
    return launch_cfg<256, 256, 4, 2, PRO_NONE, true>(a, s, 1, nullptr);
  }
  if (half) return launch_cfg<256, 128, 4, 2, PRO_NONE>(a, s, 1, nullptr);
  return launch_cfg<256, 256, 4, 2, PRO_NONE>(a, s, 1, nullptr);
}

// 256 x 256 tiles with the reduction split in `splits` K ranges, for token counts whose
// tiles fill under one round of workgroups (PRO_NONE, bf16 or fp8 weights); one range when
// `part` holds fewer than splits * t * o floats.
hipError_t launch_gemm_lds_split(const GemmArgs& a, int64_t splits, float* part, int64_t part_bytes, hipStream_t s) {
  if (a.prologue != PRO_NONE) return hipErrorInvalidValue;
  if (splits < 1 || part == nullptr || part_bytes < splits * a.t * a.o * 4) splits = 1;
  if (a.w_fp8) return launch_cfg<256, 256, 4, 2, PRO_NONE, true>(a, s, splits, part);
  return launch_cfg<256, 256, 4, 2, PRO_NONE>(a, s, splits, part);
}

// fp8 weights widened once to bf16 (exact), for the kernels that read bf16 weights only
// (kept as an A/B alternative to the fp8 direct-to-LDS variant).
__global__ void k_widen_fp8(const uint8_t* __restrict__ w8, int64_t ldw, int64_t O, int64_t K,
                            uint16_t* __restrict__ wb) {
  const int64_t per_row = K / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= O * per_row) return;
  const int64_t o = i / per_row, c = i - o * per_row;
  const uint2 q = *reinterpret_cast<const uint2*>(w8 + o * ldw + 8 * c);
  uint32_t c0, c1, c2, c3;
  fp8x4_to_bf16x4(q.x, c0, c1);
  fp8x4_to_bf16x4(q.y, c2, c3);
  *reinterpret_cast<uint4*>(wb + o * K + 8 * c) = make_uint4(c0, c1, c2, c3);
}

hipError_t launch_widen_fp8(const uint8_t* w8, int64_t ldw, int64_t o, int64_t k, uint16_t* wb, hipStream_t s) {
  if (k % 8) return hipErrorInvalidValue;
  const int64_t n = o * (k / 8);
  if (n == 0) return hipSuccess;
  k_widen_fp8<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(w8, ldw, o, k, wb);
  return hipGetLastError();
}

// Few-token variant: 128 output rows x 64 or 128 tokens per tile, split-K so that the
// grid has as many workgroups as fit one per CU (the splits' fp32 partial tiles are
// summed in slice order by a second kernel).  Measured on gfx950 for 33-128 tokens: one
// workgroup per CU beats two (twice the partial-sum traffic) and beats 256-row tiles
// (fewer tiles, so more splits); four waves of 64 x 32 measured level with eight waves.
// Three LDS stages (two K-steps in flight, lds_ring) against two, on gfx950: 4096 x 14336
// at 128 tokens 53.8 -> 47.9 us, the 64-token layer rows 10-14% faster; four stages
// measured level with three (within 3% either way).  The route's tile_wg sets another
// target workgroup count.
static int64_t small_splits(const GemmArgs& a) {
  const int64_t bn = a.t <= 64 ? 64 : 128;
  const int64_t target = a.route.tile_wg > 0 ? a.route.tile_wg : 256;
  const int64_t tiles = ((a.o + 127) / 128) * ((a.t + bn - 1) / bn);
  int64_t splits = target / tiles;
  const int64_t ksteps = a.k / BK;
  if (splits > ksteps / 2) splits = ksteps / 2;
  return splits < 1 ? 1 : splits;
}

bool gemm_lds_small_eligible(const GemmArgs& a) {
  return a.prologue == PRO_NONE && a.k % BK == 0 && a.k > 0 && w_rows_ok(a) && (a.ldx % 8) == 0;
}

int64_t gemm_lds_small_part_bytes(const GemmArgs& a) {
  const int64_t splits = small_splits(a);
  return splits > 1 ? splits * a.t * a.o * 4 : 0;
}

hipError_t launch_gemm_lds_small(const GemmArgs& a, float* part, int64_t part_bytes, hipStream_t s) {
  int64_t splits = small_splits(a);
  if (part == nullptr || part_bytes < splits * a.t * a.o * 4) splits = 1;
  if (a.w_fp8) {
    if (a.t <= 64) return launch_cfg<128, 64, 4, 2, PRO_NONE, true, 2, 3>(a, s, splits, part);
    return launch_cfg<128, 128, 4, 2, PRO_NONE, true, 2, 3>(a, s, splits, part);
  }
  if (a.t <= 64) return launch_cfg<128, 64, 4, 2, PRO_NONE, false, 2, 3>(a, s, splits, part);
  return launch_cfg<128, 128, 4, 2, PRO_NONE, false, 2, 3>(a, s, splits, part);
}

}  // namespace nml
