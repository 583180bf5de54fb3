// Group top-n select / compact / decompress kernels.
//
// Selection rule: in each group of m contiguous values along K keep the n of largest
// magnitude, ties to the lower index ("ACT" score of the Flexible (N:M) Activation
// Sparsity page, technical summary sections 2.A and 2.C).  Compressed form: kept values
// in ascending position plus one index byte (in-group position) per kept value, or two
// bits per kept value for 2:4.
//
// Work decomposition: one wavefront owns a strip of 64 consecutive groups of one row;
// lane l owns group g0 + l.  A lane loads its whole group with one to four 16-byte
// loads (8 bytes for m = 4), so consecutive lanes read consecutive memory.  Ranking is
// in registers (nm_device.h).  Compaction of the kept values goes through a per-wave
// LDS strip so that the global writes of values and index bytes are contiguous.
#include "nm_device.h"
#include "nm_launch.h"

namespace {

using namespace nmk;

constexpr int kWavesPerBlock = 4;
constexpr int kMaxN = 32;

// widths that are not a multiple of 8 (other than 4) move dword by dword
template <int M>
constexpr bool kDwordGroups = (M % 8) != 0 && M != 4;

template <int M>
__device__ __forceinline__ void load_group(const uint16_t* p, uint32_t (&d)[M / 2]) {
  if constexpr (kDwordGroups<M>) {
#pragma unroll
    for (int q = 0; q < M / 2; ++q) d[q] = reinterpret_cast<const uint32_t*>(p)[q];
  } else if constexpr (M == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    d[0] = v.x; d[1] = v.y;
  } else {
#pragma unroll
    for (int c = 0; c < M / 8; ++c) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[c];
      d[4 * c + 0] = v.x; d[4 * c + 1] = v.y; d[4 * c + 2] = v.z; d[4 * c + 3] = v.w;
    }
  }
}

template <int M>
__device__ __forceinline__ void store_group(uint16_t* p, const uint32_t (&d)[M / 2]) {
  if constexpr (kDwordGroups<M>) {
#pragma unroll
    for (int q = 0; q < M / 2; ++q) reinterpret_cast<uint32_t*>(p)[q] = d[q];
  } else if constexpr (M == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(d[0], d[1]);
  } else {
#pragma unroll
    for (int c = 0; c < M / 8; ++c)
      reinterpret_cast<uint4*>(p)[c] = make_uint4(d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]);
  }
}

// Copy `count` u16 from an LDS strip (16-byte aligned) to global memory, lanes striding by
// 64: 16-byte pieces where the destination and count allow, else dwords or single values.
__device__ __forceinline__ void copy_u16(uint16_t* dst, const uint16_t* lds, int count, int lane) {
  if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0 && (count & 7) == 0) {
    for (int e = lane; e < count / 8; e += 64)
      reinterpret_cast<uint4*>(dst)[e] = reinterpret_cast<const uint4*>(lds)[e];
  } else if ((reinterpret_cast<uintptr_t>(dst) & 3) == 0) {
    const int pairs = count >> 1;
    for (int e = lane; e < pairs; e += 64)
      reinterpret_cast<uint32_t*>(dst)[e] = reinterpret_cast<const uint32_t*>(lds)[e];
    if ((count & 1) && lane == 0) dst[count - 1] = lds[count - 1];
  } else {
    for (int e = lane; e < count; e += 64) dst[e] = lds[e];
  }
}

__device__ __forceinline__ void copy_u8(uint8_t* dst, const uint8_t* lds, int count, int lane) {
  if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0 && (count & 15) == 0) {
    for (int e = lane; e < count / 16; e += 64)
      reinterpret_cast<uint4*>(dst)[e] = reinterpret_cast<const uint4*>(lds)[e];
  } else if ((reinterpret_cast<uintptr_t>(dst) & 3) == 0) {
    const int quads = count >> 2;
    for (int e = lane; e < quads; e += 64)
      reinterpret_cast<uint32_t*>(dst)[e] = reinterpret_cast<const uint32_t*>(lds)[e];
    const int rem = count & 3;
    if (lane < rem) dst[quads * 4 + lane] = lds[quads * 4 + lane];
  } else {
    for (int e = lane; e < count; e += 64) dst[e] = lds[e];
  }
}

// NT: n as a compile-time constant (the half-density patterns), or 0 for any n.
template <int M, int NT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_select(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx, int n,
    uint16_t* __restrict__ y, int64_t ldy, uint32_t* __restrict__ mask,
    uint16_t* __restrict__ values, uint8_t* __restrict__ meta, int meta_2bit, int yblk) {
  // per-wave compaction strips (+64 dump slots for pruned elements)
  __shared__ __align__(16) uint16_t s_val[kWavesPerBlock][64 * (kMaxN + 1)];
  __shared__ __align__(16) uint8_t s_idx[kWavesPerBlock][64 * (kMaxN + 1)];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t G = k / M;
  const int64_t strips_per_row = (G + 63) >> 6;
  const int64_t strip = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const bool strip_ok = strip < rows * strips_per_row;
  const int64_t row = strip_ok ? strip / strips_per_row : 0;
  const int64_t g0 = strip_ok ? (strip - row * strips_per_row) * 64 : 0;
  const int64_t g = g0 + lane;
  const bool valid = strip_ok && g < G;
  const int nvalid = strip_ok ? (int)((G - g0) < 64 ? (G - g0) : 64) : 0;

  uint32_t d[M / 2];
  if (valid) {
    load_group<M>(x + row * ldx + g * M, d);
  } else {
#pragma unroll
    for (int q = 0; q < M / 2; ++q) d[q] = 0;
  }
  uint32_t keep = 0u;
  if (valid) {
    if constexpr (kDwordGroups<M>) keep = topn_bits_pad<M, (M <= 8 ? 8 : 16)>(d, n);
    else if constexpr (NT > 0) keep = topn_bits_n<M, NT>(d);
    else keep = topn_bits<M>(d, n);
  }

  if (y != nullptr && valid) {
    uint32_t o[M / 2];
#pragma unroll
    for (int q = 0; q < M / 2; ++q) o[q] = mask_pair(d[q], keep >> (2 * q));
    // yblk (M divides 32, k % 32 == 0): S(X) in blocks of 16 token rows, each 32-position
    // piece of the block's rows contiguous: [row / 16][k / 32][row % 16][32]
    uint16_t* yp = y + row * ldy + g * M;
    if constexpr (32 % M == 0)
      if (yblk) yp = y + (row >> 4) * (k * 16) + (((g * M) >> 5) << 9) + (row & 15) * 32 + ((g * M) & 31);
    store_group<M>(yp, o);
  }

  if constexpr (32 % M == 0) if (mask != nullptr) {
    uint32_t w = keep << ((uint32_t)(g * M) & 31u);
    if constexpr (M < 32) {
#pragma unroll
      for (int off = 1; off < 32 / M; off <<= 1) w |= __shfl_xor(w, off, 64);
    }
    const int64_t words = (k + 31) >> 5;
    if (valid && (lane % (32 / M)) == 0) mask[row * words + ((g * M) >> 5)] = w;
  }

  if (values != nullptr) {
    // compaction: kept element i of lane l goes to strip slot l*n + rank-among-kept
    uint16_t* sv = s_val[wave];
    uint8_t* si = s_idx[wave];
    const int dump = 64 * n + lane;
    int slot = lane * n;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const bool kp = (keep >> i) & 1u;
      const int a = kp ? slot : dump;
      sv[a] = (uint16_t)(d[i >> 1] >> (16 * (i & 1)));
      si[a] = (uint8_t)i;
      slot += kp ? 1 : 0;
    }
    __syncthreads();
    if (strip_ok) {
      const int64_t kc = G * n;  // compressed row length
      copy_u16(values + row * kc + g0 * n, sv, nvalid * n, lane);
      if (!meta_2bit) {
        copy_u8(meta + row * kc + g0 * n, si, nvalid * n, lane);
      } else {
        // 2:4: two kept positions per group -> one nibble; two groups per byte
        const uint32_t p0 = (uint32_t)__builtin_ctz(keep | 0x10u);
        const uint32_t p1 = 31u - (uint32_t)__builtin_clz(keep | 1u);
        uint32_t nib = (p0 & 3u) | ((p1 & 3u) << 2);
        const uint32_t other = __shfl_down(nib, 1, 64);
        const int64_t mstride = (k + 7) >> 3;
        if (valid && (lane & 1) == 0) {
          const uint32_t b = nib | ((g + 1 < G ? other : 0u) << 4);
          meta[row * mstride + (g >> 1)] = (uint8_t)b;
        }
      }
    }
  }
}

template <int M>
__global__ __launch_bounds__(256) void k_decompress(
    const uint16_t* __restrict__ values, const uint8_t* __restrict__ meta, int meta_2bit,
    int64_t rows, int64_t k, int n, uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t G = k / M;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * G) return;
  const int64_t row = gid / G, g = gid - row * G;
  const int64_t kc = G * n;
  uint32_t out[M / 2];
#pragma unroll
  for (int q = 0; q < M / 2; ++q) out[q] = 0;
  for (int j = 0; j < n; ++j) {
    const uint32_t v = values[row * kc + g * n + j];
    uint32_t pos;
    if (meta_2bit) {
      const int64_t slot = g * n + j;
      pos = (meta[row * ((k + 7) >> 3) + (slot >> 2)] >> (2 * (slot & 3))) & 3u;
    } else {
      pos = (uint32_t)meta[row * kc + g * n + j] % (uint32_t)M;
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if (pos == (uint32_t)i) out[i >> 1] |= v << (16 * (i & 1));
    }
  }
  store_group<M>(y + row * ldy + g * M, out);
}

// Scored selection: the top-n of each group by score (topn_bits_scored) instead of by
// magnitude; outputs S(X) and/or the bitmask.  Lane l owns group g0 + l as in k_select
// and reads the group's M column scores with 16-byte loads (col_score is shared by all
// rows, so it stays in cache).
template <int M, int NT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void k_select_scored(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx, int n,
    const float* __restrict__ col_score, int use_x, uint16_t* __restrict__ y, int64_t ldy,
    uint32_t* __restrict__ mask) {
  static_assert(M >= 4 && 32 % M == 0, "power-of-two widths 4..32");
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t G = k / M;
  const int64_t strips_per_row = (G + 63) >> 6;
  const int64_t strip = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  const bool strip_ok = strip < rows * strips_per_row;
  const int64_t row = strip_ok ? strip / strips_per_row : 0;
  const int64_t g0 = strip_ok ? (strip - row * strips_per_row) * 64 : 0;
  const int64_t g = g0 + lane;
  const bool valid = strip_ok && g < G;

  uint32_t d[M / 2];
  float c[M];
  if (valid) {
    load_group<M>(x + row * ldx + g * M, d);
#pragma unroll
    for (int q = 0; q < M / 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(col_score + g * M)[q];
      c[4 * q] = v.x; c[4 * q + 1] = v.y; c[4 * q + 2] = v.z; c[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < M / 2; ++q) d[q] = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) c[i] = 0.f;
  }
  const uint32_t keep = valid ? topn_bits_scored<M, NT>(d, c, n, use_x != 0) : 0u;

  if (y != nullptr && valid) {
    uint32_t o[M / 2];
#pragma unroll
    for (int q = 0; q < M / 2; ++q) o[q] = mask_pair(d[q], keep >> (2 * q));
    store_group<M>(y + row * ldy + g * M, o);
  }
  if (mask != nullptr) {
    uint32_t w = keep << ((uint32_t)(g * M) & 31u);
    if constexpr (M < 32) {
#pragma unroll
      for (int off = 1; off < 32 / M; off <<= 1) w |= __shfl_xor(w, off, 64);
    }
    const int64_t words = (k + 31) >> 5;
    if (valid && (lane % (32 / M)) == 0) mask[row * words + ((g * M) >> 5)] = w;
  }
}

}  // namespace

namespace nml {

hipError_t launch_select_scored(int m, const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, int n,
                                const float* col_score, int use_x, uint16_t* y, int64_t ldy, uint32_t* mask,
                                hipStream_t s) {
  const int64_t G = k / m;
  const int64_t strips = rows * ((G + 63) / 64);
  const int64_t blocks = (strips + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(64 * kWavesPerBlock);
#define NM_SCORED(MM)                                                                              \
  if (n == (MM) / 2)                                                                               \
    k_select_scored<MM, (MM) / 2><<<grid, block, 0, s>>>(x, rows, k, ldx, n, col_score, use_x, y, ldy, mask); \
  else                                                                                             \
    k_select_scored<MM, 0><<<grid, block, 0, s>>>(x, rows, k, ldx, n, col_score, use_x, y, ldy, mask);
  switch (m) {
    case 4: NM_SCORED(4) break;
    case 8: NM_SCORED(8) break;
    case 16: NM_SCORED(16) break;
    case 32: NM_SCORED(32) break;
    default: return hipErrorInvalidValue;
  }
#undef NM_SCORED
  return hipGetLastError();
}

hipError_t launch_select(int m, const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, int n,
                         uint16_t* y, int64_t ldy, uint32_t* mask, uint16_t* values,
                         uint8_t* meta, int meta_2bit, hipStream_t s, int yblk) {
  if (yblk && (32 % m != 0 || k % 32 != 0)) return hipErrorInvalidValue;
  const int64_t G = k / m;
  const int64_t strips = rows * ((G + 63) / 64);
  const int64_t blocks = (strips + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(64 * kWavesPerBlock);
#define NM_SELECT(MM)                                                                              \
  if (n == (MM) / 2)                                                                               \
    k_select<MM, (MM) / 2><<<grid, block, 0, s>>>(x, rows, k, ldx, n, y, ldy, mask, values, meta, meta_2bit, yblk); \
  else                                                                                             \
    k_select<MM, 0><<<grid, block, 0, s>>>(x, rows, k, ldx, n, y, ldy, mask, values, meta, meta_2bit, yblk);
  switch (m) {
    case 4: NM_SELECT(4) break;
    case 8: NM_SELECT(8) break;
    case 16: NM_SELECT(16) break;
    case 32: NM_SELECT(32) break;
    case 6: k_select<6, 0><<<grid, block, 0, s>>>(x, rows, k, ldx, n, y, ldy, nullptr, values, meta, meta_2bit, 0); break;
    case 10: k_select<10, 0><<<grid, block, 0, s>>>(x, rows, k, ldx, n, y, ldy, nullptr, values, meta, meta_2bit, 0); break;
    case 12: k_select<12, 0><<<grid, block, 0, s>>>(x, rows, k, ldx, n, y, ldy, nullptr, values, meta, meta_2bit, 0); break;
    case 14: k_select<14, 0><<<grid, block, 0, s>>>(x, rows, k, ldx, n, y, ldy, nullptr, values, meta, meta_2bit, 0); break;
    default: return hipErrorInvalidValue;
  }
#undef NM_SELECT
  return hipGetLastError();
}

hipError_t launch_decompress(int m, const uint16_t* values, const uint8_t* meta, int meta_2bit,
                             int64_t rows, int64_t k, int n, uint16_t* y, int64_t ldy, hipStream_t s) {
  const int64_t groups = rows * (k / m);
  const int64_t blocks = (groups + 255) / 256;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(256);
  switch (m) {
    case 4: k_decompress<4><<<grid, block, 0, s>>>(values, meta, meta_2bit, rows, k, n, y, ldy); break;
    case 8: k_decompress<8><<<grid, block, 0, s>>>(values, meta, meta_2bit, rows, k, n, y, ldy); break;
    case 16: k_decompress<16><<<grid, block, 0, s>>>(values, meta, meta_2bit, rows, k, n, y, ldy); break;
    case 32: k_decompress<32><<<grid, block, 0, s>>>(values, meta, meta_2bit, rows, k, n, y, ldy); break;
    case 6: k_decompress<6><<<grid, block, 0, s>>>(values, meta, meta_2bit, rows, k, n, y, ldy); break;
    case 10: k_decompress<10><<<grid, block, 0, s>>>(values, meta, meta_2bit, rows, k, n, y, ldy); break;
    case 12: k_decompress<12><<<grid, block, 0, s>>>(values, meta, meta_2bit, rows, k, n, y, ldy); break;
    case 14: k_decompress<14><<<grid, block, 0, s>>>(values, meta, meta_2bit, rows, k, n, y, ldy); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nml
