// Measurement helpers: the achievable ceilings on the machine at hand, beside the
// nominal peaks (HBM 8 TB/s, bf16 matrix 2.5 PFLOP/s).  Not part of the method.
//  * nm_probe_read: one pass over a buffer, in one of three load forms --
//      mode 0: each lane loads 16 bytes at a grid stride, four loads in flight per lane;
//      mode 1: each workgroup reads one contiguous block, sixteen 16-byte loads in flight
//              per lane;
//      mode 2: each wave streams contiguous 16 KiB chunks straight into LDS with
//              direct-to-LDS 16-byte loads (the weight streams' load path), up to 32 of
//              its loads in flight.
//  * nm_probe_mfma: 16 independent chains of v_mfma_f32_16x16x32_bf16 per wave on
//    register-resident operands (no memory traffic), the matrix-pipe rate under this
//    kernel's clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nm_probe.h"
#include "nm_device.h"

namespace {

using namespace nmk;

constexpr int kReadBlocks = 2048, kReadThreads = 256;

__global__ __launch_bounds__(kReadThreads) void k_probe_read(const u32x4* __restrict__ p, int64_t n16,
                                                              uint32_t* __restrict__ sink) {
  const int64_t tid = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  const int64_t nth = (int64_t)gridDim.x * kReadThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = tid;
  for (; i + 3 * nth < n16; i += 4 * nth) {
    const u32x4 a = p[i], b = p[i + nth], c = p[i + 2 * nth], d = p[i + 3 * nth];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += nth) acc ^= p[i];
  sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

constexpr int kBlockUnroll = 16;

// mode 1: block b reads [b * chunk, (b + 1) * chunk) (chunk a multiple of 16 * 256 * 16
// bytes except in the last block), sixteen loads in flight per lane
__global__ __launch_bounds__(kReadThreads) void k_probe_read_block(const u32x4* __restrict__ p, int64_t n16,
                                                                    int64_t chunk16, uint32_t* __restrict__ sink) {
  const int64_t b0 = (int64_t)blockIdx.x * chunk16;
  int64_t b1 = b0 + chunk16;
  b1 = b1 < n16 ? b1 : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = b0 + threadIdx.x;
  for (; i + (kBlockUnroll - 1) * kReadThreads < b1; i += kBlockUnroll * kReadThreads) {
    u32x4 v[kBlockUnroll];
#pragma unroll
    for (int u = 0; u < kBlockUnroll; ++u) v[u] = p[i + u * kReadThreads];
#pragma unroll
    for (int u = 0; u < kBlockUnroll; ++u) acc ^= v[u];
  }
  for (; i < b1; i += kReadThreads) acc ^= p[i];
  sink[(int64_t)blockIdx.x * kReadThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

typedef __attribute__((address_space(3))) void lds_void;

// mode 2: wave w of block b streams its contiguous run of 16 KiB chunks into a 16 KiB LDS
// slot with direct-to-LDS loads (16 instructions of 1 KiB per chunk); a wave waits only
// when 32 of its loads are in flight, and for all of them at the end.
constexpr int kDmaThreads = 256, kDmaChunk = 16384;
__global__ __launch_bounds__(kDmaThreads) void k_probe_read_lds(const unsigned char* __restrict__ p, int64_t nchunks,
                                                                 int64_t per_wave, uint32_t* __restrict__ sink) {
  __shared__ __align__(16) unsigned char ring[kDmaThreads / 64][kDmaChunk];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * (kDmaThreads / 64) + wave;
  const int64_t c0 = gw * per_wave;
  int64_t c1 = c0 + per_wave;
  c1 = c1 < nchunks ? c1 : nchunks;
  for (int64_t c = c0; c < c1; ++c) {
    const unsigned char* g = p + c * kDmaChunk + lane * 16;
#pragma unroll
    for (int u = 0; u < kDmaChunk / 1024; ++u)
      __builtin_amdgcn_global_load_lds(g + u * 1024, (lds_void*)(&ring[wave][u * 1024]), 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(vm_wait(32));    // at most two chunks of loads still in flight
  }
  __builtin_amdgcn_s_waitcnt(vm_wait(0));       // every load has landed
  __syncthreads();
  sink[(int64_t)blockIdx.x * kDmaThreads + threadIdx.x] =
      *reinterpret_cast<const uint32_t*>(&ring[wave][lane * 16]);
}

constexpr int kMfmaBlocks = 1024, kMfmaThreads = 256, kChains = 16;

// The launch bound admits 1024-thread blocks on purpose: it caps the kernel at 128 VGPRs,
// so the compiler keeps the accumulators in VGPRs with each chain writing its own
// registers.  With a 256-thread bound it moved them to AGPRs with overlapping source and
// destination ranges, which chains every instruction to the one before (measured 1.34
// against 2.4 PFLOP/s).
__global__ __launch_bounds__(1024) void k_probe_mfma(int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  // operands: bf16 values in (0.5, 2) that vary by lane (register resident, no loads)
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1.0f + 0.0078125f * (float)((lane * 8 + e) & 63));
    b[e] = (__bf16)(1.0f - 0.00390625f * (float)((lane * 5 + e) & 63));
  }
  f32x4 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[(int64_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int64_t nm_probe_sink_bytes(void) {
  const int64_t a = (int64_t)kReadBlocks * kReadThreads * 4, b = (int64_t)kMfmaBlocks * kMfmaThreads * 4;
  return a > b ? a : b;
}

nm_status nm_probe_read(const void* buf, int64_t bytes, void* sink, int mode, void* stream) {
  if (bytes < 0 || (bytes % 16) != 0) return NM_ESHAPE;
  if (mode < 0 || mode > 2) return NM_EINVAL;
  if (mode == 2 && (bytes % kDmaChunk) != 0) return NM_ESHAPE;
  if (bytes > 0 && (buf == nullptr || sink == nullptr)) return NM_EINVAL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 15) != 0)
    return NM_EALIGN;
  if (bytes == 0) return NM_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == 0) {
    k_probe_read<<<dim3(kReadBlocks), dim3(kReadThreads), 0, s>>>(static_cast<const u32x4*>(buf), bytes / 16,
                                                                   static_cast<uint32_t*>(sink));
  } else if (mode == 1) {
    const int64_t n16 = bytes / 16, step = (int64_t)kBlockUnroll * kReadThreads;
    const int64_t chunk16 = ((n16 + kReadBlocks - 1) / kReadBlocks + step - 1) / step * step;
    k_probe_read_block<<<dim3(kReadBlocks), dim3(kReadThreads), 0, s>>>(static_cast<const u32x4*>(buf), n16,
                                                                         chunk16, static_cast<uint32_t*>(sink));
  } else {
    const int64_t nchunks = bytes / kDmaChunk, waves = (int64_t)kReadBlocks * (kDmaThreads / 64);
    const int64_t per_wave = (nchunks + waves - 1) / waves;
    k_probe_read_lds<<<dim3(kReadBlocks), dim3(kDmaThreads), 0, s>>>(static_cast<const unsigned char*>(buf),
                                                                       nchunks, per_wave,
                                                                       static_cast<uint32_t*>(sink));
  }
  return hipGetLastError() == hipSuccess ? NM_OK : NM_EHIP;
}

int64_t nm_probe_mfma_flops(int64_t iters) {
  return iters < 0 ? 0 : (int64_t)kMfmaBlocks * (kMfmaThreads / 64) * kChains * iters * 16 * 16 * 32 * 2;
}

nm_status nm_probe_mfma(int64_t iters, void* sink, void* stream) {
  if (iters < 0) return NM_ESHAPE;
  if (sink == nullptr) return NM_EINVAL;
  if ((reinterpret_cast<uintptr_t>(sink) & 15) != 0) return NM_EALIGN;
  k_probe_mfma<<<dim3(kMfmaBlocks), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream)>>>(
      iters, static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? NM_OK : NM_EHIP;
}

}  // extern "C"
