// stream_read.hip -- the read-bandwidth references bench.py times beside the hot
// path (libpkv_probe.so, not part of the attention library): every byte of a buffer
// read once, two ways.
//   stream_read_kernel: each workgroup streams one contiguous share with 16-byte
//   vector loads into registers, sixteen in flight per lane (16 KiB per wave), two
//   workgroups per CU; each thread folds what it read into one word so the loads
//   stay live, and writes that word to a small sink.  (Contiguous shares with 16
//   loads in flight read fastest of the grid-stride and contiguous variants at 4-16
//   loads and 1-16 workgroups per CU.)
//   stream_read_lds_kernel: the decode kernels' way -- four waves per CU, each
//   streaming its contiguous share straight into LDS with global_load_lds, 16 KiB
//   per step, one step in flight while the previous one lands.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "mfma_common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;
constexpr size_t kStep = (size_t)kUnroll * kThreads;  // 16-byte words per workgroup iteration

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                              uint32_t* __restrict__ sink) {
  // Workgroup w reads words [w * share, (w + 1) * share), share a multiple of kStep; the
  // words past grid * share (fewer than grid * kStep) are read by a grid-stride tail.
  const size_t share = n16 / gridDim.x / kStep * kStep;
  const uint4* p = src + (size_t)blockIdx.x * share + threadIdx.x;
  uint32_t acc = 0;
  for (size_t off = 0; off < share; off += kStep) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = p[off + (size_t)u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  const size_t tid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (size_t i = share * gridDim.x + tid; i < n16; i += (size_t)gridDim.x * kThreads) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = acc;
}

constexpr int kDmaWaves = 4;
constexpr int kDmaStep = 16 * 1024;  // bytes one wave copies per step (16 DMAs of 1 KiB)

__global__ __launch_bounds__(kDmaWaves * 64) void stream_read_lds_kernel(const unsigned char* __restrict__ src,
                                                                       size_t bytes_per_wave) {
  __shared__ __attribute__((aligned(16))) unsigned char slots[kDmaWaves][2][kDmaStep];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const unsigned char* base = src + ((size_t)blockIdx.x * kDmaWaves + wave) * bytes_per_wave + 16 * lane;
  const size_t steps = bytes_per_wave / kDmaStep;
  for (size_t s = 0; s < steps; ++s) {
    unsigned char* dst = slots[wave][s & 1];
#pragma unroll
    for (int i = 0; i < kDmaStep / 1024; ++i) pkv::load_lds16(base + s * kDmaStep + 1024 * i, dst + 1024 * i);
    pkv::wait_vm<kDmaStep / 1024>();  // the previous step has landed; this one stays in flight
  }
  pkv::wait_vm<0>();
}

}  // namespace

extern "C" {

// Words the sink must hold for a launch of `workgroups` workgroups.
size_t pkv_probe_sink_words(int32_t workgroups) { return (size_t)workgroups * kThreads; }

// Read `bytes` (a multiple of 16, 16-byte aligned) of device memory at src once;
// sink: device array of pkv_probe_sink_words(workgroups) words.  0 on success.
int pkv_probe_stream_read(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes % 16 != 0 || workgroups <= 0 || (reinterpret_cast<uintptr_t>(src) & 15u)) return 1;
  stream_read_kernel<<<workgroups, kThreads, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const uint4*>(src),
                                                                                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The LDS-DMA read of `bytes` at src by `workgroups` workgroups of four waves:
// bytes must be a multiple of workgroups * 4 * 16 KiB.  0 on success.
int pkv_probe_stream_read_lds(const void* src, size_t bytes, int32_t workgroups, void* stream) {
  const size_t per_wave = workgroups > 0 ? bytes / ((size_t)workgroups * kDmaWaves) : 0;
  if (!src || workgroups <= 0 || per_wave == 0 || per_wave % kDmaStep != 0 ||
      per_wave * workgroups * kDmaWaves != bytes || (reinterpret_cast<uintptr_t>(src) & 15u))
    return 1;
  stream_read_lds_kernel<<<workgroups, kDmaWaves * 64, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const unsigned char*>(src), per_wave);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
