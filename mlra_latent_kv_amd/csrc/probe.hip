// Read-stream probe: the HBM read rate a plain streaming kernel reaches on this device, the
// practical ceiling next to the published peak.  Measurement support for the benchmark, not
// part of the decode path (libmla_probe.so, declared in include/mla_probe.h).
//
// Every lane reads 16 bytes per load (global_load_dwordx4), four loads in flight per lane,
// in a grid-stride sweep over the buffer; the loaded words are folded into one XOR per wave
// and stored, so the loads cannot be removed.  2048 workgroups of 256 threads (eight per CU).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "mla_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 2048;

__global__ __launch_bounds__(kThreads) void k_read_stream(const uint4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) out[(size_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = acc;
}

}  // namespace

extern "C" {

size_t mla_probe_out_words(void) { return (size_t)kBlocks * (kThreads / 64); }

int mla_probe_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream) {
  if (!buf || !out || bytes % 16) return 1;
  hipLaunchKernelGGL(k_read_stream, dim3(kBlocks), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(buf), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
