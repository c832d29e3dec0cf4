// Read-stream probe: the HBM read rate a plain streaming kernel reaches on this device, the
// practical ceiling next to the published peak.  Measurement support for the benchmark, not
// part of the decode path (libmla_probe.so, declared in include/mla_probe.h).
//
// Each of 512 workgroups (256 threads) streams one contiguous chunk of the buffer: per
// iteration every lane issues eight 16-byte non-temporal loads (global_load_dwordx4 nt) of
// consecutive 4 KiB blocks, so a workgroup has 32 KiB in flight; the few 16-byte units past
// the last whole chunk are read grid-stride.  Loaded words are folded into one XOR per wave
// and stored, so the loads cannot be removed.  (Non-temporal loads: the same hint the decode
// path's tile loads use; on MI355X a stream with it reaches ~7.0 TB/s, ~6.25 without.)
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "mla_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 512;
constexpr int kUnroll = 8;  // loads in flight per lane
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_read_stream(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ out) {
  constexpr size_t kStep = (size_t)kThreads * kUnroll;  // 16-byte units per iteration
  const size_t per = n16 / kBlocks / kStep * kStep;     // whole-iteration chunk per workgroup
  const u32x4* q = p + (size_t)blockIdx.x * per;
  uint32_t acc = 0;
  for (size_t i = threadIdx.x; i < per; i += kStep) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(q + i + kThreads * u);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // remainder past kBlocks whole chunks
  for (size_t i = (size_t)kBlocks * per + (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (size_t)kBlocks * kThreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
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
                     static_cast<const u32x4*>(buf), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
