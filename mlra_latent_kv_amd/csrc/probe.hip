// Read-stream probe: the HBM read rate a plain streaming kernel reaches on this device, the
// practical ceiling next to the published peak; and an issue probe of the matrix core and the
// vector ALU.  Measurement support for the benchmark, not part of the decode path
// (libmla_probe.so, declared in include/mla_probe.h).
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

// Page-gather probe: the same stream over a paged pool, page by page in a given order (the
// order a decode reads a shuffled paged cache).  Workgroup g takes entries
// [g n / kBlocks, (g + 1) n / kBlocks) of the page list; its four waves take every fourth
// page of that range, each page's index read once (a uniform, scalar load), and stream it
// with eight non-temporal 16-byte loads in flight per lane.
__global__ __launch_bounds__(kThreads) void k_read_pages(const char* __restrict__ pool,
                                                         uint32_t page_units,
                                                         const int32_t* __restrict__ pages,
                                                         int n_pages,
                                                         uint32_t* __restrict__ out) {
  const int first = (int)((int64_t)blockIdx.x * n_pages / kBlocks);
  const int last = (int)((int64_t)(blockIdx.x + 1) * n_pages / kBlocks);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  constexpr uint32_t kStep = 64 * kUnroll;  // units per wave and iteration
  uint32_t acc = 0;
  for (int p = first + wave; p < last; p += kThreads / 64) {
    const int pg = __builtin_amdgcn_readfirstlane(pages[p]);
    const u32x4* q = reinterpret_cast<const u32x4*>(pool + (size_t)pg * ((size_t)page_units * 16));
    for (uint32_t i = lane; i < page_units; i += kStep) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t x = i + 64 * u;
        v[u] = x < page_units ? __builtin_nontemporal_load(q + x) : u32x4{};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) out[(size_t)blockIdx.x * (kThreads / 64) + wave] = acc;
}

// Issue probe: how the matrix core and the vector ALU share a SIMD.  One workgroup of 8
// waves per CU (two per SIMD; wave w runs on SIMD w % 4, so waves 0-3 and 4-7 pair up).
// Per iteration a matrix wave issues four independent MFMA 32x32x16 bf16 chains and a vector
// wave sixteen independent exp2(0.999 x) chains (v_mul + v_exp_f32).  Modes:
//   0  all 8 waves matrix            1  waves 0-3 matrix, waves 4-7 vector
//   2  waves 0-3 matrix, 4-7 idle    3  waves 4-7 vector, 0-3 idle
//   4  all 8 waves both, interleaved in one instruction stream
//   5  all 8 waves vector            6  waves 0-3 both, interleaved, 4-7 idle (one wave
//                                       per SIMD feeding both units from one stream)
// AGPR: accumulators in the accumulation registers (MFMA written as inline asm with an "a"
// operand) instead of the architectural ones.  The per-lane results go to `out` so nothing
// is removed; their values mean nothing.
constexpr int kIssueBlocks = 256, kIssueThreads = 512;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int MODE, bool AGPR>
__global__ __launch_bounds__(kIssueThreads, 1) void k_issue_probe(float* __restrict__ out, int iters,
                                                                  float seed) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = w >> 2;
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (threadIdx.x + i));
    b[i] = (__bf16)(seed * i);
  }
  f32x16_t acc[4] = {};
  float v[16];
  for (int i = 0; i < 16; ++i) v[i] = seed * (threadIdx.x + i);
  auto mfma4 = [&]() {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (AGPR)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[c]) : "v"(a), "v"(b));
      else
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
  };
  auto exp16 = [&]() {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = __builtin_amdgcn_exp2f(v[i] * 0.999f);
  };
  if (MODE == 4 || (MODE == 6 && grp == 0)) {
    for (int it = 0; it < iters; ++it) {
      mfma4();
      exp16();
    }
  } else if (MODE != 6) {
    const bool matrix = MODE == 0 || (MODE <= 2 && grp == 0);
    const bool vector = MODE == 5 || (MODE == 1 && grp == 1) || (MODE == 3 && grp == 1);
    if (matrix)
      for (int it = 0; it < iters; ++it) mfma4();
    if (vector)
      for (int it = 0; it < iters; ++it) exp16();
  }
  float r = 0.0f;
  for (int c = 0; c < 4; ++c)
    for (int i = 0; i < 16; ++i) r += acc[c][i];
  for (int i = 0; i < 16; ++i) r += v[i];
  out[(size_t)blockIdx.x * kIssueThreads + threadIdx.x] = r;
}

template <bool AGPR>
hipError_t launch_issue(int mode, float* out, int iters, hipStream_t s) {
  const dim3 g(kIssueBlocks), t(kIssueThreads);
  switch (mode) {
    case 0: hipLaunchKernelGGL((k_issue_probe<0, AGPR>), g, t, 0, s, out, iters, 1e-3f); break;
    case 1: hipLaunchKernelGGL((k_issue_probe<1, AGPR>), g, t, 0, s, out, iters, 1e-3f); break;
    case 2: hipLaunchKernelGGL((k_issue_probe<2, AGPR>), g, t, 0, s, out, iters, 1e-3f); break;
    case 3: hipLaunchKernelGGL((k_issue_probe<3, AGPR>), g, t, 0, s, out, iters, 1e-3f); break;
    case 4: hipLaunchKernelGGL((k_issue_probe<4, AGPR>), g, t, 0, s, out, iters, 1e-3f); break;
    case 6: hipLaunchKernelGGL((k_issue_probe<6, AGPR>), g, t, 0, s, out, iters, 1e-3f); break;
    default: hipLaunchKernelGGL((k_issue_probe<5, AGPR>), g, t, 0, s, out, iters, 1e-3f); break;
  }
  return hipGetLastError();
}

}  // namespace

extern "C" {

int mla_probe_read_pages(const void* pool, size_t page_bytes, const int32_t* pages,
                         int n_pages, uint32_t* out, hipStream_t stream) {
  if (!pool || !pages || !out || n_pages < 1 || page_bytes == 0 || page_bytes % 16 ||
      page_bytes / 16 > (1u << 20))
    return 1;
  hipLaunchKernelGGL(k_read_pages, dim3(kBlocks), dim3(kThreads), 0, stream,
                     static_cast<const char*>(pool), (uint32_t)(page_bytes / 16), pages, n_pages,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

size_t mla_probe_issue_out_words(void) { return (size_t)kIssueBlocks * kIssueThreads; }

int mla_probe_issue(int mode, int agpr, int iters, float* out, hipStream_t stream) {
  if (!out || mode < 0 || mode > 6 || iters < 1 || iters > (1 << 20)) return 1;
  const hipError_t e = agpr ? launch_issue<true>(mode, out, iters, stream)
                            : launch_issue<false>(mode, out, iters, stream);
  return e == hipSuccess ? 0 : 6;
}

size_t mla_probe_out_words(void) { return (size_t)kBlocks * (kThreads / 64); }

int mla_probe_read(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream) {
  if (!buf || !out || bytes % 16) return 1;
  hipLaunchKernelGGL(k_read_stream, dim3(kBlocks), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
