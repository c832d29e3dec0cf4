// Split plan of one decode call, made on the device from seqlens by one workgroup of 256
// threads (an extra workgroup of the prologue launch, so the plan costs no launch).
//
// The main loop is split over the sequence (split-K): every sequence b with L_b tokens,
// p_b = ceil(L_b / 64) pages, is cut into n_b = ceil(p_b / c) work items of c whole pages
// (the last one ragged), item j covering tokens [64cj, min(L_b, 64c(j + 1))).  Work items
// are numbered sequence-major; split_off[b] is the first item of sequence b and
// split_off[B] = W, the item count, so the combine finds a variable number of splits per
// sequence.  Sequences with no tokens get no item.
//
// Balance: every item costs at most c pages and one workgroup set per item fills the chip
// once when W <= target, so the automatic plan takes the smallest c with
// sum_b ceil(p_b / c) <= target (binary search; the sum only falls as c grows), or
// c = max_b p_b (one item per sequence) when no c meets the target.  With num_splits given,
// c is fixed by the host.
//
// Dispatch table: the main kernels map their blocks to slots; slot s holds
// {b, t_begin, t_end, item} of the item it runs, or b = -1 when it has none.  With
// xcd_major the 8 XCDs get contiguous item ranges (slot 8g + x takes item x * ceil(W/8) + g),
// otherwise slot s takes item s.
#pragma once

#include "device_common.h"
#include "plan.h"

namespace mla {

struct PlanArgs {
  const int32_t* seqlens;
  int32_t* hdr;        // [4]: W, pages per item c, slots, target (0 when c was forced)
  int32_t* work;       // [slots][4]: b, t_begin, t_end, item
  int32_t* split_off;  // [B + 1]
  int B, max_seqlen, target, forced_pages, slots, xcd_major;
};

inline PlanArgs plan_args(const Plan& p, const int32_t* seqlens, void* workspace) {
  char* ws = static_cast<char*>(workspace);
  PlanArgs a;
  a.seqlens = seqlens;
  a.hdr = reinterpret_cast<int32_t*>(ws);
  a.work = reinterpret_cast<int32_t*>(ws + p.off_work);
  a.split_off = reinterpret_cast<int32_t*>(ws + p.off_split_off);
  a.B = p.B;
  a.max_seqlen = p.max_seqlen;
  a.target = p.target;
  a.forced_pages = p.forced_pages;
  a.slots = p.slots;
  a.xcd_major = p.xcd_major;
  return a;
}

// LDS the planner needs at least: reduction scratch; more lets it keep split_off on chip
constexpr int kPlanLdsMin = 64;

namespace plan_detail {

__device__ __forceinline__ long long max64(long long x, long long y) { return x > y ? x : y; }
__device__ __forceinline__ long long min64(long long x, long long y) { return x < y ? x : y; }

// pages of sequence b (lengths outside [0, max_seqlen] are clamped)
__device__ __forceinline__ int pages_of(const PlanArgs& a, int b) {
  const int L = min(max(a.seqlens[b], 0), a.max_seqlen);
  return (L + kPage - 1) / kPage;
}

// sum / max over the 256 threads; red: 4 slots of LDS (reused after a barrier)
__device__ __forceinline__ long long block_sum(long long v, long long* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ long long block_max(long long v, long long* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max64(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return max64(max64(red[0], red[1]), max64(red[2], red[3]));
}

}  // namespace plan_detail

// Called by all 256 threads of one workgroup; lds: lds_bytes >= kPlanLdsMin of LDS, 8-byte
// aligned.
__device__ inline void make_work_plan(const PlanArgs& a, void* lds, int lds_bytes) {
  using namespace plan_detail;
  long long* red = static_cast<long long*>(lds);     // [4]
  int* wsum = reinterpret_cast<int*>(red + 4);       // [4]
  int* so_lds = wsum + 4;                            // split_off copy, if it fits
  const bool so_in_lds = (long long)(a.B + 1) * 4 <= lds_bytes - kPlanLdsMin;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // ---- pages per item
  int c = a.forced_pages;
  if (c == 0) {
    long long P = 0, maxp = 0;
    for (int b = tid; b < a.B; b += 256) {
      const int p = pages_of(a, b);
      P += p;
      maxp = max64(maxp, p);
    }
    P = block_sum(P, red);
    maxp = max64(block_max(maxp, red), 1);
    // W(c) >= P / c, so the answer is at least ceil(P / target)
    long long lo = min64(max64((P + a.target - 1) / a.target, 1), maxp), hi = maxp;
    while (lo < hi) {  // uniform: every thread holds the same lo, hi
      const long long mid = lo + (hi - lo) / 2;
      long long n = 0;
      for (int b = tid; b < a.B; b += 256) n += (pages_of(a, b) + mid - 1) / mid;
      n = block_sum(n, red);
      if (n <= a.target) hi = mid;
      else lo = mid + 1;
    }
    c = (int)lo;
  }

  // ---- items per sequence and split_off (exclusive scan, 256 sequences per pass)
  int carry = 0;
  for (int base = 0; base < a.B; base += 256) {
    const int b = base + tid;
    const int n = b < a.B ? (pages_of(a, b) + c - 1) / c : 0;
    int x = n;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    __syncthreads();  // the previous pass is done with wsum
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int off = carry + x - n;
    for (int k = 0; k < w; ++k) off += wsum[k];
    if (b < a.B) {
      a.split_off[b] = off;
      if (so_in_lds) so_lds[b] = off;
    }
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
  }
  const int W = carry;
  if (tid == 0) {
    a.split_off[a.B] = W;
    if (so_in_lds) so_lds[a.B] = W;
    a.hdr[0] = W;
    a.hdr[1] = c;
    a.hdr[2] = a.slots;
    a.hdr[3] = a.forced_pages ? 0 : a.target;
  }
  __syncthreads();  // split_off complete (LDS and global) for the searches below

  // ---- dispatch table: the sequence of an item is the last b with split_off[b] <= item
  const int32_t* so = so_in_lds ? so_lds : a.split_off;
  const int per = (W + 7) / 8;
  for (int s = tid; s < a.slots; s += 256) {
    int item = s;
    if (a.xcd_major) {
      const int x = s & 7, g = s >> 3;
      item = g < per ? x * per + g : W;
    }
    int4 e = make_int4(-1, 0, 0, -1);
    if (item < W) {
      int lo = 0, hi = a.B;  // so[lo] <= item < so[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (so[mid] <= item) lo = mid;
        else hi = mid;
      }
      const int L = min(max(a.seqlens[lo], 0), a.max_seqlen);
      const int t0 = (item - so[lo]) * c * kPage;
      e = make_int4(lo, t0, min(L, t0 + c * kPage), item);
    }
    *reinterpret_cast<int4*>(a.work + 4 * s) = e;
  }
}

}  // namespace mla
