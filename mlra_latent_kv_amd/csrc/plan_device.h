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

// LDS the planner needs at least: reduction scratch; more lets it keep the clamped lengths
// and split_off on chip
constexpr int kPlanLdsMin = 64;
// sequences per thread whose page counts stay in registers (the first 256 * kPlanRegs; any
// further ones are re-read from seqlens)
constexpr int kPlanRegs = 4;

namespace plan_detail {

__device__ __forceinline__ long long max64(long long x, long long y) { return x > y ? x : y; }
__device__ __forceinline__ long long min64(long long x, long long y) { return x < y ? x : y; }

// length of sequence b clamped to [0, max_seqlen]
__device__ __forceinline__ int clamped_len(const PlanArgs& a, int b) {
  return min(max(a.seqlens[b], 0), a.max_seqlen);
}
__device__ __forceinline__ int pages_of_len(int L) { return (L + kPage - 1) / kPage; }
// ceil(p / c) for 0 <= p, 1 <= c < 2^21 (32-bit unsigned division)
__device__ __forceinline__ int items_of(int p, int c) {
  return (int)(((unsigned)p + (unsigned)c - 1u) / (unsigned)c);
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
// aligned.  The plan workgroup runs beside the prologue's own workgroups, so its latency is
// kept short: one read of seqlens, page counts in registers, a search range of a few steps.
__device__ inline void make_work_plan(const PlanArgs& a, void* lds, int lds_bytes) {
  using namespace plan_detail;
  long long* red = static_cast<long long*>(lds);     // [4]
  int* wsum = reinterpret_cast<int*>(red + 4);       // [4]
  int* so_lds = wsum + 4;                            // split_off copy [B + 1], if it fits
  int* len_lds = so_lds + (a.B + 1);                 // clamped lengths [B], if they fit
  const bool on_chip = (long long)(2 * a.B + 1) * 4 <= lds_bytes - kPlanLdsMin;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  int len[kPlanRegs];  // clamped lengths of sequences tid + 256 i
#pragma unroll
  for (int i = 0; i < kPlanRegs; ++i) {
    const int b = tid + 256 * i;
    len[i] = b < a.B ? clamped_len(a, b) : 0;
  }
  // f(pages of b) for every sequence this thread owns (b = tid, tid + 256, ...)
  auto for_each = [&](auto&& f) {
#pragma unroll
    for (int i = 0; i < kPlanRegs; ++i) f(pages_of_len(len[i]));
    for (int b = tid + 256 * kPlanRegs; b < a.B; b += 256) f(pages_of_len(clamped_len(a, b)));
  };

  // ---- pages per item
  int c = a.forced_pages;
  if (c == 0) {
    long long P = 0, maxp = 0, nonempty = 0;
    for_each([&](int p) {
      P += p;
      maxp = max64(maxp, p);
      nonempty += p > 0;
    });
    P = block_sum(P, red);
    nonempty = block_sum(nonempty, red);
    maxp = max64(block_max(maxp, red), 1);
    // W(c) = sum_b ceil(p_b / c) lies in [P / c, P / c + nonempty), so the answer is at
    // least ceil(P / target), and c = ceil(P / (target - nonempty)) already fits
    long long lo = min64(max64((P + a.target - 1) / a.target, 1), maxp), hi = maxp;
    if (a.target > nonempty) hi = min64(hi, max64((P + (a.target - nonempty) - 1) / (a.target - nonempty), lo));
    while (lo < hi) {  // uniform: every thread holds the same lo, hi
      const int mid = (int)(lo + (hi - lo) / 2);
      long long n = 0;
      for_each([&](int p) { n += items_of(p, mid); });
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
    const int i = base / 256;
    int L = 0;  // (a select chain: a run-time index into len[] would put it in scratch)
#pragma unroll
    for (int j = 0; j < kPlanRegs; ++j)
      if (i == j) L = len[j];
    if (i >= kPlanRegs && b < a.B) L = clamped_len(a, b);
    const int n = items_of(pages_of_len(L), c);
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
      if (on_chip) {
        so_lds[b] = off;
        len_lds[b] = L;
      }
    }
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
  }
  const int W = carry;
  if (tid == 0) {
    a.split_off[a.B] = W;
    if (on_chip) so_lds[a.B] = W;
    a.hdr[0] = W;
    a.hdr[1] = c;
    a.hdr[2] = a.slots;
    a.hdr[3] = a.forced_pages ? 0 : a.target;
  }
  __syncthreads();  // split_off complete (LDS and global) for the searches below

  // ---- dispatch table: the sequence of an item is the last b with split_off[b] <= item
  const int32_t* so = on_chip ? so_lds : a.split_off;
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
      const int L = on_chip ? len_lds[lo] : clamped_len(a, lo);
      const int t0 = (item - so[lo]) * c * kPage;
      e = make_int4(lo, t0, min(L, t0 + c * kPage), item);
    }
    *reinterpret_cast<int4*>(a.work + 4 * s) = e;
  }
}

}  // namespace mla
