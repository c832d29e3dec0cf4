// Split plan of one decode call, made on the device from seqlens by one workgroup of 256
// threads (an extra workgroup of the prologue launch, so the plan costs no launch).
//
// The main loop is split over the sequence (split-K).  A work item is a token range
// [t_begin, t_end) of one sequence; its partial result (running max, running sum, latent
// output) is merged with the other items of the sequence afterwards.  Every sequence b with
// L_b tokens, p_b = ceil(L_b / 64) pages, is cut into ceil(p_b / c) items of c whole pages
// (the last one ragged); sequences with no tokens get no item.  Items are numbered
// sequence-major; split_off[b] is the first item of sequence b and split_off[B] = W, the item
// count, so the merge finds a variable number of items per sequence.
//
// Balance: every item costs at most c pages and one workgroup set per item fills the chip
// once when W <= target, so the automatic plan takes the smallest c with
// sum_b ceil(p_b / c) <= target (binary search; the sum only falls as c grows), or
// c = max_b p_b (one item per sequence) when no c meets the target.  With num_splits given,
// c is fixed by the host.
//
// Dispatch tables: one item per dispatch slot of the main kernels.  With xcd_major the 8 XCDs
// get contiguous item ranges (slot 8g + x takes item x * ceil(W / 8) + g), otherwise slot s
// takes item s.  work[s] = {b, t_begin, t_end, item} (b = -1 for a slot without an item),
// slot_end[s] = item + 1 (0 for an idle slot), and items[i] = {b, t_begin, t_end, slot}.
//
// Device checks (MLA_FLAG_DEVICE_CHECKS): a separate kernel (k_device_checks) writes one
// result word per sequence, dbg[b] = 4 * (first bad page index + 1, or 0) + error bits; the
// plan folds them into the error word hdr[4..6] and, when a block id was out of range, makes
// a plan with no items, so nothing reads outside the pool and every output is zero.
#pragma once

#include "device_common.h"
#include "plan.h"

namespace mla {

struct PlanArgs {
  const int32_t* seqlens;
  const int32_t* dbg;  // [B] device-check results (checks only), else nullptr
  int32_t* hdr;        // [8]: W, pages per item c, slots, target (0 when c
                       // was forced), error bits, first bad sequence, its first bad page,
                       // items_cap
  int32_t* work;       // [slots][4]: b, t_begin, t_end, item of the slot's item
  int32_t* slot_end;   // [slots]: one past the slot's item (0: idle slot)
  int32_t* items;      // [items_cap][4]: b, t_begin, t_end, slot
  int32_t* split_off;  // [B + 1]
  int B, max_seqlen, target, forced_pages, slots, xcd_major, items_cap;
};

inline PlanArgs plan_args(const Plan& p, const int32_t* seqlens, void* workspace) {
  char* ws = static_cast<char*>(workspace);
  PlanArgs a;
  a.seqlens = seqlens;
  a.dbg = p.checks ? reinterpret_cast<const int32_t*>(ws + p.off_dbg) : nullptr;
  a.hdr = reinterpret_cast<int32_t*>(ws);
  a.work = reinterpret_cast<int32_t*>(ws + p.off_work);
  a.slot_end = reinterpret_cast<int32_t*>(ws + p.off_slot_end);
  a.items = reinterpret_cast<int32_t*>(ws + p.off_items);
  a.split_off = reinterpret_cast<int32_t*>(ws + p.off_split_off);
  a.B = p.B;
  a.max_seqlen = p.max_seqlen;
  a.target = p.target;
  a.forced_pages = p.forced_pages;
  a.slots = p.slots;
  a.xcd_major = p.xcd_major;
  a.items_cap = p.items_cap;
  return a;
}

// LDS the planner needs at least: reduction scratch; more lets it keep the clamped lengths
// and split_off on chip
constexpr int kPlanLdsMin = 64;
// sequences per thread whose lengths stay in registers (the first 256 * kPlanRegs; any
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

// sum / max / min over the 256 threads; red: 4 slots of LDS (reused after a barrier)
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
__device__ __forceinline__ long long block_min(long long v, long long* red) {
  return -block_max(-v, red);
}

// Exclusive scan of n(b) over b = 0 .. B-1 (256 sequences per pass): out(b, offset) is called
// for every b with its offset; returns the total.  wsum: 4 ints of LDS.
template <typename N, typename Out>
__device__ __forceinline__ long long block_scan(int B, N&& n_of, Out&& out, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  long long carry = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + tid;
    const int n = b < B ? n_of(b, base / 256) : 0;
    int x = n;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    __syncthreads();  // the previous pass is done with wsum
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    long long off = carry + x - n;
    for (int k = 0; k < w; ++k) off += wsum[k];
    if (b < B) out(b, off);
    carry += (long long)wsum[0] + wsum[1] + wsum[2] + wsum[3];
  }
  return carry;
}

// last index lo in [0, n) with v[lo] <= x, given v[0] <= x (v non-decreasing)
template <typename V>
__device__ __forceinline__ int upper_index(V&& v, int n, long long x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((long long)v(mid) <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

}  // namespace plan_detail

// Called by all 256 threads of one workgroup; lds: lds_bytes >= kPlanLdsMin of LDS, 8-byte
// aligned.  The plan workgroup runs beside the prologue's own workgroups, so its latency is
// kept short: one read of seqlens, lengths in registers, a search range of a few steps.
__device__ inline void make_work_plan(const PlanArgs& a, void* lds, int lds_bytes) {
  using namespace plan_detail;
  long long* red = static_cast<long long*>(lds);     // [4]
  int* wsum = reinterpret_cast<int*>(red + 4);       // [4]
  int* so_lds = wsum + 4;                            // split_off copy [B + 1], if it fits
  int* len_lds = so_lds + (a.B + 1);                 // clamped lengths [B], if they fit
  const bool on_chip = (long long)(2 * a.B + 1) * 4 <= lds_bytes - kPlanLdsMin;
  const int tid = threadIdx.x;

  // ---- device-check results: error word, and no items at all after a bad block id
  long long err_bits = 0, err_key = 0x7fffffffffffffffLL;
  if (a.dbg) {
    for (int b = tid; b < a.B; b += 256) {
      const int d = a.dbg[b];
      if (d & 3) {
        err_bits |= d & 3;
        err_key = min64(err_key, ((long long)b << 32) | (unsigned)(d >> 2));
      }
    }
    err_bits = block_max(err_bits & 1, red) | (block_max(err_bits & 2, red));
    err_key = block_min(err_key, red);
  }
  const bool drop_all = (err_bits & MLA_DEVERR_BLOCK) != 0;

  int len[kPlanRegs];  // clamped lengths of sequences tid + 256 i
#pragma unroll
  for (int i = 0; i < kPlanRegs; ++i) {
    const int b = tid + 256 * i;
    len[i] = b < a.B && !drop_all ? clamped_len(a, b) : 0;
  }
  // clamped length of sequence b = base + tid in scan pass i (a select chain: a run-time
  // index into len[] would put it in scratch)
  auto len_at = [&](int b, int i) {
    int L = 0;
#pragma unroll
    for (int j = 0; j < kPlanRegs; ++j)
      if (i == j) L = len[j];
    if (i >= kPlanRegs) L = drop_all ? 0 : clamped_len(a, b);
    return L;
  };

  {
    // f(pages of b) for every sequence this thread owns (b = tid, tid + 256, ...)
    auto for_each = [&](auto&& f) {
#pragma unroll
      for (int i = 0; i < kPlanRegs; ++i) f(pages_of_len(len[i]));
      for (int b = tid + 256 * kPlanRegs; b < a.B; b += 256)
        f(drop_all ? 0 : pages_of_len(clamped_len(a, b)));
    };
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
    // items per sequence and split_off
    const int W = (int)block_scan(
        a.B, [&](int b, int i) { return items_of(pages_of_len(len_at(b, i)), c); },
        [&](int b, long long off) {
          a.split_off[b] = (int)off;
          if (on_chip) {
            so_lds[b] = (int)off;
            len_lds[b] = len_at(b, b / 256);
          }
        },
        wsum);
    if (tid == 0) {
      a.split_off[a.B] = W;
      if (on_chip) so_lds[a.B] = W;
      a.hdr[0] = W;
      a.hdr[1] = c;
      a.hdr[3] = a.forced_pages ? 0 : a.target;
    }
    __syncthreads();  // split_off complete (LDS and global) for the searches below

    // dispatch tables: the sequence of an item is the last b with split_off[b] <= item
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
        const int b = upper_index([&](int i) { return so[i]; }, a.B, item);
        const int L = on_chip ? len_lds[b] : clamped_len(a, b);
        const int t0 = (item - so[b]) * c * kPage;
        e = make_int4(b, t0, min(L, t0 + c * kPage), item);
        *reinterpret_cast<int4*>(a.items + 4 * item) = make_int4(b, e.y, e.z, s);
      }
      *reinterpret_cast<int4*>(a.work + 4 * s) = e;
      a.slot_end[s] = item < W ? item + 1 : 0;
    }
  }
  if (tid == 0) {
    a.hdr[2] = a.slots;
    a.hdr[4] = (int)err_bits;
    a.hdr[5] = err_bits ? (int)(err_key >> 32) : -1;
    a.hdr[6] = err_bits ? (int)(err_key & 0xffffffff) - 1 : -1;
    a.hdr[7] = a.items_cap;
  }
}

}  // namespace mla
