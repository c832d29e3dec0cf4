// LDS tile of cached rows shared by the bf16 main loops (gfx950).
//
// A tile holds 32 consecutive tokens of one sequence (half a page): the 512 latent columns
// of each token in a 1024-byte row, then the 64 rotary-key columns of each token in a
// 128-byte row.  Tiles arrive by direct-to-LDS buffer loads, where lane i of an instruction
// always lands at byte 16*i of its destination, so the only freedom is which global 16-byte
// chunk each lane fetches.  That choice implements an XOR swizzle of the chunks inside a
// row, which keeps the reads free of LDS bank conflicts (64 banks of 4 bytes):
//  * the score step reads one 16-byte chunk per token for 16 consecutive tokens at a time
//    (ds_read_b128): the swizzle must be a bijection on any 16 consecutive rows;
//  * the value step reads with ds_read_b64_tr_b16 (32 lanes of 8 bytes at a time), either
//    4 rows x 4 chunks (32x32 MFMA operands, Sw32) or 8 rows x 2 chunks (16x16 operands,
//    Sw16); the rows of one read must land on disjoint chunk slots.
// Sw32: t mod 4 -> chunk bits 2-3, (t / 4) mod 4 -> bits 0-1.
// Sw16: t mod 8 -> chunk bits 1-3, (t / 8) mod 2 -> bit 0.
// Both repeat every 16 rows.  Rotary rows are 8 chunks and two share a 256-byte bank line;
// rope_sw(t) = (t/2) mod 8 separates 16 consecutive rows.
// The latent width DC is 512 (MLA and MLRA-4 rows of 576) or 128 (one MLRA branch with the
// rotary key, rows of 192); a 128-wide latent row is one 256-byte bank line of 16 chunks, and
// the swizzle, which only permutes chunks inside aligned groups of 16, is the same.
#pragma once

#include "device_common.h"

namespace mla {
namespace tile {

constexpr int kTT = 32;                                // tokens per tile
constexpr int kDC = 512, kDR = 64, kRow = kDC + kDR;   // latent / rotary / cached row width
constexpr int kLatRowB = kDC * 2;                      // bytes per latent row in LDS
constexpr int kRopeRowB = kDR * 2;                     // bytes per rotary row in LDS
constexpr int kRopeOff = kTT * kLatRowB;               // rotary region of a buffer
constexpr int kBufBytes = kRopeOff + kTT * kRopeRowB;  // one tile: 36864 bytes

// Tile geometry for latent width DC (the constants above are Geom<512>).
template <int DC>
struct Geom {
  static constexpr int kLatRowB = DC * 2;                   // bytes per latent row
  static constexpr int kRopeOff = kTT * kLatRowB;           // rotary region of a buffer
  static constexpr int kBufBytes = kRopeOff + kTT * kRopeRowB;
  static constexpr int kChunks = DC / 8;                    // 16-byte chunks per latent row
  static constexpr int kRowsPerLoad = 64 / kChunks;         // latent rows per 64-lane load
  static_assert(DC == 512 || DC == 128, "latent width");
};

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

enum Swizzle { Sw32, Sw16 };

template <Swizzle SW>
__device__ __forceinline__ int lat_sw(int t) {
  return SW == Sw32 ? (((t & 3) << 2) | ((t >> 2) & 3)) : (((t & 7) << 1) | ((t >> 3) & 1));
}
__device__ __forceinline__ int rope_sw(int t) { return (t >> 1) & 7; }

// Byte offset in a tile buffer of latent (row t, global 16-byte chunk c), and of the 8-byte
// piece holding element columns col..col+3 (col % 4 == 0).
template <Swizzle SW, int DC = kDC>
__device__ __forceinline__ uint32_t lat_chunk(int t, int c) {
  return (uint32_t)(t * Geom<DC>::kLatRowB + 16 * (c ^ lat_sw<SW>(t)));
}
template <Swizzle SW, int DC = kDC>
__device__ __forceinline__ uint32_t lat_piece(int t, int col) {
  return lat_chunk<SW, DC>(t, col >> 3) + 2 * (col & 7);
}
// Byte offset of rotary (row t, 16-byte chunk c), c < 8.
template <int DC = kDC>
__device__ __forceinline__ uint32_t rope_chunk(int t, int c) {
  return (uint32_t)(Geom<DC>::kRopeOff + t * kRopeRowB + 16 * (c ^ rope_sw(t)));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Cache policy of the tile loads (the instruction's cache-policy bits: 1 = sc0, 2 = nt,
// 16 = sc1): non-temporal.  Every cached row is read once per call, so nothing is gained by
// keeping it in the caches, and the streaming hint lifts the HBM read rate: a plain stream of
// direct-to-LDS loads went from 6.25 to 6.9-7.0 TB/s with it on MI355X, and the main loops
// from 5.60 to 6.37 TB/s (32-head, paged varlen workload), 4.96 to 5.37 (MLRA-4) and 4.00 to
// 4.27 (128-head, long context), same-box A/B.
#ifndef MLA_TILE_CPOL
#define MLA_TILE_CPOL 2
#endif

// 16 bytes per lane from buffer offset voff into LDS at lds + 16*lane.  Offsets at or past
// the descriptor's size read back as zeros without touching memory.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, MLA_TILE_CPOL);
}

// Loads one wave issues per tile when NW waves share it: wave w fetches its share of the
// latent rows (one instruction brings 1 KiB: one 512-wide row, or four 128-wide rows) and, if
// w < 4, rotary rows 8w..8w+7 (one instruction).
template <int NW, int DC = kDC>
__host__ __device__ constexpr int issues_per_wave(bool rope_wave) {
  return kTT / Geom<DC>::kRowsPerLoad / NW + (rope_wave ? 1 : 0);
}

// Issue wave w's loads of a tile whose first token row starts at lb (latent) / rb (rotary);
// rows >= valid read as zeros.  Lane offsets are formed here (a few VALU operations per
// load) rather than kept in registers across the loop.
template <Swizzle SW, int NW, int DC = kDC>
__device__ __forceinline__ void issue_tile(char* buf, int w, int lane, const bf16* lb,
                                           const bf16* rb, int valid, uint32_t lat_row_b,
                                           uint32_t rope_row_b) {
  using G = Geom<DC>;
  constexpr int R = kTT / G::kRowsPerLoad / NW;  // latent load instructions per wave
  const __amdgpu_buffer_rsrc_t rl = rsrc(lb, valid * lat_row_b);
  // lane -> (row t0 + lane / chunks, physical chunk lane % chunks); it lands at byte 16 lane
  // of the instruction's destination, which is exactly that row and chunk
  const int lr = lane / G::kChunks, lc = lane % G::kChunks;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int t0 = (R * w + j) * G::kRowsPerLoad, t = t0 + lr;
    dma16(rl, buf + t0 * G::kLatRowB, t * lat_row_b + 16 * (lc ^ lat_sw<SW>(t)));
  }
  if (NW <= 4 || w < 4) {  // (known true at compile time for up to 4 waves)
    const __amdgpu_buffer_rsrc_t rr = rsrc(rb, valid * rope_row_b);
    const int rt = 8 * w + (lane >> 3);
    dma16(rr, buf + G::kRopeOff + w * 1024, rt * rope_row_b + 16 * ((lane & 7) ^ rope_sw(rt)));
  }
}

// One of the loads of issue_tile: latent row R*w + part for part < R = kTT / NW, the rotary
// rows for part == R.  A wave that issues a tile's loads back to back stalls on them, so a
// caller with the latency to spare spreads them over several gaps between other work.
template <Swizzle SW, int NW>
__device__ __forceinline__ void issue_tile_part(char* buf, int w, int lane, const bf16* lb,
                                                const bf16* rb, int valid, uint32_t lat_row_b,
                                                uint32_t rope_row_b, int part) {
  constexpr int R = kTT / NW;
  if (part < R) {
    const int t = R * w + part;
    dma16(rsrc(lb, valid * lat_row_b), buf + t * kLatRowB,
          t * lat_row_b + 16 * (lane ^ lat_sw<SW>(t)));
  } else if (NW <= 4 || w < 4) {  // (known true at compile time for up to 4 waves)
    const int rt = 8 * w + (lane >> 3);
    dma16(rsrc(rb, valid * rope_row_b), buf + kRopeOff + w * 1024,
          rt * rope_row_b + 16 * ((lane & 7) ^ rope_sw(rt)));
  }
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding: vmcnt low bits
// [3:0], high bits [15:14]; expcnt [6:4] and lgkmcnt [11:8] at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also fences global
// memory, which would wait for every in-flight tile load (they write LDS asynchronously)
// and drain the prefetch ring; tile arrival is tracked with explicit vmcnt waits instead.
// The memory clobber keeps the compiler from moving LDS accesses across the barrier.  The
// same lgkmcnt(0) goes first as a builtin too: the compiler's wait analysis does not look
// into inline asm, and would otherwise still count a scalar load issued before the barrier
// as outstanding, which forces the first LDS wait after it to lgkmcnt(0) (scalar loads
// complete out of order), i.e. a wait for every operand read issued there.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt at their maxima
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS reads of tile (and query) data.  The pointer is a restrict parameter so that the
// inlined access carries alias-scope information: without it the compiler's wait analysis
// cannot tell a read of the current tile from the direct-to-LDS loads still in flight into
// other ring buffers, and inserts a wait for all of them (vmcnt(0)) before the read, which
// serialises the prefetch with the compute.  Arrival of the tile being read is guaranteed
// by the explicit vmcnt wait and barrier at the top of each tile iteration.
__device__ __forceinline__ bf16x8 lds_read16(const char* __restrict__ p) {
  return *(const bf16x8*)p;
}
// 16-byte LDS write, with the same alias-scope information as the reads (a write the wait
// analysis cannot tell apart from the tile loads in flight would first wait for all of them)
__device__ __forceinline__ void lds_write16(char* __restrict__ p, bf16x8 v) { *(bf16x8*)p = v; }
__device__ __forceinline__ s16x4 lds_read_tr(const char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// The same reads at a 32-bit LDS address.  Callers form one opaque base address per tile
// and add compile-time constants, which then go into the instructions' unsigned offset field
// instead of costing an add each.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}
__device__ __forceinline__ bf16x8 lds_read16_at(const lds_char* __restrict__ p) {
  return *(const __attribute__((address_space(3))) bf16x8*)p;
}
__device__ __forceinline__ bf16x8 lds_read16_at(uint32_t a) {
  return lds_read16_at((const lds_char*)(uintptr_t)a);
}
__device__ __forceinline__ s16x4 lds_read_tr_at(const lds_char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}
__device__ __forceinline__ s16x4 lds_read8_at(const lds_char* __restrict__ p) {
  return *(const __attribute__((address_space(3))) s16x4*)p;
}
// 16 bytes of one chunk as two 8-byte reads, first half at a, second at b.  gfx950 serves
// an 8-byte read in two LDS cycles without conflicts whenever every 32-lane half of the
// wave covers 256 distinct bytes (mod 256); a 16-byte read of the score-step pattern (16
// rows x 4 chunk columns per wave) takes eight cycles, twice the conflict-free four.
__device__ __forceinline__ bf16x8 b64_pair_at(uint32_t a, uint32_t b) {
  const s16x4 x = lds_read8_at((const lds_char*)(uintptr_t)a);
  const s16x4 y = lds_read8_at((const lds_char*)(uintptr_t)b);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ bf16x8 tr_pair_at(uint32_t lo, uint32_t hi) {
  const s16x4 a = lds_read_tr_at((const lds_char*)(uintptr_t)lo);
  const s16x4 b = lds_read_tr_at((const lds_char*)(uintptr_t)hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ f32x4 lds_load4f_at(const lds_char* __restrict__ p) {
  return *(const __attribute__((address_space(3))) f32x4*)p;
}
__device__ __forceinline__ void lds_store4f_at(lds_char* __restrict__ p, f32x4 v) {
  *(__attribute__((address_space(3))) f32x4*)p = v;
}
// Makes v opaque to the optimiser (no hoisting of expressions built from it).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Value operand of an MFMA: two transposed 4-row reads (8 tokens of one column).
__device__ __forceinline__ bf16x8 tr_pair(const char* lo, const char* hi) {
  const s16x4 a = lds_read_tr(lo);
  const s16x4 b = lds_read_tr(hi);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace tile
}  // namespace mla
