// Split-K main loop of the absorbed MLA decode step for head counts that are a multiple of
// 128 (gfx950, bf16 in, fp32 accumulation).
//
// Same contraction as the 32-head kernel (yololab MLA page, section 矩陣吸收: every head
// scores the one cached latent row plus its rotary key, and the latent row is also the
// value), organised so that each cached tile crosses HBM -> LDS once for 128 heads and
// every LDS byte read feeds as many MFMA operations as the register file allows:
//
//  * one workgroup of 4 waves per CU handles (work item: sequence b, tokens [t_begin,
//    t_end); heads 128q..128q+127);
//    wave w owns 32 heads outright: their scores, softmax state and the full 512-column
//    latent output O^T (16 accumulator blocks of 32 columns x 32 heads, 256 registers,
//    which one wave per SIMD can hold in the accumulation registers).  The absorbed query
//    (576 columns of 32 heads) stays in registers for the whole loop, so the LDS holds tiles
//    only.  No per-tile exchange between waves.
//  * MFMA 32x32x16 throughout: a 1 KiB operand read from LDS feeds 16K multiply-adds, twice
//    what the 16x16x32 shape gets from the same read, so LDS traffic per tile is half that of
//    a 16-heads-per-wave layout.
//  * tiles of 32 tokens stream through a ring of 4 LDS buffers by direct-to-LDS loads, in a
//    software pipeline: while tile k + 1 is scored, tile k's value MFMAs alternate with its
//    score MFMAs, tile k + 1's softmax runs between tile k's last value MFMAs, and tiles
//    k + 2 and k + 3 are in flight.  The value MFMAs form one stream across tile
//    boundaries: tile k's first four run around the barrier that admits tile k + 1 (their
//    operands were read behind tile k - 1's last value MFMAs), so the matrix cores stay busy
//    through the barrier and the latency of tile k + 1's first score-operand reads.
//  * scores S^T[t][h] = tile . q_cat^T (one accumulation chain over 36 K-steps of 16
//    columns); the probabilities go register-direct into the value product
//    O^T += V^T P^T (token order inside a K-step permuted to match the score layout; value
//    operand read with ds_read_b64_tr_b16 from the token-major tile).
//  * the running max of a head is raised (and O rescaled) only when a tile's max exceeds it
//    by more than kLazyTau (log2 units); otherwise the tile's weights are taken against the
//    stale max and stay below 2^kLazyTau, far inside fp32 / bf16 range.  m, l and O always
//    refer to the same max, so the partial result is the same softmax.
#include "device_common.h"
#include "launch.h"
#include "tile_bf16.h"

namespace mla {
namespace {

using namespace tile;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsWG = 128;          // heads per workgroup, 32 per wave
constexpr int kRing = 4;               // tile buffers: values, scores, two in flight
constexpr float kLazyTau = 8.0f;       // log2 headroom before the running max is raised
constexpr int kQSteps = kRow / 16;     // 36 K-steps of 16 columns: 32 latent, 4 rotary
constexpr int kIssues = issues_per_wave<kWaves>(true);  // tile loads per wave per tile

// Score MFMAs in VGPR form.  This file is built with MFMAs in their accumulation-register
// form (the default), so that O, the only other MFMA result, lives in the 256 accumulation
// registers for the whole loop; the score accumulators sit next to the softmax in VGPRs
// through these asm forms.  The compiler pads inline asm with no wait states: the first step
// takes a literal zero accumulator (no VALU write ahead of it), and the caller waits before
// the first VALU read of the result (checked on the generated code by the codegen tests).
__device__ __forceinline__ void mfma_qk_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// o *= a for one output block, in place in the accumulation registers.  (A VALU multiply in
// C++ makes the register allocator give O a VGPR home and copy all of it around the loop.)
// The caller keeps the last MFMA that wrote o well ahead of this block, and the next MFMA
// reading o well behind it.
__device__ __forceinline__ void scale_acc(f32x16& o, float a) {
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = o[i];
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %16, %0\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %0, %16\n\t"
      "v_accvgpr_read_b32 %16, %1\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %1, %16\n\t"
      "v_accvgpr_read_b32 %16, %2\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %2, %16\n\t"
      "v_accvgpr_read_b32 %16, %3\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %3, %16\n\t"
      "v_accvgpr_read_b32 %16, %4\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %4, %16\n\t"
      "v_accvgpr_read_b32 %16, %5\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %5, %16\n\t"
      "v_accvgpr_read_b32 %16, %6\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %6, %16\n\t"
      "v_accvgpr_read_b32 %16, %7\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %7, %16\n\t"
      "v_accvgpr_read_b32 %16, %8\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %8, %16\n\t"
      "v_accvgpr_read_b32 %16, %9\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %9, %16\n\t"
      "v_accvgpr_read_b32 %16, %10\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %10, %16\n\t"
      "v_accvgpr_read_b32 %16, %11\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %11, %16\n\t"
      "v_accvgpr_read_b32 %16, %12\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %12, %16\n\t"
      "v_accvgpr_read_b32 %16, %13\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %13, %16\n\t"
      "v_accvgpr_read_b32 %16, %14\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %14, %16\n\t"
      "v_accvgpr_read_b32 %16, %15\n\t"
      "v_mul_f32_e32 %16, %17, %16\n\t"
      "v_accvgpr_write_b32 %15, %16\n\t"
      : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(x[4]), "+a"(x[5]), "+a"(x[6]), "+a"(x[7]), "+a"(x[8]), "+a"(x[9]), "+a"(x[10]), "+a"(x[11]), "+a"(x[12]), "+a"(x[13]), "+a"(x[14]), "+a"(x[15]),
        "=&v"(t)
      : "v"(a));
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = x[i];
}

__global__ __launch_bounds__(kThreads, 1) void k_main_bf16_wide(
    const bf16* __restrict__ qcat, const bf16* __restrict__ latent,
    const bf16* __restrict__ rope, int64_t lat_tok, int64_t lat_seq, int64_t rope_tok,
    int64_t rope_seq, const int32_t* __restrict__ work, const int32_t* __restrict__ bt,
    int64_t bt_stride, int paged, bf16* __restrict__ part_o, float* __restrict__ part_ml, int H,
    int n_hq, const int32_t* __restrict__ seqlens, int max_seqlen, int sq, int Hw) {
  // One LDS object.  (Kept as a single struct: with separate arrays the compiler's wait
  // analysis stops telling the tile reads apart from the loads in flight and waits for all
  // of them before the first read of every tile.)
  struct Smem {
    char ring[kRing][kBufBytes];
  };
  __shared__ __align__(16) Smem sm;  // 144 KiB
  char (&ring)[kRing][kBufBytes] = sm.ring;

  // XCD-aware mapping.  Blocks are dispatched round-robin over the 8 XCDs: block 8r + x runs
  // head quad r % n_hq of dispatch slot 8(r / n_hq) + x, and the split plan gives XCD x a
  // contiguous range of work items, so the items of one sequence (which all read its query)
  // and the head quads of one item (which read the same tiles) share that XCD's L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r = bid >> 3;
  const int hq = r % n_hq;
  const int4 wi = *reinterpret_cast<const int4*>(work + 4 * (8 * (r / n_hq) + xcd));
  const int b = wi.x;
  if (b < 0) return;  // slot without a work item
  const int t_begin = wi.y, t_end = wi.z;  // page-aligned start, never empty
  int item = wi.w;  // index of the partial results
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a uniform value: the LDS destinations of the tile loads (M0) depend on it,
  // and from a value the compiler cannot prove uniform every load needs a v_readfirstlane
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, kg = lane >> 5;
  const int h0 = hq * kHeadsWG + 32 * w;  // this wave's heads

  const int n_tiles = (t_end - t_begin + kTT - 1) / kTT;
  // the tokens this wave's query token sees (s_q > 1 query tokens: token h0 / Hw is causal):
  // scores past t_lim are masked; the tiles still load to t_end for the other waves
  const int t_lim = sq > 1 ? min(t_end, causal_limit(seqlens, b, max_seqlen, sq, h0 / Hw)) : t_end;

  const uint32_t lat_row_b = (uint32_t)(lat_tok * 2), rope_row_b = (uint32_t)(rope_tok * 2);
  const int32_t* bt_row = bt + (paged ? (int64_t)b * bt_stride : 0);
  auto page_of = [&](int k) -> int32_t { return paged ? bt_row[(t_begin + kTT * k) / kPage] : 0; };
  // part < 0: every load of wave w for tile k; else only load `part` (0 .. kIssues - 1)
  auto issue = [&](int k, int64_t pg, int part = -1) {
    const int t0 = t_begin + kTT * k;
    const bf16 *lb, *rb;
    if (paged) {
      lb = latent + pg * lat_seq + (int64_t)(t0 % kPage) * lat_tok;
      rb = rope + pg * rope_seq + (int64_t)(t0 % kPage) * rope_tok;
    } else {
      lb = latent + (int64_t)b * lat_seq + (int64_t)t0 * lat_tok;
      rb = rope + (int64_t)b * rope_seq + (int64_t)t0 * rope_tok;
    }
    // valid rows, uniform (the clamp would otherwise become a vector med3, and a buffer
    // descriptor in vector registers costs a loop per load)
    const int valid = __builtin_amdgcn_readfirstlane(max(0, min(kTT, t_end - t0)));
    if (part < 0)
      issue_tile<Sw32, kWaves>(ring[k % kRing], w, lane, lb, rb, valid, lat_row_b, rope_row_b);
    else
      issue_tile_part<Sw32, kWaves>(ring[k % kRing], w, lane, lb, rb, valid, lat_row_b,
                                    rope_row_b, part);
  };

  // Absorbed query as the B operand of 32x32x16 (N = heads): lane (head l32, k-half kg),
  // K-step j covers q_cat columns 16j..16j+15, the lane's 8 at 16j + 8*kg; all 36 K-steps
  // in registers.
  //
  // Start-up order: tile 0, the query, tiles 1 and 2, then one wait for all but tiles 1 and
  // 2, so that the query and the first tile share one memory latency.  Every tile load from
  // here on goes out unconditionally, past the item's end with no valid rows (such loads
  // return zeros without touching memory), so that the number of loads in flight, and with
  // it every wait count, is the same on every path.  The explicit wait also tells the
  // compiler's wait analysis that the query registers are complete, so no wait on them,
  // which would also wait on younger tile loads, reaches the loop.
  // page of tile k, or 0 past the item's end (the block table row ends with the sequence)
  auto page_or0 = [&](int k) -> int32_t { return k < n_tiles ? page_of(k) : 0; };
  const int32_t pg0 = page_of(0), pg1 = page_or0(1), pg2 = page_or0(2);
  issue(0, pg0);
  bf16x8 qb[kQSteps];
  {
    const bf16* qrow = qcat + ((size_t)b * H + h0 + l32) * kRow + 8 * kg;
#pragma unroll
    for (int j = 0; j < kQSteps; ++j) qb[j] = *(const bf16x8*)(qrow + 16 * j);
  }
  __builtin_amdgcn_sched_barrier(0);  // every query load ahead of tiles 1, 2 (the wait counts on it)
  issue(1, pg1);
  issue(2, pg2);
  wait_vmcnt<2 * kIssues>();

  // Score reads (A = tile, M = tokens): token l32, chunk 2j + kg for latent K-step j.  The
  // swizzle permutes within aligned 16-chunk groups and repeats every 16 rows, so
  // j = 8u + j' adds 256u bytes.  Rotary K-step 32 + j: rotary chunk 2j + kg.
  //
  // The read addresses of a tile's buffer are carried from tile to tile (advanced by one
  // buffer, or wrapped to the first) and kept opaque to the optimiser: every read is one of
  // them plus a constant in the instruction's offset field, and no separate per-lane offsets
  // stay live next to them.  qa / ra follow the tile being scored, pa the tile whose values
  // are being summed (one tile behind).
  const uint32_t buf0 = lds_addr(ring[0]);
  uint32_t qa[8], ra[4], pa[2][4];
#pragma unroll
  for (int j = 0; j < 8; ++j) qa[j] = buf0 + lat_chunk<Sw32>(l32, 2 * j + kg);
#pragma unroll
  for (int j = 0; j < 4; ++j) ra[j] = buf0 + rope_chunk(l32, 2 * j + kg);
  // Value reads (A = V^T, M = 32 latent columns, K = 16 tokens): 16-lane group G holds
  // columns 16*(G&1)..+15 of the block and tokens 4*kg..+3 (first read) and 8 + 4*kg..+3
  // (second read) of the K-step; source lane li addresses token row 4*kg + li/4 (+8),
  // columns 16*(G&1) + 4*(li&3)..+3.  Column block cb = 4u + c adds 256u bytes; the second
  // K-step adds 16 KiB.
  const int G = lane >> 4, li = lane & 15;
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      pa[rr][c] = buf0 + lat_piece<Sw32>(4 * kg + (li >> 2) + 8 * rr,
                                         32 * c + 16 * (G & 1) + 4 * (li & 3));
  // buffer after the one at kt (0, 1, 2, 0, ...)
  auto next_buf = [](int kt) -> int32_t {
    return kt % kRing == kRing - 1 ? -(kRing - 1) * kBufBytes : kBufBytes;
  };

  float m_ref = -INFINITY, l_run = 0.0f;  // per head l32 (both k-halves hold the same)
  f32x16 O[16];
#pragma unroll
  for (int cb = 0; cb < 16; ++cb) O[cb] = f32x16{};

  // ---- S^T[t][h] of one tile for its 32 tokens (M) and the wave's 32 heads (N), one
  // accumulation chain over 36 K-steps (the hardware orders dependent MFMAs itself).  Tile
  // operands are read kQkAhead K-steps ahead.  mid(j) runs after MFMA j: the previous tile's
  // softmax and the next tile's loads are placed there, in the shadow of the score MFMAs.
  constexpr int kQkAhead = 4;
  constexpr int kQq = kQkAhead + 1;
  // iteration at which K-step t's tile operand is read: kQkAhead steps ahead, or kQkNear
  // steps ahead once the value MFMAs alternate with the score MFMAs (from gap kVStart on),
  // where each step is two MFMA slots
  auto read_at = [](int t, int v_start) {
    constexpr int kQkNear = 2;
    return t - (t >= v_start + kQkNear ? kQkNear : kQkAhead);
  };
  auto scores = [&](f32x16& S, int v_start, auto&& pre, auto&& mid) {
    auto a_tile = [&](int j) -> bf16x8 {
      return j < 32 ? lds_read16_at(qa[j & 7] + 256 * (j >> 3)) : lds_read16_at(ra[j - 32]);
    };
    bf16x8 aq[kQq];
#pragma unroll
    for (int t = 0; t < kQSteps; ++t)
      if (read_at(t, v_start) < 0) aq[t % kQq] = a_tile(t);
    __builtin_amdgcn_sched_barrier(0);
    pre();  // work that covers the first operand reads' latency
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kQSteps; ++j) {
#pragma unroll
      for (int t = j + 1; t < kQSteps && t <= j + kQkAhead; ++t)
        if (read_at(t, v_start) == j) aq[t % kQq] = a_tile(t);
      if (j == 0)
        mfma_qk_first(S, aq[j % kQq], qb[j]);
      else
        mfma_qk(S, aq[j % kQq], qb[j]);
      // keep the written order: the scheduler would otherwise hoist more operand reads than
      // the VGPRs left next to the query hold, or move the pieces in mid() across MFMAs
      __builtin_amdgcn_sched_barrier(0);
      mid(j);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- softmax of one tile's scores S into weight set P (tiles alternate between the two
  // sets: the value product of tile k reads set k & 1 while tile k + 1's softmax writes the
  // other).  D layout: lane (head l32, half kg), item i -> token 8*(i/4) + 4*kg + i%4.
  //  * soft_max1 / soft_max2: row max as a tree of depth 3 (a linear chain of 15 is 15
  //    dependent VALU steps), and the lazy raise of the running max, which rescale() then
  //    applies to O and l once the previous tile's values are in (the weights already use
  //    the raised max);
  //  * weight_exp / weight_pack: the weights of items i, i + 1, then their conversion to a
  //    packed pair (one conversion), summed over the rounded weights the MFMA uses as a dot
  //    product of the pair with (1, 1).
  // Each piece ends by passing its results through an empty volatile asm, which keeps it in
  // the gap between MFMAs where it is written (the compiler would otherwise sink it towards
  // its use, past branches, where it runs serially).
  // B operand of the value product (K = 16 tokens per step, N = heads): lane (head l32,
  // k-half kg) item e of step ks <-> token 16*ks + 8*(e/4) + 4*kg + e%4: the lane's own
  // scores, items 8*ks + e.
  uint32_t pw[2][2][4];
  float psum[2] = {0.0f, 0.0f};
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  bool raise = false;
  float a_raise = 1.0f;
  float t5[5];
  auto soft_max1 = [&](const f32x16& S) {
#pragma unroll
    for (int j = 0; j < 5; ++j) t5[j] = fmaxf(fmaxf(S[3 * j], S[3 * j + 1]), S[3 * j + 2]);
    asm volatile("" : "+v"(t5[0]), "+v"(t5[1]), "+v"(t5[2]), "+v"(t5[3]), "+v"(t5[4]));
  };
  auto soft_max2 = [&](const f32x16& S, int kt, int P) {
    float mx = fmaxf(fmaxf(fmaxf(t5[0], t5[1]), t5[2]), fmaxf(fmaxf(t5[3], t5[4]), S[15]));
    mx = max_xor32(mx);  // every tile holds a valid token: mx finite
    raise = false;
    if (kt == 0) {
      // O and l are still zero.  mx = -inf: the wave's query token sees none of the item's
      // tokens (s_q > 1), and never will in it; its weights are then taken against 0
      m_ref = mx == -INFINITY ? 0.0f : mx;
    } else if (__ballot(mx > m_ref + kLazyTau) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      a_raise = exp2f(m_ref - m_new);
      m_ref = m_new;
      raise = true;
    }
    psum[P] = 0.0f;
    asm volatile("" : "+v"(m_ref), "+v"(psum[P]));
  };
  // O and l to the raised max: after the previous tile's last value MFMA, before this one's
  // first (the padding covers the accumulation-register reads after that MFMA's writes)
  auto rescale = [&]() {
    if (raise) {
      asm volatile("s_nop 15\n\ts_nop 7");
      // one block at a time through VGPRs (O lives in the accumulation registers)
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {
        scale_acc(O[cb], a_raise);
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run *= a_raise;
    }
  };
  float e2[2];
  auto weight_exp = [&](const f32x16& S, int i) {  // weight of item i into e2[i & 1]
    e2[i & 1] = __builtin_amdgcn_exp2f(S[i] - m_ref);
    asm volatile("" : "+v"(e2[i & 1]));
  };
  auto weight_pack = [&](int i, int P) {
    const bf16x2 p = __builtin_convertvector(f32x2{e2[0], e2[1]}, bf16x2);
    pw[P][i >> 3][(i & 7) >> 1] = __builtin_bit_cast(uint32_t, p);
    psum[P] = __builtin_amdgcn_fdot2_f32_bf16(p, ones, psum[P], false);
    asm volatile("" : "+v"(pw[P][i >> 3][(i & 7) >> 1]), "+v"(psum[P]));
  };
  // rows past the item's end in tile kt (only the last tile can have them) get -inf
  auto mask_ragged = [&](f32x16& S, int kt) {
    const int valid = min(kTT, t_lim - t_begin - kTT * kt);  // <= 0: all masked
    if (valid < kTT) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        S[i] = 8 * (i >> 2) + 4 * kg + (i & 3) < valid ? S[i] : -INFINITY;
    }
  };
  // softmax piece q (0 .. kSoftPieces - 1) of tile kt into set P: the masked first max level,
  // the rest of the max with the raise, then per item pair p: item 2p's weight, item
  // 2p + 1's weight, the pair's conversion and row sum
  constexpr int kSoftPieces = 2 + 3 * 8;
  auto soft_piece = [&](f32x16& S, int kt, int P, int q) {
    if (q == 0) {
      mask_ragged(S, kt);
      soft_max1(S);
    } else if (q == 1) {
      soft_max2(S, kt, P);
    } else {
      const int pair = (q - 2) / 3, part = (q - 2) % 3;
      if (part < 2)
        weight_exp(S, 2 * pair + part);
      else
        weight_pack(2 * pair, P);
    }
  };

  // ---- O^T[d][h] += V^T P^T over one tile (its buffer at pa), K-step-major over the 16
  // column blocks.  The value MFMAs of consecutive tiles form one stream that never stops
  // at a tile boundary: tile k's first kFront MFMAs run around the barrier that admits tile
  // k + 1 (two before it, two behind the first score-operand reads of tile k + 1, whose
  // latency they cover), the next ones alternate with tile k + 1's score MFMAs, the rest
  // hold tile k + 1's softmax in their gaps.  Operand i of a tile goes to register slot
  // i % 4 and is read right after the value MFMA vsched(i) (a slot is refilled only after
  // the MFMA that used it has issued): two value MFMAs ahead while they alternate with
  // score MFMAs (each step is two MFMA slots), four ahead elsewhere, and the first kFront
  // operands of the next tile behind the last four MFMAs of this one.
  constexpr int kFront = 4;       // value MFMAs of tile k around the barrier of iteration k
  constexpr int kFrontPre = 2;    // ... of which issued before it
  bf16x8 vq[4];
  // operand i of the tile whose buffer is at base pa (+ buffer offset off)
  auto v_tile = [&](int i, int32_t off) -> bf16x8 {
    const int cb = i & 15, ks = i >> 4;
    const uint32_t o = 256 * (cb >> 2) + 16384 * ks;
    return tr_pair_at(pa[0][cb & 3] + off + o, pa[1][cb & 3] + off + o);
  };
  auto vsched = [](int i, int n_alt) {  // value MFMA after which operand i is read
    return i < kFront ? -1 : i < kFront + n_alt ? i - 2 : i - 4;
  };
  // value MFMA i of tile kt with weight set P; n_alt MFMAs from kFront on alternate with score
  // MFMAs; next: the stream continues with a tile after this one (its first operands are read
  // here, after pa has moved on to its buffer)
  auto value_mfma = [&](int i, int P, int kt, int n_alt, bool next) {
    const int ks = i >> 4;
    const bf16x8 pb =
        __builtin_bit_cast(bf16x8, u32x4{pw[P][ks][0], pw[P][ks][1], pw[P][ks][2], pw[P][ks][3]});
    O[i & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[i & 3], pb, O[i & 15], 0, 0, 0);
#pragma unroll
    for (int i2 = i + 1; i2 < 32 && i2 <= i + 4; ++i2)
      if (vsched(i2, n_alt) == i) vq[i2 & 3] = v_tile(i2, 0);
    if (i == 27) {  // every operand of this tile is read: move on to the next buffer
      const int32_t step = next_buf(kt);
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int c = 0; c < 4; ++c) pa[rr][c] = opaque(pa[rr][c] + step);
    }
    if (next && i >= 32 - kFront) vq[(i + kFront) & 3] = v_tile(i + kFront - 32, 0);
  };
  auto advance_qk = [&](int kt) {  // score reads move on from tile kt's buffer
    const int32_t step = next_buf(kt);
#pragma unroll
    for (int j = 0; j < 8; ++j) qa[j] = opaque(qa[j] + step);
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[j] = opaque(ra[j] + step);
  };

  // ---- software pipeline over the tiles.  Fill: tile 0's scores and softmax, and the first
  // operands of its values.  Iteration k: tile k's first value MFMAs around the barrier, the
  // score chain of tile k + 1 with tile k + 3's loads behind its first MFMAs and tile k's
  // value MFMAs alternating with its MFMAs from gap kVStart on (so each stream's operand reads
  // run twice as many MFMA slots ahead); then tile k's remaining value MFMAs, with tile
  // k + 1's softmax in their gaps (its scores are complete by then); then the lazy rescale.
  // The ring holds tile k (values), tile k + 1 (scores) and tiles k + 2, k + 3 (in flight).
  // score gap of the first alternating value MFMA: later starts leave more tail gaps for the
  // softmax but fewer alternating pairs
  constexpr int kVStart = 25;
  constexpr int kAlt = kQSteps - kVStart;  // value MFMAs alternating with score MFMAs
  // tail gap (1 .. gaps) of softmax piece q, by cumulative issue cost (cycles, measured
  // beside MFMAs: v_exp ~12, v_cvt_pk ~8, plain VALU ~6)
  auto soft_gap = [](int q, int gaps) {
    auto cost = [](int r) { return r == 0 ? 30 : r == 1 ? 50 : ((r - 2) % 3 == 2 ? 15 : 18); };
    int before = 0, total = 0;
    for (int r = 0; r < kSoftPieces; ++r) {
      if (r < q) before += cost(r);
      total += cost(r);
    }
    return 1 + before * gaps / total;
  };
  constexpr int kTail = 32 - kFront - kAlt;  // value MFMAs after the score chain
  static_assert(kTail >= 8 && kVStart >= 2 * kIssues, "value schedule");
  lds_barrier();  // tile 0 landed for every wave
  f32x16 S;
  scores(S, kQSteps, [] {}, [](int) {});
  advance_qk(0);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 11");  // the last score MFMA's result, before the first VALU read of S
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < kSoftPieces; ++q) soft_piece(S, 0, 0, q);
#pragma unroll
  for (int i = 0; i < kFront; ++i) vq[i] = v_tile(i, 0);
  auto step = [&](int k, int P) {  // P = k & 1
#pragma unroll
    for (int i = 0; i < kFrontPre; ++i) {
      value_mfma(i, P, k, kAlt, true);
      __builtin_amdgcn_sched_barrier(0);
    }
    // page of the tile issued below, read before the barrier (whose lgkmcnt(0) covers it) so
    // that no scalar load is in flight during the tile's LDS reads: scalar and LDS reads
    // share one counter and a pending scalar load would force every LDS wait to zero
    const int32_t pg = page_or0(k + 3);
    wait_vmcnt<kIssues>();  // tile k + 1 is done; only tile k + 2's loads may be out
    lds_barrier();    // tile k + 1 landed for every wave; tile k - 1's buffer is free
    scores(
        S, kVStart,
        [&] {
#pragma unroll
          for (int i = kFrontPre; i < kFront; ++i) {
            value_mfma(i, P, k, kAlt, true);
            __builtin_amdgcn_sched_barrier(0);
          }
        },
        [&](int j) {
          // the loads of tile k + 3 (into tile k - 1's buffer) go out one per gap behind
          // score MFMAs 1..9 (issued back to back they would stall the wave for ~200 cycles;
          // with two tiles in flight their latency has room)
          if (j >= 1 && j <= kIssues) issue(k + 3, pg, j - 1);
          if (j >= kVStart) value_mfma(j - kVStart + kFront, P, k, kAlt, true);
        });
    advance_qk(k + 1);
    // tail: tile k's last value MFMAs; tile k + 1's softmax in their gaps, from the second
    // gap on (the first gives the last score MFMA's result its 12 wait states), each piece
    // in the gap its cumulative issue cost falls in (about 30 cycles per gap, what one
    // MFMA covers)
#pragma unroll
    for (int i = 32 - kTail; i < 32; ++i) {
      value_mfma(i, P, k, kAlt, true);
      __builtin_amdgcn_sched_barrier(0);
      const int g = i - (32 - kTail);  // tail gap
      if (g == 0) asm volatile("s_nop 11");
#pragma unroll
      for (int q = 0; q < kSoftPieces; ++q)
        if (soft_gap(q, kTail - 1) == g) soft_piece(S, k + 1, 1 - P, q);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += sum_xor32(psum[P]);
    rescale();  // tile k + 1's raise, now that tile k's values are in
  };
  int k = 0;
  for (; k + 2 < n_tiles; k += 2) {
    step(k, 0);
    step(k + 1, 1);
  }
  if (k + 1 < n_tiles) {
    step(k, 0);
    ++k;
  }
  // last tile k = n_tiles - 1: its softmax is done and its first operands are read; its
  // values alone (set k & 1, moved to set 0 so that every register index stays a
  // compile-time constant), operands read four MFMAs ahead
  if (k & 1) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) pw[0][ks][e] = pw[1][ks][e];
    psum[0] = psum[1];
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    value_mfma(i, 0, k, 0, false);
    __builtin_amdgcn_sched_barrier(0);
  }
  l_run += sum_xor32(psum[0]);

  // ---- partial outputs, through LDS so that every global store writes whole rows.  O[cb]
  // item e is column 32cb + 8*(e/4) + 4*kg + e%4 of head h0 + l32: written straight out,
  // each store instruction would touch 32 head rows with 16 bytes each.  The wave puts its 32
  // rows (bf16) into its own stretch of the now idle LDS, then stores one 1 KiB row per
  // instruction.
  constexpr int kOutPitch = kDC * 2 + 16;  // LDS bytes per head row (+16: 2-way conflicts)
  static_assert(kWaves * 32 * kOutPitch <= sizeof(Smem), "output staging exceeds the LDS");
  wait_vmcnt<0>();  // no load into the ring is still out
  __syncthreads();  // every wave is done with the ring
  char* stage = reinterpret_cast<char*>(&sm) + w * 32 * kOutPitch;
#pragma unroll
  for (int cb = 0; cb < 16; ++cb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(bf16x4*)(stage + l32 * kOutPitch + (32 * cb + 8 * q + 4 * kg) * 2) =
          bf16x4{(bf16)O[cb][4 * q], (bf16)O[cb][4 * q + 1], (bf16)O[cb][4 * q + 2],
                 (bf16)O[cb][4 * q + 3]};
  __syncthreads();  // (only this wave reads its rows back; the barrier orders the LDS accesses)
  // the item index is made opaque here so that the output addresses are formed after the
  // loop instead of being held in registers across it
  asm volatile("" : "+s"(item));
  bf16* po = part_o + ((size_t)item * H + h0) * kDC + 8 * lane;
#pragma unroll 8
  for (int r = 0; r < 32; ++r)
    *(bf16x8*)(po + (size_t)r * kDC) = *(const bf16x8*)(stage + r * kOutPitch + 16 * lane);
  float* ml = part_ml + (size_t)item * H * 2;  // [H][2]
  if (kg == 0) {
    // a head that saw no token (l = 0) reports max -inf, which the merge skips
    ml[(size_t)(h0 + l32) * 2 + 0] = l_run > 0.0f ? m_ref : -INFINITY;
    ml[(size_t)(h0 + l32) * 2 + 1] = l_run;
  }
}

}  // namespace

hipError_t launch_main_bf16_wide(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const int n_hq = p.H / kHeadsWG;
  const unsigned blocks = (unsigned)(p.slots * n_hq);
  hipLaunchKernelGGL(k_main_bf16_wide, dim3(blocks), dim3(kThreads), 0, s, (const bf16*)a.qcat,
                     (const bf16*)a.latent, (const bf16*)a.rope, a.lat_tok, a.lat_seq, a.rope_tok,
                     a.rope_seq, a.work, a.block_table, a.bt_stride, p.paged, (bf16*)a.part_o,
                     a.part_ml, p.H, n_hq, a.seqlens, p.max_seqlen, p.sq, p.Hw);
  return hipGetLastError();
}

}  // namespace mla
