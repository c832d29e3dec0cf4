// Split-K main loop of the absorbed MLA decode step for head counts that are a multiple of
// 128 (gfx950, bf16 in, fp32 accumulation).
//
// Same contraction as the 32-head kernel (yololab MLA page, section 矩陣吸收: every head
// scores the one cached latent row plus its rotary key, and the latent row is also the
// value), organised so that each cached tile crosses HBM -> LDS once for 128 heads:
//
//  * one workgroup of 8 waves per CU handles (sequence b, split s, heads 128q..128q+127);
//    wave w owns 16 heads outright: their scores, softmax state and the full 512-column
//    latent output O^T (32 accumulator blocks of 16 columns x 16 heads, 128 VGPRs).  No
//    per-tile exchange between waves; two waves share each SIMD to hide each other's
//    latencies.
//  * tiles of 32 tokens stream through a ring of 3 LDS buffers by direct-to-LDS loads, so
//    two tiles are in flight while one is consumed; the barrier per tile only recycles the
//    buffer the waves finished with.  The rest of LDS holds the query's last 192 columns;
//    the first 384 stay in registers.  (The register file is the binding budget: O alone
//    is half of it.)
//  * scores S^T[t][h] = tile . q_cat^T with MFMA 16x16x32 (two 16-token blocks, 18 K-steps);
//    the probabilities go register-direct into the value product O^T += V^T P^T (token
//    order inside the K-step permuted to match the score layout; value operand read with
//    ds_read_b64_tr_b16 from the token-major tile).
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

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsWG = 128;          // heads per workgroup, 16 per wave
constexpr int kRing = 3;               // tile buffers
constexpr int kAhead = kRing - 1;      // tiles in flight ahead of the one being consumed
constexpr float kLazyTau = 8.0f;       // log2 headroom before the running max is raised
constexpr int kQRegSteps = 12;         // query K-steps (32 columns each) held in registers
constexpr int kQLdsSteps = 18 - kQRegSteps;  // the rest (latent 384..511 + rotary) in LDS

__global__ __launch_bounds__(kThreads, 1) void k_main_bf16_wide(
    const bf16* __restrict__ qcat, const bf16* __restrict__ latent,
    const bf16* __restrict__ rope, int64_t lat_tok, int64_t lat_seq, int64_t rope_tok,
    int64_t rope_seq, const int32_t* __restrict__ seqlens, const int32_t* __restrict__ bt,
    int64_t bt_stride, int paged, bf16* __restrict__ part_o, float* __restrict__ part_ml, int H,
    int S, int chunk, int n_hq, int units) {
  // One LDS object holds both regions.  (Kept as a single struct: with separate arrays the
  // compiler's wait analysis stops telling the tile reads apart from the loads in flight
  // and waits for all of them before the first read of every tile.)
  struct Smem {
    // query K-steps kQRegSteps..17 (columns 384..575), chunk-major: the 16-byte chunk of
    // K-step kQRegSteps + t, k-group g, head h at ((4t + g) * 128 + h) * 16, so 16
    // consecutive heads read 256 consecutive bytes
    char qlds[kQLdsSteps * 4 * kHeadsWG * 16];
    char ring[kRing][kBufBytes];
  };
  __shared__ __align__(16) Smem sm;  // 156 KiB
  char (&ring)[kRing][kBufBytes] = sm.ring;
  char* const qlds = sm.qlds;

  // XCD-aware mapping.  Blocks are dispatched round-robin over the 8 XCDs; XCD x gets a
  // contiguous range of (sequence, split) units, so the splits of one sequence (which all
  // read its query) and the head quads of one unit (which read the same tiles) share that
  // XCD's L2.
  const int per_xcd = (units + 7) / 8;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r = bid >> 3;
  const int hq = r % n_hq;
  const int unit = xcd * per_xcd + r / n_hq;
  if (unit >= units) return;
  const int b = unit / S, s = unit % S;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int h0 = hq * kHeadsWG + 16 * w;  // this wave's heads
  const int L = seqlens[b];
  const int t_begin = s * chunk;
  const int t_end = min(L, t_begin + chunk);
  float* ml = part_ml + ((size_t)b * S + s) * H * 2;  // [H][2]

  if (t_begin >= t_end) {
    if (tid < kHeadsWG) {
      ml[(size_t)(hq * kHeadsWG + tid) * 2 + 0] = -INFINITY;
      ml[(size_t)(hq * kHeadsWG + tid) * 2 + 1] = 0.0f;
    }
    return;
  }
  const int n_tiles = (t_end - t_begin + kTT - 1) / kTT;

  const uint32_t lat_row_b = (uint32_t)(lat_tok * 2), rope_row_b = (uint32_t)(rope_tok * 2);
  const int32_t* bt_row = bt + (paged ? (int64_t)b * bt_stride : 0);
  auto page_of = [&](int k) -> int32_t { return paged ? bt_row[(t_begin + kTT * k) / kPage] : 0; };
  auto issue = [&](int k, int64_t pg) {
    const int t0 = t_begin + kTT * k;
    const bf16 *lb, *rb;
    if (paged) {
      lb = latent + pg * lat_seq + (int64_t)(t0 % kPage) * lat_tok;
      rb = rope + pg * rope_seq + (int64_t)(t0 % kPage) * rope_tok;
    } else {
      lb = latent + (int64_t)b * lat_seq + (int64_t)t0 * lat_tok;
      rb = rope + (int64_t)b * rope_seq + (int64_t)t0 * rope_tok;
    }
    issue_tile<Sw16, kWaves>(ring[k % kRing], w, lane, lb, rb, min(kTT, t_end - t0), lat_row_b,
                             rope_row_b);
  };

  // Absorbed query as the B operand of 16x16x32 (N = heads): lane (head l16, k-group g16),
  // K-step j covers q_cat columns 32j..32j+31, the lane's 8 at 32j + 8*g16.  K-steps below
  // kQRegSteps in registers, the rest in qlds (this wave's 16 heads are written and read by
  // this wave only).
  // On the latent K-steps (0..15) lanes of odd k-groups hold their 8 columns as [4..7, 0..3],
  // the order in which they read the tile (see the score reads below); the contraction
  // order inside a K-step is free as long as both operands use the same one.
  const bool swap_half = g16 & 1;
  auto q_perm = [&](bf16x8 v, int j) -> bf16x8 {
    return (j < 16 && swap_half) ? __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3) : v;
  };
  bf16x8 qb[kQRegSteps];
  const uint32_t qr_off = (g16 * kHeadsWG + 16 * w + l16) * 16;  // + 8 KiB per LDS K-step
  {
    const bf16* qrow = qcat + ((size_t)b * H + h0 + l16) * kRow + 8 * g16;
#pragma unroll
    for (int j = 0; j < kQRegSteps; ++j) qb[j] = q_perm(*(const bf16x8*)(qrow + 32 * j), j);
#pragma unroll
    for (int t = 0; t < kQLdsSteps; ++t)
      *(bf16x8*)(qlds + qr_off + 8192 * t) =
          q_perm(*(const bf16x8*)(qrow + 32 * (kQRegSteps + t)), kQRegSteps + t);
  }
  // Tile 0 lands together with the query.  Draining the counter here also tells the
  // compiler's wait analysis that the query registers are complete, so no wait on them
  // (which would also wait on younger tile loads) reaches the loop.
  issue(0, page_of(0));
  wait_vmcnt<0>();
  for (int k = 1; k < kAhead && k < n_tiles; ++k) issue(k, page_of(k));

  // Score reads (A = tile, M = tokens): token 16*tb + l16, chunk 4j + g16.  The swizzle
  // permutes within aligned 16-chunk groups and repeats every 16 rows, so j = 4u + j'
  // adds 256u bytes and tb adds 16 KiB.  Latent chunks are read as two 8-byte halves, odd
  // k-groups taking the upper half first, so that the two 16-lane groups of each 32-lane
  // half touch different halves of the same chunk slots (conflict-free; a 16-byte read of
  // this pattern conflicts two ways).
  uint32_t qk_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qk_off[j] = lat_chunk<Sw16>(l16, 4 * j + g16) + (swap_half ? 8 : 0);
  uint32_t rp_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) rp_off[j] = rope_chunk(l16, 4 * j + g16);  // tb adds 2 KiB
  // Value reads (A = V^T, M = 16 latent columns, K = 32 tokens): 16-lane group g16 holds
  // tokens 4*g16..+3 and 16 + 4*g16..+3; source lane l16 addresses token row 4*g16 + l16/4
  // (+16 for the second read), columns 4*(l16 & 3)..+3 of the block.  Column block
  // cb = 8u + c adds 256u bytes; the second read adds 16 KiB.
  uint32_t pv_off[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) pv_off[c] = lat_piece<Sw16>(4 * g16 + (l16 >> 2), 16 * c + 4 * (l16 & 3));

  const bool rope_wave = w < 4;
  float m_ref = -INFINITY, l_run = 0.0f;  // per head l16 (the four k-groups hold the same)
  f32x4 O[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) O[cb] = f32x4{};

  for (int k = 0; k < n_tiles; ++k) {
    // page of the tile issued below, read before the barrier (whose lgkmcnt(0) covers it) so
    // that no scalar load is in flight during the tile's LDS reads: scalar and LDS reads
    // share one counter and a pending scalar load would force every LDS wait to zero
    const int32_t pg = k + kAhead < n_tiles ? page_of(k + kAhead) : 0;
    // this wave's loads of tile k are done once only the younger tiles' loads remain
    static_assert(kAhead == 2, "wait counts below assume two tiles in flight");
    if (k + 1 < n_tiles) {
      if (rope_wave) wait_vmcnt<issues_per_wave<kWaves>(true)>();
      else wait_vmcnt<issues_per_wave<kWaves>(false)>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();  // tile k landed for every wave; the buffer of tile k-1 is free
    if (k + kAhead < n_tiles) issue(k + kAhead, pg);
    __builtin_amdgcn_sched_barrier(0);  // no operand reads hoisted above the loads' issue
    // Per-tile LDS base addresses, opaque to the optimiser: every read below is one of these
    // plus a constant that goes into the instruction's offset field (otherwise the compiler
    // hoists one register per base + constant, or picks a base above the reads and pays an
    // add per read for the negative difference).
    const uint32_t bufa = lds_addr(ring[k % kRing]);
    uint32_t qa[4], ra[2], pa[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) qa[j] = opaque(bufa + qk_off[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) ra[j] = opaque(bufa + rp_off[j]);
#pragma unroll
    for (int c = 0; c < 8; ++c) pa[c] = opaque(bufa + pv_off[c]);
    const uint32_t qla = opaque(lds_addr(qlds) + qr_off);

    // ---- S^T[t][h] for tokens 16*tb.. (M) and the wave's 16 heads (N).  Tile operands
    // are read kQkAhead K-steps ahead of their MFMAs.
    auto a_tile = [&](int j, int tb) -> bf16x8 {
      // the other half's address: one XOR per read (o is a multiple of 256), formed here
      // rather than kept in four more registers
      const uint32_t o = 256 * (j >> 2) + 16384 * tb;
      return j < 16 ? b64_pair_at(qa[j & 3] + o, opaque(qa[j & 3] ^ 8u) + o)
                    : lds_read16_at(ra[j - 16] + 2048 * tb);
    };
    constexpr int kQkAhead = 1;
    // two accumulators per token block (even / odd K-steps): a dependent chain of 16x16x32
    // MFMAs issues at about a third of the unit's rate
    f32x4 acc2[2][2] = {};
    bf16x8 aq[kQkAhead + 1][2];
#pragma unroll
    for (int j = 0; j < kQkAhead; ++j) {
      aq[j][0] = a_tile(j, 0);
      aq[j][1] = a_tile(j, 1);
    }
#pragma unroll
    for (int j = 0; j < 18; ++j) {
      if (j + kQkAhead < 18) {
        aq[(j + kQkAhead) % (kQkAhead + 1)][0] = a_tile(j + kQkAhead, 0);
        aq[(j + kQkAhead) % (kQkAhead + 1)][1] = a_tile(j + kQkAhead, 1);
      }
      const bf16x8 qv = j < kQRegSteps ? qb[j < kQRegSteps ? j : 0]
                                       : lds_read16_at(qla + 8192 * (j - kQRegSteps));
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        acc2[tb][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[j % (kQkAhead + 1)][tb], qv,
                                                                  acc2[tb][j & 1], 0, 0, 0);
      // keep the written order: the scheduler would otherwise hoist more reads than the
      // register budget holds (O takes half of it) and spill
      __builtin_amdgcn_sched_barrier(0);
    }

    // value operands of the first column blocks, read while the softmax runs
    auto v_tile = [&](int cb) -> bf16x8 {
      const uint32_t a = pa[cb & 7] + 256 * (cb >> 3);
      return tr_pair_at(a, a + 16384);
    };
    constexpr int kPvAhead = 4;
    bf16x8 vq[kPvAhead + 1];
#pragma unroll
    for (int cb = 0; cb < kPvAhead; ++cb) vq[cb] = v_tile(cb);

    f32x4 acc[2] = {acc2[0][0] + acc2[0][1], acc2[1][0] + acc2[1][1]};

    // ---- softmax.  D layout: lane (head l16, group g16), item e of block tb ->
    // token 16*tb + 4*g16 + e
    const int valid = min(kTT, t_end - t_begin - kTT * k);
    if (valid < kTT) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * tb + 4 * g16 + e >= valid) acc[tb][e] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(acc[0][0], acc[0][1]), fmaxf(acc[0][2], acc[0][3])),
                     fmaxf(fmaxf(acc[1][0], acc[1][1]), fmaxf(acc[1][2], acc[1][3])));
    mx = max_xor32(max_xor16(mx));  // every tile holds a valid token: mx finite
    if (k == 0) {
      m_ref = mx;  // O and l are still zero
    } else if (__ballot(mx > m_ref + kLazyTau) != 0) {
      const float m_new = fmaxf(m_ref, mx);
      const float a = exp2f(m_ref - m_new);
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) O[cb] *= a;
      l_run *= a;
      m_ref = m_new;
    }
    // B operand of the value product (K = 32 tokens, N = heads): lane (head l16, k-group
    // g16) item e <-> token 4*g16 + e (e < 4) or 16 + 4*g16 + e - 4: the lane's own scores.
    bf16x8 pb;
    float psum = 0.0f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16 p = (bf16)__builtin_amdgcn_exp2f(acc[tb][e] - m_ref);
        pb[4 * tb + e] = p;
        psum += (float)p;  // normalise with the rounded weights the MFMA uses
      }
    l_run += sum_xor32(sum_xor16(psum));

    // ---- O^T[d][h] += V^T P^T over the 32 column blocks, operands kPvAhead blocks ahead
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      if (cb + kPvAhead < 32) vq[(cb + kPvAhead) % (kPvAhead + 1)] = v_tile(cb + kPvAhead);
      O[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vq[cb % (kPvAhead + 1)], pb, O[cb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- partial outputs.  O[cb] item e: column 16cb + 4*g16 + e of head h0 + l16
  bf16* po = part_o + (((size_t)b * S + s) * H + h0 + l16) * kDC + 4 * g16;
#pragma unroll
  for (int cb = 0; cb < 32; ++cb)
    *(bf16x4*)(po + 16 * cb) =
        bf16x4{(bf16)O[cb][0], (bf16)O[cb][1], (bf16)O[cb][2], (bf16)O[cb][3]};
  if (g16 == 0) {
    ml[(size_t)(h0 + l16) * 2 + 0] = m_ref;
    ml[(size_t)(h0 + l16) * 2 + 1] = l_run;
  }
}

}  // namespace

hipError_t launch_main_bf16_wide(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const int n_hq = p.H / kHeadsWG;
  const int units = p.B * p.splits;
  const unsigned blocks = (unsigned)(((units + 7) / 8) * 8 * n_hq);
  hipLaunchKernelGGL(k_main_bf16_wide, dim3(blocks), dim3(kThreads), 0, s, (const bf16*)a.qcat,
                     (const bf16*)a.latent, (const bf16*)a.rope, a.lat_tok, a.lat_seq, a.rope_tok,
                     a.rope_seq, a.seqlens, a.block_table, a.bt_stride, p.paged, (bf16*)a.part_o,
                     a.part_ml, p.H, p.splits, p.chunk, n_hq, units);
  return hipGetLastError();
}

}  // namespace mla
