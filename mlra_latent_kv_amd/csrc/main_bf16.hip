// Split-K main loop of the absorbed MLA / MLRA-4 decode step for gfx950 (bf16 in, fp32 acc).
//
// One workgroup per (work item of the split plan: sequence b, tokens [t_begin, t_end); group
// of 32 heads).  The workgroup streams the item's cached rows [c_KV (512) | k_rope (64)] in
// 32-token tiles through a ring of LDS
// buffers filled by direct-to-LDS buffer loads (no staging registers, rows past the end of
// the sequence read back as zeros), and per tile computes
//   S  = q_cat . tile^T       scores of 32 heads x 32 tokens (MFMA 32x32x16 bf16)
//   online softmax            running max / sum per head (per branch for MLRA-4)
//   O += P . tile[:, :512]    latent-space output; the value operand is read from the
//                             token-major tile with ds_read_b64_tr_b16
// and finally writes its partial (m, l, O) for the combine kernel.  This is the absorbed
// form of the yololab MLA page (section 矩陣吸收): all heads share the one cached latent, so
// each tile is a dense [heads x 576] . [576 x tokens] contraction and the latent doubles as
// the value.  For MLRA-4 ("[ICLR 2025] MLRA…", section 2.1) the latent holds four
// 128-wide branches with independent softmaxes that share the rotary score.
//
// Two workgroups share a CU (LDS <= 80 KB each, <= 256 VGPRs per wave), so every SIMD has a
// second wave to run while one waits on LDS, MFMA results or a barrier.  Each workgroup
// double-buffers its tiles: one lands while the other is consumed.
//
// Wave w (of 4) accumulates O^T for a quarter of the latent columns, [w DC/4, (w+1) DC/4).
//  * MLA (one branch, latent width DC = 512, or 128 for one MLRA branch run on its own as a
//    tensor-parallel shard with rows [c_b | k_rope] of 192): for the scores, wave w takes
//    tokens 16*(w&1).. and heads 16*(w>>1).. of the tile over all DC + 64 columns (MFMA
//    16x16x32, query in registers).  Partner waves (same heads, other 16 tokens) swap
//    per-head maxima and sums through LDS, and every wave publishes its bf16 probabilities
//    for everyone's PV step.
//  * MLRA-4: wave w's latent columns are exactly branch w; it computes its branch's scores
//    plus the full rotary score itself, so the branch's softmax and probabilities never
//    leave its registers.
#include "device_common.h"
#include "launch.h"
#include "tile_bf16.h"

namespace mla {
namespace {

using namespace tile;

constexpr int kHG = kHeadGroup;                      // heads per workgroup
constexpr int kThreads = 256;                        // 4 waves
constexpr int kPPitch = kTT + 8;                     // bf16 probability row pitch
// Tile ring depth per workgroup: two 36 KB buffers for the 576-wide rows (two workgroups per
// CU fill the LDS); the 12 KB tiles of the 192-wide rows take a deeper ring in the same room,
// so that more of the (short) per-tile compute overlaps loads in flight.
#ifndef MLA_NARROW_RING
#define MLA_NARROW_RING 2
#endif
// Lazy softmax rescale: a head's running max is raised (and O, l rescaled) only when a tile's
// max exceeds it by more than this many log2 units; otherwise the tile's weights are taken
// against the stale max and stay below 2^kLazyTau (0: raise on every increase).
#ifndef MLA_NARROW_LAZY
#define MLA_NARROW_LAZY 8
#endif
constexpr float kLazyTau = MLA_NARROW_LAZY;
// MLA path: weights taken speculatively against the running max before the halves' maxima
// are exchanged (one LDS barrier per tile instead of two); a tile that raises some head's
// max redoes its weights (0: always exchange the maxima first).
#ifndef MLA_NARROW_SPEC
#define MLA_NARROW_SPEC 1
#endif
template <int DC>
constexpr int ring_depth() { return DC == 512 ? 2 : MLA_NARROW_RING; }

// 8-byte LDS read of staged codes, through a restrict pointer like every other tile read (so
// that the wait analysis does not take it for a read of the loads in flight)
__device__ __forceinline__ uint2 lds_read8u(const char* __restrict__ p) {
  return *reinterpret_cast<const uint2*>(p);
}

// fp8 latent (F8): a tile arrives as E4M3 latent rows (DC bytes each, unswizzled) followed by
// the bf16 rotary rows (swizzled as in the widened tile) in one of two staging slots, and is
// widened once per workgroup into the single bf16 tile buffer the compute reads.
template <int DC>
constexpr int stage_bytes() { return kTT * DC + kTT * kRopeRowB; }

// Exchange buffers first, then the tile ring on a 256-byte boundary (F8: one widened tile,
// then the two staging slots).
template <int NB, int DC, bool F8>
struct Smem {
  bf16 p[NB == 1 ? kHG * kPPitch : 8];        // MLA: probabilities [h][t]
  float mx[NB == 1 ? 2 * kHG : 1];            // MLA: per-head max of each 16-token half
  float sum[NB == 1 ? 2 * kHG : 1];           // MLA: per-head probability sum of each half
  float alpha[NB == 1 ? kHG : 1];             // MLA: per-head rescale of this tile
  float mrun[NB == 1 ? kHG : 1];              // MLA: per-head running max (published)
  char gap[256];
  __attribute__((aligned(256))) char ring[F8 ? 1 : ring_depth<DC>()][Geom<DC>::kBufBytes];
  __attribute__((aligned(256))) char stage[F8 ? 2 : 1][F8 ? stage_bytes<DC>() : 16];
};

template <int NB, int DC, bool F8>
__global__ __launch_bounds__(kThreads, DC == 512 ? 2 : kNarrowWgPerCu) void k_main_bf16(
    const bf16* __restrict__ qcat, const bf16* __restrict__ latent,
    const bf16* __restrict__ rope, int64_t lat_tok, int64_t lat_seq, int64_t rope_tok,
    int64_t rope_seq, const int32_t* __restrict__ work, const int32_t* __restrict__ bt,
    int64_t bt_stride, int paged, bf16* __restrict__ part_o, float* __restrict__ part_ml, int H,
    int n_hg, const int32_t* __restrict__ seqlens, int max_seqlen, int sq, int Hw) {
  static_assert(NB == 1 || DC == 512, "MLRA-4 rows hold four 128-wide branches");
  using G = Geom<DC>;
  // tiles in flight + compute: the bf16 ring, or (F8) the two staging slots
  constexpr int kBufs = F8 ? 2 : ring_depth<DC>();
  constexpr int kIssues = issues_per_wave<4, DC>(true);  // tile loads per wave per tile
  static_assert(!F8 || kBufs == 2, "the fp8 path waits for each tile with vmcnt(0)");
  constexpr int kRowW = DC + kDR;   // cached (and absorbed-query) row width
  constexpr int kNOB = DC / 128;    // 32-column output blocks per wave
  __shared__ __align__(16) Smem<NB, DC, F8> sm;

  // XCD-aware mapping: consecutive blocks go to different XCDs, so the head groups of one
  // dispatch slot (one work item) are placed 8 blocks apart -> same XCD, dispatched back to
  // back, and their reads of the same tiles can hit that XCD's L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r = bid >> 3;
  const int hg = r % n_hg;
  const int4 wi = *reinterpret_cast<const int4*>(work + 4 * ((r / n_hg) * 8 + xcd));
  const int b = wi.x;
  if (b < 0) return;  // slot without a work item
  const int t_begin = wi.y, t_end = wi.z;  // page-aligned start, never empty
  const size_t item = (size_t)wi.w;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, kg = lane >> 5;
  const int h0 = hg * kHG;
  float* ml = part_ml + item * NB * H * 2;  // [br][H][2]
  // the tokens this head group's query token sees (s_q > 1 query tokens: token h0 / Hw is
  // causal), within the item: scores past t_lim are masked; the tiles still load to t_end
  const int t_lim = sq > 1 ? min(t_end, causal_limit(seqlens, b, max_seqlen, sq, h0 / Hw)) : t_end;

  const int n_tiles = (t_end - t_begin + kTT - 1) / kTT;

  // Tile loads: wave w brings latent rows 8w..8w+7 and the rotary keys of the same rows
  // (chunk-swizzled through the per-lane source offsets).
  const uint32_t lat_row_b = (uint32_t)(lat_tok * (F8 ? 1 : 2)), rope_row_b = (uint32_t)(rope_tok * 2);

  // tile k of the item into its ring buffer.  Past the item's end (k >= n_tiles) the same
  // loads go out with an empty buffer descriptor: they return zeros without touching memory,
  // so every wave issues the same number of loads per tile on every path and every wait below
  // is a fixed count.
  auto issue = [&](int k) {
    const int t0 = t_begin + kTT * k;
    const int valid = k < n_tiles ? min(kTT, t_end - t0) : 0;
    // latent element size: 2 bytes, or 1 for E4M3 codes (lat_tok / lat_seq count elements)
    constexpr int kLe = F8 ? 1 : 2;
    const char* lb = reinterpret_cast<const char*>(latent);
    const bf16* rb = rope;
    if (valid == 0) {
    } else if (paged) {
      const int64_t pg = bt[(int64_t)b * bt_stride + t0 / kPage];
      lb += kLe * (pg * lat_seq + (int64_t)(t0 % kPage) * lat_tok);
      rb = rope + pg * rope_seq + (int64_t)(t0 % kPage) * rope_tok;
    } else {
      lb += kLe * ((int64_t)b * lat_seq + (int64_t)t0 * lat_tok);
      rb = rope + (int64_t)b * rope_seq + (int64_t)t0 * rope_tok;
    }
    const int vu = __builtin_amdgcn_readfirstlane(valid);
    if constexpr (F8) {
      // E4M3 latent rows, row-major in the slot (one instruction = 1 KiB = 1024 / DC rows),
      // then the bf16 rotary rows 8w .. 8w + 7 swizzled as in the widened tile
      char* slot = sm.stage[k % kBufs];
      constexpr int kRowsPerLd = 1024 / DC, kCpr = DC / 16, kLd = kTT / kRowsPerLd / 4;
      const __amdgpu_buffer_rsrc_t rl = rsrc(lb, vu * lat_row_b);
#pragma unroll
      for (int j = 0; j < kLd; ++j) {
        const int r0 = (kLd * w + j) * kRowsPerLd, t = r0 + lane / kCpr;
        dma16(rl, slot + r0 * DC, t * lat_row_b + 16 * (lane % kCpr));
      }
      const __amdgpu_buffer_rsrc_t rr = rsrc(rb, vu * rope_row_b);
      const int rt = 8 * w + (lane >> 3);
      dma16(rr, slot + kTT * DC + w * 1024, rt * rope_row_b + 16 * ((lane & 7) ^ rope_sw(rt)));
    } else {
      issue_tile<Sw32, 4, DC>(sm.ring[k % kBufs], w, lane, reinterpret_cast<const bf16*>(lb), rb,
                              vu, lat_row_b, rope_row_b);
    }
  };
  // F8: widen the staged tile k (slot k % 2) into the bf16 tile buffer: every 8 E4M3 codes of
  // a latent row become one 16-byte chunk at its swizzled place (exact: E4M3 fits in bf16),
  // and the rotary rows are copied as they are (already in the buffer's layout)
  auto widen = [&](int k) {
    const char* slot = sm.stage[k % kBufs];
    char* dst = sm.ring[0];
    constexpr int kPieces = DC / 8;  // 8-code pieces per row
#pragma unroll
    for (int i = 0; i < kTT * kPieces / kThreads; ++i) {
      const int u = tid + kThreads * i, row = u / kPieces, c = u % kPieces;
      const uint2 v = lds_read8u(slot + row * DC + 8 * c);
      const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, false);
      const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, true);
      const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, false);
      const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, true);
      lds_write16(dst + lat_chunk<Sw32, DC>(row, c),
                  bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]});
    }
#pragma unroll
    for (int i = 0; i < kTT * kRopeRowB / 16 / kThreads; ++i) {
      const int u = tid + kThreads * i;
      lds_write16(dst + G::kRopeOff + 16 * u, lds_read16(slot + kTT * DC + 16 * u));
    }
  };

  // absorbed query as the MFMA B operand (N = heads).
  //  MLA, 16x16x32: lane (head 16*(w>>1) + lane%16, k-group lane/16), K-step j = 32 columns
  //  (DC / 32 latent steps, then 2 rotary ones).
  //  MLRA, 32x32x16: lane (head l32, k-half kg), K-step j = 16 columns of branch w / rope.
  constexpr int kLatSteps = DC / 32;
  constexpr int kQSteps = NB == 1 ? kLatSteps + 2 : 12;
  const int tb = w & 1, hb = w >> 1;          // MLA score block: token half, head half
  const int l16 = lane & 15, g16 = lane >> 4;
  bf16x8 qb[kQSteps];
  if (NB == 1) {
    const bf16* qrow = qcat + ((size_t)b * H + h0 + 16 * hb + l16) * kRowW + 8 * g16;
#pragma unroll
    for (int j = 0; j < kQSteps; ++j) qb[j] = *(const bf16x8*)(qrow + 32 * j);
  } else {
    const bf16* qrow = qcat + ((size_t)b * H + h0 + l32) * kRowW + 8 * kg;
#pragma unroll
    for (int j = 0; j < 8; ++j) qb[j] = *(const bf16x8*)(qrow + 128 * w + 16 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[8 + j] = *(const bf16x8*)(qrow + kDC + 16 * j);
  }

  // start-up: the query, then tiles 0 .. kBufs - 2, then one wait for all but tiles 1 ..
  // kBufs - 2.  The query's loads are older than tile 0's, so the wait completes them too,
  // and tells the compiler's wait analysis so (it would otherwise wait for every load in
  // flight before the first use of the query registers).
#pragma unroll
  for (int j = 0; j < kBufs - 1; ++j) issue(j);
  wait_vmcnt<(kBufs - 2) * kIssues>();

  float m_run = -INFINITY, l_run = 0.0f;
  if (NB == 1 && tb == 0 && g16 == 0) sm.mrun[16 * hb + l16] = -INFINITY;  // (ordered by the
                                                                           // first tile's barrier)
  f32x16 O[kNOB];
#pragma unroll
  for (int mb = 0; mb < kNOB; ++mb) O[mb] = f32x16{};

  // transposed-read sources of the value operand: rows v_row and v_row + v_delta of each
  // 16-token half, columns w DC/4 + 32mb + v_col (this wave's latent columns)
  const int g = lane >> 4, li = lane & 15;
  const int v_col = 16 * (g & 1) + 4 * (li & 3);
  const int v_row = NB == 1 ? 8 * kg + (li >> 2) : 4 * kg + (li >> 2);
  constexpr int v_delta = NB == 1 ? 4 : 8;
  uint32_t pv_off[2][2][kNOB];  // [half][read][mb]
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int mb = 0; mb < kNOB; ++mb)
        pv_off[s2][r][mb] =
            lat_piece<Sw32, DC>(16 * s2 + v_row + r * v_delta, w * (DC / 4) + 32 * mb + v_col);

  for (int k = 0; k < n_tiles; ++k) {
    // tile k has landed (the kBufs - 2 younger tiles' loads may still be out); after the
    // barrier it has landed for every wave, and tile k - 1's buffer is free for k + kBufs - 1
    wait_vmcnt<(kBufs - 2) * kIssues>();
    lds_barrier();
    // F8: slot k -> the bf16 buffer (every wave is done with tile k - 1), before the next
    // tile's loads go out: read after them, the staged codes would be waited on together
    // with those loads (the wait analysis cannot tell the two slots apart)
    if constexpr (F8) widen(k);
    issue(k + kBufs - 1);
    if constexpr (F8) lds_barrier();  // the widened tile is complete

    const int t0 = t_begin + kTT * k;
    const int valid = min(kTT, t_lim - t0);  // <= 0: every score of the tile masked
    const char* buf = sm.ring[F8 ? 0 : k % kBufs];

    bf16x8 pb[2];
    float alpha;
    if (NB == 1) {
      // ---- scores of 16 tokens x 16 heads over all 576 columns (M = tokens, N = heads)
      f32x4 acc = {};
      {
        // K-step j covers columns 32j..32j+31: chunk 4j + g16 of token t
        const int t = 16 * tb + l16;
#pragma unroll
        for (int j = 0; j < kLatSteps; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              lds_read16(buf + lat_chunk<Sw32, DC>(t, 4 * (j & 3) + g16) + 256 * (j >> 2)),
              qb[j], acc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              lds_read16(buf + rope_chunk<DC>(t, 4 * j + g16)), qb[kLatSteps + j], acc, 0, 0, 0);
      }
      // D layout: lane (head 16*hb + l16, group g16), item e -> token 16*tb + 4*g16 + e
      const int h = 16 * hb + l16;
      const int tq = 16 * tb + 4 * g16;
      // Masked without a branch: a uniform branch around the masking put the first read of
      // the last MFMA's result right behind it on the taken path, without the wait states
      // that read needs (the compiler pads straight-line code, not that path), so the max
      // could pick up the accumulator before the last K-step landed.
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = tq + e < valid ? acc[e] : -INFINITY;
      float mx = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
      mx = max_xor32(max_xor16(mx));
      // weights of this wave's 16 tokens against m_ref, and their sum (normalised with the
      // rounded weights the MFMA uses); -inf max only while every token so far is masked (a
      // query token that sees none of this item's tokens yet): taken against 0, they are 0
      bf16 pe[4];
      float psum;
      auto weights = [&](float m_ref) {
        const float m_off = m_ref == -INFINITY ? 0.0f : m_ref;
        psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pe[e] = (bf16)exp2f(acc[e] - m_off);
          psum += (float)pe[e];
        }
        psum = sum_xor32(sum_xor16(psum));
      };
#if MLA_NARROW_SPEC
      // speculative: against the running max, right unless some head's tile max passes it by
      // more than kLazyTau.  Every wave then checks all 32 heads (its value-layout head l32)
      // from the published maxima, so the (rare) redo is taken by the whole workgroup.
      weights(m_run);
      *(bf16x4*)(&sm.p[h * kPPitch + tq]) = bf16x4{pe[0], pe[1], pe[2], pe[3]};
      if (g16 == 0) {
        sm.mx[tb * kHG + h] = mx;
        sm.sum[tb * kHG + h] = psum;
      }
      lds_barrier();
      const bool raise_l = fmaxf(sm.mx[l32], sm.mx[kHG + l32]) > sm.mrun[l32] + kLazyTau;
      if (__builtin_amdgcn_ballot_w64(raise_l)) {
        mx = fmaxf(mx, sm.mx[(tb ^ 1) * kHG + h]);  // max over the tile's 32 tokens
        const bool raise_h = mx > m_run + kLazyTau;  // the first tile with a token raises
        const float m_new = raise_h ? mx : m_run;
        const float a = raise_h ? exp2f(m_run - m_new) : 1.0f;
        weights(m_new);
        lds_barrier();  // every wave has read the speculative tile's maxima
        *(bf16x4*)(&sm.p[h * kPPitch + tq]) = bf16x4{pe[0], pe[1], pe[2], pe[3]};
        if (g16 == 0) {
          sm.sum[tb * kHG + h] = psum;
          if (tb == 0) {
            sm.alpha[h] = a;
            sm.mrun[h] = m_new;
          }
        }
        lds_barrier();
        l_run = a * l_run + psum + sm.sum[(tb ^ 1) * kHG + h];
        m_run = m_new;
        alpha = sm.alpha[l32];
      } else {
        l_run += psum + sm.sum[(tb ^ 1) * kHG + h];
        alpha = 1.0f;
      }
#else
      if (g16 == 0) sm.mx[tb * kHG + h] = mx;
      lds_barrier();
      mx = fmaxf(mx, sm.mx[(tb ^ 1) * kHG + h]);  // max over the tile's 32 tokens
      const bool raise_h = mx > m_run + kLazyTau;  // lazy raise; the first tile raises
      const float m_new = raise_h ? mx : m_run;
      const float a = raise_h ? exp2f(m_run - m_new) : 1.0f;
      weights(m_new);
      *(bf16x4*)(&sm.p[h * kPPitch + tq]) = bf16x4{pe[0], pe[1], pe[2], pe[3]};
      if (g16 == 0) {
        sm.sum[tb * kHG + h] = psum;
        if (tb == 0) sm.alpha[h] = a;
      }
      lds_barrier();
      l_run = a * l_run + psum + sm.sum[(tb ^ 1) * kHG + h];
      m_run = m_new;
      alpha = sm.alpha[l32];
#endif
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        pb[s2] = lds_read16((const char*)&sm.p[l32 * kPPitch + 16 * s2 + 8 * kg]);
    } else {
      // ---- branch-w scores S^T[t][h] (M = tokens, N = heads): 128 latent + 64 rotary columns
      f32x16 acc = {};
      {
        // K-step j covers columns 128w + 16j..: chunk 16w + 2j + kg of token l32
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_read16(buf + lat_chunk<Sw32>(l32, 2 * j + kg) + 256 * w), qb[j], acc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_read16(buf + rope_chunk(l32, 2 * j + kg)), qb[8 + j], acc, 0, 0, 0);
      }
      // D layout: lane (head l32, half kg), item i -> token 8*(i/4) + 4*kg + i%4
#pragma unroll
      for (int i = 0; i < 16; ++i)
        acc[i] = 8 * (i >> 2) + 4 * kg + (i & 3) < valid ? acc[i] : -INFINITY;  // no branch
      float mx = acc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, acc[i]);
      mx = max_xor32(mx);
      const bool raise_h = mx > m_run + kLazyTau;  // lazy raise, as above
      const float m_new = raise_h ? mx : m_run;
      const float m_off = m_new == -INFINITY ? 0.0f : m_new;  // every token so far masked
      alpha = raise_h ? exp2f(m_run - m_new) : 1.0f;
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bf16 e = (bf16)exp2f(acc[i] - m_off);
        pb[i >> 3][i & 7] = e;
        psum += (float)e;
      }
      psum = sum_xor32(psum);
      l_run = alpha * l_run + psum;
      m_run = m_new;
    }

    // ---- O^T[d][h] += V^T P^T over this wave's DC / 4 latent columns
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {  // some head of the wave raised
#pragma unroll
      for (int mb = 0; mb < kNOB; ++mb) O[mb] *= alpha;
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mb = 0; mb < kNOB; ++mb)
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_pair(buf + pv_off[s2][0][mb], buf + pv_off[s2][1][mb]), pb[s2], O[mb], 0, 0, 0);
  }

  // ---- partial outputs, through LDS so that every global store writes whole rows.  O[mb]
  // item i is column d = w DC/4 + 32mb + 8*(i/4) + 4*kg + i%4 of head l32: written straight
  // out, each store instruction would touch 32 head rows with 16 bytes each.  The waves put
  // the 32 x DC block (bf16) into the now idle tile ring, then each stores its 8 rows, one
  // 1 KiB (or four 256-byte rows) per instruction.
  constexpr int kOutPitch = DC * 2 + 16;  // LDS bytes per head row (+16: 2-way conflicts)
  static_assert(kHG * kOutPitch <= G::kBufBytes, "output staging exceeds one ring buffer");
  wait_vmcnt<0>();  // the loads past the item's last tile have landed (into other buffers)
  __syncthreads();  // every wave is done with the ring
  char* stage = sm.ring[0];
#pragma unroll
  for (int mb = 0; mb < kNOB; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(bf16x4*)(stage + l32 * kOutPitch + (w * (DC / 4) + 32 * mb + 8 * q + 4 * kg) * 2) =
          bf16x4{(bf16)O[mb][4 * q], (bf16)O[mb][4 * q + 1], (bf16)O[mb][4 * q + 2],
                 (bf16)O[mb][4 * q + 3]};
  __syncthreads();
  // lane -> (row r0 + lane / chunks, 16-byte chunk lane % chunks) of the wave's 8 rows
  constexpr int kRowsPerStore = G::kRowsPerLoad;
  const int sr = lane / G::kChunks, sc = lane % G::kChunks;
  bf16* po = part_o + (item * H + h0) * DC + 8 * sc;
#pragma unroll
  for (int j = 0; j < kHG / 4 / kRowsPerStore; ++j) {
    const int r = (kHG / 4) * w + j * kRowsPerStore + sr;
    *(bf16x8*)(po + (size_t)r * DC) = *(const bf16x8*)(stage + r * kOutPitch + 16 * sc);
  }
  if (NB == 1) {
    if (tb == 0 && g16 == 0) {
      const int hs = h0 + 16 * hb + l16;
      ml[(size_t)hs * 2 + 0] = m_run;
      ml[(size_t)hs * 2 + 1] = l_run;
    }
  } else if (kg == 0) {
    ml[((size_t)w * H + h0 + l32) * 2 + 0] = m_run;
    ml[((size_t)w * H + h0 + l32) * 2 + 1] = l_run;
  }
}

}  // namespace

hipError_t launch_main_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)(p.slots * p.n_hg);
  auto kern = p.f8 ? (p.NB == 4 ? k_main_bf16<4, 512, true> : p.dcb == 512 ? k_main_bf16<1, 512, true>
                                                                           : k_main_bf16<1, 128, true>)
                   : (p.NB == 4 ? k_main_bf16<4, 512, false> : p.dcb == 512 ? k_main_bf16<1, 512, false>
                                                                            : k_main_bf16<1, 128, false>);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, s, (const bf16*)a.qcat,
                     (const bf16*)a.latent, (const bf16*)a.rope, a.lat_tok, a.lat_seq, a.rope_tok,
                     a.rope_seq, a.work, a.block_table, a.bt_stride, p.paged, (bf16*)a.part_o,
                     a.part_ml, p.H, p.n_hg, a.seqlens, p.max_seqlen, p.sq, p.Hw);
  return hipGetLastError();
}

}  // namespace mla
