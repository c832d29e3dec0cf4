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
// Wave w (of 4) accumulates O^T for latent columns [128w, 128w+128).
//  * MLA (one branch): for the scores, wave w takes tokens 16*(w&1).. and heads 16*(w>>1)..
//    of the tile over the full 576 columns (MFMA 16x16x32, query in registers).  Partner
//    waves (same heads, other 16 tokens) swap per-head maxima and sums through LDS, and
//    every wave publishes its bf16 probabilities for everyone's PV step.
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
constexpr int kBufs = 2;                             // tile ring depth per workgroup

// Exchange buffers first, then the tile ring on a 256-byte boundary.
template <int NB>
struct Smem {
  bf16 p[NB == 1 ? kHG * kPPitch : 8];        // MLA: probabilities [h][t]
  float mx[NB == 1 ? 2 * kHG : 1];            // MLA: per-head max of each 16-token half
  float sum[NB == 1 ? 2 * kHG : 1];           // MLA: per-head probability sum of each half
  float alpha[NB == 1 ? kHG : 1];             // MLA: per-head rescale of this tile
  char gap[256];
  __attribute__((aligned(256))) char ring[kBufs][kBufBytes];
};

template <int NB>
__global__ __launch_bounds__(kThreads, 2) void k_main_bf16(
    const bf16* __restrict__ qcat, const bf16* __restrict__ latent,
    const bf16* __restrict__ rope, int64_t lat_tok, int64_t lat_seq, int64_t rope_tok,
    int64_t rope_seq, const int32_t* __restrict__ work, const int32_t* __restrict__ bt,
    int64_t bt_stride, int paged, bf16* __restrict__ part_o, float* __restrict__ part_ml, int H,
    int n_hg) {
  __shared__ __align__(16) Smem<NB> sm;

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

  const int n_tiles = (t_end - t_begin + kTT - 1) / kTT;

  // Tile loads: wave w brings latent rows 8w..8w+7 and the rotary keys of the same rows
  // (chunk-swizzled through the per-lane source offsets).
  const uint32_t lat_row_b = (uint32_t)(lat_tok * 2), rope_row_b = (uint32_t)(rope_tok * 2);

  auto issue = [&](int k) {
    const int t0 = t_begin + kTT * k;
    const int valid = min(kTT, t_end - t0);
    const bf16* lb;
    const bf16* rb;
    if (paged) {
      const int64_t pg = bt[(int64_t)b * bt_stride + t0 / kPage];
      lb = latent + pg * lat_seq + (int64_t)(t0 % kPage) * lat_tok;
      rb = rope + pg * rope_seq + (int64_t)(t0 % kPage) * rope_tok;
    } else {
      lb = latent + (int64_t)b * lat_seq + (int64_t)t0 * lat_tok;
      rb = rope + (int64_t)b * rope_seq + (int64_t)t0 * rope_tok;
    }
    issue_tile<Sw32, 4>(sm.ring[k % kBufs], w, lane, lb, rb, valid, lat_row_b, rope_row_b);
  };

  // absorbed query as the MFMA B operand (N = heads).
  //  MLA, 16x16x32: lane (head 16*(w>>1) + lane%16, k-group lane/16), K-step j = 32 columns.
  //  MLRA, 32x32x16: lane (head l32, k-half kg), K-step j = 16 columns of branch w / rope.
  constexpr int kQSteps = NB == 1 ? 18 : 12;
  const int tb = w & 1, hb = w >> 1;          // MLA score block: token half, head half
  const int l16 = lane & 15, g16 = lane >> 4;
  bf16x8 qb[kQSteps];
  if (NB == 1) {
    const bf16* qrow = qcat + ((size_t)b * H + h0 + 16 * hb + l16) * kRow + 8 * g16;
#pragma unroll
    for (int j = 0; j < 18; ++j) qb[j] = *(const bf16x8*)(qrow + 32 * j);
  } else {
    const bf16* qrow = qcat + ((size_t)b * H + h0 + l32) * kRow + 8 * kg;
#pragma unroll
    for (int j = 0; j < 8; ++j) qb[j] = *(const bf16x8*)(qrow + 128 * w + 16 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[8 + j] = *(const bf16x8*)(qrow + kDC + 16 * j);
  }

  issue(0);

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 O[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) O[mb] = f32x16{};

  // transposed-read sources of the value operand: rows v_row and v_row + v_delta of each
  // 16-token half, columns 128w + 32mb + v_col (this wave's latent columns)
  const int g = lane >> 4, li = lane & 15;
  const int v_col = 16 * (g & 1) + 4 * (li & 3);
  const int v_row = NB == 1 ? 8 * kg + (li >> 2) : 4 * kg + (li >> 2);
  constexpr int v_delta = NB == 1 ? 4 : 8;
  uint32_t pv_off[2][2][4];  // [half][read][mb]; + 256w for the wave's column block
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        pv_off[s2][r][mb] = lat_piece<Sw32>(16 * s2 + v_row + r * v_delta, 32 * mb + v_col) + 256 * w;

  for (int k = 0; k < n_tiles; ++k) {
    wait_vmcnt<0>();  // with a ring of two, tile k+1 is issued only after tile k landed
    lds_barrier();  // tile k landed for every wave; buffer of tile k-1 is free
    if (k + 1 < n_tiles) issue(k + 1);

    const int t0 = t_begin + kTT * k;
    const int valid = min(kTT, t_end - t0);
    const char* buf = sm.ring[k % kBufs];

    bf16x8 pb[2];
    float alpha;
    if (NB == 1) {
      // ---- scores of 16 tokens x 16 heads over all 576 columns (M = tokens, N = heads)
      f32x4 acc = {};
      {
        // K-step j covers columns 32j..32j+31: chunk 4j + g16 of token t
        const int t = 16 * tb + l16;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              lds_read16(buf + lat_chunk<Sw32>(t, 4 * (j & 3) + g16) + 256 * (j >> 2)), qb[j],
              acc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              lds_read16(buf + rope_chunk(t, 4 * j + g16)), qb[16 + j], acc, 0, 0, 0);
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
      if (g16 == 0) sm.mx[tb * kHG + h] = mx;
      lds_barrier();
      mx = fmaxf(mx, sm.mx[(tb ^ 1) * kHG + h]);  // max over the tile's 32 tokens
      const float m_new = fmaxf(m_run, mx);  // finite: every tile holds a valid token
      const float a = exp2f(m_run - m_new);
      bf16 pe[4];
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = (bf16)exp2f(acc[e] - m_new);
        psum += (float)pe[e];  // normalise with the rounded weights the MFMA uses
      }
      psum = sum_xor32(sum_xor16(psum));
      *(bf16x4*)(&sm.p[h * kPPitch + tq]) = bf16x4{pe[0], pe[1], pe[2], pe[3]};
      if (g16 == 0) {
        sm.sum[tb * kHG + h] = psum;
        if (tb == 0) sm.alpha[h] = a;
      }
      lds_barrier();
      l_run = a * l_run + psum + sm.sum[(tb ^ 1) * kHG + h];
      m_run = m_new;
      alpha = sm.alpha[l32];
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
      const float m_new = fmaxf(m_run, mx);
      alpha = exp2f(m_run - m_new);
      float psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bf16 e = (bf16)exp2f(acc[i] - m_new);
        pb[i >> 3][i & 7] = e;
        psum += (float)e;
      }
      psum = sum_xor32(psum);
      l_run = alpha * l_run + psum;
      m_run = m_new;
    }

    // ---- O^T[d][h] += V^T P^T over this wave's 128 latent columns
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) O[mb] *= alpha;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_pair(buf + pv_off[s2][0][mb], buf + pv_off[s2][1][mb]), pb[s2], O[mb], 0, 0, 0);
  }

  // ---- partial outputs, through LDS so that every global store writes whole rows.  O[mb]
  // item i is column d = 128w + 32mb + 8*(i/4) + 4*kg + i%4 of head l32: written straight
  // out, each store instruction would touch 32 head rows with 16 bytes each.  The waves put
  // the 32 x 512 block (bf16) into the now idle tile ring, then each stores 8 of its 1 KiB
  // rows, one per instruction.
  constexpr int kOutPitch = kDC * 2 + 16;  // LDS bytes per head row (+16: 2-way conflicts)
  static_assert(kHG * kOutPitch <= kBufBytes, "output staging exceeds one ring buffer");
  __syncthreads();  // every wave is done with the ring
  char* stage = sm.ring[0];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(bf16x4*)(stage + l32 * kOutPitch + (128 * w + 32 * mb + 8 * q + 4 * kg) * 2) =
          bf16x4{(bf16)O[mb][4 * q], (bf16)O[mb][4 * q + 1], (bf16)O[mb][4 * q + 2],
                 (bf16)O[mb][4 * q + 3]};
  __syncthreads();
  bf16* po = part_o + (item * H + h0) * kDC + 8 * lane;
#pragma unroll
  for (int j = 0; j < kHG / 4; ++j) {
    const int r = (kHG / 4) * w + j;
    *(bf16x8*)(po + (size_t)r * kDC) = *(const bf16x8*)(stage + r * kOutPitch + 16 * lane);
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
  auto kern = p.NB == 1 ? k_main_bf16<1> : k_main_bf16<4>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, s, (const bf16*)a.qcat,
                     (const bf16*)a.latent, (const bf16*)a.rope, a.lat_tok, a.lat_seq, a.rope_tok,
                     a.rope_seq, a.work, a.block_table, a.bt_stride, p.paged, (bf16*)a.part_o,
                     a.part_ml, p.H, p.n_hg);
  return hipGetLastError();
}

}  // namespace mla
