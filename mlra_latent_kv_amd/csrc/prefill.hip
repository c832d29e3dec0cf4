// Un-absorbed prefill of MLA on gfx950 (bf16 in, fp32 accumulation).
//
// Many new tokens per sequence attend causally over the cache at once.  With that many query
// rows the absorbed form (every query scored over the 576-wide latent row, the 512-wide
// latent summed) costs 1088 multiply-adds per (query, key, head); the un-absorbed form
// up-projects the cached latents once per head to keys K = c W_UK^T (128) and values
// V = c W_UV (128) and then costs 192 + 128 per pair (the interview Q&A "MLA … 是什么",
// 核心机制 step 3, and the compute-heavy regime the yololab MLA page names in
// 繁榮背後的代價).  Two launches:
//
//  * k_prefill_kv: K and V of every (sequence, head, token) into the workspace, B x H x
//    L_pad x 128 each, as one MFMA GEMM [tokens x 512] . [512 x 256] per head, stored as the
//    attention's MFMA operand blocks; it also copies the rotary keys into that form;
//  * k_prefill_attn: per (sequence, head) and two blocks of 256 query tokens, a
//    flash-attention pass over the key tokens up to each block's last position: scores over
//    the 128 key columns plus the cached rotary key (64), online softmax, values summed in
//    registers.
//
// Query token i of a sequence of L tokens sits at position L - s_q + i, its rotary query is
// rotated there, and it sees the tokens up to and including itself; a token that sees none
// writes zeros.  Layouts as the multi-token decode: q_nope [B, s_q, H, 128], q_rope
// [B, s_q, H, 64], out [B, s_q, H, 128].  MLRA-4 ("[ICLR 2025] MLRA…", sections 2.1 and
// 2.2) runs the same two kernels per (head, branch) on each branch's 128-wide latent slice
// and weights (q_nope [B, s_q, H, 4, 128]), and a third launch sums the four normalised
// branch outputs times out_scale.
#include <algorithm>

#include "device_common.h"
#include "launch.h"
#include "tile_bf16.h"

namespace mla {
namespace {

using namespace tile;

constexpr int kPfDc = 512, kPfDn = 128, kPfDv = 128, kPfDr = 64;

// Direct-to-LDS load with the default cache policy.  The decode streams every cached row once
// and loads it non-temporally; the prefill re-reads what it loads (each latent chunk by every
// head, each head's weight chunks by every token block, each key and value tile by the query
// blocks of its head), so its loads stay in the caches: projection 205.7 -> 174.3 us at 128
// heads x 4096 tokens, 93 -> 85 on MLRA-4, same-process A/B on MI355X, outputs bitwise equal.
__device__ __forceinline__ void dma16_keep(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// Workspace layout: operand blocks.  Each 32-token tile of keys, values and rotary keys is
// stored as the MFMA operands the attention feeds, 1 KiB per block, lane i's 8 bf16 at
// 16 i, so the attention loads whole tiles as contiguous KiBs and reads them lane-linearly.
//   keys [B][H][tiles][8 steps j][64]:      lane (t = i % 32, g = i / 32) holds K[t][16 j + 8 g ..]
//   rotary [B][tiles][4 steps m][64]:      rope[t][16 m + 8 g ..] (as cached: already rotated)
//   values [B][H][tiles][2 ks][4 cb][64]:  V[16 ks + 4 g + e % 4 + 8 (e / 4)][32 cb + t],
//                                          e = 0..7 (the score layout's token order)
constexpr int kTileK = kTT * kPfDn * 2, kTileR = kTT * kPfDr * 2, kTileV = kTT * kPfDv * 2;

// ----------------------------------------------------------------------------- K and V
// A tile is (sequence b, block of 256 tokens, head h and latent branch br); one workgroup
// (8 waves, two per SIMD) per CU walks its share of the tiles.  Wave w computes tokens
// 64 (w & 3) .. +63 (two 32-row M blocks) of part w >> 2 (0: K, 1: V), all 128 output
// columns (four 32-column N blocks), MFMA 32x32x16 over the branch's DCB latent columns (512
// for MLA; 128 per MLRA branch, or for one MLRA branch cached on its own) in chunks of 64.
// Each chunk stages, by direct-to-LDS loads, the 256 latent rows (128 bytes of each),
// W_UK[h]'s 128 rows (their columns of the chunk) and W_UV[h]'s 64 rows of the chunk (256
// bytes each); double-buffered, so one chunk's 64 MFMAs per SIMD cover the next one's loads,
// and the next tile's first chunk loads during the current tile's output phase.
constexpr int kKvTok = 256, kKvChunk = 64, kKvWaves = 8;
constexpr int kKvABytes = kKvTok * kKvChunk * 2;     // 32 KiB
constexpr int kKvBkBytes = kPfDn * kKvChunk * 2;     // 16 KiB
constexpr int kKvBvBytes = kKvChunk * kPfDv * 2;     // 16 KiB
constexpr int kKvStage = kKvABytes + kKvBkBytes + kKvBvBytes;
constexpr int kKvLoads = kKvStage / 1024;            // 1 KiB loads per stage: 64
constexpr int kKvIssues = kKvLoads / kKvWaves;       // per wave: 8

// 128-byte rows (8 chunks, two rows per 256-byte bank line): chunk c of row r sits at
// c ^ ((r / 2) mod 8), so 16 consecutive rows read at one chunk hit 16 distinct slots
__device__ __forceinline__ uint32_t row128(int r, int c) {
  return (uint32_t)(r * 128 + 16 * (c ^ ((r >> 1) & 7)));
}

// Output tile of one part, staged for the operand-block stores: 256 rows at a 320-byte pitch
// (values; keys use 272), from the start of stage 1 on, so stage 0 can take the next tile's
// first chunk meanwhile.
constexpr int kKvOutBytes = kKvTok * (2 * kPfDv + 64);

// One bf16 into LDS through a restrict pointer: the access then carries alias-scope
// information, so the compiler does not wait for the direct-to-LDS loads in flight into the
// other stage before it.
__device__ __forceinline__ void lds_write2(char* __restrict__ p, bf16 v) { *(bf16*)p = v; }

// A workgroup's unit of work: 256 tokens of one (sequence, head and branch hb = h NB + br).
struct KvTile {
  int b, hb, t0, L;
};

template <int DCB>
__global__ __launch_bounds__(64 * kKvWaves, 1) void k_prefill_kv(
    const bf16* __restrict__ latent, int64_t lat_tok, int64_t lat_seq,
    const bf16* __restrict__ rope, int64_t rope_tok, int64_t rope_seq,
    const int32_t* __restrict__ bt, int64_t bt_stride, int paged,
    const int32_t* __restrict__ seqlens, int max_seqlen, const bf16* __restrict__ w_uk,
    const bf16* __restrict__ w_uv, bf16* __restrict__ kout, bf16* __restrict__ rout,
    bf16* __restrict__ vout, int B, int H, int NB, int L_pad) {
  struct Smem {
    char st[2][kKvStage];
    char out_tail[kKvOutBytes - kKvStage];  // the output tile runs on from stage 1 into this
  };
  __shared__ __align__(16) Smem sm;  // 144 KiB
  constexpr int dcb = DCB, n_chunks = dcb / kKvChunk;  // latent columns of a branch
  static_assert(n_chunks % 2 == 0, "every tile's first chunk goes to stage 0");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lat_row_b = (uint32_t)(lat_tok * 2);
  // tiles in (sequence, head, branch, token block) order, token block fastest; workgroup g
  // takes tiles g, g + G, g + 2G, ...: the workgroups of one XCD keep to the same few token
  // blocks, whose latent rows stay in its L2 while the heads' weights stream past
  const int n_tb = L_pad / kKvTok, HNB = H * NB;
  const int n_tiles = B * HNB * n_tb;  // below 2^31 (the plan checks)
  auto tile_at = [&](int n) {
    KvTile t;
    const int r = n / n_tb;
    t.t0 = (n - r * n_tb) * kKvTok;
    t.b = r / HNB;
    t.hb = r - t.b * HNB;
    t.L = min(max(seqlens[t.b], 0), max_seqlen);
    return t;
  };

  // chunk q of tile tl into stage q % 2, 64 loads of one KiB, 8 per wave: waves 0-3 the 256
  // latent rows (8 rows a load), waves 4-5 W_UK's 128 rows (8 a load), waves 6-7 W_UV's 64
  // rows (4 a load); rows past the sequence read as zeros (the descriptor ends at its last
  // token)
  auto issue = [&](const KvTile& tl, int q, bool live) {
    char* s = sm.st[q & 1];
    const int h = tl.hb / NB, br = tl.hb - h * NB;
    // W_UK [NB][H][128][dcb] and W_UV [NB][H][dcb][128]: the (branch, head) blocks
    const bf16* wk = w_uk + ((size_t)br * H + h) * kPfDn * dcb;
    const bf16* wv = w_uv + ((size_t)br * H + h) * dcb * kPfDv;
    const uint32_t col0_b = (uint32_t)(br * dcb * 2);  // the branch's first latent byte in a row
    const uint32_t on = live ? ~0u : 0u;  // a dead issue: empty descriptors, zeros, no reads
    if (w < 4) {  // waves 0-3: latent rows
#pragma unroll
      for (int u = 0; u < kKvIssues; ++u) {
        const int r0 = 8 * (kKvIssues * w + u), t = tl.t0 + r0;  // 8 rows of one page
        const int valid = max(0, min(8, tl.L - t));
        const bf16* base;
        if (paged) {
          const int tt = min(t, max(tl.L - 1, 0));
          const int64_t pg = valid > 0 ? bt[(int64_t)tl.b * bt_stride + tt / kPage] : 0;
          base = latent + pg * lat_seq + (int64_t)(tt % kPage) * lat_tok;
        } else {
          base = latent + (int64_t)tl.b * lat_seq + (int64_t)t * lat_tok;
        }
        const int vu = __builtin_amdgcn_readfirstlane(valid);
        const int r = lane >> 3, c = lane & 7;
        dma16_keep(rsrc(base, (vu * lat_row_b) & on), s + r0 * 128,
              r * lat_row_b + col0_b + q * 128 + 16 * (c ^ (((r0 + r) >> 1) & 7)));
      }
    } else if (w < 6) {  // waves 4-5: W_UK rows
      const auto rk = rsrc(wk, (kPfDn * dcb * 2) & on);
#pragma unroll
      for (int u = 0; u < kKvIssues; ++u) {
        const int r0 = 8 * (kKvIssues * (w - 4) + u), r = r0 + (lane >> 3), c = lane & 7;
        dma16_keep(rk, s + kKvABytes + r0 * 128, r * (dcb * 2) + q * 128 + 16 * (c ^ ((r >> 1) & 7)));
      }
    } else {  // waves 6-7: W_UV rows
      const auto rv = rsrc(wv, (dcb * kPfDv * 2) & on);
#pragma unroll
      for (int u = 0; u < kKvIssues; ++u) {
        const int r0 = 4 * (kKvIssues * (w - 6) + u), r = r0 + (lane >> 4), c = lane & 15;
        dma16_keep(rv, s + kKvABytes + kKvBkBytes + r0 * 256,
              (q * kKvChunk + r) * (kPfDv * 2) + 16 * (c ^ lat_sw<Sw32>(r)));
      }
    }
  };

  const int g = blockIdx.x, G = gridDim.x;
  if (g >= n_tiles) return;

  // the rotary keys of every (sequence, 256-token block) go into the workspace as operand
  // blocks first, workgroup g taking blocks g, g + G, ...: thread tid, pieces tid + 512 u =
  // (tile, step m, lane i) in order; zeros past the sequence
  for (int rb = g; rb < B * n_tb; rb += G) {
    const int b = rb / n_tb, t0 = (rb - b * n_tb) * kKvTok;
    const int L = min(max(seqlens[b], 0), max_seqlen);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = tid + 512 * u;
      const int tl = pc >> 8, m = (pc >> 6) & 3, i = pc & 63;
      const int t = t0 + kTT * tl + (i & 31);
      bf16x8 v = bf16x8{};
      if (t < L) {
        const bf16* row = paged ? rope + (int64_t)bt[(int64_t)b * bt_stride + t / kPage] * rope_seq +
                                      (int64_t)(t % kPage) * rope_tok
                                : rope + (int64_t)b * rope_seq + (int64_t)t * rope_tok;
        v = *(const bf16x8*)(row + 16 * m + 8 * (i >> 5));
      }
      *(bf16x8*)(rout + ((size_t)b * L_pad + t0) * kPfDr + 8 * (size_t)pc) = v;
    }
  }

  const int mq = w & 3, part = w >> 2;
  const int l32 = lane & 31, kg = lane >> 5, G16 = lane >> 4, li = lane & 15;
  issue(tile_at(g), 0, true);
  for (int n = g; n < n_tiles; n += G) {
    const KvTile cur = tile_at(n);

    f32x16 acc[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16{};
    for (int q = 0; q < n_chunks; ++q) {
      // chunk q + 1 of this tile, or the next tile's chunk 0 (stage 0, whose chunk is done),
      // goes out before chunk q is waited for; after the last tile a dead issue keeps the
      // count
      {
        const bool last = q + 1 == n_chunks;
        const int nn = last ? n + G : n;
        issue(nn == n ? cur : tile_at(min(nn, n_tiles - 1)), last ? 0 : q + 1, nn < n_tiles);
      }
      wait_vmcnt<kKvIssues>();  // chunk q has landed for this wave
      lds_barrier();  // ... and for every wave
      const char* s = sm.st[q & 1];
#pragma unroll
      for (int j = 0; j < kKvChunk / 16; ++j) {
        bf16x8 a[2], bo[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int r = 64 * mq + 32 * mb + l32;
          a[mb] = lds_read16(s + row128(r, 2 * j + kg));
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          if (part == 0) {  // W_UK rows n: 8 consecutive latent columns of row n
            bo[nb] = lds_read16(s + kKvABytes + row128(32 * nb + l32, 2 * j + kg));
          } else {          // W_UV rows c: column v, 8 consecutive rows, two transposed reads
            const int col = 32 * nb + 16 * (G16 & 1) + 4 * (li & 3);
            const int r1 = 16 * j + 8 * (G16 >> 1) + (li >> 2);
            const char* bv = s + kKvABytes + kKvBkBytes;
            bo[nb] = tr_pair(bv + lat_piece<Sw32, 128>(r1, col), bv + lat_piece<Sw32, 128>(r1 + 4, col));
          }
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb], bo[nb], acc[mb][nb], 0, 0, 0);
      }
      lds_barrier();  // every wave is done with this stage before it is refilled
    }

    // ---- output: each part's 256 x 128 tile through LDS in turn (from stage 1 on), then
    // whole operand blocks (1 KiB of contiguous workspace per wave and store), while the next
    // tile's first chunk lands in stage 0 (LDS-only barriers, so its loads stay in flight).  D layout:
    // lane (column l32 of N block nb, half kg), item i -> token 8 (i / 4) + 4 kg + i % 4 of the
    // M block.  Row pitches: 272 bytes for the keys (16 rows at one 16-byte column hit 16
    // distinct bank slots), 320 for the values (the transposed reads' 4 rows x 64 bytes per
    // half-wave are distinct).
    constexpr int kPitchK = 2 * kPfDn + 16, kPitchV = 2 * kPfDv + 64;
    static_assert(kKvTok * kPitchV == kKvOutBytes, "output tile size");
    char* o = sm.st[1];
    const size_t head_tok = ((size_t)cur.b * HNB + cur.hb) * L_pad + cur.t0;  // block's first token
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      const int pitch = pt == 0 ? kPitchK : kPitchV;
      if (part == pt) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int t = 64 * mq + 32 * mb + 8 * (i >> 2) + 4 * kg + (i & 3);
              lds_write2(o + t * pitch + 2 * (32 * nb + l32), (bf16)acc[mb][nb][i]);
            }
      }
      lds_barrier();
      // 8 tiles x 8 blocks: wave w writes blocks 8 w .. 8 w + 7 (tile w), lane by lane
      bf16* dst = (pt == 0 ? kout : vout) + head_tok * kPfDv + (size_t)w * (kTT * kPfDv);
      const char* ot = o + kTT * w * pitch;  // the wave's tile
#pragma unroll
      for (int bi = 0; bi < 8; ++bi) {
        bf16x8 v;
        if (pt == 0) {  // key step bi: token l32, columns 16 bi + 8 kg ..
          v = lds_read16(ot + l32 * kPitchK + 2 * (16 * bi + 8 * kg));
        } else {        // value block (ks, cb) = (bi / 4, bi % 4): two transposed 4-row reads
          const int ks = bi >> 2, cb = bi & 3;
          const int tr = 16 * ks + 4 * kg + (li >> 2), col = 32 * cb + 16 * (G16 & 1) + 4 * (li & 3);
          v = tr_pair(ot + tr * kPitchV + 2 * col, ot + (tr + 8) * kPitchV + 2 * col);
        }
        *(bf16x8*)(dst + 8 * (64 * bi + lane)) = v;
      }
      lds_barrier();
    }
  }
  wait_vmcnt<0>();  // the dead issue's LDS writes, before the workgroup's LDS is released
}

// ----------------------------------------------------------------------------- attention
// One workgroup (8 waves, two per SIMD) per (sequence b, head h, pair of 256-token query
// blocks); wave w holds query tokens i0 + 32w .. +31 (MFMA N = rows).  Each key tile of 32
// tokens crosses into LDS once for all 256 rows, through a ring of six 20 KiB buffers: the
// tile's 20 operand blocks exactly as the workspace stores them (8 key steps, 4 rotary
// steps, 8 value blocks), so every load is 1 KiB of contiguous memory and every LDS read is a
// lane-linear 16-byte read at one per-tile base address plus a constant.  Per tile and wave:
// S^T = K . Q^T (12 MFMAs), causal mask on the diagonal tiles, online softmax with a lazy max
// (raised only past kAtLazy log2 units), O^T += V^T P^T (8 MFMAs).
constexpr int kAtWaves = 8;
constexpr int kAtRows = 32 * kAtWaves;
constexpr int kAtRing = 6;
constexpr float kAtLazy = 8.0f;
constexpr int kAtROff = kTileK;                 // rotary blocks after the 8 key blocks
constexpr int kAtVOff = kTileK + kTileR;        // value blocks after them
constexpr int kAtBuf = kTileK + kTileR + kTileV;  // 20 KiB
// loads per wave and tile: key block w, value block w, and for waves 0-3 rotary block w
constexpr int kAtIssuesLo = 3, kAtIssuesHi = 2;

// wait until this wave has at most `younger` tiles' loads out beyond the one it needs
template <int Younger>
__device__ __forceinline__ void wait_tiles(int w) {
  if (w < 4)
    wait_vmcnt<Younger * kAtIssuesLo>();
  else
    wait_vmcnt<Younger * kAtIssuesHi>();
}

__global__ __launch_bounds__(64 * kAtWaves, 1) void k_prefill_attn(
    const bf16* __restrict__ q_nope, const bf16* __restrict__ q_rope,
    const int32_t* __restrict__ seqlens, int max_seqlen, const bf16* __restrict__ kbuf,
    const bf16* __restrict__ rbuf, const bf16* __restrict__ vbuf, bf16* __restrict__ out,
    bf16* __restrict__ obr, int B, int H, int NB, int sq, int L_pad, float qscale,
    float out_scale, RopeFreq rf) {
  struct Smem {
    char ring[kAtRing][kAtBuf];
  };
  __shared__ __align__(1024) Smem sm;  // 120 KiB
  // Causal balance: a workgroup takes query blocks n_qb - 1 - j and j of one (b, h), the
  // heavy one first, so every workgroup scans about n_qb + 1 blocks' worth of key tiles
  // (a lone middle block when n_qb is odd).  XCD-aware order: blocks go round-robin over the
  // 8 XCDs, so block 8r + x is the r-th one XCD x runs; each XCD takes whole (b, h) in turn,
  // all workgroups of one back to back: they read the same key and value tiles in the same
  // order, and started together they find most tiles in that XCD's L2.
  const int n_qb = (sq + kAtRows - 1) / kAtRows;
  const int n_wg = (n_qb + 1) / 2;
  const int x = blockIdx.x & 7, r = blockIdx.x >> 3;
  const int HB = H * NB;                    // (head, branch) pairs: hb = h NB + br
  const int bh = (r / n_wg) * 8 + x;
  if (bh >= B * HB) return;  // padding of the grid to whole groups of eight pairs
  const int jb = r % n_wg;
  const int b = bh / HB, hb = bh % HB, h = hb / NB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, kg = lane >> 5;
  const int L = min(max(seqlens[b], 0), max_seqlen);
  const char* kb = reinterpret_cast<const char*>(kbuf + ((size_t)b * HB + hb) * L_pad * kPfDn);
  const char* vb = reinterpret_cast<const char*>(vbuf + ((size_t)b * HB + hb) * L_pad * kPfDv);
  const char* rb = reinterpret_cast<const char*>(rbuf + (size_t)b * L_pad * kPfDr);
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  // a lane's operand in any block of ring buffer k: one register per tile, constants after
  const uint32_t lane_b = lds_addr(sm.ring[0]) + 16 * lane;
  auto slot = [&](int k) { return opaque(lane_b + (uint32_t)(k % kAtRing) * kAtBuf); };

  for (int pass = 0; pass < 2; ++pass) {
    const int qb = pass == 0 ? n_qb - 1 - jb : jb;
    if (pass == 1 && qb == n_qb - 1 - jb) break;  // the lone middle block
    const int i0 = qb * kAtRows;
    const int iw = i0 + 32 * w;                 // this wave's first query token
    const int ir = iw + l32;                    // this lane's query token (row)
    const int pos = L - sq + ir;                // its position (< 0: sees nothing)
    const int pos_w = L - sq + iw + 31;         // the wave's last position
    const int pos_g = min(L - sq + i0 + kAtRows - 1, L - 1);  // the block's last position
    const int n_tiles = pos_g >= 0 ? pos_g / kTT + 1 : 0;

    // tile k into its ring buffer: 1 KiB blocks, lane i's 16 bytes at 16 i.  Past n_tiles the
    // loads go out with an empty range (zeros, no memory touched) so that every wave issues
    // the same count and every wait is fixed.
    auto issue = [&](int k) {
      char* buf = sm.ring[k % kAtRing];
      const uint32_t n = k < n_tiles ? 1u : 0u;
      const size_t t = (size_t)k;
      dma16_keep(rsrc(kb + t * kTileK, n * kTileK), buf + w * 1024, w * 1024 + 16 * lane);
      dma16_keep(rsrc(vb + t * kTileV, n * kTileV), buf + kAtVOff + w * 1024, w * 1024 + 16 * lane);
      if (w < 4)
        dma16_keep(rsrc(rb + t * kTileR, n * kTileR), buf + kAtROff + w * 1024, w * 1024 + 16 * lane);
    };

    // query as the B operand (K = 192 columns, N = 32 rows): lane (row l32, half kg), K-step j
    // holds columns 16 j + 8 kg .. +7; the rotary steps 8 .. 11 rotated at the row's position;
    // scaled by softmax_scale * log2(e).  Rows past s_q load row s_q - 1 and are not stored.
    bf16x8 qb8[12];
    {
      // q_nope [B][s_q][H][NB][128] holds the branch's query at (head, branch) row hb;
      // q_rope [B][s_q][H][64] is shared by the branches of a head
      const int irc = min(ir, sq - 1);
      const size_t tok = (size_t)b * sq + irc;
      const bf16* qn = q_nope + (tok * HB + hb) * kPfDn + 8 * kg;
      const bf16* qr = q_rope + (tok * H + h) * kPfDr + 8 * kg;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 v = *(const bf16x8*)(qn + 16 * j);
#pragma unroll
        for (int e = 0; e < 8; ++e) qb8[j][e] = (bf16)((float)v[e] * qscale);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 v = *(const bf16x8*)(qr + 16 * j);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int k = (16 * j + 8 * kg + e) >> 1;  // rotation pair
          float cs, sn;
          rope_cos_sin(max(pos, 0), rf.f[k], &cs, &sn);
          const float x0 = (float)v[e], x1 = (float)v[e + 1];
          qb8[8 + j][e] = (bf16)((x0 * cs - x1 * sn) * qscale);
          qb8[8 + j][e + 1] = (bf16)((x0 * sn + x1 * cs) * qscale);
        }
      }
    }

    float m_ref = -INFINITY, l_run = 0.0f;
    f32x16 O[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) O[cb] = f32x16{};
    // tiles this wave needs (through its last position), and the limit of the causal mask:
    // a tile starting at t0 needs the mask iff t0 + kTT - 1 > lim (the wave's first position)
    const int n_w = pos_w >= 0 ? min(pos_w, L - 1) / kTT + 1 : 0;
    const int lim = L - sq + iw;

    // operand j of a tile: key steps 0-7, rotary steps 8-11
    auto key_op = [&](uint32_t sb, int j) {
      return lds_read16_at(sb + (j < 8 ? 1024 * j : kAtROff + 1024 * (j - 8)));
    };
    // causal mask: token t0 + 8 (i / 4) + 4 kg + i % 4 is seen by rows at positions >= it
    auto mask = [&](f32x16& S, int t0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = t0 + 8 * (i >> 2) + 4 * kg + (i & 3);
        S[i] = t <= pos ? S[i] : -INFINITY;
      }
    };
    // a tile's row max into the running max (mx = -inf: the tile adds nothing); the max is
    // raised lazily, only past kAtLazy log2 units, and the first tile a row sees sets it; O
    // and l are rescaled when any row of the wave raised
    auto take_max = [&](float mx) {
      const bool raise = mx > m_ref + kAtLazy || (m_ref == -INFINITY && mx != -INFINITY);
      float alpha = 1.0f;
      if (raise) {
        const float m_new = fmaxf(m_ref, mx);
        alpha = m_ref == -INFINITY ? 0.0f : exp2f(m_ref - m_new);
        m_ref = m_new;
      }
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) O[cb] *= alpha;
        l_run *= alpha;
      }
    };
    auto row_max = [&](const f32x16& S) {
      float mx = S[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, S[i]);
      return max_xor32(mx);
    };

#pragma unroll
    for (int j = 0; j < kAtRing - 1; ++j) issue(j);
    wait_tiles<kAtRing - 2>(w);  // tile 0 has landed for this wave ...
    lds_barrier();               // ... and for every wave
    f32x16 S = f32x16{};
    if (n_w > 0) {
      const uint32_t s0 = slot(0);
#pragma unroll
      for (int j = 0; j < 12; ++j)
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(key_op(s0, j), qb8[j], S, 0, 0, 0);
      if (kTT - 1 > lim) mask(S, 0);
      take_max(row_max(S));
    }
    // Software pipeline, one tile deep: iteration k scores tile k + 1 while it turns tile k's
    // scores (in S, their max already taken) into weights, then sums tile k's values.  The
    // code below is in issue order, fenced in small groups: each score MFMA goes out with the
    // key read two steps ahead and the arithmetic of one weight pair (or the value reads), so
    // the matrix core and the vector ALU work side by side.
    for (int k = 0; k < n_tiles; ++k) {
      wait_tiles<kAtRing - 3>(w);  // tile k + 1 has landed for this wave ...
      lds_barrier();  // ... and for every wave, which are all done with tile k - 1's buffer
      issue(k + kAtRing - 1);
      if (k >= n_w) continue;  // every row of the wave is before this tile (uniform)
      const uint32_t bk = slot(k), bn = slot(k + 1);
      const int tn = kTT * (k + 1);
      const float m_off = m_ref == -INFINITY ? 0.0f : m_ref;  // 0 while nothing was seen
      __builtin_amdgcn_sched_barrier(0);

      f32x16 Sn = f32x16{};
      bf16x8 kq[12], vop[8];
      uint32_t pw[8];
      float psum = 0.0f;
      kq[0] = key_op(bn, 0);
      kq[1] = key_op(bn, 1);
#pragma unroll
      for (int j = 0; j < 12; ++j) {
        if (j + 2 < 12) kq[j + 2] = key_op(bn, j + 2);
        Sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[j], qb8[j], Sn, 0, 0, 0);
        if (j < 8) {
          // weights of tile k's tokens 2j, 2j + 1 of the lane: bf16 pairs in the value
          // operand's token order, summed as the MFMA uses them
          const bf16x2 p = __builtin_convertvector(
              f32x2{__builtin_amdgcn_exp2f(S[2 * j] - m_off),
                    __builtin_amdgcn_exp2f(S[2 * j + 1] - m_off)},
              bf16x2);
          pw[j] = __builtin_bit_cast(uint32_t, p);
          psum = __builtin_amdgcn_fdot2_f32_bf16(p, ones, psum, false);
        } else {
          vop[2 * (j - 8)] = lds_read16_at(bk + kAtVOff + 1024 * (2 * (j - 8)));
          vop[2 * (j - 8) + 1] = lds_read16_at(bk + kAtVOff + 1024 * (2 * (j - 8) + 1));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run += sum_xor32(psum);
      // tile k + 1's causal mask, diagonal tiles only (a uniform branch)
      if (tn + kTT - 1 > lim) mask(Sn, tn);
      // O^T[d][row] += V^T P^T: value block 4 ks + cb holds columns 32 cb .. +31 of the
      // 16-token step ks; the weights' token order matches its rows
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pb =
            __builtin_bit_cast(bf16x8, u32x4{pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2],
                                             pw[4 * ks + 3]});
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[4 * ks + cb], pb, O[cb], 0, 0, 0);
      }
      // past n_w the scores of tile k + 1 are not used
      take_max(k + 1 < n_w ? row_max(Sn) : -INFINITY);
      S = Sn;
    }
    // no tile load is still in flight when the block ends (the ring refills for the next one,
    // or the workgroup ends), and every wave is done reading the ring
    wait_vmcnt<0>();
    lds_barrier();

    // out[row][d] = out_scale * O / l (MLA), or the branch's O / l into the branch outputs
    // (MLRA, bf16, summed in fp32 and scaled by the next launch); O^T item e of block cb:
    // column 32 cb + 8 (e / 4) + 4 kg + e % 4 of row l32
    if (ir < sq) {
      const float inv = l_run > 0.0f ? (NB == 1 ? out_scale : 1.0f) / l_run : 0.0f;
      bf16* orow = NB == 1 ? out + (((size_t)b * sq + ir) * H + h) * kPfDv
                           : obr + (((size_t)b * sq + ir) * HB + hb) * kPfDv;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(bf16x4*)(orow + 32 * cb + 8 * q + 4 * kg) =
              bf16x4{(bf16)(O[cb][4 * q] * inv), (bf16)(O[cb][4 * q + 1] * inv),
                     (bf16)(O[cb][4 * q + 2] * inv), (bf16)(O[cb][4 * q + 3] * inv)};
    }
  }
}

// ----------------------------------------------------------------------------- branch sum
// MLRA: out[b][i][h] = out_scale * sum over branches of the branch outputs (each already
// normalised by its own softmax sum), summed in fp32 and rounded once to bf16.  One thread
// per 8 columns.
__global__ __launch_bounds__(256) void k_prefill_branch_sum(const bf16* __restrict__ obr,
                                                            bf16* __restrict__ out, int NB,
                                                            int64_t rows, float out_scale) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, 8-column piece)
  if (i >= rows * (kPfDv / 8)) return;
  const int64_t row = i / (kPfDv / 8);
  const int c = (int)(i % (kPfDv / 8)) * 8;
  float acc[8] = {};
  for (int br = 0; br < NB; ++br) {
    const bf16x8 v = *(const bf16x8*)(obr + (row * NB + br) * kPfDv + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (float)v[e];
  }
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)(acc[e] * out_scale);
  *(bf16x8*)(out + row * kPfDv + c) = v;
}

}  // namespace

hipError_t launch_prefill(const PrefillPlan& p, const PrefillArgs& a, hipStream_t s,
                          void* const* events) {
  auto mark = [&](int i) {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), s) : hipSuccess;
  };
  hipError_t e = mark(0);
  if (e != hipSuccess) return e;
  const int64_t kv_tiles = (int64_t)p.B * p.H * p.NB * (p.L_pad / kKvTok);
  const unsigned kv_wg = (unsigned)std::min<int64_t>(kv_tiles, p.n_cu);  // one per CU
  hipLaunchKernelGGL(p.dcb == 512 ? k_prefill_kv<512> : k_prefill_kv<128>, dim3(kv_wg),
                     dim3(64 * kKvWaves), 0, s,
                     (const bf16*)a.latent, a.lat_tok, a.lat_seq, (const bf16*)a.rope,
                     a.rope_tok, a.rope_seq, a.block_table, a.bt_stride, p.paged, a.seqlens,
                     p.max_seqlen, (const bf16*)a.w_uk, (const bf16*)a.w_uv, (bf16*)a.kbuf,
                     (bf16*)a.rbuf, (bf16*)a.vbuf, p.B, p.H, p.NB, p.L_pad);
  e = hipGetLastError();
  if (e == hipSuccess) e = mark(1);
  if (e != hipSuccess) return e;
  RopeFreq rf;
  make_rope_freq(kPfDr, a.rope_theta, &rf);
  const int n_wg = ((p.sq + kAtRows - 1) / kAtRows + 1) / 2;  // workgroups per (b, h)
  const int64_t groups = ((int64_t)p.B * p.H * p.NB + 7) / 8;  // (b, h, branch) in eights
  hipLaunchKernelGGL(k_prefill_attn, dim3((unsigned)(groups * 8 * n_wg)), dim3(64 * kAtWaves), 0,
                     s, (const bf16*)a.q_nope, (const bf16*)a.q_rope, a.seqlens, p.max_seqlen,
                     (const bf16*)a.kbuf, (const bf16*)a.rbuf, (const bf16*)a.vbuf,
                     (bf16*)a.out, (bf16*)a.obuf, p.B, p.H, p.NB, p.sq, p.L_pad,
                     a.softmax_scale * kLog2e, a.out_scale, rf);
  e = hipGetLastError();
  if (e == hipSuccess && p.NB > 1) {
    const int64_t rows = (int64_t)p.B * p.sq * p.H;
    const int64_t pieces = rows * (kPfDv / 8);
    hipLaunchKernelGGL(k_prefill_branch_sum, dim3((unsigned)((pieces + 255) / 256)), dim3(256),
                       0, s, (const bf16*)a.obuf, (bf16*)a.out, p.NB, rows, a.out_scale);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = mark(2);
  return e;
}

}  // namespace mla
