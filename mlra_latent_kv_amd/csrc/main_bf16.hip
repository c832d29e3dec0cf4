// Split-K main loop of the absorbed MLA / MLRA-4 decode step for gfx950 (bf16 in, fp32 acc).
//
// Work item = (sequence b, sequence split s, group of 32 heads).  The workgroup streams the
// split's cached rows [c_KV (512) | k_rope (64)] in 64-token tiles (one page each) through
// LDS and, per tile:
//   S  = q_cat . tile^T       scores of 32 heads x 64 tokens (MFMA 32x32x16 bf16)
//   online softmax            running max / sum per head (per branch for MLRA-4)
//   O += P . tile[:, :512]    latent-space output (MFMA 32x32x16 bf16, operands from LDS
//                             transpose reads)
// and finally writes its partial (m, l, O) for the combine kernel.  This is the absorbed
// form of the yololab page (section 矩陣吸收): all heads share the one cached latent, so
// each tile is a dense [heads x 576] . [576 x tokens] contraction and the latent also serves
// as the value operand.  For MLRA-4 ("[ICLR 2025] MLRA…", section 2.1) the latent holds four
// 128-wide branches with independent softmaxes; the rotary score is shared by them.
//
// Wave w (of 4) owns latent columns [128w, 128w+128) (= branch w for MLRA-4) and rotary
// columns [512+16w, 512+16w+16):
//   * QK: it computes the partial score of its columns for all 32 heads x 64 tokens; the
//     four partials meet in LDS and every wave forms the full scores of the heads.
//   * PV: it accumulates O^T[d][h] for its 128 latent columns, reading the value operand
//     with ds_read_b64_tr_b16 straight from the token-major tile.
#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int kT = 64;                              // tokens per tile (one page)
constexpr int kHG = kHeadGroup;                     // heads per workgroup
constexpr int kThreads = 256;                       // 4 waves
constexpr int kDC = 512, kDR = 64, kRow = kDC + kDR;
constexpr int kChunks = kRow / 8;                   // 16-byte chunks per row (72)
constexpr int kLatChunks = kDC / 8;                 // 64
constexpr int kLoads = kT * kChunks / kThreads;     // 16-byte loads per thread per tile (18)
constexpr int kKPitch = kRow + 8;                   // LDS row pitch, bf16 elements (1168 B)
constexpr int kSPitch = kT + 4;                     // LDS score row pitch, floats

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int NB>
struct Smem {
  bf16 k[kT * kKPitch];                             // current tile, token-major
  float s[NB == 1 ? 4 : 8][kHG * kSPitch];          // per-wave partial scores [h][t]
};

__device__ __forceinline__ bf16x8 tr_pair(const bf16* p) {
  // two 4-row transposed reads: rows r..r+3 and r+4..r+7 of the same 16 columns
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * kKPitch));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <int NB>
__global__ __launch_bounds__(kThreads, 1) void k_main_bf16(
    const bf16* __restrict__ qcat, const bf16* __restrict__ latent,
    const bf16* __restrict__ rope, int64_t lat_tok, int64_t lat_seq, int64_t rope_tok,
    int64_t rope_seq, const int32_t* __restrict__ seqlens, const int32_t* __restrict__ bt,
    int64_t bt_stride, int paged, float* __restrict__ part_o, float* __restrict__ part_ml, int H,
    int S, int chunk, int n_hg, int units) {
  __shared__ __align__(16) Smem<NB> sm;

  // XCD-aware mapping: consecutive blocks go to different XCDs, so the head groups of one
  // (sequence, split) are placed 8 blocks apart -> same XCD, dispatched back to back, and
  // their repeated reads of the same tiles can hit that XCD's L2.
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r = bid >> 3;
  const int hg = r % n_hg;
  const int unit = (r / n_hg) * 8 + xcd;
  if (unit >= units) return;
  const int b = unit / S, s = unit % S;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lh = lane & 31, kg = lane >> 5;
  const int h0 = hg * kHG;
  const int L = seqlens[b];
  const int t_begin = s * chunk;
  const int t_end = min(L, t_begin + chunk);
  float* ml = part_ml + ((size_t)b * S + s) * NB * H * 2;  // [br][H][2]

  if (t_begin >= t_end) {
    if (tid < NB * kHG) {
      const int br = tid / kHG, hh = tid % kHG;
      ml[((size_t)br * H + h0 + hh) * 2 + 0] = -INFINITY;
      ml[((size_t)br * H + h0 + hh) * 2 + 1] = 0.0f;
    }
    return;
  }

  // absorbed query of this wave's columns: A operand, lane (head lh, k-group kg)
  bf16x8 qa[9];
  {
    const bf16* qrow = qcat + ((size_t)b * H + h0 + lh) * kRow + 8 * kg;
#pragma unroll
    for (int j = 0; j < 8; ++j) qa[j] = *(const bf16x8*)(qrow + 128 * w + 16 * j);
    qa[8] = *(const bf16x8*)(qrow + kDC + 16 * w);
  }

  u32x4 stage[kLoads];
  auto load_tile = [&](int t0) {
    const bf16* lb;
    const bf16* rb;
    if (paged) {
      const int64_t pg = bt[(int64_t)b * bt_stride + t0 / kT];
      lb = latent + pg * lat_seq;
      rb = rope + pg * rope_seq;
    } else {
      lb = latent + (int64_t)b * lat_seq + (int64_t)t0 * lat_tok;
      rb = rope + (int64_t)b * rope_seq + (int64_t)t0 * rope_tok;
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int c = tid + kThreads * j;
      const int row = c / kChunks, col = c % kChunks;
      const bf16* src = col < kLatChunks ? lb + row * lat_tok + col * 8
                                         : rb + row * rope_tok + (col - kLatChunks) * 8;
      stage[j] = t0 + row < t_end ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 O[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) O[mb] = f32x16{};

  // transpose-read coordinates for the PV value operand (see tr_pair)
  const int g = lane >> 4, li = lane & 15;
  const int tr_row = 8 * (g >> 1) + (li >> 2);
  const int tr_col = 128 * w + 16 * (g & 1) + 4 * (li & 3);

  load_tile(t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += kT) {
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int c = tid + kThreads * j;
      *(u32x4*)(sm.k + (c / kChunks) * kKPitch + (c % kChunks) * 8) = stage[j];
    }
    if (t0 + kT < t_end) load_tile(t0 + kT);  // prefetch the next tile into registers
    __syncthreads();

    // ---- partial scores of this wave's columns: S[h][t], M = heads, N = tokens
    f32x16 acc[2], accr[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      acc[nb] = f32x16{};
      accr[nb] = f32x16{};
      const bf16* krow = sm.k + (32 * nb + lh) * kKPitch + 8 * kg;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 kb = *(const bf16x8*)(krow + 128 * w + 16 * j);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[j], kb, acc[nb], 0, 0, 0);
      }
      const bf16x8 kb = *(const bf16x8*)(krow + kDC + 16 * w);
      if (NB == 1)
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[8], kb, acc[nb], 0, 0, 0);
      else
        accr[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[8], kb, accr[nb], 0, 0, 0);
    }
    // D layout: lane (token lh, half kg), item i -> head 8*(i/4) + 4*kg + i%4
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = 8 * (i >> 2) + 4 * kg + (i & 3);
        sm.s[w][h * kSPitch + 32 * nb + lh] = acc[nb][i];
        if (NB == 4) sm.s[4 + w][h * kSPitch + 32 * nb + lh] = accr[nb][i];
      }
    __syncthreads();

    // ---- online softmax; lane (head lh, half kg) holds tokens 16*s4 + 8*kg + i
    float v[4][8];
    float mx = -INFINITY;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int tt = 16 * s4 + 8 * kg;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        f32x4 x;
        if (NB == 1) {
          x = *(const f32x4*)(&sm.s[0][lh * kSPitch + tt + 4 * q]);
#pragma unroll
          for (int sl = 1; sl < 4; ++sl) x += *(const f32x4*)(&sm.s[sl][lh * kSPitch + tt + 4 * q]);
        } else {
          x = *(const f32x4*)(&sm.s[w][lh * kSPitch + tt + 4 * q]);
#pragma unroll
          for (int sl = 4; sl < 8; ++sl) x += *(const f32x4*)(&sm.s[sl][lh * kSPitch + tt + 4 * q]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float val = (t0 + tt + 4 * q + e < t_end) ? x[e] : -INFINITY;
          v[s4][4 * q + e] = val;
          mx = fmaxf(mx, val);
        }
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);  // finite: every tile holds a valid token
    const float alpha = exp2f(m_run - m_new);
    bf16x8 pb[4];
    float psum = 0.0f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16 e = (bf16)exp2f(v[s4][i] - m_new);
        pb[s4][i] = e;
        psum += (float)e;  // normalise with the same rounded weights the MFMA uses
      }
    psum += __shfl_xor(psum, 32, 64);
    l_run = alpha * l_run + psum;
    m_run = m_new;

    // ---- O^T[d][h] += V^T P^T over this wave's 128 latent columns
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) O[mb] *= alpha;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const bf16* vb = sm.k + (16 * s4 + tr_row) * kKPitch + tr_col;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8 va = tr_pair(vb + 32 * mb);
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[s4], O[mb], 0, 0, 0);
      }
    }
  }

  // ---- partial outputs.  O[mb] item i: column d = 128w + 32mb + 8*(i/4) + 4*kg + i%4, head lh
  float* po = part_o + (((size_t)b * S + s) * H + h0 + lh) * kDC + 128 * w + 4 * kg;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(f32x4*)(po + 32 * mb + 8 * q) =
          f32x4{O[mb][4 * q], O[mb][4 * q + 1], O[mb][4 * q + 2], O[mb][4 * q + 3]};
  const int br = NB == 1 ? 0 : w;
  if (kg == 0 && (NB == 4 || w == 0)) {
    ml[((size_t)br * H + h0 + lh) * 2 + 0] = m_run;
    ml[((size_t)br * H + h0 + lh) * 2 + 1] = l_run;
  }
}

}  // namespace

hipError_t launch_main_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const int units = p.B * p.splits;
  const unsigned blocks = (unsigned)(((units + 7) / 8) * 8 * p.n_hg);
  auto kern = p.NB == 1 ? k_main_bf16<1> : k_main_bf16<4>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, s, (const bf16*)a.qcat,
                     (const bf16*)a.latent, (const bf16*)a.rope, a.lat_tok, a.lat_seq, a.rope_tok,
                     a.rope_seq, a.seqlens, a.block_table, a.bt_stride, p.paged, a.part_o,
                     a.part_ml, p.H, p.splits, p.chunk, p.n_hg, units);
  return hipGetLastError();
}

}  // namespace mla
