// bf16 prologue and epilogue on MFMA, and the split combine that feeds the epilogue.
//
// Both weight products are small per-head GEMMs over the batch:
//   prologue  q_lat[b, c] = sum_n q_nope[b, n] W_UK[h][n][c]      ([B x d_nope] x [d_nope x d_c])
//   epilogue  out[b, v]   = sum_d o_lat[b, d] W_UV[h][d][v]       ([B x d_c] x [d_c x d_v])
// (the absorbed form's query fold and post-attention value projection; yololab MLA page,
// section 矩陣吸收).  The weights are stored with the contraction index as the row, so a
// workgroup stages its weight block in LDS row-major and reads the MFMA operand with
// ds_read_b64_tr_b16; the batch-row operand is read straight from global memory.
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace mla {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 8 consecutive rows (k) of one column (n) of a row-major LDS block, as an MFMA operand.
// Lane layout (MFMA 32x32x16 operand): lane%32 = column, lane/32 = which 8-row half.  The
// caller passes the address of this lane's source chunk (see tr_src_row / tr_src_col).
__device__ __forceinline__ bf16x8 tr8(const bf16* p, int pitch) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * pitch));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Source chunk of a lane for ds_read_b64_tr_b16: within each 16-lane group, lanes 4r..4r+3
// read 4 consecutive columns each of row r; the read hands lane i of the group column i.
__device__ __forceinline__ int tr_src_row(int lane) { return 8 * (lane >> 5) + ((lane & 15) >> 2); }
__device__ __forceinline__ int tr_src_col(int lane) { return 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }

constexpr int kRows = 32;  // batch rows per workgroup (MFMA M)

// ----------------------------------------------------------------------------- prologue
constexpr int kPCols = 128;          // latent columns per workgroup
constexpr int kPPitch = kPCols + 8;  // LDS pitch of the W_UK block (bf16)

__global__ __launch_bounds__(256) void k_prologue_bf16(
    const bf16* __restrict__ q_nope, const bf16* __restrict__ q_rope,
    const int32_t* __restrict__ seqlens, const bf16* __restrict__ w_uk, bf16* __restrict__ qcat,
    int B, int H, int NB, int dcb, float qscale, RopeFreq rf) {
  constexpr int dn = 128, dr = 64;
  __shared__ __align__(16) bf16 sW[dn * kPPitch];
  const int h = blockIdx.x, b0 = blockIdx.y * kRows, cb = blockIdx.z;
  const int dc = NB * dcb, row = dc + dr;
  const int br = (cb * kPCols) / dcb;          // branch of this column block
  const int c0 = (cb * kPCols) % dcb;          // first column inside the branch
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  const bf16* wsrc = w_uk + ((size_t)br * H + h) * dn * dcb + c0;
#pragma unroll
  for (int j = 0; j < dn * kPCols / 8 / 256; ++j) {
    const int c = tid + 256 * j, r = c >> 4, col = (c & 15) * 8;
    *(u32x4*)(sW + r * kPPitch + col) = *(const u32x4*)(wsrc + (size_t)r * dcb + col);
  }
  // A operand: q_nope rows b0 + lane%32, K-step s covers n = 16s + 8*(lane/32) .. +8
  // rows past B are clamped to B-1: their products are computed but never stored
  const int bl = lane & 31, kg = lane >> 5;
  const int b = min(b0 + bl, B - 1);
  bf16x8 qa[dn / 16];
  const bf16* qsrc = q_nope + (((size_t)b * H + h) * NB + br) * dn + 8 * kg;
#pragma unroll
  for (int s = 0; s < dn / 16; ++s) qa[s] = *(const bf16x8*)(qsrc + 16 * s);
  __syncthreads();
  f32x16 acc = {};
  const bf16* tsrc = sW + tr_src_row(lane) * kPPitch + 32 * w + tr_src_col(lane);
#pragma unroll
  for (int s = 0; s < dn / 16; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], tr8(tsrc + 16 * s * kPPitch, kPPitch), acc, 0, 0, 0);
  // D[i = batch row][j = column]: lane%32 = column, item i -> row 8*(i/4) + 4*(lane/32) + i%4
  const int col = br * dcb + c0 + 32 * w + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int bb = b0 + 8 * (i >> 2) + 4 * kg + (i & 3);
    if (bb < B) qcat[((size_t)bb * H + h) * row + col] = (bf16)(acc[i] * qscale);
  }
  // rotary part of the query, rotated at position L_b - 1 (angles in fp64)
  if (cb == 0) {
    for (int t = tid; t < kRows * (dr / 2); t += 256) {
      const int bb = b0 + t / (dr / 2), k = t % (dr / 2);
      if (bb >= B) continue;
      const int L = seqlens[bb];
      float cs, sn;
      rope_cos_sin(L > 0 ? L - 1 : 0, rf.f[k], &cs, &sn);
      const bf16* x = q_rope + ((size_t)bb * H + h) * dr + 2 * k;
      const float x0 = (float)x[0], x1 = (float)x[1];
      bf16* o = qcat + ((size_t)bb * H + h) * row + dc + 2 * k;
      o[0] = (bf16)((x0 * cs - x1 * sn) * qscale);
      o[1] = (bf16)((x0 * sn + x1 * cs) * qscale);
    }
  }
}

// ----------------------------------------------------------------------------- epilogue
constexpr int kECols = 32;           // output columns per workgroup (one wave)
constexpr int kEPitch = kECols + 8;  // LDS pitch of the W_UV block (bf16)
constexpr int kDc = 512;             // total latent width on the bf16 path (MLA 512, MLRA 4x128)

__global__ __launch_bounds__(64) void k_epilogue_bf16(const bf16* __restrict__ olat,
                                                      const bf16* __restrict__ w_uv,
                                                      bf16* __restrict__ out, int B, int H, int NB,
                                                      int dcb, float out_scale) {
  constexpr int dv = 128;
  __shared__ __align__(16) bf16 sW[kDc * kEPitch];
  const int h = blockIdx.x, b0 = blockIdx.y * kRows, v0 = blockIdx.z * kECols;
  const int lane = threadIdx.x;
  const int bl = lane & 31, kg = lane >> 5;
  // rows past B are clamped to B-1: their products are computed but never stored
  const int b = min(b0 + bl, B - 1);
  // batch-row operand for the whole contraction first, so its latency overlaps the weights
  bf16x8 a[kDc / 16];
  const bf16* arow = olat + ((size_t)b * H + h) * kDc + 8 * kg;
#pragma unroll
  for (int s = 0; s < kDc / 16; ++s) a[s] = *(const bf16x8*)(arow + 16 * s);
  // W_UV rows d (branch d/dcb), columns v0..v0+31: row d = 16*i + lane/4, chunk lane%4
  const int q = lane & 3;
#pragma unroll
  for (int i0 = 0; i0 < kDc / 16; i0 += 8) {
    u32x4 t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = 16 * (i0 + i) + (lane >> 2);
      t[i] = *(const u32x4*)(w_uv + (((size_t)(d / dcb) * H + h) * dcb + d % dcb) * dv + v0 + 8 * q);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4*)(sW + (16 * (i0 + i) + (lane >> 2)) * kEPitch + 8 * q) = t[i];
  }
  __syncthreads();
  f32x16 acc = {};
  const bf16* tsrc = sW + tr_src_row(lane) * kEPitch + tr_src_col(lane);
#pragma unroll
  for (int s = 0; s < kDc / 16; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], tr8(tsrc + 16 * s * kEPitch, kEPitch), acc, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int bb = b0 + 8 * (i >> 2) + 4 * kg + (i & 3);
    if (bb < B) out[((size_t)bb * H + h) * dv + v0 + (lane & 31)] = (bf16)(acc[i] * out_scale);
  }
}

}  // namespace

hipError_t launch_prologue_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(p.H, (p.B + kRows - 1) / kRows, p.dc / kPCols);
  RopeFreq rf;
  make_rope_freq(p.dr, a.rope_theta, &rf);
  hipLaunchKernelGGL(k_prologue_bf16, grid, dim3(256), 0, s, (const bf16*)a.q_nope,
                     (const bf16*)a.q_rope, a.seqlens, (const bf16*)a.w_uk, (bf16*)a.qcat, p.B,
                     p.H, p.NB, p.dcb, a.softmax_scale * kLog2e, rf);
  return hipGetLastError();
}

hipError_t launch_epilogue_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(p.H, (p.B + kRows - 1) / kRows, p.dv / kECols);
  hipLaunchKernelGGL(k_epilogue_bf16, grid, dim3(64), 0, s, (const bf16*)a.olat,
                     (const bf16*)a.w_uv, (bf16*)a.out, p.B, p.H, p.NB, p.dcb, a.out_scale);
  return hipGetLastError();
}

}  // namespace mla
