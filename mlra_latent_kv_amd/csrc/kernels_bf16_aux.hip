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
#include "plan_device.h"
#include "tile_bf16.h"

namespace mla {
namespace {

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

// LQ: folded query (MLA_FLAG_QUERY_LATENT): q_nope holds q_lat [B][H][dc], copied and scaled
// instead of the W_UK product.
template <bool LQ>
__global__ __launch_bounds__(256) void k_prologue_bf16(
    const bf16* __restrict__ q_nope, const bf16* __restrict__ q_rope,
    const int32_t* __restrict__ seqlens, const bf16* __restrict__ w_uk, bf16* __restrict__ qcat,
    int B, int H, int NB, int dcb, float qscale, float qscale_lat, RopeFreq rf, PlanArgs plan,
    int Hw, int sq) {
  constexpr int dn = 128, dr = 64;
  __shared__ __align__(16) bf16 sW[dn * kPPitch];
  const int h = blockIdx.x, b0 = blockIdx.y * kRows, cb = blockIdx.z;
  if (h == H) {  // the extra column of blocks: block (H, 0, 0) makes the split plan
    if (b0 == 0 && cb == 0) make_work_plan(plan, sW, (int)sizeof(sW));
    return;
  }
  const int dc = NB * dcb, row = dc + dr;
  // query row h = token qi x Hw + weight head hw (s_q > 1 tokens per sequence: token qi sits
  // at L - s_q + qi)
  const int hw = h % Hw, qi = h / Hw;
  const int br = (cb * kPCols) / dcb;          // branch of this column block
  const int c0 = (cb * kPCols) % dcb;          // first column inside the branch
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // rotary part of the query, rotated at position L_b - 1 (angles in fp64), spread over the
  // column-block workgroups of the head: the kRows * dr / 2 = 1024 (row, pair) items take one
  // per thread with d_c = 512 (gridDim.z = 4), up to four with d_c = 128 (gridDim.z = 1).
  // Their loads go out with the weight loads, so the kernel makes one memory round trip.
  constexpr int kRotPer = 4;  // most (row, pair) items per thread
  const int n_rot = (kRows * (dr / 2) + 256 * (int)gridDim.z - 1) / (256 * (int)gridDim.z);
  int bb_r[kRotPer], k_r[kRotPer], L_r[kRotPer];
  bool has_r[kRotPer];
  float x0[kRotPer], x1[kRotPer];
#pragma unroll
  for (int it = 0; it < kRotPer; ++it) {
    const int t_r = (it * (int)gridDim.z + cb) * 256 + tid;
    bb_r[it] = b0 + t_r / (dr / 2);
    k_r[it] = t_r % (dr / 2);
    has_r[it] = it < n_rot && t_r < kRows * (dr / 2) && bb_r[it] < B;
    x0[it] = x1[it] = 0.0f;
    L_r[it] = 0;
    if (it < n_rot) {  // uniform
      const int bc = min(bb_r[it], B - 1);
      const bf16* xr = q_rope + ((size_t)bc * H + h) * dr + 2 * (has_r[it] ? k_r[it] : 0);
      x0[it] = (float)xr[0];
      x1[it] = (float)xr[1];
      // position of the query token: L - s_q + qi, L as the plan clamps it
      L_r[it] = causal_limit(seqlens, bc, plan.max_seqlen, sq, qi) - 1;
    }
  }
  if constexpr (LQ) {
    // 32 rows x 128 columns of q_lat, 16 per thread as two 16-byte pieces
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int piece = tid + 256 * k, r = piece >> 4, col = cb * kPCols + 8 * (piece & 15);
      const int bb = b0 + r;
      if (bb < B) {
        const size_t bh = (size_t)bb * H + h;
        const bf16x8 v = *(const bf16x8*)(q_nope + bh * dc + col);
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)v[e] * qscale_lat);
        *(bf16x8*)(qcat + bh * row + col) = o;
      }
    }
  } else {
    const bf16* wsrc = w_uk + ((size_t)br * Hw + hw) * dn * dcb + c0;
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
      if (bb < B) qcat[((size_t)bb * H + h) * row + col] = (bf16)(acc[i] * qscale_lat);
    }
  }
#pragma unroll
  for (int it = 0; it < kRotPer; ++it) {
    if (has_r[it]) {
      float cs, sn;
      rope_cos_sin(max(L_r[it], 0), rf.f[k_r[it]], &cs, &sn);
      bf16* o = qcat + ((size_t)bb_r[it] * H + h) * row + dc + 2 * k_r[it];
      o[0] = (bf16)((x0[it] * cs - x1[it] * sn) * qscale);
      o[1] = (bf16)((x0[it] * sn + x1[it] * cs) * qscale);
    }
  }
}

}  // namespace

hipError_t launch_prologue_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(p.H + 1, (p.B + kRows - 1) / kRows, p.dc / kPCols);
  // at most four rotary (row, pair) items per thread cover the query's rotary part
  if (kRows * (p.dr / 2) > 4 * 256 * (int)grid.z) return hipErrorInvalidValue;
  RopeFreq rf;
  make_rope_freq(p.dr, a.rope_theta, &rf);
  hipLaunchKernelGGL(p.latent_q ? k_prologue_bf16<true> : k_prologue_bf16<false>, grid,
                     dim3(256), 0, s, (const bf16*)a.q_nope,
                     (const bf16*)a.q_rope, a.seqlens, (const bf16*)a.w_uk, (bf16*)a.qcat, p.B,
                     p.H, p.NB, p.dcb, a.softmax_scale * kLog2e,
                     a.softmax_scale * kLog2e * a.latent_scale, rf, a.plan, p.Hw, p.sq);
  return hipGetLastError();
}

// ------------------------------------------------------------------- combine + epilogue
// out[b, h, :] = out_scale * sum_c o_lat[b, h, c] * W_UV[c / dcb][h][c % dcb][:], where
// o_lat[b, h, c] = sum_s w_s O_s[b, h, c] is the log-sum-exp merge of the split partials
// (w_s = 2^(m_s - M) / sum_s' 2^(m_s' - M) l_s' with M the largest split max of the head's
// branch) -- the split combine and the W_UV projection of the absorbed form (yololab MLA
// page, section 矩陣吸收), with the MLRA-4 branch sum carried by the contraction over all
// 512 latent columns ("[ICLR 2025] MLRA…", section 2.2).
//
// Latent width DC = 512 (MLA, MLRA-4) or 128 (one MLRA branch as a tensor-parallel shard).
// One workgroup (4 waves) per (head h, rows b0..b0+R-1), R in {2, 4, 8, 16}:
//  1. the split statistics (M, 1/L) of every (row, branch), then the weighted sum of the split
//     partials, with all 256 threads sharing the (row, 16-byte chunk) work, into an LDS copy
//     of the merged latent output (bf16, the MFMA operand);
//  2. meanwhile the W_UV rows of the head go to LDS by direct-to-LDS loads (one contiguous
//     block per wave: wave w owns latent columns [w DC/4, (w+1) DC/4), exactly branch w for
//     MLRA-4), issued behind the first partials, half before the statistics are formed and
//     half after, so that they stream in during the merge;
//  3. each wave multiplies its DC / 4 latent columns by its W_UV rows (MFMA 32x32x16, rows of
//     the workgroup as M, padded to 32), and the four partial products (K split four ways)
//     are summed through LDS.
namespace {

constexpr int kCeDv = 128;                 // d_v of the bf16 path
constexpr int kCeRowB = kCeDv * 2;         // bytes per W_UV row in LDS
constexpr int kCeRedPitch = kCeDv + 4;     // fp32 pitch of the cross-wave sum
constexpr int kCeMaxRows = 16;

// physical 16-byte chunk of logical chunk c in W_UV row r: the transposed operand reads
// cover 4 consecutive rows x 4 consecutive chunks, which this XOR spreads over all 16
// chunk slots of a 256-byte bank line
__device__ __forceinline__ int ce_sw(int r, int c) { return c ^ (4 * (r & 3)); }

// R = 256 NC / (TPC DC / 8) rows per workgroup; each thread merges NC chunks of one row, with
// 32 chunk loads in flight.  TPC > 1 (small row blocks, for small batches): TPC adjacent
// threads share a chunk, each taking every TPC-th split, and add their sums at the end.
//
// LO (MLA_FLAG_OUTPUT_LATENT): the merged latent rows, times out_scale, are the output
// [B][H][DC]; no W_UV is read and phase 3 does not run.  gate (gated entry points, else
// null): the result is multiplied by 1 / (1 + exp(-gate)) elementwise.
template <int NC, int TPC, int DC, bool LO>
__global__ __launch_bounds__(256, 1) void k_combine_epilogue_bf16(
    const bf16* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ split_off, const bf16* __restrict__ w_uv,
    const bf16* __restrict__ gate, bf16* __restrict__ out, int B, int H, int NB, int dcb,
    float out_scale, int Hw) {
  constexpr int kCPR = DC / 8;                  // 16-byte chunks per latent row
  constexpr int R = 256 * NC / (TPC * kCPR);
  constexpr int kWRows = DC / 4;                // W_UV rows (latent columns) per wave
  constexpr int kKS = kWRows / 16;              // MFMA K-steps per wave
  constexpr int kWBytes = 4 * kWRows * kCeRowB;
  constexpr int kRedBytes = 4 * kCeMaxRows * kCeRedPitch * 4;
  static_assert(R >= 2 && R <= kCeMaxRows, "rows per workgroup");
  struct Smem {
    // per wave: its W_UV rows, chunk-swizzled; reused for the cross-wave sum
    char wuv[kWBytes > kRedBytes ? kWBytes : kRedBytes];
    char olat[kCeMaxRows][2 * DC];    // merged latent rows, chunk c at c ^ (row % 16)
    float stat_m[kCeMaxRows][4], stat_inv[kCeMaxRows][4];
  };
  __shared__ __align__(16) Smem sm;  // 145 KiB (DC = 512); wuv also holds the cross-wave sum
  char* const wuv_w = sm.wuv + (size_t)kWRows * kCeRowB * __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x % H, b0 = (blockIdx.x / H) * R;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a uniform value: the W_UV buffer descriptor depends on it, and a descriptor
  // the compiler cannot prove uniform turns every load into a per-lane loop
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // ---- 1. W_UV rows c0..c0+127 of head h: instruction i brings rows 4i..4i+3; lane l lands
  // at physical chunk l%16 of row 4i + l/16 and so fetches logical chunk ce_sw(row, l%16).
  // Instructions i0..i1-1.  Issued after the split statistics' loads and the first partials
  // (below): vector-memory loads complete in issue order, so issued first they made the
  // statistics wait for these 128 KiB too.  Half go out right after the first partials (a
  // wave then has 60 loads out, within the 63 its load counter tracks; more would stall the
  // issue), the other half behind the statistics' barrier, below the branch of the
  // statistics' rare extra loads, where the wait analysis counts them exactly.  They stream
  // in while the partials are merged.
  auto issue_wuv = [&](int i0, int i1) {
    const int c0 = kWRows * w, br = c0 / dcb;
    const bf16* wbase = w_uv + ((size_t)(br * Hw + h % Hw) * dcb + (c0 % dcb)) * kCeDv;
    const __amdgpu_buffer_rsrc_t rs = tile::rsrc(wbase, kWRows * kCeRowB);
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const int r = 4 * i + (lane >> 4);
      tile::dma16(rs, wuv_w + 1024 * i, r * kCeRowB + 16 * ce_sw(r, lane & 15));
    }
  };

  // ---- 2. merged latent.  The splits of row b are its work items split_off[b] ..
  // split_off[b + 1] - 1 (a variable number per row, none for an empty sequence).  Thread t
  // takes NC consecutive chunks of one row (within one branch: NC <= 4 chunks, a branch is 16
  // or 64 chunks).  The first batch of its split maxima and chunk loads goes out before the
  // split statistics are formed, so that the two latencies overlap.  A batch's tail past the
  // row's last split gets weight 0, and its loads (of an item that exists) are replaced by
  // zeros.
  const size_t ml_s = (size_t)NB * H * 2;  // part_ml stride of one work item
  const size_t po_s = (size_t)H * DC;      // part_o stride of one work item
  const int first = (tid / TPC) * NC, mr = first / kCPR, mc = first % kCPR;
  const int z = tid % TPC;  // which of the chunk's threads: takes splits z, z + TPC, ...
  const int mb = b0 + mr, mbr = (8 * mc) / dcb;
  // every load is unconditional, at a written work item (a predicated load leaves the
  // compiler's wait analysis with a full drain at the join); masked values are replaced
  // after the load
  const int mbl = min(mb, B - 1);
  const int mu0 = split_off[mbl], mn = mb < B ? split_off[mbl + 1] - mu0 : 0;
  auto item_of = [](int u0, int n, int s) { return max(u0 + min(s, n - 1), 0); };
  const float* mml = part_ml + (size_t)mbr * H * 2 + h * 2;
  const bf16* msrc = part_o + (size_t)h * DC + 8 * mc;
  // the longest split list among the workgroup's rows bounds the (uniform) merge loop
  int n_max = 0;
  for (int r = 0; r < R; ++r) {
    const int bb = min(b0 + r, B);
    n_max = max(n_max, split_off[min(bb + 1, B)] - split_off[bb]);
  }
  constexpr int kU = 32 / NC;  // splits in flight per thread
  float mv[kU];
  bf16x8 v[kU][NC];
  // batch starting at split s0 (a multiple of kU * TPC): this thread's splits s0 + TPC*u + z
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) mv[u] = mml[item_of(mu0, mn, s0 + TPC * u + z) * ml_s];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const size_t it = item_of(mu0, mn, s0 + TPC * u + z);
#pragma unroll
      for (int i = 0; i < NC; ++i) v[u][i] = *(const bf16x8*)(msrc + it * po_s + 8 * i);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (s0 + TPC * u + z >= mn) mv[u] = -INFINITY;
  };
  // ---- 2a. split statistics of (row, branch): M = largest split max, 1/L.  A group of P
  // consecutive lanes per (row, branch) takes splits s = q, q + P, ... and the group merges
  // its (M, L) pairs with lane shuffles (P <= 64: one wave; threads past the R * NB groups
  // load in-bounds values and drop them).  The first four (m, l) pairs of a lane are loaded
  // ahead of the merge batch (loads complete in order).
  {
    const int P = min(64, 256 / (R * NB));  // 4..64, a power of two
    const int pair = tid / P, q = tid % P;
    const bool live = pair < R * NB;
    const int r = min(pair / NB, R - 1), br = pair % NB, b = b0 + r;
    const int bl = min(b, B - 1);
    const int u0 = split_off[bl], n = live && b < B ? split_off[bl + 1] - u0 : 0;
    const float* ml = part_ml + (size_t)br * H * 2 + h * 2;
    constexpr int kPre = 4;
    float pm[kPre], pl[kPre];
#pragma unroll
    for (int it = 0; it < kPre; ++it) {
      const size_t sidx = item_of(u0, n, q + it * P);
      pm[it] = ml[sidx * ml_s];
      pl[it] = ml[sidx * ml_s + 1];
    }
    load_batch(0);
    if constexpr (!LO) issue_wuv(0, kWRows / 8);
#pragma unroll
    for (int it = 0; it < kPre; ++it)
      if (q + it * P >= n) pm[it] = -INFINITY;
    float M = -INFINITY, L = 0.0f;
    auto merge = [&](float m, float l) {
      if (m != -INFINITY) {
        const float mn = fmaxf(M, m);
        L = L * exp2f(M - mn) + l * exp2f(m - mn);
        M = mn;
      }
    };
#pragma unroll
    for (int it = 0; it < kPre; ++it) merge(pm[it], pl[it]);
    for (int s = q + kPre * P; s < n; s += P) {
      const size_t sidx = (size_t)(u0 + s);
      merge(ml[sidx * ml_s], ml[sidx * ml_s + 1]);
    }
    for (int o = 1; o < P; o <<= 1) {
      const float Mo = __shfl_xor(M, o, 64), Lo = __shfl_xor(L, o, 64);
      const float mn = fmaxf(M, Mo);
      if (mn != -INFINITY) {
        L = L * exp2f(M - mn) + Lo * exp2f(Mo - mn);
        M = mn;
      }
    }
    if (q == 0 && live) {
      sm.stat_m[r][br] = M;
      sm.stat_inv[r][br] = L > 0.0f ? 1.0f / L : 0.0f;
    }
  }
  // LDS-only barrier: __syncthreads() would first wait for every load in flight (all the
  // partials of the first batch), and the merge below would start only once they had all
  // arrived instead of load by load
  tile::lds_barrier();
  if constexpr (!LO) issue_wuv(kWRows / 8, kWRows / 4);

  // ---- 2b. weighted sum of the splits, batch by batch
  {
    f32x4 acc[NC][2];
#pragma unroll
    for (int i = 0; i < NC; ++i) acc[i][0] = acc[i][1] = f32x4{};
    const float M = sm.stat_m[mr][mbr], inv = sm.stat_inv[mr][mbr];
    for (int s0 = 0; s0 < n_max; s0 += kU * TPC) {
      if (s0 > 0) load_batch(s0);
      float wt[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        wt[u] = mv[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv[u] - M) * inv;
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int i = 0; i < NC; ++i)
          if (wt[u] == 0.0f) v[u][i] = bf16x8{};
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          acc[i][0] += wt[u] * f32x4{(float)v[u][i][0], (float)v[u][i][1], (float)v[u][i][2],
                                     (float)v[u][i][3]};
          acc[i][1] += wt[u] * f32x4{(float)v[u][i][4], (float)v[u][i][5], (float)v[u][i][6],
                                     (float)v[u][i][7]};
        }
    }
    // the chunk's TPC threads are adjacent lanes: add their shares
#pragma unroll
    for (int o = 1; o < TPC; o <<= 1)
#pragma unroll
      for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][0][e] += __shfl_xor(acc[i][0][e], o, 64);
          acc[i][1][e] += __shfl_xor(acc[i][1][e], o, 64);
        }
    if constexpr (LO) {
      // latent output: the merged chunks, scaled, are the result
#pragma unroll
      for (int i = 0; i < NC; ++i)
        if (z == 0 && mb < B) {
          bf16x8 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r[e] = (bf16)(acc[i][0][e] * out_scale);
            r[4 + e] = (bf16)(acc[i][1][e] * out_scale);
          }
          *(bf16x8*)(out + ((size_t)mb * H + h) * DC + 8 * (mc + i)) = r;
        }
    } else {
#pragma unroll
      for (int i = 0; i < NC; ++i)
        if (z == 0)
          *(bf16x8*)(sm.olat[mr] + 16 * ((mc + i) ^ (mr & 15))) =
            bf16x8{(bf16)acc[i][0][0], (bf16)acc[i][0][1], (bf16)acc[i][0][2], (bf16)acc[i][0][3],
                   (bf16)acc[i][1][0], (bf16)acc[i][1][1], (bf16)acc[i][1][2], (bf16)acc[i][1][3]};
    }
  }
  if constexpr (LO) return;
  tile::wait_vmcnt<0>();  // this wave's W_UV rows have landed
  __syncthreads();        // every merged latent row is in LDS
  // the gate logits of this thread's output piece (row tid / 16, columns 8 (tid % 16) ..),
  // loaded now so that the products below hide their latency
  const int orow = tid >> 4, ov0 = 8 * (tid & 15);
  const bool ostore = orow < R && b0 + orow < B;
  bf16x8 gv = {};
  if (gate && ostore) gv = *(const bf16x8*)(gate + ((size_t)(b0 + orow) * H + h) * kCeDv + ov0);

  // ---- 3. out[row][v] partial over this wave's DC / 4 latent columns.  A operand: lane (row
  // l32, k-half g) holds columns w DC/4 + 16j + 8g..+7 (chunk w DC/32 + 2j + g); rows >= R are
  // zero.  B operand (K = latent rows, N = v): lane (v, k-half g) holds W_UV rows 16j + 8g..+7
  // of column v, two transposed reads: source lane li of 16-lane group G addresses row
  // 16j + 8*(G>>1) + li/4 (+4), columns 16*(G&1) + 4*(li&3)..+3 of the block.
  bf16x8 a[kKS];
#pragma unroll
  for (int j = 0; j < kKS; ++j) {
    const int cc = (DC / 32) * w + 2 * j + g;
    a[j] = l32 < R ? *(const bf16x8*)(sm.olat[l32 & (kCeMaxRows - 1)] + 16 * (cc ^ (l32 & 15)))
                   : bf16x8{};
  }
  const int G = lane >> 4, li = lane & 15;
  f32x16 o[4];
#pragma unroll
  for (int vb = 0; vb < 4; ++vb) {
    o[vb] = f32x16{};
    const int col = 32 * vb + 16 * (G & 1) + 4 * (li & 3);
#pragma unroll
    for (int j = 0; j < kKS; ++j) {
      const int r1 = 16 * j + 8 * (G >> 1) + (li >> 2), r2 = r1 + 4;
      const char* base = wuv_w;
      const bf16x8 bv = tile::tr_pair(base + r1 * kCeRowB + 16 * ce_sw(r1, col >> 3) + 2 * (col & 7),
                                      base + r2 * kCeRowB + 16 * ce_sw(r2, col >> 3) + 2 * (col & 7));
      o[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], bv, o[vb], 0, 0, 0);
    }
  }

  // ---- sum of the four K quarters.  D layout: lane (v, half g), item e -> row
  // 8*(e/4) + 4*g + e%4, column 32*vb + v.  Only rows < R are stored.
  __syncthreads();  // every wave is done with its W_UV rows
  float* red = reinterpret_cast<float*>(sm.wuv);
#pragma unroll
  for (int vb = 0; vb < 4; ++vb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int row = 8 * (e >> 2) + 4 * g + (e & 3);
      if (row < kCeMaxRows) red[(w * kCeMaxRows + row) * kCeRedPitch + 32 * vb + l32] = o[vb][e];
    }
  __syncthreads();
  // thread t: row t / 16, columns 8*(t % 16)..+7
  if (ostore) {
    bf16x8 res;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) sum += red[(ww * kCeMaxRows + orow) * kCeRedPitch + ov0 + i];
      sum *= out_scale;
      // sigmoid(g) = 1 / (1 + 2^(-g log2 e))
      if (gate) sum *= 1.0f / (1.0f + __builtin_amdgcn_exp2f(-(float)gv[i] * kLog2e));
      res[i] = (bf16)sum;
    }
    *(bf16x8*)(out + ((size_t)(b0 + orow) * H + h) * kCeDv + ov0) = res;
  }
}

}  // namespace

// rows per workgroup: the largest of 16, 8, 4 that still gives every CU a workgroup, else the
// smallest block (2 rows at DC = 512, 4 at DC = 128); fewer rows per workgroup read each
// head's W_UV more often, mostly from L2
int combine_epilogue_rows(int B, int H, int dc) {
  const int r_min = dc == 128 ? 4 : 2;
  for (int R = 16; R > r_min; R /= 2)
    if ((long)H * ((B + R - 1) / R) >= 256) return R;
  return r_min;
}

namespace {
// <NC, TPC, DC, LO>: R = 256 NC / (TPC DC / 8)
template <bool LO>
auto combine_epilogue_kernel(int dc, int R) {
  return dc == 128 ? (R == 16  ? k_combine_epilogue_bf16<1, 1, 128, LO>
                      : R == 8 ? k_combine_epilogue_bf16<1, 2, 128, LO>
                               : k_combine_epilogue_bf16<1, 4, 128, LO>)
         : R == 16 ? k_combine_epilogue_bf16<4, 1, 512, LO>
         : R == 8  ? k_combine_epilogue_bf16<2, 1, 512, LO>
         : R == 4  ? k_combine_epilogue_bf16<1, 1, 512, LO>
                   : k_combine_epilogue_bf16<1, 2, 512, LO>;
}
}  // namespace

hipError_t launch_combine_epilogue_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const int R = combine_epilogue_rows(p.B, p.H, p.dc);
  const unsigned blocks = (unsigned)(p.H * ((p.B + R - 1) / R));
  auto kern = p.latent_out ? combine_epilogue_kernel<true>(p.dc, R)
                           : combine_epilogue_kernel<false>(p.dc, R);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, (const bf16*)a.part_o, a.part_ml,
                     a.split_off, (const bf16*)a.w_uv, (const bf16*)a.gate, (bf16*)a.out, p.B,
                     p.H, p.NB, p.dcb, a.out_scale * a.latent_scale, p.Hw);
  return hipGetLastError();
}

}  // namespace mla
