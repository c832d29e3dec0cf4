// fp32 path (prologue, split combine, W_UV epilogue, SIMT main loop for small fp32 shapes)
// and the rotary-key rotation.  The bf16 path's prologue and fused combine + epilogue are in
// kernels_bf16_aux.hip, its main loops in main_bf16.hip and main_bf16_wide.hip.
//
// Absorption ("超越 GQA 的推理革命…MLA…", section 矩陣吸收): the key up-projection W_UK is
// folded into the query (prologue) and the value up-projection W_UV is applied once to the
// attention-weighted latent (epilogue), so per-token keys and values are never formed.
#include <algorithm>
#include <climits>
#include <cmath>

#include "device_common.h"
#include "launch.h"
#include "plan_device.h"

namespace mla {

constexpr int kBatchBlock = 8;  // sequences per prologue / epilogue workgroup (weight reuse)

void make_rope_freq(int d_rope, float theta, RopeFreq* out) {
  for (int k = 0; k < 128; ++k)
    out->f[k] = k < d_rope / 2 ? std::pow((double)theta, -2.0 * k / d_rope) : 0.0;
}

// ----------------------------------------------------------------------------- prologue
// qcat[b,h] = [ (W_UK[br,h]^T q_nope[b,h,br])_{br} | RoPE(q_rope[b,h], L_b - 1) ] * qscale
// qscale = softmax_scale * log2(e) so the main loop can use exp2.
template <typename T>
__global__ __launch_bounds__(256) void k_prologue(const T* __restrict__ q_nope,
                                                  const T* __restrict__ q_rope,
                                                  const int32_t* __restrict__ seqlens,
                                                  const T* __restrict__ w_uk, T* __restrict__ qcat,
                                                  int B, int H, int NB, int dn, int dcb, int dr,
                                                  float qscale, RopeFreq rf, PlanArgs plan,
                                                  int lds_bytes, int latent_q, int Hw, int nq) {
  extern __shared__ __align__(16) float sq[];  // [kBatchBlock][NB][dn]; the plan block: scratch
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * kBatchBlock;
  if (h == H) {  // the extra column of blocks: block (H, 0) makes the split plan
    if (b0 == 0) make_work_plan(plan, sq, lds_bytes);
    return;
  }
  const int nb = min(kBatchBlock, B - b0);
  const int dc = NB * dcb, row = dc + dr;
  const int hw = h % Hw, qi = h / Hw;  // query row = token qi x Hw + weight head hw
  if (latent_q) {
    // folded query: q_nope holds q_lat [B][H][dc], W_UK already applied offline
    for (int i = threadIdx.x; i < nb * dc; i += blockDim.x) {
      const int j = i / dc, c = i % dc;
      const size_t bh = (size_t)(b0 + j) * H + h;
      qcat[bh * row + c] = from_f32<T>(to_f32(q_nope[bh * dc + c]) * qscale);
    }
  }
  const int per_b = NB * dn;
  for (int i = threadIdx.x; !latent_q && i < kBatchBlock * per_b; i += blockDim.x) {
    const int j = i / per_b, rest = i % per_b;
    sq[i] = j < nb ? to_f32(q_nope[((size_t)(b0 + j) * H + h) * per_b + rest]) : 0.0f;
  }
  __syncthreads();
  for (int c = threadIdx.x; !latent_q && c < dc; c += blockDim.x) {
    const int br = c / dcb, cc = c % dcb;
    const T* w = w_uk + ((size_t)br * Hw + hw) * dn * dcb + cc;
    const float* q = sq + br * dn;
    float acc[kBatchBlock];
#pragma unroll
    for (int j = 0; j < kBatchBlock; ++j) acc[j] = 0.0f;
    for (int n = 0; n < dn; ++n) {
      const float wv = to_f32(w[(size_t)n * dcb]);
#pragma unroll
      for (int j = 0; j < kBatchBlock; ++j) acc[j] = fmaf(q[j * per_b + n], wv, acc[j]);
    }
    for (int j = 0; j < nb; ++j)
      qcat[((size_t)(b0 + j) * H + h) * row + c] = from_f32<T>(acc[j] * qscale);
  }
  const int half = dr / 2;
  for (int i = threadIdx.x; i < nb * half; i += blockDim.x) {
    const int j = i / half, k = i % half;
    const int b = b0 + j;
    const int pos = causal_limit(seqlens, b, plan.max_seqlen, nq, qi) - 1;  // L - s_q + qi
    float cs, sn;
    rope_cos_sin(max(pos, 0), rf.f[k], &cs, &sn);
    const T* x = q_rope + ((size_t)b * H + h) * dr + 2 * k;
    const float x0 = to_f32(x[0]), x1 = to_f32(x[1]);
    T* o = qcat + ((size_t)b * H + h) * row + dc + 2 * k;
    o[0] = from_f32<T>((x0 * cs - x1 * sn) * qscale);
    o[1] = from_f32<T>((x0 * sn + x1 * cs) * qscale);
  }
}

hipError_t launch_prologue(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(p.H + 1, (p.B + kBatchBlock - 1) / kBatchBlock);
  const size_t lds = std::max<size_t>(
      p.latent_q ? 0 : (size_t)kBatchBlock * p.NB * p.dn * sizeof(float), 16384);
  const float qscale = a.softmax_scale * kLog2e;
  RopeFreq rf;
  make_rope_freq(p.dr, a.rope_theta, &rf);
  hipLaunchKernelGGL(k_prologue<float>, grid, dim3(256), lds, s, (const float*)a.q_nope,
                       (const float*)a.q_rope, a.seqlens, (const float*)a.w_uk, (float*)a.qcat,
                       p.B, p.H, p.NB, p.dn, p.dcb, p.dr, qscale, rf, a.plan, (int)lds,
                       p.latent_q, p.Hw, p.sq);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- device checks
// MLA_FLAG_DEVICE_CHECKS: one workgroup per sequence b checks seqlens[b] against
// [0, max_seqlen] and, for a paged cache with a known pool size, every block-table entry of
// the pages the (clamped) length uses against [0, num_pages).  It writes
// dbg[b] = 4 * (first bad page index + 1, or 0) + error bits, which the split plan folds into
// the error word.  Every read stays inside seqlens[b] and the row's used block-table entries.
__global__ __launch_bounds__(256) void k_device_checks(const int32_t* __restrict__ seqlens,
                                                       const int32_t* __restrict__ bt,
                                                       int64_t bt_stride, int paged,
                                                       int num_pages, int max_seqlen,
                                                       int32_t* __restrict__ dbg) {
  __shared__ int red[4];
  const int b = blockIdx.x;
  const int raw = seqlens[b];
  int first = INT_MAX;
  if (paged && num_pages > 0) {
    const int L = min(max(raw, 0), max_seqlen);
    const int np = (L + kPage - 1) / kPage;
    const int32_t* row = bt + (int64_t)b * bt_stride;
    for (int j = threadIdx.x; j < np; j += 256) {
      const int e = row[j];
      if (e < 0 || e >= num_pages) first = min(first, j);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = first;
    __syncthreads();
    first = min(min(red[0], red[1]), min(red[2], red[3]));
  }
  if (threadIdx.x == 0) {
    int d = (raw < 0 || raw > max_seqlen) ? MLA_DEVERR_SEQLEN : 0;
    if (first != INT_MAX) d |= MLA_DEVERR_BLOCK | (4 * (first + 1));
    dbg[b] = d;
  }
}

hipError_t launch_device_checks(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_device_checks, dim3(p.B), dim3(256), 0, s, a.seqlens, a.block_table,
                     a.bt_stride, p.paged, p.num_pages, p.max_seqlen, const_cast<int32_t*>(a.plan.dbg));
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- combine
// Per (b, h, branch): merge the splits' (m_s, l_s, O_s) with log-sum-exp weights:
//   M = max_s m_s,  o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// fp32 path: one workgroup handles 8 heads of one sequence; the split weights are formed
// once in LDS, then the partial outputs stream through.  The splits of sequence b are its
// work items split_off[b] .. split_off[b + 1] - 1 (none for an empty sequence: zeros).
constexpr int kCombHeads = 8;    // heads per combine workgroup
constexpr int kCombCols = 128;   // latent columns per combine workgroup (multiple of 4)

// Four consecutive partial values as fp32.
__device__ __forceinline__ f32x4 load4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  const bf16x4 v = *(const bf16x4*)p;
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

template <typename TP, typename TO>
__global__ __launch_bounds__(256) void k_combine(const TP* __restrict__ part_o,
                                                 const float* __restrict__ part_ml,
                                                 const int32_t* __restrict__ split_off,
                                                 TO* __restrict__ olat, int H, int S, int NB,
                                                 int dcb, float scale) {
  extern __shared__ float sw[];  // [kCombHeads][branches in this column block][S]
  const int hb = blockIdx.x, b = blockIdx.y;
  const int h0 = hb * kCombHeads;
  const int nh = min(kCombHeads, H - h0);
  const int dc = NB * dcb;
  const int d0 = blockIdx.z * kCombCols, d1 = min(dc, d0 + kCombCols);
  const int br0 = d0 / dcb, nbr = (d1 - 1) / dcb - br0 + 1;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // the work items (splits) of sequence b: u0 .. u0 + n - 1, n <= S
  const int u0 = split_off[b], n = split_off[b + 1] - u0;
  const size_t sstride = (size_t)NB * H * 2;
  // split weights: one wave per (head, branch), lanes stride over the splits
  for (int pr = wv; pr < nh * nbr; pr += blockDim.x / 64) {
    const int hl = pr / nbr, br = br0 + pr % nbr;
    const float* ml = part_ml + ((size_t)u0 * NB + br) * H * 2 + (h0 + hl) * 2;
    float M = -INFINITY;
    for (int s = lane; s < n; s += 64) M = fmaxf(M, ml[s * sstride]);
    M = wave_max(M);
    float den = 0.0f;
    if (M != -INFINITY)
      for (int s = lane; s < n; s += 64) {
        const float m = ml[s * sstride];
        if (m != -INFINITY) den = fmaf(exp2f(m - M), ml[s * sstride + 1], den);
      }
    den = wave_sum(den);
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    for (int s = lane; s < n; s += 64) {
      const float m = ml[s * sstride];
      sw[pr * S + s] = (m == -INFINITY) ? 0.0f : exp2f(m - M) * inv;
    }
  }
  __syncthreads();
  const int q4 = (d1 - d0) / 4;
  const size_t pstride = (size_t)H * dc;
  for (int it = threadIdx.x; it < nh * q4; it += blockDim.x) {
    const int hl = it / q4, d = d0 + 4 * (it % q4);
    const float* wrow = sw + (hl * nbr + d / dcb - br0) * S;
    const TP* src = part_o + ((size_t)u0 * H + h0 + hl) * dc + d;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < n; s0 += 4) {
      f32x4 v[4];
      float wt[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wt[u] = s0 + u < n ? wrow[s0 + u] : 0.0f;
        // a split whose every score underflowed has weight 0: skip its load
        v[u] = wt[u] != 0.0f ? load4(src + (size_t)(s0 + u) * pstride) : f32x4{};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += wt[u] * v[u];
    }
    TO* dst = olat + ((size_t)b * H + h0 + hl) * dc + d;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = from_f32<TO>(acc[e] * scale);
  }
}

// fp32 path (the bf16 path merges the splits inside launch_combine_epilogue_bf16).  With a
// latent output the merged rows, times out_scale, go straight to out.
hipError_t launch_combine(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((p.H + kCombHeads - 1) / kCombHeads, p.B, (p.dc + kCombCols - 1) / kCombCols);
  const int max_br = kCombCols / p.dcb + 2;
  const size_t lds = (size_t)kCombHeads * std::min(p.NB, max_br) * p.splits * sizeof(float);
  hipLaunchKernelGGL((k_combine<float, float>), grid, dim3(256), lds, s, (const float*)a.part_o,
                     a.part_ml, a.split_off, (float*)(p.latent_out ? a.out : a.olat), p.H,
                     p.splits, p.NB, p.dcb, p.latent_out ? a.out_scale : 1.0f);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- epilogue
// out[b,h,v] = out_scale * sum_br sum_c olat[b,h,br*dcb + c] * W_UV[br,h,c,v]
//              (times 1 / (1 + exp(-gate[b,h,v])) when a gate is given)
template <typename T>
__global__ __launch_bounds__(128) void k_epilogue(const float* __restrict__ olat,
                                                  const T* __restrict__ w_uv,
                                                  const T* __restrict__ gate, T* __restrict__ out,
                                                  int B, int H, int NB, int dcb, int dv,
                                                  float out_scale, int Hw) {
  extern __shared__ float so[];  // [kBatchBlock][dc]
  const int h = blockIdx.x;
  const int b0 = blockIdx.y * kBatchBlock;
  const int nb = min(kBatchBlock, B - b0);
  const int dc = NB * dcb;
  for (int i = threadIdx.x; i < kBatchBlock * dc; i += blockDim.x) {
    const int j = i / dc, d = i % dc;
    so[i] = j < nb ? olat[((size_t)(b0 + j) * H + h) * dc + d] : 0.0f;
  }
  __syncthreads();
  for (int v = threadIdx.x; v < dv; v += blockDim.x) {
    float acc[kBatchBlock];
#pragma unroll
    for (int j = 0; j < kBatchBlock; ++j) acc[j] = 0.0f;
    for (int br = 0; br < NB; ++br) {
      const T* w = w_uv + ((size_t)br * Hw + h % Hw) * dcb * dv + v;
      const float* o = so + br * dcb;
      for (int c = 0; c < dcb; ++c) {
        const float wv = to_f32(w[(size_t)c * dv]);
#pragma unroll
        for (int j = 0; j < kBatchBlock; ++j) acc[j] = fmaf(o[j * dc + c], wv, acc[j]);
      }
    }
    for (int j = 0; j < nb; ++j) {
      const size_t o = ((size_t)(b0 + j) * H + h) * dv + v;
      const float g = gate ? 1.0f / (1.0f + expf(-to_f32(gate[o]))) : 1.0f;
      out[o] = from_f32<T>(acc[j] * out_scale * g);
    }
  }
}

hipError_t launch_epilogue(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(p.H, (p.B + kBatchBlock - 1) / kBatchBlock);
  const size_t lds = (size_t)kBatchBlock * p.dc * sizeof(float);
  hipLaunchKernelGGL(k_epilogue<float>, grid, dim3(128), lds, s, (const float*)a.olat,
                     (const float*)a.w_uv, (const float*)a.gate, (float*)a.out, p.B, p.H, p.NB,
                     p.dcb, p.dv, a.out_scale, p.Hw);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- rope rotate
// RoFormer rotation of consecutive pairs by pos * theta^(-2k/d_rope) (angle reduced in fp64).
template <typename T>
__global__ __launch_bounds__(256) void k_rope_rotate(T* __restrict__ x, int64_t row_stride,
                                                     const int32_t* __restrict__ pos, int64_t n,
                                                     int dr, RopeFreq rf) {
  const int half = dr / 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * half) return;
  const int64_t r = i / half;
  const int k = (int)(i % half);
  const int p = pos[r];
  if (p < 0) return;
  float cs, sn;
  rope_cos_sin(p, rf.f[k], &cs, &sn);
  T* px = x + r * row_stride + 2 * k;
  const float x0 = to_f32(px[0]), x1 = to_f32(px[1]);
  px[0] = from_f32<T>(x0 * cs - x1 * sn);
  px[1] = from_f32<T>(x0 * sn + x1 * cs);
}

hipError_t launch_rope_rotate(void* x, int64_t row_stride, const int32_t* pos, int64_t n_rows,
                              int d_rope, float theta, int dtype, hipStream_t s) {
  const int64_t work = n_rows * (d_rope / 2);
  const dim3 grid((unsigned)((work + 255) / 256));
  RopeFreq rf;
  make_rope_freq(d_rope, theta, &rf);
  if (dtype == MLA_BF16)
    hipLaunchKernelGGL(k_rope_rotate<bf16>, grid, dim3(256), 0, s, (bf16*)x, row_stride, pos,
                       n_rows, d_rope, rf);
  else
    hipLaunchKernelGGL(k_rope_rotate<float>, grid, dim3(256), 0, s, (float*)x, row_stride, pos,
                       n_rows, d_rope, rf);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- fp32 main loop
// Generic SIMT split-K loop for small fp32 shapes: one wave per (work item, head).
// Lane t of a 64-token tile computes that token's scores for every branch; the online
// softmax keeps (m, l) per branch; lane d accumulates latent-space output columns.
__global__ __launch_bounds__(64) void k_main_f32(
    const float* __restrict__ qcat, const float* __restrict__ latent,
    const float* __restrict__ rope, int64_t lat_tok, int64_t lat_seq, int64_t rope_tok,
    int64_t rope_seq, const int32_t* __restrict__ work, const int32_t* __restrict__ bt,
    int64_t bt_stride, int paged, float* __restrict__ part_o, float* __restrict__ part_ml, int H,
    int NB, int dcb, int dr, const int32_t* __restrict__ seqlens, int max_seqlen, int nq,
    int Hw) {
  __shared__ float sq[512 + 64];
  __shared__ float sp[64 * 4];
  const int h = blockIdx.x % H;
  const int slot = blockIdx.x / H;  // slot s runs work item s
  const int b = work[4 * slot];
  if (b < 0) return;
  // tokens [t0, t1) of the item, cut at this row's causal limit (s_q > 1 query tokens)
  const int t0 = work[4 * slot + 1];
  const int t1 = min(work[4 * slot + 2], causal_limit(seqlens, b, max_seqlen, nq, h / Hw));
  const size_t item = (size_t)work[4 * slot + 3];
  const int lane = threadIdx.x;
  const int dc = NB * dcb, row = dc + dr;
  float* ml = part_ml + item * NB * H * 2;
  for (int i = lane; i < row; i += 64) sq[i] = qcat[((size_t)b * H + h) * row + i];
  __syncthreads();
  auto lat_row = [&](int t) -> const float* {
    if (paged) return latent + (int64_t)bt[(int64_t)b * bt_stride + t / 64] * lat_seq + (t % 64) * lat_tok;
    return latent + (int64_t)b * lat_seq + (int64_t)t * lat_tok;
  };
  auto rope_row = [&](int t) -> const float* {
    if (paged) return rope + (int64_t)bt[(int64_t)b * bt_stride + t / 64] * rope_seq + (t % 64) * rope_tok;
    return rope + (int64_t)b * rope_seq + (int64_t)t * rope_tok;
  };
  float m[4], l[4], alpha[4];
  for (int br = 0; br < 4; ++br) { m[br] = -INFINITY; l[br] = 0.0f; alpha[br] = 1.0f; }
  float o[8];
  for (int k = 0; k < 8; ++k) o[k] = 0.0f;
  for (int tile = t0; tile < t1; tile += 64) {
    const int t = tile + lane;
    const bool valid = t < t1;
    float sc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (valid) {
      const float* lr = lat_row(t);
      const float* rr = rope_row(t);
      float rs = 0.0f;
      for (int i = 0; i < dr; ++i) rs = fmaf(sq[dc + i], rr[i], rs);
      for (int br = 0; br < NB; ++br) {
        float acc = rs;
        for (int c = 0; c < dcb; ++c) acc = fmaf(sq[br * dcb + c], lr[br * dcb + c], acc);
        sc[br] = acc;
      }
    }
    for (int br = 0; br < NB; ++br) {
      const float mx = wave_max(sc[br]);
      const float mn = fmaxf(m[br], mx);
      alpha[br] = exp2f(m[br] - mn);
      const float pv = valid ? exp2f(sc[br] - mn) : 0.0f;
      l[br] = alpha[br] * l[br] + wave_sum(pv);
      m[br] = mn;
      sp[lane * 4 + br] = pv;
    }
    __syncthreads();
    const int nt = min(64, t1 - tile);
    for (int k = 0; k < 8; ++k) {
      const int d = lane + 64 * k;
      if (d >= dc) break;
      const int br = d / dcb;
      float acc = o[k] * alpha[br];
      for (int j = 0; j < nt; ++j) acc = fmaf(sp[j * 4 + br], lat_row(tile + j)[d], acc);
      o[k] = acc;
    }
    __syncthreads();
  }
  for (int k = 0; k < 8; ++k) {
    const int d = lane + 64 * k;
    if (d >= dc) break;
    part_o[(item * H + h) * dc + d] = o[k];
  }
  if (lane < NB) {
    ml[((size_t)lane * H + h) * 2 + 0] = m[lane];
    ml[((size_t)lane * H + h) * 2 + 1] = l[lane];
  }
}

hipError_t launch_main_f32(const Plan& p, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)p.slots * p.H));
  hipLaunchKernelGGL(k_main_f32, grid, dim3(64), 0, s, (const float*)a.qcat,
                     (const float*)a.latent, (const float*)a.rope, a.lat_tok, a.lat_seq,
                     a.rope_tok, a.rope_seq, a.work, a.block_table, a.bt_stride, p.paged,
                     (float*)a.part_o, a.part_ml, p.H, p.NB, p.dcb, p.dr, a.seqlens,
                     p.max_seqlen, p.sq, p.Hw);
  return hipGetLastError();
}

}  // namespace mla
