// Write side of the latent cache: one decode step's new token per sequence, compressed and
// appended ("超越 GQA 的推理革命…MLA…", section 鍵值聯合低秩壓縮: at write time the token is
// compressed into the joint low-rank latent c_KV; section 解耦旋轉位置編碼: the position part
// is a separate uncompressed key that carries RoPE).  For every sequence b, with t = seqlens[b]:
//   row = [ h_b W_DKV | RoPE(h_b W_KR, t) ]      (bf16 storage, fp32 accumulation)
// goes to cache position t (a paged cache takes a new page from the free list when t starts
// one), and seqlens[b] becomes t + 1.
//
// Two launches:
//  * k_append_proj: the projection [h] . [W_DKV | W_KR] as a split-K MFMA GEMM.  The weights
//    are the bytes that matter (d_model x 576 bf16, 4.7 MB at d_model 4096); each workgroup
//    takes a 256-deep K chunk of 128 output columns, stages that W block in LDS once (all of
//    its loads in flight together; read back transposed as the MFMA operand), and writes fp32
//    partials for every 32-row block of the batch.  One extra workgroup ranks the sequences
//    that need a new page (an exclusive scan in batch order).
//  * k_append_write: one workgroup per sequence: its four waves sum a quarter of the K-chunk
//    partials each (loads of up to four chunks in flight at once), the sums meet in LDS, and
//    the first wave rotates the rotary part at position t (angle reduced in fp64), rounds to
//    bf16 (the latent part of an fp8 cache: encodes it as E4M3 codes of value / scale), takes
//    its page and writes the row, then bumps the length.  Each sequence touches
//    only its own block-table entry and length, so the launch has no races.
#include <climits>

#include "append.h"
#include "device_common.h"
#include "launch.h"
#include "plan_device.h"
#include "tile_bf16.h"

namespace mla {
namespace {

constexpr int kKc = 256;       // K (d_model) per workgroup
constexpr int kColsWG = 128;   // output columns per workgroup (32 per wave)
constexpr int kRowsWG = 32;    // batch rows per workgroup
constexpr int kWPitch = kColsWG + 8;  // LDS pitch of the W block (bf16)

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 8 consecutive rows (k) of one column of a row-major LDS block as an MFMA operand (lane%32 =
// column, lane/32 = which 8-row half), from two transposed reads
__device__ __forceinline__ bf16x8 tr8(const bf16* p, int pitch) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * pitch));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__global__ __launch_bounds__(256) void k_append_proj(const bf16* __restrict__ hidden,
                                                     const bf16* __restrict__ w_dkv,
                                                     const bf16* __restrict__ w_kr,
                                                     const int32_t* __restrict__ seqlens,
                                                     AppendWs ws, int B, int d_model, int dc,
                                                     int page_size, int n_free) {
  __shared__ __align__(16) bf16 sW[kKc * kWPitch];  // 68 KB
  const int cb = blockIdx.x, kc = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ncol = dc + 64;
  if (cb == (int)gridDim.x - 1) {
    // the extra column of workgroups: (0, 0) ranks the sequences that need a page
    if (kc == 0) {
      int* wsum = reinterpret_cast<int*>(sW);
      const long long total = plan_detail::block_scan(
          B,
          [&](int b, int) {
            const int t = seqlens[b];
            return page_size && t >= 0 && t % page_size == 0 ? 1 : 0;
          },
          [&](int b, long long off) { ws.rank[b] = (int)off; }, wsum);
      if (tid == 0) ws.pages_used[0] = (int)(total < n_free ? total : n_free);
    }
    return;
  }
  const int c0 = cb * kColsWG;           // first output column of the workgroup
  const int k0 = kc * kKc;
  // W block [kKc x 128] row-major into LDS: output column c < dc is W_DKV[:, c], else
  // W_KR[:, c - dc]; columns past dc + 64 are zeros.  Thread t copies 16-byte chunks
  // (8 columns of one k row), all 16 of its loads in flight before the first LDS store; a
  // chunk never straddles the W_DKV / W_KR border (dc is a multiple of 128 and 8 | 64).
  constexpr int kChunks = kKc * (kColsWG / 8) / 256;  // per thread
  u32x4 wv[kChunks];
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int i = tid + 256 * j;
    const int r = i / (kColsWG / 8), c = c0 + (i % (kColsWG / 8)) * 8;
    wv[j] = u32x4{0, 0, 0, 0};
    if (c < dc)
      wv[j] = *(const u32x4*)(w_dkv + (size_t)(k0 + r) * dc + c);
    else if (c < ncol)
      wv[j] = *(const u32x4*)(w_kr + (size_t)(k0 + r) * 64 + (c - dc));
  }
  // A operand: hidden rows b0 + lane%32 (clamped: rows past B are computed, never stored),
  // K-step s covers k0 + 16s + 8*(lane/32) .. +8
  const int bl = lane & 31, kg = lane >> 5;
  bf16x8 a[kKc / 16];
  auto load_a = [&](int b0) {
    const bf16* hrow = hidden + (size_t)min(b0 + bl, B - 1) * d_model + k0 + 8 * kg;
#pragma unroll
    for (int s = 0; s < kKc / 16; ++s) a[s] = *(const bf16x8*)(hrow + 16 * s);
  };
  load_a(0);
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int i = tid + 256 * j;
    *(u32x4*)(sW + (i / (kColsWG / 8)) * kWPitch + (i % (kColsWG / 8)) * 8) = wv[j];
  }
  __syncthreads();
  // B operand: wave w's 32 columns; source lane of ds_read_b64_tr_b16: row 8*(lane/32) +
  // (lane%16)/4, column 16*((lane/16)%2) + 4*(lane%4) of the 32-column block
  const bf16* tsrc = sW + (8 * (lane >> 5) + ((lane & 15) >> 2)) * kWPitch + 32 * w +
                     16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int col = c0 + 32 * w + (lane & 31);
  float* part = ws.part + (size_t)kc * B * ncol;
  for (int b0 = 0; b0 < B; b0 += kRowsWG) {
    if (b0 > 0) load_a(b0);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < kKc / 16; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], tr8(tsrc + 16 * s * kWPitch, kWPitch),
                                                    acc, 0, 0, 0);
    // D[i = batch row][j = column]: lane%32 = column, item i -> row 8*(i/4) + 4*kg + i%4
    if (col < ncol) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int b = b0 + 8 * (i >> 2) + 4 * kg + (i & 3);
        if (b < B) part[(size_t)b * ncol + col] = acc[i];
      }
    }
  }
}

// One workgroup (4 waves) per sequence b.  Lane l of every wave owns the row's columns l,
// l + 64, ...; wave w sums the K-chunk partials kc = w, w + 4, ..., and the first wave adds
// the four sums.  The rotary pairs (2k, 2k + 1) of the last 64 columns are lanes 2k and 2k + 1
// of the last group.
// OCP FP8 E4M3 code of x (nearest, ties to the even code, saturating at +-448; x finite):
// below 2^-6 the grid is subnormal with step 2^-9, above it 3 mantissa bits, rounded on the
// fp32 bit pattern
__device__ __forceinline__ uint8_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a < 448.0f)) return (uint8_t)(sign | 0x7eu);
  if (a < 0.015625f) return (uint8_t)(sign | (uint32_t)rintf(a * 512.0f));  // 0 .. 8
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = (u + 0x7ffffu + ((u >> 20) & 1u)) >> 20;  // exponent and 3 mantissa bits
  const uint32_t code = r - ((127u - 7u) << 3);                // rebias 127 -> 7
  return (uint8_t)(sign | (code > 0x7eu ? 0x7eu : code));
}

// F8: the latent part is written as E4M3 codes of value / latent_scale (latent counts bytes)
template <bool F8>
__global__ __launch_bounds__(256) void k_append_write(
    AppendWs ws, int32_t* __restrict__ seqlens, int32_t* __restrict__ block_table,
    const int32_t* __restrict__ free_pages, int n_free, void* __restrict__ latent,
    bf16* __restrict__ rope, int64_t lat_tok, int64_t lat_seq, int64_t rope_tok,
    int64_t rope_seq, int64_t bt_stride, int B, int dc, int n_kc, int page_size, int max_pages,
    int capacity, RopeFreq rf, float latent_scale) {
  __shared__ float red[3][9][64];
  const int b = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ncol = dc + 64;
  const int t = seqlens[b];
  // where the row goes; a position outside the cache's capacity, or a new page that the free
  // list cannot supply, leaves the sequence untouched
  int64_t slot_lat = -1, slot_rope = -1;
  int new_page = -1;
  if (t >= 0) {
    if (page_size) {
      const int j = t / page_size;
      if (j < max_pages) {
        int pg = -1;
        if (t % page_size == 0) {
          const int r = ws.rank[b];
          if (r < n_free) pg = new_page = free_pages[r];
        } else {
          pg = block_table[(int64_t)b * bt_stride + j];
        }
        if (pg >= 0) {
          slot_lat = (int64_t)pg * lat_seq + (int64_t)(t % page_size) * lat_tok;
          slot_rope = (int64_t)pg * rope_seq + (int64_t)(t % page_size) * rope_tok;
        }
      }
    } else if (t < capacity) {
      slot_lat = (int64_t)b * lat_seq + (int64_t)t * lat_tok;
      slot_rope = (int64_t)b * rope_seq + (int64_t)t * rope_tok;
    }
  }
  if (slot_lat < 0) return;  // uniform: every lane read the same t, rank and table entry
  // sum of the K-chunk partials for this row: wave w takes chunks w, w + 4, ..., four at a
  // time with all their loads in flight (a chunk past n_kc reads chunk w, weighted 0)
  const float* part = ws.part + (size_t)b * ncol;
  const int n_grp = ncol / 64;  // 9 (d_c = 512) or 3 (d_c = 128)
  float v[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) v[i] = 0.0f;
  for (int kc0 = w; kc0 < n_kc; kc0 += 16) {
    float x[4][9];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kc = kc0 + 4 * u < n_kc ? kc0 + 4 * u : w;
      const float* p = part + (size_t)kc * B * ncol;
#pragma unroll
      for (int i = 0; i < 9; ++i) x[u][i] = i < n_grp ? p[64 * i + lane] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 9; ++i)
        if (kc0 + 4 * u < n_kc) v[i] += x[u][i];
  }
  if (w > 0) {
#pragma unroll
    for (int i = 0; i < 9; ++i) red[w - 1][i][lane] = v[i];
  }
  __syncthreads();
  if (w > 0) return;
#pragma unroll
  for (int i = 0; i < 9; ++i) v[i] += red[0][i][lane] + red[1][i][lane] + red[2][i][lane];
  // latent columns
#pragma unroll
  for (int i = 0; i < 9; ++i)
    if (i < n_grp - 1) {
      if constexpr (F8)
        static_cast<uint8_t*>(latent)[slot_lat + 64 * i + lane] = e4m3_code(v[i] / latent_scale);
      else
        static_cast<bf16*>(latent)[slot_lat + 64 * i + lane] = (bf16)v[i];
    }
  // rotary columns (the last group): pair k = lane / 2 turned by t theta^(-2k/64)
  float x = 0.0f;
#pragma unroll
  for (int i = 0; i < 9; ++i)
    if (i == n_grp - 1) x = v[i];
  const float partner = __shfl_xor(x, 1, 64);
  float cs, sn;
  rope_cos_sin(t, rf.f[lane >> 1], &cs, &sn);
  const float x0 = (lane & 1) ? partner : x, x1 = (lane & 1) ? x : partner;
  const float y = (lane & 1) ? (x0 * sn + x1 * cs) : (x0 * cs - x1 * sn);
  rope[slot_rope + lane] = (bf16)y;
  if (lane == 0) {
    if (new_page >= 0) block_table[(int64_t)b * bt_stride + t / page_size] = new_page;
    seqlens[b] = t + 1;
  }
}

}  // namespace

hipError_t launch_append(const AppendPlan& p, const AppendArgs& a, hipStream_t s) {
  const dim3 grid(p.n_cb + 1, p.n_kc);
  hipLaunchKernelGGL(k_append_proj, grid, dim3(256), 0, s, (const bf16*)a.hidden,
                     (const bf16*)a.w_dkv, (const bf16*)a.w_kr, a.seqlens, a.ws, p.B, p.d_model,
                     p.dc, p.page_size, a.n_free);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  RopeFreq rf;
  make_rope_freq(64, a.rope_theta, &rf);
  hipLaunchKernelGGL(p.f8 ? k_append_write<true> : k_append_write<false>, dim3(p.B), dim3(256),
                     0, s, a.ws, a.seqlens, a.block_table, a.free_pages, a.n_free, a.latent,
                     (bf16*)a.rope, a.lat_tok, a.lat_seq, a.rope_tok, a.rope_seq, a.bt_stride, p.B,
                     p.dc, p.n_kc, p.page_size, p.max_pages, p.capacity, rf, p.latent_scale);
  return hipGetLastError();
}

}  // namespace mla
