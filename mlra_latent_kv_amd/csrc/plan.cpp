// Validation and split plan; see plan.h.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <climits>
#include <cstdint>

namespace mla {
namespace {

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

}  // namespace

mla_status make_plan(const mla_params* p, Plan* plan) {
  if (!p || !plan) return MLA_ERR_NULL;
  if (p->dtype != MLA_F32 && p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (p->batch < 1 || p->num_heads < 1 || p->num_branches < 1 || p->d_nope < 1 || p->d_v < 1 ||
      p->d_latent < 1 || p->d_rope < 2 || (p->d_rope & 1) || p->max_seqlen < 0 ||
      p->num_splits < 0)
    return MLA_ERR_SHAPE;
  if (p->batch > (1 << 20) || p->num_heads > 4096 || p->max_seqlen > (1 << 26))
    return MLA_ERR_SHAPE;
  if (!std::isfinite(p->softmax_scale) || !std::isfinite(p->out_scale) ||
      !(p->rope_theta > 0.0f) || !std::isfinite(p->rope_theta))
    return MLA_ERR_SHAPE;
  if (p->page_size != 0 && p->page_size != kPage) return MLA_ERR_UNSUPPORTED;

  Plan q{};
  q.B = p->batch;
  q.H = p->num_heads;
  q.NB = p->num_branches;
  q.dcb = p->d_latent;
  q.dc = q.NB * q.dcb;
  q.dr = p->d_rope;
  q.dn = p->d_nope;
  q.dv = p->d_v;
  q.row = q.dc + q.dr;
  q.dtype = p->dtype;
  q.elem = p->dtype == MLA_F32 ? 4 : 2;
  q.paged = p->page_size == kPage;
  q.max_seqlen = p->max_seqlen;

  if (p->dtype == MLA_BF16) {
    const bool mla = q.NB == 1 && q.dcb == 512;
    const bool mlra = q.NB == 4 && q.dcb == 128;
    if (!(mla || mlra) || q.dr != 64 || q.dn != 128 || q.dv != 128 || q.H % kHeadGroup)
      return MLA_ERR_UNSUPPORTED;
    q.path = Path::kBf16Mfma;
    q.n_hg = q.H / kHeadGroup;
    q.wide = mla && q.H % kWideHeads == 0;
  } else {
    if ((q.NB != 1 && q.NB != 4) || q.dc > 512 || q.dr > 64 || q.dn > 256 || q.dv > 256)
      return MLA_ERR_UNSUPPORTED;
    q.path = Path::kF32Simt;
    q.n_hg = 0;
    q.wide = 0;
  }

  // strides
  if (p->latent_stride_tok < q.dc || p->rope_stride_tok < q.dr || p->latent_stride_seq < 0 ||
      p->rope_stride_seq < 0)
    return MLA_ERR_SHAPE;
  if (p->dtype == MLA_BF16 &&
      ((p->latent_stride_tok | p->latent_stride_seq | p->rope_stride_tok | p->rope_stride_seq) % 8))
    return MLA_ERR_ALIGN;
  q.n_tiles = (int)std::max<int64_t>(1, ceil_div(q.max_seqlen, kPage));
  if (q.paged) {
    if (p->max_pages_per_seq < ceil_div(q.max_seqlen, kPage) ||
        p->block_table_stride < p->max_pages_per_seq)
      return MLA_ERR_SHAPE;
  }

  // Split plan.  The device cuts sum_b ceil(L_b / 64) pages into work items of c whole pages
  // each (a sequence of p_b pages gets ceil(p_b / c) items).  Automatic: c is the smallest
  // count that keeps the items within `target` (enough workgroups to fill the chip once),
  // one item per sequence if none does; forced: c = ceil(n_tiles / num_splits).
  const int64_t wg_per_item = q.path != Path::kBf16Mfma ? q.H
                              : q.wide ? q.H / kWideHeads
                                       : q.n_hg;
  const int64_t target_wg = q.wide ? kTargetWideWorkgroups : kTargetWorkgroups;
  q.target = (int)std::max<int64_t>(1, ceil_div(target_wg, wg_per_item));
  q.xcd_major = q.wide;
  int64_t cap;
  if (p->num_splits > 0) {
    if (p->num_splits > q.n_tiles) return MLA_ERR_SHAPE;
    q.forced_pages = (int)ceil_div(q.n_tiles, p->num_splits);
    q.splits = (int)ceil_div(q.n_tiles, q.forced_pages);
    if (q.splits > kMaxSplits) return MLA_ERR_SHAPE;
    cap = (int64_t)q.B * q.splits;
  } else {
    // W <= target whenever some c meets it; otherwise one item per non-empty sequence
    q.forced_pages = 0;
    q.splits = std::min(q.n_tiles, q.target);
    cap = std::max<int64_t>(q.target, q.B);
  }
  // grid sizes and 32-bit work-item indices must fit
  if (cap + 8 > INT32_MAX / 4 || wg_per_item * (cap + 8) + 8LL * std::max(q.n_hg, 1) > INT32_MAX ||
      (int64_t)q.B * q.H > INT32_MAX)
    return MLA_ERR_SHAPE;
  q.items_cap = (int)cap;
  q.slots = (int)ceil_div(cap, 8) * 8;

  // workspace: plan, absorbed queries, per-item partials, fp32 merged latent
  size_t off = 0;
  q.off_work = 16;  // after the 4-word header
  q.off_split_off = q.off_work + (size_t)q.slots * 16;
  off = align_up(q.off_split_off + ((size_t)q.B + 1) * 4);
  q.off_qcat = off;
  off = align_up(off + (size_t)q.B * q.H * q.row * q.elem);
  q.off_part_o = off;
  off = align_up(off + (size_t)q.items_cap * q.H * q.dc * (q.dtype == MLA_BF16 ? 2 : 4));
  q.off_part_ml = off;
  off = align_up(off + (size_t)q.items_cap * q.NB * q.H * 2 * sizeof(float));
  q.off_olat = off;  // merged latent output: fp32 path only (bf16 keeps it on chip)
  if (q.dtype != MLA_BF16) off = align_up(off + (size_t)q.B * q.H * q.dc * 4);
  q.bytes = off;
  *plan = q;
  return MLA_OK;
}

mla_status check_call(const mla_params* p, const Plan& plan, int want_branches,
                      const void* q_nope, const void* q_rope, const void* latent,
                      const void* rope, const int32_t* seqlens, const int32_t* block_table,
                      const void* w_uk, const void* w_uv, const void* out,
                      const void* workspace, size_t workspace_bytes) {
  if (plan.NB != want_branches) return MLA_ERR_UNSUPPORTED;
  if (!q_nope || !q_rope || !latent || !rope || !seqlens || !w_uk || !w_uv || !out || !workspace)
    return MLA_ERR_NULL;
  if (plan.paged && !block_table) return MLA_ERR_NULL;
  if (workspace_bytes < plan.bytes) return MLA_ERR_WORKSPACE;
  const size_t ea = (size_t)plan.elem;
  if (!aligned(workspace, kWsAlign) || !aligned(seqlens, 4) || (plan.paged && !aligned(block_table, 4)))
    return MLA_ERR_ALIGN;
  if (!aligned(q_nope, ea) || !aligned(q_rope, ea) || !aligned(w_uk, ea) || !aligned(w_uv, ea) ||
      !aligned(out, ea))
    return MLA_ERR_ALIGN;
  const size_t cache_align = plan.dtype == MLA_BF16 ? 16 : 4;
  if (!aligned(latent, cache_align) || !aligned(rope, cache_align)) return MLA_ERR_ALIGN;
  // the bf16 kernels read the query and both weights with 16-byte vector loads
  if (plan.dtype == MLA_BF16 && (!aligned(q_nope, 16) || !aligned(w_uk, 16) || !aligned(w_uv, 16)))
    return MLA_ERR_ALIGN;
  (void)p;
  return MLA_OK;
}

mla_status check_rope_rotate(const void* x, int64_t row_stride, const int32_t* pos,
                             int64_t n_rows, int32_t d_rope, float theta, int32_t dtype) {
  if (dtype != MLA_F32 && dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (n_rows < 0 || d_rope < 2 || d_rope > 256 || (d_rope & 1) || row_stride < d_rope ||
      !(theta > 0.0f) || !std::isfinite(theta))
    return MLA_ERR_SHAPE;
  if (n_rows == 0) return MLA_OK;
  if (!x || !pos) return MLA_ERR_NULL;
  if (!aligned(x, dtype == MLA_F32 ? 4 : 2) || !aligned(pos, 4)) return MLA_ERR_ALIGN;
  return MLA_OK;
}

const char* status_str(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: inconsistent size, stride or bound";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: no kernel for these dims/layout";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace smaller than mla_workspace_size";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown dtype";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: pointer or stride misaligned";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown mla_status";
  }
}

}  // namespace mla
