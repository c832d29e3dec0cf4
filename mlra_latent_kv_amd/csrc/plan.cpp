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

mla_status make_plan(const mla_params* p, Plan* plan, int n_cu) {
  if (!p || !plan) return MLA_ERR_NULL;
  if (p->dtype != MLA_F32 && p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (p->batch < 1 || p->num_heads < 1 || p->num_branches < 1 || p->d_nope < 1 || p->d_v < 1 ||
      p->d_latent < 1 || p->d_rope < 2 || (p->d_rope & 1) || p->max_seqlen < 0 ||
      p->num_splits < 0 || p->num_pages < 0 || p->num_queries < 0 || p->num_queries > 16)
    return MLA_ERR_SHAPE;
  if (p->latent_format != 0 && p->latent_format != MLA_LATENT_FP8) return MLA_ERR_DTYPE;
  if (p->latent_format == MLA_LATENT_FP8 &&
      (p->dtype != MLA_BF16 || !std::isfinite(p->latent_scale) || !(p->latent_scale > 0.0f)))
    return p->dtype != MLA_BF16 ? MLA_ERR_UNSUPPORTED : MLA_ERR_SHAPE;
  if (p->flags & ~(MLA_FLAG_DEVICE_CHECKS | MLA_FLAG_QUERY_LATENT | MLA_FLAG_OUTPUT_LATENT))
    return MLA_ERR_SHAPE;
  if (p->batch > (1 << 20) || p->num_heads > 4096 || p->max_seqlen > (1 << 26))
    return MLA_ERR_SHAPE;
  if (!std::isfinite(p->softmax_scale) || !std::isfinite(p->out_scale) ||
      !(p->rope_theta > 0.0f) || !std::isfinite(p->rope_theta))
    return MLA_ERR_SHAPE;
  if (p->page_size != 0 && p->page_size != kPage) return MLA_ERR_UNSUPPORTED;

  Plan q{};
  q.B = p->batch;
  q.sq = p->num_queries > 1 ? p->num_queries : 1;
  q.Hw = p->num_heads;
  q.H = q.sq * q.Hw;  // query rows: every (token, head) pair
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
  q.n_cu = (n_cu <= 0 || n_cu > kMaxCUs) ? kMaxCUs : n_cu;
  q.checks = (p->flags & MLA_FLAG_DEVICE_CHECKS) ? 1 : 0;
  q.num_pages = q.paged ? p->num_pages : 0;
  q.latent_q = (p->flags & MLA_FLAG_QUERY_LATENT) ? 1 : 0;
  q.latent_out = (p->flags & MLA_FLAG_OUTPUT_LATENT) ? 1 : 0;
  q.f8 = p->latent_format == MLA_LATENT_FP8 ? 1 : 0;
  // the folded forms leave out the dims of the product they skip
  const bool dn_ok = q.latent_q || q.dn == 128, dv_ok = q.latent_out || q.dv == 128;

  if (p->dtype == MLA_BF16) {
    // MLA (latent 512), MLRA-4 (four branches of 128), and one MLRA branch on its own
    // (latent 128: a tensor-parallel shard of MLRA-4)
    const bool mla = q.NB == 1 && q.dcb == 512;
    const bool shard = q.NB == 1 && q.dcb == 128;
    const bool mlra = q.NB == 4 && q.dcb == 128;
    // every 32-head group (and, with 128-row quads, every wave) within one query token
    if (!(mla || shard || mlra) || q.dr != 64 || !dn_ok || !dv_ok || q.Hw % kHeadGroup)
      return MLA_ERR_UNSUPPORTED;
    q.path = Path::kBf16Mfma;
    q.n_hg = q.H / kHeadGroup;
    // (an fp8 latent runs on the 32-head kernel, which widens each tile once in LDS)
    q.wide = mla && q.H % kWideHeads == 0 && !q.f8;
  } else {
    if ((q.NB != 1 && q.NB != 4) || q.dc > 512 || q.dr > 64 || (!q.latent_q && q.dn > 256) ||
        (!q.latent_out && q.dv > 256))
      return MLA_ERR_UNSUPPORTED;
    q.path = Path::kF32Simt;
    q.n_hg = 0;
    q.wide = 0;
  }

  // strides
  if (p->latent_stride_tok < q.dc || p->rope_stride_tok < q.dr || p->latent_stride_seq < 0 ||
      p->rope_stride_seq < 0)
    return MLA_ERR_SHAPE;
  // 16-byte rows: 8 bf16 elements, or 16 fp8 codes for an fp8 latent
  if (p->dtype == MLA_BF16 &&
      ((p->latent_stride_tok | p->latent_stride_seq) % (q.f8 ? 16 : 8) ||
       (p->rope_stride_tok | p->rope_stride_seq) % 8))
    return MLA_ERR_ALIGN;
  q.n_tiles = (int)std::max<int64_t>(1, ceil_div(q.max_seqlen, kPage));
  if (q.paged) {
    if (p->max_pages_per_seq < ceil_div(q.max_seqlen, kPage) ||
        p->block_table_stride < p->max_pages_per_seq)
      return MLA_ERR_SHAPE;
  }

  // Split plan.  Page plan: the device cuts sum_b ceil(L_b / 64) pages into work items of c
  // whole pages each (a sequence of p_b pages gets ceil(p_b / c) items), one per dispatch
  // slot.  Automatic: c is the smallest count that keeps the items within `target` (enough
  // workgroups to fill the chip once), one item per sequence if none does; forced:
  // c = ceil(n_tiles / num_splits).
  const int64_t wg_per_item = q.path != Path::kBf16Mfma ? q.H
                              : q.wide ? q.H / kWideHeads
                                       : q.n_hg;
  // workgroups that fill the chip once: the wide kernel holds one per CU, the 32-head kernel
  // on 192-wide rows kNarrowWgPerCu, the others two
  const bool narrow = q.path == Path::kBf16Mfma && q.NB == 1 && q.dcb == 128;
  const int64_t target_wg = q.wide ? q.n_cu
                            : narrow ? (int64_t)kNarrowWgPerCu * q.n_cu
                                     : 2 * (int64_t)q.n_cu;
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
  q.off_work = 4 * kHdrWords;
  q.off_slot_end = q.off_work + (size_t)q.slots * 16;
  q.off_items = q.off_slot_end + (size_t)q.slots * 4;
  q.off_split_off = q.off_items + (size_t)q.items_cap * 16;
  q.off_dbg = q.off_split_off + ((size_t)q.B + 1) * 4;
  off = align_up(q.off_dbg + (size_t)q.B * 4);
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
                      const void* workspace, size_t workspace_bytes, bool gated,
                      const void* gate) {
  if (plan.NB != want_branches) return MLA_ERR_UNSUPPORTED;
  if (gated && plan.latent_out) return MLA_ERR_UNSUPPORTED;  // the gate acts on d_v outputs
  // the folded forms do not read the weight they replace
  const bool need_uk = !plan.latent_q, need_uv = !plan.latent_out;
  if (!q_nope || !q_rope || !latent || !rope || !seqlens || (need_uk && !w_uk) ||
      (need_uv && !w_uv) || !out || !workspace || (gated && !gate))
    return MLA_ERR_NULL;
  if (plan.paged && !block_table) return MLA_ERR_NULL;
  if (workspace_bytes < plan.bytes) return MLA_ERR_WORKSPACE;
  const size_t ea = (size_t)plan.elem;
  if (!aligned(workspace, kWsAlign) || !aligned(seqlens, 4) || (plan.paged && !aligned(block_table, 4)))
    return MLA_ERR_ALIGN;
  if (!aligned(q_nope, ea) || !aligned(q_rope, ea) || (need_uk && !aligned(w_uk, ea)) ||
      (need_uv && !aligned(w_uv, ea)) || !aligned(out, ea) || (gated && !aligned(gate, ea)))
    return MLA_ERR_ALIGN;
  const size_t cache_align = plan.dtype == MLA_BF16 ? 16 : 4;
  if (!aligned(latent, cache_align) || !aligned(rope, cache_align)) return MLA_ERR_ALIGN;
  // the bf16 kernels read the query, both weights and the gate, and write the output, with
  // 16-byte vector accesses
  if (plan.dtype == MLA_BF16 &&
      (!aligned(q_nope, 16) || (need_uk && !aligned(w_uk, 16)) || (need_uv && !aligned(w_uv, 16)) ||
       (gated && !aligned(gate, 16)) || !aligned(out, 16)))
    return MLA_ERR_ALIGN;
  (void)p;
  return MLA_OK;
}

mla_status make_prefill_plan(const mla_params* p, PrefillPlan* plan, int n_cu) {
  if (!p || !plan) return MLA_ERR_NULL;
  if (p->dtype != MLA_F32 && p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (p->latent_format != 0 && p->latent_format != MLA_LATENT_FP8) return MLA_ERR_DTYPE;
  if (p->batch < 1 || p->num_heads < 1 || p->num_branches < 1 || p->d_nope < 1 || p->d_v < 1 ||
      p->d_latent < 1 || p->d_rope < 2 || (p->d_rope & 1) || p->max_seqlen < 0 ||
      p->num_queries < 0 || p->num_pages < 0)
    return MLA_ERR_SHAPE;
  if (p->flags & ~(MLA_FLAG_DEVICE_CHECKS | MLA_FLAG_QUERY_LATENT | MLA_FLAG_OUTPUT_LATENT))
    return MLA_ERR_SHAPE;
  // grid dimensions (sequences, heads) and 32-bit token indices
  if (p->batch > 65535 || p->num_heads > 4096 || p->max_seqlen > (1 << 24) ||
      p->num_queries > (1 << 24))
    return MLA_ERR_SHAPE;
  if (!std::isfinite(p->softmax_scale) || !std::isfinite(p->out_scale) ||
      !(p->rope_theta > 0.0f) || !std::isfinite(p->rope_theta))
    return MLA_ERR_SHAPE;
  if (p->page_size != 0 && p->page_size != kPage) return MLA_ERR_UNSUPPORTED;
  // MLA (one 512-wide branch), MLRA-4 (four 128-wide branches) or one MLRA branch on its own
  // (128 wide) with the bf16 decode dims; no folded or gated forms, no fp8 latent, no device
  // checks
  const bool shape_ok = (p->num_branches == 1 && (p->d_latent == 512 || p->d_latent == 128)) ||
                        (p->num_branches == 4 && p->d_latent == 128);
  if (p->dtype != MLA_BF16 || !shape_ok || p->d_rope != 64 || p->d_nope != 128 ||
      p->d_v != 128 || p->flags != 0 || p->latent_format != 0)
    return MLA_ERR_UNSUPPORTED;
  if (p->latent_stride_tok < (int64_t)p->num_branches * p->d_latent || p->rope_stride_tok < 64 ||
      p->latent_stride_seq < 0 || p->rope_stride_seq < 0)
    return MLA_ERR_SHAPE;
  if ((p->latent_stride_tok | p->latent_stride_seq | p->rope_stride_tok | p->rope_stride_seq) % 8)
    return MLA_ERR_ALIGN;
  if (p->page_size == kPage && (p->max_pages_per_seq < ceil_div(p->max_seqlen, kPage) ||
                                p->block_table_stride < p->max_pages_per_seq))
    return MLA_ERR_SHAPE;
  PrefillPlan q{};
  q.B = p->batch;
  q.H = p->num_heads;
  q.sq = p->num_queries > 1 ? p->num_queries : 1;
  q.NB = p->num_branches;
  q.dcb = p->d_latent;
  q.paged = p->page_size == kPage;
  q.max_seqlen = p->max_seqlen;
  q.L_pad = (int)(ceil_div(std::max(p->max_seqlen, 1), 256) * 256);
  q.n_cu = (n_cu <= 0 || n_cu > kMaxCUs) ? kMaxCUs : n_cu;
  // projection tiles (256 tokens of one sequence, head and branch) indexed in 32 bits
  if ((int64_t)q.B * q.H * q.NB * (q.L_pad / 256) > INT32_MAX) return MLA_ERR_SHAPE;
  // attention grid, one dimension: (sequence, head and branch, pair of 256-token query blocks)
  if ((ceil_div((int64_t)q.B * q.H * q.NB, 8) * 8) * ceil_div(ceil_div(q.sq, 256), 2) > INT32_MAX)
    return MLA_ERR_SHAPE;
  // branch-sum grid: one thread per 8 output columns of each (sequence, token, head)
  if (q.NB > 1 && ceil_div((int64_t)q.B * q.sq * q.H * 16, 256) > INT32_MAX) return MLA_ERR_SHAPE;
  const size_t kv = (size_t)q.B * q.H * q.NB * q.L_pad * 128 * 2;
  const size_t r = (size_t)q.B * q.L_pad * 64 * 2;
  const size_t o = q.NB > 1 ? (size_t)q.B * q.sq * q.H * q.NB * 128 * 2 : 0;
  q.off_k = 0;
  q.off_r = align_up(kv);
  q.off_v = q.off_r + align_up(r);
  q.off_o = q.off_v + align_up(kv);
  q.bytes = q.off_o + align_up(o);
  *plan = q;
  return MLA_OK;
}

mla_status check_prefill_call(const PrefillPlan& plan, const void* q_nope, const void* q_rope,
                              const void* latent, const void* rope, const int32_t* seqlens,
                              const int32_t* block_table, const void* w_uk, const void* w_uv,
                              const void* out, const void* workspace, size_t workspace_bytes) {
  if (!q_nope || !q_rope || !latent || !rope || !seqlens || !w_uk || !w_uv || !out || !workspace)
    return MLA_ERR_NULL;
  if (plan.paged && !block_table) return MLA_ERR_NULL;
  if (workspace_bytes < plan.bytes) return MLA_ERR_WORKSPACE;
  if (!aligned(workspace, kWsAlign) || !aligned(seqlens, 4) || (plan.paged && !aligned(block_table, 4)))
    return MLA_ERR_ALIGN;
  // 16-byte vector reads of queries, cache rows and weights, 8-byte output stores
  if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(latent, 16) || !aligned(rope, 16) ||
      !aligned(w_uk, 16) || !aligned(w_uv, 16) || !aligned(out, 16))
    return MLA_ERR_ALIGN;
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

mla_status make_append_plan(const mla_append_params* p, AppendPlan* plan) {
  if (!p || !plan) return MLA_ERR_NULL;
  if (p->dtype != MLA_F32 && p->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (p->batch < 1 || p->batch > (1 << 20) || p->d_model < 1 || p->d_latent < 1 ||
      p->d_rope < 2 || p->max_pages_per_seq < 0 || p->capacity < 0 ||
      !(p->rope_theta > 0.0f) || !std::isfinite(p->rope_theta))
    return MLA_ERR_SHAPE;
  if (p->page_size != 0 && p->page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (p->latent_format != 0 && p->latent_format != MLA_LATENT_FP8) return MLA_ERR_DTYPE;
  if (p->latent_format == MLA_LATENT_FP8 &&
      (!std::isfinite(p->latent_scale) || !(p->latent_scale > 0.0f)))
    return MLA_ERR_SHAPE;
  // bf16, latent 512 (MLA, or MLRA-4's four 128-wide branches side by side) or 128 (one
  // branch), rotary key 64, d_model a multiple of 256 up to 65536
  if (p->dtype != MLA_BF16 || (p->d_latent != 512 && p->d_latent != 128) || p->d_rope != 64 ||
      p->d_model % 256 || p->d_model > 65536)
    return MLA_ERR_UNSUPPORTED;
  AppendPlan q{};
  q.B = p->batch;
  q.d_model = p->d_model;
  q.dc = p->d_latent;
  q.ncol = q.dc + 64;
  q.page_size = p->page_size;
  q.max_pages = p->max_pages_per_seq;
  q.capacity = p->capacity;
  q.f8 = p->latent_format == MLA_LATENT_FP8 ? 1 : 0;
  q.latent_scale = q.f8 ? p->latent_scale : 1.0f;
  if (q.page_size ? (q.max_pages < 1 || p->block_table_stride < q.max_pages) : q.capacity < 1)
    return MLA_ERR_SHAPE;
  if (p->latent_stride_tok < q.dc || p->rope_stride_tok < 64 || p->latent_stride_seq < 0 ||
      p->rope_stride_seq < 0)
    return MLA_ERR_SHAPE;
  q.n_cb = (int)ceil_div(q.ncol, 128);
  q.n_kc = q.d_model / 256;
  q.n_rb = (int)ceil_div(q.B, 32);
  size_t off = 0;
  q.off_part = off;
  off = align_up(off + (size_t)q.n_kc * q.B * q.ncol * 4);
  q.off_rank = off;
  off = align_up(off + (size_t)q.B * 4);
  q.bytes = off;
  *plan = q;
  return MLA_OK;
}

mla_status check_append_call(const mla_append_params* p, const AppendPlan& plan,
                             const void* hidden, const void* w_dkv, const void* w_kr,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const int32_t* free_pages,
                             int32_t n_free, const int32_t* pages_used, const void* workspace,
                             size_t workspace_bytes) {
  (void)p;
  if (!hidden || !w_dkv || !w_kr || !latent || !rope || !seqlens || !pages_used || !workspace)
    return MLA_ERR_NULL;
  if (n_free < 0) return MLA_ERR_SHAPE;
  if (plan.page_size && (!block_table || (n_free > 0 && !free_pages))) return MLA_ERR_NULL;
  if (workspace_bytes < plan.bytes) return MLA_ERR_WORKSPACE;
  // hidden rows and weight rows are read 16 bytes at a time
  if (!aligned(hidden, 16) || !aligned(w_dkv, 16) || !aligned(w_kr, 16) ||
      !aligned(latent, plan.f8 ? 1 : 2) || !aligned(rope, 2) || !aligned(seqlens, 4) ||
      !aligned(pages_used, 4) || !aligned(workspace, kWsAlign) ||
      (plan.page_size && !aligned(block_table, 4)) || (free_pages && !aligned(free_pages, 4)))
    return MLA_ERR_ALIGN;
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
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime or launch failure";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: pointer or stride misaligned";
    default: return "unknown mla_status";
  }
}

}  // namespace mla
