// extern "C" entry points of libmla_decode.so (declared in include/mla_decode.h).
//
// mla_decode / mlra_decode validate on the host, then enqueue on the caller's stream:
//   prologue  -> absorbed query q_cat = [W_UK^T q_nope | RoPE(q_rope, L-1)] * scale*log2(e),
//                and (one extra workgroup) the split plan: page-aligned work items per sequence
//   main loop -> per (work item, head group) partial (m, l, O) over the latent cache
//   combine   -> log-sum-exp merge of the splits into the latent-space output
//   epilogue  -> out = out_scale * W_UV^T o_lat (summed over MLRA branches)
// (on the bf16 path combine and epilogue are one kernel)
// Nothing is allocated, nothing synchronises, no state is kept between calls.
#include "launch.h"
#include "plan.h"

namespace {

using namespace mla;

mla_status to_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

mla_status run_decode(int want_branches, const mla_params* p, const void* q_nope,
                      const void* q_rope, const void* latent, const void* rope,
                      const int32_t* seqlens, const int32_t* block_table, const void* w_uk,
                      const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
                      void* stream, void* const* events) {
  Plan plan;
  mla_status st = make_plan(p, &plan);
  if (st != MLA_OK) return st;
  st = check_call(p, plan, want_branches, q_nope, q_rope, latent, rope, seqlens, block_table,
                  w_uk, w_uv, out, workspace, workspace_bytes);
  if (st != MLA_OK) return st;

  DecodeArgs a;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.latent = latent;
  a.rope = rope;
  a.seqlens = seqlens;
  a.block_table = block_table;
  a.w_uk = w_uk;
  a.w_uv = w_uv;
  a.out = out;
  a.lat_tok = p->latent_stride_tok;
  a.lat_seq = p->latent_stride_seq;
  a.rope_tok = p->rope_stride_tok;
  a.rope_seq = p->rope_stride_seq;
  a.bt_stride = p->block_table_stride;
  a.softmax_scale = p->softmax_scale;
  a.out_scale = p->out_scale;
  a.rope_theta = p->rope_theta;
  char* ws = static_cast<char*>(workspace);
  a.plan = plan_args(plan, seqlens, workspace);
  a.work = a.plan.work;
  a.split_off = a.plan.split_off;
  a.qcat = ws + plan.off_qcat;
  a.part_o = ws + plan.off_part_o;
  a.part_ml = reinterpret_cast<float*>(ws + plan.off_part_ml);
  a.olat = ws + plan.off_olat;

  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), s) : hipSuccess;
  };
  hipError_t e = mark(0);
  const bool bf = plan.path == Path::kBf16Mfma;
  if (e == hipSuccess) e = bf ? launch_prologue_bf16(plan, a, s) : launch_prologue(plan, a, s);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess)
    e = !bf ? launch_main_f32(plan, a, s)
        : plan.wide ? launch_main_bf16_wide(plan, a, s)
                    : launch_main_bf16(plan, a, s);
  if (e == hipSuccess) e = mark(2);
  if (bf) {
    // one kernel: the merged latent output stays on chip (events 3 and 4 coincide)
    if (e == hipSuccess) e = launch_combine_epilogue_bf16(plan, a, s);
    if (e == hipSuccess) e = mark(3);
  } else {
    if (e == hipSuccess) e = launch_combine(plan, a, s);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = launch_epilogue(plan, a, s);
  }
  if (e == hipSuccess) e = mark(4);
  return to_status(e);
}

}  // namespace

extern "C" {

mla_status mla_workspace_size(const mla_params* p, size_t* bytes) {
  if (!bytes) return MLA_ERR_NULL;
  Plan plan;
  const mla_status st = make_plan(p, &plan);
  if (st == MLA_OK) *bytes = plan.bytes;
  return st;
}

mla_status mla_num_splits(const mla_params* p, int32_t* splits) {
  if (!splits) return MLA_ERR_NULL;
  Plan plan;
  const mla_status st = make_plan(p, &plan);
  if (st == MLA_OK) *splits = plan.splits;
  return st;
}

mla_status mla_decode(const mla_params* p, const void* q_nope, const void* q_rope,
                      const void* latent, const void* rope, const int32_t* seqlens,
                      const int32_t* block_table, const void* w_uk, const void* w_uv, void* out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return run_decode(1, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, nullptr);
}

mla_status mlra_decode(const mla_params* p, const void* q_nope, const void* q_rope,
                       const void* latent, const void* rope, const int32_t* seqlens,
                       const int32_t* block_table, const void* w_uk, const void* w_uv, void* out,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return run_decode(4, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, nullptr);
}

mla_status mla_decode_timed(const mla_params* p, const void* q_nope, const void* q_rope,
                            const void* latent, const void* rope, const int32_t* seqlens,
                            const int32_t* block_table, const void* w_uk, const void* w_uv,
                            void* out, void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events) {
  return run_decode(1, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, events);
}

mla_status mlra_decode_timed(const mla_params* p, const void* q_nope, const void* q_rope,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const void* w_uk, const void* w_uv,
                             void* out, void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events) {
  return run_decode(4, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, events);
}

mla_status mla_rope_rotate(void* x, int64_t row_stride, const int32_t* pos, int64_t n_rows,
                           int32_t d_rope, float theta, int32_t dtype, void* stream) {
  const mla_status st = check_rope_rotate(x, row_stride, pos, n_rows, d_rope, theta, dtype);
  if (st != MLA_OK || n_rows == 0) return st;
  return to_status(launch_rope_rotate(x, row_stride, pos, n_rows, d_rope, theta, dtype,
                                      static_cast<hipStream_t>(stream)));
}

const char* mla_status_str(int32_t status) { return status_str(status); }

}  // extern "C"
