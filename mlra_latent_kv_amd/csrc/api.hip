// extern "C" entry points of libmla_decode.so (declared in include/mla_decode.h).
//
// mla_decode / mlra_decode validate on the host, then enqueue on the caller's stream:
//   prologue  -> absorbed query q_cat = [W_UK^T q_nope | RoPE(q_rope, L-1)] * scale*log2(e),
//                and (one extra workgroup) the split plan: page-aligned work items per sequence
//   main loop -> per (work item, head group) partial (m, l, O) over the latent cache
//   combine   -> log-sum-exp merge of the splits into the latent-space output
//   epilogue  -> out = out_scale * W_UV^T o_lat (summed over MLRA branches), times
//                sigmoid(gate) for the gated entry points
// (on the bf16 path combine and epilogue are one kernel).  MLA_FLAG_QUERY_LATENT replaces
// the prologue's W_UK product by the given latent query; MLA_FLAG_OUTPUT_LATENT writes the
// merged latent output (times out_scale) instead of the W_UV product.
// Nothing is allocated, nothing synchronises, no state is kept between calls.
#include <atomic>

#include "append.h"
#include "launch.h"
#include "plan.h"

// Scratch of mla_decode_noalloc: the workspace (split plan, absorbed queries, split
// partials) in a file-scope device array, so that call allocates nothing.  Every GPU the
// library runs on holds its own copy until the process ends.  Host code never uses this name
// as an address (on the host it is only a stand-in symbol): the device address comes from
// hipGetSymbolAddress, once per device (noalloc_scratch below).
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace mla;

mla_status to_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Compute units of the current device, queried once per device and cached (the split plan's
// workgroup targets follow it, so a partitioned device gets a plan for its own CUs).
constexpr int kCuCacheDevices = 64;
std::atomic<int> g_cu_count[kCuCacheDevices];

hipError_t device_cu_count(int* n_cu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kCuCacheDevices) {
    const int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *n_cu = v;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n < 1) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < kCuCacheDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *n_cu = n;
  return hipSuccess;
}

mla_status run_decode(int want_branches, const mla_params* p, const void* q_nope,
                      const void* q_rope, const void* latent, const void* rope,
                      const int32_t* seqlens, const int32_t* block_table, const void* w_uk,
                      const void* w_uv, void* out, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, void* const* events, const void* gate = nullptr,
                      bool gated = false) {
  // validation against the plan mla_workspace_size describes (sized for kMaxCUs), then the
  // plan for this device's compute units, which needs no more workspace
  Plan plan;
  mla_status st = make_plan(p, &plan);
  if (st != MLA_OK) return st;
  st = check_call(p, plan, want_branches, q_nope, q_rope, latent, rope, seqlens, block_table,
                  w_uk, w_uv, out, workspace, workspace_bytes, gated, gate);
  if (st != MLA_OK) return st;
  int n_cu = 0;
  if (device_cu_count(&n_cu) != hipSuccess) return MLA_ERR_HIP;
  st = make_plan(p, &plan, n_cu);
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
  a.gate = gated ? gate : nullptr;
  a.lat_tok = p->latent_stride_tok;
  a.lat_seq = p->latent_stride_seq;
  a.rope_tok = p->rope_stride_tok;
  a.rope_seq = p->rope_stride_seq;
  a.bt_stride = p->block_table_stride;
  a.softmax_scale = p->softmax_scale;
  a.out_scale = p->out_scale;
  a.rope_theta = p->rope_theta;
  a.latent_scale = plan.f8 ? p->latent_scale : 1.0f;
  char* ws = static_cast<char*>(workspace);
  a.plan = plan_args(plan, seqlens, workspace);
  a.work = a.plan.work;
  a.slot_end = a.plan.slot_end;
  a.items = a.plan.items;
  a.split_off = a.plan.split_off;
  a.qcat = ws + plan.off_qcat;
  a.part_o = ws + plan.off_part_o;
  a.part_ml = reinterpret_cast<float*>(ws + plan.off_part_ml);
  a.olat = ws + plan.off_olat;

  hipStream_t s = stream;
  auto mark = [&](int i) {
    return events ? hipEventRecord(static_cast<hipEvent_t>(events[i]), s) : hipSuccess;
  };
  hipError_t e = mark(0);
  const bool bf = plan.path == Path::kBf16Mfma;
  if (e == hipSuccess && plan.checks) e = launch_device_checks(plan, a, s);
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
    // latent output: the combine writes out directly and there is no epilogue
    if (e == hipSuccess) e = launch_combine(plan, a, s);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess && !plan.latent_out) e = launch_epilogue(plan, a, s);
  }
  if (e == hipSuccess) e = mark(4);
  return to_status(e);
}

// Device address of `scratch` on the current device, looked up on the first call on each
// device (with that device current) and cached.
std::atomic<char*> g_scratch[kCuCacheDevices];

hipError_t noalloc_scratch(char** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kCuCacheDevices) return hipErrorInvalidDevice;
  char* v = g_scratch[dev].load(std::memory_order_acquire);
  if (!v) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    v = static_cast<char*>(a);
    g_scratch[dev].store(v, std::memory_order_release);
  }
  *ptr = v;
  return hipSuccess;
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
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_decode(1, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, nullptr);
}

mla_status mlra_decode(const mla_params* p, const void* q_nope, const void* q_rope,
                       const void* latent, const void* rope, const int32_t* seqlens,
                       const int32_t* block_table, const void* w_uk, const void* w_uv, void* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_decode(4, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, nullptr);
}

mla_status mla_decode_gated(const mla_params* p, const void* q_nope, const void* q_rope,
                            const void* latent, const void* rope, const int32_t* seqlens,
                            const int32_t* block_table, const void* w_uk, const void* w_uv,
                            const void* gate, void* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return run_decode(1, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, nullptr, gate, true);
}

mla_status mlra_decode_gated(const mla_params* p, const void* q_nope, const void* q_rope,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const void* w_uk, const void* w_uv,
                             const void* gate, void* out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return run_decode(4, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, nullptr, gate, true);
}

mla_status mla_decode_timed(const mla_params* p, const void* q_nope, const void* q_rope,
                            const void* latent, const void* rope, const int32_t* seqlens,
                            const int32_t* block_table, const void* w_uk, const void* w_uv,
                            void* out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                            void* const* events) {
  return run_decode(1, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, events);
}

mla_status mlra_decode_timed(const mla_params* p, const void* q_nope, const void* q_rope,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const void* w_uk, const void* w_uv,
                             void* out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                             void* const* events) {
  return run_decode(4, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    workspace, workspace_bytes, stream, events);
}

mla_status mla_decode_noalloc(const mla_params* p, const void* q_nope, const void* q_rope,
                              const void* latent, const void* rope, const int32_t* seqlens,
                              const int32_t* block_table, const void* w_uk, const void* w_uv,
                              void* out, hipStream_t stream) {
  // host checks first (no HIP call): arguments, and the call's workspace must fit the static
  // scratch.  The pointer checks run here with a stand-in for the scratch address (aligned,
  // never dereferenced); run_decode repeats them with the real one.
  Plan plan;
  mla_status st = make_plan(p, &plan);
  if (st != MLA_OK) return st;
  if (plan.bytes > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  st = check_call(p, plan, 1, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                  reinterpret_cast<const void*>(kWsAlign), (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  if (st != MLA_OK) return st;
  char* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return MLA_ERR_HIP;
  return run_decode(1, p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                    ws, (size_t)MLA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

mla_status mla_rope_rotate(void* x, int64_t row_stride, const int32_t* pos, int64_t n_rows,
                           int32_t d_rope, float theta, int32_t dtype, hipStream_t stream) {
  const mla_status st = check_rope_rotate(x, row_stride, pos, n_rows, d_rope, theta, dtype);
  if (st != MLA_OK || n_rows == 0) return st;
  return to_status(launch_rope_rotate(x, row_stride, pos, n_rows, d_rope, theta, dtype,
                                      stream));
}

mla_status mla_append_workspace_size(const mla_append_params* p, size_t* bytes) {
  if (!bytes) return MLA_ERR_NULL;
  AppendPlan plan;
  const mla_status st = make_append_plan(p, &plan);
  if (st == MLA_OK) *bytes = plan.bytes;
  return st;
}

mla_status mla_cache_append(const mla_append_params* p, const void* hidden, const void* w_dkv,
                            const void* w_kr, void* latent, void* rope, int32_t* seqlens,
                            int32_t* block_table, const int32_t* free_pages, int32_t n_free,
                            int32_t* pages_used, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  AppendPlan plan;
  mla_status st = make_append_plan(p, &plan);
  if (st != MLA_OK) return st;
  st = check_append_call(p, plan, hidden, w_dkv, w_kr, latent, rope, seqlens, block_table,
                         free_pages, n_free, pages_used, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  AppendArgs a;
  a.hidden = hidden;
  a.w_dkv = w_dkv;
  a.w_kr = w_kr;
  a.latent = latent;
  a.rope = rope;
  a.seqlens = seqlens;
  a.block_table = block_table;
  a.free_pages = free_pages;
  a.n_free = n_free;
  a.lat_tok = p->latent_stride_tok;
  a.lat_seq = p->latent_stride_seq;
  a.rope_tok = p->rope_stride_tok;
  a.rope_seq = p->rope_stride_seq;
  a.bt_stride = p->block_table_stride;
  a.rope_theta = p->rope_theta;
  char* ws = static_cast<char*>(workspace);
  a.ws.part = reinterpret_cast<float*>(ws + plan.off_part);
  a.ws.rank = reinterpret_cast<int32_t*>(ws + plan.off_rank);
  a.ws.pages_used = pages_used;
  return to_status(launch_append(plan, a, stream));
}

mla_status mla_prefill_workspace_size(const mla_params* p, size_t* bytes) {
  if (!bytes) return MLA_ERR_NULL;
  PrefillPlan plan;
  const mla_status st = make_prefill_plan(p, &plan);
  if (st == MLA_OK) *bytes = plan.bytes;
  return st;
}

namespace {
mla_status run_prefill(const mla_params* p, const void* q_nope, const void* q_rope,
                       const void* latent, const void* rope, const int32_t* seqlens,
                       const int32_t* block_table, const void* w_uk, const void* w_uv, void* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                       void* const* events) {
  PrefillPlan plan;
  mla_status st = make_prefill_plan(p, &plan);
  if (st != MLA_OK) return st;
  st = check_prefill_call(plan, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv,
                          out, workspace, workspace_bytes);
  if (st != MLA_OK) return st;
  int n_cu = 0;  // the device is asked only for a valid call
  if (device_cu_count(&n_cu) != hipSuccess) return MLA_ERR_HIP;
  if (n_cu > 0 && n_cu < plan.n_cu) plan.n_cu = n_cu;
  PrefillArgs a;
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
  a.kbuf = static_cast<char*>(workspace) + plan.off_k;
  a.rbuf = static_cast<char*>(workspace) + plan.off_r;
  a.vbuf = static_cast<char*>(workspace) + plan.off_v;
  a.obuf = static_cast<char*>(workspace) + plan.off_o;
  return to_status(launch_prefill(plan, a, stream, events));
}
}  // namespace

mla_status mla_prefill(const mla_params* p, const void* q_nope, const void* q_rope,
                       const void* latent, const void* rope, const int32_t* seqlens,
                       const int32_t* block_table, const void* w_uk, const void* w_uv, void* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_prefill(p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                     workspace, workspace_bytes, stream, nullptr);
}

mla_status mla_prefill_timed(const mla_params* p, const void* q_nope, const void* q_rope,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const void* w_uk, const void* w_uv,
                             void* out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, void* const* events) {
  return run_prefill(p, q_nope, q_rope, latent, rope, seqlens, block_table, w_uk, w_uv, out,
                     workspace, workspace_bytes, stream, events);
}

const char* mla_status_str(int32_t status) { return status_str(status); }

}  // extern "C"
