// Host-side argument validation and launch plan for the decode step.
// Pure C++ (no HIP): the same source is compiled into the HIP library and, on its own,
// into a host-only test binary.
#pragma once

#include <cstddef>
#include <cstdint>

#include "mla_decode.h"

namespace mla {

constexpr int kPage = MLA_PAGE_SIZE;   // tokens per page
constexpr int kHeadGroup = 32;         // heads per workgroup of the 32-head bf16 kernels
constexpr int kWideHeads = 128;        // heads per workgroup of the wide bf16 kernel
// workgroups per CU of the 32-head kernel on 192-wide rows (one MLRA branch): its tiles and
// registers are small, so several workgroups share a CU and hide each other's per-tile chain
#ifndef MLA_NARROW_OCC
#define MLA_NARROW_OCC 4
#endif
constexpr int kNarrowWgPerCu = MLA_NARROW_OCC;
constexpr int kMaxCUs = 256;           // compute units the workspace is sized for (MI355X);
                                       // a device reporting more is planned as if it had 256
constexpr size_t kWsAlign = 256;
constexpr int kMaxSplits = 512;        // bound on work items per sequence (the fp32 combine
                                       // keeps one weight per item in LDS)
constexpr int kHdrWords = 8;           // plan header words at the start of the workspace

enum class Path { kBf16Mfma, kF32Simt };

struct Plan {
  // H: query rows per sequence, s_q tokens x Hw heads (token-major); Hw: heads of the weights
  int B, H, NB, dcb, dc, dr, dn, dv, row;
  int sq, Hw;
  int dtype, elem;
  int paged;
  int max_seqlen;
  int n_tiles;   // ceil(max_seqlen / 64), >= 1
  int n_cu;      // compute units the plan is made for (1 .. kMaxCUs)
  int checks;    // MLA_FLAG_DEVICE_CHECKS given: a check kernel runs before the prologue
  int num_pages; // pool pages for the block-id check (0: not checked)
  int latent_q;  // MLA_FLAG_QUERY_LATENT: the query arrives folded (no W_UK product)
  int latent_out;  // MLA_FLAG_OUTPUT_LATENT: out is the latent-space output (no W_UV)
  int f8;          // MLA_LATENT_FP8: the latent cache holds E4M3 codes (scale latent_scale)
  // Split plan.  The device cuts the batch into work items of whole pages, one per dispatch
  // slot (see plan_device.h); the host only bounds it.
  int target;        // slots the automatic plan fills (one workgroup set per CU slot)
  int forced_pages;  // pages per work item when num_splits is given, else 0
  int splits;        // most work items one sequence can be cut into
  int items_cap;     // most work items of one call: sizes the partials
  int slots;         // dispatch slots of the main kernels (rounded up to 8)
  int xcd_major;     // page plan: slot 8g + x takes item x * ceil(W / 8) + g
  int n_hg;      // head groups of the bf16 kernel (H / 32); 0 on the fp32 path
  int wide;      // 1: bf16 MLA with H % 128 == 0 runs the 128-heads-per-workgroup kernel
  Path path;
  // workspace layout (byte offsets); part_o holds bf16 on the bf16 path, fp32 otherwise.
  // The plan comes first: header int32[8], work int32[slots][4], slot_end int32[slots],
  // items int32[items_cap][4], split_off int32[B + 1], device-check results int32[B].
  size_t off_work, off_slot_end, off_items, off_split_off, off_dbg;
  size_t off_qcat, off_part_o, off_part_ml, off_olat, bytes;
};

// Validates *p (shape, dtype, support, strides) and fills *plan for a device with n_cu
// compute units (n_cu <= 0 or > kMaxCUs: kMaxCUs, the bound the workspace size uses).
// Touches no device.
mla_status make_plan(const mla_params* p, Plan* plan, int n_cu = 0);

// Per-call checks on top of make_plan: required pointers, alignment, workspace size,
// and the branch count the entry point accepts (1 for mla_decode, 4 for mlra_decode).
mla_status check_call(const mla_params* p, const Plan& plan, int want_branches,
                      const void* q_nope, const void* q_rope, const void* latent,
                      const void* rope, const int32_t* seqlens, const int32_t* block_table,
                      const void* w_uk, const void* w_uv, const void* out,
                      const void* workspace, size_t workspace_bytes, bool gated = false,
                      const void* gate = nullptr);

mla_status check_rope_rotate(const void* x, int64_t row_stride, const int32_t* pos,
                             int64_t n_rows, int32_t d_rope, float theta, int32_t dtype);

// Cache append (mla_cache_append): launch shape and workspace layout.
struct AppendPlan {
  int B, d_model, dc, ncol;   // ncol = dc + 64 output columns per row
  int page_size, max_pages, capacity;
  int f8;                     // MLA_LATENT_FP8: latent written as E4M3 codes of value / latent_scale
  float latent_scale;
  int n_cb, n_kc, n_rb;       // projection grid: column blocks of 128, K chunks of 256, row blocks of 32
  size_t off_part, off_rank, bytes;
};

// Validates *p and fills *plan.  Touches no device.
mla_status make_append_plan(const mla_append_params* p, AppendPlan* plan);

// Per-call checks on top of make_append_plan: pointers, alignment, workspace size.
mla_status check_append_call(const mla_append_params* p, const AppendPlan& plan,
                             const void* hidden, const void* w_dkv, const void* w_kr,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const int32_t* free_pages,
                             int32_t n_free, const int32_t* pages_used, const void* workspace,
                             size_t workspace_bytes);

// Prefill (mla_prefill): the un-absorbed many-query step.  The workspace holds the keys and
// values up-projected from the latent (B x H x NB x L_pad x 128 bf16 each) and a copy of the
// rotary keys (B x L_pad x 64 bf16), all as MFMA operand blocks of 32-token tiles, and with
// MLRA branches (NB = 4) each branch's normalised output (B x s_q x H x NB x 128 bf16) for the
// branch sum.
struct PrefillPlan {
  int B, H, sq;       // sequences, weight heads, query tokens per sequence (rows s_q x H)
  int NB, dcb;        // latent branches (1 MLA, 4 MLRA) and latent columns per branch
  int paged, max_seqlen;
  int L_pad;          // key rows per (sequence, head, branch) in the workspace: max_seqlen
                      // rounded up to the projection's 256-token blocks
  int n_cu;           // compute units: the projection runs one workgroup per CU
  size_t off_k, off_r, off_v, off_o, bytes;
};

// Validates *p for the prefill and fills *plan for a device with n_cu compute units (n_cu <= 0
// or > kMaxCUs: kMaxCUs; the caller may lower plan->n_cu to the device's count afterwards).
// Touches no device.
mla_status make_prefill_plan(const mla_params* p, PrefillPlan* plan, int n_cu = 0);

// Per-call checks on top of make_prefill_plan: pointers, alignment, workspace size.
mla_status check_prefill_call(const PrefillPlan& plan, const void* q_nope, const void* q_rope,
                              const void* latent, const void* rope, const int32_t* seqlens,
                              const int32_t* block_table, const void* w_uk, const void* w_uv,
                              const void* out, const void* workspace, size_t workspace_bytes);

const char* status_str(int32_t s);

}  // namespace mla
