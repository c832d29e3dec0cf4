// Host-side argument validation and launch plan for the decode step.
// Pure C++ (no HIP): the same source is compiled into the HIP library and, on its own,
// into a host-only test binary.
#pragma once

#include <cstddef>
#include <cstdint>

#include "mla_decode.h"

namespace mla {

constexpr int kPage = MLA_PAGE_SIZE;   // tokens per page == tokens per main-loop tile
constexpr int kHeadGroup = 32;         // heads per workgroup of the bf16 main kernel
constexpr int kTargetWorkgroups = 512; // two per CU of an MI355X (32-head kernel runs 2 per CU)
constexpr int kWideHeads = 128;        // heads per workgroup of the wide bf16 kernel
constexpr int kTargetWideWorkgroups = 256;  // one per CU (the wide kernel fills a CU's LDS)
constexpr size_t kWsAlign = 256;
constexpr int kMaxSplits = 512;        // bound on work items per sequence (the fp32 combine
                                       // keeps one weight per item in LDS)

enum class Path { kBf16Mfma, kF32Simt };

struct Plan {
  int B, H, NB, dcb, dc, dr, dn, dv, row;
  int dtype, elem;
  int paged;
  int max_seqlen;
  int n_tiles;   // ceil(max_seqlen / 64), >= 1
  // Split plan.  The device cuts the batch into work items of whole pages (see
  // plan_device.h); the host only bounds it.
  int target;        // work items the automatic plan aims for (a workgroup set per CU slot)
  int forced_pages;  // pages per work item when num_splits is given, else 0
  int splits;        // most work items one sequence can be cut into (<= kMaxSplits)
  int items_cap;     // most work items of one call: sizes the partials
  int slots;         // dispatch slots of the main kernels (items_cap rounded up to 8)
  int xcd_major;     // 1: slot 8g + x takes item x * ceil(W / 8) + g (XCD-contiguous items)
  int n_hg;      // head groups of the bf16 kernel (H / 32); 0 on the fp32 path
  int wide;      // 1: bf16 MLA with H % 128 == 0 runs the 128-heads-per-workgroup kernel
  Path path;
  // workspace layout (byte offsets); part_o holds bf16 on the bf16 path, fp32 otherwise.
  // The plan comes first: header int32[4], work int32[slots][4], split_off int32[B + 1].
  size_t off_work, off_split_off, off_qcat, off_part_o, off_part_ml, off_olat, bytes;
};

// Validates *p (shape, dtype, support, strides) and fills *plan.  Touches no device.
mla_status make_plan(const mla_params* p, Plan* plan);

// Per-call checks on top of make_plan: required pointers, alignment, workspace size,
// and the branch count the entry point accepts (1 for mla_decode, 4 for mlra_decode).
mla_status check_call(const mla_params* p, const Plan& plan, int want_branches,
                      const void* q_nope, const void* q_rope, const void* latent,
                      const void* rope, const int32_t* seqlens, const int32_t* block_table,
                      const void* w_uk, const void* w_uv, const void* out,
                      const void* workspace, size_t workspace_bytes);

mla_status check_rope_rotate(const void* x, int64_t row_stride, const int32_t* pos,
                             int64_t n_rows, int32_t d_rope, float theta, int32_t dtype);

const char* status_str(int32_t s);

}  // namespace mla
