// Internal launch interface between the C ABI (api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "plan.h"
#include "plan_device.h"

namespace mla {

struct DecodeArgs {
  const void* q_nope;
  const void* q_rope;
  const void* latent;
  const void* rope;
  const int32_t* seqlens;
  const int32_t* block_table;
  const void* w_uk;
  const void* w_uv;
  void* out;
  int64_t lat_tok, lat_seq, rope_tok, rope_seq, bt_stride;
  float softmax_scale, out_scale, rope_theta;
  // workspace regions
  PlanArgs plan;    // split plan, written by the prologue launch
  const int32_t* work;       // [slots][4] dispatch table: b, t_begin, t_end, item (b < 0: none)
  const int32_t* split_off;  // [B + 1] first work item of each sequence
  void* qcat;       // [B][H][row] storage dtype, pre-scaled by softmax_scale*log2(e)
  void* part_o;     // [item][H][d_c], unnormalised partial latent outputs: bf16 on the bf16
                    // path (the same rounding as the latent output), fp32 otherwise
  float* part_ml;   // [item][NB][H][2]  (running max in log2 units, running sum)
  void* olat;       // [B][H][d_c] fp32, fp32 path only (the bf16 path keeps it on chip)
};

struct RopeFreq;
// theta^(-2k/d_rope), k < d_rope/2, in fp64 (RoFormer frequencies)
void make_rope_freq(int d_rope, float theta, RopeFreq* out);

hipError_t launch_prologue(const Plan& p, const DecodeArgs& a, hipStream_t s);       // fp32 path
hipError_t launch_prologue_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_main_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_main_bf16_wide(const Plan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_main_f32(const Plan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine(const Plan& p, const DecodeArgs& a, hipStream_t s);        // fp32 path
hipError_t launch_epilogue(const Plan& p, const DecodeArgs& a, hipStream_t s);       // fp32 path
// bf16 path: split combine and W_UV epilogue in one kernel (the latent output stays on chip)
hipError_t launch_combine_epilogue_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s);
int combine_epilogue_rows(int B, int H);
hipError_t launch_rope_rotate(void* x, int64_t row_stride, const int32_t* pos, int64_t n_rows,
                              int d_rope, float theta, int dtype, hipStream_t s);

}  // namespace mla
