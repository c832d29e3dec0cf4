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
  const void* gate;  // [B][H][d_v] gate logits of the gated entry points, else null
  int64_t lat_tok, lat_seq, rope_tok, rope_seq, bt_stride;
  float softmax_scale, out_scale, rope_theta;
  float latent_scale;  // value of one latent unit: the fp8 latent's scale, else 1
  // workspace regions
  PlanArgs plan;    // split plan, written by the prologue launch
  const int32_t* work;       // [slots][4]: b, t_begin, t_end, item of the slot's first item
                             // (b < 0: the slot has none)
  const int32_t* slot_end;   // [slots]: one past the slot's last item
  const int32_t* items;      // [items_cap][4]: b, t_begin, t_end, slot of every item
  const int32_t* split_off;  // [B + 1] first work item of each sequence
  void* qcat;       // [B][H][row] storage dtype, pre-scaled by softmax_scale*log2(e)
  void* part_o;     // [item][H][d_c], unnormalised partial latent outputs: bf16 on the bf16
                    // path (the same rounding as the latent output), fp32 otherwise
  float* part_ml;   // [item][NB][H][2]  (running max in log2 units, running sum)
  void* olat;       // [B][H][d_c] fp32, fp32 path only (the bf16 path keeps it on chip)
};

// mla_prefill: the un-absorbed many-query step (prefill.hip)
struct PrefillArgs {
  const void* q_nope;   // [B][s_q][H][128]
  const void* q_rope;   // [B][s_q][H][64], not rotated
  const void* latent;
  const void* rope;
  const int32_t* seqlens;
  const int32_t* block_table;
  const void* w_uk;     // [NB][H][128][dcb]
  const void* w_uv;     // [NB][H][dcb][128]
  void* out;            // [B][s_q][H][128]
  int64_t lat_tok, lat_seq, rope_tok, rope_seq, bt_stride;
  float softmax_scale, out_scale, rope_theta;
  // workspace: keys and values as operand blocks [B][H NB][L_pad / 32][8 KiB] each, the
  // rotary keys [B][L_pad / 32][4 KiB], and (NB > 1) the branch outputs [B][s_q][H NB][128] bf16
  void* kbuf;
  void* rbuf;
  void* vbuf;
  void* obuf;
};
// events (tracing, else null): three hipEvent_t recorded before the projection, between the
// two kernels and after the attention
hipError_t launch_prefill(const PrefillPlan& p, const PrefillArgs& a, hipStream_t s,
                          void* const* events);

struct RopeFreq;
// theta^(-2k/d_rope), k < d_rope/2, in fp64 (RoFormer frequencies)
void make_rope_freq(int d_rope, float theta, RopeFreq* out);

// MLA_FLAG_DEVICE_CHECKS only: per-sequence checks of seqlens and block ids, before the plan
hipError_t launch_device_checks(const Plan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_prologue(const Plan& p, const DecodeArgs& a, hipStream_t s);       // fp32 path
hipError_t launch_prologue_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_main_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_main_bf16_wide(const Plan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_main_f32(const Plan& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine(const Plan& p, const DecodeArgs& a, hipStream_t s);        // fp32 path
hipError_t launch_epilogue(const Plan& p, const DecodeArgs& a, hipStream_t s);       // fp32 path
// bf16 path: split combine and W_UV epilogue in one kernel (the latent output stays on chip)
hipError_t launch_combine_epilogue_bf16(const Plan& p, const DecodeArgs& a, hipStream_t s);
int combine_epilogue_rows(int B, int H, int dc);
hipError_t launch_rope_rotate(void* x, int64_t row_stride, const int32_t* pos, int64_t n_rows,
                              int d_rope, float theta, int dtype, hipStream_t s);

}  // namespace mla
