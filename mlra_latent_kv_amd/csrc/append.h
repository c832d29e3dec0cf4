// Host plan and launch interface of the cache-append step (append.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace mla {

struct AppendWs {
  float* part;         // [n_kc][B][d_c + 64] fp32 K-chunk partials of the projection
  int32_t* rank;       // [B] rank of each sequence among those that need a new page
  int32_t* pages_used; // [1] (caller's device output): free pages taken
};

struct AppendArgs {
  const void* hidden;
  const void* w_dkv;
  const void* w_kr;
  void* latent;
  void* rope;
  int32_t* seqlens;
  int32_t* block_table;
  const int32_t* free_pages;
  int n_free;
  int64_t lat_tok, lat_seq, rope_tok, rope_seq, bt_stride;
  float rope_theta;
  AppendWs ws;
};

hipError_t launch_append(const AppendPlan& p, const AppendArgs& a, hipStream_t s);

}  // namespace mla
