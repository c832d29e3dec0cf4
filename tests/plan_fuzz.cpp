// Host-only exercise of the validation / split-plan code (plan.cpp), built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_abi.py.
#include <cstdio>
#include <cstring>
#include <random>

#include "plan.h"

int main() {
  std::mt19937_64 rng(12345);
  auto pick = [&](std::initializer_list<long long> v) {
    std::uniform_int_distribution<size_t> d(0, v.size() - 1);
    return *(v.begin() + d(rng));
  };
  long long ok = 0, bad = 0;
  for (int it = 0; it < 200000; ++it) {
    mla_params p;
    std::memset(&p, 0, sizeof(p));
    p.batch = (int)pick({-1, 0, 1, 3, 64, 1 << 20, (1 << 20) + 1, 2147483647});
    p.num_heads = (int)pick({0, 1, 4, 32, 96, 128, 4096, 4097});
    p.num_branches = (int)pick({0, 1, 2, 4});
    p.d_nope = (int)pick({0, 16, 128, 257});
    p.d_v = (int)pick({0, 16, 128, 300});
    p.d_latent = (int)pick({0, 32, 128, 512, 513});
    p.d_rope = (int)pick({0, 1, 8, 64, 66});
    p.page_size = (int)pick({0, 64, 16});
    p.max_seqlen = (int)pick({-1, 0, 1, 63, 64, 65, 131072, 1 << 26, (1 << 26) + 1});
    p.max_pages_per_seq = (int)pick({0, 1, 2048, 1 << 20});
    p.num_splits = (int)pick({-1, 0, 1, 7, 1 << 20});
    p.dtype = (int)pick({0, 1, 2});
    p.latent_stride_tok = pick({0, 40, 576, 577, 1 << 30});
    p.latent_stride_seq = pick({-8, 0, 576 * 64, 576LL * 131072});
    p.rope_stride_tok = pick({0, 40, 576});
    p.rope_stride_seq = pick({0, 576 * 64});
    p.block_table_stride = pick({0, 2048, 1 << 20});
    p.softmax_scale = (float)pick({0, 1});
    p.out_scale = 0.5f;
    p.rope_theta = (float)pick({0, 10000});
    mla::Plan plan;
    const mla_status st = mla::make_plan(&p, &plan);
    if (st == MLA_OK) {
      ++ok;
      // invariants of an accepted plan
      const long long pages = p.max_seqlen > 0 ? (p.max_seqlen + 63) / 64 : 1;
      const bool forced = p.num_splits > 0;
      const long long per = forced ? plan.forced_pages : 0;
      if (plan.splits < 1 || plan.splits > mla::kMaxSplits || plan.splits > pages ||
          plan.target < 1 || plan.items_cap < 1 || plan.slots % 8 ||
          plan.slots < plan.items_cap || plan.slots - plan.items_cap >= 8 ||
          (forced && (per < 1 || per * plan.splits < pages || per * (plan.splits - 1) >= pages ||
                      plan.items_cap != (long long)p.batch * plan.splits)) ||
          (!forced && (plan.forced_pages != 0 || plan.items_cap < plan.target ||
                       plan.items_cap < p.batch)) ||
          plan.off_work != 16 || plan.off_split_off != 16 + 16 * (size_t)plan.slots ||
          plan.off_qcat < plan.off_split_off + 4 * ((size_t)p.batch + 1) ||
          plan.off_part_o < plan.off_qcat || plan.off_part_ml < plan.off_part_o ||
          plan.off_olat < plan.off_part_ml || plan.bytes < plan.off_olat) {
        std::printf("bad plan at iteration %d\n", it);
        return 1;
      }
    } else {
      ++bad;
    }
  }
  std::printf("accepted %lld rejected %lld\n", ok, bad);
  return ok > 0 && bad > 0 ? 0 : 2;
}
