// Host-only driver for tests/test_planner_sanitized_cpu.py: applies the plan rule
// (csrc/planner.cpp, built with address and undefined-behaviour sanitizers) to
// random length mixes, page sizes, windows and schedules, including lengths that
// reach the 16M-token ranges of the radix ordering, and checks every item of
// every plan against the request it belongs to. Exits non-zero on any failure.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "planner.h"

namespace {
int failures = 0;
void check(bool ok, const char* what, int plan) {
  if (!ok && failures++ < 10) std::fprintf(stderr, "plan %d: %s\n", plan, what);
}
}  // namespace

int main(int argc, char** argv) {
  const int n_plans = argc > 1 ? std::atoi(argv[1]) : 2000;
  std::mt19937_64 rng(173);
  long items = 0;
  for (int p = 0; p < n_plans; ++p) {
    const int batch = static_cast<int>(rng() % 40);
    const int P = std::vector<int>{1, 2, 5, 16, 32, 64, 256}[rng() % 7];
    const bool prefill = rng() & 1;
    std::vector<int64_t> qo(batch), kv(batch);
    for (int b = 0; b < batch; ++b) {
      const int64_t hi = rng() % 16 == 0 ? 20000000 : (rng() % 4 == 0 ? 200000 : 3000);
      kv[b] = rng() % 5 == 0 ? 0 : static_cast<int64_t>(rng() % hi);
      qo[b] = prefill ? (kv[b] == 0 ? static_cast<int64_t>(rng() % 3)
                                    : 1 + static_cast<int64_t>(rng() % std::min<int64_t>(kv[b], 4096)))
                      : 1;
    }
    pkv::PlanInput in{};
    in.qo_lens = qo.data();
    in.kv_lens = kv.data();
    in.batch = batch;
    in.page_size = P;
    in.num_kv_heads = 1 + static_cast<int>(rng() % 8);
    in.group_size = 1 + static_cast<int>(rng() % 16);
    in.rows_per_tile = prefill ? 128 : in.group_size;
    in.causal = prefill && (rng() & 1);
    in.window_left = rng() % 4 == 0 ? static_cast<int>(rng() % 5000) : -1;
    in.num_cus = 256;
    in.wg_per_cu = 1 + static_cast<int>(rng() % 16);
    in.min_chunk_tokens = 1 + static_cast<int>(rng() % 1024);
    in.group_all = rng() % 3 == 0;
    pkv::HostPlan hp;
    std::string err;
    if (!pkv::build_plan(in, &hp, &err)) continue;
    items += static_cast<long>(hp.items.size());
    std::vector<int64_t> slot_uses(static_cast<size_t>(hp.num_slots), 0);
    for (const pkv::PlanItem& x : hp.items) {
      check(x.b >= 0 && x.b < batch, "request index out of range", p);
      if (x.b < 0 || x.b >= batch) continue;
      check(x.kv_begin <= x.kv_end && x.kv_end <= kv[x.b], "KV range outside the request", p);
      check(x.page_begin <= x.page_end, "page range reversed", p);
      check(x.kv_end <= static_cast<int64_t>(x.page_end) * P, "KV range past its pages", p);
      check(x.g >= 0 && x.g < in.num_kv_heads, "KV head out of range", p);
      check(x.slot >= -1 && x.slot < hp.num_slots, "slot out of range", p);
      if (x.slot >= 0 && x.slot < hp.num_slots) ++slot_uses[static_cast<size_t>(x.slot)];
    }
    for (int64_t u : slot_uses) check(u == 1, "a partial-state slot is not written exactly once", p);
    for (const pkv::MergeGroup& g : hp.groups)
      check(g.slot_begin >= 0 && g.num_chunks >= 1 &&
                static_cast<int64_t>(g.slot_begin) + g.num_chunks <= hp.num_slots,
            "merge group slots out of range", p);
  }
  std::printf("plans %d items %ld failures %d\n", n_plans, items, failures);
  return failures == 0 ? 0 : 1;
}
