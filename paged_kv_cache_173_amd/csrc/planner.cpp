// Host-side work-chunk planner (see planner.h for the rule's source).
#include "planner.h"

#include <algorithm>
#include <limits>

namespace pkv {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct TileExtent {
  int32_t b, tile;
  int64_t kv_end, page_lo, pages;
};

}  // namespace

bool build_plan(const PlanInput& in, HostPlan* out, std::string* err) {
  const int64_t P = in.page_size, G = in.group_size, R = in.rows_per_tile;
  out->items.clear();
  out->groups.clear();

  // Per (request, tile): the KV extent the tile's rows may see. It ends
  // after the last row's causal limit and, with a sliding window, starts at
  // the first row's window start (rounded down to a page).
  std::vector<TileExtent> tiles;
  tiles.reserve(static_cast<size_t>(std::max(in.batch, 0)));
  int64_t page_sum = 0;
  for (int32_t b = 0; b < in.batch; ++b) {
    const int64_t Q = in.qo_lens[b], L = in.kv_lens[b];
    const int64_t rows = Q * G;
    const int64_t n_tiles = ceil_div(rows, R);
    for (int64_t t = 0; t < n_tiles; ++t) {
      int64_t extent = L;
      if (in.causal) {
        const int64_t last_row = std::min((t + 1) * R, rows) - 1;
        const int64_t q_last = last_row / G;
        extent = std::clamp<int64_t>(L - Q + q_last + 1, 0, L);
      }
      int64_t kv_lo = 0;
      if (in.window_left >= 0) kv_lo = std::max<int64_t>(0, L - Q + (t * R) / G - in.window_left);
      const int64_t page_lo = kv_lo / P;
      const int64_t pages = std::max<int64_t>(0, ceil_div(extent, P) - page_lo);
      tiles.push_back({b, static_cast<int32_t>(t), extent, page_lo, pages});
      page_sum += pages;
    }
  }

  // Chunk size: enough chunks to cover num_cus * wg_per_cu slots, never
  // shorter than min_chunk_tokens (in whole pages).
  const int64_t work = static_cast<int64_t>(in.num_kv_heads) * page_sum;
  const int64_t target = static_cast<int64_t>(in.num_cus) * in.wg_per_cu;
  const int64_t c_min = std::max<int64_t>(1, ceil_div(in.min_chunk_tokens, P));
  const int64_t c = std::max<int64_t>(c_min, ceil_div(work, target));
  if (c > std::numeric_limits<int32_t>::max()) {
    *err = "chunk size overflows int32";
    return false;
  }

  // Items in (b, tile, g, j) order, with their token counts. Slots are at
  // most the items, so both counts fit int32 once the items do.
  int64_t n_items = 0;
  for (const TileExtent& te : tiles)
    n_items += std::max<int64_t>(1, ceil_div(te.pages, c)) * in.num_kv_heads;
  if (n_items > std::numeric_limits<int32_t>::max()) {
    *err = "item count overflows int32";
    return false;
  }
  std::vector<PlanItem> gen(static_cast<size_t>(n_items));
  std::vector<uint32_t> tokens(static_cast<size_t>(n_items));
  size_t n = 0;
  int64_t slot = 0;
  uint32_t max_tokens = 0;
  for (const TileExtent& te : tiles) {
    const int64_t n_chunks = std::max<int64_t>(1, ceil_div(te.pages, c));
    for (int32_t g = 0; g < in.num_kv_heads; ++g) {
      int64_t slot_begin = -1;
      const bool grouped = n_chunks > 1 || in.group_all;
      if (grouped) {
        slot_begin = slot;
        MergeGroup mg{};
        mg.b = te.b;
        mg.tile = te.tile;
        mg.g = g;
        mg.slot_begin = static_cast<int32_t>(slot_begin);
        mg.num_chunks = static_cast<int32_t>(n_chunks);
        out->groups.push_back(mg);
        slot += n_chunks;
      }
      for (int64_t j = 0; j < n_chunks; ++j) {
        PlanItem& it = gen[n];
        it.b = te.b;
        it.g = g;
        it.tile = te.tile;
        it.page_begin = static_cast<int32_t>(te.page_lo + j * c);
        it.page_end = static_cast<int32_t>(te.page_lo + std::min((j + 1) * c, te.pages));
        const int64_t k0 = std::min((te.page_lo + j * c) * P, te.kv_end);
        const int64_t k1 = std::min((te.page_lo + (j + 1) * c) * P, te.kv_end);
        it.kv_begin = static_cast<int32_t>(k0);
        it.kv_end = static_cast<int32_t>(k1);
        it.slot = grouped ? static_cast<int32_t>(slot_begin + j) : -1;
        tokens[n] = static_cast<uint32_t>(k1 - k0);
        max_tokens = std::max(max_tokens, tokens[n]);
        ++n;
      }
    }
  }
  // Longest first; ties keep the (b, tile, g, j) order above. The key
  // max_tokens - tokens is sorted ascending by a stable least-significant-digit
  // radix sort over 11-bit digits (one pass while every item is shorter than
  // 2048 tokens, at most three).
  constexpr int kDigitBits = 11;
  constexpr uint32_t kDigits = 1u << kDigitBits;
  std::vector<uint32_t> order(n), next(n);
  for (size_t i = 0; i < n; ++i) order[i] = static_cast<uint32_t>(i);
  std::vector<uint32_t> count(kDigits + 1);
  for (int shift = 0; shift < 32 && (max_tokens >> shift) != 0; shift += kDigitBits) {
    std::fill(count.begin(), count.end(), 0u);
    for (size_t i = 0; i < n; ++i) ++count[((max_tokens - tokens[i]) >> shift) % kDigits + 1];
    for (uint32_t d = 0; d < kDigits; ++d) count[d + 1] += count[d];
    for (size_t i = 0; i < n; ++i) {
      const uint32_t k = order[i];
      next[count[((max_tokens - tokens[k]) >> shift) % kDigits]++] = k;
    }
    order.swap(next);
  }
  out->items.resize(n);
  for (size_t i = 0; i < n; ++i) out->items[i] = gen[order[i]];
  out->chunk_pages = static_cast<int32_t>(c);
  out->num_slots = static_cast<int32_t>(slot);
  return true;
}

std::vector<int32_t> interleave_items(const std::vector<PlanItem>& a,
                                      const std::vector<PlanItem>& b) {
  auto cost = [](const PlanItem& it) -> int64_t { return int64_t{it.kv_end} - it.kv_begin + 1; };
  int64_t total_a = 0, total_b = 0;
  for (const PlanItem& it : a) total_a += cost(it);
  for (const PlanItem& it : b) total_b += cost(it);
  std::vector<int32_t> order;
  order.reserve(a.size() + b.size());
  size_t i = 0, j = 0;
  int64_t done_a = 0, done_b = 0;
  while (i < a.size() || j < b.size()) {
    // done_a / total_a <= done_b / total_b, in integers (both totals > 0 when
    // their list is non-empty; products stay far below 2^63)
    const bool take_a = j == b.size() || (i < a.size() && done_a * total_b <= done_b * total_a);
    if (take_a) {
      done_a += cost(a[i]);
      order.push_back(static_cast<int32_t>(i++));
    } else {
      done_b += cost(b[j]);
      order.push_back(-static_cast<int32_t>(j++) - 1);
    }
  }
  return order;
}

}  // namespace pkv
