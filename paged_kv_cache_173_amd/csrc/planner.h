// Host-side work-chunk planner: pure C++17, no HIP dependency.
//
// The FlashInfer article ("FlashInfer", section "Plan and run") describes a
// plan step that inspects sequence lengths and cache metadata, chooses a
// schedule and prepares workspace data, and a run step that reuses it; the
// section "Purpose and scope" notes that one fixed schedule leaves work
// unevenly spread. This file is this library's schedule: split each
// (request, query tile, KV head) group's KV range into equal page chunks so
// that the total work fills num_cus * wg_per_cu workgroup slots, and order
// the resulting items longest first.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace pkv {

// One workgroup's unit of work.
struct PlanItem {
  int32_t b, g, tile, page_begin, page_end, kv_begin, kv_end, slot;  // slot -1: final output
};
static_assert(sizeof(PlanItem) == 32, "PlanItem is 8 int32");

// A (request, tile, KV head) group whose KV range was split into chunks (or
// any group, with group_all). A cascade's suffix group also names the prefix
// states its merge adds: base_num_chunks slots from base_slot_begin of the
// prefix part, at row base_row of each (all 0 elsewhere).
struct MergeGroup {
  int32_t b, tile, g, slot_begin, num_chunks, base_slot_begin, base_num_chunks, base_row;
};
static_assert(sizeof(MergeGroup) == 32, "MergeGroup is 8 int32");

struct PlanInput {
  const int64_t* qo_lens;  // per request
  const int64_t* kv_lens;  // per request
  int32_t batch;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t group_size;      // G = num_qo_heads / num_kv_heads
  int32_t rows_per_tile;   // G for decode, 128 for prefill
  bool causal;
  int32_t window_left;     // W >= 0: a row at position p sees keys >= p - W; < 0: no window
  int32_t num_cus;
  int32_t wg_per_cu;
  int32_t min_chunk_tokens;
  // Every (request, tile, KV head) group becomes a merge group with partial-
  // state slots, also when it is one chunk (so that a merge can add a further
  // state to every row).
  bool group_all = false;
};

struct HostPlan {
  int32_t chunk_pages = 0;
  int32_t num_slots = 0;
  std::vector<PlanItem> items;
  std::vector<MergeGroup> groups;
};

// Applies the rule. Returns false (with *err set) if a count overflows int32.
bool build_plan(const PlanInput& in, HostPlan* out, std::string* err);

// Launch order of one grid that runs the items of two plans (the mixed
// prefill + decode launch): entry >= 0 is item `entry` of `a`, entry < 0 is
// item -entry-1 of `b`. Each list keeps its own order. An item costs its KV
// token count plus one; the next entry comes from the list whose emitted share
// of its own total cost is smaller (a on ties), so the two kinds advance at the
// same relative pace and every stretch of the grid mixes them.
std::vector<int32_t> interleave_items(const std::vector<PlanItem>& a,
                                      const std::vector<PlanItem>& b);

}  // namespace pkv
