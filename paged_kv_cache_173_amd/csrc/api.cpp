// C ABI of libpkv.so (declared in include/pkv.h): argument validation, the
// host plan, workspace layout, the plan's host-to-device copy, and kernel
// launches. Plan/run split, stable workspaces and reuse of a plan follow the
// FlashInfer article, section "Plan and run".
#include "pkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <limits>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "kernels.h"
#include "planner.h"

namespace {

thread_local std::string g_error;

constexpr uint32_t kPlanMagic = 0x31564b50u;  // "PKV1"
constexpr int64_t kAlign = 256;
constexpr int32_t kRowsPerPrefillTile = 128;
// The mixed prefill + decode kernel runs 128-row prefill items (one row block
// per wave, two workgroups per CU), whatever the prefill kernel uses.
constexpr int32_t kRowsPerPodPrefillTile = 128;
constexpr int32_t kMaxDecodeGroup = 16;

pkv_status fail(pkv_status st, const std::string& msg) {
  g_error = msg;
  return st;
}

pkv_status ok() {
  g_error.clear();
  return PKV_OK;
}

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pkv_status hip_fail(hipError_t e, const char* what) {
  return fail(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

pkv_status check_heads(int32_t num_qo_heads, int32_t num_kv_heads) {
  if (num_qo_heads <= 0 || num_kv_heads <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_qo_heads and num_kv_heads must be positive");
  if (num_qo_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_qo_heads must be a multiple of num_kv_heads");
  return PKV_OK;
}

pkv_status check_head_dim_dtype(int32_t head_dim, pkv_dtype dtype) {
  if (head_dim <= 0) return fail(PKV_ERR_INVALID_ARG, "head_dim must be positive");
  if (head_dim != pkv::kHeadDimSupported)
    return fail(PKV_ERR_UNSUPPORTED, "only head_dim 128 is implemented");
  if (dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(dtype == PKV_F32 ? PKV_ERR_UNSUPPORTED : PKV_ERR_INVALID_ARG,
                "attention storage dtype must be PKV_F16 or PKV_BF16");
  return PKV_OK;
}

pkv_status check_sched(const pkv_sched* s) {
  if (s->num_cus <= 0 || s->wg_per_cu <= 0 || s->min_chunk_tokens <= 0)
    return fail(PKV_ERR_INVALID_ARG, "sched fields must be positive");
  return PKV_OK;
}

pkv_status resolve_sched(const pkv_sched* in, pkv_kind kind, pkv_sched* out) {
  if (in != nullptr) {
    *out = *in;
    return check_sched(out);
  }
  int32_t dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return pkv_default_sched_for(kind, dev, out);
}

// Page table on the host: monotone indptr, last_page_len within [1, P] for a
// request with pages and 0 for an empty one. Fills per-request KV lengths.
pkv_status check_page_table(const int32_t* kv_indptr, const int32_t* last_page_len,
                            int32_t batch, int32_t page_size, std::vector<int64_t>* kv_lens) {
  if (batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch must be >= 0");
  if (page_size <= 0) return fail(PKV_ERR_INVALID_ARG, "page_size must be positive");
  if (kv_indptr == nullptr || (batch > 0 && last_page_len == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "kv_indptr / last_page_len host arrays are NULL");
  if (kv_indptr[0] < 0) return fail(PKV_ERR_INVALID_ARG, "kv_indptr[0] must be >= 0");
  kv_lens->resize(batch);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = static_cast<int64_t>(kv_indptr[b + 1]) - kv_indptr[b];
    if (n < 0) return fail(PKV_ERR_INVALID_ARG, "kv_indptr is not monotone at " + std::to_string(b));
    const int32_t lpl = last_page_len[b];
    if (n == 0) {
      if (lpl != 0)
        return fail(PKV_ERR_INVALID_ARG,
                    "last_page_len must be 0 for request " + std::to_string(b) + " with no pages");
      (*kv_lens)[b] = 0;
    } else {
      if (lpl < 1 || lpl > page_size)
        return fail(PKV_ERR_INVALID_ARG, "last_page_len[" + std::to_string(b) +
                                             "] must be in [1, page_size]");
      const int64_t L = (n - 1) * page_size + lpl;
      if (L > INT32_MAX) return fail(PKV_ERR_INVALID_ARG, "KV length overflows int32");
      (*kv_lens)[b] = L;
    }
  }
  return PKV_OK;
}

pkv_status check_qo_indptr(const int32_t* qo_indptr, int32_t batch, std::vector<int64_t>* qo_lens) {
  if (qo_indptr == nullptr) return fail(PKV_ERR_INVALID_ARG, "qo_indptr host array is NULL");
  if (qo_indptr[0] < 0) return fail(PKV_ERR_INVALID_ARG, "qo_indptr[0] must be >= 0");
  qo_lens->resize(batch);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t q = static_cast<int64_t>(qo_indptr[b + 1]) - qo_indptr[b];
    if (q < 0) return fail(PKV_ERR_INVALID_ARG, "qo_indptr is not monotone at " + std::to_string(b));
    (*qo_lens)[b] = q;
  }
  return PKV_OK;
}

pkv_status check_kv(const pkv_paged_kv* kv, const pkv_plan_info* plan) {
  if (kv == nullptr || kv->k == nullptr || kv->v == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "paged KV (or its k / v pointer) is NULL");
  if (kv->page_size != plan->page_size || kv->num_kv_heads != plan->num_kv_heads ||
      kv->head_dim != plan->head_dim || kv->dtype != plan->dtype)
    return fail(PKV_ERR_PLAN_MISMATCH, "paged KV geometry / dtype differs from the plan's");
  if (kv->page_stride % 8 || kv->token_stride % 8 || kv->head_stride % 8 || kv->page_stride < 0 ||
      kv->token_stride < 0 || kv->head_stride < 0)
    return fail(PKV_ERR_INVALID_ARG, "KV strides must be non-negative multiples of 8 elements");
  if (!aligned16(kv->k) || !aligned16(kv->v))
    return fail(PKV_ERR_INVALID_ARG, "k / v must be 16-byte aligned");
  if (kv->token_stride < kv->head_dim || kv->token_stride > (INT32_MAX / 32))
    return fail(PKV_ERR_INVALID_ARG, "token_stride must be in [head_dim, 2^26)");
  if (kv->page_stride >= (int64_t{1} << 30))
    return fail(PKV_ERR_INVALID_ARG, "page_stride must be below 2^30 elements");
  return PKV_OK;
}

pkv_status check_scale(float sm_scale) {
  if (!(sm_scale > 0.f) || sm_scale > 3.0e38f)
    return fail(PKV_ERR_INVALID_ARG, "sm_scale must be finite and positive");
  return PKV_OK;
}

pkv_status check_plan(const pkv_plan_info* plan, pkv_kind kind) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  if (plan->magic != kPlanMagic || plan->abi_version != PKV_ABI_VERSION)
    return fail(PKV_ERR_PLAN_MISMATCH, "not a plan made by this library version");
  if (plan->kind != kind) return fail(PKV_ERR_PLAN_MISMATCH, "plan kind differs from this call");
  return PKV_OK;
}

// The window of a plan call's variant (-1 for none), validated.
pkv_status plan_window(const pkv_variant* v, int32_t* window_left) {
  *window_left = v != nullptr ? v->window_left : -1;
  if (*window_left < -1) return fail(PKV_ERR_INVALID_ARG, "window_left must be -1 or >= 0");
  return PKV_OK;
}

// Validates a run call's variant against the plan part and fills the
// kernels' variant arguments (all off for NULL).
pkv_status resolve_variant(const pkv_variant* v, const pkv_plan_part& part, float sm_scale,
                           pkv::VariantArgs* out) {
  *out = pkv::VariantArgs{-1, 0.f, 0.f, nullptr};
  int32_t w;
  pkv_status st;
  if ((st = plan_window(v, &w))) return st;
  if (w != part.window_left)
    return fail(PKV_ERR_PLAN_MISMATCH, "window_left differs from the one the plan was made for");
  if (v == nullptr) return PKV_OK;
  const float c = v->logits_soft_cap;
  if (!(c >= 0.f) || c > 3.0e38f)
    return fail(PKV_ERR_INVALID_ARG, "logits_soft_cap must be finite and >= 0");
  if (reinterpret_cast<uintptr_t>(v->sinks) % 4 != 0)
    return fail(PKV_ERR_INVALID_ARG, "sinks must be 4-byte aligned");
  out->window_left = w;
  out->sinks = v->sinks;
  if (c > 0.f) {
    const double cin = 2.0 * 1.4426950408889634 * sm_scale / c;
    const double cout = static_cast<double>(c) / sm_scale;
    if (!(cin < 3.0e38) || !(cout < 3.0e38) || !(cin > 1e-37) || !(cout > 1e-37))
      return fail(PKV_ERR_INVALID_ARG, "logits_soft_cap out of range for this sm_scale");
    out->cap_in = static_cast<float>(cin);
    out->cap_out = static_cast<float>(cout);
  }
  return PKV_OK;
}

const pkv::VariantArgs kNoVariant{-1, 0.f, 0.f, nullptr};

struct Layout {
  int64_t int_bytes = 0;
  int64_t float_bytes = 0;
};

// Places one part's tables (items, merge groups: 8 int32 each; KV lengths:
// batch int32) and partial states (num_slots slots of rows_per_tile rows: O
// [128] and (m, l)) at the current end of each workspace.
void place_counts(int64_t num_items, int64_t num_groups, int64_t num_slots, int32_t chunk_pages,
                  int64_t batch, int32_t rows_per_tile, int32_t causal, Layout* lay,
                  pkv_plan_part* part, int32_t window_left = -1) {
  part->num_items = static_cast<int32_t>(num_items);
  part->num_groups = static_cast<int32_t>(num_groups);
  part->chunk_pages = chunk_pages;
  part->rows_per_tile = rows_per_tile;
  part->num_slots = static_cast<int32_t>(num_slots);
  part->causal = causal;
  part->window_left = window_left;
  part->items_off = lay->int_bytes;
  lay->int_bytes = align_up(lay->int_bytes + num_items * 32);
  part->groups_off = lay->int_bytes;
  lay->int_bytes = align_up(lay->int_bytes + num_groups * 32);
  part->kv_len_off = lay->int_bytes;
  lay->int_bytes = align_up(lay->int_bytes + batch * 4);
  part->part_o_off = lay->float_bytes;
  lay->float_bytes =
      align_up(lay->float_bytes + num_slots * rows_per_tile * pkv::kHeadDimSupported * 4);
  part->part_ml_off = lay->float_bytes;
  lay->float_bytes = align_up(lay->float_bytes + num_slots * rows_per_tile * 8);
}

void place_part(const pkv::HostPlan& hp, int64_t batch, int32_t rows_per_tile, int32_t causal,
                Layout* lay, pkv_plan_part* part, int32_t window_left = -1) {
  place_counts(static_cast<int64_t>(hp.items.size()), static_cast<int64_t>(hp.groups.size()),
               hp.num_slots, hp.chunk_pages, batch, rows_per_tile, causal, lay, part,
               window_left);
}

void write_part(const pkv::HostPlan& hp, const std::vector<int64_t>& kv_lens,
                const pkv_plan_part& part, char* host) {
  int32_t* lens = reinterpret_cast<int32_t*>(host + part.kv_len_off);
  for (size_t b = 0; b < kv_lens.size(); ++b) lens[b] = static_cast<int32_t>(kv_lens[b]);
  if (!hp.items.empty())
    std::memcpy(host + part.items_off, hp.items.data(), hp.items.size() * sizeof(pkv::PlanItem));
  if (!hp.groups.empty())
    std::memcpy(host + part.groups_off, hp.groups.data(),
                hp.groups.size() * sizeof(pkv::MergeGroup));
}

// The last plan copy out of each host staging buffer: an event recorded on the
// copy's stream right after it. A plan call waits for that event before it
// writes the same buffer again, so one staging buffer serves every plan call
// without the plan waiting for its own copy (or for the work queued before it).
struct StagingCopy {
  hipEvent_t done = nullptr;
  hipDevice_t device = -1;
};
std::mutex g_staging_mu;
std::unordered_map<const void*, StagingCopy> g_staging;

// Sets *h to host_ws once no earlier plan copy still reads it, or to NULL when
// host_ws is NULL or smaller than `need` (nothing is written then).
pkv_status claim_staging(void* host_ws, size_t host_ws_bytes, int64_t need, char** h) {
  *h = nullptr;
  if (host_ws == nullptr || host_ws_bytes < static_cast<size_t>(need)) return PKV_OK;
  hipEvent_t done = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_staging_mu);
    auto it = g_staging.find(host_ws);
    if (it != g_staging.end()) done = it->second.done;
  }
  // Only a plan call on this same buffer replaces its event, and such calls
  // do not overlap (documented), so the handle stays valid without the lock.
  if (done != nullptr) {
    const hipError_t e = hipEventSynchronize(done);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(plan staging copy)");
  }
  *h = static_cast<char*>(host_ws);
  return PKV_OK;
}

// Records the completion of a copy out of host_ws queued on `stream`.
pkv_status record_staging(const void* host_ws, hipStream_t stream) {
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  std::lock_guard<std::mutex> lock(g_staging_mu);
  StagingCopy& c = g_staging[host_ws];
  if (c.done != nullptr && c.device != dev) {
    (void)hipEventDestroy(c.done);
    c.done = nullptr;
  }
  if (c.done == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    e = hipEventCreateWithFlags(&c.done, hipEventDisableTiming);
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) {
      c.done = nullptr;
      g_staging.erase(host_ws);
      return hip_fail(e, "hipEventCreateWithFlags(plan staging copy)");
    }
    c.device = dev;
  }
  if ((e = hipEventRecord(c.done, stream)) != hipSuccess)
    return hip_fail(e, "hipEventRecord(plan staging copy)");
  return PKV_OK;
}

// Checks the workspaces, then queues the copy of host_ws[0:int_bytes] to
// int_ws on the stream and records its completion for host_ws.
pkv_status commit_plan(const Layout& lay, void* int_ws, size_t int_ws_bytes, void* float_ws,
                       size_t float_ws_bytes, void* host_ws, size_t host_ws_bytes,
                       hipStream_t stream, pkv_plan_info* out) {
  out->int_ws_required = lay.int_bytes;
  out->float_ws_required = lay.float_bytes;
  if ((lay.int_bytes > 0 && (int_ws == nullptr || int_ws_bytes < static_cast<size_t>(lay.int_bytes))) ||
      (lay.float_bytes > 0 &&
       (float_ws == nullptr || float_ws_bytes < static_cast<size_t>(lay.float_bytes))) ||
      (lay.int_bytes > 0 &&
       (host_ws == nullptr || host_ws_bytes < static_cast<size_t>(lay.int_bytes))))
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL,
                "workspace too small: need int " + std::to_string(lay.int_bytes) + " B, float " +
                    std::to_string(lay.float_bytes) + " B, host " + std::to_string(lay.int_bytes) +
                    " B");
  if (!aligned16(int_ws) || !aligned16(float_ws))
    return fail(PKV_ERR_INVALID_ARG, "workspaces must be 16-byte aligned");
  out->int_ws = int_ws;
  out->float_ws = float_ws;
  if (lay.int_bytes > 0) {
    hipError_t e = hipMemcpyAsync(int_ws, host_ws, lay.int_bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
    pkv_status st = record_staging(host_ws, stream);
    if (st) return st;
  }
  return PKV_OK;
}

void fill_header(pkv_plan_info* out, pkv_kind kind, pkv_dtype dtype, int32_t batch, int32_t hq,
                 int32_t hkv, int32_t head_dim, int32_t page_size, int32_t total_qo,
                 const pkv_sched& sched) {
  std::memset(out, 0, sizeof(*out));
  out->magic = kPlanMagic;
  out->abi_version = PKV_ABI_VERSION;
  out->kind = kind;
  out->dtype = dtype;
  out->batch = batch;
  out->num_qo_heads = hq;
  out->num_kv_heads = hkv;
  out->head_dim = head_dim;
  out->page_size = page_size;
  out->total_qo = total_qo;
  out->sched = sched;
}

// Both cascade levels: every group writes partial states, which the level-1
// merge combines (each suffix group with its prefix states).
pkv::PlanInput all_groups(pkv::PlanInput in) {
  in.group_all = true;
  return in;
}

pkv::PlanInput make_input(const std::vector<int64_t>& qo, const std::vector<int64_t>& kv,
                          int32_t page_size, int32_t hkv, int32_t G, int32_t rows, bool causal,
                          const pkv_sched& s, int32_t window_left = -1) {
  pkv::PlanInput in{};
  in.qo_lens = qo.data();
  in.kv_lens = kv.data();
  in.batch = static_cast<int32_t>(kv.size());
  in.page_size = page_size;
  in.num_kv_heads = hkv;
  in.group_size = G;
  in.rows_per_tile = rows;
  in.causal = causal;
  in.window_left = window_left;
  in.num_cus = s.num_cus;
  in.wg_per_cu = s.wg_per_cu;
  in.min_chunk_tokens = s.min_chunk_tokens;
  return in;
}

pkv::PageMode page_mode(int32_t page_size) {
  return page_size % 16 == 0 ? pkv::kPagedUniform : pkv::kPagedGeneric;
}

const char* ws_at(const void* base, int64_t off) { return static_cast<const char*>(base) + off; }
float* f_at(void* base, int64_t off) {
  return reinterpret_cast<float*>(static_cast<char*>(base) + off);
}
const int32_t* i_at(const void* base, int64_t off) {
  return reinterpret_cast<const int32_t*>(ws_at(base, off));
}

// The decode kernel's arguments for one planned part.
pkv::DecodeArgs decode_args(const pkv_plan_info* plan, const pkv_plan_part& part, const void* q,
                            const pkv_paged_kv* kv, const int32_t* kv_indptr_d,
                            const int32_t* kv_indices_d, float sm_scale, void* o, float* lse,
                            const pkv::VariantArgs& var) {
  pkv::DecodeArgs a{};
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.page_stride = kv->page_stride;
  a.token_stride = kv->token_stride;
  a.head_stride = kv->head_stride;
  a.kv_indptr = kv_indptr_d;
  a.kv_indices = kv_indices_d;
  a.items = i_at(plan->int_ws, part.items_off);
  a.page_size = plan->page_size;
  a.num_qo_heads = plan->num_qo_heads;
  a.group = plan->num_qo_heads / plan->num_kv_heads;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.o = o;
  a.lse = lse;
  a.part_o = f_at(plan->float_ws, part.part_o_off);
  a.part_ml = f_at(plan->float_ws, part.part_ml_off);
  a.kv_lens = i_at(plan->int_ws, part.kv_len_off);
  a.var = var;
  return a;
}

// The prefill kernel's arguments for one planned part.
pkv::PrefillArgs prefill_args(const pkv_plan_info* plan, const pkv_plan_part& part, const void* q,
                              const pkv_paged_kv* kv, const int32_t* qo_indptr_d,
                              const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                              float sm_scale, void* o, float* lse, int32_t num_qo_heads,
                              const pkv::VariantArgs& var) {
  pkv::PrefillArgs a{};
  a.q = q;
  a.k = kv->k;
  a.v = kv->v;
  a.page_stride = kv->page_stride;
  a.token_stride = kv->token_stride;
  a.head_stride = kv->head_stride;
  a.qo_indptr = qo_indptr_d;
  a.kv_indptr = kv_indptr_d;
  a.kv_indices = kv_indices_d;
  a.items = i_at(plan->int_ws, part.items_off);
  a.kv_lens = i_at(plan->int_ws, part.kv_len_off);
  a.page_size = plan->page_size;
  a.num_qo_heads = num_qo_heads;
  a.group = num_qo_heads / plan->num_kv_heads;
  a.causal = part.causal;
  a.rows_per_tile = part.rows_per_tile;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.o = o;
  a.lse = lse;
  a.part_o = f_at(plan->float_ws, part.part_o_off);
  a.part_ml = f_at(plan->float_ws, part.part_ml_off);
  a.var = var;
  return a;
}

// The prefix states a cascade's suffix merge adds (none elsewhere).
struct BaseStates {
  const float* o = nullptr;
  const float* ml = nullptr;
  int32_t rows = 0;
  int32_t tile_slots = 0;
  int64_t states_per_group = 0;
};

// Merges a part's split groups (if any) into its final rows.
pkv_status merge_part(const pkv_plan_part& part, bool prefill, const int32_t* qo_indptr_d,
                      int32_t num_qo_heads, int32_t group, const void* int_ws, void* float_ws,
                      void* o, float* lse, const float* sinks, pkv_dtype dtype,
                      pkv::OutKind out_kind, hipStream_t stream, const BaseStates& base = {}) {
  if (part.num_groups == 0) return PKV_OK;
  pkv::MergeGroupsArgs m{};
  m.groups = i_at(int_ws, part.groups_off);
  m.rows_per_tile = part.rows_per_tile;
  m.num_qo_heads = num_qo_heads;
  m.group = group;
  m.prefill = prefill ? 1 : 0;
  m.qo_indptr = qo_indptr_d;
  m.part_o = f_at(float_ws, part.part_o_off);
  m.part_ml = f_at(float_ws, part.part_ml_off);
  m.o = o;
  m.lse = lse;
  m.sinks = sinks;
  m.base_o = base.o;
  m.base_ml = base.ml;
  m.base_rows = base.rows;
  m.base_tile_slots = base.tile_slots;
  const int64_t states = part.num_slots + base.states_per_group * part.num_groups;
  const hipError_t e = pkv::launch_merge_groups(m, dtype, out_kind, part.num_groups, states, stream);
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return PKV_OK;
}

// The caller's timing events (hipEvent_t passed as void*, either may be NULL),
// carried by the attention kernel's own dispatch.
pkv::LaunchEvents launch_events(void* start, void* stop) {
  return {static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)};
}

// Launches one decode pass (items, then the merge of split groups) writing
// final rows to o / lse.
pkv_status run_decode_part(const pkv_plan_info* plan, const pkv_plan_part& part, const void* q,
                           const pkv_paged_kv* kv, const int32_t* kv_indptr_d,
                           const int32_t* kv_indices_d, float sm_scale, void* o, float* lse,
                           pkv::OutKind out_kind, hipStream_t stream,
                           const pkv::LaunchEvents& ev = {},
                           const pkv::VariantArgs& var = kNoVariant,
                           const BaseStates& base = {}) {
  const pkv::DecodeArgs a =
      decode_args(plan, part, q, kv, kv_indptr_d, kv_indices_d, sm_scale, o, lse, var);
  const hipError_t e = pkv::launch_decode(a, plan->dtype, out_kind, page_mode(plan->page_size),
                                          part.num_items, stream, ev);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  return merge_part(part, false, nullptr, plan->num_qo_heads, a.group, plan->int_ws,
                    plan->float_ws, o, lse, var.sinks, plan->dtype, out_kind, stream, base);
}

// Launches one prefill pass and, when `merge` is set, the merge of its split
// groups into o / lse (the cascade's level 0 leaves its chunk states for the
// level-1 merge instead).
pkv_status run_prefill_part(const pkv_plan_info* plan, const pkv_plan_part& part, const void* q,
                            const pkv_paged_kv* kv, const int32_t* qo_indptr_d,
                            const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                            float sm_scale, void* o, float* lse, int32_t num_qo_heads,
                            pkv::OutKind out_kind, hipStream_t stream,
                            const pkv::LaunchEvents& ev = {},
                            const pkv::VariantArgs& var = kNoVariant, bool merge = true) {
  const pkv::PrefillArgs a = prefill_args(plan, part, q, kv, qo_indptr_d, kv_indptr_d,
                                          kv_indices_d, sm_scale, o, lse, num_qo_heads, var);
  const hipError_t e = pkv::launch_prefill(a, plan->dtype, out_kind, page_mode(plan->page_size),
                                           part.num_items, stream, ev);
  if (e != hipSuccess) return hip_fail(e, "prefill kernel launch");
  if (!merge) return PKV_OK;
  return merge_part(part, true, qo_indptr_d, num_qo_heads, a.group, plan->int_ws, plan->float_ws,
                    o, lse, var.sinks, plan->dtype, out_kind, stream);
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_error.c_str(); }

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

size_t pkv_plan_info_size(void) { return sizeof(pkv_plan_info); }

pkv_status pkv_default_sched(int32_t device, pkv_sched* out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CU count)");
  out->num_cus = cus;
  out->wg_per_cu = 4;
  // Chunks of 128 tokens: the single 1024-token decode (32 heads) runs 256
  // items instead of 128 and its step drops from 14.5 to 13.0 us; 64 tokens
  // gains no more and 32 loses it again.
  out->min_chunk_tokens = 128;
  return ok();
}

pkv_status pkv_default_sched_for(pkv_kind kind, int32_t device, pkv_sched* out) {
  if (kind != PKV_KIND_DECODE && kind != PKV_KIND_PREFILL)
    return fail(PKV_ERR_INVALID_ARG, "kind must be PKV_KIND_DECODE or PKV_KIND_PREFILL");
  pkv_status st = pkv_default_sched(device, out);
  if (st) return st;
  int32_t cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return hip_fail(e, "hipSetDevice");
  const int32_t occ = kind == PKV_KIND_DECODE ? pkv::decode_occupancy() : pkv::prefill_occupancy();
  if (cur != device) (void)hipSetDevice(cur);
  // Decode: about two and a half waves of items per resident workgroup (rounded
  // down), so that the longest-first order evens out the last wave (one wave
  // left ~5 % idle at the end on the 64-request and 4 x 128k-token workloads).
  // Prefill: one wave; its tiles already give several items per workgroup.
  if (occ > 0) out->wg_per_cu = kind == PKV_KIND_DECODE ? (5 * occ) / 2 : occ;
  return ok();
}

pkv_status pkv_workspace_size(pkv_kind kind, int32_t batch, int32_t num_qo_heads,
                              int32_t num_kv_heads, int32_t head_dim, int64_t max_items,
                              size_t* int_ws_bytes, size_t* float_ws_bytes,
                              size_t* host_ws_bytes) {
  if (int_ws_bytes == nullptr || float_ws_bytes == nullptr || host_ws_bytes == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "output pointers must be non-NULL");
  if (batch < 0 || max_items < 0) return fail(PKV_ERR_INVALID_ARG, "batch and max_items must be >= 0");
  if (num_qo_heads <= 0 || num_kv_heads <= 0 || num_qo_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_qo_heads must be a positive multiple of num_kv_heads");
  if (head_dim != pkv::kHeadDimSupported)
    return fail(PKV_ERR_UNSUPPORTED, "only head_dim 128 is implemented");
  if (max_items > std::numeric_limits<int32_t>::max())
    return fail(PKV_ERR_INVALID_ARG, "max_items overflows int32");
  const int32_t G = num_qo_heads / num_kv_heads;
  // A plan of any lengths with at most max_items items: its merge groups and
  // partial-state slots are never more than its items, so max_items of each,
  // placed the way the kind's plan call places its parts, bounds every table.
  // Two-part kinds give each part the whole bound.
  const int64_t n = max_items;
  Layout lay;
  pkv_plan_part part[2]{};
  switch (kind) {
    case PKV_KIND_DECODE:
      if (G > kMaxDecodeGroup) return fail(PKV_ERR_UNSUPPORTED, "decode supports G <= 16");
      place_counts(n, n, n, 0, batch, G, 0, &lay, &part[0]);
      break;
    case PKV_KIND_PREFILL:
      if (G > kRowsPerPrefillTile) return fail(PKV_ERR_UNSUPPORTED, "prefill supports G <= 128");
      place_counts(n, n, n, 0, batch, kRowsPerPrefillTile, 0, &lay, &part[0]);
      break;
    case PKV_KIND_BLOCK_SPARSE:   // batch = query blocks
      if (G > kRowsPerPrefillTile) return fail(PKV_ERR_UNSUPPORTED, "prefill supports G <= 128");
      lay.int_bytes = align_up((static_cast<int64_t>(batch) + 1) * 4);
      place_counts(n, n, n, 0, batch, kRowsPerPrefillTile, 0, &lay, &part[0]);
      break;
    case PKV_KIND_CASCADE: {      // batch = requests (suffixes)
      if (G > kMaxDecodeGroup) return fail(PKV_ERR_UNSUPPORTED, "cascade supports G <= 16");
      lay.int_bytes = kAlign;
      place_counts(n, n, n, 0, 1, kRowsPerPrefillTile, 0, &lay, &part[0]);
      place_counts(n, n, n, 0, batch, G, 0, &lay, &part[1]);
      break;
    }
    case PKV_KIND_POD:            // batch = prefill requests + decode requests
      if (G > kMaxDecodeGroup) return fail(PKV_ERR_UNSUPPORTED, "the mixed launch supports G <= 16");
      place_counts(n, n, n, 0, batch, kRowsPerPodPrefillTile, 0, &lay, &part[0]);
      place_counts(n, n, n, 0, batch, G, 0, &lay, &part[1]);
      lay.int_bytes = align_up(lay.int_bytes + n * 4);
      break;
    default:
      return fail(PKV_ERR_INVALID_ARG, "unknown plan kind");
  }
  *int_ws_bytes = static_cast<size_t>(lay.int_bytes);
  *float_ws_bytes = static_cast<size_t>(lay.float_bytes);
  *host_ws_bytes = static_cast<size_t>(lay.int_bytes);
  return ok();
}

pkv_status pkv_plan_export(const pkv_plan_info* plan, const void* host_ws, int32_t part,
                           int32_t* items_out, int32_t items_cap, int32_t* groups_out,
                           int32_t groups_cap) {
  if (plan == nullptr) return fail(PKV_ERR_INVALID_ARG, "plan is NULL");
  if (plan->magic != kPlanMagic || plan->abi_version != PKV_ABI_VERSION)
    return fail(PKV_ERR_PLAN_MISMATCH, "not a plan made by this library version");
  const bool two_parts = plan->kind == PKV_KIND_CASCADE || plan->kind == PKV_KIND_POD;
  if (part < 0 || part > (two_parts ? 1 : 0))
    return fail(PKV_ERR_INVALID_ARG, "part must be 0 (or 1 for a cascade or mixed-batch plan)");
  const pkv_plan_part& pp = plan->part[part];
  if (items_cap < pp.num_items || groups_cap < pp.num_groups)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL,
                "need room for " + std::to_string(pp.num_items) + " items and " +
                    std::to_string(pp.num_groups) + " groups");
  if ((pp.num_items > 0 || pp.num_groups > 0) && host_ws == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "host_ws is NULL");
  if ((pp.num_items > 0 && items_out == nullptr) || (pp.num_groups > 0 && groups_out == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "output arrays must be non-NULL when the part has rows");
  const char* h = static_cast<const char*>(host_ws);
  if (pp.num_items > 0)
    std::memcpy(items_out, h + pp.items_off, static_cast<size_t>(pp.num_items) * 32);
  if (pp.num_groups > 0)
    std::memcpy(groups_out, h + pp.groups_off, static_cast<size_t>(pp.num_groups) * 32);
  return ok();
}

pkv_status pkv_plan_host(pkv_kind kind, const int32_t* qo_indptr_h, const int32_t* kv_indptr_h,
                         const int32_t* last_page_len_h, int32_t batch, int32_t num_qo_heads,
                         int32_t num_kv_heads, int32_t page_size, int32_t causal,
                         int32_t window_left, const pkv_sched* sched, int32_t* items_out,
                         int32_t items_cap, int32_t* groups_out, int32_t groups_cap,
                         int32_t* counts_out) {
  if (sched == nullptr) return fail(PKV_ERR_INVALID_ARG, "pkv_plan_host needs an explicit sched");
  if (counts_out == nullptr) return fail(PKV_ERR_INVALID_ARG, "counts_out is NULL");
  pkv_status st = check_sched(sched);
  if (st) return st;
  if ((st = check_heads(num_qo_heads, num_kv_heads))) return st;
  if (kind != PKV_KIND_DECODE && kind != PKV_KIND_PREFILL)
    return fail(PKV_ERR_INVALID_ARG, "kind must be PKV_KIND_DECODE or PKV_KIND_PREFILL");
  if (window_left < -1) return fail(PKV_ERR_INVALID_ARG, "window_left must be -1 or >= 0");
  if (window_left < -1) return fail(PKV_ERR_INVALID_ARG, "window_left must be -1 or >= 0");
  std::vector<int64_t> kv_lens, qo_lens;
  if ((st = check_page_table(kv_indptr_h, last_page_len_h, batch, page_size, &kv_lens))) return st;
  const int32_t G = num_qo_heads / num_kv_heads;
  int32_t rows;
  if (kind == PKV_KIND_DECODE) {
    qo_lens.assign(batch, 1);
    rows = G;
    causal = 0;
  } else {
    if ((st = check_qo_indptr(qo_indptr_h, batch, &qo_lens))) return st;
    rows = kRowsPerPrefillTile;
  }
  pkv::HostPlan hp;
  std::string err;
  if (!pkv::build_plan(make_input(qo_lens, kv_lens, page_size, num_kv_heads, G, rows, causal != 0,
                                  *sched, window_left),
                       &hp, &err))
    return fail(PKV_ERR_INVALID_ARG, err);
  counts_out[0] = static_cast<int32_t>(hp.items.size());
  counts_out[1] = static_cast<int32_t>(hp.groups.size());
  counts_out[2] = hp.chunk_pages;
  counts_out[3] = hp.num_slots;
  if (static_cast<int64_t>(hp.items.size()) > items_cap ||
      static_cast<int64_t>(hp.groups.size()) > groups_cap)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "items_cap / groups_cap too small");
  if (!hp.items.empty()) {
    if (items_out == nullptr) return fail(PKV_ERR_INVALID_ARG, "items_out is NULL");
    std::memcpy(items_out, hp.items.data(), hp.items.size() * sizeof(pkv::PlanItem));
  }
  if (!hp.groups.empty()) {
    if (groups_out == nullptr) return fail(PKV_ERR_INVALID_ARG, "groups_out is NULL");
    std::memcpy(groups_out, hp.groups.data(), hp.groups.size() * sizeof(pkv::MergeGroup));
  }
  return ok();
}

pkv_status pkv_decode_plan(const int32_t* kv_indptr_h, const int32_t* last_page_len_h,
                           int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t page_size, pkv_dtype dtype,
                           const pkv_variant* variant, const pkv_sched* sched, void* int_ws,
                           size_t int_ws_bytes, void* float_ws, size_t float_ws_bytes,
                           void* host_ws, size_t host_ws_bytes, void* stream,
                           pkv_plan_info* out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  pkv_status st;
  int32_t window_left;
  if ((st = plan_window(variant, &window_left))) return st;
  if ((st = check_heads(num_qo_heads, num_kv_heads))) return st;
  if ((st = check_head_dim_dtype(head_dim, dtype))) return st;
  const int32_t G = num_qo_heads / num_kv_heads;
  if (G > kMaxDecodeGroup)
    return fail(PKV_ERR_UNSUPPORTED, "decode supports num_qo_heads / num_kv_heads <= 16");
  std::vector<int64_t> kv_lens;
  if ((st = check_page_table(kv_indptr_h, last_page_len_h, batch, page_size, &kv_lens))) return st;
  pkv_sched s;
  if ((st = resolve_sched(sched, PKV_KIND_DECODE, &s))) return st;
  std::vector<int64_t> qo_lens(batch, 1);
  pkv::HostPlan hp;
  std::string err;
  if (!pkv::build_plan(
          make_input(qo_lens, kv_lens, page_size, num_kv_heads, G, G, false, s, window_left), &hp,
          &err))
    return fail(PKV_ERR_INVALID_ARG, err);
  fill_header(out, PKV_KIND_DECODE, dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
              batch, s);
  Layout lay;
  place_part(hp, batch, G, 0, &lay, &out->part[0], window_left);
  char* h = nullptr;
  if ((st = claim_staging(host_ws, host_ws_bytes, lay.int_bytes, &h))) return st;
  if (h != nullptr) write_part(hp, kv_lens, out->part[0], h);
  if ((st = commit_plan(lay, int_ws, int_ws_bytes, float_ws, float_ws_bytes, host_ws,
                        host_ws_bytes, static_cast<hipStream_t>(stream), out)))
    return st;
  return ok();
}

pkv_status pkv_decode_run(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                          const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                          float sm_scale, const pkv_variant* variant, void* o, float* lse,
                          void* stream) {
  return pkv_decode_run_timed(plan, q, kv, kv_indptr_d, kv_indices_d, sm_scale, variant, o, lse,
                              stream, nullptr, nullptr);
}

pkv_status pkv_decode_run_timed(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                                const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                                float sm_scale, const pkv_variant* variant, void* o, float* lse,
                                void* stream, void* attention_start, void* attention_done) {
  pkv_status st;
  if ((st = check_scale(sm_scale))) return st;
  if ((st = check_plan(plan, PKV_KIND_DECODE))) return st;
  if ((st = check_kv(kv, plan))) return st;
  pkv::VariantArgs var;
  if ((st = resolve_variant(variant, plan->part[0], sm_scale, &var))) return st;
  if (plan->batch > 0 && (q == nullptr || o == nullptr || kv_indptr_d == nullptr ||
                          kv_indices_d == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "q, o, kv_indptr or kv_indices is NULL");
  if (!aligned16(q) || !aligned16(o)) return fail(PKV_ERR_INVALID_ARG, "q / o must be 16-byte aligned");
  if ((st = run_decode_part(plan, plan->part[0], q, kv, kv_indptr_d, kv_indices_d, sm_scale, o,
                            lse, pkv::kOutStorage, static_cast<hipStream_t>(stream),
                            launch_events(attention_start, attention_done), var)))
    return st;
  return ok();
}

pkv_status pkv_prefill_plan(const int32_t* qo_indptr_h, const int32_t* kv_indptr_h,
                            const int32_t* last_page_len_h, int32_t batch, int32_t num_qo_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            pkv_dtype dtype, int32_t causal, const pkv_variant* variant,
                            const pkv_sched* sched, void* int_ws, size_t int_ws_bytes,
                            void* float_ws, size_t float_ws_bytes, void* host_ws,
                            size_t host_ws_bytes, void* stream, pkv_plan_info* out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  pkv_status st;
  int32_t window_left;
  if ((st = plan_window(variant, &window_left))) return st;
  if ((st = check_heads(num_qo_heads, num_kv_heads))) return st;
  if ((st = check_head_dim_dtype(head_dim, dtype))) return st;
  if (causal != 0 && causal != 1) return fail(PKV_ERR_INVALID_ARG, "causal must be 0 or 1");
  const int32_t G = num_qo_heads / num_kv_heads;
  if (G > kRowsPerPrefillTile)
    return fail(PKV_ERR_UNSUPPORTED, "prefill supports num_qo_heads / num_kv_heads <= 128");
  std::vector<int64_t> kv_lens, qo_lens;
  if ((st = check_page_table(kv_indptr_h, last_page_len_h, batch, page_size, &kv_lens))) return st;
  if ((st = check_qo_indptr(qo_indptr_h, batch, &qo_lens))) return st;
  int64_t total_qo = 0;
  for (int64_t qn : qo_lens) total_qo += qn;
  if (total_qo * num_qo_heads > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "total query rows overflow int32");
  pkv_sched s;
  if ((st = resolve_sched(sched, PKV_KIND_PREFILL, &s))) return st;
  pkv::HostPlan hp;
  std::string err;
  if (!pkv::build_plan(make_input(qo_lens, kv_lens, page_size, num_kv_heads, G,
                                  kRowsPerPrefillTile, causal != 0, s, window_left),
                       &hp, &err))
    return fail(PKV_ERR_INVALID_ARG, err);
  fill_header(out, PKV_KIND_PREFILL, dtype, batch, num_qo_heads, num_kv_heads, head_dim,
              page_size, static_cast<int32_t>(total_qo), s);
  Layout lay;
  place_part(hp, batch, kRowsPerPrefillTile, causal, &lay, &out->part[0], window_left);
  char* h = nullptr;
  if ((st = claim_staging(host_ws, host_ws_bytes, lay.int_bytes, &h))) return st;
  if (h != nullptr) write_part(hp, kv_lens, out->part[0], h);
  if ((st = commit_plan(lay, int_ws, int_ws_bytes, float_ws, float_ws_bytes, host_ws,
                        host_ws_bytes, static_cast<hipStream_t>(stream), out)))
    return st;
  return ok();
}

pkv_status pkv_prefill_run(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                           const int32_t* qo_indptr_d, const int32_t* kv_indptr_d,
                           const int32_t* kv_indices_d, float sm_scale,
                           const pkv_variant* variant, void* o, float* lse, void* stream) {
  return pkv_prefill_run_timed(plan, q, kv, qo_indptr_d, kv_indptr_d, kv_indices_d, sm_scale,
                               variant, o, lse, stream, nullptr, nullptr);
}

pkv_status pkv_prefill_run_timed(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                                 const int32_t* qo_indptr_d, const int32_t* kv_indptr_d,
                                 const int32_t* kv_indices_d, float sm_scale,
                                 const pkv_variant* variant, void* o, float* lse, void* stream,
                                 void* attention_start, void* attention_done) {
  pkv_status st;
  if ((st = check_scale(sm_scale))) return st;
  if ((st = check_plan(plan, PKV_KIND_PREFILL))) return st;
  if ((st = check_kv(kv, plan))) return st;
  pkv::VariantArgs var;
  if ((st = resolve_variant(variant, plan->part[0], sm_scale, &var))) return st;
  if (plan->total_qo > 0 && (q == nullptr || o == nullptr || qo_indptr_d == nullptr ||
                             kv_indptr_d == nullptr || kv_indices_d == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "q, o, qo_indptr, kv_indptr or kv_indices is NULL");
  if (!aligned16(q) || !aligned16(o)) return fail(PKV_ERR_INVALID_ARG, "q / o must be 16-byte aligned");
  if ((st = run_prefill_part(plan, plan->part[0], q, kv, qo_indptr_d, kv_indptr_d, kv_indices_d,
                             sm_scale, o, lse, plan->num_qo_heads, pkv::kOutStorage,
                             static_cast<hipStream_t>(stream),
                             launch_events(attention_start, attention_done), var)))
    return st;
  return ok();
}

pkv_status pkv_single_decode(const void* q, const void* k, const void* v, int32_t kv_len,
                             int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                             pkv_dtype dtype, float sm_scale, const pkv_sched* sched,
                             void* float_ws, size_t float_ws_bytes, int64_t* float_ws_required,
                             void* o, float* lse, void* stream) {
  pkv_status st;
  if ((st = check_scale(sm_scale))) return st;
  if ((st = check_heads(num_qo_heads, num_kv_heads))) return st;
  if ((st = check_head_dim_dtype(head_dim, dtype))) return st;
  if (kv_len < 0) return fail(PKV_ERR_INVALID_ARG, "kv_len must be >= 0");
  const int32_t G = num_qo_heads / num_kv_heads;
  if (G > kMaxDecodeGroup)
    return fail(PKV_ERR_UNSUPPORTED, "decode supports num_qo_heads / num_kv_heads <= 16");
  pkv_sched s;
  if ((st = resolve_sched(sched, PKV_KIND_DECODE, &s))) return st;
  // The contiguous cache is a run of 16-token pages; the plan rule picks c.
  constexpr int32_t kVirtualPage = 16;
  std::vector<int64_t> qo_lens(1, 1), kv_lens(1, kv_len);
  pkv::HostPlan hp;
  std::string err;
  if (!pkv::build_plan(make_input(qo_lens, kv_lens, kVirtualPage, num_kv_heads, G, G, false, s),
                       &hp, &err))
    return fail(PKV_ERR_INVALID_ARG, err);
  const int64_t n_pages = (static_cast<int64_t>(kv_len) + kVirtualPage - 1) / kVirtualPage;
  const int64_t c = hp.chunk_pages;
  const int32_t nchunks = static_cast<int32_t>(std::max<int64_t>(1, (n_pages + c - 1) / c));
  // float_ws: the partial states O [Hkv * nchunks][G][128] and (m, l)
  // [Hkv * nchunks][G][2].
  const int64_t slots = static_cast<int64_t>(num_kv_heads) * nchunks;
  const int64_t o_bytes = align_up(slots * G * head_dim * 4);
  const int64_t need = nchunks > 1 ? o_bytes + slots * G * 8 : 0;
  if (float_ws_required != nullptr) *float_ws_required = need;
  if (need > 0 && (float_ws == nullptr || float_ws_bytes < static_cast<size_t>(need)))
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "float workspace too small: need " +
                                                 std::to_string(need) + " B");
  if (q == nullptr || o == nullptr || (kv_len > 0 && (k == nullptr || v == nullptr)))
    return fail(PKV_ERR_INVALID_ARG, "q, o, or (kv_len > 0) k or v is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(float_ws))
    return fail(PKV_ERR_INVALID_ARG, "q, k, v, o and float_ws must be 16-byte aligned");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  pkv::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.token_stride = static_cast<int64_t>(num_kv_heads) * head_dim;
  a.head_stride = head_dim;
  a.page_stride = a.token_stride * kVirtualPage;
  a.items = nullptr;
  a.implicit_nchunks = nchunks;
  a.implicit_chunk_tokens = static_cast<int32_t>(c * kVirtualPage);
  a.implicit_kv_len = kv_len;
  a.page_size = kVirtualPage;
  a.num_qo_heads = num_qo_heads;
  a.group = G;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.o = o;
  a.lse = lse;
  if (nchunks > 1) {
    a.part_o = static_cast<float*>(float_ws);
    a.part_ml = f_at(float_ws, o_bytes);
  }
  hipError_t e = pkv::launch_decode(a, dtype, pkv::kOutStorage, pkv::kContiguous,
                                    num_kv_heads * nchunks, hs);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  if (nchunks > 1) {
    pkv::MergeGroupsArgs m{};
    m.groups = nullptr;
    m.implicit_nchunks = nchunks;
    m.rows_per_tile = G;
    m.num_qo_heads = num_qo_heads;
    m.group = G;
    m.prefill = 0;
    m.part_o = a.part_o;
    m.part_ml = a.part_ml;
    m.o = o;
    m.lse = lse;
    e = pkv::launch_merge_groups(m, dtype, pkv::kOutStorage, num_kv_heads, slots, hs);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  }
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free single decode: the split partial states live in a fixed
// device array of this library instead of a caller workspace. In host code
// `scratch` names a host-side stand-in, not device memory: its device address
// is taken once per device (hipGetSymbolAddress, that device current) and only
// that address is passed to kernels. Every call on a device shares the array;
// nothing in it needs to start at zero (each chunk writes its whole partial
// state before the merge launch reads it), and calls that overlap on one
// device race.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kScratchBytes = int64_t{32} << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device.
pkv_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PKV_ERR_UNSUPPORTED, "device index above the library's limit of 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_single_decode_noalloc(const void* q, const void* k, const void* v, int32_t kv_len,
                                     int32_t num_qo_heads, int32_t num_kv_heads,
                                     int32_t head_dim, pkv_dtype dtype, float sm_scale,
                                     const pkv_sched* sched, void* o, float* lse, void* stream) {
  void* ws = nullptr;
  pkv_status st = scratch_of_current_device(&ws);
  if (st) return st;
  int64_t need = 0;
  st = pkv_single_decode(q, k, v, kv_len, num_qo_heads, num_kv_heads, head_dim, dtype, sm_scale,
                         sched, ws, static_cast<size_t>(kScratchBytes), &need, o, lse, stream);
  if (st == PKV_ERR_WORKSPACE_TOO_SMALL)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL,
                "the partial states need " + std::to_string(need) +
                    " B; the fixed scratch holds " + std::to_string(kScratchBytes) +
                    " B (fewer chunks: a sched with a larger min_chunk_tokens or fewer slots)");
  return st;
}

static pkv_status check_merge_args(int32_t n, int32_t num_heads, int32_t head_dim,
                                   pkv_dtype v_dtype) {
  if (n < 0 || num_heads <= 0 || head_dim <= 0)
    return fail(PKV_ERR_INVALID_ARG, "n must be >= 0, num_heads and head_dim positive");
  if (v_dtype != PKV_F16 && v_dtype != PKV_BF16 && v_dtype != PKV_F32)
    return fail(PKV_ERR_INVALID_ARG, "v_dtype must be PKV_F16, PKV_BF16 or PKV_F32");
  return PKV_OK;
}

pkv_status pkv_merge_state(const void* va, const float* sa, const void* vb, const float* sb,
                           void* vo, float* so, int32_t n, int32_t num_heads, int32_t head_dim,
                           pkv_dtype v_dtype, void* stream) {
  pkv_status st;
  if ((st = check_merge_args(n, num_heads, head_dim, v_dtype))) return st;
  if (n > 0 && (!va || !sa || !vb || !sb || !vo))
    return fail(PKV_ERR_INVALID_ARG, "va, sa, vb, sb and vo must be non-NULL");
  hipError_t e = pkv::launch_merge2(va, sa, vb, sb, vo, so, static_cast<int64_t>(n) * num_heads,
                                    head_dim, v_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return ok();
}

pkv_status pkv_merge_state_in_place(void* v, float* s, const void* v_other, const float* s_other,
                                    int32_t n, int32_t num_heads, int32_t head_dim,
                                    pkv_dtype v_dtype, void* stream) {
  pkv_status st;
  if ((st = check_merge_args(n, num_heads, head_dim, v_dtype))) return st;
  if (n > 0 && (!v || !s || !v_other || !s_other))
    return fail(PKV_ERR_INVALID_ARG, "v, s, v_other and s_other must be non-NULL");
  hipError_t e = pkv::launch_merge2(v, s, v_other, s_other, v, s,
                                    static_cast<int64_t>(n) * num_heads, head_dim, v_dtype,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return ok();
}

pkv_status pkv_merge_states(const void* v, const float* s, int32_t n, int32_t num_states,
                            int32_t num_heads, int32_t head_dim, pkv_dtype v_dtype, void* vo,
                            float* so, void* stream) {
  pkv_status st;
  if ((st = check_merge_args(n, num_heads, head_dim, v_dtype))) return st;
  if (num_states < 0) return fail(PKV_ERR_INVALID_ARG, "num_states must be >= 0");
  if (n > 0 && (!vo || (num_states > 0 && (!v || !s))))
    return fail(PKV_ERR_INVALID_ARG, "v, s and vo must be non-NULL");
  hipError_t e = pkv::launch_merge_n(v, s, n, num_states, num_heads, head_dim, v_dtype, vo, so,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return ok();
}

pkv_status pkv_cascade_plan(int32_t prefix_num_pages, int32_t prefix_last_page_len,
                            const int32_t* suffix_indptr_h, const int32_t* suffix_last_page_len_h,
                            int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t page_size, pkv_dtype dtype,
                            const pkv_sched* sched, void* int_ws, size_t int_ws_bytes,
                            void* float_ws, size_t float_ws_bytes, void* host_ws,
                            size_t host_ws_bytes, void* stream, pkv_plan_info* out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  pkv_status st;
  if ((st = check_heads(num_qo_heads, num_kv_heads))) return st;
  if ((st = check_head_dim_dtype(head_dim, dtype))) return st;
  const int32_t G = num_qo_heads / num_kv_heads;
  if (G > kMaxDecodeGroup)
    return fail(PKV_ERR_UNSUPPORTED, "cascade decode supports num_qo_heads / num_kv_heads <= 16");
  if (prefix_num_pages < 0) return fail(PKV_ERR_INVALID_ARG, "prefix_num_pages must be >= 0");
  // Level 0: one "request" whose query tokens are the batch's decode tokens.
  const int32_t pre_indptr[2] = {0, prefix_num_pages};
  const int32_t pre_lpl[1] = {prefix_last_page_len};
  std::vector<int64_t> pre_len, suf_len;
  if ((st = check_page_table(pre_indptr, pre_lpl, 1, page_size, &pre_len))) return st;
  if ((st = check_page_table(suffix_indptr_h, suffix_last_page_len_h, batch, page_size, &suf_len)))
    return st;
  pkv_sched s0, s1;
  if ((st = resolve_sched(sched, PKV_KIND_PREFILL, &s0))) return st;
  if ((st = resolve_sched(sched, PKV_KIND_DECODE, &s1))) return st;
  // Default level 0: one item per CU. Its items all run in one round whatever
  // their number, so half as many prefix chunks as the prefill default halve
  // the states it writes and the merge reads.
  if (sched == nullptr) s0.wg_per_cu = 1;
  std::vector<int64_t> pre_qo(1, batch), suf_qo(batch, 1);
  pkv::HostPlan hp0, hp1;
  std::string err;
  if (!pkv::build_plan(all_groups(make_input(pre_qo, pre_len, page_size, num_kv_heads, G,
                                             kRowsPerPrefillTile, false, s0)),
                       &hp0, &err) ||
      !pkv::build_plan(all_groups(make_input(suf_qo, suf_len, page_size, num_kv_heads, G, G,
                                             false, s1)),
                       &hp1, &err))
    return fail(PKV_ERR_INVALID_ARG, err);
  // Level 0 is one request, unmasked: every (tile, g) group has the same
  // chunks, and group (tile, g) owns slots (tile * Hkv + g) * n0 ... Suffix
  // group (b, g) merges the prefix states of its G rows: packed rows b*G ..
  // b*G + G - 1 of KV head g at level 0 (the query token of request b is
  // level-0 query token b).
  const int32_t n0 = hp0.groups.empty() ? 0 : hp0.groups[0].num_chunks;
  for (pkv::MergeGroup& mg : hp1.groups) {
    const int64_t packed = static_cast<int64_t>(mg.b) * G;
    const int64_t tile = packed / kRowsPerPrefillTile;
    mg.base_slot_begin = static_cast<int32_t>((tile * num_kv_heads + mg.g) * n0);
    mg.base_num_chunks = n0;
    mg.base_row = static_cast<int32_t>(packed % kRowsPerPrefillTile);
  }
  fill_header(out, PKV_KIND_CASCADE, dtype, batch, num_qo_heads, num_kv_heads, head_dim,
              page_size, batch, s1);
  Layout lay;
  // int ws: [level-0 qo_indptr (2), level-0 kv_indptr (2)] then both parts' tables
  lay.int_bytes = kAlign;
  place_part(hp0, 1, kRowsPerPrefillTile, 0, &lay, &out->part[0]);
  place_part(hp1, batch, G, 0, &lay, &out->part[1]);
  char* h = nullptr;
  if ((st = claim_staging(host_ws, host_ws_bytes, lay.int_bytes, &h))) return st;
  if (h != nullptr) {
    const int32_t hdr[4] = {0, batch, 0, prefix_num_pages};
    std::memcpy(h, hdr, sizeof(hdr));
    write_part(hp0, pre_len, out->part[0], h);
    write_part(hp1, suf_len, out->part[1], h);
  }
  if ((st = commit_plan(lay, int_ws, int_ws_bytes, float_ws, float_ws_bytes, host_ws,
                        host_ws_bytes, static_cast<hipStream_t>(stream), out)))
    return st;
  return ok();
}

pkv_status pkv_cascade_run(const pkv_plan_info* plan, const void* q, const pkv_paged_kv* kv,
                           const int32_t* prefix_indices_d, const int32_t* suffix_indptr_d,
                           const int32_t* suffix_indices_d, float sm_scale, void* o, float* lse,
                           void* stream) {
  pkv_status st;
  if ((st = check_scale(sm_scale))) return st;
  if ((st = check_plan(plan, PKV_KIND_CASCADE))) return st;
  if ((st = check_kv(kv, plan))) return st;
  if (plan->batch == 0) return ok();
  if (q == nullptr || o == nullptr || suffix_indptr_d == nullptr || suffix_indices_d == nullptr ||
      (plan->part[0].num_items > 0 && prefix_indices_d == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "q, o, prefix / suffix tables must be non-NULL");
  if (!aligned16(q) || !aligned16(o)) return fail(PKV_ERR_INVALID_ARG, "q / o must be 16-byte aligned");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int32_t* hdr = i_at(plan->int_ws, 0);
  // Level 0: the prefix's chunk states of every (request, head) row, the
  // prefix read once; every item writes a partial state.
  if ((st = run_prefill_part(plan, plan->part[0], q, kv, hdr, hdr + 2, prefix_indices_d, sm_scale,
                             nullptr, nullptr, plan->num_qo_heads, pkv::kOutStorage, hs, {},
                             kNoVariant, /*merge=*/false)))
    return st;
  // Level 1: the suffix chunks per request (batch decode, every group a merge
  // group), then one merge of each group's prefix states and suffix chunks.
  const pkv_plan_part& p0 = plan->part[0];
  const int32_t n0 = p0.num_groups > 0 ? p0.num_slots / p0.num_groups : 0;
  BaseStates base;
  base.o = f_at(plan->float_ws, p0.part_o_off);
  base.ml = f_at(plan->float_ws, p0.part_ml_off);
  base.rows = p0.rows_per_tile;
  base.tile_slots = plan->num_kv_heads * n0;
  base.states_per_group = n0;
  if ((st = run_decode_part(plan, plan->part[1], q, kv, suffix_indptr_d, suffix_indices_d,
                            sm_scale, o, lse, pkv::kOutStorage, hs, {}, kNoVariant, base)))
    return st;
  return ok();
}

pkv_status pkv_pod_plan(const int32_t* qo_indptr_h, const int32_t* kv_indptr_p_h,
                        const int32_t* last_page_len_p_h, int32_t batch_p, int32_t causal,
                        const int32_t* kv_indptr_d_h, const int32_t* last_page_len_d_h,
                        int32_t batch_d, int32_t num_qo_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t page_size, pkv_dtype dtype,
                        const pkv_sched* sched, void* int_ws, size_t int_ws_bytes,
                        void* float_ws, size_t float_ws_bytes, void* host_ws,
                        size_t host_ws_bytes, void* stream, pkv_plan_info* out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  pkv_status st;
  if ((st = check_heads(num_qo_heads, num_kv_heads))) return st;
  if ((st = check_head_dim_dtype(head_dim, dtype))) return st;
  if (causal != 0 && causal != 1) return fail(PKV_ERR_INVALID_ARG, "causal must be 0 or 1");
  const int32_t G = num_qo_heads / num_kv_heads;
  if (G > kMaxDecodeGroup)
    return fail(PKV_ERR_UNSUPPORTED, "the mixed launch supports num_qo_heads / num_kv_heads <= 16");
  std::vector<int64_t> kv_p, qo_p, kv_d;
  if ((st = check_page_table(kv_indptr_p_h, last_page_len_p_h, batch_p, page_size, &kv_p)))
    return st;
  if ((st = check_qo_indptr(qo_indptr_h, batch_p, &qo_p))) return st;
  if ((st = check_page_table(kv_indptr_d_h, last_page_len_d_h, batch_d, page_size, &kv_d)))
    return st;
  int64_t total_qo = 0;
  for (int64_t qn : qo_p) total_qo += qn;
  if (total_qo * num_qo_heads > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "total query rows overflow int32");
  pkv_sched sp, sd;
  if ((st = resolve_sched(sched, PKV_KIND_PREFILL, &sp))) return st;
  if ((st = resolve_sched(sched, PKV_KIND_DECODE, &sd))) return st;
  std::vector<int64_t> qo_d(batch_d, 1);
  pkv::HostPlan hp, hd;
  std::string err;
  if (!pkv::build_plan(make_input(qo_p, kv_p, page_size, num_kv_heads, G, kRowsPerPodPrefillTile,
                                  causal != 0, sp),
                       &hp, &err) ||
      !pkv::build_plan(make_input(qo_d, kv_d, page_size, num_kv_heads, G, G, false, sd), &hd,
                       &err))
    return fail(PKV_ERR_INVALID_ARG, err);
  const std::vector<int32_t> order = pkv::interleave_items(hp.items, hd.items);
  fill_header(out, PKV_KIND_POD, dtype, batch_p, num_qo_heads, num_kv_heads, head_dim, page_size,
              static_cast<int32_t>(total_qo), sp);
  out->batch2 = batch_d;
  out->num_blocks = static_cast<int32_t>(order.size());
  Layout lay;
  place_part(hp, batch_p, kRowsPerPodPrefillTile, causal, &lay, &out->part[0]);
  place_part(hd, batch_d, G, 0, &lay, &out->part[1]);
  out->order_off = lay.int_bytes;
  lay.int_bytes = align_up(lay.int_bytes + static_cast<int64_t>(order.size()) * 4);
  char* h = nullptr;
  if ((st = claim_staging(host_ws, host_ws_bytes, lay.int_bytes, &h))) return st;
  if (h != nullptr) {
    write_part(hp, kv_p, out->part[0], h);
    write_part(hd, kv_d, out->part[1], h);
    if (!order.empty()) std::memcpy(h + out->order_off, order.data(), order.size() * 4);
  }
  if ((st = commit_plan(lay, int_ws, int_ws_bytes, float_ws, float_ws_bytes, host_ws,
                        host_ws_bytes, static_cast<hipStream_t>(stream), out)))
    return st;
  return ok();
}

pkv_status pkv_pod_run(const pkv_plan_info* plan, const pkv_paged_kv* kv, const void* q_p,
                       const int32_t* qo_indptr_d, const int32_t* kv_indptr_p_d,
                       const int32_t* kv_indices_p_d, void* o_p, float* lse_p, const void* q_d,
                       const int32_t* kv_indptr_d_d, const int32_t* kv_indices_d_d, void* o_d,
                       float* lse_d, float sm_scale, void* stream) {
  return pkv_pod_run_timed(plan, kv, q_p, qo_indptr_d, kv_indptr_p_d, kv_indices_p_d, o_p, lse_p,
                           q_d, kv_indptr_d_d, kv_indices_d_d, o_d, lse_d, sm_scale, stream,
                           nullptr, nullptr);
}

pkv_status pkv_pod_run_timed(const pkv_plan_info* plan, const pkv_paged_kv* kv, const void* q_p,
                             const int32_t* qo_indptr_d, const int32_t* kv_indptr_p_d,
                             const int32_t* kv_indices_p_d, void* o_p, float* lse_p,
                             const void* q_d, const int32_t* kv_indptr_d_d,
                             const int32_t* kv_indices_d_d, void* o_d, float* lse_d,
                             float sm_scale, void* stream, void* attention_start,
                             void* attention_done) {
  pkv_status st;
  if ((st = check_scale(sm_scale))) return st;
  if ((st = check_plan(plan, PKV_KIND_POD))) return st;
  if ((st = check_kv(kv, plan))) return st;
  if (plan->total_qo > 0 && (q_p == nullptr || o_p == nullptr || qo_indptr_d == nullptr ||
                             kv_indptr_p_d == nullptr || kv_indices_p_d == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "q_p, o_p, qo_indptr, kv_indptr_p or kv_indices_p is NULL");
  if (plan->batch2 > 0 && (q_d == nullptr || o_d == nullptr || kv_indptr_d_d == nullptr ||
                           kv_indices_d_d == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "q_d, o_d, kv_indptr_d or kv_indices_d is NULL");
  if (!aligned16(q_p) || !aligned16(o_p) || !aligned16(q_d) || !aligned16(o_d))
    return fail(PKV_ERR_INVALID_ARG, "q / o must be 16-byte aligned");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  pkv::PodArgs a{};
  a.p = prefill_args(plan, plan->part[0], q_p, kv, qo_indptr_d, kv_indptr_p_d, kv_indices_p_d,
                     sm_scale, o_p, lse_p, plan->num_qo_heads, kNoVariant);
  a.d = decode_args(plan, plan->part[1], q_d, kv, kv_indptr_d_d, kv_indices_d_d, sm_scale, o_d,
                    lse_d, kNoVariant);
  a.order = i_at(plan->int_ws, plan->order_off);
  const hipError_t e = pkv::launch_pod(a, plan->dtype, page_mode(plan->page_size), plan->num_blocks,
                                       s, launch_events(attention_start, attention_done));
  if (e != hipSuccess) return hip_fail(e, "mixed prefill + decode kernel launch");
  if ((st = merge_part(plan->part[0], true, qo_indptr_d, plan->num_qo_heads, a.p.group,
                       plan->int_ws, plan->float_ws, o_p, lse_p, nullptr, plan->dtype,
                       pkv::kOutStorage, s)))
    return st;
  if ((st = merge_part(plan->part[1], false, nullptr, plan->num_qo_heads, a.d.group, plan->int_ws,
                       plan->float_ws, o_d, lse_d, nullptr, plan->dtype, pkv::kOutStorage, s)))
    return st;
  return ok();
}

pkv_status pkv_block_sparse_plan(const int32_t* bsr_indptr_h, const int32_t* bsr_indices_h,
                                 int32_t num_block_rows, int32_t num_qo_tokens,
                                 int32_t num_kv_tokens, int32_t row_block, int32_t col_block,
                                 int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                 pkv_dtype dtype, const pkv_sched* sched, void* int_ws,
                                 size_t int_ws_bytes, void* float_ws, size_t float_ws_bytes,
                                 void* host_ws, size_t host_ws_bytes, void* stream,
                                 pkv_plan_info* out) {
  if (out == nullptr) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  pkv_status st;
  if ((st = check_heads(num_qo_heads, num_kv_heads))) return st;
  if ((st = check_head_dim_dtype(head_dim, dtype))) return st;
  const int32_t G = num_qo_heads / num_kv_heads;
  if (G > kRowsPerPrefillTile)
    return fail(PKV_ERR_UNSUPPORTED, "block-sparse supports num_qo_heads / num_kv_heads <= 128");
  if (row_block <= 0 || col_block <= 0)
    return fail(PKV_ERR_INVALID_ARG, "row_block and col_block must be positive");
  if (num_qo_tokens < 0 || num_kv_tokens < 0)
    return fail(PKV_ERR_INVALID_ARG, "token counts must be >= 0");
  if (static_cast<int64_t>(num_qo_tokens) * num_qo_heads > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "query rows overflow int32");
  const int64_t want_rows = (static_cast<int64_t>(num_qo_tokens) + row_block - 1) / row_block;
  if (num_block_rows != want_rows)
    return fail(PKV_ERR_INVALID_ARG, "num_block_rows must be ceil(num_qo_tokens / row_block)");
  if (bsr_indptr_h == nullptr || bsr_indptr_h[0] != 0)
    return fail(PKV_ERR_INVALID_ARG, "bsr_indptr_h must be non-NULL with bsr_indptr_h[0] = 0");
  const int64_t num_col_blocks = (static_cast<int64_t>(num_kv_tokens) + col_block - 1) / col_block;
  if (num_col_blocks * col_block * static_cast<int64_t>(num_kv_heads) * head_dim >
      (int64_t{1} << 40))
    return fail(PKV_ERR_INVALID_ARG, "keys too large");
  if (static_cast<int64_t>(col_block) * num_kv_heads * head_dim >= (int64_t{1} << 30))
    return fail(PKV_ERR_INVALID_ARG, "col_block * num_kv_heads * head_dim must be below 2^30");
  std::vector<int64_t> qo_lens(num_block_rows), kv_lens(num_block_rows);
  const int64_t last_block_len = num_kv_tokens - (num_col_blocks - 1) * col_block;
  for (int32_t i = 0; i < num_block_rows; ++i) {
    const int32_t b0 = bsr_indptr_h[i], b1 = bsr_indptr_h[i + 1];
    if (b1 < b0) return fail(PKV_ERR_INVALID_ARG, "bsr_indptr is not monotone at " + std::to_string(i));
    if (b1 > b0 && bsr_indices_h == nullptr)
      return fail(PKV_ERR_INVALID_ARG, "bsr_indices_h is NULL");
    int64_t len = 0;
    for (int32_t e = b0; e < b1; ++e) {
      const int32_t j = bsr_indices_h[e];
      if (j < 0 || j >= num_col_blocks || (e > b0 && j <= bsr_indices_h[e - 1]))
        return fail(PKV_ERR_INVALID_ARG, "bsr_indices of block row " + std::to_string(i) +
                                             " must ascend within [0, ceil(num_kv_tokens / C))");
      len += (j == num_col_blocks - 1) ? last_block_len : col_block;
    }
    qo_lens[i] = std::min<int64_t>(row_block, num_qo_tokens - static_cast<int64_t>(i) * row_block);
    kv_lens[i] = len;
  }
  pkv_sched s;
  if ((st = resolve_sched(sched, PKV_KIND_PREFILL, &s))) return st;
  pkv::HostPlan hp;
  std::string err;
  if (!pkv::build_plan(make_input(qo_lens, kv_lens, col_block, num_kv_heads, G,
                                  kRowsPerPrefillTile, false, s),
                       &hp, &err))
    return fail(PKV_ERR_INVALID_ARG, err);
  fill_header(out, PKV_KIND_BLOCK_SPARSE, dtype, num_block_rows, num_qo_heads, num_kv_heads,
              head_dim, col_block, num_qo_tokens, s);
  Layout lay;
  // int ws: the query-block offsets [num_block_rows + 1], then the part's tables
  lay.int_bytes = align_up((static_cast<int64_t>(num_block_rows) + 1) * 4);
  place_part(hp, num_block_rows, kRowsPerPrefillTile, 0, &lay, &out->part[0]);
  char* h = nullptr;
  if ((st = claim_staging(host_ws, host_ws_bytes, lay.int_bytes, &h))) return st;
  if (h != nullptr) {
    int32_t* qo = reinterpret_cast<int32_t*>(h);
    for (int32_t i = 0; i <= num_block_rows; ++i)
      qo[i] = static_cast<int32_t>(std::min<int64_t>(static_cast<int64_t>(i) * row_block,
                                                     num_qo_tokens));
    write_part(hp, kv_lens, out->part[0], h);
  }
  if ((st = commit_plan(lay, int_ws, int_ws_bytes, float_ws, float_ws_bytes, host_ws,
                        host_ws_bytes, static_cast<hipStream_t>(stream), out)))
    return st;
  return ok();
}

pkv_status pkv_block_sparse_run(const pkv_plan_info* plan, const void* q, const void* k,
                                const void* v, const int32_t* bsr_indptr_d,
                                const int32_t* bsr_indices_d, float sm_scale, void* o, float* lse,
                                void* stream) {
  pkv_status st;
  if ((st = check_scale(sm_scale))) return st;
  if ((st = check_plan(plan, PKV_KIND_BLOCK_SPARSE))) return st;
  if (plan->total_qo == 0) return ok();
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || bsr_indptr_d == nullptr ||
      bsr_indices_d == nullptr)
    return fail(PKV_ERR_INVALID_ARG, "q, k, v, o and the BSR arrays must be non-NULL");
  if (!aligned16(q) || !aligned16(o) || !aligned16(k) || !aligned16(v))
    return fail(PKV_ERR_INVALID_ARG, "q / k / v / o must be 16-byte aligned");
  // The dense keys viewed as pages of col_block tokens: page j = key block j.
  pkv_paged_kv kv{};
  kv.k = k;
  kv.v = v;
  kv.token_stride = static_cast<int64_t>(plan->num_kv_heads) * plan->head_dim;
  kv.head_stride = plan->head_dim;
  kv.page_stride = kv.token_stride * plan->page_size;
  kv.page_size = plan->page_size;
  kv.num_kv_heads = plan->num_kv_heads;
  kv.head_dim = plan->head_dim;
  kv.dtype = plan->dtype;
  if ((st = run_prefill_part(plan, plan->part[0], q, &kv, i_at(plan->int_ws, 0), bsr_indptr_d,
                             bsr_indices_d, sm_scale, o, lse, plan->num_qo_heads,
                             pkv::kOutStorage, static_cast<hipStream_t>(stream))))
    return st;
  return ok();
}

pkv_status pkv_append_paged_kv(const void* append_k, const void* append_v, int32_t nnz,
                               const int32_t* batch_indices_d, const int32_t* positions_d,
                               void* k_cache, void* v_cache, const pkv_paged_kv* layout,
                               const int32_t* kv_indptr_d, const int32_t* kv_indices_d,
                               const int32_t* last_page_len_d, int32_t batch, void* stream) {
  if (layout == nullptr) return fail(PKV_ERR_INVALID_ARG, "layout is NULL");
  if (nnz < 0 || batch < 0) return fail(PKV_ERR_INVALID_ARG, "nnz and batch must be >= 0");
  if (layout->page_size <= 0) return fail(PKV_ERR_INVALID_ARG, "page_size must be positive");
  if (layout->num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be positive");
  pkv_status st;
  if ((st = check_head_dim_dtype(layout->head_dim, layout->dtype))) return st;
  if (layout->num_kv_heads > 32)
    return fail(PKV_ERR_UNSUPPORTED, "append supports num_kv_heads <= 32");
  if (layout->page_stride % 8 || layout->token_stride % 8 || layout->head_stride % 8 ||
      layout->page_stride < 0 || layout->token_stride < 0 || layout->head_stride < 0 ||
      layout->page_stride >= (int64_t{1} << 30) || layout->token_stride > (INT32_MAX / 32))
    return fail(PKV_ERR_INVALID_ARG,
                "KV strides must be non-negative multiples of 8 elements (page_stride < 2^30, "
                "token_stride < 2^26)");
  if (nnz == 0) return ok();
  if (!append_k || !append_v || !batch_indices_d || !positions_d || !k_cache || !v_cache ||
      (batch > 0 && (!kv_indptr_d || !kv_indices_d || !last_page_len_d)))
    return fail(PKV_ERR_INVALID_ARG, "append / cache / page-table pointers must be non-NULL");
  if (!aligned16(append_k) || !aligned16(append_v) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_ERR_INVALID_ARG, "append_k / append_v / k_cache / v_cache must be 16-byte aligned");
  if (batch == 0) return ok();   // no request: every row is skipped
  pkv::AppendArgs a{};
  a.append_k = append_k;
  a.append_v = append_v;
  a.append_stride = static_cast<int64_t>(layout->num_kv_heads) * layout->head_dim;
  a.batch_indices = batch_indices_d;
  a.positions = positions_d;
  a.k = k_cache;
  a.v = v_cache;
  a.page_stride = layout->page_stride;
  a.token_stride = layout->token_stride;
  a.head_stride = layout->head_stride;
  a.kv_indptr = kv_indptr_d;
  a.kv_indices = kv_indices_d;
  a.last_page_len = last_page_len_d;
  a.batch = batch;
  a.page_size = layout->page_size;
  a.num_kv_heads = layout->num_kv_heads;
  a.nnz = nnz;
  hipError_t e = pkv::launch_append(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append kernel launch");
  return ok();
}

pkv_status pkv_append_positions(const int32_t* append_indptr_h, const int32_t* kv_indptr_h,
                                const int32_t* last_page_len_h, int32_t batch, int32_t page_size,
                                int32_t* batch_indices_h, int32_t* positions_h) {
  std::vector<int64_t> kv_lens;
  pkv_status st;
  if ((st = check_page_table(kv_indptr_h, last_page_len_h, batch, page_size, &kv_lens))) return st;
  if (append_indptr_h == nullptr) return fail(PKV_ERR_INVALID_ARG, "append_indptr_h is NULL");
  if (append_indptr_h[0] != 0) return fail(PKV_ERR_INVALID_ARG, "append_indptr_h[0] must be 0");
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = static_cast<int64_t>(append_indptr_h[b + 1]) - append_indptr_h[b];
    if (n < 0)
      return fail(PKV_ERR_INVALID_ARG, "append_indptr_h is not monotone at " + std::to_string(b));
    if (n > kv_lens[b])
      return fail(PKV_ERR_INVALID_ARG, "request " + std::to_string(b) +
                                           " appends more tokens than its KV length");
  }
  if (append_indptr_h[batch] > 0 && (batch_indices_h == nullptr || positions_h == nullptr))
    return fail(PKV_ERR_INVALID_ARG, "batch_indices_h / positions_h are NULL");
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t first = append_indptr_h[b];
    const int32_t count = append_indptr_h[b + 1] - first;
    const int64_t start = kv_lens[b] - count;
    for (int32_t i = 0; i < count; ++i) {
      batch_indices_h[first + i] = b;
      positions_h[first + i] = static_cast<int32_t>(start + i);
    }
  }
  return ok();
}

}  // extern "C"
