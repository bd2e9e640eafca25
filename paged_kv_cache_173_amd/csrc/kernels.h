// Kernel argument blocks and host-side launchers (implemented in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {

constexpr int32_t kHeadDimSupported = 128;

// How a kernel finds the address of logical token t of a request.
enum PageMode : int32_t {
  kContiguous = 0,    // no page table: token t at t * token_stride
  kPagedUniform = 1,  // page_size % 16 == 0: a 16-token block never straddles a page
  kPagedGeneric = 2,  // any page_size: one page-table lookup per lane and token
};

enum OutKind : int32_t { kOutStorage = 0, kOutF32 = 1 };

// Attention variants shared by the decode and prefill kernels (all off:
// window_left < 0, cap_out = 0, sinks = NULL; the launchers then pick the
// plain kernels).
//   * Sliding window: a row at position p sees keys t >= p - window_left.
//   * Logit soft cap c: the raw score s = q.k becomes
//     cap_out * tanh(s * sm_scale / c) with cap_out = c / sm_scale, so that
//     sm_scale times it is c * tanh(sm_scale * s / c); the kernels form
//     tanh(y) = 1 - 2 / (exp2(2 y log2 e) + 1) with cap_in = 2 log2(e) sm_scale / c.
//   * Sinks: sinks[h] (natural log) joins the softmax of every row of query
//     head h as a key with a zero value, once, where the final row is written.
struct VariantArgs {
  int32_t window_left = -1;
  float cap_in = 0.f;
  float cap_out = 0.f;
  const float* sinks = nullptr;   // device [num_qo_heads] or NULL
};

inline bool variant_on(const VariantArgs& v) {
  return v.window_left >= 0 || v.cap_out > 0.f || v.sinks != nullptr;
}

// A split-KV partial state, as the kernels write it: for each row, O (fp32
// [128], already divided by l) and the pair (m, l) in the log2 domain: m a
// reference exponent (the row's running maximum of sm_scale * log2(e) * q.k),
// l = sum over the chunk's keys of 2^(x_t - m). The row's natural-log LSE is
// (m + log2 l) * ln 2; keeping m and l apart instead lets a merge weight the
// chunk by l * 2^(m - M) with m - M exact, so states stay exact to fp32
// rounding even when every logit is ~1e5 in magnitude. An empty chunk is
// (O = 0, m = -inf, l = 0).
//
// Merge group record (int32[8]) of a plan part: {b, tile, g, slot_begin,
// num_chunks, base_slot_begin, base_num_chunks, base_row}: the group's chunks
// are slots slot_begin .. slot_begin + num_chunks - 1 of the part; a cascade's
// suffix group also merges base_num_chunks states of the prefix part
// (slots base_slot_begin.., rows base_row.. of each), before its own chunks. Its
// rows may run past the prefix tile's last row; row base_row + r >= base_rows
// is row base_row + r - base_rows of the next tile, whose slots start
// base_tile_slots later.

struct DecodeArgs {
  const void* q;            // [batch, Hq, 128] storage dtype
  const void* k;            // K page pool base
  const void* v;            // V page pool base
  int64_t page_stride, token_stride, head_stride;  // elements
  const int32_t* kv_indptr;   // device [batch+1] (paged modes)
  const int32_t* kv_indices;  // device page ids (paged modes)
  const int32_t* items;       // device [num_items][8], or NULL: implicit uniform chunks
  int32_t implicit_nchunks;   // implicit mode: chunks per KV head (single request)
  int32_t implicit_chunk_tokens;
  int32_t implicit_kv_len;
  int32_t page_size;
  int32_t num_qo_heads;
  int32_t group;              // G <= 16
  float scale_log2;           // sm_scale * log2(e)
  void* o;                    // final output rows [batch*Hq][128]
  float* lse;                 // final LSE [batch*Hq] or NULL
  float* part_o;              // partial states [slot][G][128]
  float* part_ml;             // [slot][G][2]: (m, l)
  const int32_t* kv_lens;     // device [batch] KV length per request (variants only)
  VariantArgs var;
};

struct PrefillArgs {
  const void* q;            // [total_qo, Hq, 128] storage dtype
  const void* k;
  const void* v;
  int64_t page_stride, token_stride, head_stride;  // elements
  const int32_t* qo_indptr;   // device [batch+1]
  const int32_t* kv_indptr;   // device [batch+1]
  const int32_t* kv_indices;  // device page ids
  const int32_t* items;       // device [num_items][8]
  const int32_t* kv_lens;     // device [batch] KV length per request
  int32_t page_size;
  int32_t num_qo_heads;
  int32_t group;              // G <= 128
  int32_t causal;
  int32_t rows_per_tile;      // query rows of an item (128: the plan and the kernel agree)
  float scale_log2;           // sm_scale * log2(e)
  void* o;                    // final output rows [total_qo*Hq][128]
  float* lse;                 // [total_qo*Hq] or NULL
  float* part_o;              // [slot][128 rows][128]
  float* part_ml;             // [slot][128 rows][2]: (m, l)
  VariantArgs var;
};

struct AppendArgs {
  const void* append_k;       // [nnz] rows of [Hkv, 128], 2-byte elements
  const void* append_v;
  int64_t append_stride;      // elements between consecutive appended rows
  const int32_t* batch_indices;   // device [nnz]
  const int32_t* positions;       // device [nnz]
  void* k;                    // K page pool base (written)
  void* v;                    // V page pool base (written)
  int64_t page_stride, token_stride, head_stride;  // elements
  const int32_t* kv_indptr;   // device [batch+1]
  const int32_t* kv_indices;  // device page ids
  const int32_t* last_page_len;   // device [batch]
  int32_t batch;
  int32_t page_size;
  int32_t num_kv_heads;       // <= 32
  int64_t nnz;
};

// One launch of prefill and decode items (the mixed-batch kernel): entry i of
// `order` names the item workgroup i runs (>= 0: prefill item; < 0: decode
// item -e-1). The two halves keep their own argument blocks; both read the
// same page pools.
struct PodArgs {
  PrefillArgs p;
  DecodeArgs d;
  const int32_t* order;       // device [num_prefill_items + num_decode_items]
};

struct MergeGroupsArgs {
  const int32_t* groups;      // device [num_groups][8], or NULL: implicit (single decode:
                              // group g = KV head g, chunks in slots g*n .. g*n + n - 1)
  int32_t implicit_nchunks;
  int32_t rows_per_tile;      // rows per partial slot
  int32_t num_qo_heads;
  int32_t group;              // G
  int32_t prefill;            // row mapping: 0 decode, 1 GQA-packed prefill rows
  const int32_t* qo_indptr;   // device, prefill mapping only
  const float* part_o;
  const float* part_ml;
  void* o;
  float* lse;                 // or NULL
  const float* sinks;         // device [num_qo_heads] sink logits, or NULL
  // The cascade: partial states of the prefix part (slots of base_rows rows),
  // merged before each group's own chunks (see the group record), or NULL.
  const float* base_o;
  const float* base_ml;
  int32_t base_rows;
  int32_t base_tile_slots;    // slots from a prefix tile's group to the next tile's
};

// Events a launch may carry on its own dispatch packet (hipExtLaunchKernel):
// `start` takes the kernel's begin timestamp and `stop` its end timestamp, so
// their elapsed time is the kernel's run time alone, without the queue's
// dispatch latency. Either may be null.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Workgroups of the decode / prefill kernel resident per CU (0 on error).
int32_t decode_occupancy();
int32_t prefill_occupancy();

hipError_t launch_decode(const DecodeArgs& a, int32_t storage_dtype, OutKind out,
                         PageMode mode, int32_t grid, hipStream_t stream,
                         const LaunchEvents& ev = {});

hipError_t launch_prefill(const PrefillArgs& a, int32_t storage_dtype, OutKind out,
                          PageMode mode, int32_t grid, hipStream_t stream,
                          const LaunchEvents& ev = {});

// num_chunks: the chunks of all groups together (chooses the mapping).
hipError_t launch_merge_groups(const MergeGroupsArgs& a, int32_t storage_dtype, OutKind out,
                               int32_t num_groups, int64_t num_chunks, hipStream_t stream);

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

// Mixed prefill + decode launch; outputs are in the storage dtype.
hipError_t launch_pod(const PodArgs& a, int32_t storage_dtype, PageMode mode, int32_t grid,
                      hipStream_t stream, const LaunchEvents& ev = {});

// Public merges: v dtype in {F16, BF16, F32}; rows = n * H.
hipError_t launch_merge2(const void* va, const float* sa, const void* vb, const float* sb,
                         void* vo, float* so, int64_t rows, int32_t head_dim, int32_t v_dtype,
                         hipStream_t stream);
hipError_t launch_merge_n(const void* v, const float* s, int64_t n, int32_t num_states,
                          int32_t num_heads, int32_t head_dim, int32_t v_dtype, void* vo,
                          float* so, hipStream_t stream);
// Cascade's final merge: fp32 states a and b -> storage-dtype o, float lse.
hipError_t launch_merge2_f32_to(const float* va, const float* sa, const float* vb,
                                const float* sb, void* vo, float* so, int64_t rows,
                                int32_t head_dim, int32_t out_dtype, hipStream_t stream);

}  // namespace pkv
