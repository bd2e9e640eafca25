// Attention-state merge kernels for gfx950.
//
// States of disjoint KV parts (O_k, LSE_k) combine into the state of their
// union by rescaling with the LSEs: s* = max_k LSE_k, w_k = exp(LSE_k - s*),
// O = sum w_k O_k / sum w_k, LSE = s* + ln(sum w_k); if every LSE_k is -inf
// the row saw no key and the result is (0, -inf) (FlashInfer article,
// sections "Attention states" and "Extreme-negative-logit correction"; docs
// index "flashinfer.cascade" > "Merge Attention States").
//
// Mapping: every output row gets one wave whose lanes stride over head_dim and
// read the states in ascending k (four rows per workgroup), except the rows of
// split groups of many chunks, whose chunks four waves share. The planned
// merges read the kernels' split-KV partial states, (O, m, l) in the log2
// domain (kernels.h); the public merges take natural-log LSEs.
// Every reduction runs in a fixed order, so a run is reproducible bit for bit.
// The work is a few MB at most and HBM-bound; fp32 throughout, output rounded
// once.
#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

template <class V>
__device__ __forceinline__ float load_f(const V* p) {
  return static_cast<float>(*p);
}

template <class OUT>
__device__ __forceinline__ void store_f(OUT* p, float x) {
  *p = static_cast<OUT>(x);
}

// Merge of the chunks of one planned split group: blockIdx.x = group. Chunk k
// of row r is the partial state (O_k, m_k, l_k) in slot sb + k (log2 domain,
// see kernels.h): w_k = l_k 2^(m_k - M), M = max_k m_k. A cascade's suffix
// group merges the prefix states of its rows first (states k < bn), then its
// own chunks: the level-0 pass leaves one state per prefix chunk, so no
// separate merge of the prefix runs.
// With WPR = 1 wave per row, wave w of blockIdx.y takes row 4 * blockIdx.y + w
// and adds up the chunks' outputs in ascending chunk order; with WPR = 4
// (groups of many chunks), the four waves of blockIdx.y take row blockIdx.y
// and split its chunks (k = w, w+4, ...), and their four partial sums add up
// in LDS in a fixed order. Every wave reads the row's (m_k, l_k) with its 64
// lanes in parallel (max and sum); lane l owns output columns 2l and 2l+1. The
// output loads go out in batches of kBatch chunks, the first batch before the
// reductions (which do not need it), so a wave's first kBatch chunks cost
// about one memory round trip. Every reduction runs in a fixed order, so every
// run gives the same bits.
template <class OUT, int WPR>
__global__ __launch_bounds__(256) void merge_groups_kernel(const MergeGroupsArgs a) {
  constexpr int D = kHeadDim;
  constexpr int kBatch = 8;
  __shared__ float s_red[WPR == 4 ? 4 : 1][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int b = 0, tile = 0, g, sb, n, bsb = 0, bn = 0, brow = 0;
  if (a.groups != nullptr) {
    const int32_t* gr = a.groups + 8 * blockIdx.x;
    b = gr[0];
    tile = gr[1];
    g = gr[2];
    sb = gr[3];
    n = gr[4];
    bsb = gr[5];
    bn = gr[6];
    brow = gr[7];
  } else {
    g = blockIdx.x;
    n = a.implicit_nchunks;
    sb = g * n;
  }
  const int R = a.rows_per_tile;
  const int r = WPR == 4 ? static_cast<int>(blockIdx.y) : 4 * static_cast<int>(blockIdx.y) + wave;
  if (r >= R) return;       // WPR = 1: uniform across the wave; WPR = 4: never taken
  RowMap map{a.num_qo_heads, a.group, a.prefill != 0};
  const int64_t orow = map.out_row(a.qo_indptr, b, tile, g, r, R);
  if (orow < 0) return;     // uniform across the wave (WPR = 4: the workgroup)
  // State k of the row: k < bn the prefix state k (cascade; a prefix row past
  // its tile's last row lives in the next tile's slots), then chunk k - bn.
  const int nk = bn + n;
  auto state_row = [&](int k) -> int64_t {
    if (k >= bn) return (static_cast<int64_t>(sb) + k - bn) * R + r;
    const int br = brow + r;
    const int64_t s0 = static_cast<int64_t>(bsb) + k;
    return br < a.base_rows ? s0 * a.base_rows + br
                            : (s0 + a.base_tile_slots) * a.base_rows + br - a.base_rows;
  };
  auto ml_at = [&](int k) -> float2 {
    return *reinterpret_cast<const float2*>((k < bn ? a.base_ml : a.part_ml) + 2 * state_row(k));
  };
  auto o_at = [&](int k) -> float2 {
    return *reinterpret_cast<const float2*>((k < bn ? a.base_o : a.part_o) + state_row(k) * D +
                                            2 * lane);
  };
  // This wave's states: k = k_first, k_first + k_step, ...
  const int k_first = WPR == 4 ? wave : 0;
  constexpr int k_step = WPR == 4 ? 4 : 1;

  float2 v[kBatch], mk[kBatch];
  auto load_batch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int k = k0 + k_step * i;
      if (k < nk) {
        mk[i] = ml_at(k);
        v[i] = o_at(k);
      }
    }
  };
  load_batch(k_first);

  // Lane l holds (m, l) of state l (the first 64 states) for both reductions.
  const float2 ml0 = lane < nk ? ml_at(lane) : make_float2(neg_inf(), 0.f);
  float M = ml0.x;
  for (int k = lane + 64; k < nk; k += 64) M = fmaxf(M, ml_at(k).x);
  M = wave_reduce_max(M);
  // An attention sink of the row's head is one more state (0, sink): it
  // enters the maximum and the sum, and adds nothing to the output.
  const float sink = a.sinks != nullptr ? a.sinks[orow % a.num_qo_heads] * kLog2e : neg_inf();
  M = fmaxf(M, sink);
  const float Mu = (M == neg_inf()) ? 0.f : M;
  float L = lane < nk ? ml0.y * fast_exp2(ml0.x - Mu) : 0.f;
  for (int k = lane + 64; k < nk; k += 64) {
    const float2 ml = ml_at(k);
    L += ml.y * fast_exp2(ml.x - Mu);
  }
  L = wave_reduce_sum(L) + fast_exp2(sink - Mu);

  float o0 = 0.f, o1 = 0.f;
  for (int k0 = k_first; k0 < nk; k0 += k_step * kBatch) {
    if (k0 != k_first) load_batch(k0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (k0 + k_step * i < nk) {
        const float w = mk[i].y * fast_exp2(mk[i].x - Mu);
        o0 += w * v[i].x;
        o1 += w * v[i].y;
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const float lse = L > 0.f ? (M + fast_log2(L)) * kLn2 : neg_inf();
  if constexpr (WPR == 4) {
    s_red[wave][2 * lane] = o0;
    s_red[wave][2 * lane + 1] = o1;
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < D) {
      const float sum = ((s_red[0][tid] + s_red[1][tid]) + s_red[2][tid]) + s_red[3][tid];
      store_f(static_cast<OUT*>(a.o) + orow * D + tid, sum * inv);
    }
    if (tid == 0 && a.lse != nullptr) a.lse[orow] = lse;
  } else {
    OUT* out = static_cast<OUT*>(a.o) + orow * D + 2 * lane;
    store_f(out, o0 * inv);
    store_f(out + 1, o1 * inv);
    if (lane == 0 && a.lse != nullptr) a.lse[orow] = lse;
  }
}

// Generic row merge of K states: state k of row `row` is at
// v + (row_base(row) + k * k_stride) * D (values) and s[s_base(row) + k*s_k_stride].
// Used for merge_states ([n, K, H, D]) and the two-input forms.
template <class VIN, class VOUT>
__global__ __launch_bounds__(256) void merge_rows_kernel(const VIN* va, const float* sa,
                                                         const VIN* vb, const float* sb,
                                                         int64_t rows, int32_t H, int32_t K,
                                                         int32_t D, VOUT* vo, float* so) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  // vb == nullptr: K states interleaved as [n, K, H, D]; else two arrays [rows, D].
  const int64_t i = row / H, h = row - (row / H) * H;
  auto v_ptr = [&](int k) -> const VIN* {
    if (vb != nullptr) return (k == 0 ? va : vb) + row * D;
    return va + ((i * K + k) * H + h) * D;
  };
  auto s_val = [&](int k) -> float {
    if (vb != nullptr) return k == 0 ? sa[row] : sb[row];
    return sa[(i * K + k) * H + h];
  };
  float M = neg_inf();
  for (int k = 0; k < K; ++k) M = fmaxf(M, s_val(k));
  const float Mu = (M == neg_inf()) ? 0.f : M;
  float L = 0.f;
  for (int k = 0; k < K; ++k) L += fast_exp2((s_val(k) - Mu) * kLog2e);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int d = lane; d < D; d += 64) {
    float acc = 0.f;
    for (int k = 0; k < K; ++k) {
      const float w = fast_exp2((s_val(k) - Mu) * kLog2e);
      acc += w * load_f(v_ptr(k) + d);
    }
    store_f(vo + row * D + d, acc * inv);
  }
  if (lane == 0 && so != nullptr) so[row] = L > 0.f ? M + __logf(L) : neg_inf();
}

template <class V>
hipError_t merge_rows(const void* va, const float* sa, const void* vb, const float* sb,
                      int64_t rows, int32_t H, int32_t K, int32_t D, void* vo, float* so,
                      hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t grid = (rows + 3) / 4;
  hipLaunchKernelGGL((merge_rows_kernel<V, V>), dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                     s, static_cast<const V*>(va), sa, static_cast<const V*>(vb), sb, rows, H, K,
                     D, static_cast<V*>(vo), so);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge_groups(const MergeGroupsArgs& a, int32_t storage_dtype, OutKind out,
                               int32_t num_groups, int64_t num_chunks, hipStream_t stream) {
  if (num_groups <= 0) return hipSuccess;
  // Groups of 32 chunks or more on average: four waves per row, so that each
  // wave has at most a quarter of the batches in a row; otherwise one wave
  // per row (four rows per workgroup).
  const bool split = num_chunks >= 32 * static_cast<int64_t>(num_groups);
  const dim3 grid(num_groups, split ? a.rows_per_tile : (a.rows_per_tile + 3) / 4);
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a); };
  if (out == kOutF32) {
    split ? go(merge_groups_kernel<float, 4>) : go(merge_groups_kernel<float, 1>);
  } else if (storage_dtype == 0) {
    split ? go(merge_groups_kernel<_Float16, 4>) : go(merge_groups_kernel<_Float16, 1>);
  } else {
    split ? go(merge_groups_kernel<__bf16, 4>) : go(merge_groups_kernel<__bf16, 1>);
  }
  return hipGetLastError();
}

hipError_t launch_merge2(const void* va, const float* sa, const void* vb, const float* sb,
                         void* vo, float* so, int64_t rows, int32_t head_dim, int32_t v_dtype,
                         hipStream_t stream) {
  switch (v_dtype) {
    case 0: return merge_rows<_Float16>(va, sa, vb, sb, rows, 1, 2, head_dim, vo, so, stream);
    case 1: return merge_rows<__bf16>(va, sa, vb, sb, rows, 1, 2, head_dim, vo, so, stream);
    default: return merge_rows<float>(va, sa, vb, sb, rows, 1, 2, head_dim, vo, so, stream);
  }
}

hipError_t launch_merge_n(const void* v, const float* s, int64_t n, int32_t num_states,
                          int32_t num_heads, int32_t head_dim, int32_t v_dtype, void* vo,
                          float* so, hipStream_t stream) {
  const int64_t rows = n * num_heads;
  switch (v_dtype) {
    case 0:
      return merge_rows<_Float16>(v, s, nullptr, nullptr, rows, num_heads, num_states, head_dim,
                                  vo, so, stream);
    case 1:
      return merge_rows<__bf16>(v, s, nullptr, nullptr, rows, num_heads, num_states, head_dim, vo,
                                so, stream);
    default:
      return merge_rows<float>(v, s, nullptr, nullptr, rows, num_heads, num_states, head_dim, vo,
                               so, stream);
  }
}

hipError_t launch_merge2_f32_to(const float* va, const float* sa, const float* vb,
                                const float* sb, void* vo, float* so, int64_t rows,
                                int32_t head_dim, int32_t out_dtype, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((rows + 3) / 4));
  if (out_dtype == 0) {
    hipLaunchKernelGGL((merge_rows_kernel<float, _Float16>), grid, dim3(256), 0, stream, va, sa,
                       vb, sb, rows, 1, 2, head_dim, static_cast<_Float16*>(vo), so);
  } else {
    hipLaunchKernelGGL((merge_rows_kernel<float, __bf16>), grid, dim3(256), 0, stream, va, sa, vb,
                       sb, rows, 1, 2, head_dim, static_cast<__bf16*>(vo), so);
  }
  return hipGetLastError();
}

}  // namespace pkv
