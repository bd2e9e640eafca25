// Paged prefill / append kernel for gfx950 (also level 0 of the cascade).
//
// What it computes: for one work item (request b, KV head g, a tile of 128
// GQA-packed query rows, KV token range [k0, k1)) the attention state of
// every row over the visible keys of that range: with the bottom-right causal
// mask, query token i of a request with Q query tokens and L keys sees key t
// iff t <= i + L - Q. Online softmax with IEEE -inf; a row that sees no key
// in the range yields O = 0, LSE = -inf (FlashInfer article, sections
// "Attention states" and "Extreme-negative-logit correction"; docs index
// "flashinfer.prefill", "KV-Cache Layout in FlashInfer").
//
// How it maps to CDNA4:
//   * Workgroup = 4 waves, wave w owns rows 32w .. 32w+31 of the tile; a row
//     is (query token, query head) with the G heads of a KV group packed
//     together, so each K/V tile read from HBM serves G heads.
//   * KV advances in 64-token tiles, double-buffered in LDS. The tiles go
//     from HBM straight into LDS (buffer / global loads with the LDS flag), so
//     no registers hold them in flight and no instructions copy them: wave w
//     fetches the 16-token group w of the next tile (four 1 KB loads for K,
//     four for V) while every wave computes the current one. The page id of a
//     group is read one tile before its loads are issued. With page_size a
//     multiple of 16 a group lies in one page: one descriptor per wave and
//     tile, ranged to the group's valid tokens so that tokens past the item
//     read as zero; other page sizes look up every token and repeat the last
//     valid one past the end (its weight is exactly 0).
//   * LDS rows are 256 B (one token's 128 values, unpadded) with the 16-byte
//     chunks XOR-swizzled per row: K by (row mod 16), V by 4 * (row mod 4).
//     Neither the K operand reads (32 rows, one chunk) nor the transposing V
//     reads (ds_read_b64_tr_b16: 4 rows x 16 values per 16 lanes) then hit a
//     bank twice in one cycle.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16}: K rows are the A operand
//     (from LDS), the wave's 32 q rows are the B operand (registers for the
//     whole item). Lane l then holds 16 scores of row l % 32 per 32 tokens,
//     so the row max and sum are lane-local plus one permlane32 swap.
//   * O^T = V^T P^T on the same MFMA: P is rounded to the storage dtype and
//     is taken straight from the score registers (the token order inside a
//     16-token step is permuted identically on both operands); the fp32
//     accumulator of row l % 32 stays in lane l, so the rescale is lane-local.
//   * The scale multiplies the fp32 scores (q is not pre-scaled), in the
//     log2 domain; LSE = (m + log2 l) * ln 2.
#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int KT = 64;                       // KV tokens per tile
constexpr int kTileRows = 128;
constexpr int kRowBytes = kHeadDim * 2;      // one token row in LDS
constexpr int kTileBytes = KT * kRowBytes;   // 16 KB per K or V tile

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Byte offset in an LDS tile of 16-byte chunk c of token row t.
__device__ __forceinline__ int k_at(int t, int c) { return t * kRowBytes + 16 * (c ^ (t & 15)); }
__device__ __forceinline__ int v_at(int t, int c) { return t * kRowBytes + 16 * (c ^ (4 * (t & 3))); }

// Cache policy of the KV tile loads. Every query tile of a (request, KV
// head) reads the same KV, so the tiles stay cacheable.
constexpr int kKvPolicy = kCacheDefault;

// 16 bytes per lane from global memory straight into LDS: lane i writes
// dst + 16 i (dst wave-uniform). Buffer form: bytes past the descriptor's
// range read as zero.
__device__ __forceinline__ void buffer_to_lds_16B(__amdgpu_buffer_rsrc_t r, lds_void* dst,
                                                  uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, byte_off, 0, 0, kKvPolicy);
}
__device__ __forceinline__ void global_to_lds_16B(const void* src, lds_void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, kKvPolicy);
}
__device__ __forceinline__ s16x4 lds_read_tr16_b64(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left free): the direct-to-LDS loads
// of this wave have landed.
__device__ __forceinline__ void wait_lds_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Stores 4 consecutive output values (rounded once to OUT).
template <class OUT>
__device__ __forceinline__ void store4(OUT* p, float x0, float x1, float x2, float x3) {
  if constexpr (sizeof(OUT) == 4) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x0, x1, x2, x3};
  } else {
    const uint32_t a = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, out_cast<OUT>(x0))) |
                       (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, out_cast<OUT>(x1))) << 16);
    const uint32_t b = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, out_cast<OUT>(x2))) |
                       (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, out_cast<OUT>(x3))) << 16);
    *reinterpret_cast<u32x2*>(p) = u32x2{a, b};
  }
}

template <class T, class OUT, int MODE>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillArgs a) {
  using elem = typename T::elem;
  constexpr int D = kHeadDim;
  // Two stages, four distinct arrays: the compiler then sees that the loads
  // into one stage never alias the operand reads of the other and does not
  // wait for the loads in flight before reading the current tile.
  __shared__ __attribute__((aligned(1024))) char sKa[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sVa[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sKb[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sVb[kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, half = lane >> 5;
  const int G = a.group;

  const int32_t* it = a.items + 8 * blockIdx.x;
  const int b = it[0], g = it[1], tile = it[2], k0 = it[5], k1 = it[6], slot = it[7];
  const int q0 = a.qo_indptr[b];
  const int Q = a.qo_indptr[b + 1] - q0;
  const int L = a.kv_lens[b];

  // This lane's query row.
  const int prow = tile * kTileRows + 32 * wave + lr;     // GQA-packed row in the request
  const bool row_ok = prow < Q * G;
  const int qtok = prow / G;
  const int head = g * G + (prow - qtok * G);
  const int lim = qtok + L - Q;                            // last visible key (causal)
  // Smallest causal limit of the wave (its first row): tiles that end at or
  // before it need no causal mask for any row of the wave.
  const int lim_wave = (tile * kTileRows + 32 * wave) / G + L - Q;

  // q^T as the B operand: lane holds q[row lr][d = 16kk + 8*half .. +7].
  u32x4 qv[8];
  {
    const elem* qp = static_cast<const elem*>(a.q) +
                     (static_cast<int64_t>(q0 + qtok) * a.num_qo_heads + head) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qv[kk] = row_ok ? load_16B(qp + 16 * kk) : u32x4{0, 0, 0, 0};
  }

  // ---- staging: wave w fetches token rows 16w .. 16w+15 of a tile; load j
  // (0..3) covers rows 16w + 4j + lane/16, lane % 16 being the LDS chunk slot.
  const char* kbase = static_cast<const char*>(a.k) + static_cast<int64_t>(g) * a.head_stride * 2;
  const char* vbase = static_cast<const char*>(a.v) + static_cast<int64_t>(g) * a.head_stride * 2;
  const int P = a.page_size;
  const int64_t ps_bytes = a.page_stride * 2;
  const uint32_t ts_bytes = static_cast<uint32_t>(a.token_stride) * 2;
  const int page0 = a.kv_indptr[b];
  const int npages = a.kv_indptr[b + 1] - page0;
  const __amdgpu_buffer_rsrc_t pt = make_rsrc(a.kv_indices + page0, 4u * static_cast<uint32_t>(npages));
  const int srow = lane >> 4, spos = lane & 15;
  // Global chunk fetched by this lane for load j (the inverse of the swizzle).
  auto k_chunk = [&](int j) { return spos ^ (4 * j + srow); };
  const int v_chunk = spos ^ (4 * srow);
  auto lds_dst = [&](char* tile_base, int j) -> lds_void* {
    return (lds_void*)(tile_base + (16 * wave + 4 * j) * kRowBytes);
  };

  // Page-uniform mode: page id of the group of tile ti (wave-uniform).
  const int pshift = (P & (P - 1)) == 0 ? __builtin_ctz(P) : -1;
  auto group_page = [&](int ti) -> int {      // page index in the request
    const int tc = min(k0 + ti * KT + 16 * wave, k1 - 1);
    // (uniform; readfirstlane keeps it in SGPRs when the division runs on VALU)
    return __builtin_amdgcn_readfirstlane(pshift >= 0 ? (tc >> pshift) : tc / P);
  };
  // Generic mode: page index and slot of the lane's token for load j of tile ti.
  auto lane_token = [&](int ti, int j) -> int { return min(k0 + ti * KT + 16 * wave + 4 * j + srow, k1 - 1); };

  int pid_next[4];   // page ids for the next tile's loads (uniform mode: [0] only)
  auto fetch_pids = [&](int ti) {
    if constexpr (MODE == kPagedUniform) {
      pid_next[0] = __builtin_amdgcn_raw_buffer_load_b32(pt, 4u * group_page(ti), 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pid_next[j] = __builtin_amdgcn_raw_buffer_load_b32(pt, 4u * (lane_token(ti, j) / P), 0, 0);
    }
  };
  auto issue_tile = [&](int ti, char* kdst, char* vdst) {
    if constexpr (MODE == kPagedUniform) {
      const int t = k0 + ti * KT + 16 * wave;
      const int pi = group_page(ti);
      const int pid = __builtin_amdgcn_readfirstlane(pid_next[0]);
      const int sl = min(t, k1 - 1) - pi * P;
      const int nvalid = __builtin_amdgcn_readfirstlane(max(0, min(16, k1 - t)));   // (v_med3)
      const int64_t goff = static_cast<int64_t>(pid) * ps_bytes + static_cast<int64_t>(sl) * ts_bytes;
      const uint32_t nbytes = static_cast<uint32_t>(nvalid) * ts_bytes;
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + goff, nbytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + goff, nbytes);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t row = static_cast<uint32_t>(4 * j + srow) * ts_bytes;
        buffer_to_lds_16B(rk, lds_dst(kdst, j), row + 16 * k_chunk(j));
        buffer_to_lds_16B(rv, lds_dst(vdst, j), row + 16 * v_chunk);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tc = lane_token(ti, j);
        const int sl = tc - (tc / P) * P;
        const int64_t off = static_cast<int64_t>(pid_next[j]) * ps_bytes + static_cast<int64_t>(sl) * ts_bytes;
        global_to_lds_16B(kbase + off + 16 * k_chunk(j), lds_dst(kdst, j));
        global_to_lds_16B(vbase + off + 16 * v_chunk, lds_dst(vdst, j));
      }
    }
  };

  float m_run = neg_inf();   // running max of row lr (log2 domain)
  float l_run = 0.f;         // this lane's share of the running sum (exact weights)
  float lq_run = 0.f;        // the same sum over the rounded weights fed to the PV MFMA
  f32x16 acc[4];             // acc[mb][i]: row lr, d = 32mb + 8(i/4) + 4*half + i%4
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;

  const int ntiles = (k1 - k0 + KT - 1) / KT;
  if (ntiles > 0) {
    fetch_pids(0);
    issue_tile(0, sKa, sVa);   // waits for the page ids it needs
    fetch_pids(1);
  }
  wait_lds_loads();
  __syncthreads();

  // Operand addresses that do not depend on the tile.
  // K (A operand of S^T): row 32blk + lr, chunk 2kk + half.
  // V (A operand of O^T, transposing read): 16-lane group q16 = lane/16 reads
  // rows base + (lane%16)/4 at d = 32mb + 16(q16 & 1) + 4(lane & 3).
  const int vq = (lane >> 2) & 3;                           // row within the 4-row block
  const int vchunk_lo = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vbyte = 8 * (lane & 1);

  // One tile: compute from (kt, vt) while the next tile streams into (kn, vn).
  auto step = [&](int ti, const char* kt, const char* vt, char* kn, char* vn) {
    const int tb = k0 + ti * KT;
    if (ti + 1 < ntiles) {
      issue_tile(ti + 1, kn, vn);
      fetch_pids(ti + 2);
    }

    // S^T for two 32-token blocks.
    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[blk][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kt + k_at(32 * blk + lr, 2 * kk + half));
        s[blk] = T::mfma_32x32x16(kf, qv[kk], s[blk]);
      }
    }

    // Mask (only where the tile reaches past k1 or past this row's causal
    // limit). The running max is taken on the raw scores and scaled once
    // (scale > 0), and the scale is folded into the exponent's FMA below.
    const bool need_mask = (tb + KT > k1) || (a.causal && tb + KT - 1 > lim_wave);
    if (need_mask) {
      // Last key this lane's row may see in the tile, relative to the
      // lane's first token (one compare and select per score, no branches).
      const int tlast = (a.causal ? min(k1 - 1, lim) : k1 - 1) - (tb + 4 * half);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * blk + 8 * (i >> 2) + (i & 3) > tlast) s[blk][i] = neg_inf();
    }
    float tmax = neg_inf();
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[blk][i]);
    tmax = max_across_halves(tmax) * a.scale_log2;
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    // P rounded once to the storage dtype. O is normalised by the sum of the
    // same rounded weights (an exact convex combination of V rows); the LSE
    // uses the sum of the unrounded weights.
    u32x4 pk[4];                       // pk[st]: the B operand of 16-token step st
    float psum = 0.f, pqsum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int blk = st >> 1, hf = st & 1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = fast_exp2(fmaf(s[blk][8 * hf + 2 * j], a.scale_log2, -m_use));
        const float x1 = fast_exp2(fmaf(s[blk][8 * hf + 2 * j + 1], a.scale_log2, -m_use));
        pk[st][j] = T::pack2(x0, x1);
        pqsum = T::add_pair(pk[st][j], pqsum);
        psum += x0 + x1;
      }
    }
    l_run = l_run * alpha + psum;
    lq_run = lq_run * alpha + pqsum;
    // Rescale only when some row's running max moved (wave-uniform branch).
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] *= alpha;
    }

    // O^T += V^T P^T over four 16-token steps. Step st covers tokens
    // 16st + 4*half + {0..3} (first read) and + {8..11} (second read), the
    // order in which pk[st] holds them.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int r0 = 16 * st + 4 * half + vq;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int c = 4 * mb + vchunk_lo;
        const s16x4 lo = lds_read_tr16_b64(vt + v_at(r0, c) + vbyte);
        const s16x4 hi = lds_read_tr16_b64(vt + v_at(r0 + 8, c) + vbyte);
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        acc[mb] = T::mfma_32x32x16(u32x4{l2[0], l2[1], h2[0], h2[1]}, pk[st], acc[mb]);
      }
    }

    wait_lds_loads();
    __syncthreads();
  };
  for (int ti = 0; ti < ntiles; ti += 2) {
    step(ti, sKa, sVa, sKb, sVb);
    if (ti + 1 < ntiles) step(ti + 1, sKb, sVb, sKa, sVa);
  }

  // Finalize row lr.
  const float l_tot = sum_across_halves(l_run);
  const float lq_tot = sum_across_halves(lq_run);
  if (!row_ok) return;
  const float inv = lq_tot > 0.f ? 1.f / lq_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : neg_inf();
  if (slot < 0) {
    const int64_t orow = static_cast<int64_t>(q0 + qtok) * a.num_qo_heads + head;
    OUT* o = static_cast<OUT*>(a.o) + orow * D;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * mb + 8 * q4 + 4 * half;
        store4<OUT>(o + d, acc[mb][4 * q4] * inv, acc[mb][4 * q4 + 1] * inv,
                    acc[mb][4 * q4 + 2] * inv, acc[mb][4 * q4 + 3] * inv);
      }
    if (half == 0 && a.lse != nullptr) a.lse[orow] = lse;
  } else {
    const int64_t srow_out = static_cast<int64_t>(slot) * kTileRows + 32 * wave + lr;
    float* po = a.part_o + srow_out * D;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * mb + 8 * q4 + 4 * half;
        *reinterpret_cast<f32x4*>(po + d) =
            f32x4{acc[mb][4 * q4] * inv, acc[mb][4 * q4 + 1] * inv, acc[mb][4 * q4 + 2] * inv,
                  acc[mb][4 * q4 + 3] * inv};
      }
    if (half == 0) a.part_lse[srow_out] = lse;
  }
}

template <class T, class OUT>
hipError_t launch_prefill_t(const PrefillArgs& a, PageMode mode, int32_t grid, hipStream_t s) {
  if (mode == kPagedUniform)
    hipLaunchKernelGGL((prefill_kernel<T, OUT, kPagedUniform>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_kernel<T, OUT, kPagedGeneric>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int32_t prefill_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&prefill_kernel<BF16, __bf16, kPagedUniform>), 256,
          0) != hipSuccess)
    return 0;
  return n;
}

hipError_t launch_prefill(const PrefillArgs& a, int32_t storage_dtype, OutKind out,
                          PageMode mode, int32_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (storage_dtype == 0) {
    return out == kOutF32 ? launch_prefill_t<F16, float>(a, mode, grid, stream)
                          : launch_prefill_t<F16, _Float16>(a, mode, grid, stream);
  }
  return out == kOutF32 ? launch_prefill_t<BF16, float>(a, mode, grid, stream)
                        : launch_prefill_t<BF16, __bf16>(a, mode, grid, stream);
}

}  // namespace pkv
