// Paged decode work item for gfx950: one query token per request, GQA-packed.
//
// The body of the decode kernel (decode.hip) and of the decode half of the
// mixed prefill + decode kernel (pod.hip).
//
// What it computes: for one work item (request b, KV head g, KV token range
// [t0, t1)) the attention state of the G query heads of group g over those
// tokens, with an online (running-max) softmax; a whole range gives the final
// output, a chunk gives a partial state (O, m, l) that the merge kernel
// combines (FlashInfer article, sections "Attention states" and
// "Extreme-negative-logit correction"; the page walk follows the page-table
// layout of the docs index, "KV-Cache Layout in FlashInfer").
//
// How it maps to CDNA4:
//   * A workgroup = 4 waves; wave w takes 16-token blocks w, w+4, ... of the
//     item and the four running states merge through LDS at the end.
//   * Scores: S^T = K Q^T on v_mfma_f32_16x16x32_{f16,bf16}. K is the A
//     operand: lane l loads 16 contiguous bytes of token (l % 16)'s K row
//     straight from HBM into registers; q (G <= 16 heads, padded to 16) is the
//     B operand, held in registers for the whole item. Lane l receives the
//     scores of head l % 16 for tokens 4*(l/16) + i, i = 0..3.
//   * PV: O^T = V^T P^T on v_mfma_f32_16x16x4_f32. V is the A operand: lane l
//     loads 16 contiguous bytes (d = 8*(l%16) .. +7) of token 4*(l/16) + i,
//     so 16 lanes read one 256-byte row; each of the 8 values feeds its own
//     MFMA (d is the row label). P stays fp32 and is exactly the score
//     registers the lane already holds, so there is no transpose and no
//     cross-lane traffic; every lane accumulates head l % 16, so the online
//     softmax rescale is lane-local.
//   * Row max across the 4 token rows of a block: v_permlane16/32_swap.
//   * Loads: one scalar buffer descriptor per 16-token block (page base,
//     range = the block's valid rows, so tail tokens read as zero) and
//     per-lane offsets fixed for the whole item; non-temporal, because the KV
//     cache is streamed once per call and must not evict reused data.
//   * Two register sets: block k+8's K is issued into block k's K registers
//     as soon as the scores have read them, its V after the PV product, so
//     about two blocks per wave are in flight; page ids are read one step
//     ahead. The loop has no branch around a load, so each wait covers only
//     the block about to be used.
//   * -inf is a real IEEE -inf; exp2 of (-inf) - (-inf) is avoided by
//     subtracting 0 when the running max is still -inf. An empty item yields
//     O = 0, LSE = -inf.
//   * Variants (VAR instances, paged modes; the FlashInfer article, section
//     "Custom attention templates", names them): the scores of a block are
//     soft-capped before the mask, tokens below the sliding window's start
//     (L - 1 - window_left) are masked like tail tokens, and a head's sink
//     joins the softmax in the epilogue of an item that writes the final row
//     (split items leave it to the merge).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;
constexpr int kDecodeWaves = kWaves;
constexpr int kBlock = 16;  // tokens per wave iteration
// K/V pages are read once per call: stream them past the caches.
constexpr int kCachePolicy = kCacheStream;

// LDS of the cross-wave merge at the end of an item: running maxima and sums
// [wave][16] and each wave's accumulator rows [16][128] (floats), whose
// 16-byte chunks are XOR-swizzled by row so that the 16 rows a lane group
// writes at one column land in different banks.
struct DecodeLds {
  float* m;
  float* l;
  float* acc[kWaves];
  __device__ __forceinline__ float* acc_of(int w) const {
    return w == 0 ? acc[0] : w == 1 ? acc[1] : w == 2 ? acc[2] : acc[3];
  }
};
__device__ __forceinline__ int acc_at(int row, int d) { return row * kHeadDim + (d ^ ((row & 15) << 2)); }

template <class T, class OUT, int MODE, bool VAR>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int b, int g, int t0, int t1,
                                            int slot, const DecodeLds& lds) {
  // The item is the same for every lane; saying so keeps it (and the page-table
  // reads and descriptors built from it) in SGPRs in any kernel this body is
  // inlined into.
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  t0 = __builtin_amdgcn_readfirstlane(t0);
  t1 = __builtin_amdgcn_readfirstlane(t1);
  slot = __builtin_amdgcn_readfirstlane(slot);
  static_assert(!VAR || MODE != kContiguous, "variants need the paged item table");
  using elem = typename T::elem;
  constexpr int D = kHeadDim;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is the same for all 64 lanes; saying so keeps everything
  // derived from it (block index, page id, buffer descriptor) in SGPRs.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane & 15, grp = lane >> 4;
  const int G = a.group;

  // q^T as the B operand: lane holds q[head hl][d = 32j + 8*grp .. +7].
  const elem* qrow = static_cast<const elem*>(a.q) +
                     (static_cast<int64_t>(b) * a.num_qo_heads + g * G + hl) * D + 8 * grp;
  u32x4 qv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qv[j] = hl < G ? load_16B(qrow + 32 * j) : u32x4{0, 0, 0, 0};

  const elem* kbase = static_cast<const elem*>(a.k) + static_cast<int64_t>(g) * a.head_stride;
  const elem* vbase = static_cast<const elem*>(a.v) + static_cast<int64_t>(g) * a.head_stride;
  const int32_t* pages = nullptr;
  if (MODE != kContiguous) pages = a.kv_indices + __builtin_amdgcn_readfirstlane(a.kv_indptr[b]);
  const int P = a.page_size;

  // Element offset of token t (relative to the request) in the pools.
  auto token_off = [&](int t) -> int64_t {
    if (MODE == kContiguous) return static_cast<int64_t>(t) * a.token_stride;
    const int pi = t / P;
    const int sl = t - pi * P;
    return static_cast<int64_t>(pages[pi]) * a.page_stride +
           static_cast<int64_t>(sl) * a.token_stride;
  };

  const int last = t1 - 1;
  // First token the query sees under the sliding window (VAR only).
  int wlo = 0;
  if constexpr (VAR) {
    if (a.var.window_left >= 0) wlo = a.kv_lens[b] - 1 - a.var.window_left;
  }
  const bool capped = VAR && a.var.cap_out > 0.f;

  // Issue the K and V loads of 16-token block `blk`. Paged-uniform and
  // contiguous modes: one scalar buffer descriptor per block, based at the
  // block's first token row of head g and ending after its last valid token
  // row, and per-lane byte offsets that are the same for every block; tail
  // tokens past t1 fall outside the descriptor and read as zero. Generic
  // mode: a page-table lookup per lane and token (tail tokens clamped).
  const uint32_t ts_bytes = static_cast<uint32_t>(a.token_stride) * sizeof(elem);
  const int nblk_total = (t1 - t0 + kBlock - 1) / kBlock;
  const uint32_t koff = hl * ts_bytes + 8 * grp * sizeof(elem);
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (4 * grp + i) * ts_bytes + 8 * hl * sizeof(elem);
  // Bytes of the descriptor of block `blk`: its valid token rows, or 0 for a
  // block past the item (every lane then reads zero and nothing is fetched).
  auto nbytes = [&](int blk) -> uint32_t {
    const int nvalid = min(kBlock, t1 - (t0 + kBlock * blk));
    return nvalid > 0 ? static_cast<uint32_t>(nvalid - 1) * ts_bytes + kHeadDim * sizeof(elem)
                      : 0u;
  };
  auto issue_k = [&](int blk, int64_t base, u32x4* kr) {
    if (MODE != kPagedGeneric) {
      const auto rk = make_rsrc(kbase + base, nbytes(blk));
#pragma unroll
      for (int j = 0; j < 4; ++j) kr[j] = buffer_load_16B<kCachePolicy>(rk, koff + 32 * j * sizeof(elem));
    } else if (blk < nblk_total) {
      const int tb = t0 + kBlock * blk;
      const elem* kp = kbase + token_off(min(tb + hl, last)) + 8 * grp;
#pragma unroll
      for (int j = 0; j < 4; ++j) kr[j] = load_16B_stream(kp + 32 * j);
    }
  };
  auto issue_v = [&](int blk, int64_t base, u32x4* vr) {
    if (MODE != kPagedGeneric) {
      const auto rv = make_rsrc(vbase + base, nbytes(blk));
#pragma unroll
      for (int i = 0; i < 4; ++i) vr[i] = buffer_load_16B<kCachePolicy>(rv, voff[i]);
    } else if (blk < nblk_total) {
      const int tb = t0 + kBlock * blk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[i] = load_16B_stream(vbase + token_off(min(tb + 4 * grp + i, last)) + 8 * hl);
    }
  };

  float m_run = neg_inf();  // running max (log2 domain) of head hl
  float l_run = 0.f;        // this lane's share of the running sum
  f32x4 acc[8];             // acc[j][r]: head hl, d = 32*grp + 8*r + j
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One 16-token block: scores on MFMA, then (after the caller reuses the K
  // registers) online softmax and PV on MFMA.
  auto scores = [&](const u32x4* kc) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) s = T::mfma_16x16x32(kc[j], qv[j], s);
    return s;
  };
  auto softmax_pv = [&](int blk, f32x4 s, const u32x4* vc) {
    const int tb = t0 + kBlock * blk;
    // Raw scores (soft-capped for the variant), -inf where masked. The block
    // maximum is taken on them and scaled once, and each weight is
    // 2^(s * scale_log2 - m) from one fused multiply-add: no rounded product
    // of a large score with the scale enters a weight, so weights stay exact
    // to fp32 rounding of their own (small) exponent even when every logit is
    // ~1e5 in magnitude.
    float r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tb + 4 * grp + i;
      float si = s[i];
      bool vis = t < t1;
      if constexpr (VAR) {
        if (capped) si = soft_cap(si, a.var.cap_in, a.var.cap_out);
        vis = vis && t >= wlo;
      }
      r[i] = vis ? si : neg_inf();
    }
    float bm = fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3]));
    bm = max_across_rows(bm) * a.scale_log2;
    const float m_new = fmaxf(m_run, bm);
    const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(r[i], a.scale_log2, -m_use));
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
    // Rescale only when some head's running max moved (wave-uniform branch).
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x8 vf = T::to_f32(vc[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[j], p[i], acc[j], 0, 0, 0);
    }
  };

  // Two register sets. While block blk (set X) is computed, block blk+4
  // (set Y) is in flight; block blk+8's K is issued into X's K registers as
  // soon as the scores have read them, and its V into X's V registers after
  // the PV product. The loads are issued unconditionally (a block past the
  // item gets an empty descriptor) and the loop body has no early exit, so
  // each wait covers only the block about to be used. The page id of block
  // blk+12 is read one step before it is needed.
  const int nblk = nblk_total;
  // Paged-uniform mode: blocks per page = P / 16; the page index of block
  // blk is t0 / P + blk / (P / 16) (shifts when P / 16 is a power of two).
  const int bpp = P / kBlock;
  const int bpp_shift = (MODE == kPagedUniform && (bpp & (bpp - 1)) == 0) ? __builtin_ctz(bpp) : -1;
  const int page0 = MODE == kPagedUniform ? t0 / P : 0;
  auto pid_of = [&](int blk) -> int {
    if (MODE != kPagedUniform) return 0;
    blk = min(blk, nblk - 1);                   // always a page of this item
    const int pi = bpp_shift >= 0 ? page0 + (blk >> bpp_shift) : page0 + blk / bpp;
    return pages[pi];
  };
  auto base_from = [&](int blk, int pid) -> int64_t {
    const int tb = t0 + kBlock * blk;
    if (MODE == kContiguous) return static_cast<int64_t>(tb) * a.token_stride;
    if (MODE == kPagedGeneric) return 0;
    const int slot0 = bpp_shift >= 0 ? (blk & (bpp - 1)) * kBlock : (blk % bpp) * kBlock;
    return static_cast<int64_t>(pid) * a.page_stride +
           static_cast<int64_t>(slot0) * a.token_stride;
  };
  int blk = wave;
  u32x4 kA[4], vA[4], kB[4], vB[4];
  if (nblk > 0) {
    {
      const int64_t b0 = base_from(blk, pid_of(blk));
      const int64_t b1 = base_from(blk + kWaves, pid_of(blk + kWaves));
      issue_k(blk, b0, kA);
      issue_v(blk, b0, vA);
      issue_k(blk + kWaves, b1, kB);
      issue_v(blk + kWaves, b1, vB);
    }
    int pid_next = pid_of(blk + 2 * kWaves);
    const int steps = blk < nblk ? (nblk - blk + kWaves - 1) / kWaves : 0;
#define PKV_DECODE_STEP(KX, VX)                                                    \
  {                                                                                \
    const int64_t base_next = base_from(blk + 2 * kWaves, pid_next);               \
    pid_next = pid_of(blk + 3 * kWaves);                                           \
    const f32x4 s = scores(KX);                                                    \
    issue_k(blk + 2 * kWaves, base_next, KX);                                      \
    softmax_pv(blk, s, VX);                                                        \
    issue_v(blk + 2 * kWaves, base_next, VX);                                      \
    blk += kWaves;                                                                 \
  }
    int st = 0;
    for (; st + 2 <= steps; st += 2) {
      PKV_DECODE_STEP(kA, vA)
      PKV_DECODE_STEP(kB, vB)
    }
    if (st < steps) PKV_DECODE_STEP(kA, vA)
  }
#undef PKV_DECODE_STEP

  // Merge the four waves' states (all in the log2 domain).
  l_run = sum_across_rows(l_run);
  if (grp == 0) {
    lds.m[wave * 16 + hl] = m_run;
    lds.l[wave * 16 + hl] = l_run;
  }
  if (hl < G) {
    float* dst = lds.acc_of(wave);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 32 * grp + 8 * r;
      *reinterpret_cast<f32x4*>(dst + acc_at(hl, c)) = f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
      *reinterpret_cast<f32x4*>(dst + acc_at(hl, c + 4)) = f32x4{acc[4][r], acc[5][r], acc[6][r], acc[7][r]};
    }
  }
  __syncthreads();

  const int64_t row0 = static_cast<int64_t>(b) * a.num_qo_heads + g * G;
  const bool split = slot >= 0;
  for (int e = tid; e < G * D; e += 256) {
    const int row = e >> 7, d = e & (D - 1);
    float M = lds.m[row];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, lds.m[w * 16 + row]);
    // A sink (log2 domain) is one more term of the sum, with a zero value;
    // a split item leaves it to the merge.
    float sink = neg_inf();
    if constexpr (VAR) {
      if (a.var.sinks != nullptr && !split) sink = a.var.sinks[g * G + row] * kLog2e;
      M = fmaxf(M, sink);
    }
    const float Mu = (M == neg_inf()) ? 0.f : M;
    float L = 0.f, O = 0.f;
    if constexpr (VAR) L = fast_exp2(sink - Mu);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(lds.m[w * 16 + row] - Mu);
      L += f * lds.l[w * 16 + row];
      O += f * lds.acc_of(w)[acc_at(row, d)];
    }
    const float o = L > 0.f ? O / L : 0.f;
    if (!split) {
      const float lse = L > 0.f ? (M + fast_log2(L)) * kLn2 : neg_inf();
      static_cast<OUT*>(a.o)[(row0 + row) * D + d] = out_cast<OUT>(o);
      if (d == 0 && a.lse != nullptr) a.lse[row0 + row] = lse;
    } else {
      // The chunk's partial state: O, and (m, l) = the reference exponent and
      // the weight sum in the log2 domain.
      const int64_t srow = static_cast<int64_t>(slot) * G + row;
      a.part_o[srow * D + d] = o;
      if (d == 0) *reinterpret_cast<f32x2*>(a.part_ml + 2 * srow) = f32x2{M, L};
    }
  }
}

}  // namespace

}  // namespace pkv
