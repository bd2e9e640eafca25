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
//   * KV advances in 64-token tiles staged through LDS, double-buffered: the
//     global loads of tile i+1 are in flight while tile i is computed.
//     K is stored row-major [token][d] (rows padded to 272 B); V is stored
//     transposed [d][token] (rows padded to 136 B, columns XOR-swizzled per
//     16 rows) so that the PV operand reads are 8-byte LDS loads and neither
//     the staging writes nor the reads have bank conflicts.
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

constexpr int KT = 64;                 // KV tokens per tile
constexpr int KROW = kHeadDim + 8;     // K row stride in LDS (elements)
constexpr int VROW = KT + 4;           // V^T row stride in LDS (elements)
constexpr int kTileRows = 128;

// Column (in elements) of logical token column `c` in row `d` of the
// transposed V tile. The XOR with 4 * (d >> 4) keeps 4-token (8-byte) groups
// together and makes both access patterns free of LDS bank conflicts: the
// staging writes (16 lanes writing rows 8 apart, same column) land in 16
// distinct bank pairs, and the MFMA operand reads (lanes reading 16
// consecutive rows, same column) still do.
__device__ __forceinline__ int vt_col(int d, int c) { return c ^ (4 * (d >> 4)); }

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
  __shared__ __attribute__((aligned(16))) elem sK[2][KT * KROW];
  __shared__ __attribute__((aligned(16))) elem sV[2][D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  const elem* kbase = static_cast<const elem*>(a.k) + static_cast<int64_t>(g) * a.head_stride;
  const elem* vbase = static_cast<const elem*>(a.v) + static_cast<int64_t>(g) * a.head_stride;
  const int32_t* pages = a.kv_indices + a.kv_indptr[b];
  const int P = a.page_size;
  auto token_off = [&](int t) -> int64_t {
    const int pi = t / P;
    const int sl = t - pi * P;
    return static_cast<int64_t>(pages[pi]) * a.page_stride +
           static_cast<int64_t>(sl) * a.token_stride;
  };

  // Staging: K thread (c = tid % 16 d-chunk, tokens tid/16 + 16*rep);
  //          V thread (c = tid % 16 d-chunk, tokens 4*(tid/16) + u).
  const int sc = tid & 15, sr = tid >> 4;
  u32x4 kst[4], vst[4];
  auto stage_load = [&](int tb) {
    const int last = k1 - 1;
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
      const int t = min(tb + sr + 16 * rep, last);
      kst[rep] = load_16B(kbase + token_off(t) + 8 * sc);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = min(tb + 4 * sr + u, last);
      vst[u] = load_16B(vbase + token_off(t) + 8 * sc);
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int rep = 0; rep < 4; ++rep)
      *reinterpret_cast<u32x4*>(&sK[buf][(sr + 16 * rep) * KROW + 8 * sc]) = kst[rep];
    // Transpose 4 tokens x 8 d into 8 rows of V^T (4 tokens each).
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // d = 8*sc + 2w (low halves) and 8*sc + 2w + 1 (high halves)
      const uint32_t lo01 = __builtin_amdgcn_perm(vst[1][w], vst[0][w], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(vst[3][w], vst[2][w], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(vst[1][w], vst[0][w], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(vst[3][w], vst[2][w], 0x07060302u);
      // rows 8*sc + 2w (+1) share (row >> 4) = sc >> 1: see vt_col
      const int col = vt_col(8 * sc, 4 * sr);
      *reinterpret_cast<u32x2*>(&sV[buf][(8 * sc + 2 * w) * VROW + col]) = u32x2{lo01, lo23};
      *reinterpret_cast<u32x2*>(&sV[buf][(8 * sc + 2 * w + 1) * VROW + col]) = u32x2{hi01, hi23};
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
    stage_load(k0);
    stage_store(0);
  }
  __syncthreads();

  for (int ti = 0; ti < ntiles; ++ti) {
    const int buf = ti & 1;
    const int tb = k0 + ti * KT;
    const bool more = ti + 1 < ntiles;
    if (more) stage_load(tb + KT);

    // S^T for two 32-token blocks.
    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[blk][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(
            &sK[buf][(32 * blk + lr) * KROW + 16 * kk + 8 * half]);
        s[blk] = T::mfma_32x32x16(kf, qv[kk], s[blk]);
      }
    }

    // Mask (only where the tile reaches past k1 or past this row's causal
    // limit). The running max is taken on the raw scores and scaled once
    // (scale > 0), and the scale is folded into the exponent's FMA below.
    const bool need_mask = (tb + KT > k1) || (a.causal && tb + KT - 1 > lim_wave);
    float tmax = neg_inf();
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[blk][i];
        if (need_mask) {
          const int t = tb + 32 * blk + 8 * (i >> 2) + 4 * half + (i & 3);
          if (t >= k1 || (a.causal && t > lim)) x = neg_inf();
        }
        s[blk][i] = x;
        tmax = fmaxf(tmax, x);
      }
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

    // O^T += V^T P^T over four 16-token steps.
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const elem* vrow = &sV[buf][(32 * mb + lr) * VROW];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + vt_col(32 * mb + lr, 16 * st + 4 * half));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + vt_col(32 * mb + lr, 16 * st + 4 * half + 8));
        acc[mb] = T::mfma_32x32x16(u32x4{lo[0], lo[1], hi[0], hi[1]}, pk[st], acc[mb]);
      }
    }

    if (more) stage_store(buf ^ 1);
    __syncthreads();
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
    const int64_t srow = static_cast<int64_t>(slot) * kTileRows + 32 * wave + lr;
    float* po = a.part_o + srow * D;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * mb + 8 * q4 + 4 * half;
        *reinterpret_cast<f32x4*>(po + d) =
            f32x4{acc[mb][4 * q4] * inv, acc[mb][4 * q4 + 1] * inv, acc[mb][4 * q4 + 2] * inv,
                  acc[mb][4 * q4 + 3] * inv};
      }
    if (half == 0) a.part_lse[srow] = lse;
  }
}

template <class T, class OUT>
hipError_t launch_prefill_t(const PrefillArgs& a, int32_t grid, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<T, OUT, kPagedGeneric>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int32_t prefill_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&prefill_kernel<BF16, __bf16, kPagedGeneric>), 256,
          0) != hipSuccess)
    return 0;
  return n;
}

hipError_t launch_prefill(const PrefillArgs& a, int32_t storage_dtype, OutKind out,
                          PageMode /*mode*/, int32_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (storage_dtype == 0) {
    return out == kOutF32 ? launch_prefill_t<F16, float>(a, grid, stream)
                          : launch_prefill_t<F16, _Float16>(a, grid, stream);
  }
  return out == kOutF32 ? launch_prefill_t<BF16, float>(a, grid, stream)
                        : launch_prefill_t<BF16, __bf16>(a, grid, stream);
}

}  // namespace pkv
