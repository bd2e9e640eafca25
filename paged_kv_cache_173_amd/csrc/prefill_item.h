// Paged prefill / append work item for gfx950 (also level 0 of the cascade).
//
// The body of the prefill kernel (prefill.hip) and of the prefill half of the
// mixed prefill + decode kernel (pod.hip).
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
//   * Workgroup = 4 waves, wave w owns rows 32w .. 32w+31 of the 128-row tile;
//     a row is (query token, query head) with the G heads of a KV group packed
//     together, so each K/V tile read from HBM serves G heads.
//   * KV advances in 32-token tiles (KT) through a four-deep LDS ring per
//     operand (sK0..sK3, sV0..sV3, 8 KB each, 64 KB per workgroup): K is
//     loaded four tiles ahead, V three. Tiles go from HBM straight into LDS
//     (buffer / global loads with the LDS flag), so no registers hold them in
//     flight and no instructions copy them: wave w fetches kRpw = KT / NW = 8
//     token rows of each tile (two 1 KB loads for K, two for V). Each
//     iteration ends with s_waitcnt vmcnt(2 * kLoadsPerIter) (loads complete
//     in issue order; every iteration issues the same loads, tiles past the
//     item reading zero) and a fence-free barrier. Page ids are read two
//     iterations ahead. With page_size a power of two >= 16 a wave's rows of a
//     tile lie in one page: one descriptor per wave and tile, ranged to the
//     valid tokens so that tokens past the item read as zero; other page
//     sizes look up every token and repeat the last valid one past the end
//     (its weight is exactly 0).
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
//   * Software pipeline: iteration j computes S(j+1) on the MFMAs while the
//     VALU forms tile j's weights, then tile j's PV product runs beside the
//     row maxima of tile j+1; the reference exponent of a row moves only when
//     a score exceeds it by more than 2^8 (lazy rescaling).
//   * The scale multiplies the fp32 scores (q is not pre-scaled), in the
//     log2 domain, fused with the subtraction of the reference; LSE =
//     (m + log2 l) * ln 2. A split item writes its partial state as O and the
//     pair (m, l).
//   * Variants (VAR instances; the FlashInfer article, section "Custom
//     attention templates", names them): a tile's scores are soft-capped as
//     soon as they leave the MFMAs, before the mask; the sliding window masks
//     keys below a row's window start in the same wave-uniform mask step as
//     the causal limit (the plan already starts each item at the page of its
//     first row's window); a head's sink joins the final sum of an item that
//     writes the final row (split items leave it to the merge).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int KT = 32;                       // KV tokens per tile
constexpr int kTileRows = 128;
constexpr int kRowBytes = kHeadDim * 2;      // one token row in LDS
constexpr int kTileBytes = KT * kRowBytes;   // 8 KB per K or V tile

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

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left free): at most N of this wave's
// vector-memory loads (direct-to-LDS loads included; they count in issue
// order) are still in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for the LDS tiles without a memory fence: the wave's own
// LDS reads are complete (lgkmcnt(0)) and the direct-to-LDS loads it needs
// were waited for by the caller, so no vector-memory wait is forced here (a
// fence would wait for every load in flight, including the prefetches).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Stores 4 consecutive output values (rounded once to OUT, nearest even; a
// 16-bit OUT is packed two values per conversion).
template <class OUT>
__device__ __forceinline__ void store4(OUT* p, float x0, float x1, float x2, float x3) {
  if constexpr (sizeof(OUT) == 4) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x0, x1, x2, x3};
  } else {
    using S = std::conditional_t<std::is_same_v<OUT, __bf16>, BF16, F16>;
    static_assert(std::is_same_v<OUT, typename S::elem>, "16-bit outputs are fp16 or bf16");
    *reinterpret_cast<u32x2*>(p) = u32x2{S::pack2(x0, x1), S::pack2(x2, x3)};
  }
}

// Lazy rescaling: the exponent reference of a row moves only when the row's
// scaled maximum exceeds it by more than this many powers of two, so weights
// stay <= 2^8 (exact in fp32 and in the fp16 / bf16 range) and the running
// state is rescaled a few times per row instead of on most tiles.
constexpr float kRescaleSlack = 8.f;

// K and V tiles in LDS, four buffers each: tile t lives in buffer t % 4.
// Eight distinct arrays, so the compiler sees that the loads streaming into
// one buffer never alias the operand reads of another (a kernel that uses
// them gets its own copy).
__shared__ __attribute__((aligned(1024))) char sK0[kTileBytes];
__shared__ __attribute__((aligned(1024))) char sK1[kTileBytes];
__shared__ __attribute__((aligned(1024))) char sK2[kTileBytes];
__shared__ __attribute__((aligned(1024))) char sK3[kTileBytes];
__shared__ __attribute__((aligned(1024))) char sV0[kTileBytes];
__shared__ __attribute__((aligned(1024))) char sV1[kTileBytes];
__shared__ __attribute__((aligned(1024))) char sV2[kTileBytes];
__shared__ __attribute__((aligned(1024))) char sV3[kTileBytes];

// NW = waves per workgroup (4 or 8); RB = row blocks per wave: wave w owns
// rows 32*RB*w .. 32*RB*(w+1)-1 of an item of 32*NW*RB rows, in RB blocks of
// 32. The NW waves share every K / V tile (each stages KT/NW of its rows). Every K and V operand read from LDS
// feeds RB MFMAs (one per block). The kernels use RB = 1 (two waves per SIMD,
// 187-221 VGPRs by instance). RB = 2 halves the LDS reads per MFMA but needs about 330
// registers per lane, so one wave per SIMD; with the compiler placing the
// score accumulators in AGPRs (every softmax touch then copies them out) it
// gave bit-identical results 23 % slower on the causal prefill workload.
template <class T, class OUT, int MODE, bool VAR, int RB = 1, int NW = 4>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, const int32_t* it) {
  static_assert(NW == 4 || NW == 8, "a tile's 32 rows are staged in groups of four per load");
  using elem = typename T::elem;
  constexpr int D = kHeadDim;
  constexpr int kRows = 32 * NW * RB;     // query rows of one item
  constexpr int kRpw = KT / NW;           // tile rows each wave stages
  constexpr int kLpw = kRpw / 4;          // its loads per K or V tile (four rows each)
  auto kbuf = [&](auto ph) -> char* {
    constexpr int i = decltype(ph)::value & 3;
    if constexpr (i == 0) return sK0;
    else if constexpr (i == 1) return sK1;
    else if constexpr (i == 2) return sK2;
    else return sK3;
  };
  auto vbuf = [&](auto ph) -> char* {
    constexpr int i = decltype(ph)::value & 3;
    if constexpr (i == 0) return sV0;
    else if constexpr (i == 1) return sV1;
    else if constexpr (i == 2) return sV2;
    else return sV3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, half = lane >> 5;
  const int G = a.group;
#ifdef PKV_DEBUG_LDS_POISON
  // Debug builds: every LDS tile buffer starts as NaN (0xFFFF is a NaN in fp16
  // and bf16), so a tile read before its load has landed poisons the output
  // instead of reading rows left by an earlier item.
  {
    char* const bufs[8] = {sK0, sK1, sK2, sK3, sV0, sV1, sV2, sV3};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      for (int off = 16 * tid; off < kTileBytes; off += 16 * blockDim.x)
        *reinterpret_cast<u32x4*>(bufs[i] + off) = u32x4{~0u, ~0u, ~0u, ~0u};
    __syncthreads();
  }
#endif

  // The item's fields and the request's table entries are the same for every
  // lane; saying so keeps them (and the descriptors built from them) in SGPRs
  // whatever kernel this body is inlined into.
  const auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  const int b = uni(it[0]), g = uni(it[1]), tile = uni(it[2]), k0 = uni(it[5]), k1 = uni(it[6]),
            slot = uni(it[7]);
  const int q0 = uni(a.qo_indptr[b]);
  const int Q = uni(a.qo_indptr[b + 1]) - q0;
  const int L = uni(a.kv_lens[b]);

  // This lane's query rows (one per block).
  const int row0 = tile * kRows + 32 * RB * wave;          // the wave's first row
  bool row_ok[RB];
  int qtok[RB], head[RB], lim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int prow = row0 + 32 * rb + lr;                  // GQA-packed row in the request
    row_ok[rb] = prow < Q * G;
    qtok[rb] = prow / G;
    head[rb] = g * G + (prow - qtok[rb] * G);
    lim[rb] = qtok[rb] + L - Q;                            // last visible key (causal)
  }
  // Smallest causal limit of the wave (its first row): tiles that end at or
  // before it need no causal mask for any row of the wave.
  const int lim_wave = row0 / G + L - Q;
  // Keys past this one need a mask for some row of the wave (the causal
  // limit of the wave's first row, or the item's end).
  const int mask_from = a.causal ? min(k1 - 1, lim_wave) : k1 - 1;
  // Sliding window (VAR): the row's first visible key, and the largest of
  // them in the wave (its last row's): tiles starting below it need the
  // window mask for some row of the wave.
  int wlo[RB], win_from = 0;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) wlo[rb] = 0;
  if constexpr (VAR) {
    if (a.var.window_left >= 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) wlo[rb] = lim[rb] - a.var.window_left;
      win_from = (row0 + 32 * RB - 1) / G + L - Q - a.var.window_left;
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) wlo[rb] = INT32_MIN / 4;
      win_from = INT32_MIN / 4;
    }
  }
  const bool capped = VAR && a.var.cap_out > 0.f;

  // q^T as the B operand: lane holds q[row][d = 16kk + 8*half .. +7] of each block.
  u32x4 qv[RB][8];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const elem* qp = static_cast<const elem*>(a.q) +
                     (static_cast<int64_t>(q0 + qtok[rb]) * a.num_qo_heads + head[rb]) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qv[rb][kk] = row_ok[rb] ? load_16B(qp + 16 * kk) : u32x4{0, 0, 0, 0};
  }

  // ---- staging: wave w fetches token rows kRpw*w .. kRpw*(w+1)-1 of a tile;
  // load j (0 .. kLpw-1) covers rows kRpw*w + 4j + lane/16, lane % 16 being
  // the LDS chunk slot.
  const char* kbase = static_cast<const char*>(a.k) + static_cast<int64_t>(g) * a.head_stride * 2;
  const char* vbase = static_cast<const char*>(a.v) + static_cast<int64_t>(g) * a.head_stride * 2;
  const int P = a.page_size;
  const uint32_t ps_bytes = static_cast<uint32_t>(a.page_stride) * 2;   // < 2^31 (checked on the host)
  const uint32_t ts_bytes = static_cast<uint32_t>(a.token_stride) * 2;
  const int page0 = uni(a.kv_indptr[b]);
  const int npages = uni(a.kv_indptr[b + 1]) - page0;
  const __amdgpu_buffer_rsrc_t pt = make_rsrc(a.kv_indices + page0, 4u * static_cast<uint32_t>(npages));
  const int srow = lane >> 4, spos = lane & 15;
  // Global chunk fetched by this lane for load j (the inverse of the swizzle).
  auto k_chunk = [&](int j) { return spos ^ ((kRpw * wave + 4 * j + srow) & 15); };
  const int v_chunk = spos ^ (4 * srow);
  auto lds_dst = [&](char* tile_base, int j) -> lds_void* {
    return (lds_void*)(tile_base + (kRpw * wave + 4 * j) * kRowBytes);
  };

  // Page-uniform mode (page_size a power of two >= 16): page index (in the
  // request) of the wave's kRpw-token group of tile ti. Item starts are page
  // aligned, so a group never straddles a page; the token is clamped into the
  // item, so the index is in range.
  const int pshift = __builtin_ctz(static_cast<unsigned>(P));
  auto group_page = [&](int ti) -> int {
    const int tc = min(k0 + ti * KT + kRpw * wave, k1 - 1);
    return tc >> pshift;
  };
  // Generic mode: the lane's token for load j of tile ti (clamped likewise).
  auto lane_token = [&](int ti, int j) -> int {
    return min(k0 + ti * KT + kRpw * wave + 4 * j + srow, k1 - 1);
  };

  // Page ids of one tile's loads, fetched two iterations before they are
  // used: vector-memory loads complete in issue order, so a consumer of an id
  // waits for every load issued before it, and two iterations is when the
  // tile loads issued just before it are due anyway. Uniform mode: the group's
  // id (wave-uniform); generic mode: the ids of the lane's kLpw tokens. Loads
  // past the page list read zero (the descriptor's range).
  struct Pids { int p[2]; };
  auto fetch_pids = [&](int ti) -> Pids {
    Pids r;
    if constexpr (MODE == kPagedUniform) {
      r.p[0] = __builtin_amdgcn_raw_buffer_load_b32(pt, 0, 4u * group_page(ti), 0);
      r.p[1] = 0;
    } else {
#pragma unroll
      for (int j = 0; j < kLpw; ++j)
        r.p[j] = __builtin_amdgcn_raw_buffer_load_b32(pt, 4u * (lane_token(ti, j) / P), 0, 0);
    }
    return r;
  };
  // Where the wave's group of a tile sits in the pool (uniform mode): its
  // byte offset from the K / V base and its number of valid bytes (tokens
  // past the item read as zero). K and V of a tile share it.
  struct Group { uint64_t off; uint32_t nbytes; };
  auto group_of = [&](int ti, const Pids& pid) -> Group {
    const int t = k0 + ti * KT + kRpw * wave;
    const uint32_t id = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(pid.p[0]));
    const uint32_t sl = static_cast<uint32_t>(min(t, k1 - 1) & (P - 1));
    // clamp(k1 - t, 0, kRpw): wave-uniform (readfirstlane: the compiler forms
    // the clamp with a vector med3)
    const uint32_t nvalid = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(max(0, min(kRpw, k1 - t))));
    return {static_cast<uint64_t>(id) * ps_bytes + sl * ts_bytes, nvalid * ts_bytes};
  };
  auto issue_group = [&](const Group& gr, const char* base, char* dst, bool is_k) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + gr.off, gr.nbytes);
#pragma unroll
    for (int j = 0; j < kLpw; ++j) {
      const uint32_t row = static_cast<uint32_t>(4 * j + srow) * ts_bytes;
      buffer_to_lds_16B(r, lds_dst(dst, j), row + 16 * (is_k ? k_chunk(j) : v_chunk));
    }
  };
  // Loads K (is_k) or V of tile ti into dst.
  auto issue = [&](int ti, const Pids& pid, const char* base, char* dst, bool is_k) {
    if constexpr (MODE == kPagedUniform) {
      issue_group(group_of(ti, pid), base, dst, is_k);
    } else {
#pragma unroll
      for (int j = 0; j < kLpw; ++j) {
        const int tc = lane_token(ti, j);
        const int sl = tc - (tc / P) * P;
        const uint64_t off = static_cast<uint64_t>(static_cast<uint32_t>(pid.p[j])) * ps_bytes + sl * ts_bytes;
        global_to_lds_16B(base + off + 16 * (is_k ? k_chunk(j) : v_chunk), lds_dst(dst, j));
      }
    }
  };

  // Row state (one per block). The exponent reference m_ref (log2 domain,
  // scaled) is the row maximum seen so far up to the lazy slack; weights are
  // exp2(scale_log2 * s - m_ref) rounded once to the storage dtype, and the
  // normalisation of O uses the sum of those rounded weights (O is then an
  // exact convex combination of V rows). The LSE needs the sum of the
  // unrounded weights when the rounding is coarse: one bf16 rounding is off by
  // up to 2^-8 relative, ln(1 + 2^-8) = 3.9e-3 in the LSE for a row with few
  // keys, so bf16 keeps a second, fp32 sum; fp16's 2^-11 (4.9e-4) uses the
  // rounded sum for both.
  float m_ref[RB], neg_m[RB], thr[RB], l_run[RB], l_lse[RB];
  // neg_m: -m_ref, or 0 while m_ref = -inf. thr: the raw-score threshold
  // (m_ref + slack) / scale_log2: a tile needs the rescale path only if some
  // lane holds a score above it (any rounding in it only moves the point at
  // which the reference is refreshed). l_run / l_lse: this lane's share of the
  // row's rounded / unrounded weight sum.
  const float inv_scale_log2 = 1.f / a.scale_log2;
  constexpr bool kExactLse = std::is_same_v<T, BF16>;
  f32x16 acc[RB][4];          // acc[rb][mb][i]: row lr of block rb, d = 32mb + 8(i/4) + 4*half + i%4
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_ref[rb] = neg_inf();
    neg_m[rb] = 0.f;
    thr[rb] = neg_inf();
    l_run[rb] = 0.f;
    l_lse[rb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rb][mb][i] = 0.f;
  }

  const int ntiles = (k1 - k0 + KT - 1) / KT;

  // Operand addresses. Both swizzles only permute 16-byte chunks inside a
  // row, so every read address of a tile is one per-lane base XOR a constant:
  //  * K (A operand of S^T): row lr, chunk 2kk + half, stored at chunk
  //    (2kk + half) ^ (lr & 15): byte lr*256 + 16*(half ^ (lr & 15)), XOR 32kk.
  //  * V (A operand of O^T, transposing read): 16-lane group q16 = lane/16
  //    reads row 16st + 4*half + vq (+8 for the second read), vq = (lane/4)&3,
  //    at d = 32mb + 16(q16 & 1) + 4(lane & 3): chunk 4mb + vchunk_lo stored
  //    at chunk (4mb + vchunk_lo) ^ 4vq: byte (4*half + vq)*256 +
  //    16*vchunk_lo + 8*(lane & 1) + 64*vq, XOR 64mb, plus 4096st (+2048).
  // The twelve per-lane offsets live in registers; a buffer's base (and the
  // 16-token step, +4096, and the +8 rows, +2048, of the V reads) is the
  // instruction's immediate offset.
  const int k_lane = lr * kRowBytes + 16 * (half ^ (lr & 15));
  const int vq = (lane >> 2) & 3;
  const int vchunk_lo = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int v_lane = (4 * half + vq) * kRowBytes + 16 * vchunk_lo + 8 * (lane & 1) + 64 * vq;
  int ka[8], va[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) ka[kk] = k_lane ^ (32 * kk);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) va[mb] = v_lane ^ (64 * mb);

  // S^T of one tile for every block: K rows are the A operand (LDS, one read
  // per step for all blocks), q^T the B operand.
  auto qk = [&](const char* kt, f32x16 (&s)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[rb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4 kf = *reinterpret_cast<const u32x4*>(kt + ka[kk]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb] = T::mfma_32x32x16(kf, qv[rb][kk], s[rb]);
    }
  };
  // Masks tile ti's scores where the tile reaches past k1 or past the row's
  // causal limit (wave-uniform test; one compare and select per score).
  auto mask = [&](int ti, f32x16 (&s)[RB]) {
    const int tb = k0 + ti * KT;
    if constexpr (VAR) {
      if (capped) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) s[rb][i] = soft_cap(s[rb][i], a.var.cap_in, a.var.cap_out);
      }
      if (tb + KT - 1 > mask_from || tb < win_from) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int tlast = (a.causal ? min(k1 - 1, lim[rb]) : k1 - 1) - (tb + 4 * half);
          const int tfirst = wlo[rb] - (tb + 4 * half);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = 8 * (i >> 2) + (i & 3);
            if (off > tlast || off < tfirst) s[rb][i] = neg_inf();
          }
        }
      }
    } else if (tb + KT - 1 > mask_from) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int tlast = (a.causal ? min(k1 - 1, lim[rb]) : k1 - 1) - (tb + 4 * half);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + (i & 3) > tlast) s[rb][i] = neg_inf();
      }
    }
  };
  // Largest raw score this lane holds of a tile (half of its row's keys).
  auto lane_max = [&](const f32x16& s) -> float {
    float t = neg_inf();
#pragma unroll
    for (int i = 0; i < 16; ++i) t = fmaxf(t, s[i]);
    return t;
  };
  // Moves block rb's reference where some lane's scores outgrew the threshold
  // (wave-uniform branch): every row takes its full maximum over both halves,
  // and O and the sums are rescaled by the same factor.
  auto maybe_rescale = [&](int rb, float lmax) {
    if (__builtin_amdgcn_ballot_w64(lmax > thr[rb]) != 0) {
      const float m_new = fmaxf(m_ref[rb], max_across_halves(lmax) * a.scale_log2);
      const float alpha = (m_new == neg_inf()) ? 1.f : fast_exp2(m_ref[rb] - m_new);
      m_ref[rb] = m_new;
      neg_m[rb] = (m_new == neg_inf()) ? 0.f : -m_new;
      thr[rb] = (m_new == neg_inf()) ? neg_inf() : (m_new + kRescaleSlack) * inv_scale_log2;
      l_run[rb] *= alpha;
      if constexpr (kExactLse) l_lse[rb] *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[rb][mb] *= alpha;
    }
  };
  // The two halves of a pipelined iteration. The instruction order is written
  // out: each step issues an LDS read two MFMA steps ahead of its use, one MFMA
  // per block, and a slice of the VALU work of the other tile, and a
  // scheduling fence (sched_barrier) keeps the compiler from regrouping the
  // steps.
  auto k_read = [&](const char* kt, int kk) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(kt + ka[kk]);
  };
  auto v_read = [&](const char* vt, int i) -> u32x4 {   // step i = (st, mb) = (i/4, i%4)
    const char* p = vt + 4096 * (i >> 2) + va[i & 3];
    const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16_b64(p));
    const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16_b64(p + 8 * kRowBytes));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // S(j+1) (8 MFMA steps over d) with the weights of tile j, one pair of
  // scores per block and step; kf[0..1] hold the first two K operands on
  // entry. The last two steps read the first two V operands of the PV product
  // into vf[0..1]. The weight work is skewed over three steps so that no
  // instruction waits for a result of its own step: step kk takes the
  // exponentials of pair kk (arguments formed one step earlier), forms the
  // arguments of pair kk+1, and packs and sums pair kk-1. The empty asm
  // statements keep the sums in their step (otherwise the compiler sinks them
  // into one dependent chain in front of the PV product).
  auto qk_weights = [&](const char* kt, u32x4 (&kf)[3], f32x16 (&s)[RB], const f32x16 (&sc)[RB],
                        u32x4 (&pk)[RB][2], const char* vt, u32x4 (&vf)[3]) {
    float sum[RB], xsum[RB], a0[RB], a1[RB], x0p[RB], x1p[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      sum[rb] = l_run[rb];
      xsum[rb] = l_lse[rb];
      a0[rb] = fmaf(sc[rb][0], a.scale_log2, neg_m[rb]);
      a1[rb] = fmaf(sc[rb][1], a.scale_log2, neg_m[rb]);
      x0p[rb] = x1p[rb] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      if (kk + 2 < 8) kf[(kk + 2) % 3] = k_read(kt, kk + 2);
      else vf[kk - 6] = v_read(vt, kk - 6);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        s[rb] = T::mfma_32x32x16(kf[kk % 3], qv[rb][kk], kk == 0 ? f32x16{} : s[rb]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float x0 = fast_exp2(a0[rb]), x1 = fast_exp2(a1[rb]);
        if (kk + 1 < 8) {
          a0[rb] = fmaf(sc[rb][2 * kk + 2], a.scale_log2, neg_m[rb]);
          a1[rb] = fmaf(sc[rb][2 * kk + 3], a.scale_log2, neg_m[rb]);
        }
        if (kk > 0) {
          pk[rb][(kk - 1) >> 2][(kk - 1) & 3] = T::pack2(x0p[rb], x1p[rb]);
          sum[rb] = T::add_pair(pk[rb][(kk - 1) >> 2][(kk - 1) & 3], sum[rb]);
          if constexpr (kExactLse) xsum[rb] += x0p[rb] + x1p[rb];
          asm volatile("" : "+v"(sum[rb]));
          if constexpr (kExactLse) asm volatile("" : "+v"(xsum[rb]));
        }
        x0p[rb] = x0;
        x1p[rb] = x1;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      pk[rb][1][3] = T::pack2(x0p[rb], x1p[rb]);
      sum[rb] = T::add_pair(pk[rb][1][3], sum[rb]);
      if constexpr (kExactLse) xsum[rb] += x0p[rb] + x1p[rb];
      l_run[rb] = sum[rb];
      l_lse[rb] = xsum[rb];
    }
  };
  // PV of tile j (8 MFMA steps) with the lane maxima of tile j+1's scores, one
  // pair per block and step; leaves the lane maxima (raw scores) in t.
  auto pv_max = [&](const char* vt, u32x4 (&vf)[3], const u32x4 (&pk)[RB][2],
                    const f32x16 (&sn)[RB], float (&t)[RB], auto&& hook) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) t[rb] = neg_inf();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i + 2 < 8) vf[(i + 2) % 3] = v_read(vt, i + 2);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][i & 3] = T::mfma_32x32x16(vf[i % 3], pk[rb][i >> 2], acc[rb][i & 3]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        t[rb] = fmaxf(fmaxf(t[rb], sn[rb][2 * i]), sn[rb][2 * i + 1]);
        asm volatile("" : "+v"(t[rb]));   // likewise for the running maxima
      }
      if (i == 4) hook();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Software pipeline over KV tiles. Iteration j: the loads of K(j+4) and
  // V(j+3) are issued; the MFMA units compute S(j+1) while the VALU forms the
  // weights of tile j; then the PV product of tile j runs while the VALU takes
  // tile j+1's row maxima. The iteration ends by waiting for the loads of
  // K(j+2) and V(j+1) (issued two iterations earlier; the last two
  // iterations' loads stay in flight) and one barrier. A buffer is refilled
  // only in the iteration after the barrier that follows its last read.
  // Every iteration issues the same loads (tiles past the item read zero, or
  // repeat the last token in generic mode), so the wait counts are constants.
  // Loads per iteration and wave: page ids (one uniform id, or one per lane
  // token) and the kLpw loads of K and of V.
  constexpr int kLoadsPerIter = MODE == kPagedUniform ? 1 + 2 * kLpw : 3 * kLpw;
  // Page ids of the K loads of tiles j+4 and j+5 and of the V load of tile j+3.
  Pids pid_k0, pid_k1, pid_v;
  Group grp_v{0, 0};   // uniform mode: where the V load of tile j+3 reads
  Group grp_k{0, 0};   // uniform mode: where the K load of tile j+4 reads
  // `ph` is j % 4 as a compile-time constant, so buffer choices are constants.
  auto body = [&](int j, auto ph, f32x16 (&s_cur)[RB], f32x16 (&s_nxt)[RB]) {
    constexpr int p = decltype(ph)::value;
    char* kn = kbuf(std::integral_constant<int, p>{});                  // receives K(j+4)
    char* vn = vbuf(std::integral_constant<int, (p + 3) & 3>{});        // receives V(j+3)
    const char* kt = kbuf(std::integral_constant<int, (p + 1) & 3>{});  // holds K(j+1)
    const char* vt = vbuf(std::integral_constant<int, p>{});            // holds V(j)
    u32x4 kf[3], vf[3];
    // The first K operands land while the loads below are issued.
    kf[0] = k_read(kt, 0);
    kf[1] = k_read(kt, 1);
    __builtin_amdgcn_sched_barrier(0);
    const Pids pnn = fetch_pids(j + 6);
    if constexpr (MODE == kPagedUniform) {
      issue_group(grp_k, kbase, kn, true);
      issue_group(grp_v, vbase, vn, false);
      grp_v = grp_k;
    } else {
      issue(j + 4, pid_k0, kbase, kn, true);
      issue(j + 3, pid_v, vbase, vn, false);
      pid_v = pid_k0;
    }
    pid_k0 = pid_k1;
    pid_k1 = pnn;

    u32x4 pk[RB][2];
    qk_weights(kt, kf, s_nxt, s_cur, pk, vt, vf);
    // The weights are complete here (kept from sinking past the branch).
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) asm volatile("" ::"v"(pk[rb][0]), "v"(pk[rb][1]));
    mask(j + 1, s_nxt);
    float t[RB];
    // The next iteration's K group is formed among the PV MFMAs, so that its
    // scalar address arithmetic is off the path to the next tile's loads.
    pv_max(vt, vf, pk, s_nxt, t, [&] {
      if constexpr (MODE == kPagedUniform) grp_k = group_of(j + 5, pid_k0);
    });
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) maybe_rescale(rb, t[rb]);
    wait_vm<2 * kLoadsPerIter>();
    lds_barrier();
  };

  if (ntiles > 0) {
    // Issue order: every tile the end-of-iteration wait of iteration j must
    // cover (K(j+2), V(j+1)) has at least 2 * kLoadsPerIter loads issued
    // after it by then, as in the steady state: iteration 0 needs K(2) and
    // V(1), followed here by p5, K(3), V(2) (kLoadsPerIter loads) and by
    // iteration 0's own kLoadsPerIter. The two page-id fetches sit between
    // the tile loads to make up that count.
    const Pids p0 = fetch_pids(0), p1 = fetch_pids(1), p2 = fetch_pids(2), p3 = fetch_pids(3);
    issue(0, p0, kbase, sK0, true);
    issue(0, p0, vbase, sV0, false);
    issue(1, p1, kbase, sK1, true);
    pid_k0 = fetch_pids(4);
    issue(2, p2, kbase, sK2, true);
    issue(1, p1, vbase, sV1, false);
    pid_k1 = fetch_pids(5);
    issue(3, p3, kbase, sK3, true);
    issue(2, p2, vbase, sV2, false);
    pid_v = p3;
    if constexpr (MODE == kPagedUniform) {
      grp_v = group_of(3, p3);
      grp_k = group_of(4, pid_k0);
    }
    // K(0), V(0) and K(1) have landed (2 * kLoadsPerIter loads follow K(1));
    // p4, K(2), V(1), p5, K(3), V(2) may still be in flight.
    wait_vm<2 * kLoadsPerIter>();
    lds_barrier();

    f32x16 sA[RB], sB[RB];
    qk(sK0, sA);
    mask(0, sA);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) maybe_rescale(rb, lane_max(sA[rb]));
    // Every wave has read K(0) before iteration 0 refills its buffer.
    lds_barrier();
    constexpr std::integral_constant<int, 0> ph0{};
    constexpr std::integral_constant<int, 1> ph1{};
    constexpr std::integral_constant<int, 2> ph2{};
    constexpr std::integral_constant<int, 3> ph3{};
    // Every tile runs the same body, the last one included: its "next" tile
    // lies past the item (its K buffer holds zeros or repeated rows, already
    // waited for like any other), every score of it is masked to -inf, so it
    // moves no reference and its scores are dropped when the loop ends.
    for (int j = 0;; j += 4) {
      body(j, ph0, sA, sB);
      if (j + 1 == ntiles) break;
      body(j + 1, ph1, sB, sA);
      if (j + 2 == ntiles) break;
      body(j + 2, ph2, sA, sB);
      if (j + 3 == ntiles) break;
      body(j + 3, ph3, sB, sA);
      if (j + 4 == ntiles) break;
    }
  }

  // Finalize each block's row lr.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l_tot = sum_across_halves(l_run[rb]);
    float l_ex = kExactLse ? sum_across_halves(l_lse[rb]) : l_tot;
    if (!row_ok[rb]) continue;
    float m_fin = m_ref[rb];
    float o_scale = 1.f;   // factor on the accumulator besides 1 / l_tot
    if constexpr (VAR) {
      // The head's sink (log2 domain) is one more term of both sums, with a
      // zero value: move the reference to the larger of the two and add it.
      if (a.var.sinks != nullptr && slot < 0) {
        const float sink = a.var.sinks[head[rb]] * kLog2e;
        const float m_new = fmaxf(m_fin, sink);
        if (m_new != neg_inf()) {
          o_scale = fast_exp2(m_fin - m_new);
          const float w_sink = fast_exp2(sink - m_new);
          l_tot = l_tot * o_scale + w_sink;
          l_ex = l_ex * o_scale + w_sink;
          m_fin = m_new;
        }
      }
    }
    const float inv = l_tot > 0.f ? o_scale * __builtin_amdgcn_rcpf(l_tot) : 0.f;
    if (slot < 0) {
      const float lse = l_ex > 0.f ? (m_fin + fast_log2(l_ex)) * kLn2 : neg_inf();
      const int64_t orow = static_cast<int64_t>(q0 + qtok[rb]) * a.num_qo_heads + head[rb];
      OUT* o = static_cast<OUT*>(a.o) + orow * D;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * mb + 8 * q4 + 4 * half;
          store4<OUT>(o + d, acc[rb][mb][4 * q4] * inv, acc[rb][mb][4 * q4 + 1] * inv,
                      acc[rb][mb][4 * q4 + 2] * inv, acc[rb][mb][4 * q4 + 3] * inv);
        }
      if (half == 0 && a.lse != nullptr) a.lse[orow] = lse;
    } else {
      const int64_t srow_out = static_cast<int64_t>(slot) * kRows + 32 * RB * wave + 32 * rb + lr;
      float* po = a.part_o + srow_out * D;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = 32 * mb + 8 * q4 + 4 * half;
          *reinterpret_cast<f32x4*>(po + d) =
              f32x4{acc[rb][mb][4 * q4] * inv, acc[rb][mb][4 * q4 + 1] * inv,
                    acc[rb][mb][4 * q4 + 2] * inv, acc[rb][mb][4 * q4 + 3] * inv};
        }
      // The chunk's (m, l): its exponent reference and the (unrounded) weight sum.
      if (half == 0) *reinterpret_cast<f32x2*>(a.part_ml + 2 * srow_out) = f32x2{m_fin, l_ex};
    }
  }
}

}  // namespace

}  // namespace pkv
