// Appending new K/V rows into a paged cache for gfx950.
//
// What it computes: appended row n names its request b = batch_indices[n] and
// its position t = positions[n] in that request; the page table already
// describes the cache after the append, so token t of request b lives in page
// kv_indices[kv_indptr[b] + t / P] at slot t % P (NHD page memory
// [page, slot, kv_head, d]). Row n of the appended K and V is copied there,
// for every KV head, and nothing else is written (docs index "flashinfer.page"
// > "Append new K/V tensors to Paged KV-Cache"; the page walk is the one of the
// FlashInfer article, section "Block-sparse cache representation", and of the
// docs index "KV-Cache Layout in FlashInfer" > "Page Table Layout").
//
// Rows whose request is outside [0, batch), whose position is outside the
// request's KV length, or whose page index falls past the request's pages are
// skipped (no write).
//
// Mapping: one wave per appended row; lane l moves 16 bytes of KV head
// 4i + l/16 (16 lanes cover one 256-byte head row), so every load and store is
// a fully used 1 KB wave access. HBM-bound: each row reads and writes
// Hkv * 128 * 2 bytes for K and the same for V.
#include "device_common.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kRowsPerBlock = 4;     // one wave per appended row

__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock +
                    __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (n >= a.nnz) return;
  const int b = a.batch_indices[n];
  const int t = a.positions[n];
  if (b < 0 || b >= a.batch || t < 0) return;
  const int p0 = a.kv_indptr[b];
  const int np = a.kv_indptr[b + 1] - p0;
  if (np <= 0) return;
  const int64_t len = static_cast<int64_t>(np - 1) * a.page_size + a.last_page_len[b];
  const int pi = t / a.page_size;
  if (t >= len || pi >= np) return;
  const int64_t page = a.kv_indices[p0 + pi];
  const int slot = t - pi * a.page_size;

  // Wave-uniform row bases; the lane's byte offsets inside the row are added
  // per head group.
  const int64_t dst = (page * a.page_stride + static_cast<int64_t>(slot) * a.token_stride) * 2;
  const int64_t src = n * a.append_stride * 2;
  const char* ak = static_cast<const char*>(a.append_k) + src;
  const char* av = static_cast<const char*>(a.append_v) + src;
  char* k = static_cast<char*>(a.k) + dst;
  char* v = static_cast<char*>(a.v) + dst;
  const int c = 16 * (lane & 15);             // byte offset of this lane's 16 bytes in a head row
  const int64_t hs = a.head_stride * 2;
  for (int h = lane >> 4; h < a.num_kv_heads; h += 4) {
    const u32x4 kx = load_16B(ak + h * (2 * kHeadDim) + c);
    const u32x4 vx = load_16B(av + h * (2 * kHeadDim) + c);
    *reinterpret_cast<u32x4*>(k + h * hs + c) = kx;
    *reinterpret_cast<u32x4*>(v + h * hs + c) = vx;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.nnz <= 0) return hipSuccess;
  const int64_t grid = (a.nnz + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
