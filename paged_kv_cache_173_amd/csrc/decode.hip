// Paged decode kernel for gfx950: one work item (request, KV head, token
// range) per workgroup; the item's computation is decode_item (decode_item.h).
#include <hip/hip_ext.h>

#include "decode_item.h"

namespace pkv {

namespace {

template <class T, class OUT, int MODE, bool VAR>
__global__ __launch_bounds__(256, 3) void decode_kernel(const DecodeArgs a) {
  __shared__ float s_m[kDecodeWaves * 16];
  __shared__ float s_l[kDecodeWaves * 16];
  __shared__ __attribute__((aligned(16))) float s_acc[kDecodeWaves][16 * kHeadDim];
  int b, g, t0, t1, slot;
  if (a.items != nullptr) {
    const int32_t* it = a.items + 8 * blockIdx.x;
    b = it[0];
    g = it[1];
    t0 = it[5];
    t1 = it[6];
    slot = it[7];
  } else {
    const int n = a.implicit_nchunks;
    g = blockIdx.x / n;
    const int j = blockIdx.x - g * n;
    b = 0;
    t0 = j * a.implicit_chunk_tokens;
    t1 = min(t0 + a.implicit_chunk_tokens, a.implicit_kv_len);
    slot = n > 1 ? static_cast<int>(blockIdx.x) : -1;
  }

  decode_item<T, OUT, MODE, VAR>(a, b, g, t0, t1, slot,
                                 DecodeLds{s_m, s_l, {s_acc[0], s_acc[1], s_acc[2], s_acc[3]}});
}

template <class T, class OUT>
hipError_t launch_decode_t(const DecodeArgs& a, PageMode mode, int32_t grid, hipStream_t s,
                           const LaunchEvents& ev) {
  if (variant_on(a.var)) {
    if (mode == kContiguous) return hipErrorInvalidValue;
    if (mode == kPagedUniform)
      hipExtLaunchKernelGGL((decode_kernel<T, OUT, kPagedUniform, true>), dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
    else
      hipExtLaunchKernelGGL((decode_kernel<T, OUT, kPagedGeneric, true>), dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
    return hipGetLastError();
  }
  switch (mode) {
    case kContiguous:
      hipExtLaunchKernelGGL((decode_kernel<T, OUT, kContiguous, false>), dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
      break;
    case kPagedUniform:
      hipExtLaunchKernelGGL((decode_kernel<T, OUT, kPagedUniform, false>), dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
      break;
    default:
      hipExtLaunchKernelGGL((decode_kernel<T, OUT, kPagedGeneric, false>), dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

int32_t decode_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&decode_kernel<F16, _Float16, kPagedUniform, false>), 256,
          0) != hipSuccess)
    return 0;
  return n;
}

hipError_t launch_decode(const DecodeArgs& a, int32_t storage_dtype, OutKind out, PageMode mode,
                         int32_t grid, hipStream_t stream, const LaunchEvents& ev) {
  if (grid <= 0) return hipSuccess;
  if (storage_dtype == 0) {
    return out == kOutF32 ? launch_decode_t<F16, float>(a, mode, grid, stream, ev)
                          : launch_decode_t<F16, _Float16>(a, mode, grid, stream, ev);
  }
  return out == kOutF32 ? launch_decode_t<BF16, float>(a, mode, grid, stream, ev)
                        : launch_decode_t<BF16, __bf16>(a, mode, grid, stream, ev);
}

}  // namespace pkv
