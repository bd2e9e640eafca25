// Paged prefill / append kernel for gfx950: one work item (request, KV head,
// 128-row query tile, token range) per workgroup; the item's computation is
// prefill_item (prefill_item.h).
#include <hip/hip_ext.h>

#include "prefill_item.h"

namespace pkv {

namespace {

template <class T, class OUT, int MODE, bool VAR>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const PrefillArgs a) {
  prefill_item<T, OUT, MODE, VAR, 1>(a, a.items + 8 * blockIdx.x);
}

template <class T, class OUT, bool VAR>
void launch_prefill_mode(const PrefillArgs& a, PageMode mode, int32_t grid, hipStream_t s,
                         const LaunchEvents& ev) {
  if (mode == kPagedUniform) {
    hipExtLaunchKernelGGL((prefill_kernel<T, OUT, kPagedUniform, VAR>), dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
  } else {
    hipExtLaunchKernelGGL((prefill_kernel<T, OUT, kPagedGeneric, VAR>), dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
  }
}

template <class T, class OUT>
hipError_t launch_prefill_t(const PrefillArgs& a, PageMode mode, int32_t grid, hipStream_t s,
                            const LaunchEvents& ev) {
  // The uniform kernel locates pages with shifts: other page sizes use the
  // per-token lookups of the generic kernel.
  if (mode == kPagedUniform && (a.page_size & (a.page_size - 1)) != 0) mode = kPagedGeneric;
  if (variant_on(a.var))
    launch_prefill_mode<T, OUT, true>(a, mode, grid, s, ev);
  else
    launch_prefill_mode<T, OUT, false>(a, mode, grid, s, ev);
  return hipGetLastError();
}

}  // namespace

int32_t prefill_occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&prefill_kernel<BF16, __bf16, kPagedUniform, false>), 256,
          0) != hipSuccess)
    return 0;
  return n;
}

hipError_t launch_prefill(const PrefillArgs& a, int32_t storage_dtype, OutKind out,
                          PageMode mode, int32_t grid, hipStream_t stream,
                          const LaunchEvents& ev) {
  if (grid <= 0) return hipSuccess;
  if (a.rows_per_tile != kTileRows) return hipErrorInvalidValue;
  if (storage_dtype == 0) {
    return out == kOutF32 ? launch_prefill_t<F16, float>(a, mode, grid, stream, ev)
                          : launch_prefill_t<F16, _Float16>(a, mode, grid, stream, ev);
  }
  return out == kOutF32 ? launch_prefill_t<BF16, float>(a, mode, grid, stream, ev)
                        : launch_prefill_t<BF16, __bf16>(a, mode, grid, stream, ev);
}

}  // namespace pkv
