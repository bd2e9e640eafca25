// Mixed prefill + decode in one launch for gfx950 (POD attention: prefill and
// decode of a mixed batch fused into one kernel; named in the page "FlashInfer:
// A Kernel Library That Puts Attention, GEMM, and MoE Behind One API", section
// "The Feature List: What Is Actually Covered", and in the docs index,
// "flashinfer.pod" > "PODWithPagedKVCacheWrapper").
//
// What it computes: exactly what a prefill run over the prefill requests and
// a decode run over the decode requests compute (the same items of the same
// plans, the same arithmetic: prefill_item and decode_item); only the launch
// is shared. Workgroup i runs entry order[i] of an interleaved table:
// order[i] >= 0 is prefill item order[i], order[i] < 0 is decode item
// -order[i] - 1.
//
// Why one launch on CDNA4: a prefill item keeps the MFMA units and LDS busy
// and reads little from HBM; a decode item streams K/V from HBM and does
// little arithmetic. Interleaving them in one grid puts both kinds on every
// CU at once, so the HBM traffic of the decode items hides under the MFMA
// time of the prefill items instead of following it. The kernel takes the
// prefill item's resources (256 VGPRs, 64 KB of LDS: two workgroups per CU);
// a decode item borrows the K tile buffers for its cross-wave merge
// (16 x 128 floats = 8 KB per wave, one buffer each) and a V buffer for the
// maxima and sums. No item uses both halves, so they never share LDS.
#include <hip/hip_ext.h>

#include "decode_item.h"
#include "prefill_item.h"

namespace pkv {

namespace {

template <class T, int MODE>
__global__ __launch_bounds__(256, 2) void pod_kernel(const PodArgs a) {
  using OUT = typename T::elem;
  const int e = a.order[blockIdx.x];
  if (e >= 0) {
    prefill_item<T, OUT, MODE, false, 1>(a.p, a.p.items + 8 * e);
  } else {
    const int32_t* it = a.d.items + 8 * (-e - 1);
    float* m = reinterpret_cast<float*>(sV0);
    decode_item<T, OUT, MODE, false>(
        a.d, it[0], it[1], it[5], it[6], it[7],
        DecodeLds{m, m + kDecodeWaves * 16,
                  {reinterpret_cast<float*>(sK0), reinterpret_cast<float*>(sK1),
                   reinterpret_cast<float*>(sK2), reinterpret_cast<float*>(sK3)}});
  }
}

static_assert(16 * kHeadDim * sizeof(float) <= kTileBytes, "a wave's merge rows fit one tile buffer");

template <class T>
hipError_t launch_pod_t(const PodArgs& a, PageMode mode, int32_t grid, hipStream_t s,
                        const LaunchEvents& ev) {
  // Like the prefill launcher: the uniform kernel needs a power-of-two page.
  if (mode == kPagedUniform && (a.p.page_size & (a.p.page_size - 1)) != 0) mode = kPagedGeneric;
  if (mode == kPagedUniform)
    hipExtLaunchKernelGGL((pod_kernel<T, kPagedUniform>), dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
  else
    hipExtLaunchKernelGGL((pod_kernel<T, kPagedGeneric>), dim3(grid), dim3(256), 0, s, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pod(const PodArgs& a, int32_t storage_dtype, PageMode mode, int32_t grid,
                      hipStream_t stream, const LaunchEvents& ev) {
  if (grid <= 0) return hipSuccess;
  if (mode == kContiguous) return hipErrorInvalidValue;
  return storage_dtype == 0 ? launch_pod_t<F16>(a, mode, grid, stream, ev)
                            : launch_pod_t<BF16>(a, mode, grid, stream, ev);
}

}  // namespace pkv
