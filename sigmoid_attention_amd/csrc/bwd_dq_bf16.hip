// dQ kernel (launch of the pass body in dq_body.h over the work list).
#include "dq_body.h"

namespace sa {

template <int D, int CPT, bool CAUSAL, bool GATED, bool SPLIT, bool VL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(const KArgs a) {
  using T = DqTraits<D, CPT, GATED>;
  __shared__ __attribute__((aligned(1024))) char smem[T::NSTAGE * T::STAGE];
  const Item it = block_item<VL>(a);
  if (VL && !it.valid) return;
  dq_body<D, CPT, CAUSAL, GATED, SPLIT, VL>(a, it, smem, a.out0);
}

template <int D, int CPT, bool C, bool G, bool SP>
static hipError_t launch_one(const KArgs& a, hipStream_t st) {
  if (a.varlen)
    hipLaunchKernelGGL((dq_kernel<D, CPT, C, G, SP, true>), dim3(a.nitems), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((dq_kernel<D, CPT, C, G, SP, false>), dim3(a.nitems), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int CPT>
static hipError_t dispatch(const KArgs& a, bool c, bool g, bool sp, hipStream_t st) {
  if (c) {
    if (g) return sp ? launch_one<D, CPT, true, true, true>(a, st) : launch_one<D, CPT, true, true, false>(a, st);
    return sp ? launch_one<D, CPT, true, false, true>(a, st) : launch_one<D, CPT, true, false, false>(a, st);
  }
  if (g) return sp ? launch_one<D, CPT, false, true, true>(a, st) : launch_one<D, CPT, false, true, false>(a, st);
  return sp ? launch_one<D, CPT, false, false, true>(a, st) : launch_one<D, CPT, false, false, false>(a, st);
}

int dq_tile_rows(int d) { return d == 64 ? DqTraits<64, 2, false>::BM : DqTraits<128, 1, false>::BM; }

hipError_t launch_dq_bf16(const KArgs& a, int d, bool causal, bool gated, bool split,
                          hipStream_t st) {
  return d == 64 ? dispatch<64, 2>(a, causal, gated, split, st)
                 : dispatch<128, 1>(a, causal, gated, split, st);
}

}  // namespace sa
