// dK/dV kernel (launch of the pass body in dkdv_body.h over the work list).
#include "dkdv_body.h"

namespace sa {

template <int D, int CPT, bool CAUSAL, bool GATED, bool SPLIT, bool DG, bool VL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1)))
void dkdv_kernel(const KArgs a) {
  using T = DkvTraits<D, CPT>;
  __shared__ __attribute__((aligned(1024))) char smem[T::NSTAGE * T::STAGE];
  const Item it = block_item<VL>(a);
  if (VL && !it.valid) return;
  dkdv_body<D, CPT, CAUSAL, GATED, SPLIT, DG, VL>(a, it, smem, a.out0, a.out1);
}

template <int D, int CPT, bool C, bool G, bool SP, bool DG = false>
static hipError_t launch_one(const KArgs& a, hipStream_t st) {
  if (a.varlen)
    hipLaunchKernelGGL((dkdv_kernel<D, CPT, C, G, SP, false, true>), dim3(a.nitems), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((dkdv_kernel<D, CPT, C, G, SP, DG, false>), dim3(a.nitems), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int CPT>
static hipError_t dispatch(const KArgs& a, bool c, bool g, bool sp, hipStream_t st) {
  if (a.aux) {   // gate gradient (gated only)
    if (c) return sp ? launch_one<D, CPT, true, true, true, true>(a, st) : launch_one<D, CPT, true, true, false, true>(a, st);
    return sp ? launch_one<D, CPT, false, true, true, true>(a, st) : launch_one<D, CPT, false, true, false, true>(a, st);
  }
  if (c) {
    if (g) return sp ? launch_one<D, CPT, true, true, true>(a, st) : launch_one<D, CPT, true, true, false>(a, st);
    return sp ? launch_one<D, CPT, true, false, true>(a, st) : launch_one<D, CPT, true, false, false>(a, st);
  }
  if (g) return sp ? launch_one<D, CPT, false, true, true>(a, st) : launch_one<D, CPT, false, true, false>(a, st);
  return sp ? launch_one<D, CPT, false, false, true>(a, st) : launch_one<D, CPT, false, false, false>(a, st);
}

int dkdv_tile_rows(int d) { return d == 64 ? DkvTraits<64, 2>::BK : DkvTraits<128, 1>::BK; }

// At d = 128 the query tiles of the LDS ring hold 32 rows (three stages, 48 KB) for short
// sequences and 64 rows (96 KB; the workgroup is alone on its CU at one wave per SIMD)
// from kLongRows query rows on: half the barriers and ring waits per query, measured 2-5 %
// faster from 4096 rows, 1.5 % slower at 512. The arithmetic, and so the result, is the
// same either way.
constexpr int kLongRows = 1024;

hipError_t launch_dkdv_bf16(const KArgs& a, int d, bool causal, bool gated, bool split,
                            hipStream_t st) {
  if (d == 64) return dispatch<64, 2>(a, causal, gated, split, st);
  const int rows_q = a.varlen ? a.Lmax : (a.nsorted > 0 ? len_at(a, 0) : 0);
  return rows_q >= kLongRows ? dispatch<128, 2>(a, causal, gated, split, st)
                             : dispatch<128, 1>(a, causal, gated, split, st);
}

}  // namespace sa
