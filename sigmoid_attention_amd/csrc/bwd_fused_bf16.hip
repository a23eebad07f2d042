// Both backward kernels in one launch (d = 64): the work list is the dK/dV pass's items
// followed by the dQ pass's items, each workgroup running the body of the pass its item
// belongs to. The bodies, their arithmetic and their outputs are those of the separate
// dQ and dK/dV kernels ("Better Models, Faster Training: Sigmoid Attention for
// single-cell Foundation Models", section 4: one kernel for dQ, one for dK/dV, no
// atomics); only the dispatch is shared, so the workgroups of one pass fill the slots
// the other pass's last, shorter items leave idle.
#include "dkdv_body.h"
#include "dq_body.h"

namespace sa {

template <bool CAUSAL, bool GATED, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_kernel(const KArgs a, void* dq) {
  using TQ = DqTraits<64, 2, GATED>;
  using TK = DkvTraits<64, 2>;
  constexpr int kBytesQ = TQ::NSTAGE * TQ::STAGE, kBytesK = TK::NSTAGE * TK::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[kBytesQ > kBytesK ? kBytesQ : kBytesK];
  // both passes list the same sequences with the same number of 128-row tiles each
  const int g = remap_block(blockIdx.x, 2 * a.nitems, a.xcd_chunk);
  if (g < a.nitems) {
    const Item it = uniform_item(decode_item(a, g, 0));
    dkdv_body<64, 2, CAUSAL, GATED, SPLIT, false, false>(a, it, smem, a.out0, a.out1);
  } else {
    const Item it = uniform_item(decode_item(a, g - a.nitems, CAUSAL ? 1 : 0));
    dq_body<64, 2, CAUSAL, GATED, SPLIT, false>(a, it, smem, dq);
  }
}

template <bool C, bool G, bool SP>
static hipError_t launch_one(const KArgs& a, void* dq, hipStream_t st) {
  hipLaunchKernelGGL((bwd_kernel<C, G, SP>), dim3(2 * a.nitems), dim3(256), 0, st, a, dq);
  return hipGetLastError();
}

// a: the dK/dV pass's plan (out0 = dK, out1 = dV); requires d = 64 and equal tile rows
// for both passes.
hipError_t launch_bwd_bf16(const KArgs& a, void* dq, bool causal, bool gated, bool split,
                           hipStream_t st) {
  static_assert(DqTraits<64, 2, false>::BM == DkvTraits<64, 2>::BK, "tile rows differ");
  if (causal) {
    if (gated) return split ? launch_one<true, true, true>(a, dq, st) : launch_one<true, true, false>(a, dq, st);
    return split ? launch_one<true, false, true>(a, dq, st) : launch_one<true, false, false>(a, dq, st);
  }
  if (gated) return split ? launch_one<false, true, true>(a, dq, st) : launch_one<false, true, false>(a, dq, st);
  return split ? launch_one<false, false, true>(a, dq, st) : launch_one<false, false, false>(a, dq, st);
}

}  // namespace sa
