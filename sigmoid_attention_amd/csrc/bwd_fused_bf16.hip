// Both backward kernels in one launch (d = 64, padded or packed batches): the work list
// is the dK/dV pass's items followed by the dQ pass's items (for causal batches of one
// length, both passes' tile blocks merged by cost), each workgroup running the body of
// the pass its item belongs to. The bodies, their arithmetic and their outputs are those of the separate
// dQ and dK/dV kernels ("Better Models, Faster Training: Sigmoid Attention for
// single-cell Foundation Models", section 4: one kernel for dQ, one for dK/dV, no
// atomics); only the dispatch is shared, so the workgroups of one pass fill the slots
// the other pass's last, shorter items leave idle.
#include "dkdv_body.h"
#include "dq_body.h"

namespace sa {

// a: the dK/dV pass's plan (nitems dK/dV items); nq_items dQ items follow them, with
// tiles_q query tiles per (sequence, head) in packed mode (VL).
template <bool CAUSAL, bool GATED, bool SPLIT, bool VL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_kernel(const KArgs a, void* dq, int nq_items, int tiles_q) {
  using TQ = DqTraits<64, 2, GATED>;
  using TK = DkvTraits<64, 2>;
  constexpr int kBytesQ = TQ::NSTAGE * TQ::STAGE, kBytesK = TK::NSTAGE * TK::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[kBytesQ > kBytesK ? kBytesQ : kBytesK];
  const int g = remap_block(blockIdx.x, a.nitems + nq_items, a.xcd_chunk);
  bool dq_item = g >= a.nitems;
  Item it;
  if (CAUSAL && a.nblocks > 0) {                    // both passes' blocks, merged by cost
    it = VL ? varlen_block_item(a, g, &dq_item) : decode_block_item(a, g, &dq_item);
  } else if (!dq_item) {
    it = VL ? varlen_item(a, g, a.tiles_per_seq, 1) : decode_item(a, g, 0);
  } else {
    const int gq = g - a.nitems;
    it = VL ? varlen_item(a, gq, tiles_q, 0) : decode_item(a, gq, CAUSAL ? 1 : 0);
  }
  it = uniform_item(it);
  dq_item = __builtin_amdgcn_readfirstlane(dq_item ? 1 : 0) != 0;
  if (VL && !it.valid) return;
  if (!dq_item)
    dkdv_body<64, 2, CAUSAL, GATED, SPLIT, false, VL>(a, it, smem, a.out0, a.out1);
  else
    dq_body<64, 2, CAUSAL, GATED, SPLIT, VL>(a, it, smem, dq);
}

template <bool C, bool G, bool SP>
static hipError_t launch_one(const KArgs& a, void* dq, int nq_items, int tiles_q, hipStream_t st) {
  const dim3 grid(a.nitems + nq_items);
  if (a.varlen)
    hipLaunchKernelGGL((bwd_kernel<C, G, SP, true>), grid, dim3(256), 0, st, a, dq, nq_items, tiles_q);
  else
    hipLaunchKernelGGL((bwd_kernel<C, G, SP, false>), grid, dim3(256), 0, st, a, dq, nq_items, tiles_q);
  return hipGetLastError();
}

// a: the dK/dV pass's plan (out0 = dK, out1 = dV) at d = 64; the dQ pass uses the same
// 128-row tiles: in the padded layout its items mirror the dK/dV items (nq_items =
// a.nitems), in packed mode there are nq_items = B * H * tiles_q of them.
hipError_t launch_bwd_bf16(const KArgs& a, void* dq, int nq_items, int tiles_q, bool causal,
                           bool gated, bool split, hipStream_t st) {
  static_assert(DqTraits<64, 2, false>::BM == DkvTraits<64, 2>::BK, "tile rows differ");
  if (causal) {
    if (gated) return split ? launch_one<true, true, true>(a, dq, nq_items, tiles_q, st)
                            : launch_one<true, true, false>(a, dq, nq_items, tiles_q, st);
    return split ? launch_one<true, false, true>(a, dq, nq_items, tiles_q, st)
                 : launch_one<true, false, false>(a, dq, nq_items, tiles_q, st);
  }
  if (gated) return split ? launch_one<false, true, true>(a, dq, nq_items, tiles_q, st)
                          : launch_one<false, true, false>(a, dq, nq_items, tiles_q, st);
  return split ? launch_one<false, false, true>(a, dq, nq_items, tiles_q, st)
               : launch_one<false, false, false>(a, dq, nq_items, tiles_q, st);
}

}  // namespace sa
