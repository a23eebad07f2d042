// Kernel-argument block and the work-list decoding shared by the host planner and
// the kernels. The work list of a pass is a sequence of items (b, h, tile); only tiles
// that hold at least one valid row are listed, so fully padded tiles are never
// computed (block-sparse padding, section 4 of the sigmoid-attention paper).
//
// Order: batch entries sorted by decreasing valid length (longest work first); within
// an entry, bidirectional passes list head-major (all tiles of one head together, so
// K/V of that head stays hot in one L2) and causal passes list tile-major with the
// most expensive tiles first. A blockIdx -> item remap then gives each XCD a
// contiguous chunk of items per round, so that the tiles sharing one head's K/V run on
// the same XCD and its L2.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define SA_HD __host__ __device__
#else
#define SA_HD
#endif

namespace sa {

constexpr int kMaxBatch = 256;
constexpr int kNumXcd = 8;

struct KArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* out0;            // o (fwd), dq (dq pass), dk (dk/dv pass)
  void* out1;            // dv (dk/dv pass)
  float* aux;            // per-head float plane [B][H][Lmax] or null: dg (dk/dv pass),
                         // row mass (forward)
  const float* gate;     // [B][gsb] device floats or null
  int64_t sb, sh, sl;    // element strides of the 4-D tensors
  int64_t gsb;           // gate batch stride (elements)
  int32_t H;
  int32_t Lmax;
  int32_t nitems;        // compute items in the launch
  int32_t nsorted;       // batch entries with n > 0
  int32_t tile;          // rows per item (queries for fwd/dq, keys for dk/dv)
  int32_t xcd_chunk;     // items per XCD per round; 0 disables the remap
  int32_t causal;
  int32_t reverse;       // list tiles last-first (causal query-side passes)
  int32_t gate_sink;
  int32_t out_f32;       // outputs are float (else bf16)
  float c1;              // -s * log2(e): logit scale folded into the exp2 argument
  float scale;           // s
  float gate_eps;
  float gate_tau;
  int32_t off[kMaxBatch + 1];  // prefix item counts by sorted position
  float c2[kMaxBatch];         // -beta * log2(e) by sorted position
  uint16_t len[kMaxBatch];     // valid length by sorted position
  uint8_t bidx[kMaxBatch];     // batch index by sorted position
};

struct Item {
  int b;      // batch index
  int h;      // head
  int t;      // tile index (rows t*tile .. t*tile+tile-1)
  int n;      // valid length of batch entry b
  float c2;   // -beta_b * log2(e)
};

// blockIdx -> item index. Rounds of kNumXcd*chunk items; in each round XCD x (which
// receives blocks w with w % 8 == x) takes the contiguous items [x*chunk, x*chunk+chunk).
// Bijective; blocks past the last full round map to themselves.
SA_HD inline int remap_block(int w, int nitems, int chunk) {
  if (chunk <= 0) return w;
  const int round = kNumXcd * chunk;
  const int full = (nitems / round) * round;
  if (w >= full) return w;
  const int x = w % kNumXcd;
  const int s = w / kNumXcd;
  return (s / chunk) * round + x * chunk + (s % chunk);
}

SA_HD inline Item decode_item(const KArgs& a, int g) {
  // largest p with off[p] <= g (off is non-decreasing, off[0] = 0)
  int lo = 0, hi = a.nsorted - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.off[mid] <= g) lo = mid; else hi = mid - 1;
  }
  Item it;
  const int p = lo;
  it.b = a.bidx[p];
  it.n = a.len[p];
  it.c2 = a.c2[p];
  const int T = (it.n + a.tile - 1) / a.tile;
  const int local = g - a.off[p];
  if (a.causal) {
    it.h = local % a.H;
    it.t = local / a.H;
  } else {
    it.h = local / T;
    it.t = local % T;
  }
  if (a.reverse) it.t = T - 1 - it.t;
  return it;
}

}  // namespace sa
