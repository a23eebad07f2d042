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
//
// Causal batches whose sequences all have one length (fixed-length training batches) are
// listed block-major instead: one block per tile index, holding that tile of every
// (sequence, head), the blocks in decreasing cost, so that list scheduling starts the
// longest items first across the whole batch and not only within each sequence. In the
// one-call backward the blocks of both passes are merged by cost. The XCD remap is off in
// this mode (blockIdx = item, or the snake placement of remap_block when one round of
// resident workgroups holds the list, which keeps each item's XCD): with a multiple of 8
// (sequence, head) pairs per block, every tile of one head then lands on the same XCD,
// XCD g mod 8. Packed causal batches use the same
// block-major order, with costs taken at the maximum lengths (the lengths themselves are
// on the device).
//
// Packed variable-length batches (device-side cu_seqlens) use a third mode: the grid is
// B x H x ceil(max_rows / tile) items in (b, h, tile) order with the tile fastest, each
// workgroup reads its sequence's bounds from device memory and exits at once when its
// tile starts past the sequence's rows. Query and key lengths may differ; the causal
// rule is then aligned at the bottom right (key j allowed for query i iff
// j <= i + nk - nq), which is what a query shard of a longer sequence needs.
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
constexpr int kMaxBlocks = 128;       // block-major lists: at most this many tile blocks
constexpr unsigned kDqBlock = 0x8000u;  // block code bit: a dQ block of the one-call list

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
  int32_t Lmax;          // padded length (packed mode: the longest query row count)
  int32_t nitems;        // compute items in the launch
  int32_t nsorted;       // batch entries with n > 0 (packed mode, block-major: B)
  int32_t tile;          // rows per item (queries for fwd/dq, keys for dk/dv)
  int32_t xcd_chunk;     // items per XCD per round; 0 disables the remap
  int32_t causal;
  int32_t reverse;       // list tiles last-first (causal query-side passes)
  int32_t gate_sink;
  int32_t out_f32;       // outputs are float (else bf16)
  int32_t f16_pv;        // forward with hi+lo operands: P V on f16 operands where V fits
  float c1;              // -s * log2(e): logit scale folded into the exp2 argument
  float scale;           // s
  float gate_eps;
  float gate_tau;
  // packed variable-length mode (varlen != 0): the per-batch tables below are unused
  int32_t varlen;
  int32_t tiles_per_seq;       // ceil(max rows / tile)
  int32_t tiles_over_keys;     // 1: a pass whose tiles are key rows (dk/dv)
  const int32_t* cu_q;         // device [B + 1] query row bounds
  const int32_t* cu_k;         // device [B + 1] key row bounds
  const float* bias;           // device [B] or null (then beta_b = -ln(nk_b))
  // block-major mode (nblocks > 0; padded causal batches of one length, packed causal
  // batches): item g is (sorted position or sequence, head) (g % (nsorted * H)) / H,
  // g % H of block g / (nsorted * H), whose code holds the tile index (low 15 bits) and
  // kDqBlock
  int32_t nblocks;
  uint32_t blocks[kMaxBlocks];   // one dword each: read with a scalar load
  int32_t off[kMaxBatch + 1];  // prefix item counts by sorted position
  float c2[kMaxBatch];         // -beta * log2(e) by sorted position
  // valid length << 8 | batch index, by sorted position: one dword per entry, so that
  // the work-item decode reads it with a scalar load (through the scalar cache)
  uint32_t lenb[kMaxBatch];
};

// passed by value as the kernels' argument: stay within the 4 KiB a launch carries
static_assert(sizeof(KArgs) <= 4096, "kernel-argument block above 4 KiB");

SA_HD inline int len_at(const KArgs& a, int p) { return (int)(a.lenb[p] >> 8); }
SA_HD inline int bidx_at(const KArgs& a, int p) { return (int)(a.lenb[p] & 0xffu); }

struct Item {
  int b;         // batch index
  int h;         // head
  int t;         // tile index (rows t*tile .. t*tile+tile-1)
  int nq;        // query rows of this sequence
  int nk;        // key rows of this sequence
  int diag;      // causal: key j allowed for query i iff j <= i + diag
  int valid;     // 0: the item lies past its sequence (packed mode only)
  float c2;      // -beta_b * log2(e)
  int64_t qoff;  // element offset of query row 0 of (b, h) (q, o, dO, dq)
  int64_t koff;  // element offset of key row 0 of (b, h) (k, v, dk, dv)
  int64_t goff;  // gate index of key 0 of sequence b
};

// blockIdx -> item index. Rounds of kNumXcd*chunk items; in each round XCD x (which
// receives blocks w with w % 8 == x) takes the contiguous items [x*chunk, x*chunk+chunk).
// Bijective; blocks past the last full round map to themselves.
// chunk == kSnake (a block-major list that fits one round of resident workgroups): blocks
// w, w + kNumCu, w + 2 kNumCu, ... share a CU under round-robin dispatch, so every second
// span of kNumCu blocks takes its items in reverse order of groups of kNumXcd (a CU that
// receives one of the costliest items receives cheaper ones in its other slots; the
// order inside a group keeps each item's XCD). A last partial span maps to itself.
constexpr int kNumCu = 256;
constexpr int kSnake = -1;
SA_HD inline int remap_block(int w, int nitems, int chunk) {
  if (chunk == kSnake) {
    const int span = w / kNumCu, base = span * kNumCu, c = w - base;
    if ((span & 1) && base + kNumCu <= nitems)
      return base + (kNumCu / kNumXcd - 1 - c / kNumXcd) * kNumXcd + c % kNumXcd;
    return w;
  }
  if (chunk <= 0) return w;
  const int round = kNumXcd * chunk;
  const int full = (nitems / round) * round;
  if (w >= full) return w;
  const int x = w % kNumXcd;
  const int s = w / kNumXcd;
  return (s / chunk) * round + x * chunk + (s % chunk);
}

// Item (head h, tile t) of the sequence at sorted position p.
SA_HD inline Item item_at(const KArgs& a, int p, int h, int t) {
  Item it;
  it.b = bidx_at(a, p);
  it.nq = it.nk = len_at(a, p);
  it.diag = 0;
  it.valid = 1;
  it.c2 = a.c2[p];
  it.h = h;
  it.t = t;
  it.qoff = it.koff = (int64_t)it.b * a.sb + (int64_t)it.h * a.sh;
  it.goff = (int64_t)it.b * a.gsb;
  return it;
}

// Item g of a block-major list; *dq_block is set for a dQ block of the one-call list.
SA_HD inline Item decode_block_item(const KArgs& a, int g, bool* dq_block) {
  const int m = a.nsorted * a.H;
  const int blk = g / m;
  const int r = g - blk * m;
  const int p = r / a.H;
  const unsigned code = a.blocks[blk];
  *dq_block = (code & kDqBlock) != 0u;
  return item_at(a, p, r - p * a.H, (int)(code & (kDqBlock - 1u)));
}

// `reverse` lists a sequence's tiles last-first (the causal query-side passes); a
// block-major list carries its tile order in the block codes instead.
SA_HD inline Item decode_item(const KArgs& a, int g, int reverse) {
  if (a.nblocks > 0) {
    bool dq_block;
    return decode_block_item(a, g, &dq_block);
  }
  // largest p with off[p] <= g (off is non-decreasing, off[0] = 0)
  int lo = 0, hi = a.nsorted - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.off[mid] <= g) lo = mid; else hi = mid - 1;
  }
  const int p = lo;
  const int T = (len_at(a, p) + a.tile - 1) / a.tile;
  const int local = g - a.off[p];
  int h, t;
  if (a.causal) {
    h = local % a.H;
    t = local / a.H;
  } else {
    h = local / T;
    t = local % T;
  }
  if (reverse) t = T - 1 - t;
  return item_at(a, p, h, t);
}

SA_HD inline Item decode_item(const KArgs& a, int g) { return decode_item(a, g, a.reverse); }

}  // namespace sa
