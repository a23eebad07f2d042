// Device helpers for the gfx950 (CDNA4) sigmoid-attention kernels: MFMA and LDS
// wrappers, the swizzled LDS tile layout, register-staged tile loads, and the
// exp2/rcp form of the logistic function.
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (64 lanes, l = lane):
//   A[i][k]: lane l holds i = l % 32, k = 8*(l/32) + 0..7        (8 bf16)
//   B[k][j]: lane l holds j = l % 32, k = 8*(l/32) + 0..7        (8 bf16)
//   D[i][j]: lane l, register r holds i = 8*(r/4) + 4*(l/32) + r%4, j = l % 32
// A product whose result feeds the next MFMA as an operand is computed transposed
// (S^T = K Q^T), so each lane owns one query column and 16 keys of it; those 16
// registers are consumed directly as the k-slots of the next MFMA, with the k-slot
// -> key permutation  slot 8*h + m  <->  key 8*(m/4) + 4*h + m%4  (h = l/32) applied
// identically to the other operand.
//
// ds_read_b64_tr_b16: within each 16-lane group, source lane j points at 4 bf16;
// output lane 16g+m receives element (m & 3) of source lanes 16g + (m >> 2) + 4e,
// e = 0..3. With source lane j addressing row r0 + j/4, column c0 + 4*(j%4) of a
// row-major tile, output lane m gets rows r0..r0+3 of column c0 + m: a column read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kargs.h"

namespace sa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

#define SA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f16(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Make the compiler wait for a register's pending load here, so that loop bodies that
// use it do not conservatively wait for every load in flight (including prefetches).
template <typename V>
__device__ __forceinline__ void settle(V& x) {
  asm volatile("" : "+v"(x));
}

// ---------------------------------------------------------------------------------
// LDS tile layout: [rows][D] bf16; the 16-byte chunks of row r are permuted by
// XOR with xsw<D>(r). The map is chosen (by exhaustive search over XOR maps of the row
// bits) so that both read patterns below touch distinct banks in every pass, for LDS
// widths of 32 or 64 four-byte banks: the row-operand read (32 consecutive rows, one
// chunk) and the transposed column read (4 consecutive rows x 4 chunks).
// ---------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ constexpr int xsw(int r) {
  if (D == 64) return ((r & 3) << 1) ^ ((r >> 2) & 3);
  return ((r & 1) << 2) ^ ((r & 2) * 5) ^ ((r >> 2) & 3);
}

template <int D>
__device__ __forceinline__ uint32_t swz(int row, int col) {
  return (uint32_t)(row * (D * 2) + (((col >> 3) ^ xsw<D>(row)) << 4) + ((col & 7) << 1));
}

__device__ __forceinline__ bf16x8 lds_read16(const char* base, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const char* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((SA_LDS bf16x4*)(base + off));
}

__device__ __forceinline__ bf16x8 cat(const bf16x4& a, const bf16x4& b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// Column operand of a 32x32x16 MFMA from a row-major swizzled tile: lane l receives
// rows row0 + (slot->row map) of column col0 + l%32 for the 16 k-slots of k-step
// `ks` (rows row0 + 16*ks + 8*(m/4) + 4*(l/32) + m%4). Two transposed reads.
template <int D>
__device__ __forceinline__ bf16x8 lds_col_operand(const char* tile, int row0, int col0) {
  const int l = lane_id();
  const int g = l >> 4, j = l & 15;
  const int r = row0 + 4 * (g >> 1) + (j >> 2);
  const int c = col0 + 16 * (g & 1) + 4 * (j & 3);
  const bf16x4 lo = lds_read_tr(tile, swz<D>(r, c));
  const bf16x4 hi = lds_read_tr(tile, swz<D>(r + 8, c));
  return cat(lo, hi);
}

// Row operand: lane l receives row row0 + l%32, columns col0 + 8*(l/32) + 0..7.
template <int D>
__device__ __forceinline__ bf16x8 lds_row_operand(const char* tile, int row0, int col0) {
  const int l = lane_id();
  return lds_read16(tile, swz<D>(row0 + (l & 31), col0 + 8 * (l >> 5)));
}

// Per-lane byte offsets of the two operand reads above inside a swizzled tile, for row
// blocks that start at a multiple of 16 rows (the swizzle depends on the low four row
// bits only, so such a block is the first one shifted by row0 * 2D bytes). With a tile
// address known at compile time, every read is then one LDS instruction with an
// immediate offset: no per-read address arithmetic.
template <int D>
struct LdsLane {
  uint32_t row[D / 16];     // row operand of k-step ks
  uint32_t col[D / 32][2];  // column operand of column block dt: rows r and r + 8
  __device__ __forceinline__ LdsLane() {
    const int l = lane_id();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) row[ks] = swz<D>(l & 31, 16 * ks + 8 * (l >> 5));
    const int g = l >> 4, j = l & 15;
    const int r = 4 * (g >> 1) + (j >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int c = 32 * dt + 16 * (g & 1) + 4 * (j & 3);
      col[dt][0] = swz<D>(r, c);
      col[dt][1] = swz<D>(r + 8, c);
    }
  }
  // row0 must be a multiple of 16
  __device__ __forceinline__ bf16x8 rowop(const char* tile, int row0, int ks) const {
    return lds_read16(tile + row0 * (2 * D), row[ks]);
  }
  __device__ __forceinline__ bf16x8 colop(const char* tile, int row0, int dt) const {
    const char* t = tile + row0 * (2 * D);
    return cat(lds_read_tr(t, col[dt][0]), lds_read_tr(t, col[dt][1]));
  }
};

// ---------------------------------------------------------------------------------
// Staging of a [ROWS][D] bf16 tile: 16-byte global loads into registers (issued one
// tile ahead, so their latency hides behind the current tile's MFMA work), then
// 16-byte LDS stores into the swizzled layout. Consecutive threads load consecutive
// 16-byte chunks, so each wave reads whole rows. Rows past the valid length are
// clamped to the last valid row: padded memory is never read, and the caller masks
// those rows out of the result.
// ---------------------------------------------------------------------------------
template <int ROWS, int D, int NTHREADS>
struct TileRegs {
  static constexpr int CPR = D / 8;                       // 16-byte chunks per row
  static constexpr int ITERS = ROWS * CPR / NTHREADS;
  static_assert(ROWS * CPR % NTHREADS == 0, "tile must split evenly over the threads");
  u32x4 r[ITERS];

  __device__ __forceinline__ void load(const bf16* src, int64_t sl, int row_base, int last_row) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int P = it * NTHREADS + (int)threadIdx.x;
      const int row = P / CPR;
      int grow = row_base + row;
      grow = grow < last_row ? grow : last_row;
      r[it] = *reinterpret_cast<const u32x4*>(src + (int64_t)grow * sl + (P % CPR) * 8);
    }
  }
  __device__ __forceinline__ void store(char* lds_tile) const {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int P = it * NTHREADS + (int)threadIdx.x;
      *reinterpret_cast<u32x4*>(lds_tile + swz<D>(P / CPR, (P % CPR) * 8)) = r[it];
    }
  }
};

// ---------------------------------------------------------------------------------
// Direct global -> LDS staging (global_load_lds_dwordx4) of a [ROWS][D] bf16 tile in the
// swizzled layout above, without passing through registers. One wave instruction moves
// 64 x 16 bytes into one contiguous 1 KB block of LDS: lane L fills bytes [16L, 16L+16)
// of the block. The swizzle is applied on the source side: the 16-byte slot `s` of tile
// row `r` holds logical chunk s ^ xsw(r), so lane L loads that chunk. Rows past the
// valid length are clamped to the last valid row (padded memory is never read; the
// caller masks those keys). The data is in LDS once vmcnt reaches zero for the issuing
// wave; a barrier then makes it visible to the workgroup.
// ---------------------------------------------------------------------------------
// One global_load_lds_dwordx4: 16 bytes per lane from base + voff into LDS at
// lds_addr + 16 * lane. Written as inline assembly so that the compiler does not see an
// LDS write in flight and does not make every later LDS read wait for it (it cannot tell
// that the ring stage being filled is not the one being read). Completion is awaited
// explicitly (vmcnt) before the barrier that publishes the stage. M0 is used by
// nothing else in these kernels.
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  // base and lds_addr are wave-uniform; make them scalar for the s-register operands
  // (readfirstlane returns int: go through uint32_t so the low half is not sign-extended)
  const uint64_t b = reinterpret_cast<uintptr_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t bs = (uint64_t)lo | ((uint64_t)hi << 32);
  const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  // Wait states the hardware does not enforce: 5 between a VALU write of an SGPR (the
  // readfirstlane above) and a memory instruction reading it, 1 between an SALU write
  // of M0 and an LDS DMA that uses it.
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(bs), "s"(ls) : "memory");
}

template <int ROWS, int D, int NWAVES>
struct DirectTile {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int BLOCKS = ROWS * CPR / 64;    // 1 KB blocks per tile
  static constexpr int PER_WAVE = BLOCKS / NWAVES;
  static_assert(BLOCKS % NWAVES == 0, "tile must split evenly over the waves");

  // Rows row_base .. row_base + ROWS - 1 of src (element row stride sl, which must keep
  // ROWS * sl * 2 below 2^32), rows past last_row clamped to last_row. The per-lane
  // source offsets are recomputed at each call (a few VALU operations per tile) rather
  // than held in registers.
  __device__ __forceinline__ static void load(char* lds_tile, const bf16* src, int64_t sl,
                                              int row_base, int last_row) {
    const int l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const char* base = reinterpret_cast<const char*>(src + (int64_t)row_base * sl);
    const int lim = last_row - row_base;
    const uint32_t rb = (uint32_t)sl * 2u;
    const uint32_t lds = (uint32_t)(uintptr_t)(SA_LDS char*)lds_tile;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int blk = i * NWAVES + w;
      const int P = blk * 64 + l;
      const int row = P / CPR;
      const uint32_t col = (uint32_t)(((P % CPR) ^ xsw<D>(row)) * 16);
      const int r = row < lim ? row : lim;
      lds_dma16(base, (uint32_t)r * rb + col, lds + (uint32_t)blk * 1024u);
    }
  }
};

// Direct loads of one ring stage holding two tiles with the same layout and strides (K
// and V, or Q and dO), the second TILE bytes after the first. A tile whose rows are all
// valid takes the fast path: this wave's two 1 KB blocks of a tile sit NWAVES blocks
// apart, and the swizzle depends on the low four row bits only, which the two blocks
// share, so one per-lane offset (computed once) serves every interior tile and both
// blocks: the second block's source is the first's plus a fixed number of rows. Per tile
// the fast path issues four loads with no vector arithmetic and one wait for SGPRs
// written by vector instructions per tensor. Edge tiles clamp rows to the last valid row
// (DirectTile).
// A wave-uniform 64-bit value in scalar registers (readfirstlane returns int: go through
// uint32_t so that the low half is not sign-extended)
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return (uint64_t)lo | ((uint64_t)hi << 32);
}

template <int ROWS, int D, int NWAVES>
struct DirectPair {
  using Tile = DirectTile<ROWS, D, NWAVES>;
  static constexpr int CPR = D / 8;
  static constexpr int TILE = ROWS * D * 2;
  static constexpr int ROWS_APART = NWAVES * 64 / CPR;   // rows between this wave's blocks
  static_assert(Tile::PER_WAVE % 2 == 0, "pairs of blocks per wave and tile");
  static_assert(ROWS_APART % 16 == 0, "this wave's blocks must share the low four row bits");
  uint32_t voff;       // per-lane byte offset of block 0 within an interior tile
  uint32_t rb;         // row stride in bytes
  int w;               // wave index (uniform)

  __device__ __forceinline__ DirectPair(int64_t sl) {
    const int l = lane_id();
    w = __builtin_amdgcn_readfirstlane(wave_id());
    rb = (uint32_t)sl * 2u;
    const int P = w * 64 + l;
    const int row = P / CPR;
    voff = (uint32_t)row * rb + (uint32_t)(((P % CPR) ^ xsw<D>(row)) * 16);
  }

  // Block i of this wave (i = 0 .. PER_WAVE - 1) lies i * ROWS_APART rows further in the
  // source and i * NWAVES KB further in LDS, with the same per-lane offset.
  __device__ __forceinline__ void fast(const char* base, uint32_t lds) const {
#pragma unroll
    for (int pr = 0; pr < Tile::PER_WAVE / 2; ++pr) {
      const uint64_t b0 = uniform_u64(reinterpret_cast<uintptr_t>(base) +
                                      (uint64_t)(2 * pr * ROWS_APART) * rb);
      const uint64_t b1 = uniform_u64(b0 + (uint64_t)ROWS_APART * rb);
      const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(
          lds + (uint32_t)(2 * pr * NWAVES) * 1024u);
      const uint32_t lds1 = (uint32_t)__builtin_amdgcn_readfirstlane(
          lds + (uint32_t)((2 * pr + 1) * NWAVES) * 1024u);
      // 5 wait states between a vector write of an SGPR operand and the memory instruction
      // reading it (once for both loads), 1 between the SALU write of M0 and the LDS DMA
      asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %3\n\t"
                   "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %4"
                   :: "v"(voff), "s"(lds0), "s"(lds1), "s"(b0), "s"(b1) : "memory");
    }
  }

  // rows row_base .. row_base + ROWS - 1 of a and b into the stage at lds_stage
  __device__ __forceinline__ void load(char* lds_stage, const bf16* a, const bf16* b, int64_t sl,
                                       int row_base, int last_row) const {
    if (row_base + ROWS - 1 <= last_row) {
      const uint32_t lds = (uint32_t)(uintptr_t)(SA_LDS char*)lds_stage + (uint32_t)w * 1024u;
      const int64_t off = (int64_t)row_base * sl;
      fast(reinterpret_cast<const char*>(a + off), lds);
      fast(reinterpret_cast<const char*>(b + off), lds + (uint32_t)TILE);
    } else {
      Tile::load(lds_stage, a, sl, row_base, last_row);
      Tile::load(lds_stage + TILE, b, sl, row_base, last_row);
    }
  }
};

// The work item of this workgroup, with every field made explicitly wave-uniform (scalar
// registers), so that the tensor base pointers derived from it stay in scalar registers.
// Packed mode: the item's sequence bounds come from the device arrays cu_q / cu_k.
// Packed-mode item g of a pass with T tiles per (sequence, head), over key rows or query
// rows.
__device__ __forceinline__ Item varlen_item_at(const KArgs& a, int b, int h, int t,
                                               int over_keys) {
  Item it;
  it.t = t;
  it.h = h;
  it.b = b;
  const int q0 = a.cu_q[it.b], k0 = a.cu_k[it.b];
  it.nq = a.cu_q[it.b + 1] - q0;
  it.nk = a.cu_k[it.b + 1] - k0;
  it.diag = it.nk - it.nq;
  const int rows = over_keys ? it.nk : it.nq;
  it.valid = it.t * a.tile < rows ? 1 : 0;
  // -beta * log2(e); the default beta = -ln(nk) gives log2(nk)
  it.c2 = a.bias ? -a.bias[it.b] * 1.4426950408889634f
                 : (it.nk > 0 ? __builtin_amdgcn_logf((float)it.nk) : 0.0f);
  it.qoff = (int64_t)q0 * a.sl + (int64_t)it.h * a.sh;
  it.koff = (int64_t)k0 * a.sl + (int64_t)it.h * a.sh;
  it.goff = k0;
  return it;
}

__device__ __forceinline__ Item varlen_item(const KArgs& a, int g, int T, int over_keys) {
  const int bh = g / T;
  return varlen_item_at(a, bh / a.H, bh % a.H, g % T, over_keys);
}

// Packed-mode item g of a block-major list (causal batches): block g / (B * H) holds one
// tile of every (sequence, head); *dq_block is set for a dQ block of the one-call list.
__device__ __forceinline__ Item varlen_block_item(const KArgs& a, int g, bool* dq_block) {
  const int m = a.nsorted * a.H;
  const int blk = g / m;
  const int r = g - blk * m;
  const unsigned code = a.blocks[blk];
  *dq_block = (code & kDqBlock) != 0u;
  const int b = r / a.H;
  return varlen_item_at(a, b, r - b * a.H, (int)(code & (kDqBlock - 1u)),
                        *dq_block ? 0 : a.tiles_over_keys);
}

__device__ __forceinline__ Item varlen_item(const KArgs& a, int g) {
  if (a.nblocks > 0) {
    bool dq_block;
    return varlen_block_item(a, g, &dq_block);
  }
  return varlen_item(a, g, a.tiles_per_seq, a.tiles_over_keys);
}

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t u = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Every field of a work item is the same for the whole workgroup: keep it in scalar
// registers, so that base pointers built from it do too.
__device__ __forceinline__ Item uniform_item(Item it) {
  it.b = __builtin_amdgcn_readfirstlane(it.b);
  it.h = __builtin_amdgcn_readfirstlane(it.h);
  it.t = __builtin_amdgcn_readfirstlane(it.t);
  it.nq = __builtin_amdgcn_readfirstlane(it.nq);
  it.nk = __builtin_amdgcn_readfirstlane(it.nk);
  it.diag = __builtin_amdgcn_readfirstlane(it.diag);
  it.valid = __builtin_amdgcn_readfirstlane(it.valid);
  it.c2 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, it.c2)));
  it.qoff = uniform64(it.qoff);
  it.koff = uniform64(it.koff);
  it.goff = uniform64(it.goff);
  return it;
}

template <bool VL>
__device__ __forceinline__ Item block_item(const KArgs& a) {
  const int g = remap_block(blockIdx.x, a.nitems, a.xcd_chunk);
  return uniform_item(VL ? varlen_item(a, g) : decode_item(a, g));
}

// Wait until every vector-memory operation of this wave has completed (including direct
// loads into LDS), then synchronise the workgroup.
__device__ __forceinline__ void wait_vmem_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// ---------------------------------------------------------------------------------
// Logistic function: sigma(x) = 1 / (1 + 2^t), t = -x * log2(e) = acc * c1 + c2 with
// c1 = -s*log2(e), c2 = -beta*log2(e). Hardware v_exp_f32 / v_rcp_f32; for large t
// exp2 -> +inf and rcp -> 0, for very negative t exp2 -> 0 and rcp -> 1: no NaN.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float sigmoid_l2(float acc, float c1, float c2) {
  const float t = __builtin_fmaf(acc, c1, c2);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// 8 floats to f16, round to nearest even.
__device__ __forceinline__ f16x8 pack8_f16(const f32x16& v, int base) {
  f16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (_Float16)v[base + i];
  return r;
}

// Logistic function scaled by 2^14: 2^14 / (1 + 2^t) = 1 / (2^-14 + 2^(t - 14)), with
// c2s = c2 - 14 folded into the exp2 argument, so the scale costs nothing. In [0, 2^14],
// so the value and its f16 rounding stay normal down to sigma = 2^-28.
constexpr float kPScale = 16384.0f;
constexpr float kPScaleInv = 1.0f / 16384.0f;
__device__ __forceinline__ float sigmoid_l2s(float acc, float c1, float c2s) {
  const float t = __builtin_fmaf(acc, c1, c2s);
  return __builtin_amdgcn_rcpf(kPScaleInv + __builtin_amdgcn_exp2f(t));
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int base) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)v[base + i];
  return r;
}

// Split 8 floats v[base..base+7] into bf16 hi (round to nearest even) and bf16 lo =
// bf16(v - hi), so that hi + lo carries about 16 significant bits. The residual
// v - hi is exact in float and is formed by one v_dot2c_f32_bf16 per element:
// v + (hi0, hi1) . (-1, 0).
// The two selector pairs (-1, 0) and (0, -1) live in scalar registers (the instruction
// takes its first source from one), built once per kernel from their bit patterns
// 0x0000bf80 and 0xbf800000: as an inline-constant operand of a packed bf16 instruction
// they would not carry the intended halves.
struct SplitSel {
  bf16x2 m0, m1;
  __device__ __forceinline__ SplitSel() {
    uint32_t b0 = 0x0000bf80u, b1 = 0xbf800000u;
    asm volatile("" : "+s"(b0), "+s"(b1));
    m0 = __builtin_bit_cast(bf16x2, b0);
    m1 = __builtin_bit_cast(bf16x2, b1);
  }
};

__device__ __forceinline__ void split8(const f32x16& v, int base, bf16x8& hi, bf16x8& lo,
                                       const SplitSel& sel) {
  const bf16x2 m0 = sel.m0, m1 = sel.m1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = v[base + 2 * i], b = v[base + 2 * i + 1];
    bf16x2 h;
    h[0] = (bf16)a;
    h[1] = (bf16)b;
    const float ra = __builtin_amdgcn_fdot2_f32_bf16(h, m0, a, false);
    const float rb = __builtin_amdgcn_fdot2_f32_bf16(h, m1, b, false);
    hi[2 * i] = h[0];
    hi[2 * i + 1] = h[1];
    lo[2 * i] = (bf16)ra;
    lo[2 * i + 1] = (bf16)rb;
  }
}

// Key (or query) index held by register r of lane l in a 32x32 MFMA result, relative
// to the tile's row 0.
__device__ __forceinline__ int acc_row(int r, int l) { return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); }

// Store a 32-column x 32-row float accumulator tile, transposed in registers (lane l
// owns output row `row`, registers hold 16 of the 32 columns col0 + acc_row(r, l)), as
// bf16 with a scale: four 8-byte stores per lane.
__device__ __forceinline__ void store_row_bf16(bf16* dst_row, const f32x16& acc, int col0,
                                               float mul) {
  const int l = lane_id();
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[4 * a + e] * mul);
    *reinterpret_cast<bf16x4*>(dst_row + col0 + 8 * a + 4 * (l >> 5)) = v;
  }
}

__device__ __forceinline__ void store_row_f32(float* dst_row, const f32x16& acc, int col0,
                                              float mul) {
  const int l = lane_id();
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = acc[4 * a + e] * mul;
    *reinterpret_cast<f32x4*>(dst_row + col0 + 8 * a + 4 * (l >> 5)) = v;
  }
}

// Store one lane's output row (bf16 or float output type, chosen at run time).
__device__ __forceinline__ void store_row(void* base, int64_t row_off, bool out_f32,
                                          const f32x16& acc, int col0, float mul) {
  if (out_f32) store_row_f32(reinterpret_cast<float*>(base) + row_off, acc, col0, mul);
  else store_row_bf16(reinterpret_cast<bf16*>(base) + row_off, acc, col0, mul);
}

}  // namespace sa
