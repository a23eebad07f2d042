// Host side of the C ABI declared in include/sigattn.h: argument validation, the
// length-aware work planner (valid tiles only, longest sequences first, XCD-grouped)
// and kernel launch on the caller's stream. Nothing here allocates, frees or
// synchronises.
#include "../../include/sigattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <vector>

#include "aux_args.h"
#include "dec_args.h"
#include "kargs.h"

namespace sa {
hipError_t launch_fwd_bf16(const KArgs& a, int d, bool causal, bool gated, bool split, hipStream_t st);
hipError_t launch_dq_bf16(const KArgs& a, int d, bool causal, bool gated, bool split, hipStream_t st);
hipError_t launch_dkdv_bf16(const KArgs& a, int d, bool causal, bool gated, bool split, hipStream_t st);
hipError_t launch_bwd_bf16(const KArgs& a, void* dq, int nq_items, int tiles_q, bool causal,
                           bool gated, bool split, hipStream_t st);
int fwd_tile_rows(int d);
int dq_tile_rows(int d);
int dkdv_tile_rows(int d);
hipError_t launch_zero_rows(const ZArgs& z, int B, int H, hipStream_t st);
hipError_t launch_plane_tail(const PArgs& pa, hipStream_t st);
hipError_t launch_f32(const DArgs& a, int pass, hipStream_t st);
hipError_t launch_cache_build(const BuildArgs& a, int B, hipStream_t st);
hipError_t launch_cache_append(const AppendArgs& a, int B, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t noalloc_scratch(hipStream_t stream, float** out);
int calib_mfma_per_iter();
hipError_t launch_mfma_calib(float* sink, int64_t* clk, int nblocks, int iters, hipStream_t st);
}  // namespace sa

namespace {

using sa::KArgs;

constexpr double kLog2eD = 1.4426950408889634;

static_assert(SIGATTN_NOALLOC_WORKSPACE_BYTES == sa::kNoAllocFloats * (int64_t)sizeof(float),
              "the header's limit must match the static workspace");

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(const sigattn_problem* p) { return p->dtype == SIGATTN_BF16 ? 2 : 4; }
int out_elem_size(const sigattn_problem* p) { return p->out_dtype == SIGATTN_BF16 ? 2 : 4; }

double beta_of(const sigattn_problem* p, int b) {
  if (p->bias) return (double)p->bias[b];
  const int n = p->seqlens[b];
  return n > 0 ? -std::log((double)n) : 0.0;   // b = -ln(n); unused when n = 0
}

double scale_of(const sigattn_problem* p) {
  return p->scale != 0.0f ? (double)p->scale : 1.0 / std::sqrt((double)p->d);
}

int tile_rows_d(int d, int pass);

// Rows of d elements at offsets sum_i idx_i * stride_i (0 <= idx_i < count_i) must not
// overlap, or outputs written through the shared strides would race. Sufficient test:
// with the dimensions of count > 1 sorted by stride, each stride is at least the extent
// of the dimensions below it (the first at least d).
bool rows_disjoint(int64_t d, const int64_t* stride, const int64_t* count, int n) {
  int64_t st[4], ct[4];
  int m = 0;
  for (int i = 0; i < n && m < 4; ++i)
    if (count[i] > 1) { st[m] = stride[i]; ct[m] = count[i]; ++m; }
  for (int i = 1; i < m; ++i)
    for (int j = i; j > 0 && st[j] < st[j - 1]; --j) {
      std::swap(st[j], st[j - 1]);
      std::swap(ct[j], ct[j - 1]);
    }
  int64_t extent = d;   // elements spanned by the dimensions below
  for (int i = 0; i < m; ++i) {
    if (st[i] < extent) return false;
    // extent of dims 0..i: the last row starts at (count-1)*stride (+ below), spans d more
    const double e = (double)st[i] * (double)(ct[i] - 1) + (double)extent;
    if (e > 9.0e18) return false;
    extent = st[i] * (ct[i] - 1) + extent;
  }
  return true;
}

sigattn_status validate_problem(const sigattn_problem* p) {
  if (!p) return SIGATTN_ERR_INVALID_ARG;
  if (p->struct_size != sizeof(sigattn_problem)) return SIGATTN_ERR_INVALID_ARG;
  if (p->B < 0 || p->H < 1 || p->Lmax < 1) return SIGATTN_ERR_INVALID_ARG;
  if (p->B > SIGATTN_MAX_BATCH || p->Lmax > SIGATTN_MAX_LEN) return SIGATTN_ERR_UNSUPPORTED;
  if (p->d != 64 && p->d != 128) return SIGATTN_ERR_UNSUPPORTED;
  if (p->dtype != SIGATTN_BF16 && p->dtype != SIGATTN_F32) return SIGATTN_ERR_UNSUPPORTED;
  if (p->out_dtype != SIGATTN_BF16 && p->out_dtype != SIGATTN_F32) return SIGATTN_ERR_UNSUPPORTED;
  if (p->dtype == SIGATTN_F32 && p->out_dtype != SIGATTN_F32) return SIGATTN_ERR_UNSUPPORTED;
  if (p->fast_math < 0 || p->fast_math > 2) return SIGATTN_ERR_INVALID_ARG;
  if (p->stride_b < 0 || p->stride_h < 0 || p->stride_l < p->d) return SIGATTN_ERR_INVALID_ARG;
  // tile loads address up to 128 rows from a per-tile base with 32-bit byte offsets
  if (p->stride_l > SIGATTN_MAX_ROW_STRIDE) return SIGATTN_ERR_UNSUPPORTED;
  if (p->B > 0 && !p->seqlens) return SIGATTN_ERR_INVALID_ARG;
  for (int b = 0; b < p->B; ++b)
    if (p->seqlens[b] < 0 || p->seqlens[b] > p->Lmax) return SIGATTN_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return SIGATTN_ERR_INVALID_ARG;
  if (!std::isfinite(p->scale) || p->scale < 0.0f) return SIGATTN_ERR_INVALID_ARG;
  if (p->bias)
    for (int b = 0; b < p->B; ++b)
      if (!std::isfinite(p->bias[b])) return SIGATTN_ERR_INVALID_ARG;
  if (p->gate) {
    if (reinterpret_cast<uintptr_t>(p->gate) & 3u) return SIGATTN_ERR_ALIGNMENT;
    if (p->gate_stride_b < 0 || (p->gate_stride_b != 0 && p->gate_stride_b < p->Lmax))
      return SIGATTN_ERR_INVALID_ARG;
    if (!std::isfinite(p->gate_eps) || p->gate_eps < 0.0f) return SIGATTN_ERR_INVALID_ARG;
    if (!std::isfinite(p->gate_tau) || p->gate_tau < 0.0f) return SIGATTN_ERR_INVALID_ARG;
    if (p->gate_sink < 0) return SIGATTN_ERR_INVALID_ARG;
  }
  // every row must start on a 16-byte boundary
  const int64_t es = elem_size(p);
  if (((p->stride_l * es) & 15) || ((p->stride_h * es) & 15) || ((p->stride_b * es) & 15))
    return SIGATTN_ERR_ALIGNMENT;
  // rows of different (batch entry, head, position) must not overlap: outputs share these
  // strides
  {
    const int64_t stride[3] = {p->stride_b, p->stride_h, p->stride_l};
    const int64_t count[3] = {p->B, p->H, p->Lmax};
    if (!rows_disjoint(p->d, stride, count, 3)) return SIGATTN_ERR_INVALID_ARG;
  }
  for (int pass = 0; pass < 3; ++pass) {
    const int tile = tile_rows_d(p->d, pass);
    int64_t items = 0;
    for (int b = 0; b < p->B; ++b) items += (int64_t)p->H * ((p->seqlens[b] + tile - 1) / tile);
    if (items > SIGATTN_MAX_ITEMS) return SIGATTN_ERR_UNSUPPORTED;
  }
  return SIGATTN_OK;
}

sigattn_status check_tensors(const void* const* in, int nin, void* const* out, int nout) {
  for (int i = 0; i < nin; ++i) {
    if (!in[i]) return SIGATTN_ERR_INVALID_ARG;
    if (!aligned16(in[i])) return SIGATTN_ERR_ALIGNMENT;
  }
  for (int o = 0; o < nout; ++o) {
    if (!out[o]) return SIGATTN_ERR_INVALID_ARG;
    if (!aligned16(out[o])) return SIGATTN_ERR_ALIGNMENT;
    for (int i = 0; i < nin; ++i)
      if (out[o] == in[i]) return SIGATTN_ERR_INVALID_ARG;
    for (int o2 = 0; o2 < o; ++o2)
      if (out[o] == out[o2]) return SIGATTN_ERR_INVALID_ARG;
  }
  return SIGATTN_OK;
}

int tile_rows_d(int d, int pass) {
  return pass == 0 ? sa::fwd_tile_rows(d) : pass == 1 ? sa::dq_tile_rows(d) : sa::dkdv_tile_rows(d);
}

int tile_rows(const sigattn_problem* p, int pass) { return tile_rows_d(p->d, pass); }

int xcd_chunk_default() {
  static int v = [] {
    const char* e = std::getenv("SIGATTN_XCD_CHUNK");
    return e ? std::atoi(e) : 16;
  }();
  return v;
}

// 32 x 32 units of work in tile t of a causal (nq, nk) pair, causal rule aligned at the
// bottom right (tiles of `tile` rows, one 32-row slice per wave): a query slice sees the
// keys up to its last row, a key slice the queries from its first row on.
double causal_tile_units(int nq, int nk, int tile, int t, bool key_side) {
  const int sq = (nq + 31) / 32, sk = (nk + 31) / 32;
  double u = 0.0;
  for (int w = 0; w < tile / 32; ++w) {
    const int r = t * (tile / 32) + w;
    if (r >= (key_side ? sk : sq)) break;
    u += std::max(0, key_side ? std::min(sq, sk - r) : std::min(sk, r + 1 + sk - sq));
  }
  return u;
}

// Measured cost of a dK/dV unit relative to a dQ unit (1.46 and 1.03 us per wave at two
// waves per SIMD), which orders the merged blocks of the one-call backward.
constexpr double kDkdvUnitCost = 1.42;

// Block-major list of a causal batch: one block per tile, costliest first. `which` is the
// pass (0 forward, 1 dQ, 2 dK/dV) or 3 for the one-call backward, whose dK/dV blocks (tk
// key tiles) and dQ blocks (tq query tiles) are merged by cost, dQ blocks flagged. Lists
// of more than kMaxBlocks blocks keep the default order.
void set_blocks(KArgs* a, int which, int nq, int nk, int tq, int tk) {
  a->nblocks = 0;
  struct Block { double cost; uint32_t code; };
  std::vector<Block> blocks;
  if (which == 2 || which == 3)
    for (int t = 0; t < tk; ++t)
      blocks.push_back({kDkdvUnitCost * causal_tile_units(nq, nk, a->tile, t, true),
                        (uint32_t)t});
  if (which != 2)
    for (int t = tq - 1; t >= 0; --t)
      blocks.push_back({causal_tile_units(nq, nk, a->tile, t, false),
                        (uint32_t)t | (which == 3 ? sa::kDqBlock : 0u)});
  if (blocks.empty() || (int)blocks.size() > sa::kMaxBlocks) return;
  std::stable_sort(blocks.begin(), blocks.end(),
                   [](const Block& x, const Block& y) { return x.cost > y.cost; });
  a->nblocks = (int)blocks.size();
  for (int i = 0; i < a->nblocks; ++i) a->blocks[i] = blocks[i].code;
  a->xcd_chunk = 0;
}

// Workgroups of a pass resident on one CU (the kernels' waves per SIMD; a workgroup has
// one wave on each of the CU's four SIMDs). Pass 3: the one-call backward.
int slots_per_cu(int pass, int d) {
  if (pass == 0) return d == 64 ? 3 : 2;
  if (pass == 2) return d == 64 ? 2 : 1;
  return 2;
}

// A block-major list that one round of resident workgroups holds is spread over the CUs
// by the snake remap (remap_block); longer lists are list-scheduled in order.
void snake_if_one_round(KArgs* a, int pass, int d, int nitems) {
  if (a->nblocks > 0 && nitems <= sa::kNumCu * slots_per_cu(pass, d)) a->xcd_chunk = sa::kSnake;
}

// Padded batches: block-major only when causal and every listed sequence has one length.
void order_blocks(KArgs* a, int which) {
  a->nblocks = 0;
  if (!a->causal || a->nsorted == 0 || sa::len_at(*a, 0) != sa::len_at(*a, a->nsorted - 1))
    return;
  const int n = sa::len_at(*a, 0);
  const int T = (n + a->tile - 1) / a->tile;
  set_blocks(a, which, n, n, T, T);
}

// Fill the kernel-argument block of one pass: the sorted, padded-tile-free work list.
void plan_pass(const sigattn_problem* p, int pass, KArgs* a) {
  std::memset(a, 0, sizeof(*a));
  const int tile = tile_rows(p, pass);
  std::vector<int> order;
  for (int b = 0; b < p->B; ++b)
    if (p->seqlens[b] > 0) order.push_back(b);
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return p->seqlens[x] > p->seqlens[y]; });
  a->nsorted = (int)order.size();
  a->off[0] = 0;
  for (int i = 0; i < a->nsorted; ++i) {
    const int b = order[i];
    const int n = p->seqlens[b];
    const int T = (n + tile - 1) / tile;
    a->off[i + 1] = a->off[i] + p->H * T;
    a->lenb[i] = ((uint32_t)n << 8) | (uint32_t)b;
    a->c2[i] = (float)(-beta_of(p, b) * kLog2eD);
  }
  a->nitems = a->off[a->nsorted];
  a->H = p->H;
  a->Lmax = p->Lmax;
  a->tile = tile;
  a->xcd_chunk = xcd_chunk_default();
  a->causal = p->causal;
  a->reverse = (p->causal && pass != 2) ? 1 : 0;
  a->sb = p->stride_b;
  a->sh = p->stride_h;
  a->sl = p->stride_l;
  const double s = scale_of(p);
  a->scale = (float)s;
  a->c1 = (float)(-s * kLog2eD);
  a->gate = p->gate;
  a->gsb = p->gate_stride_b ? p->gate_stride_b : p->Lmax;
  a->gate_eps = p->gate_eps;
  a->gate_tau = p->gate_tau;
  a->gate_sink = p->gate_sink;
  a->out_f32 = p->out_dtype == SIGATTN_F32 ? 1 : 0;
  a->f16_pv = (pass == 0 && p->fast_math == 2) ? 1 : 0;
  order_blocks(a, pass);
  snake_if_one_round(a, pass, p->d, a->nitems);
}

bool needs_zero_fill(const sigattn_problem* p) {
  for (int b = 0; b < p->B; ++b)
    if (p->seqlens[b] < p->Lmax) return true;
  return false;
}

sigattn_status zero_fill(const sigattn_problem* p, void* o0, void* o1, hipStream_t st,
                         void* o2 = nullptr) {
  if (!needs_zero_fill(p)) return SIGATTN_OK;
  sa::ZArgs z;
  std::memset(&z, 0, sizeof(z));
  z.o0 = o0;
  z.o1 = o1;
  z.o2 = o2;
  int nmin = p->Lmax;
  for (int b = 0; b < p->B; ++b) nmin = p->seqlens[b] < nmin ? p->seqlens[b] : nmin;
  z.block0 = nmin / sa::kZeroRows;   // nmin < Lmax here, so at least one block remains
  z.sb = p->stride_b;
  z.sh = p->stride_h;
  z.sl = p->stride_l;
  z.Lmax = p->Lmax;
  z.esize = out_elem_size(p);
  z.row_bytes = p->d * z.esize;
  for (int b = 0; b < p->B; ++b) z.len[b] = (uint16_t)p->seqlens[b];
  return sa::launch_zero_rows(z, p->B, p->H, st) == hipSuccess ? SIGATTN_OK : SIGATTN_ERR_HIP;
}

// Zero the padded entries of a per-head float plane and, if `sum` is set, reduce it over
// heads; enqueued after the pass that wrote the valid entries.
sigattn_status plane_tail(const sigattn_problem* p, float* plane, float* sum, hipStream_t st) {
  sa::PArgs pa;
  std::memset(&pa, 0, sizeof(pa));
  pa.plane = plane;
  pa.sum = sum;
  pa.B = p->B;
  pa.H = p->H;
  pa.Lmax = p->Lmax;
  for (int b = 0; b < p->B; ++b) pa.len[b] = (uint16_t)p->seqlens[b];
  return sa::launch_plane_tail(pa, st) == hipSuccess ? SIGATTN_OK : SIGATTN_ERR_HIP;
}

sigattn_status run_f32(const sigattn_problem* p, int pass, const void* q, const void* k,
                       const void* v, const void* dout, void* o0, void* o1, float* aux,
                       hipStream_t st) {
  sa::DArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.out0 = o0; a.out1 = o1; a.aux = aux;
  a.gate = p->gate;
  a.sb = p->stride_b; a.sh = p->stride_h; a.sl = p->stride_l;
  a.gsb = p->gate_stride_b ? p->gate_stride_b : p->Lmax;
  a.B = p->B; a.H = p->H; a.Lmax = p->Lmax; a.d = p->d;
  a.causal = p->causal;
  a.gate_sink = p->gate_sink;
  a.scale = (float)scale_of(p);
  a.gate_eps = p->gate_eps;
  a.gate_tau = p->gate_tau;
  for (int b = 0; b < p->B; ++b) {
    a.len[b] = p->seqlens[b];
    a.beta[b] = (float)beta_of(p, b);
  }
  if (sa::launch_f32(a, pass, st) != hipSuccess) return SIGATTN_ERR_HIP;
  return zero_fill(p, o0, o1, st);
}

// aux: the per-head float plane of the pass (row mass for the forward, gate gradient for
// the dk/dv pass) or null; aux_sum: its sum over heads or null.
sigattn_status run_pass(const sigattn_problem* p, int pass, const void* q, const void* k,
                        const void* v, const void* dout, void* o0, void* o1, void* stream,
                        float* aux = nullptr, float* aux_sum = nullptr) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (p->B == 0) return SIGATTN_OK;
  sigattn_status s;
  if (p->dtype == SIGATTN_F32) {
    s = run_f32(p, pass, q, k, v, dout, o0, o1, aux, st);
    if (s != SIGATTN_OK || !aux) return s;
    return plane_tail(p, aux, aux_sum, st);
  }
  KArgs a;
  plan_pass(p, pass, &a);
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.out0 = o0; a.out1 = o1; a.aux = aux;
  const bool causal = p->causal != 0, gated = p->gate != nullptr;
  if (a.nitems > 0) {
    hipError_t e;
    const bool split = p->fast_math != 1;
    if (pass == 0) e = sa::launch_fwd_bf16(a, p->d, causal, gated, split, st);
    else if (pass == 1) e = sa::launch_dq_bf16(a, p->d, causal, gated, split, st);
    else e = sa::launch_dkdv_bf16(a, p->d, causal, gated, split, st);
    if (e != hipSuccess) return SIGATTN_ERR_HIP;
  }
  if ((s = zero_fill(p, o0, o1, st)) != SIGATTN_OK || !aux) return s;
  return plane_tail(p, aux, aux_sum, st);
}

// A per-head float plane or its head sum: 4-byte aligned, distinct from every tensor.
sigattn_status check_plane(const void* plane, const void* const* others, int nothers) {
  if (!plane) return SIGATTN_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(plane) & 3u) return SIGATTN_ERR_ALIGNMENT;
  for (int i = 0; i < nothers; ++i)
    if (others[i] == plane) return SIGATTN_ERR_INVALID_ARG;
  return SIGATTN_OK;
}

// ---------------------------------- packed batches ----------------------------------

sigattn_status validate_varlen(const sigattn_varlen* p) {
  if (!p) return SIGATTN_ERR_INVALID_ARG;
  if (p->struct_size != sizeof(sigattn_varlen)) return SIGATTN_ERR_INVALID_ARG;
  if (p->B < 0 || p->H < 1 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0)
    return SIGATTN_ERR_INVALID_ARG;
  if (p->d != 64 && p->d != 128) return SIGATTN_ERR_UNSUPPORTED;
  if (p->out_dtype != SIGATTN_BF16 && p->out_dtype != SIGATTN_F32) return SIGATTN_ERR_UNSUPPORTED;
  if (p->fast_math < 0 || p->fast_math > 2) return SIGATTN_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return SIGATTN_ERR_INVALID_ARG;
  if (p->stride_t < 0 || p->stride_h < 0) return SIGATTN_ERR_INVALID_ARG;
  if (p->stride_t > SIGATTN_MAX_ROW_STRIDE) return SIGATTN_ERR_UNSUPPORTED;
  if (((p->stride_t * 2) & 15) || ((p->stride_h * 2) & 15)) return SIGATTN_ERR_ALIGNMENT;
  {
    // packed rows of different (row, head) must not overlap; the row count is on the
    // device, bounded by B times the larger of the two maximum lengths
    const int64_t rows = (int64_t)p->B * (p->max_seqlen_q > p->max_seqlen_k ? p->max_seqlen_q
                                                                             : p->max_seqlen_k);
    const int64_t stride[2] = {p->stride_t, p->stride_h};
    const int64_t count[2] = {rows > 2 ? rows : 2, p->H};
    if (!rows_disjoint(p->d, stride, count, 2)) return SIGATTN_ERR_INVALID_ARG;
  }
  if (!std::isfinite(p->scale) || p->scale < 0.0f) return SIGATTN_ERR_INVALID_ARG;
  if (p->B > 0 && (!p->cu_seqlens_q || !p->cu_seqlens_k)) return SIGATTN_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(p->cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(p->cu_seqlens_k) & 3u) ||
      (reinterpret_cast<uintptr_t>(p->bias) & 3u) || (reinterpret_cast<uintptr_t>(p->gate) & 3u))
    return SIGATTN_ERR_ALIGNMENT;
  if (p->gate) {
    if (!std::isfinite(p->gate_eps) || p->gate_eps < 0.0f) return SIGATTN_ERR_INVALID_ARG;
    if (!std::isfinite(p->gate_tau) || p->gate_tau < 0.0f) return SIGATTN_ERR_INVALID_ARG;
    if (p->gate_sink < 0) return SIGATTN_ERR_INVALID_ARG;
  }
  for (int pass = 0; pass < 3; ++pass) {
    const int64_t rows = pass == 2 ? p->max_seqlen_k : p->max_seqlen_q;
    const int tile = pass == 0 ? sa::fwd_tile_rows(p->d) : pass == 1 ? sa::dq_tile_rows(p->d)
                                                                    : sa::dkdv_tile_rows(p->d);
    if ((int64_t)p->B * p->H * ((rows + tile - 1) / tile) > SIGATTN_MAX_ITEMS)
      return SIGATTN_ERR_UNSUPPORTED;
  }
  return SIGATTN_OK;
}

// The kernel arguments of a packed-batch pass.
void plan_varlen(const sigattn_varlen* p, int pass, const void* q, const void* k,
                 const void* v, const void* dout, void* o0, void* o1, KArgs& a) {
  std::memset(&a, 0, sizeof(a));
  const int tile = tile_rows_d(p->d, pass);
  const int64_t rows = pass == 2 ? p->max_seqlen_k : p->max_seqlen_q;
  a.varlen = 1;
  a.tile = tile;
  a.tiles_per_seq = (int32_t)((rows + tile - 1) / tile);
  a.tiles_over_keys = pass == 2 ? 1 : 0;
  a.nitems = (int32_t)((int64_t)p->B * p->H * a.tiles_per_seq);
  a.Lmax = p->max_seqlen_q;   // packed mode: the longest query row count (kernel choice)
  a.cu_q = p->cu_seqlens_q;
  a.cu_k = p->cu_seqlens_k;
  a.bias = p->bias;
  a.H = p->H;
  a.xcd_chunk = xcd_chunk_default();
  a.causal = p->causal;
  a.sl = p->stride_t;
  a.sh = p->stride_h;
  const double s = p->scale != 0.0f ? (double)p->scale : 1.0 / std::sqrt((double)p->d);
  a.scale = (float)s;
  a.c1 = (float)(-s * kLog2eD);
  a.gate = p->gate;
  a.gate_eps = p->gate_eps;
  a.gate_tau = p->gate_tau;
  a.gate_sink = p->gate_sink;
  a.out_f32 = p->out_dtype == SIGATTN_F32 ? 1 : 0;
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.out0 = o0; a.out1 = o1;
  a.f16_pv = (pass == 0 && p->fast_math == 2) ? 1 : 0;
  if (p->causal && p->B > 0) {
    // block-major, costs at the maximum lengths; item g reads sequence (g % (B H)) / H
    a.nsorted = p->B;
    const int t = a.tiles_per_seq;
    set_blocks(&a, pass, p->max_seqlen_q, p->max_seqlen_k, pass == 2 ? 0 : t, pass == 2 ? t : 0);
    snake_if_one_round(&a, pass, p->d, a.nitems);
  }
}

sigattn_status run_varlen(const sigattn_varlen* p, int pass, const void* q, const void* k,
                          const void* v, const void* dout, void* o0, void* o1, void* stream) {
  KArgs a;
  plan_varlen(p, pass, q, k, v, dout, o0, o1, a);
  if (a.nitems == 0) return SIGATTN_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool causal = p->causal != 0, gated = p->gate != nullptr, split = p->fast_math != 1;
  hipError_t e;
  if (pass == 0) e = sa::launch_fwd_bf16(a, p->d, causal, gated, split, st);
  else if (pass == 1) e = sa::launch_dq_bf16(a, p->d, causal, gated, split, st);
  else e = sa::launch_dkdv_bf16(a, p->d, causal, gated, split, st);
  return e == hipSuccess ? SIGATTN_OK : SIGATTN_ERR_HIP;
}

// ------------------------------------ KV cache ------------------------------------

constexpr int64_t kMaxCacheCap = int64_t(1) << 24;

sigattn_status validate_cache(const sigattn_cache* c) {
  if (!c) return SIGATTN_ERR_INVALID_ARG;
  if (c->struct_size != sizeof(sigattn_cache)) return SIGATTN_ERR_INVALID_ARG;
  if (c->B < 0 || c->H < 1 || c->cap < 1) return SIGATTN_ERR_INVALID_ARG;
  if (c->B > SIGATTN_MAX_BATCH || c->cap > kMaxCacheCap) return SIGATTN_ERR_UNSUPPORTED;
  if (c->d != 64 && c->d != 128) return SIGATTN_ERR_UNSUPPORTED;
  if (c->stride_b < 0 || c->stride_h < 0 || c->stride_l < c->d) return SIGATTN_ERR_INVALID_ARG;
  if (c->stride_l > SIGATTN_MAX_ROW_STRIDE) return SIGATTN_ERR_UNSUPPORTED;
  if (((c->stride_l * 2) & 15) || ((c->stride_h * 2) & 15) || ((c->stride_b * 2) & 15))
    return SIGATTN_ERR_ALIGNMENT;
  if (!c->k || !c->v || !c->count || !c->seen) return SIGATTN_ERR_INVALID_ARG;
  if (!aligned16(c->k) || !aligned16(c->v)) return SIGATTN_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(c->count) & 3u) || (reinterpret_cast<uintptr_t>(c->seen) & 3u) ||
      (reinterpret_cast<uintptr_t>(c->gate) & 3u))
    return SIGATTN_ERR_ALIGNMENT;
  if (c->k == c->v || c->count == c->seen) return SIGATTN_ERR_INVALID_ARG;
  if (!std::isfinite(c->gate_eps) || c->gate_eps < 0.0f) return SIGATTN_ERR_INVALID_ARG;
  if (!std::isfinite(c->gate_tau) || c->gate_tau < 0.0f) return SIGATTN_ERR_INVALID_ARG;
  if (c->gate_sink < 0) return SIGATTN_ERR_INVALID_ARG;
  return SIGATTN_OK;
}

sa::CacheView cache_view(const sigattn_cache* c) {
  sa::CacheView v;
  std::memset(&v, 0, sizeof(v));
  v.k = c->k;
  v.v = c->v;
  v.gate = c->gate;
  v.count = c->count;
  v.seen = c->seen;
  v.sb = c->stride_b;
  v.sh = c->stride_h;
  v.sl = c->stride_l;
  v.H = c->H;
  v.cap = c->cap;
  v.d = c->d;
  v.gate_eps = c->gate_eps;
  v.gate_tau = c->gate_tau;
  v.gate_sink = c->gate_sink;
  return v;
}

int64_t decode_chunks(const sigattn_cache* c) { return (c->cap + sa::kDecChunk - 1) / sa::kDecChunk; }

int64_t decode_ws_bytes(const sigattn_cache* c) {
  return (int64_t)c->B * c->H * decode_chunks(c) * c->d * (int64_t)sizeof(float);
}

// q/o rows ([B][H][d] with element strides sb, sh) must start on 16-byte boundaries
bool rows16(int64_t sb, int64_t sh, int esize) {
  return sb >= 0 && sh >= 0 && ((sb * esize) & 15) == 0 && ((sh * esize) & 15) == 0;
}

// Single-query decode. internal_ws: the partial sums go to the library's static device
// workspace (the allocation-free entry point) instead of the caller's `workspace`.
sigattn_status decode_call(const sigattn_cache* c, const void* q, int64_t stride_b,
                           int64_t stride_h, const float* bias, float scale, void* o,
                           int32_t out_dtype, void* workspace, int64_t workspace_bytes,
                           void* stream, bool internal_ws) {
  sigattn_status s = validate_cache(c);
  if (s != SIGATTN_OK) return s;
  if (out_dtype != SIGATTN_BF16 && out_dtype != SIGATTN_F32) return SIGATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || scale < 0.0f) return SIGATTN_ERR_INVALID_ARG;
  if (c->B > 0 && !bias) return SIGATTN_ERR_INVALID_ARG;
  for (int b = 0; b < c->B; ++b)
    if (!std::isfinite(bias[b])) return SIGATTN_ERR_INVALID_ARG;
  if (!q || !o || (!internal_ws && !workspace)) return SIGATTN_ERR_INVALID_ARG;
  const int osize = out_dtype == SIGATTN_F32 ? 4 : 2;
  if (!aligned16(q) || !aligned16(o) || !aligned16(workspace) || !rows16(stride_b, stride_h, 2) ||
      !rows16(stride_b, stride_h, osize))
    return SIGATTN_ERR_ALIGNMENT;
  if (stride_h < c->d && c->H > 1) return SIGATTN_ERR_INVALID_ARG;
  if (internal_ws) {
    if (decode_ws_bytes(c) > SIGATTN_NOALLOC_WORKSPACE_BYTES) return SIGATTN_ERR_UNSUPPORTED;
  } else if (workspace_bytes < decode_ws_bytes(c)) {
    return SIGATTN_ERR_INVALID_ARG;
  }
  const void* bufs[7] = {c->k, c->v, c->gate, c->count, c->seen, q, workspace};
  for (int i = 0; i < 7; ++i) {
    if (bufs[i] && bufs[i] == o) return SIGATTN_ERR_INVALID_ARG;
    if (i < 6 && bufs[i] && bufs[i] == workspace) return SIGATTN_ERR_INVALID_ARG;
  }
  if (c->B == 0) return SIGATTN_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  if (internal_ws && sa::noalloc_scratch(st, &ws) != hipSuccess) return SIGATTN_ERR_HIP;
  sa::DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.c = cache_view(c);
  a.q = q;
  a.out = o;
  a.ws = ws;
  a.qsb = stride_b;
  a.qsh = stride_h;
  a.B = c->B;
  a.nchunk = (int32_t)decode_chunks(c);
  a.out_f32 = out_dtype == SIGATTN_F32 ? 1 : 0;
  const double sc = scale != 0.0f ? (double)scale : 1.0 / std::sqrt((double)c->d);
  a.c1 = (float)(-sc * kLog2eD);
  for (int b = 0; b < c->B; ++b) a.c2[b] = (float)(-(double)bias[b] * kLog2eD);
  return sa::launch_decode(a, st) == hipSuccess ? SIGATTN_OK : SIGATTN_ERR_HIP;
}

}  // namespace

extern "C" {

sigattn_status sigattn_validate(const sigattn_problem* p) { return validate_problem(p); }

sigattn_status sigattn_fwd(const sigattn_problem* p, const void* q, const void* k,
                           const void* v, void* o, void* stream) {
  sigattn_status s = validate_problem(p);
  if (s != SIGATTN_OK) return s;
  const void* in[3] = {q, k, v};
  void* out[1] = {o};
  if ((s = check_tensors(in, 3, out, 1)) != SIGATTN_OK) return s;
  return run_pass(p, 0, q, k, v, nullptr, o, nullptr, stream);
}

sigattn_status sigattn_fwd_rowsum(const sigattn_problem* p, const void* q, const void* k,
                                  const void* v, void* o, float* row_mass, void* stream) {
  sigattn_status s = validate_problem(p);
  if (s != SIGATTN_OK) return s;
  const void* in[3] = {q, k, v};
  void* out[1] = {o};
  if ((s = check_tensors(in, 3, out, 1)) != SIGATTN_OK) return s;
  const void* others[5] = {q, k, v, o, p->gate};
  if ((s = check_plane(row_mass, others, 5)) != SIGATTN_OK) return s;
  return run_pass(p, 0, q, k, v, nullptr, o, nullptr, stream, row_mass, nullptr);
}

sigattn_status sigattn_bwd_dq(const sigattn_problem* p, const void* q, const void* k,
                              const void* v, const void* dout, void* dq, void* stream) {
  sigattn_status s = validate_problem(p);
  if (s != SIGATTN_OK) return s;
  const void* in[4] = {q, k, v, dout};
  void* out[1] = {dq};
  if ((s = check_tensors(in, 4, out, 1)) != SIGATTN_OK) return s;
  return run_pass(p, 1, q, k, v, dout, dq, nullptr, stream);
}

sigattn_status sigattn_bwd_dkdv(const sigattn_problem* p, const void* q, const void* k,
                                const void* v, const void* dout, void* dk, void* dv,
                                void* stream) {
  sigattn_status s = validate_problem(p);
  if (s != SIGATTN_OK) return s;
  const void* in[4] = {q, k, v, dout};
  void* out[2] = {dk, dv};
  if ((s = check_tensors(in, 4, out, 2)) != SIGATTN_OK) return s;
  return run_pass(p, 2, q, k, v, dout, dk, dv, stream);
}

sigattn_status sigattn_bwd(const sigattn_problem* p, const void* q, const void* k,
                           const void* v, const void* dout, void* dq, void* dk, void* dv,
                           void* stream) {
  sigattn_status s = validate_problem(p);
  if (s != SIGATTN_OK) return s;
  const void* in[4] = {q, k, v, dout};
  void* out[3] = {dq, dk, dv};
  if ((s = check_tensors(in, 4, out, 3)) != SIGATTN_OK) return s;
  if (p->B == 0) return SIGATTN_OK;
  if (p->dtype == SIGATTN_F32 || p->d != 64) {
    // one kernel after the other (at d = 128 the dK/dV kernel runs one wave per SIMD and
    // the dQ kernel two, so sharing a launch would hold the dQ items to one)
    if ((s = run_pass(p, 2, q, k, v, dout, dk, dv, stream)) != SIGATTN_OK) return s;
    return run_pass(p, 1, q, k, v, dout, dq, nullptr, stream);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  KArgs a;
  plan_pass(p, 2, &a);
  order_blocks(&a, 3);
  snake_if_one_round(&a, 3, p->d, 2 * a.nitems);
  a.q = q; a.k = k; a.v = v; a.dout = dout; a.out0 = dk; a.out1 = dv;
  if (a.nitems > 0 && sa::launch_bwd_bf16(a, dq, a.nitems, 0, p->causal != 0, p->gate != nullptr,
                                          p->fast_math != 1, st) != hipSuccess)
    return SIGATTN_ERR_HIP;
  return zero_fill(p, dk, dv, st, dq);
}

sigattn_status sigattn_bwd_dkdv_dg(const sigattn_problem* p, const void* q, const void* k,
                                   const void* v, const void* dout, void* dk, void* dv,
                                   float* dg_head, float* dg, void* stream) {
  sigattn_status s = validate_problem(p);
  if (s != SIGATTN_OK) return s;
  if (!p->gate) return SIGATTN_ERR_INVALID_ARG;
  const void* in[4] = {q, k, v, dout};
  void* out[2] = {dk, dv};
  if ((s = check_tensors(in, 4, out, 2)) != SIGATTN_OK) return s;
  const void* others[7] = {q, k, v, dout, dk, dv, p->gate};
  if ((s = check_plane(dg_head, others, 7)) != SIGATTN_OK) return s;
  if (dg) {
    const void* others2[8] = {q, k, v, dout, dk, dv, p->gate, dg_head};
    if ((s = check_plane(dg, others2, 8)) != SIGATTN_OK) return s;
  }
  return run_pass(p, 2, q, k, v, dout, dk, dv, stream, dg_head, dg);
}

sigattn_status sigattn_fwd_varlen(const sigattn_varlen* p, const void* q, const void* k,
                                  const void* v, void* o, void* stream) {
  sigattn_status s = validate_varlen(p);
  if (s != SIGATTN_OK) return s;
  const void* in[3] = {q, k, v};
  void* out[1] = {o};
  if ((s = check_tensors(in, 3, out, 1)) != SIGATTN_OK) return s;
  return run_varlen(p, 0, q, k, v, nullptr, o, nullptr, stream);
}

sigattn_status sigattn_bwd_dq_varlen(const sigattn_varlen* p, const void* q, const void* k,
                                     const void* v, const void* dout, void* dq, void* stream) {
  sigattn_status s = validate_varlen(p);
  if (s != SIGATTN_OK) return s;
  const void* in[4] = {q, k, v, dout};
  void* out[1] = {dq};
  if ((s = check_tensors(in, 4, out, 1)) != SIGATTN_OK) return s;
  return run_varlen(p, 1, q, k, v, dout, dq, nullptr, stream);
}

sigattn_status sigattn_bwd_dkdv_varlen(const sigattn_varlen* p, const void* q,
                                       const void* k, const void* v, const void* dout,
                                       void* dk, void* dv, void* stream) {
  sigattn_status s = validate_varlen(p);
  if (s != SIGATTN_OK) return s;
  const void* in[4] = {q, k, v, dout};
  void* out[2] = {dk, dv};
  if ((s = check_tensors(in, 4, out, 2)) != SIGATTN_OK) return s;
  return run_varlen(p, 2, q, k, v, dout, dk, dv, stream);
}

sigattn_status sigattn_bwd_varlen(const sigattn_varlen* p, const void* q, const void* k,
                                  const void* v, const void* dout, void* dq, void* dk, void* dv,
                                  void* stream) {
  sigattn_status s = validate_varlen(p);
  if (s != SIGATTN_OK) return s;
  const void* in[4] = {q, k, v, dout};
  void* out[3] = {dq, dk, dv};
  if ((s = check_tensors(in, 4, out, 3)) != SIGATTN_OK) return s;
  if (p->d != 64) {
    if ((s = run_varlen(p, 2, q, k, v, dout, dk, dv, stream)) != SIGATTN_OK) return s;
    return run_varlen(p, 1, q, k, v, dout, dq, nullptr, stream);
  }
  KArgs a;
  plan_varlen(p, 2, q, k, v, dout, dk, dv, a);
  const int tile = tile_rows_d(p->d, 1);
  const int tiles_q = (int)((p->max_seqlen_q + tile - 1) / tile);
  const int nq_items = (int)((int64_t)p->B * p->H * tiles_q);
  if (a.nitems + nq_items == 0) return SIGATTN_OK;
  if (p->causal) {
    set_blocks(&a, 3, p->max_seqlen_q, p->max_seqlen_k, tiles_q, a.tiles_per_seq);
    snake_if_one_round(&a, 3, p->d, a.nitems + nq_items);
  }
  return sa::launch_bwd_bf16(a, dq, nq_items, tiles_q, p->causal != 0, p->gate != nullptr,
                             p->fast_math != 1, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? SIGATTN_OK : SIGATTN_ERR_HIP;
}

sigattn_status sigattn_cache_build(const sigattn_cache* c, const sigattn_problem* p,
                                   const void* k, const void* v, void* stream) {
  sigattn_status s = validate_cache(c);
  if (s != SIGATTN_OK) return s;
  if ((s = validate_problem(p)) != SIGATTN_OK) return s;
  if (p->dtype != SIGATTN_BF16) return SIGATTN_ERR_UNSUPPORTED;
  if (p->B != c->B || p->H != c->H || p->d != c->d) return SIGATTN_ERR_INVALID_ARG;
  if ((p->gate == nullptr) != (c->gate == nullptr)) return SIGATTN_ERR_INVALID_ARG;
  for (int b = 0; b < p->B; ++b)
    if (p->seqlens[b] > c->cap) return SIGATTN_ERR_INVALID_ARG;
  const void* in[2] = {k, v};
  if (!k || !v) return SIGATTN_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v)) return SIGATTN_ERR_ALIGNMENT;
  const void* outs[5] = {c->k, c->v, c->gate, c->count, c->seen};
  for (const void* i : in)
    for (const void* o : outs)
      if (o && i == o) return SIGATTN_ERR_INVALID_ARG;
  if (p->B == 0) return SIGATTN_OK;
  sa::BuildArgs a;
  std::memset(&a, 0, sizeof(a));
  a.c = cache_view(c);
  a.k = k;
  a.v = v;
  a.gate = p->gate;
  a.sb = p->stride_b;
  a.sh = p->stride_h;
  a.sl = p->stride_l;
  a.gsb = p->gate_stride_b ? p->gate_stride_b : p->Lmax;
  a.Lmax = p->Lmax;
  for (int b = 0; b < p->B; ++b) a.len[b] = (uint16_t)p->seqlens[b];
  return sa::launch_cache_build(a, p->B, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? SIGATTN_OK : SIGATTN_ERR_HIP;
}

sigattn_status sigattn_cache_append(const sigattn_cache* c, const void* k_new,
                                    const void* v_new, int64_t stride_b, int64_t stride_h,
                                    const float* g_new, int32_t* status, void* stream) {
  sigattn_status s = validate_cache(c);
  if (s != SIGATTN_OK) return s;
  if (!k_new || !v_new || k_new == v_new) return SIGATTN_ERR_INVALID_ARG;
  if ((g_new == nullptr) != (c->gate == nullptr)) return SIGATTN_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !rows16(stride_b, stride_h, 2))
    return SIGATTN_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(g_new) & 3u) || (reinterpret_cast<uintptr_t>(status) & 3u))
    return SIGATTN_ERR_ALIGNMENT;
  const void* outs[5] = {c->k, c->v, c->gate, c->count, c->seen};
  for (const void* o : outs) {
    if (!o) continue;
    if (o == k_new || o == v_new || o == g_new || o == status) return SIGATTN_ERR_INVALID_ARG;
  }
  if (c->B == 0) return SIGATTN_OK;
  sa::AppendArgs a;
  std::memset(&a, 0, sizeof(a));
  a.c = cache_view(c);
  a.k = k_new;
  a.v = v_new;
  a.gate = g_new;
  a.nsb = stride_b;
  a.nsh = stride_h;
  a.status = status;
  return sa::launch_cache_append(a, c->B, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? SIGATTN_OK : SIGATTN_ERR_HIP;
}

int64_t sigattn_decode_workspace_size(const sigattn_cache* c) {
  if (validate_cache(c) != SIGATTN_OK) return -1;
  return decode_ws_bytes(c);
}

sigattn_status sigattn_decode(const sigattn_cache* c, const void* q, int64_t stride_b,
                              int64_t stride_h, const float* bias, float scale, void* o,
                              int32_t out_dtype, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  return decode_call(c, q, stride_b, stride_h, bias, scale, o, out_dtype, workspace,
                     workspace_bytes, stream, false);
}

sigattn_status sigattn_decode_noalloc(const sigattn_cache* c, const void* q, int64_t stride_b,
                                      int64_t stride_h, const float* bias, float scale, void* o,
                                      int32_t out_dtype, void* stream) {
  return decode_call(c, q, stride_b, stride_h, bias, scale, o, out_dtype, nullptr, 0, stream,
                     true);
}

int64_t sigattn_plan(const sigattn_problem* p, int32_t pass, int32_t* items, int64_t cap,
                     int32_t* tile_rows_out) {
  if (validate_problem(p) != SIGATTN_OK || pass < 0 || pass > 3) return -1;
  if (pass == 3 && p->d != 64) return -1;
  if (cap > 0 && !items) return -1;
  if (p->B == 0) return 0;
  KArgs a;
  plan_pass(p, pass == 3 ? 2 : pass, &a);
  if (tile_rows_out) *tile_rows_out = a.tile;
  if (pass < 3) {
    for (int w = 0; w < a.nitems && w < cap; ++w) {
      const sa::Item it = sa::decode_item(a, sa::remap_block(w, a.nitems, a.xcd_chunk));
      items[3 * w + 0] = it.b;
      items[3 * w + 1] = it.h;
      items[3 * w + 2] = it.t;
    }
    return a.nitems;
  }
  // the one-call backward: the dK/dV list, then the dQ list (the dQ pass's order with
  // the dK/dV pass's tiles), or both merged block-major; dQ items as (b, h, -1 - tile)
  order_blocks(&a, 3);
  const int total = 2 * a.nitems;
  snake_if_one_round(&a, 3, p->d, total);
  for (int w = 0; w < total && w < cap; ++w) {
    const int g = sa::remap_block(w, total, a.xcd_chunk);
    bool dq_item = g >= a.nitems;
    sa::Item it;
    if (p->causal && a.nblocks > 0) it = sa::decode_block_item(a, g, &dq_item);
    else if (!dq_item) it = sa::decode_item(a, g, 0);
    else it = sa::decode_item(a, g - a.nitems, p->causal ? 1 : 0);
    items[3 * w + 0] = it.b;
    items[3 * w + 1] = it.h;
    items[3 * w + 2] = dq_item ? -1 - it.t : it.t;
  }
  return total;
}

sigattn_status sigattn_calibrate_mfma(int32_t nblocks, int32_t iters, float* sink,
                                      int64_t* clk, void* stream) {
  if (nblocks < 1 || nblocks > SIGATTN_MAX_CALIB_BLOCKS || iters < 1 ||
      iters > SIGATTN_MAX_CALIB_ITERS || (int64_t)nblocks * iters > SIGATTN_MAX_CALIB_WORK ||
      !sink || !clk)
    return SIGATTN_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(sink) & 3u) || (reinterpret_cast<uintptr_t>(clk) & 7u))
    return SIGATTN_ERR_ALIGNMENT;
  return sa::launch_mfma_calib(sink, clk, nblocks, iters, reinterpret_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? SIGATTN_OK
             : SIGATTN_ERR_HIP;
}

double sigattn_calibrate_mfma_flops(int32_t nblocks, int32_t iters) {
  if (nblocks < 1 || iters < 1) return 0.0;
  // 4 waves per workgroup; 32 x 32 x 16 products, 2 flops each
  return (double)nblocks * 4.0 * (double)iters * sa::calib_mfma_per_iter() * 32.0 * 32.0 * 16.0 * 2.0;
}

const char* sigattn_status_string(sigattn_status s) {
  switch (s) {
    case SIGATTN_OK: return "ok";
    case SIGATTN_ERR_INVALID_ARG: return "invalid argument";
    case SIGATTN_ERR_UNSUPPORTED: return "unsupported problem";
    case SIGATTN_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case SIGATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int sigattn_version(void) { return SIGATTN_VERSION; }

}  // extern "C"
