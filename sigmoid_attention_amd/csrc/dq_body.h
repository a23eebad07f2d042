// Backward pass, query side, on gfx950:
//   dQ_i = s sum_j dS_ij k_j,  dS_ij = (dO_i . V'_j) P_ij (1 - P_ij)
// P is recomputed from Q and K rather than stored ("Better Models, Faster Training:
// Sigmoid Attention for single-cell Foundation Models", section 4, backward pass
// decomposition: one kernel for dQ, one for dK/dV, no atomics). The factor
// P(1 - P) is the diagonal of the sigmoid Jacobian (appendix A.1.2).
//
// One workgroup = 4 waves = one item (b, h, query tile of 128). Each wave keeps its 32
// Q and dO rows in registers as B operands. K and V stream through the same 3-stage LDS
// ring as the forward (direct loads two tiles ahead, one barrier per tile). Per 32-key
// chunk c (a unit): S^T = K Q^T and dP^T = V dO^T (MFMA) of chunk c+1 are computed while
// the VALU turns S(c), dP(c) into dS(c) (fp32, then bf16 hi + lo when SPLIT), and
// dQ^T += K^T dS^T (K^T read with transposed LDS loads) for the first key half of c;
// the second key half is deferred into the next unit.
#pragma once

#include <type_traits>

#include "common.h"

namespace sa {

template <int D, int CPT, bool GATED>
struct DqTraits {
  static constexpr int kThreads = 256;
  static constexpr int kWaves = 4;
  static constexpr int BM = kWaves * 32;        // queries per work item
  static constexpr int BN = 32 * CPT;           // keys per LDS tile
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int TILE = BN * D * 2;
  static constexpr int TAB = GATED ? 2 * BN * 4 : 0;
  static constexpr int STAGE = 2 * TILE + TAB;  // K tile, V tile, gate table
  static constexpr int NSTAGE = 3;
};

enum DqMode { kDqInterior = 0, kDqMasked = 1 };

__device__ __forceinline__ constexpr int dq_arc(int r) { return 8 * (r >> 2) + (r & 3); }

// The dQ pass of one work item `it` (wave-uniform), by the 4 waves of a 256-thread
// workgroup: `smem` is the LDS ring (DqTraits::NSTAGE * STAGE bytes, 1024-aligned) and
// dQ goes to `out`. VL: packed batch (separate query and key lengths, bottom-right
// causal diagonal).
template <int D, int CPT, bool CAUSAL, bool GATED, bool SPLIT, bool VL>
__device__ __forceinline__ void dq_body(const KArgs& a, const Item& it, char* smem, void* out) {
  using T = DqTraits<D, CPT, GATED>;

  const int l = lane_id(), w = wave_id();
  const int lk = 4 * (l >> 5);
  const SplitSel sel;
  const int nq = it.nq, nk = VL ? it.nk : it.nq, diag = VL ? it.diag : 0;
  const int lastq = nq - 1, lastk = nk - 1;
  const int64_t koff = VL ? it.koff : it.qoff;
  const bf16* Qg = (const bf16*)a.q + it.qoff;
  const bf16* Kg = (const bf16*)a.k + koff;
  const bf16* Vg = (const bf16*)a.v + koff;
  const bf16* dOg = (const bf16*)a.dout + it.qoff;
  const float* Gg = GATED ? a.gate + it.goff : nullptr;
  const int64_t sl = a.sl;
  const int item_q0 = it.t * T::BM;
  const int q0 = item_q0 + w * 32;
  const float c1 = a.c1, c2 = it.c2;

  int kend = nk;
  if (CAUSAL) {
    const int e = (item_q0 + T::BM < nq ? item_q0 + T::BM : nq) + diag;
    kend = e < 0 ? 0 : (e < nk ? e : nk);
  }
  const int nch = (kend + 31) / 32;
  const int ntiles = (nch + CPT - 1) / CPT;
  int wch = q0 < nq ? nch : 0;
  if (CAUSAL && q0 < nq) {
    const int lk_allowed = (q0 + 32 < nq ? q0 + 32 : nq) - 1 + diag;
    wch = lk_allowed < 0 ? 0 : (lk_allowed / 32 + 1 < nch ? lk_allowed / 32 + 1 : nch);
  }

  const DirectPair<T::BN, D, T::kWaves> dma(sl);
  auto issue_tile = [&](int t) {
    dma.load(smem + (t % T::NSTAGE) * T::STAGE, Kg, Vg, sl, t * T::BN, lastk);
  };
  // gate table of tile t (as in the forward), written by wave 0 from gate values read
  // one tile ahead, so that the wait for them does not also wait for the direct loads
  const bool gate_lane = GATED && w == 0 && l < T::BN;
  auto gate_value = [&](int t) {
    const int key = t * T::BN + l;
    return Gg[key < lastk ? key : lastk];
  };
  auto store_table = [&](int t, float g) {
    if (gate_lane) {
      float* tab = reinterpret_cast<float*>(smem + (t % T::NSTAGE) * T::STAGE + 2 * T::TILE);
      const int key = t * T::BN + l;
      const bool keep = key < nk && !(key >= a.gate_sink && g < a.gate_tau);
      tab[l] = keep ? c2 - __builtin_amdgcn_logf(g + a.gate_eps) : __builtin_inff();
      tab[T::BN + l] = keep ? g : 0.0f;
    }
  };
  // gate values for the tables of tiles 0 and t + 1; the table of tile 0 is written once
  // the loads issued after them are awaited, before the barrier that publishes the tile
  float gfirst = 0.0f, gnext = 0.0f;
  if (gate_lane && ntiles > 0) gfirst = gate_value(0);
  if (gate_lane && ntiles > 1) gnext = gate_value(1);
  if (ntiles > 0) issue_tile(0);
  if (ntiles > 1) issue_tile(1);

  bf16x8 qop[T::KS], doop[T::KS];
  {
    int row = q0 + (l & 31);
    row = row < lastq ? row : lastq;
    const bf16* qr = Qg + (int64_t)row * sl + 8 * (l >> 5);
    const bf16* dr = dOg + (int64_t)row * sl + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      qop[ks] = *reinterpret_cast<const bf16x8*>(qr + 16 * ks);
      doop[ks] = *reinterpret_cast<const bf16x8*>(dr + 16 * ks);
    }
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      settle(qop[ks]);
      settle(doop[ks]);
    }
  }

  f32x16 acc[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) acc[dt] = zero16();

  if (ntiles > 0) store_table(0, gfirst);
  wait_vmem_and_barrier();

  // S^T and dP^T of chunk 0
  f32x16 s_cur = zero16(), dp_cur = zero16();
#pragma unroll
  for (int ks = 0; ks < (D == 64 ? T::KS : 0); ++ks) {
    s_cur = mfma(lds_row_operand<D>(smem, 0, 16 * ks), qop[ks], s_cur);
    dp_cur = mfma(lds_row_operand<D>(smem + T::TILE, 0, 16 * ks), doop[ks], dp_cur);
  }

  // dS of the 4 entries r0..r0+3 (fp32) into ds
  auto ds4 = [&](auto mode_tag, int r0, int kb, const float* tab, int krow, f32x16& ds) {
    constexpr int MODE = decltype(mode_tag)::value;
    f32x4 tc2, tg;
    if (GATED) {
      tc2 = *reinterpret_cast<const f32x4*>(tab + krow + 2 * r0 + lk);
      tg = *reinterpret_cast<const f32x4*>(tab + T::BN + krow + 2 * r0 + lk);
    }
    int lim = nk - 1 - kb - lk;
    if (CAUSAL) {
      const int ld = q0 + (l & 31) + diag - kb - lk;
      lim = ld < lim ? ld : lim;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + e;
      const float p = sigmoid_l2(s_cur[r], c1, GATED ? tc2[e] : c2);
      const float sp = __builtin_fmaf(-p, p, p);   // p (1 - p)
      float x = dp_cur[r] * (GATED ? sp * tg[e] : sp);
      if (MODE == kDqMasked) x = dq_arc(r) <= lim ? x : 0.0f;
      ds[r] = x;
    }
  };
  auto to_bf16 = [&](const f32x16& v, int h, bf16x8& hi, bf16x8& lo) {
    if (SPLIT) split8(v, 8 * h, hi, lo, sel);
    else hi = pack8(v, 8 * h);
  };

  bf16x8 dsh = {}, dsl = {}, dkc[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) dkc[dt] = bf16x8{};
  auto dq_mfma = [&](int dt, const bf16x8& kc, const bf16x8& hi, const bf16x8& lo) {
    acc[dt] = mfma(kc, hi, acc[dt]);
    if (SPLIT) acc[dt] = mfma(kc, lo, acc[dt]);
  };

  // One unit (chunk c): steps pair VALU work with MFMAs that do not depend on it.
  //   1: dS entries 0-3              | deferred dQ (second key half of chunk c-1)
  //   2: entries 4-7, to bf16 (h=0)  | S^T of chunk c+1
  //   3: entries 8-11                | dP^T of chunk c+1
  //   4: entries 12-15, to bf16 (h=1)| dQ for the first key half of chunk c
  const LdsLane<D> lane;
  auto unit = [&](auto mode_tag, const char* Kc, int krow, const char* Kn, int kn_row,
                  const char* Vn, const float* tab, int kb) {
    bf16x8 kop[T::KS], vop[T::KS], kc0[T::DT], kc1[T::DT];
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) kop[ks] = lane.rowop(Kn, kn_row, ks);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) kc0[dt] = lane.colop(Kc, krow, dt);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) vop[ks] = lane.rowop(Vn, kn_row, ks);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) kc1[dt] = lane.colop(Kc, krow + 16, dt);
    __builtin_amdgcn_sched_barrier(0);

    f32x16 ds;
    bf16x8 h0, l0, h1, l1;
    f32x16 s_next = zero16(), dp_next = zero16();
    // step 1
    ds4(mode_tag, 0, kb, tab, krow, ds);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) dq_mfma(dt, dkc[dt], dsh, dsl);
    __builtin_amdgcn_sched_barrier(0);
    // step 2
    ds4(mode_tag, 4, kb, tab, krow, ds);
    to_bf16(ds, 0, h0, l0);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) s_next = mfma(kop[ks], qop[ks], s_next);
    __builtin_amdgcn_sched_barrier(0);
    // step 3
    ds4(mode_tag, 8, kb, tab, krow, ds);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) dp_next = mfma(vop[ks], doop[ks], dp_next);
    __builtin_amdgcn_sched_barrier(0);
    // step 4
    ds4(mode_tag, 12, kb, tab, krow, ds);
    to_bf16(ds, 1, h1, l1);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) dq_mfma(dt, kc0[dt], h0, l0);
    __builtin_amdgcn_sched_barrier(0);
    s_cur = s_next;
    dp_cur = dp_next;
    dsh = h1;
    dsl = l1;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) dkc[dt] = kc1[dt];
  };

  // d = 128 (four times the operand registers): no cross-unit pipelining. S^T and dP^T of
  // chunk c are formed at the start of its unit, the K^T operands read per key half.
  auto unit_flat = [&](auto mode_tag, const char* Kc, int krow, const float* tab, int kb) {
    s_cur = zero16();
    dp_cur = zero16();
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      s_cur = mfma(lane.rowop(Kc, krow, ks), qop[ks], s_cur);
      dp_cur = mfma(lane.rowop(Kc + T::TILE, krow, ks), doop[ks], dp_cur);
    }
    f32x16 ds;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ds4(mode_tag, 8 * h, kb, tab, krow, ds);
      ds4(mode_tag, 8 * h + 4, kb, tab, krow, ds);
      bf16x8 hi, lo;
      to_bf16(ds, h, hi, lo);
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
        dq_mfma(dt, lane.colop(Kc, krow + 16 * h, dt), hi, lo);
    }
  };
  constexpr bool PIPE = D == 64;

  int cfirst = nk / 32;
  if (CAUSAL) {
    const int c = q0 + diag + 1 < 0 ? 0 : (q0 + diag + 1) / 32;
    cfirst = c < cfirst ? c : cfirst;
  }
  int tmask = cfirst / CPT;
  tmask = tmask < ntiles ? tmask : ntiles;
  if (q0 >= nq) tmask = 0;

  // `stage`: the ring slot of tile t, a compile-time constant in the unrolled interior
  // loop (LDS addresses fold into immediate offsets), or -1 when computed
  auto tile_body = [&](auto mode_tag, auto stage_tag, int t) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr int SG = decltype(stage_tag)::value;
    if (t > 0) wait_vmem_and_barrier();
    // gnext was read during the previous tile (or before the first) and has arrived
    if (t + 1 < ntiles) store_table(t + 1, gnext);
    if (t + 2 < ntiles) {
      if (gate_lane) gnext = gate_value(t + 2);
      issue_tile(t + 2);
    }
    const int st = SG >= 0 ? SG : t % T::NSTAGE;
    const int st1 = SG >= 0 ? (SG + 1) % T::NSTAGE : (t + 1) % T::NSTAGE;
    const char* cur = smem + st * T::STAGE;
    const char* nxt = smem + st1 * T::STAGE;
    const float* tab = reinterpret_cast<const float*>(cur + 2 * T::TILE);
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int c = t * CPT + cc;
      if (MODE == kDqInterior || c < wch) {
        const char* Kn = (cc + 1 < CPT) ? cur : nxt;
        const int kn_row = ((cc + 1) % CPT) * 32;
        if (PIPE) unit(mode_tag, cur, cc * 32, Kn, kn_row, Kn + T::TILE, tab, c * 32);
        else unit_flat(mode_tag, cur, cc * 32, tab, c * 32);
      }
    }
  };
  using Int = std::integral_constant<int, kDqInterior>;
  using Msk = std::integral_constant<int, kDqMasked>;
  using Dyn = std::integral_constant<int, -1>;
  int t = 0;
  for (; t + 3 <= tmask; t += 3) {
    tile_body(Int{}, std::integral_constant<int, 0>{}, t);
    tile_body(Int{}, std::integral_constant<int, 1>{}, t + 1);
    tile_body(Int{}, std::integral_constant<int, 2>{}, t + 2);
  }
  for (; t < tmask; ++t) tile_body(Int{}, Dyn{}, t);
  for (; t < ntiles; ++t) tile_body(Msk{}, Dyn{}, t);

#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) dq_mfma(dt, dkc[dt], dsh, dsl);

  const int query = q0 + (l & 31);
  if (query < nq) {
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
      store_row(out, it.qoff + (int64_t)query * sl, a.out_f32, acc[dt], 32 * dt, a.scale);
  }
}

}  // namespace sa
