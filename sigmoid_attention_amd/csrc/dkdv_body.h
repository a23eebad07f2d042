// Backward pass, key side, on gfx950:
//   dV_j = g_j sum_i P_ij dO_i,   dK_j = s sum_i dS_ij q_i,
//   dS_ij = (dO_i . V'_j) P_ij (1 - P_ij)
// with P recomputed ("Better Models, Faster Training: Sigmoid Attention for single-cell
// Foundation Models", section 4, backward decomposition; appendix A.1.2 Jacobian).
// Each key row belongs to exactly one workgroup, so results are accumulated in
// registers and written once: no atomics, bitwise deterministic.
//
// One workgroup = 4 waves = one item (b, h, key tile of 128). Each wave keeps 32 key rows
// of K and V in registers (B operands), so in S = Q K^T and dP = dO V^T every lane owns
// one key column and the per-key gate terms are per-lane constants. Q and dO stream
// through a 3-stage LDS ring filled by direct loads two tiles ahead. Per 32-query chunk
// c (a unit): the logistic function of S(c) runs while the MFMAs of dP(c) and S(c+1)
// execute; then dS, the bf16 operands, and dV^T += dO^T P, dK^T += Q^T dS (dO^T and Q^T
// read with transposed LDS loads).
//
// With DG the pass also writes the per-head gate gradient
//   dg_hj = sum_i dS_ij / (g_j + eps) + v_j . sum_i P_ij dO_i
// (chain rule through both places the gate enters: log g_j on the logits and g_j on the
// values, "Sigmoid Attention as a Better Substrate for Learned KV Cache Eviction", gate
// paragraphs): each lane sums the float dS of its key column as it goes, and the dot
// product with v_j reads the dV accumulator before the gate factor in the epilogue.
#pragma once

#include <type_traits>

#include "common.h"

namespace sa {

template <int D, int CPT>
struct DkvTraits {
  static constexpr int kThreads = 256;
  static constexpr int kWaves = 4;
  static constexpr int BK = kWaves * 32;   // keys per item
  static constexpr int BQ = 32 * CPT;      // queries per LDS tile
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int TILE = BQ * D * 2;
  static constexpr int STAGE = 2 * TILE;   // Q tile, dO tile
  static constexpr int NSTAGE = 3;
};

enum DkvMode { kKvInterior = 0, kKvMasked = 1 };

__device__ __forceinline__ constexpr int kv_arc(int r) { return 8 * (r >> 2) + (r & 3); }

// The dK/dV pass of one work item `it` (wave-uniform), by the 4 waves of a 256-thread
// workgroup: `smem` is the LDS ring (DkvTraits::NSTAGE * STAGE bytes, 1024-aligned), dK
// goes to `out_k` and dV to `out_v`. VL: packed batch (separate query and key lengths,
// bottom-right causal diagonal). K, V, dK and dV of 32 keys take 96 registers per lane
// at d = 64 (two waves per SIMD) and 192 at d = 128 (one wave per SIMD).
template <int D, int CPT, bool CAUSAL, bool GATED, bool SPLIT, bool DG, bool VL>
__device__ __forceinline__ void dkdv_body(const KArgs& a, const Item& it, char* smem,
                                          void* out_k, void* out_v) {
  using T = DkvTraits<D, CPT>;

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
  const int64_t sl = a.sl;
  const int item_k0 = it.t * T::BK;
  const int k0 = item_k0 + w * 32;          // first key of this wave
  const int mykey = k0 + (l & 31);          // key column owned by this lane
  const float c1 = a.c1;

  // per-lane key constants: logit offset (exp2 domain; +inf drops the key) and factor
  float c2 = it.c2, gmul = 1.0f, gval = 1.0f;
  if (GATED) {
    gval = a.gate[it.goff + (mykey < lastk ? mykey : lastk)];
    const bool keep = mykey < nk && !(mykey >= a.gate_sink && gval < a.gate_tau);
    c2 = keep ? c2 - __builtin_amdgcn_logf(gval + a.gate_eps) : __builtin_inff();
    gmul = keep ? gval : 0.0f;
  }
  float ds_sum = 0.0f;   // DG: sum over this lane's queries of dS / g_j

  // query chunks of the item: all valid queries, or (causal) those from the first query
  // allowed for the item's first key (key j is seen by queries i >= j - diag); this
  // wave's first contributing chunk is c_lo
  const int nch = (nq + 31) / 32;
  const int c_start = CAUSAL ? (item_k0 - diag > 0 ? item_k0 - diag : 0) / 32 : 0;
  const int t0 = c_start / CPT;
  const int ntiles = (nch + CPT - 1) / CPT;
  int c_lo = CAUSAL ? (k0 - diag > 0 ? k0 - diag : 0) / 32 : 0;
  if (k0 >= nk) c_lo = nch;                 // all keys of this wave are padding
  // S of the first unit is formed before the tile loop when its tile is one of the two
  // loaded first, else at the start of that unit (with 32-query tiles the first chunks
  // of waves 2 and 3 lie past them; a causal shift can put them later still)
  const bool s_late = CAUSAL && c_lo < nch && c_lo / CPT > t0 + 1;

  const DirectPair<T::BQ, D, T::kWaves> dma(sl);
  auto issue_tile = [&](int t) {
    dma.load(smem + (t % T::NSTAGE) * T::STAGE, Qg, dOg, sl, t * T::BQ, lastq);
  };
  if (t0 < ntiles) issue_tile(t0);
  if (t0 + 1 < ntiles) issue_tile(t0 + 1);

  // K and V rows as B operands: lane holds key mykey, d = 16ks + 8(l/32) + 0..7
  bf16x8 kreg[T::KS], vreg[T::KS];
  {
    const int row = mykey < lastk ? mykey : lastk;
    const bf16* kr = Kg + (int64_t)row * sl + 8 * (l >> 5);
    const bf16* vr = Vg + (int64_t)row * sl + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      kreg[ks] = *reinterpret_cast<const bf16x8*>(kr + 16 * ks);
      vreg[ks] = *reinterpret_cast<const bf16x8*>(vr + 16 * ks);
    }
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      settle(kreg[ks]);
      settle(vreg[ks]);
    }
  }

  f32x16 dk[T::DT], dv[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) { dk[dt] = zero16(); dv[dt] = zero16(); }

  wait_vmem_and_barrier();

  // S of this wave's first chunk (its tile is one of the two loaded above)
  f32x16 s_cur = zero16();
  if (c_lo < nch && !s_late) {
    const char* st = smem + ((c_lo / CPT) % T::NSTAGE) * T::STAGE;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks)
      s_cur = mfma(lds_row_operand<D>(st, (c_lo % CPT) * 32, 16 * ks), kreg[ks], s_cur);
  }

  // logistic of the 16 entries of S(c), masked (query < nq; query >= key - diag if causal)
  auto sig16 = [&](auto mode_tag, int qb0, f32x16& p) {
    constexpr int MODE = decltype(mode_tag)::value;
    // keep query >= mykey - diag and query <= lastq: query = qb0 + lk + arc(r)
    const int hi_lim = lastq - qb0 - lk;
    const int lo_lim = mykey - diag - qb0 - lk;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = sigmoid_l2(s_cur[r], c1, c2);
      if (MODE == kKvMasked) {
        bool ok = kv_arc(r) <= hi_lim;
        if (CAUSAL) ok = ok && kv_arc(r) >= lo_lim;
        x = ok ? x : 0.0f;
      }
      p[r] = x;
    }
  };
  // masked entries have P = 0 and a finite dP, so their dS is exactly 0
  auto accumulate_ds = [&](const f32x16& ds) {
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      s0 += ds[r];
      s1 += ds[r + 1];
      s2 += ds[r + 2];
      s3 += ds[r + 3];
    }
    ds_sum += (s0 + s1) + (s2 + s3);
  };
  auto to_bf16 = [&](const f32x16& v, int h, bf16x8& hi, bf16x8& lo) {
    if (SPLIT) split8(v, 8 * h, hi, lo, sel);
    else hi = pack8(v, 8 * h);
  };
  auto kv_mfma = [&](f32x16& acc, const bf16x8& op, const bf16x8& hi, const bf16x8& lo) {
    acc = mfma(op, hi, acc);
    if (SPLIT) acc = mfma(op, lo, acc);
  };

  // One unit (query chunk c), steps paired as VALU | MFMA:
  //   1: logistic of S(c)                     | dP(c), S(c+1)
  //   2: dS = dP P (1 - P), bf16 of h = 0     | -
  //   3: bf16 of h = 1                        | dV, dK for the first query half of c
  //   4: -                                    | dV, dK for the second query half
  // (at d = 64 the MFMA-only step overlaps the VALU steps of the other wave on the SIMD)
  const LdsLane<D> lane;
  auto unit = [&](auto mode_tag, const char* Qc, const char* dOc, int qrow, const char* Qn,
                  int qn_row, int qb0) {
    bf16x8 dor[T::KS], qnr[T::KS];
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) dor[ks] = lane.rowop(dOc, qrow, ks);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) qnr[ks] = lane.rowop(Qn, qn_row, ks);
    __builtin_amdgcn_sched_barrier(0);
    // step 1
    f32x16 p, dp = zero16(), s_next = zero16();
    sig16(mode_tag, qb0, p);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) dp = mfma(dor[ks], vreg[ks], dp);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) s_next = mfma(qnr[ks], kreg[ks], s_next);
    __builtin_amdgcn_sched_barrier(0);
    // step 2
    bf16x8 do0[T::DT], qc0[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      do0[dt] = lane.colop(dOc, qrow, dt);
      qc0[dt] = lane.colop(Qc, qrow, dt);
    }
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = dp[r] * __builtin_fmaf(-p[r], p[r], p[r]);
    if (DG) accumulate_ds(ds);
    bf16x8 ph0, pl0, dh0, dl0, ph1, pl1, dh1, dl1;
    to_bf16(p, 0, ph0, pl0);
    to_bf16(ds, 0, dh0, dl0);
    __builtin_amdgcn_sched_barrier(0);
    // step 3
    bf16x8 do1[T::DT], qc1[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      do1[dt] = lane.colop(dOc, qrow + 16, dt);
      qc1[dt] = lane.colop(Qc, qrow + 16, dt);
    }
    to_bf16(p, 1, ph1, pl1);
    to_bf16(ds, 1, dh1, dl1);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      kv_mfma(dv[dt], do0[dt], ph0, pl0);
      kv_mfma(dk[dt], qc0[dt], dh0, dl0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // step 4
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      kv_mfma(dv[dt], do1[dt], ph1, pl1);
      kv_mfma(dk[dt], qc1[dt], dh1, dl1);
    }
    __builtin_amdgcn_sched_barrier(0);
    s_cur = s_next;
  };

  // Tile loops: [t0, tm1) masked (the causal diagonal chunk), [tm1, tm2) interior,
  // [tm2, ntiles) masked (the tile holding the last valid query when nq % 32 != 0 or
  // when it holds fewer than CPT chunks).
  // Every wave passes one barrier per tile.
  // masked under the causal rule: chunks up to the one holding query k0 + 31 - diag
  int tm1 = t0;
  if (CAUSAL && k0 + 31 - diag >= 0) tm1 = (k0 + 31 - diag) / 32 / CPT + 1;
  // the tile holding the last query chunk is masked when that chunk is partial or when
  // the tile reaches past the last chunk (nch not a multiple of CPT)
  int tm2 = (nq % 32 != 0 || nch % CPT != 0) ? (nch - 1) / CPT : ntiles;
  if (c_lo >= nch) { tm1 = ntiles; tm2 = ntiles; }
  tm1 = tm1 < ntiles ? tm1 : ntiles;
  tm2 = tm2 > tm1 ? tm2 : tm1;
  tm2 = tm2 < ntiles ? tm2 : ntiles;

  // `stage_tag`: the ring slot of tile t, a compile-time constant in the unrolled interior
  // loop (LDS addresses fold into immediate offsets), or -1 when computed
  auto tile_body = [&](auto mode_tag, auto stage_tag, int t) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr int SG = decltype(stage_tag)::value;
    if (t > t0) wait_vmem_and_barrier();
    if (t + 2 < ntiles) issue_tile(t + 2);
    const int st = SG >= 0 ? SG : t % T::NSTAGE;
    const int st1 = SG >= 0 ? (SG + 1) % T::NSTAGE : (t + 1) % T::NSTAGE;
    const char* cur = smem + st * T::STAGE;
    const char* nxt = smem + st1 * T::STAGE;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int c = t * CPT + cc;
      if (MODE == kKvInterior || (c >= c_lo && c < nch)) {
        if (MODE == kKvMasked && s_late && c == c_lo) {
          s_cur = zero16();
#pragma unroll
          for (int ks = 0; ks < T::KS; ++ks)
            s_cur = mfma(lds_row_operand<D>(cur, cc * 32, 16 * ks), kreg[ks], s_cur);
        }
        const char* Qn = (cc + 1 < CPT) ? cur : nxt;
        unit(mode_tag, cur, cur + T::TILE, cc * 32, Qn, ((cc + 1) % CPT) * 32, c * 32);
      }
    }
  };
  using Msk = std::integral_constant<int, kKvMasked>;
  using Int = std::integral_constant<int, kKvInterior>;
  using Dyn = std::integral_constant<int, -1>;
  for (int t = t0; t < tm1; ++t) tile_body(Msk{}, Dyn{}, t);
  {
    // interior tiles: up to a multiple of the ring size one at a time, then whole turns
    // of the ring with compile-time slots
    int t = tm1;
    for (; t < tm2 && t % T::NSTAGE != 0; ++t) tile_body(Int{}, Dyn{}, t);
    for (; t + 3 <= tm2; t += 3) {
      tile_body(Int{}, std::integral_constant<int, 0>{}, t);
      tile_body(Int{}, std::integral_constant<int, 1>{}, t + 1);
      tile_body(Int{}, std::integral_constant<int, 2>{}, t + 2);
    }
    for (; t < tm2; ++t) tile_body(Int{}, Dyn{}, t);
  }
  for (int t = tm2; t < ntiles; ++t) tile_body(Msk{}, Dyn{}, t);

  if (DG) {
    // v_j . (sum_i P_ij dO_i): this lane holds features 32 dt + 8 m + lk + e of the dV
    // accumulator (before the gate factor); the partner lane (l ^ 32) holds the rest
    float vdot = 0.0f;
    if (mykey < nk) {
      const bf16* vr = Vg + (int64_t)mykey * sl + lk;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x4 v4 = *reinterpret_cast<const bf16x4*>(vr + 32 * dt + 8 * m);
#pragma unroll
          for (int e = 0; e < 4; ++e) vdot = __builtin_fmaf((float)v4[e], dv[dt][4 * m + e], vdot);
        }
    }
    ds_sum += __shfl_xor(ds_sum, 32, 64);
    vdot += __shfl_xor(vdot, 32, 64);
    if (l < 32 && mykey < nk) {
      // dS = g_j * ds_sum terms (the kernel's dP omits the gate factor of V'_j)
      const float dg = gmul != 0.0f ? gval / (gval + a.gate_eps) * ds_sum + vdot : 0.0f;
      a.aux[((int64_t)it.b * a.H + it.h) * a.Lmax + mykey] = dg;
    }
  }

  if (mykey < nk) {
    const int64_t roff = koff + (int64_t)mykey * sl;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      store_row(out_k, roff, a.out_f32, dk[dt], 32 * dt, a.scale * gmul);
      store_row(out_v, roff, a.out_f32, dv[dt], 32 * dt, gmul);
    }
  }
}

}  // namespace sa
