// Forward pass of padded sigmoid attention on gfx950:
//   O = sigma(s Q K^T + beta [+ log(g + eps)]) V'      (element-wise sigmoid, no row
// statistics), "Better Models, Faster Training: Sigmoid Attention for single-cell
// Foundation Models", section 3 equation; one fused pass that never materialises the
// n x n matrix and never visits fully padded tiles (section 4, block-sparse computation).
//
// One workgroup = 4 waves = one work item (b, h, query tile of BM rows). Each wave owns
// QB blocks of 32 queries held in registers as the B operand of S^T = K Q^T, so the fp32
// result already has the register layout of the B operand of O^T += V^T P^T (P never goes
// through LDS). K and V stream through a 3-stage LDS ring filled by direct global->LDS
// loads two tiles ahead; one barrier per tile.
//
// Per 32-key chunk c a wave runs a software pipeline: the MFMAs of S(c+1) are issued
// while the VALU evaluates the logistic function of S(c) (computed one chunk earlier), and
// the P V MFMAs of each 16-key half follow the VALU work of that half. At d = 64 the two transcendentals per pair (exp2, rcp; a
// quarter of the FMA rate on gfx950) cost about as much as the two products, so keeping
// both pipes busy at once is what sets the speed.
//
// Chunk modes (wave-uniform): interior chunks compute every pair; chunks that reach past
// the valid length, or cross the wave's diagonal under the causal rule, zero the pairs
// with key >= nk or key > query + diag. With a gate, a per-key table in LDS supplies the logit
// offset (+inf for padded or dropped keys, which makes P exactly 0) and value factor.
//
// With RS the pass also writes the row mass sum_j P_ij of every valid query (the
// row-sum diagnostic of "Sigmoid Attention as a Better Substrate for Learned KV Cache
// Eviction": without row normalisation the total weight of a row is free). Each lane
// adds the masked weights of its query column before the value gate is applied; the
// two lanes holding one query are combined in the epilogue.
#include <type_traits>

#include "common.h"

namespace sa {

template <int D, int QB, int CPT, bool GATED>
struct FwdTraits {
  static constexpr int kThreads = 256;
  static constexpr int kWaves = 4;
  static constexpr int BM = kWaves * QB * 32;   // queries per work item
  static constexpr int BN = 32 * CPT;           // keys per LDS tile
  static constexpr int KS = D / 16;             // k-steps of S^T = K Q^T
  static constexpr int DT = D / 32;             // 32-column blocks of O
  static constexpr int TILE = BN * D * 2;       // bytes of one K (or V) tile
  static constexpr int TAB = GATED ? 2 * BN * 4 : 0;   // per-key gate table
  static constexpr int STAGE = 2 * TILE + TAB;  // K tile, V tile, gate table
  static constexpr int NSTAGE = 3;
};

enum ChunkMode { kInterior = 0, kMasked = 1 };

// Register row (within a 32-row MFMA result) of entry r, without the lane term 4*(l/32).
__device__ __forceinline__ constexpr int arc(int r) { return 8 * (r >> 2) + (r & 3); }

// Waves per SIMD the register budget is sized for: 3 at d = 64 (168 registers, which the
// unit without the deferred half fits), 2 at d = 128 and for the row-mass variant.
#ifndef SA_FWD64_QB
#define SA_FWD64_QB 1
#endif
template <int D, int QB, bool RS>
struct FwdOcc {
  static constexpr int value = (D == 64 && !RS) ? 3 : 2;
};

// F16 (with SPLIT): P V on f16 operands where V fits, hi + lo bf16 otherwise.
template <int D, int QB, int CPT, bool CAUSAL, bool GATED, bool SPLIT, bool RS, bool VL,
          bool F16 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FwdOcc<D, QB, RS>::value, FwdOcc<D, QB, RS>::value)))
void fwd_kernel(const KArgs a) {
  static_assert(SPLIT || !F16, "f16 operands replace the hi + lo split");
  using T = FwdTraits<D, QB, CPT, GATED>;
  __shared__ __attribute__((aligned(1024))) char smem[T::NSTAGE * T::STAGE];
  // F16: per ring slot, set when some value of that tile's V does not fit f16
  __shared__ int vflag[T::NSTAGE];

  const int l = lane_id(), w = wave_id();
  const int lk = 4 * (l >> 5);
  const SplitSel sel;
  // VL: packed batch (separate query and key lengths, bottom-right causal diagonal);
  // otherwise nk = nq and diag = 0 are compile-time facts
  const Item it = block_item<VL>(a);
  if (VL && !it.valid) return;
  const int nq = it.nq, nk = VL ? it.nk : it.nq, diag = VL ? it.diag : 0;
  const int lastq = nq - 1, lastk = nk - 1;
  const int64_t koff = VL ? it.koff : it.qoff;
  const bf16* Qg = (const bf16*)a.q + it.qoff;
  const bf16* Kg = (const bf16*)a.k + koff;
  const bf16* Vg = (const bf16*)a.v + koff;
  const float* Gg = GATED ? a.gate + it.goff : nullptr;
  const int64_t sl = a.sl;
  const int item_q0 = it.t * T::BM;
  const int q0 = item_q0 + w * QB * 32;   // first query of this wave
  const float c1 = a.c1, c2 = it.c2;
  // F16 keeps P as 2^14 sigma: 14 comes off the exp2 argument, 2^-14 off the result
  const float c2s = F16 ? c2 - 14.0f : c2;
  const float out_scale = F16 ? kPScaleInv : 1.0f;

  // keys of the item: all of them, or (causal) those up to the item's last query + diag
  int kend = nk;
  if (CAUSAL) {
    const int e = (item_q0 + T::BM < nq ? item_q0 + T::BM : nq) + diag;
    kend = e < 0 ? 0 : (e < nk ? e : nk);
  }
  const int nch = (kend + 31) / 32;                 // 32-key chunks of the item
  const int ntiles = (nch + CPT - 1) / CPT;
  // chunks this wave computes: none if all its queries are padding; under the causal
  // rule only chunks holding a key allowed for its last valid query
  int wch = q0 < nq ? nch : 0;
  if (CAUSAL && q0 < nq) {
    const int lk_allowed = (q0 + QB * 32 < nq ? q0 + QB * 32 : nq) - 1 + diag;
    wch = lk_allowed < 0 ? 0 : (lk_allowed / 32 + 1 < nch ? lk_allowed / 32 + 1 : nch);
  }

  const DirectPair<T::BN, D, T::kWaves> dma(sl);
  auto issue_tile = [&](int t) {
    dma.load(smem + (t % T::NSTAGE) * T::STAGE, Kg, Vg, sl, t * T::BN, lastk);
  };
  // gate table of tile t: logit offset in the exp2 domain (+inf drops the key, which
  // gives P = 0 exactly) and value factor, one entry per key, written by wave 0 (lanes
  // below BN) from the gate value g of its key. The values are read one tile ahead
  // (gate_value), so that the wait for them falls where nothing else is in flight: a
  // wait right behind the direct loads of a tile would wait for those too (the
  // compiler does not count them and waits for every load).
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
      tab[l] = keep ? c2s - __builtin_amdgcn_logf(g + a.gate_eps) : __builtin_inff();
      tab[T::BN + l] = keep ? g : 0.0f;
    }
  };
  float gfirst = 0.0f, gnext = 0.0f;   // gate values for the tables of tiles 0 and t + 1
  // first two tiles: gate values and direct loads; the table of tile 0 is written once
  // the loads issued after them are awaited, before the barrier that publishes the tile
  auto start_ring = [&]() {
    if (gate_lane && ntiles > 0) gfirst = gate_value(0);
    if (gate_lane && ntiles > 1) gnext = gate_value(1);
    if (ntiles > 0) issue_tile(0);
    if (ntiles > 1) issue_tile(1);
  };
  // F16: P V runs on f16 operands where V allows. P is kept as 2^14 sigma (in [0, 2^14],
  // normal in f16 down to sigma = 2^-28) and rounded once to f16, 2^-11 relative, 8x
  // finer than bf16: one f16 product instead of the bf16 hi + lo pair. V's bf16 values
  // with 2^-17 <= |v| < 2^16 are exact in f16; smaller ones fall into the f16 subnormals
  // (absolute error at most 2^-25, zero below 2^-25), larger ones do not fit and flag
  // the tile (below); during tile t each thread converts its two
  // 16-byte chunks of tile t+1's V in place and flags the tile if a value did not fit.
  // If any tile of the item was flagged, the workgroup computes the item again from the
  // start on bf16 hi + lo operands, with V loaded afresh and left unconverted. The tile
  // loops themselves never branch on the flags: an exit from them costs the register
  // allocation far more than the rare second pass.
  static_assert(T::TILE == 16 * 2 * T::kThreads, "two 16-byte V chunks per thread");
  auto convert_v = [&](int t) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    char* vt = smem + (t % T::NSTAGE) * T::STAGE + T::TILE;
    u16x2 emax = {0, 0};   // largest |bf16| bit pattern seen, per half
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4* p = reinterpret_cast<u32x4*>(vt + 16 * (threadIdx.x + T::kThreads * i));
      const u32x4 c = *p;
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        emax = __builtin_elementwise_max(emax, __builtin_bit_cast(u16x2, c[e] & 0x7fff7fffu));
        f16x2 h;
        h[0] = (_Float16)__builtin_bit_cast(float, c[e] << 16);
        h[1] = (_Float16)__builtin_bit_cast(float, c[e] & 0xffff0000u);
        o[e] = __builtin_bit_cast(uint32_t, h);
      }
      *p = o;
    }
    // |v| >= 2^16 is a bf16 exponent field >= 143 (0x4780 with the mantissa bits below);
    // that includes infinities, and NaN, which would not need the second pass but is rare
    const bool bad = emax[0] >= 0x4780 || emax[1] >= 0x4780;
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && l == 0) vflag[t % T::NSTAGE] = 1;
  };
  if (F16 && threadIdx.x < T::NSTAGE) vflag[threadIdx.x] = 0;
  start_ring();

  // Q rows as B operands: lane holds query q0 + 32qb + l%32, d = 16ks + 8(l/32) + 0..7.
  bf16x8 qop[QB][T::KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    int row = q0 + 32 * qb + (l & 31);
    row = row < lastq ? row : lastq;
    const bf16* qr = Qg + (int64_t)row * sl + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) qop[qb][ks] = *reinterpret_cast<const bf16x8*>(qr + 16 * ks);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) settle(qop[qb][ks]);

  f32x16 acc[QB][T::DT];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) acc[qb][dt] = zero16();
  float mass[QB];   // RS: sum of this lane's weights per query block
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mass[qb] = 0.0f;

  if (ntiles > 0) store_table(0, gfirst);
  wait_vmem_and_barrier();

  // S of unit 0 (chunk 0, query block 0)
  f32x16 s_cur;
  {
    s_cur = zero16();
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks)
      s_cur = mfma(lds_row_operand<D>(smem, 0, 16 * ks), qop[0][ks], s_cur);
  }
  int vbad = 0;   // f16 operands: some tile of this item had V beyond f16
  if (F16 && ntiles > 0) {
    convert_v(0);
    __syncthreads();
  }

  // The work of a chunk is split into units u = (chunk c, query block qb). Unit u
  // evaluates the logistic function of S(u) while the MFMAs of S(u+1) run, then adds
  // P(u) V(c) into O. S(u+1) uses the K rows of the same chunk for qb + 1 < QB, else
  // those of chunk c + 1 (already in LDS: tiles t and t+1 are both visible in tile t).
  //
  // Logistic of the 4 entries r0..r0+3 of S(u) (one row group of the MFMA result),
  // masked as the chunk mode requires, into p.
  auto sig4 = [&](auto mode_tag, int qb, int r0, int kb, const float* tab, int krow,
                  f32x16& p) {
    constexpr int MODE = decltype(mode_tag)::value;
    f32x4 tc2, tg;
    if (GATED) {
      tc2 = *reinterpret_cast<const f32x4*>(tab + krow + 2 * r0 + lk);
      tg = *reinterpret_cast<const f32x4*>(tab + T::BN + krow + 2 * r0 + lk);
    }
    // masked chunks keep key <= lim + kb + lk: key < nk, and key <= query + diag when
    // causal
    int lim = nk - 1 - kb - lk;
    if (CAUSAL) {
      const int ld = q0 + 32 * qb + (l & 31) + diag - kb - lk;
      lim = ld < lim ? ld : lim;
    }
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + e;
      float x = F16 ? sigmoid_l2s(s_cur[r], c1, GATED ? tc2[e] : c2s)
                    : sigmoid_l2(s_cur[r], c1, GATED ? tc2[e] : c2s);
      if (MODE == kMasked) x = arc(r) <= lim ? x : 0.0f;
      if (RS) part += x;
      if (GATED) x *= tg[e];
      p[r] = x;
    }
    if (RS) mass[qb] += part;
  };
  auto to_bf16 = [&](const f32x16& p, int h, bf16x8& ph, bf16x8& pl) {
    if (SPLIT) split8(p, 8 * h, ph, pl, sel);
    else ph = pack8(p, 8 * h);
  };

  auto pv = [&](int qb, int dt, const bf16x8& vo, const bf16x8& hi, const bf16x8& lo) {
    acc[qb][dt] = mfma(vo, hi, acc[qb][dt]);
    if (SPLIT) acc[qb][dt] = mfma(vo, lo, acc[qb][dt]);
  };

  // One unit (query block qb against one 32-key chunk). Program order is fixed by
  // scheduling barriers into steps that pair VALU work with MFMAs that do not depend on
  // it; the K and V operand reads are issued first so that their latency hides behind the
  // first VALU step. Nothing is carried into the next unit but S(u+1); the second key
  // half's P V closes the unit and overlaps the VALU work of the other waves on the SIMD
  // (three at d = 64):
  //   1: logistic of entries 0-3           | S(u+1), first half of the k-steps
  //   2: entries 4-7, to bf16 (h = 0)      | S(u+1), second half
  //   3: entries 8-11                      | P V (h = 0)
  //   4: entries 12-15, to bf16 (h = 1)    | -
  //   5: -                                 | P V (h = 1)
  const LdsLane<D> lane;
  auto unit = [&](auto mode_tag, auto f16_tag, int qb, const char* Kn, int kn_row,
                  int qb_next, const char* Vt, int v_row, const float* tab, int kb) {
    constexpr bool OPF16 = decltype(f16_tag)::value;
    bf16x8 kop[T::KS];
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) kop[ks] = lane.rowop(Kn, kn_row, ks);
    bf16x8 vop0[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) vop0[dt] = lane.colop(Vt, v_row, dt);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 p;
    bf16x8 ph0, pl0, ph1, pl1;
    f16x8 p16_0, p16_1;
    f32x16 s_next = zero16();
    sig4(mode_tag, qb, 0, kb, tab, v_row, p);
#pragma unroll
    for (int ks = 0; ks < T::KS / 2; ++ks) s_next = mfma(kop[ks], qop[qb_next][ks], s_next);
    __builtin_amdgcn_sched_barrier(0);
    sig4(mode_tag, qb, 4, kb, tab, v_row, p);
    if constexpr (OPF16) p16_0 = pack8_f16(p, 0);
    else to_bf16(p, 0, ph0, pl0);
#pragma unroll
    for (int ks = T::KS / 2; ks < T::KS; ++ks) s_next = mfma(kop[ks], qop[qb_next][ks], s_next);
    __builtin_amdgcn_sched_barrier(0);
    // f16 operands: the second half of the unit runs at raised wave priority (measured
    // 2-3 % faster there; no gain with hi + lo operands, whose units are VALU-heavier)
    if constexpr (OPF16) __builtin_amdgcn_s_setprio(1);
    bf16x8 vop1[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) vop1[dt] = lane.colop(Vt, v_row + 16, dt);
    sig4(mode_tag, qb, 8, kb, tab, v_row, p);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      if constexpr (OPF16) acc[qb][dt] = mfma_f16(__builtin_bit_cast(f16x8, vop0[dt]), p16_0, acc[qb][dt]);
      else pv(qb, dt, vop0[dt], ph0, pl0);
    }
    __builtin_amdgcn_sched_barrier(0);
    sig4(mode_tag, qb, 12, kb, tab, v_row, p);
    if constexpr (OPF16) p16_1 = pack8_f16(p, 8);
    else to_bf16(p, 1, ph1, pl1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      if constexpr (OPF16) acc[qb][dt] = mfma_f16(__builtin_bit_cast(f16x8, vop1[dt]), p16_1, acc[qb][dt]);
      else pv(qb, dt, vop1[dt], ph1, pl1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (OPF16) __builtin_amdgcn_s_setprio(0);
    s_cur = s_next;
  };
  auto chunk = [&](auto mode_tag, auto f16_tag, const char* Kc, int kc_row, const char* Kn,
                   int kn_row, const char* Vt, int v_row, const float* tab, int kb) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const char* K1 = qb + 1 < QB ? Kc : Kn;
      const int k1_row = qb + 1 < QB ? kc_row : kn_row;
      const int qb1 = qb + 1 < QB ? qb + 1 : 0;
      unit(mode_tag, f16_tag, qb, K1, k1_row, qb1, Vt, v_row, tab, kb);
    }
  };

  // Tiles before `tmask` hold only interior chunks for this wave; the rest run the
  // masked body. Two loops without a mode branch inside; every wave passes the same
  // number of barriers (one per tile).
  int cfirst = nk / 32;                                 // first chunk reaching past nk
  if (CAUSAL) {
    // first chunk holding a key past query q0's last allowed key q0 + diag
    const int c = q0 + diag + 1 < 0 ? 0 : (q0 + diag + 1) / 32;
    cfirst = c < cfirst ? c : cfirst;
  }
  int tmask = cfirst / CPT;
  tmask = tmask < ntiles ? tmask : ntiles;
  if (q0 >= nq) tmask = 0;                              // nothing to compute

  // One tile. `stage` is the ring slot of tile t: a compile-time constant in the unrolled
  // interior loop (the LDS addresses then fold into immediate offsets), or -1 when it
  // has to be computed.
  auto tile_body = [&](auto mode_tag, auto stage_tag, auto f16_tag, int t) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr int SG = decltype(stage_tag)::value;
    constexpr bool OPF16 = decltype(f16_tag)::value;
    if (t > 0) wait_vmem_and_barrier();
    const int st = SG >= 0 ? SG : t % T::NSTAGE;
    const int st1 = SG >= 0 ? (SG + 1) % T::NSTAGE : (t + 1) % T::NSTAGE;
    // every thread reads the flag after the barrier that follows all its writers
    if constexpr (OPF16) vbad |= vflag[st];
    // gnext was read during the previous tile (or before the first) and has arrived
    if (t + 1 < ntiles) store_table(t + 1, gnext);
    if (t + 2 < ntiles) {
      if (gate_lane) gnext = gate_value(t + 2);
      issue_tile(t + 2);
    }
    if constexpr (OPF16) {
      // tile t+2's slot was last read at the start of tile t-1
      if (threadIdx.x == 0) vflag[(st + 2) % T::NSTAGE] = 0;
      if (t + 1 < ntiles) convert_v(t + 1);
    }
    const char* cur = smem + st * T::STAGE;
    const char* nxt = smem + st1 * T::STAGE;
    const float* tab = reinterpret_cast<const float*>(cur + 2 * T::TILE);
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int c = t * CPT + cc;
      if (MODE == kInterior || c < wch) {
        const char* Kn = (cc + 1 < CPT) ? cur : nxt;
        const int kn_row = ((cc + 1) % CPT) * 32;
        chunk(mode_tag, f16_tag, cur, cc * 32, Kn, kn_row, cur + T::TILE, cc * 32, tab, c * 32);
      }
    }
  };
  using Int = std::integral_constant<int, kInterior>;
  using Msk = std::integral_constant<int, kMasked>;
  using Dyn = std::integral_constant<int, -1>;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using Op16 = std::true_type;     // f16 operands
  using OpBf = std::false_type;    // bf16 operands (hi + lo when SPLIT)
  auto tile_loops = [&](auto f16_tag) {
    int t = 0;
    for (; t + 3 <= tmask; t += 3) {
      tile_body(Int{}, S0{}, f16_tag, t);
      tile_body(Int{}, S1{}, f16_tag, t + 1);
      tile_body(Int{}, S2{}, f16_tag, t + 2);
    }
    for (; t < tmask; ++t) tile_body(Int{}, Dyn{}, f16_tag, t);
    for (; t < ntiles; ++t) tile_body(Msk{}, Dyn{}, f16_tag, t);
  };
  if constexpr (F16) {
    tile_loops(Op16{});
    if (__builtin_amdgcn_readfirstlane(vbad)) {
      // again from the start on bf16 hi + lo operands: wait for the loads still in flight
      // and for every wave to leave the ring, then refill it
      wait_vmem_and_barrier();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        mass[qb] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) acc[qb][dt] = zero16();
      }
      start_ring();
      if (ntiles > 0) store_table(0, gfirst);
      wait_vmem_and_barrier();
      s_cur = zero16();
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks)
        s_cur = mfma(lds_row_operand<D>(smem, 0, 16 * ks), qop[0][ks], s_cur);
      tile_loops(OpBf{});
    }
  } else {
    tile_loops(OpBf{});
  }

  // epilogue: valid query rows only (rows >= n are zero-filled by a separate kernel)
  if (RS) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      mass[qb] += __shfl_xor(mass[qb], 32, 64);
      const int query = q0 + 32 * qb + (l & 31);
      if (l < 32 && query < nq)
        a.aux[((int64_t)it.b * a.H + it.h) * a.Lmax + query] = mass[qb] * out_scale;
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int query = q0 + 32 * qb + (l & 31);
    if (query < nq) {
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
        store_row(a.out0, it.qoff + (int64_t)query * sl, a.out_f32, acc[qb][dt], 32 * dt,
                  out_scale);
    }
  }
}

template <int D, int QB, int CPT, bool C, bool G, bool SP, bool RS>
static hipError_t launch_one(const KArgs& a, hipStream_t st) {
  const dim3 grid(a.nitems), block(256);
  if constexpr (SP) {
    if (a.f16_pv) {
      if (a.varlen) hipLaunchKernelGGL((fwd_kernel<D, QB, CPT, C, G, true, false, true, true>), grid, block, 0, st, a);
      else hipLaunchKernelGGL((fwd_kernel<D, QB, CPT, C, G, true, RS, false, true>), grid, block, 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.varlen)
    hipLaunchKernelGGL((fwd_kernel<D, QB, CPT, C, G, SP, false, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((fwd_kernel<D, QB, CPT, C, G, SP, RS, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <int D, int QB, int CPT, bool RS>
static hipError_t dispatch_rs(const KArgs& a, bool c, bool g, bool sp, hipStream_t st) {
  if (c) {
    if (g) return sp ? launch_one<D, QB, CPT, true, true, true, RS>(a, st) : launch_one<D, QB, CPT, true, true, false, RS>(a, st);
    return sp ? launch_one<D, QB, CPT, true, false, true, RS>(a, st) : launch_one<D, QB, CPT, true, false, false, RS>(a, st);
  }
  if (g) return sp ? launch_one<D, QB, CPT, false, true, true, RS>(a, st) : launch_one<D, QB, CPT, false, true, false, RS>(a, st);
  return sp ? launch_one<D, QB, CPT, false, false, true, RS>(a, st) : launch_one<D, QB, CPT, false, false, false, RS>(a, st);
}

template <int D, int QB, int CPT>
static hipError_t dispatch(const KArgs& a, bool c, bool g, bool sp, hipStream_t st) {
  return a.aux ? dispatch_rs<D, QB, CPT, true>(a, c, g, sp, st) : dispatch_rs<D, QB, CPT, false>(a, c, g, sp, st);
}

int fwd_tile_rows(int d) { return d == 64 ? FwdTraits<64, SA_FWD64_QB, 2, false>::BM : FwdTraits<128, 1, 1, false>::BM; }

hipError_t launch_fwd_bf16(const KArgs& a, int d, bool causal, bool gated, bool split,
                           hipStream_t st) {
  return d == 64 ? dispatch<64, SA_FWD64_QB, 2>(a, causal, gated, split, st)
                 : dispatch<128, 1, 1>(a, causal, gated, split, st);
}

}  // namespace sa
