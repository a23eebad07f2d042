// Backward pass, key side, on gfx950:
//   dV_j = g_j sum_i P_ij dO_i,   dK_j = s sum_i dS_ij q_i,
//   dS_ij = (dO_i . V'_j) P_ij (1 - P_ij)
// with P recomputed ("Better Models, Faster Training: Sigmoid Attention for single-cell
// Foundation Models", section 4, backward decomposition; appendix A.1.2 Jacobian).
// Each key row belongs to exactly one workgroup, so results are accumulated in
// registers and written once: no atomics, bitwise deterministic.
//
// One workgroup = 4 waves = one item (b, h, key tile of 128). Each wave keeps 32 key
// rows of K and V in registers (B operands). Q and dO tiles of 64 queries are
// double-buffered in LDS, the next tile's global loads in flight during the current.
// Per 32-query chunk: S = Q K^T and dP = dO V^T (MFMA), P and dS in fp32 registers
// (lane = key column), then dV^T += dO^T P and dK^T += Q^T dS (MFMA, with dO^T and
// Q^T read by transposed LDS loads; P and dS as hi + lo when SPLIT).
#include "common.h"

namespace sa {

template <int D>
struct DkvTraits {
  static constexpr int kThreads = 256;
  static constexpr int kWaves = 4;
  static constexpr int BK = kWaves * 32;       // keys per item
  static constexpr int BQ = 64;                // queries per LDS stage
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int TILE_BYTES = BQ * D * 2;
  static constexpr int STAGE = 2 * TILE_BYTES;   // Q, dO
};

template <int D, bool CAUSAL, bool GATED, bool SPLIT>
__global__ __launch_bounds__(256) void dkdv_kernel(const KArgs a) {
  using T = DkvTraits<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * T::STAGE];

  const int l = lane_id(), w = wave_id();
  const SplitSel sel;
  const Item it = decode_item(a, remap_block(blockIdx.x, a.nitems, a.xcd_chunk));
  const int n = it.n;
  const int last = n - 1;
  const int64_t hoff = (int64_t)it.b * a.sb + (int64_t)it.h * a.sh;
  const bf16* Qg = (const bf16*)a.q + hoff;
  const bf16* Kg = (const bf16*)a.k + hoff;
  const bf16* Vg = (const bf16*)a.v + hoff;
  const bf16* dOg = (const bf16*)a.dout + hoff;
  const int64_t sl = a.sl;
  const int item_k0 = it.t * T::BK;
  const int k0 = item_k0 + w * 32;          // first key of this wave
  const int mykey = k0 + (l & 31);          // key column owned by this lane
  const float c1 = a.c1;

  // per-lane key constants: logit offset (exp2 domain; +inf drops the key) and factor
  float c2 = it.c2, gmul = 1.0f;
  if (GATED) {
    const float g = a.gate[(int64_t)it.b * a.gsb + (mykey < last ? mykey : last)];
    const bool keep = mykey < n && !(mykey >= a.gate_sink && g < a.gate_tau);
    c2 = keep ? c2 - __builtin_amdgcn_logf(g + a.gate_eps) : __builtin_inff();
    gmul = keep ? g : 0.0f;
  }

  // K and V rows as B operands: lane holds key mykey, d = 16ks + 8(l/32) + 0..7
  bf16x8 kop[T::KS], vop[T::KS];
  {
    const int row = mykey < last ? mykey : last;
    const bf16* kr = Kg + (int64_t)row * sl + 8 * (l >> 5);
    const bf16* vr = Vg + (int64_t)row * sl + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      kop[ks] = *reinterpret_cast<const bf16x8*>(kr + 16 * ks);
      vop[ks] = *reinterpret_cast<const bf16x8*>(vr + 16 * ks);
    }
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      settle(kop[ks]);
      settle(vop[ks]);
    }
  }

  f32x16 dk[T::DT], dv[T::DT];
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt) { dk[dt] = zero16(); dv[dt] = zero16(); }

  // query tiles: all valid queries, or those at or after the item's first key (causal)
  const int qt0 = CAUSAL ? item_k0 / T::BQ : 0;
  const int nqt = (n + T::BQ - 1) / T::BQ;

  TileRegs<T::BQ, D, T::kThreads> qreg, doreg;
  auto load = [&](int qt) {
    qreg.load(Qg, sl, qt * T::BQ, last);
    doreg.load(dOg, sl, qt * T::BQ, last);
  };
  auto store = [&](int qt) {
    char* st = smem + (qt & 1) * T::STAGE;
    qreg.store(st);
    doreg.store(st + T::TILE_BYTES);
  };

  if (qt0 < nqt) {
    load(qt0);
    store(qt0);
  }
  for (int qt = qt0; qt < nqt; ++qt) {
    if (qt + 1 < nqt) load(qt + 1);
    __syncthreads();
    const int qb0 = qt * T::BQ;
    // causal: skip tiles whose every query comes before every key of this wave
    if (!CAUSAL || qb0 + T::BQ - 1 >= k0) {
      const char* Qt = smem + (qt & 1) * T::STAGE;
      const char* dOt = Qt + T::TILE_BYTES;
      const bool edge = qb0 + T::BQ > n;
      const bool diag = CAUSAL && (qb0 < k0 + 31);

#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
          const bf16x8 qa = lds_row_operand<D>(Qt, 32 * c, 16 * ks);
          const bf16x8 da = lds_row_operand<D>(dOt, 32 * c, 16 * ks);
          s = mfma(qa, kop[ks], s);
          dp = mfma(da, vop[ks], dp);
        }
        f32x16 p, ds;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = sigmoid_l2(s[r], c1, c2);
          ds[r] = dp[r] * __builtin_fmaf(-p[r], p[r], p[r]);
        }
        if (edge || diag) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int query = qb0 + 32 * c + acc_row(r, l);
            const bool ok = query < n && (!CAUSAL || mykey <= query);
            p[r] = ok ? p[r] : 0.0f;
            ds[r] = ok ? ds[r] : 0.0f;
          }
        }
        bf16x8 pb0, pb1, db0, db1, pl0, pl1, dl0, dl1;
        if (SPLIT) {
          split8(p, 0, pb0, pl0, sel);
          split8(p, 8, pb1, pl1, sel);
          split8(ds, 0, db0, dl0, sel);
          split8(ds, 8, db1, dl1, sel);
        } else {
          pb0 = pack8(p, 0);
          pb1 = pack8(p, 8);
          db0 = pack8(ds, 0);
          db1 = pack8(ds, 8);
        }
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const bf16x8 doT0 = lds_col_operand<D>(dOt, 32 * c, 32 * dt);
          const bf16x8 doT1 = lds_col_operand<D>(dOt, 32 * c + 16, 32 * dt);
          dv[dt] = mfma(doT0, pb0, dv[dt]);
          dv[dt] = mfma(doT1, pb1, dv[dt]);
          if (SPLIT) {
            dv[dt] = mfma(doT0, pl0, dv[dt]);
            dv[dt] = mfma(doT1, pl1, dv[dt]);
          }
          const bf16x8 qT0 = lds_col_operand<D>(Qt, 32 * c, 32 * dt);
          const bf16x8 qT1 = lds_col_operand<D>(Qt, 32 * c + 16, 32 * dt);
          dk[dt] = mfma(qT0, db0, dk[dt]);
          dk[dt] = mfma(qT1, db1, dk[dt]);
          if (SPLIT) {
            dk[dt] = mfma(qT0, dl0, dk[dt]);
            dk[dt] = mfma(qT1, dl1, dk[dt]);
          }
        }
      }
    }
    if (qt + 1 < nqt) store(qt + 1);
  }

  if (mykey < n) {
    const int64_t roff = hoff + (int64_t)mykey * sl;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) {
      store_row(a.out0, roff, a.out_f32, dk[dt], 32 * dt, a.scale * gmul);
      store_row(a.out1, roff, a.out_f32, dv[dt], 32 * dt, gmul);
    }
  }
}

template <int D, bool C, bool G, bool SP>
static hipError_t launch_one(const KArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((dkdv_kernel<D, C, G, SP>), dim3(a.nitems), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch(const KArgs& a, bool c, bool g, bool sp, hipStream_t st) {
  if (c) {
    if (g) return sp ? launch_one<D, true, true, true>(a, st) : launch_one<D, true, true, false>(a, st);
    return sp ? launch_one<D, true, false, true>(a, st) : launch_one<D, true, false, false>(a, st);
  }
  if (g) return sp ? launch_one<D, false, true, true>(a, st) : launch_one<D, false, true, false>(a, st);
  return sp ? launch_one<D, false, false, true>(a, st) : launch_one<D, false, false, false>(a, st);
}

int dkdv_tile_rows(int d) { return d == 64 ? DkvTraits<64>::BK : DkvTraits<128>::BK; }

hipError_t launch_dkdv_bf16(const KArgs& a, int d, bool causal, bool gated, bool split,
                            hipStream_t st) {
  return d == 64 ? dispatch<64>(a, causal, gated, split, st) : dispatch<128>(a, causal, gated, split, st);
}

}  // namespace sa
