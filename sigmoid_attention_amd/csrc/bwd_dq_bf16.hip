// Backward pass, query side, on gfx950:
//   dQ_i = s sum_j dS_ij k_j,  dS_ij = (dO_i . V'_j) P_ij (1 - P_ij)
// P is recomputed from Q and K rather than stored ("Better Models, Faster Training:
// Sigmoid Attention for single-cell Foundation Models", section 4, backward pass
// decomposition: one kernel for dQ, one for dK/dV, no atomics). The factor
// P(1 - P) is the diagonal of the sigmoid Jacobian (appendix A.1.2).
//
// One workgroup = 4 waves = one item (b, h, query tile). Each wave keeps its Q and dO
// rows in registers (B operands). K and V tiles are double-buffered in LDS, the next
// tile's global loads in flight during the current tile. Per 32-key chunk:
// S^T = K Q^T and dP^T = V dO^T (MFMA), then P, dS in fp32 registers, then
// dQ^T += K^T dS^T (MFMA with K^T read by transposed LDS loads; dS as hi + lo when
// SPLIT).
#include "common.h"

namespace sa {

template <int D, int QB>
struct DqTraits {
  static constexpr int kThreads = 256;
  static constexpr int kWaves = 4;
  static constexpr int BM = kWaves * QB * 32;
  static constexpr int BN = 64;
  static constexpr int KS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int STAGE = 2 * TILE_BYTES + 2 * BN * 4;   // K, V, per-key gate table
};

template <int D, int QB, bool CAUSAL, bool GATED, bool SPLIT>
__global__ __launch_bounds__(256) void dq_kernel(const KArgs a) {
  using T = DqTraits<D, QB>;
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
  const float* Gg = GATED ? a.gate + (int64_t)it.b * a.gsb : nullptr;
  const int64_t sl = a.sl;
  const int item_q0 = it.t * T::BM;
  const int q0 = item_q0 + w * QB * 32;
  const float c1 = a.c1, c2 = it.c2;

  bf16x8 qop[QB][T::KS], doop[QB][T::KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    int row = q0 + 32 * qb + (l & 31);
    row = row < last ? row : last;
    const bf16* qr = Qg + (int64_t)row * sl + 8 * (l >> 5);
    const bf16* dr = dOg + (int64_t)row * sl + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      qop[qb][ks] = *reinterpret_cast<const bf16x8*>(qr + 16 * ks);
      doop[qb][ks] = *reinterpret_cast<const bf16x8*>(dr + 16 * ks);
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      settle(qop[qb][ks]);
      settle(doop[qb][ks]);
    }

  f32x16 acc[QB][T::DT];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) acc[qb][dt] = zero16();

  int kend = n;
  if (CAUSAL) kend = (item_q0 + T::BM < n) ? item_q0 + T::BM : n;
  const int nkt = (kend + T::BN - 1) / T::BN;

  TileRegs<T::BN, D, T::kThreads> kreg, vreg;
  float greg = 0.0f;
  auto load = [&](int kt) {
    const int kb = kt * T::BN;
    kreg.load(Kg, sl, kb, last);
    vreg.load(Vg, sl, kb, last);
    if (GATED && w == 0) {
      const int key = kb + l;
      greg = Gg[key < last ? key : last];
    }
  };
  auto store = [&](int kt) {
    char* st = smem + (kt & 1) * T::STAGE;
    kreg.store(st);
    vreg.store(st + T::TILE_BYTES);
    if (GATED && w == 0) {
      const int key = kt * T::BN + l;
      const bool keep = key < n && !(key >= a.gate_sink && greg < a.gate_tau);
      float* tab = reinterpret_cast<float*>(st + 2 * T::TILE_BYTES);
      tab[l] = keep ? c2 - __builtin_amdgcn_logf(greg + a.gate_eps) : __builtin_inff();
      tab[T::BN + l] = greg;
    }
  };

  load(0);
  store(0);
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) load(kt + 1);
    __syncthreads();
    const int kb = kt * T::BN;
    if (!CAUSAL || kb <= q0 + QB * 32 - 1) {
      const char* Kt = smem + (kt & 1) * T::STAGE;
      const char* Vt = Kt + T::TILE_BYTES;
      const float* tab = reinterpret_cast<const float*>(Kt + 2 * T::TILE_BYTES);
      const bool edge = kb + T::BN > n;
      const bool diag = CAUSAL && (kb + T::BN - 1 > q0);

#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 kop[T::KS], vop[T::KS];
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
          kop[ks] = lds_row_operand<D>(Kt, 32 * c, 16 * ks);
          vop[ks] = lds_row_operand<D>(Vt, 32 * c, 16 * ks);
        }
        f32x4 gc2[4], gg[4];
        if (GATED) {
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
            const int k4 = 32 * c + 8 * a4 + 4 * (l >> 5);
            gc2[a4] = *reinterpret_cast<const f32x4*>(tab + k4);
            gg[a4] = *reinterpret_cast<const f32x4*>(tab + T::BN + k4);
          }
        }
        bf16x8 dsb[QB][2], dsl[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          f32x16 s = zero16(), dp = zero16();
#pragma unroll
          for (int ks = 0; ks < T::KS; ++ks) {
            s = mfma(kop[ks], qop[qb][ks], s);
            dp = mfma(vop[ks], doop[qb][ks], dp);
          }
          f32x16 ds;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = sigmoid_l2(s[r], c1, GATED ? gc2[r >> 2][r & 3] : c2);
            const float sp = __builtin_fmaf(-p, p, p);   // p (1 - p)
            ds[r] = dp[r] * (GATED ? sp * gg[r >> 2][r & 3] : sp);
          }
          if (edge || diag) {
            const int query = q0 + 32 * qb + (l & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb + 32 * c + acc_row(r, l);
              const bool ok = key < n && (!CAUSAL || key <= query);
              ds[r] = ok ? ds[r] : 0.0f;
            }
          }
          if (SPLIT) {
            split8(ds, 0, dsb[qb][0], dsl[qb][0], sel);
            split8(ds, 8, dsb[qb][1], dsl[qb][1], sel);
          } else {
            dsb[qb][0] = pack8(ds, 0);
            dsb[qb][1] = pack8(ds, 8);
          }
        }
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
#pragma unroll
          for (int ks2 = 0; ks2 < 2; ++ks2) {
            const bf16x8 kT = lds_col_operand<D>(Kt, 32 * c + 16 * ks2, 32 * dt);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              acc[qb][dt] = mfma(kT, dsb[qb][ks2], acc[qb][dt]);
              if (SPLIT) acc[qb][dt] = mfma(kT, dsl[qb][ks2], acc[qb][dt]);
            }
          }
        }
      }
    }
    if (kt + 1 < nkt) store(kt + 1);
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int query = q0 + 32 * qb + (l & 31);
    if (query < n) {
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
        store_row(a.out0, hoff + (int64_t)query * sl, a.out_f32, acc[qb][dt], 32 * dt, a.scale);
    }
  }
}

template <int D, int QB, bool C, bool G, bool SP>
static hipError_t launch_one(const KArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((dq_kernel<D, QB, C, G, SP>), dim3(a.nitems), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int QB>
static hipError_t dispatch(const KArgs& a, bool c, bool g, bool sp, hipStream_t st) {
  if (c) {
    if (g) return sp ? launch_one<D, QB, true, true, true>(a, st) : launch_one<D, QB, true, true, false>(a, st);
    return sp ? launch_one<D, QB, true, false, true>(a, st) : launch_one<D, QB, true, false, false>(a, st);
  }
  if (g) return sp ? launch_one<D, QB, false, true, true>(a, st) : launch_one<D, QB, false, true, false>(a, st);
  return sp ? launch_one<D, QB, false, false, true>(a, st) : launch_one<D, QB, false, false, false>(a, st);
}

int dq_tile_rows(int d) { return d == 64 ? DqTraits<64, 1>::BM : DqTraits<128, 1>::BM; }

hipError_t launch_dq_bf16(const KArgs& a, int d, bool causal, bool gated, bool split,
                          hipStream_t st) {
  return d == 64 ? dispatch<64, 1>(a, causal, gated, split, st)
                 : dispatch<128, 1>(a, causal, gated, split, st);
}

}  // namespace sa
