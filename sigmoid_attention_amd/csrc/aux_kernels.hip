// Auxiliary kernels:
//  * zero_rows: writes exact zeros into the padded rows (i >= n_b) of up to three
//    outputs, so that every output element is defined. The grid starts at the row block
//    of the shortest sequence's first padded row; blocks below a longer sequence's
//    length exit at once. Padded input slots are never
//    read (padded tiles are skipped, "Better Models, Faster Training: Sigmoid Attention
//    for single-cell Foundation Models", section 4).
//  * plane_tail: per-head float planes [B][H][Lmax] (gate gradient, row mass): zeros
//    for j >= n_b, and the sum over heads of the gate gradient, in head order (the gate
//    is shared by the heads, so its gradient is the sum of the per-head ones).
//  * the float32 debug path: one wave per output row, plain loops with a wave-wide
//    reduction for each dot product. It is slow and simple on purpose; it computes the
//    same definitions as the bf16 kernels (section 3 equation; gate injection and
//    hard drop from "Sigmoid Attention as a Better Substrate for Learned KV Cache
//    Eviction"; backward through the diagonal Jacobian, appendix A.1.2).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aux_args.h"

namespace sa {

__global__ __launch_bounds__(256) void zero_rows_kernel(const ZArgs z) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int n = z.len[b];
  const int row0 = (z.block0 + blockIdx.x) * kZeroRows;
  if (row0 + kZeroRows <= n) return;
  const int cpr = z.row_bytes / 16;
  const int64_t hoff = ((int64_t)b * z.sb + (int64_t)h * z.sh) * z.esize;
  for (int idx = threadIdx.x; idx < kZeroRows * cpr; idx += blockDim.x) {
    const int row = row0 + idx / cpr;
    if (row < n || row >= z.Lmax) continue;
    const int64_t off = hoff + (int64_t)row * z.sl * z.esize + (int64_t)(idx % cpr) * 16;
    const uint4 zero = {0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>((char*)z.o0 + off) = zero;
    if (z.o1) *reinterpret_cast<uint4*>((char*)z.o1 + off) = zero;
    if (z.o2) *reinterpret_cast<uint4*>((char*)z.o2 + off) = zero;
  }
}

hipError_t launch_zero_rows(const ZArgs& z, int B, int H, hipStream_t st) {
  dim3 grid((z.Lmax + kZeroRows - 1) / kZeroRows - z.block0, H, B);
  hipLaunchKernelGGL(zero_rows_kernel, grid, dim3(256), 0, st, z);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void plane_tail_kernel(const PArgs pa) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= pa.Lmax) return;
  const int n = pa.len[b];
  float* row = pa.plane + (int64_t)b * pa.H * pa.Lmax + j;
  float acc = 0.0f;
  for (int h = 0; h < pa.H; ++h) {
    if (j >= n) row[(int64_t)h * pa.Lmax] = 0.0f;
    else acc += row[(int64_t)h * pa.Lmax];
  }
  if (pa.sum) pa.sum[(int64_t)b * pa.Lmax + j] = acc;
}

hipError_t launch_plane_tail(const PArgs& pa, hipStream_t st) {
  dim3 grid((pa.Lmax + 255) / 256, pa.B);
  hipLaunchKernelGGL(plane_tail_kernel, grid, dim3(256), 0, st, pa);
  return hipGetLastError();
}

// ------------------------------- float32 debug path -------------------------------

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// dot product of two d-long rows spread over the 64 lanes (d / 64 elements per lane)
__device__ __forceinline__ float row_dot(const float* a, const float* b, int d, int lane) {
  float s = 0.0f;
  for (int c = lane; c < d; c += 64) s = fmaf(a[c], b[c], s);
  return wave_sum(s);
}

struct KeyRule {
  const DArgs& a;
  int b, n;
  __device__ bool kept(int j) const {
    if (!a.gate || a.gate_tau <= 0.0f) return true;
    const float g = a.gate[(int64_t)b * a.gsb + j];
    return !(j >= a.gate_sink && g < a.gate_tau);
  }
  __device__ float gate(int j) const { return a.gate ? a.gate[(int64_t)b * a.gsb + j] : 1.0f; }
  __device__ float logit(float dot, int j) const {
    float x = a.scale * dot + a.beta[b];
    if (a.gate) x += logf(gate(j) + a.gate_eps);
    return x;
  }
};

__device__ __forceinline__ float logistic(float x) { return 1.0f / (1.0f + expf(-x)); }

// pass 0: O, pass 1: dQ (one wave per query row); pass 2: dK, dV (one wave per key row)
__global__ __launch_bounds__(256) void f32_kernel(const DArgs a, int pass) {
  const int lane = threadIdx.x & 63;
  const int64_t row_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows_per_b = (int64_t)a.H * a.Lmax;
  const int b = (int)(row_id / rows_per_b);
  if (b >= a.B) return;
  const int h = (int)((row_id % rows_per_b) / a.Lmax);
  const int i = (int)(row_id % a.Lmax);
  const int n = a.len[b];
  if (i >= n) return;
  const int64_t hoff = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const float* Q = (const float*)a.q + hoff;
  const float* K = (const float*)a.k + hoff;
  const float* V = (const float*)a.v + hoff;
  const float* dO = (const float*)a.dout + hoff;
  const KeyRule rule{a, b, n};
  const int64_t sl = a.sl;
  constexpr int MAXC = 2;  // d / 64 elements per lane, d <= 128
  float acc0[MAXC] = {0.0f, 0.0f}, acc1[MAXC] = {0.0f, 0.0f};

  const int64_t plane_idx = ((int64_t)b * a.H + h) * a.Lmax + i;
  if (pass == 0 || pass == 1) {
    const float* qi = Q + (int64_t)i * sl;
    const float* doi = dO + (int64_t)i * sl;
    float mass = 0.0f;
    for (int j = 0; j < n; ++j) {
      if (a.causal && j > i) break;
      if (!rule.kept(j)) continue;
      const float* kj = K + (int64_t)j * sl;
      const float* vj = V + (int64_t)j * sl;
      const float p = logistic(rule.logit(row_dot(qi, kj, a.d, lane), j));
      const float g = rule.gate(j);
      mass += p;
      if (pass == 0) {
        for (int c = lane, e = 0; c < a.d; c += 64, ++e) acc0[e] = fmaf(p * g, vj[c], acc0[e]);
      } else {
        const float ds = g * row_dot(doi, vj, a.d, lane) * p * (1.0f - p);
        for (int c = lane, e = 0; c < a.d; c += 64, ++e) acc0[e] = fmaf(ds, kj[c], acc0[e]);
      }
    }
    float* out = (float*)a.out0 + hoff + (int64_t)i * sl;
    const float mul = pass == 0 ? 1.0f : a.scale;
    for (int c = lane, e = 0; c < a.d; c += 64, ++e) out[c] = acc0[e] * mul;
    if (pass == 0 && a.aux && lane == 0) a.aux[plane_idx] = mass;
  } else {
    const int j = i;  // this wave owns key row j
    const float* kj = K + (int64_t)j * sl;
    const float* vj = V + (int64_t)j * sl;
    const bool keep = rule.kept(j);
    const float g = rule.gate(j);
    float ds_sum = 0.0f;
    if (keep) {
      for (int qi_ = a.causal ? j : 0; qi_ < n; ++qi_) {
        const float* qi = Q + (int64_t)qi_ * sl;
        const float* doi = dO + (int64_t)qi_ * sl;
        const float p = logistic(rule.logit(row_dot(qi, kj, a.d, lane), j));
        const float ds = g * row_dot(doi, vj, a.d, lane) * p * (1.0f - p);
        ds_sum += ds;
        for (int c = lane, e = 0; c < a.d; c += 64, ++e) {
          acc1[e] = fmaf(p, doi[c], acc1[e]);   // dV before the gate factor
          acc0[e] = fmaf(ds, qi[c], acc0[e]);   // dK before the scale
        }
      }
    }
    float* dk = (float*)a.out0 + hoff + (int64_t)j * sl;
    float* dv = (float*)a.out1 + hoff + (int64_t)j * sl;
    for (int c = lane, e = 0; c < a.d; c += 64, ++e) {
      dk[c] = keep ? acc0[e] * a.scale : 0.0f;
      dv[c] = keep ? acc1[e] * g : 0.0f;
    }
    if (a.aux) {
      // gate gradient: sum_i dS_ij / (g_j + eps) + v_j . sum_i P_ij dO_i
      float vd = 0.0f;
      for (int c = lane, e = 0; c < a.d; c += 64, ++e) vd = fmaf(vj[c], acc1[e], vd);
      vd = wave_sum(vd);
      if (lane == 0) a.aux[plane_idx] = keep ? ds_sum / (g + a.gate_eps) + vd : 0.0f;
    }
  }
}

hipError_t launch_f32(const DArgs& a, int pass, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.H * a.Lmax;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, pass);
  return hipGetLastError();
}

}  // namespace sa
