// KV cache with threshold eviction and single-query decode, on gfx950.
//
// "Sigmoid Attention as a Better Substrate for Learned KV Cache Eviction", gate
// paragraphs: a token-wise gate g_j enters the logits as log(g_j + eps) and the values as
// g_j v_j; at inference, entries with g_j < tau are physically removed after prefill and
// every entry written during decode is kept or removed by the same rule; kept entries keep
// their logit and value scaling. The cache therefore holds only kept entries, in position
// order, with their gates; the positions below `sink` are never removed.
//
//  * cache_build: compaction of a prefill. One workgroup per (sequence, block of 256
//    positions) counts the kept positions before its block, scans its own block's keep
//    flags (wave ballots) and copies the kept K and V rows of every head to their slots.
//  * cache_append: one decode-time write per sequence; the counters live on the device,
//    so a serving loop never reads the gates back to the host.
//  * decode: o = sum_j sigma(s q . k_j + beta [+ log(g_j + eps)]) [g_j] v_j over the live
//    entries. One query against a stream of cache rows is a matrix-vector product: it is
//    bound by HBM bandwidth, not by the matrix cores, so it runs on the vector ALUs. Each
//    cache row is read by 8 lanes with non-temporal 16-byte loads, so that each load
//    instruction covers whole 128-byte lines (a streamed row is never read again); the
//    dot product uses v_dot2_f32_bf16 and a butterfly over the row's lanes; eight steps
//    of loads are issued before their math so that enough bytes are in flight. The rows
//    of one (b, h) are split into chunks of 512 entries, one workgroup each, so that the
//    work is even whatever the cache lengths; a chunk's partial sum of weighted values is
//    a plain sum (no row maximum or normaliser to merge, unlike softmax), written to a
//    workspace and added up in chunk order by a second kernel: deterministic, no atomics.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.h"
#include "dec_args.h"

namespace sa {

// Workspace of the allocation-free decode entry point: the per-chunk partial sums live in
// this file-scope device array instead of caller memory. Each GPU the library runs on
// holds its own copy until the process ends. In host code the name `scratch` is only a
// host-side stand-in: its device address is looked up per device (noalloc_scratch) and
// only that address is ever handed to a kernel.
static __device__ __align__(256) float scratch[kNoAllocFloats];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the device that `stream` belongs to, looked up once per
// device with that device current (hipGetSymbolAddress), then cached.
hipError_t noalloc_scratch(hipStream_t stream, float** out) {
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

// ------------------------------------ cache build ------------------------------------

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__global__ __launch_bounds__(256) void cache_build_kernel(const BuildArgs a) {
  const int b = blockIdx.y;
  const int n = a.len[b];
  const int r0 = blockIdx.x * kBuildRows;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const bool count_owner = n == 0 ? blockIdx.x == 0 : (n - 1) / kBuildRows == (int)blockIdx.x;
  if (r0 >= n && !count_owner) return;
  const float* g = a.gate ? a.gate + (int64_t)b * a.gsb : nullptr;
  const float tau = a.c.gate_tau;
  const int sink = a.c.gate_sink;
  auto keep = [&](int j) { return !g || tau <= 0.0f || j < sink || g[j] >= tau; };

  __shared__ int red[4];
  __shared__ int wtot[4];
  __shared__ int slot[kBuildRows];

  // kept positions before this block
  int cnt = 0;
  for (int j = tid; j < r0; j += 256) cnt += keep(j) ? 1 : 0;
  cnt = wave_sum_i(cnt);
  if (l == 0) red[w] = cnt;
  // this block's keep flags: exclusive prefix by wave ballots
  const int row = r0 + tid;
  const bool f = row < n && keep(row);
  const uint64_t mask = __ballot(f);
  const int before = __popcll(mask & ((1ull << l) - 1ull));
  if (l == 0) wtot[w] = __popcll(mask);
  __syncthreads();
  const int base = red[0] + red[1] + red[2] + red[3];
  int pre = before;
  for (int v = 0; v < w; ++v) pre += wtot[v];
  const int total = base + wtot[0] + wtot[1] + wtot[2] + wtot[3];
  const int s = base + pre;
  slot[tid] = f ? s : -1;
  if (f && a.c.gate) a.c.gate[(int64_t)b * a.c.cap + s] = g ? g[row] : 1.0f;
  __syncthreads();

  // copy the kept rows of every head, 16 bytes per thread and step
  const int cpr = a.c.d / 8;
  const int per_row = a.c.H * cpr;
  const int rows = (n - r0 < kBuildRows) ? (n - r0) : kBuildRows;
  for (int idx = tid; idx < rows * per_row; idx += 256) {
    const int r = idx / per_row;
    const int dst_slot = slot[r];
    if (dst_slot < 0) continue;
    const int rem = idx - r * per_row;
    const int h = rem / cpr;
    const int c = rem - h * cpr;
    const int64_t src = (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)(r0 + r) * a.sl + 8 * c;
    const int64_t dst = (int64_t)b * a.c.sb + (int64_t)h * a.c.sh + (int64_t)dst_slot * a.c.sl + 8 * c;
    *reinterpret_cast<uint4*>((bf16*)a.c.k + dst) = *reinterpret_cast<const uint4*>((const bf16*)a.k + src);
    *reinterpret_cast<uint4*>((bf16*)a.c.v + dst) = *reinterpret_cast<const uint4*>((const bf16*)a.v + src);
  }
  if (count_owner && tid == 0) {
    a.c.count[b] = total;
    a.c.seen[b] = n;
  }
}

hipError_t launch_cache_build(const BuildArgs& a, int B, hipStream_t st) {
  dim3 grid((a.Lmax + kBuildRows - 1) / kBuildRows, B);
  hipLaunchKernelGGL(cache_build_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------ cache append -----------------------------------

__global__ __launch_bounds__(256) void cache_append_kernel(const AppendArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int cnt = a.c.count[b];
  const int pos = a.c.seen[b];
  const float g = a.gate ? a.gate[b] : 1.0f;
  const bool keep = !a.gate || a.c.gate_tau <= 0.0f || pos < a.c.gate_sink || g >= a.c.gate_tau;
  const bool fits = cnt >= 0 && cnt < a.c.cap;
  if (keep && fits) {
    const int cpr = a.c.d / 8;
    for (int idx = tid; idx < a.c.H * cpr; idx += 256) {
      const int h = idx / cpr, c = idx - h * cpr;
      const int64_t src = (int64_t)b * a.nsb + (int64_t)h * a.nsh + 8 * c;
      const int64_t dst = (int64_t)b * a.c.sb + (int64_t)h * a.c.sh + (int64_t)cnt * a.c.sl + 8 * c;
      *reinterpret_cast<uint4*>((bf16*)a.c.k + dst) = *reinterpret_cast<const uint4*>((const bf16*)a.k + src);
      *reinterpret_cast<uint4*>((bf16*)a.c.v + dst) = *reinterpret_cast<const uint4*>((const bf16*)a.v + src);
    }
    if (tid == 0 && a.c.gate) a.c.gate[(int64_t)b * a.c.cap + cnt] = g;
  }
  __syncthreads();   // every thread has read the counters before they change
  if (tid == 0) {
    a.c.count[b] = cnt + ((keep && fits) ? 1 : 0);
    a.c.seen[b] = pos + 1;
    if (keep && !fits && a.status) *a.status = 1;
  }
}

hipError_t launch_cache_append(const AppendArgs& a, int B, hipStream_t st) {
  hipLaunchKernelGGL(cache_append_kernel, dim3(B), dim3(256), 0, st, a);
  return hipGetLastError();
}

// --------------------------------------- decode --------------------------------------

// live entries of sequence b, clamped to the cache's capacity so that a corrupted
// counter can never address rows outside the cache
__device__ __forceinline__ int live_count(const CacheView& c, int b) {
  const int m = c.count[b];
  return m < 0 ? 0 : (m > c.cap ? c.cap : m);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// 16 bytes of a cache row, which is read once per decode: a non-temporal load
__device__ __forceinline__ bf16x8 stream_load(const bf16* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return __builtin_bit_cast(bf16x8, v);
}

template <int I>
__device__ __forceinline__ bf16x2 pair(const bf16x8& v) {
  return __builtin_shufflevector(v, v, 2 * I, 2 * I + 1);
}

// dot product of 8 bf16 pairs in float: v_dot2_f32_bf16, accumulating into acc
__device__ __forceinline__ float dot8(const bf16x8& a, const bf16x8& b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(pair<0>(a), pair<0>(b), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(pair<1>(a), pair<1>(b), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(pair<2>(a), pair<2>(b), acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(pair<3>(a), pair<3>(b), acc, false);
}

template <int D, bool GATED>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a) {
  constexpr int LPK = 8;                   // lanes per cache row
  constexpr int NL = D / 64;               // 16-byte loads per lane and row (one per 128 B)
  constexpr int KPS = 64 / LPK;            // rows per wave step
  constexpr int U = 8;                     // steps whose loads are issued together
  constexpr int KPW = kDecChunk / 4;       // rows per wave and chunk
  constexpr int NIT = KPW / (U * KPS);
  static_assert(NIT * U * KPS == KPW, "chunk must split into whole iterations");

  const int bh = blockIdx.x / a.nchunk;
  const int chunk = blockIdx.x - bh * a.nchunk;
  const int b = bh / a.c.H, h = bh - b * a.c.H;
  const int m = live_count(a.c, b);
  const int c0 = chunk * kDecChunk;
  if (c0 >= m) return;

  const int l = lane_id(), w = wave_id();
  const int ks = l / LPK, sub = l % LPK;
  // this lane's features: 64 i + 8 sub .. 64 i + 8 sub + 7 for i < NL, so that each load
  // instruction of a wave covers whole 128-byte lines of its rows
  const bf16* qp = (const bf16*)a.q + (int64_t)b * a.qsb + (int64_t)h * a.qsh + 8 * sub;
  bf16x8 qv[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) qv[i] = *reinterpret_cast<const bf16x8*>(qp + 64 * i);
  const int64_t hoff = (int64_t)b * a.c.sb + (int64_t)h * a.c.sh;
  const bf16* Kb = (const bf16*)a.c.k + hoff + 8 * sub;
  const bf16* Vb = (const bf16*)a.c.v + hoff + 8 * sub;
  const float* Gb = GATED ? a.c.gate + (int64_t)b * a.c.cap : nullptr;
  const float c1 = a.c1, c2 = a.c2[b], eps = a.c.gate_eps;
  const int64_t sl = a.c.sl;
  const int last = m - 1;

  float acc[8 * NL];
#pragma unroll
  for (int e = 0; e < 8 * NL; ++e) acc[e] = 0.0f;

  const int wbase = c0 + w * KPW;
  for (int it = 0; it < NIT; ++it) {
    const int jb = wbase + it * U * KPS;
    if (jb >= m) break;   // wave-uniform
    bf16x8 kr[U][NL], vr[U][NL];
    float gv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * KPS + ks;
      const int64_t row = (int64_t)(j < last ? j : last) * sl;   // rows past m read row m-1
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        kr[u][i] = stream_load(Kb + row + 64 * i);
        vr[u][i] = stream_load(Vb + row + 64 * i);
      }
      if (GATED) gv[u] = Gb[j < last ? j : last];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * KPS + ks;
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < NL; ++i) dot = dot8(qv[i], kr[u][i], dot);
#pragma unroll
      for (int off = 1; off < LPK; off <<= 1) dot += __shfl_xor(dot, off, 64);
      float t = __builtin_fmaf(dot, c1, c2);
      if (GATED) t -= __builtin_amdgcn_logf(gv[u] + eps);
      float p = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
      if (GATED) p *= gv[u];
      p = j < m ? p : 0.0f;
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[8 * i + e] = __builtin_fmaf(p, (float)vr[u][i][e], acc[8 * i + e]);
    }
  }

  // sum over the rows held by the wave's lanes, then over the four waves in order
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8 * NL; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  __shared__ float red[4][D];
  if (ks == 0) {
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[w][64 * i + 8 * sub + e] = acc[8 * i + e];
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < D)
    a.ws[((int64_t)bh * a.nchunk + chunk) * D + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

__global__ __launch_bounds__(256) void decode_reduce_kernel(const DecodeArgs a) {
  const int D = a.c.d;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.B * a.c.H * D) return;
  const int bh = (int)(idx / D), e = (int)(idx - (int64_t)bh * D);
  const int b = bh / a.c.H, h = bh - b * a.c.H;
  const int m = live_count(a.c, b);
  const int nch = (m + kDecChunk - 1) / kDecChunk;
  float s = 0.0f;
  for (int c = 0; c < nch; ++c) s += a.ws[((int64_t)bh * a.nchunk + c) * D + e];
  const int64_t off = (int64_t)b * a.qsb + (int64_t)h * a.qsh + e;
  if (a.out_f32) reinterpret_cast<float*>(a.out)[off] = s;
  else reinterpret_cast<bf16*>(a.out)[off] = (bf16)s;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  const int grid = a.B * a.c.H * a.nchunk;
  if (grid > 0) {
    const bool g = a.c.gate != nullptr;
    if (a.c.d == 64) {
      if (g) hipLaunchKernelGGL((decode_kernel<64, true>), dim3(grid), dim3(256), 0, st, a);
      else hipLaunchKernelGGL((decode_kernel<64, false>), dim3(grid), dim3(256), 0, st, a);
    } else {
      if (g) hipLaunchKernelGGL((decode_kernel<128, true>), dim3(grid), dim3(256), 0, st, a);
      else hipLaunchKernelGGL((decode_kernel<128, false>), dim3(grid), dim3(256), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t elems = (int64_t)a.B * a.c.H * a.c.d;
  if (elems > 0)
    hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((elems + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sa
