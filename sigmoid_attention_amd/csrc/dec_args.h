// Argument blocks of the KV-cache kernels (cache build from a prefill, threshold append,
// single-query decode and its chunk reduction).
#pragma once
#include <stdint.h>

#include "kargs.h"

namespace sa {

constexpr int kDecChunk = 512;   // cache entries per decode workgroup
constexpr int kBuildRows = 256;  // prefill rows per cache-build workgroup
// floats of the static device workspace of the allocation-free decode (16 MiB per GPU)
constexpr int64_t kNoAllocFloats = int64_t(1) << 22;

struct CacheView {
  void* k;               // [B][H][cap][d] bf16
  void* v;
  float* gate;           // [B][cap] or null (ungated cache)
  int32_t* count;        // [B] live entries
  int32_t* seen;         // [B] positions written
  int64_t sb, sh, sl;    // element strides of k and v
  int32_t H, cap, d;
  float gate_eps, gate_tau;
  int32_t gate_sink;
};

struct BuildArgs {
  CacheView c;
  const void* k;         // prefill K, V: [B][H][Lmax][d] bf16
  const void* v;
  const float* gate;     // prefill gate [B][gsb] or null
  int64_t sb, sh, sl, gsb;
  int32_t Lmax;
  uint16_t len[kMaxBatch];   // valid prefill length by batch index
};

struct AppendArgs {
  CacheView c;
  const void* k;         // new entries [B][H][d] bf16
  const void* v;
  const float* gate;     // [B] or null
  int64_t nsb, nsh;      // element strides of the new entries
  int32_t* status;       // set to 1 when an entry to keep finds its cache full; or null
};

struct DecodeArgs {
  CacheView c;
  const void* q;         // [B][H][d] bf16
  void* out;             // [B][H][d], float or bf16, strides of q
  float* ws;             // [B*H][nchunk][d] float partial sums
  int64_t qsb, qsh;      // element strides of q and out
  int32_t B;
  int32_t nchunk;        // ceil(cap / kDecChunk)
  int32_t out_f32;
  float c1;              // -s * log2(e)
  float c2[kMaxBatch];   // -beta_b * log2(e)
};

}  // namespace sa
