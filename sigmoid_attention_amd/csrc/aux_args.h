// Argument blocks of the auxiliary kernels (padded-row zero fill, float32 debug path).
#pragma once
#include <stdint.h>

#include "kargs.h"

namespace sa {

constexpr int kZeroRows = 32;

struct ZArgs {
  void* o0;
  void* o1;              // second output or null
  void* o2;              // third output or null
  int64_t sb, sh, sl;    // element strides
  int32_t Lmax;
  int32_t block0;        // first row block holding a padded row (shortest sequence's)
  int32_t row_bytes;     // d * element size (a multiple of 16)
  int32_t esize;         // element size in bytes
  uint16_t len[kMaxBatch];   // valid length by batch index
};

// Per-head float planes [B][H][Lmax] (gate gradient, row mass): zero the entries
// j >= n_b and, when sum is set, write sum[b][j] = sum over h of plane[b][h][j].
struct PArgs {
  float* plane;
  float* sum;            // [B][Lmax] or null
  int32_t B, H, Lmax;
  uint16_t len[kMaxBatch];   // valid length by batch index
};

struct DArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* out0;
  void* out1;
  float* aux;            // dg plane of the dk/dv pass, row-mass plane of the forward
  const float* gate;
  int64_t sb, sh, sl, gsb;
  int32_t B, H, Lmax, d;
  int32_t causal;
  int32_t gate_sink;
  float scale;
  float gate_eps;
  float gate_tau;
  int32_t len[kMaxBatch];    // by batch index
  float beta[kMaxBatch];     // by batch index
};

}  // namespace sa
