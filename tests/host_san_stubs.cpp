// Host-only stand-ins for the device side of libsigattn, for a sanitized CPU build of the
// host code (argument validation, the work planner, the C entry points). Every launcher
// returns success without touching a device; the tile heights are those of the kernels.
// Used by tests/test_abi_sanitized.py only.
#include <hip/hip_runtime.h>

#include "../sigmoid_attention_amd/csrc/aux_args.h"
#include "../sigmoid_attention_amd/csrc/dec_args.h"
#include "../sigmoid_attention_amd/csrc/kargs.h"

namespace sa {
hipError_t launch_fwd_bf16(const KArgs&, int, bool, bool, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_dq_bf16(const KArgs&, int, bool, bool, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_dkdv_bf16(const KArgs&, int, bool, bool, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_bf16(const KArgs&, void*, int, int, bool, bool, bool, hipStream_t) {
  return hipSuccess;
}
int fwd_tile_rows(int) { return 128; }
int dq_tile_rows(int) { return 128; }
int dkdv_tile_rows(int) { return 128; }
hipError_t launch_zero_rows(const ZArgs&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_plane_tail(const PArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_f32(const DArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_cache_build(const BuildArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_cache_append(const AppendArgs&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipSuccess; }
hipError_t noalloc_scratch(hipStream_t, float** out) {
  static float fake[1];
  *out = fake;
  return hipSuccess;
}
int calib_mfma_per_iter() { return 16; }
hipError_t launch_mfma_calib(float*, int64_t*, int, int, hipStream_t) { return hipSuccess; }
}  // namespace sa
