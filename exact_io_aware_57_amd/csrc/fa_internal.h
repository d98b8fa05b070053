// Internal interface between the host entry points (fa_api.hip) and the kernel
// launchers (fa_fwd_bf16.hip, fa_fwd_f32.hip).  Not installed, not part of the
// C interface in include/fa.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One forward problem, already validated on the host.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;               // may be null
  const int32_t* seqlens;   // may be null
  int B, H, N, d;
  int Hkv;                  // key/value heads; divides H (H: plain multi-head)
  float scale;
  int causal;
};

// Each launcher enqueues exactly one kernel on `stream` and returns the HIP
// error of the launch itself.
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);

}  // namespace fa
