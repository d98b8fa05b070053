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

// One decode problem (few queries against a key/value cache), already
// validated; opart [rows, S, d] and lpart [rows, S] (rows = B * H * Nq) are the
// caller's workspace, S the number of key splits, QBLK the workgroups per
// key/value head along the query rows.
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;               // may be null
  const int32_t* seqlens;   // may be null
  float* opart;
  float* lpart;
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int S, QBLK;
};

// Each forward launcher enqueues exactly one kernel on `stream` and returns the
// HIP error of the launch itself; launch_decode enqueues the split kernel and
// the merge kernel.
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_bf16_d256(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
int decode_rows_per_block();   // query rows per split-kernel workgroup
int decode_tile_keys();        // keys per tile of the split kernel

}  // namespace fa
