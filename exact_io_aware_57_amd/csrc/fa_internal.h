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
  // FP8 inputs only: the tensors are descale * value(code)
  float descale_q = 1.0f, descale_k = 1.0f, descale_v = 1.0f;
  int num_cu = 256;         // compute units of the device the launch runs on
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
hipError_t launch_fwd_fp8(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// Backward pass.  lse2 and delta point into the caller's workspace: per query
// row (rows of each head padded to Npad, a multiple of bwd_row_pad()) the
// forward LSE times log2(e) and D = dO . O.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* seqlens;   // may be null
  float* lse2;
  float* delta;
  int B, H, Hkv, N, Npad, d;
  float scale;
  int causal;
};

// Enqueues the row-dot kernel, the dK/dV kernel and the dQ kernel.
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);
int bwd_row_pad();
int decode_rows_per_block();   // query rows per split-kernel workgroup
int decode_tile_keys();        // keys per tile of the split kernel

}  // namespace fa
