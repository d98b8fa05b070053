// Fused exact attention forward pass in float32 for gfx950.
//
// The same method as the bf16 kernel (tiles of keys streamed through LDS, a
// running row max and a running sum of exponentials, one fused kernel:
// FlashAttention (UR), sections "Tiling and block-based processing", "Online
// computation of softmax" and "Fusing the operations into one CUDA kernel"),
// with every product, exponential and sum in float32 on the vector ALUs.  It is
// the accuracy path (small problems, float32 tolerances), not the throughput
// path: gfx950 has no reduced-precision shortcut that would keep float32
// accuracy, and the matrix cores' float32 rate equals the vector rate.
//
// Layout of the work: D/32 consecutive threads share one query row, each owning
// 32 of its D dimensions of q and of the output accumulator; a score is a
// partial dot product per thread summed across those threads with lane shuffles.
// K/V tiles of 32 keys are staged in LDS and read as broadcasts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int BNF = 32;  // keys per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdParams p) {
  constexpr int TPQ = D / 32;           // threads per query row
  constexpr int QPB = kThreads / TPQ;   // query rows per workgroup
  __shared__ __attribute__((aligned(16))) float Ks[BNF][D];
  __shared__ __attribute__((aligned(16))) float Vs[BNF][D];

  const int N = p.N;
  const int tid = threadIdx.x;
  const int sub = tid % TPQ;
  const int qloc = tid / TPQ;
  const int ntiles = (N + QPB - 1) / QPB;
  const int bh = blockIdx.x / ntiles;
  const int qt = blockIdx.x - bh * ntiles;
  const int b = bh / p.H;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  // key/value head of this query head: groups of H / Hkv consecutive heads
  const size_t kvoff = ((size_t)b * p.Hkv + (bh - b * p.H) / (p.H / p.Hkv)) * (size_t)N * D;
  const float* __restrict__ Qh = reinterpret_cast<const float*>(p.q) + hoff;
  const float* __restrict__ Kh = reinterpret_cast<const float*>(p.k) + kvoff;
  const float* __restrict__ Vh = reinterpret_cast<const float*>(p.v) + kvoff;
  float* __restrict__ Oh = reinterpret_cast<float*>(p.o) + hoff;

  int kv_valid = N;
  if (p.seqlens) {
    const int L = p.seqlens[b];
    kv_valid = L < 0 ? 0 : (L > N ? N : L);
  }
  const int qi = qt * QPB + qloc;
  const int qc = min(qi, N - 1);
  int kv_end = kv_valid;
  if (CAUSAL) kv_end = min(kv_end, qt * QPB + QPB);

  float qv[32], acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    qv[c] = Qh[(size_t)qc * D + sub * 32 + c];
    acc[c] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  for (int k0 = 0; k0 < kv_end; k0 += BNF) {
    __syncthreads();
    for (int idx = tid; idx < BNF * D / 4; idx += kThreads) {
      const int row = idx / (D / 4);
      const int c4 = idx % (D / 4);
      const int key = min(k0 + row, N - 1);
      reinterpret_cast<float4*>(&Ks[row][0])[c4] = reinterpret_cast<const float4*>(Kh + (size_t)key * D)[c4];
      reinterpret_cast<float4*>(&Vs[row][0])[c4] = reinterpret_cast<const float4*>(Vh + (size_t)key * D)[c4];
    }
    __syncthreads();

    float s[BNF];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      float part = 0.0f;
#pragma unroll
      for (int c = 0; c < 32; ++c) part = __builtin_fmaf(qv[c], Ks[j][sub * 32 + c], part);
#pragma unroll
      for (int w = 1; w < TPQ; w <<= 1) part += __shfl_xor(part, w, TPQ);
      const int key = k0 + j;
      const bool ok = key < kv_valid && (!CAUSAL || key <= qi);
      s[j] = ok ? part * p.scale : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m, tmax);
    if (m_new == -INFINITY) continue;  // nothing valid for this row yet
    const float alpha = (m == -INFINITY) ? 0.0f : expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < 32; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      const float pj = expf(s[j] - m_new);
      l += pj;
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] = __builtin_fmaf(pj, Vs[j][sub * 32 + c], acc[c]);
    }
    m = m_new;
  }

  if (qi < N) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) Oh[(size_t)qi * D + sub * 32 + c] = acc[c] * inv;
    if (p.lse && sub == 0) p.lse[(size_t)bh * N + qi] = l > 0.0f ? m + logf(l) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  constexpr int QPB = kThreads / (D / 32);
  const int ntiles = (p.N + QPB - 1) / QPB;
  const dim3 grid((unsigned)ntiles * (unsigned)p.H * (unsigned)p.B);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_f32_kernel<D, CAUSAL>), grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  if (p.d == 256) return p.causal ? launch<256, true>(p, stream) : launch<256, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace fa
