// Decoding against a key/value cache with the keys split across workgroups,
// and the merge of the partial results, bf16 in / bf16 out, for gfx950.
//
// Problem: per (batch, head) Nq new queries attend to the cache of that batch's
// valid keys (the pages mention inference kernels built on the same method,
// FlashAttention (UR), section on specialised solutions).  Query i is the
// (L - Nq + i)-th position of a sequence of L valid keys; causal drops the keys
// after it.  Grouped heads as in the forward pass (H_kv key/value heads).
//
// A decode step has little work per key (Nq x group query rows) and a long key
// range, so one workgroup per (batch, key/value head) would leave most of the
// chip idle.  The keys are split into S contiguous chunks of whole tiles; each
// workgroup computes, for all query rows of one key/value head, the softmax-
// weighted average over its chunk and the chunk's log-sum-exp, exactly as one
// K/V stream of the forward pass does (FlashAttention (UR), sections "Tiling
// and block-based processing" and "Online computation of softmax").  A second
// kernel then combines the chunks: LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s, the same combination the online softmax
// applies tile by tile, here applied to whole partial results.
//
// Split kernel: 4 waves; the query rows of a key/value head (head-major, then
// query index) are taken 32 per wave, 128 per workgroup.  K/V tiles of 64 keys
// are double-buffered in LDS by direct global->LDS loads, S^T = K Q^T and
// O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 with the operand layouts of
// the forward kernels.  The step reads the whole cache once per key/value head,
// so it is bound by HBM bandwidth; the softmax keeps the exact running max.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kDecBN = 64;        // keys per tile
constexpr int kDecRows = 128;     // query rows per workgroup (4 waves x 32)

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeParams p) {
  using T = Tile<D, kDecBN>;
  constexpr int BN = kDecBN;
  constexpr int KB = T::KB;
  constexpr int DC = T::DC;
  constexpr int DB = T::DB;
  constexpr int NLD = T::NLD;
  constexpr int NQK = KB * DC;
  constexpr int NPV = KB * 2 * DB;
  __shared__ __attribute__((aligned(1024))) char kbuf[2][T::MAT];
  __shared__ __attribute__((aligned(1024))) char vbuf[2][T::MAT];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  int wg = blockIdx.x;
  const int split = wg % p.S;
  wg /= p.S;
  const int qblk = wg % p.QBLK;
  wg /= p.QBLK;
  const int b = wg / p.Hkv;
  const int hk = wg - b * p.Hkv;
  const int group = p.H / p.Hkv;
  const int R = group * p.Nq;   // query rows of this key/value head

  int L = p.Nk;
  if (p.seqlens) {
    const int x = p.seqlens[b];
    L = x < 0 ? 0 : (x > p.Nk ? p.Nk : x);
  }
  const int ntl = (L + BN - 1) / BN;
  const int per = (ntl + p.S - 1) / p.S;
  const int t0 = min(ntl, split * per);
  const int t1 = min(ntl, t0 + per);   // this workgroup's tiles: [t0, t1)

  // This lane's query row; rows past R compute on a copy of the last row and
  // store nothing.
  const int r = qblk * kDecRows + wave * 32 + r32;
  const bool row_ok = r < R;
  const int rr = row_ok ? r : R - 1;
  const int h = hk * group + rr / p.Nq;
  const int qi = rr - (rr / p.Nq) * p.Nq;
  const int lim = CAUSAL ? L - p.Nq + qi : L - 1;   // last key the row may see
  const bool wave_rows = qblk * kDecRows + wave * 32 < R;

  const __bf16* __restrict__ Kh = reinterpret_cast<const __bf16*>(p.k) + ((size_t)b * p.Hkv + hk) * (size_t)p.Nk * D;
  const __bf16* __restrict__ Vh = reinterpret_cast<const __bf16*>(p.v) + ((size_t)b * p.Hkv + hk) * (size_t)p.Nk * D;
  const size_t qrow = ((size_t)b * p.H + h) * (size_t)p.Nq + qi;   // row of q, o, lse

  bf16x8 qf[DC];
  {
    const u32x4* row = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(p.q) + qrow * D);
#pragma unroll
    for (int s = 0; s < DC; ++s) qf[s] = __builtin_bit_cast(bf16x8, row[2 * s + hi]);
  }
  const int kx = kswz<D>(r32);
  const int kbase = r32 * T::ROW + (((kx >> 1) << 1 | (hi ^ (kx & 1))) << 4);
  const int i16 = lane & 15;
  const int g16 = (lane >> 4) & 1;
  const int vrow = 4 * hi + (i16 >> 2);
  const int vbase = vrow * T::ROW + (((2 * g16 + ((i16 & 3) >> 1)) ^ vswz<D>(vrow)) << 4) + (i16 & 1) * 8;

  int ld_row[NLD], ld_kc[NLD], ld_vc[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int pos = (wave * NLD + i) * 64 + lane;
    const int row = pos / T::CH;
    const int cst = pos % T::CH;
    ld_row[i] = row;
    ld_kc[i] = (cst ^ kswz<D>(row)) * 8;
    ld_vc[i] = (cst ^ vswz<D>(row)) * 8;
  }
  auto load = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int key = min(t * BN + ld_row[i], p.Nk - 1);
      dma16(Kh + (size_t)key * D + ld_kc[i], kbuf[t & 1] + (wave * NLD + i) * 1024);
      dma16(Vh + (size_t)key * D + ld_vc[i], vbuf[t & 1] + (wave * NLD + i) * 1024);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sc = p.scale * kLog2e;

  auto tile = [&](int t) __attribute__((always_inline)) {
    const char* Ks = kbuf[t & 1];
    const char* Vs = vbuf[t & 1];
    u32x4 kfr[NQK];
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int s_ = i / KB, kb = i % KB;
      kfr[i] = *reinterpret_cast<const u32x4*>(Ks + kb * 32 * T::ROW + (kbase ^ (s_ << 5)));
    }
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int s_ = i / KB, kb = i % KB;
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kfr[i]), qf[s_], sacc[kb], 0, 0, 0);
    }
    const int k0 = t * BN;
    if (k0 + BN > L || (CAUSAL && k0 + BN - 1 > L - p.Nq)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
          sacc[kb][e] = (key < L && key <= lim) ? sacc[kb][e] : -INFINITY;
        }
    }
    // exact running max (the step is bound by HBM; the rescale costs nothing)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    mx = pair_max(mx) * sc;
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == -INFINITY || m_run == m_new) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float mref = m_new == -INFINITY ? 0.0f : m_new;
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[cb][e] *= alpha;
    uint32_t pk[KB][8];
    float part[KB * 8];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][2 * j], sc, -mref));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][2 * j + 1], sc, -mref));
        part[kb * 8 + j] = p0 + p1;
        pk[kb][j] = pack_bf16(p0, p1);
      }
    l_run += tree_sum(part);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int kb = i / (2 * DB), u = (i / DB) & 1, cb = i % DB;
      char* vb = const_cast<char*>(Vs) + (kb * 32 + 16 * u) * T::ROW + (vbase ^ (cb << 6));
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * T::ROW));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, v0);
      const u32x2 hi2 = __builtin_bit_cast(u32x2, v1);
      const u32x4 a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
      const u32x4 b4 = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
      oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4),
                                                         oacc[cb], 0, 0, 0);
    }
  };

  if (t0 < t1) {
    load(t0);
    wait_vmem();
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
      if (t + 1 < t1) load(t + 1);   // into the buffer the previous tile used
      if (wave_rows) tile(t);
      wait_vmem();
      __syncthreads();
    }
  }

  const float l = pair_sum(l_run);
  if (row_ok) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* orow = p.opart + (qrow * p.S + split) * D;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = cb * 32 + 8 * g + 4 * hi;
        typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
        const f32x4 w = {oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv, oacc[cb][4 * g + 2] * inv,
                         oacc[cb][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + col) = w;
      }
    if (hi == 0) p.lpart[qrow * p.S + split] = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
  }
}

// Merge: one wave per query row; lane c holds columns c, c + 64, ...
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int rows) {
  constexpr int CPL = D / 64;   // columns per lane
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const float* lp = p.lpart + (size_t)row * p.S;
  float mx = -INFINITY;
  for (int s = lane; s < p.S; s += 64) mx = fmaxf(mx, lp[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  __bf16* orow = reinterpret_cast<__bf16*>(p.o) + (size_t)row * D;
  if (mx == -INFINITY) {   // no split saw a key
#pragma unroll
    for (int c = 0; c < CPL; ++c) orow[lane + 64 * c] = (__bf16)0.0f;
    if (p.lse && lane == 0) p.lse[row] = -INFINITY;
    return;
  }
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
  float tot = 0.0f;
  const float* op = p.opart + (size_t)row * p.S * D;
  for (int s = 0; s < p.S; ++s) {
    const float ls = lp[s];
    if (ls == -INFINITY) continue;   // an empty split (uniform across the wave)
    const float w = __builtin_amdgcn_exp2f((ls - mx) * kLog2e);
    tot += w;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = __builtin_fmaf(w, op[(size_t)s * D + lane + 64 * c], acc[c]);
  }
  const float inv = 1.0f / tot;
#pragma unroll
  for (int c = 0; c < CPL; ++c) orow[lane + 64 * c] = (__bf16)(acc[c] * inv);
  if (p.lse && lane == 0) p.lse[row] = mx + log2f(tot) * kLn2;
}

template <int D, bool CAUSAL>
hipError_t launch_split(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.B * (unsigned)p.Hkv * (unsigned)p.QBLK * (unsigned)p.S);
  DecodeParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_split_kernel<D, CAUSAL>), grid, dim3(256), args, 0, stream);
}

template <int D>
hipError_t launch_merge(const DecodeParams& p, hipStream_t stream) {
  int rows = p.B * p.H * p.Nq;
  const dim3 grid((unsigned)((rows + 3) / 4));
  DecodeParams arg = p;
  void* args[] = {&arg, &rows};
  return hipLaunchKernel(reinterpret_cast<const void*>(&decode_merge_kernel<D>), grid, dim3(256), args, 0, stream);
}

}  // namespace

int decode_rows_per_block() { return kDecRows; }
int decode_tile_keys() { return kDecBN; }

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  hipError_t e;
  if (p.d == 64) e = p.causal ? launch_split<64, true>(p, stream) : launch_split<64, false>(p, stream);
  else e = p.causal ? launch_split<128, true>(p, stream) : launch_split<128, false>(p, stream);
  if (e != hipSuccess) return e;
  return p.d == 64 ? launch_merge<64>(p, stream) : launch_merge<128>(p, stream);
}

}  // namespace fa
