// Fused exact attention forward pass, bf16 in / bf16 out, for CDNA4 (gfx950).
//
// What is computed: O = softmax(scale * Q K^T) V per (batch, head), plus the row
// log-sum-exp (FlashAttention (UR), section "The problem of standard attention").
// How: the method of FlashAttention (UR), sections "Tiling and block-based
// processing", "Online computation of softmax" and "Fusing the operations into
// one CUDA kernel": one kernel loads a tile of queries once, streams K/V tiles
// through on-chip memory, and keeps a running row max and a running sum of
// exponentials, so the N x N score matrix only ever exists as a register tile.
// FlashAttention-2 (HI), "Technical architecture", gives the three changes kept
// here: (1) few non-matmul operations, (2) one head spread over many compute
// units by giving each workgroup its own tile of query rows, (3) a split of the
// work inside a workgroup that needs no exchange of softmax state between
// waves.
//
// Mapping to gfx950:
//  * A workgroup is 4 waves and owns BM = 4 * 32 * QB query rows of one
//    (batch, head); each wave owns 32 * QB rows outright, so softmax state never
//    crosses waves.  K/V tiles of 64 keys are shared by the 4 waves through LDS,
//    double-buffered: the global loads of tile t+1 are in flight while tile t is
//    computed.
//  * Both products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//    S is computed transposed, S^T = K Q^T, so that in the accumulator layout
//    each lane holds 16 keys of ONE query: the row max and the row sum are
//    in-lane reductions plus a single exchange with lane^32.
//  * O is accumulated transposed too, O^T = V^T P^T: the B operand (P^T) is the
//    S^T accumulator converted to bf16 in place (no LDS round trip), and the A
//    operand (V^T, keys contiguous) is read from the row-major V tile with the
//    gfx950 transposing LDS read ds_read_b64_tr_b16.  Each lane again holds one
//    query's outputs, so the softmax rescale is a per-lane scalar.
//  * Non-matmul work per score: one FMA (scale and max subtraction folded), one
//    v_exp_f32 (base 2), a third of a v_max3, half a v_cvt_pk_bf16_f32 and half
//    a v_dot2 (the row sum over the same bf16-rounded P that feeds the second
//    product).  The output is rescaled only when a row max grows by more than
//    2^8 in the exponent (the result is the same; P may reach 2^8 in between),
//    and divided by the row sum once at the end.
//  * Masks are applied only on tiles that straddle a boundary (causal diagonal,
//    last valid key); tiles wholly above a wave's causal diagonal are skipped.
//  * Workgroups are renumbered so that each XCD (each its own L2) receives a
//    contiguous run of (head, query tile) pairs, and causal query tiles are
//    issued heaviest first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BN = 64;            // keys per K/V tile
constexpr int KB = BN / 32;       // 32-key blocks per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;      // lazy-rescale threshold, log2 units

template <int D>
struct Tile {
  static constexpr int CH = D / 8;                  // 16-byte chunks per row
  static constexpr int DC = D / 16;                 // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;                 // 32-row blocks of O^T
  static constexpr int ROW = D * 2;                 // bytes per row
  static constexpr int MAT = BN * ROW;              // one K or V tile
  static constexpr int STAGE = 2 * MAT;             // K + V
  static constexpr int NLD = BN * CH / kThreads;    // 16-byte loads per thread per matrix
  static_assert(BN * CH % kThreads == 0, "tile load must split evenly");
};

// K tile: 16-byte chunk c of row r sits at chunk c ^ (r & 7).  The S^T A-operand
// read (8 lanes = 8 consecutive rows, same chunk) then touches 8 distinct
// 16-byte bank groups.
__device__ __forceinline__ int kswz(int row) { return row & 7; }
// V tile: the transposing read takes 4 consecutive rows x 32 bytes per 16
// lanes; an even XOR keeps each 32-byte pair together and spreads the 4 rows
// over distinct banks (row = 128 B for d=64, 256 B for d=128).
template <int D>
__device__ __forceinline__ int vswz(int row) { return D == 64 ? (row & 6) : ((row & 3) << 1); }

// Value of x from the other half-wave (lane ^ 32) combined with x.  The
// permlane32 swap exchanges the two half-waves between its two results, so one
// of the pair is x and the other the partner's value in every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;  // round to nearest even (v_cvt_pk_bf16_f32)
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, int QB, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(FwdParams p) {
  using T = Tile<D>;
  constexpr int QW = 32 * QB;             // query rows per wave
  constexpr int BM = kWaves * QW;         // query rows per workgroup
  __shared__ __attribute__((aligned(16))) char smem[2 * T::STAGE];

  const int N = p.N;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  // ---- workgroup -> (batch*head, query tile) --------------------------------
  // The dispatcher hands workgroup i to XCD i % 8.  Renumber so that XCD x gets
  // the contiguous logical range [x*per, (x+1)*per): neighbouring query tiles of
  // one head then share that XCD's L2 for their K/V reads.
  const int ntiles = (N + BM - 1) / BM;
  const int total = gridDim.x;
  const int bid = blockIdx.x;
  const int per = total >> 3;
  const int lid = (bid < (per << 3)) ? (bid & 7) * per + (bid >> 3) : bid;
  const int bh = lid / ntiles;
  int qt = lid - bh * ntiles;
  if (CAUSAL) qt = ntiles - 1 - qt;  // heaviest tiles first
  const int b = bh / p.H;

  const size_t hoff = (size_t)bh * (size_t)N * D;
  const __bf16* __restrict__ Qh = reinterpret_cast<const __bf16*>(p.q) + hoff;
  const __bf16* __restrict__ Kh = reinterpret_cast<const __bf16*>(p.k) + hoff;
  const __bf16* __restrict__ Vh = reinterpret_cast<const __bf16*>(p.v) + hoff;
  __bf16* __restrict__ Oh = reinterpret_cast<__bf16*>(p.o) + hoff;

  int kv_valid = N;
  if (p.seqlens) {
    const int L = p.seqlens[b];
    kv_valid = L < 0 ? 0 : (L > N ? N : L);
  }
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * QW;
  int kv_end = kv_valid;
  if (CAUSAL) kv_end = min(kv_end, q0 + BM);
  const int ntk = (kv_end + BN - 1) / BN;

  // ---- Q tile -> registers (B operand of S^T = K Q^T) -----------------------
  // B[k][j] for lane l: j = l % 32 (query), k = 8*(l/32) + e (head dim).
  bf16x8 qf[QB][T::DC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = min(qw0 + qb * 32 + r32, N - 1);
    const u32x4* row = reinterpret_cast<const u32x4*>(Qh + (size_t)qi * D);
#pragma unroll
    for (int s = 0; s < T::DC; ++s) qf[qb][s] = __builtin_bit_cast(bf16x8, row[2 * s + hi]);
  }

  // ---- per-lane LDS offsets ---------------------------------------------------
  // K read for k-step s: row r32 of a 32-key block, chunk 2s + hi.
  int koff[T::DC];
#pragma unroll
  for (int s = 0; s < T::DC; ++s) koff[s] = r32 * T::ROW + ((((2 * s + hi) ^ kswz(r32))) << 4);
  // V transposing read: within each 16-lane group, lane 4j+q supplies row k0+j,
  // columns c0+4q..c0+4q+3; the group returns V[k0..k0+3][c0+i] to lane i.
  // Here k0 = (block row) + 4*hi and c0 = 32*cb + 16*g.
  const int i16 = lane & 15;
  const int g16 = (lane >> 4) & 1;
  const int vrow = 4 * hi + (i16 >> 2);
  const int vsw = vswz<D>(vrow);
  int voff[T::DB];
#pragma unroll
  for (int cb = 0; cb < T::DB; ++cb) {
    const int chunk = cb * 4 + 2 * g16 + ((i16 & 3) >> 1);
    voff[cb] = vrow * T::ROW + ((chunk ^ vsw) << 4) + (i16 & 1) * 8;
  }

  // ---- K/V tile staging ---------------------------------------------------------
  u32x4 kst[T::NLD], vst[T::NLD];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < T::NLD; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / T::CH;
      const int c = idx % T::CH;
      const int key = min(t * BN + row, N - 1);  // rows past the end are read clamped and masked
      kst[i] = *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + c * 8);
      vst[i] = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + c * 8);
    }
  };
  auto sstore = [&](int stage) {
    char* base = smem + stage * T::STAGE;
#pragma unroll
    for (int i = 0; i < T::NLD; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / T::CH;
      const int c = idx % T::CH;
      *reinterpret_cast<u32x4*>(base + row * T::ROW + ((c ^ kswz(row)) << 4)) = kst[i];
      *reinterpret_cast<u32x4*>(base + T::MAT + row * T::ROW + ((c ^ vswz<D>(row)) << 4)) = vst[i];
    }
  };

  // ---- running state ------------------------------------------------------------
  f32x16 oacc[QB][T::DB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < T::DB; ++cb) oacc[qb][cb] = f32x16{};
  }
  const float sc = p.scale * kLog2e;  // scores enter exp2 as s * scale * log2(e)
  bf16x2 ones;
  ones[0] = (__bf16)1.0f;
  ones[1] = (__bf16)1.0f;

  if (ntk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int t = 0; t < ntk; ++t) {
    const int st = t & 1;
    if (t + 1 < ntk) gload(t + 1);
    const int k0 = t * BN;
    const bool active = !CAUSAL || (k0 <= qw0 + QW - 1);
    if (active) {
      const char* Ks = smem + st * T::STAGE;
      const char* Vs = Ks + T::MAT;

      // S^T = K Q^T: lane holds S[q = qw0 + 32qb + r32][k0 + 32kb + 8(r/4) + 4hi + r%4].
      f32x16 sacc[QB][KB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[qb][kb] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int s = 0; s < T::DC; ++s) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Ks + kb * 32 * T::ROW + koff[s]));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][s], sacc[qb][kb], 0, 0, 0);
        }
      }

      // Masks, only where the tile straddles the valid-key end or the diagonal.
      const bool need_mask = (k0 + BN > kv_valid) || (CAUSAL && k0 + BN - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qi = qw0 + qb * 32 + r32;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              const bool ok = key < kv_valid && (!CAUSAL || key <= qi);
              sacc[qb][kb][r] = ok ? sacc[qb][kb][r] : -INFINITY;
            }
        }
      }

      // Online softmax.  pk holds P^T as packed bf16 pairs (accumulator registers
      // 2j and 2j+1), ready to be the B operand of O^T += V^T P^T.
      uint32_t pk[QB][KB][8];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
        mx = pair_max(mx);
        const float tmax = mx * sc;
        const bool need = tmax > m_run[qb] + kTau;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
          const float m_new = need ? tmax : m_run[qb];
          const float alpha = (m_new == m_run[qb]) ? 1.0f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
          l_run[qb] *= alpha;
#pragma unroll
          for (int cb = 0; cb < T::DB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][cb][r] *= alpha;
          m_run[qb] = m_new;
        }
        const float mref = (m_run[qb] == -INFINITY) ? 0.0f : m_run[qb];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][2 * j], sc, -mref));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][2 * j + 1], sc, -mref));
            const uint32_t pp = pack_bf16(p0, p1);
            l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), ones, l_run[qb], false);
            pk[qb][kb][j] = pp;
          }
      }

      // O^T += V^T P^T.  MFMA (kb, u) takes accumulator registers 8u..8u+7 of
      // block kb, i.e. keys 32kb + 16u + {0..3, 8..11} + 4hi; the A operand
      // supplies the same keys as two transposing reads of 4 rows each.
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          char* vb = const_cast<char*>(Vs) + (kb * 32 + 16 * u) * T::ROW;
#pragma unroll
          for (int cb = 0; cb < T::DB; ++cb) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + voff[cb]));
            const s16x4 hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * T::ROW + voff[cb]));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 hi2 = __builtin_bit_cast(u32x2, hv);
            const u32x4 a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
            const bf16x8 a = __builtin_bit_cast(bf16x8, a4);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              const u32x4 b4 = {pk[qb][kb][4 * u], pk[qb][kb][4 * u + 1], pk[qb][kb][4 * u + 2], pk[qb][kb][4 * u + 3]};
              oacc[qb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, b4), oacc[qb][cb], 0, 0, 0);
            }
          }
        }
      }
    }
    if (t + 1 < ntk) sstore(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) ---------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = pair_sum(l_run[qb]);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int qi = qw0 + qb * 32 + r32;
    if (qi < N) {
      __bf16* orow = Oh + (size_t)qi * D;
#pragma unroll
      for (int cb = 0; cb < T::DB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = cb * 32 + 8 * g + 4 * hi;
          const u32x2 w = {pack_bf16(oacc[qb][cb][4 * g] * inv, oacc[qb][cb][4 * g + 1] * inv),
                           pack_bf16(oacc[qb][cb][4 * g + 2] * inv, oacc[qb][cb][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + col) = w;
        }
      if (p.lse && hi == 0) {
        p.lse[(size_t)bh * N + qi] = l > 0.0f ? (m_run[qb] + log2f(l)) * kLn2 : -INFINITY;
      }
    }
  }
}

template <int D, int QB, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  constexpr int BM = kWaves * 32 * QB;
  const int ntiles = (p.N + BM - 1) / BM;
  const dim3 grid((unsigned)ntiles * (unsigned)p.H * (unsigned)p.B);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, QB, CAUSAL>), grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, 2, true>(p, stream) : launch<64, 2, false>(p, stream);
  return p.causal ? launch<128, 2, true>(p, stream) : launch<128, 2, false>(p, stream);
}

}  // namespace fa
