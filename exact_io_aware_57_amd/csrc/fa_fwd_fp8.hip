// Fused exact attention forward pass over FP8 (e4m3) inputs with per-tensor
// scales, bf16 output, for gfx950.
//
// FlashAttention (UR), section "FlashAttention-3 (2024)", names FP8 support as
// the next precision step of the method, without a scheme.  Here Q, K and V are
// e4m3 codes with one float scale each (the tensors are descale * value), the
// method is unchanged (tiles of K/V streamed through LDS, online softmax, sections
// "Tiling and block-based processing" and "Online computation of softmax"), and
// both products run on the 8-bit matrix instruction v_mfma_f32_32x32x64_f8f6f4,
// which does four times the work of the bf16 32x32x16 product per instruction
// at twice its rate:
//  * S^T = K Q^T: K rows from LDS and this lane's query row from registers,
//    64 head-dimension elements per product (lane half h holds elements
//    64 s + 32 h .. +31 of k-step s on both sides).
//  * P: each row keeps a reference max that moves (and rescales the
//    accumulator) only when a tile's max exceeds it by more than 0.75 in the
//    base-2 exponent, so 0 <= P <= 2^0.75; P * 2^8 (the factor folded into the
//    exponent) is then at most 431, below the largest e4m3 value (448), and is
//    rounded to e4m3 (round to nearest even; values down to 2^-14 keep 3
//    significant bits); the 2^-8 comes out in the final division and the LSE.
//    The reference key has P = 1, so the row sum l >= 1 in these units.  The
//    row sum adds the float32 P * 2^8.
//  * O^T += V^T P^T: the 64 keys of a tile are one product per 32 output
//    columns.  Lane half h of P^T holds keys 32 kb + 8 g + 4 h + e (the keys
//    its score registers hold), so V^T must supply the same keys: four
//    transposing 8-bit LDS reads (ds_read_b64_tr_b8, 8 keys of one column per
//    lane each) with per-lane row addresses that pick exactly those keys.
//  * O = sv * O^T / l rounded to bf16; LSE = ln2 (m - 8 + log2 l).
// The workgroup is 4 waves x 32 query rows, K/V tiles of 64 keys double-
// buffered in LDS by direct global->LDS loads, two workgroups per compute unit.
// On small grids (at most 256 such workgroups, 1024 keys or more) a workgroup
// has two groups of 4 waves on the same rows, each streaming half of the key
// tiles, merged at the end by the rule for split results.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// Lazy-rescale threshold of the FP8 kernel in base-2 exponent units: P stays at
// most 2^0.75, so P * 2^8 <= 430.5 stays below the largest e4m3 value (448)
// with room for rounding of the exponent's argument.
constexpr float kFp8Tau = 0.75f;

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int D>
struct Tile8 {
  static constexpr int BN = 64;                      // keys per tile
  static constexpr int ROW = D;                      // bytes per row
  static constexpr int CH = D / 16;                  // 16-byte chunks per row
  static constexpr int MAT = BN * ROW;               // one K or V tile
  static constexpr int NLD = MAT / (1024 * kWaves);  // 1 KB wave-loads per wave per matrix
  static constexpr int KS = D / 64;                  // k-steps of S^T
  static constexpr int DB = D / 32;                  // 32-column blocks of O^T
  static_assert(MAT % (1024 * kWaves) == 0, "tile load must split evenly over the waves");
};

// K (read as rows: 16 lanes, 16 consecutive rows, one 16-byte chunk): the XOR
// puts the rows that share a 256-byte bank line in distinct chunks.
template <int D>
__device__ __forceinline__ int kswz8(int r) { return D == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
// V (read transposed only: 32 lanes, rows {0..3, 8..11} + 4h of a 16-row group,
// two adjacent chunks): the XOR sends rows that share bank lines to distinct
// chunk pairs.
template <int D>
__device__ __forceinline__ int vswz8(int r) {
  return D == 64 ? (((r >> 3) & 1) << 1) : ((((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2));
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // neutral block scales (2^0): the plain 8-bit product
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// KS key groups of 4 waves share the workgroup's 128 query rows: group g
// streams the g-th contiguous share of the key tiles through its own LDS
// stages, and group 1 hands its reference max, row sum and O^T to group 0 at
// the end, which combines them as a merge of split results.  Two groups keep
// 8 waves per compute unit busy on grids too small for two 4-wave workgroups
// per compute unit.
template <int D, bool CAUSAL, int KS>
__global__ __launch_bounds__(kThreads * KS, KS == 1 ? 2 : 1) void fwd_fp8_kernel(FwdParams p) {
  static_assert(KS == 1 || KS == 2, "one or two key groups");
  using T = Tile8<D>;
  constexpr int BN = T::BN;
  constexpr int QW = 32;
  constexpr int BM = kWaves * QW;
  __shared__ __attribute__((aligned(1024))) char stage0[KS][2 * T::MAT];
  __shared__ __attribute__((aligned(1024))) char stage1[KS][2 * T::MAT];
  // the merge passes one float per accumulator register of a 32-column block
  // of O^T (16 per lane, 256 lanes) through stage0
  static_assert(KS == 1 || 16 * 256 * 4 <= KS * 2 * T::MAT, "the key-group exchange fits stage0");

  const int N = p.N;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(KS == 1 ? tid >> 6 : (tid >> 6) & 3);
  const int kgrp = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  const int ntiles = (N + BM - 1) / BM;
  const int total = gridDim.x;
  const int bid = blockIdx.x;
  const int per = total >> 3;
  const int lid = (bid < (per << 3)) ? (bid & 7) * per + (bid >> 3) : bid;
  const int bh = lid / ntiles;
  int qt = lid - bh * ntiles;
  if (CAUSAL) qt = ntiles - 1 - qt;
  const int b = bh / p.H;

  const size_t hoff = (size_t)bh * (size_t)N * D;
  const size_t kvoff = ((size_t)b * p.Hkv + (bh - b * p.H) / (p.H / p.Hkv)) * (size_t)N * D;
  const uint8_t* __restrict__ Qh = reinterpret_cast<const uint8_t*>(p.q) + hoff;
  const uint8_t* __restrict__ Kh = reinterpret_cast<const uint8_t*>(p.k) + kvoff;
  const uint8_t* __restrict__ Vh = reinterpret_cast<const uint8_t*>(p.v) + kvoff;
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

  // Q row of this lane's query: k-step s, lane half h -> bytes 64 s + 32 h .. +31
  i32x8 qf[T::KS];
  {
    const int qi = min(qw0 + r32, N - 1);
    const u32x4* row = reinterpret_cast<const u32x4*>(Qh + (size_t)qi * D);
#pragma unroll
    for (int s = 0; s < T::KS; ++s) {
      const u32x4 a = row[4 * s + 2 * hi], c = row[4 * s + 2 * hi + 1];
      qf[s] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    }
  }

  // K operand of key block kb, k-step s: row 32 kb + r32, chunks 4 s + 2 h and
  // 4 s + 2 h + 1 (swizzled, adjacent after the XOR).
  const int kx = kswz8<D>(r32);
  const int kbase = r32 * T::ROW + (((2 * hi) ^ kx) << 4);
  // V^T operand of column block cb, read t4: this lane supplies row
  // 16 t4 + 8 (i / 8) + 4 h + (i / 2) % 4 (i = lane % 16), 8 bytes of chunk
  // 2 cb + g16 (g16 = lane / 16 % 2), and receives column 32 cb + lane % 32 of
  // the 8 rows its group supplies: keys 16 t4 + {0..3, 8..11} + 4 h.
  const int i16 = lane & 15;
  const int g16 = (lane >> 4) & 1;
  const int vrow = 8 * (i16 >> 3) + 4 * hi + ((i16 >> 1) & 3);
  const int vbase = vrow * T::ROW + ((g16 ^ vswz8<D>(vrow)) << 4) + 8 * (i16 & 1);

  int ld_row[T::NLD], ld_kc[T::NLD], ld_vc[T::NLD];
#pragma unroll
  for (int i = 0; i < T::NLD; ++i) {
    const int pos = (wave * T::NLD + i) * 64 + lane;
    const int row = pos / T::CH;
    const int cst = pos % T::CH;
    ld_row[i] = row;
    ld_kc[i] = (cst ^ kswz8<D>(row)) * 16;
    ld_vc[i] = (cst ^ vswz8<D>(row)) * 16;
  }
  auto issue_loads = [&](int t, char* base) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::NLD; ++i) {
      const int key = min(t * BN + ld_row[i], N - 1);  // rows past the end are read clamped and masked
      char* dst = base + (wave * T::NLD + i) * 1024;
      load_to_lds16(Kh + (size_t)key * D + ld_kc[i], dst);
      load_to_lds16(Vh + (size_t)key * D + ld_vc[i], dst + T::MAT);
    }
  };

  f32x16 oacc[T::DB];
#pragma unroll
  for (int cb = 0; cb < T::DB; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sc = p.scale * p.descale_q * p.descale_k * kLog2e;

  // One tile body for masked and unmasked tiles: the mask overwrites the score
  // tile in place under a runtime branch, and the rare rescale multiplies O^T
  // before the one copy of the second product.  Separate inlined bodies for
  // the two cases (or for the two rescale outcomes) leave O^T in different
  // registers on each path, and the compiler then copies all of it (32
  // v_mov_b64) at the join on every tile: 1.43 -> 1.26 ms on the long-context
  // shape, results bitwise unchanged.
  auto tile = [&](const char* Ks, int k0) __attribute__((always_inline)) {
    const char* Vs = Ks + T::MAT;
    // per-tile copies of the lane's LDS offsets (an empty asm keeps the
    // compiler from holding every derived address across the loop)
    int kb0 = kbase, vb0 = vbase;
    asm volatile("" : "+v"(kb0), "+v"(vb0));
    // ---- S^T: lane holds S[q = qw0 + r32][k0 + 32 kb + 8 (r / 4) + 4 h + r % 4]
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < T::KS; ++s) {
        const int off = kb * 32 * T::ROW + (kb0 ^ (s << 6));
        const u32x4 x = *reinterpret_cast<const u32x4*>(Ks + off);
        const u32x4 y = *reinterpret_cast<const u32x4*>(Ks + (off ^ 16));
        const i32x8 a = {(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        sacc[kb] = mfma_fp8(a, qf[s], sacc[kb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if ((k0 + BN > kv_valid) || (CAUSAL && k0 + BN - 1 > qw0)) {
      const int qi = qw0 + r32;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = key < kv_valid && (!CAUSAL || key <= qi);
          sacc[kb][r] = ok ? sacc[kb][r] : -INFINITY;
        }
    }
    // ---- reference max: moved (with a rescale) only when a row's tile max
    // exceeds it by more than kFp8Tau; every P is then at most 2^kFp8Tau.  An
    // exact running max rescales on most early tiles (any of the wave's 32 rows
    // growing); the threshold removes those multiplies (long context 1.28 ->
    // 1.20 ms).
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = pair_max(mx) * sc;
    const bool grow = mx > m_run + kFp8Tau;
    float alpha = 1.0f;
    bool rescale = false;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      alpha = (m_new == m_run) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);   // exp2(-inf) = 0
      l_run *= alpha;
      m_run = m_new;
      rescale = true;
    }
    const float mref = m_run == -INFINITY ? 0.0f : m_run;
    // exponentials of P * 2^8 directly (the 2^8 folded into the FMA's offset):
    // the e4m3 operand needs no multiply, and l sums P * 2^8
    const float mref8 = 8.0f - mref;
    // ---- P (float32, <= 2^kFp8Tau), row sum, and P * 2^8 as e4m3 in the slot order of
    // the second product: dword w holds registers 4 (w % 4) .. +3 of block w / 4
    float part[2][4];
    i32x8 pb;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][4 * g + e], sc, mref8));
        part[kb][g] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], w, true);
        pb[4 * kb + g] = w;
      }
    const float tsum = ((part[0][0] + part[0][1]) + (part[0][2] + part[0][3])) +
                       ((part[1][0] + part[1][1]) + (part[1][2] + part[1][3]));
    l_run += tsum;
    __builtin_amdgcn_sched_barrier(0);
    // ---- O^T = alpha O^T + V^T P^T, one product per 32 output columns
    auto pv = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int cb = 0; cb < T::DB; ++cb) {
        i32x8 a;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_i32x2*)(const_cast<char*>(Vs) + t4 * 16 * T::ROW + (vb0 ^ (cb << 5))));
          a[2 * t4] = v[0];
          a[2 * t4 + 1] = v[1];
        }
        oacc[cb] = mfma_fp8(a, pb, oacc[cb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (rescale) {
      keep_branch();
#pragma unroll
      for (int cb = 0; cb < T::DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
    }
    pv();
  };

  if constexpr (KS == 1) {
    // one group: the loop as written before the key split (the generic form
    // below compiles to a different schedule that measured about 1% slower)
    auto step1 = [&](int t, const char* cur, char* next) __attribute__((always_inline)) {
      if (t + 1 < ntk) issue_loads(t + 1, next);
      const int k0 = t * BN;
      const bool active = !CAUSAL || (k0 <= qw0 + QW - 1);
      if (active) {
        tile(cur, k0);
      }
      wait_vmem();
      __syncthreads();
    };
    if (ntk > 0) issue_loads(0, stage0[0]);
    wait_vmem();
    __syncthreads();
    for (int t = 0; t < ntk; t += 2) {
      step1(t, stage0[0], stage1[0]);
      if (t + 1 < ntk) step1(t + 1, stage1[0], stage0[0]);
    }
  } else {
  // Group g takes tiles [t_begin, t_end); both groups run the same number of
  // steps, so every workgroup barrier is reached by all 8 waves.
  const int nsteps = (ntk + KS - 1) / KS;
  const int t_begin = kgrp * nsteps;
  const int t_end = min(ntk, t_begin + nsteps);
  char* const st0 = stage0[kgrp];
  char* const st1 = stage1[kgrp];
  auto step = [&](int s, const char* cur, char* next) __attribute__((always_inline)) {
    const int t = t_begin + s;
    if (t + 1 < t_end) issue_loads(t + 1, next);
    const int k0 = t * BN;
    const bool active = t < t_end && (!CAUSAL || (k0 <= qw0 + QW - 1));
    if (active) {
      tile(cur, k0);
    }
    wait_vmem();
    __syncthreads();
  };

  if (t_begin < t_end) issue_loads(t_begin, st0);
  wait_vmem();
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    step(s, st0, st1);
    if (s + 1 < nsteps) step(s + 1, st1, st0);
  }
  }

  if constexpr (KS == 2) {
    // The stage buffers are free after the loop's last barrier.  Both groups
    // hold the same rows in the same lane layout, so the exchange is lane for
    // lane; both reference maxima carry the same 2^8 factor in P.
    float* xch = reinterpret_cast<float*>(&stage0[0][0]);
    const int slot = wave * 64 + lane;
    if (kgrp == 1) {
      xch[slot] = m_run;
      xch[256 + slot] = l_run;
    }
    __syncthreads();
    float wa = 0.0f, wb = 0.0f;
    if (kgrp == 0) {
      const float mb = xch[slot];
      const float lb = xch[256 + slot];
      const float m = fmaxf(m_run, mb);
      wa = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
      wb = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mb - m);
      l_run = l_run * wa + lb * wb;
      m_run = m;
    }
#pragma unroll
    for (int cb = 0; cb < T::DB; ++cb) {
      __syncthreads();
      if (kgrp == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[r * 256 + slot] = oacc[cb][r];
      }
      __syncthreads();
      if (kgrp == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = oacc[cb][r] * wa + xch[r * 256 + slot] * wb;
      }
    }
    if (kgrp != 0) return;
  }

  // ---- epilogue: O = sv O^T / l, LSE = ln2 (m - 8 + log2 l) (both sums carry 2^8)
  const float l = pair_sum(l_run);
  const float inv = l > 0.0f ? p.descale_v / l : 0.0f;   // l and O^T both carry the factor 2^8
  const int qi = qw0 + r32;
  if (qi < N) {
    __bf16* orow = Oh + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < T::DB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = cb * 32 + 8 * g + 4 * hi;
        const u32x2 w = {pack_bf16(oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv),
                         pack_bf16(oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + col) = w;
      }
    if (p.lse && hi == 0) p.lse[(size_t)bh * N + qi] = l > 0.0f ? (m_run - 8.0f + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, int KS>
hipError_t launch8(const FwdParams& p, hipStream_t stream) {
  constexpr int BM = kWaves * 32;
  const int ntiles = (p.N + BM - 1) / BM;
  const dim3 grid((unsigned)ntiles * (unsigned)p.H * (unsigned)p.B);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_fp8_kernel<D, CAUSAL, KS>), grid, dim3(kThreads * KS), args,
                         0, stream);
}

template <int D>
hipError_t launch8_d(const FwdParams& p, hipStream_t stream) {
  // Grids of at most 256 workgroups of 128 rows (one per compute unit) split
  // each workgroup's keys over two groups of 4 waves, from 1024 keys.
  const long long groups = (long long)p.B * p.H * ((p.N + 127) / 128);
  if (groups <= 256 && p.N >= 1024) return p.causal ? launch8<D, true, 2>(p, stream) : launch8<D, false, 2>(p, stream);
  return p.causal ? launch8<D, true, 1>(p, stream) : launch8<D, false, 1>(p, stream);
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return launch8_d<64>(p, stream);
  return launch8_d<128>(p, stream);
}

}  // namespace fa
