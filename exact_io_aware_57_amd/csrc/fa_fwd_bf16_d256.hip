// Fused exact attention forward pass for head size 256, bf16 in / bf16 out,
// for gfx950.
//
// Same computation and method as the head sizes 64 and 128 (FlashAttention
// (UR), sections "Tiling and block-based processing", "Online computation of
// softmax" and "Fusing the operations into one CUDA kernel"; head size 256 is
// among the cases FlashAttention (UR), section "FlashAttention-2 (2023)", lists
// as supported).  What changes at d = 256 is the register budget: the Q
// fragments of one wave's 32 query rows take 64 registers and its transposed
// output accumulator O^T (256 x 32 fp32) 128, so two waves per SIMD (256
// registers each) cannot hold them with the score tile and the operand
// buffers at 64-key tiles.  This kernel therefore runs one wave per SIMD (4
// waves per compute unit) and uses that wave's whole 512-entry register file:
// it is compiled without the option that keeps MFMA accumulators in ordinary
// VGPRs, so S^T and O^T live in the accumulation registers.  It serves grids
// too small for the 8-wave ping-pong kernel, which takes head size 256 with
// 32-key tiles on larger grids (two waves per SIMD hide each other's tile
// loads and softmax).
//
//  * Workgroup: 4 waves x 32 query rows of one (batch, head); K/V tiles of 64
//    keys (32 KB each at d = 256), double-buffered in LDS (128 KB) and filled by
//    direct global->LDS loads issued one tile ahead.
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with the
//    operand layouts of the other head sizes (K rows and transposing reads of
//    the row-major V tile from swizzled LDS); the LDS operand reads are issued
//    a fixed number of products ahead of their use, so that they are in flight
//    under the matrix work without holding a whole tile's operands in
//    registers.
//  * Softmax per score: one FMA, one v_exp_f32 (base 2), half a pack to bf16,
//    half a v_dot2 for the row sum of the rounded P (the normaliser of O) and
//    one float32 add for the row sum of the unrounded P (the LSE output); the
//    reference max of a
//    row moves only when a tile's max exceeds it by more than 2^8 in the
//    exponent.  Masks only on tiles that straddle the causal diagonal or the
//    last valid key; tiles above a wave's diagonal are skipped.
//  * XCD-aware renumbering of workgroups and heaviest-first causal order, as
//    for the other head sizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kD = 256;
constexpr int kBN = 64;
constexpr int kAhead = 4;   // LDS operand reads in flight ahead of their product

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_d256_kernel(FwdParams p) {
  using T = Tile<kD, kBN>;
  constexpr int D = kD, BN = kBN;
  constexpr int KB = T::KB;          // 2 key blocks of 32
  constexpr int DC = T::DC;          // 16 k-steps of S^T
  constexpr int DB = T::DB;          // 8 row blocks of O^T
  constexpr int NQK = KB * DC;       // 32 products for S^T
  constexpr int NPV = KB * 2 * DB;   // 32 products for O^T
  constexpr int QW = 32;
  constexpr int BM = kWaves * QW;
  __shared__ __attribute__((aligned(1024))) char stage0[T::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[T::STAGE];

  const int N = p.N;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  // workgroup -> (batch*head, query tile): XCD x gets a contiguous logical range
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
  const __bf16* __restrict__ Qh = reinterpret_cast<const __bf16*>(p.q) + hoff;
  const __bf16* __restrict__ Kh = reinterpret_cast<const __bf16*>(p.k) + kvoff;
  const __bf16* __restrict__ Vh = reinterpret_cast<const __bf16*>(p.v) + kvoff;
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

  // Q fragments (B operand of S^T = K Q^T): lane l holds query qw0 + l % 32,
  // head-dim elements 16 s + 8 (l / 32) + 0..7 of k-step s.
  bf16x8 qf[DC];
  {
    const int qi = min(qw0 + r32, N - 1);
    const u32x4* row = reinterpret_cast<const u32x4*>(Qh + (size_t)qi * D);
#pragma unroll
    for (int s = 0; s < DC; ++s) qf[s] = __builtin_bit_cast(bf16x8, row[2 * s + hi]);
  }

  // K operand of k-step s, key block kb: row 32 kb + r32, global chunk 2 s + hi,
  // stored at chunk (2 s + hi) ^ kswz(row); XOR with 32 s moves between k-steps.
  const int kx = kswz<D>(r32);
  const int kbase = r32 * T::ROW + ((((kx >> 1) << 1) | (hi ^ (kx & 1))) << 4);
  // V^T operand (transposing read) of row block cb: XOR with 64 cb.
  const int i16 = lane & 15;
  const int g16 = (lane >> 4) & 1;
  const int vrow = 4 * hi + (i16 >> 2);
  const int vbase = vrow * T::ROW + (((2 * g16 + ((i16 & 3) >> 1)) ^ vswz<D>(vrow)) << 4) + (i16 & 1) * 8;

  // Tile loads: wave-load i of this wave fills LDS rows 16 wave + 2 i + hi
  // (chunk r32 of each), i.e. global chunk r32 ^ swz(row) of that key.
  // The lane index is passed through an empty asm so that the 16 per-lane
  // addresses are recomputed at each use instead of being held in registers
  // across the loop (the same for the LDS read offsets below).
  auto issue_loads = [&](int t, char* base) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lr = ln & 31, lh = ln >> 5;
#pragma unroll
    for (int i = 0; i < T::NLD; ++i) {
      const int row = 16 * wave + 2 * i + lh;
      const int key = min(t * BN + row, N - 1);  // rows past the end are read clamped and masked
      char* dst = base + (wave * T::NLD + i) * 1024;
      load_to_lds16(Kh + (size_t)key * D + ((lr ^ kswz<D>(row)) << 3), dst);
      load_to_lds16(Vh + (size_t)key * D + ((lr ^ vswz<D>(row)) << 3), dst + T::MAT);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) oacc[cb] = f32x16{};
  // l_run sums the bf16-rounded P (the normaliser of O), le_run the float32 P
  // before rounding (the LSE output).
  float m_run = -INFINITY, l_run = 0.0f, le_run = 0.0f;
  const float sc = p.scale * kLog2e;
  bf16x2 ones;
  ones[0] = (__bf16)1.0f;
  ones[1] = (__bf16)1.0f;

  auto tile = [&](const bool MASK, const char* Ks, int k0) __attribute__((always_inline)) {
    const char* Vs = Ks + T::MAT;
    int kb0 = kbase, vb0 = vbase;
    asm volatile("" : "+v"(kb0), "+v"(vb0));
    // ---- S^T = K Q^T: product i is k-step i / KB of key block i % KB ----
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
    auto read_k = [&](int i) __attribute__((always_inline)) {
      const int s = i / KB, kb = i % KB;
      return *reinterpret_cast<const u32x4*>(Ks + kb * 32 * T::ROW + (kb0 ^ (s << 5)));
    };
    u32x4 kf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kf[i] = read_k(i);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int s = i / KB, kb = i % KB;
      const u32x4 a = kf[i % kAhead];
      if (i + kAhead < NQK) kf[i % kAhead] = read_k(i + kAhead);
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[s], sacc[kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- mask, online softmax (lazy rescale), P^T as packed bf16 ----
    if (MASK) {
      const int qi = qw0 + r32;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = key < kv_valid && (!CAUSAL || key <= qi);
          sacc[kb][r] = ok ? sacc[kb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = pair_max(mx);
    const float tmax = mx * sc;
    const bool need = tmax > m_run + kTau;
    float alpha = 1.0f;
    bool rescale = false;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? tmax : m_run;
      alpha = (m_new == m_run) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      le_run *= alpha;
      m_run = m_new;
      rescale = true;
    }
    const float mref = (MASK && m_run == -INFINITY) ? 0.0f : m_run;
    uint32_t pk[KB][8];
    float te0 = 0.0f, te1 = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][2 * j], sc, -mref));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][2 * j + 1], sc, -mref));
        const uint32_t pp = pack_bf16(p0, p1);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), ones, l_run, false);
        te0 += p0;
        te1 += p1;
        pk[kb][j] = pp;
      }
    le_run += te0 + te1;

    // ---- O^T = alpha O^T + V^T P^T: product i is row block i % DB, half u of
    // key block kb (keys 32 kb + 16 u + {0..3, 8..11} + 4 hi) ----
    auto pv = [&]() __attribute__((always_inline)) {
      auto read_v = [&](int i, s16x4& lo, s16x4& hv) __attribute__((always_inline)) {
        const int kb = i / (2 * DB), u = (i / DB) & 1, cb = i % DB;
        char* vb = const_cast<char*>(Vs) + (kb * 32 + 16 * u) * T::ROW + (vb0 ^ (cb << 6));
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
        hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * T::ROW));
      };
      s16x4 vlo[kAhead], vhi[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) read_v(i, vlo[i], vhi[i]);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const int kb = i / (2 * DB), u = (i / DB) & 1, cb = i % DB;
        const u32x2 lo2 = __builtin_bit_cast(u32x2, vlo[i % kAhead]);
        const u32x2 hi2 = __builtin_bit_cast(u32x2, vhi[i % kAhead]);
        const u32x4 a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
        if (i + kAhead < NPV) read_v(i + kAhead, vlo[i % kAhead], vhi[i % kAhead]);
        const u32x4 b4 = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4),
                                                           oacc[cb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (rescale) {
      keep_branch();
      // one 16-register block at a time through the VALU (a barrier per block
      // keeps the scheduler from moving all of O^T into VGPRs at once)
#pragma unroll
      for (int cb = 0; cb < DB; ++cb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
      pv();
    } else {
      pv();
    }
  };

  auto step = [&](int t, const char* cur, char* next) __attribute__((always_inline)) {
    if (t + 1 < ntk) issue_loads(t + 1, next);
    const int k0 = t * BN;
    const bool active = !CAUSAL || (k0 <= qw0 + QW - 1);
    if (active) {
      const bool need_mask = (k0 + BN > kv_valid) || (CAUSAL && k0 + BN - 1 > qw0);
      if (need_mask)
        tile(true, cur, k0);
      else
        tile(false, cur, k0);
    }
    wait_vmem();
    __syncthreads();
  };

  if (ntk > 0) issue_loads(0, stage0);
  wait_vmem();
  __syncthreads();
  for (int t = 0; t < ntk; t += 2) {
    step(t, stage0, stage1);
    if (t + 1 < ntk) step(t + 1, stage1, stage0);
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 (m + log2 l) ----
  const float l = pair_sum(l_run);
  const float le = pair_sum(le_run);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const int qi = qw0 + r32;
  if (qi < N) {
    __bf16* orow = Oh + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = cb * 32 + 8 * g + 4 * hi;
        const u32x2 w = {pack_bf16(oacc[cb][4 * g] * inv, oacc[cb][4 * g + 1] * inv),
                         pack_bf16(oacc[cb][4 * g + 2] * inv, oacc[cb][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + col) = w;
        __builtin_amdgcn_sched_barrier(0);
      }
    if (p.lse && hi == 0) p.lse[(size_t)bh * N + qi] = le > 0.0f ? (m_run + log2f(le)) * kLn2 : -INFINITY;
  }
}

template <bool CAUSAL>
hipError_t launch_d256(const FwdParams& p, hipStream_t stream) {
  constexpr int BM = kWaves * 32;
  const int ntiles = (p.N + BM - 1) / BM;
  const dim3 grid((unsigned)ntiles * (unsigned)p.H * (unsigned)p.B);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_d256_kernel<CAUSAL>), grid, dim3(kThreads), args, 0,
                         stream);
}

}  // namespace

hipError_t launch_fwd_bf16_d256(const FwdParams& p, hipStream_t stream) {
  return p.causal ? launch_d256<true>(p, stream) : launch_d256<false>(p, stream);
}

}  // namespace fa
