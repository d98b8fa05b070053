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
//    crosses waves.  K/V tiles of BN keys are shared by the 4 waves through LDS,
//    double-buffered and filled by direct global->LDS loads
//    (global_load_lds_dwordx4): the loads of tile t+1 are in flight while tile t
//    is computed, and no VGPRs or LDS-write instructions are spent on staging.
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
//    v_exp_f32 (base 2), half a v_cvt_pk_bf16_f32 and the row sum: in the
//    8-wave kernel one float32 add (a tree per tile over the unrounded P; the
//    bf16-rounded P feeds the second product, so the weights sum to 1 within
//    the 2^-8 of that rounding), in the 4-wave kernel half a v_dot2 over the
//    rounded P, which normalises O, plus one float32 add over the unrounded P,
//    which gives the LSE.  v_dot2 runs on the matrix pipeline and slows
//    several-fold next to another wave's products, which the 8-wave kernel
//    always has.  The
//    reference max of a row changes rarely: the kernels do not even compute a
//    tile's max unless the tile's sum of P exceeds 2^8, which every P <= 2^8
//    rules out (P may reach 2^8 in between); the 4-wave kernel with 128-key
//    tiles at head size 64 instead computes each tile's max and moves the
//    reference when the max exceeds it by more than 2^8 in the exponent.  The
//    output is divided by the row sum once at the end.
//  * Masks are applied only on tiles that straddle a boundary (causal diagonal,
//    last valid key), by a branch that overwrites the score tile in place;
//    tiles wholly above a wave's causal diagonal are skipped.
//  * Workgroups are renumbered so that each XCD (each its own L2) receives a
//    contiguous run of (head, query tile) pairs, and causal query tiles are
//    issued heaviest first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D, int QB, int BN, int OCC, bool CAUSAL, int KS>
__global__ __launch_bounds__(kThreads * KS, OCC) void fwd_bf16_kernel(FwdParams p) {
  // KS key groups of 4 waves share the workgroup's query rows: group g streams
  // the g-th contiguous share of the key tiles through its own LDS stages, and
  // the groups' partial results (reference max, row sum, O^T) are combined at
  // the end, through LDS, by the same rule as a merge of split results.  With
  // KS = 2 the longest workgroups of a causal grid take half as many steps,
  // and a small grid keeps more waves per compute unit busy.
  static_assert(KS == 1 || KS == 2, "one or two key groups");
  using T = Tile<D, BN>;
  constexpr int KB = T::KB;
  constexpr int QW = 32 * QB;             // query rows per wave
  // Max-free softmax (below) on every instantiation but 128-key tiles at head
  // size 64, where computing the tile's max measured faster (BERT- and GPT-2-
  // shaped 0.0265 -> 0.0254 and 0.0341 -> 0.0327 ms; at 2048 keys with 128-key
  // tiles 2-4% slower).
  constexpr bool kMaxFree = !(D == 64 && BN == 128);
  constexpr int BM = kWaves * QW;         // query rows per workgroup
  // Two K/V stages (per key group) as separate LDS objects, so the compiler
  // can tell that the direct loads into one stage never alias the reads of the
  // other.
  __shared__ __attribute__((aligned(1024))) char stage0[KS][T::STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[KS][T::STAGE];
  // the merge of the key groups passes one float per accumulator register of a
  // 32-column block of O^T through stage0
  static_assert(KS == 1 || QB * 16 * 256 * 4 <= KS * T::STAGE, "the key-group exchange fits stage0");

  const int N = p.N;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // row wave within the key group
  const int kgrp = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);  // key group
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  // ---- workgroup -> (batch*head, query tile): XCD-contiguous ranges, causal
  // work balanced over the compute units (grid_tile) ----------------------------
  const int ntiles = (N + BM - 1) / BM;
  int bh, qt;
  if (CAUSAL || !p.seqlens || !grid_tile_lengths(blockIdx.x, gridDim.x, ntiles, p.B, p.H, N, BN, p.seqlens, p.num_cu, bh, qt))
    grid_tile(blockIdx.x, gridDim.x, ntiles, p.B * p.H, CAUSAL, p.num_cu, bh, qt);
  const int b = bh / p.H;

  const size_t hoff = (size_t)bh * (size_t)N * D;
  // key/value head of this query head: groups of H / Hkv consecutive heads
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
  // key tiles [t_begin, t_end) of this key group; every group runs nsteps steps
  const int ntk_all = (kv_end + BN - 1) / BN;
  const int nsteps = (ntk_all + KS - 1) / KS;
  const int t_begin = kgrp * nsteps;
  const int t_end = min(ntk_all, t_begin + nsteps);

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
  for (int s = 0; s < T::DC; ++s) koff[s] = r32 * T::ROW + ((((2 * s + hi) ^ kswz<D>(r32))) << 4);
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

  // ---- K/V tile loads: global -> LDS directly ------------------------------------
  // One global_load_lds_dwordx4 writes 64 consecutive 16-byte LDS chunks (lane i
  // to base + 16 i).  Lane i of wave-load j therefore fills LDS chunk
  // p = 64 j + i, i.e. row p / CH, stored chunk p % CH, and fetches the global
  // chunk that the swizzle puts there.
  int ld_row[T::NLD], ld_kc[T::NLD], ld_vc[T::NLD];
#pragma unroll
  for (int i = 0; i < T::NLD; ++i) {
    const int pos = (wave * T::NLD + i) * 64 + lane;
    const int row = pos / T::CH;
    const int cst = pos % T::CH;
    ld_row[i] = row;
    ld_kc[i] = (cst ^ kswz<D>(row)) * 8;
    ld_vc[i] = (cst ^ vswz<D>(row)) * 8;
  }
  auto issue_loads = [&](int t, char* base) {
#pragma unroll
    for (int i = 0; i < T::NLD; ++i) {
      const int key = min(t * BN + ld_row[i], N - 1);  // rows past the end are read clamped and masked
      char* dst = base + (wave * T::NLD + i) * 1024;
      load_to_lds16(Kh + (size_t)key * D + ld_kc[i], dst);
      load_to_lds16(Vh + (size_t)key * D + ld_vc[i], dst + T::MAT);
    }
  };

  // ---- running state ------------------------------------------------------------
  f32x16 oacc[QB][T::DB];
  // Two row sums: l_run over the bf16-rounded P that the second product uses
  // (the normaliser of O, so that the weights applied to V sum to one), and
  // le_run over the float32 P before rounding (the LSE output).
  float m_run[QB], l_run[QB], le_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
    le_run[qb] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < T::DB; ++cb) oacc[qb][cb] = f32x16{};
  }
  const float sc = p.scale * kLog2e;  // scores enter exp2 as s * scale * log2(e)
  bf16x2 ones;
  ones[0] = (__bf16)1.0f;
  ones[1] = (__bf16)1.0f;

  // One K/V tile: S^T = K Q^T, (mask), online softmax, O^T += V^T P^T.  One
  // body serves masked and unmasked tiles (the mask overwrites the score tile
  // in place under a runtime branch) and the rare rescale multiplies O^T before
  // the one copy of the second product: with separate inlined bodies per case
  // O^T sits in different registers on each path and the compiler copies all
  // of it at the join (16-32 v_mov_b64 per tile); results are bitwise the same.
  auto tile = [&](const char* Ks, int k0) __attribute__((always_inline)) {
    const char* Vs = Ks + T::MAT;

    // S^T: lane holds S[q = qw0 + 32qb + r32][k0 + 32kb + 8(r/4) + 4hi + r%4].
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

    uint32_t pk[QB][KB][8];   // P^T as packed bf16 pairs (accumulator registers 2j, 2j+1)
    float alpha[QB];
    bool rescale = false;     // wave-uniform: some row max moved by more than 2^kTau
    const bool mask = (k0 + BN > kv_valid) || (CAUSAL && k0 + BN - 1 > qw0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (mask) {
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
      alpha[qb] = 1.0f;
      if constexpr (kMaxFree) {
        // Exponentials against the current reference max without computing
        // the tile's max (as in the 8-wave kernel): every p is at most 2^kTau
        // whenever the tile's sum of p is; the max is computed, and the tile
        // redone against it, only when the sum is larger, not a number, or the
        // row has no reference yet.
        auto exps = [&](float mref, float& te) __attribute__((always_inline)) {
          float ts = 0.0f, te0 = 0.0f;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][2 * j], sc, -mref));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][2 * j + 1], sc, -mref));
              const uint32_t pp = pack_bf16(p0, p1);
              ts = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), ones, ts, false);
              te0 += p0 + p1;
              pk[qb][kb][j] = pp;
            }
          te = te0;
          return ts;
        };
        float le;
        float ls = exps(m_run[qb] == -INFINITY ? 0.0f : m_run[qb], le);
        // The redo below overwrites le; without this use the compiler sinks the
        // float32 sum past the branch and keeps every unrounded P live across
        // it (about 30 more registers: three instead of four waves per SIMD).
        pin(le);
        const bool bad = !(ls <= kMaxTileSum) || m_run[qb] == -INFINITY;
        if (__builtin_amdgcn_ballot_w64(bad) != 0) {
          keep_branch();
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
          mx = pair_max(mx);
          const float m_new = fmaxf(m_run[qb], mx * sc);
          alpha[qb] = (m_run[qb] == -INFINITY || m_new == m_run[qb]) ? 1.0f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
          l_run[qb] *= alpha[qb];
          le_run[qb] *= alpha[qb];
          m_run[qb] = m_new;
          rescale = true;
          ls = exps(m_run[qb] == -INFINITY ? 0.0f : m_run[qb], le);
        }
        l_run[qb] += ls;
        le_run[qb] += le;
        continue;
      }
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
        alpha[qb] = (m_new == m_run[qb]) ? 1.0f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        l_run[qb] *= alpha[qb];
        le_run[qb] *= alpha[qb];
        m_run[qb] = m_new;
        rescale = true;
      }
      const float mref = (mask && m_run[qb] == -INFINITY) ? 0.0f : m_run[qb];
      float te0 = 0.0f, te1 = 0.0f;
      // this kernel keeps the row sum on v_dot2 over the packed P (measured
      // faster here than float32 adds, unlike the 8-wave kernel)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][2 * j], sc, -mref));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][2 * j + 1], sc, -mref));
          const uint32_t pp = pack_bf16(p0, p1);
          l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), ones, l_run[qb], false);
          te0 += p0;
          te1 += p1;
          pk[qb][kb][j] = pp;
        }
      le_run[qb] += te0 + te1;
      pin(le_run[qb]);   // keeps the float32 sum ahead of the second product
    }

    // O^T = alpha O^T + V^T P^T.  MFMA (kb, u) takes accumulator registers
    // 8u..8u+7 of block kb, i.e. keys 32kb + 16u + {0..3, 8..11} + 4hi; the A
    // operand supplies the same keys as two transposing reads of 4 rows each.
    auto pv = [&]() __attribute__((always_inline)) {
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
    };
    if (rescale) {
      keep_branch();
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int cb = 0; cb < T::DB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][cb][r] *= alpha[qb];
    }
    pv();
  };

  // One step: start the loads of tile t+1 into `next`, compute tile t from
  // `cur`, then wait for this wave's loads and meet the other waves.
  char* const st0 = stage0[kgrp];
  char* const st1 = stage1[kgrp];
  auto step = [&](int s, const char* cur, char* next) __attribute__((always_inline)) {
    const int t = t_begin + s;
    if (t + 1 < t_end) issue_loads(t + 1, next);
    const int k0 = t * BN;
    const bool active = t < t_end && (!CAUSAL || (k0 <= qw0 + QW - 1));
    if (active) tile(cur, k0);
    wait_vmem();
    __syncthreads();
  };

  if (t_begin < t_end) issue_loads(t_begin, st0);
  wait_vmem();
  __syncthreads();
  // Unrolled by two so that each access names a fixed stage.
  for (int s = 0; s < nsteps; s += 2) {
    step(s, st0, st1);
    if (s + 1 < nsteps) step(s + 1, st1, st0);
  }

  if constexpr (KS == 2) {
    // Key group 1 hands its (reference max, row sum, O^T) to group 0 through
    // LDS, lane for lane (both groups hold the same rows in the same layout),
    // a 32-column block of O^T at a time; group 0 rescales both to the larger
    // reference and adds.  The stage buffers are free after the loop's last
    // barrier.
    float* xch = reinterpret_cast<float*>(&stage0[0][0]);
    const int slot = wave * 64 + lane;
    float wa[QB] = {}, wb[QB] = {};
    if (kgrp == 1) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        xch[(3 * qb) * 256 + slot] = m_run[qb];
        xch[(3 * qb + 1) * 256 + slot] = l_run[qb];
        xch[(3 * qb + 2) * 256 + slot] = le_run[qb];
      }
    }
    __syncthreads();
    if (kgrp == 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mb = xch[(3 * qb) * 256 + slot];
        const float lb = xch[(3 * qb + 1) * 256 + slot];
        const float leb = xch[(3 * qb + 2) * 256 + slot];
        const float m = fmaxf(m_run[qb], mb);
        wa[qb] = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[qb] - m);
        wb[qb] = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mb - m);
        l_run[qb] = l_run[qb] * wa[qb] + lb * wb[qb];
        le_run[qb] = le_run[qb] * wa[qb] + leb * wb[qb];
        m_run[qb] = m;
      }
    }
#pragma unroll
    for (int cb = 0; cb < T::DB; ++cb) {
      __syncthreads();
      if (kgrp == 1) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) xch[(qb * 16 + r) * 256 + slot] = oacc[qb][cb][r];
      }
      __syncthreads();
      if (kgrp == 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            oacc[qb][cb][r] = oacc[qb][cb][r] * wa[qb] + xch[(qb * 16 + r) * 256 + slot] * wb[qb];
      }
    }
    if (kgrp != 0) return;
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l) ---------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = pair_sum(l_run[qb]);
    const float le = pair_sum(le_run[qb]);
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
        p.lse[(size_t)bh * N + qi] = le > 0.0f ? (m_run[qb] + log2f(le)) * kLn2 : -INFINITY;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Ping-pong kernel: 8 waves in two groups of 4 (waves w and w+4 share a SIMD).
// Each wave owns 32 query rows and alternates an MFMA phase (O^T += V^T P^T for
// tile t-1, then S^T = K Q^T for tile t) with a softmax phase on the VALU.  The
// two groups run one phase apart, separated by workgroup barriers, so on every
// SIMD one wave keeps the matrix core busy while the other runs its softmax:
// VALU work of one wave executes alongside MFMA work of another, which it does
// not do within one wave.
// K and V have two LDS buffers each.  At every even phase 2t the workgroup
// issues the loads of K_{t+1} and V_t (direct global->LDS), and waits for them
// at the end of phase 2t+1, before any wave reads them.  At head size 128 and
// 256 that odd-phase barrier is the only one per tile.  The loads take the
// scalar-base form (head base in SGPRs, 32-bit lane offset): the group that is
// entering its softmax phase issues its loads while the other group's products
// have started, where the 64-bit-address form is slow to issue (long context
// 1.826 -> 1.809 ms, head size 256 1.884 -> 1.859 ms, results bitwise equal).
// Head size 256 runs this kernel with 32-key tiles: Q fragments (64 registers),
// O^T (128), the score tile (16) and P (8) then fit the 256 registers of a wave
// at two waves per SIMD, provided the matrix phase reads each LDS operand two
// products ahead of its use instead of a whole tile's operands up front, and
// the tile loads recompute their addresses instead of holding them.
// ---------------------------------------------------------------------------


template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_bf16_pp_kernel(FwdParams p) {
  using T = Tile<D, BN>;
  constexpr int KB = T::KB;
  constexpr int NW = 8;
  constexpr int BM = NW * 32;
  constexpr int NLD = T::MAT / (1024 * NW);   // 1 KB wave-loads per wave per matrix
  static_assert(T::MAT % (1024 * NW) == 0, "tile load must split evenly over 8 waves");
  __shared__ __attribute__((aligned(1024))) char kbuf[2][T::MAT];
  __shared__ __attribute__((aligned(1024))) char vbuf[2][T::MAT];

  const int N = p.N;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
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
  // key/value head of this query head: groups of H / Hkv consecutive heads
  const size_t kvoff = ((size_t)b * p.Hkv + (bh - b * p.H) / (p.H / p.Hkv)) * (size_t)N * D;
  const __bf16* __restrict__ Qh = reinterpret_cast<const __bf16*>(p.q) + hoff;
  const __bf16* __restrict__ Kh = uniform_ptr(reinterpret_cast<const __bf16*>(p.k) + kvoff);
  const __bf16* __restrict__ Vh = uniform_ptr(reinterpret_cast<const __bf16*>(p.v) + kvoff);
  __bf16* __restrict__ Oh = reinterpret_cast<__bf16*>(p.o) + hoff;

  int kv_valid = N;
  if (p.seqlens) {
    const int L = p.seqlens[b];
    kv_valid = L < 0 ? 0 : (L > N ? N : L);
  }
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;
  int kv_end = kv_valid;
  if (CAUSAL) kv_end = min(kv_end, q0 + BM);
  const int ntk = (kv_end + BN - 1) / BN;               // tiles the workgroup streams
  int last = ntk - 1;                                    // last tile this wave needs
  if (CAUSAL) last = min(last, (qw0 + 31) / BN);

  bf16x8 qf[T::DC];
  {
    const int qi = min(qw0 + r32, N - 1);
    const u32x4* row = reinterpret_cast<const u32x4*>(Qh + (size_t)qi * D);
#pragma unroll
    for (int s = 0; s < T::DC; ++s) qf[s] = __builtin_bit_cast(bf16x8, row[2 * s + hi]);
  }
  // Per-lane LDS base offsets.  The swizzled chunk index splits into bits that
  // depend on the lane only and bits that depend on the k-step (K) or the
  // column block (V), and the two never overlap the row offset, so every
  // operand address is one XOR of a lane base with a compile-time constant.
  //   K, k-step s: chunk (2s + hi) ^ kswz(r32) = ((s ^ (x >> 1)) << 1) | (hi ^ (x & 1))
  //   V, block cb: chunk (4cb + c4) ^ vswz(vrow), vswz a multiple of 2 below 8 (d=64)
  //                or of 4 below 16 (d=128)
  const int kx = kswz<D>(r32);
  const int kbase = r32 * T::ROW + (((kx >> 1) << 1 | (hi ^ (kx & 1))) << 4);   // k-step 0
  const int i16 = lane & 15;
  const int g16 = (lane >> 4) & 1;
  const int vrow = 4 * hi + (i16 >> 2);
  const int vbase = vrow * T::ROW + (((2 * g16 + ((i16 & 3) >> 1)) ^ vswz<D>(vrow)) << 4) + (i16 & 1) * 8;  // block 0
  auto koff = [&](int s_) { return kbase ^ (s_ << 5); };
  auto voff = [&](int cb) { return vbase ^ (cb << 6); };
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
  // At head size 256 the load addresses are recomputed at each tile from the
  // lane index (passed through an empty asm) instead of being held.
  auto ld_addr = [&](int i, int& row, int& kc, int& vc) __attribute__((always_inline)) {
    if constexpr (D >= 256) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int pos = (wave * NLD + i) * 64 + ln;
      row = pos / T::CH;
      const int cst = pos % T::CH;
      kc = (cst ^ kswz<D>(row)) * 8;
      vc = (cst ^ vswz<D>(row)) * 8;
    } else {
      row = ld_row[i];
      kc = ld_kc[i];
      vc = ld_vc[i];
    }
  };
  auto load_k = [&](int t) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      int row, kc, vc;
      ld_addr(i, row, kc, vc);
      const int key = min(t * BN + row, N - 1);
      dma16s(Kh, (uint32_t)(((size_t)key * D + kc) * 2), kbuf[t & 1] + (wave * NLD + i) * 1024);
    }
  };
  auto load_v = [&](int t) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      int row, kc, vc;
      ld_addr(i, row, kc, vc);
      const int key = min(t * BN + row, N - 1);
      dma16s(Vh, (uint32_t)(((size_t)key * D + vc) * 2), vbuf[t & 1] + (wave * NLD + i) * 1024);
    }
  };

  f32x16 oacc[T::DB];
#pragma unroll
  for (int cb = 0; cb < T::DB; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 sacc[KB];
  uint32_t pk[KB][8];
  const float sc = p.scale * kLog2e;

  // MFMA phase: O^T = alpha O^T + V_{tv}^T P^T (if DO_PV) and S^T = K_{tk} Q^T
  // (if DO_QK).  The K operands are requested up front (the scheduling fence
  // keeps the compiler from pulling them back next to their uses).  With both
  // products, S^T runs first and the V operand reads are interleaved with it;
  // a phase with one product only issues its products in order.
  constexpr int NPV = KB * 2 * T::DB;   // MFMAs of O^T += V^T P^T per tile
  constexpr int NQK = KB * T::DC;       // MFMAs of S^T = K Q^T per tile
  auto mfma_phase = [&](const bool DO_PV, int tv, const bool DO_QK, int tk) __attribute__((always_inline)) {
    // The wave in its matrix phase gets the higher issue priority of the two
    // waves sharing its SIMD, so the partner's softmax instructions do not
    // delay its products (measured: 1.915 -> 1.896 ms on the long context).
    __builtin_amdgcn_s_setprio(1);
    if constexpr (D >= 256) {
      // Head size 256: no room for a tile's operands at once; each operand is
      // read two products ahead of its use.
      const char* Ks2 = kbuf[tk & 1];
      const char* Vs2 = vbuf[tv & 1];
      int kb0 = kbase, vb0 = vbase;
      asm volatile("" : "+v"(kb0), "+v"(vb0));
      if (DO_QK) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
        auto read_k = [&](int i) __attribute__((always_inline)) {
          return *reinterpret_cast<const u32x4*>(Ks2 + (i % KB) * 32 * T::ROW + (kb0 ^ ((i / KB) << 5)));
        };
        u32x4 kr[2];
        kr[0] = read_k(0);
        kr[1] = read_k(1);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
          const u32x4 a = kr[i & 1];
          if (i + 2 < NQK) kr[i & 1] = read_k(i + 2);
          sacc[i % KB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[i / KB], sacc[i % KB], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (DO_PV) {
        auto read_v = [&](int i, s16x4& lo, s16x4& hv) __attribute__((always_inline)) {
          const int kb = i / (2 * T::DB), u = (i / T::DB) & 1, cb = i % T::DB;
          const char* vb = Vs2 + (kb * 32 + 16 * u) * T::ROW + (vb0 ^ (cb << 6));
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
          hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * T::ROW));
        };
        s16x4 vl[2], vh[2];
        read_v(0, vl[0], vh[0]);
        read_v(1, vl[1], vh[1]);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
          const int kb = i / (2 * T::DB), u = (i / T::DB) & 1, cb = i % T::DB;
          const u32x2 lo2 = __builtin_bit_cast(u32x2, vl[i & 1]);
          const u32x2 hi2 = __builtin_bit_cast(u32x2, vh[i & 1]);
          const u32x4 a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
          if (i + 2 < NPV) read_v(i + 2, vl[i & 1], vh[i & 1]);
          const u32x4 b4 = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4),
                                                             oacc[cb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) pin(sacc[kb]);
#pragma unroll
      for (int cb = 0; cb < T::DB; ++cb) pin(oacc[cb]);
      __builtin_amdgcn_s_setprio(0);
      return;
    }
    // Both products (the steady state): one stream of products, S^T product i
    // then O^T product i, each operand read from LDS a fixed number of
    // products ahead through a small register ring.  The first product's
    // operand is then the first read in flight, and at most about ten LDS
    // reads are outstanding (the LDS wait counter tracks fifteen): with all
    // K operands requested up front the compiler issued the first product's
    // operand eleventh, and the last products each waited on the counter
    // (long context 1.854 -> 1.826 ms, results bitwise equal).
    static_assert(NQK == NPV, "the product stream pairs one S^T and one O^T product");
    {
      if (DO_PV && DO_QK) {
        const char* Vr = vbuf[tv & 1];
        const char* Kr = kbuf[tk & 1];
        constexpr int RK = 4, RV = 4;   // ring depths: reads run RK - 1 (RV - 1) products ahead
        u32x4 kr[RK];
        s16x4 vr[RV][2];
        auto rdk = [&](int i) __attribute__((always_inline)) {
          const int s_ = i / KB, kb = i % KB;
          kr[i % RK] = *reinterpret_cast<const u32x4*>(Kr + kb * 32 * T::ROW + koff(s_));
        };
        auto rdv = [&](int i) __attribute__((always_inline)) {
          const int kb = i / (2 * T::DB), u = (i / T::DB) & 1, cb = i % T::DB;
          char* vb = const_cast<char*>(Vr) + (kb * 32 + 16 * u) * T::ROW + voff(cb);
          vr[i % RV][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
          vr[i % RV][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * T::ROW));
        };
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
        for (int i = 0; i < RK - 1; ++i) rdk(i);
#pragma unroll
        for (int i = 0; i < RV - 1; ++i) rdv(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
          if (i + RK - 1 < NQK) rdk(i + RK - 1);
          {
            const int s = i / KB, kb = i % KB;
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kr[i % RK]), qf[s], sacc[kb], 0, 0, 0);
          }
          if (i + RV - 1 < NPV) rdv(i + RV - 1);
          {
            const int kb = i / (2 * T::DB), u = (i / T::DB) & 1, cb = i % T::DB;
            const u32x4 b4 = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
            const u32x2 lo2 = __builtin_bit_cast(u32x2, vr[i % RV][0]);
            const u32x2 hi2 = __builtin_bit_cast(u32x2, vr[i % RV][1]);
            const u32x4 a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
            oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4),
                                                               oacc[cb], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) pin(sacc[kb]);
#pragma unroll
        for (int cb = 0; cb < T::DB; ++cb) pin(oacc[cb]);
        __builtin_amdgcn_s_setprio(0);
        return;
      }
    }
    // One product only (the first and last phases of a workgroup): K operands
    // are requested up front (they feed the longer S^T chain); the V operands
    // are read next to their products when the tile has more than one key
    // block, so the registers for all of them are not needed at once.
    constexpr bool V_UPFRONT = (KB == 1);
    s16x4 vfr[NPV][2];
    u32x4 kfr[NQK];
    const char* Vs = vbuf[tv & 1];
    const char* Ks = kbuf[tk & 1];
    auto read_v = [&](int i) __attribute__((always_inline)) {
      const int kb = i / (2 * T::DB), u = (i / T::DB) & 1, cb = i % T::DB;
      char* vb = const_cast<char*>(Vs) + (kb * 32 + 16 * u) * T::ROW + voff(cb);
      vfr[i][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vb);
      vfr[i][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + 8 * T::ROW));
    };
#pragma unroll
    for (int i = 0; i < (NPV > NQK ? NPV : NQK); ++i) {
      if (V_UPFRONT && DO_PV && i < NPV) read_v(i);
      if (DO_QK && i < NQK) {
        const int s_ = i / KB, kb = i % KB;   // key blocks interleaved: KB chains
        kfr[i] = *reinterpret_cast<const u32x4*>(Ks + kb * 32 * T::ROW + koff(s_));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    auto products = [&]() __attribute__((always_inline)) {
      if (DO_QK) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
      }
#pragma unroll
      for (int i = 0; i < (NPV > NQK ? NPV : NQK); ++i) {
        if (!V_UPFRONT && DO_PV && i < NPV) read_v(i);
        if (DO_PV && i < NPV) {
          const int kb = i / (2 * T::DB), u = (i / T::DB) & 1, cb = i % T::DB;
          const u32x4 b4 = {pk[kb][4 * u], pk[kb][4 * u + 1], pk[kb][4 * u + 2], pk[kb][4 * u + 3]};
          const u32x2 lo2 = __builtin_bit_cast(u32x2, vfr[i][0]);
          const u32x2 hi2 = __builtin_bit_cast(u32x2, vfr[i][1]);
          const u32x4 a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), __builtin_bit_cast(bf16x8, b4),
                                                             oacc[cb], 0, 0, 0);
        }
        if (DO_QK && i < NQK) {
          const int s = i / KB, kb = i % KB;
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kfr[i]), qf[s], sacc[kb], 0, 0, 0);
        }
      }
    };
    products();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) pin(sacc[kb]);
#pragma unroll
    for (int cb = 0; cb < T::DB; ++cb) pin(oacc[cb]);
    __builtin_amdgcn_s_setprio(0);
  };
  // Online softmax of sacc (tile t) into pk.  The mask, where the tile crosses
  // the valid-key end or this wave's causal diagonal, overwrites sacc in place.
  auto softmax = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * BN;
    const bool need_mask = (k0 + BN > kv_valid) || (CAUSAL && k0 + BN - 1 > qw0);
    if (need_mask) {
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
    // Exponentials against the current reference max, without computing
    // this tile's max: every p is at most 2^kTau whenever the lane's sum of
    // its p over the tile is (all p are >= 0), so the max is computed only
    // on the rare tiles where that sum is larger (or not a number, or the
    // row has no reference yet); those tiles are recomputed against it.
    auto exps = [&](float mref) __attribute__((always_inline)) {
      float part[KB * 8];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][2 * j], sc, -mref));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][2 * j + 1], sc, -mref));
          const uint32_t pp = pack_bf16(p0, p1);
          part[kb * 8 + j] = p0 + p1;
          pk[kb][j] = pp;
        }
#pragma unroll
      for (int w = KB * 4; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) part[i] = part[i] + part[i + w];
      return part[0];
    };
    float ls = exps(m_run == -INFINITY ? 0.0f : m_run);
    const bool bad = !(ls <= kMaxTileSum) || m_run == -INFINITY;
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      keep_branch();
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx * sc);
      const float alpha = (m_run == -INFINITY || m_new == m_run) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int cb = 0; cb < T::DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
      ls = exps(m_run == -INFINITY ? 0.0f : m_run);
    }
    l_run += ls;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) pin(pk[kb][j]);
    pin(l_run);
  };

  // Global phase counter, identical in every wave.  Phase 2t starts the loads of
  // K_{t+1} and V_t; phase 2t+1 ends by waiting for them.
  // The barrier after an odd phase is what the data needs: the tile loads are
  // complete and visible, and the buffers the next loads overwrite were last
  // read in the two phases before it.  The barrier after an even phase only
  // keeps the two groups one phase apart; the softmax phase reads no LDS, so
  // without it a group that finishes its softmax early starts its products
  // beside the other group's last products instead of waiting.  At head size
  // 128 and 256 that measured faster (long context 1.790 -> 1.775 ms, d = 256
  // 1.841 -> 1.804 ms, non-causal d = 128 0.873 -> 0.861 ms, median of
  // same-process runs; results bitwise equal); at head size 64, where the
  // softmax phase is the longer one, it was 2-4% slower, so it stays there.
  constexpr bool kEvenBarrier = D < 128;
  const int n_phases = 2 * ntk + 2;
  int ph = 0;
  auto issue_tile = [&]() __attribute__((always_inline)) {
    if ((ph & 1) == 0) {
      const int t = ph >> 1;
      if (t < ntk) {
        if (t + 1 < ntk) load_k(t + 1);
        load_v(t);
      }
    }
  };
  // At head size 128 and 256 the wave entering its matrix phase issues its
  // share of an even phase's loads after its products, not before them: the
  // issue then no longer delays the tile's first products, while the other
  // group, entering its softmax phase, still issues at the start (long context
  // 1.823 -> 1.811 ms, d = 256 1.837 -> 1.790 ms, non-causal d = 128
  // 0.890 -> 0.883 ms; results bitwise equal).  Issuing between the products
  // measured the same.  The loads still precede the wait at the end of the
  // next phase, and the buffers they fill were last read before the barrier
  // that ends the phase before.
  constexpr bool kLateMatrixIssue = D >= 128;
  auto begin_phase = [&](const bool matrix_next = false) __attribute__((always_inline)) {
    if (!(kLateMatrixIssue && matrix_next)) issue_tile();
  };
  auto after_matrix = [&]() __attribute__((always_inline)) {
    if (kLateMatrixIssue) issue_tile();
  };
  auto end_phase = [&]() __attribute__((always_inline)) {
    if (ph & 1) wait_vmem();
    __builtin_amdgcn_sched_barrier(0);
    if (kEvenBarrier || (ph & 1)) __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    ++ph;
  };
  if (ntk > 0) {
    load_k(0);
    wait_vmem();
    __syncthreads();
    if (grp == 1) {              // the second group starts one phase late
      begin_phase();
      end_phase();
    }
    if (last >= 0) {
      begin_phase(true);
      mfma_phase(false, 0, true, 0);
      after_matrix();
      end_phase();
      for (int t = 0; t < last; ++t) {
        begin_phase();
        softmax(t);
        end_phase();
        begin_phase(true);
        mfma_phase(true, t, true, t + 1);
        after_matrix();
        end_phase();
      }
      begin_phase();
      softmax(last);
      end_phase();
      begin_phase(true);
      mfma_phase(true, last, false, 0);
      after_matrix();
      end_phase();
    }
    while (ph < n_phases) {      // keep loading and meeting the barriers
      begin_phase();
      end_phase();
    }
  }

  const float l = pair_sum(l_run);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
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
    if (p.lse && hi == 0) p.lse[(size_t)bh * N + qi] = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, int BN, bool CAUSAL>
hipError_t launch_pp(const FwdParams& p, hipStream_t stream) {
  const int ntiles = (p.N + 255) / 256;
  const dim3 grid((unsigned)ntiles * (unsigned)p.H * (unsigned)p.B);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_pp_kernel<D, BN, CAUSAL>), grid, dim3(512), args, 0, stream);
}

template <int D, int QB, int BN, int OCC, bool CAUSAL, int KS = 1>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  constexpr int BM = kWaves * 32 * QB;
  const int ntiles = (p.N + BM - 1) / BM;
  const dim3 grid((unsigned)ntiles * (unsigned)p.H * (unsigned)p.B);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, QB, BN, OCC, CAUSAL, KS>), grid,
                         dim3(kThreads * KS), args, 0, stream);
}

#if defined(FA_FORCE_FWD)
// Candidate builds for the kernel-choice measurements (built only with
// -DFA_FORCE_FWD=<id>, never in the library itself): every bf16 forward call
// runs the one kernel form <id> names, so that rocprofv3 counters of each
// candidate can be taken on the same workload.
//   1 8-wave, 64-key tiles     2 8-wave, 128-key tiles (d 64)   3 8-wave, 32-key tiles (d 128)
//   4 4-wave, 32-key tiles     5 4-wave, 64-key tiles           6 4-wave, 128-key tiles (d 64)
//   7 4-wave two key groups, 64-key tiles   8 4-wave two key groups, 128-key tiles (d 64)
template <int D, bool C>
hipError_t launch_candidate(int id, const FwdParams& p, hipStream_t stream) {
  switch (id) {
    case 1: return launch_pp<D, 64, C>(p, stream);
    case 2: if constexpr (D == 64) return launch_pp<64, 128, C>(p, stream); break;
    case 3: if constexpr (D == 128) return launch_pp<128, 32, C>(p, stream); break;
    case 4: return launch<D, 1, 32, 2, C>(p, stream);
    case 5: return launch<D, 1, 64, 2, C>(p, stream);
    case 6: if constexpr (D == 64) return launch<64, 1, 128, 2, C>(p, stream); break;
    case 7: return launch<D, 1, 64, (D == 64 ? 2 : 1), C, 2>(p, stream);
    case 8: if constexpr (D == 64) return launch<64, 1, 128, 1, C, 2>(p, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;
}
#endif

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
#if defined(FA_FORCE_FWD)
  if (p.d == 64) return p.causal ? launch_candidate<64, true>(FA_FORCE_FWD, p, stream)
                                 : launch_candidate<64, false>(FA_FORCE_FWD, p, stream);
  if (p.d == 128) return p.causal ? launch_candidate<128, true>(FA_FORCE_FWD, p, stream)
                                  : launch_candidate<128, false>(FA_FORCE_FWD, p, stream);
#endif
  // Kernel choice by head size, key range and grid size (workgroups of the
  // ping-pong kernel: 256 query rows each), from same-process timings of every
  // candidate on gfx950 over grids of 32 to 2048 such workgroups.
  const long long pp_groups = (long long)p.B * p.H * ((p.N + 255) / 256);
  // The ping-pong kernel addresses a head's K and V by 32-bit byte offsets
  // from the head's base (the scalar-base form of its tile loads).
  const bool pp_fits = (unsigned long long)p.N * (unsigned long long)p.d * 2ull <= 0xFFFFFFFFull;
  if (p.d == 256) {
    // 32-key tiles: the score tile, the Q fragments (64 registers) and O^T (128)
    // of a wave then fit two waves per SIMD.  On grids of 256 (non-causal) and
    // 512 (causal) workgroups the ping-pong kernel takes 11-29% less time than
    // the one-wave-per-SIMD head-size-256 kernel (128 query rows per
    // workgroup), which takes 12-18% less on grids of 64 and 128.
    if (pp_groups >= 256 && pp_fits)
      return p.causal ? launch_pp<256, 32, true>(p, stream) : launch_pp<256, 32, false>(p, stream);
    return launch_fwd_bf16_d256(p, stream);
  }
  if (p.d == 64) {
    // At head size 64 the softmax outweighs the products and each tile's fixed
    // costs (load issue, barriers) weigh more, so long key ranges take 128-key
    // tiles, which halve them per score.  The ping-pong kernel needs a full
    // grid: 256 workgroups, and causal grids need 4096 keys or more (at 2048
    // causal keys the 4-wave kernel takes 11-13% less time even at 2048
    // workgroups).  Elsewhere the 4-wave kernel (128 rows per workgroup, two
    // workgroups per compute unit) runs 128-key tiles from 2048 keys up (3-12%
    // less time than 64-key tiles on grids under 1024 workgroups, within 3%
    // above) and 64-key tiles below, where a workgroup sees only a few tiles.
    const bool pp_long = p.causal ? (pp_groups >= 256 && p.N >= 4096) : (pp_groups >= 256 && p.N >= 2048);
    if (pp_long && pp_fits) return p.causal ? launch_pp<64, 128, true>(p, stream) : launch_pp<64, 128, false>(p, stream);
    // Below that the 4-wave kernel runs, also on full grids: under 2048 keys it
    // takes 4-8% less time than the ping-pong kernel with 64-key tiles
    // (non-causal) and 16-33% less (causal, 1024 and 1536 keys, 256 to 512
    // heads).  Small grids split each workgroup's keys over two groups of 4
    // waves, so that 128-row workgroups of 8 waves cover the chip: from 1024
    // keys on grids of at most 256 such workgroups with 128-key tiles (one
    // workgroup per compute unit; 11-17% less time than one key group,
    // non-causal, and 7-9% less than two groups with 64-key tiles, causal).
    // Causal grids up to 512 workgroups, which still fit the chip in one round
    // at two 8-wave workgroups per compute unit, take 64-key tiles: the
    // longest workgroups, which set the time of a small causal launch, take
    // half as many steps (4-10% less time than one group on grids of 128 to
    // 256 workgroups; 2-9% more on grids of 768 to 1024, which no longer fit
    // in one round).
    const long long w4_groups = (long long)p.B * p.H * ((p.N + 127) / 128);
    if (p.N >= 1024 && w4_groups <= 256)
      return p.causal ? launch<64, 1, 128, 1, true, 2>(p, stream) : launch<64, 1, 128, 1, false, 2>(p, stream);
    if (p.causal && w4_groups <= 512) return launch<64, 1, 64, 2, true, 2>(p, stream);
    if (p.N >= 2048) return p.causal ? launch<64, 1, 128, 2, true>(p, stream) : launch<64, 1, 128, 2, false>(p, stream);
    return p.causal ? launch<64, 1, 64, 2, true>(p, stream) : launch<64, 1, 64, 2, false>(p, stream);
  }
  // Head size 128: grids of at most 128 ping-pong workgroups leave compute
  // units idle; from 768 keys they run the 4-wave kernel with two key groups
  // and 64-key tiles instead (128-row workgroups of 8 waves, one per compute
  // unit: 19-27% less time than the ping-pong kernel on grids of 32 to 128,
  // causal or not; on grids of 192 and 256 it is 10-16% faster for some causal
  // shapes and 8-37% slower for others).  Larger grids take the ping-pong
  // kernel from 1024 keys up (4-28% less time than the 4-wave kernel with one
  // key group on grids of 256 to 512 workgroups) and the 4-wave kernel below
  // (10-14% less time than the ping-pong kernel at 512 keys on 512 and 1024
  // heads).
  if (pp_groups <= 128 && p.N >= 768)
    return p.causal ? launch<128, 1, 64, 1, true, 2>(p, stream) : launch<128, 1, 64, 1, false, 2>(p, stream);
  if (p.N >= 1024 && pp_fits)
    return p.causal ? launch_pp<128, 64, true>(p, stream) : launch_pp<128, 64, false>(p, stream);
  return p.causal ? launch<128, 1, 32, 2, true>(p, stream) : launch<128, 1, 32, 2, false>(p, stream);
}

}  // namespace fa
