// Gradients of exact attention (dQ, dK, dV), bf16 in / bf16 out, for gfx950.
//
// The pages quote their speed-ups for training but print no backward
// algorithm (FlashAttention (UR), "Experimental results"; FlashAttention-2 (HI),
// "Performance and efficiency").  What is computed is the chain rule through
// the forward definition, for a loss whose gradient with respect to O is dO:
//     P = softmax(scale Q K^T) (row-wise, masked),  dV = P^T dO,  dP = dO V^T,
//     dS = P o (dP - D),  D_i = dO_i . O_i,  dQ = scale dS K,  dK = scale dS^T Q.
// As in the forward pass, the N x N matrices never reach HBM: P is recomputed
// tile by tile from Q, K and the forward pass's row log-sum-exp, the same
// recomputation that lets the forward pass keep no attention matrix
// (FlashAttention (UR), "Tiling and block-based processing").
//
// Three kernels, no atomics, a fixed order of every sum (bitwise repeatable):
//  1. bwd_rowdot_kernel: D_i = dO_i . O_i and lse2_i = LSE_i log2(e) per query
//     row, into the caller's workspace (rows padded to a multiple of 128 per
//     head, the padding set to lse2 = +inf, D = 0).
//  2. bwd_dkdv_kernel: one workgroup per (batch, key/value head, 128 keys);
//     each wave holds its 32 keys' K and V rows as matrix operands and the
//     transposed accumulators dV^T, dK^T, and streams 128-query tiles of Q, dO,
//     lse2 and D (every query head of the group in turn) through LDS:
//         S = Q K^T, P = exp2(S scale log2e - lse2), dP = dO V^T,
//         dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
//     Lanes own keys and registers hold queries, so P and dS feed the next
//     products straight from the accumulators, as P^T does in the forward
//     kernels with the roles of queries and keys exchanged.
//  3. bwd_dq_kernel: one workgroup per (batch, head, 128 queries); each wave
//     holds its 32 queries' Q and dO rows and dQ^T, and streams 64-key tiles of
//     K and V:  S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D),
//     dQ^T += K^T dS^T.
//     On grids of at least 256 workgroups of 256 queries, dQ runs in a
//     ping-pong form instead (bwd_dq_pp_kernel): 8 waves in two groups that
//     alternate the products with the exponentials, one phase apart.
// Computing dQ in its own pass recomputes S and dP once more (7 products per
// score instead of 5) in exchange for no atomic accumulation of dQ across key
// tiles.
//
// Q and dO (kernel 2) and K (kernel 3) are read from LDS both as rows (A
// operand of S, dP) and transposed (A operand of dK^T, dV^T, dQ^T, via
// ds_read_b64_tr_b16), so their 16-byte chunks are stored with one XOR
// swizzle that keeps both access patterns free of bank conflicts.
// The dK/dV kernel runs one wave per SIMD: its 256 VGPRs hold the operands and
// the gradient accumulators, with a few values parked in the accumulation
// registers; the dQ kernels fit two waves per SIMD in 256 registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBT = 64;         // rows of a loaded tile (two per query tile of kernel 2; the key tile of kernel 3)
constexpr int kRowsWG = 128;    // rows held per workgroup (4 waves x 32)
constexpr int kQT = 128;        // query rows per streamed tile of the dK/dV kernel

// Swizzle for tiles read both as rows and transposed: chunk c of row r is stored
// at c ^ swz(r).  Rows: 16 lanes read one chunk of 16 consecutive rows, which
// land in 16 distinct 16-byte bank groups.  Transposed: 32 lanes read 64 bytes
// of 4 consecutive rows 4a..4a+3, which land in 4 distinct 64-byte bank windows
// (d = 128: bits 2-3 of the swizzle differ; d = 64, two rows per 256 bytes:
// rows 4a and 4a+2 differ in bit 2).
template <int D>
__device__ __forceinline__ int bswz(int row) {
  return D == 64 ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)) : (((row & 3) << 2) | ((row >> 2) & 3));
}

// ---------------------------------------------------------------------------
// 1. D_i = dO_i . O_i and lse2_i; 16 lanes per row (8 elements each at d = 128,
// 4 at d = 64), 16 rows per workgroup.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(BwdParams p) {
  constexpr int EPL = D / 16;   // elements per lane
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * 16 + (tid >> 4);   // padded row index
  const int sub = tid & 15;
  const long long bh = row / p.Npad;
  const int i = (int)(row - bh * p.Npad);
  if (bh >= (long long)p.B * p.H) return;
  float acc = 0.0f;
  float lse = -INFINITY;
  if (i < p.N) {
    const size_t off = ((size_t)bh * p.N + i) * D + sub * EPL;
    const __bf16* o = reinterpret_cast<const __bf16*>(p.o) + off;
    const __bf16* g = reinterpret_cast<const __bf16*>(p.dout) + off;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
    lse = p.lse[(size_t)bh * p.N + i];
  }
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, 16);
  if (sub == 0) {
    p.delta[row] = acc;
    // a row with no allowed key (LSE = -inf) gets P = exp2(s - inf) = 0
    p.lse2[row] = lse == -INFINITY ? INFINITY : lse * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// Shared operand addressing for a 64-row tile stored with bswz.
// ---------------------------------------------------------------------------
template <int D>
struct TileAddr {
  using T = Tile<D, kBT>;
  int row_base;   // A operand of k-step s, rows blk*32 + r32: XOR with 32 s
  int tr_base0;   // transposed read of rows 16u + 4hi + {0..3} of a 32-row block: XOR with 64 cb
  int tr_base1;   // the same for rows 16u + 8 + 4hi + {0..3}
  __device__ __forceinline__ TileAddr(int lane) {
    const int r32 = lane & 31, hi = lane >> 5;
    const int x = bswz<D>(r32);
    row_base = r32 * T::ROW + ((((x >> 1) << 1) | (hi ^ (x & 1))) << 4);
    const int i16 = lane & 15, g16 = (lane >> 4) & 1;
    const int vrow = 4 * hi + (i16 >> 2);
    const int c0 = 2 * g16 + ((i16 & 3) >> 1);
    tr_base0 = vrow * T::ROW + ((c0 ^ bswz<D>(vrow)) << 4) + (i16 & 1) * 8;
    tr_base1 = (vrow + 8) * T::ROW + ((c0 ^ bswz<D>(vrow + 8)) << 4) + (i16 & 1) * 8;
  }
};

// Transposing read pair of rows (blk*32 + 16u) + {4hi + 0..3, 8 + 4hi + 0..3},
// columns of row block cb: the A operand X^T[col][row] of one product.
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char* tile, int tb0, int tb1, int blk, int u, int cb) {
  using T = Tile<D, kBT>;
  const char* base = tile + (blk * 32 + 16 * u) * T::ROW;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + (tb0 ^ (cb << 6))));
  const s16x4 hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + (tb1 ^ (cb << 6))));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
  const u32x2 hi2 = __builtin_bit_cast(u32x2, hv);
  const u32x4 a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
  return __builtin_bit_cast(bf16x8, a4);
}

template <int D>
__device__ __forceinline__ bf16x8 read_row(const char* tile, int rb, int blk, int s) {
  using T = Tile<D, kBT>;
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + blk * 32 * T::ROW + (rb ^ (s << 5))));
}

// A sequence of N products in order, product i taking the A operand rd(i):
// each operand is read from LDS AHEAD products before its product, so the
// reads are in flight under the matrix work (a scheduling fence after every
// product keeps the compiler from hoisting a whole tile's reads).
template <int N, int AHEAD, typename RD, typename MF>
__device__ __forceinline__ void products(RD rd, MF mf) {
  bf16x8 ring[AHEAD];
#pragma unroll
  for (int i = 0; i < AHEAD && i < N; ++i) ring[i] = rd(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bf16x8 a = ring[i % AHEAD];
    if (i + AHEAD < N) ring[i % AHEAD] = rd(i + AHEAD);
    mf(i, a);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// N1 products then N2 products, their A operands read through one ring of
// AHEAD registers, so that the second sequence's first operands are read
// during the first sequence.
template <int N1, int N2, int AHEAD, typename RD1, typename MF1, typename RD2, typename MF2>
__device__ __forceinline__ void products2(RD1 rd1, MF1 mf1, RD2 rd2, MF2 mf2) {
  auto rd = [&](int g) __attribute__((always_inline)) { return g < N1 ? rd1(g) : rd2(g - N1); };
  bf16x8 ring[AHEAD];
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) ring[i] = rd(i);
#pragma unroll
  for (int g = 0; g < N1 + N2; ++g) {
    const bf16x8 a = ring[g % AHEAD];
    if (g + AHEAD < N1 + N2) ring[g % AHEAD] = rd(g + AHEAD);
    if (g < N1)
      mf1(g, a);
    else
      mf2(g - N1, a);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Direct global->LDS load of one 64-row tile (rows clamped to [0, N-1]).
// Wave-load j (j = wave * NLD + i) fills LDS rows RPL j .. RPL j + RPL - 1, lane
// l writing stored chunk l % CH of row RPL j + l / CH, so it fetches the global
// chunk that the swizzle puts there.  The swizzle reads only row bits 0-3, and
// RPL * NLD = 16, so it splits into a lane part and a constant per i:
// bswz(RPL j + lr) = bswz(lr) ^ bswz(RPL i) for lr < RPL.  A load then costs
// four address instructions (add, clamp, xor, shift-add) instead of about
// fifteen.
template <int D>
struct LoadLane {
  using T = Tile<D, kBT>;
  static constexpr int RPL = 64 / T::CH;   // rows per wave-load
  static_assert(RPL * T::NLD == 16, "a wave's loads span 16 rows, a whole period of the swizzle");
  int lr;        // row within a wave-load
  uint32_t lc;   // byte offset of the lane's chunk before the per-load constant
  // the lane index through an empty asm: the per-lane parts are recomputed at
  // each tile instead of being held in registers across the loop
  __device__ __forceinline__ explicit LoadLane(int lane) {
    asm volatile("" : "+v"(lane));
    lr = lane / T::CH;
    lc = (uint32_t)(((lane % T::CH) ^ bswz<D>(lr)) << 4);
  }
  // wave-load i of this wave's part of the tile at rows r0 .. r0 + 63
  __device__ __forceinline__ void load(const __bf16* src, int r0, int N, char* dst, int wave, int i) const {
    const int j = wave * T::NLD + i;
    const int r = min(r0 + j * RPL + lr, N - 1);
    dma16s(src, (uint32_t)r * (uint32_t)(D * 2) + (lc ^ (uint32_t)(bswz<D>(RPL * i) << 4)), dst + j * 1024);
  }
};

template <int D>
__device__ __forceinline__ void load_tile(const __bf16* src, int r0, int N, char* dst, int wave, int lane) {
  const LoadLane<D> ll(lane);
#pragma unroll
  for (int i = 0; i < Tile<D, kBT>::NLD; ++i) ll.load(src, r0, N, dst, wave, i);
}

// ---------------------------------------------------------------------------
// 2. dK, dV.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
  using T = Tile<D, kBT>;
  constexpr int DC = T::DC, DB = T::DB;
  constexpr int QMAT = 2 * T::MAT;                  // one 128-row tile of Q or dO
  constexpr int STAGE = 2 * QMAT + 2 * kQT * 4;      // Q, dO, lse2[128], D[128]
  static_assert(STAGE % 1024 == 0, "a stage offset leaves the swizzled low address bits alone");
  __shared__ __attribute__((aligned(1024))) char stages[2 * STAGE];

  const int N = p.N;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  const int nkt = (N + kRowsWG - 1) / kRowsWG;
  const int total = gridDim.x;
  const int bid = blockIdx.x;
  const int per = total >> 3;
  const int lid = (bid < (per << 3)) ? (bid & 7) * per + (bid >> 3) : bid;
  const int bg = lid / nkt;
  const int kt = lid - bg * nkt;   // ascending: under a causal mask the first key tiles have the most queries
  const int b = bg / p.Hkv;
  const int g = bg - b * p.Hkv;
  const int G = p.H / p.Hkv;

  int L = N;
  if (p.seqlens) {
    const int x = p.seqlens[b];
    L = x < 0 ? 0 : (x > N ? N : x);
  }
  const int k0 = kt * kRowsWG;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + r32;          // this lane's key
  const bool wave_live = kw0 < L;     // keys at or past L get zero gradients

  const size_t kvoff = ((size_t)b * p.Hkv + g) * (size_t)N * D;
  // K, V rows of this lane's key as B operands: element 16 s + 8 hi + e
  bf16x8 kf[DC], vf[DC];
  {
    const int kr = min(key, N - 1);
    const u32x4* krow = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(p.k) + kvoff + (size_t)kr * D);
    const u32x4* vrow = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(p.v) + kvoff + (size_t)kr * D);
#pragma unroll
    for (int s = 0; s < DC; ++s) {
      kf[s] = __builtin_bit_cast(bf16x8, krow[2 * s + hi]);
      vf[s] = __builtin_bit_cast(bf16x8, vrow[2 * s + hi]);
    }
  }

  const int nqt = (N + kQT - 1) / kQT;
  const int qstart = CAUSAL ? k0 / kQT : 0;
  const int per_head = nqt - qstart;
  const int n_it = L > k0 ? G * per_head : 0;   // no valid key in this workgroup: nothing to accumulate

  auto issue_loads = [&](int it, char* base) __attribute__((always_inline)) {
    const int hq = g * G + it / per_head;
    const int q0 = (qstart + it % per_head) * kQT;
    const size_t hoff = ((size_t)b * p.H + hq) * (size_t)N * D;
    load_tile<D>(reinterpret_cast<const __bf16*>(p.q) + hoff, q0, N, base, wave, lane);
    load_tile<D>(reinterpret_cast<const __bf16*>(p.q) + hoff, q0 + kBT, N, base + T::MAT, wave, lane);
    load_tile<D>(reinterpret_cast<const __bf16*>(p.dout) + hoff, q0, N, base + QMAT, wave, lane);
    load_tile<D>(reinterpret_cast<const __bf16*>(p.dout) + hoff, q0 + kBT, N, base + QMAT + T::MAT, wave, lane);
    if (wave < 2 && lane < 32) {   // 128 floats of lse2 (wave 0) or D (wave 1)
      const float* src = (wave == 0 ? p.lse2 : p.delta) + ((size_t)b * p.H + hq) * (size_t)p.Npad + q0;
      dma16s(src, (uint32_t)(lane * 16), base + 2 * QMAT + wave * kQT * 4);
    }
  };

  f32x16 dvacc[DB], dkacc[DB];
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) {
    dvacc[cb] = f32x16{};
    dkacc[cb] = f32x16{};
  }
  const float sc = p.scale * kLog2e;
  const TileAddr<D> ad(lane);

  // One 128-query tile from the stage at byte offset soff.  The offset goes into
  // the lane bases (opaque, so each is one register per tile); lse2 and D of
  // query qo sit at stages + lb + 4 qo and + 4 (kQT + qo), the lane part 16 hi
  // in lb.  spread(c, i) issues wave-load i of chunk c of the next tile.
  auto tile = [&](const bool mask, const int soff, int q0, auto&& spread) __attribute__((always_inline)) {
    const char* Qs = stages;
    const char* Gs = stages + QMAT;
    int rb = ad.row_base + soff, tb0 = ad.tr_base0 + soff, tb1 = ad.tr_base1 + soff, lb = 2 * QMAT + 16 * hi + soff;
    asm volatile("" : "+v"(rb), "+v"(tb0), "+v"(tb1), "+v"(lb));
    // The tile's 4 x NP products read their A operands from LDS through one
    // ring of AH registers that runs across the phases: the first operands of
    // a phase are read during the previous one (through the softmax too).
    // Long-context backward 7.091 -> 7.006 ms against a ring restarted at each
    // phase (same-process A/B, gradients bitwise equal); a ring of 6 the same.
    constexpr int NSP = 2 * DC, NGP = 4 * DB, NP = NSP + NGP, NB = kQT / 32, AH = 4;
    auto rd = [&](int g) __attribute__((always_inline)) {
      const int qb = g / NP, j = g % NP;
      if (j < NSP) return j < DC ? read_row<D>(Qs, rb, qb, j) : read_row<D>(Gs, rb, qb, j - DC);
      const int i = j - NSP;
      return read_tr<D>((i & 1) ? Qs : Gs, tb0, tb1, qb, i / (2 * DB), (i / 2) % DB);
    };
    bf16x8 ring[AH];
#pragma unroll
    for (int g = 0; g < AH; ++g) ring[g] = rd(g);
    auto next_operand = [&](int g) __attribute__((always_inline)) {
      const bf16x8 a = ring[g % AH];
      if (g + AH < NB * NP) ring[g % AH] = rd(g + AH);
      return a;
    };
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      // S[q][key] = Q K^T and dP[q][key] = dO V^T for 32 queries
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int i = 0; i < NSP; ++i) {
        const bf16x8 a = next_operand(qb * NP + i);
        if (i < DC)
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[i], sacc, 0, 0, 0);
        else
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[i - DC], pacc, 0, 0, 0);
        if (i < T::NLD) spread(qb, i);
        __builtin_amdgcn_sched_barrier(0);
      }
      // register r holds query q0 + 32 qb + 8 (r / 4) + 4 hi + r % 4
      uint32_t pk[8], dk[8];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
        const int qo = qb * 32 + 8 * gq + 4 * hi;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(stages + lb + 4 * (qb * 32 + 8 * gq));
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(stages + lb + 4 * (kQT + qb * 32 + 8 * gq));
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * gq + e], sc, -l4[e]));
        if (mask) {   // wave-uniform: only tiles on the diagonal or at a ragged end
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int q = q0 + qo + e;
            const bool ok = q < N && key < L && (!CAUSAL || key <= q);
            pv[e] = ok ? pv[e] : 0.0f;
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) dsv[e] = pv[e] * (pacc[4 * gq + e] - d4[e]);
        pk[2 * gq] = pack_bf16(pv[0], pv[1]);
        pk[2 * gq + 1] = pack_bf16(pv[2], pv[3]);
        dk[2 * gq] = pack_bf16(dsv[0], dsv[1]);
        dk[2 * gq + 1] = pack_bf16(dsv[2], dsv[3]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries, 16 at a time:
      // half u takes registers 8u..8u+7, queries 16u + 4hi + {0..3, 8..11}
      // product i: half u = i / (2 DB), column block cb = (i / 2) % DB, dV (even i) or dK (odd i)
      bf16x8 bp[2], bs[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bp[u] = __builtin_bit_cast(bf16x8, u32x4{pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]});
        bs[u] = __builtin_bit_cast(bf16x8, u32x4{dk[4 * u], dk[4 * u + 1], dk[4 * u + 2], dk[4 * u + 3]});
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NGP; ++i) {
        const bf16x8 a = next_operand(qb * NP + NSP + i);
        const int u = i / (2 * DB), cb = (i / 2) % DB;
        if (i & 1)
          dkacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bs[u], dkacc[cb], 0, 0, 0);
        else
          dvacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp[u], dvacc[cb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Every wave with a valid key works on every tile: the first query tile of a
  // causal workgroup starts at the workgroup's first key, so it reaches every
  // wave's keys.  Waves whose keys all lie at or past L only load.  One code
  // path per tile (the mask a wave-uniform branch inside it, the stage an
  // offset) keeps the accumulators in the same registers from tile to tile.
  static_assert(kQT == kRowsWG, "query tiles start at the workgroup's first key");
  static_assert(kQT / 32 == 4, "four 32-query blocks issue the four 64-row chunks of the next tile");
  auto step = [&](int it) __attribute__((always_inline)) {
    const bool more = it + 1 < n_it;
    const int soff = (it & 1) * STAGE;
    char* next = stages + (STAGE - soff);
    const int q0 = (qstart + it % per_head) * kQT;
    // The next tile's loads are spread over this tile's four 32-query blocks:
    // block c issues chunk c (Q rows 0-63, Q rows 64-127, dO rows 0-63, dO rows
    // 64-127), one wave-load after each of its first NLD products, so that the
    // loads queue beside the products instead of stalling the wave at once.
    // The loads are unconditional (no branch per load): after the last tile
    // they fetch that tile again into the idle stage, in bounds and waited for
    // like the others (long-context backward 6.851 -> 6.745 ms, same-process).
    const int itn = more ? it + 1 : it;
    const int hqn = g * G + itn / per_head;
    const int q0n = (qstart + itn % per_head) * kQT;
    const size_t hoffn = ((size_t)b * p.H + hqn) * (size_t)N * D;
    const __bf16* qsrc = reinterpret_cast<const __bf16*>(p.q) + hoffn;
    const __bf16* gsrc = reinterpret_cast<const __bf16*>(p.dout) + hoffn;
    const LoadLane<D> ll(lane);
    if (wave < 2 && lane < 32) {   // 128 floats of lse2 (wave 0) or D (wave 1)
      const float* src = (wave == 0 ? p.lse2 : p.delta) + ((size_t)b * p.H + hqn) * (size_t)p.Npad + q0n;
      dma16s(src, (uint32_t)(lane * 16), next + 2 * QMAT + wave * kQT * 4);
    }
    auto spread = [&](int c, int i) __attribute__((always_inline)) {
      ll.load(c < 2 ? qsrc : gsrc, q0n + (c & 1) * kBT, N, next + (c >> 1) * QMAT + (c & 1) * T::MAT, wave, i);
    };
    const bool need_mask = (q0 + kQT > N) || (kw0 + 32 > L) || (CAUSAL && q0 < kw0 + 31);
    tile(need_mask, soff, q0, spread);
    wait_vmem();
    __syncthreads();
  };

  if (n_it > 0) issue_loads(0, stages);
  wait_vmem();
  __syncthreads();
  if (wave_live) {
    for (int it = 0; it < n_it; ++it) step(it);
  } else {
    for (int it = 0; it < n_it; ++it) {   // the same barriers, loads only
      if (it + 1 < n_it) issue_loads(it + 1, stages + ((it + 1) & 1) * STAGE);
      wait_vmem();
      __syncthreads();
    }
  }

  // dV^T, dK^T register r: column 32 cb + 8 (r / 4) + 4 hi + r % 4 of this lane's key
  if (key < N) {
    __bf16* dvrow = reinterpret_cast<__bf16*>(p.dv) + kvoff + (size_t)key * D;
    __bf16* dkrow = reinterpret_cast<__bf16*>(p.dk) + kvoff + (size_t)key * D;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = cb * 32 + 8 * gq + 4 * hi;
        const u32x2 wv = {pack_bf16(dvacc[cb][4 * gq], dvacc[cb][4 * gq + 1]),
                          pack_bf16(dvacc[cb][4 * gq + 2], dvacc[cb][4 * gq + 3])};
        const u32x2 wk = {pack_bf16(dkacc[cb][4 * gq] * p.scale, dkacc[cb][4 * gq + 1] * p.scale),
                          pack_bf16(dkacc[cb][4 * gq + 2] * p.scale, dkacc[cb][4 * gq + 3] * p.scale)};
        *reinterpret_cast<u32x2*>(dvrow + col) = wv;
        *reinterpret_cast<u32x2*>(dkrow + col) = wk;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdParams p) {
  using T = Tile<D, kBT>;
  constexpr int DC = T::DC, DB = T::DB;
  constexpr int STAGE = 2 * T::MAT;   // K, V
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE];

  const int N = p.N;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r32 = lane & 31;
  const int hi = lane >> 5;

  const int ntiles = (N + kRowsWG - 1) / kRowsWG;
  const int total = gridDim.x;
  const int bid = blockIdx.x;
  const int per = total >> 3;
  const int lid = (bid < (per << 3)) ? (bid & 7) * per + (bid >> 3) : bid;
  const int bh = lid / ntiles;
  int qt = lid - bh * ntiles;
  if (CAUSAL) qt = ntiles - 1 - qt;   // heaviest first
  const int b = bh / p.H;

  const size_t hoff = (size_t)bh * (size_t)N * D;
  const size_t kvoff = ((size_t)b * p.Hkv + (bh - b * p.H) / (p.H / p.Hkv)) * (size_t)N * D;
  const __bf16* __restrict__ Kh = reinterpret_cast<const __bf16*>(p.k) + kvoff;
  const __bf16* __restrict__ Vh = reinterpret_cast<const __bf16*>(p.v) + kvoff;

  int L = N;
  if (p.seqlens) {
    const int x = p.seqlens[b];
    L = x < 0 ? 0 : (x > N ? N : x);
  }
  const int q0 = qt * kRowsWG;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + r32;
  int kv_end = L;
  if (CAUSAL) kv_end = min(kv_end, q0 + kRowsWG);
  const int ntk = (kv_end + kBT - 1) / kBT;

  bf16x8 qf[DC], gf[DC];
  {
    const int qr = min(qi, N - 1);
    const u32x4* qrow = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(p.q) + hoff + (size_t)qr * D);
    const u32x4* grow = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(p.dout) + hoff + (size_t)qr * D);
#pragma unroll
    for (int s = 0; s < DC; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, qrow[2 * s + hi]);
      gf[s] = __builtin_bit_cast(bf16x8, grow[2 * s + hi]);
    }
  }
  const float lse2 = p.lse2[(size_t)bh * p.Npad + min(qi, p.Npad - 1)];
  const float dsum = p.delta[(size_t)bh * p.Npad + min(qi, p.Npad - 1)];

  f32x16 dqacc[DB];
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) dqacc[cb] = f32x16{};
  const float sc = p.scale * kLog2e;
  const TileAddr<D> ad(lane);

  auto tile = [&](const bool MASK, const char* st, int k0) __attribute__((always_inline)) {
    const char* Ks = st;
    const char* Vs = st + T::MAT;
    int rb = ad.row_base, tb0 = ad.tr_base0, tb1 = ad.tr_base1;
    asm volatile("" : "+v"(rb), "+v"(tb0), "+v"(tb1));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T[key][q] = K Q^T and dP^T[key][q] = V dO^T for 32 keys
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      products<2 * DC, 2>(
          [&](int i) __attribute__((always_inline)) { return i < DC ? read_row<D>(Ks, rb, kb, i) : read_row<D>(Vs, rb, kb, i - DC); },
          [&](int i, const bf16x8& a) __attribute__((always_inline)) {
            if (i < DC)
              sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i], sacc, 0, 0, 0);
            else
              pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gf[i - DC], pacc, 0, 0, 0);
          });
      // register r holds key k0 + 32 kb + 8 (r / 4) + 4 hi + r % 4
      uint32_t dk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float dsv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * j + e;
          float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], sc, -lse2));
          if (MASK) {
            const int kk = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool ok = kk < L && (!CAUSAL || kk <= qi);
            pr = ok ? pr : 0.0f;
          }
          dsv[e] = pr * (pacc[r] - dsum);
        }
        dk[j] = pack_bf16(dsv[0], dsv[1]);
      }
      // dQ^T += K^T dS^T over these 32 keys, 16 at a time
      bf16x8 bs[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        bs[u] = __builtin_bit_cast(bf16x8, u32x4{dk[4 * u], dk[4 * u + 1], dk[4 * u + 2], dk[4 * u + 3]});
      products<2 * DB, 2>(
          [&](int i) __attribute__((always_inline)) { return read_tr<D>(Ks, tb0, tb1, kb, i / DB, i % DB); },
          [&](int i, const bf16x8& a) __attribute__((always_inline)) {
            dqacc[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bs[i / DB], dqacc[i % DB], 0, 0, 0);
          });
    }
  };

  auto issue_loads = [&](int t, char* base) __attribute__((always_inline)) {
    load_tile<D>(Kh, t * kBT, N, base, wave, lane);
    load_tile<D>(Vh, t * kBT, N, base + T::MAT, wave, lane);
  };

  auto step = [&](int t, const char* cur, char* next) __attribute__((always_inline)) {
    if (t + 1 < ntk) issue_loads(t + 1, next);
    const int k0 = t * kBT;
    const bool active = !CAUSAL || (k0 <= qw0 + 31);
    if (active) {
      const bool need_mask = (k0 + kBT > L) || (CAUSAL && k0 + kBT - 1 > qw0);
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

  if (qi < N) {
    __bf16* orow = reinterpret_cast<__bf16*>(p.dq) + hoff + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = cb * 32 + 8 * gq + 4 * hi;
        const u32x2 w = {pack_bf16(dqacc[cb][4 * gq] * p.scale, dqacc[cb][4 * gq + 1] * p.scale),
                         pack_bf16(dqacc[cb][4 * gq + 2] * p.scale, dqacc[cb][4 * gq + 3] * p.scale)};
        *reinterpret_cast<u32x2*>(orow + col) = w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------------------
// 3b. dQ, ping-pong form for large grids: 8 waves in two groups of 4 (waves w
// and w + 4 share a SIMD), 256 queries per workgroup (32 per wave), BT-key
// tiles (64 as launched; 32-key tiles measured slower).  Each wave alternates a matrix phase (dQ^T += K^T dS^T of tile t - 1,
// then S^T and dP^T of tile t) with a VALU phase (P and dS of tile t); the two
// groups run one phase apart, so on every SIMD one wave keeps the matrix core
// busy while the other computes exponentials, as in the 8-wave forward kernel.
// K has three LDS buffers (tile t - 1 is read transposed by the dQ product
// while tile t is read as rows and tile t + 1 loads), V two.  At every even
// phase 2t the workgroup issues the loads of tile t + 1 and waits for them at
// the end of phase 2t + 1; the first reads of that tile come at phase 2t + 2,
// and the buffers it overwrites were last read in phases 2t - 2 and 2t - 1.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int BT>
__global__ __launch_bounds__(512, 1) void bwd_dq_pp_kernel(BwdParams p) {
  constexpr int KB = BT / 32;         // 32-key blocks per tile
  constexpr int BM = 256;             // queries per workgroup
  constexpr int ROW = D * 2;          // bytes per row
  constexpr int MAT = BT * ROW;       // one K or V tile
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int RPL = 64 / CH;        // rows per 1 KB wave-load
  constexpr int NWL = MAT / 1024;     // wave-loads per matrix
  constexpr int DC = D / 16, DB = D / 32;
  static_assert(NWL % 8 == 0 || NWL == 4, "wave-loads split over 8 waves");
  __shared__ __attribute__((aligned(1024))) char kbuf[3][MAT];
  __shared__ __attribute__((aligned(1024))) char vbuf[2][MAT];

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
  if (CAUSAL) qt = ntiles - 1 - qt;   // heaviest first
  const int b = bh / p.H;

  const size_t hoff = (size_t)bh * (size_t)N * D;
  const size_t kvoff = ((size_t)b * p.Hkv + (bh - b * p.H) / (p.H / p.Hkv)) * (size_t)N * D;
  const __bf16* Kh = uniform_ptr(reinterpret_cast<const __bf16*>(p.k) + kvoff);
  const __bf16* Vh = uniform_ptr(reinterpret_cast<const __bf16*>(p.v) + kvoff);

  int L = N;
  if (p.seqlens) {
    const int x = p.seqlens[b];
    L = x < 0 ? 0 : (x > N ? N : x);
  }
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + r32;
  int kv_end = L;
  if (CAUSAL) kv_end = min(kv_end, q0 + BM);
  const int ntk = (kv_end + BT - 1) / BT;              // tiles the workgroup streams
  int last = ntk - 1;                                   // last tile this wave needs
  if (CAUSAL) last = min(last, (qw0 + 31) / BT);

  bf16x8 qf[DC], gf[DC];
  {
    const int qr = min(qi, N - 1);
    const u32x4* qrow = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(p.q) + hoff + (size_t)qr * D);
    const u32x4* grow = reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(p.dout) + hoff + (size_t)qr * D);
#pragma unroll
    for (int s = 0; s < DC; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, qrow[2 * s + hi]);
      gf[s] = __builtin_bit_cast(bf16x8, grow[2 * s + hi]);
    }
  }
  // rows past the padded end read the last padded row; their results are not stored
  const float lse2 = p.lse2[(size_t)bh * p.Npad + min(qi, p.Npad - 1)];
  const float dsum = p.delta[(size_t)bh * p.Npad + min(qi, p.Npad - 1)];

  // Tile loads: wave-load j of a matrix fills rows RPL j .. RPL j + RPL - 1
  // (the split of the swizzle as in load_tile: bswz(RPL j + lr) = bswz(lr) ^
  // bswz(RPL j)).  Wave w issues K wave-load w and V wave-load w (d = 128), or
  // K wave-load w (waves 0-3) or V wave-load w - 4 (waves 4-7, d = 64).
  auto load_kv = [&](int t) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lr = ln / CH;
    const uint32_t lc = (uint32_t)(((ln % CH) ^ bswz<D>(lr)) << 4);
    auto one = [&](const __bf16* src, char* dst, int j) __attribute__((always_inline)) {
      const int r = min(t * BT + j * RPL + lr, N - 1);
      dma16s(src, (uint32_t)r * (uint32_t)ROW + (lc ^ (uint32_t)(bswz<D>(RPL * j) << 4)), dst + j * 1024);
    };
    if constexpr (NWL % 8 == 0) {
#pragma unroll
      for (int i = 0; i < NWL / 8; ++i) {
        one(Kh, kbuf[t % 3], wave + 8 * i);
        one(Vh, vbuf[t & 1], wave + 8 * i);
      }
    } else {
      if (wave < 4)
        one(Kh, kbuf[t % 3], wave);
      else
        one(Vh, vbuf[t & 1], wave - 4);
    }
  };

  f32x16 dqacc[DB];
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) dqacc[cb] = f32x16{};
  f32x16 sacc[KB], pacc[KB];                  // S^T, dP^T of the tile in flight
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    sacc[kb] = f32x16{};
    pacc[kb] = f32x16{};
  }
  uint32_t dk[KB][8] = {};                    // dS^T of the previous tile, bf16 pairs
  const float sc = p.scale * kLog2e;
  const TileAddr<D> ad(lane);

  // Matrix phase: dQ^T += K_tq^T dS^T (if DO_DQ), then S^T and dP^T of tile ts
  // (if DO_S), the S^T and dP^T products interleaved (two accumulation chains).
  // With both, one operand ring runs through the two sequences, so the first
  // S^T operands are read during the last dQ^T products (long-context backward
  // 7.116 -> 7.062 ms in a same-process A/B, gradients bitwise equal).
  auto mfma_phase = [&](const bool DO_DQ, int tq, const bool DO_S, int ts) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    int rb = ad.row_base, tb0 = ad.tr_base0, tb1 = ad.tr_base1;
    asm volatile("" : "+v"(rb), "+v"(tb0), "+v"(tb1));
    // product i: key block kb = i / (2 DB), half u = (i / DB) % 2, column block cb = i % DB
    const char* Kq = kbuf[tq % 3];
    auto rd_dq = [&](int i) __attribute__((always_inline)) { return read_tr<D>(Kq, tb0, tb1, i / (2 * DB), (i / DB) & 1, i % DB); };
    auto mf_dq = [&](int i, const bf16x8& a) __attribute__((always_inline)) {
      const int kb = i / (2 * DB), u = (i / DB) & 1;
      const bf16x8 bs = __builtin_bit_cast(bf16x8, u32x4{dk[kb][4 * u], dk[kb][4 * u + 1], dk[kb][4 * u + 2], dk[kb][4 * u + 3]});
      dqacc[i % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bs, dqacc[i % DB], 0, 0, 0);
    };
    // product i: chain c = i % (2 KB) (S^T of block c / 2, or dP^T of it if c is odd), k-step i / (2 KB)
    const char* Ks = kbuf[ts % 3];
    const char* Vs = vbuf[ts & 1];
    auto rd_s = [&](int i) __attribute__((always_inline)) {
      const int c = i % (2 * KB), st = i / (2 * KB);
      return (c & 1) ? read_row<D>(Vs, rb, c >> 1, st) : read_row<D>(Ks, rb, c >> 1, st);
    };
    auto mf_s = [&](int i, const bf16x8& a) __attribute__((always_inline)) {
      const int c = i % (2 * KB), st = i / (2 * KB);
      if (c & 1)
        pacc[c >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gf[st], pacc[c >> 1], 0, 0, 0);
      else
        sacc[c >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], sacc[c >> 1], 0, 0, 0);
    };
    if (DO_S) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[kb] = f32x16{};
        pacc[kb] = f32x16{};
      }
    }
    if (DO_DQ && DO_S)
      products2<2 * DB * KB, 2 * DC * KB, 4>(rd_dq, mf_dq, rd_s, mf_s);
    else if (DO_DQ)
      products<2 * DB * KB, 2>(rd_dq, mf_dq);
    else if (DO_S)
      products<2 * DC * KB, 4>(rd_s, mf_s);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      pin(sacc[kb]);
      pin(pacc[kb]);
    }
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) pin(dqacc[cb]);
    __builtin_amdgcn_s_setprio(0);
  };

  // VALU phase: P = exp2(S scale log2e - lse2) (masked), dS = P (dP - D), packed.
  // Register r holds key 32 t + 8 (r / 4) + 4 hi + r % 4 of this lane's query.
  auto valu_phase = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * BT;
    auto body = [&](const bool MASK) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float dsv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int r = 2 * j + e;
            float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], sc, -lse2));
            if (MASK) {
              const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
              const bool ok = kk < L && (!CAUSAL || kk <= qi);
              pr = ok ? pr : 0.0f;
            }
            dsv[e] = pr * (pacc[kb][r] - dsum);
          }
          dk[kb][j] = pack_bf16(dsv[0], dsv[1]);
        }
    };
    const bool need_mask = (k0 + BT > L) || (CAUSAL && k0 + BT - 1 > qw0);
    if (need_mask)
      body(true);
    else
      body(false);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) pin(dk[kb][j]);
  };

  // Global phase counter, identical in every wave (all waves meet every
  // barrier, including waves past their last tile).
  const int n_phases = 2 * ntk + 2;
  int ph = 0;
  auto issue_tile = [&]() __attribute__((always_inline)) {
    if ((ph & 1) == 0) {
      const int t = ph >> 1;
      if (t + 1 < ntk) load_kv(t + 1);
    }
  };
  // The wave entering its matrix phase issues its share of the loads after
  // its products (as in the 8-wave forward kernel), so the issue does not
  // delay the phase's first products (long-context backward 7.426 -> 7.373
  // ms, gradients bitwise equal).
  auto begin_phase = [&](const bool matrix_next = false) __attribute__((always_inline)) {
    if (!matrix_next) issue_tile();
  };
  auto after_matrix = [&]() __attribute__((always_inline)) { issue_tile(); };
  auto end_phase = [&]() __attribute__((always_inline)) {
    if (ph & 1) wait_vmem();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    ++ph;
  };
  if (ntk > 0) {
    load_kv(0);
    wait_vmem();
    __syncthreads();
    if (grp == 1) {   // the second group starts one phase late
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
        valu_phase(t);
        end_phase();
        begin_phase(true);
        mfma_phase(true, t, true, t + 1);
        after_matrix();
        end_phase();
      }
      begin_phase();
      valu_phase(last);
      end_phase();
      begin_phase(true);
      mfma_phase(true, last, false, 0);
      after_matrix();
      end_phase();
    }
    while (ph < n_phases) {   // keep loading and meeting the barriers
      begin_phase();
      end_phase();
    }
  }

  if (qi < N) {
    __bf16* orow = reinterpret_cast<__bf16*>(p.dq) + hoff + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int col = cb * 32 + 8 * gq + 4 * hi;
        const u32x2 w = {pack_bf16(dqacc[cb][4 * gq] * p.scale, dqacc[cb][4 * gq + 1] * p.scale),
                         pack_bf16(dqacc[cb][4 * gq + 2] * p.scale, dqacc[cb][4 * gq + 3] * p.scale)};
        *reinterpret_cast<u32x2*>(orow + col) = w;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int D>
hipError_t launch_all(const BwdParams& p, hipStream_t stream) {
  BwdParams arg = p;
  void* args[] = {&arg};
  const long long rows = (long long)p.B * p.H * p.Npad;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_rowdot_kernel<D>), dim3((unsigned)((rows + 15) / 16)),
                                 dim3(256), args, 0, stream);
  if (e != hipSuccess) return e;
  const unsigned nt = (unsigned)((p.N + kRowsWG - 1) / kRowsWG);
  const void* kv = p.causal ? reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, true>)
                            : reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, false>);
  e = hipLaunchKernel(kv, dim3(nt * (unsigned)p.B * (unsigned)p.Hkv), dim3(kThreads), args, 0, stream);
  if (e != hipSuccess) return e;
  // dQ: the ping-pong form once its grid (256 queries per workgroup) fills the
  // chip, else the 4-wave form with two workgroups per compute unit.  Both
  // sum every dQ row over 32-key blocks in the same order (bitwise equal).
  const unsigned ntp = (unsigned)((p.N + 255) / 256);
  if (ntp * (unsigned)p.B * (unsigned)p.H >= 256u) {
    const void* dqp = p.causal ? reinterpret_cast<const void*>(&bwd_dq_pp_kernel<D, true, 64>)
                               : reinterpret_cast<const void*>(&bwd_dq_pp_kernel<D, false, 64>);
    return hipLaunchKernel(dqp, dim3(ntp * (unsigned)p.B * (unsigned)p.H), dim3(512), args, 0, stream);
  }
  const void* dq = p.causal ? reinterpret_cast<const void*>(&bwd_dq_kernel<D, true>)
                            : reinterpret_cast<const void*>(&bwd_dq_kernel<D, false>);
  return hipLaunchKernel(dq, dim3(nt * (unsigned)p.B * (unsigned)p.H), dim3(kThreads), args, 0, stream);
}

}  // namespace

int bwd_row_pad() { return kQT; }

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  return p.d == 64 ? launch_all<64>(p, stream) : launch_all<128>(p, stream);
}

}  // namespace fa
