// Device-side building blocks shared by the attention kernels for gfx950:
// operand vector types, the LDS layout (swizzles and tile geometry), lane-pair
// reductions, bf16 packing, ordering helpers and the global->LDS load.
// Internal to the library (not part of include/fa.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;      // lazy-rescale threshold, log2 units
constexpr float kMaxTileSum = 256.0f;   // 2^kTau

template <int D, int BN>
struct Tile {
  static constexpr int KB = BN / 32;                // 32-key blocks per tile
  static constexpr int CH = D / 8;                  // 16-byte chunks per row
  static constexpr int DC = D / 16;                 // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;                 // 32-row blocks of O^T
  static constexpr int ROW = D * 2;                 // bytes per row
  static constexpr int MAT = BN * ROW;              // one K or V tile
  static constexpr int STAGE = 2 * MAT;             // K + V
  static constexpr int NLD = MAT / (1024 * kWaves); // 1 KB wave-loads per wave per matrix
  static_assert(MAT % (1024 * kWaves) == 0, "tile load must split evenly over the waves");
};

// LDS swizzles (16-byte chunk c of row r is stored at chunk c ^ swz(r)), chosen
// by measurement on gfx950, where ds_read_b128 is serviced 16 lanes (256 bytes)
// at a time and ds_read_b64_tr_b16 32 lanes at a time.
// K: the S^T A-operand read sends 16 consecutive rows, same chunk, through one
// cycle; the XOR spreads them over all 64 banks (d=64 rows are 128 bytes, so
// two rows share a 256-byte bank line).
template <int D>
__device__ __forceinline__ int kswz(int row) { return D == 64 ? ((row >> 1) & 7) : (row & 15); }
// V: 16 lanes of the transposing read cover 4 consecutive rows x 32 bytes, 32
// lanes 4 rows x 64 bytes; an XOR by a multiple of 2 chunks keeps each 32-byte
// pair together and places the 4 rows in distinct banks.
template <int D>
__device__ __forceinline__ int vswz(int row) { return D == 64 ? ((row & 3) << 1) : ((row & 3) << 2); }

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

// Sum of v[0..N) (N a power of two) as a balanced tree, overwriting v.  The
// softmax row sums use it on the float32 probabilities: plain adds, where a
// v_dot2 over the packed bf16 values would run on the matrix pipeline at a
// fraction of the VALU rate whenever another wave's products are running.
template <int N>
__device__ __forceinline__ float tree_sum(float (&v)[N]) {
  static_assert((N & (N - 1)) == 0, "power of two");
#pragma unroll
  for (int w = N / 2; w >= 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) v[i] = v[i] + v[i + w];
  return v[0];
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;  // round to nearest even (v_cvt_pk_bf16_f32)
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// An empty volatile asm: marks a rarely taken branch (the softmax rescale) so
// that the compiler keeps it a branch instead of executing its body on every
// tile with a neutral factor.
__device__ __forceinline__ void keep_branch() { asm volatile("" ::: "memory"); }

// Empty volatile asm that consumes a register value: the computation of the
// value cannot be moved after this point (register-only arithmetic may
// otherwise migrate across a workgroup barrier, which orders memory only).
template <typename V>
__host__ __device__ __forceinline__ void pin(const V& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(v));
#endif
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup -> (batch * head, query tile) for a grid of ntiles query tiles per
// head and bh_count heads.
// Without the causal mask every tile costs the same.  The dispatcher hands
// workgroup i to XCD i % 8; XCD x gets the contiguous logical range
// [x * per, (x + 1) * per), so neighbouring query tiles of one head share that
// XCD's L2 for their K/V reads.
// With the causal mask query tile qt costs about qt + 1 key tiles.  On a grid
// of at most four rounds of ncu workgroups (ncu compute units) the whole grid
// is resident at once, and the hardware places workgroups i, i + ncu, i + 2 ncu,
// ... on one compute unit (measured on gfx950), so the logical order decides
// how much work each unit gets: tiles are ranked heaviest first (query tile
// descending, then head), and odd rounds take their ranks in reverse order of
// the groups of 8 (keeping i % 8, hence the XCD of a head when bh_count is a
// multiple of 8).  The sums over a unit's workgroups are then nearly equal
// (GPT-2-shaped causal: at most 30 key tiles per unit against a mean of 27,
// where one tile per head for every round put 48 on some units and 6 on
// others).  Larger causal grids are dispatched as units free up: their tiles go
// heaviest first within each XCD's contiguous range.
// Rank (heaviest first) of workgroup bid on a grid of at most four rounds of
// ncu: even rounds take ranks in order, odd rounds in reverse order of the
// groups of 8, keeping bid % 8.
__device__ __forceinline__ int snake_rank(int bid, int total, int ncu) {
  const int r = bid / ncu;
  if ((r & 1) && (r + 1) * ncu <= total) {
    const int c = bid - r * ncu;
    return r * ncu + ((((ncu >> 3) - 1 - (c >> 3)) << 3) | (c & 7));
  }
  return bid;
}

__device__ __forceinline__ void grid_tile(int bid, int total, int ntiles, int bh_count, bool causal, int ncu, int& bh,
                                          int& qt) {
  if (causal && total <= 4 * ncu && (ncu & 7) == 0) {
    const int k = snake_rank(bid, total, ncu);
    const int qr = k / bh_count;
    bh = k - qr * bh_count;
    qt = ntiles - 1 - qr;
    return;
  }
  const int per = total >> 3;
  const int lid = (bid < (per << 3)) ? (bid & 7) * per + (bid >> 3) : bid;
  bh = lid / ntiles;
  qt = lid - bh * ntiles;
  if (causal) qt = ntiles - 1 - qt;  // heaviest tiles first
}

// The same for a grid without the causal mask whose batches have their own key
// lengths (seqlens, B entries): a tile of batch b costs about ceil(L_b / bn)
// key tiles.  When the whole grid is resident at once (as above) the tiles are
// ranked by that cost, longest batches first (ties by batch index), and the
// ranks go to the units in the same alternating order as the causal tiles, so
// that every unit gets a similar sum.  Within a batch consecutive ranks take
// consecutive heads, so the query tiles of one head stay on one XCD when H is a
// multiple of 8.  Every wave computes the same mapping: lane j < B holds batch
// j's cost and its rank among the batches.  Returns false (mapping not taken)
// for grids of more than four rounds or more than 64 batches.
__device__ __forceinline__ bool grid_tile_lengths(int bid, int total, int ntiles, int B, int H, int N, int bn,
                                                  const int32_t* seqlens, int ncu, int& bh, int& qt) {
  if (!(total <= 4 * ncu && (ncu & 7) == 0 && B <= 64)) return false;
  const int lane = (int)(threadIdx.x & 63);
  int c = -1;
  if (lane < B) {
    const int L = seqlens[lane];
    c = ((L < 0 ? 0 : (L > N ? N : L)) + bn - 1) / bn;
  }
  int rank = 0;
  for (int j = 0; j < B; ++j) {
    const int cj = __builtin_amdgcn_readlane(c, j);
    rank += (cj > c || (cj == c && j < lane)) ? 1 : 0;
  }
  const int k = snake_rank(bid, total, ncu);
  const int per_b = H * ntiles;
  const int pos = k / per_b;   // < B: the grid has B * H * ntiles workgroups
  const int rest = k - pos * per_b;
  // the ranks of lanes 0..B-1 are a permutation of 0..B-1: exactly one bit
  const unsigned long long m = __builtin_amdgcn_ballot_w64(lane < B && rank == pos);
  const int b = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(m));
  qt = rest / H;
  bh = b * H + (rest - qt * H);
  return true;
}

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_base + 16 i (global_load_lds_dwordx4).  The builtin exists only for
// the device target; clang's host pass drops a kernel whose body names it, so
// its use is confined to the device pass.
__device__ __forceinline__ void load_to_lds16(const void* src, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
#endif
}


// 16 bytes per lane from global memory straight into LDS (lane i of the wave to
// lds_base + 16 i).  Issued as inline assembly so that the compiler does not
// treat the LDS buffers being filled as aliasing the ones being read; the
// kernel waits for these loads itself (vmcnt) before the barrier that publishes
// them.  M0 carries the LDS base; the s_nop is the wait state the hardware
// requires between an M0 write and its use by an LDS DMA.
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  const unsigned l = (unsigned)(uintptr_t)((lds_void*)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(l), "v"(src) : "memory", "m0");
}

// The same load addressed as a wave-uniform base (SGPR pair) plus a 32-bit
// per-lane byte offset (VGPR): global_load_lds_dwordx4 voffset, sbase.  On
// gfx950 a vector-memory instruction that reads a 64-bit address from VGPRs is
// slow to issue while another wave on the SIMD runs products whose
// accumulators are VGPRs (four such loads: about 1090 ticks, against 85 with
// no products beside them); this form reads one VGPR and issues in about 120.
// `base` must be the same in every lane; `off` < 2^32.
// A wave-uniform pointer moved to SGPRs once (readfirstlane of both halves),
// so that loops taking it as a scalar base do not re-read it from VGPRs.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t b = (uint64_t)(uintptr_t)p;
  const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  return reinterpret_cast<P*>((uintptr_t)u);
}

__device__ __forceinline__ void dma16s(const void* base, uint32_t off, void* lds_base) {
  const unsigned l = (unsigned)(uintptr_t)((lds_void*)lds_base);
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(l), "v"(off), "s"(bu)
               : "memory", "m0");
}

}  // namespace
}  // namespace fa
