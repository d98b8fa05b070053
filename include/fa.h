/*
 * fa.h - C interface of the fused exact attention forward pass for AMD MI355X
 * (CDNA4, gfx950).
 *
 * The operation is exact attention as the pages define it,
 *     O = softmax(scale * Q K^T) V,  row-wise softmax over the keys,
 * (FlashAttention (UR), section "The problem of standard attention"; the same
 * formula in FlashAttention (FA)), computed tile by tile with an online softmax
 * so that the N x N score matrix never reaches device memory (FlashAttention
 * (UR), sections "Tiling and block-based processing", "Online computation of
 * softmax" and "Fusing the operations into one CUDA kernel").  One call
 * computes every (batch, head) of a [B, H, N, d] problem.
 *
 * Layout.  q, k, v and o are dense row-major [B, H, N, d] arrays (d fastest,
 * then the sequence index, then the head, then the batch).  lse is a dense
 * [B, H, N] float array.  seqlens is an int32 [B] array.  All of them are
 * DEVICE pointers (memory the current HIP device can read and write).
 *
 * Masks ("masking" is one of the fused steps on the pages; its meaning here):
 *   causal != 0 : query i attends to key j only if j <= i;
 *   seqlens     : batch b has seqlens[b] valid keys; keys j >= seqlens[b] are
 *                 dropped for every query of that batch; queries are not
 *                 dropped.  NULL means all N keys are valid.
 * Both masks combine with AND.  A row with no valid key gets O = 0 and
 * LSE = -inf.
 *
 * LSE.  lse[b,h,i] = log(sum_j exp(scale * q_i . k_j)) over the valid keys, in
 * natural log, float32.  It is not on the pages; it is the statistic a later
 * merge of partial results, or a backward pass, needs.
 *
 * Ownership and execution.  The caller owns every buffer.  The library
 * allocates no device or host memory and keeps no state across calls besides a
 * cache of device properties (and, for fa_decode_noalloc only, one static
 * device array per GPU, described there).  A call validates its arguments on the host,
 * enqueues one kernel on `stream` (a hipStream_t; NULL = the default stream)
 * and returns without synchronising.  Calls are thread-safe.
 *
 * Errors.  Argument checks happen on the host before anything is enqueued and
 * return a negative fa_status; nothing is written then.  seqlens values live on
 * the device and are not checked on the host: the kernel clamps each to
 * [0, N].  Faults inside the kernel (for example a pointer that is not device
 * memory) surface through the HIP runtime at the next synchronisation, as for
 * any kernel.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* NULL tensor, B/H/N < 1, H_kv not dividing H, bad scale, size overflow */
  FA_ERR_UNSUPPORTED = -2, /* d not supported by the entry point, or the current device is not gfx950 */
  FA_ERR_MISALIGNED = -3,  /* q, k, v, o not 16-byte aligned, or lse / seqlens not 4-byte aligned */
  FA_ERR_NO_DEVICE = -4,   /* no HIP device is present or current */
  FA_ERR_LAUNCH = -5,      /* the HIP runtime refused the kernel launch */
  FA_ERR_SCRATCH_TOO_SMALL = -6 /* fa_decode_noalloc: the partial results exceed its static scratch */
} fa_status;

/*
 * bf16 forward pass (the hot path).
 *   q, k, v : const __hip_bfloat16*  [B, H, N, d]
 *   o       : __hip_bfloat16*        [B, H, N, d]   output, round to nearest even
 *   lse     : float*                 [B, H, N]      output; may be NULL (not written)
 *   B, H, N : batch, heads, sequence length (>= 1); queries and keys share N
 *   d       : head dimension, 64, 128 or 256
 *   scale   : softmax scale (the pages' 1/sqrt(d_k)); finite and > 0
 *   causal  : 0 or non-zero
 *   seqlens : const int32_t* [B] key-padding lengths on the device, or NULL
 *   stream  : hipStream_t to enqueue on, or NULL
 * Arithmetic: S = Q K^T and O += P V on bf16 matrix cores with float32
 * accumulation; softmax statistics in float32; P is rounded to bf16 for the
 * second product.  The row sum is taken over that rounded P in the kernels for
 * partial grids and short key ranges, and over the float32 P before rounding
 * in the 8-wave kernel for full grids and long key ranges (the weights then
 * sum to 1 within 2^-8, the unit roundoff of bf16).
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t* seqlens, void* stream);

/*
 * float32 forward pass: same arguments and semantics with float tensors; every
 * product, exponential and sum is float32 (no reduced-precision matrix path).
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               const int32_t* seqlens, void* stream);

/*
 * Grouped-query / multi-query forward pass (FlashAttention (UR), section
 * "FlashAttention-2 (2023)": multi-query attention among the supported
 * architectures).  q and o are [B, H, N, d]; k and v are [B, H_kv, N, d] with
 * 1 <= H_kv <= H and H_kv dividing H.  Query heads
 * g*(H/H_kv) .. (g+1)*(H/H_kv)-1 attend to key/value head g: H_kv = H is
 * fa_fwd, H_kv = 1 is multi-query attention.  Every other argument, the
 * arithmetic and the errors are those of fa_fwd (bf16) and fa_fwd_f32 (float);
 * an H_kv that does not divide H returns FA_ERR_INVALID_ARG.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, int causal,
               const int32_t* seqlens, void* stream);
int fa_fwd_gqa_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                   int B, int H, int H_kv, int N, int d, float scale, int causal,
                   const int32_t* seqlens, void* stream);

/*
 * Decoding against a key/value cache, keys split across workgroups.
 *   q, o     : [B, H, Nq, d] bf16 (Nq new queries per head), o written
 *   k, v     : [B, H_kv, Nk, d] bf16 (the cache; H_kv divides H, grouped as
 *              in fa_fwd_gqa)
 *   lse      : float [B, H, Nq] output, natural log; may be NULL
 *   seqlens  : int32 [B] valid cache length per batch on the device (clamped
 *              to [0, Nk]), or NULL for Nk
 *   causal   : query i of batch b is position L_b - Nq + i of its sequence
 *              and sees only keys j <= L_b - Nq + i (non-zero), or every
 *              valid key (0)
 *   num_splits : key chunks per (batch, key/value head); 0 = chosen by the
 *              library from the shape
 *   workspace, workspace_size : caller-owned device memory of at least
 *              fa_decode_workspace_size(...) bytes (16-byte aligned), used for
 *              the partial results; its contents on entry do not matter
 * The keys of each valid cache are split into num_splits contiguous chunks of
 * whole 64-key tiles; one kernel computes each chunk's softmax average and
 * log-sum-exp, a second kernel combines the chunks (LSE = log sum exp LSE_s,
 * O = sum exp(LSE_s - LSE) O_s; FlashAttention (UR), section "Online
 * computation of softmax", applied to whole partial results).  Arithmetic as
 * fa_fwd; partial results are float32.  Returns FA_OK or a negative fa_status
 * (FA_ERR_INVALID_ARG also for a workspace smaller than required); nothing is
 * enqueued on error.
 */
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
              const int32_t* seqlens, int num_splits, void* workspace, size_t workspace_size, void* stream);

/* Bytes of workspace fa_decode needs for these arguments (0 for invalid ones). */
size_t fa_decode_workspace_size(int B, int H, int H_kv, int Nq, int Nk, int d, int num_splits);

/*
 * fa_decode without a workspace, for callers that cannot allocate device memory
 * around the call (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, arithmetic and results are those of
 * fa_decode (same kernels, same key splits); the partial results go to a static
 * device array of FA_DECODE_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends.  The call allocates nothing and frees
 * nothing.
 *   Limit: fa_decode_workspace_size(...) of the same arguments must not exceed
 *   FA_DECODE_NOALLOC_SCRATCH_BYTES, else FA_ERR_SCRATCH_TOO_SMALL is returned
 *   and nothing is enqueued (the bench decode step, B=8 H=32 Nq=1 d=128 with 8
 *   key splits, needs about 1 MiB).
 *   Sharing: every call on one GPU uses that GPU's one array, so calls that
 *   overlap on one GPU (different streams or threads without ordering between
 *   them) race and must not be issued; calls ordered on one stream are safe.
 *   The array's previous contents never matter: every partial result a call
 *   reads, it has written.
 *   The first call on a device looks up that device's array address (once,
 *   with that device current).
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                      const int32_t* seqlens, int num_splits, void* stream);

/*
 * FP8 forward pass: Q, K, V as e4m3 codes with one scale per tensor.
 *   q        : uint8 [B, H, N, d] e4m3 codes (OCP 8-bit float: 1 sign, 4
 *              exponent bits with bias 7, 3 mantissa bits, max 448, NaN only
 *              for 0x7F / 0xFF); the query tensor is q_descale * value(q)
 *   k, v     : uint8 [B, H_kv, N, d] e4m3 codes, scaled by k_descale, v_descale
 *   o        : __hip_bfloat16 [B, H, N, d] output;  lse : float [B, H, N] or NULL
 *   d        : 64 or 128;  descales: finite and > 0;  other arguments as fa_fwd_gqa
 * FlashAttention (UR), section "FlashAttention-3 (2024)", names FP8 support.
 * Arithmetic: S = Q K^T on 8-bit matrix cores with float32 accumulation; the
 * softmax in float32 with a reference row max that moves only when a tile's
 * max exceeds it by more than 2^0.75, so P <= 2^0.75; P scaled by 2^8 and
 * rounded to e4m3 (relative error <= 2^-4) for O += P V on 8-bit matrix cores;
 * the row sum l adds the float32 P.  Returns FA_OK or a negative fa_status;
 * nothing is enqueued on error.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, float q_descale, float k_descale, float v_descale,
               int causal, const int32_t* seqlens, void* stream);

/*
 * Backward pass: dQ, dK, dV for a loss whose gradient with respect to the
 * forward output O is dout.  The pages print no backward algorithm; this is the
 * chain rule through the forward definition:
 *   P = softmax(scale Q K^T) (masked), dV = P^T dO, dP = dO V^T,
 *   dS = P o (dP - D) with D_i = dO_i . O_i, dQ = scale dS K, dK = scale dS^T Q,
 * with P recomputed tile by tile from Q, K and the forward LSE, as the forward
 * pass computes it without storing the attention matrix (FlashAttention (UR),
 * "Tiling and block-based processing").
 *   q, o, dout : [B, H, N, d] bf16 (o and lse are the forward pass's outputs)
 *   k, v       : [B, H_kv, N, d] bf16 (H_kv divides H, grouped as fa_fwd_gqa)
 *   lse        : float [B, H, N], the forward pass's row log-sum-exp (required)
 *   dq         : [B, H, N, d] bf16 output
 *   dk, dv     : [B, H_kv, N, d] bf16 outputs; with grouped heads, the sum over
 *                the query heads that share the key/value head
 *   d          : 64 or 128 (FA_ERR_UNSUPPORTED otherwise, and for heads of
 *                4 GiB or more, N * d * 2 >= 2^32 bytes: the kernels address a
 *                head's rows by 32-bit offsets)
 *   scale, causal, seqlens : as for the forward call that produced o and lse
 *   workspace, workspace_size : caller-owned device memory of at least
 *                fa_bwd_workspace_size(B, H, N) bytes (16-byte aligned) for the
 *                per-row D and LSE log2(e); its contents on entry do not matter
 * Arithmetic: bf16 products on matrix cores with float32 accumulation; P and dS
 * are rounded to bf16 as operands of the gradient products; every sum has a
 * fixed order (no atomics), so results are bitwise repeatable.  Keys at or past
 * a batch's padding length get zero dK, dV.  Enqueues three kernels on stream;
 * returns FA_OK or a negative fa_status (FA_ERR_INVALID_ARG also for a
 * workspace smaller than required); nothing is enqueued on error.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int causal,
           const int32_t* seqlens, void* workspace, size_t workspace_size, void* stream);

/* Bytes of workspace fa_bwd needs (0 for invalid arguments). */
size_t fa_bwd_workspace_size(int B, int H, int N);

/*
 * Measurement aid, not part of the attention path: enqueues on `stream` a
 * kernel of FA_CLOCK_SAMPLE_UNITS workgroups in which workgroup w writes
 * out[3w] = the core clock counter of the compute unit it runs on (s_memtime,
 * core clock cycles; the counters of different units are not aligned),
 * out[3w+1] = the constant 100 MHz counter (s_memrealtime) and out[3w+2] =
 * the unit's place (XCD id << 16 | shader engine << 8 | unit).  out is a
 * device pointer to 3 * FA_CLOCK_SAMPLE_UNITS uint64 values.  Two samples
 * around a batch of attention launches on the same stream, paired by unit,
 * give each unit's average core clock over the batch:
 * 100 MHz * d(cycles) / d(ticks).  Returns FA_OK or a negative fa_status.
 */
#define FA_CLOCK_SAMPLE_UNITS 256
int fa_clock_sample(unsigned long long* out, void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* fa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
