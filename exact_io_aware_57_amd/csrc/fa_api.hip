// Host entry points of the C interface declared in include/fa.h: argument
// validation, the device check and dispatch to the kernel launchers.  Nothing
// here allocates memory or synchronises the device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"

// Static scratch of fa_decode_noalloc: the split kernel's partial results live
// here instead of in a caller workspace.  Each GPU the library runs on holds its
// own copy of this array (FA_DECODE_NOALLOC_SCRATCH_BYTES) until the process
// ends, and every fa_decode_noalloc call on that GPU uses it (calls that overlap
// on one GPU race).  Host code never passes the array's name to a kernel: on
// the host it only stands in for the symbol, and the device address of the
// current GPU's copy comes from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {
// Workgroup w reads the core clock counter of the compute unit it runs on
// (s_memtime, counting core clock cycles; the counters of different units are
// not aligned with one another), the constant 100 MHz counter (s_memrealtime)
// and the unit's place: XCD id << 16 | shader engine << 8 | unit, from the
// XCC_ID and HW_ID registers.  Two samples around other work, paired by unit,
// give each unit's average core clock in between.
__global__ void clock_sample_kernel(unsigned long long* out) {
  if (threadIdx.x == 0) {
    const unsigned hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);        // HW_ID
    const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15;  // XCC_ID
    out[3 * blockIdx.x] = __builtin_amdgcn_s_memtime();
    out[3 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
    out[3 * blockIdx.x + 2] = (xcc << 16) | (((hw >> 13) & 7) << 8) | ((hw >> 8) & 15);
  }
}
}  // namespace

namespace {

constexpr int kMaxDevices = 64;
// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other;
// and the device's compute-unit count (filled by the same check).
std::atomic<int> g_arch_ok[kMaxDevices];
std::atomic<int> g_num_cu[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FA_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  int v = g_arch_ok[dev].load(std::memory_order_acquire);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FA_ERR_NO_DEVICE;
    }
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_num_cu[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch_ok[dev].store(v, std::memory_order_release);
  }
  return v == 1 ? FA_OK : FA_ERR_UNSUPPORTED;
}

// Compute units of the current device (after check_device() accepted it).
int current_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  const int n = g_num_cu[dev].load(std::memory_order_relaxed);
  return n > 0 ? n : 256;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Device address of each GPU's copy of `scratch` (above), looked up once per
// device with that device current.
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, or null if the lookup
// failed.  dev is the current device (check_device() has accepted it).
void* scratch_address(int dev) {
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    void* found = nullptr;
    if (hipGetSymbolAddress(&found, HIP_SYMBOL(scratch)) != hipSuccess || !found) {
      (void)hipGetLastError();
      return nullptr;
    }
    ptr = found;
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

int validate(const fa::FwdParams& p) {
  if (!p.q || !p.k || !p.v || !p.o) return FA_ERR_INVALID_ARG;
  if (p.B < 1 || p.H < 1 || p.N < 1) return FA_ERR_INVALID_ARG;
  if (p.Hkv < 1 || p.Hkv > p.H || p.H % p.Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(p.scale) || !(p.scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (p.d != 64 && p.d != 128 && p.d != 256) return FA_ERR_UNSUPPORTED;
  // Every element offset must fit the 64-bit index arithmetic of the kernels and
  // the workgroup count must fit one grid dimension.
  const uint64_t elems = (uint64_t)p.B * (uint64_t)p.H * (uint64_t)p.N * (uint64_t)p.d;
  if (elems > (uint64_t(1) << 40)) return FA_ERR_INVALID_ARG;
  if ((uint64_t)p.B * (uint64_t)p.H * (uint64_t)p.N > (uint64_t)INT32_MAX) return FA_ERR_INVALID_ARG;
  if (!aligned(p.q, 16) || !aligned(p.k, 16) || !aligned(p.v, 16) || !aligned(p.o, 16)) return FA_ERR_MISALIGNED;
  if (p.lse && !aligned(p.lse, 4)) return FA_ERR_MISALIGNED;
  if (p.seqlens && !aligned(p.seqlens, 4)) return FA_ERR_MISALIGNED;
  return FA_OK;
}

int run(fa::FwdParams p, void* stream, bool bf16) {
  int st = validate(p);
  if (st != FA_OK) return st;
  st = check_device();
  if (st != FA_OK) return st;
  p.num_cu = current_cus();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = !bf16 ? fa::launch_fwd_f32(p, s) : fa::launch_fwd_bf16(p, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Key splits of a decode problem: enough workgroups to cover the chip twice,
// at least 4 tiles per split, at most 128 splits.
int decode_splits(int B, int H, int H_kv, int Nq, int Nk, int requested) {
  if (requested > 0) return requested;
  const long long rows = (long long)(H / H_kv) * Nq;
  const long long qblk = (rows + fa::decode_rows_per_block() - 1) / fa::decode_rows_per_block();
  const long long base = (long long)B * H_kv * qblk;
  const long long tiles = ((long long)Nk + fa::decode_tile_keys() - 1) / fa::decode_tile_keys();
  long long s = (512 + base - 1) / base;
  const long long s_max = tiles / 4 > 1 ? tiles / 4 : 1;
  if (s > s_max) s = s_max;
  if (s > 128) s = 128;
  return (int)(s < 1 ? 1 : s);
}

bool decode_shape_ok(int B, int H, int H_kv, int Nq, int Nk, int d) {
  return B >= 1 && H >= 1 && Nq >= 1 && Nk >= 1 && H_kv >= 1 && H_kv <= H && H % H_kv == 0 && (d == 64 || d == 128);
}

size_t workspace_bytes(int B, int H, int Nq, int d, int S) {
  const size_t rows = (size_t)B * H * Nq;
  return rows * (size_t)S * (size_t)d * sizeof(float) + rows * (size_t)S * sizeof(float);
}

int bwd_npad(int N) {
  const int pad = fa::bwd_row_pad();
  return (N + pad - 1) / pad * pad;
}

size_t bwd_workspace_bytes(int B, int H, int N) { return 2 * (size_t)B * H * (size_t)bwd_npad(N) * sizeof(float); }

// Validation and launch of one decode step.  ws == nullptr means the static
// scratch (fa_decode_noalloc): the problem must then fit its fixed size.
int decode_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int Nq,
                       int Nk, int d, float scale, int causal, const int32_t* seqlens, int num_splits, void* ws,
                       size_t ws_size, void* stream) {
  const bool use_scratch = ws == nullptr;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || H_kv < 1 || H_kv > H || H % H_kv != 0 || num_splits < 0)
    return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)B * H * Nq * d > (uint64_t(1) << 40) || (uint64_t)B * H_kv * Nk * d > (uint64_t(1) << 40))
    return FA_ERR_INVALID_ARG;
  const int S = decode_splits(B, H, H_kv, Nq, Nk, num_splits);
  const long long rows = (long long)(H / H_kv) * Nq;
  const long long qblk = (rows + fa::decode_rows_per_block() - 1) / fa::decode_rows_per_block();
  if ((long long)B * H_kv * qblk * S > INT32_MAX || (long long)B * H * Nq > INT32_MAX) return FA_ERR_INVALID_ARG;
  const size_t need = workspace_bytes(B, H, Nq, d, S);
  if (use_scratch) {
    if (need > (size_t)FA_DECODE_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH_TOO_SMALL;
  } else if (ws_size < need) {
    return FA_ERR_INVALID_ARG;
  }
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || (ws && !aligned(ws, 16)))
    return FA_ERR_MISALIGNED;
  if (lse && !aligned(lse, 4)) return FA_ERR_MISALIGNED;
  if (seqlens && !aligned(seqlens, 4)) return FA_ERR_MISALIGNED;
  const int st = check_device();
  if (st != FA_OK) return st;
  if (use_scratch) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
      (void)hipGetLastError();
      return FA_ERR_NO_DEVICE;
    }
    ws = scratch_address(dev);
    if (!ws) return FA_ERR_NO_DEVICE;
  }
  const size_t orows = (size_t)B * H * Nq;
  float* opart = reinterpret_cast<float*>(ws);
  float* lpart = opart + orows * (size_t)S * (size_t)d;
  fa::DecodeParams p{q, k, v, o, lse, seqlens, opart, lpart, B, H, H_kv, Nq, Nk, d, scale, causal ? 1 : 0, S, (int)qblk};
  return fa::launch_decode(p, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t fa_bwd_workspace_size(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  return bwd_workspace_bytes(B, H, N);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
           void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int causal, const int32_t* seqlens,
           void* workspace, size_t workspace_size, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || H_kv < 1 || H_kv > H || H % H_kv != 0) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // the kernels address a head's rows by 32-bit byte offsets from its base
  if ((uint64_t)N * (uint64_t)d * 2u > 0xFFFFFFFFull) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)B * H * N * d > (uint64_t(1) << 40)) return FA_ERR_INVALID_ARG;
  const long long tiles = ((long long)N + 127) / 128;
  if ((long long)B * H * tiles > INT32_MAX || (long long)B * H * (N + 64) > INT32_MAX) return FA_ERR_INVALID_ARG;
  if (workspace_size < bwd_workspace_bytes(B, H, N)) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16))
    return FA_ERR_MISALIGNED;
  if (!aligned(lse, 4)) return FA_ERR_MISALIGNED;
  if (seqlens && !aligned(seqlens, 4)) return FA_ERR_MISALIGNED;
  const int st = check_device();
  if (st != FA_OK) return st;
  const int Npad = bwd_npad(N);
  float* lse2 = reinterpret_cast<float*>(workspace);
  float* delta = lse2 + (size_t)B * H * Npad;
  fa::BwdParams p{q, k, v, o, dout, lse, dq, dk, dv, seqlens, lse2, delta, B, H, H_kv, N, Npad, d, scale,
                  causal ? 1 : 0};
  return fa::launch_bwd(p, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_decode_workspace_size(int B, int H, int H_kv, int Nq, int Nk, int d, int num_splits) {
  if (!decode_shape_ok(B, H, H_kv, Nq, Nk, d) || num_splits < 0) return 0;
  return workspace_bytes(B, H, Nq, d, decode_splits(B, H, H_kv, Nq, Nk, num_splits));
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
              const int32_t* seqlens, int num_splits, void* workspace, size_t workspace_size, void* stream) {
  if (!workspace) return FA_ERR_INVALID_ARG;
  return decode_impl(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, seqlens, num_splits, workspace,
                     workspace_size, stream);
}

int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal,
                      const int32_t* seqlens, int num_splits, void* stream) {
  return decode_impl(q, k, v, o, lse, B, H, H_kv, Nq, Nk, d, scale, causal, seqlens, num_splits, nullptr, 0, stream);
}

int fa_clock_sample(unsigned long long* out, void* stream) {
  if (!out) return FA_ERR_INVALID_ARG;
  if (!aligned(out, 8)) return FA_ERR_MISALIGNED;
  const int st = check_device();
  if (st != FA_OK) return st;
  void* args[] = {&out};
  return hipLaunchKernel(reinterpret_cast<const void*>(&clock_sample_kernel), dim3(FA_CLOCK_SAMPLE_UNITS), dim3(64),
                         args, 0,
                         reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? FA_OK
             : FA_ERR_LAUNCH;
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           const int32_t* seqlens, void* stream) {
  fa::FwdParams p{q, k, v, o, lse, seqlens, B, H, N, d, H, scale, causal ? 1 : 0};
  return run(p, stream, true);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               const int32_t* seqlens, void* stream) {
  fa::FwdParams p{q, k, v, o, lse, seqlens, B, H, N, d, H, scale, causal ? 1 : 0};
  return run(p, stream, false);
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, int causal,
               const int32_t* seqlens, void* stream) {
  fa::FwdParams p{q, k, v, o, lse, seqlens, B, H, N, d, H_kv, scale, causal ? 1 : 0};
  return run(p, stream, true);
}

int fa_fwd_gqa_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                   int B, int H, int H_kv, int N, int d, float scale, int causal,
                   const int32_t* seqlens, void* stream) {
  fa::FwdParams p{q, k, v, o, lse, seqlens, B, H, N, d, H_kv, scale, causal ? 1 : 0};
  return run(p, stream, false);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, float q_descale, float k_descale, float v_descale,
               int causal, const int32_t* seqlens, void* stream) {
  fa::FwdParams p{q, k, v, o, lse, seqlens, B, H, N, d, H_kv, scale, causal ? 1 : 0, q_descale, k_descale, v_descale};
  int st = validate(p);
  if (st != FA_OK) return st;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  for (float s : {q_descale, k_descale, v_descale})
    if (!std::isfinite(s) || !(s > 0.0f)) return FA_ERR_INVALID_ARG;
  st = check_device();
  if (st != FA_OK) return st;
  p.num_cu = current_cus();
  return fa::launch_fwd_fp8(p, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG:
      return "FA_ERR_INVALID_ARG: null tensor, non-positive size, key/value heads not dividing heads, bad scale or size overflow";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: head dimension not supported by this entry point (64, 128, or 256 for the "
             "forward pass), or device is not gfx950";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED: q/k/v/o need 16-byte alignment, lse/seqlens 4-byte";
    case FA_ERR_NO_DEVICE: return "FA_ERR_NO_DEVICE: no current HIP device";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime refused the kernel launch";
    case FA_ERR_SCRATCH_TOO_SMALL:
      return "FA_ERR_SCRATCH_TOO_SMALL: the decode step needs more partial-result memory than the static scratch of "
             "fa_decode_noalloc holds (FA_DECODE_NOALLOC_SCRATCH_BYTES); use fa_decode with a workspace, or fewer "
             "splits or rows per call";
    default: return "unknown fa_status";
  }
}

}  // extern "C"
