// Host entry points of the C interface declared in include/fa.h: argument
// validation, the device check and dispatch to the kernel launchers.  Nothing
// here allocates memory or synchronises the device.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa.h"
#include "fa_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// Per-device verdict of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return FA_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  int v = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FA_ERR_NO_DEVICE;
    }
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? FA_OK : FA_ERR_UNSUPPORTED;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int validate(const fa::FwdParams& p) {
  if (!p.q || !p.k || !p.v || !p.o) return FA_ERR_INVALID_ARG;
  if (p.B < 1 || p.H < 1 || p.N < 1) return FA_ERR_INVALID_ARG;
  if (p.Hkv < 1 || p.Hkv > p.H || p.H % p.Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(p.scale) || !(p.scale > 0.0f)) return FA_ERR_INVALID_ARG;
  if (p.d != 64 && p.d != 128) return FA_ERR_UNSUPPORTED;
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

int run(const fa::FwdParams& p, void* stream, bool bf16) {
  int st = validate(p);
  if (st != FA_OK) return st;
  st = check_device();
  if (st != FA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = bf16 ? fa::launch_fwd_bf16(p, s) : fa::launch_fwd_f32(p, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

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

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARG:
      return "FA_ERR_INVALID_ARG: null tensor, non-positive size, key/value heads not dividing heads, bad scale or size overflow";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension not 64/128, or device is not gfx950";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED: q/k/v/o need 16-byte alignment, lse/seqlens 4-byte";
    case FA_ERR_NO_DEVICE: return "FA_ERR_NO_DEVICE: no current HIP device";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: the HIP runtime refused the kernel launch";
    default: return "unknown fa_status";
  }
}

}  // extern "C"
