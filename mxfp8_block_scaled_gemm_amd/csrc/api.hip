// C ABI of libmxgemm (declared in include/mxgemm.h): host-side validation,
// then one launch per call.  Validation is a pure function of the arguments
// and runs before anything is enqueued ([cute] page, AllReduceMHC checks every
// buffer before its first launch), so a rejected call launches nothing and
// writes nothing.
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "mx_launch.hpp"
#include "mxgemm.h"

namespace {

using mxg::GemmArgs;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 0 = not checked yet, 1 = gfx950, 2 = something else.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

// Is the current device a gfx950?  MXG_FORCE_ARCH overrides the reported
// architecture name (used to exercise the rejection path).
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MXG_ERR_DEVICE;
  const char* forced = std::getenv("MXG_FORCE_ARCH");
  if (forced) return std::strncmp(forced, "gfx950", 6) == 0 ? MXG_OK : MXG_ERR_DEVICE;
  if (dev >= kMaxDevices) return MXG_ERR_DEVICE;
  int state = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXG_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? MXG_OK : MXG_ERR_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? MXG_OK : MXG_ERR_DEVICE; }

int validate_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint8_t* q,
                      const uint8_t* s) {
  if (!x || !q || !s) return MXG_ERR_NULL;
  if (M < 1 || K < 32 || K % 32 != 0 || ld_x < K || M > (int64_t)1 << 31 || K > (int64_t)1 << 30)
    return MXG_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(q) || ld_x % 8 != 0) return MXG_ERR_ALIGN;
  return MXG_OK;
}

int validate_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ld_x,
                  const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q,
                  const uint8_t* w_s, const uint16_t* out, size_t ws_bytes, const void* ws) {
  if (!a_q || !a_s || !w_q || !w_s || !out) return MXG_ERR_NULL;
  if (M < 1 || M > MXG_MAX_ROWS || N < 16 || N % 16 != 0 || K < 128 || K % 128 != 0 ||
      N > (int64_t)1 << 24 || K > (int64_t)1 << 20)
    return MXG_ERR_SHAPE;
  if (N * K > ((int64_t)1 << 31) - 1) return MXG_ERR_SHAPE;
  if (x && (ld_x < K || ld_x * M > ((int64_t)1 << 30))) return MXG_ERR_SHAPE;
  if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(w_q) || !aligned16(w_s) ||
      !aligned16(out) || (x && (!aligned16(x) || ld_x % 8 != 0)))
    return MXG_ERR_ALIGN;
  const size_t need = mxg_gemm_workspace_bytes(M, N, K);
  if (need > 0 && (!ws || ws_bytes < need)) return MXG_ERR_WORKSPACE;
  return MXG_OK;
}

int validate_pack(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                  const uint8_t* wp_q, const uint8_t* wp_s) {
  if (!w_q || !w_s || !wp_q || !wp_s) return MXG_ERR_NULL;
  if (N < 16 || N % 16 != 0 || K < 128 || K % 128 != 0 || N > (int64_t)1 << 24 ||
      K > (int64_t)1 << 20 || N * K > ((int64_t)1 << 31) - 1)
    return MXG_ERR_SHAPE;
  if (!aligned16(w_q) || !aligned16(w_s) || !aligned16(wp_q) || !aligned16(wp_s))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

}  // namespace

extern "C" {

const char* mxg_strerror(int status) {
  switch (status) {
    case MXG_OK: return "success";
    case MXG_ERR_NULL: return "a required pointer is NULL";
    case MXG_ERR_ALIGN: return "a pointer or row stride is not 16-byte aligned";
    case MXG_ERR_SHAPE: return "a size is out of range or sizes are inconsistent";
    case MXG_ERR_WORKSPACE: return "workspace missing or too small";
    case MXG_ERR_DEVICE: return "device is not gfx950, or the kernel launch failed";
    default: return "unknown status";
  }
}

int mxg_version(void) { return 100; }

size_t mxg_gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

int mxfp8_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* q, uint8_t* s,
                   void* stream) {
  int st = validate_quantize(x, M, K, ld_x, q, s);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return launched(mxg::launch_quantize(x, M, K, ld_x, q, s, (hipStream_t)stream));
}

int mxfp8_pack_weights(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                       uint8_t* wp_q, uint8_t* wp_s, void* stream) {
  int st = validate_pack(w_q, w_s, N, K, wp_q, wp_s);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return launched(mxg::launch_pack(w_q, w_s, N, K, wp_q, wp_s, (hipStream_t)stream));
}

int mxfp8_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* x_bf16, int64_t ld_x,
               uint8_t* a_q, uint8_t* a_s, const uint8_t* w_q, const uint8_t* w_s, uint16_t* out,
               void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate_gemm(M, N, K, x_bf16, ld_x, a_q, a_s, w_q, w_s, out, workspace_bytes,
                         workspace);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  GemmArgs a{x_bf16, ld_x, a_q, a_s, w_q, w_s, out, (int)M, (int)N, (int)K};
  return launched(mxg::launch_gemm(a, (hipStream_t)stream));
}

}  // extern "C"
