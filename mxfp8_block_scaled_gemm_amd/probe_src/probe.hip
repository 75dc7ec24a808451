// HBM read ceiling of a single launch: reads a packed MXFP8 weight exactly as
// the small-row GEMM's weight stream does (one workgroup of 16 waves per
// 16-row tile; every wave issues all of its 128-wide K steps up front, each
// step two non-temporal 16-byte code loads and one scale-byte load per lane)
// and does nothing else.  Its per-launch time is the floor any kernel
// streaming that weight in one launch meets on this machine: launch and
// drain included, no arithmetic, no activations, no output.  The loaded
// words are folded into one value that is stored only when it equals a
// pattern no weight produces by accident, so no load can be dropped and
// nothing is written.
//
// A measurement aid, built into its own library (libmxprobe.so) beside the
// GEMM library and not part of its interface.
#include <cstdlib>
#include <cstring>

#include "mx_device.hpp"
#include "mxgemm.h"
#include "mxprobe.h"

namespace mxg {

constexpr int kProbeWaves = 16;
constexpr int kProbeSlots = 4;    // steps per wave: K up to 8192

__global__ __launch_bounds__(kProbeWaves * 64) void hbm_read_kernel(const uint8_t* w_q,
                                                                     const uint8_t* w_s,
                                                                     int steps, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int t = blockIdx.x;
  const auto rq = make_rsrc(w_q + (size_t)t * steps * 2048, (uint32_t)(steps * 2048));
  const auto rs = make_rsrc(w_s + (size_t)t * steps * 64, (uint32_t)(steps * 64));
  v4i lo[kProbeSlots], hi[kProbeSlots];
  uint32_t sc[kProbeSlots];
#pragma unroll
  for (int j = 0; j < kProbeSlots; ++j) {
    const int s = wave + kProbeWaves * j;
    const bool ok = s < steps;
    lo[j] = buf_ld16_nt(rq, ok ? (uint32_t)(s * 2048 + 16 * lane) : kOutOfRange);
    hi[j] = buf_ld16_nt(rq, ok ? (uint32_t)(s * 2048 + 1024 + 16 * lane) : kOutOfRange);
    sc[j] = buf_ld8(rs, ok ? (uint32_t)(s * 64 + lane) : kOutOfRange);
  }
  v4i acc = lo[0] ^ hi[0];
  uint32_t a = sc[0];
#pragma unroll
  for (int j = 1; j < kProbeSlots; ++j) {
    acc ^= lo[j] ^ hi[j];
    a ^= sc[j];
  }
  const uint32_t x = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) ^ (a << 24);
  if (x == 0x9E3779B9u && acc[0] == 0x7F4A7C15) sink[0] = x;
}

}  // namespace mxg

extern "C" int mxg_hbm_read_probe(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                                  uint32_t* sink, void* stream) {
  if (!w_q || !w_s || !sink) return MXG_ERR_NULL;
  if (N < 16 || N % 16 != 0 || N > ((int64_t)1 << 24) || K < 128 || K % 128 != 0 ||
      K > 128 * mxg::kProbeWaves * mxg::kProbeSlots)
    return MXG_ERR_SHAPE;
  const auto addr = [](const void* p) { return reinterpret_cast<uintptr_t>(p); };
  if ((addr(w_q) & 15u) || (addr(w_s) & 15u) || (addr(sink) & 3u)) return MXG_ERR_ALIGN;
  // gfx950 only (MXG_FORCE_ARCH stands in for the device's name in tests)
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MXG_ERR_DEVICE;
  if (const char* forced = std::getenv("MXG_FORCE_ARCH")) {
    if (std::strncmp(forced, "gfx950", 6) != 0) return MXG_ERR_DEVICE;
  } else {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess ||
        std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return MXG_ERR_DEVICE;
  }
  hipLaunchKernelGGL(mxg::hbm_read_kernel, dim3((unsigned)(N / 16)), dim3(mxg::kProbeWaves * 64),
                     0, (hipStream_t)stream, w_q, w_s, (int)(K / 128), sink);
  return hipGetLastError() == hipSuccess ? MXG_OK : MXG_ERR_DEVICE;
}
