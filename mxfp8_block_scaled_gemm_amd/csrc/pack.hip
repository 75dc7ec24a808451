// One-time repack of an MXFP8 weight into the tile order the GEMM streams.
//
// The GEMM feeds 16 weight rows x 128 K to each scaled MFMA (the weight is
// the A operand; [mxfp8] page, launch_low_latency computes out^T).  In the
// packed order the 2 KiB of codes and the 64 scale bytes of one (16-row tile,
// 128-K step) are contiguous and already in lane order, so a wave reads its
// operands as two fully contiguous 1 KiB loads plus one 64-byte load.
//
//   codes:  wp[((t*S + s)*2 + h)*1024 + 16*l + b] = W[16t + l%16][128s + 64h + 16(l/16) + b]
//   scales: wps[(t*S + s)*64 + l]                 = Ws[16t + l%16][4s + l/16]
// with S = K/128, t < N/16, s < S, h < 2, lane l < 64, b < 16.  A pure
// permutation of the bytes of [N, K] codes and [N, K/32] scales.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxg {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ w_q,
                                                   const uint8_t* __restrict__ w_s, int64_t N,
                                                   int64_t K, uint8_t* __restrict__ wp_q,
                                                   uint8_t* __restrict__ wp_s) {
  const int64_t S = K >> 7;
  const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // 16-byte output chunk
  const int64_t nchunks = (N / 16) * S * 128;
  if (chunk >= nchunks) return;
  const int l = (int)(chunk & 63);
  const int h = (int)((chunk >> 6) & 1);
  const int64_t ts = chunk >> 7;                                         // t * S + s
  const int64_t t = ts / S, s = ts % S;
  const int64_t row = 16 * t + (l & 15);
  st16(wp_q + chunk * 16, ld16(w_q + row * K + 128 * s + 64 * h + 16 * (l >> 4)));
  if (h == 0) wp_s[ts * 64 + l] = w_s[row * (K >> 5) + 4 * s + (l >> 4)];
}

hipError_t launch_pack(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                       uint8_t* wp_q, uint8_t* wp_s, hipStream_t stream) {
  const int64_t nchunks = (N / 16) * (K / 128) * 128;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, stream,
                     w_q, w_s, N, K, wp_q, wp_s);
  return hipGetLastError();
}

}  // namespace mxg
