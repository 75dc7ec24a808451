// HBM read ceiling of a single launch: reads the same bytes the small-row
// GEMM's weight stream reads, with the same access pattern (one workgroup of
// 16 waves per 16-row weight tile, every wave issuing all of its 2 KiB steps
// up front as non-temporal 16-byte buffer loads), and does nothing else.
// Its per-launch time is the floor any kernel streaming those bytes in one
// launch meets on this machine: launch and drain included, no arithmetic,
// no activations, no output.  The loaded words are folded into one value
// that is stored only when it equals a pattern the caller never writes, so
// no load can be dropped and nothing is written.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxg {

constexpr int kProbeWaves = 16;
constexpr int kProbeSlots = 4;    // steps per wave: tiles up to 128 KiB

__global__ __launch_bounds__(kProbeWaves * 64) void hbm_read_kernel(const uint8_t* src,
                                                                     uint32_t tile_bytes,
                                                                     uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const auto r = make_rsrc(src + (size_t)blockIdx.x * tile_bytes, tile_bytes);
  v4i v[2 * kProbeSlots];
#pragma unroll
  for (int j = 0; j < kProbeSlots; ++j) {
    const uint32_t step = (uint32_t)(wave + kProbeWaves * j) * 2048u;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      v[2 * j + h] = buf_ld16_nt(r, step + 1024u * h + 16u * lane);
  }
  v4i acc = v[0];
#pragma unroll
  for (int i = 1; i < 2 * kProbeSlots; ++i) acc ^= v[i];
  const uint32_t x = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  if (x == 0x9E3779B9u && acc[0] == 0x7F4A7C15) sink[0] = x;
}

hipError_t launch_hbm_read(const uint8_t* src, int tiles, uint32_t tile_bytes, uint32_t* sink,
                           hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(tiles), dim3(kProbeWaves * 64), 0, stream, src,
                     tile_bytes, sink);
  return hipGetLastError();
}

}  // namespace mxg
