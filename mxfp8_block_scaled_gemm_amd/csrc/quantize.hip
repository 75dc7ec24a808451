// BF16 -> MXFP8 activation quantizer ([mxfp8] page: pinned_mm and wide_mm
// quantize a BF16 input with mxfp8_e4m3_quantize before the GEMM; [cute] page,
// AllReduceMHC: mxfp8_out receives the layer input as MXFP8).
//
// Four lanes own one 32-element block: each loads 8 BF16 values (16 bytes,
// so a wave reads 1 KiB contiguous per row segment), the block amax is an
// integer max over BF16 magnitude bits reduced with two lane shuffles, and
// each lane writes its 8 codes as one 8-byte store.  Bit-exact by
// construction: the exponent is integer arithmetic and the only rounding is
// the hardware RNE convert of x / 2^e.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxg {

constexpr int kQuantThreads = 256;              // 64 blocks of 32 per workgroup

__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ld_x,
    uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int64_t nb = K >> 5;                                  // blocks per row
  const int64_t b = (int64_t)blockIdx.x * (kQuantThreads / 4) + (threadIdx.x >> 2);
  const int sub = threadIdx.x & 3;
  const bool valid = b < nb;
  for (int64_t row = blockIdx.y; row < M; row += gridDim.y) {
    v4i v = {0, 0, 0, 0};
    if (valid) v = ld16(x + row * ld_x + b * 32 + sub * 8);
    uint32_t a = halves_max(bf16x2_absmax2(bf16x2_absmax2((uint32_t)v[0], (uint32_t)v[1]),
                                           bf16x2_absmax2((uint32_t)v[2], (uint32_t)v[3])));
    a = quad_max(a);
    const int e = block_exponent(a);
    const BlockScale bs = block_scale(e);
    if (valid) {
      uint2 c;
      c.x = enc4_e4m3((uint32_t)v[0], (uint32_t)v[1], bs);
      c.y = enc4_e4m3((uint32_t)v[2], (uint32_t)v[3], bs);
      *reinterpret_cast<uint2*>(q + row * K + b * 32 + sub * 8) = c;
      if (sub == 0) s[row * nb + b] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                           uint8_t* q, uint8_t* s, hipStream_t stream) {
  const int64_t nb = K >> 5;
  const int64_t gx = (nb + kQuantThreads / 4 - 1) / (kQuantThreads / 4);
  const int64_t gy = M < 65535 ? M : 65535;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(kQuantThreads), 0,
                     stream, x, M, K, ld_x, q, s);
  return hipGetLastError();
}

}  // namespace mxg
