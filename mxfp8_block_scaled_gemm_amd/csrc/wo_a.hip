// Rotary embedding fused into the MXFP8 quantizer of the grouped WO-A
// projection's input ([o_proj] page, dsv41_o_proj: the fused WO-A kernel
// takes the attention output, the token positions and the layer's
// cos_sin_cache; _can_fuse_wo_a: 448 "nope" + 64 rotary dims per head).
//
// Row m of the input is H heads of D BF16 values at o + m*ld_row + h*ld_head.
// The last D - nope dims of every head are rotated by the angle table row of
// positions[m]: dims (nope + 2i, nope + 2i + 1) form pair i, which turns
// forward by theta_i,
//     y1 = x1 cos - x2 sin,   y2 = x2 cos + x1 sin,
// each product and difference an FP32 operation of its own (the library is
// built without floating-point contraction), the results rounded to BF16 as
// the unfused path stores them.  The flattened row of H*D values, in which
// group g's input is the hpg*D contiguous columns of heads g*hpg..g*hpg+hpg-1,
// is then quantized to MXFP8 exactly as quantize.hip does: 32-dim blocks never
// straddle the rotary boundary (nope % 32 == 0), so rotation and quantization
// fuse per block.
//
// A position outside [0, max_pos) reads angle row 0 (no memory outside the
// table is touched) and sets bit 1 of the error word.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxg {

constexpr int kRopeThreads = 256;              // 64 blocks of 32 per workgroup

__global__ __launch_bounds__(kRopeThreads) void rope_quant_kernel(RopeQuantArgs p) {
  const int nb_head = p.D >> 5;                               // blocks per head
  const int nb = p.H * nb_head;                               // blocks per row
  const int b = blockIdx.x * (kRopeThreads / 4) + (threadIdx.x >> 2);
  const int sub = threadIdx.x & 3;
  const bool valid = b < nb;
  const int h = b / nb_head;
  const int d0 = (b - h * nb_head) * 32 + sub * 8;            // first of this lane's 8 dims
  const int half = (p.D - p.nope) >> 1;
  for (int row = blockIdx.y; row < p.M; row += gridDim.y) {
    v4i v = {0, 0, 0, 0};
    if (valid) v = ld16(p.o + (int64_t)row * p.ld_row + (int64_t)h * p.ld_head + d0);
    if (valid && d0 >= p.nope) {
      int64_t pos = p.positions[row];
      if (pos < 0 || pos >= p.max_pos) {
        if (sub == 0 && b == p.nope / 32) atomicOr(p.error, 2u);
        pos = 0;
      }
      const int i0 = (d0 - p.nope) >> 1;                      // pairs i0 .. i0+3
      const float* cs = p.cos_sin + pos * (2 * half);
      const v4f c = *reinterpret_cast<const v4f*>(cs + i0);
      const v4f s = *reinterpret_cast<const v4f*>(cs + half + i0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x1 = bf16_lo((uint32_t)v[k]), x2 = bf16_hi((uint32_t)v[k]);
        const float y1 = x1 * c[k] - x2 * s[k];
        const float y2 = x2 * c[k] + x1 * s[k];
        v[k] = (int)pk_bf16(y1, y2);
      }
    }
    uint32_t a = halves_max(bf16x2_absmax2(bf16x2_absmax2((uint32_t)v[0], (uint32_t)v[1]),
                                           bf16x2_absmax2((uint32_t)v[2], (uint32_t)v[3])));
    a = quad_max(a);
    const int e = block_exponent(a);
    const BlockScale bs = block_scale(e);
    if (valid) {
      uint2 code;
      code.x = enc4_e4m3((uint32_t)v[0], (uint32_t)v[1], bs);
      code.y = enc4_e4m3((uint32_t)v[2], (uint32_t)v[3], bs);
      const int64_t K = (int64_t)nb * 32;
      *reinterpret_cast<uint2*>(p.q + row * K + b * 32 + sub * 8) = code;
      if (sub == 0) p.s[(int64_t)row * nb + b] = (uint8_t)(e + 127);
    }
  }
}

hipError_t launch_rope_quant(const RopeQuantArgs& a, hipStream_t stream) {
  const int nb = a.H * (a.D >> 5);
  const int gx = (nb + kRopeThreads / 4 - 1) / (kRopeThreads / 4);
  const int gy = a.M < 65535 ? a.M : 65535;
  hipLaunchKernelGGL(rope_quant_kernel, dim3(gx, gy), dim3(kRopeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mxg
