// RMSNorm + MXFP8 quantize of BF16 rows in one launch ([step] page:
// AttentionStep.run normalises the leading columns of fused_wqa_wkv's output
// in _split_qkv_and_norm before wq_b reads them as MXFP8; [cute] page:
// AllReduceMHC normalises its collapse with norm_weight / norm_eps and can
// write the result as MXFP8 with swizzled 128x4 scales).
//
// One workgroup per row: each thread owns whole 32-element blocks (64 bytes
// of x and of the gain, four 16-byte loads each), sums their squares in
// FP32, the row's sum comes from a wave reduction plus one LDS exchange,
// then each thread normalises its blocks, rounds them to BF16 and quantizes
// the BF16 values as mxfp8_quantize does (integer amax of the BF16 bits,
// E8M0 exponent, hardware RNE convert of y / 2^e).  The work is a few KB
// per row: launch latency, not bandwidth, bounds it.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxg {

constexpr int kNormThreads = 256;
constexpr int kNormBlocksPerThread = 2;   // K <= 256 * 2 * 32 = 16384

// Byte offset of the scale of row m, block b in 128 x 4 tiles: tiles run
// along K first (kb4 = K/128 tiles per 128 rows), 512 bytes each, and inside
// a tile row m sits at (m % 32) * 16 + ((m % 128) / 32) * 4, block b at b % 4.
__device__ __forceinline__ int64_t scale_off_128x4(int64_t m, int64_t b, int64_t kb4) {
  return ((m >> 7) * kb4 + (b >> 2)) * 512 + (m & 31) * 16 + ((m & 127) >> 5) * 4 + (b & 3);
}

__global__ __launch_bounds__(kNormThreads) void rmsnorm_quant_kernel(
    const uint16_t* __restrict__ x, int64_t K, int64_t ld_x, const uint16_t* __restrict__ w,
    float eps, uint16_t* __restrict__ y, int64_t ld_y, uint8_t* __restrict__ q,
    uint8_t* __restrict__ s, int layout) {
  __shared__ float s_sum[kNormThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m = blockIdx.x, KB = K >> 5;
  const uint16_t* xr = x + m * ld_x;

  v4i xv[kNormBlocksPerThread][4], wv[kNormBlocksPerThread][4];
#pragma unroll
  for (int i = 0; i < kNormBlocksPerThread; ++i) {
    const int64_t b = tid + (int64_t)kNormThreads * i;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xv[i][k] = b < KB ? ld16(xr + b * 32 + 8 * k) : v4i{0, 0, 0, 0};
      wv[i][k] = b < KB ? ld16(w + b * 32 + 8 * k) : v4i{0, 0, 0, 0};
    }
  }

  // Sum of squares (FP32, each product and sum rounded on its own).
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormBlocksPerThread; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t u = (uint32_t)xv[i][k][h];
        const float a = bf16_lo(u), c = bf16_hi(u);
        ss = ss + a * a;
        ss = ss + c * c;
      }
  ss = wave_sum(ss);
  if (lane == 0) s_sum[wave] = ss;
  __syncthreads();
  float tot = s_sum[0];
#pragma unroll
  for (int i = 1; i < kNormThreads / 64; ++i) tot = tot + s_sum[i];
  const float r = 1.0f / __builtin_sqrtf(tot / (float)K + eps);

#pragma unroll
  for (int i = 0; i < kNormBlocksPerThread; ++i) {
    const int64_t b = tid + (int64_t)kNormThreads * i;
    if (b >= KB) continue;
    // y = BF16(x * r * w), packed two per word in element order.
    uint32_t yw[16];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t xu = (uint32_t)xv[i][k][h], wu = (uint32_t)wv[i][k][h];
        const float lo = (bf16_lo(xu) * r) * bf16_lo(wu);
        const float hi = (bf16_hi(xu) * r) * bf16_hi(wu);
        yw[4 * k + h] = pk_bf16(lo, hi);
      }
    uint32_t amax = 0;
#pragma unroll
    for (int k = 0; k < 16; k += 2) amax = bf16x2_absmax2(amax, bf16x2_absmax2(yw[k], yw[k + 1]));
    const int e = block_exponent(halves_max(amax));
    const BlockScale bs = block_scale(e);
    uint32_t c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = enc4_e4m3(yw[2 * k], yw[2 * k + 1], bs);
    uint8_t* qo = q + m * K + b * 32;
    st16(qo, v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]});
    st16(qo + 16, v4i{(int)c[4], (int)c[5], (int)c[6], (int)c[7]});
    if (y) {
      uint16_t* yo = y + m * ld_y + b * 32;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        st16(yo + 8 * k, v4i{(int)yw[4 * k], (int)yw[4 * k + 1], (int)yw[4 * k + 2],
                             (int)yw[4 * k + 3]});
    }
    const int64_t so = layout == 1 ? scale_off_128x4(m, b, K >> 7) : m * KB + b;
    s[so] = (uint8_t)(e + 127);
  }
}

hipError_t launch_rmsnorm_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                   const uint16_t* w, float eps, uint16_t* y, int64_t ld_y,
                                   uint8_t* q, uint8_t* s, int layout, hipStream_t stream) {
  if (K > (int64_t)kNormThreads * kNormBlocksPerThread * 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_quant_kernel, dim3((unsigned)M), dim3(kNormThreads), 0, stream, x, K,
                     ld_x, w, eps, y, ld_y, q, s, layout);
  return hipGetLastError();
}

}  // namespace mxg
