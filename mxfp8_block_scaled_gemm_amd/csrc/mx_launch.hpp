// Host-side launchers of the libmxgemm kernels.  Each takes already
// validated arguments (the C ABI in api.hip validates) and only enqueues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

struct GemmArgs {
  const uint16_t* x;     // BF16 activations to quantize in-kernel, or nullptr
  int64_t ld_x;          // row stride of x (elements)
  uint8_t* a_q;          // MXFP8 activation codes [M, K]  (written when x != nullptr)
  uint8_t* a_s;          // activation scale bytes [M, K/32] (written when x != nullptr)
  const uint8_t* w_q;    // packed weight codes (pack.hip order), N*K bytes
  const uint8_t* w_s;    // packed weight scale bytes, N*K/32 bytes
  uint16_t* out;         // BF16 [M, N]
  int M, N, K;
};

hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                           uint8_t* q, uint8_t* s, hipStream_t stream);

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);

hipError_t launch_pack(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                       uint8_t* wp_q, uint8_t* wp_s, hipStream_t stream);

}  // namespace mxg
