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
  const uint8_t* w_q;    // weight codes [N, K]
  const uint8_t* w_s;    // weight scale bytes [N, K/32]
  uint16_t* out;         // BF16 [M, N]
  int M, N, K;
};

hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                           uint8_t* q, uint8_t* s, hipStream_t stream);

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);

}  // namespace mxg
