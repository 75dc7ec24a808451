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
  // MXFP8 activations read with row stride lda bytes (scales: lda / 32).
  // Grouped GEMM (group_tiles > 0): weight tile t (rows [16t, 16t+16))
  // belongs to group t / group_tiles, whose activations start a_group bytes
  // (scales: a_group / 32) further along each row.  Only with x == nullptr.
  int64_t lda = 0;       // 0: K
  int group_tiles = 0;
  int64_t a_group = 0;
};

hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                           uint8_t* q, uint8_t* s, hipStream_t stream);

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);

// Rotary embedding + MXFP8 of the grouped WO-A input (wo_a.hip).
struct RopeQuantArgs {
  const uint16_t* o;          // BF16, head h of row m at o + m*ld_row + h*ld_head
  int64_t ld_row, ld_head;
  const int64_t* positions;   // [M]
  const float* cos_sin;       // FP32 [max_pos, D - nope]: cos, then sin
  int64_t max_pos;
  uint8_t* q;                 // out: codes [M, H*D]
  uint8_t* s;                 // out: scale bytes [M, H*D/32]
  uint32_t* error;            // bit 1 set when a position is out of range
  int M, H, D, nope;
};

hipError_t launch_rope_quant(const RopeQuantArgs& a, hipStream_t stream);

hipError_t launch_pack(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                       uint8_t* wp_q, uint8_t* wp_s, hipStream_t stream);

}  // namespace mxg
