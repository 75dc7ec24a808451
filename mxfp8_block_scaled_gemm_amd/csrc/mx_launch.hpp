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
  const uint8_t* w_q;    // weight codes, N*K bytes (packed, or row-major with w_rm)
  const uint8_t* w_s;    // weight scale bytes, N*K/32 bytes
  uint16_t* out;         // BF16 [M, N]
  int M, N, K;
  // MXFP8 activations read with row stride lda bytes (scales: lda / 32).
  // Grouped GEMM (group_tiles > 0): weight tile t (rows [16t, 16t+16))
  // belongs to group t / group_tiles, whose activations start a_group bytes
  // (scales: a_group / 32) further along each row.  Only with x == nullptr.
  int64_t lda = 0;       // 0: K
  int group_tiles = 0;
  int64_t a_group = 0;
  // Workspace of a K-split plan: tile-group counters at ctr (zero on entry,
  // zero again on exit) and FP32 partial tiles at part.  May be null when
  // gemm_workspace_bytes() is 0 for the shape.
  uint32_t* ctr = nullptr;
  float* part = nullptr;
  int P = 1, Sp = 0;     // K split of the 2D kernel (set by the launcher)
  // Activation scales in 128 x 4 tiles instead of row-major (MXFP8 input,
  // no grouping, lda == K).
  bool a_sf128 = false;
  // Weights row-major ([N, K] codes, [N, K/32] scales) instead of packed.
  bool w_rm = false;
  // M <= 16 kernel: workgroups per 16-row weight tile (1, 2 or 4; set by the
  // launcher).
  int rsplit = 1;
  // BF16 input only: RMS-normalise each row of x (gain norm_w [K], BF16;
  // norm_eps inside the square root) before the quantize, as
  // launch_rmsnorm_quantize does; the normalised BF16 rows are also written
  // to norm_y [M, K] when it is non-null.
  const uint16_t* norm_w = nullptr;
  float norm_eps = 0.f;
  uint16_t* norm_y = nullptr;
  // Also write the MXFP8 of output columns [0, qn) (qn % 32 == 0, qn <= N),
  // quantized from the BF16 outputs as launch_quantize would: codes to
  // out_q [M, qn], scale bytes to out_s [M, qn / 32].  Only the 2D kernel
  // with two or more weight tiles per workgroup and at most 64 rows does it;
  // launch_gemm reports whether the call did.
  uint8_t* out_q = nullptr;
  uint8_t* out_s = nullptr;
  int qn = 0;
};

// Bytes of FP32 partials the GEMM of this shape needs (0: no K split).
size_t gemm_partial_bytes(int M, int N, int K, int group_tiles = 0);

// Workspace layout.  The first 64 KiB are the counter region:
//   word kCtrError (byte 20)  error word: an in-kernel wait that expired, or a
//                             WO-A position outside its angle table
//   kGemmCtrOffset ..         K-split tile counters (one word per tile group)
// Every counter is back at zero when a call ends, so calls of any shape can
// share one zero-filled workspace in turn.  K-split FP32 partial sums (and
// WO-A's rotated input) follow from kGemmPartOffset; they need no clearing.
constexpr int kCtrError = 5;
constexpr size_t kCtrBytes = 8192;            // smallest workspace any call needs
constexpr size_t kCtrRegionBytes = 64 * 1024;
constexpr size_t kGemmCtrOffset = 8192;
constexpr size_t kGemmPartOffset = kCtrRegionBytes;

hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                           uint8_t* q, uint8_t* s, hipStream_t stream);

// *quantized_out (when given) is set to whether out_q / out_s were written.
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream, bool* quantized_out = nullptr);

// 64 x 64-tile GEMM for more than 64 rows (gemm_big.hip): MXFP8 input,
// N % 64 == 0, row-major activation scales.
bool gemm_big_fits(const GemmArgs& a);
hipError_t launch_gemm_big(const GemmArgs& a, int cus, hipStream_t stream);
// The wide form of the same (K split across waves, NT tiles per workgroup):
// whether it takes the shape, the tile count whose grid fits one round on
// `cus` CUs (0: none), and the launch (nt 0: that count).
bool gemm_wide_fits(const GemmArgs& a);
int gemm_wide_tiles(const GemmArgs& a, int cus);
hipError_t launch_gemm_wide(const GemmArgs& a, int cus, hipStream_t stream, int nt = 0);

// RMSNorm + MXFP8 of BF16 rows (rmsnorm.hip); layout 1 = 128 x 4 scale tiles.
hipError_t launch_rmsnorm_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                                   const uint16_t* w, float eps, uint16_t* y, int64_t ld_y,
                                   uint8_t* q, uint8_t* s, int layout, hipStream_t stream);

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
