/*
 * mxgemm.h -- C ABI of libmxgemm: small-row MXFP8 block-scaled GEMMs for the
 * attention projections of a decode step, on AMD MI355X (gfx950).
 *
 * Sources ("pages") are the vLLM API documentation pages
 *   [mxfp8]  vllm.models.deepseek_v41.nvidia.specialized_decode.attention.mxfp8
 *   [step]   vllm.models.deepseek_v41.nvidia.specialized_decode.attention.step
 *   [cute]   vllm.models.deepseek_v41.nvidia.ops.cute_dsl
 *   [o_proj] vllm.models.deepseek_v41.nvidia.ops.o_proj
 *
 * Data formats
 *   MXFP8 tensor  E4M3 ("FN": bias 7, max 448, no infinity) element codes, one
 *                 byte each, row-major [rows, K], plus one UE8M0 scale byte
 *                 (value 2^(byte-127)) per 32 consecutive K elements, row-major
 *                 [rows, K/32].  ([mxfp8] compile_low_latency: Float8E4M3FN
 *                 operands, Float8E8M0FNU scales, sf_vec_size 32.)
 *   weights       a column-major K x N matrix on the [mxfp8] page
 *                 (launch_low_latency), i.e. N rows of K contiguous codes:
 *                 w_q [N, K], w_s [N, K/32] here (MXG_WEIGHTS_ROW_MAJOR).
 *                 The GEMMs read that layout as it is, or the same bytes
 *                 once repacked by mxfp8_pack_weights into the order their
 *                 kernels stream (MXG_WEIGHTS_PACKED, the default), as a
 *                 layer preprocesses its weights once for its GEMM backend.
 *                 On MI355X the packed layout streams 25-40 % faster.
 *   BF16          uint16_t bit patterns.  Outputs are BF16 [M, N] row-major,
 *                 each element the FP32-accumulated sum rounded to nearest even,
 *                 with no scale and no bias ([mxfp8] compile_low_latency).
 *
 * Conventions (all entry points)
 *   - Every buffer is device memory owned by the caller; the library allocates
 *     nothing and keeps no state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream) and the call returns without waiting for it.
 *   - Arguments are validated on the host before anything is launched
 *     ([cute] AllReduceMHC validates every buffer before its first launch):
 *     on any error nothing is launched and no output is written.
 *   - Device pointers must be 16-byte aligned, and row strides must keep every
 *     row 16-byte aligned ([mxfp8] launch_low_latency passes 16-byte aligned
 *     operand pointers, and a 32-byte aligned weight scale pointer, which
 *     meets this).
 *   - Row counts: 1 <= M <= MXG_MAX_ROWS for the chain and WO-A ([mxfp8]:
 *     the low-latency kernel covers up to 48 rows with 16-, 32- or 48-row
 *     activation tiles; more rows go to another kernel), and up to
 *     MXG_MAX_GEMM_ROWS for mxfp8_gemm / mxfp8_gemm_ex, which serve rows
 *     above 48 as 64-row blocks of another kernel shape.
 *   - K must be a multiple of 128 (at most MXG_MAX_K) and N a multiple of 16
 *     for the GEMMs ([mxfp8] mxfp8_eligible requires the weight's K to be a
 *     multiple of 128).
 *   - Inputs holding NaN/Inf (BF16), the E4M3 NaN codes 0x7F/0xFF or the
 *     E8M0 NaN byte 0xFF are outside the contract: the results are unspecified
 *     (the hardware propagates NaN).
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define MXG_OK 0
#define MXG_ERR_NULL 1      /* a required pointer is NULL                      */
#define MXG_ERR_ALIGN 2     /* a pointer or row stride is not 16-byte aligned   */
#define MXG_ERR_SHAPE 3     /* a size is out of range or sizes are inconsistent */
#define MXG_ERR_WORKSPACE 4 /* workspace missing or smaller than required       */
#define MXG_ERR_DEVICE 5    /* current device is not gfx950, or a launch failed */

#define MXG_MAX_ROWS 48       /* rows of the chain, WO-A and the low-latency GEMM range */
#define MXG_MAX_GEMM_ROWS 256 /* rows of mxfp8_gemm / mxfp8_gemm_ex (above 48: 64-row blocks) */
#define MXG_MAX_K 16384     /* largest contraction of the GEMM entry points */

/* Human-readable text of a status code (static storage; never NULL). */
const char *mxg_strerror(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int mxg_version(void);

/*
 * mxfp8_quantize -- BF16 -> MXFP8 ([mxfp8] pinned_mm and wide_mm quantize a
 * BF16 input with mxfp8_e4m3_quantize; [cute] AllReduceMHC's mxfp8_out
 * receives the layer input as MXFP8).
 *
 * For each row m and each 32-element block b of columns [0, K):
 *   amax = max |x|;  e = clamp(floor(log2 amax) - 8, -127, 127), and e = -127
 *   when amax = 0;  s[m, b] = e + 127;  q[m, k] = E4M3(x[m, k] * 2^-e), rounded
 *   to nearest even and saturated to +-448, sign kept.
 * (The pages do not print the scale rule; this is the benchmark's rule,
 * 2^(floor(log2 amax) - 8), 8 being E4M3's largest exponent.)
 *
 *   x     BF16 [M, ld_x] (reads columns [0, K) of each row)
 *   M     rows, >= 1 (any count: weights may be quantized with this too)
 *   K     columns to quantize, multiple of 32
 *   ld_x  row stride of x in elements, >= K, multiple of 8
 *   q     out: E4M3 codes [M, K]
 *   s     out: scale bytes [M, K/32]
 * Codes and scales are a deterministic function of the BF16 bits.
 */
int mxfp8_quantize(const uint16_t *x, int64_t M, int64_t K, int64_t ld_x,
                   uint8_t *q, uint8_t *s, void *stream);

/*
 * Layouts of an MXFP8 weight's bytes (mxg_weight.layout, mxfp8_gemm_ex).
 * Both hold the same N*K code bytes and N*K/32 scale bytes, and give results
 * equal bit for bit.  A 16-row x 128-K step of the row-major layout is 16
 * rows of 128 bytes, so each of a wave's two 16-byte-per-lane code loads
 * reads 64 bytes of 16 rows, where a packed step is 2 KiB in lane order.
 */
#define MXG_WEIGHTS_PACKED 0    /* mxfp8_pack_weights order (fastest)   */
#define MXG_WEIGHTS_ROW_MAJOR 1 /* [N, K] codes, [N, K/32] scales       */

/* Layouts of MXFP8 scale bytes written by mxfp8_rmsnorm_quantize. */
#define MXG_SCALES_ROW_MAJOR 0 /* [M, K/32], row-major                          */
#define MXG_SCALES_128X4 1     /* 128 x 4 tiles ([mxfp8] module text: F8_128x4) */

/* Bytes of a 128x4-tiled scale buffer for M rows of K columns:
 * ceil(M/128)*128 rows times ceil(K/128)*4 scale columns. */
size_t mxg_scale_bytes_128x4(int64_t M, int64_t K);

/*
 * mxfp8_rmsnorm_quantize -- RMSNorm of BF16 rows followed by the MXFP8
 * quantize of the normalised rows, in one launch ([step] AttentionStep.run:
 * _split_qkv_and_norm normalises the leading columns of fused_wqa_wkv's
 * output before they go to wq_b as MXFP8; [cute] AllReduceMHC: norm_weight
 * and norm_eps, with mxfp8_out receiving the normalised layer input as MXFP8
 * with swizzled 128x4 scales).
 *
 * For each row m:
 *   r = 1 / sqrt(mean_{k<K} x[m,k]^2 + eps)  (FP32, sum in any order)
 *   y[m,k] = BF16_RNE(x[m,k] * r * w[k])      (FP32 products)
 *   (q, s) = the quantize of mxfp8_quantize applied to the BF16 row y[m, :].
 * The pages print no formula; the mean runs over the K normalised columns
 * and eps sits inside the square root.
 *
 *   x             BF16 [M, ld_x]; columns [0, K) of each row are normalised
 *   M             rows, 1 <= M <= 65535
 *   K             columns, multiple of 128, <= MXG_MAX_K
 *   ld_x          row stride of x in elements, >= K, multiple of 8
 *   w             BF16 [K] per-column gain (norm weight)
 *   eps           >= 0, finite
 *   y             out (optional, NULL = not written): BF16 [M, ld_y]
 *   ld_y          row stride of y in elements, >= K, multiple of 8
 *   q             out: E4M3 codes [M, K]
 *   s             out: scale bytes, laid out per scale_layout:
 *                 MXG_SCALES_ROW_MAJOR: [M, K/32];
 *                 MXG_SCALES_128X4: mxg_scale_bytes_128x4(M, K) bytes, the
 *                 scale of row m, block b at
 *                   ((m/128)*(K/128) + b/4)*512 + (m%32)*16 + ((m%128)/32)*4 + b%4;
 *                 padding bytes are not written (zero them once, as the
 *                 pages' MXFP8 buffers are zero-allocated)
 * Codes and scales are a deterministic function of the BF16 row y.  Status
 * as above; nothing is launched or written on an error.
 */
int mxfp8_rmsnorm_quantize(const uint16_t *x, int64_t M, int64_t K, int64_t ld_x,
                           const uint16_t *w, float eps, uint16_t *y, int64_t ld_y,
                           uint8_t *q, uint8_t *s, int32_t scale_layout, void *stream);

/*
 * mxfp8_pack_weights -- one-time repack of an MXFP8 weight into the tile
 * order the GEMM kernels stream.  A pure permutation of bytes:
 *   wp_q[((t*S + s)*2 + h)*1024 + 16*l + b] = w_q[16t + l%16][128s + 64h + 16(l/16) + b]
 *   wp_s[(t*S + s)*64 + l]                  = w_s[16t + l%16][4s + l/16]
 * with S = K/128, tile t < N/16, step s < S, half h < 2, lane l < 64,
 * byte b < 16: the 2 KiB of codes and 64 scale bytes that one 16-row x 128-K
 * scaled MFMA consumes are contiguous, in the order its lanes hold them.
 *
 *   w_q, w_s    row-major MXFP8 weight, [N, K] codes and [N, K/32] scales
 *   N, K        N % 16 == 0, K % 128 == 0
 *   wp_q, wp_s  out: N*K and N*K/32 bytes (must not overlap the inputs)
 */
int mxfp8_pack_weights(const uint8_t *w_q, const uint8_t *w_s, int64_t N, int64_t K,
                       uint8_t *wp_q, uint8_t *wp_s, void *stream);

/*
 * mxfp8_gemm -- out = dequant(a) . dequant(w)^T  ([mxfp8] launch_low_latency:
 * out = a (rows x K) times the [K, N] weight; the kernel there computes out^T
 * with the weight's N as its M, as this one does).  FP32 accumulation, BF16
 * output, no scale, no bias.
 *
 *   M, N, K   1 <= M <= MXG_MAX_GEMM_ROWS, N % 16 == 0, K % 128 == 0,
 *             K <= MXG_MAX_K.  Up to 48 rows the low-latency kernels serve
 *             the call; above 48 ([mxfp8] module text: more rows go to
 *             another kernel there) it runs as a grid of 64-row blocks over
 *             the same weight in one launch, with BF16 input quantized by
 *             its own launch first
 *   x_bf16    NULL: a_q/a_s are inputs.  Non-NULL: BF16 [M, ld_x] activations
 *             that the kernel quantizes itself (as mxfp8_quantize does) and
 *             whose codes/scales it also WRITES to a_q/a_s (the pages'
 *             wide_mm quantizes a BF16 x before its GEMM; here both run in
 *             one launch when M*K <= 65536, else a quantize launch runs
 *             first on the same stream).
 *   ld_x      row stride of x_bf16 in elements (ignored when x_bf16 is NULL)
 *   a_q, a_s  MXFP8 activations [M, K] / [M, K/32]
 *   w_q, w_s  MXFP8 weight [N, K] / [N, K/32], packed by mxfp8_pack_weights
 *             (mxfp8_gemm_ex also reads it unpacked)
 *   out       BF16 [M, N]
 *   workspace, workspace_bytes
 *             caller-owned device scratch of at least mxg_gemm_workspace_bytes()
 *             bytes: cross-workgroup counters and K-split partial sums.  It
 *             must be zero-filled once when allocated; every call leaves its
 *             counters (the first 64 KiB) at zero again, and the partial
 *             sums after them need no clearing, so calls of any shape can
 *             share one workspace in turn.  Calls that share a workspace must
 *             not overlap (issue them on one stream).
 *
 * Small-row GEMMs are bound by the weight stream from HBM; the library picks
 * the kernel and the K split per shape.  Results do not depend on the choice
 * beyond FP32 summation order, and are deterministic for a given shape.
 */
int mxfp8_gemm(int64_t M, int64_t N, int64_t K, const uint16_t *x_bf16,
               int64_t ld_x, uint8_t *a_q, uint8_t *a_s, const uint8_t *w_q,
               const uint8_t *w_s, uint16_t *out, void *workspace,
               size_t workspace_bytes, void *stream);

/* Workspace bytes mxfp8_gemm needs for these sizes. */
size_t mxg_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * mxfp8_gemm_noalloc -- mxfp8_gemm for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same operation, arguments (less the
 * workspace), kernels and results as mxfp8_gemm.  The cross-workgroup
 * counters and K-split partial sums that mxfp8_gemm keeps in the caller's
 * workspace live instead in a library-owned device array of
 * MXG_NOALLOC_SCRATCH_BYTES bytes, one per GPU the library runs on, held
 * until the process ends.  The call itself allocates nothing.
 *   - Shapes whose mxg_gemm_workspace_bytes() exceeds
 *     MXG_NOALLOC_SCRATCH_BYTES are rejected with MXG_ERR_WORKSPACE before
 *     anything is launched.
 *   - Every call on one GPU uses that GPU's one array and each call leaves
 *     its counters at zero for the next: calls issued in order (one stream,
 *     or streams ordered by events) are safe; calls that may run at the same
 *     time on one GPU race and give wrong results.
 * Status as for mxfp8_gemm.
 */
#define MXG_NOALLOC_SCRATCH_BYTES (16u << 20)
int mxfp8_gemm_noalloc(int64_t M, int64_t N, int64_t K, const uint16_t *x_bf16,
                       int64_t ld_x, uint8_t *a_q, uint8_t *a_s, const uint8_t *w_q,
                       const uint8_t *w_s, uint16_t *out, void *stream);

/*
 * mxfp8_gemm_ex -- mxfp8_gemm with the layouts of the activation scales and
 * of the weight given by the caller.
 *   a_scale_layout   MXG_SCALES_ROW_MAJOR: a_s is [M, K/32], as in mxfp8_gemm;
 *                    MXG_SCALES_128X4: a_s is mxg_scale_bytes_128x4(M, K)
 *                    bytes in 128 x 4 tiles (offsets as in
 *                    mxfp8_rmsnorm_quantize), MXFP8 input only (x_bf16 NULL).
 *                    ([mxfp8] module text: the low-latency and cute-dsl
 *                    backends read the same F8_128x4 activation scales, so a
 *                    tensor from mxfp8_rmsnorm_quantize with MXG_SCALES_128X4,
 *                    or another producer of that layout, needs no repack.)
 *   w_layout         MXG_WEIGHTS_PACKED: w_q/w_s from mxfp8_pack_weights, as
 *                    in mxfp8_gemm; MXG_WEIGHTS_ROW_MAJOR: w_q [N, K] and
 *                    w_s [N, K/32] as the [mxfp8] page's launch_low_latency
 *                    takes them (a column-major [K, N] weight), read without
 *                    a repack.
 *   other arguments  as mxfp8_gemm.
 * The kernels, plans and summation order do not depend on either layout, so
 * results equal mxfp8_gemm's on the same values bit for bit.  With
 * MXG_SCALES_128X4 the direct kernels (up to 48 rows) or the 64-row blocks
 * of the 2D kernel serve the call.  An unknown layout, or 128 x 4 scales with
 * BF16 input, is MXG_ERR_SHAPE; other status as above.
 */
int mxfp8_gemm_ex(int64_t M, int64_t N, int64_t K, const uint16_t *x_bf16, int64_t ld_x,
                  uint8_t *a_q, uint8_t *a_s, int32_t a_scale_layout, const uint8_t *w_q,
                  const uint8_t *w_s, int32_t w_layout, uint16_t *out, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * An MXFP8 weight of shape [N, K] and the layout of its bytes:
 *   MXG_WEIGHTS_PACKED     (0, the default of a zero-initialised field) q and
 *                          s as mxfp8_pack_weights writes them;
 *   MXG_WEIGHTS_ROW_MAJOR  q [N, K] codes, s [N, K/32] scale bytes, row-major.
 * Any other layout value is rejected with MXG_ERR_SHAPE.
 */
typedef struct {
  const uint8_t *q; /* N*K codes      */
  const uint8_t *s; /* N*K/32 scales  */
  int64_t N, K;
  int32_t layout;   /* MXG_WEIGHTS_* */
} mxg_weight;

/*
 * mxfp8_proj_chain -- three projections back to back, in the
 * order of a decode step's attention ([step] page, AttentionStep.run:
 * fused_wqa_wkv on the MXFP8 layer input, the leading columns of its output
 * requantized to MXFP8 for wq_b, and wo_b on its own MXFP8 input):
 *   A:  out_a = a . wA^T                       (a: MXFP8 [M, wA.K])
 *   requantize out_a[:, 0:wB.K] to MXFP8 -> (b_q, b_s), as mxfp8_quantize does
 *   B:  out_b = b . wB^T
 *   C:  out_c = c . wC^T                       (c: MXFP8 [M, wC.K])
 * Each stage reads its activations only once the previous stage has finished
 * (C included).  Weights never depend on the previous stage, and the pages
 * overlap the next weight read with the previous kernel ([mxfp8] page: the
 * low-latency kernel loads its weights before its grid dependency wait).
 * The stages run as three launches in stream order (each stage's weight
 * read starts when the previous launch ends): on MI355X a dependency between
 * workgroups of one persistent launch measured slower than a launch boundary.
 * The requantize runs inside one of them: in A's epilogue where A's kernel
 * holds whole 32-column blocks of its output per workgroup, otherwise in B's
 * activation staging.
 *
 * Shapes: 1 <= M <= 48; each weight N % 16 == 0, K % 128 == 0; wB.K <= wA.N,
 * wB.K % 128 == 0.  out_a/out_b/out_c are BF16 [M, N] row-major, b_q/b_s
 * [M, wB.K] / [M, wB.K/32] (written).  The workspace rules of mxfp8_gemm
 * apply, with mxg_chain_workspace_bytes() as the size.
 *
 * Optional norm ([step] page: _split_qkv_and_norm normalises those leading
 * columns before wq_b): with norm_weight non-NULL (BF16 [wB.K], 16-byte
 * aligned; norm_eps >= 0), out_a[:, 0:wB.K] is RMS-normalised as
 * mxfp8_rmsnorm_quantize does and the BF16 result is what is requantized;
 * it is also written to b_bf16 ([M, wB.K] BF16) when that is non-NULL.
 * B normalises the rows while staging them up to 16 rows; above that the
 * norm takes one more launch between A and B.  norm_weight NULL: the plain
 * requantize.
 */
typedef struct {
  int64_t M;
  const uint8_t *a_q, *a_s;
  mxg_weight wA, wB, wC;
  uint16_t *out_a;
  uint8_t *b_q, *b_s;
  uint16_t *out_b;
  const uint8_t *c_q, *c_s;
  uint16_t *out_c;
  void *workspace;
  size_t workspace_bytes;
  const uint16_t *norm_weight; /* optional RMSNorm gain [wB.K] (NULL: none)  */
  float norm_eps;
  uint16_t *b_bf16;            /* optional: the normalised BF16 [M, wB.K]  */
} mxg_chain;

int mxfp8_proj_chain(const mxg_chain *chain, void *stream);

/* Workspace bytes mxfp8_proj_chain needs (pointers in *chain are not read). */
size_t mxg_chain_workspace_bytes(const mxg_chain *chain);

/*
 * wo_a_fused_quantize -- the grouped WO-A projection with rotary embedding in
 * front and MXFP8 of its output behind, optionally followed by wo_b ([o_proj]
 * page, dsv41_o_proj: the fused WO-A kernel returns the MXFP8 codes and
 * scales that wo_b takes as its input; _can_fuse_wo_a: FP8 WO-A with per-32
 * scales, at most 8 heads per group, 448 + 64 head dims, o_lora_rank a
 * multiple of 128).  For each row m (token):
 *   1. y = o[m] with the last rope = D - nope dims of every head rotated by
 *      positions[m]: pair i = dims (nope + 2i, nope + 2i + 1), angle row
 *      cos_sin[positions[m]] = [cos theta_0 .. cos theta_{rope/2-1},
 *      sin theta_0 .. sin theta_{rope/2-1}], y1 = x1 cos - x2 sin,
 *      y2 = x2 cos + x1 sin in FP32 without fused multiply-add, rounded to
 *      BF16; the nope dims pass through.
 *   2. group g (heads g*hpg .. g*hpg + hpg - 1, hpg = H/G) is the hpg*D
 *      values of those heads, concatenated, quantized to MXFP8 as
 *      mxfp8_quantize does;
 *   3. z[m, g*R + r] = BF16 of that group input times row g*R + r of wa
 *      (R = wa.N / G), i.e. the G group outputs concatenated;
 *   4. (z_q, z_s) = MXFP8 of z, as mxfp8_quantize does;
 *   5. if wb.q != NULL: out = dequant(z_q, z_s) . dequant(wb)^T, BF16.
 * Every intermediate is rounded to BF16 before it is quantized, as in the
 * unfused path (rotary output, z).
 *
 *   M           1 <= M <= MXG_MAX_ROWS
 *   o           BF16 attention output; head h of row m starts at
 *               o + m*ld_row + h*ld_head, its D values contiguous
 *   ld_row, ld_head
 *               strides in elements: ld_head >= D, ld_row >= (H-1)*ld_head + D,
 *               both multiples of 8
 *   positions   int64 [M] token positions, each in [0, max_pos)
 *   cos_sin     FP32 [max_pos, rope] angle table as above (16-byte aligned)
 *   n_heads H, head_dim D, nope_dim, n_groups G
 *               H % G == 0, H/G <= 8, D and nope multiples of 32,
 *               0 < nope < D (rope = D - nope)
 *   wa          MXFP8 weight (either layout) with N = G*R rows,
 *               group g = rows [g*R, g*R + R), and K = hpg*D; R % 128 == 0
 *   z           optional out: BF16 [M, G*R] (NULL: kept in the workspace)
 *   z_q, z_s    out: MXFP8 of z, [M, G*R] codes, [M, G*R/32] scale bytes
 *   wb, out     optional wo_b: a weight with K = G*R, N % 16 == 0, and
 *               its BF16 output [M, wb.N]; wb.q == NULL skips step 5
 *   workspace, workspace_bytes
 *               at least mxg_wo_a_workspace_bytes() bytes, zero-filled once
 *               when allocated.  After a call, bytes [65536, 65536 + M*H*D)
 *               hold the MXFP8 codes of the rotated input [M, H*D] (step 2)
 *               and its scale bytes [M, H*D/32] follow at the next multiple
 *               of 256; without z, z follows them.  Byte offset 20 is an error word: bit 1
 *               is set when a position is outside [0, max_pos); that row then
 *               uses angle row 0 and its results are not meaningful.  The
 *               word is never cleared by the library.  Calls sharing a
 *               workspace must not overlap.
 * Validation happens before any launch; positions are device data, so their
 * range is the one check made on the device.
 */
typedef struct {
  int64_t M;
  const uint16_t *o;
  int64_t ld_row, ld_head;
  const int64_t *positions;
  const float *cos_sin;
  int64_t max_pos;
  int32_t n_heads, head_dim, nope_dim, n_groups;
  mxg_weight wa;
  uint16_t *z;
  uint8_t *z_q, *z_s;
  mxg_weight wb;
  uint16_t *out;
  void *workspace;
  size_t workspace_bytes;
} mxg_wo_a;

int wo_a_fused_quantize(const mxg_wo_a *p, void *stream);

/* Workspace bytes wo_a_fused_quantize needs (pointers in *p are not read). */
size_t mxg_wo_a_workspace_bytes(const mxg_wo_a *p);

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_H */
