/*
 * mxprobe.h -- C ABI of libmxprobe: a measurement aid that sits beside
 * libmxgemm (see mxgemm.h for the data formats and status codes) and is not
 * a step of the GEMM path.
 *
 * mxg_hbm_read_probe reads a weight packed by mxfp8_pack_weights (N rows, K
 * columns) exactly as the GEMMs' weight stream reads it (one workgroup of 16
 * waves per 16-row tile, each wave issuing all of its 128-wide K steps at
 * once) and computes nothing.  Timing it against mxfp8_gemm on the same
 * weight gives the single-launch streaming ceiling the GEMM is measured
 * against.
 *   w_q, w_s    packed weight codes (N*K bytes) and scales (N*K/32 bytes),
 *               16-byte aligned
 *   N, K        N % 16 == 0, K % 128 == 0, K <= 8192
 *   sink        a 4-byte aligned device word the kernel writes only for one
 *               improbable folded value of the data (so no load can be
 *               optimized away)
 *   stream      hipStream_t as void* (NULL: the default stream)
 * Status as in mxgemm.h (1 NULL, 2 alignment, 3 shape, 5 not gfx950 or the
 * launch failed); nothing is launched on an error.
 */
#ifndef MXPROBE_H
#define MXPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int mxg_hbm_read_probe(const uint8_t *w_q, const uint8_t *w_s, int64_t N, int64_t K,
                       uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXPROBE_H */
