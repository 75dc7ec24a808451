// Argument checks of the libmxgemm C ABI: pure host functions of the
// arguments (no device access, no HIP), run before anything is enqueued
// ([cute] page: AllReduceMHC checks every buffer before its first launch), so
// a rejected call launches nothing and writes nothing.  They live in a plain
// C++ file so that the same code can also be built with the host sanitizers
// (AddressSanitizer, UndefinedBehaviorSanitizer) for the CPU test suite.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mxgemm.h"

namespace mxg {
namespace check {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint8_t* q,
             const uint8_t* s);
int rmsnorm(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* w, float eps,
            const uint16_t* y, int64_t ld_y, const uint8_t* q, const uint8_t* s, int32_t layout);
bool gemm_shape(int64_t M, int64_t N, int64_t K);
int gemm(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ld_x, const uint8_t* a_q,
         const uint8_t* a_s, const uint8_t* w_q, const uint8_t* w_s, const uint16_t* out);
// Weight shape and layout of the chain's and WO-A's weights.
bool weight(const mxg_weight& w);
// mxfp8_gemm_ex's layouts: known values, and 128 x 4 scales only on MXFP8 input.
int gemm_layouts(int32_t a_scale_layout, int32_t w_layout, const uint16_t* x);
// Chain and WO-A structures, everything but the workspace.
int chain(const mxg_chain* c);
bool wo_a_shape(const mxg_wo_a& p);
int wo_a(const mxg_wo_a* p);
int pack(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K, const uint8_t* wp_q,
         const uint8_t* wp_s);
// A caller workspace of `bytes` bytes for a call that needs `need`.
int workspace(const void* ws, size_t bytes, size_t need);

}  // namespace check
}  // namespace mxg
