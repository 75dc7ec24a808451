// Argument checks of the libmxgemm C ABI (declared in validate.hpp), and the
// exported helpers that are pure functions of their arguments.
#include "validate.hpp"

namespace mxg {
namespace check {

int quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint8_t* q,
             const uint8_t* s) {
  if (!x || !q || !s) return MXG_ERR_NULL;
  if (M < 1 || K < 32 || K % 32 != 0 || ld_x < K || M > (int64_t)1 << 31 || K > (int64_t)1 << 30 ||
      ld_x > ((int64_t)1 << 40) / M)
    return MXG_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(q) || ld_x % 8 != 0) return MXG_ERR_ALIGN;
  return MXG_OK;
}

int rmsnorm(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* w, float eps,
            const uint16_t* y, int64_t ld_y, const uint8_t* q, const uint8_t* s, int32_t layout) {
  if (!x || !w || !q || !s) return MXG_ERR_NULL;
  // (strides are bounded by division: a product could overflow)
  if (M < 1 || M > 65535 || K < 128 || K % 128 != 0 || K > MXG_MAX_K || ld_x < K ||
      ld_x > ((int64_t)1 << 30) / M || !(eps >= 0.f) || eps > 3.0e38f ||
      (layout != MXG_SCALES_ROW_MAJOR && layout != MXG_SCALES_128X4))
    return MXG_ERR_SHAPE;
  if (y && (ld_y < K || ld_y > ((int64_t)1 << 30) / M)) return MXG_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(q) || ld_x % 8 != 0 ||
      (y && (!aligned16(y) || ld_y % 8 != 0)))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

bool gemm_shape(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= MXG_MAX_GEMM_ROWS && N >= 16 && N % 16 == 0 && K >= 128 && K % 128 == 0 &&
         N <= ((int64_t)1 << 24) && K <= MXG_MAX_K && N * K <= ((int64_t)1 << 31) - 1;
}

int gemm(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ld_x, const uint8_t* a_q,
         const uint8_t* a_s, const uint8_t* w_q, const uint8_t* w_s, const uint16_t* out) {
  if (!a_q || !a_s || !w_q || !w_s || !out) return MXG_ERR_NULL;
  if (!gemm_shape(M, N, K)) return MXG_ERR_SHAPE;
  if (x && (ld_x < K || ld_x > ((int64_t)1 << 30) / M)) return MXG_ERR_SHAPE;
  if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(w_q) || !aligned16(w_s) ||
      !aligned16(out) || (x && (!aligned16(x) || ld_x % 8 != 0)))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

bool weight(const mxg_weight& w) {
  return (w.layout == MXG_WEIGHTS_PACKED || w.layout == MXG_WEIGHTS_ROW_MAJOR) && w.N >= 16 && w.N % 16 == 0 && w.K >= 128 && w.K % 128 == 0 && w.N <= ((int64_t)1 << 24) &&
         w.K <= MXG_MAX_K && w.N * w.K <= ((int64_t)1 << 31) - 1;
}

int chain(const mxg_chain* c) {
  if (!c) return MXG_ERR_NULL;
  if (!c->a_q || !c->a_s || !c->wA.q || !c->wA.s || !c->wB.q || !c->wB.s || !c->wC.q ||
      !c->wC.s || !c->out_a || !c->b_q || !c->b_s || !c->out_b || !c->c_q || !c->c_s ||
      !c->out_c)
    return MXG_ERR_NULL;
  if (c->M < 1 || c->M > MXG_MAX_ROWS || !weight(c->wA) || !weight(c->wB) || !weight(c->wC) ||
      c->wB.K > c->wA.N)
    return MXG_ERR_SHAPE;
  const void* ptrs[] = {c->a_q, c->a_s, c->wA.q, c->wA.s, c->wB.q, c->wB.s, c->wC.q, c->wC.s,
                        c->out_a, c->b_q, c->b_s, c->out_b, c->c_q, c->c_s, c->out_c};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MXG_ERR_ALIGN;
  if (c->norm_weight && (!(c->norm_eps >= 0.f) || c->norm_eps > 3.0e38f)) return MXG_ERR_SHAPE;
  if ((c->norm_weight && !aligned16(c->norm_weight)) || (c->b_bf16 && !aligned16(c->b_bf16)))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

bool wo_a_shape(const mxg_wo_a& p) {
  const int64_t H = p.n_heads, D = p.head_dim, nope = p.nope_dim, G = p.n_groups;
  if (p.M < 1 || p.M > MXG_MAX_ROWS || H < 1 || G < 1 || H % G != 0 || H / G > 8) return false;
  if (D < 64 || D % 32 != 0 || nope < 32 || nope >= D || nope % 32 != 0 || D > 4096) return false;
  if (H * D > ((int64_t)1 << 20) || p.max_pos < 1 || p.max_pos > ((int64_t)1 << 31) / (D - nope))
    return false;
  if (p.ld_head < D || p.ld_head > ((int64_t)1 << 30) / H) return false;   // no overflow below
  if (p.ld_row < (H - 1) * p.ld_head + D || p.ld_row > ((int64_t)1 << 30)) return false;
  if (((p.M - 1) * p.ld_row + H * p.ld_head) * 2 >= ((int64_t)1 << 31)) return false;
  if (!weight(p.wa) || p.wa.N % G != 0 || (p.wa.N / G) % 128 != 0 || p.wa.K != (H / G) * D)
    return false;
  if (p.wb.q && (!weight(p.wb) || p.wb.K != p.wa.N)) return false;
  return true;
}

int wo_a(const mxg_wo_a* p) {
  if (!p) return MXG_ERR_NULL;
  if (!p->o || !p->positions || !p->cos_sin || !p->wa.q || !p->wa.s || !p->z_q || !p->z_s)
    return MXG_ERR_NULL;
  if (p->wb.q && (!p->wb.s || !p->out)) return MXG_ERR_NULL;
  if (!wo_a_shape(*p)) return MXG_ERR_SHAPE;
  const void* ptrs[] = {p->o, p->cos_sin, p->wa.q, p->wa.s, p->z_q, p->z_s};
  for (const void* q : ptrs)
    if (!aligned16(q)) return MXG_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(p->positions) & 7u) || p->ld_row % 8 || p->ld_head % 8)
    return MXG_ERR_ALIGN;
  if (p->z && !aligned16(p->z)) return MXG_ERR_ALIGN;
  if (p->wb.q && (!aligned16(p->wb.q) || !aligned16(p->wb.s) || !aligned16(p->out)))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

int gemm_layouts(int32_t a_scale_layout, int32_t w_layout, const uint16_t* x) {
  if (a_scale_layout != MXG_SCALES_ROW_MAJOR && a_scale_layout != MXG_SCALES_128X4)
    return MXG_ERR_SHAPE;
  if (w_layout != MXG_WEIGHTS_PACKED && w_layout != MXG_WEIGHTS_ROW_MAJOR) return MXG_ERR_SHAPE;
  if (x && a_scale_layout == MXG_SCALES_128X4) return MXG_ERR_SHAPE;
  return MXG_OK;
}

int pack(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K, const uint8_t* wp_q,
         const uint8_t* wp_s) {
  if (!w_q || !w_s || !wp_q || !wp_s) return MXG_ERR_NULL;
  if (N < 16 || N % 16 != 0 || K < 128 || K % 128 != 0 || N > (int64_t)1 << 24 ||
      K > (int64_t)1 << 20 || N * K > ((int64_t)1 << 31) - 1)
    return MXG_ERR_SHAPE;
  if (!aligned16(w_q) || !aligned16(w_s) || !aligned16(wp_q) || !aligned16(wp_s))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

int workspace(const void* ws, size_t bytes, size_t need) {
  if (need > 0 && (!ws || bytes < need)) return MXG_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MXG_ERR_ALIGN;
  return MXG_OK;
}

}  // namespace check
}  // namespace mxg

extern "C" {

const char* mxg_strerror(int status) {
  switch (status) {
    case MXG_OK: return "success";
    case MXG_ERR_NULL: return "a required pointer is NULL";
    case MXG_ERR_ALIGN: return "a pointer or row stride is not 16-byte aligned";
    case MXG_ERR_SHAPE: return "a size is out of range or sizes are inconsistent";
    case MXG_ERR_WORKSPACE: return "workspace missing or too small";
    case MXG_ERR_DEVICE: return "device is not gfx950, or the kernel launch failed";
    default: return "unknown status";
  }
}

int mxg_version(void) { return 200; }

size_t mxg_scale_bytes_128x4(int64_t M, int64_t K) {
  if (M < 1 || K < 1) return 0;
  return (size_t)((M + 127) / 128) * 128 * (size_t)((K + 127) / 128) * 4;
}

}  // extern "C"
