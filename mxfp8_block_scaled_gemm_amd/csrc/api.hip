// C ABI of libmxgemm (declared in include/mxgemm.h): host-side validation,
// then one launch per call.  Validation is a pure function of the arguments
// and runs before anything is enqueued ([cute] page, AllReduceMHC checks every
// buffer before its first launch), so a rejected call launches nothing and
// writes nothing.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "mx_launch.hpp"
#include "mxgemm.h"

// Scratch of mxfp8_gemm_noalloc (see there): one copy per GPU.
constexpr size_t kScratchBytes = MXG_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

using mxg::GemmArgs;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 0 = not checked yet, 1 = gfx950, 2 = something else.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

// Is the current device a gfx950?  MXG_FORCE_ARCH overrides the reported
// architecture name (used to exercise the rejection path).
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MXG_ERR_DEVICE;
  const char* forced = std::getenv("MXG_FORCE_ARCH");
  if (forced) return std::strncmp(forced, "gfx950", 6) == 0 ? MXG_OK : MXG_ERR_DEVICE;
  if (dev >= kMaxDevices) return MXG_ERR_DEVICE;
  int state = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXG_ERR_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? MXG_OK : MXG_ERR_DEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? MXG_OK : MXG_ERR_DEVICE; }

int validate_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint8_t* q,
                      const uint8_t* s) {
  if (!x || !q || !s) return MXG_ERR_NULL;
  if (M < 1 || K < 32 || K % 32 != 0 || ld_x < K || M > (int64_t)1 << 31 || K > (int64_t)1 << 30)
    return MXG_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(q) || ld_x % 8 != 0) return MXG_ERR_ALIGN;
  return MXG_OK;
}

int validate_rmsnorm(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, const uint16_t* w,
                     float eps, const uint16_t* y, int64_t ld_y, const uint8_t* q,
                     const uint8_t* s, int32_t layout) {
  if (!x || !w || !q || !s) return MXG_ERR_NULL;
  if (M < 1 || M > 65535 || K < 128 || K % 128 != 0 || K > MXG_MAX_K || ld_x < K ||
      ld_x * M > ((int64_t)1 << 30) || !(eps >= 0.f) || eps > 3.0e38f ||
      (layout != MXG_SCALES_ROW_MAJOR && layout != MXG_SCALES_128X4))
    return MXG_ERR_SHAPE;
  if (y && (ld_y < K || ld_y * M > ((int64_t)1 << 30))) return MXG_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(q) || ld_x % 8 != 0 ||
      (y && (!aligned16(y) || ld_y % 8 != 0)))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

bool gemm_shape_ok(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= MXG_MAX_GEMM_ROWS && N >= 16 && N % 16 == 0 && K >= 128 && K % 128 == 0 &&
         N <= ((int64_t)1 << 24) && K <= MXG_MAX_K && N * K <= ((int64_t)1 << 31) - 1;
}

int validate_gemm_args(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ld_x,
                       const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q,
                       const uint8_t* w_s, const uint16_t* out) {
  if (!a_q || !a_s || !w_q || !w_s || !out) return MXG_ERR_NULL;
  if (!gemm_shape_ok(M, N, K)) return MXG_ERR_SHAPE;
  if (x && (ld_x < K || ld_x * M > ((int64_t)1 << 30))) return MXG_ERR_SHAPE;
  if (!aligned16(a_q) || !aligned16(a_s) || !aligned16(w_q) || !aligned16(w_s) ||
      !aligned16(out) || (x && (!aligned16(x) || ld_x % 8 != 0)))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

int validate_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ld_x,
                  const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q,
                  const uint8_t* w_s, const uint16_t* out, size_t ws_bytes, const void* ws) {
  const int st = validate_gemm_args(M, N, K, x, ld_x, a_q, a_s, w_q, w_s, out);
  if (st != MXG_OK) return st;
  const size_t need = mxg_gemm_workspace_bytes(M, N, K);
  if (need > 0 && (!ws || ws_bytes < need)) return MXG_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return MXG_ERR_ALIGN;
  return MXG_OK;
}

bool weight_ok(const mxg_weight& w) {
  return w.N >= 16 && w.N % 16 == 0 && w.K >= 128 && w.K % 128 == 0 && w.N <= ((int64_t)1 << 24) &&
         w.K <= MXG_MAX_K && w.N * w.K <= ((int64_t)1 << 31) - 1;
}

int validate_chain(const mxg_chain* c, size_t need) {
  if (!c) return MXG_ERR_NULL;
  if (!c->a_q || !c->a_s || !c->wA.q || !c->wA.s || !c->wB.q || !c->wB.s || !c->wC.q ||
      !c->wC.s || !c->out_a || !c->b_q || !c->b_s || !c->out_b || !c->c_q || !c->c_s ||
      !c->out_c)
    return MXG_ERR_NULL;
  if (c->M < 1 || c->M > MXG_MAX_ROWS || !weight_ok(c->wA) || !weight_ok(c->wB) ||
      !weight_ok(c->wC) || c->wB.K > c->wA.N)
    return MXG_ERR_SHAPE;
  const void* ptrs[] = {c->a_q, c->a_s, c->wA.q, c->wA.s, c->wB.q, c->wB.s, c->wC.q, c->wC.s,
                        c->out_a, c->b_q, c->b_s, c->out_b, c->c_q, c->c_s, c->out_c};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MXG_ERR_ALIGN;
  if (c->norm_weight && (!(c->norm_eps >= 0.f) || c->norm_eps > 3.0e38f)) return MXG_ERR_SHAPE;
  if ((c->norm_weight && !aligned16(c->norm_weight)) || (c->b_bf16 && !aligned16(c->b_bf16)))
    return MXG_ERR_ALIGN;
  if (!c->workspace || c->workspace_bytes < need) return MXG_ERR_WORKSPACE;
  if (!aligned16(c->workspace)) return MXG_ERR_ALIGN;
  return MXG_OK;
}

// K-split state of a direct GEMM in workspace ws, partials from part_off on.
void set_ksplit(GemmArgs& a, void* ws, size_t part_off) {
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  a.ctr = w ? reinterpret_cast<uint32_t*>(w + mxg::kGemmCtrOffset) : nullptr;
  a.part = w ? reinterpret_cast<float*>(w + part_off) : nullptr;
}

// Workspace bytes a direct GEMM needs with its partials from part_off on.
size_t direct_need(int M, int N, int K, size_t part_off, int group_tiles = 0) {
  const size_t pb = mxg::gemm_partial_bytes(M, N, K, group_tiles);
  return pb ? part_off + pb : 0;
}

int chain_direct(const mxg_chain& c, hipStream_t stream) {
  const int M = (int)c.M;
  GemmArgs a{nullptr, 0, const_cast<uint8_t*>(c.a_q), const_cast<uint8_t*>(c.a_s), c.wA.q, c.wA.s,
             c.out_a, M, (int)c.wA.N, (int)c.wA.K};
  set_ksplit(a, c.workspace, mxg::kGemmPartOffset);
  hipError_t e = mxg::launch_gemm(a, stream);
  if (e != hipSuccess) return MXG_ERR_DEVICE;
  GemmArgs b{c.out_a, c.wA.N, c.b_q, c.b_s, c.wB.q, c.wB.s, c.out_b, M, (int)c.wB.N, (int)c.wB.K};
  // B quantizes A's leading columns while staging them (RMS-normalising
  // them first when a gain is given), or launches that step on its own
  // first where its kernel cannot.
  b.norm_w = c.norm_weight;
  b.norm_eps = c.norm_eps;
  b.norm_y = c.b_bf16;
  set_ksplit(b, c.workspace, mxg::kGemmPartOffset);
  if ((e = mxg::launch_gemm(b, stream)) != hipSuccess) return MXG_ERR_DEVICE;
  GemmArgs cc{nullptr, 0, const_cast<uint8_t*>(c.c_q), const_cast<uint8_t*>(c.c_s), c.wC.q,
              c.wC.s, c.out_c, M, (int)c.wC.N, (int)c.wC.K};
  set_ksplit(cc, c.workspace, mxg::kGemmPartOffset);
  return launched(mxg::launch_gemm(cc, stream));
}

// ------------------------------------------------------------------ WO-A

struct WoALayout {
  size_t xq, xs, z, end;   // workspace offsets
};

WoALayout wo_a_layout(const mxg_wo_a& p) {
  const size_t M = (size_t)p.M, HD = (size_t)p.n_heads * (size_t)p.head_dim;
  const size_t GR = (size_t)p.wa.N;
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  WoALayout l;
  l.xq = mxg::kCtrRegionBytes;
  l.xs = up(l.xq + M * HD);
  l.z = up(l.xs + M * HD / 32);
  l.end = up(l.z + (p.z ? 0 : 2 * M * GR));
  return l;
}

bool wo_a_shape_ok(const mxg_wo_a& p) {
  const int64_t H = p.n_heads, D = p.head_dim, nope = p.nope_dim, G = p.n_groups;
  if (p.M < 1 || p.M > MXG_MAX_ROWS || H < 1 || G < 1 || H % G != 0 || H / G > 8) return false;
  if (D < 64 || D % 32 != 0 || nope < 32 || nope >= D || nope % 32 != 0 || D > 4096) return false;
  if (H * D > ((int64_t)1 << 20) || p.max_pos < 1 || p.max_pos > ((int64_t)1 << 31) / (D - nope))
    return false;
  if (p.ld_head < D || p.ld_row < (H - 1) * p.ld_head + D) return false;
  if (((p.M - 1) * p.ld_row + H * p.ld_head) * 2 >= ((int64_t)1 << 31)) return false;
  if (!weight_ok(p.wa) || p.wa.N % G != 0 || (p.wa.N / G) % 128 != 0 || p.wa.K != (H / G) * D)
    return false;
  if (p.wb.q && (!weight_ok(p.wb) || p.wb.K != p.wa.N)) return false;
  return true;
}

size_t wo_a_need(const mxg_wo_a& p);

int validate_wo_a(const mxg_wo_a* p) {
  if (!p) return MXG_ERR_NULL;
  if (!p->o || !p->positions || !p->cos_sin || !p->wa.q || !p->wa.s || !p->z_q || !p->z_s)
    return MXG_ERR_NULL;
  if (p->wb.q && (!p->wb.s || !p->out)) return MXG_ERR_NULL;
  if (!wo_a_shape_ok(*p)) return MXG_ERR_SHAPE;
  const void* ptrs[] = {p->o, p->cos_sin, p->wa.q, p->wa.s, p->z_q, p->z_s};
  for (const void* q : ptrs)
    if (!aligned16(q)) return MXG_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(p->positions) & 7u) || p->ld_row % 8 || p->ld_head % 8)
    return MXG_ERR_ALIGN;
  if (p->z && !aligned16(p->z)) return MXG_ERR_ALIGN;
  if (p->wb.q && (!aligned16(p->wb.q) || !aligned16(p->wb.s) || !aligned16(p->out)))
    return MXG_ERR_ALIGN;
  if (!p->workspace || p->workspace_bytes < wo_a_need(*p)) return MXG_ERR_WORKSPACE;
  if (!aligned16(p->workspace)) return MXG_ERR_ALIGN;
  return MXG_OK;
}

// Workspace bytes of WO-A: the rotated input's codes (and z when the caller
// keeps none), then the K-split partials of either GEMM.
size_t wo_a_need(const mxg_wo_a& p) {
  const WoALayout l = wo_a_layout(p);
  size_t need = l.end;
  const int R = (int)p.wa.N / p.n_groups;
  need = std::max(need, direct_need((int)p.M, (int)p.wa.N, (int)p.wa.K, l.end, R / 16));
  if (p.wb.q) need = std::max(need, direct_need((int)p.M, (int)p.wb.N, (int)p.wb.K, l.end));
  return need;
}

int wo_a_run(const mxg_wo_a& p, hipStream_t stream) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(p.workspace);
  const WoALayout l = wo_a_layout(p);
  const int M = (int)p.M, H = p.n_heads, D = p.head_dim, G = p.n_groups;
  const int HD = H * D, GR = (int)p.wa.N, R = GR / G, Kg = (int)p.wa.K;
  uint8_t* xq = ws + l.xq;
  uint8_t* xs = ws + l.xs;
  uint16_t* z = p.z ? p.z : reinterpret_cast<uint16_t*>(ws + l.z);
  // 1-2. rotary + MXFP8 of every head, groups side by side in each row.
  mxg::RopeQuantArgs rq{p.o, p.ld_row, p.ld_head, p.positions, p.cos_sin, p.max_pos, xq, xs,
                        reinterpret_cast<uint32_t*>(ws + 4 * mxg::kCtrError), M, H, D,
                        p.nope_dim};
  hipError_t e = mxg::launch_rope_quant(rq, stream);
  if (e != hipSuccess) return MXG_ERR_DEVICE;
  // 3. grouped projection: weight tile t reads group t / (R/16)'s columns.
  GemmArgs ga{nullptr, 0, xq, xs, p.wa.q, p.wa.s, z, M, GR, Kg};
  ga.lda = HD;
  ga.group_tiles = R / 16;
  ga.a_group = Kg;
  set_ksplit(ga, p.workspace, l.end);
  if ((e = mxg::launch_gemm(ga, stream)) != hipSuccess) return MXG_ERR_DEVICE;
  // 4-5. MXFP8 of z, written by wo_b's GEMM when there is one.
  if (p.wb.q) {
    GemmArgs gb{z, GR, p.z_q, p.z_s, p.wb.q, p.wb.s, p.out, M, (int)p.wb.N, (int)p.wb.K};
    set_ksplit(gb, p.workspace, l.end);
    return launched(mxg::launch_gemm(gb, stream));
  }
  return launched(mxg::launch_quantize(z, M, GR, GR, p.z_q, p.z_s, stream));
}

int validate_pack(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                  const uint8_t* wp_q, const uint8_t* wp_s) {
  if (!w_q || !w_s || !wp_q || !wp_s) return MXG_ERR_NULL;
  if (N < 16 || N % 16 != 0 || K < 128 || K % 128 != 0 || N > (int64_t)1 << 24 ||
      K > (int64_t)1 << 20 || N * K > ((int64_t)1 << 31) - 1)
    return MXG_ERR_SHAPE;
  if (!aligned16(w_q) || !aligned16(w_s) || !aligned16(wp_q) || !aligned16(wp_s))
    return MXG_ERR_ALIGN;
  return MXG_OK;
}

// ------------------------------------------------ allocation-free GEMM
//
// mxfp8_gemm_noalloc keeps the K-split state of mxfp8_gemm (counters and FP32
// partial sums, laid out as in a caller's workspace) in this library-owned
// array: one copy per GPU, zero at load like any static object, and every
// call leaves its counters at zero again.  In host code the array's name is
// only a stand-in for the symbol; its address on each device is taken once
// with hipGetSymbolAddress while that device is current, and only that
// pointer is handed to kernels.
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device (looked up once per device).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXG_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MXG_ERR_DEVICE;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MXG_OK;
}

}  // namespace

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

int mxg_version(void) { return 100; }

size_t mxg_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!gemm_shape_ok(M, N, K)) return mxg::kCtrBytes;
  return std::max(mxg::kCtrBytes, direct_need((int)M, (int)N, (int)K, mxg::kGemmPartOffset));
}

size_t mxg_chain_workspace_bytes(const mxg_chain* c) {
  if (!c || c->M < 1 || c->M > MXG_MAX_ROWS || !weight_ok(c->wA) || !weight_ok(c->wB) ||
      !weight_ok(c->wC))
    return mxg::kCtrBytes;
  const int M = (int)c->M;
  size_t need = mxg::kCtrBytes;
  for (const mxg_weight* w : {&c->wA, &c->wB, &c->wC})
    need = std::max(need, direct_need(M, (int)w->N, (int)w->K, mxg::kGemmPartOffset));
  return need;
}

int mxfp8_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* q, uint8_t* s,
                   void* stream) {
  int st = validate_quantize(x, M, K, ld_x, q, s);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return launched(mxg::launch_quantize(x, M, K, ld_x, q, s, (hipStream_t)stream));
}

size_t mxg_scale_bytes_128x4(int64_t M, int64_t K) {
  if (M < 1 || K < 1) return 0;
  return (size_t)((M + 127) / 128) * 128 * (size_t)((K + 127) / 128) * 4;
}

int mxfp8_rmsnorm_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                           const uint16_t* w, float eps, uint16_t* y, int64_t ld_y, uint8_t* q,
                           uint8_t* s, int32_t scale_layout, void* stream) {
  int st = validate_rmsnorm(x, M, K, ld_x, w, eps, y, ld_y, q, s, scale_layout);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return launched(mxg::launch_rmsnorm_quantize(x, M, K, ld_x, w, eps, y, ld_y, q, s,
                                               scale_layout, (hipStream_t)stream));
}

int mxg_hbm_read_probe(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                       uint32_t* sink, void* stream) {
  if (!w_q || !w_s || !sink) return MXG_ERR_NULL;
  if (N < 16 || N % 16 != 0 || N > ((int64_t)1 << 24) || K < 128 || K % 128 != 0 || K > 8192)
    return MXG_ERR_SHAPE;
  if (!aligned16(w_q) || !aligned16(w_s) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return MXG_ERR_ALIGN;
  int st = check_device();
  if (st != MXG_OK) return st;
  return launched(
      mxg::launch_hbm_read(w_q, w_s, (int)(N / 16), (int)(K / 128), sink, (hipStream_t)stream));
}

int mxfp8_pack_weights(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                       uint8_t* wp_q, uint8_t* wp_s, void* stream) {
  int st = validate_pack(w_q, w_s, N, K, wp_q, wp_s);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return launched(mxg::launch_pack(w_q, w_s, N, K, wp_q, wp_s, (hipStream_t)stream));
}

int mxfp8_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* x_bf16, int64_t ld_x,
               uint8_t* a_q, uint8_t* a_s, const uint8_t* w_q, const uint8_t* w_s, uint16_t* out,
               void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate_gemm(M, N, K, x_bf16, ld_x, a_q, a_s, w_q, w_s, out, workspace_bytes,
                         workspace);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  GemmArgs a{x_bf16, ld_x, a_q, a_s, w_q, w_s, out, (int)M, (int)N, (int)K};
  set_ksplit(a, workspace, mxg::kGemmPartOffset);
  return launched(mxg::launch_gemm(a, (hipStream_t)stream));
}

int mxfp8_gemm_noalloc(int64_t M, int64_t N, int64_t K, const uint16_t* x_bf16, int64_t ld_x,
                       uint8_t* a_q, uint8_t* a_s, const uint8_t* w_q, const uint8_t* w_s,
                       uint16_t* out, void* stream) {
  int st = validate_gemm_args(M, N, K, x_bf16, ld_x, a_q, a_s, w_q, w_s, out);
  if (st != MXG_OK) return st;
  if (mxg_gemm_workspace_bytes(M, N, K) > kScratchBytes) return MXG_ERR_WORKSPACE;
  if ((st = check_device()) != MXG_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MXG_OK) return st;
  GemmArgs a{x_bf16, ld_x, a_q, a_s, w_q, w_s, out, (int)M, (int)N, (int)K};
  set_ksplit(a, ws, mxg::kGemmPartOffset);
  return launched(mxg::launch_gemm(a, (hipStream_t)stream));
}

int mxfp8_gemm_ex(int64_t M, int64_t N, int64_t K, const uint8_t* a_q, const uint8_t* a_s,
                  int32_t a_scale_layout, const uint8_t* w_q, const uint8_t* w_s, uint16_t* out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (a_scale_layout == MXG_SCALES_ROW_MAJOR)
    return mxfp8_gemm(M, N, K, nullptr, 0, const_cast<uint8_t*>(a_q), const_cast<uint8_t*>(a_s),
                      w_q, w_s, out, workspace, workspace_bytes, stream);
  if (a_scale_layout != MXG_SCALES_128X4) return MXG_ERR_SHAPE;
  int st = validate_gemm(M, N, K, nullptr, 0, a_q, a_s, w_q, w_s, out, workspace_bytes,
                         workspace);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  GemmArgs a{nullptr, 0, const_cast<uint8_t*>(a_q), const_cast<uint8_t*>(a_s), w_q, w_s, out,
             (int)M, (int)N, (int)K};
  a.a_sf128 = true;
  set_ksplit(a, workspace, mxg::kGemmPartOffset);
  return launched(mxg::launch_gemm(a, (hipStream_t)stream));
}

int mxfp8_proj_chain(const mxg_chain* c, void* stream) {
  if (!c) return MXG_ERR_NULL;
  int st = validate_chain(c, mxg_chain_workspace_bytes(c));
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return chain_direct(*c, (hipStream_t)stream);
}

size_t mxg_wo_a_workspace_bytes(const mxg_wo_a* p) {
  if (!p || !wo_a_shape_ok(*p)) return mxg::kCtrRegionBytes;
  return wo_a_need(*p);
}

int wo_a_fused_quantize(const mxg_wo_a* p, void* stream) {
  int st = validate_wo_a(p);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return wo_a_run(*p, (hipStream_t)stream);
}

}  // extern "C"
