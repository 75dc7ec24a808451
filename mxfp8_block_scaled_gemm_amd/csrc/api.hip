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
#include "validate.hpp"

// Scratch of mxfp8_gemm_noalloc (see there): one copy per GPU.
constexpr size_t kScratchBytes = MXG_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

using mxg::GemmArgs;
namespace check = mxg::check;

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

int validate_gemm(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ld_x,
                  const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q,
                  const uint8_t* w_s, const uint16_t* out, size_t ws_bytes, const void* ws) {
  const int st = check::gemm(M, N, K, x, ld_x, a_q, a_s, w_q, w_s, out);
  if (st != MXG_OK) return st;
  return check::workspace(ws, ws_bytes, mxg_gemm_workspace_bytes(M, N, K));
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
  a.w_rm = c.wA.layout == MXG_WEIGHTS_ROW_MAJOR;
  set_ksplit(a, c.workspace, mxg::kGemmPartOffset);
  // A writes the MXFP8 of its leading wB.K columns itself where its kernel
  // can (each 32-column block in one workgroup's epilogue); otherwise B
  // quantizes them while staging them (RMS-normalising them first when a
  // gain is given, which needs whole rows), or launches that step on its own
  // first where its kernel cannot.
  if (!c.norm_weight) {
    a.out_q = c.b_q;
    a.out_s = c.b_s;
    a.qn = (int)c.wB.K;
  }
  bool a_quantized = false;
  hipError_t e = mxg::launch_gemm(a, stream, &a_quantized);
  if (e != hipSuccess) return MXG_ERR_DEVICE;
  GemmArgs b{a_quantized ? nullptr : c.out_a, c.wA.N, c.b_q, c.b_s, c.wB.q, c.wB.s, c.out_b, M,
             (int)c.wB.N, (int)c.wB.K};
  b.w_rm = c.wB.layout == MXG_WEIGHTS_ROW_MAJOR;
  b.norm_w = c.norm_weight;
  b.norm_eps = c.norm_eps;
  b.norm_y = c.b_bf16;
  set_ksplit(b, c.workspace, mxg::kGemmPartOffset);
  if ((e = mxg::launch_gemm(b, stream)) != hipSuccess) return MXG_ERR_DEVICE;
  GemmArgs cc{nullptr, 0, const_cast<uint8_t*>(c.c_q), const_cast<uint8_t*>(c.c_s), c.wC.q,
              c.wC.s, c.out_c, M, (int)c.wC.N, (int)c.wC.K};
  cc.w_rm = c.wC.layout == MXG_WEIGHTS_ROW_MAJOR;
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

size_t wo_a_need(const mxg_wo_a& p);

int validate_wo_a(const mxg_wo_a* p) {
  const int st = check::wo_a(p);
  if (st != MXG_OK) return st;
  if (!p->workspace) return MXG_ERR_WORKSPACE;
  return check::workspace(p->workspace, p->workspace_bytes, wo_a_need(*p));
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
  ga.w_rm = p.wa.layout == MXG_WEIGHTS_ROW_MAJOR;
  set_ksplit(ga, p.workspace, l.end);
  if ((e = mxg::launch_gemm(ga, stream)) != hipSuccess) return MXG_ERR_DEVICE;
  // 4-5. MXFP8 of z, written by wo_b's GEMM when there is one.
  if (p.wb.q) {
    GemmArgs gb{z, GR, p.z_q, p.z_s, p.wb.q, p.wb.s, p.out, M, (int)p.wb.N, (int)p.wb.K};
    gb.w_rm = p.wb.layout == MXG_WEIGHTS_ROW_MAJOR;
    set_ksplit(gb, p.workspace, l.end);
    return launched(mxg::launch_gemm(gb, stream));
  }
  return launched(mxg::launch_quantize(z, M, GR, GR, p.z_q, p.z_s, stream));
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

size_t mxg_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!check::gemm_shape(M, N, K)) return mxg::kCtrBytes;
  return std::max(mxg::kCtrBytes, direct_need((int)M, (int)N, (int)K, mxg::kGemmPartOffset));
}

size_t mxg_chain_workspace_bytes(const mxg_chain* c) {
  if (!c || c->M < 1 || c->M > MXG_MAX_ROWS || !check::weight(c->wA) || !check::weight(c->wB) ||
      !check::weight(c->wC))
    return mxg::kCtrBytes;
  const int M = (int)c->M;
  size_t need = mxg::kCtrBytes;
  for (const mxg_weight* w : {&c->wA, &c->wB, &c->wC})
    need = std::max(need, direct_need(M, (int)w->N, (int)w->K, mxg::kGemmPartOffset));
  return need;
}

int mxfp8_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x, uint8_t* q, uint8_t* s,
                   void* stream) {
  int st = check::quantize(x, M, K, ld_x, q, s);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return launched(mxg::launch_quantize(x, M, K, ld_x, q, s, (hipStream_t)stream));
}

int mxfp8_rmsnorm_quantize(const uint16_t* x, int64_t M, int64_t K, int64_t ld_x,
                           const uint16_t* w, float eps, uint16_t* y, int64_t ld_y, uint8_t* q,
                           uint8_t* s, int32_t scale_layout, void* stream) {
  int st = check::rmsnorm(x, M, K, ld_x, w, eps, y, ld_y, q, s, scale_layout);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return launched(mxg::launch_rmsnorm_quantize(x, M, K, ld_x, w, eps, y, ld_y, q, s,
                                               scale_layout, (hipStream_t)stream));
}

int mxfp8_pack_weights(const uint8_t* w_q, const uint8_t* w_s, int64_t N, int64_t K,
                       uint8_t* wp_q, uint8_t* wp_s, void* stream) {
  int st = check::pack(w_q, w_s, N, K, wp_q, wp_s);
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
  int st = check::gemm(M, N, K, x_bf16, ld_x, a_q, a_s, w_q, w_s, out);
  if (st != MXG_OK) return st;
  if (mxg_gemm_workspace_bytes(M, N, K) > kScratchBytes) return MXG_ERR_WORKSPACE;
  if ((st = check_device()) != MXG_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MXG_OK) return st;
  GemmArgs a{x_bf16, ld_x, a_q, a_s, w_q, w_s, out, (int)M, (int)N, (int)K};
  set_ksplit(a, ws, mxg::kGemmPartOffset);
  return launched(mxg::launch_gemm(a, (hipStream_t)stream));
}

int mxfp8_gemm_ex(int64_t M, int64_t N, int64_t K, const uint16_t* x_bf16, int64_t ld_x,
                  uint8_t* a_q, uint8_t* a_s, int32_t a_scale_layout, const uint8_t* w_q,
                  const uint8_t* w_s, int32_t w_layout, uint16_t* out, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int st = check::gemm_layouts(a_scale_layout, w_layout, x_bf16);
  if (st != MXG_OK) return st;
  if ((st = validate_gemm(M, N, K, x_bf16, ld_x, a_q, a_s, w_q, w_s, out, workspace_bytes,
                          workspace)) != MXG_OK)
    return st;
  if ((st = check_device()) != MXG_OK) return st;
  GemmArgs a{x_bf16, ld_x, a_q, a_s, w_q, w_s, out, (int)M, (int)N, (int)K};
  a.a_sf128 = a_scale_layout == MXG_SCALES_128X4;
  a.w_rm = w_layout == MXG_WEIGHTS_ROW_MAJOR;
  set_ksplit(a, workspace, mxg::kGemmPartOffset);
  return launched(mxg::launch_gemm(a, (hipStream_t)stream));
}

int mxfp8_proj_chain(const mxg_chain* c, void* stream) {
  int st = check::chain(c);
  if (st != MXG_OK) return st;
  if (!c->workspace) return MXG_ERR_WORKSPACE;
  if ((st = check::workspace(c->workspace, c->workspace_bytes, mxg_chain_workspace_bytes(c))) !=
      MXG_OK)
    return st;
  if ((st = check_device()) != MXG_OK) return st;
  return chain_direct(*c, (hipStream_t)stream);
}

size_t mxg_wo_a_workspace_bytes(const mxg_wo_a* p) {
  if (!p || !check::wo_a_shape(*p)) return mxg::kCtrRegionBytes;
  return wo_a_need(*p);
}

int wo_a_fused_quantize(const mxg_wo_a* p, void* stream) {
  int st = validate_wo_a(p);
  if (st != MXG_OK) return st;
  if ((st = check_device()) != MXG_OK) return st;
  return wo_a_run(*p, (hipStream_t)stream);
}

}  // extern "C"
