// The C ABI's argument checks (mxfp8_block_scaled_gemm_amd/csrc/validate.cpp)
// driven through the rejection and acceptance cases of the ABI tests, built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py.  Pointers are fake addresses that are never
// dereferenced.  Extreme strides and sizes check that no size product
// overflows.  Prints each mismatch and exits non-zero if any.
#include <cmath>
#include <cstdio>
#include <limits>

#include "validate.hpp"

namespace c = mxg::check;

static int failures = 0;
static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    std::printf("line %d: %s -> %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

template <class T>
static T* P(int k) {                                     // 16-byte aligned fake address
  return reinterpret_cast<T*>((uintptr_t)0x10000 * (uintptr_t)(k + 1));
}
template <class T>
static T* Off(int k, int bytes) {
  return reinterpret_cast<T*>((uintptr_t)0x10000 * (uintptr_t)(k + 1) + (uintptr_t)bytes);
}

static mxg_weight W(int k, int64_t N, int64_t K) { return mxg_weight{P<uint8_t>(k), P<uint8_t>(k + 1), N, K}; }

int main() {
  const int64_t big = std::numeric_limits<int64_t>::max();
  const uint16_t* x = P<const uint16_t>(0);
  const uint8_t *aq = P<const uint8_t>(1), *as = P<const uint8_t>(2), *wq = P<const uint8_t>(3),
                *ws = P<const uint8_t>(4);
  const uint16_t* out = P<const uint16_t>(5);

  // mxfp8_gemm arguments
  EXPECT(c::gemm(4, 1024, 2048, nullptr, 0, aq, as, wq, ws, out), MXG_OK);
  EXPECT(c::gemm(4, 1024, 2048, x, 2048, aq, as, wq, ws, out), MXG_OK);
  EXPECT(c::gemm(4, 1024, 2048, nullptr, 0, nullptr, as, wq, ws, out), MXG_ERR_NULL);
  EXPECT(c::gemm(4, 1024, 2048, nullptr, 0, aq, as, wq, nullptr, out), MXG_ERR_NULL);
  EXPECT(c::gemm(0, 1024, 2048, nullptr, 0, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(257, 1024, 2048, nullptr, 0, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(-1, 1024, 2048, nullptr, 0, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(4, 1024, 100, nullptr, 0, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(4, 128, 16384 + 128, nullptr, 0, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(4, 1000, 2048, nullptr, 0, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(4, big, big, nullptr, 0, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(big, 1024, 2048, nullptr, 0, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(4, 1024, 2048, x, 1024, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(4, 1024, 2048, x, big, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(256, 1024, 2048, x, big / 2, aq, as, wq, ws, out), MXG_ERR_SHAPE);
  EXPECT(c::gemm(4, 1024, 2048, nullptr, 0, Off<const uint8_t>(1, 8), as, wq, ws, out), MXG_ERR_ALIGN);
  EXPECT(c::gemm(4, 1024, 2048, nullptr, 0, aq, as, Off<const uint8_t>(3, 1), ws, out), MXG_ERR_ALIGN);
  EXPECT(c::gemm(4, 1024, 2048, Off<const uint16_t>(0, 2), 2048, aq, as, wq, ws, out), MXG_ERR_ALIGN);
  EXPECT(c::gemm(4, 1024, 2048, x, 2052, aq, as, wq, ws, out), MXG_ERR_ALIGN);
  EXPECT(c::workspace(nullptr, 0, 0), MXG_OK);
  EXPECT(c::workspace(nullptr, 0, 65536), MXG_ERR_WORKSPACE);
  EXPECT(c::workspace(P<void>(7), 16, 65536), MXG_ERR_WORKSPACE);
  EXPECT(c::workspace(Off<void>(7, 4), 1 << 30, 65536), MXG_ERR_ALIGN);
  EXPECT(c::workspace(P<void>(7), 1 << 30, 65536), MXG_OK);

  // mxfp8_quantize
  EXPECT(c::quantize(x, 4, 64, 64, P<uint8_t>(1), P<uint8_t>(2)), MXG_OK);
  EXPECT(c::quantize(nullptr, 4, 64, 64, P<uint8_t>(1), P<uint8_t>(2)), MXG_ERR_NULL);
  EXPECT(c::quantize(x, 0, 64, 64, P<uint8_t>(1), P<uint8_t>(2)), MXG_ERR_SHAPE);
  EXPECT(c::quantize(x, 4, 48, 64, P<uint8_t>(1), P<uint8_t>(2)), MXG_ERR_SHAPE);
  EXPECT(c::quantize(x, 4, 64, 32, P<uint8_t>(1), P<uint8_t>(2)), MXG_ERR_SHAPE);
  EXPECT(c::quantize(x, 1 << 20, 64, big, P<uint8_t>(1), P<uint8_t>(2)), MXG_ERR_SHAPE);
  EXPECT(c::quantize(x, big, big, big, P<uint8_t>(1), P<uint8_t>(2)), MXG_ERR_SHAPE);
  EXPECT(c::quantize(Off<const uint16_t>(0, 2), 4, 64, 64, P<uint8_t>(1), P<uint8_t>(2)), MXG_ERR_ALIGN);
  EXPECT(c::quantize(x, 4, 64, 68, P<uint8_t>(1), P<uint8_t>(2)), MXG_ERR_ALIGN);

  // mxfp8_rmsnorm_quantize
  const uint16_t* g = P<const uint16_t>(1);
  const uint16_t* y = P<const uint16_t>(2);
  uint8_t *q = P<uint8_t>(3), *s = P<uint8_t>(4);
  EXPECT(c::rmsnorm(x, 4, 1536, 2048, g, 1e-6f, y, 1536, q, s, 0), MXG_OK);
  EXPECT(c::rmsnorm(x, 4, 1536, 2048, g, 1e-6f, nullptr, 0, q, s, 1), MXG_OK);
  EXPECT(c::rmsnorm(nullptr, 4, 1536, 2048, g, 1e-6f, y, 1536, q, s, 0), MXG_ERR_NULL);
  EXPECT(c::rmsnorm(x, 4, 1536, 2048, nullptr, 1e-6f, y, 1536, q, s, 0), MXG_ERR_NULL);
  EXPECT(c::rmsnorm(x, 0, 1536, 2048, g, 1e-6f, y, 1536, q, s, 0), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 65536, 1536, 2048, g, 1e-6f, y, 1536, q, s, 0), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 4, 1600, 2048, g, 1e-6f, y, 1600, q, s, 0), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 4, 1536, 1024, g, 1e-6f, y, 1536, q, s, 0), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 65535, 1536, big, g, 1e-6f, y, 1536, q, s, 0), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 65535, 1536, 2048, g, 1e-6f, y, big, q, s, 0), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 4, 1536, 2048, g, -1.f, y, 1536, q, s, 0), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 4, 1536, 2048, g, std::nanf(""), y, 1536, q, s, 0), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 4, 1536, 2048, g, INFINITY, y, 1536, q, s, 0), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 4, 1536, 2048, g, 1e-6f, y, 1536, q, s, 2), MXG_ERR_SHAPE);
  EXPECT(c::rmsnorm(x, 4, 1536, 2052, g, 1e-6f, y, 1536, q, s, 0), MXG_ERR_ALIGN);
  EXPECT(c::rmsnorm(x, 4, 1536, 2048, g, 1e-6f, Off<const uint16_t>(2, 2), 1536, q, s, 0), MXG_ERR_ALIGN);

  // mxfp8_pack_weights, the read probe
  EXPECT(c::pack(aq, as, 4096, 5120, P<uint8_t>(8), P<uint8_t>(9)), MXG_OK);
  EXPECT(c::pack(aq, as, 4096, 5120, nullptr, P<uint8_t>(9)), MXG_ERR_NULL);
  EXPECT(c::pack(aq, as, 4100, 5120, P<uint8_t>(8), P<uint8_t>(9)), MXG_ERR_SHAPE);
  EXPECT(c::pack(aq, as, big, big, P<uint8_t>(8), P<uint8_t>(9)), MXG_ERR_SHAPE);
  EXPECT(c::pack(aq, as, 4096, 5120, Off<uint8_t>(8, 4), P<uint8_t>(9)), MXG_ERR_ALIGN);

  // mxfp8_proj_chain
  mxg_chain ch{};
  ch.M = 8;
  ch.a_q = P<uint8_t>(0); ch.a_s = P<uint8_t>(1);
  ch.wA = W(2, 2048, 5120); ch.wB = W(4, 8192, 1536); ch.wC = W(6, 5120, 8192);
  ch.out_a = P<uint16_t>(8); ch.b_q = P<uint8_t>(9); ch.b_s = P<uint8_t>(10);
  ch.out_b = P<uint16_t>(11); ch.c_q = P<uint8_t>(12); ch.c_s = P<uint8_t>(13);
  ch.out_c = P<uint16_t>(14);
  EXPECT(c::chain(&ch), MXG_OK);
  EXPECT(c::chain(nullptr), MXG_ERR_NULL);
  { mxg_chain b = ch; b.M = 0; EXPECT(c::chain(&b), MXG_ERR_SHAPE); }
  { mxg_chain b = ch; b.M = 49; EXPECT(c::chain(&b), MXG_ERR_SHAPE); }
  { mxg_chain b = ch; b.out_b = nullptr; EXPECT(c::chain(&b), MXG_ERR_NULL); }
  { mxg_chain b = ch; b.wB = W(4, 8192, 100); EXPECT(c::chain(&b), MXG_ERR_SHAPE); }
  { mxg_chain b = ch; b.wB = W(4, 8192, 4096); EXPECT(c::chain(&b), MXG_ERR_SHAPE); }
  { mxg_chain b = ch; b.wC = W(6, big, big); EXPECT(c::chain(&b), MXG_ERR_SHAPE); }
  { mxg_chain b = ch; b.a_q = Off<uint8_t>(0, 8); EXPECT(c::chain(&b), MXG_ERR_ALIGN); }
  { mxg_chain b = ch; b.norm_weight = P<uint16_t>(16); b.norm_eps = -1.f; EXPECT(c::chain(&b), MXG_ERR_SHAPE); }
  { mxg_chain b = ch; b.norm_weight = P<uint16_t>(16); b.norm_eps = std::nanf(""); EXPECT(c::chain(&b), MXG_ERR_SHAPE); }
  { mxg_chain b = ch; b.norm_weight = Off<uint16_t>(16, 2); EXPECT(c::chain(&b), MXG_ERR_ALIGN); }
  { mxg_chain b = ch; b.norm_weight = P<uint16_t>(16); b.b_bf16 = Off<uint16_t>(17, 4); EXPECT(c::chain(&b), MXG_ERR_ALIGN); }

  // wo_a_fused_quantize
  mxg_wo_a wa{};
  wa.M = 4; wa.o = P<uint16_t>(0); wa.ld_row = 64 * 512; wa.ld_head = 512;
  wa.positions = P<int64_t>(2); wa.cos_sin = P<float>(3); wa.max_pos = 65536;
  wa.n_heads = 64; wa.head_dim = 512; wa.nope_dim = 448; wa.n_groups = 8;
  wa.wa = W(4, 8192, 4096); wa.z = P<uint16_t>(6); wa.z_q = P<uint8_t>(7); wa.z_s = P<uint8_t>(8);
  wa.wb = W(9, 5120, 8192); wa.out = P<uint16_t>(11);
  EXPECT(c::wo_a(&wa), MXG_OK);
  EXPECT(c::wo_a(nullptr), MXG_ERR_NULL);
  { mxg_wo_a b = wa; b.positions = nullptr; EXPECT(c::wo_a(&b), MXG_ERR_NULL); }
  { mxg_wo_a b = wa; b.out = nullptr; EXPECT(c::wo_a(&b), MXG_ERR_NULL); }
  { mxg_wo_a b = wa; b.M = 49; EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.n_groups = 7; EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.nope_dim = 512; EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.ld_head = 256; EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.ld_head = big; EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.ld_row = big; EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.max_pos = 0; EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.max_pos = big; EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.wa = W(4, 8192, 2048); EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.wb = W(9, 5120, 4096); EXPECT(c::wo_a(&b), MXG_ERR_SHAPE); }
  { mxg_wo_a b = wa; b.o = Off<uint16_t>(0, 8); EXPECT(c::wo_a(&b), MXG_ERR_ALIGN); }
  { mxg_wo_a b = wa; b.positions = Off<int64_t>(2, 4); EXPECT(c::wo_a(&b), MXG_ERR_ALIGN); }
  { mxg_wo_a b = wa; b.ld_head = 516; b.ld_row = 64 * 516; EXPECT(c::wo_a(&b), MXG_ERR_ALIGN); }

  // exported helpers
  if (mxg_scale_bytes_128x4(129, 1536) != 256 * 48 || mxg_scale_bytes_128x4(0, 1536) != 0) {
    std::printf("mxg_scale_bytes_128x4 mismatch\n");
    ++failures;
  }
  for (int st = -1; st < 8; ++st)
    if (!mxg_strerror(st)) ++failures;
  std::printf("validators: %d mismatches\n", failures);
  return failures ? 1 : 0;
}
