// Host side of the stage programs: splitting stages into units, balancing
// them over the grid, and carving the workspace (counters and K-split
// partials).
#include <algorithm>
#include <atomic>

#include "mx_stages.hpp"

namespace mxg {

namespace {

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// LDS bytes of a stage whose segments are Sp steps long: one activation
// buffer (codes, scales) plus the two alternating partial-tile buffers.
size_t stage_lds(int M, int Sp, int MB) {
  return (size_t)M * (Sp * 128 + 16) + (((size_t)M * (Sp * 4 + 4) + 15) & ~(size_t)15) +
         (size_t)2 * kStageStreamWaves * MB * 64 * 16;
}

// K parts per 16-row tile: the split whose busiest workgroup streams the
// fewest weight steps, counting a small cost per unit and the latency of
// the cross-workgroup partial sum when P > 1.  -1 if nothing fits in LDS.
int choose_kparts(int M, int N, int K, int G, size_t extra_lds) {
  const int S = K / 128, tiles = N / 16, MB = (M + 15) / 16;
  int best = -1;
  long best_cost = 0;
  for (int P = 1; P <= 64; P *= 2) {
    if (P > S) break;
    const int Sp = ceil_div(S, P);
    if (stage_lds(M, Sp, MB) + extra_lds > (size_t)kStageLdsMax) continue;
    const long cost = (long)ceil_div(tiles * P, G) * (Sp + 2) + (P > 1 ? 8 : 0);
    if (best < 0 || cost < best_cost) {
      best = P;
      best_cost = cost;
    }
  }
  return best;
}

}  // namespace

int stage_grid() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int g = cached[dev].load(std::memory_order_relaxed);
  if (g == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    g = cus;   // one 1024-thread workgroup per CU: all co-resident
    cached[dev].store(g, std::memory_order_relaxed);
  }
  return g;
}

ProgramBuilder::ProgramBuilder(int M, int G, uint8_t* ws, size_t data_start)
    : M_(M), ws_(ws), ctr_off_(kTileCtrBase), off_(std::max(data_start, kCtrRegionBytes)) {
  pg_ = Program{};
  pg_.G = G;
  pg_.ws = ws;
}

uint32_t* ProgramBuilder::carve_counters(size_t n) {
  uint32_t* p = ws_ ? reinterpret_cast<uint32_t*>(ws_ + ctr_off_) : nullptr;
  ctr_off_ += n * 4;
  if (ctr_off_ > kCtrRegionBytes) ctr_overflow_ = true;
  return p;
}

uint8_t* ProgramBuilder::carve(size_t bytes) {
  off_ = (off_ + 255) & ~(size_t)255;
  uint8_t* p = ws_ ? ws_ + off_ : nullptr;
  off_ += bytes;
  return p;
}

int ProgramBuilder::add_gemm(int N, int K, const uint8_t* wq, const uint8_t* wsc, int dep,
                             uint16_t* out, int ld_out, int act, int D, int nope) {
  StageDesc& d = pg_.st[pg_.nstages];
  d = StageDesc{};
  d.dep = dep;
  d.M = M_;
  d.N = N;
  d.K = K;
  d.S = K / 128;
  d.tiles = N / 16;
  d.group_tiles = d.tiles;
  d.wq = wq;
  d.ws = wsc;
  d.act = act;
  d.lda = K;
  d.D = D;
  d.nope = nope;
  d.out = out;
  d.ld_out = ld_out;
  const size_t extra = act == kActRope ? (size_t)M_ * (D - nope) * 4 : 0;
  d.P = choose_kparts(M_, N, K, pg_.G, extra);
  if (d.P < 0) {
    bad_ = true;
    d.P = 1;
  }
  d.Sp = (d.S + d.P - 1) / d.P;
  d.units = d.tiles * d.P;
  if (d.P > 1) {
    d.tile_ctr = carve_counters((size_t)d.tiles);
    d.part = reinterpret_cast<float*>(carve((size_t)d.tiles * d.P * mb() * 64 * 16));
  }
  return pg_.nstages++;
}

bool ProgramBuilder::finish() {
  if (ctr_overflow_ || bad_ || pg_.nstages == 0) return false;
  int rot = 0, act_ld = 0, scl_ld = 0;
  for (int i = 0; i < pg_.nstages; ++i) {
    StageDesc& d = pg_.st[i];
    if (d.tiles % d.group_tiles != 0) return false;
    act_ld = std::max(act_ld, d.Sp * 128 + 16);
    scl_ld = std::max(scl_ld, d.Sp * 4 + 4);
    // Rotate each stage's ranges so that the workgroups holding one unit
    // more in one stage are not the same ones in the next.
    d.rot = rot;
    rot = (rot + d.units) % pg_.G;
    // Workgroup b, f = (b - rot) mod G places from the rotation, takes the
    // units [f*uq + min(f, ur), ...) of count uq + (f < ur): the workgroups
    // with units are those with uq > 0 or f < ur.
    d.uq = d.units / pg_.G;
    d.ur = d.units % pg_.G;
    for (int x = 0; x < kGroups; ++x) d.arrive_target[x] = 0;
    for (int b = 0; b < pg_.G; ++b) {
      const int f = ((b - d.rot) % pg_.G + pg_.G) % pg_.G;
      if (d.uq > 0 || f < d.ur) ++d.arrive_target[b % kGroups];
    }
    if (d.dep >= 0) {
      pg_.st[d.dep].consumed = 1;
      pg_.synced = 1;
    }
  }
  pg_.act_ld = act_ld;
  pg_.scl_ld = scl_ld;
  return stage_lds_bytes(pg_, mb()) <= (size_t)kStageLdsMax;
}

}  // namespace mxg
