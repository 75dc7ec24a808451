// Host side of the stage programs: splitting stages into units, balancing
// them over the grid, and carving the workspace (counters and K-split
// partials).
#include <algorithm>
#include <atomic>

#include "mx_stages.hpp"

namespace mxg {

namespace {

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// LDS bytes of a GEMM unit's staged activations (codes, scales) for Sp steps.
size_t act_lds(int M, int Sp) { return (size_t)M * (Sp * 128 + 16); }
size_t scl_lds(int M, int Sp) { return ((size_t)M * (Sp * 4 + 4) + 15) & ~(size_t)15; }
size_t red_lds(int MB) { return (size_t)kStageStreamWaves * MB * 64 * 16; }

}  // namespace

int choose_kparts(int M, int N, int K, int G) {
  const int S = K / 128, tiles = N / 16, MB = (M + 15) / 16;
  int best = -1;
  long best_cost = 0;
  for (int P = 1; P <= 16; P *= 2) {
    if (P > S) break;
    const int Sp = ceil_div(S, P);
    if (Sp > kStageStreamWaves * kStageStepsPerWave) continue;
    if (act_lds(M, Sp) + scl_lds(M, Sp) + red_lds(MB) > (size_t)kStageLdsMax) continue;
    // weight steps the busiest workgroup streams, plus a per-unit overhead
    const long cost = (long)ceil_div(tiles * P, G) * (Sp + 2);
    if (best < 0 || cost < best_cost) {
      best = P;
      best_cost = cost;
    }
  }
  return best;
}

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

ProgramBuilder::ProgramBuilder(int M, int G, uint8_t* ws)
    : M_(M), ws_(ws), ctr_off_(kTileCtrBase), off_(kCtrRegionBytes) {
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

int ProgramBuilder::add_quant(const uint16_t* x, int ld_x, int K, uint8_t* q, uint8_t* s,
                              int dep) {
  StageDesc& d = pg_.st[pg_.nstages];
  d = StageDesc{};
  d.kind = kStageQuant;
  d.dep = dep;
  d.M = M_;
  d.x = x;
  d.ld_x = ld_x;
  d.qK = K;
  d.q = q;
  d.s = s;
  d.units = ceil_div(M_ * (K / 32), 64);
  return pg_.nstages++;
}

int ProgramBuilder::add_gemm(int N, int K, const uint8_t* wq, const uint8_t* wsc,
                             const uint8_t* aq, const uint8_t* as, int groups, int64_t a_gs_q,
                             int64_t a_gs_s, uint16_t* out, int ld_out, int dep) {
  StageDesc& d = pg_.st[pg_.nstages];
  d = StageDesc{};
  d.kind = kStageGemm;
  d.dep = dep;
  d.M = M_;
  d.N = N;
  d.K = K;
  d.tiles = N / 16;
  d.group_tiles = d.tiles / groups;
  d.wq = wq;
  d.ws = wsc;
  d.aq = aq;
  d.as = as;
  d.a_gs_q = a_gs_q;
  d.a_gs_s = a_gs_s;
  d.out = out;
  d.ld_out = ld_out;
  d.P = std::max(1, choose_kparts(M_, N, K, pg_.G));
  d.Sp = ceil_div(K / 128, d.P);
  d.units = d.tiles * d.P;
  if (d.P > 1) {
    d.tile_ctr = carve_counters((size_t)d.tiles);
    d.part = reinterpret_cast<float*>(carve((size_t)d.tiles * d.P * mb() * 64 * 16));
  }
  return pg_.nstages++;
}

bool ProgramBuilder::finish() {
  if (ctr_overflow_) return false;
  size_t act = 0, scl = 0;
  int rot = 0;
  for (int i = 0; i < pg_.nstages; ++i) {
    StageDesc& d = pg_.st[i];
    if (d.kind == kStageGemm) {
      if (choose_kparts(M_, d.N, d.K, pg_.G) < 0) return false;
      act = std::max(act, act_lds(M_, d.Sp));
      scl = std::max(scl, scl_lds(M_, d.Sp));
    }
    // Rotate each stage's start so that the workgroups left with one unit
    // more in one stage are not the same ones in the next.
    d.rot = rot;
    rot = (rot + d.units) % pg_.G;
    // Workgroups b with units in this stage: (b - rot) mod G < units.
    for (int x = 0; x < kGroups; ++x) d.arrive_target[x] = 0;
    for (int b = 0; b < pg_.G; ++b) {
      const int f = ((b - d.rot) % pg_.G + pg_.G) % pg_.G;
      if (f < d.units) ++d.arrive_target[b % kGroups];
    }
    if (d.dep >= 0) {
      pg_.st[d.dep].consumed = 1;
      pg_.synced = 1;
    }
  }
  pg_.lds_act_bytes = (int)((act + 15) & ~(size_t)15);
  pg_.lds_scl_bytes = (int)scl;
  return (size_t)pg_.lds_act_bytes + pg_.lds_scl_bytes + red_lds(mb()) <= (size_t)kStageLdsMax;
}

}  // namespace mxg
