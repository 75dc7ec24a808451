// Stage programs run by the persistent stage kernel (stages.hip), and the
// host-side builder that lays them out over the grid and the workspace.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxg {

constexpr int kStageStreamWaves = 12;   // weight stream + MFMA waves
constexpr int kStageIoWaves = 4;        // dependency / activation / output waves
constexpr int kStageThreads = (kStageStreamWaves + kStageIoWaves) * 64;
constexpr int kMaxStages = 4;
constexpr int kStageLdsMax = 160 * 1024 - 64;   // dynamic LDS; a few static words follow

// How a GEMM stage gets its MXFP8 activations (staged into LDS per segment).
constexpr int kActMx = 0;     // MXFP8 codes + scales in memory
constexpr int kActBf16 = 1;   // BF16 in memory, quantized while staging
constexpr int kActRope = 2;   // BF16 attention heads: rotary on the last dims, then quantized

// Workspace layout: a fixed counter region, then K-split partial sums.
//   word 5 (byte 20)          error word (an expired wait sets bit 0)
//   kArriveBase + (s*8+x)*128 arrivals of workgroup group x (b mod 8) that
//                             finished stage s, one 128-byte line each
//   kExitBase + x*128         exits of group x;  kExitTop: groups done
//   kTileCtrBase ..           K-split tile counters
// Arrivals are spread over 8 lines because same-address device atomics
// serialize.  Every counter is back at zero when a call ends, and no program
// puts partial sums in the counter region, so programs of any shape can
// share a workspace one after another.
constexpr int kGroups = 8;
constexpr int kCtrError = 5;
constexpr size_t kArriveBase = 256;
constexpr size_t kExitBase = kArriveBase + (size_t)kMaxStages * kGroups * 128;
constexpr size_t kExitTop = kExitBase + (size_t)kGroups * 128;
constexpr size_t kTileCtrBase = 8192;
constexpr size_t kCtrBytes = kTileCtrBase;
constexpr size_t kCtrRegionBytes = 64 * 1024;

// One GEMM stage: out[M, N] = dequant(act) . dequant(W)^T.
// Work units are (16-row weight tile t, K part p) in part-major order
// v = p * tiles + t; part p covers 128-wide K steps [p*Sp, min(S, p*Sp+Sp)).
// A "segment" is the activation block one unit reads: (part, group).
struct StageDesc {
  int dep;                     // stage whose output the activations read (-1: none)
  int consumed;                // a later stage depends on this one
  int M, N, K, S;              // S = K / 128
  int tiles, P, Sp, units, rot;
  int uq, ur;                  // units / G, units % G (workgroup f from rot takes uq, +1 if f < ur)
  int group_tiles;             // weight tiles per activation group
  uint16_t arrive_target[kGroups];  // workgroups of each group with units here
  const uint8_t* wq;           // packed weight codes (mxfp8_pack_weights order)
  const uint8_t* ws;           // packed weight scales
  int act;                     // kActMx / kActBf16 / kActRope
  // kActMx: codes of row m, group g, column k at aq + g*a_group + m*lda + k;
  // scale bytes at as + (g*a_group + m*lda + k) / 32.
  const uint8_t* aq;
  const uint8_t* as;
  int64_t lda, a_group;
  // kActBf16: x + g*a_group + m*ld_x + k.  kActRope: group g is heads
  // g*hpg .. g*hpg + hpg - 1 (hpg = K / D), head h of row m at
  // x + m*ld_x + h*ld_head, its last D - nope dims rotated by positions[m].
  const uint16_t* x;
  int64_t ld_x, ld_head;
  int D, nope;
  const int64_t* positions;
  const float* cos_sin;
  int64_t max_pos;
  // kActBf16 / kActRope: the codes of each segment are also written, by the
  // workgroup that owns the segment's first unit: q + m*ldq + g*K + k and
  // s + (m*ldq + g*K + k) / 32 (q may be null).
  uint8_t* q;
  uint8_t* s;
  int64_t ldq;
  uint16_t* out;               // BF16 [M, ld_out]; tile t writes columns [16t, 16t+16)
  int ld_out;
  float* part;                 // K-split partials [tiles][P][MB*64] v4f (P > 1)
  uint32_t* tile_ctr;          // K-split arrival counters [tiles] (P > 1)
};

struct Program {
  int nstages, G;
  int synced;                  // some stage is consumed: arrivals and exit counting run
  int act_ld, scl_ld;          // LDS bytes per activation row (codes, scales), max over stages
  uint8_t* ws;                 // workspace (counter region first)
  StageDesc st[kMaxStages];
};

// LDS bytes of the stage kernel for a program with MB 16-row activation tiles.
size_t stage_lds_bytes(const Program& pg, int MB);

// Builds a program; with a null workspace it only measures the bytes needed.
// K-split partials are carved from data_start on (the counter region comes
// first in every workspace).
class ProgramBuilder {
 public:
  ProgramBuilder(int M, int G, uint8_t* ws, size_t data_start = kCtrRegionBytes);
  // Adds a GEMM stage (its K split chosen here); returns its index.  The
  // activation source fields default to MXFP8 with lda = K and are set by
  // the caller through stage().  act, D and nope size the LDS.
  int add_gemm(int N, int K, const uint8_t* wq, const uint8_t* wsc, int dep, uint16_t* out,
               int ld_out, int act = kActMx, int D = 0, int nope = 0);
  StageDesc& stage(int i) { return pg_.st[i]; }
  // Assigns unit rotations, arrival targets and LDS sizes; false if a stage
  // cannot run.
  bool finish();
  size_t workspace_bytes() const { return off_; }
  int mb() const { return (M_ + 15) / 16; }
  const Program& program() const { return pg_; }

 private:
  Program pg_;
  int M_;
  uint8_t* ws_;
  size_t ctr_off_, off_;
  bool ctr_overflow_ = false;
  bool bad_ = false;
  uint8_t* carve(size_t bytes);
  uint32_t* carve_counters(size_t n);
};

// Workgroups the stage kernel runs with on the current device (one per CU).
int stage_grid();

hipError_t launch_program(const Program& pg, int MB, hipStream_t stream);

}  // namespace mxg
