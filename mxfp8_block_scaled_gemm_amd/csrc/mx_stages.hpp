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
constexpr int kStageStepsPerWave = 4;   // 128-K steps a stream wave holds per unit
constexpr int kMaxStages = 4;
constexpr int kStageLdsMax = 160 * 1024 - 64;   // dynamic LDS; a few static words follow

constexpr int kStageQuant = 1;          // BF16 -> MXFP8 of a row range
constexpr int kStageGemm = 2;           // (grouped) MXFP8 GEMM, BF16 out

// Workspace layout: a fixed counter region, then K-split partial sums.
//   word 5 (byte 20)          error word (an expired wait sets it)
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

struct StageDesc {
  int kind, dep, units, rot;
  int consumed;                // a later stage reads this stage's output
  uint16_t arrive_target[kGroups];  // workgroups of each group with units here
  // GEMM
  int M, N, K, P, Sp, tiles, group_tiles;
  const uint8_t* wq;           // packed weight codes (all groups, N rows)
  const uint8_t* ws;           // packed weight scales
  const uint8_t* aq;           // activation codes [M, K] of group 0
  const uint8_t* as;           // activation scales [M, K/32] of group 0
  int64_t a_gs_q, a_gs_s;      // bytes between consecutive groups' activations
  uint16_t* out;               // BF16 [M, ld_out]; tile t writes columns [16t, 16t+16)
  int ld_out;
  float* part;                 // K-split partials [tiles][P][MB*64] v4f (P > 1)
  uint32_t* tile_ctr;          // K-split arrival counters [tiles] (P > 1)
  // QUANT: rows [0, M) of x, columns [0, qK) -> q [M, qK], s [M, qK/32]
  const uint16_t* x;
  int ld_x, qK;
  uint8_t* q;
  uint8_t* s;
};

struct Program {
  int nstages, G;
  int synced;                  // some stage is consumed: arrivals and exit counting run
  int lds_act_bytes, lds_scl_bytes;
  uint8_t* ws;                 // workspace (counter region first)
  StageDesc st[kMaxStages];
};

// Builds a program; with a null workspace it only measures the bytes needed.
class ProgramBuilder {
 public:
  ProgramBuilder(int M, int G, uint8_t* ws);
  // Returns the stage index.
  int add_quant(const uint16_t* x, int ld_x, int K, uint8_t* q, uint8_t* s, int dep);
  int add_gemm(int N, int K, const uint8_t* wq, const uint8_t* wsc, const uint8_t* aq,
               const uint8_t* as, int groups, int64_t a_gs_q, int64_t a_gs_s, uint16_t* out,
               int ld_out, int dep);
  // Assigns unit rotations and LDS sizes; returns false if a stage cannot run.
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
  uint8_t* carve(size_t bytes);
  uint32_t* carve_counters(size_t n);
};

// K parts per 16-row tile for a GEMM stage of this shape on G workgroups.
int choose_kparts(int M, int N, int K, int G);

// Workgroups the stage kernel runs with on the current device (one per CU).
int stage_grid();

hipError_t launch_program(const Program& pg, int MB, hipStream_t stream);

}  // namespace mxg
