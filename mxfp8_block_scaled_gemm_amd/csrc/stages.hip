// Persistent stage-program kernel: a short program of dependent stages
// (activation quantize, MXFP8 GEMM, grouped GEMM, requantize) run by one
// launch of one workgroup per CU.
//
// Why: a single small-row GEMM streams 2-40 MB of weights and a launch costs
// about as much as streaming a few MB, and the decode step runs several
// projections back to back ([step] page, AttentionStep: fused_wqa_wkv, wq_b,
// wo_b; [mxfp8] page: the low-latency kernel loads its weights before its
// grid dependency wait so the weight read overlaps the previous kernel).
// Here every stage's weight stream is independent of the data, so the weight
// loads of the next unit are always in flight while the current unit waits
// for its input; only the activations wait for the previous stage.
//
// Workgroup = 16 waves:
//   waves 0..11  "stream" waves: weight loads (packed tile order, predicated
//                by buffer ranges, non-temporal) for the current and the next
//                unit, and the scaled MFMAs;
//   waves 12..15 "io" waves: dependency waits, activation staging into LDS
//                (or quantizing a BF16 input), the reduction of the 12 partial
//                tiles, the BF16 output or the K-split partial, and
//                publishing completion.
// Splitting the roles keeps each wave's in-order load counter free of the
// other role's loads, so no stream wave ever waits for an activation and no
// activation waits behind a weight.
//
// Work units: a GEMM stage is cut into (16-row weight tile) x (K part) units;
// a quantize stage into 64-block chunks.  Unit u of stage s runs on
// workgroup (u + rot_s) mod G, every workgroup taking its units stage by
// stage.  A tile cut into P > 1 K parts is finished by whichever part
// arrives last, which sums the P FP32 partials in part order (the result
// does not depend on arrival order).
//
// Cross-workgroup data (quantized activations, outputs read by a later
// stage, K-split partials) is written and read device-coherent (sc1), and a
// workgroup counts one arrival per stage on one of 8 counters (same-address
// device atomics serialize, so arrivals are spread over 8 lines); a
// dependent stage's io wave polls the 8 counters.  Every spin is bounded (an
// expired wait sets the workspace's error word and lets the kernel finish).
// The last workgroup out resets the counters, so a zeroed workspace stays
// valid for the next call.  Dependencies only point to earlier stages and
// the grid never exceeds the number of co-resident workgroups, so every wait
// is satisfied.
#include "mx_device.hpp"
#include "mx_launch.hpp"
#include "mx_stages.hpp"

namespace mxg {

namespace {

constexpr int kStream = kStageStreamWaves;      // 12
constexpr int kIo = kStageIoWaves;              // 4
constexpr int kIoThreads = kIo * 64;
constexpr int kSPW = kStageStepsPerWave;        // 4
constexpr uint32_t kSpinLimit = 1u << 20;       // polls (with sleeps): well under a second
constexpr int kCoherent = 16;                   // sc1: device-coherent access

__device__ __forceinline__ uint32_t* ctr_word(const Program& pg, size_t byte_off) {
  return reinterpret_cast<uint32_t*>(pg.ws + byte_off);
}
__device__ __forceinline__ uint32_t* arrive_word(const Program& pg, int s, int x) {
  return ctr_word(pg, kArriveBase + ((size_t)s * kGroups + x) * 128);
}

// Device-coherent (sc1) buffer accesses for data that crosses workgroups
// within a launch: written through and read past the per-XCD caches, so a
// plain store + s_waitcnt before the arrival counter replaces a full L2
// write-back fence.
__device__ __forceinline__ v4i ld16_c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherent));
}
__device__ __forceinline__ uint32_t ld4_c(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kCoherent);
}
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st16_c(__amdgpu_buffer_rsrc_t r, uint32_t off, v4i v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, (int)off, 0, kCoherent);
}
__device__ __forceinline__ void st8_c(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v2u{v.x, v.y}, r, (int)off, 0, kCoherent);
}
__device__ __forceinline__ void st1_c(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, (int)off, 0, kCoherent);
}

// Workgroup barrier that orders LDS only: outstanding global loads (the
// weight stream) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier among the 4 io waves only (an LDS counter that only grows during
// the launch; the k-th use waits for 4k arrivals, one per wave).
__device__ __forceinline__ void io_sync(uint32_t* bar, uint32_t& k, int lane) {
  ++k;
  if (lane == 0) __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kIo * k)
    __builtin_amdgcn_s_sleep(1);
}

// Wait until every group's arrival count for stage d reached its target
// (io wave 0 polls, lanes 0..7 one group each; the others wait in io_sync).
__device__ void wait_stage(const Program& pg, int d, int iw, int lane, uint32_t* bar,
                           uint32_t& k) {
  if (iw == 0) {
    const StageDesc& sd = pg.st[d];
    uint32_t target = lane < kGroups ? sd.arrive_target[lane] : 0;
    const uint32_t* w = arrive_word(pg, d, lane < kGroups ? lane : 0);
    uint32_t it = 0;
    while (true) {
      const uint32_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__builtin_amdgcn_ballot_w64(lane < kGroups && v < target) == 0) break;
      if (++it > kSpinLimit) {
        if (lane == 0)
          __hip_atomic_fetch_or(ctr_word(pg, kCtrError * 4), 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  io_sync(bar, k, lane);
}

// This workgroup finished its units of stage s: once all io waves' stores
// have landed, count one arrival for the workgroup's group.
__device__ void arrive_stage(const Program& pg, int s, int b, int iw, int lane, uint32_t* bar,
                             uint32_t& k) {
  __builtin_amdgcn_s_waitcnt(0);                        // this wave's stores done
  io_sync(bar, k, lane);
  if (iw == 0 && lane == 0)
    __hip_atomic_fetch_add(arrive_word(pg, s, b % kGroups), 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int first_unit(const StageDesc& sd, int b, int G) {
  const int f = (b - sd.rot) % G;
  return f < 0 ? f + G : f;
}

// Unit cursor over the workgroup's units, stage by stage.
struct Cursor {
  int s, u;
};

// Move c to the next unit at or after c (GEMM units only if gemm_only).
__device__ bool seek(const Program& pg, int b, int G, Cursor& c, bool gemm_only) {
  while (c.s < pg.nstages) {
    const StageDesc& sd = pg.st[c.s];
    if ((!gemm_only || sd.kind == kStageGemm) && c.u < sd.units) return true;
    ++c.s;
    if (c.s < pg.nstages) c.u = first_unit(pg.st[c.s], b, G);
  }
  return false;
}

__device__ __forceinline__ Cursor start(const Program& pg, int b, int G) {
  return Cursor{0, first_unit(pg.st[0], b, G)};
}

// K range of a GEMM unit, in 128-wide steps.
struct UnitRange {
  int t, p, k0, k1;
};
__device__ __forceinline__ UnitRange unit_range(const StageDesc& sd, int u) {
  UnitRange r;
  r.t = u / sd.P;
  r.p = u - r.t * sd.P;
  const int S = sd.K >> 7;
  r.k0 = r.p * sd.Sp;
  r.k1 = min(r.k0 + sd.Sp, S);
  return r;
}

struct WeightBuf {
  v4i lo[kSPW], hi[kSPW];
  uint32_t sc[kSPW];
};

// Issue the weight loads of one unit for stream wave w (all slots issued;
// slots beyond the unit's steps are out of range and touch no memory).
__device__ __forceinline__ void load_weights(const StageDesc& sd, int u, bool valid, int w,
                                             int lane, WeightBuf& wb) {
  const int S = sd.K >> 7;
  UnitRange r = unit_range(sd, valid ? u : 0);
  const auto rw = make_rsrc(sd.wq + (int64_t)r.t * S * 2048, (uint32_t)(S * 2048));
  const auto rs = make_rsrc(sd.ws + (int64_t)r.t * S * 64, (uint32_t)(S * 64));
#pragma unroll
  for (int j = 0; j < kSPW; ++j) {
    const int step = r.k0 + w + kStream * j;
    const bool ok = valid && step < r.k1;
    wb.lo[j] = buf_ld16_nt(rw, ok ? (uint32_t)(step * 2048 + lane * 16) : kOutOfRange);
    wb.hi[j] = buf_ld16_nt(rw, ok ? (uint32_t)(step * 2048 + 1024 + lane * 16) : kOutOfRange);
    wb.sc[j] = buf_ld8(rs, ok ? (uint32_t)(step * 64 + lane) : kOutOfRange);
  }
}

struct Lds {
  uint8_t* act;   // [M][Sp*128 + 16] codes of the unit's K range
  uint8_t* scl;   // [M][Sp*4 + 4] scale bytes
  v4f* red;       // [kStream][MB][64] partial tiles
  uint32_t* bar;  // io-wave barrier counter
};

// One GEMM unit on a stream wave: MFMAs over its steps, partial tile to LDS.
template <int MB>
__device__ __forceinline__ void stream_compute(const StageDesc& sd, int u, int w, int lane,
                                               const WeightBuf& wb, Lds& L) {
  const int g = lane >> 4, r = lane & 15;
  const UnitRange ur = unit_range(sd, u);
  const int ldA = sd.Sp * 128 + 16, ldS = sd.Sp * 4 + 4;
  lds_barrier();                                        // B1: activations staged
  v4f acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kSPW; ++j) {
    const int sl = w + kStream * j;                     // step within the unit
    if (ur.k0 + sl < ur.k1) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = 16 * mb + r;
        v4i blo = {0, 0, 0, 0}, bhi = {0, 0, 0, 0};
        int bsc = 0;
        if (m < sd.M) {
          const uint8_t* a = L.act + m * ldA + sl * 128 + 16 * g;
          blo = *reinterpret_cast<const v4i*>(a);
          bhi = *reinterpret_cast<const v4i*>(a + 64);
          bsc = L.scl[m * ldS + 4 * sl + g];
        }
        acc[mb] = mfma_mx16(cat8(wb.lo[j], wb.hi[j]), cat8(blo, bhi), acc[mb], (int)wb.sc[j], bsc);
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) L.red[(w * MB + mb) * 64 + lane] = acc[mb];
  lds_barrier();                                        // B2: partials in LDS
}

template <int MB>
__device__ void stream_loop(const Program& pg, int b, int G, int w, int lane, Lds& L) {
  Cursor cur = start(pg, b, G);
  bool have = seek(pg, b, G, cur, true);
  WeightBuf A, B;
  load_weights(pg.st[have ? cur.s : 0], cur.u, have, w, lane, A);
  while (have) {
    Cursor nx = cur;
    nx.u += G;
    bool hn = seek(pg, b, G, nx, true);
    load_weights(pg.st[hn ? nx.s : 0], nx.u, hn, w, lane, B);
    stream_compute<MB>(pg.st[cur.s], cur.u, w, lane, A, L);
    if (!hn) break;
    cur = nx;
    nx.u += G;
    hn = seek(pg, b, G, nx, true);
    load_weights(pg.st[hn ? nx.s : 0], nx.u, hn, w, lane, A);
    stream_compute<MB>(pg.st[cur.s], cur.u, w, lane, B, L);
    if (!hn) break;
    cur = nx;
  }
}

// ----------------------------------------------------------------- io waves

// Quantize one 64-block chunk of a BF16 matrix (4 lanes per 32-block); the
// codes go out device-coherent, for the stage that reads them.
__device__ void io_quant_unit(const StageDesc& sd, int u, int lt) {
  const int nbr = sd.qK >> 5;                           // blocks per row
  const int total = sd.M * nbr;
  const int blk = u * 64 + (lt >> 2), sub = lt & 3;
  const bool ok = blk < total;
  const int row = ok ? blk / nbr : 0, cb = ok ? blk - row * nbr : 0;
  const auto rx = make_rsrc(sd.x, (uint32_t)(((sd.M - 1) * sd.ld_x + sd.qK) * 2));
  const uint32_t xo = (uint32_t)((row * sd.ld_x + cb * 32 + sub * 8) * 2);
  const v4i v = sd.dep >= 0 ? ld16_c(rx, ok ? xo : kOutOfRange) : buf_ld16(rx, ok ? xo : kOutOfRange);
  uint32_t a = halves_max(bf16x2_absmax2(bf16x2_absmax2((uint32_t)v[0], (uint32_t)v[1]),
                                         bf16x2_absmax2((uint32_t)v[2], (uint32_t)v[3])));
  a = quad_max(a);
  const int e = block_exponent(a);
  const BlockScale bs = block_scale(e);
  if (ok) {
    uint2 c;
    c.x = enc4_e4m3((uint32_t)v[0], (uint32_t)v[1], bs);
    c.y = enc4_e4m3((uint32_t)v[2], (uint32_t)v[3], bs);
    const auto rq = make_rsrc(sd.q, (uint32_t)(sd.M * sd.qK));
    const auto rs = make_rsrc(sd.s, (uint32_t)(sd.M * nbr));
    st8_c(rq, (uint32_t)(row * sd.qK + cb * 32 + sub * 8), c);
    if (sub == 0) st1_c(rs, (uint32_t)(row * nbr + cb), (uint8_t)(e + 127));
  }
}

// Stage a GEMM unit's activations (its K range, all M rows) into LDS;
// activations made earlier in this launch are read device-coherent.
__device__ void io_stage_act(const StageDesc& sd, const UnitRange& ur, int lt, Lds& L) {
  const int ldA = sd.Sp * 128 + 16, ldS = sd.Sp * 4 + 4;
  const int gi = ur.t / sd.group_tiles;
  const int KB = sd.K >> 5;
  const auto ra = make_rsrc(sd.aq + (int64_t)gi * sd.a_gs_q, (uint32_t)(sd.M * sd.K));
  const auto rs = make_rsrc(sd.as + (int64_t)gi * sd.a_gs_s, (uint32_t)(sd.M * KB));
  const bool coh = sd.dep >= 0;
  const int ns = ur.k1 - ur.k0;
  const int cpr = ns * 8;                               // 16-byte chunks per row
  const int nck = sd.M * cpr;
  for (int c = lt; c < nck; c += kIoThreads) {
    const int row = c / cpr, col = (c - row * cpr) * 16;
    const uint32_t off = (uint32_t)(row * sd.K + ur.k0 * 128 + col);
    *reinterpret_cast<v4i*>(L.act + row * ldA + col) = coh ? ld16_c(ra, off) : buf_ld16(ra, off);
  }
  const int nsc = sd.M * ns;                            // scale dwords (4 blocks each)
  for (int c = lt; c < nsc; c += kIoThreads) {
    const int row = c / ns, cd = c - row * ns;
    const uint32_t off = (uint32_t)(row * KB + (ur.k0 + cd) * 4);
    *reinterpret_cast<uint32_t*>(L.scl + row * ldS + cd * 4) =
        coh ? ld4_c(rs, off) : __builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, 0);
  }
}

__device__ __forceinline__ void store_out(const StageDesc& sd, int m, int n, v4f v) {
  uint2 o;
  o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  if (sd.consumed) {
    const auto ro = make_rsrc(sd.out, (uint32_t)(sd.M * sd.ld_out * 2));
    st8_c(ro, (uint32_t)((m * sd.ld_out + n) * 2), o);
  } else {
    *reinterpret_cast<uint2*>(sd.out + (int64_t)m * sd.ld_out + n) = o;
  }
}

template <int MB>
__device__ void io_gemm_unit(const StageDesc& sd, int u, int iw, int lane, Lds& L) {
  const int lt = iw * 64 + lane;
  const UnitRange ur = unit_range(sd, u);
  io_stage_act(sd, ur, lt, L);
  lds_barrier();                                        // B1
  lds_barrier();                                        // B2
  if (iw >= MB) return;                                 // wave iw owns activation tile iw
  // Sum the stream waves' partial tiles in wave order.
  const int mb = iw;
  v4f sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < kStream; ++w) sum += L.red[(w * MB + mb) * 64 + lane];
  const int m = 16 * mb + (lane & 15);
  const int n = 16 * ur.t + 4 * (lane >> 4);
  if (sd.P == 1) {
    if (m < sd.M) store_out(sd, m, n, sum);
    return;
  }
  // K split: park the FP32 partial (device-coherent); the last of the
  // tile's MB*P partial writers sums the P partials in part order.
  const uint32_t tile_bytes = (uint32_t)(sd.P * MB * 64 * 16);
  const auto rp = make_rsrc(reinterpret_cast<uint8_t*>(sd.part) + (int64_t)ur.t * tile_bytes,
                            tile_bytes);
  st16_c(rp, (uint32_t)(((ur.p * MB + mb) * 64 + lane) * 16), __builtin_bit_cast(v4i, sum));
  __builtin_amdgcn_s_waitcnt(0);
  uint32_t old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(sd.tile_ctr + ur.t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old != (uint32_t)(MB * sd.P - 1)) return;
#pragma unroll
  for (int k = 0; k < MB; ++k) {
    v4f tot = __builtin_bit_cast(v4f, ld16_c(rp, (uint32_t)((k * 64 + lane) * 16)));
    for (int p = 1; p < sd.P; ++p)
      tot += __builtin_bit_cast(v4f, ld16_c(rp, (uint32_t)(((p * MB + k) * 64 + lane) * 16)));
    const int mm = 16 * k + (lane & 15);
    if (mm < sd.M) store_out(sd, mm, n, tot);
  }
  if (lane == 0)
    __hip_atomic_store(sd.tile_ctr + ur.t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MB>
__device__ void io_loop(const Program& pg, int b, int G, int iw, int lane, Lds& L) {
  uint32_t k = 0;                                       // io_sync uses so far
  Cursor cur = start(pg, b, G);
  int waited = -1;                                      // stage whose dependency was met
  while (seek(pg, b, G, cur, false)) {
    const StageDesc& sd = pg.st[cur.s];
    if (sd.dep >= 0 && waited != cur.s) {
      wait_stage(pg, sd.dep, iw, lane, L.bar, k);
      waited = cur.s;
    }
    if (sd.kind == kStageGemm)
      io_gemm_unit<MB>(sd, cur.u, iw, lane, L);
    else
      io_quant_unit(sd, cur.u, iw * 64 + lane);
    const int s = cur.s;
    cur.u += G;
    if (sd.consumed && cur.u >= sd.units) arrive_stage(pg, s, b, iw, lane, L.bar, k);
  }
  if (!pg.synced) return;
  // Exit counting: the last workgroup out resets the arrival counters.
  if (iw != 0) return;
  uint32_t last = 0;
  if (lane == 0) {
    const int x = b % kGroups;
    const uint32_t members = (uint32_t)((G - x + kGroups - 1) / kGroups);
    const uint32_t o = __hip_atomic_fetch_add(ctr_word(pg, kExitBase + x * 128), 1u,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (o == members - 1)
      last = __hip_atomic_fetch_add(ctr_word(pg, kExitTop), 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(kGroups - 1);
  }
  last = __builtin_amdgcn_readfirstlane(last);
  if (!last) return;
  for (int i = lane; i < kMaxStages * kGroups; i += 64)
    __hip_atomic_store(arrive_word(pg, i / kGroups, i % kGroups), 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (lane < kGroups)
    __hip_atomic_store(ctr_word(pg, kExitBase + lane * 128), 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (lane == 0)
    __hip_atomic_store(ctr_word(pg, kExitTop), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MB>
__global__ __launch_bounds__(kStageThreads) void stage_kernel(Program pg) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t io_bar;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = gridDim.x, b = blockIdx.x;
  Lds L;
  L.act = smem;
  L.scl = smem + pg.lds_act_bytes;
  L.red = reinterpret_cast<v4f*>(smem + pg.lds_act_bytes + pg.lds_scl_bytes);
  L.bar = &io_bar;
  if (threadIdx.x == 0) io_bar = 0;
  __syncthreads();
  if (wave < kStream)
    stream_loop<MB>(pg, b, G, wave, lane, L);
  else
    io_loop<MB>(pg, b, G, wave - kStream, lane, L);
}

template <int MB>
hipError_t launch_mb(const Program& pg, hipStream_t stream) {
  auto kern = stage_kernel<MB>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kStageLdsMax);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const size_t lds = (size_t)pg.lds_act_bytes + pg.lds_scl_bytes + (size_t)kStream * MB * 64 * 16;
  hipLaunchKernelGGL(kern, dim3(pg.G), dim3(kStageThreads), lds, stream, pg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_program(const Program& pg, int MB, hipStream_t stream) {
  if (MB <= 1) return launch_mb<1>(pg, stream);
  if (MB == 2) return launch_mb<2>(pg, stream);
  return launch_mb<3>(pg, stream);
}

}  // namespace mxg
