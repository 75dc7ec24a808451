// MXFP8 GEMM for more than 64 activation rows ([mxfp8] page, module text:
// above the low-latency row range the projections run on another kernel).
//
// A workgroup of 4 or 8 waves computes a 64 x 64 output tile over the whole
// K: weight tiles 4 bx .. 4 bx + 3 (16 rows each; wave w, and with 8 waves
// also wave w + 4, streams tile 4 bx + w from HBM straight into its MFMA A
// operands, packed order; two waves of one tile take the even and the odd
// K-steps of each chunk and add their sums at the end) against
// activation rows 64 by .. 64 by + 63 (four 16-row MFMA B tiles, staged
// through LDS in chunks of 4 K-steps, double-buffered).  Every weight step
// a wave loads feeds four scaled MFMAs and every activation byte staged
// feeds four waves, so a weight byte is read once per 64 rows and an
// activation byte once per 64 weight rows; no K split, no cross-workgroup
// sum.  The row tiles of one weight tile group are dispatched 8 workgroups
// apart, i.e. to one XCD close in time, so the repeat weight reads hit that
// XCD's L2.
#include <type_traits>

#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxg {

namespace {

constexpr int kCS = 4;                              // K-steps (128 wide) per chunk
constexpr int kBigRows = 64;                        // activation rows per workgroup
constexpr int kLdA = kCS * 128 + 16;                // LDS bytes per code row of a chunk
constexpr int kLdS = kCS * 4 + 4;                   // LDS bytes per scale row of a chunk
constexpr int kBufBytes = kBigRows * kLdA + kBigRows * kLdS;
// Staging per thread per chunk: 64 rows x kCS*128 code bytes in 16-byte
// pieces, and 64 rows x kCS*4 scale bytes in dwords.
constexpr int kPiecesPerRow = kCS * 128 / 16;
constexpr int kDwordsPerRow = kCS;
constexpr int kScalePieces = kBigRows * kDwordsPerRow;   // dwords per chunk

// WV = 4: one wave per weight tile; WV = 8: two per tile, taking the even
// and the odd K-steps of each chunk (more loads in flight per workgroup).
template <int WV>
__global__ __launch_bounds__(WV * 64) void gemm_big_kernel(GemmArgs p) {
  constexpr int kBigThreads = WV * 64;
  constexpr int kHalves = WV / 4;                    // waves per weight tile
  constexpr int kStCodes = kBigRows * kPiecesPerRow / kBigThreads;
  constexpr int kStScales = (kScalePieces + kBigThreads - 1) / kBigThreads;
  static_assert(kBigRows * kPiecesPerRow % kBigThreads == 0, "staging must tile the chunk");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int M = p.M, N = p.N, K = p.K, S = K >> 7, KB = K >> 5;
  const int nch = (S + kCS - 1) / kCS;

  // (bx, by): 64 weight rows x 64 activation rows; the RB row tiles of one
  // bx go 8 workgroups apart (same XCD).
  const int X = N >> 6, RB = (M + kBigRows - 1) / kBigRows;
  int bx, by;
  if ((X & 7) == 0) {
    const int id = blockIdx.x, within = id % (8 * RB);
    bx = (id / (8 * RB)) * 8 + (within & 7);
    by = within >> 3;
  } else {
    by = blockIdx.x / X;
    bx = blockIdx.x - by * X;
  }
  const int row0 = by * kBigRows;
  const int Mb = min(M - row0, kBigRows);
  const int tile = 4 * bx + (wave & 3), kh = wave >> 2;   // my tile; my share of each chunk's steps

  const auto ra = make_rsrc(p.a_q + (int64_t)row0 * K, (uint32_t)((Mb - 1) * K + K));
  const auto rs = make_rsrc(p.a_s + (int64_t)row0 * KB, (uint32_t)((Mb - 1) * KB + KB));
  const auto rw = make_rsrc(p.w_q + (int64_t)tile * S * 2048, (uint32_t)(S * 2048));
  const auto rws = make_rsrc(p.w_s + (int64_t)tile * S * 64, (uint32_t)(S * 64));

  // Activation chunk c: rows [0, Mb), steps [kCS c, kCS c + kCS) -> registers.
  v4i st[kStCodes];
  uint32_t ss[kStScales];
  auto stage_load = [&](int c) {
    const int ns = min(kCS, S - kCS * c);
#pragma unroll
    for (int i = 0; i < kStCodes; ++i) {
      const int piece = tid + i * kBigThreads;
      const int row = piece / kPiecesPerRow, col = (piece % kPiecesPerRow) * 16;
      const bool ok = row < Mb && (col >> 7) < ns;
      st[i] = buf_ld16(ra, ok ? (uint32_t)(row * K + kCS * 128 * c + col) : kOutOfRange);
    }
#pragma unroll
    for (int i = 0; i < kStScales; ++i) {
      const int piece = tid + i * kBigThreads;
      const int row = piece / kDwordsPerRow, col = (piece % kDwordsPerRow) * 4;
      const bool ok = piece < kScalePieces && row < Mb && (col >> 2) < ns;
      ss[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rs, ok ? row * KB + kCS * 4 * c + col : (int)kOutOfRange, 0, 0);
    }
  };
  auto stage_park = [&](int buf) {
    uint8_t* act = smem + buf * kBufBytes;
    uint8_t* scl = act + kBigRows * kLdA;
#pragma unroll
    for (int i = 0; i < kStCodes; ++i) {
      const int piece = tid + i * kBigThreads;
      const int row = piece / kPiecesPerRow, col = (piece % kPiecesPerRow) * 16;
      *reinterpret_cast<v4i*>(act + row * kLdA + col) = st[i];
    }
#pragma unroll
    for (int i = 0; i < kStScales; ++i) {
      const int piece = tid + i * kBigThreads;
      const int row = piece / kDwordsPerRow, col = (piece % kDwordsPerRow) * 4;
      if (piece < kScalePieces) *reinterpret_cast<uint32_t*>(scl + row * kLdS + col) = ss[i];
    }
  };

  // Weight steps of chunk c for this wave's tile, in register set W.
  constexpr int kHS = kCS / kHalves;                 // my steps per chunk
  const WeightLane wl = weight_lane(p.w_rm, K, lane);
  v4i wlo[2][kHS], whi[2][kHS];
  uint32_t wsc[2][kHS];
  auto weight_load = [&](auto set_tag, int c) {
    constexpr int W = decltype(set_tag)::value;
#pragma unroll
    for (int jj = 0; jj < kHS; ++jj) {
      const int s = kCS * c + kHalves * jj + kh;
      const bool ok = s < S;
      const uint32_t lo = s * wl.step_q + wl.lane_q;
      wlo[W][jj] = buf_ld16_nt(rw, ok ? lo : kOutOfRange);
      whi[W][jj] = buf_ld16_nt(rw, ok ? lo + wl.half_q : kOutOfRange);
      wsc[W][jj] = buf_ld8(rws, ok ? s * wl.step_s + wl.lane_s : kOutOfRange);
    }
  };

  v4f acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](auto set_tag, int c) {
    constexpr int W = decltype(set_tag)::value;
    const uint8_t* act = smem + (c & 1) * kBufBytes;
    const uint8_t* scl = act + kBigRows * kLdA;
    const int ns = min(kCS, S - kCS * c);
#pragma unroll
    for (int jj = 0; jj < kHS; ++jj) {
      const int j = kHalves * jj + kh;
      if (j < ns) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint8_t* a = act + (16 * mt + r) * kLdA + j * 128 + 16 * g;
          const v4i blo = *reinterpret_cast<const v4i*>(a);
          const v4i bhi = *reinterpret_cast<const v4i*>(a + 64);
          const int bsc = scl[(16 * mt + r) * kLdS + 4 * j + g];
          acc[mt] = mfma_mx16(cat8(wlo[W][jj], whi[W][jj]), cat8(blo, bhi), acc[mt],
                              (int)wsc[W][jj], bsc);
        }
      }
    }
  };

  // One chunk: prefetch chunk c + 1 (activations to registers, weights to
  // the other register set), compute chunk c from LDS, park chunk c + 1.
  auto chunk = [&](auto set_tag, int c) {
    constexpr int W = decltype(set_tag)::value;
    const bool next = c + 1 < nch;
    if (next) {
      stage_load(c + 1);
      weight_load(std::integral_constant<int, 1 - W>{}, c + 1);
    }
    __syncthreads();                                  // chunk c parked; buffer (c+1)&1 free
    compute(std::integral_constant<int, W>{}, c);
    if (next) stage_park((c + 1) & 1);
  };

  stage_load(0);
  weight_load(std::integral_constant<int, 0>{}, 0);
  stage_park(0);
  for (int c = 0; c < nch; c += 2) {
    chunk(std::integral_constant<int, 0>{}, c);
    if (c + 1 < nch) chunk(std::integral_constant<int, 1>{}, c + 1);
  }

  if constexpr (kHalves == 2) {
    // The two halves of each tile's steps: waves 4..7 hand their sums to
    // waves 0..3 through LDS (after the last chunk's reads), which add them.
    __syncthreads();
    v4f* red = reinterpret_cast<v4f*>(smem);            // [4 tiles][4 mt][64]
    if (kh == 1) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) red[((wave & 3) * 4 + mt) * 64 + lane] = acc[mt];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] += red[((wave & 3) * 4 + mt) * 64 + lane];
  }
  // Lane (g, r) of acc[mt] holds out[row0 + 16 mt + r][16 tile + 4 g + i].
  const int n = 16 * tile + 4 * g;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int m = 16 * mt + r;
    if (m < Mb) {
      uint2 o;
      o.x = pk_bf16(acc[mt][0], acc[mt][1]);
      o.y = pk_bf16(acc[mt][2], acc[mt][3]);
      *reinterpret_cast<uint2*>(p.out + (int64_t)(row0 + m) * N + n) = o;
    }
  }
}

// ------------------------------------------------------------ wide form
//
// 64 activation rows x NT weight tiles per workgroup over the whole K, with
// K split across the 8 waves instead of the tiles: chunk c holds K-steps
// [8c, 8c + 8) of the 64 rows in LDS, and wave w takes step 8c + w of every
// tile and every 16-row block.  It loads that step's weight operands for
// its NT tiles itself (registers, one chunk ahead), reads each of the four
// 16-row activation operands of the step from LDS once, and feeds each to
// NT MFMAs.  An activation byte is therefore read from LDS once per
// workgroup (the 64 x 64 form reads it once per tile wave), and a chunk
// takes one barrier for 8 steps.  At the end the 8 waves' partial tiles are
// summed through LDS in wave order.
constexpr int kWW = 8;                              // waves
constexpr int kWCS = kWW;                           // K-steps per chunk: one per wave
constexpr int kWLdA = kWCS * 128 + 16;              // LDS bytes per code row of a chunk
constexpr int kWLdS = kWCS * 4 + 4;                 // LDS bytes per scale row of a chunk
constexpr int kWBuf = kBigRows * kWLdA + kBigRows * kWLdS;
constexpr int kWThreads = kWW * 64;
constexpr int kWRowsPerWave = kBigRows / kWW;      // rows each wave loads into LDS per chunk
static_assert(kBigRows * kWCS == kWThreads, "one scale dword per thread");
static_assert(kWCS * 128 == 16 * 64, "a chunk row is one 16-byte load per lane");

// s_waitcnt immediate that waits until at most n vector loads of this wave
// are outstanding (export and LDS counters left unconstrained).
constexpr int vmcnt_at_most(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | ((n >> 4) << 14); }

template <int NT>
constexpr size_t wide_lds_bytes() {
  constexpr size_t ring = 2 * (size_t)kWBuf;
  constexpr size_t red = (size_t)kWW * NT * 4 * 64 * 16;   // partial tiles of every wave
  return ring > red ? ring : red;
}

template <int NT>
__global__ __launch_bounds__(kWThreads) void gemm_wide_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int M = p.M, N = p.N, K = p.K, S = K >> 7, KB = K >> 5;
  const int nch = (S + kWCS - 1) / kWCS;

  // (bx, by): 16 NT weight rows x 64 activation rows; the RB row blocks of
  // one bx go 8 workgroups apart (same XCD), so the repeat weight reads hit
  // that XCD's L2.
  const int X = N / (16 * NT), RB = (M + kBigRows - 1) / kBigRows;
  int bx, by;
  if ((X & 7) == 0) {
    const int id = blockIdx.x, within = id % (8 * RB);
    bx = (id / (8 * RB)) * 8 + (within & 7);
    by = within >> 3;
  } else {
    by = blockIdx.x / X;
    bx = blockIdx.x - by * X;
  }
  const int row0 = by * kBigRows;
  const int Mb = min(M - row0, kBigRows);

  const auto ra = make_rsrc(p.a_q + (int64_t)row0 * K, (uint32_t)(Mb * K));
  const auto rs = make_rsrc(p.a_s + (int64_t)row0 * KB, (uint32_t)(Mb * KB));
  const auto rw = make_rsrc(p.w_q + (int64_t)NT * bx * S * 2048, (uint32_t)(NT * S * 2048));
  const auto rws = make_rsrc(p.w_s + (int64_t)NT * bx * S * 64, (uint32_t)(NT * S * 64));
  const WeightLane wl = weight_lane(p.w_rm, K, lane);
  constexpr int kWaitWeightsOnly = vmcnt_at_most(3 * NT);   // one chunk's weight loads

  // Activation chunk c -> LDS buffer c & 1 without registers: wave w loads
  // rows w, w + 8, .. straight into LDS, each row's 1 KiB of the chunk by one
  // 16-byte-per-lane load (lane l: bytes 16 l ..).  Rows past Mb load out of
  // range; columns past the last step are never read.  The scale dword of
  // row tid / 8, step tid % 8 goes through a register.
  uint32_t ss;
  auto stage_load = [&](int c) {
    uint8_t* act = smem + (c & 1) * kWBuf;
#pragma unroll
    for (int i = 0; i < kWRowsPerWave; ++i) {
      const int row = wave + kWW * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(act + row * kWLdA), 16,
          row < Mb ? (uint32_t)(row * K + kWCS * 128 * c + 16 * lane) : kOutOfRange, 0, 0, 0);
    }
    const int row = tid >> 3, k4 = tid & 7;
    const bool ok = row < Mb && kWCS * c + k4 < S;
    ss = __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? row * KB + 4 * (kWCS * c + k4) : (int)kOutOfRange,
                                              0, 0);
  };
  auto stage_park = [&](int buf) {
    uint8_t* scl = smem + buf * kWBuf + kBigRows * kWLdA;
    *reinterpret_cast<uint32_t*>(scl + (tid >> 3) * kWLdS + 4 * (tid & 7)) = ss;
  };

  // Weight operands of step 8c + wave for the NT tiles, in register set W
  // (two sets: the weights run one chunk ahead of the MFMAs; two chunks
  // ahead measured slower on MI355X, e.g. 15.97 against 15.12 us at M 256,
  // N 4096, K 5120).
  v4i wlo[2][NT], whi[2][NT];
  uint32_t wsc[2][NT];
  auto weight_load = [&](auto set_tag, int c) {
    constexpr int W = decltype(set_tag)::value;
    const int s = kWCS * c + wave;
    const bool ok = s < S;
    const uint32_t lo = s * wl.step_q + wl.lane_q, sco = s * wl.step_s + wl.lane_s;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t tq = (uint32_t)(t * S * 2048), ts = (uint32_t)(t * S * 64);
      wlo[W][t] = buf_ld16_nt(rw, ok ? tq + lo : kOutOfRange);
      whi[W][t] = buf_ld16_nt(rw, ok ? tq + lo + wl.half_q : kOutOfRange);
      wsc[W][t] = buf_ld8(rws, ok ? ts + sco : kOutOfRange);
    }
  };

  v4f acc[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[t][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](auto set_tag, int c) {
    constexpr int W = decltype(set_tag)::value;
    if (kWCS * c + wave >= S) return;                  // wave-uniform: past the last step
    const uint8_t* act = smem + (c & 1) * kWBuf;
    const uint8_t* scl = act + kBigRows * kWLdA;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint8_t* a = act + (16 * mt + r) * kWLdA + wave * 128 + 16 * g;
      const v8i b = cat8(*reinterpret_cast<const v4i*>(a), *reinterpret_cast<const v4i*>(a + 64));
      const int bsc = scl[(16 * mt + r) * kWLdS + 4 * wave + g];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t][mt] = mfma_mx16(cat8(wlo[W][t], whi[W][t]), b, acc[t][mt], (int)wsc[W][t], bsc);
    }
  };

  // One chunk: once every wave is past chunk c - 1 (its buffer is then
  // free), issue chunk c + 1 (activations into LDS, weights into the other
  // register set), compute chunk c, then wait for this wave's part of chunk
  // c + 1's activations (issued ahead of its weights, which stay in flight)
  // and park its scales; the next barrier publishes it.  Chunks past the last load out of range and compute
  // nothing, so every chunk issues the same loads and the load-counter waits
  // stay exact.
  auto chunk = [&](auto set_tag, int c) {
    constexpr int W = decltype(set_tag)::value;
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    stage_load(c + 1);
    weight_load(std::integral_constant<int, 1 - W>{}, c + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(std::integral_constant<int, W>{}, c);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitWeightsOnly);
    stage_park((c + 1) & 1);
  };

  stage_load(0);
  weight_load(std::integral_constant<int, 0>{}, 0);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitWeightsOnly);
  stage_park(0);
  for (int c = 0; c < nch; c += 2) {
    chunk(std::integral_constant<int, 0>{}, c);
    chunk(std::integral_constant<int, 1>{}, c + 1);
  }

  // The 8 waves' partial tiles, summed in wave order: item i = (t, mt, lane)
  // of the NT x 4 output blocks.
  __syncthreads();                                    // every wave past its last chunk
  v4f* red = reinterpret_cast<v4f*>(smem);            // [wave][NT][4][64]
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) red[((wave * NT + t) * 4 + mt) * 64 + lane] = acc[t][mt];
  __syncthreads();
  constexpr int kItems = NT * 4 * 64;
#pragma unroll
  for (int i0 = 0; i0 < kItems; i0 += kWThreads) {
    const int i = i0 + tid;
    if (kItems % kWThreads != 0 && i >= kItems) break;
    v4f sum = red[i];
#pragma unroll
    for (int w = 1; w < kWW; ++w) sum += red[w * kItems + i];
    const int t = i >> 8, mt = (i >> 6) & 3, l = i & 63;
    // lane (g, r) of block (t, mt) holds out[row0 + 16 mt + r][16 tile + 4 g + 0..3]
    const int m = 16 * mt + (l & 15), n = 16 * (NT * bx + t) + 4 * (l >> 4);
    if (m < Mb) {
      uint2 o;
      o.x = pk_bf16(sum[0], sum[1]);
      o.y = pk_bf16(sum[2], sum[3]);
      *reinterpret_cast<uint2*>(p.out + (int64_t)(row0 + m) * N + n) = o;
    }
  }
}

}  // namespace

bool gemm_big_fits(const GemmArgs& a) {
  return a.M > kBigRows && a.N % 64 == 0 && a.x == nullptr && a.group_tiles == 0 &&
         (a.lda == 0 || a.lda == a.K) && !a.a_sf128;
}

bool gemm_wide_fits(const GemmArgs& a) {
  return a.M > 48 && a.N % 16 == 0 && a.x == nullptr && a.group_tiles == 0 &&
         (a.lda == 0 || a.lda == a.K) && !a.a_sf128;
}

template <int WV>
static hipError_t launch_big(const GemmArgs& a, int grid, hipStream_t stream) {
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_big_kernel<WV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kBufBytes);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(gemm_big_kernel<WV>, dim3(grid), dim3(WV * 64), 2 * kBufBytes, stream, a);
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_wide(const GemmArgs& a, hipStream_t stream) {
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_wide_kernel<NT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)wide_lds_bytes<NT>());
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int grid = (a.N / (16 * NT)) * ((a.M + kBigRows - 1) / kBigRows);
  hipLaunchKernelGGL(gemm_wide_kernel<NT>, dim3(grid), dim3(kWThreads), wide_lds_bytes<NT>(),
                     stream, a);
  return hipGetLastError();
}

// Weight tiles per workgroup of the wide form: the count (4, 2 or 1) whose
// grid is the largest that still runs in one round on `cus` CUs (one
// workgroup per CU: its LDS ring takes 135 KiB), or 0 when every count
// needs a second round.
int gemm_wide_tiles(const GemmArgs& a, int cus) {
  const int rb = (a.M + kBigRows - 1) / kBigRows;
  int best = 0, best_grid = 0;
  for (int nt : {4, 2, 1}) {
    if (a.N % (16 * nt) != 0) continue;
    const int grid = (a.N / (16 * nt)) * rb;
    if (grid <= cus && grid > best_grid) best = nt, best_grid = grid;
  }
  return best;
}

// The wide form with `nt` tiles per workgroup (0: the one-round count, or
// else the fewest workgroups).
hipError_t launch_gemm_wide(const GemmArgs& a, int cus, hipStream_t stream, int nt) {
  if (nt == 0) nt = gemm_wide_tiles(a, cus);
  if (nt == 0) nt = a.N % 64 == 0 ? 4 : a.N % 32 == 0 ? 2 : 1;
  if (nt == 4) return launch_wide<4>(a, stream);
  if (nt == 2) return launch_wide<2>(a, stream);
  return launch_wide<1>(a, stream);
}

// Eight waves (two per weight tile) when the grid fits one workgroup per CU:
// 17-20 % faster there (M = 256, N 4096, K 5120: 17.3 against 20.7 us); four
// waves on larger grids, where two 4-wave workgroups share a CU but a single
// 8-wave one does not (M = 256, N 8192, K 1536: 10.8 against 13.3 us).
hipError_t launch_gemm_big(const GemmArgs& a, int cus, hipStream_t stream) {
  const int grid = (a.N / 64) * ((a.M + kBigRows - 1) / kBigRows);
  if (grid <= cus) return launch_big<8>(a, grid, stream);
  return launch_big<4>(a, grid, stream);
}

}  // namespace mxg
