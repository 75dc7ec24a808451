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
      o.x = f32_to_bf16(acc[mt][0]) | (f32_to_bf16(acc[mt][1]) << 16);
      o.y = f32_to_bf16(acc[mt][2]) | (f32_to_bf16(acc[mt][3]) << 16);
      *reinterpret_cast<uint2*>(p.out + (int64_t)(row0 + m) * N + n) = o;
    }
  }
}

}  // namespace

bool gemm_big_fits(const GemmArgs& a) {
  return a.M > kBigRows && a.N % 64 == 0 && a.x == nullptr && a.group_tiles == 0 &&
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
