// Small-row MXFP8 block-scaled GEMM: out[M, N] = dequant(a) . dequant(w)^T,
// BF16 out, for M = 1..48 ([mxfp8] page: launch_low_latency, and the wide
// activation tiles of 16, 32 or 48 rows in wide_mm / wide_tactic).
//
// As in the pages' low-latency kernel the weight is the MFMA's A operand and
// the activations its B operand (the kernel computes out^T): one scaled
// 16 x 16 x 128 MFMA covers 16 weight rows x up to 16 activation rows.  At
// these row counts the GEMM is bound by the weight stream from HBM
// (N*K*33/32 bytes for 2*M*N*K flops), and the design serves that stream:
//   * weights arrive pre-packed in tile order (pack.hip), so each wave reads
//     its A operand as fully contiguous 1 KiB loads and its scales as one
//     64-byte load per step;
//   * a workgroup owns one 16-row weight tile and the whole K; its 8 waves
//     split K (wave w takes 128-wide steps w, w+8, ...) and each wave issues
//     every weight load it will need up front, predicated by buffer range
//     checks rather than branches, so nothing waits on anything until the
//     stream is in flight;
//   * the activations (at most M*K bytes, read by every workgroup) are
//     staged once per workgroup: loaded with coalesced 16-byte accesses
//     before the weight loads are issued, quantized in registers when they
//     come as BF16, and parked in LDS, from where each wave reads its B
//     operands;
//   * the 8 partial tiles are summed through LDS in wave order
//     (deterministic), rounded to BF16 and stored.
// Rows above 16 (the 32- and 48-row buckets) take a second kernel that reads
// its activations straight from global memory.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxg {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

__host__ __device__ constexpr int act_ld(int K) { return K + 16; }          // LDS bytes per code row
__host__ __device__ constexpr int scale_ld(int K) { return (K >> 5) + 4; }  // LDS bytes per scale row

// Weight tile of workgroup b.  Workgroups are dispatched to the 8 XCDs round
// robin (b mod 8), and each XCD has its own L2.  Four consecutive tiles share
// every 128-byte line of the BF16 output rows, so when the tile count allows,
// those four tiles go to workgroups of one XCD: their partial-line writes then
// merge in one L2 instead of four.
__device__ __forceinline__ int xcd_tile(int b, int tiles) {
  if (tiles & 31) return b;
  const int xcd = b & 7, k = b >> 3;
  return 4 * (xcd + 8 * (k >> 2)) + (k & 3);
}

// Quantize one 8-element BF16 chunk (16 bytes) whose block of 32 is spread
// over the 4 lanes tid & ~3 .. (tid & ~3) + 3; returns the 8 codes and the
// block's exponent.  All 64 lanes must call it (it shuffles).
__device__ __forceinline__ uint2 quant_chunk8(v4i v, int& e) {
  uint32_t a = halves_max(bf16x2_absmax2(bf16x2_absmax2((uint32_t)v[0], (uint32_t)v[1]),
                                         bf16x2_absmax2((uint32_t)v[2], (uint32_t)v[3])));
  a = quad_max(a);
  e = block_exponent(a);
  const BlockScale bs = block_scale(e);
  uint2 c;
  c.x = enc4_e4m3((uint32_t)v[0], (uint32_t)v[1], bs);
  c.y = enc4_e4m3((uint32_t)v[2], (uint32_t)v[3], bs);
  return c;
}

// ----------------------------------------------------------- M <= 16 rows
//
// W waves split K; SPW: weight steps a wave holds in registers (>= its step
// count); CH: 16-byte activation chunks each thread stages (>= M*K/16/(64W)
// for MXFP8 input, M*K/8/(64W) for BF16 input).
template <int W, int SPW, int CH, bool FQ>
__global__ __launch_bounds__(W * 64) void gemm_m16_kernel(GemmArgs p) {
  constexpr int kThreads = W * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int M = p.M, K = p.K, KB = K >> 5, S = K >> 7;
  const int t = xcd_tile(blockIdx.x, p.N >> 4);
  const int ldA = act_ld(K), ldS = scale_ld(K);
  uint8_t* s_act = smem;                                   // [M][ldA] codes
  uint8_t* s_scl = smem + M * ldA;                         // [M][ldS] scale bytes
  v4f* s_red = reinterpret_cast<v4f*>(smem + ((M * ldA + M * ldS + 15) & ~15));  // [W][64]

  // 1. Activation staging loads (L2-resident, small): issued first so that
  //    waiting for them does not wait for the weight stream.
  v4i st[CH];
  uint32_t sc[FQ ? 1 : 2];
  const int nck = FQ ? (M * K) >> 3 : (M * K) >> 4;        // 16-byte chunks
  auto chunk = [&](int i) {                                // chunk id, or -1
    const int c = tid + i * kThreads;
    return c < nck ? c : -1;
  };
  if constexpr (!FQ) {
    // Rows of K codes at stride lda (and K/32 scale bytes at stride lda/32),
    // starting at this tile's group.
    const int64_t grp = p.group_tiles ? (int64_t)(t / p.group_tiles) * p.a_group : 0;
    const int lda = (int)p.lda, ldas = lda >> 5;
    const auto ra = make_rsrc(p.a_q + grp, (uint32_t)((M - 1) * lda + K));
    const int cpr = K >> 4;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = chunk(i);
      const int row = c / cpr, col = (c - row * cpr) * 16;
      st[i] = buf_ld16(ra, c >= 0 ? (uint32_t)(row * lda + col) : kOutOfRange);
    }
    const auto rs = make_rsrc(p.a_s + (grp >> 5), (uint32_t)((M - 1) * ldas + KB));
    const int nsc = (M * KB) >> 2, spr = KB >> 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / spr, col = (c - row * spr) * 4;
      sc[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rs, c < nsc ? row * ldas + col : (int)kOutOfRange, 0, 0);
    }
  } else {
    const auto rx = make_rsrc(p.x, (uint32_t)(((M - 1) * p.ld_x + K) * 2));
    const int cpr = K >> 3;                                // 8-element chunks per row
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = chunk(i);
      const int row = c / cpr, col = (c - row * cpr) * 8;
      st[i] = buf_ld16(rx, c >= 0 ? (uint32_t)(row * p.ld_x + col) * 2u : kOutOfRange);
    }
  }

  // Keep the staging loads ahead of the weight stream: the load counter
  // drains in issue order, so the staging data can then be waited for
  // while the weights are still in flight.
  __builtin_amdgcn_sched_barrier(0);

  // 2. The weight stream: all of this wave's steps, packed tile order.
  const int my = S > wave ? (S - wave + W - 1) / W : 0;
  const auto rw = make_rsrc(p.w_q + (int64_t)t * S * 2048, (uint32_t)(S * 2048));
  const auto rws = make_rsrc(p.w_s + (int64_t)t * S * 64, (uint32_t)(S * 64));
  v4i wlo[SPW], whi[SPW];
  uint32_t wsc[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int s = wave + W * j;
    const bool ok = j < my;
    wlo[j] = buf_ld16_nt(rw, ok ? (uint32_t)(s * 2048 + lane * 16) : kOutOfRange);
    whi[j] = buf_ld16_nt(rw, ok ? (uint32_t)(s * 2048 + 1024 + lane * 16) : kOutOfRange);
    wsc[j] = buf_ld8(rws, ok ? (uint32_t)(s * 64 + lane) : kOutOfRange);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. Park the activations in LDS (quantizing BF16 on the way).
  if constexpr (!FQ) {
    const int cpr = K >> 4;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = chunk(i);
      if (c >= 0) {
        const int row = c / cpr, col = (c - row * cpr) * 16;
        *reinterpret_cast<v4i*>(s_act + row * ldA + col) = st[i];
      }
    }
    const int spr = KB >> 2;
    const int nsc = (M * KB) >> 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kThreads;
      if (c < nsc) {
        const int row = c / spr, col = (c - row * spr) * 4;
        *reinterpret_cast<uint32_t*>(s_scl + row * ldS + col) = sc[i];
      }
    }
  } else {
    const int cpr = K >> 3;
    const bool writer = blockIdx.x == 0;   // one workgroup writes the codes out
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = chunk(i);
      int e;
      const uint2 codes = quant_chunk8(st[i], e);
      if (c >= 0) {
        const int row = c / cpr, col = (c - row * cpr) * 8;
        *reinterpret_cast<uint2*>(s_act + row * ldA + col) = codes;
        if ((c & 3) == 0) s_scl[row * ldS + (col >> 5)] = (uint8_t)(e + 127);
        if (writer) {
          *reinterpret_cast<uint2*>(p.a_q + (int64_t)row * K + col) = codes;
          if ((c & 3) == 0) p.a_s[(int64_t)row * KB + (col >> 5)] = (uint8_t)(e + 127);
        }
      }
    }
  }
  __syncthreads();

  // 4. MFMAs as the weight steps land.
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const bool live = r < M;
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    if (j < my) {
      const int s = wave + W * j;
      v4i blo = {0, 0, 0, 0}, bhi = {0, 0, 0, 0};
      int bsc = 0;
      if (live) {
        const uint8_t* a = s_act + r * ldA + s * 128 + 16 * g;
        blo = *reinterpret_cast<const v4i*>(a);
        bhi = *reinterpret_cast<const v4i*>(a + 64);
        bsc = s_scl[r * ldS + 4 * s + g];
      }
      acc = mfma_mx16(cat8(wlo[j], whi[j]), cat8(blo, bhi), acc, (int)wsc[j], bsc);
    }
  }

  // 5. Sum the W K-slices in wave order; BF16 out.
  s_red[wave * 64 + lane] = acc;
  __syncthreads();
  if (tid < 64) {
    v4f sum = s_red[lane];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += s_red[w * 64 + lane];
    const int m = lane & 15, n = 16 * t + 4 * (lane >> 4);
    if (m < M) {
      uint2 o;
      o.x = f32_to_bf16(sum[0]) | (f32_to_bf16(sum[1]) << 16);
      o.y = f32_to_bf16(sum[2]) | (f32_to_bf16(sum[3]) << 16);
      *reinterpret_cast<uint2*>(p.out + (int64_t)m * p.N + n) = o;
    }
  }
}

// ----------------------------------------------------------- M = 17..48 rows
//
// MB activation tiles of 16 rows share each weight tile.  Activations are
// read straight from global memory per step (too many rows to stage the whole
// K in LDS); SPW weight steps per chunk.
template <int MB, int SPW, bool FQ>
__global__ __launch_bounds__(kThreads) void gemm_wide_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int K = p.K, KB = K >> 5, S = K >> 7;
  const int t = xcd_tile(blockIdx.x, p.N >> 4);
  const int my = S > wave ? (S - wave + kWaves - 1) / kWaves : 0;
  const auto rw = make_rsrc(p.w_q + (int64_t)t * S * 2048, (uint32_t)(S * 2048));
  const auto rws = make_rsrc(p.w_s + (int64_t)t * S * 64, (uint32_t)(S * 64));
  const int64_t grp = p.group_tiles ? (int64_t)(t / p.group_tiles) * p.a_group : 0;

  v4f acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < my; c0 += SPW) {
    v4i wlo[SPW], whi[SPW];
    uint32_t wsc[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int s = wave + kWaves * (c0 + j);
      const bool ok = c0 + j < my;
      wlo[j] = buf_ld16_nt(rw, ok ? (uint32_t)(s * 2048 + lane * 16) : kOutOfRange);
      whi[j] = buf_ld16_nt(rw, ok ? (uint32_t)(s * 2048 + 1024 + lane * 16) : kOutOfRange);
      wsc[j] = buf_ld8(rws, ok ? (uint32_t)(s * 64 + lane) : kOutOfRange);
    }
    if constexpr (!FQ) {
      v4i alo[SPW][MB], ahi[SPW][MB];
      int asc[SPW][MB];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int s = wave + kWaves * min(c0 + j, my - 1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = 16 * mb + r;
          if (m < p.M && c0 + j < my) {
            const uint8_t* ap = p.a_q + grp + (int64_t)m * p.lda + s * 128 + 16 * g;
            alo[j][mb] = ld16(ap);
            ahi[j][mb] = ld16(ap + 64);
            asc[j][mb] = p.a_s[(grp >> 5) + (int64_t)m * (p.lda >> 5) + 4 * s + g];
          } else {
            alo[j][mb] = ahi[j][mb] = v4i{0, 0, 0, 0};
            asc[j][mb] = 0;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        if (c0 + j < my) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb] = mfma_mx16(cat8(wlo[j], whi[j]), cat8(alo[j][mb], ahi[j][mb]), acc[mb],
                                (int)wsc[j], asc[j][mb]);
        }
      }
    } else {
      // BF16 activations quantized in registers: lane (g, r) holds K
      // [16g, 16g+16) and [64+16g, ..+16) of row m, i.e. half of MFMA block
      // g/2 and half of block 2 + g/2; lane g ^ 1 holds the other halves.
      v4i x0[SPW][MB], x1[SPW][MB], x2[SPW][MB], x3[SPW][MB];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int s = wave + kWaves * min(c0 + j, my - 1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = 16 * mb + r;
          if (m < p.M && c0 + j < my) {
            const uint16_t* xp = p.x + (int64_t)m * p.ld_x + s * 128 + 16 * g;
            x0[j][mb] = ld16(xp);
            x1[j][mb] = ld16(xp + 8);
            x2[j][mb] = ld16(xp + 64);
            x3[j][mb] = ld16(xp + 72);
          } else {
            x0[j][mb] = x1[j][mb] = x2[j][mb] = x3[j][mb] = v4i{0, 0, 0, 0};
          }
        }
      }
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        if (c0 + j < my) {
          const int s = wave + kWaves * (c0 + j);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            uint32_t alo = 0, ahi = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              alo = bf16x2_absmax2(alo, bf16x2_absmax2((uint32_t)x0[j][mb][i], (uint32_t)x1[j][mb][i]));
              ahi = bf16x2_absmax2(ahi, bf16x2_absmax2((uint32_t)x2[j][mb][i], (uint32_t)x3[j][mb][i]));
            }
            alo = halves_max(alo);
            ahi = halves_max(ahi);
            alo = max(alo, (uint32_t)__shfl_xor((int)alo, 16));
            ahi = max(ahi, (uint32_t)__shfl_xor((int)ahi, 16));
            const int elo = block_exponent(alo), ehi = block_exponent(ahi);
            // The MFMA takes block b's scale from lanes g == b: g = 0 and 3
            // own it; g = 1 needs block 1 (first halves of g = 2, 3) and g = 2
            // needs block 2 (second halves of g = 0, 1).
            const int give = (g == 1) ? ehi : elo;
            const int src = (g == 1) ? lane + 16 : ((g == 2) ? lane - 16 : lane);
            const int got = __shfl(give, src);
            const int e = (g == 0) ? elo : ((g == 3) ? ehi : got);
            const BlockScale blo = block_scale(elo), bhi = block_scale(ehi);
            v4i clo, chi;
            clo[0] = (int)enc4_e4m3((uint32_t)x0[j][mb][0], (uint32_t)x0[j][mb][1], blo);
            clo[1] = (int)enc4_e4m3((uint32_t)x0[j][mb][2], (uint32_t)x0[j][mb][3], blo);
            clo[2] = (int)enc4_e4m3((uint32_t)x1[j][mb][0], (uint32_t)x1[j][mb][1], blo);
            clo[3] = (int)enc4_e4m3((uint32_t)x1[j][mb][2], (uint32_t)x1[j][mb][3], blo);
            chi[0] = (int)enc4_e4m3((uint32_t)x2[j][mb][0], (uint32_t)x2[j][mb][1], bhi);
            chi[1] = (int)enc4_e4m3((uint32_t)x2[j][mb][2], (uint32_t)x2[j][mb][3], bhi);
            chi[2] = (int)enc4_e4m3((uint32_t)x3[j][mb][0], (uint32_t)x3[j][mb][1], bhi);
            chi[3] = (int)enc4_e4m3((uint32_t)x3[j][mb][2], (uint32_t)x3[j][mb][3], bhi);
            const int m = 16 * mb + r;
            if (blockIdx.x == 0 && m < p.M) {
              uint8_t* qp = p.a_q + (int64_t)m * K + s * 128 + 16 * g;
              st16(qp, clo);
              st16(qp + 64, chi);
              p.a_s[(int64_t)m * KB + 4 * s + g] = (uint8_t)(e + 127);
            }
            acc[mb] = mfma_mx16(cat8(wlo[j], whi[j]), cat8(clo, chi), acc[mb], (int)wsc[j],
                                e + 127);
          }
        }
      }
    }
  }

  __shared__ v4f red[kWaves][MB][64];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < MB * 64) {
    const int mb = tid >> 6, ln = tid & 63;
    v4f sum = red[0][mb][ln];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += red[w][mb][ln];
    const int m = 16 * mb + (ln & 15);
    const int n = 16 * t + 4 * (ln >> 4);
    if (m < p.M) {
      uint2 o;
      o.x = f32_to_bf16(sum[0]) | (f32_to_bf16(sum[1]) << 16);
      o.y = f32_to_bf16(sum[2]) | (f32_to_bf16(sum[3]) << 16);
      *reinterpret_cast<uint2*>(p.out + (int64_t)m * p.N + n) = o;
    }
  }
}

// ------------------------------------------------------------------ launch

constexpr int kM16Waves = 16;

size_t gemm_m16_lds_bytes(int M, int K) {
  return (size_t)((M * act_ld(K) + M * scale_ld(K) + 15) & ~15) + kM16Waves * 64 * sizeof(v4f);
}

template <int SPW, int CH, bool FQ>
static hipError_t launch_m16(const GemmArgs& a, hipStream_t stream) {
  auto kern = gemm_m16_kernel<kM16Waves, SPW, CH, FQ>;
  const size_t lds = gemm_m16_lds_bytes(a.M, a.K);
  static bool configured = false;   // raise the dynamic-LDS limit once per instance
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(a.N / 16), dim3(kM16Waves * 64), lds, stream, a);
  return hipGetLastError();
}

template <int SPW, bool FQ>
static hipError_t launch_m16_ch(const GemmArgs& a, int ch, hipStream_t stream) {
  if constexpr (FQ) {
    if (ch <= 2) return launch_m16<SPW, 2, FQ>(a, stream);
    return launch_m16<SPW, 4, FQ>(a, stream);
  } else {
    if (ch <= 2) return launch_m16<SPW, 2, FQ>(a, stream);
    if (ch <= 4) return launch_m16<SPW, 4, FQ>(a, stream);
    if (ch <= 8) return launch_m16<SPW, 8, FQ>(a, stream);
    return launch_m16<SPW, 16, FQ>(a, stream);
  }
}

template <bool FQ>
static hipError_t launch_m16_spw(const GemmArgs& a, int spw, int ch, hipStream_t stream) {
  if (spw <= 1) return launch_m16_ch<1, FQ>(a, ch, stream);
  if (spw <= 2) return launch_m16_ch<2, FQ>(a, ch, stream);
  if (spw <= 3) return launch_m16_ch<3, FQ>(a, ch, stream);
  return launch_m16_ch<4, FQ>(a, ch, stream);
}

template <int MB, int SPW, bool FQ>
static hipError_t launch_wide(const GemmArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_wide_kernel<MB, SPW, FQ>), dim3(a.N / 16), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

// Whether the M <= 16 kernel can stage this activation in LDS.
bool gemm_m16_fits(int M, int K) { return M <= 16 && gemm_m16_lds_bytes(M, K) <= 160 * 1024; }

hipError_t launch_gemm(const GemmArgs& args, hipStream_t stream) {
  GemmArgs a = args;
  if (a.lda == 0) a.lda = a.K;
  const bool fq = a.x != nullptr;
  if (fq && (a.group_tiles != 0 || a.lda != a.K)) return hipErrorInvalidValue;
  const int S = a.K / 128;
  const int steps = (S + kM16Waves - 1) / kM16Waves;       // weight steps per wave
  const int per = fq ? a.M * a.K / 8 : a.M * a.K / 16;     // 16-byte staging chunks
  const int ch = (per + kM16Waves * 64 - 1) / (kM16Waves * 64);
  if (gemm_m16_fits(a.M, a.K) && steps <= 4) {
    if (!fq && ch <= 16) return launch_m16_spw<false>(a, steps, ch, stream);
    // In-kernel quantize while the weight stream is in flight when the
    // activation is small (every workgroup quantizes all of it, which costs
    // more than a separate launch from about 8 rows of 5120); larger
    // activations are quantized by their own launch first.
    if (fq && ch <= 4) return launch_m16_spw<true>(a, steps, ch, stream);
    if (fq) {
      hipError_t e = launch_quantize(a.x, a.M, a.K, a.ld_x, a.a_q, a.a_s, stream);
      if (e != hipSuccess) return e;
      GemmArgs b = a;
      b.x = nullptr;
      return launch_gemm(b, stream);
    }
  }
  const int mb = (a.M + 15) / 16;
  if (!fq) {
    if (mb == 1) return launch_wide<1, 8, false>(a, stream);
    if (mb == 2) return launch_wide<2, 6, false>(a, stream);
    return launch_wide<3, 4, false>(a, stream);
  }
  if (mb == 1) return launch_wide<1, 6, true>(a, stream);
  if (mb == 2) return launch_wide<2, 4, true>(a, stream);
  return launch_wide<3, 3, true>(a, stream);
}

}  // namespace mxg
