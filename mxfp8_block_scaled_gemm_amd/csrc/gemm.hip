// Small-row MXFP8 block-scaled GEMM: out[M, N] = dequant(a) . dequant(w)^T,
// BF16 out, for M = 1..48 ([mxfp8] page: launch_low_latency, and the wide
// activation tiles of 16, 32 or 48 rows in wide_mm / wide_tactic).
//
// Like the pages' low-latency kernel, the weight is the MFMA's A operand and
// the activations its B operand, so one 16 x 16 x 128 scaled MFMA covers 16
// weight rows x up to 16 activation rows, and the kernel computes out^T tile
// by tile.  At these row counts the GEMM is bound by the weight stream from
// HBM (N*K*33/32 bytes against 2*M*N*K flops), so the design is about that
// stream:
//   * a workgroup owns 16*T weight rows and the whole K; its W waves split K
//     (wave w takes 128-wide K steps w, w+W, ...), so every workgroup streams
//     16*T full rows and the grid is N/(16*T) workgroups;
//   * each wave issues all weight loads of a chunk of SPW steps up front
//     (two 16-byte loads per lane per step: per instruction every weight row
//     is read as one 64-byte contiguous segment), then the activation loads,
//     then runs the MFMAs;
//   * the W partial 16x16 tiles are summed through LDS in a fixed order
//     (deterministic), rounded to BF16 and stored.
// With FQ the kernel takes BF16 activations and quantizes them itself in
// registers (the same rule as mxfp8_quantize); workgroup 0 also writes the
// codes and scales out.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxg {

template <int MB, int T, int W, int SPW, bool FQ>
__global__ __launch_bounds__(W * 64) void gemm_kernel(GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int K = p.K, KB = K >> 5, S = K >> 7;
  const int n0 = blockIdx.x * (16 * T);
  const int my = S > wave ? (S - wave + W - 1) / W : 0;   // steps owned by this wave

  v4f acc[T][MB];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[t][mb] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < my; c0 += SPW) {
    v4i wlo[SPW][T], whi[SPW][T];
    int wsc[SPW][T];
    // Weight stream first: it is the long-latency HBM traffic.  Steps past the
    // wave's last are clamped to it (loads stay in bounds, MFMAs are skipped).
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int s = wave + W * min(c0 + j, my - 1);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int n = n0 + 16 * t + r;
        const uint8_t* wp = p.w_q + (int64_t)n * K + s * 128 + 16 * g;
        wlo[j][t] = ld16(wp);
        whi[j][t] = ld16(wp + 64);
        wsc[j][t] = p.w_s[(int64_t)n * KB + 4 * s + g];
      }
    }
    if constexpr (!FQ) {
      v4i alo[SPW][MB], ahi[SPW][MB];
      int asc[SPW][MB];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int s = wave + W * min(c0 + j, my - 1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = 16 * mb + r;
          if (m < p.M) {
            const uint8_t* ap = p.a_q + (int64_t)m * K + s * 128 + 16 * g;
            alo[j][mb] = ld16(ap);
            ahi[j][mb] = ld16(ap + 64);
            asc[j][mb] = p.a_s[(int64_t)m * KB + 4 * s + g];
          } else {
            alo[j][mb] = v4i{0, 0, 0, 0};
            ahi[j][mb] = v4i{0, 0, 0, 0};
            asc[j][mb] = 0;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        if (c0 + j < my) {
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[t][mb] = mfma_mx16(cat8(wlo[j][t], whi[j][t]), cat8(alo[j][mb], ahi[j][mb]),
                                     acc[t][mb], wsc[j][t], asc[j][mb]);
        }
      }
    } else {
      // BF16 activations: lane (g, r) holds K [16g, 16g+16) and [64+16g, ..+16)
      // of row m, i.e. half of MFMA block g/2 and half of block 2 + g/2; the
      // partner lane (g ^ 1) holds the other halves.
      v4i x0[SPW][MB], x1[SPW][MB], x2[SPW][MB], x3[SPW][MB];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int s = wave + W * min(c0 + j, my - 1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = 16 * mb + r;
          if (m < p.M) {
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
          const int s = wave + W * (c0 + j);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            uint32_t alo = 0, ahi = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              alo = max(alo, bf16_pair_absmax_bits((uint32_t)x0[j][mb][i]));
              alo = max(alo, bf16_pair_absmax_bits((uint32_t)x1[j][mb][i]));
              ahi = max(ahi, bf16_pair_absmax_bits((uint32_t)x2[j][mb][i]));
              ahi = max(ahi, bf16_pair_absmax_bits((uint32_t)x3[j][mb][i]));
            }
            alo = max(alo, (uint32_t)__shfl_xor((int)alo, 16));
            ahi = max(ahi, (uint32_t)__shfl_xor((int)ahi, 16));
            const int elo = block_exponent(alo), ehi = block_exponent(ahi);
            // The MFMA takes block b's scale from lanes g == b: g = 0 and 3 own
            // it already; g = 1 needs block 1 (first halves of g = 2, 3) and
            // g = 2 needs block 2 (second halves of g = 0, 1).
            const int give = (g == 1) ? ehi : elo;
            const int src = (g == 1) ? lane + 16 : ((g == 2) ? lane - 16 : lane);
            const int got = __shfl(give, src);
            const int e = (g == 0) ? elo : ((g == 3) ? ehi : got);
            v4i clo, chi;
            clo[0] = (int)enc4_e4m3((uint32_t)x0[j][mb][0], (uint32_t)x0[j][mb][1], -elo);
            clo[1] = (int)enc4_e4m3((uint32_t)x0[j][mb][2], (uint32_t)x0[j][mb][3], -elo);
            clo[2] = (int)enc4_e4m3((uint32_t)x1[j][mb][0], (uint32_t)x1[j][mb][1], -elo);
            clo[3] = (int)enc4_e4m3((uint32_t)x1[j][mb][2], (uint32_t)x1[j][mb][3], -elo);
            chi[0] = (int)enc4_e4m3((uint32_t)x2[j][mb][0], (uint32_t)x2[j][mb][1], -ehi);
            chi[1] = (int)enc4_e4m3((uint32_t)x2[j][mb][2], (uint32_t)x2[j][mb][3], -ehi);
            chi[2] = (int)enc4_e4m3((uint32_t)x3[j][mb][0], (uint32_t)x3[j][mb][1], -ehi);
            chi[3] = (int)enc4_e4m3((uint32_t)x3[j][mb][2], (uint32_t)x3[j][mb][3], -ehi);
            const int m = 16 * mb + r;
            if (blockIdx.x == 0 && m < p.M) {
              uint8_t* qp = p.a_q + (int64_t)m * K + s * 128 + 16 * g;
              st16(qp, clo);
              st16(qp + 64, chi);
              p.a_s[(int64_t)m * KB + 4 * s + g] = (uint8_t)(e + 127);
            }
            const v8i b = cat8(clo, chi);
#pragma unroll
            for (int t = 0; t < T; ++t)
              acc[t][mb] = mfma_mx16(cat8(wlo[j][t], whi[j][t]), b, acc[t][mb], wsc[j][t], e + 127);
          }
        }
      }
    }
  }

  // Sum the W K-slices in wave order and store BF16.
  __shared__ v4f red[W][T * MB][64];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[wave][t * MB + mb][lane] = acc[t][mb];
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid < T * MB * 64) {
    const int tm = tid >> 6, ln = tid & 63;
    v4f sum = red[0][tm][ln];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red[w][tm][ln];
    const int t = tm / MB, mb = tm % MB;
    const int m = 16 * mb + (ln & 15);
    const int n = n0 + 16 * t + 4 * (ln >> 4);
    if (m < p.M) {
      uint2 o;
      o.x = f32_to_bf16(sum[0]) | (f32_to_bf16(sum[1]) << 16);
      o.y = f32_to_bf16(sum[2]) | (f32_to_bf16(sum[3]) << 16);
      *reinterpret_cast<uint2*>(p.out + (int64_t)m * p.N + n) = o;
    }
  }
}

template <int MB, int T, int W, int SPW, bool FQ>
static hipError_t launch_one(const GemmArgs& a, hipStream_t stream) {
  static_assert(T * MB <= W, "the reduction uses one thread per output lane");
  dim3 grid(a.N / (16 * T));
  hipLaunchKernelGGL((gemm_kernel<MB, T, W, SPW, FQ>), grid, dim3(W * 64), 0, stream, a);
  return hipGetLastError();
}

// Tile choice per activation-row bucket (16, 32 or 48 rows, the pages' tile
// sizes) and per quantize mode; SPW bounds the registers that hold one chunk.
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  const int mb = (a.M + 15) / 16;
  const bool fq = a.x != nullptr;
  if (!fq) {
    if (mb == 1) return launch_one<1, 1, 8, 8, false>(a, stream);
    if (mb == 2) return launch_one<2, 1, 8, 6, false>(a, stream);
    return launch_one<3, 1, 8, 4, false>(a, stream);
  }
  if (mb == 1) return launch_one<1, 1, 8, 6, true>(a, stream);
  if (mb == 2) return launch_one<2, 1, 8, 4, true>(a, stream);
  return launch_one<3, 1, 8, 3, true>(a, stream);
}

}  // namespace mxg
