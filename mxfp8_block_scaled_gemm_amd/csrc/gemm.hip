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
//   * M <= 16 kernel: a workgroup owns one 16-row weight tile and the whole
//     K; its 16 waves split K (wave w takes 128-wide steps w, w+16, ...) and
//     each wave issues every weight load it will need up front, predicated
//     by buffer range checks rather than branches, so nothing waits on
//     anything until the stream is in flight;
//   * the activations (at most M*K bytes, read by every workgroup) are
//     staged per workgroup: loaded with coalesced 16-byte accesses before
//     the weight loads are issued, quantized in registers when they come as
//     BF16 (one 32-element block per lane), and parked in LDS, from where
//     each wave reads its B operands;
//   * the 16 partial tiles are summed through LDS in wave order
//     (deterministic), rounded to BF16 and stored;
//   * 2D kernel (rows above 16, and shapes whose tile count fits the chip
//     badly): a workgroup takes 1, 2 or 4 weight tiles over one K part, the
//     activations go through LDS in 2048-wide K chunks, and K parts are
//     summed across workgroups in part order by the last to arrive.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mxg {

constexpr int kM16Waves = 16;   // waves per workgroup of the GEMM kernels
constexpr int kRowBlock = 64;   // activation rows one 2D-kernel workgroup serves

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

// Byte offset of the dword holding the scales of blocks [4 q, 4 q + 4) of
// activation row m: row-major at row stride ldas, or (sf128) in 128 x 4
// tiles (S = K/128 tiles per 128 rows), where those four bytes are
// contiguous.  With sf128, m counts from the tensor's first row.
__device__ __forceinline__ int act_scale_dword(int m, int q, int ldas, bool sf128, int S) {
  return sf128 ? ((m >> 7) * S + q) * 512 + (m & 31) * 16 + ((m & 127) >> 5) * 4
               : m * ldas + 4 * q;
}

// Quantize one whole 32-element BF16 block held by this lane (4 x 16 bytes)
// to its 32 E4M3 codes (2 x 16 bytes) and its exponent.  One lane per block
// keeps the per-block work (amax, exponent, scale) to one copy, where lanes
// sharing a block would each repeat it.
__device__ __forceinline__ void quant_block32(const v4i* v, v4i& c0, v4i& c1, int& e) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    m = bf16x2_absmax2(m, bf16x2_absmax2(bf16x2_absmax2((uint32_t)v[k][0], (uint32_t)v[k][1]),
                                         bf16x2_absmax2((uint32_t)v[k][2], (uint32_t)v[k][3])));
  e = block_exponent(halves_max(m));
  const BlockScale bs = block_scale(e);
  uint32_t c[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    c[2 * k] = enc4_e4m3((uint32_t)v[k][0], (uint32_t)v[k][1], bs);
    c[2 * k + 1] = enc4_e4m3((uint32_t)v[k][2], (uint32_t)v[k][3], bs);
  }
  c0 = v4i{(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  c1 = v4i{(int)c[4], (int)c[5], (int)c[6], (int)c[7]};
}

// Fixed-order sum of `slices` partial 16 x 16 tiles parked in LDS as FP32
// [slice][64 lanes][4] (slice i at red + i * stride floats), spread over 256
// threads: thread t (t < 256) adds element t of every slice in slice order,
// so each of the 256 sums is (((s0 + s1) + s2) + ...), the same order as one
// wave adding whole slices.
__device__ __forceinline__ float sum_slices(const float* red, int slices, int stride, int t) {
  float v = red[t];
  for (int i = 1; i < slices; ++i) v += red[i * stride + t];
  return v;
}

// Element t of a 256-element tile sum is value t % 4 of D lane t / 4.  Each
// lane quad gathers its four values as BF16 with DPP quad permutes; the
// quad's first thread (t % 4 == 0) returns true with D lane t / 4's values
// 0..3 in o.  All 64 lanes of each calling wave must take part (the permutes
// read neighbouring lanes).
__device__ __forceinline__ bool quad_bf16(float v, int t, uint2& o) {
  const uint32_t h = f32_to_bf16(v);
  const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  const uint32_t pr = h | (nb << 16);                       // on even t: values (t, t + 1)
  const uint32_t np = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)pr, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  o.x = pr;
  o.y = np;
  return (t & 3) == 0;
}

// ----------------------------------------------------------- M <= 16 rows
//
// W waves split K; SPW: weight steps a wave holds in registers (>= its step
// count); CH: what each thread stages: 16-byte code chunks (>= M*K/16/(64W))
// for MXFP8 input, whole 32-element blocks (>= M*K/32/(64W)) for BF16 input.
//
// HALF: the weight has G < tiles <= 1.5 G tiles for a grid of G workgroups.
// Workgroup b takes full tile xcd_tile(b, G) and, for b < 2 (tiles - G), half
// (b & 1) of leftover tile G + b / 2: rows 8 (b & 1) .. + 8, whose operand
// bytes are whole 128-byte lines of the packed tile, in an MFMA of its own
// whose other A rows stay zero.  Every workgroup then streams one tile or one
// and a half, with no sum across workgroups; slots [0, SPW/2) hold the full
// tile's steps, slots [SPW/2, SPW) the half tile's.
//
// NRM (BF16 input, not HALF): the rows of x are RMS-normalised before the
// quantize.  Every workgroup stages whole rows, so it computes each row's
// factor 1 / sqrt(mean(x^2) + eps) itself, then y = BF16((x * r) * w) is
// quantized as any BF16 input is.  Two forms, with the same arithmetic in the
// same order (bit-identical results):
//   NRM = 1: blocks in thread order; block sums of squares through LDS, one
//            wave per row adds them in block order, the gain parked in LDS;
//            two workgroup barriers ahead of the quantize.
//   NRM = 2: K <= 2048 (at most 64 blocks a row): wave w stages whole rows
//            w, w + W, ..., lane l block l, and holds its blocks' gains in
//            registers, so each wave finishes its rows' norm with no barrier
//            (the barriers cannot pass before every wave has issued its weight
//            loads, and the norm's work then stood between that point and the
//            MFMAs).
// It runs with 8 waves, built for two workgroups per CU (at most 128
// registers per lane): with 16 waves the norm needs more than the 64
// registers that two such workgroups per CU allow, and with one workgroup per
// CU a weight of more tiles than CUs takes a second round.
template <int W, int SPW, int CH, bool FQ, bool HALF = false, int NRM = 0>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(NRM ? W / 2 : 1)))
void gemm_m16_kernel(GemmArgs p) {
  static_assert(!NRM || (FQ && !HALF), "the norm runs in the BF16 staging");
  constexpr int kThreads = W * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int M = p.M, K = p.K, KB = K >> 5, S = K >> 7;
  // With rsplit = 2 or 4 a workgroup takes rows [16/rsplit * part, ...) of
  // weight tile t, so that a small N still gives every CU a workgroup: its
  // lanes load only those rows' operand bytes (whole 128-byte lines of the
  // packed tile) and the other lanes' A rows stay zero.
  const int rsplit = HALF ? 1 : p.rsplit, sh = rsplit == 1 ? 4 : (rsplit == 2 ? 3 : 2);
  const int G = gridDim.x;
  const int unit = xcd_tile(blockIdx.x, HALF ? G : (p.N >> 4) * rsplit);
  const int t = unit / rsplit, part = unit - t * rsplit;
  const bool mine = (r >> sh) == part;                     // my A row is this workgroup's
  // HALF: my half of a leftover tile (th), if I have one.
  const int th = G + (blockIdx.x >> 1), hpart = blockIdx.x & 1;
  const bool has_half = HALF && (int)blockIdx.x < 2 * ((p.N >> 4) - G);
  const bool mine_h = has_half && (r >> 3) == hpart;
  const int ldA = act_ld(K), ldS = scale_ld(K);
  uint8_t* s_act = smem;                                   // [M][ldA] codes
  uint8_t* s_scl = smem + M * ldA;                         // [M][ldS] scale bytes
  // Partial tiles [W][64] (HALF: [2][W][64] over the activations, written
  // once every wave is past its MFMAs).
  v4f* s_red = reinterpret_cast<v4f*>(HALF ? smem : smem + ((M * ldA + M * ldS + 15) & ~15));

  // 1. Activation staging loads (L2-resident, small): issued first so that
  //    waiting for them does not wait for the weight stream.
  // Scale dwords are an eighth of the 16-byte code chunks.
  constexpr int SCR = FQ ? 1 : (CH + 7) / 8;
  v4i st[FQ ? 4 * CH : CH];
  uint32_t sc[SCR];
  const int nck = FQ ? (M * K) >> 5 : (M * K) >> 4;        // 32-blocks, or 16-byte chunks
  auto chunk = [&](int i) {                                // chunk id, or -1
    if constexpr (NRM == 2) {                              // row wave + W i, block lane
      const int row = wave + W * i;
      return row < M && lane < KB ? row * KB + lane : -1;
    }
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
    const auto rs = make_rsrc(p.a_s + (grp >> 5),
                              (uint32_t)(p.a_sf128 ? 128 * KB : (M - 1) * ldas + KB));
    const int nsc = (M * KB) >> 2, spr = KB >> 2;
#pragma unroll
    for (int i = 0; i < SCR; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / spr, col = (c - row * spr) * 4;
      sc[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rs, c < nsc ? act_scale_dword(row, col >> 2, ldas, p.a_sf128, S) : (int)kOutOfRange, 0,
          0);
    }
  } else {
    const auto rx = make_rsrc(p.x, (uint32_t)(((M - 1) * p.ld_x + K) * 2));
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = chunk(i);                              // block: row c / KB, 32 columns
      const int row = c / KB, col = (c - row * KB) * 32;
      const uint32_t off = (uint32_t)(row * p.ld_x + col) * 2u;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        st[4 * i + k] = buf_ld16(rx, c >= 0 ? off + 16 * k : kOutOfRange);
    }
  }
  // The norm's gain (K BF16 values), one 16-byte piece per thread (K <= 8 x
  // threads), staged through LDS so that it holds no registers across the
  // weight stream (two workgroups per CU need at most 64 per lane).
  v4i gst = {0, 0, 0, 0};
  if constexpr (NRM == 1)
    gst = buf_ld16(make_rsrc(p.norm_w, (uint32_t)(K * 2)),
                   tid < (K >> 3) ? (uint32_t)(tid * 16) : kOutOfRange);
  // NRM = 2: the 32 gains of block `lane` (the same for every row).
  v4i gw[NRM == 2 ? 4 : 1];
  if constexpr (NRM == 2) {
    const auto rg = make_rsrc(p.norm_w, (uint32_t)(K * 2));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      gw[k] = buf_ld16(rg, lane < KB ? (uint32_t)(lane * 64 + 16 * k) : kOutOfRange);
  }

  // Keep the staging loads ahead of the weight stream: the load counter
  // drains in issue order, so the staging data can then be waited for
  // while the weights are still in flight.  (An execution barrier here, so
  // that every wave issues its staging loads before any wave's weights,
  // measured slower on MI355X: the weight stream then starts later.)
  __builtin_amdgcn_sched_barrier(0);

  // 2. The weight stream: all of this wave's steps, packed tile order.
  constexpr int SF = HALF ? SPW / 2 : SPW;                 // slots of the full tile
  const int my = S > wave ? (S - wave + W - 1) / W : 0;
  const auto rw = make_rsrc(p.w_q + (int64_t)t * S * 2048, (uint32_t)(S * 2048));
  const auto rws = make_rsrc(p.w_s + (int64_t)t * S * 64, (uint32_t)(S * 64));
  const auto rwh = make_rsrc(p.w_q + (int64_t)th * S * 2048, has_half ? (uint32_t)(S * 2048) : 0u);
  const auto rwsh = make_rsrc(p.w_s + (int64_t)th * S * 64, has_half ? (uint32_t)(S * 64) : 0u);
  const WeightLane wl = weight_lane(p.w_rm, K, lane);
  v4i wlo[SPW], whi[SPW];
  uint32_t wsc[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const bool full = j < SF;
    const int jj = full ? j : j - SF;
    const int s = wave + W * jj;
    const bool ok = jj < my && (full ? mine : mine_h);
    const auto rq = full ? rw : rwh;
    const auto rsc = full ? rws : rwsh;
    const uint32_t lo = s * wl.step_q + wl.lane_q;
    wlo[j] = buf_ld16_nt(rq, ok ? lo : kOutOfRange);
    whi[j] = buf_ld16_nt(rq, ok ? lo + wl.half_q : kOutOfRange);
    wsc[j] = buf_ld8(rsc, ok ? s * wl.step_s + wl.lane_s : kOutOfRange);
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
    for (int i = 0; i < SCR; ++i) {
      const int c = tid + i * kThreads;
      if (c < nsc) {
        const int row = c / spr, col = (c - row * spr) * 4;
        *reinterpret_cast<uint32_t*>(s_scl + row * ldS + col) = sc[i];
      }
    }
  } else {
    const bool writer = blockIdx.x == 0;   // one workgroup writes the codes out
    if constexpr (NRM) {
      // Block sums of squares (each product and sum rounded on its own); a
      // row's blocks are then added in a fixed order: lane l takes blocks l,
      // l + 64, ... in order, then wave_sum across the lanes.
      auto block_ss = [&](int i) {
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint32_t u = (uint32_t)st[4 * i + k][h];
            const float a = bf16_lo(u), b = bf16_hi(u);
            ss = ss + a * a;
            ss = ss + b * b;
          }
        return ss;
      };
      float rr[CH];                                        // each chunk's row factor
      uint8_t* s_gain = reinterpret_cast<uint8_t*>(s_red) + W * 64 * sizeof(v4f);  // [K] BF16
      if constexpr (NRM == 1) {
        float* s_ss = reinterpret_cast<float*>(s_red);     // [M][KB], then r [M]
        float* s_r = s_ss + M * KB;
        if (tid < (K >> 3)) *reinterpret_cast<v4i*>(s_gain + tid * 16) = gst;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int c = chunk(i);
          if (c >= 0) s_ss[c] = block_ss(i);               // c = row * KB + block
        }
        __syncthreads();
        for (int row = wave; row < M; row += W) {          // W waves, up to 16 rows
          float t = 0.f;
          for (int b = lane; b < KB; b += 64) t = t + s_ss[row * KB + b];
          t = wave_sum(t);
          if (lane == 0) s_r[row] = 1.0f / __builtin_sqrtf(t / (float)K + p.norm_eps);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int c = chunk(i);
          rr[i] = s_r[c >= 0 ? c / KB : 0];
        }
      } else {
        // One block per lane: the lane's sum is its only term (0 + ss = ss).
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          rr[i] = 0.f;
          if (wave + W * i < M) {                          // wave-uniform
            const float t = wave_sum(chunk(i) >= 0 ? block_ss(i) : 0.f);
            rr[i] = 1.0f / __builtin_sqrtf(t / (float)K + p.norm_eps);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = chunk(i);
        if (c >= 0) {
          const float r = rr[i];
          const uint8_t* gb = s_gain + (c - (c / KB) * KB) * 64;   // the block's 32 gains
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v4i gk;
            if constexpr (NRM == 2) gk = gw[k];
            else gk = *reinterpret_cast<const v4i*>(gb + 16 * k);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const uint32_t xu = (uint32_t)st[4 * i + k][h], wu = (uint32_t)gk[h];
              const float lo = (bf16_lo(xu) * r) * bf16_lo(wu);
              const float hi = (bf16_hi(xu) * r) * bf16_hi(wu);
              st[4 * i + k][h] = (int)pk_bf16(lo, hi);
            }
          }
          if (writer && p.norm_y) {
            const int row = c / KB, col = (c - row * KB) * 32;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              *reinterpret_cast<v4i*>(p.norm_y + (int64_t)row * K + col + 8 * k) = st[4 * i + k];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = chunk(i);
      if (c >= 0) {
        v4i c0, c1;
        int e;
        quant_block32(&st[4 * i], c0, c1, e);
        const int row = c / KB, cb = c - row * KB, col = cb * 32;
        *reinterpret_cast<v4i*>(s_act + row * ldA + col) = c0;
        *reinterpret_cast<v4i*>(s_act + row * ldA + col + 16) = c1;
        s_scl[row * ldS + cb] = (uint8_t)(e + 127);
        if (writer) {
          *reinterpret_cast<v4i*>(p.a_q + (int64_t)row * K + col) = c0;
          *reinterpret_cast<v4i*>(p.a_q + (int64_t)row * K + col + 16) = c1;
          p.a_s[(int64_t)row * KB + cb] = (uint8_t)(e + 127);
        }
      }
    }
  }
  __syncthreads();

  // 4. MFMAs as the weight steps land.
  v4f acc = {0.f, 0.f, 0.f, 0.f}, acch = {0.f, 0.f, 0.f, 0.f};
  const bool live = r < M;
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const bool full = j < SF;
    const int jj = full ? j : j - SF;
    if (jj < my && (full || has_half)) {                   // wave-uniform
      const int s = wave + W * jj;
      v4i blo = {0, 0, 0, 0}, bhi = {0, 0, 0, 0};
      int bsc = 0;
      if (live) {
        const uint8_t* a = s_act + r * ldA + s * 128 + 16 * g;
        blo = *reinterpret_cast<const v4i*>(a);
        bhi = *reinterpret_cast<const v4i*>(a + 64);
        bsc = s_scl[r * ldS + 4 * s + g];
      }
      if (full)
        acc = mfma_mx16(cat8(wlo[j], whi[j]), cat8(blo, bhi), acc, (int)wsc[j], bsc);
      else
        acch = mfma_mx16(cat8(wlo[j], whi[j]), cat8(blo, bhi), acch, (int)wsc[j], bsc);
    }
  }

  // 5. Sum the W K-slices in wave order (spread over four waves per tile);
  //    BF16 out.
  if constexpr (HALF) __syncthreads();                     // activations no longer read
  s_red[wave * 64 + lane] = acc;
  if constexpr (HALF) s_red[(W + wave) * 64 + lane] = acch;
  __syncthreads();
  const float* redf = reinterpret_cast<const float*>(s_red);
  uint2 o;
  if (tid < 256 && quad_bf16(sum_slices(redf, W, 256, tid), tid, o)) {
    const int l = tid >> 2;                                 // D lane of this output quad
    const int m = l & 15, n = 16 * t + 4 * (l >> 4);
    // output rows n .. n+3 are weight rows 4 (l / 16) .. of the tile
    if (m < M && ((4 * (l >> 4)) >> sh) == part)
      *reinterpret_cast<uint2*>(p.out + (int64_t)m * p.N + n) = o;
  }
  if constexpr (HALF) {
    const int t4 = tid - 256;
    if (has_half && t4 >= 0 && t4 < 256 &&                 // wave-uniform
        quad_bf16(sum_slices(redf + W * 256, W, 256, t4), t4, o)) {
      const int l = t4 >> 2;
      const int m = l & 15, n = 16 * th + 4 * (l >> 4);
      if (m < M && ((4 * (l >> 4)) >> 3) == hpart)
        *reinterpret_cast<uint2*>(p.out + (int64_t)m * p.N + n) = o;
    }
  }
}

typedef unsigned v4u32 __attribute__((ext_vector_type(4)));

// Words between the K split's tile-group counters: one 128-byte line each.
// Workgroups of different tile groups arrive at nearly the same time, and
// device-scope atomics on one line serialize (measured on MI355X: M = 32 /
// 48, N 4096, K 5120 took 9.07 / 9.92 us with the counters packed, 8.66 /
// 9.68 spread out).
constexpr int kCtrStride = 32;

// ------------------------------------- 2D tiling (any M; 64-row blocks above 48)
//
// When one full-K weight tile per workgroup does not suit the shape (rows
// above 16: every workgroup would pull all M*K activation bytes through its
// CU; or a tile count that leaves part of the chip with a second round), a
// workgroup takes T weight tiles over one of P K parts.  The activation
// traffic per workgroup falls by P, the weight bytes per workgroup stay
// near one tile's, and the grid stays near one workgroup per CU.
//
// Workgroup (tile group tg, part q): tiles [T tg, T tg + T), steps
// [q Sp, q Sp + ns).  Wave w serves tile w mod T, taking the steps
// w / T + (16 / T) j of it, so slot j lies in K-chunk j / T (16 steps,
// staged through LDS; chunk c is read by slots [c T, c T + T)).  As in the
// M <= 16 kernel, every weight load is issued up front, after the first
// (or every) activation chunk's loads.  The 16 / T partial tiles of each
// tile are summed through LDS in wave order; with P > 1 the FP32 tile sums
// go to the workspace and the last of the P workgroups of a tile group to
// arrive adds them in part order (deterministic) and stores BF16.
template <int MB, int T, int SPW, int NB, int CHM, bool FQ, bool NRM = false, bool WL = false>
__global__ __launch_bounds__(kM16Waves * 64) void gemm_2d_kernel(GemmArgs p0) {
  // Row block y: rows [64 y, 64 y + 64) of the activations and the output,
  // with their own K-split partials and tile counters (a GEMM of more than
  // 64 rows is a grid of 64-row GEMMs over the same weight).  The grid is
  // one-dimensional, X = tile groups x K parts per row block: workgroup id
  // serves (x, y) with the RB row blocks of x dispatched 8 apart, i.e. to the
  // same XCD (workgroups go to the 8 XCDs round robin) close in time, so the
  // weight tiles they share are read from HBM once and from that L2 after.
  const int X = (p0.N >> 4) / T * p0.P, RB = (p0.M + kRowBlock - 1) / kRowBlock;
  int bx = blockIdx.x, by = 0;
  if (RB > 1) {
    if ((X & 7) == 0) {
      const int id = blockIdx.x, within = id % (8 * RB);
      bx = (id / (8 * RB)) * 8 + (within & 7);
      by = within >> 3;
    } else {
      by = blockIdx.x / X;
      bx = blockIdx.x - by * X;
    }
  }
  const int row0 = kRowBlock * by;
  GemmArgs p = p0;
  p.M = min(p0.M - row0, kRowBlock);
  p.a_q += (int64_t)row0 * p0.lda;
  if (!p0.a_sf128) p.a_s += (int64_t)row0 * (p0.lda >> 5);
  p.out += (int64_t)row0 * p0.N;
  if (p0.part) p.part += (int64_t)by * (p0.N >> 4) * p0.P * MB * 64 * 4;
  if (p0.ctr) p.ctr += (int64_t)by * ((p0.N >> 4) / T) * kCtrStride;
  // Row index of this block's first row in the scale addressing: row-major
  // scales were offset above; 128 x 4 tiles are addressed from the first row.
  const int srow0 = p0.a_sf128 ? row0 : 0;
  // Registers per thread per K chunk: CHM 16-byte code chunks, or with BF16
  // input (M <= 32) MB whole 32-element blocks per thread (64 per row).
  constexpr int FQB = FQ ? MB : 0;                      // BF16 blocks per thread per chunk
  constexpr int CHL = FQ ? 4 * FQB : CHM;
  static_assert(!FQ || MB <= 2, "BF16 staging serves up to 32 rows");
  static_assert(!NRM || (FQ && NB == 1), "the norm runs in the BF16 staging of one chunk");
  static_assert(!WL || (!FQ && !NRM && NB == 1 && T * MB <= 8), "wave-local: MXFP8 input");
  // Partial tiles each wave parks for the sums: its tile's row tiles, or
  // (wave-local) every tile's.
  constexpr int RU = WL ? T * MB : MB;
  constexpr int W = kM16Waves, kT = W * 64, WPT = W / T;  // waves per tile
  constexpr int kLdA = 16 * 128 + 16;                   // LDS bytes per code row of a chunk
  constexpr int kLdS = 16 * 4 + 4;                      // LDS bytes per scale row of a chunk
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ uint32_t s_last;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int M = p.M, K = p.K, S = K >> 7, Sp = p.Sp, P = p.P;
  const int ngroups = (p.N >> 4) / T;
  const int q = bx / ngroups;
  const int tg = xcd_tile(bx - q * ngroups, ngroups);
  const int k0 = q * Sp, ns = min(Sp, S - k0);          // this part's steps
  const int nch = (ns + 15) >> 4;
  const int tt = wave % T, wi = wave / T;               // my tile, my index among its waves
  const int tile = tg * T + tt;
  uint8_t* s_act = smem;                                // [M][kLdA]
  uint8_t* s_scl = smem + M * kLdA;                     // [M][kLdS]
  v4f* s_red = reinterpret_cast<v4f*>(smem);            // [W][MB][64], after the last chunk

  // A tile group lies in one activation group (the plan keeps T | group_tiles).
  const int64_t grp = p.group_tiles ? (int64_t)(tg * T / p.group_tiles) * p.a_group : 0;
  const int lda = (int)p.lda, ldas = lda >> 5;
  const auto ra = make_rsrc(p.a_q + grp, (uint32_t)((M - 1) * lda + K));
  const auto rs = make_rsrc(p.a_s + (grp >> 5),
                            (uint32_t)(p.a_sf128 ? ((p0.M + 127) >> 7) * 128 * (K >> 5)
                                                 : (M - 1) * ldas + (K >> 5)));
  // Chunk c: steps [k0 + 16c, k0 + 16c + 16) within the part.
  auto stage_load = [&](int c, v4i (&st)[CHL], uint32_t& sc) {
    const int nsc_steps = min(16, ns - 16 * c);
    const int cpr = nsc_steps * 8, nck = M * cpr;
    const int col0 = (k0 + 16 * c) * 128;
#pragma unroll
    for (int i = 0; i < CHM; ++i) {
      const int cc = tid + i * kT;
      const int row = cc / cpr, col = (cc - row * cpr) * 16;
      st[i] = buf_ld16(ra, cc < nck ? (uint32_t)(row * lda + col0 + col) : kOutOfRange);
    }
    const int nsc = M * nsc_steps;
    const int row = tid / nsc_steps, cd = tid - row * nsc_steps;
    sc = __builtin_amdgcn_raw_buffer_load_b32(
        rs, tid < nsc ? act_scale_dword(srow0 + row, k0 + 16 * c + cd, ldas, p.a_sf128, S)
                      : (int)kOutOfRange,
        0, 0);
  };
  auto stage_park = [&](int c, const v4i (&st)[CHL], uint32_t sc) {
    const int nsc_steps = min(16, ns - 16 * c);
    const int cpr = nsc_steps * 8, nck = M * cpr;
#pragma unroll
    for (int i = 0; i < CHM; ++i) {
      const int cc = tid + i * kT;
      if (cc < nck) {
        const int row = cc / cpr, col = (cc - row * cpr) * 16;
        *reinterpret_cast<v4i*>(s_act + row * kLdA + col) = st[i];
      }
    }
    const int nsc = M * nsc_steps;
    if (tid < nsc) {
      const int row = tid / nsc_steps, cd = tid - row * nsc_steps;
      *reinterpret_cast<uint32_t*>(s_scl + row * kLdS + cd * 4) = sc;
    }
  };

  // BF16 input: the chunk's 32-element blocks (64 per row), FQB whole blocks
  // per thread, quantized while parked; the first tile group's workgroups
  // also write the codes out.  Thread block f: block tid + f * threads; with
  // the norm (one chunk of at most 64 blocks a row), row wave + 16 f, block
  // lane, so that each wave holds whole rows.  nblk: none.
  auto blk_of = [&](int f, int bpr, int nblk) {
    if constexpr (NRM) {
      const int row = wave + kM16Waves * f;
      return row < M && lane < bpr ? row * bpr + lane : nblk;
    }
    return tid + f * kT;
  };
  auto load_bf16 = [&](int c, v4i (&st)[CHL]) {
    const int nsc_steps = min(16, ns - 16 * c);
    const int col0 = (k0 + 16 * c) * 128;
    const auto rx = make_rsrc(p.x, (uint32_t)(((M - 1) * p.ld_x + K) * 2));
    const int bpr = nsc_steps * 4, nblk = M * bpr;
#pragma unroll
    for (int f = 0; f < FQB; ++f) {
      const int blk = blk_of(f, bpr, nblk);
      const int row = blk / bpr, cb = blk - row * bpr;
      const uint32_t off = (uint32_t)(row * p.ld_x + col0 + cb * 32) * 2u;
#pragma unroll
      for (int h = 0; h < 4; ++h)
        st[4 * f + h] = buf_ld16(rx, blk < nblk ? off + 16 * h : kOutOfRange);
    }
  };
  auto park_bf16 = [&](int c, const v4i (&st)[CHL], uint8_t* act, int ldA_, uint8_t* scl,
                       int ldS_) {
    const int nsc_steps = min(16, ns - 16 * c);
    const int bpr = nsc_steps * 4, nblk = M * bpr;
    const int col0 = (k0 + 16 * c) * 128;
#pragma unroll
    for (int f = 0; f < FQB; ++f) {
      const int blk = blk_of(f, bpr, nblk);
      if (blk < nblk) {
        const int row = blk / bpr, cb = blk - row * bpr;
        v4i c0, c1;
        int e;
        quant_block32(&st[4 * f], c0, c1, e);
        *reinterpret_cast<v4i*>(act + row * ldA_ + cb * 32) = c0;
        *reinterpret_cast<v4i*>(act + row * ldA_ + cb * 32 + 16) = c1;
        scl[row * ldS_ + cb] = (uint8_t)(e + 127);
        if (tg == 0) {
          uint8_t* qo = p.a_q + (int64_t)row * K + col0 + cb * 32;
          *reinterpret_cast<v4i*>(qo) = c0;
          *reinterpret_cast<v4i*>(qo + 16) = c1;
          p.a_s[((int64_t)row * K + col0 + cb * 32) >> 5] = (uint8_t)(e + 127);
        }
      }
    }
  };

  // 1. Activations (chunk 0, or all chunks) ahead of the weight stream; with
  //    the norm, its gain too (one 16-byte piece per thread, K <= 2048).
  v4i st[NB][CHL];
  uint32_t sc[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    if (!WL && c < nch) {
      if constexpr (FQ)
        load_bf16(c, st[c]);
      else
        stage_load(c, st[c], sc[c]);
    }
  }
  // Wave-local: no staging.  Wave w takes steps w + 16 j (j < SPW) of every
  // tile of the group and loads the MFMA B operands of those steps itself
  // (row 16 mb + r's 32 code bytes and scale byte, rows past M clamped to
  // row M - 1, whose outputs are never stored), each used for T MFMAs.
  v4i blo[WL ? SPW : 1][MB], bhi[WL ? SPW : 1][MB];
  uint32_t bsc[WL ? SPW : 1][MB];
  if constexpr (WL) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int stp = wave + kM16Waves * j;
      const bool ok = stp < ns;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = min(16 * mb + r, M - 1);
        const uint32_t off = (uint32_t)(m * lda + (k0 + stp) * 128 + 16 * g);
        blo[j][mb] = buf_ld16(ra, ok ? off : kOutOfRange);
        bhi[j][mb] = buf_ld16(ra, ok ? off + 64 : kOutOfRange);
        bsc[j][mb] = buf_ld8(
            rs, ok ? (uint32_t)(act_scale_dword(srow0 + m, k0 + stp, ldas, p.a_sf128, S) + g)
                   : kOutOfRange);
      }
    }
  }
  // The norm's gain: the 32 values of block `lane` (the same for every row).
  v4i gw[NRM ? 4 : 1];
  if constexpr (NRM) {
    const auto rg = make_rsrc(p.norm_w, (uint32_t)(K * 2));
#pragma unroll
    for (int k = 0; k < 4; ++k)
      gw[k] = buf_ld16(rg, lane < (K >> 5) ? (uint32_t)(lane * 64 + 16 * k) : kOutOfRange);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. The weight stream: slot j = step wi + WPT j of my tile.
  const auto rw = make_rsrc(p.w_q, (uint32_t)((p.N >> 4) * S * 2048));
  const auto rws = make_rsrc(p.w_s, (uint32_t)((p.N >> 4) * S * 64));
  constexpr int NW = WL ? SPW * T : SPW;                // weight slots per wave
  const WeightLane wl = weight_lane(p.w_rm, K, lane);
  v4i wlo[NW], whi[NW];
  uint32_t wsc[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    // wave-local: slot j = step wave + 16 (j / T) of tile j % T
    const int stp = WL ? wave + kM16Waves * (j / T) : wi + WPT * j;
    const int wt = WL ? tg * T + j % T : tile;
    const bool ok = stp < ns;
    const uint32_t ks = (uint32_t)(k0 + stp);
    const uint32_t lo = (uint32_t)wt * (uint32_t)(16 * K) + ks * wl.step_q + wl.lane_q;
    wlo[j] = buf_ld16_nt(rw, ok ? lo : kOutOfRange);
    whi[j] = buf_ld16_nt(rw, ok ? lo + wl.half_q : kOutOfRange);
    wsc[j] = buf_ld8(rws, ok ? (uint32_t)wt * (uint32_t)(K / 2) + ks * wl.step_s + wl.lane_s
                             : kOutOfRange);
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. Chunk by chunk: park it, (prefetch the next), the MFMAs of its slots.
  //    When every chunk is in registers and the part fits LDS, all chunks
  //    are parked side by side behind one barrier and each wave then runs
  //    its MFMAs as its own weights land.
  v4f acc[RU];
#pragma unroll
  for (int u = 0; u < RU; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
  constexpr int NCH = (SPW + T - 1) / T;
  if constexpr (WL) {
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      if (wave + kM16Waves * j < ns) {                  // wave-uniform
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[t * MB + mb] = mfma_mx16(cat8(wlo[j * T + t], whi[j * T + t]),
                                         cat8(blo[j][mb], bhi[j][mb]), acc[t * MB + mb],
                                         (int)wsc[j * T + t], (int)bsc[j][mb]);
      }
    }
  } else if constexpr (NB == NCH && NB > 1) {
    const int ldA = Sp * 128 + 16, ldS = Sp * 4 + 4;
    uint8_t* w_scl = smem + M * ldA;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      if (FQ && c < nch) park_bf16(c, st[c], s_act + 2048 * c, ldA, w_scl + 64 * c, ldS);
      if (!FQ && c < nch) {
        const int nsc_steps = min(16, ns - 16 * c);
        const int cpr = nsc_steps * 8, nck = M * cpr;
#pragma unroll
        for (int i = 0; i < CHM; ++i) {
          const int cc = tid + i * kT;
          if (cc < nck) {
            const int row = cc / cpr, col = (cc - row * cpr) * 16;
            *reinterpret_cast<v4i*>(s_act + row * ldA + 2048 * c + col) = st[c][i];
          }
        }
        const int nsc = M * nsc_steps;
        if (tid < nsc) {
          const int row = tid / nsc_steps, cd = tid - row * nsc_steps;
          *reinterpret_cast<uint32_t*>(w_scl + row * ldS + 64 * c + cd * 4) = sc[c];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int stp = wi + WPT * j;
      if (stp < ns) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = min(16 * mb + r, M - 1);        // rows past M: never stored
          const uint8_t* a = s_act + m * ldA + stp * 128 + 16 * g;
          const v4i blo = *reinterpret_cast<const v4i*>(a);
          const v4i bhi = *reinterpret_cast<const v4i*>(a + 64);
          const int bsc = w_scl[m * ldS + 4 * stp + g];
          acc[mb] = mfma_mx16(cat8(wlo[j], whi[j]), cat8(blo, bhi), acc[mb], (int)wsc[j], bsc);
        }
      }
    }
    __syncthreads();                                    // LDS reused for the sums
  } else {
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c < nch) {                                      // uniform
      if constexpr (NRM) {
        // RMSNorm of the staged rows (the part is all of K, one chunk, at
        // most 64 blocks a row): as in the M <= 16 kernel, block sums of
        // squares (each product and sum rounded on its own), added across
        // the wave's lanes (lane l: block l) by wave_sum, then
        // y = BF16((x * r) * w) replaces the staged values.  Each wave holds
        // whole rows: no barrier.
        const int KB = K >> 5;
#pragma unroll
        for (int f = 0; f < FQB; ++f) {
          const int row = wave + kM16Waves * f;
          if (row < M) {                                // wave-uniform
            const bool mine = lane < KB;
            float t = 0.f;
            if (mine) {
#pragma unroll
              for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                  const uint32_t u = (uint32_t)st[0][4 * f + k][h];
                  const float x0 = bf16_lo(u), x1 = bf16_hi(u);
                  t = t + x0 * x0;
                  t = t + x1 * x1;
                }
            }
            t = wave_sum(t);
            const float rr = 1.0f / __builtin_sqrtf(t / (float)K + p.norm_eps);
            if (mine) {
#pragma unroll
              for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                  const uint32_t xu = (uint32_t)st[0][4 * f + k][h], wu = (uint32_t)gw[k][h];
                  const float lo = (bf16_lo(xu) * rr) * bf16_lo(wu);
                  const float hi = (bf16_hi(xu) * rr) * bf16_hi(wu);
                  st[0][4 * f + k][h] = (int)pk_bf16(lo, hi);
                }
              if (tg == 0 && p.norm_y) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                  *reinterpret_cast<v4i*>(p.norm_y + (int64_t)row * K + lane * 32 + 8 * k) =
                      st[0][4 * f + k];
              }
            }
          }
        }
      }
      if constexpr (FQ)
        park_bf16(c, st[NB > 1 ? c : 0], s_act, kLdA, s_scl, kLdS);
      else
        stage_park(c, st[NB > 1 ? c : 0], sc[NB > 1 ? c : 0]);
      __syncthreads();
      if (NB == 1 && c + 1 < nch) {
        if constexpr (FQ)
          load_bf16(c + 1, st[0]);
        else
          stage_load(c + 1, st[0], sc[0]);
      }
#pragma unroll
      for (int j = c * T; j < c * T + T && j < SPW; ++j) {
        const int stp = wi + WPT * j;
        if (stp < ns) {
          const int sl = stp - 16 * c;                  // step within the chunk
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const int m = min(16 * mb + r, M - 1);      // rows past M: never stored
            const uint8_t* a = s_act + m * kLdA + sl * 128 + 16 * g;
            const v4i blo = *reinterpret_cast<const v4i*>(a);
            const v4i bhi = *reinterpret_cast<const v4i*>(a + 64);
            const int bsc = s_scl[m * kLdS + 4 * sl + g];
            acc[mb] = mfma_mx16(cat8(wlo[j], whi[j]), cat8(blo, bhi), acc[mb], (int)wsc[j], bsc);
          }
        }
      }
      __syncthreads();
    }
  }
  }

  // 4. Per (tile, row block) unit: sum its WPT partial tiles in wave order.
  // Unit u = (tile t, row tile mb), t * MB + mb, has NSL partial tiles
  // (slices) in wave order, slice i of unit u at s_red[(u + T MB i) * 64]:
  // WPT waves per tile, or every wave when wave-local.
  constexpr int NSL = WL ? kM16Waves : WPT;
#pragma unroll
  for (int u = 0; u < RU; ++u) s_red[(wave * RU + u) * 64 + lane] = acc[u];
  __syncthreads();
  // Output MXFP8 (out_q): the tile group's BF16 outputs are also put in an
  // LDS tile [16 MB rows][16 T columns] beside the partial tiles and, after
  // a barrier, quantized per 32 columns, one block per thread.
  const bool qz = T >= 2 && p.out_q != nullptr && 16 * T * tg < p.qn;   // workgroup-uniform
  uint16_t* s_q = reinterpret_cast<uint16_t*>(smem + kM16Waves * RU * 64 * 16);
  auto q_put = [&](int m, int n, uint2 o) {
    *reinterpret_cast<uint2*>(s_q + m * (16 * T) + (n - 16 * T * tg)) = o;
  };
  auto q_flush = [&]() {
    __syncthreads();
    constexpr int BPR = T / 2 > 0 ? T / 2 : 1;          // 32-column blocks per row
    const int row = tid / BPR, cb = tid - row * BPR, col = 16 * T * tg + 32 * cb;
    if (row < M && col < p.qn) {
      const v4i* v = reinterpret_cast<const v4i*>(s_q + row * (16 * T) + 32 * cb);
      v4i blk[4] = {v[0], v[1], v[2], v[3]};
      v4i c0, c1;
      int e;
      quant_block32(blk, c0, c1, e);
      uint8_t* qo = p.out_q + (int64_t)row * p.qn + col;
      *reinterpret_cast<v4i*>(qo) = c0;
      *reinterpret_cast<v4i*>(qo + 16) = c1;
      p.out_s[(int64_t)row * (p.qn >> 5) + (col >> 5)] = (uint8_t)(e + 127);
    }
  };
  if (P == 1 && T * MB <= kM16Waves / 4) {
    // Few units: each spread over four waves (one of its 256 sums per thread).
    const int u = wave >> 2, t4 = tid & 255, l = t4 >> 2;
    if (u < T * MB) {                                   // wave-uniform
      const int rt = u / MB, rmb = u - rt * MB;
      const int m = 16 * rmb + (l & 15), n = 16 * (tg * T + rt) + 4 * (l >> 4);
      uint2 o;
      if (quad_bf16(sum_slices(reinterpret_cast<const float*>(s_red) + u * 256, NSL, T * MB * 256, t4),
                    t4, o) &&
          m < M) {
        *reinterpret_cast<uint2*>(p.out + (int64_t)m * p.N + n) = o;
        if (qz) q_put(m, n, o);
      }
    }
    if (qz) q_flush();
    return;
  }
  // Otherwise wave tt * MB + mb sums tile tt's row block mb.
  const bool red = wave < T * MB;
  const int rt = wave / MB, rmb = wave - rt * MB;        // tile and row block I sum
  v4f sum = {0.f, 0.f, 0.f, 0.f};
  if (red) {
    sum = s_red[(rt * MB + rmb) * 64 + lane];
#pragma unroll
    for (int i = 1; i < NSL; ++i) sum += s_red[((rt + T * i) * MB + rmb) * 64 + lane];
  }
  const int otile = tg * T + rt;
  const int m = 16 * rmb + (lane & 15), n = 16 * otile + 4 * (lane >> 4);
  if (P == 1) {
    if (red && m < M) {
      uint2 o;
      o.x = pk_bf16(sum[0], sum[1]);
      o.y = pk_bf16(sum[2], sum[3]);
      *reinterpret_cast<uint2*>(p.out + (int64_t)m * p.N + n) = o;
      if (qz) q_put(m, n, o);
    }
    if (qz) q_flush();
    return;
  }
  // K split: FP32 tile sums to the workspace (device-coherent), then one
  // arrival per workgroup on the tile group's counter.
  const uint32_t pstride = (uint32_t)(P * MB * 64 * 16);        // bytes per tile
  const auto rp = make_rsrc(reinterpret_cast<uint8_t*>(p.part), (uint32_t)((p.N >> 4) * pstride));
  if (red)
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(v4u32, sum), rp,
        (int)(otile * pstride + ((q * MB + rmb) * 64 + lane) * 16), 0, 16);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(p.ctr + tg * kCtrStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(P - 1);
  __syncthreads();
  if (!s_last) return;
  if (red) {
    // the P parts' sums, added in part order
    v4f tot = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                          rp, (int)(otile * pstride + (rmb * 64 + lane) * 16), 0, 16));
    for (int qq = 1; qq < P; ++qq)
      tot += __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                         rp, (int)(otile * pstride + ((qq * MB + rmb) * 64 + lane) * 16),
                                         0, 16));
    if (m < M) {
      uint2 o;
      o.x = pk_bf16(tot[0], tot[1]);
      o.y = pk_bf16(tot[2], tot[3]);
      *reinterpret_cast<uint2*>(p.out + (int64_t)m * p.N + n) = o;
      if (qz) q_put(m, n, o);
    }
  }
  if (tid == 0) __hip_atomic_store(p.ctr + tg * kCtrStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (qz) q_flush();
}

// ------------------------------------------------------------------ launch

size_t gemm_m16_lds_bytes(int M, int K, int W) {
  return (size_t)((M * act_ld(K) + M * scale_ld(K) + 15) & ~15) + (size_t)W * 64 * sizeof(v4f);
}

// HALF: the two sets of partial tiles overlay the activations.
size_t gemm_m16_half_lds_bytes(int M, int K, int W) {
  const size_t act = (size_t)((M * act_ld(K) + M * scale_ld(K) + 15) & ~15);
  const size_t red = (size_t)2 * W * 64 * sizeof(v4f);
  return act > red ? act : red;
}

template <int W, int SPW, int CH, bool FQ, bool HALF = false, int NRM = 0>
static hipError_t launch_m16(const GemmArgs& a, int grid, hipStream_t stream) {
  auto kern = gemm_m16_kernel<W, SPW, CH, FQ, HALF, NRM>;
  const size_t lds = HALF       ? gemm_m16_half_lds_bytes(a.M, a.K, W)
                     : NRM == 1 ? gemm_m16_lds_bytes(a.M, a.K, W) + (size_t)a.K * 2
                                : gemm_m16_lds_bytes(a.M, a.K, W);
  static bool configured = false;   // raise the dynamic-LDS limit once per instance
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(W * 64), lds, stream, a);
  return hipGetLastError();
}

// Staging registers per thread: 16-byte code chunks (MXFP8 input) or whole
// 32-element blocks (BF16 input), rounded up to an instantiated count.
template <int W, int SPW, bool FQ>
static hipError_t launch_m16_ch(const GemmArgs& a, int ch, hipStream_t stream) {
  const int grid = a.N / 16 * a.rsplit;
  if constexpr (FQ) {
    if (ch <= 1) return launch_m16<W, SPW, 1, FQ>(a, grid, stream);
    if (ch <= 2) return launch_m16<W, SPW, 2, FQ>(a, grid, stream);
  } else {
    if (ch <= 2) return launch_m16<W, SPW, 2, FQ>(a, grid, stream);
    if (ch <= 4) return launch_m16<W, SPW, 4, FQ>(a, grid, stream);
    if constexpr (W == 16) {
      if (ch <= 8) return launch_m16<W, SPW, 8, FQ>(a, grid, stream);
      if (ch <= 16) return launch_m16<W, SPW, 16, FQ>(a, grid, stream);
    }
  }
  return hipErrorInvalidValue;
}

// HALF launches: 16 waves, one workgroup per CU (grid = G), SPW = 2 x the
// full tile's slots.
template <int SPW, bool FQ>
static hipError_t launch_m16_half_ch(const GemmArgs& a, int G, int ch, hipStream_t stream) {
  if constexpr (FQ) {
    if (ch <= 1) return launch_m16<16, SPW, 1, FQ, true>(a, G, stream);
    if (ch <= 2) return launch_m16<16, SPW, 2, FQ, true>(a, G, stream);
  } else {
    if (ch <= 2) return launch_m16<16, SPW, 2, FQ, true>(a, G, stream);
    if (ch <= 4) return launch_m16<16, SPW, 4, FQ, true>(a, G, stream);
    if constexpr (SPW < 8) {                               // 8 slots + 8 chunks would spill
      if (ch <= 8) return launch_m16<16, SPW, 8, FQ, true>(a, G, stream);
    }
  }
  return hipErrorInvalidValue;
}

template <bool FQ>
static hipError_t launch_m16_half(const GemmArgs& a, int G, int sf, int ch, hipStream_t stream) {
  if (sf <= 1) return launch_m16_half_ch<2, FQ>(a, G, ch, stream);
  if (sf <= 2) return launch_m16_half_ch<4, FQ>(a, G, ch, stream);
  if (sf <= 3) return launch_m16_half_ch<6, FQ>(a, G, ch, stream);
  if (sf <= 4) return launch_m16_half_ch<8, FQ>(a, G, ch, stream);
  return hipErrorInvalidValue;
}

// The normalising BF16 staging: 8 waves, one workgroup per weight tile
// (rsplit as chosen), up to two 32-blocks per thread, up to 4 weight steps
// per wave (K <= 4096).  K <= 2048 and M <= 16 take the per-wave form (a
// wave's rows in one or two staging chunks, at most 2 weight steps a wave).
constexpr int kNormWaves = 8;

template <int SPW, int NRM>
static hipError_t launch_m16_norm_ch(const GemmArgs& a, int ch, hipStream_t stream) {
  const int grid = a.N / 16 * a.rsplit;
  if (ch <= 1) return launch_m16<kNormWaves, SPW, 1, true, false, NRM>(a, grid, stream);
  if (ch <= 2) return launch_m16<kNormWaves, SPW, 2, true, false, NRM>(a, grid, stream);
  return hipErrorInvalidValue;
}

static bool m16_norm_per_wave(int M, int K) { return K <= 2048 && M <= 2 * kNormWaves; }

static hipError_t launch_m16_norm(const GemmArgs& a, int spw, int ch, bool shared,
                                  hipStream_t stream) {
  if (m16_norm_per_wave(a.M, a.K) && !shared)
    return launch_m16_norm_ch<2, 2>(a, (a.M + kNormWaves - 1) / kNormWaves, stream);
  if (spw <= 2) return launch_m16_norm_ch<2, 1>(a, ch, stream);
  if (spw <= 4) return launch_m16_norm_ch<4, 1>(a, ch, stream);   // more would spill
  return hipErrorInvalidValue;
}

// Largest staging-register count instantiated for W waves (W = 4: one
// MXFP8 row only).
int m16_max_ch(int W, bool fq) { return fq ? (W == 4 ? 0 : 2) : (W == 4 ? 4 : 16); }

// Most weight steps per wave instantiated for W waves.
int m16_max_spw(int W) { return W == 4 ? 16 : 4; }

template <bool FQ>
static hipError_t launch_m16_w(const GemmArgs& a, int W, int spw, int ch, hipStream_t stream) {
  if constexpr (!FQ) {
    if (W == 4) {
      if (spw <= 4) return launch_m16_ch<4, 4, FQ>(a, ch, stream);
      if (spw <= 8) return launch_m16_ch<4, 8, FQ>(a, ch, stream);
      if (spw <= 10) return launch_m16_ch<4, 10, FQ>(a, ch, stream);
      if (spw <= 12) return launch_m16_ch<4, 12, FQ>(a, ch, stream);
      return launch_m16_ch<4, 16, FQ>(a, ch, stream);
    }
  }
  if (W != 16) return hipErrorInvalidValue;
  if (spw <= 1) return launch_m16_ch<16, 1, FQ>(a, ch, stream);
  if (spw <= 2) return launch_m16_ch<16, 2, FQ>(a, ch, stream);
  if (spw <= 3) return launch_m16_ch<16, 3, FQ>(a, ch, stream);
  return launch_m16_ch<16, 4, FQ>(a, ch, stream);
}

size_t gemm_2d_lds_bytes(int M, int MB) {
  const size_t act = (size_t)M * (16 * 128 + 16) + (size_t)M * (16 * 4 + 4);
  const size_t red = (size_t)kM16Waves * MB * 64 * sizeof(v4f);
  return ((act > red ? act : red) + 15) & ~(size_t)15;
}

namespace {

// A 2D plan: T tiles per workgroup, P K parts of Sp steps, SPW weight slots
// per wave.
struct Plan {
  int T, P, Sp, SPW;
  double cost;
};

constexpr int kSlotSizes[] = {1, 2, 3, 4, 6, 8};

int round_slots(int spw) {
  for (int v : kSlotSizes)
    if (spw <= v) return v;
  return 0;
}

// The time model of a plan: the busiest workgroup's bytes, weights at its
// share of HBM bandwidth and activations at the rate one CU pulls them from
// L2, plus the cross-workgroup sum of a K split: a fixed 1.2 us and the last
// arriving workgroup's read of the other P - 1 parts' FP32 tiles (1 KiB per
// weight tile and 16-row tile) at 60 GB/s.  Rates from measurements on
// MI355X (about 6.5 TB/s of weights streamed chip-wide; about 46 GB/s of
// activations into one CU while every CU reads the same lines); the split's
// terms were fitted to every plan timed at 17 / 24 / 32 / 48 rows on N x K =
// 2048 x 5120, 4096 x 5120, 5120 x 8192 and 8192 x 1536, where the chosen
// plan is then within 0.2 us of the fastest (a flat 1.5 us picked (4, 8) at
// 2048 x 5120, up to 1.1 us slower than (2, 4)).  T = P = 1 also models the
// M <= 16 kernel (one full-K tile per workgroup).
double plan_cost(int M, int N, int K, int T, int P, int cus, int rb = 1) {
  const int tiles = N / 16, S = K / 128, MB = (M + 15) / 16;
  const int Sp = (S + P - 1) / P;
  const int groups = tiles / T, wgs = groups * P * rb;
  const int rounds = (wgs + cus - 1) / cus;
  const int active = wgs < cus ? wgs : cus;
  const double wb = (double)T * Sp * 2112.0, ab = (double)M * Sp * 132.0;
  const double split = P > 1 ? 1.2e-6 + (double)(P - 1) * T * MB * 1024.0 / 60e9 : 0.0;
  return rounds * (wb / (6.5e12 / active) + ab / 46e9) + split;
}

// The 2D plan of least modelled time.
Plan choose_plan(int M, int N, int K, int group_tiles, int cus) {
  // More than 64 rows: 64-row blocks, each with the plan's tile groups and
  // K parts (and their own counters).
  const int rb = (M + kRowBlock - 1) / kRowBlock;
  if (M > kRowBlock) M = kRowBlock;
  const int tiles = N / 16, S = K / 128, MB = (M + 15) / 16;
  // MXG_PLAN="T,P" restricts the choice to that plan where it is valid
  // (tests and plan sweeps; ignored otherwise).
  int wantT = 0, wantP = 0;
  if (const char* e = std::getenv("MXG_PLAN")) {
    const char* c = std::strchr(e, ',');
    if (c) {
      wantT = std::atoi(e);
      wantP = std::atoi(c + 1);
    }
  }
  Plan best{0, 0, 0, 0, 1e30};
  for (int pass = 0; pass < 2 && best.T == 0; ++pass)
  for (int T : {1, 2, 4}) {
    if (tiles % T || (group_tiles && group_tiles % T) || T * MB > 16) continue;
    if (pass == 0 && wantT && T != wantT) continue;
    for (int P : {1, 2, 3, 4, 6, 8}) {
      if (pass == 0 && wantP && P != wantP) continue;
      if (P > S) break;
      const int Sp = (S + P - 1) / P;
      if ((P - 1) * Sp >= S) continue;                  // no empty part
      const int spw = round_slots((T * Sp + 15) / 16);
      if (spw == 0) continue;
      if (P > 1 && kGemmCtrOffset + (size_t)rb * (tiles / T) * kCtrStride * 4 > kCtrRegionBytes)
        continue;                                       // counters beyond their region
      const double cost = plan_cost(M, N, K, T, P, cus, rb);
      if (cost < best.cost) best = Plan{T, P, Sp, spw, cost};
    }
  }
  return best;
}

int device_cus() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
      cached = cus;
    else
      return 256;
  }
  return cached;
}

// Wave-local form (MXFP8 input, at most 64 rows, T * MB <= 8): SL steps
// per wave.
template <int MB, int T, int SL>
hipError_t launch_2d_wl(const GemmArgs& a, hipStream_t stream) {
  constexpr int CHM = (MB * 16 * 16 * 8 + kM16Waves * 64 - 1) / (kM16Waves * 64);
  auto kern = gemm_2d_kernel<MB, T, SL, 1, CHM, false, false, true>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 64);
    if (e != hipSuccess) return e;
    configured = true;
  }
  size_t lds = (size_t)kM16Waves * T * MB * 64 * 16;
  if (a.out_q) lds += (size_t)512 * MB * T;
  hipLaunchKernelGGL(kern, dim3((a.N / 16 / T) * a.P), dim3(kM16Waves * 64), lds, stream, a);
  return hipGetLastError();
}

template <int MB, int T>
hipError_t launch_2d_wl_sl(const GemmArgs& a, int sl, hipStream_t stream) {
  if (sl <= 1) return launch_2d_wl<MB, T, 1>(a, stream);
  if (sl <= 2) return launch_2d_wl<MB, T, 2>(a, stream);
  return launch_2d_wl<MB, T, 3>(a, stream);
}

// Whether the wave-local form takes the plan: MXFP8 input, one row block,
// T * MB <= 8, at most 3 steps per wave.
bool wl_fits(const GemmArgs& a, int T, int Sp) {
  const int MB = (a.M + 15) / 16, sl = (Sp + 15) / 16;
  if (sl == 3 && ((MB == 1 && T == 4) || (MB == 2 && T == 4) || (MB == 3 && T == 2))) return false;
  return a.x == nullptr && a.M <= 48 && T * MB <= 8 && sl <= 3;
}

hipError_t launch_2d_wave_local(const GemmArgs& a, int T, hipStream_t stream) {
  const int MB = (a.M + 15) / 16, sl = (a.Sp + 15) / 16;
  if (MB == 1) {
    if (T == 1) return launch_2d_wl_sl<1, 1>(a, sl, stream);
    if (T == 2) return launch_2d_wl_sl<1, 2>(a, sl, stream);
    return launch_2d_wl_sl<1, 4>(a, sl, stream);
  }
  if (MB == 2) {
    if (T == 1) return launch_2d_wl_sl<2, 1>(a, sl, stream);
    if (T == 2) return launch_2d_wl_sl<2, 2>(a, sl, stream);
    return launch_2d_wl_sl<2, 4>(a, sl, stream);
  }
  if (T == 1) return launch_2d_wl_sl<3, 1>(a, sl, stream);
  return launch_2d_wl_sl<3, 2>(a, sl, stream);
}

template <int MB, int T, int SPW, bool FQ>
hipError_t launch_2d(const GemmArgs& a, hipStream_t stream) {
  constexpr int CHM = (MB * 16 * 16 * 8 + kM16Waves * 64 - 1) / (kM16Waves * 64);
  constexpr int CHL = FQ ? 4 * MB : CHM;                 // staging registers per chunk (v4i)
  constexpr int NCH = (SPW + T - 1) / T;
  // The whole part's activations in registers (then in LDS at once) while
  // they fit beside the weight slots; otherwise chunk by chunk.
  constexpr bool kRegs = NCH * CHL * 4 + SPW * 9 + MB * 4 <= 120;
  const int Mb = a.M < kRowBlock ? a.M : kRowBlock;      // rows of one row block
  const size_t whole_lds = (size_t)Mb * (a.Sp * 128 + 16) + (size_t)Mb * (a.Sp * 4 + 4);
  const bool whole = kRegs && NCH > 1 && whole_lds <= 160 * 1024 - 64;
  const dim3 grid((a.N / 16 / T) * a.P * ((a.M + kRowBlock - 1) / kRowBlock));
  // with out_q: the partial tiles, then the BF16 output tile of 16 MB x 16 T
  size_t lds_min = gemm_2d_lds_bytes(Mb, MB);
  if (a.out_q) lds_min = std::max(lds_min, (size_t)kM16Waves * MB * 64 * 16 + (size_t)512 * MB * T);
  if (whole) {
    auto kern = gemm_2d_kernel<MB, T, SPW, (kRegs ? NCH : 1), CHM, FQ>;
    static bool configured = false;
    if (!configured) {
      // 160 KiB of LDS per workgroup, less the kernel's static word
      hipError_t e = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         160 * 1024 - 64);
      if (e != hipSuccess) return e;
      configured = true;
    }
    size_t lds = lds_min;
    if (whole_lds > lds) lds = (whole_lds + 15) & ~(size_t)15;
    hipLaunchKernelGGL(kern, grid, dim3(kM16Waves * 64), lds, stream, a);
  } else {
    auto kern = gemm_2d_kernel<MB, T, SPW, 1, CHM, FQ>;
    static bool configured = false;
    if (!configured) {
      hipError_t e = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         160 * 1024 - 64);
      if (e != hipSuccess) return e;
      configured = true;
    }
    hipLaunchKernelGGL(kern, grid, dim3(kM16Waves * 64), lds_min, stream, a);
  }
  return hipGetLastError();
}

template <int MB, int T, bool FQ>
hipError_t launch_2d_spw(const GemmArgs& a, int spw, hipStream_t stream) {
  switch (spw) {
    case 1: return launch_2d<MB, T, 1, FQ>(a, stream);
    case 2: return launch_2d<MB, T, 2, FQ>(a, stream);
    case 3: return launch_2d<MB, T, 3, FQ>(a, stream);
    case 4: return launch_2d<MB, T, 4, FQ>(a, stream);
    case 6: return launch_2d<MB, T, 6, FQ>(a, stream);
    default: return launch_2d<MB, T, 8, FQ>(a, stream);
  }
}

template <int MB, bool FQ>
hipError_t launch_2d_t(const GemmArgs& a, int T, int spw, hipStream_t stream) {
  if (T == 1) return launch_2d_spw<MB, 1, FQ>(a, spw, stream);
  if (T == 2) return launch_2d_spw<MB, 2, FQ>(a, spw, stream);
  return launch_2d_spw<MB, 4, FQ>(a, spw, stream);
}

// The RMSNorm in the 2D kernel's BF16 staging: two weight tiles per
// workgroup, no K split, the part one staging chunk (K <= 2048), at most 32
// rows (a wave's rows in registers: no LDS beyond the chunk's).
bool gemm_2d_norm_fits(const GemmArgs& a) {
  return a.x && a.norm_w && a.M <= 32 && a.K <= 2048 && (a.N / 16) % 2 == 0 && a.group_tiles == 0 &&
         (a.lda == 0 || a.lda == a.K) &&
         gemm_2d_lds_bytes(a.M, (a.M + 15) / 16) <= 160 * 1024 - 64;
}

template <int MB, int SPW>
hipError_t launch_2d_norm_k(const GemmArgs& a, hipStream_t stream) {
  constexpr int CHM = (MB * 16 * 16 * 8 + kM16Waves * 64 - 1) / (kM16Waves * 64);
  auto kern = gemm_2d_kernel<MB, 2, SPW, 1, CHM, true, true>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 64);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const size_t lds = gemm_2d_lds_bytes(a.M, MB);
  hipLaunchKernelGGL(kern, dim3(a.N / 32), dim3(kM16Waves * 64), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_2d_norm(const GemmArgs& args, hipStream_t stream) {
  GemmArgs a = args;
  const int S = a.K / 128;
  a.P = 1;
  a.Sp = S;
  a.out_q = a.out_s = nullptr;
  const bool one = (2 * S + 15) / 16 <= 1;               // weight slots per wave: 1 or 2
  if (a.M <= 16) return one ? launch_2d_norm_k<1, 1>(a, stream) : launch_2d_norm_k<1, 2>(a, stream);
  return one ? launch_2d_norm_k<2, 1>(a, stream) : launch_2d_norm_k<2, 2>(a, stream);
}

// With BF16 input only for M <= 32 (larger row counts would spill the
// staging registers); the caller quantizes the others first.
template <bool FQ>
hipError_t launch_2d_mb(const GemmArgs& a, int T, int spw, hipStream_t stream) {
  const int mb = a.M > kRowBlock ? kRowBlock / 16 : (a.M + 15) / 16;
  if (mb == 1) return launch_2d_t<1, FQ>(a, T, spw, stream);
  if constexpr (FQ) {
    if (mb == 2) return launch_2d_t<2, FQ>(a, T, spw, stream);
    return hipErrorInvalidValue;
  } else {
    if (mb == 2) return launch_2d_t<2, FQ>(a, T, spw, stream);
    if (mb == 3) return launch_2d_t<3, FQ>(a, T, spw, stream);
    return launch_2d_t<4, FQ>(a, T, spw, stream);
  }
}

}  // namespace

size_t gemm_partial_bytes(int M, int N, int K, int group_tiles) {
  const Plan pl = choose_plan(M, N, K, group_tiles, device_cus());
  const int rb = (M + kRowBlock - 1) / kRowBlock;
  const int MB = M > kRowBlock ? kRowBlock / 16 : (M + 15) / 16;
  return pl.P > 1 ? (size_t)rb * (N / 16) * pl.P * MB * 64 * 16 : 0;
}

// MXG_DIRECT_KERNEL ("m16" / "2d" / "m16h") forces the kernel where it
// applies (tests use it to cover each on the same shapes); 0 = choose.
int forced_kernel() {
  const char* e = std::getenv("MXG_DIRECT_KERNEL");
  if (!e) return 0;
  if (std::strcmp(e, "m16") == 0) return 1;
  if (std::strcmp(e, "2d") == 0) return 2;
  if (std::strcmp(e, "m16h") == 0) return 3;
  return 0;
}

// Whether the M <= 16 kernel's HALF form takes the shape: G < tiles <= 1.5 G
// (one tile per workgroup plus half a leftover tile for some), at most 4
// full-tile slots per wave (K <= 8192), the activation in LDS, no grouping.
// MXFP8 input of at most 8 chunks per thread (4 with 8 weight slots, which
// would spill with more), or BF16 input of at most two 32-blocks per thread
// (M * K <= 65536).
bool gemm_m16_half_fits(const GemmArgs& a, int G) {
  const int tiles = a.N / 16, S = a.K / 128;
  if (a.M > 16 || a.group_tiles != 0 || tiles <= G || 2 * (tiles - G) > G || S > 64) return false;
  if (gemm_m16_half_lds_bytes(a.M, a.K, 16) > 160 * 1024) return false;
  return a.x ? a.M * a.K <= 65536 : a.M * a.K / 16 <= (S > 48 ? 4 : 8) * 1024;
}

// Whether the M <= 16 kernel can stage this activation in LDS.
bool gemm_m16_fits(int M, int K, int W) {
  return M <= 16 && gemm_m16_lds_bytes(M, K, W) <= 160 * 1024;
}

// Waves per workgroup of the M <= 16 kernel.  With one MXFP8 row, 4 waves
// holding up to 16 weight steps each (fewer waves to launch, fewer partial
// tiles to sum, the activation a few hundred bytes) measured 6-8 % faster
// than 16 waves at K = 1536, 4096 and 8192 on MI355X, but 3 % slower at
// K = 5120 (10 steps per wave against 2 or 3), which keeps 16.  With more
// rows, or BF16 input, the activation staging and quantize spread over 16
// waves win (4 and 8 waves measured 0.2-0.9 us slower than 16 for BF16
// input at N 4096, K 5120, M = 1..8).  MXG_M16_WAVES=16 forces 16 waves for
// one row as well (tests cover both); 0 is returned when the kernel cannot
// take the shape.
int m16_waves(int M, int K, bool fq) {
  const int S = K / 128;
  const char* e = std::getenv("MXG_M16_WAVES");
  const int want = e && std::atoi(e) == 16 ? 16 : 0;
  for (int W : {4, 16}) {
    if (want && W != want) continue;
    if (W == 4 && (M != 1 || fq || K == 5120)) continue;
    const int steps = (S + W - 1) / W;
    const int per = fq ? M * K / 32 : M * K / 16;
    const int ch = (per + W * 64 - 1) / (W * 64);
    if (steps <= m16_max_spw(W) && ch <= m16_max_ch(W, fq) && gemm_m16_fits(M, K, W)) return W;
  }
  return 0;
}

// Workgroups per 16-row weight tile in the M <= 16 kernel: 2 when the tile
// count leaves at least half the CUs idle and K >= 4096, else 1.  Measured on
// MI355X: 2.5-7 % faster at N = 1024 and 2048 with K = 4096 or 5120 (e.g.
// BF16 M = 4, N 2048, K 5120: 4.97 against 5.34 us), 2 % slower at K = 2048
// (launch-bound); a split of 4 was slower wherever the tiles filled a quarter
// of the chip or more.  MXG_M16_RSPLIT=1|2|4 forces the split (tests cover
// all three).
int m16_row_split(int N, int K, bool) {
  if (const char* e = std::getenv("MXG_M16_RSPLIT")) {
    const int v = std::atoi(e);
    if (v == 1 || v == 2 || v == 4) return v;
  }
  return (N / 16) * 2 <= device_cus() && K >= 4096 ? 2 : 1;
}

// MXFP8 input of at most 4 rows on a weight of G < tiles <= 1.5 G tiles and
// K >= 4096: two half-tile workgroups per tile (2 x tiles workgroups of 16
// waves).  Measured on MI355X at N 5120, K 8192: 9.8-10.5 us at M = 1 and
// 10.4-11.3 at M = 4, against 10.5-11.1 and 11.1-11.4 for the 2D kernel and
// 11.2 and 11.6 for one tile plus half a leftover tile per workgroup.
bool m16_half_tiles_wide(int M, int N, int K, bool fq) {
  const int tiles = N / 16, G = device_cus();
  return !fq && M <= 4 && K >= 4096 && tiles > G && 2 * (tiles - G) <= G;
}

hipError_t launch_gemm(const GemmArgs& args, hipStream_t stream, bool* quantized_out) {
  if (quantized_out) *quantized_out = false;
  GemmArgs a = args;
  if (a.lda == 0) a.lda = a.K;
  const bool fq = a.x != nullptr;
  if (fq && (a.group_tiles != 0 || a.lda != a.K)) return hipErrorInvalidValue;
  if (a.a_sf128 && (fq || a.group_tiles != 0 || a.lda != a.K)) return hipErrorInvalidValue;
  if (a.M > 48) {
    // More than 48 rows: the 2D kernel over 64-row blocks (one block up to
    // 64 rows), MXFP8 input (BF16 input is quantized by its own launch
    // first).
    if (a.group_tiles != 0) return hipErrorInvalidValue;
    a.out_q = a.out_s = nullptr;                         // not on row blocks
    if (fq) {
      hipError_t e = launch_quantize(a.x, a.M, a.K, a.ld_x, a.a_q, a.a_s, stream);
      if (e != hipSuccess) return e;
      a.x = nullptr;
    }
    // Above 48 rows (measured on MI355X, us, wide / 64 x 64 / row blocks):
    //   * above 64 rows at K >= 4096: the wide form (K split across the waves; 2 or 4 weight
    //     tiles per workgroup, in one round where a count allows): N 4096,
    //     K 5120, M = 96 / 256: 11.2 / 15.1 against 15.7 / 16.2 and 15.0 /
    //     26.7; N 5120, K 8192, M = 128 / 256: 20.2 / 35.8 against 24.3 /
    //     39.7; N 2048, K 16384, M = 128: 23.5 against 43.5 and 30.5;
    //   * above 64 rows at K < 4096: the 64 x 64 form, whose 4-step chunks suit short K
    //     better than the wide form's 8 steps (N 8192, K 1536, M = 96 / 256:
    //     7.4 / 10.3 against 8.2 / 14.7 and 8.5 / 15.5);
    //   * 49-64 rows: the wide form where two or more weight tiles per
    //     workgroup fill one round (N 5120, K 8192, M = 56: 15.4 against
    //     17.9; N 8192, K 1536, M = 64: 6.9 against 7.3), else the row
    //     blocks, whose K split fills the CUs (N 2048, K 16384, M = 64: 14.7
    //     against 24.1 in the wide form's 128 workgroups);
    //   * else (a shape neither takes) the row blocks below.
    // MXG_BIG_KERNEL=wide|64 forces a form where it takes the shape, and
    // MXG_DIRECT_KERNEL=2d keeps the row blocks.
    const char* bk = std::getenv("MXG_BIG_KERNEL");
    const int bforce = !bk ? 0 : std::strcmp(bk, "wide") == 0 ? 1 : std::strcmp(bk, "64") == 0 ? 2 : 0;
    if (a.M <= 64 && forced_kernel() != 2 && gemm_wide_fits(a) &&
        (bforce == 1 || (bforce == 0 && gemm_wide_tiles(a, device_cus()) >= 2)))
      return launch_gemm_wide(a, device_cus(), stream);
    if (a.M > 64 && forced_kernel() != 2) {
      if (gemm_wide_fits(a) && (bforce == 1 || (bforce == 0 && a.K >= 4096)))
        return launch_gemm_wide(a, device_cus(), stream);
      if (gemm_big_fits(a) && bforce != 1) return launch_gemm_big(a, device_cus(), stream);
    }
    const Plan pl = choose_plan(a.M, a.N, a.K, 0, device_cus());
    if (pl.T == 0) return hipErrorInvalidValue;
    a.P = pl.P;
    a.Sp = pl.Sp;
    if (pl.P > 1 && (a.ctr == nullptr || a.part == nullptr)) return hipErrorInvalidValue;
    return launch_2d_mb<false>(a, pl.T, pl.SPW, stream);
  }
  const int S = a.K / 128;
  int force = forced_kernel();                             // tests: 1 = M <= 16, 2 = 2D, 3 = HALF
  if (a.norm_w) {
    // Where the norm runs (every workgroup normalises the rows it stages, so
    // its vector work grows with the rows and the workgroups; measured on
    // MI355X, the chain at N 8192, K 1536 for B):
    //   * M <= 4: in the M <= 16 kernel's BF16 staging (M = 1 / 2 / 4: 19.6 /
    //     19.8 / 20.5 us for the chain against 19.9 / 20.2 / 20.7 in the 2D
    //     kernel, 22.8 / 23.0 / 23.4 with a launch; 19.5 / 19.5 / 20.0
    //     without the norm);
    //   * 5 <= M <= 16: in the 2D kernel's staging, two tiles per workgroup,
    //     no K split (M = 8 / 12 / 16: 22.8 / 24.2 / 25.2 us against 23.2 /
    //     25.8 / 27.8 in the M <= 16 kernel and 24.9 / 25.6 / 26.0 with a
    //     launch);
    //   * above 16 rows, or where neither form takes the shape: RMSNorm +
    //     MXFP8 as its own launch, and the GEMM reads the codes (M = 32:
    //     32.3 us against 34.7 in the 2D kernel).
    // MXG_NORM_KERNEL=2d|m16|launch forces the form where it takes the shape
    // (tests and sweeps); m16lds forces the M <= 16 kernel's shared (NRM = 1)
    // form where the per-wave one would run.
    const char* nk = std::getenv("MXG_NORM_KERNEL");
    const int nforce = !nk ? 0 : std::strcmp(nk, "2d") == 0 ? 1 : std::strcmp(nk, "m16") == 0 ? 2
                                 : std::strcmp(nk, "launch") == 0 ? 3
                                 : std::strcmp(nk, "m16lds") == 0 ? 4 : 0;
    const bool norm2d = gemm_2d_norm_fits(a) && force != 1 && force != 3 &&
                        (nforce == 1 || (nforce == 0 && (force == 2 || (a.M > 4 && a.M <= 16))));
    if (norm2d) return launch_2d_norm(a, stream);
    constexpr int NW = kNormWaves, NT = NW * 64;
    const int per_cu = (a.N / 16 + device_cus() - 1) / device_cus();
    const bool inline_ok = a.x && a.M <= 16 && (a.M * a.K / 32) * per_cu <= 2048 &&
                           a.M * a.K / 32 <= 2 * NT && a.K <= 8 * NT && (S + NW - 1) / NW <= 4 &&
                           gemm_m16_lds_bytes(a.M, a.K, NW) + (size_t)a.K * 2 <= 160 * 1024 &&
                           force != 2 && force != 3 && nforce != 1 && nforce != 3;
    if (inline_ok) {
      GemmArgs b = a;
      b.rsplit = m16_row_split(a.N, a.K, true);
      return launch_m16_norm(b, (S + NW - 1) / NW, (a.M * a.K / 32 + NT - 1) / NT, nforce == 4,
                             stream);
    }
    hipError_t e = launch_rmsnorm_quantize(a.x, a.M, a.K, a.ld_x, a.norm_w, a.norm_eps, a.norm_y,
                                           a.K, a.a_q, a.a_s, 0, stream);
    if (e != hipSuccess) return e;
    GemmArgs b = a;
    b.x = nullptr;
    b.norm_w = nullptr;
    return launch_gemm(b, stream, quantized_out);
  }
  // A weight of G < tiles <= 1.5 G tiles with BF16 input: one tile per CU
  // plus half a leftover tile for some, no sum across workgroups.  A read of
  // the weight alone in this order takes 8.0 us on MI355X at N 5120, K 8192,
  // against 8.9 us for one tile per workgroup (a second round on a quarter of
  // the CUs) and 8.3 us for 640 half tiles; with BF16 input the GEMM measured
  // 11.5 / 12.2 us at M = 1 / 4 against 12.3 / 13.4 for the next best form.
  // (With MXFP8 input two half-tile workgroups per tile measured faster up to
  // 4 rows, and the 2D kernel above; see m16_row_split.)
  if ((force == 3 || (force == 0 && a.x)) && gemm_m16_half_fits(a, device_cus())) {
    GemmArgs h = a;
    h.rsplit = 1;
    const int sf = (S + 15) / 16;
    if (!a.x) return launch_m16_half<false>(h, device_cus(), sf, (a.M * a.K / 16 + 1023) / 1024,
                                            stream);
    return launch_m16_half<true>(h, device_cus(), sf, (a.M * a.K / 32 + 1023) / 1024, stream);
  }
  if (force == 3) force = 0;                               // HALF does not take the shape
  Plan pl = choose_plan(a.M, a.N, a.K, a.group_tiles, device_cus());
  // BF16 input, at most 12 weight steps (K <= 1536) and at least two weight
  // tiles per CU: T = 2 or 4 tiles per workgroup in the 2D kernel, no K
  // split, so that each CU quantizes the rows once instead of once per tile.
  // Measured on MI355X (us, the M <= 16 kernel -> this plan): N 8192, K 1536
  // (T = 2), M = 1 / 4 / 8 / 16: 4.87 / 4.91 / 5.08 / 5.97 -> 4.77 / 4.82 /
  // 4.92 / 5.37; N 16384, K 1536 (T = 4), M = 1 / 4 / 8: 7.85 / 7.84 / 8.09
  // -> 6.53 / 6.54 / 6.62.  With a longer K the M <= 16 kernel's weight
  // stream wins (N 8192, K 4096, M = 1: 8.74 against 9.78 with T = 2).
  {
    const int tiles = a.N / 16, cus = device_cus();
    const int T = tiles >= 4 * cus ? 4 : 2;
    if (force == 0 && fq && a.M <= 16 && a.K <= 1536 && a.group_tiles == 0 && tiles >= 2 * cus &&
        tiles % T == 0) {
      pl = Plan{T, 1, S, round_slots((T * S + 15) / 16), 0.0};
      force = 2;                                           // the 2D kernel below
    }
  }
  // MXFP8 input, at most 16 rows, on at least two tiles per CU where the
  // M <= 16 kernel's LDS (the whole activation) admits one workgroup per CU,
  // so its tiles take a second round: the 2D kernel with one tile per
  // workgroup and no K split stages the activation in 2048-column chunks,
  // and two of its workgroups share a CU.  Measured on MI355X (N 8192,
  // K 4096, M = 16): 9.66 us in the M <= 16 kernel, 9.00 in this plan (9.51
  // in the model's (2, 1)); at 8 and 12 rows, where two M <= 16 workgroups
  // fit a CU, that kernel stays faster (7.97 / 8.15 against 8.43 / 8.61).
  {
    const int tiles = a.N / 16, cus = device_cus();
    const size_t lds_cu = 160 * 1024;
    if (force == 0 && !fq && a.M <= 16 && tiles >= 2 * cus &&
        2 * gemm_m16_lds_bytes(a.M, a.K, 16) > lds_cu &&
        2 * gemm_2d_lds_bytes(a.M, (a.M + 15) / 16) <= lds_cu) {
      const int spw = round_slots((S + 15) / 16);
      if (spw) {
        pl = Plan{1, 1, S, spw, 0.0};
        force = 2;
      }
    }
  }
  // One full-K tile per workgroup with the whole activation in LDS unless
  // the model gives a 2D plan at most 3/4 of its time: the M <= 16 kernel
  // keeps more loads in flight per CU (two workgroups share a CU when their
  // LDS fits) and has less fixed cost, which the model leaves out.  (With
  // BF16 input either choice pays about as much for the quantize: in-kernel
  // in the M <= 16 kernel, a launch before the 2D kernel.)
  const bool m16_fast = pl.cost >= 0.75 * plan_cost(a.M, a.N, a.K, 1, 1, device_cus());
  // In-kernel quantize up to 2048 32-blocks (M*K <= 65536) per workgroup a
  // CU runs: measured faster than a quantize launch up to there (every
  // workgroup repeats the whole quantize, so a grid of two rounds counts
  // double).
  const int per_cu = (a.N / 16 + device_cus() - 1) / device_cus();
  const bool fq_inline = fq && (a.M * a.K / 32) * per_cu <= 2048;
  const bool wide_halves = force == 0 && m16_half_tiles_wide(a.M, a.N, a.K, fq) &&
                           std::getenv("MXG_M16_WAVES") == nullptr &&
                           std::getenv("MXG_M16_RSPLIT") == nullptr;
  const int W = wide_halves && gemm_m16_fits(a.M, a.K, 16) && (S + 15) / 16 <= m16_max_spw(16)
                    ? 16
                    : m16_waves(a.M, a.K, fq && fq_inline);
  if (W && (force == 1 || (force == 0 && (m16_fast || wide_halves)))) {
    const int steps = (S + W - 1) / W;                     // weight steps per wave
    const int per = fq ? a.M * a.K / 32 : a.M * a.K / 16;  // 32-blocks, or 16-byte chunks
    const int ch = (per + W * 64 - 1) / (W * 64);
    a.rsplit = wide_halves ? 2 : m16_row_split(a.N, a.K, fq);
    if (!fq) return launch_m16_w<false>(a, W, steps, ch, stream);
    // In-kernel quantize while the weight stream is in flight when the
    // activation is small enough (every workgroup quantizes all of it, one
    // 32-block per lane at a time); larger activations are quantized by
    // their own launch first.
    if (fq_inline) return launch_m16_w<true>(a, W, steps, ch, stream);
    hipError_t e = launch_quantize(a.x, a.M, a.K, a.ld_x, a.a_q, a.a_s, stream);
    if (e != hipSuccess) return e;
    GemmArgs b = a;
    b.x = nullptr;
    return launch_gemm(b, stream, quantized_out);
  }
  // Otherwise the 2D kernel.  BF16 input is quantized while staging when
  // M <= 32 and a workgroup's share is small (M * Sp <= 1024: at most four
  // 32-blocks per thread over its K part), else by its own launch first.
  if (pl.T == 0) return hipErrorInvalidValue;
  GemmArgs b = a;
  b.P = pl.P;
  b.Sp = pl.Sp;
  if (pl.P > 1 && (b.ctr == nullptr || b.part == nullptr)) return hipErrorInvalidValue;
  // (Only where the kernel holds the whole part's BF16 blocks in registers:
  // chunk by chunk, the in-kernel quantize measured no faster.)
  const int nch_fq = (pl.SPW + pl.T - 1) / pl.T, mb_fq = (a.M + 15) / 16;
  const bool fq_regs = nch_fq * 16 * mb_fq + pl.SPW * 9 + 4 * mb_fq <= 120 &&
                       (size_t)a.M * (pl.Sp * 128 + 16) + (size_t)a.M * (pl.Sp * 4 + 4) <=
                           160 * 1024 - 64;
  // The output's MXFP8 in the epilogue where a workgroup holds whole 32-column
  // blocks (two or more weight tiles).
  const bool qz = b.out_q && pl.T >= 2 && b.qn > 0 && b.qn % 32 == 0 && b.qn <= b.N;
  if (!qz) b.out_q = b.out_s = nullptr;
  hipError_t e;
  if (fq && a.M <= 32 && a.M * pl.Sp <= 1024 && fq_regs) {
    e = launch_2d_mb<true>(b, pl.T, pl.SPW, stream);
  } else {
    if (fq && (e = launch_quantize(a.x, a.M, a.K, a.ld_x, a.a_q, a.a_s, stream)) != hipSuccess)
      return e;
    b.x = nullptr;
    // The wave-local form where every wave has a step of the part (Sp >= 12
    // of 16 waves) and each B operand feeds two or more weight tiles; with a
    // shorter part its idle waves leave fewer loads in flight than the
    // staged form, and one tile per workgroup gains nothing.  Measured on
    // MI355X (MXFP8 input, M = 17 / 24 / 32, staged -> wave-local, us):
    // N 8192 K 1536, plan (2, 1): 5.29 / 5.50 / 5.68 -> 4.91 / 5.20 / 5.36;
    // N 5120 K 8192, (4, 3): 13.65 / 14.09 / 13.88 -> 12.45 / 12.83 / 13.31;
    // N 8192 K 4096, (2, 1): 11.17 / 11.85 / 12.22 -> 10.35 / 11.20 / 11.97;
    // and the other way at N 4096 K 5120, (4, 4), Sp = 10: 8.70 / 8.80 ->
    // 8.79 / 8.99, and N 2048 K 5120, (4, 8), Sp = 5: 7.8 -> 8.4.
    // MXG_WAVE_LOCAL=1|0 forces the form on (where it takes the plan) or off.
    const char* wle = std::getenv("MXG_WAVE_LOCAL");
    const bool wl = wl_fits(b, pl.T, pl.Sp) &&
                    (wle ? wle[0] == '1' : pl.T >= 2 && pl.Sp >= 12);
    if (wl)
      e = launch_2d_wave_local(b, pl.T, stream);
    else
      e = launch_2d_mb<false>(b, pl.T, pl.SPW, stream);
  }
  if (e == hipSuccess && qz && quantized_out) *quantized_out = true;
  return e;
}

}  // namespace mxg
