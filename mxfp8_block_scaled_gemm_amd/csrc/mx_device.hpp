// Device helpers shared by the libmxgemm kernels (gfx950 only).
//
// MXFP8 here: E4M3 ("FN") element codes with one UE8M0 power-of-two scale per
// 32 consecutive K elements ([mxfp8] page, compile_low_latency: Float8E4M3FN
// operands, Float8E8M0FNU scales, sf_vec_size 32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- BF16

// Low / high BF16 of a packed pair, widened exactly to FP32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// FP32 -> BF16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two FP32 values -> packed BF16 (lo in bits 0-15, hi in 16-31), round to
// nearest, ties to even, in one instruction (v_cvt_pk_bf16_f32): for every
// finite input the same bits as f32_to_bf16, and a NaN stays a NaN.
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  const v2f v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, v2bf16));
}

// Sum over a wave's 64 lanes, the same value in every lane, with no LDS
// round trip: DPP adds within each row of 16 lanes with partners l ^ 1 and
// l ^ 2 (quad permutes), then 7 - l and 15 - l within the half row and the
// row (mirrors; after the steps before them these add the same values as
// partners l ^ 4 and l ^ 8 would), then the four row sums, read from lanes
// 0, 16, 32 and 48, added as (r0 + r1) + (r2 + r3).  All 64 lanes must be
// active.
template <int CTRL>
__device__ __forceinline__ float add_dpp(float t) {
  return t + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(t), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float t) {
  t = add_dpp<0xB1>(t);    // quad_perm [1, 0, 3, 2]
  t = add_dpp<0x4E>(t);    // quad_perm [2, 3, 0, 1]
  t = add_dpp<0x141>(t);   // row_half_mirror
  t = add_dpp<0x140>(t);   // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 48));
  return (r0 + r1) + (r2 + r3);
}

// Maximum over the 4 lanes of each aligned lane quad (DPP quad permutes:
// no LDS round trip).
__device__ __forceinline__ uint32_t quad_max(uint32_t a) {
  uint32_t b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  a = a > b ? a : b;
  b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, false);           // [2,3,0,1]
  return a > b ? a : b;
}

// ------------------------------------------------------- scale exponent

// Exponent e of the block scale 2^e from the block's amax (BF16 magnitude
// bits): e = floor(log2 amax) - 8 (8 = E4M3's largest exponent, 448 =
// 1.75 * 2^8), clamped to the UE8M0 range; an all-zero block takes the
// smallest scale, byte 0.  Pure integer arithmetic on the bit fields.
__device__ __forceinline__ int block_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  int E = (int)(amax_bits >> 7);
  int p = E > 0 ? E - 127 : (31 - __clz((int)amax_bits)) - 133;  // subnormal: m * 2^-133
  int e = p - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// --------------------------------------------------------------- E4M3

typedef short v2s __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// Larger BF16 magnitude (as bits) over two packed pairs, per 16-bit half.
// For non-negative floats the bit patterns order like the values, so a
// block's amax is an integer maximum of its magnitude bits.
__device__ __forceinline__ uint32_t bf16x2_absmax2(uint32_t a, uint32_t b) {
  const v2u16 x = __builtin_bit_cast(v2u16, a & 0x7FFF7FFFu);
  const v2u16 y = __builtin_bit_cast(v2u16, b & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}
__device__ __forceinline__ uint32_t halves_max(uint32_t m) {
  const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
  return lo > hi ? lo : hi;
}

// The block's scale 2^e and saturation bound 448 * 2^e as FP32, built from
// their bit fields (2^-127 is an FP32 subnormal; the bound is always normal).
struct BlockScale {
  float scale, bound;
};
__device__ __forceinline__ BlockScale block_scale(int e) {
  BlockScale b;
  b.scale = __uint_as_float(e > -127 ? (uint32_t)(e + 127) << 23 : 0x00400000u);
  b.bound = __uint_as_float(((uint32_t)(e + 135) << 23) | 0x00600000u);
  return b;
}

// Two FP32 values -> two E4M3 codes of x / 2^e, round to nearest even,
// saturated to +-448: the hardware MX convert divides by the scale and
// rounds to nearest even over the whole E4M3 grid (subnormals included) but
// gives NaN above 464, so the inputs are first clamped to +-448 * 2^e (exact:
// both are powers of two times representable values).  The codes land in the
// low (HI = false) or high (HI = true) 16 bits of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t enc2_e4m3(float a, float b, BlockScale bs, uint32_t old) {
  const float ca = __builtin_amdgcn_fmed3f(a, -bs.bound, bs.bound);
  const float cb = __builtin_amdgcn_fmed3f(b, -bs.bound, bs.bound);
  return __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(v2s, old), ca, cb,
                                                         bs.scale, HI));
}

// Four BF16 values (two packed pairs) -> four E4M3 codes in one dword,
// element order preserved (lowest address in the lowest byte).
__device__ __forceinline__ uint32_t enc4_e4m3(uint32_t w0, uint32_t w1, BlockScale bs) {
  uint32_t r = enc2_e4m3<false>(bf16_lo(w0), bf16_hi(w0), bs, 0u);
  return enc2_e4m3<true>(bf16_lo(w1), bf16_hi(w1), bs, r);
}

// ---------------------------------------------------------------- MFMA

// D = A . B + C on one 16 x 16 x 128 tile of E4M3 operands, each lane's
// operand carrying one UE8M0 scale byte (byte 0 of sa / sb).
//
// Lane layout of v_mfma_scale_f32_16x16x128_f8f6f4 (g = lane / 16,
// r = lane % 16, measured on gfx950):
//   A: row r; operand bytes 0..15 are K [16g, 16g+16), bytes 16..31 are
//      K [64+16g, 64+16g+16); the scale byte scales row r over K [32g, 32g+32).
//   B: the same with column r in place of row r.
//   D: lane holds D[4g + i][r] for i = 0..3.
__device__ __forceinline__ v4f mfma_mx16(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ v8i cat8(v4i lo, v4i hi) {
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// 16-byte global load / store.
__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }
__device__ __forceinline__ void st16(void* p, v4i v) { *reinterpret_cast<v4i*>(p) = v; }

// ------------------------------------------------------- weight layouts
//
// A 16-row weight tile t holds codes [16tK, 16(t+1)K) and scale bytes
// [tK/2, (t+1)K/2) both in the row-major layout ([N, K] codes, [N, K/32]
// scales) and in the packed one (pack.hip); only the order inside the tile
// differs.  For the 128-wide K step s, lane l of a scaled 16x16x128 MFMA
// (A row r = l % 16, K group g = l / 16) takes codes K[16g, 16g+16) ("lo")
// and K[64+16g, 64+16g+16) ("hi") of row r, and the scale of row r over
// block K[32g, 32g+32).  Inside the tile they sit at
//   lo: s * step_q + lane_q,   hi: lo + half_q,   scale: s * step_s + lane_s.
struct WeightLane {
  uint32_t step_q, half_q, lane_q, step_s, lane_s;
};
__device__ __forceinline__ WeightLane weight_lane(bool row_major, int K, int lane) {
  const int r = lane & 15, g = lane >> 4;
  if (row_major)
    return {128u, 64u, (uint32_t)(r * K + 16 * g), 4u, (uint32_t)(r * (K >> 5) + g)};
  return {2048u, 1024u, (uint32_t)(16 * lane), 64u, (uint32_t)lane};
}

// ------------------------------------------------------- buffer loads
//
// Raw buffer loads with a byte range: an access at or beyond `bytes` returns
// zero without touching memory, which predicates a load without a branch
// (so the number of outstanding loads stays static for s_waitcnt).
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ v4i buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// Streaming variant for data read exactly once (the weights): non-temporal
// cache policy, so the stream does not evict reused lines.
__device__ __forceinline__ v4i buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
__device__ __forceinline__ uint32_t buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

}  // namespace mxg
