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

// Larger of the two BF16 magnitudes of a packed pair, as magnitude bits.
// For non-negative floats the bit patterns order like the values, so the
// block maximum is an integer maximum.
__device__ __forceinline__ uint32_t bf16_pair_absmax_bits(uint32_t w) {
  uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
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

// Scales two FP32 values by 2^-e (exact), saturates them to +-448 and
// converts them to E4M3 with round-to-nearest-even; the two codes land in the
// low (HI = false) or high (HI = true) 16 bits of `old`.  The hardware
// conversion rounds to nearest even on the whole E4M3 grid, subnormals
// included, but returns NaN above 464, hence the clamp first.
template <bool HI>
__device__ __forceinline__ uint32_t enc2_e4m3(float a, float b, int neg_e, uint32_t old) {
  float va = __builtin_amdgcn_ldexpf(a, neg_e);
  float vb = __builtin_amdgcn_ldexpf(b, neg_e);
  va = __builtin_fminf(__builtin_fmaxf(va, -448.0f), 448.0f);
  vb = __builtin_fminf(__builtin_fmaxf(vb, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(va, vb, (int)old, HI);
}

// Four BF16 values (two packed pairs) -> four E4M3 codes in one dword,
// element order preserved (lowest address in the lowest byte).
__device__ __forceinline__ uint32_t enc4_e4m3(uint32_t w0, uint32_t w1, int neg_e) {
  uint32_t r = enc2_e4m3<false>(bf16_lo(w0), bf16_hi(w0), neg_e, 0u);
  return enc2_e4m3<true>(bf16_lo(w1), bf16_hi(w1), neg_e, r);
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

}  // namespace mxg
