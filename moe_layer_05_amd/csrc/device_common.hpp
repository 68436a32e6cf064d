// Device helpers shared by the kernels of the fused MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr float kFp8Max = 448.0f;   // largest finite OCP E4M3 value

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------- E4M3

// float32 -> OCP E4M3 code: nearest, ties to the even mantissa, saturating to
// +-448, sign kept (tiny negatives give 0x80).  Integer-exact: the magnitude
// is clamped, subnormals (< 2^-6) are scaled by 2^9 and rounded to an
// integer mantissa, normals have their float32 mantissa rounded to 3 bits and
// their exponent re-biased from 127 to 7.  Not for NaN.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), kFp8Max);
  uint32_t code;
  if (a < 0.015625f) {                        // 2^-6: subnormal range
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // 0..8, exact scaling
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);         // RNE to 3 mantissa bits
    code = (b >> 20) - ((127u - 7u) << 3);
  }
  return code | sign;
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp) and
// exponential; for very negative z, e^-z is +inf and the result is -0.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Activation scale from an amax stored as float bits: amax / 448, 1 if zero.
__device__ __forceinline__ float scale_from_amax_bits(uint32_t amax_bits) {
  float amax = __uint_as_float(amax_bits);
  return amax > 0.0f ? amax / kFp8Max : 1.0f;
}

// ---------------------------------------------------------------- waves

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------- amax

// A per-tensor amax is gathered in kAmaxSlots words, each on its own 128-byte
// line, so thousands of waves updating it do not serialise on one address;
// after the producer kernel has finished, one wave reads all slots.  Layout of
// an amax block: slot i at word i * kAmaxStride, then the final value (written
// once by the consumer) at word kAmaxFinal.
constexpr int kAmaxSlots = 64;
constexpr int kAmaxStride = 32;
constexpr int kAmaxFinal = kAmaxSlots * kAmaxStride;
constexpr int kAmaxWords = kAmaxFinal + 32;

// Non-negative floats order like their bit patterns: atomicMax on the bits.
__device__ __forceinline__ void amax_slot_max(uint32_t* block, uint32_t key, float v) {
  atomicMax(block + (key % kAmaxSlots) * kAmaxStride, __float_as_uint(v));
}

// Word to clear for index t < kAmaxSlots * nblocks of consecutive amax blocks.
__device__ __forceinline__ int amax_zero_index(int t) {
  return (t / kAmaxSlots) * kAmaxWords + (t % kAmaxSlots) * kAmaxStride;
}

// The maximum over all slots of an amax block, in every lane of the wave.
__device__ __forceinline__ float amax_slots_reduce(const uint32_t* block) {
  const int lane = threadIdx.x & (kWave - 1);
  return wave_max(__uint_as_float(block[lane * kAmaxStride]));
}

}  // namespace moe
