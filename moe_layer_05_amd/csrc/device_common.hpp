// Device helpers shared by the kernels of the fused MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr float kFp8Max = 448.0f;   // largest finite OCP E4M3 value
constexpr float kE5m2Max = 57344.0f;  // largest finite OCP E5M2 value

// Operand formats of the expert products: bfloat16, or FP8 codes in E4M3 or
// E5M2 (the FP8 explainer of the kongchang.com page names both).
constexpr int kFmtBF16 = 0;
constexpr int kFmtE4M3 = 1;
constexpr int kFmtE5M2 = 2;

template <int FMT>
constexpr float fp8_max() {
  return FMT == kFmtE5M2 ? kE5m2Max : kFp8Max;
}

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

// Four consecutive partial outputs at element `idx` of a partial-row buffer:
// float32, or bfloat16 (nearest even) when `bf16`.
__device__ __forceinline__ void store_part4(void* buf, bool bf16, int64_t idx, float a, float b,
                                            float c, float d) {
  if (bf16) {
    uint2 pk;
    pk.x = f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
    pk.y = f32_to_bf16_bits(c) | (f32_to_bf16_bits(d) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(buf) + idx) = pk;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(buf) + idx) = make_float4(a, b, c, d);
  }
}

// Per-row dequantisation scales of four consecutive weight rows r..r+3 (r a
// multiple of 4, so one 16-byte load), each times the activation row's scale.
__device__ __forceinline__ void row_scales4(const float* ws, int r, float sa, float (&out)[4]) {
  const float4 w = *reinterpret_cast<const float4*>(ws + r);
  out[0] = w.x * sa;
  out[1] = w.y * sa;
  out[2] = w.z * sa;
  out[3] = w.w * sa;
}
// The same for a gate row group and its up row group.
__device__ __forceinline__ void row_scales4(const float* ws, int rg, int ru, float sa,
                                            float (&g)[4], float (&u)[4]) {
  row_scales4(ws, rg, sa, g);
  row_scales4(ws, ru, sa, u);
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

// Four codes E4M3(v / s) in one word, first value in the low byte.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d, float s) {
  return f32_to_e4m3(a / s) | (f32_to_e4m3(b / s) << 8) | (f32_to_e4m3(c / s) << 16) |
         (f32_to_e4m3(d / s) << 24);
}

// float32 -> OCP E5M2 code: nearest, ties to the even mantissa, saturating to
// +-57344, sign kept.  As f32_to_e4m3: subnormals (< 2^-14) are scaled by
// 2^16 and rounded to an integer mantissa (0..4; 4 is the smallest normal's
// code), normals have their float32 mantissa rounded to 2 bits and their
// exponent re-biased from 127 to 15.  Not for NaN.
__device__ __forceinline__ uint32_t f32_to_e5m2(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), kE5m2Max);
  uint32_t code;
  if (a < 6.103515625e-05f) {                 // 2^-14: subnormal range
    code = (uint32_t)__builtin_rintf(a * 65536.0f);
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0xFFFFFu + ((b >> 21) & 1u);         // RNE to 2 mantissa bits
    code = (b >> 21) - ((127u - 15u) << 2);
  }
  return code | sign;
}

__device__ __forceinline__ uint32_t e5m2_pack4(float a, float b, float c, float d, float s) {
  return f32_to_e5m2(a / s) | (f32_to_e5m2(b / s) << 8) | (f32_to_e5m2(c / s) << 16) |
         (f32_to_e5m2(d / s) << 24);
}

// Four codes of format FMT (E4M3 or E5M2) of v / s in one word.
template <int FMT>
__device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d, float s) {
  if constexpr (FMT == kFmtE5M2) return e5m2_pack4(a, b, c, d, s);
  else return e4m3_pack4(a, b, c, d, s);
}

// silu(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp) and
// exponential; for very negative z, e^-z is +inf and the result is -0.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Activation scale from an amax stored as float bits: amax / max of the
// format (448 for E4M3), 1 if zero.
__device__ __forceinline__ float scale_from_amax_bits(uint32_t amax_bits,
                                                      float fmax = kFp8Max) {
  float amax = __uint_as_float(amax_bits);
  return amax > 0.0f ? amax / fmax : 1.0f;
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

// Whole-wave reductions with DPP row operations: each step moves data between
// lanes inside the register file (a few cycles, no LDS round trip).  Steps:
// swap neighbours, swap pairs, mirror halves of 8, mirror rows of 16 (every
// lane then holds its row's result), then broadcast lane 15 of a row into the
// next row and lane 31 into rows 2 and 3; lane 63 ends with the full result,
// which is read back as a wave-uniform value.  Every lane of the wave must be
// active.
namespace dpp {
constexpr int kSwap1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kSwap2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kHalfMirror = 0x141;  // row_half_mirror
constexpr int kMirror = 0x140;      // row_mirror
constexpr int kBcast15 = 0x142;     // row_bcast:15 (rows 1 and 3 written)
constexpr int kBcast31 = 0x143;     // row_bcast:31 (rows 2 and 3 written)

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t move(uint32_t v) {
  // lanes outside the written rows keep their own value
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}
}  // namespace dpp

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_dpp(uint32_t v, Op op) {
  v = op(v, dpp::move<dpp::kSwap1, 0xF>(v));
  v = op(v, dpp::move<dpp::kSwap2, 0xF>(v));
  v = op(v, dpp::move<dpp::kHalfMirror, 0xF>(v));
  v = op(v, dpp::move<dpp::kMirror, 0xF>(v));
  v = op(v, dpp::move<dpp::kBcast15, 0xA>(v));
  v = op(v, dpp::move<dpp::kBcast31, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// row of 16 (lanes without a source add 0), then the row totals carried into
// the following rows.  Every lane of the wave must be active.
__device__ __forceinline__ int wave_inclusive_sum_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, dpp::kBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, dpp::kBcast31, 0xC, 0xF, false);
  return v;
}

// max of non-negative or any floats (IEEE fmaxf), sum of floats (the order of
// the additions is fixed by the steps above)
__device__ __forceinline__ float wave_max_dpp(float v) {
  return __uint_as_float(wave_reduce_dpp(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  return __uint_as_float(wave_reduce_dpp(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
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

// The maximum over all slots of an amax block, in every lane of the wave
// (every lane active).
__device__ __forceinline__ float amax_slots_reduce(const uint32_t* block) {
  const int lane = threadIdx.x & (kWave - 1);
  return wave_max_dpp(__uint_as_float(block[lane * kAmaxStride]));
}

}  // namespace moe
