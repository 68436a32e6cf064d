// a0 and the intermediate quantisation of a4: FP8 (E4M3 or E5M2) per tensor,
// or per row.
//
// FP8 E4M3 (4 exponent, 3 mantissa bits) with one scale per tensor:
// kongchang.com page, FP8 explainer under "Triton Backend Routing"; aib.vote
// page, third paragraph ("tensor-quantized" FP8 MoE).
//
// Two grid-wide steps: an amax reduction (wave max, one atomicMax of the
// float bits per wave into one of 64 slots) and the quantisation, whose waves
// each reduce the slots, form s = amax / 448 and write E4M3(v / s) with an
// IEEE division, so the codes are exactly those of a float32 reference; its
// first thread also stores the final amax for later kernels.  Both kernels
// stream with 16-byte loads and are bandwidth-bound.
//
// The per-row form (one scale per token row of x, per pair row of the
// intermediate) carries the kongchang.com page's concern in "Triton Backend
// Routing: A Practical Path to FP8 Quantization" -- value distributions
// differ, so one uniform scale loses precision -- from experts down to rows:
// a row's own scale keeps its small values out of the E4M3 subnormal range.
#include "device_common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

// amax over n bfloat16 values (n % 8 == 0), 8 per thread per step.
__global__ __launch_bounds__(256) void amax_bf16_kernel(const uint4* __restrict__ x, int64_t n8,
                                                        uint32_t* __restrict__ amax) {
  float m = 0.0f;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n8;
       j += (int64_t)gridDim.x * blockDim.x) {
    uint4 q = x[j];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(q.x)), fabsf(bf16_hi(q.x))),
                       fmaxf(fabsf(bf16_lo(q.y)), fabsf(bf16_hi(q.y)))));
    m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(q.z)), fabsf(bf16_hi(q.z))),
                       fmaxf(fabsf(bf16_lo(q.w)), fabsf(bf16_hi(q.w)))));
  }
  m = wave_max_dpp(m);
  if ((threadIdx.x & (kWave - 1)) == 0 && m > 0.0f)
    amax_slot_max(amax, blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave, m);
}

// codes = FP8(x / s), 8 bfloat16 in -> 8 codes out per thread per step.
template <int FMT>
__global__ __launch_bounds__(256) void quant_bf16_kernel(const uint4* __restrict__ x, int64_t n8,
                                                         uint32_t* __restrict__ amax,
                                                         uint2* __restrict__ codes,
                                                         float* __restrict__ scale_out) {
  const float m = amax_slots_reduce(amax);
  const float s = scale_from_amax_bits(__float_as_uint(m), fp8_max<FMT>());
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    amax[kAmaxFinal] = __float_as_uint(m);
    if (scale_out) *scale_out = s;
  }
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n8;
       j += (int64_t)gridDim.x * blockDim.x) {
    uint4 q = x[j];
    uint2 o;
    o.x = fp8_pack4<FMT>(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y), s);
    o.y = fp8_pack4<FMT>(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w), s);
    codes[j] = o;
  }
}

// codes = FP8(a / s) for float32 a (n % 8 == 0), the amax came from the
// producer of a.
template <int FMT>
__global__ __launch_bounds__(256) void quant_f32_kernel(const float4* __restrict__ a, int64_t n8,
                                                        uint32_t* __restrict__ amax,
                                                        uint2* __restrict__ codes) {
  const float m = amax_slots_reduce(amax);
  const float s = scale_from_amax_bits(__float_as_uint(m), fp8_max<FMT>());
  if (blockIdx.x == 0 && threadIdx.x == 0) amax[kAmaxFinal] = __float_as_uint(m);
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n8;
       j += (int64_t)gridDim.x * blockDim.x) {
    float4 p = a[2 * j], q = a[2 * j + 1];
    uint2 o;
    o.x = fp8_pack4<FMT>(p.x, p.y, p.z, p.w, s);
    o.y = fp8_pack4<FMT>(q.x, q.y, q.z, q.w, s);
    codes[j] = o;
  }
}

// Per-row form: one wave per row (grid-stride over rows).  The wave reduces
// the row's amax from 16-byte loads, forms s = amax / 448 with the same
// arithmetic as the per-tensor form, and writes the codes on a second read of
// the row (from cache: a row is at most a few tens of KB).
template <bool BF16>
__device__ __forceinline__ void load8(const void* src, int64_t j, float (&v)[8]) {
  if constexpr (BF16) {
    const uint4 q = static_cast<const uint4*>(src)[j];
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  } else {
    const float4 p = static_cast<const float4*>(src)[2 * j];
    const float4 q = static_cast<const float4*>(src)[2 * j + 1];
    v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
    v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
  }
}

template <bool BF16, int FMT>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ src,
                                                         int64_t rows, int c8,
                                                         uint2* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t r = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; r < rows;
       r += nw) {
    const int64_t base = r * c8;
    float m = 0.0f;
#pragma unroll 4
    for (int j = lane; j < c8; j += kWave) {
      float v[8];
      load8<BF16>(src, base + j, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    }
    m = wave_max_dpp(m);
    const float s = scale_from_amax_bits(__float_as_uint(m), fp8_max<FMT>());
    if (lane == 0) scales[r] = s;
#pragma unroll 4
    for (int j = lane; j < c8; j += kWave) {
      float v[8];
      load8<BF16>(src, base + j, v);
      uint2 o;
      o.x = fp8_pack4<FMT>(v[0], v[1], v[2], v[3], s);
      o.y = fp8_pack4<FMT>(v[4], v[5], v[6], v[7], s);
      codes[base + j] = o;
    }
  }
}

// Clears the slots of n consecutive amax blocks.
__global__ void zero_amax_kernel(uint32_t* p, int nblocks) {
  for (int t = threadIdx.x; t < nblocks * kAmaxSlots; t += blockDim.x) p[amax_zero_index(t)] = 0u;
}

unsigned stream_grid(int64_t n8, int num_cus) {
  int64_t blocks = (n8 + 255) / 256;
  int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  return (unsigned)(blocks > 0 ? blocks : 1);
}

}  // namespace

hipError_t prepare_quant_kernels() {
  const void* fns[] = {reinterpret_cast<const void*>(&amax_bf16_kernel),
                       reinterpret_cast<const void*>(&quant_bf16_kernel<kFmtE4M3>),
                       reinterpret_cast<const void*>(&quant_bf16_kernel<kFmtE5M2>),
                       reinterpret_cast<const void*>(&quant_f32_kernel<kFmtE4M3>),
                       reinterpret_cast<const void*>(&quant_f32_kernel<kFmtE5M2>),
                       reinterpret_cast<const void*>(&zero_amax_kernel),
                       reinterpret_cast<const void*>(&quant_rows_kernel<true, kFmtE4M3>),
                       reinterpret_cast<const void*>(&quant_rows_kernel<false, kFmtE4M3>),
                       reinterpret_cast<const void*>(&quant_rows_kernel<true, kFmtE5M2>),
                       reinterpret_cast<const void*>(&quant_rows_kernel<false, kFmtE5M2>)};
  for (const void* f : fns) {
    const hipError_t e = prepare_kernel(f, 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_zero_amax(uint32_t* p, int nblocks, hipStream_t stream) {
  zero_amax_kernel<<<1, 64, 0, stream>>>(p, nblocks);
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const void* x, int64_t n, uint32_t* amax, int num_cus,
                            hipStream_t stream) {
  const int64_t n8 = n / 8;
  amax_bf16_kernel<<<stream_grid(n8, num_cus), 256, 0, stream>>>(
      static_cast<const uint4*>(x), n8, amax);
  return hipGetLastError();
}

hipError_t launch_quant_bf16(int fmt, const void* x, int64_t n, uint32_t* amax, uint8_t* codes,
                             float* scale_out, int num_cus, hipStream_t stream) {
  const int64_t n8 = n / 8;
  auto k = fmt == kFmtE5M2 ? &quant_bf16_kernel<kFmtE5M2> : &quant_bf16_kernel<kFmtE4M3>;
  k<<<stream_grid(n8, num_cus), 256, 0, stream>>>(
      static_cast<const uint4*>(x), n8, amax, reinterpret_cast<uint2*>(codes), scale_out);
  return hipGetLastError();
}

hipError_t launch_quant_f32(int fmt, const float* a, int64_t n, uint32_t* amax, uint8_t* codes,
                            int num_cus, hipStream_t stream) {
  const int64_t n8 = n / 8;
  auto k = fmt == kFmtE5M2 ? &quant_f32_kernel<kFmtE5M2> : &quant_f32_kernel<kFmtE4M3>;
  k<<<stream_grid(n8, num_cus), 256, 0, stream>>>(
      reinterpret_cast<const float4*>(a), n8, amax, reinterpret_cast<uint2*>(codes));
  return hipGetLastError();
}

hipError_t launch_quant_rows(int fmt, const void* src, bool bf16, int64_t rows, int C,
                             uint8_t* codes, float* scales, int num_cus, hipStream_t stream) {
  int64_t blocks = (rows + 3) / 4;                 // 4 waves (rows) per block
  if (blocks > (int64_t)num_cus * 8) blocks = (int64_t)num_cus * 8;
  const unsigned grid = (unsigned)(blocks > 0 ? blocks : 1);
  const bool e5 = fmt == kFmtE5M2;
  auto k = bf16 ? (e5 ? &quant_rows_kernel<true, kFmtE5M2> : &quant_rows_kernel<true, kFmtE4M3>)
                : (e5 ? &quant_rows_kernel<false, kFmtE5M2> : &quant_rows_kernel<false, kFmtE4M3>);
  k<<<grid, 256, 0, stream>>>(src, rows, C / 8, reinterpret_cast<uint2*>(codes), scales);
  return hipGetLastError();
}

}  // namespace moe
