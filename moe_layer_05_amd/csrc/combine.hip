// a6: routing-weighted combine of the expert outputs.
//
// Combining the chosen experts' outputs is part of the layer's work around the
// matrix products (toolboxkart.tech page, "Why MoE inference needs specialized
// kernels"); the down projection's epilogue already applied the dequantisation
// scales, so this sums, for each token, its K rows times their routing
// weights over the S parts of the down product's reduction in a fixed order
// (k = 0..K-1, then part 0..S-1: deterministic, no atomics) and rounds to
// bfloat16 (nearest even).  8 outputs per thread: K*S row loads (up to 8 rows
// in flight per thread), one 16-byte store.  At prefill the partial rows are
// bfloat16, which halves their write and read traffic.
#include "device_common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kBatch = 8;     // rows loaded per thread before they are added

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ dw,
                                                      const float* __restrict__ w, int splits,
                                                      int64_t T, int K, int H,
                                                      uint4* __restrict__ out) {
  const int h8 = H / 8;
  const int64_t n8 = T * (int64_t)h8;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n8;
       j += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = j / h8;
    const int hc = (int)(j - t * h8) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int64_t src = (t * K) * (int64_t)H + hc;           // element index of row k = 0
    const int64_t part = T * K * (int64_t)H;
    const int rows = K * splits;                     // row q: k = q / splits, part q % splits
    for (int q0 = 0; q0 < rows; q0 += kBatch) {
      float4 p[kBatch][2];                           // all loads of a batch before the adds
      float wk[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int q = q0 + b;
        if (q < rows) {
          const int k = q / splits;
          const int64_t r = src + (int64_t)k * H + (q % splits) * part;
          if constexpr (BF16) {
            const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(dw) + r);
            p[b][0] = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
            p[b][1] = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
          } else {
            const float* f = static_cast<const float*>(dw) + r;
            p[b][0] = *reinterpret_cast<const float4*>(f);
            p[b][1] = *reinterpret_cast<const float4*>(f + 4);
          }
          wk[b] = w[t * K + k];
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (q0 + b < rows) {
          const float c = wk[b];
          s[0] += c * p[b][0].x; s[1] += c * p[b][0].y; s[2] += c * p[b][0].z;
          s[3] += c * p[b][0].w; s[4] += c * p[b][1].x; s[5] += c * p[b][1].y;
          s[6] += c * p[b][1].z; s[7] += c * p[b][1].w;
        }
      }
    }
    uint4 o;
    o.x = f32_to_bf16_bits(s[0]) | (f32_to_bf16_bits(s[1]) << 16);
    o.y = f32_to_bf16_bits(s[2]) | (f32_to_bf16_bits(s[3]) << 16);
    o.z = f32_to_bf16_bits(s[4]) | (f32_to_bf16_bits(s[5]) << 16);
    o.w = f32_to_bf16_bits(s[6]) | (f32_to_bf16_bits(s[7]) << 16);
    out[j] = o;
  }
}

}  // namespace

hipError_t prepare_combine_kernels() {
  const hipError_t e = prepare_kernel(reinterpret_cast<const void*>(&combine_kernel<false>), 0);
  if (e != hipSuccess) return e;
  return prepare_kernel(reinterpret_cast<const void*>(&combine_kernel<true>), 0);
}

hipError_t launch_combine(const void* dw, bool dw_bf16, const float* w, int splits, int64_t T,
                          int K, int H, void* out, int num_cus, hipStream_t stream) {
  const int64_t n8 = T * (int64_t)(H / 8);
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > (int64_t)num_cus * 8) blocks = (int64_t)num_cus * 8;
  const unsigned grid = (unsigned)(blocks > 0 ? blocks : 1);
  if (dw_bf16)
    combine_kernel<true><<<grid, 256, 0, stream>>>(dw, w, splits, T, K, H,
                                                   static_cast<uint4*>(out));
  else
    combine_kernel<false><<<grid, 256, 0, stream>>>(dw, w, splits, T, K, H,
                                                    static_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
