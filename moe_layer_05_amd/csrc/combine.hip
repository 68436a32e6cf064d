// a6: routing-weighted combine of the expert outputs.
//
// Combining the chosen experts' outputs is part of the layer's work around the
// matrix products (toolboxkart.tech page, "Why MoE inference needs specialized
// kernels"); the down projection's epilogue already multiplied each pair's
// output by its routing weight and scales, so this sums, for each token, its K
// rows over the S parts of the down product's reduction in a fixed order
// (k = 0..K-1, then part 0..S-1: deterministic, no atomics) and rounds to
// bfloat16 (nearest even).  8 outputs per thread: K*S x 32-byte loads, one
// 16-byte store.
#include "device_common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ dw, int splits,
                                                      int64_t T, int K, int H,
                                                      uint4* __restrict__ out) {
  const int h8 = H / 8;
  const int64_t n8 = T * (int64_t)h8;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n8;
       j += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = j / h8;
    const int hc = (int)(j - t * h8) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* src = dw + (t * K) * (int64_t)H + hc;
    const int64_t part = T * K * (int64_t)H;
    for (int k = 0; k < K; ++k) {
      for (int sp = 0; sp < splits; ++sp) {
        const float* r = src + (int64_t)k * H + sp * part;
        const float4 p = *reinterpret_cast<const float4*>(r);
        const float4 q = *reinterpret_cast<const float4*>(r + 4);
        s[0] += p.x; s[1] += p.y; s[2] += p.z; s[3] += p.w;
        s[4] += q.x; s[5] += q.y; s[6] += q.z; s[7] += q.w;
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

hipError_t launch_combine(const float* dw, int splits, int64_t T, int K, int H, void* out,
                          int num_cus, hipStream_t stream) {
  const int64_t n8 = T * (int64_t)(H / 8);
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > (int64_t)num_cus * 8) blocks = (int64_t)num_cus * 8;
  combine_kernel<<<(unsigned)(blocks > 0 ? blocks : 1), 256, 0, stream>>>(
      dw, splits, T, K, H, static_cast<uint4*>(out));
  return hipGetLastError();
}

}  // namespace moe
