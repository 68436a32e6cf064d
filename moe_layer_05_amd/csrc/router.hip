// a1: top-K router kernel.  One wavefront per token; the per-token selection
// is route_token (route_device.hpp).  For per-tensor FP8 the same launch also
// reduces the amax of x (a0's first half): kAmaxSlots more workgroups, each
// storing the maximum of its share into its own slot of x's amax block, so
// every slot is written by every call and none needs clearing first.
#include "internal.hpp"
#include "route_device.hpp"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;
constexpr int kXBatch = 8;                  // 16-byte loads in flight per thread

template <int VPL>   // logits per lane: ceil(E / 64)
__global__ __launch_bounds__(kRouterThreads) void router_kernel(
    const float* __restrict__ logits, int64_t T, int E, int K, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ wts,
    uint32_t* __restrict__ zero_amax, int n_amax, const uint4* __restrict__ x, int64_t n8,
    uint32_t* __restrict__ amax_x, int route_blocks) {
  if ((int)blockIdx.x >= route_blocks) {
    // amax of x: workgroup j of kAmaxSlots takes every kAmaxSlots-th stretch
    const int j = blockIdx.x - route_blocks;
    const int64_t stride = (int64_t)kAmaxSlots * kRouterThreads;
    float m = 0.0f;
    for (int64_t base = (int64_t)j * kRouterThreads + threadIdx.x; base < n8;
         base += stride * kXBatch) {
      uint4 q[kXBatch];                     // all loads of a batch before any use
#pragma unroll
      for (int i = 0; i < kXBatch; ++i) {
        const int64_t k = base + (int64_t)i * stride;
        q[i] = k < n8 ? x[k] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kXBatch; ++i) {
        m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(q[i].x)), fabsf(bf16_hi(q[i].x))),
                           fmaxf(fabsf(bf16_lo(q[i].y)), fabsf(bf16_hi(q[i].y)))));
        m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(q[i].z)), fabsf(bf16_hi(q[i].z))),
                           fmaxf(fabsf(bf16_lo(q[i].w)), fabsf(bf16_hi(q[i].w)))));
      }
    }
    __shared__ float wmax[kRouterThreads / kWave];
    m = wave_max_dpp(m);
    if ((threadIdx.x & (kWave - 1)) == 0) wmax[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float b = wmax[0];
#pragma unroll
      for (int w = 1; w < kRouterThreads / kWave; ++w) b = fmaxf(b, wmax[w]);
      amax_x[j * kAmaxStride] = __float_as_uint(b);
    }
    return;
  }
  // clears the amax slots of this call's other quantisations (n_amax blocks)
  if (blockIdx.x == 0 && (int)threadIdx.x < n_amax * kAmaxSlots)
    zero_amax[amax_zero_index(threadIdx.x)] = 0u;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (t >= T) return;
  route_token<VPL>(logits + t * (int64_t)E, E, K, renorm, ids + t * K, wts + t * K);
}

}  // namespace

hipError_t prepare_router_kernels() {
  const void* fns[] = {reinterpret_cast<const void*>(&router_kernel<1>),
                       reinterpret_cast<const void*>(&router_kernel<2>),
                       reinterpret_cast<const void*>(&router_kernel<4>),
                       reinterpret_cast<const void*>(&router_kernel<8>),
                       reinterpret_cast<const void*>(&router_kernel<16>)};
  for (const void* f : fns) {
    const hipError_t e = prepare_kernel(f, 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_router(const float* logits, int64_t T, int E, int K, int renorm,
                         int32_t* ids, float* wts, uint32_t* zero_amax,
                         int n_amax, hipStream_t stream, const void* x, int64_t n,
                         uint32_t* amax_x) {
  const int waves_per_block = kRouterThreads / kWave;
  const int64_t blocks = (T + waves_per_block - 1) / waves_per_block;
  const int route_blocks = (int)(blocks > 0 ? blocks : 1);
  const bool with_amax = x != nullptr && amax_x != nullptr && n > 0;
  if (with_amax && n % 8 != 0) return hipErrorInvalidValue;
  const uint4* x8 = with_amax ? static_cast<const uint4*>(x) : nullptr;
  const int64_t n8 = with_amax ? n / 8 : 0;
  dim3 grid((unsigned)(route_blocks + (with_amax ? kAmaxSlots : 0))), block(kRouterThreads);
  const int vpl = (E + kWave - 1) / kWave;
#define MOE_ROUTER_LAUNCH(N)                                                          \
  router_kernel<N><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, ids, wts, zero_amax, \
                                               n_amax, x8, n8, amax_x, route_blocks)
  if (vpl <= 1) MOE_ROUTER_LAUNCH(1);
  else if (vpl <= 2) MOE_ROUTER_LAUNCH(2);
  else if (vpl <= 4) MOE_ROUTER_LAUNCH(4);
  else if (vpl <= 8) MOE_ROUTER_LAUNCH(8);
  else MOE_ROUTER_LAUNCH(16);
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
