// a1: top-K router kernel.  One wavefront per token; the per-token selection
// is route_token (route_device.hpp).
#include "internal.hpp"
#include "route_device.hpp"

namespace moe {
namespace {

template <int VPL>   // logits per lane: ceil(E / 64)
__global__ __launch_bounds__(256) void router_kernel(
    const float* __restrict__ logits, int64_t T, int E, int K, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ wts,
    uint32_t* __restrict__ zero_amax, int n_amax) {
  // clears the amax slots of this call's quantisations (n_amax blocks)
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
                         int n_amax, hipStream_t stream) {
  const int waves_per_block = 4;
  const int64_t blocks = (T + waves_per_block - 1) / waves_per_block;
  dim3 grid((unsigned)(blocks > 0 ? blocks : 1)), block(waves_per_block * kWave);
  const int vpl = (E + kWave - 1) / kWave;
#define MOE_ROUTER_CASE(N)                                                     \
  case N:                                                                      \
    router_kernel<N><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, ids, \
                                                 wts, zero_amax, n_amax);     \
    break;
  switch (vpl) {
    MOE_ROUTER_CASE(1)
    MOE_ROUTER_CASE(2)
    MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(16)
    default:
      if (vpl == 3) { router_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, ids, wts, zero_amax, n_amax); break; }
      if (vpl <= 8) { router_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, ids, wts, zero_amax, n_amax); break; }
      router_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, K, renorm, ids, wts, zero_amax, n_amax);
  }
#undef MOE_ROUTER_CASE
  return hipGetLastError();
}

}  // namespace moe
