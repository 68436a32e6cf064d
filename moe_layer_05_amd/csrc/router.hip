// a1: top-K router.  One wavefront per token.
//
// The router picks, per token, the few experts it activates (toolboxkart.tech
// page, "Why MoE inference needs specialized kernels"; kongchang.com page, "Why
// MoE Inference Is So Sensitive to Kernel Engineering").  The order is: larger
// logit first, equal logits -> lower expert id.  Each lane holds up to
// ceil(E/64) logits in registers; each of the K rounds takes a wave-wide
// maximum of a 64-bit key (order-preserving float bits << 32 | ~expert id), so
// the decision is exact on the float32 logits and ties resolve to the lower
// id.  The winner's lane retires that logit.
#include "device_common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

// Order-preserving map of float bits to uint32 (finite floats; -0 folded to +0
// by the caller).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

template <int VPL>   // logits per lane: ceil(E / 64)
__global__ __launch_bounds__(256) void router_kernel(
    const float* __restrict__ logits, int64_t T, int E, int K, int renorm,
    int32_t* __restrict__ ids, float* __restrict__ wts,
    uint32_t* __restrict__ zero_amax, int n_amax) {
  // clears the amax slots of this call's quantisations (n_amax blocks)
  if (blockIdx.x == 0 && (int)threadIdx.x < n_amax * kAmaxSlots)
    zero_amax[amax_zero_index(threadIdx.x)] = 0u;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (t >= T) return;
  const float* row = logits + t * (int64_t)E;

  float v[VPL];
  uint32_t avail = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    int e = j * kWave + lane;
    v[j] = (e < E) ? row[e] + 0.0f : 0.0f;     // + 0.0f folds -0 into +0
    if (e < E) avail |= 1u << j;
  }

  int my_id = 0;
  float my_val = 0.0f;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;                          // every finite key is > 0
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      if (avail & (1u << j)) {
        uint32_t e = (uint32_t)(j * kWave + lane);
        uint64_t key = ((uint64_t)order_key(v[j]) << 32) | (uint32_t)(~e);
        best = key > best ? key : best;
      }
    }
    best = wave_max_u64(best);
    uint32_t win = ~(uint32_t)best;
    if ((int)(win & (kWave - 1)) == lane) avail &= ~(1u << (win / kWave));
    if (k == lane) {
      my_id = (int)win;
      my_val = key_value((uint32_t)(best >> 32));
    }
  }

  const float top = __shfl(my_val, 0);
  float ex = (lane < K) ? expf(my_val - top) : 0.0f;
  float denom;
  if (renorm) {
    denom = wave_sum(ex);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (j * kWave + lane < E) s += expf(v[j] - top);
    denom = wave_sum(s);
  }
  if (lane < K) {
    ids[t * K + lane] = my_id;
    wts[t * K + lane] = ex / denom;
  }
}

}  // namespace

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
