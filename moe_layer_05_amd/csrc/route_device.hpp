// Device side of a1 (top-K routing of one token by one wavefront), shared by
// the router kernel and the fused front kernel of small batches.
//
// The router picks, per token, the few experts it activates (toolboxkart.tech
// page, "Why MoE inference needs specialized kernels"; kongchang.com page, "Why
// MoE Inference Is So Sensitive to Kernel Engineering").  The order is: larger
// logit first, equal logits -> lower expert id.  Each lane holds up to
// ceil(E/64) logits in registers; each of the K rounds takes a wave-wide
// maximum of a 64-bit key (order-preserving float bits << 32 | ~expert id), so
// the decision is exact on the float32 logits and ties resolve to the lower
// id.  The winner's lane retires that logit.
#pragma once

#include "device_common.hpp"

namespace moe {

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


// The logits of one token, lane l holding logits l, l + 64, ... (-0 folded
// into +0; positions past E are 0 and never chosen).
template <int VPL>
__device__ __forceinline__ void load_logits(const float* __restrict__ row, int E, float (&v)[VPL]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int e = j * kWave + lane;
    v[j] = (e < E) ? row[e] + 0.0f : 0.0f;
  }
}

// Routes one token from its loaded logits; lanes 0..K-1 write the chosen ids
// and weights (softmax renormalised over the K, or over all E).  The whole
// wave must be active.
template <int VPL>   // logits per lane: ceil(E / 64)
__device__ __forceinline__ void route_values(const float (&v)[VPL], int E, int K, int renorm,
                                             int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t avail = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j)
    if (j * kWave + lane < E) avail |= 1u << j;

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
    best = wave_max_u64_dpp(best);
    uint32_t win = ~(uint32_t)best;
    if ((int)(win & (kWave - 1)) == lane) avail &= ~(1u << (win / kWave));
    if (k == lane) {
      my_id = (int)win;
      my_val = key_value((uint32_t)(best >> 32));
    }
  }

  const float top = __uint_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
  float ex = (lane < K) ? expf(my_val - top) : 0.0f;
  float denom;
  if (renorm) {
    denom = wave_sum_dpp(ex);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (j * kWave + lane < E) s += expf(v[j] - top);
    denom = wave_sum_dpp(s);
  }
  if (lane < K) {
    ids[lane] = my_id;
    wts[lane] = ex / denom;
  }
}

// load_logits then route_values.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int K,
                                            int renorm, int32_t* __restrict__ ids,
                                            float* __restrict__ wts) {
  float v[VPL];
  load_logits<VPL>(row, E, v);
  route_values<VPL>(v, E, K, renorm, ids, wts);
}

}  // namespace moe
