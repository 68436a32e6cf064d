// Device side of a1 (top-K routing of one token by one wavefront), shared by
// the router kernel and the fused front kernel of small batches.
//
// The router picks, per token, the few experts it activates (toolboxkart.tech
// page, "Why MoE inference needs specialized kernels"; kongchang.com page, "Why
// MoE Inference Is So Sensitive to Kernel Engineering").  The order is: larger
// logit first, equal logits -> lower expert id.  Each lane holds up to
// ceil(E/64) logits in registers; each of the K rounds picks the largest
// remaining logit and, among equal ones, the lowest id, with exact float32
// comparisons.  The winner's lane retires that logit.
#pragma once

#include "device_common.hpp"

namespace moe {

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
// wave must be active.  Each round takes the wave-wide maximum logit (a
// 32-bit max over the lanes' own best), then the lowest expert id holding
// it: one ballot when a single lane holds it, a 32-bit minimum of the ids
// otherwise (ties: logits equal as floats, -0 already folded into +0) -- the
// same choice as a maximum of the 64-bit key (logit, -id).
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
    // the lane's best: the largest of its available logits, the lowest id
    // (smallest j) among equal ones; a lane with none offers -inf and no id
    float lv = -__builtin_inff();
    uint32_t le = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      if ((avail & (1u << j)) && (le == 0xFFFFFFFFu || v[j] > lv)) {
        lv = v[j];
        le = (uint32_t)(j * kWave + lane);
      }
    }
    const float top = wave_max_dpp(lv);
    const uint64_t cand = __ballot(le != 0xFFFFFFFFu && lv == top);
    uint32_t win;
    if (__popcll(cand) == 1) {
      win = (uint32_t)__builtin_amdgcn_readlane((int)le, __builtin_ctzll(cand));
    } else {
      const uint32_t mine = ((cand >> lane) & 1) ? le : 0xFFFFFFFFu;
      win = wave_reduce_dpp(mine, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
    }
    if ((int)(win & (kWave - 1)) == lane) avail &= ~(1u << (win / kWave));
    if (k == lane) {
      my_id = (int)win;
      my_val = top;
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
