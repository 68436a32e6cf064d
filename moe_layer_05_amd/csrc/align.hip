// a2: align -- stable counting sort of the token-expert pairs by expert, each
// expert's run padded to a multiple of block_m with the sentinel T*K.
//
// Grouping the tokens of each expert is what lets every expert run one
// grouped matrix product over a variable number of tokens (kongchang.com page,
// "Why MoE Inference Is So Sensitive to Kernel Engineering": the number of
// tokens each expert receives is variable; "Swap-AB": grouped GEMMs).
//
// One workgroup of 1024 threads (16 waves) walks the pairs in chunks of 1024.
// Inside a chunk, each lane finds the lanes of its wave holding the same
// expert with one ballot per bit of the expert id (a wave-level multisplit),
// so its rank among equal experts of its wave is a popcount; the per-wave
// counts go to LDS (one writer per wave and expert, no atomics), and the rank
// in the whole pair list is the running count of earlier chunks plus the
// counts of earlier waves plus the in-wave rank.  Every step is a pure
// function of the input order, so the layout is deterministic and stable.
#include "device_common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int P, int E, int BM,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ num_post_pad, int32_t* __restrict__ rank) {
  extern __shared__ int smem[];
  int* cnt = smem;                                   // [E] running counts
  int* seg = smem + E;                               // [E] segment starts
  int* wsum = smem + 2 * E;                          // [16] scan scratch
  uint8_t* wc = reinterpret_cast<uint8_t*>(smem + 2 * E + kAlignWaves);  // [16][E]

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int nbits = (E > 1) ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;

  for (int e = tid; e < E; e += kAlignThreads) cnt[e] = 0;

  for (int base = 0; base < P; base += kAlignThreads) {
    for (int j = tid; j < kAlignWaves * E; j += kAlignThreads) wc[j] = 0;
    __syncthreads();
    const int i = base + tid;
    const bool valid = i < P;
    const int e = valid ? ids[i] : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    const int rw = __popcll(peers & lt_mask);
    if (valid && rw == 0) wc[wave * E + e] = (uint8_t)__popcll(peers);
    __syncthreads();
    if (valid) {
      int r = cnt[e] + rw;
      for (int w = 0; w < wave; ++w) r += wc[w * E + e];
      rank[i] = r;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kAlignThreads) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < kAlignWaves; ++w) s += wc[w * E + ee];
      cnt[ee] += s;
    }
    __syncthreads();
  }

  // Exclusive scan of the padded counts over experts (E <= 1024: one each).
  const int my_pad = (tid < E) ? (cnt[tid] + BM - 1) / BM * BM : 0;
  int incl = my_pad;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  const int start = before + incl - my_pad;
  if (tid < E) seg[tid] = start;
  if (tid == kAlignThreads - 1) num_post_pad[0] = before + incl;
  if (tid < E && my_pad > 0) {
    const int c = cnt[tid];
    for (int b = 0; b < my_pad / BM; ++b) block_expert[start / BM + b] = tid;
    for (int p = start + c; p < start + my_pad; ++p) sorted_ids[p] = P;
  }
  __syncthreads();

  for (int i = tid; i < P; i += kAlignThreads) sorted_ids[seg[ids[i]] + rank[i]] = i;
}

}  // namespace

size_t align_lds_bytes(int E) {
  return (size_t)(2 * E + kAlignWaves) * sizeof(int) + (size_t)kAlignWaves * E;
}

hipError_t launch_align(const int32_t* ids, int P, int E, int BM, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_post_pad, int32_t* rank,
                        hipStream_t stream) {
  align_kernel<<<1, kAlignThreads, align_lds_bytes(E), stream>>>(
      ids, P, E, BM, sorted_ids, block_expert, num_post_pad, rank);
  return hipGetLastError();
}

}  // namespace moe
