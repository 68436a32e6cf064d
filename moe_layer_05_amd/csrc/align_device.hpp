// a2 (device side): align -- stable counting sort of the token-expert pairs by expert, each
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
//
// (At prefill sizes the fused forward lays out two layouts at once, split by
// the experts' pair counts, with the multi-workgroup kernels of align.hip.)
#pragma once

#include "device_common.hpp"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;

struct AlignOut {
  int32_t* sorted_ids;
  int32_t* block_expert;
  int32_t* num_post_pad;
  int BM;
};

// Block-wide exclusive scans of two ints per thread (1024 threads) sharing
// one pair of barriers; returns the exclusive prefixes and the totals (every
// thread).  `wsum` holds 2 * kAlignWaves ints.
__device__ __forceinline__ int2 block_exclusive_scan2(int v0, int v1, int* wsum, int2* total) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int i0 = wave_inclusive_sum_dpp(v0);
  const int i1 = wave_inclusive_sum_dpp(v1);
  __syncthreads();
  if (lane == kWave - 1) {
    wsum[wave] = i0;
    wsum[kAlignWaves + wave] = i1;
  }
  __syncthreads();
  int2 before = make_int2(0, 0), all = make_int2(0, 0);
#pragma unroll
  for (int w = 0; w < kAlignWaves; ++w) {
    const int a = wsum[w], b = wsum[kAlignWaves + w];
    if (w < wave) {
      before.x += a;
      before.y += b;
    }
    all.x += a;
    all.y += b;
  }
  *total = all;
  return make_int2(before.x + i0 - v0, before.y + i1 - v1);
}

// The whole align step by one workgroup of kAlignThreads threads; `smem`
// holds align_lds_words(E) ints.  `ids` may have been written earlier in the
// same kernel by this workgroup (a workgroup barrier must separate them).
__device__ __forceinline__ void align_block(const int32_t* ids, int P, int E, AlignOut out,
                                            int32_t* __restrict__ rank, int* smem) {
  int* cnt = smem;                                   // [E] running counts
  int* seg = smem + E;                               // [E] segment starts
  int* wsum = smem + 2 * E;                          // [2][16] scan scratch
  uint8_t* wc = reinterpret_cast<uint8_t*>(smem + 2 * E + 2 * kAlignWaves);  // [16][E]

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int nbits = (E > 1) ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;

  for (int e = tid; e < E; e += kAlignThreads) cnt[e] = 0;

  int e0 = 0, r0 = 0;                                // this thread's pair of the first chunk
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
      if (base == 0) {
        e0 = e;
        r0 = r;
      } else {
        rank[i] = r;
      }
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
  const int c_e = (tid < E) ? cnt[tid] : 0;
  const int pad = (c_e + out.BM - 1) / out.BM * out.BM;
  int2 tot;
  const int start = block_exclusive_scan2(pad, 0, wsum, &tot).x;
  if (tid < E) seg[tid] = start;
  if (tid == 0) out.num_post_pad[0] = tot.x;
  if (tid < E && pad > 0) {
    for (int b = 0; b < pad / out.BM; ++b) out.block_expert[start / out.BM + b] = tid;
    for (int q = start + c_e; q < start + pad; ++q) out.sorted_ids[q] = P;
  }
  __syncthreads();

  for (int i = tid; i < P; i += kAlignThreads) {
    const int e = i < kAlignThreads ? e0 : ids[i];
    const int r = i < kAlignThreads ? r0 : rank[i];
    out.sorted_ids[seg[e] + r] = i;
  }
}

// The same step by one wave for at most 64 pairs (the front launch of small
// batches), with no barrier: lane i holds pair i; its peers (the lanes with
// the same expert) come from the same ballot multisplit, so its rank among
// them is a popcount, and the first lane of each expert knows the expert's
// count.  The segment starts are an exclusive scan of the padded counts over
// the expert ids, through `lds` (E ints): lane l scans experts
// [l * ceil(E/64), ...) and a wave prefix joins the lanes.  The padding is
// written first, over every position, then the pairs over theirs (the two
// store passes ordered by a wait).
__device__ __forceinline__ void align_wave(const int32_t* ids, int P, int E, AlignOut out,
                                           int* lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int nbits = (E > 1) ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
  const bool valid = lane < P;
  const int e = valid ? ids[lane] : 0;
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(valid && bit);
    peers &= bit ? m : ~m;
  }
  const int rank = __popcll(peers & lt_mask);
  const bool first = valid && rank == 0;
  const int cnt = __popcll(peers);
  const int nblk = first ? (cnt + out.BM - 1) / out.BM : 0;   // blocks of expert e

  // blocks per expert id in LDS, then their exclusive prefix over the ids
  const int cpl = (E + kWave - 1) / kWave;
  for (int i = 0; i < cpl; ++i) {
    const int x = lane * cpl + i;
    if (x < E) lds[x] = 0;
  }
  if (first) lds[e] = nblk;
  int mine = 0;
  for (int i = 0; i < cpl; ++i) {
    const int x = lane * cpl + i;
    if (x < E) mine += lds[x];
  }
  const int incl = wave_inclusive_sum_dpp(mine);
  const int total = __builtin_amdgcn_readlane(incl, kWave - 1) * out.BM;
  int run = incl - mine;
  for (int i = 0; i < cpl; ++i) {
    const int x = lane * cpl + i;
    if (x < E) {
      const int c = lds[x];
      lds[x] = run;
      run += c;
    }
  }
  const int seg = lds[e] * out.BM;                 // valid lanes: their expert's start
  if (lane == 0) out.num_post_pad[0] = total;
  if (first)
    for (int b = 0; b < nblk; ++b) out.block_expert[seg / out.BM + b] = e;
  for (int q = lane; q < total; q += kWave) out.sorted_ids[q] = P;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the padding stores before the pairs'
  if (valid) out.sorted_ids[seg + rank] = lane;
}

// LDS of align_block: counts, segment starts, scan scratch (ints) and the
// per-wave counts (bytes).
constexpr size_t align_lds_words(int E) {
  return (size_t)(2 * E + 2 * kAlignWaves) + ((size_t)kAlignWaves * E + 3) / 4;
}

}  // namespace moe
