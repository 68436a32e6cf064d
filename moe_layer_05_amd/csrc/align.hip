// a2: align kernel -- one workgroup runs align_block (align_device.hpp).
#include <algorithm>

#include "align_device.hpp"
#include "internal.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int P, int E, AlignOut out, int32_t* __restrict__ rank) {
  extern __shared__ int smem[];
  align_block(ids, P, E, out, rank, smem);
}

// Align plus a0 in one launch (small batches routed by the router kernel):
// workgroup 0 runs align_block; workgroups 1.. write the FP8 codes of x, with
// one scale per tensor (the router launch left the amax of x in the slots of
// amax_x: each workgroup folds them, workgroup 1 stores the final word) or one
// scale per token row (a wave per row, as quant_rows_kernel).  The codes are
// formed with the same arithmetic as the quantisation kernels.
struct XQuant {
  const uint4* x;            // [T][H] bfloat16, 8 per uint4
  int64_t n8;                // T * H / 8
  int h8;                    // H / 8
  uint32_t* amax_x;          // per tensor: amax block of x (slots in, final word out)
  uint2* codes;              // 8 codes per uint2
  float* row_scales;         // per row: [T] scales out, or nullptr for one scale
};

template <int FMT>
__global__ __launch_bounds__(kAlignThreads) void align_quant_kernel(
    const int32_t* __restrict__ ids, int P, int E, AlignOut out, int32_t* __restrict__ rank,
    XQuant q) {
  extern __shared__ int smem[];
  if (blockIdx.x == 0) {
    align_block(ids, P, E, out, rank, smem);
    return;
  }
  const int nq = gridDim.x - 1, b = blockIdx.x - 1;
  const int lane = threadIdx.x & (kWave - 1);
  if (q.row_scales) {
    const int64_t T = q.n8 / q.h8;
    for (int64_t r = (int64_t)b * kAlignWaves + threadIdx.x / kWave; r < T;
         r += (int64_t)nq * kAlignWaves) {
      const uint4* row = q.x + r * q.h8;
      float m = 0.0f;
      for (int j = lane; j < q.h8; j += kWave) {
        const uint4 v = row[j];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))),
                           fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)))));
        m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))),
                           fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)))));
      }
      m = wave_max_dpp(m);
      const float sc = scale_from_amax_bits(__float_as_uint(m), fp8_max<FMT>());
      if (lane == 0) q.row_scales[r] = sc;
      for (int j = lane; j < q.h8; j += kWave) {
        const uint4 v = row[j];
        uint2 o;
        o.x = fp8_pack4<FMT>(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y), sc);
        o.y = fp8_pack4<FMT>(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w), sc);
        q.codes[r * q.h8 + j] = o;
      }
    }
    return;
  }
  const float m = amax_slots_reduce(q.amax_x);
  const float sc = scale_from_amax_bits(__float_as_uint(m), fp8_max<FMT>());
  if (b == 0 && threadIdx.x == 0) q.amax_x[kAmaxFinal] = __float_as_uint(m);
  for (int64_t j = (int64_t)b * kAlignThreads + threadIdx.x; j < q.n8;
       j += (int64_t)nq * kAlignThreads) {
    const uint4 v = q.x[j];
    uint2 o;
    o.x = fp8_pack4<FMT>(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y), sc);
    o.y = fp8_pack4<FMT>(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w), sc);
    q.codes[j] = o;
  }
}

// ---- Multi-workgroup form, for many pairs.  (1) Each workgroup ranks the
// pairs of its chunk of kAlignThreads among equal experts (the same wave
// multisplit as align_block) and writes the chunk's per-expert counts;
// (2) one workgroup turns the counts into per-chunk offsets (in place) and
// lays out both padded layouts; (3) each workgroup scatters its chunk.  The
// position of a pair is a pure function of the input order, so the result
// equals the one-workgroup form exactly.

__global__ __launch_bounds__(kAlignThreads) void align_count_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ rank) {
  extern __shared__ int smem[];
  uint8_t* wc = reinterpret_cast<uint8_t*>(smem);   // [16][E] per-wave counts
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int nbits = (E > 1) ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;
  for (int j = tid; j < kAlignWaves * E; j += kAlignThreads) wc[j] = 0;
  __syncthreads();
  const int i = blockIdx.x * kAlignThreads + tid;
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
    int r = rw;
    for (int w = 0; w < wave; ++w) r += wc[w * E + e];
    rank[i] = r;                                     // rank inside the chunk
  }
  for (int ee = tid; ee < E; ee += kAlignThreads) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) c += wc[w * E + ee];
    counts[(int64_t)blockIdx.x * E + ee] = c;
  }
}

// counts [C][E] -> exclusive offsets over the chunks (in place); seg [3][E]
// receives the small and big segment starts and the per-expert totals;
// n_clear words at `clear` are zeroed (the tiled products' work counters).
__global__ __launch_bounds__(kAlignThreads) void align_scan_kernel(
    int32_t* __restrict__ counts, int C, int E, int P, AlignOut small, AlignOut big, int thr,
    int32_t* __restrict__ seg, uint32_t* __restrict__ clear, int n_clear) {
  __shared__ int wsum[2 * kAlignWaves];
  const int tid = threadIdx.x;
  if (tid < n_clear) clear[tid] = 0u;
  int c_e = 0;
  if (tid < E) {
    constexpr int kBatch = 32;                       // loads in flight per thread
    for (int c0 = 0; c0 < C; c0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        v[k] = c0 + k < C ? counts[(int64_t)(c0 + k) * E + tid] : 0;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        if (c0 + k < C) counts[(int64_t)(c0 + k) * E + tid] = c_e;
        c_e += v[k];
      }
    }
  }
  const bool is_big = c_e >= thr;
  const int pad_s = (tid < E && !is_big) ? (c_e + small.BM - 1) / small.BM * small.BM : 0;
  const int pad_b = (tid < E && is_big) ? (c_e + big.BM - 1) / big.BM * big.BM : 0;
  int2 tot;
  const int2 start = block_exclusive_scan2(pad_s, pad_b, wsum, &tot);
  if (tid < E) {
    seg[tid] = start.x;
    seg[E + tid] = start.y;
    seg[2 * E + tid] = c_e;
  }
  if (tid == 0) {
    small.num_post_pad[0] = tot.x;
    big.num_post_pad[0] = tot.y;
  }
  if (tid < E && pad_s > 0) {
    for (int b = 0; b < pad_s / small.BM; ++b) small.block_expert[start.x / small.BM + b] = tid;
    for (int q = start.x + c_e; q < start.x + pad_s; ++q) small.sorted_ids[q] = P;
  }
  if (tid < E && pad_b > 0) {
    for (int b = 0; b < pad_b / big.BM; ++b) big.block_expert[start.y / big.BM + b] = tid;
    for (int q = start.y + c_e; q < start.y + pad_b; ++q) big.sorted_ids[q] = P;
  }
}

__global__ __launch_bounds__(kAlignThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ seg, const int32_t* __restrict__ rank, AlignOut small,
    AlignOut big, int thr) {
  const int i = blockIdx.x * kAlignThreads + threadIdx.x;
  if (i >= P) return;
  const int e = ids[i];
  const int r = offs[(int64_t)blockIdx.x * E + e] + rank[i];
  if (seg[2 * E + e] >= thr) big.sorted_ids[seg[E + e] + r] = i;
  else small.sorted_ids[seg[e] + r] = i;
}

}  // namespace

hipError_t prepare_align_kernels() {
  const void* fns[] = {reinterpret_cast<const void*>(&align_kernel),
                       reinterpret_cast<const void*>(&align_quant_kernel<kFmtE4M3>),
                       reinterpret_cast<const void*>(&align_quant_kernel<kFmtE5M2>),
                       reinterpret_cast<const void*>(&align_count_kernel),
                       reinterpret_cast<const void*>(&align_scan_kernel),
                       reinterpret_cast<const void*>(&align_scatter_kernel)};
  for (const void* f : fns) {
    const hipError_t e = prepare_kernel(f, 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t align_multi_workspace_bytes(int P, int E) {
  const size_t C = ((size_t)P + kAlignThreads - 1) / kAlignThreads;
  return (C * E + 3 * (size_t)E) * sizeof(int32_t);
}

hipError_t launch_align_split_multi(const int32_t* ids, int P, int E, int BM_small,
                                    int32_t* sorted_small, int32_t* bexp_small,
                                    int32_t* npp_small, int BM_big, int32_t* sorted_big,
                                    int32_t* bexp_big, int32_t* npp_big, int thr, int32_t* rank,
                                    int32_t* scratch, uint32_t* clear, int n_clear,
                                    hipStream_t stream) {
  if (n_clear < 0 || n_clear > kAlignThreads || (n_clear > 0 && clear == nullptr))
    return hipErrorInvalidValue;
  AlignOut small{sorted_small, bexp_small, npp_small, BM_small};
  AlignOut big{sorted_big, bexp_big, npp_big, BM_big};
  const int C = (P + kAlignThreads - 1) / kAlignThreads;
  int32_t* counts = scratch;                         // [C][E]
  int32_t* seg = scratch + (size_t)C * E;            // [3][E]
  align_count_kernel<<<C, kAlignThreads, (size_t)kAlignWaves * E, stream>>>(ids, P, E, counts,
                                                                           rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  align_scan_kernel<<<1, kAlignThreads, 0, stream>>>(counts, C, E, P, small, big, thr, seg,
                                                    clear, n_clear);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  align_scatter_kernel<<<C, kAlignThreads, 0, stream>>>(ids, P, E, counts, seg, rank, small, big,
                                                       thr);
  return hipGetLastError();
}

size_t align_lds_bytes(int E) { return align_lds_words(E) * sizeof(int); }

hipError_t launch_align(const int32_t* ids, int P, int E, int BM, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_post_pad, int32_t* rank,
                        hipStream_t stream) {
  AlignOut out{sorted_ids, block_expert, num_post_pad, BM};
  align_kernel<<<1, kAlignThreads, align_lds_bytes(E), stream>>>(ids, P, E, out, rank);
  return hipGetLastError();
}

hipError_t launch_align_quant(const int32_t* ids, int P, int E, int BM, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* num_post_pad, int32_t* rank,
                              int fmt, const void* x, int64_t T, int H, uint32_t* amax_x,
                              uint8_t* codes, float* row_scales, int num_cus,
                              hipStream_t stream) {
  AlignOut out{sorted_ids, block_expert, num_post_pad, BM};
  XQuant q{static_cast<const uint4*>(x), T * (int64_t)H / 8, H / 8, amax_x,
           reinterpret_cast<uint2*>(codes), row_scales};
  int64_t nq = row_scales ? (T + kAlignWaves - 1) / kAlignWaves
                          : (q.n8 + kAlignThreads - 1) / kAlignThreads;
  nq = std::max<int64_t>(1, std::min<int64_t>(nq, num_cus));
  const dim3 grid((unsigned)(1 + nq));
  if (fmt == kFmtE5M2)
    align_quant_kernel<kFmtE5M2><<<grid, kAlignThreads, align_lds_bytes(E), stream>>>(
        ids, P, E, out, rank, q);
  else
    align_quant_kernel<kFmtE4M3><<<grid, kAlignThreads, align_lds_bytes(E), stream>>>(
        ids, P, E, out, rank, q);
  return hipGetLastError();
}

}  // namespace moe
