// a2: align kernel -- one workgroup runs align_block (align_device.hpp).
#include "align_device.hpp"
#include "internal.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int P, int E, AlignOut small, AlignOut big, int thr,
    int32_t* __restrict__ rank) {
  extern __shared__ int smem[];
  align_block(ids, P, E, small, big, thr, rank, smem);
}

}  // namespace

size_t align_lds_bytes(int E) { return align_lds_words(E) * sizeof(int); }

hipError_t launch_align(const int32_t* ids, int P, int E, int BM, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_post_pad, int32_t* rank,
                        hipStream_t stream) {
  AlignOut small{sorted_ids, block_expert, num_post_pad, BM};
  AlignOut big{nullptr, nullptr, nullptr, 256};
  align_kernel<<<1, kAlignThreads, align_lds_bytes(E), stream>>>(ids, P, E, small, big,
                                                                 0x7FFFFFFF, rank);
  return hipGetLastError();
}

hipError_t launch_align_split(const int32_t* ids, int P, int E, int BM_small,
                              int32_t* sorted_small, int32_t* bexp_small, int32_t* npp_small,
                              int BM_big, int32_t* sorted_big, int32_t* bexp_big,
                              int32_t* npp_big, int thr, int32_t* rank, hipStream_t stream) {
  AlignOut small{sorted_small, bexp_small, npp_small, BM_small};
  AlignOut big{sorted_big, bexp_big, npp_big, BM_big};
  align_kernel<<<1, kAlignThreads, align_lds_bytes(E), stream>>>(ids, P, E, small, big, thr,
                                                                 rank);
  return hipGetLastError();
}

}  // namespace moe
