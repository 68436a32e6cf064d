// LDS rings fed by direct-to-LDS loads and the 16x16 MFMA step of the
// weight-streaming products (gemm_decode.hip, down_small.hip), gfx950 only.
//
// A chunk is 256 bytes of a K-contiguous row.  A 16-row tile of one chunk
// (4 KB) is loaded by four direct-to-LDS instructions: instruction i covers
// tile rows 4i + g4 (g4 = lane / 16) and lane piece r16 = lane % 16; the lane
// reads the row's 16-byte piece r16 ^ (4i + g4), so LDS row R position x holds
// piece x ^ R, and a read of piece q of row R at position q ^ R by the 16 lanes
// of a group hits 16 different bank groups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace moe {
namespace {

constexpr int kChunk = 256;           // bytes of each row per pipeline step
constexpr int kTileBytes = 16 * kChunk;   // one 16-row tile of one chunk in LDS
constexpr int kAuxNT = 2;             // cache policy bits of a non-temporal load

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Four 16-byte LDS reads and the wait for them, in one block: the compiler
// does not see these reads, so it adds no conservative wait on the weight
// loads into LDS that precede them (the kernel places those waits itself).
// The outputs are early-clobber: a read's data may land before a later read
// of the block has taken its address, so no output may share a register with
// an address.
__device__ __forceinline__ void lds_read4(uint4 (&d)[4], uint32_t a0, uint32_t a1, uint32_t a2,
                                          uint32_t a3) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %5\n"
      "ds_read_b128 %2, %6\n"
      "ds_read_b128 %3, %7\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The same for a run-time number of whole stages (0 <= stages < D) of L
// loads each: the counter takes an immediate, so this branches (uniformly)
// to the matching wait.
template <int L, int D>
__device__ __forceinline__ void wait_stages(int stages) {
  static_assert((D - 1) * L <= 63, "vmcnt range");
  switch (stages) {
    case 1: if constexpr (D > 1) wait_vmcnt<1 * L>(); break;
    case 2: if constexpr (D > 2) wait_vmcnt<2 * L>(); break;
    case 3: if constexpr (D > 3) wait_vmcnt<3 * L>(); break;
    case 4: if constexpr (D > 4) wait_vmcnt<4 * L>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

template <int FMT>
struct Tile {
  // 16x16 accumulate of one 256-byte chunk: A = 16 weight rows, B = 16 tokens.
  static __device__ __forceinline__ v4f mma(const uint4 (&a)[4], const uint4 (&b)[4], v4f acc) {
    if constexpr (FMT != kFmtBF16) {
      constexpr int kF = FMT == kFmtE5M2 ? 1 : 0;  // operand format: 0 E4M3, 1 E5M2
      v8i a0 = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
      v8i b0 = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w,
                (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
      v8i a1 = {(int)a[2].x, (int)a[2].y, (int)a[2].z, (int)a[2].w,
                (int)a[3].x, (int)a[3].y, (int)a[3].z, (int)a[3].w};
      v8i b1 = {(int)b[2].x, (int)b[2].y, (int)b[2].z, (int)b[2].w,
                (int)b[3].x, (int)b[3].y, (int)b[3].z, (int)b[3].w};
      // the same format for both operands; scale operands 0 select the
      // unscaled instruction (v_mfma_f32_16x16x128_f8f6f4), measured bit for
      // bit equal to unit scales and issued about 3% faster
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, b0, acc, kF, kF, 0, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, b1, acc, kF, kF, 0, 0, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v8bf av = __builtin_bit_cast(v8bf, a[j]);
        v8bf bv = __builtin_bit_cast(v8bf, b[j]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
      }
    }
    return acc;
  }
};

}  // namespace
}  // namespace moe
