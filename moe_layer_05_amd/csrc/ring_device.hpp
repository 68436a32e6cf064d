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

// All NT tiles of one ring stage, tile t at byte offset t * kTileBytes from the
// four MFMA-layout read addresses: up to three tiles (twelve reads) per asm
// block, each block ending in its own wait (early-clobber outputs, as above).
template <int T, int NT>
__device__ __forceinline__ void lds_read_tiles(uint4 (&d)[NT][4], uint32_t a0, uint32_t a1,
                                               uint32_t a2, uint32_t a3) {
  if constexpr (T < NT) {
    constexpr int rem = NT - T;
    constexpr int n = (rem >= 3 && rem != 4) ? 3 : (rem >= 2 ? 2 : 1);
    static_assert((T + n) * kTileBytes <= 65536, "LDS read offset range");
    if constexpr (n == 3) {
      asm volatile(
          "ds_read_b128 %0, %12 offset:%16\n"
          "ds_read_b128 %1, %13 offset:%16\n"
          "ds_read_b128 %2, %14 offset:%16\n"
          "ds_read_b128 %3, %15 offset:%16\n"
          "ds_read_b128 %4, %12 offset:%17\n"
          "ds_read_b128 %5, %13 offset:%17\n"
          "ds_read_b128 %6, %14 offset:%17\n"
          "ds_read_b128 %7, %15 offset:%17\n"
          "ds_read_b128 %8, %12 offset:%18\n"
          "ds_read_b128 %9, %13 offset:%18\n"
          "ds_read_b128 %10, %14 offset:%18\n"
          "ds_read_b128 %11, %15 offset:%18\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(d[T][0]), "=&v"(d[T][1]), "=&v"(d[T][2]), "=&v"(d[T][3]),
            "=&v"(d[T + 1][0]), "=&v"(d[T + 1][1]), "=&v"(d[T + 1][2]), "=&v"(d[T + 1][3]),
            "=&v"(d[T + 2][0]), "=&v"(d[T + 2][1]), "=&v"(d[T + 2][2]), "=&v"(d[T + 2][3])
          : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "n"(T * kTileBytes),
            "n"((T + 1) * kTileBytes), "n"((T + 2) * kTileBytes)
          : "memory");
    } else if constexpr (n == 2) {
      asm volatile(
          "ds_read_b128 %0, %8 offset:%12\n"
          "ds_read_b128 %1, %9 offset:%12\n"
          "ds_read_b128 %2, %10 offset:%12\n"
          "ds_read_b128 %3, %11 offset:%12\n"
          "ds_read_b128 %4, %8 offset:%13\n"
          "ds_read_b128 %5, %9 offset:%13\n"
          "ds_read_b128 %6, %10 offset:%13\n"
          "ds_read_b128 %7, %11 offset:%13\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(d[T][0]), "=&v"(d[T][1]), "=&v"(d[T][2]), "=&v"(d[T][3]),
            "=&v"(d[T + 1][0]), "=&v"(d[T + 1][1]), "=&v"(d[T + 1][2]), "=&v"(d[T + 1][3])
          : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "n"(T * kTileBytes), "n"((T + 1) * kTileBytes)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %4 offset:%8\n"
          "ds_read_b128 %1, %5 offset:%8\n"
          "ds_read_b128 %2, %6 offset:%8\n"
          "ds_read_b128 %3, %7 offset:%8\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(d[T][0]), "=&v"(d[T][1]), "=&v"(d[T][2]), "=&v"(d[T][3])
          : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "n"(T * kTileBytes)
          : "memory");
    }
    lds_read_tiles<T + n, NT>(d, a0, a1, a2, a3);
  }
}

// An empty asm that takes a tile's registers as read and written after every
// memory operation before it: the products that use the tile cannot be
// scheduled above loads issued before this point.
__device__ __forceinline__ void after_issue(uint4 (&x)[4]) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  v4u t0 = __builtin_bit_cast(v4u, x[0]), t1 = __builtin_bit_cast(v4u, x[1]);
  v4u t2 = __builtin_bit_cast(v4u, x[2]), t3 = __builtin_bit_cast(v4u, x[3]);
  asm volatile("" : "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t3)::"memory");
  x[0] = __builtin_bit_cast(uint4, t0);
  x[1] = __builtin_bit_cast(uint4, t1);
  x[2] = __builtin_bit_cast(uint4, t2);
  x[3] = __builtin_bit_cast(uint4, t3);
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
