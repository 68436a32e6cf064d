// a3-a6 for large token blocks (prefill): a grouped, LDS-pipelined MFMA GEMM
// over blocks of 256 tokens of one expert.
//
// An expert that receives hundreds of tokens turns its products into dense
// matrix work; grouped GEMMs over the experts' token blocks are what the layer
// is made of (kongchang.com page, "Swap-AB": grouped and batched GEMMs are
// abundant in MoE).  The expert weight rows still take the MFMA row side, as
// in the decode kernel (toolboxkart.tech page, section 1; aib.vote page,
// second paragraph), so each lane's four accumulators are four consecutive
// output features and the epilogue stores them as one vector.  The epilogues
// apply the dequantisation scales and SiLU-and-mul in the same pass (aib.vote
// page, third paragraph); the routing weight is applied by the combine.
//
// Workgroup tile: 256 weight rows x 256 tokens, 8 waves in a 2 x 4 grid, each
// wave 128 x 64 = 8 x 4 MFMA 16x16 tiles (fp8: one 16x16x128 per tile and
// k-step; bf16: two 16x16x32).  Two waves per SIMD: while one waits for its
// LDS reads, the other issues MFMAs.  The k-step is 128 bytes of the reduction
// dimension; weight and token tiles of a k-step (32 KB each) move HBM/L2 ->
// LDS with direct-to-LDS loads, two stages deep (128 KB), one barrier per
// k-step.  LDS rows are 128 bytes with the 16-byte granule index XOR-ed by
// (row & 7); a lane of lane group g4 takes granules g4 and g4 + 4 of its row
// (any fixed assignment of k positions works, as A and B share it), which the
// hardware reads without bank conflicts (granule pairs 2 g4, 2 g4 + 1 would
// conflict on half the cycles).
//
// Gate/up: the 256 weight rows are 128 gate rows and the 128 up rows of the
// same intermediate columns, so SiLU(g) * u is formed in registers.  Down:
// 256 consecutive rows of W2.  The token rows are gathered through the sorted
// pair ids; padding slots read a valid row and their columns are not stored,
// and a wave whose 64 token slots are all padding skips its MFMAs.
#include <algorithm>

#include "device_common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kTM = 256;            // weight rows per workgroup tile
constexpr int kTN = 256;            // tokens per workgroup tile (= block size)
constexpr int kBK = 128;            // bytes of the reduction dimension per k-step
constexpr int kStageBytes = (kTM + kTN) * kBK;   // 64 KB
constexpr int kTileLds = 2 * kStageBytes;        // 128 KB

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Four 16-byte LDS reads and the wait for them.
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

template <int FMT>
__device__ __forceinline__ v4f tile_mma(const uint4 (&a)[2], const uint4 (&b)[2], v4f acc) {
  if constexpr (FMT != kFmtBF16) {
    constexpr int kF = FMT == kFmtE5M2 ? 1 : 0;    // operand format: 0 E4M3, 1 E5M2
    v8i av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
              (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
    v8i bv = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w,
              (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
    // scale operands 0: the unscaled instruction (v_mfma_f32_16x16x128_f8f6f4),
    // bit for bit equal to unit scales and issued about 3% faster
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, kF, kF, 0, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[0]),
                                                  __builtin_bit_cast(v8bf, b[0]), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[1]),
                                                   __builtin_bit_cast(v8bf, b[1]), acc, 0, 0, 0);
  }
}

// Eight 16-byte LDS reads and the wait for them.
__device__ __forceinline__ void lds_read8(uint4 (&d)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %9\n"
      "ds_read_b128 %2, %10\n"
      "ds_read_b128 %3, %11\n"
      "ds_read_b128 %4, %12\n"
      "ds_read_b128 %5, %13\n"
      "ds_read_b128 %6, %14\n"
      "ds_read_b128 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]),
        "=&v"(d[6]), "=&v"(d[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

constexpr int kWaves = 8;
constexpr int kLoadsPerWave = 32 / kWaves;       // 1 KB loads per tile (A or B) per wave

template <int MODE, int FMT>
__global__ __launch_bounds__(512, 1) void moe_gemm_tile_kernel(GemmParams p) {
  constexpr bool FP8 = FMT != kFmtBF16;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // Persistent: one workgroup per compute unit takes tiles until none is
  // left.  The routed blocks are cut into 8 contiguous ranges, one per XCD
  // (workgroups are handed to the XCDs in turn, blockIdx & 7), and each XCD's
  // tiles form a list walked in panels of 8 blocks x 4 column tiles, so the
  // 32 tiles running at once on an XCD read 8 token slices and 4 weight
  // slices per k-step from its L2.  A workgroup takes the next tile of its
  // XCD's list from an atomic counter, and once that list is empty the next
  // tile of another XCD's list: the XCDs' lists cost different times (an
  // expert with one block reads mostly padding token rows, which hit L2;
  // measured per workgroup, static turns ended 846..1220 us into a 1220 us
  // gate/up launch), so idle compute units take over the tail.  Every tile is
  // taken exactly once and computed the same way by whichever workgroup, so
  // the results do not depend on the schedule.
  constexpr int kPB = 8, kPN = 4;
  const int nb = p.num_post_pad[0] / kTN;
  const int xcd = blockIdx.x & 7;
  auto range = [&](int x, int& b0, int& b1) {
    b0 = (x * nb) >> 3;
    b1 = ((x + 1) * nb) >> 3;
  };
  // tile l of XCD x's list -> (block b, column tile n)
  auto tile_of = [&](int x, int l, int& b, int& n) {
    int b0, b1;
    range(x, b0, b1);
    const int gw = p.groups;
    const int bp = l / (kPB * gw);
    const int bpw = min(kPB, (b1 - b0) - bp * kPB);
    const int rem = l - bp * kPB * gw;
    const int np = rem / (bpw * kPN);
    const int npw = min(kPN, gw - np * kPN);
    const int inner = rem - np * bpw * kPN;
    b = b0 + bp * kPB + inner / npw;
    n = np * kPN + inner % npw;
  };
  // the next tile as x << 24 | l, or -1 when every list is empty (one thread)
  auto grab = [&]() -> int {
    for (int d = 0; d < 8; ++d) {
      const int x = (xcd + d) & 7;
      int b0, b1;
      range(x, b0, b1);
      const int cnt = (b1 - b0) * p.groups;
      if (cnt == 0) continue;
      const int l = (int)atomicAdd(p.tile_queue + x, 1u);
      if (l < cnt) return (x << 24) | l;
    }
    return -1;
  };
  __shared__ int s_next;

  const int row_bytes = (int)p.row_bytes;
  const int nfull = row_bytes / kBK;
  const int nk = (row_bytes + kBK - 1) / kBK;

  // ---- loads into LDS.  Load instruction i (1 KB) of a tile covers tile
  // rows 8i .. 8i + 7: lane -> row 8i + (lane >> 3), LDS position lane & 7,
  // which holds the row's 16-byte granule (lane & 7) ^ (lane >> 3).  Wave w
  // issues loads i = 4w .. 4w + 3 of the weight tile and of the token tile.
  const int lrow = lane >> 3;
  const uint32_t gq = (uint32_t)(((lane & 7) ^ lrow) * 16);
  uint8_t* a_lds = smem + wave * kLoadsPerWave * 1024;                 // + stage * kStageBytes
  uint8_t* b_lds = smem + kTM * kBK + wave * kLoadsPerWave * 1024;

  // A tile's identity (kept for its epilogue) and the load addresses of the
  // tile being loaded (replaced by the next tile's during the last k-step).
  struct Tile {
    int n, e;
    const int32_t* blk;
    int nsub;                                      // 16-token tiles of this wave holding a pair
    int rot;                                       // first k-step of the sweep
  };
  const uint8_t* a_src[kLoadsPerWave];
  const uint8_t* b_src[kLoadsPerWave];
  auto setup = [&](int code, Tile& s) {
    int b;
    tile_of(code >> 24, code & 0xFFFFFF, b, s.n);
    // The tiles of XCD x's panels sweep the full k-steps from step
    // x * nfull / 8 on, wrapping round (a partial last step stays last): the
    // eight XCDs then read different column ranges at a time (measured on
    // MI355X, FP8 Zipf T = 4096: gate/up stage 1457 -> 1443 us).
    s.rot = (int)(((int64_t)(code >> 24) * nfull) / 8);
    s.e = __builtin_amdgcn_readfirstlane(p.block_expert[b]);
    s.blk = p.sorted_ids + (int64_t)b * kTN;
    {
      // the pairs of a block are a prefix of it, the rest is padding
      const uint64_t live = __ballot(s.blk[64 * (wave >> 1) + lane] < p.P);
      s.nsub = __builtin_amdgcn_readfirstlane((__popcll(live) + 15) >> 4);
    }
    const uint8_t* wexp = p.W + (int64_t)s.e * p.w_expert_bytes;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int r = (kLoadsPerWave * wave + i) * 8 + lrow;   // tile row 0..255
      int wr;
      if constexpr (MODE == kGateUp) {
        const int col = s.n * 128 + (r & 127);
        wr = (col < p.I) ? ((r < 128) ? col : p.I + col) : 0;
      } else {
        const int h = s.n * kTM + r;
        wr = (h < p.H) ? h : 0;
      }
      a_src[i] = wexp + (int64_t)wr * row_bytes;
      const int32_t pair = s.blk[r];
      const int64_t brow = pair < p.P ? (int64_t)(pair / p.b_row_div) : 0;
      b_src[i] = p.B + brow * row_bytes;
    }
  };
  auto issue = [&](int stage, int k, int rot) {
    const bool tail = k >= nfull;
    if (!tail) {
      k += rot;
      if (k >= nfull) k -= nfull;
    }
    const uint32_t off = (uint32_t)k * kBK;
    const uint32_t o = (!tail || off + gq < (uint32_t)row_bytes) ? off + gq : 0u;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
      // weights through the caches: the other token blocks of the panel
      // read the same weight slice
      __builtin_amdgcn_global_load_lds((const void*)(a_src[i] + o),
                                       (lds_void*)(a_lds + stage * kStageBytes + i * 1024), 16,
                                       0, 0);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(b_src[i] + o),
                                       (lds_void*)(b_lds + stage * kStageBytes + i * 1024), 16,
                                       0, 0);
  };

  // ---- MFMA-layout reads: lane holds row l16 of a 16-row tile and the 32
  // bytes of granules g4 and g4 + 4 of the k-step.
  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t sw = (uint32_t)(l16 & 7);
  const uint32_t r0 = lds_addr(smem) + l16 * kBK + ((g4 ^ sw) * 16);
  const uint32_t r1 = lds_addr(smem) + l16 * kBK + (((g4 + 4) ^ sw) * 16);
  // first row of weight tile ai / token tile bj of this wave inside a stage
  auto a_row = [&](int ai) -> int {
    if constexpr (MODE == kGateUp) return (ai < 4 ? 0 : 128) + 64 * wm + 16 * (ai & 3);
    else return 128 * wm + 16 * ai;
  };
  const int b_row0 = kTM + 64 * wn;

  v4f acc[8][4];
  auto compute = [&](int stage, bool tail, uint32_t off) {
    const uint32_t sb = (uint32_t)stage * kStageBytes;
    uint4 bt[8];                                   // token tile bj: bt[2 bj], bt[2 bj + 1]
    uint32_t ba[8];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      const uint32_t o = sb + (uint32_t)(b_row0 + 16 * bj) * kBK;
      ba[2 * bj] = r0 + o;
      ba[2 * bj + 1] = r1 + o;
    }
    lds_read8(bt, ba);
    if (tail) {
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
        if (off + g4 * 16 >= (uint32_t)row_bytes) bt[2 * bj] = make_uint4(0, 0, 0, 0);
        if (off + (g4 + 4) * 16 >= (uint32_t)row_bytes) bt[2 * bj + 1] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int ai = 0; ai < 8; ai += 2) {
      uint4 cur[4];
      const uint32_t o0 = sb + (uint32_t)a_row(ai) * kBK;
      const uint32_t o1 = sb + (uint32_t)a_row(ai + 1) * kBK;
      lds_read4(cur, r0 + o0, r1 + o0, r0 + o1, r1 + o1);
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
        const uint4 bb[2] = {bt[2 * bj], bt[2 * bj + 1]};
        const uint4 a0[2] = {cur[0], cur[1]};
        const uint4 a1[2] = {cur[2], cur[3]};
        acc[ai][bj] = tile_mma<FMT>(a0, bb, acc[ai][bj]);
        acc[ai + 1][bj] = tile_mma<FMT>(a1, bb, acc[ai + 1][bj]);
      }
    }
  };

  // ------------------------------------------------------------ epilogue
  // Lane (g4, l16) holds weight rows 4*g4 + v of each 16-row sub-tile for
  // token column l16; per-row scales as in the decode form.
  const bool rows = FP8 && p.row_scales;
  auto epilogue = [&](const Tile& s) {
    float scale = 1.0f;
    const int64_t wrow0 = (int64_t)s.e * (MODE == kGateUp ? 2 * p.I : p.H);
    if constexpr (FP8)
      if (!rows) scale = scale_from_amax_bits(*p.act_amax, fp8_max<FMT>()) * p.w_scale[s.e];
    if constexpr (MODE == kGateUp) {
      float local_max = 0.0f;
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
        const int32_t pair = s.blk[64 * wn + 16 * bj + l16];
        if (pair >= p.P) continue;
        const float sa = rows ? p.act_scale[pair / p.b_row_div] : 1.0f;
#pragma unroll
        for (int ai = 0; ai < 4; ++ai) {
          const int col = s.n * 128 + 64 * wm + 16 * ai + 4 * g4;
          if (col >= p.I) continue;
          float sg[4] = {scale, scale, scale, scale}, su[4] = {scale, scale, scale, scale};
          if (rows) row_scales4(p.w_scale + wrow0, col, p.I + col, sa, sg, su);
          float av[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float gt = acc[ai][bj][v] * sg[v];
            const float up = acc[ai + 4][bj][v] * su[v];
            av[v] = silu_fast(gt) * up;
            local_max = fmaxf(local_max, fabsf(av[v]));
          }
          if constexpr (FP8) {
            float* dst = static_cast<float*>(p.a_out) + (int64_t)pair * p.I + col;
            *reinterpret_cast<float4*>(dst) = make_float4(av[0], av[1], av[2], av[3]);
          } else {
            uint16_t* dst = static_cast<uint16_t*>(p.a_out) + (int64_t)pair * p.I + col;
            uint2 pk;
            pk.x = f32_to_bf16_bits(av[0]) | (f32_to_bf16_bits(av[1]) << 16);
            pk.y = f32_to_bf16_bits(av[2]) | (f32_to_bf16_bits(av[3]) << 16);
            *reinterpret_cast<uint2*>(dst) = pk;
          }
        }
      }
      if constexpr (FP8) {
        if (!rows) {
          local_max = wave_max(local_max);
          if (lane == 0 && local_max > 0.0f)
            amax_slot_max(p.a_amax, (uint32_t)(blockIdx.x * kWaves + wave), local_max);
        }
      }
    } else {
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) {
        const int32_t pair = s.blk[64 * wn + 16 * bj + l16];
        if (pair >= p.P) continue;
        const float sa = rows ? p.act_scale[pair] : 1.0f;
#pragma unroll
        for (int ai = 0; ai < 8; ++ai) {
          const int h = s.n * kTM + 128 * wm + 16 * ai + 4 * g4;
          if (h >= p.H) continue;
          float sc[4] = {scale, scale, scale, scale};
          if (rows) row_scales4(p.w_scale + wrow0, h, sa, sc);
          store_part4(p.dw, p.dw_bf16, (int64_t)pair * p.H + h, acc[ai][bj][0] * sc[0],
                      acc[ai][bj][1] * sc[1], acc[ai][bj][2] * sc[2], acc[ai][bj][3] * sc[3]);
        }
      }
    }
  };

  // ---- the walk: during a tile's last k-step the first stage of the next
  // tile is loaded, so a tile's start and its epilogue overlap with loads.
  // The next tile is taken at a tile's first k-step (thread 0, into s_next)
  // and read at its last, after the barriers between.
  if (tid == 0) s_next = grab();
  __syncthreads();
  const int first = s_next;
  if (first < 0) return;                           // uniform: every thread read s_next
  Tile cur, nxt;
  setup(first, cur);
  issue(0, 0, cur.rot);
  int stage = 0;
  for (;;) {
    bool has_next = false;
#pragma unroll
    for (int ai = 0; ai < 8; ++ai)
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) acc[ai][bj] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < nk; ++k) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads of this stage
      __syncthreads();                                   // all waves: stage in, other stage read
      if (k == 0) {
        // every thread read s_next (the current tile) before this barrier
        if (tid == 0) s_next = grab();
        if (nk == 1) __syncthreads();
      }
      if (k + 1 < nk) {
        issue(stage ^ 1, k + 1, cur.rot);
      } else {
        const int next = s_next;
        has_next = next >= 0;
        if (has_next) {
          setup(next, nxt);
          issue(stage ^ 1, 0, nxt.rot);
        }
      }
      if (__builtin_amdgcn_readfirstlane(cur.nsub) > 0) compute(stage, k >= nfull, (uint32_t)k * kBK);
      stage ^= 1;
    }
    epilogue(cur);
    if (!has_next) break;
    cur = nxt;
  }
}

// Run once per device by the entry points before any launch
// (prepare_tile_kernels): the 128 KB LDS limit.
template <int MODE, int FMT>
hipError_t ready_tile() {
  return prepare_kernel(reinterpret_cast<const void*>(&moe_gemm_tile_kernel<MODE, FMT>), kTileLds);
}

template <int MODE, int FMT>
hipError_t launch_tile(const GemmParams& p, dim3 grid, hipStream_t stream) {
  moe_gemm_tile_kernel<MODE, FMT><<<grid, dim3(64 * kWaves), kTileLds, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t prepare_tile_kernels() {
  hipError_t e = ready_tile<kGateUp, kFmtBF16>();
  if (e == hipSuccess) e = ready_tile<kGateUp, kFmtE4M3>();
  if (e == hipSuccess) e = ready_tile<kGateUp, kFmtE5M2>();
  if (e == hipSuccess) e = ready_tile<kDown, kFmtBF16>();
  if (e == hipSuccess) e = ready_tile<kDown, kFmtE4M3>();
  if (e == hipSuccess) e = ready_tile<kDown, kFmtE5M2>();
  return e;
}

int tile_block_m() { return kTN; }

int tile_groups(int mode, int rows) {
  return mode == kGateUp ? (rows + 127) / 128 : (rows + kTM - 1) / kTM;
}

hipError_t launch_gemm_tile(int mode, int fmt, const GemmParams& p, int64_t nblk_cap,
                            int num_cus, hipStream_t stream) {
  if (p.BM != kTN || p.tile_queue == nullptr) return hipErrorInvalidValue;
  const int64_t tiles = nblk_cap * p.groups;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7FFFFFFF || p.row_bytes > (1 << 24)) return hipErrorInvalidValue;
  // one workgroup per compute unit (a multiple of 8: one share per XCD)
  int64_t wgs = std::min<int64_t>(std::max(num_cus / 8, 1), (tiles + 7) / 8) * 8;
  dim3 grid((unsigned)wgs);
  if (mode == kGateUp) {
    if (fmt == kFmtE4M3) return launch_tile<kGateUp, kFmtE4M3>(p, grid, stream);
    if (fmt == kFmtE5M2) return launch_tile<kGateUp, kFmtE5M2>(p, grid, stream);
    return launch_tile<kGateUp, kFmtBF16>(p, grid, stream);
  }
  if (fmt == kFmtE4M3) return launch_tile<kDown, kFmtE4M3>(p, grid, stream);
  if (fmt == kFmtE5M2) return launch_tile<kDown, kFmtE5M2>(p, grid, stream);
  return launch_tile<kDown, kFmtBF16>(p, grid, stream);
}

}  // namespace moe
