// a3-a6 for thin token blocks: grouped expert GEMMs with the expert weight rows
// on the MFMA row side (the Swap-AB idea), and fused epilogues.
//
// Thin decode batches leave a matrix unit's row side mostly empty if tokens
// take it; transposing the product, C^T = W X^T, puts the large expert
// dimension there instead and costs nothing mathematically (toolboxkart.tech
// page, section 1 "Swap-AB makes better use of the WGMMA tile"; kongchang.com
// page, "Swap-AB: Making WGMMA Run at Full Utilization"; aib.vote page, second
// paragraph: top-k=8 joins the selected experts' intermediate dimensions into
// one large dimension).  The fused epilogues apply the dequantisation scales,
// SiLU-and-mul, the routing weight and the aggregation in the same pass as the
// product (aib.vote page, third paragraph).
//
// On gfx950 the row side of a 16x16 MFMA is 16 weight rows; tokens take the 16
// columns.  A block of the aligned layout holds the BM (<= 64) tokens of one
// expert, so each expert's weights stream from HBM once per call when BM >= its
// token count.  Both operands are K-contiguous rows (W[row][k], X[token][k]):
// lane l holds row (l % 16) and a 64-byte run of k chosen by (l / 16).  The
// MFMA pairs A and B elements by the same (lane group, byte) position, so any
// fixed assignment of k to those positions gives the full dot product; this
// lets every lane load 4 x 16 contiguous bytes per row per 256-byte chunk
// with no shuffles.  Weights go HBM -> VGPR directly (they are read once), one
// chunk ahead of the MFMAs.
//
// Work item = (block b, tile n).  Gate/up: a wave owns 16 intermediate columns
// c0..c0+15, i.e. gate rows c0.. and up rows I+c0.., so SiLU(g)*u is local to
// the lane; a workgroup (4 waves) covers 64 columns.  Down: a wave owns RA*16
// rows of H; a workgroup covers 64*RA rows.  The grid is persistent and sized
// from the capacity bound; each workgroup reads the device-side pair count and
// leaves when no item is left, so the host never waits for the routing.
#include "device_common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

constexpr int kChunk = 256;          // bytes of each row per pipeline step
constexpr int kLaneBytes = 64;       // bytes of each row per lane group per step

template <bool FP8>
struct Tile {
  // 16x16 accumulate of one 256-byte chunk: A = 16 weight rows, B = 16 tokens.
  static __device__ __forceinline__ v4f mma(const uint4 (&a)[4], const uint4 (&b)[4], v4f acc) {
    if constexpr (FP8) {
      v8i a0 = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
      v8i b0 = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w,
                (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
      v8i a1 = {(int)a[2].x, (int)a[2].y, (int)a[2].z, (int)a[2].w,
                (int)a[3].x, (int)a[3].y, (int)a[3].z, (int)a[3].w};
      v8i b1 = {(int)b[2].x, (int)b[2].y, (int)b[2].z, (int)b[2].w,
                (int)b[3].x, (int)b[3].y, (int)b[3].z, (int)b[3].w};
      // format 0 = E4M3 for both operands; scales 2^(127-127) = 1
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, b0, acc, 0, 0, 0, 127, 0, 127);
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, b1, acc, 0, 0, 0, 127, 0, 127);
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

__device__ __forceinline__ void load_run(uint4 (&d)[4], const uint8_t* p, int64_t off,
                                         int64_t row_bytes, bool tail, bool ok) {
  if (!ok) {
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = make_uint4(0, 0, 0, 0);
    return;
  }
  if (!tail) {
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = *reinterpret_cast<const uint4*>(p + off + 16 * j);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      d[j] = (off + 16 * j < row_bytes) ? *reinterpret_cast<const uint4*>(p + off + 16 * j)
                                        : make_uint4(0, 0, 0, 0);
  }
}

template <int MODE, bool FP8, int NSUB, int RA>
__global__ __launch_bounds__(256, 2) void moe_gemm_swapab_kernel(GemmParams p) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int g4 = lane >> 4;        // lane group: which 64-byte run of the chunk
  const int r16 = lane & 15;       // row (A) / token slot (B) inside the tile
  const int nblocks = p.num_post_pad[0] / p.BM;
  const int nitems = nblocks * p.tiles;
  const int64_t row_bytes = p.row_bytes;
  const int nfull = (int)(row_bytes / kChunk);
  const int nchunks = nfull + ((row_bytes % kChunk) ? 1 : 0);

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int b = item / p.tiles;
    const int n = item - b * p.tiles;
    const int e = p.block_expert[b];

    // valid tokens in this block (sentinels sit at the end of a block)
    const int32_t sid = (lane < p.BM) ? p.sorted_ids[(int64_t)b * p.BM + lane] : p.P;
    const int count = __popcll(__ballot(sid < p.P));
    const int nsub = (count + 15) >> 4;

    // weight rows of this wave
    const uint8_t* wexp = p.W + (int64_t)e * p.w_expert_bytes;
    const uint8_t* a_ptr[RA];
    bool a_ok[RA];
    int row0[RA];
#pragma unroll
    for (int ra = 0; ra < RA; ++ra) {
      if constexpr (MODE == kGateUp) {
        const int c0 = n * 64 + wave * 16;           // intermediate column
        row0[ra] = c0;
        a_ok[ra] = c0 < p.I;
        const int row = (ra == 0 ? c0 : p.I + c0) + r16;
        a_ptr[ra] = wexp + (int64_t)row * row_bytes + g4 * kLaneBytes;
      } else {
        const int r0 = n * (64 * RA) + (wave * RA + ra) * 16;
        row0[ra] = r0;
        a_ok[ra] = r0 < p.H;
        a_ptr[ra] = wexp + (int64_t)(r0 + r16) * row_bytes + g4 * kLaneBytes;
      }
    }
    const bool wave_on = a_ok[0];
    if (!wave_on) continue;                          // no barriers below

    // activation rows of this wave's token slots
    const uint8_t* b_ptr[NSUB];
    bool b_ok[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const int32_t pair = (s < nsub) ? p.sorted_ids[(int64_t)b * p.BM + s * 16 + r16] : p.P;
      b_ok[s] = pair < p.P;
      const int64_t brow = b_ok[s] ? (int64_t)(pair / p.b_row_div) : 0;
      b_ptr[s] = p.B + brow * row_bytes + g4 * kLaneBytes;
    }

    v4f acc[RA][NSUB];
#pragma unroll
    for (int ra = 0; ra < RA; ++ra)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[ra][s] = v4f{0.f, 0.f, 0.f, 0.f};

    uint4 a0[RA][4], a1[RA][4], b0[NSUB][4], b1[NSUB][4];

    auto load = [&](uint4 (&ad)[RA][4], uint4 (&bd)[NSUB][4], int c) {
      const bool tail = c >= nfull;
      const int64_t off = (int64_t)c * kChunk;
#pragma unroll
      for (int ra = 0; ra < RA; ++ra) load_run(ad[ra], a_ptr[ra], off, row_bytes - g4 * kLaneBytes, tail, a_ok[ra]);
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
        if (s < nsub) load_run(bd[s], b_ptr[s], off, row_bytes - g4 * kLaneBytes, tail, b_ok[s]);
    };
    auto compute = [&](uint4 (&ad)[RA][4], uint4 (&bd)[NSUB][4]) {
#pragma unroll
      for (int ra = 0; ra < RA; ++ra) {
        if (!a_ok[ra]) continue;
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
          if (s < nsub) acc[ra][s] = Tile<FP8>::mma(ad[ra], bd[s], acc[ra][s]);
      }
    };

    load(a0, b0, 0);
    for (int c = 0;;) {
      const bool more1 = c + 1 < nchunks;
      if (more1) load(a1, b1, c + 1);
      compute(a0, b0);
      if (!more1) break;
      ++c;
      const bool more2 = c + 1 < nchunks;
      if (more2) load(a0, b0, c + 1);
      compute(a1, b1);
      if (!more2) break;
      ++c;
    }

    // ------------------------------------------------------------ epilogue
    float scale = 1.0f;
    if constexpr (FP8) scale = scale_from_amax_bits(*p.act_amax) * p.w_scale[e];

    if constexpr (MODE == kGateUp) {
      float local_max = 0.0f;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if (s >= nsub) continue;
        const int32_t pair = p.sorted_ids[(int64_t)b * p.BM + s * 16 + r16];
        if (pair >= p.P) continue;
        const int col = row0[0] + 4 * g4;
        float av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float g = acc[0][s][v] * scale;
          const float u = acc[1][s][v] * scale;
          av[v] = g / (1.0f + __expf(-g)) * u;
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
      if constexpr (FP8) {
        local_max = wave_max(local_max);
        if (lane == 0 && local_max > 0.0f) atomic_max_nonneg(p.a_amax, local_max);
      }
    } else {
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if (s >= nsub) continue;
        const int32_t pair = p.sorted_ids[(int64_t)b * p.BM + s * 16 + r16];
        if (pair >= p.P) continue;
        const float sc = scale * p.topk_w[pair];
#pragma unroll
        for (int ra = 0; ra < RA; ++ra) {
          if (!a_ok[ra]) continue;
          float* dst = p.dw + (int64_t)pair * p.H + row0[ra] + 4 * g4;
          *reinterpret_cast<float4*>(dst) =
              make_float4(acc[ra][s][0] * sc, acc[ra][s][1] * sc, acc[ra][s][2] * sc,
                          acc[ra][s][3] * sc);
        }
      }
    }
  }
}

template <int MODE, bool FP8, int RA>
hipError_t launch_nsub(const GemmParams& p, int nsub_max, dim3 grid, hipStream_t stream) {
  dim3 block(256);
  switch (nsub_max) {
    case 1: moe_gemm_swapab_kernel<MODE, FP8, 1, RA><<<grid, block, 0, stream>>>(p); break;
    case 2: moe_gemm_swapab_kernel<MODE, FP8, 2, RA><<<grid, block, 0, stream>>>(p); break;
    case 4: moe_gemm_swapab_kernel<MODE, FP8, 4, RA><<<grid, block, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int swapab_down_rows_per_item() { return 64 * kDownRA; }

hipError_t launch_gemm_swapab(int mode, bool fp8, const GemmParams& p, int max_items,
                              int num_cus, hipStream_t stream) {
  const int nsub_max = p.BM / 16;
  int g = num_cus * 2;
  if (g > max_items) g = max_items;
  if (g < 1) g = 1;
  dim3 grid(g);
  if (mode == kGateUp) {
    return fp8 ? launch_nsub<kGateUp, true, 2>(p, nsub_max, grid, stream)
               : launch_nsub<kGateUp, false, 2>(p, nsub_max, grid, stream);
  }
  return fp8 ? launch_nsub<kDown, true, kDownRA>(p, nsub_max, grid, stream)
             : launch_nsub<kDown, false, kDownRA>(p, nsub_max, grid, stream);
}

}  // namespace moe
