// a3-a6 for thin token blocks: grouped expert GEMMs with the expert weight rows
// on the MFMA row side (the Swap-AB idea), fused epilogues, and a weight
// stream shaped for HBM3E.
//
// Thin decode batches leave a matrix unit's row side mostly empty if tokens
// take it; transposing the product, C^T = W X^T, puts the large expert
// dimension there instead and costs nothing mathematically (toolboxkart.tech
// page, section 1 "Swap-AB makes better use of the WGMMA tile"; kongchang.com
// page, "Swap-AB: Making WGMMA Run at Full Utilization"; aib.vote page, second
// paragraph: top-k=8 joins the selected experts' intermediate dimensions into
// one large dimension).  The epilogues apply the dequantisation scales and
// SiLU-and-mul in the same pass as the product (aib.vote page, third
// paragraph); the combine applies the routing weights.
//
// On gfx950 the row side of a 16x16 MFMA is 16 weight rows; tokens take the 16
// columns.  Both operands are K-contiguous rows (W[row][k], X[token][k]):
// lane l holds row (l % 16) and a 64-byte run of k chosen by (l / 16) in each
// 256-byte chunk.  The MFMA pairs A and B elements by the same (lane group,
// byte) position, so any fixed assignment of k to those positions gives the
// full dot product; every lane therefore loads 4 x 16 contiguous bytes per row
// per chunk with no shuffles.
//
// Decode is a weight stream: every byte of an active expert is read once and
// used by at most a few tokens.  The kernel is shaped for that:
//  - both operands move HBM/L2 -> LDS with direct-to-LDS loads (no VGPR
//    staging); weight loads are non-temporal (the data is not reused, and
//    streaming it past the last-level cache raises the sustained read rate of
//    HBM3E), activation rows (x, x codes, a, a codes: small, shared by all row
//    groups of an expert) go through the caches;
//  - each wave owns a ring of D chunk stages in LDS and keeps D - 1 of them in
//    flight; it waits on its own vector-memory counter, so no workgroup
//    barrier is needed (one wave per workgroup); a stage is read into
//    registers before its refill is issued, so the refill overlaps the
//    stage's products;
//  - gate/up waves start their sweep of the rows at different chunks, so the
//    waves running at one time spread their reads over the rows' columns;
//  - the unit of work is one wave: (block b, row group g, k-split s), where a
//    row group is RA 16-row MFMA tiles; the grid is not persistent: one wave
//    per unit of the capacity bound, so the hardware dispatcher balances the
//    waves over the compute units, and units past the device-side block count
//    leave at once (the host never reads the routing);
//  - the down product may split its reduction dimension I into S parts; each
//    part writes its own partial rows and the combine adds the parts
//    in a fixed order, so results stay deterministic.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"
#include "ring_device.hpp"

namespace moe {
namespace {

// Rows of fewer chunks than this are short: their waves are short, and more
// of them in flight wins (fewer weight tiles per wave, shallower rings).
constexpr int kShortRow = 24;

// Ring depth for RA weight tiles and NSUB token tiles per wave: each wave
// holds D * (RA + NSUB) * 4 KB of LDS, and 160 KB per compute unit.  A stage
// is refilled as soon as it has been read, so nearly all D stages are loading
// at any time, and shallow rings (more waves per compute unit) often measured
// faster, though not for every shape (MI355X, per call):
//  - one token tile, two weight tiles: short rows D = 2 (FP8 64 tokens down
//    525 -> 512 us, TP8 slice 16 tokens gate/up 33 -> 31 us); long rows
//    D = 3 for gate/up (bf16 8 tokens 284 -> 277 us) and 4 for the down
//    product (bf16 32 tokens: D = 3 146 -> 154 us);
//  - one token tile, four weight tiles: D = 2 for gate/up (FP8 1 token
//    40.4 -> 39.2 us), 3 for the down product;
//  - two token tiles, four weight tiles: D = 2 for gate/up (bf16 64 tokens
//    298 -> 294 us), 3 for the down product (D = 2: 151 -> 159 us).
// Within the 6-bit vector-memory counter.
constexpr int ring_depth(int mode, int ra, int nsub, bool short_rows) {
  return ra >= 8      ? 2
         : nsub == 1  ? (ra == 2 ? (short_rows ? 2 : (mode == kGateUp ? 3 : 4))
                                 : (mode == kGateUp ? 2 : 3))
         : nsub == 2  ? (ra == 4 && mode == kGateUp ? 2 : 3)
                      : 2;
}

// A grid that one round of waves with this deeper ring holds takes it: with
// few waves the chip has room, and each wave's own loads in flight set the
// pace (TP8 slice, 1 token, gate/up 96 waves: depth 4 11 us, depth 2 13 us).
constexpr int deep_depth(int ra, int nsub) {
  return ra >= 8 ? 2 : nsub == 1 ? (ra == 2 ? 4 : 3) : nsub == 2 ? 3 : 2;
}

template <int MODE, int FMT, int NSUB, int RA, int D>
__global__ __launch_bounds__(64) void moe_gemm_decode_kernel(GemmParams p) {
  constexpr bool FP8 = FMT != kFmtBF16;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // loads per chunk, all into LDS: 4 per 16-row weight tile, 4 per 16-token tile
  constexpr int kTiles = RA + NSUB;
  constexpr int kLoads = 4 * kTiles;
  static_assert((D - 1) * kLoads <= 63, "ring deeper than the vmcnt counter");

  const int lane = threadIdx.x;
  const int g4 = lane >> 4;
  const int r16 = lane & 15;

  const int64_t unit = blockIdx.x;                 // one wave per workgroup
  const int per_block = p.groups * p.splits;
  const int b = (int)(unit / per_block);
  if (b >= p.num_post_pad[0] / p.BM) return;       // past the routed blocks
  const int rem = (int)(unit - (int64_t)b * per_block);
  const int grp = rem % p.groups;
  const int split = rem / p.groups;
  const int e = __builtin_amdgcn_readfirstlane(p.block_expert[b]);

  const int row_bytes = (int)p.row_bytes;
  const int nchunks = (row_bytes + kChunk - 1) / kChunk;
  const int nfull = row_bytes / kChunk;
  // Even parts: part s takes chunks [s * n / S, (s + 1) * n / S), so no part is
  // empty (the host keeps n / S >= 8) and only the last one holds the row's
  // partial chunk.
  const int c_begin = (int)((int64_t)split * nchunks / p.splits);
  const int c_end = (int)((int64_t)(split + 1) * nchunks / p.splits);

  // valid tokens of this block (sentinels sit at the end of a block)
  const int32_t* blk = p.sorted_ids + (int64_t)b * p.BM;
  const int32_t sid = (lane < p.BM) ? blk[lane] : p.P;
  const int count = __popcll(__ballot(sid < p.P));
  const int nsub = (count + 15) >> 4;

  // ---- tiles: RA weight tiles (16 rows each) then NSUB token tiles (16
  // activation rows each), 256 bytes of each row per chunk, HBM/L2 -> LDS.
  // Load instruction i of a tile covers tile rows 4i + g4 with lane piece
  // r16; LDS slot (row rr, position q) holds the row's 16-byte piece q ^ rr,
  // so the MFMA-layout reads (16 rows, one piece) hit 16 bank groups.
  const uint8_t* wexp = p.W + (int64_t)e * p.w_expert_bytes;
  int row0[RA];
  bool a_ok[RA];
  const uint8_t* src[kTiles][4];                   // the lane's row start per load
#pragma unroll
  for (int ra = 0; ra < RA; ++ra) {
    int base;
    if constexpr (MODE == kGateUp) {
      // pairs of tiles: gate rows c0.., up rows I + c0..
      const int c0 = (grp * (RA / 2) + ra / 2) * 16;
      row0[ra] = c0;
      a_ok[ra] = c0 < p.I;
      base = (ra & 1) ? p.I + c0 : c0;
    } else {
      const int r0 = (grp * RA + ra) * 16;
      row0[ra] = r0;
      a_ok[ra] = r0 < p.H;
      base = r0;
    }
    if (!a_ok[ra]) base = 0;                       // a valid row; never stored
#pragma unroll
    for (int i = 0; i < 4; ++i) src[ra][i] = wexp + (int64_t)(base + 4 * i + g4) * row_bytes;
  }
  if (!a_ok[0]) return;                            // no tile of this wave exists
#pragma unroll
  for (int s = 0; s < NSUB; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = s * 16 + 4 * i + g4;
      const int32_t pair = slot < p.BM ? blk[slot] : p.P;
      // padding slots read activation row 0; their columns are never stored
      const int64_t brow = pair < p.P ? (int64_t)(pair / p.b_row_div) : 0;
      src[RA + s][i] = p.B + brow * row_bytes;
    }
  uint32_t pc[4];                                  // the lane's piece offset per load
#pragma unroll
  for (int i = 0; i < 4; ++i) pc[i] = (uint32_t)((r16 ^ (4 * i + g4)) * 16);
  // Gate/up waves sweep their full chunks starting at chunk c_begin + rot and
  // wrapping round, rot = unit mod the chunk count: waves that run together
  // then read different column ranges of their rows rather than the same
  // one (measured on MI355X, bf16 H = 4096, 64 tokens: gate/up 319 -> 299 us;
  // the down product's rows measured no gain, so they keep the plain order).
  const int c_full = min(c_end, nfull);
  const int rot = MODE == kGateUp && c_full > c_begin ? (int)(unit % (c_full - c_begin)) : 0;

  uint8_t* ring = smem;
  uint32_t rd[4];                                  // MFMA-layout read addresses
#pragma unroll
  for (int j = 0; j < 4; ++j) rd[j] = lds_addr(ring) + r16 * kChunk + (((4 * j + g4) ^ r16) * 16);

  v4f acc[RA][NSUB];
#pragma unroll
  for (int ra = 0; ra < RA; ++ra)
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[ra][s] = v4f{0.f, 0.f, 0.f, 0.f};

  // Every load of the loop goes to LDS and is counted by the explicit waits;
  // the compiler sees no load whose register result it must wait for.
  auto issue = [&](int d, int c) {
    int q = c + rot;                               // the chunk read at position c
    if (q >= c_full) q -= c_full - c_begin;
    const uint32_t off = (uint32_t)q * kChunk;
#pragma unroll
    for (int t = 0; t < RA; ++t)                   // weights: read once, non-temporal
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(
            (const void*)(src[t][i] + off + pc[i]),
            (lds_void*)(ring + (d * kTiles + t) * kTileBytes + i * 1024), 16, 0, kAuxNT);
#pragma unroll
    for (int t = RA; t < kTiles; ++t)              // activations: shared, cached
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(
            (const void*)(src[t][i] + off + pc[i]),
            (lds_void*)(ring + (d * kTiles + t) * kTileBytes + i * 1024), 16, 0, 0);
  };
  // tail: pieces past the row end are read from the row start (valid memory)
  // and zeroed on the token side after the read.
  auto issue_tail = [&](int c) {
    const uint32_t off = (uint32_t)c * kChunk;
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = off + pc[i] < (uint32_t)row_bytes;
        __builtin_amdgcn_global_load_lds(
            (const void*)(src[t][i] + (in ? off + pc[i] : 0u)),
            (lds_void*)(ring + t * kTileBytes + i * 1024), 16, 0, 0);
      }
  };
  auto consume = [&](int d, bool tail, uint32_t off) {
    uint4 bt[NSUB][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      const uint32_t o = (uint32_t)(d * kTiles + RA + s) * kTileBytes;
      lds_read4(bt[s], rd[0] + o, rd[1] + o, rd[2] + o, rd[3] + o);
      if (tail) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (off + (4 * j + g4) * 16 >= (uint32_t)row_bytes) bt[s][j] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int ra = 0; ra < RA; ++ra) {
      uint4 a[4];
      const uint32_t o = (uint32_t)(d * kTiles + ra) * kTileBytes;
      lds_read4(a, rd[0] + o, rd[1] + o, rd[2] + o, rd[3] + o);
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[ra][s] = Tile<FMT>::mma(a, bt[s], acc[ra][s]);
    }
  };
  // Consume stage d and refill it with chunk c: the whole stage is read into
  // registers first, so the refill's loads leave before the products issue
  // (the products of a stage take longer to issue than its reads).
  auto consume_refill = [&](int d, int c) {
    uint4 tl[kTiles][4];
    const uint32_t sb = (uint32_t)(d * kTiles) * kTileBytes;
    lds_read_tiles<0, kTiles>(tl, rd[0] + sb, rd[1] + sb, rd[2] + sb, rd[3] + sb);
    issue(d, c);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) after_issue(tl[t]);
#pragma unroll
    for (int ra = 0; ra < RA; ++ra)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[ra][s] = Tile<FMT>::mma(tl[ra], tl[RA + s], acc[ra][s]);
  };

  // Ring of D chunks over the full chunks of this part: chunk c + d is
  // consumed and chunk c + D + d issued into its stage, so D - 1 chunks stay
  // in flight; the last chunks drain with full waits.
  const int nc = c_full - c_begin;
  if (nc >= D) {
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, c_begin + d);
    int c = c_begin;
    for (; c + 2 * D <= c_full; c += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        wait_vmcnt<(D - 1) * kLoads>();
        consume_refill(d, c + D + d);
      }
    }
    // Drain: stages hold chunks c .. c + D - 1, and ex = c_full - c - D
    // (0 <= ex < D) chunks remain to be loaded into the stages as they free.
    // Before consuming stage d, the stages loaded after it are the D - 1 - d
    // later ones and the min(d, ex) refilled ones.
    const int ex = c_full - c - D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      wait_stages<kLoads, D>(D - 1 - d + min(d, ex));
      if (d < ex) consume_refill(d, c + D + d);
      else consume(d, false, 0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (d < ex) {
        wait_stages<kLoads, D>(ex - 1 - d);
        consume(d, false, 0);
      }
    }
  } else if (nc > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (d < nc) issue(d, c_begin + d);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (d < nc) {
        wait_stages<kLoads, D>(nc - 1 - d);
        consume(d, false, 0);
      }
    }
  }
  // The row's partial last chunk, when this part holds it.
  if (c_end > nfull) {
    issue_tail(nfull);
    wait_vmcnt<0>();
    consume(0, true, (uint32_t)nfull * kChunk);
  }

  // ------------------------------------------------------------ epilogue
  // Lane (g4, r16) holds rows 4*g4 + v of each 16-row weight tile for token
  // column r16.  Per tensor: one scale for the whole block; per row: the
  // weight row's scale times the activation row's.
  float scale = 1.0f;
  const bool rows = FP8 && p.row_scales;
  const int64_t wrow0 = (int64_t)e * (MODE == kGateUp ? 2 * p.I : p.H);
  if constexpr (FP8)
    if (!rows) scale = scale_from_amax_bits(*p.act_amax, fp8_max<FMT>()) * p.w_scale[e];

  if constexpr (MODE == kGateUp) {
    float local_max = 0.0f;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (s >= nsub) continue;
      const int32_t pair = blk[s * 16 + r16];
      if (pair >= p.P) continue;
      const float sa = rows ? p.act_scale[pair / p.b_row_div] : 1.0f;
#pragma unroll
      for (int cg = 0; cg < RA / 2; ++cg) {
        if (!a_ok[2 * cg]) continue;
        const int col = row0[2 * cg] + 4 * g4;
        float sg[4] = {scale, scale, scale, scale}, su[4] = {scale, scale, scale, scale};
        if (rows) row_scales4(p.w_scale + wrow0, col, p.I + col, sa, sg, su);
        float av[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gt = acc[2 * cg][s][v] * sg[v];
          const float up = acc[2 * cg + 1][s][v] * su[v];
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
        if (lane == 0 && local_max > 0.0f) amax_slot_max(p.a_amax, (uint32_t)unit, local_max);
      }
    }
  } else {
    const int64_t part = (int64_t)split * p.dw_split_stride;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (s >= nsub) continue;
      const int32_t pair = blk[s * 16 + r16];
      if (pair >= p.P) continue;
      const float sa = rows ? p.act_scale[pair] : 1.0f;
#pragma unroll
      for (int ra = 0; ra < RA; ++ra) {
        if (!a_ok[ra]) continue;
        float sc[4] = {scale, scale, scale, scale};
        if (rows) row_scales4(p.w_scale + wrow0, row0[ra] + 4 * g4, sa, sc);
        store_part4(p.dw, p.dw_bf16, part + (int64_t)pair * p.H + row0[ra] + 4 * g4,
                    acc[ra][s][0] * sc[0], acc[ra][s][1] * sc[1], acc[ra][s][2] * sc[2],
                    acc[ra][s][3] * sc[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent form.  A wave walks units u = blockIdx.x, blockIdx.x + gridDim.x,
// ... (grid = the waves the chip holds at once) and its chunk stream runs
// across unit boundaries: the next units' first chunks load while the current
// one finishes, so a unit costs no start-up latency.  Everything a unit needs
// besides its rows -- its block's pair ids, its expert id and (FP8) the
// expert's weight scale -- also arrives by direct-to-LDS loads in the same
// ordered stream, ahead of use, into small per-wave slots; no register load
// whose wait would drain the stream sits on the path.  Rows may end in a
// partial chunk (as in the one-wave-per-unit form).  Per-tensor scales only:
// the host launches the one-wave-per-unit form for per-row scales.
//
// Schedule, in steps t = k * cps + j (unit k, chunk j, cps chunks per unit):
// during step t the wave reads stage t % D into registers, issues the chunk of
// step t + D into it, then runs the stage's products (and, at a unit's last
// chunk, the unit's epilogue).  At the start of step t everything issued
// during steps up to t - D has landed (loads complete in order; stores only
// add to the counter).  The chunks of unit k start to be issued at step
// k * cps - D, which reads unit k's ids and expert id and issues those of unit
// k + m, m = ceil(D / cps): issued at step (k - m) * cps - D <= k * cps - 2 D,
// they have landed.  With NS = 2 m + 1 slots, unit k + NS's ids overwrite
// slot k at step (k + m + 1) * cps - D >= (k + 1) * cps, a step after unit k's
// epilogue at step (k + 1) * cps - 1.
constexpr int kMetaBytes = 272;       // pair ids [64], expert id, weight scale (16-byte slots)

// Units whose ids are issued ahead, and slots, for cps chunks per unit.
__host__ __device__ constexpr int meta_ahead(int d, int cps) { return (d + cps - 1) / cps; }
__host__ __device__ constexpr int meta_slots(int d, int cps) { return 2 * meta_ahead(d, cps) + 1; }

__device__ __forceinline__ uint32_t lds_read_u32(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n"
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(v)
               : "v"(a)
               : "memory");
  return v;
}

template <int MODE, int FMT, int NSUB, int RA, int D>
__global__ __launch_bounds__(64) void moe_gemm_stream_kernel(GemmParams p) {
  constexpr bool FP8 = FMT != kFmtBF16;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int kTiles = RA + NSUB;
  constexpr int kLoads = 4 * kTiles;
  static_assert((D - 1) * kLoads <= 63, "ring deeper than the vmcnt counter");

  const int lane = threadIdx.x;
  const int g4 = lane >> 4;
  const int r16 = lane & 15;

  // plain loads, before the stream starts
  const int per_block = p.groups * p.splits;
  const int64_t total = (int64_t)(p.num_post_pad[0] / p.BM) * per_block;
  const int64_t u0 = blockIdx.x, du = gridDim.x;
  if (u0 >= total) return;
  float act_scale = 1.0f;
  if constexpr (FP8) act_scale = scale_from_amax_bits(*p.act_amax, fp8_max<FMT>());

  const int nw = (int)((total - 1 - u0) / du) + 1;         // units of this wave
  const int row_bytes = (int)p.row_bytes;
  const int nchunks = (row_bytes + kChunk - 1) / kChunk;
  const bool part_tail = row_bytes % kChunk != 0;           // the last chunk is partial
  const int cps = nchunks / p.splits;                       // chunks per unit
  const int nsteps = nw * cps;
  const int ahead = meta_ahead(D, cps), nslots = meta_slots(D, cps);

  uint8_t* ring = smem;
  uint8_t* meta = smem + D * kTiles * kTileBytes;
  const uint32_t meta_a = lds_addr(meta);
  auto unit_pos = [&](int k, int& b, int& grp, int& split) {
    const int64_t u = u0 + (int64_t)k * du;
    b = (int)(u / per_block);
    const int rem = (int)(u - (int64_t)b * per_block);
    grp = rem % p.groups;
    split = rem / p.groups;
  };
  auto meta_issue = [&](int k) {                   // ids and expert id of unit k
    int b, grp, split;
    unit_pos(k, b, grp, split);
    uint8_t* slot = meta + (k % nslots) * kMetaBytes;
    const int32_t* blk = p.sorted_ids + (int64_t)b * p.BM;
    __builtin_amdgcn_global_load_lds((const void*)(blk + (lane < p.BM ? lane : 0)),
                                     (lds_void*)slot, 4, 0, 0);
    if (lane == 0)                                 // one word: lane 0 writes at the slot base
      __builtin_amdgcn_global_load_lds((const void*)(p.block_expert + b),
                                       (lds_void*)(slot + 256), 4, 0, 0);
  };

  uint32_t pc[4];                                  // the lane's piece offset per load
#pragma unroll
  for (int i = 0; i < 4; ++i) pc[i] = (uint32_t)((r16 ^ (4 * i + g4)) * 16);
  uint32_t rd[4];                                  // MFMA-layout read addresses
#pragma unroll
  for (int j = 0; j < 4; ++j) rd[j] = lds_addr(ring) + r16 * kChunk + (((4 * j + g4) ^ r16) * 16);

  // ---- load side: the unit whose chunks are being issued
  const uint8_t* src[kTiles][4];
  int l_cbegin = 0;
  auto load_setup = [&](int k) {                   // unit k's ids and expert id have landed
    int b, grp, split;
    unit_pos(k, b, grp, split);
    const uint32_t slot = meta_a + (uint32_t)((k % nslots) * kMetaBytes);
    const int e = __builtin_amdgcn_readfirstlane((int)lds_read_u32(slot + 256));
    const uint8_t* wexp = p.W + (int64_t)e * p.w_expert_bytes;
#pragma unroll
    for (int ra = 0; ra < RA; ++ra) {
      int base;
      if constexpr (MODE == kGateUp) {
        const int c0 = (grp * (RA / 2) + ra / 2) * 16;
        base = c0 < p.I ? ((ra & 1) ? p.I + c0 : c0) : 0;
      } else {
        const int r0 = (grp * RA + ra) * 16;
        base = r0 < p.H ? r0 : 0;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) src[ra][i] = wexp + (int64_t)(base + 4 * i + g4) * row_bytes;
    }
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = s * 16 + 4 * i + g4;
        const int32_t pair = q < p.BM ? (int32_t)lds_read_u32(slot + 4 * q) : p.P;
        const int64_t brow = pair < p.P ? (int64_t)(pair / p.b_row_div) : 0;
        src[RA + s][i] = p.B + brow * row_bytes;
      }
    l_cbegin = split * cps;
    if constexpr (FP8) {                            // the expert's weight scale, for the epilogue
      if (lane == 0)
        __builtin_amdgcn_global_load_lds((const void*)(p.w_scale + e),
                                         (lds_void*)(meta + (k % nslots) * kMetaBytes + 260), 4,
                                         0, 0);
    }
  };
  // pieces past the row end (partial last chunk) are read from the row start
  // (valid memory) and zeroed on the token side after the read
  auto issue = [&](int d, int c) {
    const uint32_t off = (uint32_t)c * kChunk;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (off + pc[i] < (uint32_t)row_bytes) ? off + pc[i] : 0u;
#pragma unroll
    for (int t = 0; t < RA; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(
            (const void*)(src[t][i] + o[i]),
            (lds_void*)(ring + (d * kTiles + t) * kTileBytes + i * 1024), 16, 0, kAuxNT);
#pragma unroll
    for (int t = RA; t < kTiles; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(
            (const void*)(src[t][i] + o[i]),
            (lds_void*)(ring + (d * kTiles + t) * kTileBytes + i * 1024), 16, 0, 0);
  };
  // Gate/up units (one part per row) sweep their full chunks from position
  // unit mod the full-chunk count on, wrapping round, and read a partial last
  // chunk last: the same order as the one-wave-per-unit form.
  const int nrot = cps - (part_tail ? 1 : 0);
  // issue the chunk of step t (into stage t % D), setting up its unit first
  auto issue_step = [&](int t) {
    const int k = t / cps, j = t - k * cps;
    if (j == 0) {
      load_setup(k);
      if (k + ahead < nw) meta_issue(k + ahead);
    }
    int q = j;
    if (MODE == kGateUp && j < nrot) {
      q += (int)((u0 + (int64_t)k * du) % nrot);
      if (q >= nrot) q -= nrot;
    }
    issue(t % D, l_cbegin + q);
  };

  // ---- compute side
  v4f acc[RA][NSUB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int ra = 0; ra < RA; ++ra)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[ra][s] = v4f{0.f, 0.f, 0.f, 0.f};
  };
  // Consume stage d, then (refill >= 0) issue step `refill` into it: the
  // whole stage is read into registers first, so the refill's loads leave
  // before the products issue (the products of a stage take longer to issue
  // than its reads).
  auto consume = [&](int d, bool tail, uint32_t off, int refill) {
    uint4 tl[kTiles][4];
    const uint32_t sb = (uint32_t)(d * kTiles) * kTileBytes;
    lds_read_tiles<0, kTiles>(tl, rd[0] + sb, rd[1] + sb, rd[2] + sb, rd[3] + sb);
    if (tail) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (off + (4 * j + g4) * 16 >= (uint32_t)row_bytes) tl[RA + s][j] = make_uint4(0, 0, 0, 0);
    }
    if (refill >= 0) issue_step(refill);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) after_issue(tl[t]);
#pragma unroll
    for (int ra = 0; ra < RA; ++ra)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[ra][s] = Tile<FMT>::mma(tl[ra], tl[RA + s], acc[ra][s]);
  };
  auto epilogue = [&](int k) {
    int b, grp, split;
    unit_pos(k, b, grp, split);
    const uint32_t slot = meta_a + (uint32_t)((k % nslots) * kMetaBytes);
    float scale = 1.0f;
    if constexpr (FP8) scale = act_scale * __uint_as_float(lds_read_u32(slot + 260));
    if constexpr (MODE == kGateUp) {
      float local_max = 0.0f;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const int q = s * 16 + r16;
        const int32_t pair = q < p.BM ? (int32_t)lds_read_u32(slot + 4 * q) : p.P;
        if (pair >= p.P) continue;
#pragma unroll
        for (int cg = 0; cg < RA / 2; ++cg) {
          const int c0 = (grp * (RA / 2) + cg) * 16;
          if (c0 >= p.I) continue;
          const int col = c0 + 4 * g4;
          float av[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float gt = acc[2 * cg][s][v] * scale;
            const float up = acc[2 * cg + 1][s][v] * scale;
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
        local_max = wave_max(local_max);
        if (lane == 0 && local_max > 0.0f)
          amax_slot_max(p.a_amax, (uint32_t)(u0 + (int64_t)k * du), local_max);
      }
    } else {
      const int64_t part = (int64_t)split * p.dw_split_stride;
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const int q = s * 16 + r16;
        const int32_t pair = q < p.BM ? (int32_t)lds_read_u32(slot + 4 * q) : p.P;
        if (pair >= p.P) continue;
#pragma unroll
        for (int ra = 0; ra < RA; ++ra) {
          const int r0 = (grp * RA + ra) * 16;
          if (r0 >= p.H) continue;
          store_part4(p.dw, p.dw_bf16, part + (int64_t)pair * p.H + r0 + 4 * g4,
                      acc[ra][s][0] * scale, acc[ra][s][1] * scale, acc[ra][s][2] * scale,
                      acc[ra][s][3] * scale);
        }
      }
    }
  };

  // ---- the stream
  for (int k = 0; k < ahead && k < nw; ++k) meta_issue(k);
  wait_vmcnt<0>();
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < nsteps) issue_step(d);
  zero_acc();
  for (int t = 0; t < nsteps; ++t) {
    const int later = nsteps - 1 - t;                // steps issued after this one, at most D - 1
    if (later >= D - 1) wait_vmcnt<(D - 1) * kLoads>();
    else wait_stages<kLoads, D>(later);
    const int j = t % cps;
    const bool tail = part_tail && j == cps - 1 &&
                      (int)((u0 + (int64_t)(t / cps) * du) % per_block) / p.groups ==
                          p.splits - 1;
    consume(t % D, tail, (uint32_t)(nchunks - 1) * kChunk, t + D < nsteps ? t + D : -1);
    if ((t + 1) % cps == 0) {
      epilogue(t / cps);
      zero_acc();
    }
  }
}

// Kernel preparation (dynamic LDS limits), run once per device by the entry
// points before any launch (prepare_decode_kernels).
template <int MODE, int FMT, int NSUB, int RA, int D>
hipError_t ready_one() {
  return prepare_kernel(
      reinterpret_cast<const void*>(&moe_gemm_decode_kernel<MODE, FMT, NSUB, RA, D>),
      D * (RA + NSUB) * kTileBytes);
}

// LDS of the stream form: the ring and the id slots for cps chunks per unit.
constexpr int stream_lds(int d, int tiles, int cps) {
  return d * tiles * kTileBytes + meta_slots(d, cps) * kMetaBytes;
}

template <int MODE, int FMT, int NSUB, int RA, int D>
hipError_t ready_stream() {                        // the limit for the most slots (cps = 1)
  return prepare_kernel(
      reinterpret_cast<const void*>(&moe_gemm_stream_kernel<MODE, FMT, NSUB, RA, D>),
      stream_lds(D, RA + NSUB, 1));
}

template <int MODE, int FMT, int NSUB, int RA, int D>
hipError_t launch_one(const GemmParams& p, dim3 grid, hipStream_t stream) {
  const int lds = D * (RA + NSUB) * kTileBytes;
  moe_gemm_decode_kernel<MODE, FMT, NSUB, RA, D><<<grid, dim3(64), lds, stream>>>(p);
  return hipGetLastError();
}

// The persistent form (ring depth DS) when each resident wave gets 2 to 7
// units on average (with one unit the unit's ids cost an extra round trip;
// with many units, and for one-chunk rows, the one-wave-per-unit grid with
// ring depth DC measured faster); the parts of the reduction must be equal.
// Grid = the waves resident on `num_cus` compute units.
template <int MODE, int FMT, int NSUB, int RA, int DC, int DS>
hipError_t launch_best(const GemmParams& p, dim3 grid, int num_cus, hipStream_t stream) {
  const int64_t nchunks = (p.row_bytes + kChunk - 1) / kChunk;
  const int cps = (int)(nchunks / p.splits);
  const int lds = stream_lds(DS, RA + NSUB, cps > 0 ? cps : 1);
  const int64_t resident = (int64_t)num_cus * std::max(1, (160 * 1024) / lds);
  // The persistent form carries one weight scale per unit in its metadata
  // slots, so per-row scales take the classic form.
  const bool stream_ok = !p.row_scales && DS > 1 && nchunks % p.splits == 0 && cps >= 1 &&
                         grid.x >= 2 * resident && grid.x < 8 * resident;
  if (!stream_ok) return launch_one<MODE, FMT, NSUB, RA, DC>(p, grid, stream);
  const unsigned g = (unsigned)std::min<int64_t>(grid.x, resident);
  moe_gemm_stream_kernel<MODE, FMT, NSUB, RA, DS><<<dim3(g), dim3(64), lds, stream>>>(p);
  return hipGetLastError();
}

// Rows of several chunks: both forms with the ring depth of the shape.
template <int MODE, int FMT, int NSUB, int RA, bool SHORT>
hipError_t launch_depth(const GemmParams& p, dim3 grid, int num_cus, hipStream_t stream) {
  constexpr int D = ring_depth(MODE, RA, NSUB, SHORT);
  constexpr int DD = deep_depth(RA, NSUB);
  if constexpr (DD > D) {
    const int64_t deep = (int64_t)num_cus * ((160 * 1024) / (DD * (RA + NSUB) * kTileBytes));
    if ((int64_t)grid.x <= deep) return launch_one<MODE, FMT, NSUB, RA, DD>(p, grid, stream);
  }
  return launch_best<MODE, FMT, NSUB, RA, D, D>(p, grid, num_cus, stream);
}

template <int MODE, int FMT, int RA>
hipError_t launch_nsub(const GemmParams& p, int nsub_max, dim3 grid, int num_cus,
                       hipStream_t stream) {
  if constexpr (RA >= 8) {
    if (nsub_max > 2) return hipErrorInvalidValue;   // would not fit the registers
  }
  if (p.row_bytes <= kChunk) {
    // one chunk per row: the one-wave-per-unit form needs no ring, so the LDS
    // holds more waves; the stream form keeps its ring across units
    switch (nsub_max) {
      case 1:
        return launch_best<MODE, FMT, 1, RA, 1, ring_depth(MODE, RA, 1, true)>(p, grid, num_cus,
                                                                              stream);
      case 2:
        return launch_best<MODE, FMT, 2, RA, 1, ring_depth(MODE, RA, 2, true)>(p, grid, num_cus,
                                                                              stream);
      case 4:
        if constexpr (RA < 8)
          return launch_best<MODE, FMT, 4, RA, 1, ring_depth(MODE, RA, 4, true)>(p, grid, num_cus,
                                                                                 stream);
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
  const bool sh = (p.row_bytes + kChunk - 1) / kChunk < kShortRow;
  switch (nsub_max) {
    case 1:
      return sh ? launch_depth<MODE, FMT, 1, RA, true>(p, grid, num_cus, stream)
                : launch_depth<MODE, FMT, 1, RA, false>(p, grid, num_cus, stream);
    case 2:
      return sh ? launch_depth<MODE, FMT, 2, RA, true>(p, grid, num_cus, stream)
                : launch_depth<MODE, FMT, 2, RA, false>(p, grid, num_cus, stream);
    case 4:
      if constexpr (RA < 8)
        return sh ? launch_depth<MODE, FMT, 4, RA, true>(p, grid, num_cus, stream)
                  : launch_depth<MODE, FMT, 4, RA, false>(p, grid, num_cus, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int MODE, int RA>
hipError_t launch_dtype(int fmt, const GemmParams& p, int nsub_max, dim3 grid, int num_cus,
                        hipStream_t stream) {
  if (fmt == kFmtE4M3) return launch_nsub<MODE, kFmtE4M3, RA>(p, nsub_max, grid, num_cus, stream);
  if (fmt == kFmtE5M2) return launch_nsub<MODE, kFmtE5M2, RA>(p, nsub_max, grid, num_cus, stream);
  return launch_nsub<MODE, kFmtBF16, RA>(p, nsub_max, grid, num_cus, stream);
}

template <int MODE, int FMT, int RA, int NSUB>
hipError_t ready_shape() {
  constexpr int DS = ring_depth(MODE, RA, NSUB, true), DL = ring_depth(MODE, RA, NSUB, false);
  hipError_t e = ready_one<MODE, FMT, NSUB, RA, 1>();
  if (e == hipSuccess) e = ready_one<MODE, FMT, NSUB, RA, DS>();
  if (e == hipSuccess) e = ready_stream<MODE, FMT, NSUB, RA, DS>();
  if constexpr (DL != DS) {
    if (e == hipSuccess) e = ready_one<MODE, FMT, NSUB, RA, DL>();
    if (e == hipSuccess) e = ready_stream<MODE, FMT, NSUB, RA, DL>();
  }
  constexpr int DD = deep_depth(RA, NSUB);
  if constexpr (DD != DS && DD != DL)
    if (e == hipSuccess) e = ready_one<MODE, FMT, NSUB, RA, DD>();
  return e;
}

template <int MODE, int FMT, int RA>
hipError_t ready_ra() {
  hipError_t e = ready_shape<MODE, FMT, RA, 1>();
  if (e == hipSuccess) e = ready_shape<MODE, FMT, RA, 2>();
  if constexpr (RA < 8)                            // RA = 8 takes at most 2 token tiles
    if (e == hipSuccess) e = ready_shape<MODE, FMT, RA, 4>();
  return e;
}

}  // namespace

hipError_t prepare_decode_kernels() {
  hipError_t e = hipSuccess;
  auto all = [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    if (e == hipSuccess) e = ready_ra<kGateUp, F, 2>();
    if (e == hipSuccess) e = ready_ra<kGateUp, F, 4>();
    if (e == hipSuccess) e = ready_ra<kDown, F, 2>();
    if (e == hipSuccess) e = ready_ra<kDown, F, 4>();
    if (e == hipSuccess) e = ready_ra<kDown, F, 8>();
  };
  all(std::integral_constant<int, kFmtBF16>{});
  all(std::integral_constant<int, kFmtE4M3>{});
  all(std::integral_constant<int, kFmtE5M2>{});
  return e;
}

namespace {

// Waves of one shape that the chip holds at once: one wave per workgroup with
// D * (RA + NSUB) 4 KB LDS tiles, 160 KB of LDS per compute unit.
int64_t resident_waves(int mode, int ra, int nsub, int64_t row_bytes, int num_cus) {
  const bool sh = (row_bytes + kChunk - 1) / kChunk < kShortRow;
  const int d = row_bytes <= kChunk ? 1 : ring_depth(mode, ra, nsub, sh);
  const int per_cu = (160 * 1024) / (d * (ra + nsub) * kTileBytes);
  return (int64_t)std::max(num_cus, 1) * (per_cu > 0 ? per_cu : 1);
}

// Compute units the split rule counts at most: the largest gfx950 part, so
// the workspace a call needs does not depend on the device.
constexpr int kSplitCus = 256;

// Parts of the down product's reduction for RA weight tiles per wave: split
// until the expected units (est_blocks routed blocks; the layout's capacity
// holds more) give each resident wave about two, keeping >= 8 chunks per
// part.  Measured on MI355X, bf16 H = 4096, I = 14336: 64 tokens (32-token
// blocks) two parts 152 us, four 160 us, eight 183 us; 8 tokens one part
// 195 us, two 144 us, four 149 us.
int down_splits(int64_t est_blocks, int rows, int nchunks, int ra, int nsub, int64_t row_bytes,
                int cus) {
  const int64_t units = est_blocks * ((rows + 16 * ra - 1) / (16 * ra));
  const int64_t resident = resident_waves(kDown, ra, nsub, row_bytes, std::min(cus, kSplitCus));
  int sp = 1;
  while (units * sp < 2 * resident && nchunks / (2 * sp) >= 8 && sp < 16) sp *= 2;
  return sp;
}

// Busy fraction of the rounds a grid of `units` waves takes (the last round
// may be partly empty).
double round_fill(int64_t units, int64_t resident) {
  const double r = (double)units / (double)resident;
  return r / std::ceil(r);
}

}  // namespace

DecodeShape decode_shape(int mode, int64_t nblk_cap, int64_t est_blocks, int rows,
                         int64_t row_bytes, int bm, int num_cus) {
  DecodeShape s{};
  const int nchunks = (int)((row_bytes + kChunk - 1) / kChunk);
  const int nsub = bm / 16;
  // RA = 2 or 4 weight tiles per wave.  Short rows make short waves, where
  // more of them in flight wins: RA = 2.  With long rows a partly empty last
  // round of resident waves costs a whole wave time, so the other RA is taken
  // when its grid fills the rounds clearly better (small grids).
  auto pick = [&](int pref, auto units_of) {
    if (nchunks < kShortRow) return 2;
    const int alt = 6 - pref;
    const double fp =
        round_fill(units_of(pref), resident_waves(mode, pref, nsub, row_bytes, num_cus));
    const double fa =
        round_fill(units_of(alt), resident_waves(mode, alt, nsub, row_bytes, num_cus));
    return fa > fp + 0.05 ? alt : pref;
  };
  if (mode == kGateUp) {
    // rows = I: a wave owns RA / 2 groups of 16 columns (16 gate and 16 up
    // rows each); more token tiles call for more weight tiles per wave, so
    // the weights keep most of the LDS ring.
    auto units = [&](int ra) { return nblk_cap * ((rows + 8 * ra - 1) / (8 * ra)); };
    s.ra = pick(nsub == 1 ? 2 : 4, units);
    s.groups = (rows + 8 * s.ra - 1) / (8 * s.ra);
    s.splits = 1;
  } else {
    // rows = H: RA 16-row tiles per wave; short rows take more tiles; the
    // reduction is split as down_splits says.
    auto splits_of = [&](int ra) {
      return down_splits(est_blocks, rows, nchunks, ra, nsub, row_bytes, num_cus);
    };
    auto units = [&](int ra) {
      return nblk_cap * ((rows + 16 * ra - 1) / (16 * ra)) * splits_of(ra);
    };
    // one-chunk rows: 8 weight tiles per wave with 2 token tiles (measured
    // on the TP8 slice: T = 256 down 48.8 -> 42.1 us; with 1 token tile 4
    // tiles stay faster)
    s.ra = row_bytes <= kChunk ? (nsub == 2 ? 8 : 4)
                               : row_bytes < 512 ? 4 : pick(nsub == 1 ? 2 : 4, units);
    s.groups = (rows + 16 * s.ra - 1) / (16 * s.ra);
    s.splits = splits_of(s.ra);
  }
  return s;
}

int decode_max_splits(int64_t est_blocks, int rows, int64_t row_bytes, int bm) {
  const int nchunks = (int)((row_bytes + kChunk - 1) / kChunk);
  int m = 1;
  for (int ra : {2, 4, 8})
    m = std::max(m, down_splits(est_blocks, rows, nchunks, ra, bm / 16, row_bytes, kSplitCus));
  return m;
}

hipError_t launch_gemm_decode(int mode, int fmt, const GemmParams& p, int ra, int64_t nblk_cap,
                              int num_cus, hipStream_t stream) {
  const int nsub_max = p.BM / 16;
  const int64_t wgs = nblk_cap * p.groups * p.splits;   // one wave each
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7FFFFFFF || p.row_bytes > (1 << 24)) return hipErrorInvalidValue;
  dim3 grid((unsigned)wgs);
  if (mode == kGateUp) {
    if (ra == 2) return launch_dtype<kGateUp, 2>(fmt, p, nsub_max, grid, num_cus, stream);
    if (ra == 4) return launch_dtype<kGateUp, 4>(fmt, p, nsub_max, grid, num_cus, stream);
    return hipErrorInvalidValue;
  }
  if (ra == 2) return launch_dtype<kDown, 2>(fmt, p, nsub_max, grid, num_cus, stream);
  if (ra == 4) return launch_dtype<kDown, 4>(fmt, p, nsub_max, grid, num_cus, stream);
  if (ra == 8) return launch_dtype<kDown, 8>(fmt, p, nsub_max, grid, num_cus, stream);
  return hipErrorInvalidValue;
}

}  // namespace moe
