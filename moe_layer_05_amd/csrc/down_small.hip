// a5 + a6 in one launch for calls of at most 8 token-expert pairs (one decode
// token at K <= 8, a few at smaller K): the down product and the
// routing-weighted combine.
//
// The pages make the fused layer one pass over the selected experts whose
// epilogue applies the scales and aggregates the experts' outputs (aib.vote
// page, third paragraph), and single-token decode the shape where the fixed
// work around the expert GEMMs weighs most (aib.vote page, second paragraph:
// M < 64 or M = 1; toolboxkart.tech page, "Why MoE inference needs
// specialized kernels").  With so few pairs every pair fits one column of a
// 16x16 MFMA tile, which lets one accumulator hold the down products of all
// of a call's experts at once:
//  - column p of the B operand holds pair p's intermediate row (bfloat16, or
//    its FP8 codes); while the wave streams expert e's weight rows it zeroes
//    (in registers) the columns of the pairs not routed to e, so column p
//    accumulates exactly W2[e(p)] a_p, whatever the number of experts;
//  - a workgroup owns 16 output rows and its waves split the steps (chunk of
//    the reduction dimension, expert); after the stream each wave scales its
//    accumulator (the dequantisation scales, then the routing weight of the
//    column's pair) into LDS, and each (token, row) output sums its K pairs'
//    values over the waves in a fixed order, rounded once to bfloat16: no
//    partial rows in HBM, no combine launch, no atomics, the same bits every
//    run.
// The weight stream is the decode one: direct-to-LDS loads (weights
// non-temporal) into a ring of stages per wave, waits on the wave's own
// vector-memory counter; each stage also brings the chunk of the pair rows.
// (Forming the intermediate's FP8 codes in this kernel instead, from the
// float32 rows and the amax, was measured slower: every workgroup needs all
// codes, so the divisions and roundings ran once per workgroup.)
#include <algorithm>

#include "device_common.hpp"
#include "internal.hpp"
#include "ring_device.hpp"

namespace moe {
namespace {

constexpr int kSmallD = 4;            // ring stages per wave
constexpr int kSmallMaxWaves = 8;     // waves per workgroup
constexpr int kSmallLdsMax = 160 * 1024;
constexpr int kSmallMaxResidentWaves = 20;   // per compute unit at the kernel's < 100 VGPRs

struct SmallDownArgs {
  const uint8_t* W;           // w2 [E][H][I] (bytes)
  int64_t w_expert_bytes;     // H * I * elem
  int row_bytes;              // I * elem
  const uint8_t* B;           // rows of a [P][row_bytes] (bfloat16, or FP8 codes)
  const int32_t* ids;         // [P] expert of each pair
  const float* wts;           // [P] routing weights
  const float* w_scale;       // FP8: [E] per tensor, [E][H] per row
  const uint32_t* act_amax;   // FP8 per tensor: the final amax word of a
  const float* act_scale;     // FP8 per row: [P]
  int P, K, H, I;
  int region;                 // LDS bytes per wave
  int depth;                  // ring stages per wave (1..kSmallD)
  uint16_t* out;              // [P / K][H] bfloat16
};

// NB: quarter token tiles (4 pair rows each) streamed per stage (1 or 2).  ROWS: FP8
// with one scale per weight row and per pair row (else one per tensor).
//
// Work of a workgroup: steps t = c * nexp + j (chunk c of the row, j-th
// distinct expert of the call), chunk-major; wave w takes the steps
// [w S / nw, (w + 1) S / nw), S = nexp * nchunks, so one wave may cover
// several experts of one chunk or several chunks of all experts, and the
// workgroup's rows are summed over every step by the LDS reduction.
template <int FMT, int NB, bool ROWS>
__global__ __launch_bounds__(kSmallMaxWaves * kWave) void moe_down_small_kernel(SmallDownArgs p) {
  constexpr bool FP8 = FMT != kFmtBF16;
  constexpr int kLoads = 4 + NB;                    // per stage: 16 weight rows, 4 * NB pair rows
  constexpr int kStage = kTileBytes + NB * 1024;
  static_assert(NB == 1 || NB == 2, "pair rows per stage");
  static_assert(!ROWS || FP8, "per-row scales are FP8 only");
  static_assert((kSmallD - 1) * kLoads <= 63, "ring deeper than the vmcnt counter");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int g4 = lane >> 4;
  const int r16 = lane & 15;
  const int h0 = blockIdx.x * 16;
  const int row_bytes = p.row_bytes;
  const int nchunks = (row_bytes + kChunk - 1) / kChunk;
  const int nfull = row_bytes / kChunk;
  const int depth = p.depth;                        // ring stages, 1..kSmallD
  uint8_t* ring = smem + (size_t)wave * p.region;

  // ---- the call's experts: lane p < P holds pair p's expert; lane j holds
  // the j-th distinct expert in pair order (P <= 8)
  const int my_e = lane < p.P ? p.ids[lane] : -1;
  bool first = lane < p.P;
  for (int q = 0; q < 16; ++q) {
    const int eq = __shfl(my_e, q);
    if (q < lane && eq == my_e) first = false;
  }
  const uint64_t fm = __ballot(first);
  const int nexp = __popcll(fm);
  int pos = 0;
  {
    uint64_t m = fm;
    for (int k = 0; m; ++k, m &= m - 1)
      if (k == lane) pos = __builtin_ctzll(m);
  }
  const int elist = __shfl(my_e, pos);

  // ---- this wave's steps (the host keeps nw <= K * nchunks <= S, so every
  // wave has at least one)
  const int S = nexp * nchunks;
  const int t0 = (int)((int64_t)wave * S / nw);
  const int nsteps = (int)((int64_t)(wave + 1) * S / nw) - t0;
  const int cfirst = nexp > 0 ? t0 / nexp : 0;
  const int jfirst = t0 - cfirst * nexp;

  // ---- what the epilogue multiplies column r16 by, loaded now so the loads
  // overlap the stream: the routing weight and (FP8) the scales -- the
  // expert's weight scale times a's, or per output row h0 + 4 g4 + v the
  // weight row's scale times the pair row's.  (Unconditional loads at
  // clamped indices: a load under a branch whose result merges with a
  // constant makes the compiler wait for it at once.)
  const bool col_ok = r16 < p.P;
  const int cr = col_ok ? r16 : 0;
  const int col_e = __shfl(my_e, cr);
  const float col_w = p.wts[cr];
  float col_ws = 1.0f, col_as = 1.0f;
  uint32_t amax_bits = 0;
  float4 col_ws4 = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
  if constexpr (ROWS) {
    col_ws4 = *reinterpret_cast<const float4*>(p.w_scale + (int64_t)col_e * p.H + h0 + 4 * g4);
    col_as = p.act_scale[cr];
  } else if constexpr (FP8) {
    col_ws = p.w_scale[col_e];
    amax_bits = *p.act_amax;
  }

  // ---- weight rows h0 + 4i + g4 and pair rows 4i + g4, the lane's piece per load
  uint32_t pc[4];
  int64_t wrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pc[i] = (uint32_t)((r16 ^ (4 * i + g4)) * 16);
    wrow[i] = (int64_t)(h0 + 4 * i + g4) * row_bytes;
  }
  const uint8_t* brow[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = min(4 * i + g4, p.P - 1);         // rows past the pairs: any valid row
    brow[i] = p.B + (int64_t)r * row_bytes;
  }

  // stage d <- step (chunk c, expert j); pieces past a partial row's end are
  // read from the row start (valid memory) and zeroed on the B side
  auto issue = [&](int d, int c, int j) {
    const int e = __builtin_amdgcn_readlane(elist, j);
    const uint8_t* wexp = p.W + (int64_t)e * p.w_expert_bytes;
    const uint32_t off = (uint32_t)c * kChunk;
    uint8_t* st = ring + d * kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = off + pc[i];
      __builtin_amdgcn_global_load_lds((const void*)(wexp + wrow[i] + (o < (uint32_t)row_bytes ? o : 0u)),
                                       (lds_void*)(st + i * 1024), 16, 0, kAuxNT);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const uint32_t o = off + pc[i];
      __builtin_amdgcn_global_load_lds((const void*)(brow[i] + (o < (uint32_t)row_bytes ? o : 0u)),
                                       (lds_void*)(st + kTileBytes + i * 1024), 16, 0, 0);
    }
  };

  int ic = cfirst, ij = jfirst;                     // next step to issue
  for (int d = 0; d < depth && d < nsteps; ++d) {
    issue(d, ic, ij);
    if (++ij == nexp) { ij = 0; ++ic; }
  }

  // ---- the stream: one accumulator, column p = pair p
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  uint32_t rd_w[4], rd_b[4];                         // weight row r16; pair row brr
  const int brr = r16 < 4 * NB ? r16 : 0;            // (masked when past the pairs)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rd_w[j] = (uint32_t)(r16 * kChunk + (((4 * j + g4) ^ r16) * 16));
    rd_b[j] = (uint32_t)(kTileBytes + brr * kChunk + (((4 * j + g4) ^ brr) * 16));
  }
  const uint32_t ring_base = lds_addr(ring);

  int c = cfirst, j = jfirst, d = 0;                 // step to consume and its stage
  for (int t = 0; t < nsteps; ++t) {
    wait_stages<kLoads, kSmallD>(min(depth - 1, nsteps - 1 - t));
    const int e = __builtin_amdgcn_readlane(elist, j);
    const bool on = (__ballot(my_e == e) >> r16) & 1;   // pair r16 routed to e
    uint4 bt[4], a[4];
    const uint32_t sb = ring_base + (uint32_t)(d * kStage);
    lds_read4(bt, sb + rd_b[0], sb + rd_b[1], sb + rd_b[2], sb + rd_b[3]);
    lds_read4(a, sb + rd_w[0], sb + rd_w[1], sb + rd_w[2], sb + rd_w[3]);
    const uint32_t off = (uint32_t)c * kChunk;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      if (!on || (c >= nfull && off + (4 * jj + g4) * 16 >= (uint32_t)row_bytes))
        bt[jj] = make_uint4(0, 0, 0, 0);
    acc = Tile<FMT>::mma(a, bt, acc);
    if (t + depth < nsteps) {
      issue(d, ic, ij);
      if (++ij == nexp) { ij = 0; ++ic; }
    }
    if (++j == nexp) { j = 0; ++c; }
    if (++d == depth) d = 0;
  }

  // ---- scaled contributions meet in LDS (each wave's own ring, idle now:
  // its last wait was for every load): red[pair][row] = (acc * scale) * w,
  // lane (g4, r16) holding rows 4 g4 + v of pair r16
  float* red = reinterpret_cast<float*>(ring);
  {
    float sc[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (ROWS) {
      sc[0] = col_ws4.x * col_as; sc[1] = col_ws4.y * col_as;
      sc[2] = col_ws4.z * col_as; sc[3] = col_ws4.w * col_as;
    } else if constexpr (FP8) {
      sc[0] = sc[1] = sc[2] = sc[3] = scale_from_amax_bits(amax_bits, fp8_max<FMT>()) * col_ws;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
      red[r16 * 16 + 4 * g4 + v] = col_ok ? (acc[v] * sc[v]) * col_w : 0.0f;
  }
  __syncthreads();

  // out[t][h] = bf16(sum over k, then over the waves), a fixed order
  const int T = p.P / p.K;
  for (int o = threadIdx.x; o < T * 16; o += blockDim.x) {
    const int tok = o >> 4;
    const int row = o & 15;
    float s = 0.0f;
    for (int k = 0; k < p.K; ++k) {
      const int pair = tok * p.K + k;
      for (int w = 0; w < nw; ++w)
        s += reinterpret_cast<const float*>(smem + (size_t)w * p.region)[pair * 16 + row];
    }
    p.out[(int64_t)tok * p.H + h0 + row] = (uint16_t)f32_to_bf16_bits(s);
  }
}

template <int FMT, int NB, bool ROWS>
hipError_t ready_small() {
  return prepare_kernel(reinterpret_cast<const void*>(&moe_down_small_kernel<FMT, NB, ROWS>),
                        kSmallLdsMax);
}

template <int FMT, bool ROWS>
void launch_small(const SmallDownArgs& a, int nb, int nw, hipStream_t stream) {
  const dim3 grid(a.H / 16), block(nw * kWave);
  const size_t lds = (size_t)nw * a.region;
  if (nb == 1) moe_down_small_kernel<FMT, 1, ROWS><<<grid, block, lds, stream>>>(a);
  else moe_down_small_kernel<FMT, 2, ROWS><<<grid, block, lds, stream>>>(a);
}

int stream_tiles(int P) { return P <= 4 ? 1 : 2; }

}  // namespace

// Waves per workgroup and ring depth: the shape whose workgroups all fit on
// the chip at once (one round) and keep the most weight bytes loading per
// compute unit (counted up to 128 KB; about 64 KB per unit already covers
// HBM3E's latency-bandwidth product), fewer waves on ties.  The steps per
// wave are counted for the fewest experts a call can have (K).
SmallDownPlan small_down_plan(int64_t P, int K, int H, int I, int welem, int num_cus) {
  SmallDownPlan best{};
  // up to 8 pairs: each stage's pair rows are then at most half its weight
  // bytes (measured with 16 pairs, bf16 T = 8: 469 us per step against 442
  // with the down product and combine launches -- the pair rows doubled each
  // stage's L2 reads)
  if (P < 1 || P > 8 || K < 1 || P % K != 0 || H % 16 != 0 || I % 16 != 0) return best;
  const int row_bytes = I * welem;
  const int nchunks = (row_bytes + kChunk - 1) / kChunk;
  const int stage = kTileBytes + stream_tiles((int)P) * 1024;
  const int groups = H / 16;
  const int cus = std::max(num_cus, 1);
  const int64_t steps_min = (int64_t)K * nchunks;
  double best_score = -1.0;
  for (int nw = 1; nw <= kSmallMaxWaves && nw <= steps_min; ++nw) {
    const int64_t steps_pw = steps_min / nw;
    for (int depth = 1; depth <= kSmallD && depth <= std::max<int64_t>(1, steps_pw); ++depth) {
      const int region = depth * stage;
      const int wg_lds = nw * region;
      if (wg_lds > kSmallLdsMax) continue;
      const int per_cu = std::min(kSmallLdsMax / wg_lds, kSmallMaxResidentWaves / nw);
      if (per_cu < 1) continue;
      const int rounds = (groups + cus * per_cu - 1) / (cus * per_cu);
      const double wgs = std::min<double>(per_cu, (double)groups / ((double)cus * rounds));
      const double inflight = std::min(wgs * nw * depth * kTileBytes, 128.0 * 1024);
      const double score = inflight / rounds;
      if (score > best_score * 1.0001) {
        best_score = score;
        best.waves = nw;
        best.region = region;
        best.depth = depth;
      }
    }
  }
  return best;
}

hipError_t launch_down_small(int fmt, const SmallDownPlan& plan, const uint8_t* w2,
                             int64_t w_expert_bytes, const void* b_rows, const int32_t* ids,
                             const float* wts, const float* w_scale, const uint32_t* act_amax,
                             const float* act_scale, int P, int K, int H, int I, void* out,
                             hipStream_t stream) {
  if (plan.waves < 1 || plan.waves > kSmallMaxWaves || plan.depth < 1 || plan.depth > kSmallD)
    return hipErrorInvalidValue;
  const bool fp8 = fmt != kFmtBF16;
  const bool rows = act_scale != nullptr;
  if (!b_rows || !ids || !wts || !out) return hipErrorInvalidValue;
  if (fp8 && (!w_scale || (!rows && !act_amax))) return hipErrorInvalidValue;
  SmallDownArgs a{};
  a.W = w2;
  a.w_expert_bytes = w_expert_bytes;
  a.row_bytes = I * (fp8 ? 1 : 2);
  a.B = static_cast<const uint8_t*>(b_rows);
  a.ids = ids;
  a.wts = wts;
  a.w_scale = w_scale;
  a.act_amax = act_amax;
  a.act_scale = act_scale;
  a.P = P;
  a.K = K;
  a.H = H;
  a.I = I;
  a.region = plan.region;
  a.depth = plan.depth;
  a.out = static_cast<uint16_t*>(out);
  const int nb = stream_tiles(P);
  const int nw = plan.waves;
  if (fmt == kFmtBF16) launch_small<kFmtBF16, false>(a, nb, nw, stream);
  else if (fmt == kFmtE4M3 && rows) launch_small<kFmtE4M3, true>(a, nb, nw, stream);
  else if (fmt == kFmtE4M3) launch_small<kFmtE4M3, false>(a, nb, nw, stream);
  else if (rows) launch_small<kFmtE5M2, true>(a, nb, nw, stream);
  else launch_small<kFmtE5M2, false>(a, nb, nw, stream);
  return hipGetLastError();
}

hipError_t prepare_down_small_kernels() {
  const hipError_t es[] = {
      ready_small<kFmtBF16, 1, false>(), ready_small<kFmtBF16, 2, false>(),
      ready_small<kFmtE4M3, 1, false>(), ready_small<kFmtE4M3, 2, false>(),
      ready_small<kFmtE4M3, 1, true>(),  ready_small<kFmtE4M3, 2, true>(),
      ready_small<kFmtE5M2, 1, false>(), ready_small<kFmtE5M2, 2, false>(),
      ready_small<kFmtE5M2, 1, true>(),  ready_small<kFmtE5M2, 2, true>()};
  for (hipError_t e : es)
    if (e != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace moe
