// Inverse rotary position embedding of attention heads fused with their
// per-head FP8 quantisation, for any token count.
//
// The pages name this kernel beside the MoE layer: it had been recompiled for
// every new number of tokens until its variable-length arguments stopped
// being specialised (toolboxkart.tech page, section 3; aib.vote page, fourth
// paragraph).  Here every size is a kernel argument of one ahead-of-time
// compiled kernel, so no token count, head count or head size compiles
// anything.
//
// What it computes, per token t and head h (D features, the first R rotated):
//   pairs (i, i + R/2) ("half" layout) or (2i, 2i + 1) ("interleaved"),
//   c = table[p][i], s = table[p][R/2 + i], p = positions[t]:
//     y1 = x1 * c + x2 * s,  y2 = x2 * c - x1 * s      (rotation by -theta)
//   features from R on pass through; then
//   scale[t][h] = amax|y| / max of the format (1 when 0),
//   codes = FP8(y / scale) (E4M3 or E5M2, nearest even, saturating).
// Each product and each sum rounds on its own in float32 (no fused
// multiply-add): the rotated value decides an integer code, so it is formed
// exactly as a float32 reference forms it.
//
// Layout of the work: one row (t, h) per group of G lanes, G the power of two
// >= D / 8; lane j of a group holds features 8j .. 8j + 7 (one 16-byte load
// of x, one 8-byte store of codes).  Half layout: the partner of feature f <
// R/2 is f + R/2, eight features in the lane R/16 further on (R % 16 == 0), so
// one shuffle of four words fetches all eight partners.  Interleaved: the
// partners are in the same lane (R % 8 == 0).  The row amax is a butterfly
// over the group.  HBM-bound: every byte of x is read once and every code
// written once; the table rows come from the caches.
#include "device_common.hpp"
#include "internal.hpp"

#pragma clang fp contract(off)

namespace moe {
namespace {

constexpr int kRopeThreads = 256;

struct RopeArgs {
  const uint4* x;            // bf16 rows, 8 per uint4
  int64_t x_stride8;         // token stride in uint4 units
  const int64_t* positions;
  const float* table;        // [max_pos][R]
  int64_t max_pos;
  int64_t rows;              // T * NH
  int NH, D, R;
  int gshift;                // log2 of the lanes per row
  uint2* codes;              // 8 codes per uint2
  float* scales;             // [T * NH]
};

__device__ __forceinline__ void unpack8(const uint4& q, float (&v)[8]) {
  v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
}

template <int FMT, bool INTERLEAVED>
__global__ __launch_bounds__(kRopeThreads) void inv_rope_quant_kernel(RopeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int G = 1 << a.gshift;
  const int j = lane & (G - 1);                       // lane inside the row group
  const int rows_per_block = kRopeThreads >> a.gshift;
  const int d8 = a.D >> 3;                            // lanes that hold features
  const bool holds = j < d8;
  const int f0 = 8 * j;                               // first feature of this lane
  const int half = a.R >> 1;
  for (int64_t row0 = (int64_t)blockIdx.x * rows_per_block; row0 < a.rows;
       row0 += (int64_t)gridDim.x * rows_per_block) {
    const int64_t row = row0 + (threadIdx.x >> a.gshift);
    const bool live = row < a.rows && holds;
    const int64_t t = row / a.NH;
    const int h = (int)(row - t * a.NH);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    uint4 q = make_uint4(0, 0, 0, 0);
    if (live) q = a.x[t * a.x_stride8 + (int64_t)h * d8 + j];
    // half layout: the partner lane's words (every lane takes part)
    uint4 pq = q;
    if constexpr (!INTERLEAVED) {
      const int off = a.R >> 4;                        // lanes between partners
      const int src = j < off ? lane + off : lane - off;
      const int srcl = (j < 2 * off) ? src : lane;
      pq.x = (uint32_t)__shfl((int)q.x, srcl);
      pq.y = (uint32_t)__shfl((int)q.y, srcl);
      pq.z = (uint32_t)__shfl((int)q.z, srcl);
      pq.w = (uint32_t)__shfl((int)q.w, srcl);
    }
    unpack8(q, v);
    if (live && f0 < a.R) {
      int64_t p = a.positions[t];
      p = p < 0 ? 0 : (p >= a.max_pos ? a.max_pos - 1 : p);
      const float* cs = a.table + p * a.R;
      if constexpr (INTERLEAVED) {
        // features f0 .. f0 + 7 are four pairs; angle index f / 2
        const float4 c4 = *reinterpret_cast<const float4*>(cs + (f0 >> 1));
        const float4 s4 = *reinterpret_cast<const float4*>(cs + half + (f0 >> 1));
        const float c[4] = {c4.x, c4.y, c4.z, c4.w}, s[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x1 = v[2 * i], x2 = v[2 * i + 1];
          v[2 * i] = (x1 * c[i]) + (x2 * s[i]);
          v[2 * i + 1] = (x2 * c[i]) - (x1 * s[i]);
        }
      } else {
        float w[8];
        unpack8(pq, w);
        const bool first = f0 < half;
        const int i0 = first ? f0 : f0 - half;         // angle index of feature 0
        const float4 ca = *reinterpret_cast<const float4*>(cs + i0);
        const float4 cb = *reinterpret_cast<const float4*>(cs + i0 + 4);
        const float4 sa = *reinterpret_cast<const float4*>(cs + half + i0);
        const float4 sb = *reinterpret_cast<const float4*>(cs + half + i0 + 4);
        const float c[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
        const float s[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float mine = v[i], other = w[i];
          v[i] = first ? (mine * c[i]) + (other * s[i])     // x1' = x1 c + x2 s
                       : (mine * c[i]) - (other * s[i]);    // x2' = x2 c - x1 s
        }
      }
    }
    // amax of the row over its group, scale, codes
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    for (int o = 1; o < G; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float sc = scale_from_amax_bits(__float_as_uint(m), fp8_max<FMT>());
    if (live) {
      uint2 o;
      o.x = fp8_pack4<FMT>(v[0], v[1], v[2], v[3], sc);
      o.y = fp8_pack4<FMT>(v[4], v[5], v[6], v[7], sc);
      a.codes[row * d8 + j] = o;
      if (j == 0) a.scales[row] = sc;
    }
  }
}

template <int FMT, bool IL>
const void* rope_fn() {
  return reinterpret_cast<const void*>(&inv_rope_quant_kernel<FMT, IL>);
}

}  // namespace

hipError_t prepare_rope_kernels() {
  const void* fns[] = {rope_fn<kFmtE4M3, false>(), rope_fn<kFmtE4M3, true>(),
                       rope_fn<kFmtE5M2, false>(), rope_fn<kFmtE5M2, true>()};
  for (const void* f : fns) {
    const hipError_t e = prepare_kernel(f, 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_inv_rope_quant(int fmt, bool interleaved, const void* x, int64_t x_stride,
                                 const int64_t* positions, const float* table, int64_t max_pos,
                                 int64_t T, int NH, int D, int R, uint8_t* codes, float* scales,
                                 int num_cus, hipStream_t stream) {
  RopeArgs a{};
  a.x = static_cast<const uint4*>(x);
  a.x_stride8 = x_stride / 8;
  a.positions = positions;
  a.table = table;
  a.max_pos = max_pos;
  a.rows = T * NH;
  a.NH = NH;
  a.D = D;
  a.R = R;
  int g = 0;
  while ((1 << g) < D / 8) ++g;
  a.gshift = g;
  a.codes = reinterpret_cast<uint2*>(codes);
  a.scales = scales;
  const int rows_per_block = kRopeThreads >> g;
  int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = (int64_t)num_cus * 16;
  if (blocks > cap) blocks = cap;
  const dim3 grid((unsigned)(blocks > 0 ? blocks : 1)), block(kRopeThreads);
  const bool e5 = fmt == kFmtE5M2;
  if (e5 && interleaved) inv_rope_quant_kernel<kFmtE5M2, true><<<grid, block, 0, stream>>>(a);
  else if (e5) inv_rope_quant_kernel<kFmtE5M2, false><<<grid, block, 0, stream>>>(a);
  else if (interleaved) inv_rope_quant_kernel<kFmtE4M3, true><<<grid, block, 0, stream>>>(a);
  else inv_rope_quant_kernel<kFmtE4M3, false><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace moe
