// a1 + a0 + a2 in one launch for small batches: routing, the E4M3 codes of x
// and the align layout.
//
// At decode sizes each of these steps is a few microseconds of work behind a
// kernel launch that costs about as much; the pages point at exactly this
// overhead around the expert GEMMs of a thin batch (toolboxkart.tech page,
// "Why MoE inference needs specialized kernels": routing, data movement and
// combining add work; aib.vote page, third paragraph: one GPU pass).
//  - Workgroup 0 (16 waves): wave t routes token t (route_token, at most 16
//    tokens) into LDS, then after a workgroup barrier wave 0 runs the align
//    step on those ids (align_wave, up to 64 pairs) or the whole workgroup
//    does (align_block).
//  - (FP8) Workgroups 1..n: each reduces the amax of all of x and writes the
//    codes FP8(x / s), s = amax / max (448 for E4M3, 57344 for E5M2), of its
//    own slice (the same arithmetic
//    as the two-kernel path, so the codes are identical); workgroup 1 stores
//    the final amax word for the GEMM epilogue and clears the slots of the
//    intermediate's amax.  With per-row scales workgroup 1 + t quantises
//    token row t on that row's own amax and stores its scale.
#include "align_device.hpp"
#include "internal.hpp"
#include "route_device.hpp"

namespace moe {
namespace {

constexpr int kFrontMaxT = 16;             // tokens: one wave each
constexpr int64_t kXMaxBytes = 256 << 10;   // x read whole by each quantising workgroup
constexpr int kXBatch = 8;                  // 16-byte loads in flight per thread
constexpr int64_t kXSlice = 2048;           // 16-byte pieces quantised per workgroup

struct FrontArgs {
  const float* logits;
  int T, E, K, renorm;
  int32_t* ids;
  float* wts;
  // FP8 only
  const uint4* x;            // [T][H] bfloat16, 8 per uint4
  int64_t n8;                // T * H / 8
  uint32_t* amax_x;          // amax block of x (final word written here)
  uint32_t* amax_a;          // amax block of a (slots cleared here)
  uint2* qx;                 // codes of x, 8 per uint2
  float* sx_rows;            // per-row scales of x [T], or nullptr for one scale
  // align
  AlignOut out;
  int32_t* rank;
  int ids_lds_offset;        // ints: the routed ids in LDS, after the align step's words
};

// Workgroup 0: routing and align.  Workgroups 1..: (FP8) each reduces the
// amax of all of x (a few hundred KB at most, from L2) and writes the codes
// of its own slice, so the divisions are spread over many compute units and
// need no exchange between workgroups.
template <int VPL, int FMT>
__global__ __launch_bounds__(kAlignThreads) void front_kernel(FrontArgs a) {
  constexpr bool FP8 = FMT != kFmtBF16;
  extern __shared__ int smem[];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);

  if constexpr (FP8) {
    if (blockIdx.x > 0 && a.sx_rows) {
      // per-row scales: workgroup b quantises token row b - 1 on its own amax
      const int64_t h8 = a.n8 / a.T;
      const int64_t base = (int64_t)(blockIdx.x - 1) * h8;
      float m = 0.0f;
      for (int64_t j = tid; j < h8; j += kAlignThreads) {
        const uint4 q = a.x[base + j];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(q.x)), fabsf(bf16_hi(q.x))),
                           fmaxf(fabsf(bf16_lo(q.y)), fabsf(bf16_hi(q.y)))));
        m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(q.z)), fabsf(bf16_hi(q.z))),
                           fmaxf(fabsf(bf16_lo(q.w)), fabsf(bf16_hi(q.w)))));
      }
      m = wave_max_dpp(m);
      float* wmax = reinterpret_cast<float*>(smem);
      if (lane == 0) wmax[wave] = m;
      __syncthreads();
      m = wave_max_dpp(wmax[lane & (kAlignWaves - 1)]);
      const float s = scale_from_amax_bits(__float_as_uint(m), fp8_max<FMT>());
      if (tid == 0) a.sx_rows[blockIdx.x - 1] = s;
      for (int64_t j = tid; j < h8; j += kAlignThreads) {
        const uint4 q = a.x[base + j];
        uint2 o;
        o.x = fp8_pack4<FMT>(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y), s);
        o.y = fp8_pack4<FMT>(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w), s);
        a.qx[base + j] = o;
      }
      return;
    }
    if (blockIdx.x > 0) {
      float m = 0.0f;
      for (int64_t base = 0; base < a.n8; base += kXBatch * kAlignThreads) {
        uint4 q[kXBatch];               // all loads of a batch before any use
#pragma unroll
        for (int i = 0; i < kXBatch; ++i) {
          const int64_t j = base + tid + (int64_t)i * kAlignThreads;
          q[i] = j < a.n8 ? a.x[j] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kXBatch; ++i) {
          m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(q[i].x)), fabsf(bf16_hi(q[i].x))),
                             fmaxf(fabsf(bf16_lo(q[i].y)), fabsf(bf16_hi(q[i].y)))));
          m = fmaxf(m, fmaxf(fmaxf(fabsf(bf16_lo(q[i].z)), fabsf(bf16_hi(q[i].z))),
                             fmaxf(fabsf(bf16_lo(q[i].w)), fabsf(bf16_hi(q[i].w)))));
        }
      }
      m = wave_max_dpp(m);
      float* wmax = reinterpret_cast<float*>(smem);
      if (lane == 0) wmax[wave] = m;
      __syncthreads();
      m = wave_max_dpp(wmax[lane & (kAlignWaves - 1)]);
      const float s = scale_from_amax_bits(__float_as_uint(m), fp8_max<FMT>());
      if (blockIdx.x == 1) {
        if (tid == 0) a.amax_x[kAmaxFinal] = __float_as_uint(m);
        if (tid < kAmaxSlots) a.amax_a[amax_zero_index(tid)] = 0u;
      }
      const int64_t per = (a.n8 + gridDim.x - 2) / (gridDim.x - 1);
      const int64_t j0 = (int64_t)(blockIdx.x - 1) * per;
      const int64_t j1 = j0 + per < a.n8 ? j0 + per : a.n8;
      for (int64_t j = j0 + tid; j < j1; j += kAlignThreads) {
        const uint4 q = a.x[j];
        uint2 o;
        o.x = fp8_pack4<FMT>(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y), s);
        o.y = fp8_pack4<FMT>(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w), s);
        a.qx[j] = o;
      }
      return;
    }
  }

  // The ids go to LDS (the align step reads them there) and from there to
  // their output.  Up to 64 pairs one wave aligns them with no barrier
  // (measured at T = 1: routing 4.1 us, the 16-wave align 2.9 us of a 7 us
  // launch); more take the workgroup's align.
  static_assert(kFrontMaxT <= kAlignWaves, "one wave per token");
  int* s_ids = smem + a.ids_lds_offset;
  if (wave < a.T)
    route_token<VPL>(a.logits + (int64_t)wave * a.E, a.E, a.K, a.renorm, s_ids + wave * a.K,
                     a.wts + (int64_t)wave * a.K);
  __syncthreads();              // ids visible to the workgroup
  const int P = a.T * a.K;
  if (tid < P) a.ids[tid] = s_ids[tid];
  if (P <= kWave) {
    if (wave == 0) align_wave(s_ids, P, a.E, a.out, smem);
  } else {
    align_block(s_ids, P, a.E, a.out, a.rank, smem);
  }
}

template <int FMT>
hipError_t launch_vpl(const FrontArgs& a, int vpl, size_t lds, hipStream_t stream) {
  constexpr bool FP8 = FMT != kFmtBF16;
  // FP8: one workgroup per kXSlice 16-byte pieces of x, or per token row
  // with per-row scales, after workgroup 0
  const unsigned nq = !FP8 ? 0u
                      : a.sx_rows ? (unsigned)a.T
                                  : (unsigned)((a.n8 + kXSlice - 1) / kXSlice);
  const dim3 grid(1 + (nq > 0 ? nq : (FP8 ? 1u : 0u))), block(kAlignThreads);
  if (vpl <= 1) front_kernel<1, FMT><<<grid, block, lds, stream>>>(a);
  else if (vpl <= 2) front_kernel<2, FMT><<<grid, block, lds, stream>>>(a);
  else if (vpl <= 4) front_kernel<4, FMT><<<grid, block, lds, stream>>>(a);
  else if (vpl <= 8) front_kernel<8, FMT><<<grid, block, lds, stream>>>(a);
  else front_kernel<16, FMT><<<grid, block, lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t prepare_front_kernels() {
#define MOE_FRONT_FNS(F)                                      \
  reinterpret_cast<const void*>(&front_kernel<1, F>),         \
      reinterpret_cast<const void*>(&front_kernel<2, F>),     \
      reinterpret_cast<const void*>(&front_kernel<4, F>),     \
      reinterpret_cast<const void*>(&front_kernel<8, F>),     \
      reinterpret_cast<const void*>(&front_kernel<16, F>)
  const void* fns[] = {MOE_FRONT_FNS(kFmtBF16), MOE_FRONT_FNS(kFmtE4M3), MOE_FRONT_FNS(kFmtE5M2)};
#undef MOE_FRONT_FNS
  for (const void* f : fns) {
    const hipError_t e = prepare_kernel(f, 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

bool front_fits(int64_t T, int H, int K, bool fp8) {
  // one wave per token, the pairs in one align chunk, and (FP8) x small
  // enough for every quantising workgroup to read all of it
  return T <= kFrontMaxT && T * K <= kAlignThreads &&
         (!fp8 || T * (int64_t)H * 2 <= kXMaxBytes);
}

hipError_t launch_front(const float* logits, int64_t T, int E, int K, int renorm, int32_t* ids,
                        float* wts, int fmt, const void* x, int H, uint32_t* amax_x,
                        uint32_t* amax_a, uint8_t* qx, float* sx_rows, int BM,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_pad,
                        int32_t* rank, hipStream_t stream) {
  FrontArgs a{};
  a.logits = logits;
  a.T = (int)T;
  a.E = E;
  a.K = K;
  a.renorm = renorm;
  a.ids = ids;
  a.wts = wts;
  a.x = static_cast<const uint4*>(x);
  a.n8 = T * (int64_t)H / 8;
  a.amax_x = amax_x;
  a.amax_a = amax_a;
  a.qx = reinterpret_cast<uint2*>(qx);
  a.sx_rows = sx_rows;
  a.out = AlignOut{sorted_ids, block_expert, num_post_pad, BM};
  a.rank = rank;
  const int vpl = (E + kWave - 1) / kWave;
  a.ids_lds_offset = (int)align_lds_words(E);
  size_t lds = (align_lds_words(E) + (size_t)T * K) * sizeof(int);
  if (lds < kAlignWaves * sizeof(float)) lds = kAlignWaves * sizeof(float);
  if (fmt == kFmtE4M3) return launch_vpl<kFmtE4M3>(a, vpl, lds, stream);
  if (fmt == kFmtE5M2) return launch_vpl<kFmtE5M2>(a, vpl, lds, stream);
  return launch_vpl<kFmtBF16>(a, vpl, lds, stream);
}

}  // namespace moe
