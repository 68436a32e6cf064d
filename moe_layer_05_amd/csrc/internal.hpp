// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kGateUp = 0;
constexpr int kDown = 1;

// Arguments of the grouped expert GEMMs (gate/up and down).
struct GemmParams {
  const uint8_t* W;            // expert weights [E][R][L] (bytes)
  int64_t w_expert_bytes;      // bytes of one expert's matrix
  int64_t row_bytes;           // bytes of one row of W and of B (L * elem)
  const uint8_t* B;            // activation rows (x / codes of x / a / codes of a)
  int b_row_div;               // B row of a pair: pair / b_row_div
  const int32_t* sorted_ids;   // aligned layout
  const int32_t* block_expert;
  const int32_t* num_post_pad;
  int BM;                      // tokens per block
  int P;                       // pairs (= sentinel)
  int groups;                  // row groups per block (one wave each)
  int splits;                  // parts of the reduction dimension
  const float* w_scale;        // [E] (FP8), [E][rows] with row_scales, or nullptr
  const uint32_t* act_amax;    // final amax bits of B's quantisation (FP8 per tensor) or nullptr
  // FP8 with one scale per weight row and per activation row: w_scale holds
  // one scale per output row of each expert (2I for gate/up, H for down) and
  // act_scale one per row of B; act_amax and a_amax are unused.
  int row_scales;
  const float* act_scale;      // [rows of B] float32, with row_scales
  // gate/up
  void* a_out;                 // [P][I] float32 (FP8 path) or bfloat16
  uint32_t* a_amax;            // amax block (slots) of a (FP8) or nullptr
  int I;
  // down
  void* dw;                    // [splits][P][H] scaled expert outputs, float32 or bfloat16
  int64_t dw_split_stride;     // elements between parts (P * H)
  int dw_bf16;                 // the partial rows are bfloat16 (prefill) instead of float32
  int H;
  // tiled products: 8 work counters (one per XCD's tile list), zero at launch
  uint32_t* tile_queue;
};

// Work decomposition of a decode GEMM launch (chosen on the host from the
// shape only): RA 16-row tiles per wave, row groups per block, k-splits.
struct DecodeShape {
  int ra, groups, splits;
};

// a1; zero_amax: n_amax consecutive amax blocks cleared by the launch.  With
// x set (n bfloat16 values, n % 8 == 0), kAmaxSlots more workgroups of the
// same launch store the amax of x into the slots of amax_x, one each (a0's
// first half: every slot is written, none needs clearing).
hipError_t launch_router(const float* logits, int64_t T, int E, int K, int renorm,
                         int32_t* ids, float* wts, uint32_t* zero_amax, int n_amax,
                         hipStream_t stream, const void* x = nullptr, int64_t n = 0,
                         uint32_t* amax_x = nullptr);

size_t align_lds_bytes(int E);
hipError_t launch_align(const int32_t* ids, int P, int E, int BM, int32_t* sorted_ids,
                        int32_t* block_expert, int32_t* num_post_pad, int32_t* rank,
                        hipStream_t stream);

// a2 and a0 in one launch: workgroup 0 aligns, the others write the FP8 codes
// of x [T][H] (fmt E4M3 or E5M2) with one scale per tensor, from the amax
// slots of amax_x (final word stored), or, with row_scales set, one scale per
// token row (written to row_scales).
hipError_t launch_align_quant(const int32_t* ids, int P, int E, int BM, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* num_post_pad, int32_t* rank,
                              int fmt, const void* x, int64_t T, int H, uint32_t* amax_x,
                              uint8_t* codes, float* row_scales, int num_cus,
                              hipStream_t stream);

// a1 + a0 + a2 by one workgroup for small batches (front_fits): routing,
// (FP8) the codes of x with the final amax word and the amax slots of a
// cleared -- or, when sx_rows is set, the codes of x with one scale per token
// row, written to sx_rows -- and the align layout with block size BM.
bool front_fits(int64_t T, int H, int K, bool fp8);
hipError_t launch_front(const float* logits, int64_t T, int E, int K, int renorm, int32_t* ids,
                        float* wts, int fmt, const void* x, int H, uint32_t* amax_x,
                        uint32_t* amax_a, uint8_t* qx, float* sx_rows, int BM,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_pad,
                        int32_t* rank, hipStream_t stream);

// Two layouts at once (prefill), by three multi-workgroup launches: experts
// with >= thr pairs in blocks of BM_big, the others in blocks of BM_small;
// scratch holds align_multi_workspace_bytes(P, E); the n_clear words at
// `clear` are zeroed by the same launches (the tiled products' counters).
size_t align_multi_workspace_bytes(int P, int E);
hipError_t launch_align_split_multi(const int32_t* ids, int P, int E, int BM_small,
                                    int32_t* sorted_small, int32_t* bexp_small,
                                    int32_t* npp_small, int BM_big, int32_t* sorted_big,
                                    int32_t* bexp_big, int32_t* npp_big, int thr, int32_t* rank,
                                    int32_t* scratch, uint32_t* clear, int n_clear,
                                    hipStream_t stream);

hipError_t launch_zero_amax(uint32_t* p, int nblocks, hipStream_t stream);
hipError_t launch_amax_bf16(const void* x, int64_t n, uint32_t* amax, int num_cus,
                            hipStream_t stream);
// fmt: kFmtE4M3 or kFmtE5M2 (device_common.hpp).
hipError_t launch_quant_bf16(int fmt, const void* x, int64_t n, uint32_t* amax, uint8_t* codes,
                             float* scale_out, int num_cus, hipStream_t stream);
// Per-row FP8: scales[r] = amax|row r| / max (1 when 0), codes = FP8(v /
// scales[r]); rows of C values (C % 8 == 0), bfloat16 or float32.
hipError_t launch_quant_rows(int fmt, const void* src, bool bf16, int64_t rows, int C,
                             uint8_t* codes, float* scales, int num_cus, hipStream_t stream);
hipError_t launch_quant_f32(int fmt, const float* a, int64_t n, uint32_t* amax, uint8_t* codes,
                            int num_cus, hipStream_t stream);

// Resolve a kernel in the runtime ahead of its first launch (with the dynamic
// LDS limit it needs when lds > 0): the first launch of a kernel otherwise
// pays the runtime's lookup, which a first call at a new token count would
// show.  Each file prepares every kernel it may launch; the entry points run
// all of it once per device before their first launch there, which also sets
// the LDS limits the GEMM launches rely on.
inline hipError_t prepare_kernel(const void* fn, int lds) {
  if (lds > 0) return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  hipFuncAttributes attr;
  return hipFuncGetAttributes(&attr, fn);
}
hipError_t prepare_decode_kernels();
hipError_t prepare_tile_kernels();
hipError_t prepare_router_kernels();
hipError_t prepare_align_kernels();
hipError_t prepare_front_kernels();
hipError_t prepare_quant_kernels();
hipError_t prepare_combine_kernels();
hipError_t prepare_rope_kernels();

// Inverse rotary embedding of [T][NH][D] bfloat16 heads (token stride x_stride
// elements) with the cos/sin table [max_pos][R], then one FP8 scale per
// (token, head): codes [T][NH][D], scales [T][NH].
hipError_t launch_inv_rope_quant(int fmt, bool interleaved, const void* x, int64_t x_stride,
                                 const int64_t* positions, const float* table, int64_t max_pos,
                                 int64_t T, int NH, int D, int R, uint8_t* codes, float* scales,
                                 int num_cus, hipStream_t stream);

// The shape is chosen for num_cus compute units (the current device's);
// nblk_cap is the layout's block capacity, est_blocks the blocks a call
// is expected to route (one per active expert).
DecodeShape decode_shape(int mode, int64_t nblk_cap, int64_t est_blocks, int rows,
                         int64_t row_bytes, int bm, int num_cus);
// The most parts any shape choice splits the down product's reduction into,
// whatever the device (bounds the workspace of the partial rows).
int decode_max_splits(int64_t est_blocks, int rows, int64_t row_bytes, int bm);
hipError_t launch_gemm_decode(int mode, int fmt, const GemmParams& p, int ra, int64_t nblk_cap,
                              int num_cus, hipStream_t stream);

// Tiled products for large token blocks (BM = tile_block_m()); groups are
// the column tiles per block.
int tile_block_m();
int tile_groups(int mode, int rows);
hipError_t launch_gemm_tile(int mode, int fmt, const GemmParams& p, int64_t nblk_cap,
                            int num_cus, hipStream_t stream);

// Down product + combine in one launch for calls of at most 8 pairs
// (down_small.hip); waves == 0 when the call does not fit (then the down
// product and the combine launches run).  b_rows: bfloat16 a, or the FP8
// codes of a with act_amax (the final amax word, per tensor) or act_scale
// (one scale per pair row).
struct SmallDownPlan {
  int waves, region, depth;
};
SmallDownPlan small_down_plan(int64_t P, int K, int H, int I, int welem, int num_cus);
hipError_t launch_down_small(int fmt, const SmallDownPlan& plan, const uint8_t* w2,
                             int64_t w_expert_bytes, const void* b_rows, const int32_t* ids,
                             const float* wts, const float* w_scale, const uint32_t* act_amax,
                             const float* act_scale, int P, int K, int H, int I, void* out,
                             hipStream_t stream);
hipError_t prepare_down_small_kernels();

// out[t] = bf16(sum over k, then parts, of w[t*K+k] * dw[part][t*K+k]); dw
// float32, or bfloat16 when dw_bf16
hipError_t launch_combine(const void* dw, bool dw_bf16, const float* w, int splits, int64_t T,
                          int K, int H, void* out, int num_cus, hipStream_t stream);

}  // namespace moe
