// C ABI of the fused MoE layer (declared in include/moe.h): host-side argument
// checks, workspace layout and the launch sequence.  No device memory is
// allocated and nothing synchronises the host.
#include <algorithm>
#include <mutex>
#include <vector>

#include "moe.h"
#include "device_common.hpp"
#include "internal.hpp"

namespace moe {
namespace {

constexpr size_t kAlignBytes = 256;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;

size_t round_up(size_t x) { return (x + kAlignBytes - 1) / kAlignBytes * kAlignBytes; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device state, filled once per device id (any id the runtime reports):
// every kernel of the library resolved (so no later call, at whatever token
// count, pays a kernel's first lookup) and the compute-unit count.
struct DeviceState {
  bool prepared = false;
  int cus = 0;
  void* scratch = nullptr;        // this device's copy of `scratch` (device address)
};
std::mutex g_dev_mu;
std::vector<DeviceState> g_dev;   // indexed by device id; guarded by g_dev_mu

DeviceState& device_state(int dev) {
  if ((size_t)dev >= g_dev.size()) g_dev.resize((size_t)dev + 1);
  return g_dev[(size_t)dev];
}

// Workspace of moe_fused_forward_noalloc: one copy per device, held until the
// process ends.  In host code this name is a stand-in, not a device address;
// the address of the current device's copy comes from hipGetSymbolAddress
// (kept in DeviceState::scratch) and is the only form host code passes on.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Resolves every kernel on the current device once, and the address of its
// scratch copy; returns the first error.
hipError_t prepare_all() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceState& st = device_state(dev);
  if (st.prepared) return hipSuccess;
  e = prepare_decode_kernels();
  if (e == hipSuccess) e = prepare_tile_kernels();
  if (e == hipSuccess) e = prepare_router_kernels();
  if (e == hipSuccess) e = prepare_align_kernels();
  if (e == hipSuccess) e = prepare_front_kernels();
  if (e == hipSuccess) e = prepare_quant_kernels();
  if (e == hipSuccess) e = prepare_down_small_kernels();
  if (e == hipSuccess) e = prepare_combine_kernels();
  if (e == hipSuccess) e = prepare_rope_kernels();
  if (e == hipSuccess) e = hipGetSymbolAddress(&st.scratch, HIP_SYMBOL(scratch));
  if (e == hipSuccess && st.scratch == nullptr) e = hipErrorInvalidSymbol;
  if (e == hipSuccess) st.prepared = true;
  return e;
}

// The current device's scratch address (prepare_all has run on it), or null.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  const DeviceState& st = device_state(dev);
  return st.prepared ? st.scratch : nullptr;
}

// Compute-unit count of the current device (256, MI355X's, when no device
// can be queried: the host-only size queries then still answer).
int num_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceState& st = device_state(dev);
  if (st.cus == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    st.cus = n;
  }
  return st.cus;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool block_m_ok(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

// Upper bound of the number of blocks of the aligned layout: each active
// expert adds at most one partly filled block, and at most min(E, P) experts
// are active.
int64_t max_blocks(int64_t P, int E, int bm) {
  const int64_t active = P < E ? P : E;
  return P / bm + active;
}

// Experts with at least this many pairs take the tiled products when the
// call is large enough to have such experts (prefill); the rest keep the
// weight-streaming kernels.
constexpr int kTileThreshold = 16;

// Largest x (bytes) whose amax the router launch reduces itself (kAmaxSlots
// workgroups); measured: 512 KB (T = 64, H = 4096) saves a launch, 58.7 MB
// (T = 4096, H = 7168) is slower than the many-workgroup amax launch.
constexpr int64_t kRouterAmaxMaxBytes = 8 << 20;

struct FusedLayout {
  size_t ids, wts, sorted, bexp, npp, rank, scal, srow, qx, a, qa, dw, ascr, total;
  size_t sorted_t, bexp_t, npp_t;     // tiled layout (prefill)
  size_t tq;                          // tile counters of the two tiled products (2 x 8)
  int bm;
  int64_t cap, nblk;
  bool tiled;
  int64_t cap_t, nblk_t;
  DecodeShape gu, dn;
};

bool is_fp8(moe_wdtype wd) { return wd == MOE_FP8_E4M3 || wd == MOE_FP8_E5M2; }
bool wdtype_ok(moe_wdtype wd) { return wd == MOE_BF16 || is_fp8(wd); }
// Operand format of the kernels for a weight type.
int fmt_of(moe_wdtype wd) {
  return wd == MOE_FP8_E5M2 ? kFmtE5M2 : wd == MOE_FP8_E4M3 ? kFmtE4M3 : kFmtBF16;
}

bool rows_mode(const moe_fused_args* a) {
  return is_fp8(a->wdtype) && a->fp8_scales == MOE_SCALES_ROW;
}

bool use_tiles(int64_t T, int E, int K) {
  return T >= 256 && T * (int64_t)K >= 32LL * E;
}

// Workspace layout of a call; the kernel shapes are chosen for `cus` compute
// units, the sizes do not depend on it.
FusedLayout fused_layout(int64_t T, int H, int I, int E, int K, moe_wdtype wd, bool rows,
                         int cus) {
  FusedLayout L{};
  const int64_t P = T * K;
  const bool fp8 = is_fp8(wd);
  rows = rows && fp8;
  const int welem = fp8 ? 1 : 2;
  L.tiled = use_tiles(T, E, K);
  L.bm = L.tiled ? kTileThreshold : moe_fused_block_m(T, H, I, E, K, wd);
  // In the split layout every small expert has fewer than kTileThreshold =
  // BM pairs, so it takes exactly one block.
  L.nblk = L.tiled ? std::min<int64_t>(E, P) : max_blocks(P, E, L.bm);
  L.cap = L.nblk * L.bm;
  if (L.tiled) {
    const int bmt = tile_block_m();
    const int64_t big_experts = std::min<int64_t>(E, P / kTileThreshold);
    L.nblk_t = P / bmt + big_experts;
    L.cap_t = L.nblk_t * bmt;
  }
  const int64_t est = std::min<int64_t>(E, P);   // one block per active expert
  L.gu = decode_shape(kGateUp, L.nblk, est, I, (int64_t)H * welem, L.bm, cus);
  L.dn = decode_shape(kDown, L.nblk, est, H, (int64_t)I * welem, L.bm, cus);
  if (L.tiled) L.dn.splits = 1;          // the tiled products write one part
  const int dw_parts = L.tiled ? 1 : decode_max_splits(est, H, (int64_t)I * welem, L.bm);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += round_up(bytes); return o; };
  L.ids = take(P * 4);
  L.wts = take(P * 4);
  L.sorted = take(L.cap * 4);
  L.bexp = take(L.nblk * 4);
  L.npp = take(4);
  L.sorted_t = take(L.tiled ? L.cap_t * 4 : 0);
  L.bexp_t = take(L.tiled ? L.nblk_t * 4 : 0);
  L.npp_t = take(4);
  L.tq = take(L.tiled ? 16 * 4 : 0);
  L.rank = take(P * 4);
  L.ascr = take(L.tiled ? align_multi_workspace_bytes((int)P, E) : 0);
  L.scal = take(2 * kAmaxWords * 4);     // amax blocks of x and of a
  L.srow = take(rows ? (size_t)(T + P) * 4 : 0);   // per-row scales of x and of a
  L.qx = take(fp8 ? (size_t)T * H : 0);
  L.a = take((size_t)P * I * (fp8 ? 4 : 2));
  L.qa = take(fp8 ? (size_t)P * I : 0);
  L.dw = take((size_t)dw_parts * P * H * (L.tiled ? 2 : 4));   // bfloat16 at prefill
  L.total = off;
  return L;
}

moe_status check_shape(int64_t T, int H, int I, int E, int K) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0) return MOE_ERR_SHAPE;
  if (K > E) return MOE_ERR_SHAPE;
  if (E > kMaxE || K > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (H % 16 != 0 || I % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)K >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is negative or inconsistent";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the supported range";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP call failed";
  }
  return "unknown moe_status";
}

moe_status moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t K,
                          int32_t renormalize, int32_t* topk_ids, float* topk_weights,
                          hipStream_t stream) {
  if (T < 0 || E <= 0 || K <= 0) return MOE_ERR_SHAPE;
  if (K > E) return MOE_ERR_SHAPE;
  if (E > kMaxE || K > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  if (prepare_all() != hipSuccess) return MOE_ERR_HIP;
  return hip_status(
      launch_router(logits, T, E, K, renormalize, topk_ids, topk_weights, nullptr, 0, stream));
}

size_t moe_align_capacity(int64_t T, int32_t K, int32_t E, int32_t block_m) {
  if (T < 0 || K <= 0 || E <= 0 || !block_m_ok(block_m)) return 0;
  return (size_t)(max_blocks(T * K, E, block_m) * block_m);
}

size_t moe_align_workspace_bytes(int64_t T, int32_t K, int32_t E, int32_t block_m) {
  if (T < 0 || K <= 0 || E <= 0 || !block_m_ok(block_m)) return 0;
  return round_up((size_t)(T * K) * 4);
}

moe_status moe_align(const int32_t* topk_ids, int64_t T, int32_t K, int32_t E, int32_t block_m,
                     int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_pad,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (T < 0 || E <= 0 || K <= 0) return MOE_ERR_SHAPE;
  if (K > E) return MOE_ERR_SHAPE;
  if (E > kMaxE || !block_m_ok(block_m)) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)K >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (!num_post_pad) return MOE_ERR_NULL;
  if (T > 0 && (!topk_ids || !sorted_ids || !block_expert || !workspace)) return MOE_ERR_NULL;
  if (workspace_bytes < moe_align_workspace_bytes(T, K, E, block_m)) return MOE_ERR_WORKSPACE;
  if (T == 0) return MOE_OK;
  if (prepare_all() != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_align(topk_ids, (int)(T * K), E, block_m, sorted_ids, block_expert,
                                 num_post_pad, static_cast<int32_t*>(workspace), stream));
}

size_t moe_act_quant_workspace_bytes(void) { return round_up(kAmaxWords * 4); }

moe_status moe_act_quant_fp8(const void* x, int64_t n, uint8_t* codes, float* scale,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (n < 0) return MOE_ERR_SHAPE;
  if (n % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (!scale || !workspace) return MOE_ERR_NULL;
  if (n > 0 && (!x || !codes)) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(workspace)) return MOE_ERR_UNSUPPORTED;
  if (workspace_bytes < moe_act_quant_workspace_bytes()) return MOE_ERR_WORKSPACE;
  if (prepare_all() != hipSuccess) return MOE_ERR_HIP;
  uint32_t* amax = static_cast<uint32_t*>(workspace);
  const int cus = num_cus();
  hipError_t e = launch_zero_amax(amax, 1, stream);
  if (e == hipSuccess && n > 0) e = launch_amax_bf16(x, n, amax, cus, stream);
  if (e == hipSuccess) e = launch_quant_bf16(kFmtE4M3, x, n, amax, codes, scale, cus, stream);
  return hip_status(e);
}

moe_status moe_act_quant_fp8_rows(const void* x, int64_t rows, int32_t cols, moe_wdtype fmt,
                                  uint8_t* codes, float* scales, hipStream_t stream) {
  if (rows < 0 || cols < 0) return MOE_ERR_SHAPE;
  if (!is_fp8(fmt)) return MOE_ERR_UNSUPPORTED;
  if (cols % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes)) return MOE_ERR_UNSUPPORTED;
  if (prepare_all() != hipSuccess) return MOE_ERR_HIP;
  return hip_status(
      launch_quant_rows(fmt_of(fmt), x, true, rows, cols, codes, scales, num_cus(), stream));
}

int32_t moe_fused_block_m(int64_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                          moe_wdtype wdtype) {
  (void)H; (void)I; (void)wdtype;
  // One block per active expert whenever an expert can hold all its tokens,
  // so each expert's weights stream from HBM once.  An expert receives at
  // most T pairs; with many experts it receives about T*K/E, so the block is
  // sized for a few times that mean (blocks up to 64 tokens).
  if (T <= 16) return 16;
  const int64_t mean = (E > 0) ? (T * (int64_t)K + E - 1) / E : T;
  if (mean <= 8) return 16;
  if (T <= 32 || mean <= 16) return 32;
  return 64;
}

size_t moe_fused_workspace_bytes(const moe_fused_args* a) {
  if (!a) return 0;
  if (check_shape(a->T, a->H, a->I, a->E, a->K) != MOE_OK) return 0;
  if (!wdtype_ok(a->wdtype)) return 0;
  if (is_fp8(a->wdtype) && a->fp8_scales != MOE_SCALES_TENSOR &&
      a->fp8_scales != MOE_SCALES_ROW)
    return 0;
  return fused_layout(a->T, a->H, a->I, a->E, a->K, a->wdtype, rows_mode(a), 256).total;
}

moe_status moe_fused_workspace_layout(const moe_fused_args* a, moe_fused_layout* out) {
  if (!a || !out) return MOE_ERR_NULL;
  moe_status st = check_shape(a->T, a->H, a->I, a->E, a->K);
  if (st != MOE_OK) return st;
  if (!wdtype_ok(a->wdtype)) return MOE_ERR_UNSUPPORTED;
  const bool fp8 = is_fp8(a->wdtype);
  if (fp8 && a->fp8_scales != MOE_SCALES_TENSOR && a->fp8_scales != MOE_SCALES_ROW)
    return MOE_ERR_UNSUPPORTED;
  const bool rows = rows_mode(a);
  const FusedLayout L = fused_layout(a->T, a->H, a->I, a->E, a->K, a->wdtype, rows, 256);
  const size_t none = MOE_NO_SECTION;
  moe_fused_layout o{};
  o.total = L.total;
  o.block_m = L.bm;
  o.tiled = L.tiled ? 1 : 0;
  o.tile_block_m = L.tiled ? tile_block_m() : 0;
  o.tile_threshold = L.tiled ? kTileThreshold : 0;
  o.capacity = L.cap;
  o.tile_capacity = L.tiled ? L.cap_t : 0;
  o.topk_ids = L.ids;
  o.topk_weights = L.wts;
  o.sorted_ids = L.sorted;
  o.block_expert = L.bexp;
  o.num_post_pad = L.npp;
  o.tile_sorted_ids = L.tiled ? L.sorted_t : none;
  o.tile_block_expert = L.tiled ? L.bexp_t : none;
  o.tile_num_post_pad = L.tiled ? L.npp_t : none;
  const bool tensor_fp8 = fp8 && !rows;
  o.x_amax = tensor_fp8 ? L.scal + (size_t)kAmaxFinal * 4 : none;
  o.x_codes = fp8 ? L.qx : none;
  o.x_scales = rows ? L.srow : none;
  o.a = L.a;
  o.a_amax = tensor_fp8 ? L.scal + (size_t)(kAmaxWords + kAmaxFinal) * 4 : none;
  o.a_codes = fp8 ? L.qa : none;
  o.a_scales = rows ? L.srow + (size_t)a->T * 4 : none;
  *out = o;
  return MOE_OK;
}

}  // extern "C"

namespace {

// Records events[s] on the stream when the array and its entry s are set.
hipError_t mark(hipEvent_t* events, int s, hipStream_t stream) {
  return (events && events[s]) ? hipEventRecord(events[s], stream) : hipSuccess;
}

// Host-only checks of a fused call (no HIP call); the workspace pointer is
// checked only when `with_workspace`.  T == 0 passes once the shape is valid.
moe_status check_fused(const moe_fused_args* a, bool with_workspace) {
  if (!a) return MOE_ERR_NULL;
  moe_status st = check_shape(a->T, a->H, a->I, a->E, a->K);
  if (st != MOE_OK) return st;
  if (!wdtype_ok(a->wdtype)) return MOE_ERR_UNSUPPORTED;
  const bool fp8 = is_fp8(a->wdtype);
  if (fp8 && a->fp8_scales != MOE_SCALES_TENSOR && a->fp8_scales != MOE_SCALES_ROW)
    return MOE_ERR_UNSUPPORTED;
  if (a->T == 0) return MOE_OK;
  const bool rows = rows_mode(a);
  if (!a->x || !a->router_logits || !a->w13 || !a->w2 || !a->out) return MOE_ERR_NULL;
  if (with_workspace && !a->workspace) return MOE_ERR_NULL;
  if (fp8 && (!a->w13_scale || !a->w2_scale)) return MOE_ERR_NULL;
  if (rows && (!aligned16(a->w13_scale) || !aligned16(a->w2_scale))) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(a->x) || !aligned16(a->w13) || !aligned16(a->w2) || !aligned16(a->out))
    return MOE_ERR_UNSUPPORTED;
  if (with_workspace && !aligned16(a->workspace)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status fused_forward_impl(const moe_fused_args* a, hipStream_t stream, hipEvent_t* ev) {
  moe_status st = check_fused(a, true);
  if (st != MOE_OK || a->T == 0) return st;
  const bool fp8 = is_fp8(a->wdtype);
  const int fmt = fmt_of(a->wdtype);
  const bool rows = rows_mode(a);
  const int64_t T = a->T;
  const int H = a->H, I = a->I, E = a->E, K = a->K;
  const int cus = num_cus();
  const FusedLayout L = fused_layout(T, H, I, E, K, a->wdtype, rows, cus);
  if (a->workspace_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (prepare_all() != hipSuccess) return MOE_ERR_HIP;

  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  int32_t* ids = a->topk_ids_out ? a->topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* wts = a->topk_weights_out ? a->topk_weights_out : reinterpret_cast<float*>(ws + L.wts);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
  int32_t* bexp = reinterpret_cast<int32_t*>(ws + L.bexp);
  int32_t* npp = reinterpret_cast<int32_t*>(ws + L.npp);
  int32_t* rank = reinterpret_cast<int32_t*>(ws + L.rank);
  uint32_t* amax_x = reinterpret_cast<uint32_t*>(ws + L.scal);   // amax blocks
  uint32_t* amax_a = amax_x + kAmaxWords;
  float* sx = reinterpret_cast<float*>(ws + L.srow);             // [T] (per-row scales)
  float* sa = sx + T;                                             // [P]
  uint8_t* qx = ws + L.qx;
  void* abuf = ws + L.a;
  uint8_t* qa = ws + L.qa;
  void* dw = ws + L.dw;
  const int P = (int)(T * K);
  const int welem = fp8 ? 1 : 2;

  int32_t* sorted_t = reinterpret_cast<int32_t*>(ws + L.sorted_t);
  int32_t* bexp_t = reinterpret_cast<int32_t*>(ws + L.bexp_t);
  int32_t* npp_t = reinterpret_cast<int32_t*>(ws + L.npp_t);
  hipError_t e = mark(ev, MOE_STAGE_ROUTE, stream);
  if (!L.tiled && front_fits(T, H, K, fp8)) {
    // a1 + a0 + a2 in one launch; the act-quant and align stages are empty
    if (e == hipSuccess)
      e = launch_front(a->router_logits, T, E, K, a->renormalize, ids, wts, fmt, a->x, H, amax_x,
                       amax_a, qx, rows ? sx : nullptr, L.bm, sorted, bexp, npp, rank, stream);
    if (e == hipSuccess) e = mark(ev, MOE_STAGE_ACT_QUANT, stream);
    if (e == hipSuccess) e = mark(ev, MOE_STAGE_ALIGN, stream);
  } else {
    // a1.  Per-tensor FP8 with a small x: the same launch clears the amax
    // slots of a and stores the amax of x in the slots of x (a0's first
    // half, one launch less).  A large x (prefill) needs more workgroups than
    // that launch adds: the router clears both amax blocks and a launch of
    // its own reduces x.
    const bool tensor_fp8 = fp8 && !rows;
    const bool amax_in_router = tensor_fp8 && T * (int64_t)H * 2 <= kRouterAmaxMaxBytes;
    if (e == hipSuccess) {
      if (amax_in_router)
        e = launch_router(a->router_logits, T, E, K, a->renormalize, ids, wts, amax_a, 1,
                          stream, a->x, T * H, amax_x);
      else
        e = launch_router(a->router_logits, T, E, K, a->renormalize, ids, wts, amax_x,
                          tensor_fp8 ? 2 : 0, stream);
    }
    // a0.  Without tiles (decode batches) the align launch also writes the
    // codes of x -- from the router's amax slots, or per token row -- so the
    // act-quant stage is empty; a large x has its amax reduced first by a
    // launch of its own.
    if (e == hipSuccess) e = mark(ev, MOE_STAGE_ACT_QUANT, stream);
    const bool quant_in_align = fp8 && !L.tiled;
    if (fp8 && !rows && !amax_in_router && e == hipSuccess)
      e = launch_amax_bf16(a->x, T * H, amax_x, cus, stream);
    if (fp8 && L.tiled && e == hipSuccess) {
      e = rows ? launch_quant_rows(fmt, a->x, true, T, H, qx, sx, cus, stream)
               : launch_quant_bf16(fmt, a->x, T * H, amax_x, qx, nullptr, cus, stream);
    }
    // a2
    if (e == hipSuccess) e = mark(ev, MOE_STAGE_ALIGN, stream);
    if (e == hipSuccess) {
      if (L.tiled)
        e = launch_align_split_multi(ids, P, E, L.bm, sorted, bexp, npp, tile_block_m(),
                                     sorted_t, bexp_t, npp_t, kTileThreshold, rank,
                                     reinterpret_cast<int32_t*>(ws + L.ascr),
                                     reinterpret_cast<uint32_t*>(ws + L.tq), 16, stream);
      else if (quant_in_align)
        e = launch_align_quant(ids, P, E, L.bm, sorted, bexp, npp, rank, fmt, a->x, T, H, amax_x,
                               qx, rows ? sx : nullptr, cus, stream);
      else
        e = launch_align(ids, P, E, L.bm, sorted, bexp, npp, rank, stream);
    }
  }

  // a3 + a4
  GemmParams g{};
  g.sorted_ids = sorted;
  g.block_expert = bexp;
  g.num_post_pad = npp;
  g.BM = L.bm;
  g.P = P;
  g.I = I;
  g.H = H;
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_GATE_UP, stream);
  if (e == hipSuccess) {
    g.W = static_cast<const uint8_t*>(a->w13);
    g.w_expert_bytes = (int64_t)2 * I * H * welem;
    g.row_bytes = (int64_t)H * welem;
    g.B = fp8 ? qx : static_cast<const uint8_t*>(a->x);
    g.b_row_div = K;
    g.groups = L.gu.groups;
    g.splits = L.gu.splits;
    g.w_scale = fp8 ? a->w13_scale : nullptr;
    g.row_scales = rows ? 1 : 0;
    g.act_amax = fp8 && !rows ? amax_x + kAmaxFinal : nullptr;
    g.act_scale = rows ? sx : nullptr;
    g.a_out = abuf;
    g.a_amax = fp8 && !rows ? amax_a : nullptr;
    e = launch_gemm_decode(kGateUp, fmt, g, L.gu.ra, L.nblk, cus, stream);
    if (e == hipSuccess && L.tiled) {
      GemmParams t = g;
      t.sorted_ids = sorted_t;
      t.block_expert = bexp_t;
      t.num_post_pad = npp_t;
      t.BM = tile_block_m();
      t.tile_queue = reinterpret_cast<uint32_t*>(ws + L.tq);
      t.groups = tile_groups(kGateUp, I);
      t.splits = 1;
      e = launch_gemm_tile(kGateUp, fmt, t, L.nblk_t, cus, stream);
    }
  }
  // intermediate quantisation (FP8)
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_INTER_QUANT, stream);
  if (e == hipSuccess && rows)
    e = launch_quant_rows(fmt, abuf, false, P, I, qa, sa, cus, stream);
  else if (e == hipSuccess && fp8)
    e = launch_quant_f32(fmt, static_cast<const float*>(abuf), (int64_t)P * I, amax_a, qa, cus,
                         stream);
  // At most 8 pairs: the down product and the combine in one launch.
  const SmallDownPlan small = L.tiled ? SmallDownPlan{} : small_down_plan(P, K, H, I, welem, cus);
  if (small.waves > 0) {
    if (e == hipSuccess) e = mark(ev, MOE_STAGE_DOWN, stream);
    if (e == hipSuccess)
      e = launch_down_small(fmt, small, static_cast<const uint8_t*>(a->w2), (int64_t)H * I * welem,
                            fp8 ? static_cast<const void*>(qa) : abuf, ids, wts,
                            fp8 ? a->w2_scale : nullptr, fp8 && !rows ? amax_a + kAmaxFinal : nullptr,
                            rows ? sa : nullptr, P, K, H, I, a->out, stream);
    if (e == hipSuccess) e = mark(ev, MOE_STAGE_COMBINE, stream);
    if (e == hipSuccess) e = mark(ev, MOE_STAGE_COUNT, stream);
    return hip_status(e);
  }
  // a5
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_DOWN, stream);
  if (e == hipSuccess) {
    g.W = static_cast<const uint8_t*>(a->w2);
    g.w_expert_bytes = (int64_t)H * I * welem;
    g.row_bytes = (int64_t)I * welem;
    g.B = fp8 ? qa : static_cast<const uint8_t*>(abuf);
    g.b_row_div = 1;
    g.groups = L.dn.groups;
    g.splits = L.dn.splits;
    g.w_scale = fp8 ? a->w2_scale : nullptr;
    g.act_amax = fp8 && !rows ? amax_a + kAmaxFinal : nullptr;
    g.act_scale = rows ? sa : nullptr;
    g.dw = dw;
    g.dw_split_stride = (int64_t)P * H;
    g.dw_bf16 = L.tiled ? 1 : 0;
    e = launch_gemm_decode(kDown, fmt, g, L.dn.ra, L.nblk, cus, stream);
    if (e == hipSuccess && L.tiled) {
      GemmParams t = g;
      t.sorted_ids = sorted_t;
      t.block_expert = bexp_t;
      t.num_post_pad = npp_t;
      t.BM = tile_block_m();
      t.tile_queue = reinterpret_cast<uint32_t*>(ws + L.tq) + 8;
      t.groups = tile_groups(kDown, H);
      t.splits = 1;
      e = launch_gemm_tile(kDown, fmt, t, L.nblk_t, cus, stream);
    }
  }
  // a6
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_COMBINE, stream);
  if (e == hipSuccess)
    e = launch_combine(dw, L.tiled, wts, L.dn.splits, T, K, H, a->out, cus, stream);
  if (e == hipSuccess) e = mark(ev, MOE_STAGE_COUNT, stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

moe_status moe_fused_forward(const moe_fused_args* a, hipStream_t stream) {
  return fused_forward_impl(a, stream, nullptr);
}

moe_status moe_fused_forward_timed(const moe_fused_args* a, hipStream_t stream,
                                   hipEvent_t* events) {
  if (!events) return MOE_ERR_NULL;
  return fused_forward_impl(a, stream, events);
}

moe_status moe_inv_rope_fp8_quant_per_head(const void* x, int64_t x_token_stride,
                                           const int64_t* positions, const float* cos_sin,
                                           int64_t max_pos, int64_t T, int32_t NH, int32_t D,
                                           int32_t R, int32_t interleaved, moe_wdtype fmt,
                                           uint8_t* codes, float* scales, hipStream_t stream) {
  if (T < 0 || NH <= 0 || D <= 0 || R <= 0 || max_pos <= 0) return MOE_ERR_SHAPE;
  if (R > D || (R & 1)) return MOE_ERR_SHAPE;
  if (!is_fp8(fmt)) return MOE_ERR_UNSUPPORTED;
  if (D % 8 != 0 || D > 512) return MOE_ERR_UNSUPPORTED;
  if (interleaved ? (R % 8 != 0) : (R % 16 != 0)) return MOE_ERR_UNSUPPORTED;
  if (x_token_stride < (int64_t)NH * D || x_token_stride % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)NH >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !positions || !cos_sin || !codes || !scales) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(cos_sin)) return MOE_ERR_UNSUPPORTED;
  if (prepare_all() != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_inv_rope_quant(fmt_of(fmt), interleaved != 0, x, x_token_stride,
                                          positions, cos_sin, max_pos, T, NH, D, R, codes,
                                          scales, num_cus(), stream));
}

moe_status moe_fused_forward_noalloc(const moe_fused_args* a, hipStream_t stream) {
  // every check on the host first: arguments, then the size against the
  // scratch buffer; nothing is enqueued on an error
  const moe_status st = check_fused(a, false);
  if (st != MOE_OK || a->T == 0) return st;
  if (moe_fused_workspace_bytes(a) > kScratchBytes) return MOE_ERR_WORKSPACE;
  if (prepare_all() != hipSuccess) return MOE_ERR_HIP;
  moe_fused_args b = *a;
  b.workspace = device_scratch();
  if (!b.workspace) return MOE_ERR_HIP;
  b.workspace_bytes = kScratchBytes;
  return fused_forward_impl(&b, stream, nullptr);
}

}  // extern "C"
