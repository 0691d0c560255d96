// C ABI of libgnf4: argument validation, path choice and kernel dispatch.
// Every entry point is declared and documented in include/gnf4.h.

#include <limits.h>
#include <string.h>

#include <mutex>

#include "dgrad_tile.h"
#include "gnf4_internal.h"
#include "route_core.h"

namespace gnf4 {

namespace {
thread_local int g_last_hip_error = 0;

gnf4_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return GNF4_ERR_HIP;
}

// Rows per group at or below which a group takes the decode path.  One
// constant for every shape (no per-shape tables): below it a tile of 32
// MFMA rows would be mostly padding, above it the fp32 decode path's
// per-row multiply-adds cost more than the matrix core.
constexpr int kDecodeMaxRows = 8;
// A batch averaging at least this many rows per group (prefill) puts every
// group on the tile path: a decode launch there only has its workgroups
// scan the group list for the rare small group, which costs more than the
// tile kernel spends on such a group.
constexpr int64_t kTileOnlyRowsPerGroup = 32;

// The automatic path choice, from host-known sizes only.
static bool auto_tile_only(int64_t M, int64_t G) {
  const int64_t g_eff = G < M ? G : M;
  return g_eff > 0 && M >= kTileOnlyRowsPerGroup * g_eff;
}

bool is_device_ptr(const void* p) {
  if (p == nullptr) return false;
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  const hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return false;
  }
  return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Workspace of one grouped GEMM call: the tile path's staged activation
// rows first (stage_bytes: the exponents of M + 1 rows, then M + 1 fp16 rows
// of the padded width; fewer are used when the rows are staged per token),
// then the decode path's split-K partials, each region 256-byte aligned.
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

void set_stage_regions(void* ws, int64_t M, int32_t*& row_exp, uint16_t*& xh) {
  row_exp = static_cast<int32_t*>(ws);
  xh = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) +
                                   align256((size_t)(M + 1) * sizeof(int32_t)));
}

// Workspace of gnf4_grouped_gemm_gather_noalloc: one library-owned array per
// GPU, held until the process ends.  Its host-side name is only a stand-in;
// kernels get the device address that hipGetSymbolAddress returns for the
// current device (scratch_address).
constexpr size_t kNoAllocScratchBytes = (size_t)GNF4_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static thread_local int cached_dev = -1, cached = 0;
  if (dev != cached_dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached_dev = dev;
    cached = n;
  }
  return cached;
}

}  // namespace gnf4

using namespace gnf4;

extern "C" {

const char* gnf4_status_string(gnf4_status s) {
  switch (s) {
    case GNF4_OK: return "ok";
    case GNF4_ERR_INVALID_ARG: return "invalid argument (null pointer, bad dimension or misalignment)";
    case GNF4_ERR_NOT_DEVICE_PTR:
      return "pointer is not device memory: libgnf4 runs on the GPU only; the CPU reference "
             "computation is the oracle shipped with the tests, not a fallback";
    case GNF4_ERR_UNSUPPORTED: return "size beyond the supported limits";
    case GNF4_ERR_WORKSPACE: return "workspace missing or too small";
    case GNF4_ERR_HIP: return "HIP runtime error (see gnf4_last_hip_error)";
  }
  return "unknown status";
}

int gnf4_last_hip_error(void) { return g_last_hip_error; }

const char* gnf4_version(void) { return "0.1.0"; }

static bool valid_dtype(int32_t d) { return d == GNF4_DTYPE_BF16 || d == GNF4_DTYPE_F32; }
// scale kind of an MXFP4 stack inside gemm_common: E8M0 bytes, one per 32 codes
constexpr int32_t kScaleE8M0 = 2;
static size_t dtype_bytes(int32_t d) {
  return d == GNF4_DTYPE_BF16 ? 2 : d == kScaleE8M0 ? 1 : 4;
}

gnf4_status gnf4_pack(const void* w, int32_t w_dtype, int64_t E, int64_t N, int64_t K,
                      uint8_t* packed, float* absmax, void* stream) {
  return gnf4_pack_ex(w, w_dtype, E, N, K, packed, absmax, GNF4_DTYPE_F32, stream);
}

gnf4_status gnf4_pack_ex(const void* w, int32_t w_dtype, int64_t E, int64_t N, int64_t K,
                         uint8_t* packed, void* absmax, int32_t absmax_dtype, void* stream) {
  if (!w || !packed || !absmax) return GNF4_ERR_INVALID_ARG;
  if (E <= 0 || N <= 0 || K <= 0 || K % kBlock != 0) return GNF4_ERR_INVALID_ARG;
  if (!valid_dtype(w_dtype) || !valid_dtype(absmax_dtype)) return GNF4_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(packed, 4) || !aligned(absmax, dtype_bytes(absmax_dtype)))
    return GNF4_ERR_INVALID_ARG;
  if (E > INT64_MAX / N || E * N > INT64_MAX / K) return GNF4_ERR_INVALID_ARG;
  if (!is_device_ptr(w) || !is_device_ptr(packed) || !is_device_ptr(absmax))
    return GNF4_ERR_NOT_DEVICE_PTR;
  const int64_t n_blocks = E * N * (K / kBlock);
  const hipError_t e = launch_pack(w, w_dtype, n_blocks, packed, absmax, absmax_dtype,
                                   (hipStream_t)stream);
  return e == hipSuccess ? GNF4_OK : hip_fail(e);
}

size_t gnf4_route_sort_workspace_size(int64_t T, int64_t E, int32_t top_k) {
  if (T < 0 || E <= 0) return 0;
  return plan_route(T, E, top_k).ws_bytes;
}

gnf4_status gnf4_route_sort(const float* logits, int64_t T, int64_t E, int32_t top_k,
                            int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                            int32_t* sorted_slots, int32_t* slot_rows, int32_t* group_sizes,
                            int32_t* group_expert_ids, int32_t* num_groups, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (T < 0 || E <= 0 || top_k < 1 || top_k > E) return GNF4_ERR_INVALID_ARG;
  if (E > 1024 || top_k > 32) return GNF4_ERR_UNSUPPORTED;
  if (T > (int64_t)INT_MAX / top_k) return GNF4_ERR_UNSUPPORTED;
  if (!expert_offsets || !group_sizes || !group_expert_ids || !num_groups)
    return GNF4_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_slots)) return GNF4_ERR_INVALID_ARG;
  const void* dev_ptrs[] = {expert_offsets, group_sizes, group_expert_ids, num_groups};
  for (const void* p : dev_ptrs)
    if (!aligned(p, 4)) return GNF4_ERR_INVALID_ARG;
  if (T > 0) {
    const void* more[] = {logits, topk_ids, topk_w, sorted_slots};
    for (const void* p : more)
      if (!aligned(p, 4)) return GNF4_ERR_INVALID_ARG;
    for (const void* p : more)
      if (!is_device_ptr(p)) return GNF4_ERR_NOT_DEVICE_PTR;
    if (slot_rows) {  // optional output
      if (!aligned(slot_rows, 4)) return GNF4_ERR_INVALID_ARG;
      if (!is_device_ptr(slot_rows)) return GNF4_ERR_NOT_DEVICE_PTR;
    }
  }
  for (const void* p : dev_ptrs)
    if (!is_device_ptr(p)) return GNF4_ERR_NOT_DEVICE_PTR;
  const RoutePlan plan = plan_route(T, E, top_k);
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return GNF4_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return GNF4_ERR_INVALID_ARG;
    if (!is_device_ptr(workspace)) return GNF4_ERR_NOT_DEVICE_PTR;
  }
  const hipError_t e = launch_route_sort(logits, (int)T, (int)E, top_k, topk_ids, topk_w,
                                         expert_offsets, sorted_slots, slot_rows, group_sizes,
                                         group_expert_ids, num_groups,
                                         static_cast<int32_t*>(workspace), plan,
                                         (hipStream_t)stream);
  return e == hipSuccess ? GNF4_OK : hip_fail(e);
}

static gnf4_status gemm_common(const uint16_t* x, const uint8_t* packed, const void* absmax,
                               int32_t absmax_dtype, int64_t E, int64_t N, int64_t K, const int32_t* sizes,
                               const int32_t* ids, int64_t G, int64_t M, uint16_t* y,
                               void* ws, size_t ws_bytes, int32_t path, int32_t split_k,
                               void* stream, const int32_t* slots = nullptr, int32_t slot_div = 1,
                               int64_t T = 0, bool ws_is_scratch = false) {
  if (E <= 0 || N <= 0 || K < kBlock || K % kBlock != 0 || M < 0 || G < 0)
    return GNF4_ERR_INVALID_ARG;
  if (path < 0 || path > 2 || split_k < 0 || split_k > 16) return GNF4_ERR_INVALID_ARG;
  if (slots && (slot_div < 1 || T < 0)) return GNF4_ERR_INVALID_ARG;
  if (M == 0 || G == 0) return GNF4_OK;
  if (N * (K / 2) >= ((int64_t)1 << 31) || M * K >= ((int64_t)1 << 31) ||
      M * N >= ((int64_t)1 << 31) || E >= INT_MAX || G >= 65536)
    return GNF4_ERR_UNSUPPORTED;
  if (slots && (T * slot_div >= ((int64_t)1 << 31) || T * K >= ((int64_t)1 << 31)))
    return GNF4_ERR_UNSUPPORTED;
  if (!x || !packed || !absmax || !sizes || !ids || !y) return GNF4_ERR_INVALID_ARG;
  if (!valid_dtype(absmax_dtype) && absmax_dtype != kScaleE8M0) return GNF4_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(absmax, dtype_bytes(absmax_dtype)) ||
      !aligned(sizes, 4) ||
      !aligned(ids, 4) || !aligned(y, 2) || (slots && !aligned(slots, 4)))
    return GNF4_ERR_INVALID_ARG;
  const void* ptrs[] = {x, packed, absmax, sizes, ids, y};
  for (const void* p : ptrs)
    if (!is_device_ptr(p)) return GNF4_ERR_NOT_DEVICE_PTR;
  if (slots && !is_device_ptr(slots)) return GNF4_ERR_NOT_DEVICE_PTR;

  GemmArgs a;
  a.slots = slots;
  a.slot_div = slot_div;
  a.T = (int)T;
  a.x = x;
  a.packed = packed;
  a.absmax = absmax;
  a.abs_bf16 = absmax_dtype == GNF4_DTYPE_BF16;
  a.mxfp4 = absmax_dtype == kScaleE8M0;
  a.sizes = sizes;
  a.ids = ids;
  a.y = y;
  a.partial = nullptr;
  a.row_exp = nullptr;
  a.xh = nullptr;
  a.xh_ld = 0;
  a.E = (int)E;
  a.N = (int)N;
  a.K = (int)K;
  a.G = (int)G;
  a.M = (int)M;
  bool run_decode = true, run_tile = true;
  if (path == 1) {
    a.rows_max_decode = INT_MAX;
    a.rows_min_tile = INT_MAX;
    run_tile = false;
  } else if (path == 2) {
    a.rows_max_decode = 0;
    a.rows_min_tile = 1;
    run_decode = false;
  } else if (auto_tile_only(M, G)) {
    a.rows_max_decode = 0;
    a.rows_min_tile = 1;
    run_decode = false;
  } else {
    a.rows_max_decode = kDecodeMaxRows;
    a.rows_min_tile = kDecodeMaxRows + 1;
    // No group can exceed M rows, and with the gather fused a group of a
    // top-k routing holds at most T rows (a token picks each expert once).
    // Then the decode launch serves every group, whatever its size (a group
    // that breaks that bound is still computed, on the decode path), and
    // the tile launch and its staging are skipped.
    if (M <= kDecodeMaxRows || (slots && T <= kDecodeMaxRows)) {
      a.rows_max_decode = INT_MAX;
      a.rows_min_tile = INT_MAX;
      run_tile = false;
    }
  }
  const hipStream_t s = (hipStream_t)stream;
  if (validate_requested()) {
    int32_t bad = 0;
    const hipError_t ve = validate_groups(sizes, ids, G, E, M, slots, T * (int64_t)slot_div, s,
                                          &bad);
    if (ve != hipSuccess) return hip_fail(ve);
    if (bad) return GNF4_ERR_INVALID_ARG;
  }
  size_t dec_off = 0;  // where the decode partials start in the workspace
  if (ws && (run_tile || ws_bytes > 0)) {
    if (!aligned(ws, 16)) return GNF4_ERR_INVALID_ARG;
    if (!ws_is_scratch && !is_device_ptr(ws)) return GNF4_ERR_NOT_DEVICE_PTR;
  }
  StagePlan sp{};
  if (run_tile) {
    dec_off = stage_bytes(M, K);
    if (!ws || ws_bytes < dec_off) return GNF4_ERR_WORKSPACE;
    set_stage_regions(ws, M, a.row_exp, a.xh);
    sp = plan_stage(a);
    a.xh_ld = sp.ld;
  }
  if (run_decode) {
    DecodePlan p = plan_decode(M, N, K, G, split_k, device_cu_count());
    if (p.L == 0) return GNF4_ERR_UNSUPPORTED;  // this split_k leaves too much K per split
    const size_t need = decode_workspace_bytes(p, M, N);
    if (need > 0) {
      if (!ws || ws_bytes < dec_off + need) {
        if (split_k > 0) return GNF4_ERR_WORKSPACE;
        p = plan_decode(M, N, K, G, 1, device_cu_count());  // no room to split: one pass
        if (p.L == 0) return GNF4_ERR_WORKSPACE;  // K needs splitting, which needs workspace
      } else {
        a.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + dec_off);
      }
    }
    const hipError_t e = launch_decode(a, p, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (run_tile) {
    hipError_t e = launch_stage_x(a, sp, a.mxfp4, s);  // MXFP4 operands in natural K order
    if (e == hipSuccess) e = launch_tile(a, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return GNF4_OK;
}

gnf4_status gnf4_gather_rows(const uint16_t* x, int64_t T, int64_t K, const int32_t* sorted_slots,
                             int32_t top_k, int64_t M, uint16_t* x_sorted, void* stream) {
  if (T < 0 || M < 0 || top_k < 1 || K < kBlock || K % kBlock != 0) return GNF4_ERR_INVALID_ARG;
  if (M == 0) return GNF4_OK;
  if (T * top_k >= ((int64_t)1 << 31) || M * K >= ((int64_t)1 << 31) || M >= ((int64_t)1 << 31))
    return GNF4_ERR_UNSUPPORTED;
  if (!x || !sorted_slots || !x_sorted) return GNF4_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(x_sorted, 16) || !aligned(sorted_slots, 4))
    return GNF4_ERR_INVALID_ARG;
  if (!is_device_ptr(x) || !is_device_ptr(sorted_slots) || !is_device_ptr(x_sorted))
    return GNF4_ERR_NOT_DEVICE_PTR;
  const hipError_t e = launch_gather(x, sorted_slots, top_k, (int)T, (int)M, (int)K, x_sorted,
                                     (hipStream_t)stream);
  return e == hipSuccess ? GNF4_OK : hip_fail(e);
}

// Path of a dgrad call: 2 = tile, 1 = GEMV.  Automatic: a batch averaging
// at least 32 rows per group (prefill) takes the tile path; the GEMV path
// re-reads the weights once per 4 rows of dy.
static int dgrad_path(int32_t path, int64_t M, int64_t G) {
  if (path == 0) return auto_tile_only(M, G) ? 2 : 1;
  return path;
}

size_t gnf4_grouped_dgrad_workspace_size_ex(int64_t M, int64_t N, int64_t K, int64_t G,
                                            int64_t E, int32_t path) {
  (void)E;
  if (M <= 0 || N <= 0 || K < kBlock || G <= 0) return 0;
  if (dgrad_path(path, M, G) == 2) return stage_bytes(M, N);
  return dgrad_workspace_bytes(plan_dgrad(M, N, K, G, device_cu_count()), M, K);
}

size_t gnf4_grouped_dgrad_workspace_size(int64_t M, int64_t N, int64_t K, int64_t G,
                                         int64_t E) {
  return gnf4_grouped_dgrad_workspace_size_ex(M, N, K, G, E, 0);
}

gnf4_status gnf4_grouped_dgrad_ex(const uint16_t* dy, const uint8_t* packed, const void* absmax,
                                  int64_t E, int64_t N, int64_t K, const int32_t* group_sizes,
                                  const int32_t* group_expert_ids, int64_t G, int64_t M,
                                  uint16_t* dx, void* workspace, size_t workspace_bytes,
                                  int32_t absmax_dtype, int32_t path, void* stream) {
  if (E <= 0 || N <= 0 || K < kBlock || K % kBlock != 0 || M < 0 || G < 0)
    return GNF4_ERR_INVALID_ARG;
  if (path < 0 || path > 2) return GNF4_ERR_INVALID_ARG;
  if (M == 0 || G == 0) return GNF4_OK;
  if (N * (K / 2) >= ((int64_t)1 << 31) || M * K >= ((int64_t)1 << 31) ||
      M * N >= ((int64_t)1 << 31) || E * N >= ((int64_t)1 << 31) || G >= 65536)
    return GNF4_ERR_UNSUPPORTED;
  if (!dy || !packed || !absmax || !group_sizes || !group_expert_ids || !dx)
    return GNF4_ERR_INVALID_ARG;
  if (!valid_dtype(absmax_dtype)) return GNF4_ERR_INVALID_ARG;
  if (!aligned(dy, 2) || !aligned(dx, 2) || !aligned(packed, 16) ||
      !aligned(absmax, dtype_bytes(absmax_dtype)) ||
      !aligned(group_sizes, 4) || !aligned(group_expert_ids, 4))
    return GNF4_ERR_INVALID_ARG;
  const void* ptrs[] = {dy, packed, absmax, group_sizes, group_expert_ids, dx};
  for (const void* p : ptrs)
    if (!is_device_ptr(p)) return GNF4_ERR_NOT_DEVICE_PTR;
  DgradArgs a;
  a.dy = dy;
  a.packed = packed;
  a.absmax = absmax;
  a.abs_bf16 = absmax_dtype == GNF4_DTYPE_BF16;
  a.sizes = group_sizes;
  a.ids = group_expert_ids;
  a.dx = dx;
  a.partial = nullptr;
  a.E = (int)E;
  a.N = (int)N;
  a.K = (int)K;
  a.G = (int)G;
  a.M = (int)M;
  const hipStream_t s = (hipStream_t)stream;
  if (validate_requested()) {
    int32_t bad = 0;
    const hipError_t ve = validate_groups(group_sizes, group_expert_ids, G, E, M, nullptr, 0, s,
                                          &bad);
    if (ve != hipSuccess) return hip_fail(ve);
    if (bad) return GNF4_ERR_INVALID_ARG;
  }
  const int run = dgrad_path(path, M, G);
  if (run == 2) {
    if (!workspace || workspace_bytes < stage_bytes(M, N)) return GNF4_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return GNF4_ERR_INVALID_ARG;
    if (!is_device_ptr(workspace)) return GNF4_ERR_NOT_DEVICE_PTR;
    // dy staged by the forward's pre-pass as an [M, N] matrix, natural order
    GemmArgs g{};
    g.x = dy;
    g.slots = nullptr;
    g.slot_div = 1;
    g.T = 0;
    g.M = (int)M;
    g.K = (int)N;
    set_stage_regions(workspace, M, g.row_exp, g.xh);
    const StagePlan sp = plan_stage(g);
    hipError_t e = launch_stage_x(g, sp, true, s);
    if (e == hipSuccess) e = launch_dgrad_tile(a, g.row_exp, g.xh, sp.ld, 1, s);
    return e == hipSuccess ? GNF4_OK : hip_fail(e);
  }
  DgradPlan p = plan_dgrad(M, N, K, G, device_cu_count());
  const size_t need = dgrad_workspace_bytes(p, M, K);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) {
      p.S = 1;  // no room for split partials: one split over all of N
      p.rows_per_split = (int)N;
    } else {
      if (!aligned(workspace, 16)) return GNF4_ERR_INVALID_ARG;
      if (!is_device_ptr(workspace)) return GNF4_ERR_NOT_DEVICE_PTR;
      a.partial = static_cast<float*>(workspace);
    }
  }
  const hipError_t e = launch_dgrad(a, p, s);
  return e == hipSuccess ? GNF4_OK : hip_fail(e);
}

gnf4_status gnf4_grouped_dgrad(const uint16_t* dy, const uint8_t* packed, const void* absmax,
                               int64_t E, int64_t N, int64_t K, const int32_t* group_sizes,
                               const int32_t* group_expert_ids, int64_t G, int64_t M,
                               uint16_t* dx, void* workspace, size_t workspace_bytes,
                               int32_t absmax_dtype, void* stream) {
  return gnf4_grouped_dgrad_ex(dy, packed, absmax, E, N, K, group_sizes, group_expert_ids, G, M,
                               dx, workspace, workspace_bytes, absmax_dtype, 0, stream);
}

gnf4_status gnf4_grouped_gemm_mxfp4(const uint16_t* x, int64_t T, const int32_t* sorted_slots,
                                    int32_t top_k, const uint8_t* packed, const uint8_t* scales,
                                    int64_t E, int64_t N, int64_t K, const int32_t* group_sizes,
                                    const int32_t* group_expert_ids, int64_t G, int64_t M,
                                    uint16_t* y, void* workspace, size_t workspace_bytes,
                                    int32_t path, int32_t split_k, void* stream) {
  if (sorted_slots) {
    if (top_k < 1 || T < 0) return GNF4_ERR_INVALID_ARG;
    return gemm_common(x, packed, scales, kScaleE8M0, E, N, K, group_sizes, group_expert_ids, G,
                       M, y, workspace, workspace_bytes, path, split_k, stream, sorted_slots,
                       top_k, T);
  }
  return gemm_common(x, packed, scales, kScaleE8M0, E, N, K, group_sizes, group_expert_ids, G, M,
                     y, workspace, workspace_bytes, path, split_k, stream);
}

// The routed one-token GEMM's decode plan: top_k rows, one per pick.
static DecodePlan route_gemm_plan(int32_t top_k, int64_t N, int64_t K) {
  return plan_decode(top_k, N, K, top_k, 0, device_cu_count());
}

size_t gnf4_route_gemm_one_token_workspace_size(int64_t E, int32_t top_k, int64_t N, int64_t K) {
  (void)E;
  if (top_k < 1 || N <= 0 || K < kBlock) return 0;
  return decode_workspace_bytes(route_gemm_plan(top_k, N, K), top_k, N);
}

gnf4_status gnf4_route_gemm_one_token(const float* logits, int64_t E, int32_t top_k,
                                      const uint16_t* x, const uint8_t* packed,
                                      const void* absmax, int32_t absmax_dtype, int64_t N,
                                      int64_t K, uint16_t* y, int32_t* topk_ids, float* topk_w,
                                      int32_t* expert_offsets, int32_t* sorted_slots,
                                      int32_t* slot_rows, int32_t* group_sizes,
                                      int32_t* group_expert_ids, int32_t* num_groups,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (E < 1 || top_k < 1 || top_k > E || N <= 0 || K < kBlock || K % kBlock != 0)
    return GNF4_ERR_INVALID_ARG;
  // at most two experts per lane of the ranking wavefronts; top_k as
  // gnf4_route_sort
  if (E > 128 || top_k > 32) return GNF4_ERR_UNSUPPORTED;
  if (N * (K / 2) >= ((int64_t)1 << 31) || E * N >= ((int64_t)1 << 31)) return GNF4_ERR_UNSUPPORTED;
  if (!valid_dtype(absmax_dtype)) return GNF4_ERR_INVALID_ARG;
  const void* out4[] = {topk_ids, topk_w, expert_offsets, sorted_slots, group_sizes,
                        group_expert_ids, num_groups, logits};
  for (const void* p : out4)
    if (!p || !aligned(p, 4)) return GNF4_ERR_INVALID_ARG;
  if (!x || !packed || !absmax || !y) return GNF4_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(absmax, dtype_bytes(absmax_dtype)) ||
      !aligned(y, 2) || (slot_rows && !aligned(slot_rows, 4)))
    return GNF4_ERR_INVALID_ARG;
  for (const void* p : out4)
    if (!is_device_ptr(p)) return GNF4_ERR_NOT_DEVICE_PTR;
  const void* more[] = {x, packed, absmax, y};
  for (const void* p : more)
    if (!is_device_ptr(p)) return GNF4_ERR_NOT_DEVICE_PTR;
  if (slot_rows && !is_device_ptr(slot_rows)) return GNF4_ERR_NOT_DEVICE_PTR;

  GemmArgs a{};
  a.x = x;
  a.packed = packed;
  a.absmax = absmax;
  a.abs_bf16 = absmax_dtype == GNF4_DTYPE_BF16;
  a.mxfp4 = false;
  a.sizes = group_sizes;       // written by the launch; read by a split-K reduce
  a.ids = group_expert_ids;
  a.slots = sorted_slots;
  a.slot_div = top_k;
  a.T = 1;
  a.y = y;
  a.partial = nullptr;
  a.row_exp = nullptr;
  a.E = (int)E;
  a.N = (int)N;
  a.K = (int)K;
  a.G = (int)E;
  a.M = top_k;
  a.rows_max_decode = INT_MAX;
  a.rows_min_tile = INT_MAX;
  DecodePlan p = route_gemm_plan(top_k, N, K);
  if (p.L == 0) return GNF4_ERR_UNSUPPORTED;
  const size_t need = decode_workspace_bytes(p, top_k, N);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) {
      p = plan_decode(top_k, N, K, top_k, 1, device_cu_count());  // no room to split: one pass
      if (p.L == 0) return GNF4_ERR_WORKSPACE;
    } else {
      if (!aligned(workspace, 16)) return GNF4_ERR_INVALID_ARG;
      if (!is_device_ptr(workspace)) return GNF4_ERR_NOT_DEVICE_PTR;
      a.partial = static_cast<float*>(workspace);
    }
  }
  RouteOneOut ro;
  ro.E = (int)E;
  ro.K = top_k;
  ro.topk_ids = topk_ids;
  ro.topk_w = topk_w;
  ro.offsets = expert_offsets;
  ro.sorted = sorted_slots;
  ro.rows = slot_rows;
  ro.gsizes = group_sizes;
  ro.gids = group_expert_ids;
  ro.ngroups = num_groups;
  const hipError_t e = launch_decode_routed(a, p, logits, ro, (hipStream_t)stream);
  return e == hipSuccess ? GNF4_OK : hip_fail(e);
}

size_t gnf4_moe_ffn_one_token_workspace_size(int32_t top_k) {
  if (top_k < 1) return 0;
  return ffn_sync_bytes(top_k);
}

gnf4_status gnf4_moe_ffn_one_token(const float* logits, int64_t E, int32_t top_k,
                                   const uint16_t* x, const uint8_t* gate_up_packed,
                                   const void* gate_up_absmax, const uint8_t* down_packed,
                                   const void* down_absmax, int32_t absmax_dtype, int64_t H,
                                   int64_t I, uint16_t* h, uint16_t* y, int32_t* topk_ids,
                                   float* topk_w, int32_t* expert_offsets, int32_t* sorted_slots,
                                   int32_t* slot_rows, int32_t* group_sizes,
                                   int32_t* group_expert_ids, int32_t* num_groups,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (E < 1 || top_k < 1 || top_k > E || H < kBlock || H % kBlock != 0 || I < kBlock ||
      I % kBlock != 0)
    return GNF4_ERR_INVALID_ARG;
  if (E > 128 || top_k > 32) return GNF4_ERR_UNSUPPORTED;
  if (2 * I * (H / 2) >= ((int64_t)1 << 31) || H * (I / 2) >= ((int64_t)1 << 31) ||
      E * 2 * I >= ((int64_t)1 << 31) || E * H >= ((int64_t)1 << 31))
    return GNF4_ERR_UNSUPPORTED;
  if (!valid_dtype(absmax_dtype)) return GNF4_ERR_INVALID_ARG;
  const void* out4[] = {topk_ids, topk_w, expert_offsets, sorted_slots, group_sizes,
                        group_expert_ids, num_groups, logits};
  for (const void* p : out4)
    if (!p || !aligned(p, 4)) return GNF4_ERR_INVALID_ARG;
  if (!x || !gate_up_packed || !gate_up_absmax || !down_packed || !down_absmax || !h || !y)
    return GNF4_ERR_INVALID_ARG;
  const size_t ab = dtype_bytes(absmax_dtype);
  if (!aligned(x, 16) || !aligned(gate_up_packed, 16) || !aligned(down_packed, 16) ||
      !aligned(gate_up_absmax, ab) || !aligned(down_absmax, ab) || !aligned(h, 16) ||
      !aligned(y, 2) || (slot_rows && !aligned(slot_rows, 4)))
    return GNF4_ERR_INVALID_ARG;
  const size_t need = gnf4_moe_ffn_one_token_workspace_size(top_k);
  if (!workspace || workspace_bytes < need) return GNF4_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return GNF4_ERR_INVALID_ARG;
  for (const void* p : out4)
    if (!is_device_ptr(p)) return GNF4_ERR_NOT_DEVICE_PTR;
  const void* more[] = {x, gate_up_packed, gate_up_absmax, down_packed, down_absmax, h, y,
                        workspace};
  for (const void* p : more)
    if (!is_device_ptr(p)) return GNF4_ERR_NOT_DEVICE_PTR;
  if (slot_rows && !is_device_ptr(slot_rows)) return GNF4_ERR_NOT_DEVICE_PTR;
  FfnPlan plan;
  if (!plan_ffn(E, top_k, H, I, device_cu_count(), plan)) return GNF4_ERR_UNSUPPORTED;
  RouteOneOut ro;
  ro.E = (int)E;
  ro.K = top_k;
  ro.topk_ids = topk_ids;
  ro.topk_w = topk_w;
  ro.offsets = expert_offsets;
  ro.sorted = sorted_slots;
  ro.rows = slot_rows;
  ro.gsizes = group_sizes;
  ro.gids = group_expert_ids;
  ro.ngroups = num_groups;
  const hipError_t e = launch_ffn_one_token(
      plan, logits, x, gate_up_packed, gate_up_absmax, down_packed, down_absmax,
      absmax_dtype == GNF4_DTYPE_BF16, (int)E, top_k, (int)H, (int)I, h, y,
      static_cast<int32_t*>(workspace), ro, (hipStream_t)stream);
  return e == hipSuccess ? GNF4_OK : hip_fail(e);
}

int gnf4_moe_ffn_one_token_supported(int64_t E, int32_t top_k, int64_t H, int64_t I) {
  if (E < 1 || top_k < 1 || top_k > E || E > 128 || top_k > 32 || H < kBlock ||
      H % kBlock != 0 || I < kBlock || I % kBlock != 0)
    return 0;
  FfnPlan plan;
  return plan_ffn(E, top_k, H, I, device_cu_count(), plan) ? 1 : 0;
}

gnf4_status gnf4_swiglu(const uint16_t* gate_up, int64_t M, int64_t I, uint16_t* h,
                        void* stream) {
  if (M < 0 || I <= 0) return GNF4_ERR_INVALID_ARG;
  if (M == 0) return GNF4_OK;
  if (M > ((int64_t)1 << 40) / I) return GNF4_ERR_UNSUPPORTED;
  if (!gate_up || !h || !aligned(gate_up, 2) || !aligned(h, 2)) return GNF4_ERR_INVALID_ARG;
  if (!is_device_ptr(gate_up) || !is_device_ptr(h)) return GNF4_ERR_NOT_DEVICE_PTR;
  const hipError_t e = launch_swiglu(gate_up, M, I, h, (hipStream_t)stream);
  return e == hipSuccess ? GNF4_OK : hip_fail(e);
}

gnf4_status gnf4_combine(const uint16_t* y, const int32_t* slot_rows, const float* topk_w,
                         int64_t T, int32_t top_k, int64_t M, int64_t H, uint16_t* out,
                         void* stream) {
  if (T < 0 || M < 0 || H <= 0 || top_k < 1) return GNF4_ERR_INVALID_ARG;
  if (T == 0) return GNF4_OK;
  if (T > (int64_t)INT_MAX / top_k) return GNF4_ERR_UNSUPPORTED;
  if (!slot_rows || !topk_w || !out || (M > 0 && !y)) return GNF4_ERR_INVALID_ARG;
  if (!aligned(slot_rows, 4) || !aligned(topk_w, 4) || !aligned(out, 2) ||
      (y && !aligned(y, 2)))
    return GNF4_ERR_INVALID_ARG;
  if (!is_device_ptr(slot_rows) || !is_device_ptr(topk_w) || !is_device_ptr(out) ||
      (M > 0 && !is_device_ptr(y)))
    return GNF4_ERR_NOT_DEVICE_PTR;
  const hipError_t e = launch_combine(y, slot_rows, topk_w, T, top_k, M, H, out,
                                      (hipStream_t)stream);
  return e == hipSuccess ? GNF4_OK : hip_fail(e);
}

gnf4_status gnf4_grouped_gemm_gather(const uint16_t* x, int64_t T, const int32_t* sorted_slots,
                                     int32_t top_k, const uint8_t* packed, const void* absmax,
                                     int64_t E, int64_t N, int64_t K, const int32_t* group_sizes,
                                     const int32_t* group_expert_ids, int64_t G, int64_t M,
                                     uint16_t* y, void* workspace, size_t workspace_bytes,
                                     int32_t path, int32_t split_k, int32_t absmax_dtype,
                                     void* stream) {
  if (!sorted_slots) return GNF4_ERR_INVALID_ARG;
  return gemm_common(x, packed, absmax, absmax_dtype, E, N, K, group_sizes, group_expert_ids, G,
                     M, y, workspace, workspace_bytes, path, split_k, stream, sorted_slots, top_k,
                     T);
}

size_t gnf4_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

gnf4_status gnf4_grouped_gemm_gather_noalloc(const uint16_t* x, int64_t T,
                                             const int32_t* sorted_slots, int32_t top_k,
                                             const uint8_t* packed, const void* absmax, int64_t E,
                                             int64_t N, int64_t K, const int32_t* group_sizes,
                                             const int32_t* group_expert_ids, int64_t G,
                                             int64_t M, uint16_t* y, int32_t path,
                                             int32_t split_k, int32_t absmax_dtype,
                                             void* stream) {
  if (!sorted_slots) return GNF4_ERR_INVALID_ARG;
  if (E <= 0 || N <= 0 || K < kBlock || K % kBlock != 0 || M < 0 || G < 0 || T < 0 ||
      top_k < 1)
    return GNF4_ERR_INVALID_ARG;
  if (path < 0 || path > 2 || split_k < 0 || split_k > 16) return GNF4_ERR_INVALID_ARG;
  if (M == 0 || G == 0) return GNF4_OK;
  // the scratch must hold what the workspace of gnf4_grouped_gemm_gather would
  const size_t need = gnf4_grouped_gemm_workspace_size_ex(M, N, K, G, E, path, split_k);
  if (need > kNoAllocScratchBytes) return GNF4_ERR_UNSUPPORTED;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e);
  return gemm_common(x, packed, absmax, absmax_dtype, E, N, K, group_sizes, group_expert_ids, G,
                     M, y, ws, kNoAllocScratchBytes, path, split_k, stream, sorted_slots, top_k,
                     T, true);
}

size_t gnf4_grouped_gemm_workspace_size_ex(int64_t M, int64_t N, int64_t K, int64_t G,
                                           int64_t E, int32_t path, int32_t split_k) {
  (void)E;
  if (M <= 0 || N <= 0 || K < kBlock || G <= 0) return 0;
  const bool tile_only = path == 2 || (path == 0 && auto_tile_only(M, G));
  const bool tile = tile_only || (path == 0 && M > kDecodeMaxRows);
  const size_t tile_bytes = tile ? stage_bytes(M, K) : 0;
  if (tile_only) return tile_bytes;
  const DecodePlan p = plan_decode(M, N, K, G, split_k, device_cu_count());
  return tile_bytes + decode_workspace_bytes(p, M, N);
}

size_t gnf4_grouped_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t G, int64_t E) {
  return gnf4_grouped_gemm_workspace_size_ex(M, N, K, G, E, 0, 0);
}

gnf4_status gnf4_grouped_gemm(const uint16_t* x_sorted, const uint8_t* packed,
                              const float* absmax, int64_t E, int64_t N, int64_t K,
                              const int32_t* group_sizes, const int32_t* group_expert_ids,
                              int64_t G, int64_t M, uint16_t* y, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return gemm_common(x_sorted, packed, absmax, GNF4_DTYPE_F32, E, N, K, group_sizes,
                     group_expert_ids, G, M, y, workspace, workspace_bytes, 0, 0, stream);
}

gnf4_status gnf4_grouped_gemm_ex(const uint16_t* x_sorted, const uint8_t* packed,
                                 const void* absmax, int64_t E, int64_t N, int64_t K,
                                 const int32_t* group_sizes, const int32_t* group_expert_ids,
                                 int64_t G, int64_t M, uint16_t* y, void* workspace,
                                 size_t workspace_bytes, int32_t path, int32_t split_k,
                                 int32_t absmax_dtype, void* stream) {
  return gemm_common(x_sorted, packed, absmax, absmax_dtype, E, N, K, group_sizes,
                     group_expert_ids, G, M, y, workspace, workspace_bytes, path, split_k,
                     stream);
}

}  // extern "C"
