// C ABI of libw4a16: argument checking, device check, variant selection and
// launch of the gfx950 kernels.  Every check runs on the host before any HIP
// call, so a rejected call touches no device state.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/w4a16.h"
#include "w4a16_internal.h"

namespace {

constexpr int64_t kMaxRows = 2147483647LL;
// Stands in for the static scratch in the host-side argument checks of
// w4a16_head_gather_noalloc (they test a workspace pointer for null and
// alignment only; the kernels get the real device address).
constexpr uintptr_t kScratchAligned = 256;
constexpr int64_t kMaxK = 1LL << 20;

std::atomic<int32_t> g_variant{-1};
std::once_flag g_env_once;

void read_env_variant() {
  int32_t v = W4A16_VARIANT_AUTO;
  if (const char* e = std::getenv("W4A16_VARIANT")) {
    if (std::strcmp(e, "dot") == 0) v = W4A16_VARIANT_DOT;
    if (std::strcmp(e, "mfma") == 0) v = W4A16_VARIANT_MFMA;
  }
  int32_t expected = -1;
  g_variant.compare_exchange_strong(expected, v);
}

int32_t current_variant() {
  std::call_once(g_env_once, read_env_variant);
  return g_variant.load();
}

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other;
// and the device's compute-unit count (sizes the split-K plans).
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];
thread_local int t_cus = 256;  // CUs of the device of this thread's last checked call

w4a16_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return W4A16_ERR_UNSUPPORTED;
  int known = g_arch[dev].load();
  if (known == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return W4A16_ERR_HIP;
    g_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1);
    known = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch[dev].store(known);
  }
  t_cus = g_cus[dev].load();
  return known == 1 ? W4A16_OK : W4A16_ERR_UNSUPPORTED;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

w4a16_status check_kt(int64_t K, int32_t T) {
  if (K < W4A16_GROUP || K > kMaxK || K % W4A16_GROUP != 0) return W4A16_ERR_BAD_SHAPE;
  if (T < 1 || T > W4A16_MAX_T) return W4A16_ERR_BAD_SHAPE;
  return W4A16_OK;
}

// The variant a call with T activation rows runs: the selection, except
// that the dot kernel is built for T <= kDotMaxT only; AUTO is the matrix
// cores (measured faster at every T on MI355X).
int resolve_variant(int32_t v, int32_t T) {
  if (v == W4A16_VARIANT_DOT && T <= w4a16::kDotMaxT) return v;
  return W4A16_VARIANT_MFMA;
}

w4a16::Plan make_plan(w4a16::GemvArgs& a, int32_t T) {
  const int v = resolve_variant(current_variant(), T);
  return v == W4A16_VARIANT_DOT ? w4a16::plan_dot(a, T) : w4a16::plan_mfma(a, T, t_cus);
}

w4a16::GemvArgs gemv_args(const uint8_t* packed, const uint16_t* scales, bool tiled, const uint16_t* x, float* y,
                          const int32_t* row_ids, int64_t n_out, int64_t n_rows, int64_t K) {
  w4a16::GemvArgs a{};
  a.packed = packed;
  a.scales = scales;
  a.x = x;
  a.y = y;
  a.row_ids = row_ids;
  a.n_out = n_out;
  a.n_rows = n_rows;
  a.K = (int32_t)K;
  a.G = (int32_t)(K / W4A16_GROUP);
  a.tiled = tiled ? 1 : 0;
  a.tile_bytes = tiled ? w4a16::tiled_tile_bytes(a.G) : 0;
  return a;
}

// Checks shared by both layouts of the gathered head.
w4a16_status check_gather(const int32_t* row_ids, int64_t n_ids, int64_t n_rows, const uint16_t* x_bf16, int64_t K,
                          int32_t T, float* y_f32, int32_t* argmax_id, float* argmax_val, void* workspace,
                          size_t workspace_bytes) {
  if (!x_bf16) return W4A16_ERR_NULL_POINTER;
  if (!y_f32 && !argmax_id) return W4A16_ERR_NULL_POINTER;
  if (argmax_val && !argmax_id) return W4A16_ERR_NULL_POINTER;
  if (n_ids < 1 || n_ids > kMaxRows || n_rows < 1 || n_rows > kMaxRows) return W4A16_ERR_BAD_SHAPE;
  if (!row_ids && n_ids != n_rows) return W4A16_ERR_BAD_SHAPE;
  if (w4a16_status s = check_kt(K, T)) return s;
  if (!aligned(x_bf16, 16) || !aligned(y_f32, 4) || !aligned(row_ids, 4) || !aligned(argmax_id, 4) ||
      !aligned(argmax_val, 4))
    return W4A16_ERR_MISALIGNED;
  if (argmax_id) {
    const int64_t need = (int64_t)w4a16::max_workgroups(n_ids) * T * (int64_t)sizeof(int2);
    if (!workspace || workspace_bytes < (size_t)need || !aligned(workspace, 16)) return W4A16_ERR_WORKSPACE;
  }
  return check_device();
}

// Launches the planned kernel and, when argmax_id is set, the argmax reduction.
w4a16_status run(w4a16::GemvArgs& a, int32_t T, int32_t* argmax_id, float* argmax_val, const w4a16::Plan& p,
                 hipStream_t stream) {
  if (w4a16::launch(a, p, T, stream) != hipSuccess) return W4A16_ERR_HIP;
  if (argmax_id && w4a16::launch_argmax_final(a.partial, p.grid, T, argmax_id, argmax_val, stream) != hipSuccess)
    return W4A16_ERR_HIP;
  return W4A16_OK;
}

// Argmax partials of w4a16_head_gather_noalloc: a static device array, one
// per GPU the library runs on, held until the process ends.  Its host-side
// name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = size_t(1) << 21;  // 2 MiB = W4A16_NOALLOC_SCRATCH_BYTES
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];

// The device address of this device's scratch array (the current device, as
// check_device found it), or nullptr if HIP cannot give it.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

// Grouped launches: table layout and tile choice.
namespace {

constexpr uint32_t kTableMagic = 0x57344231u;  // "W4B1"

struct TableHeader {
  uint32_t magic;
  uint32_t version;
  int32_t count;
  int32_t T;
  int32_t variant;
  int32_t rt;
  int32_t tiled;  // 1: every problem tiled (tiled-layout kernels, one tile per wave); 2: every problem row-major
  int32_t threads;
  int32_t lds;
  int32_t n_argmax;  // argmax records after the count argument records (host copy)
  int64_t grid;
  int64_t ws_bytes;  // workspace w4a16_matmul_batch_ws uses (0: none)
  int64_t reserved;
};
static_assert(sizeof(TableHeader) == 64, "table header size");

// A grouped problem's argmax reduction, launched after the grouped kernel.
struct ArgmaxRecord {
  const int2* partial;
  int64_t nparts;  // the problem's workgroups
  int32_t* id;
  float* val;
};
static_assert(sizeof(ArgmaxRecord) == 32 && sizeof(w4a16::GemvArgs) == 144, "batch table record sizes");

// Tile of grouped launches, from the MI355X sweeps.  All problems tiled:
// at T <= 2 shared workgroups of one tile per wave; above, run workgroups
// of four tiles per wave, a problem whose activations do not fit running
// shared workgroups inside the same kernel.  Eight waves up to T = 6: two
// such workgroups share a CU, and at K = 5,120 each still holds its outputs
// in LDS beside the activations (27B-class body pass at T = 5 and 6: +1.5
// and +1.0 points against runs of six tiles).  From T = 7 sixteen waves,
// one workgroup a CU, whose LDS holds both up to T = 11 (at T = 8: +1.7-2.3
// points against eight waves of six, which must store per tile; at T = 9-10
// about +4); from T = 12 their runs take K in slices to keep the outputs in
// LDS (at T = 12 +0.9 points against runs of three tiles, which fit whole).
// Every problem row-major: up to T = 2 shared workgroups of two 16-row
// tiles per wave, four waves at T = 1 and eight at T = 2 (27B-class body
// pass: 75.3% of 8 TB/s at T = 2 against 70.7% for four waves of four
// tiles), above that the tiled layout's runs (at T = 4 / 8 / 16: 71.4 /
// 64.7 / 58.5% against 70.7 / 63.1 / 56.2% for eight waves of two tiles).
// Both layouts mixed: four waves of two tiles at T = 1, of four from T = 2
// (the same pass row-major with the either-layout kernels: +5.6% at T = 8,
// +8.3% at T = 4 against eight waves of four).  W4A16_BATCH_TILE =
// "split|shared|run,rt,waves" overrides it (for measurement).
w4a16::Tile batch_tile(int T, bool all_tiled, bool all_row, int64_t kmax) {
  w4a16::Tile t;
  if ((all_tiled || all_row) && T > 2)
    t = w4a16::Tile{w4a16::kRun, 4, T <= 6 ? 8 : 16};
  else if (all_tiled)
    t = w4a16::Tile{w4a16::kShared, 1, w4a16::shared_waves(T, kmax)};
  else if (all_row)
    t = w4a16::Tile{w4a16::kShared, 2, T == 1 ? 4 : 8};
  else
    t = T == 1 ? w4a16::Tile{w4a16::kShared, 2, 4} : w4a16::Tile{w4a16::kShared, 4, 4};
  w4a16::tile_override(true, &t);
  return t;
}

// The header of a table written by w4a16_batch_plan, or null.
const TableHeader* valid_table(const void* table_host) {
  if (!table_host || !aligned(table_host, 8)) return nullptr;
  const auto* hdr = static_cast<const TableHeader*>(table_host);
  if (hdr->magic != kTableMagic || hdr->version != W4A16_ABI_VERSION || hdr->count < 1 ||
      hdr->count > W4A16_MAX_BATCH || hdr->T < 1 || hdr->T > W4A16_MAX_T || hdr->grid < 1 || hdr->ws_bytes < 0 ||
      hdr->n_argmax < 0 || hdr->n_argmax > hdr->count)
    return nullptr;
  return hdr;
}

// A planned grouped launch.  Plans need no workspace (ws_bytes 0): the
// workgroups copy every problem's bf16 activations straight into LDS.
w4a16_status run_batch(const void* table_host, const void* table_dev, hipStream_t stream) {
  if (!table_host || !table_dev) return W4A16_ERR_NULL_POINTER;
  if (!aligned(table_dev, 16) || !aligned(table_host, 8)) return W4A16_ERR_MISALIGNED;
  const TableHeader* hdr = valid_table(table_host);
  if (!hdr) return W4A16_ERR_BAD_SHAPE;
  w4a16::Plan p{};
  if (hdr->variant != w4a16::kSplit && hdr->variant != w4a16::kShared && hdr->variant != w4a16::kRun)
    return W4A16_ERR_BAD_SHAPE;
  if (hdr->rt != 1 && hdr->rt != 2 && hdr->rt != 4) return W4A16_ERR_BAD_SHAPE;
  if (hdr->threads < 64 || hdr->threads > 1024 || hdr->threads % 64 || hdr->lds < 0 || hdr->lds > 163840)
    return W4A16_ERR_BAD_SHAPE;
  // layout of the launch's kernels: 0 either (mixed), 1 tiled (one tile per wave), 2 row-major
  if (hdr->tiled < 0 || hdr->tiled > 2 || (hdr->tiled == 1 && hdr->rt != 1)) return W4A16_ERR_BAD_SHAPE;
  if (hdr->variant == w4a16::kRun && hdr->tiled == 0) return W4A16_ERR_BAD_SHAPE;  // runs read one layout
  if (w4a16_status s = check_device()) return s;
  p.variant = hdr->variant;
  p.rt = hdr->rt;
  p.tiled = hdr->tiled == 1;
  p.rowmajor = hdr->tiled == 2;
  p.threads = hdr->threads;
  p.grid = hdr->grid;
  p.lds = hdr->lds;
  const auto* args = reinterpret_cast<const w4a16::GemvArgs*>(static_cast<const TableHeader*>(table_dev) + 1);
  if (w4a16::launch_batch(args, hdr->count, p, hdr->T, stream) != hipSuccess) return W4A16_ERR_HIP;
  const auto* recs = reinterpret_cast<const ArgmaxRecord*>(reinterpret_cast<const w4a16::GemvArgs*>(hdr + 1) +
                                                           hdr->count);
  for (int32_t i = 0; i < hdr->n_argmax; ++i)
    if (w4a16::launch_argmax_final(recs[i].partial, recs[i].nparts, hdr->T, recs[i].id, recs[i].val, stream) !=
        hipSuccess)
      return W4A16_ERR_HIP;
  return W4A16_OK;
}

}  // namespace

extern "C" {

w4a16_status w4a16_matmul(const uint8_t* packed_u4, const uint16_t* scales_bf16, const uint16_t* x_bf16,
                          float* y_f32, int64_t N, int64_t K, int32_t T, hipStream_t stream) {
  if (!packed_u4 || !scales_bf16 || !x_bf16 || !y_f32) return W4A16_ERR_NULL_POINTER;
  if (N < 1 || N > kMaxRows) return W4A16_ERR_BAD_SHAPE;
  if (w4a16_status s = check_kt(K, T)) return s;
  if (!aligned(packed_u4, 16) || !aligned(x_bf16, 16) || !aligned(scales_bf16, 2) || !aligned(y_f32, 4))
    return W4A16_ERR_MISALIGNED;
  if (w4a16_status s = check_device()) return s;
  w4a16::GemvArgs a = gemv_args(packed_u4, scales_bf16, false, x_bf16, y_f32, nullptr, N, N, K);
  const w4a16::Plan p = make_plan(a, T);
  return run(a, T, nullptr, nullptr, p, stream);
}

w4a16_status w4a16_matmul_tiled(const void* tiled, const uint16_t* x_bf16, float* y_f32, int64_t N, int64_t K,
                                int32_t T, hipStream_t stream) {
  if (!tiled || !x_bf16 || !y_f32) return W4A16_ERR_NULL_POINTER;
  if (N < 1 || N > kMaxRows) return W4A16_ERR_BAD_SHAPE;
  if (w4a16_status s = check_kt(K, T)) return s;
  if (!aligned(tiled, 16) || !aligned(x_bf16, 16) || !aligned(y_f32, 4)) return W4A16_ERR_MISALIGNED;
  if (w4a16_status s = check_device()) return s;
  w4a16::GemvArgs a =
      gemv_args(static_cast<const uint8_t*>(tiled), nullptr, true, x_bf16, y_f32, nullptr, N, N, K);
  const w4a16::Plan p = w4a16::plan_mfma(a, T, t_cus);
  return run(a, T, nullptr, nullptr, p, stream);
}

size_t w4a16_workspace_bytes(int64_t n_out, int32_t T) {
  if (n_out < 1 || n_out > kMaxRows || T < 1 || T > W4A16_MAX_T) return 0;
  return (size_t)w4a16::max_workgroups(n_out) * (size_t)T * sizeof(int2);
}

w4a16_status w4a16_head_gather(const int32_t* row_ids, int64_t n_ids, const uint8_t* packed_u4,
                               const uint16_t* scales_bf16, int64_t n_rows, const uint16_t* x_bf16, int64_t K,
                               int32_t T, float* y_f32, int32_t* argmax_id, float* argmax_val, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  if (!packed_u4 || !scales_bf16) return W4A16_ERR_NULL_POINTER;
  if (!aligned(packed_u4, 16) || !aligned(scales_bf16, 2)) return W4A16_ERR_MISALIGNED;
  if (w4a16_status s = check_gather(row_ids, n_ids, n_rows, x_bf16, K, T, y_f32, argmax_id, argmax_val, workspace,
                                    workspace_bytes))
    return s;
  w4a16::GemvArgs a = gemv_args(packed_u4, scales_bf16, false, x_bf16, y_f32, row_ids, n_ids, n_rows, K);
  a.partial = argmax_id ? static_cast<int2*>(workspace) : nullptr;
  const w4a16::Plan p = make_plan(a, T);
  return run(a, T, argmax_id, argmax_val, p, stream);
}

w4a16_status w4a16_head_gather_noalloc(const int32_t* row_ids, int64_t n_ids, const uint8_t* packed_u4,
                                       const uint16_t* scales_bf16, int64_t n_rows, const uint16_t* x_bf16,
                                       int64_t K, int32_t T, float* y_f32, int32_t* argmax_id, float* argmax_val,
                                       hipStream_t stream) {
  static_assert(kScratchBytes == W4A16_NOALLOC_SCRATCH_BYTES, "scratch size in the header");
  if (!packed_u4 || !scales_bf16) return W4A16_ERR_NULL_POINTER;
  if (!aligned(packed_u4, 16) || !aligned(scales_bf16, 2)) return W4A16_ERR_MISALIGNED;
  // the argmax partials must fit the static array; checked before anything else uses it
  if (argmax_id && n_ids >= 1 && n_ids <= kMaxRows && T >= 1 && T <= W4A16_MAX_T &&
      w4a16_workspace_bytes(n_ids, T) > kScratchBytes)
    return W4A16_ERR_SCRATCH;
  if (w4a16_status s = check_gather(row_ids, n_ids, n_rows, x_bf16, K, T, y_f32, argmax_id, argmax_val,
                                    argmax_id ? reinterpret_cast<void*>(kScratchAligned) : nullptr, kScratchBytes))
    return s;
  void* ws = nullptr;
  if (argmax_id && !(ws = scratch_ptr())) return W4A16_ERR_HIP;
  w4a16::GemvArgs a = gemv_args(packed_u4, scales_bf16, false, x_bf16, y_f32, row_ids, n_ids, n_rows, K);
  a.partial = argmax_id ? static_cast<int2*>(ws) : nullptr;
  const w4a16::Plan p = make_plan(a, T);
  return run(a, T, argmax_id, argmax_val, p, stream);
}

w4a16_status w4a16_head_gather_tiled(const int32_t* row_ids, int64_t n_ids, const void* tiled, int64_t n_rows,
                                     const uint16_t* x_bf16, int64_t K, int32_t T, float* y_f32, int32_t* argmax_id,
                                     float* argmax_val, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  if (!tiled) return W4A16_ERR_NULL_POINTER;
  if (!aligned(tiled, 16)) return W4A16_ERR_MISALIGNED;
  if (w4a16_status s = check_gather(row_ids, n_ids, n_rows, x_bf16, K, T, y_f32, argmax_id, argmax_val, workspace,
                                    workspace_bytes))
    return s;
  w4a16::GemvArgs a =
      gemv_args(static_cast<const uint8_t*>(tiled), nullptr, true, x_bf16, y_f32, row_ids, n_ids, n_rows, K);
  a.partial = argmax_id ? static_cast<int2*>(workspace) : nullptr;
  const w4a16::Plan p = w4a16::plan_mfma(a, T, t_cus);
  return run(a, T, argmax_id, argmax_val, p, stream);
}

size_t w4a16_tiled_tile_bytes(int64_t K) {
  if (K < W4A16_GROUP || K > kMaxK || K % W4A16_GROUP != 0) return 0;
  return (size_t)w4a16::tiled_tile_bytes(K / W4A16_GROUP);
}

size_t w4a16_tiled_bytes(int64_t N, int64_t K) {
  if (N < 1 || N > kMaxRows) return 0;
  return (size_t)((N + 15) / 16) * w4a16_tiled_tile_bytes(K);
}

w4a16_status w4a16_repack_tiled(const uint8_t* packed_u4, const uint16_t* scales_bf16, int64_t N, int64_t K,
                                void* tiled, size_t tiled_bytes, hipStream_t stream) {
  if (!packed_u4 || !scales_bf16 || !tiled) return W4A16_ERR_NULL_POINTER;
  if (N < 1 || N > kMaxRows) return W4A16_ERR_BAD_SHAPE;
  if (w4a16_status s = check_kt(K, 1)) return s;
  if (!aligned(packed_u4, 16) || !aligned(scales_bf16, 2) || !aligned(tiled, 16)) return W4A16_ERR_MISALIGNED;
  if (tiled_bytes < w4a16_tiled_bytes(N, K)) return W4A16_ERR_WORKSPACE;
  if (w4a16_status s = check_device()) return s;
  return w4a16::launch_repack(packed_u4, scales_bf16, nullptr, N, N, (int32_t)K, static_cast<uint8_t*>(tiled),
                              stream) == hipSuccess
             ? W4A16_OK
             : W4A16_ERR_HIP;
}

w4a16_status w4a16_repack_tiled_rows(const uint8_t* packed_u4, const uint16_t* scales_bf16, int64_t n_rows, int64_t K,
                                     const int32_t* row_ids, int64_t n_ids, void* tiled, size_t tiled_bytes,
                                     hipStream_t stream) {
  if (!packed_u4 || !scales_bf16 || !row_ids || !tiled) return W4A16_ERR_NULL_POINTER;
  if (n_rows < 1 || n_rows > kMaxRows || n_ids < 1 || n_ids > kMaxRows) return W4A16_ERR_BAD_SHAPE;
  if (w4a16_status s = check_kt(K, 1)) return s;
  if (!aligned(packed_u4, 16) || !aligned(scales_bf16, 2) || !aligned(row_ids, 4) || !aligned(tiled, 16))
    return W4A16_ERR_MISALIGNED;
  if (tiled_bytes < w4a16_tiled_bytes(n_ids, K)) return W4A16_ERR_WORKSPACE;
  if (w4a16_status s = check_device()) return s;
  return w4a16::launch_repack(packed_u4, scales_bf16, row_ids, n_rows, n_ids, (int32_t)K,
                              static_cast<uint8_t*>(tiled), stream) == hipSuccess
             ? W4A16_OK
             : W4A16_ERR_HIP;
}

size_t w4a16_batch_table_bytes(int32_t count) {
  if (count < 1 || count > W4A16_MAX_BATCH) return 0;
  return sizeof(TableHeader) + (size_t)count * (sizeof(w4a16::GemvArgs) + sizeof(ArgmaxRecord));
}

w4a16_status w4a16_batch_plan(const w4a16_problem* problems, int32_t count, int32_t T, void* table_host,
                              size_t table_bytes) {
  if (!problems || !table_host) return W4A16_ERR_NULL_POINTER;
  if (count < 1 || count > W4A16_MAX_BATCH || T < 1 || T > W4A16_MAX_T) return W4A16_ERR_BAD_SHAPE;
  if (table_bytes < w4a16_batch_table_bytes(count) || !aligned(table_host, 8)) return W4A16_ERR_WORKSPACE;
  for (int32_t i = 0; i < count; ++i) {
    const w4a16_problem& q = problems[i];
    if (q.layout != W4A16_LAYOUT_ROW_MAJOR && q.layout != W4A16_LAYOUT_TILED) return W4A16_ERR_BAD_SHAPE;
    if (q.reserved != 0) return W4A16_ERR_BAD_SHAPE;
    const bool tiled = q.layout == W4A16_LAYOUT_TILED;
    if (!q.packed_u4 || (!tiled && !q.scales_bf16) || !q.x_bf16 || !q.y_f32) return W4A16_ERR_NULL_POINTER;
    if (q.N < 1 || q.N > kMaxRows) return W4A16_ERR_BAD_SHAPE;
    if (w4a16_status s = check_kt(q.K, T)) return s;
    if (!aligned(q.packed_u4, 16) || !aligned(q.x_bf16, 16) || (!tiled && !aligned(q.scales_bf16, 2)) ||
        !aligned(q.y_f32, 4) || !aligned(q.argmax_id, 4) || !aligned(q.argmax_val, 4))
      return W4A16_ERR_MISALIGNED;
    if (q.argmax_val && !q.argmax_id) return W4A16_ERR_NULL_POINTER;
    if (q.argmax_id && (!q.workspace || !aligned(q.workspace, 16) ||
                        q.workspace_bytes < w4a16_workspace_bytes(q.N, T)))
      return W4A16_ERR_WORKSPACE;
  }
  auto* hdr = static_cast<TableHeader*>(table_host);
  auto* args = reinterpret_cast<w4a16::GemvArgs*>(hdr + 1);
  auto* recs = reinterpret_cast<ArgmaxRecord*>(args + count);
  bool all_tiled = true, all_row = true;
  int64_t kmax = 0;
  for (int32_t i = 0; i < count; ++i) {
    all_tiled = all_tiled && problems[i].layout == W4A16_LAYOUT_TILED;
    all_row = all_row && problems[i].layout == W4A16_LAYOUT_ROW_MAJOR;
    kmax = std::max(kmax, problems[i].K);
  }
  w4a16::Tile bt = batch_tile(T, all_tiled, all_row, kmax);
  // Every problem runs the same kernel (a run problem whose activations do
  // not fit runs shared workgroups inside the run kernel); a plan that still
  // differs between problems falls back to shared workgroups.
  for (int attempt = 0; attempt < 2; ++attempt) {
    int64_t grid = 0;
    int lds = 0, threads = 64, rt = 0, n_argmax = 0;
    bool uniform = true;
    for (int32_t i = 0; i < count; ++i) {
      const w4a16_problem& q = problems[i];
      const bool tiled = q.layout == W4A16_LAYOUT_TILED;
      w4a16::GemvArgs a = gemv_args(q.packed_u4, tiled ? nullptr : q.scales_bf16, tiled, q.x_bf16, q.y_f32,
                                    nullptr, q.N, q.N, q.K);
      a.partial = q.argmax_id ? static_cast<int2*>(q.workspace) : nullptr;
      const w4a16::Plan p = w4a16::plan_tile(a, T, bt, all_tiled, all_row, true);
      uniform = uniform && p.variant == bt.shape;
      rt = p.rt;
      a.wg_start = grid;
      grid += p.grid;
      lds = std::max(lds, p.lds);
      threads = std::max(threads, p.threads);
      args[i] = a;
      if (q.argmax_id) recs[n_argmax++] = ArgmaxRecord{a.partial, p.grid, q.argmax_id, q.argmax_val};
    }
    if (!uniform) {
      bt = w4a16::Tile{w4a16::kShared, 1, std::min(bt.nw, all_tiled ? 16 : 8)};
      continue;
    }
    if (grid > 0x7fffffffLL) return W4A16_ERR_BAD_SHAPE;
    *hdr = TableHeader{kTableMagic, W4A16_ABI_VERSION, count, T, bt.shape, rt, all_tiled ? 1 : all_row ? 2 : 0, threads,
                       lds, n_argmax, grid, 0, 0};
    return W4A16_OK;
  }
  return W4A16_ERR_BAD_SHAPE;  // not reached: shared tiles always plan
}

size_t w4a16_batch_workspace_bytes(const void* table_host) {
  const TableHeader* hdr = valid_table(table_host);
  return hdr ? (size_t)hdr->ws_bytes : 0;
}

w4a16_status w4a16_matmul_batch(const void* table_host, const void* table_dev, hipStream_t stream) {
  return run_batch(table_host, table_dev, stream);
}

w4a16_status w4a16_matmul_batch_ws(const void* table_host, const void* table_dev, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;  // no plan needs one (w4a16_batch_workspace_bytes is 0)
  (void)workspace_bytes;
  return run_batch(table_host, table_dev, stream);
}

size_t w4a16_topk_workspace_bytes(int64_t n, int32_t T, int32_t k) {
  if (n < 1 || n > kMaxRows || T < 1 || T > W4A16_MAX_T || k < 1 || k > W4A16_MAX_TOPK) return 0;
  return (size_t)T * (size_t)w4a16::topk_chunks(n) * (size_t)k * 8u;
}

w4a16_status w4a16_topk(const float* scores, int64_t n, int32_t T, const int32_t* row_ids, int32_t k,
                        int32_t* top_ids, float* top_vals, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!scores || !top_ids) return W4A16_ERR_NULL_POINTER;
  if (n < 1 || n > kMaxRows || T < 1 || T > W4A16_MAX_T || k < 1 || k > W4A16_MAX_TOPK) return W4A16_ERR_BAD_SHAPE;
  if (!aligned(scores, 4) || !aligned(row_ids, 4) || !aligned(top_ids, 4) || !aligned(top_vals, 4))
    return W4A16_ERR_MISALIGNED;
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < w4a16_topk_workspace_bytes(n, T, k))
    return W4A16_ERR_WORKSPACE;
  if (w4a16_status s = check_device()) return s;
  return w4a16::launch_topk(scores, n, T, row_ids, k, top_ids, top_vals, workspace, stream) == hipSuccess
             ? W4A16_OK
             : W4A16_ERR_HIP;
}

w4a16_status w4a16_greedy_accept(const int32_t* target_ids, const int32_t* draft_ids, int32_t n_seq, int32_t rows,
                                 int32_t* n_accepted, int32_t* tokens, hipStream_t stream) {
  if (!target_ids || !n_accepted || (rows > 1 && !draft_ids)) return W4A16_ERR_NULL_POINTER;
  if (n_seq < 1 || n_seq > W4A16_MAX_BATCH || rows < 1 || rows > W4A16_MAX_T) return W4A16_ERR_BAD_SHAPE;
  if (!aligned(target_ids, 4) || !aligned(draft_ids, 4) || !aligned(n_accepted, 4) || !aligned(tokens, 4))
    return W4A16_ERR_MISALIGNED;
  if (w4a16_status s = check_device()) return s;
  return w4a16::launch_greedy(target_ids, draft_ids, n_seq, rows, n_accepted, tokens, stream) == hipSuccess
             ? W4A16_OK
             : W4A16_ERR_HIP;
}

w4a16_status w4a16_draft_union(const int32_t* base_ids, int32_t n_base, const int32_t* seq_ids, int32_t n_seq,
                               int64_t n_rows, int32_t* union_ids, int32_t* n_union, hipStream_t stream) {
  static_assert(W4A16_MAX_SEQ_IDS == w4a16::kMaxSeqIds && W4A16_MAX_UNION_VOCAB == w4a16::kMaxUnionVocab,
                "limits of the union kernel");
  if (!union_ids || !n_union || (n_base > 0 && !base_ids) || (n_seq > 0 && !seq_ids)) return W4A16_ERR_NULL_POINTER;
  if (n_base < 0 || n_seq < 0 || n_seq > W4A16_MAX_SEQ_IDS || (int64_t)n_base + n_seq < 1 ||
      (int64_t)n_base + n_seq > kMaxRows || n_rows < 1 || n_rows > W4A16_MAX_UNION_VOCAB)
    return W4A16_ERR_BAD_SHAPE;
  if (!aligned(base_ids, 4) || !aligned(seq_ids, 4) || !aligned(union_ids, 4) || !aligned(n_union, 4))
    return W4A16_ERR_MISALIGNED;
  if (w4a16_status s = check_device()) return s;
  return w4a16::launch_draft_union(base_ids, n_base, seq_ids, n_seq, (int)n_rows, union_ids, n_union, stream) ==
                 hipSuccess
             ? W4A16_OK
             : W4A16_ERR_HIP;
}

w4a16_status w4a16_set_tile(int32_t batch, const char* spec) {
  if (batch != 0 && batch != 1) return W4A16_ERR_BAD_SHAPE;
  return w4a16::set_tile_override(batch == 1, spec) ? W4A16_OK : W4A16_ERR_BAD_SHAPE;
}

w4a16_status w4a16_set_variant(int32_t variant) {
  if (variant != W4A16_VARIANT_AUTO && variant != W4A16_VARIANT_DOT && variant != W4A16_VARIANT_MFMA)
    return W4A16_ERR_BAD_VARIANT;
  std::call_once(g_env_once, read_env_variant);
  g_variant.store(variant);
  return W4A16_OK;
}

int32_t w4a16_get_variant(void) { return current_variant(); }

w4a16_status w4a16_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                               hipStream_t stream) {
  if (!src || !sink) return W4A16_ERR_NULL_POINTER;
  if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 50) || workgroups < 1 || workgroups > 65536)
    return W4A16_ERR_BAD_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return W4A16_ERR_MISALIGNED;
  if (w4a16_status s = check_device()) return s;
  return w4a16::launch_stream_read(src, (int64_t)bytes, sink, workgroups, stream) == hipSuccess ? W4A16_OK
                                                                                                   : W4A16_ERR_HIP;
}

const char* w4a16_status_string(int32_t status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_NULL_POINTER: return "a required pointer is NULL";
    case W4A16_ERR_BAD_SHAPE: return "a size is out of range";
    case W4A16_ERR_MISALIGNED: return "a pointer is not aligned as required";
    case W4A16_ERR_WORKSPACE: return "argmax requested without a large enough 16-byte aligned workspace";
    case W4A16_ERR_UNSUPPORTED: return "the current device is not gfx950";
    case W4A16_ERR_HIP: return "a HIP runtime call failed";
    case W4A16_ERR_BAD_VARIANT: return "unknown kernel variant";
    case W4A16_ERR_SCRATCH:
      return "the argmax partials need more than the library's static scratch (W4A16_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int32_t w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

}  // extern "C"
