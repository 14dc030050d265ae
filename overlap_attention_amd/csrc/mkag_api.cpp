// C-ABI layer of the AllGather+GEMM entry points (include/mkag.h): argument
// validation on the host before anything is enqueued, the per-(device, stream)
// workspace (chunk flags, control block, status), the decomposition into staging
// chunks and output tiles, the initial split from the cost model, and the launch.
#include "../../include/mkag.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "mkag_args.h"

extern "C" __attribute__((visibility("hidden"))) hipError_t mkag_kernel_launch(const mkag::Args* a,
                                                                              hipStream_t stream);
extern "C" __attribute__((visibility("hidden"))) hipError_t mkag_kernel_occupancy(int* blocks_per_cu);
// The thread's last-error message, kept by the ring-attention layer for both APIs.
extern "C" __attribute__((visibility("hidden"))) void mkra_set_last_error(const char* msg);

namespace {

mk_status fail(mk_status s, const std::string& msg) {
  mkra_set_last_error(msg.c_str());
  return s;
}
mk_status hip_fail(hipError_t e, const char* what) {
  return fail(MK_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

struct Workspace {
  int device = -1;
  hipStream_t stream = nullptr;
  uint64_t epoch = 0;
  mkag::Ctrl* ctrl = nullptr;
  mkag::Status* status = nullptr;
  uint64_t* flags = nullptr;
  size_t flags_cap = 0;
  uint64_t gathered_epoch = 0;  // epoch of a phase-1 call not yet consumed by phase 2
  uint64_t gathered_sig[8] = {};  // that call's tensors and shape
};

std::mutex g_mu;
std::vector<Workspace*> g_ws;
std::vector<int> g_occ;  // workgroups per CU, per device (0 = not queried yet)
std::vector<int> g_cus;

Workspace* find_ws(int device, hipStream_t stream, bool create) {
  for (Workspace* w : g_ws)
    if (w->device == device && w->stream == stream) return w;
  if (!create) return nullptr;
  Workspace* w = new Workspace();
  w->device = device;
  w->stream = stream;
  g_ws.push_back(w);
  return w;
}

int64_t numel(const mk_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

bool contiguous(const mk_tensor* t) {
  int64_t expect = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->stride[i] != expect) return false;
    expect *= t->shape[i];
  }
  return true;
}

mk_status check_tensor(const mk_tensor* t, const char* name, int ndim) {
  if (t == nullptr) return fail(MK_E_INVAL, std::string(name) + ": null descriptor");
  if (t->ndim != ndim) return fail(MK_E_INVAL, std::string(name) + ": wrong number of dimensions");
  if (t->dtype != MK_BF16) return fail(MK_E_INVAL, std::string(name) + ": must be bf16");
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(MK_E_INVAL, std::string(name) + ": negative extent");
  if (!contiguous(t)) return fail(MK_E_INVAL, std::string(name) + ": not contiguous");
  if (numel(t) > 0) {
    if (t->data == nullptr) return fail(MK_E_INVAL, std::string(name) + ": null data pointer");
    if ((reinterpret_cast<uintptr_t>(t->data) & 15u) != 0)
      return fail(MK_E_INVAL, std::string(name) + ": data not 16-byte aligned");
  }
  return MK_OK;
}

bool overlaps(const mk_tensor* a, const mk_tensor* b) {
  if (numel(a) == 0 || numel(b) == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a->data), a1 = a0 + numel(a) * 2;
  uintptr_t b0 = reinterpret_cast<uintptr_t>(b->data), b1 = b0 + numel(b) * 2;
  return a0 < b1 && b0 < a1;
}

mk_status check_device_pointer(const void* p, int dev, const char* name) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(MK_E_INVAL, std::string(name) + ": not a HIP allocation");
  }
  if (attr.type != hipMemoryTypeDevice || attr.device != dev)
    return fail(MK_E_INVAL, std::string(name) + ": not device memory of the current device");
  return MK_OK;
}

// Same integer Eq. (2) as the kernel.
int eq2_target(int64_t b, int64_t rp, int64_t rs, int64_t cp, int64_t cs) {
  if (rs <= 0) return 0;
  const uint64_t ws = (uint64_t)rs * (uint64_t)cs;
  const uint64_t wt = ws + (uint64_t)(rp > 0 ? rp : 0) * (uint64_t)cp;
  const int64_t n = (int64_t)((2ull * (uint64_t)b * ws + wt) / (2ull * wt));
  const int64_t hi = std::min<int64_t>(b - 1, rs);
  const int64_t lo = hi < 1 ? hi : 1;
  return (int)std::max(lo, std::min(hi, n));
}

mk_status run(const mk_tensor* a_shards, int n_ranks, int rank, const mk_tensor* w, mk_tensor* a_full, mk_tensor* c,
              hipStream_t stream, const mk_ag_gemm_opts* user_opts, mk_ag_gemm_stats* stats) {
  mkra_set_last_error("");
  mk_ag_gemm_opts opts;
  mk_ag_gemm_default_opts(&opts);
  if (user_opts != nullptr) opts = *user_opts;
  mk_status s;
  if ((s = check_tensor(a_shards, "a_shards", 3)) != MK_OK) return s;
  if ((s = check_tensor(w, "w", 2)) != MK_OK) return s;
  if ((s = check_tensor(a_full, "a_full", 2)) != MK_OK) return s;
  if ((s = check_tensor(c, "c", 2)) != MK_OK) return s;
  const int64_t n = a_shards->shape[0], m_loc = a_shards->shape[1], k = a_shards->shape[2];
  const int64_t n_out = w->shape[0];
  if (n_ranks < 1 || n != n_ranks) return fail(MK_E_INVAL, "a_shards.shape[0] must equal n_ranks >= 1");
  if (rank < 0 || rank >= n_ranks) return fail(MK_E_INVAL, "rank must be in [0, n_ranks)");
  if (w->shape[1] != k) return fail(MK_E_INVAL, "w must be [N_out, K] with the K of a_shards");
  if (a_full->shape[0] != n * m_loc || a_full->shape[1] != k) return fail(MK_E_INVAL, "a_full must be [N*M_loc, K]");
  if (c->shape[0] != n * m_loc || c->shape[1] != n_out) return fail(MK_E_INVAL, "c must be [N*M_loc, N_out]");
  if (overlaps(a_full, a_shards) || overlaps(a_full, w) || overlaps(c, a_shards) || overlaps(c, w) ||
      overlaps(c, a_full))
    return fail(MK_E_INVAL, "a_full/c overlap an input or each other");
  if (opts.split_mode != MK_SPLIT_ADAPTIVE && opts.split_mode != MK_SPLIT_FIXED &&
      opts.split_mode != MK_SPLIT_ADAPTIVE_PAPER)
    return fail(MK_E_INVAL, "opts.split_mode");
  if (opts.fixed_staging_wgs < 0 || opts.initial_staging_wgs < 0 || opts.grid_wgs < 0 || opts.spin_timeout_us < 0 ||
      opts.controller_period_us < 0)
    return fail(MK_E_INVAL, "negative option");
  if (opts.phase < 0 || opts.phase > 2) return fail(MK_E_INVAL, "opts.phase must be 0, 1 or 2");
  if (opts.disable_staging != 0 && (opts.disable_staging != 1 || opts.phase != 0))
    return fail(MK_E_INVAL, "opts.disable_staging must be 0, or 1 on the fused call (phase 0)");
  if (m_loc == 0) {
    if (stats != nullptr) std::memset(stats, 0, sizeof(*stats));
    return MK_OK;  // nothing to gather or compute
  }
  if (k == 0 || k % mkag::kBK != 0) return fail(MK_E_UNSUPPORTED, "K must be a positive multiple of 64");
  if (n_out % 8 != 0) return fail(MK_E_UNSUPPORTED, "N_out must be a multiple of 8");
  // K <= 2^22 keeps a lane's byte offset inside a tile (255 rows of 2K bytes) in 32 bits.
  if (m_loc > (1 << 24) || k > (1 << 22) || n_out > (1 << 24) || n > 4096)
    return fail(MK_E_INVAL, "extent too large");

  mkag::Args a;
  std::memset(&a, 0, sizeof(a));
  a.a_shards = static_cast<const uint16_t*>(a_shards->data);
  a.w = static_cast<const uint16_t*>(w->data);
  a.a_full = static_cast<uint16_t*>(a_full->data);
  a.c = static_cast<uint16_t*>(c->data);
  a.n_ranks = (int)n;
  a.rank = rank;
  a.m_loc = (int)m_loc;
  a.k = (int)k;
  a.n_out = (int)n_out;
  a.n_chunks = (int)((m_loc + mkag::kChunkRows - 1) / mkag::kChunkRows);
  a.n_rtiles = (int)((m_loc + mkag::kBM - 1) / mkag::kBM);
  a.n_ntiles = (int)((n_out + mkag::kBN - 1) / mkag::kBN);
  const int64_t n_flags = n * (int64_t)a.n_chunks;
  const int64_t n_stage = n_flags * mkag::kPieces;
  const int64_t n_compute = n * (int64_t)a.n_rtiles * a.n_ntiles;
  if (n_compute > (int64_t)INT32_MAX / 2) return fail(MK_E_INVAL, "too many output tiles");
  a.n_stage_tasks = (int)n_stage;
  a.n_compute = (int)n_compute;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if ((s = check_device_pointer(a_shards->data, dev, "a_shards")) != MK_OK) return s;
  if ((s = check_device_pointer(w->data, dev, "w")) != MK_OK) return s;
  if ((s = check_device_pointer(a_full->data, dev, "a_full")) != MK_OK) return s;
  if (n_out > 0 && (s = check_device_pointer(c->data, dev, "c")) != MK_OK) return s;

  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_occ.size() <= dev) {
    g_occ.resize(dev + 1, 0);
    g_cus.resize(dev + 1, 0);
  }
  if (g_occ[dev] == 0) {
    hipDeviceProp_t prop;
    if ((e = hipGetDeviceProperties(&prop, dev)) != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    int occ = 0;
    if ((e = mkag_kernel_occupancy(&occ)) != hipSuccess) return hip_fail(e, "occupancy query");
    g_occ[dev] = std::max(occ, 1);
    g_cus[dev] = prop.multiProcessorCount;
  }
  const int capacity = g_cus[dev] * g_occ[dev];
  int grid = opts.grid_wgs > 0 ? std::min(opts.grid_wgs, capacity) : capacity;
  grid = (int)std::max<int64_t>(1, std::min<int64_t>(grid, n_compute + std::min<int64_t>(n_stage, 16)));
  a.grid = grid;
  // Queues: one per XCD (workgroup i serves queue i mod n_xcd); queue x owns the column
  // tiles x, x + n_xcd, ..., so the workgroups of one XCD stream the same W rows through
  // its L2 while they walk the chunks in order.
  a.n_xcd = std::max(1, std::min({mkag::kMaxXcd, grid, a.n_ntiles}));
  for (int x = 0; x < a.n_xcd; ++x) a.xcd_ntiles[x] = (a.n_ntiles - x + a.n_xcd - 1) / a.n_xcd;

  // Cost model (controller priors and initial split): an output tile's FLOPs at half of
  // one CU's bf16 MFMA peak (4096 FLOP/clk at 2.4 GHz); a chunk's read + write bytes at
  // 40 GB/s per workgroup. Ticks are 100 MHz.
  const double tile_flops = 2.0 * mkag::kBM * mkag::kBN * (double)k;
  a.cost_compute0 = std::max<int64_t>(1, (int64_t)(tile_flops / (0.5 * 4096.0 * 2.4e9) * 1e8));
  const double piece_bytes = 2.0 * 2.0 * std::min<int64_t>(mkag::kPieceRows, m_loc) * (double)k;
  a.cost_stage0 = std::max<int64_t>(1, (int64_t)(piece_bytes / 40e9 * 1e8));
  a.split_fixed = opts.split_mode == MK_SPLIT_FIXED ? 1 : 0;
  a.ctrl_paper = opts.split_mode == MK_SPLIT_ADAPTIVE_PAPER ? 1 : 0;
  int init;
  if (a.split_fixed)
    init = std::min(opts.fixed_staging_wgs, grid - 1 > 0 ? grid - 1 : 0);
  else if (opts.initial_staging_wgs > 0)
    init = std::min(opts.initial_staging_wgs, grid - 1 > 0 ? grid - 1 : 0);
  else
    init = eq2_target(grid, n_compute, n_stage, a.cost_compute0, a.cost_stage0);
  a.disable_staging = opts.disable_staging ? 1 : 0;
  if (a.disable_staging) init = 0;
  a.initial_stagers = init;
  a.timeout_ticks = (uint64_t)(opts.spin_timeout_us > 0 ? opts.spin_timeout_us : 10000000) * 100ull;
  a.ctrl_period_ticks = (uint64_t)(opts.controller_period_us > 0 ? opts.controller_period_us : 20) * 100ull;

  Workspace* ws = find_ws(dev, stream, true);
  if (ws->ctrl == nullptr) {
    if ((e = hipMalloc(reinterpret_cast<void**>(&ws->ctrl), sizeof(mkag::Ctrl))) != hipSuccess)
      return hip_fail(e, "workspace allocation");
    if ((e = hipMalloc(reinterpret_cast<void**>(&ws->status), sizeof(mkag::Status))) != hipSuccess)
      return hip_fail(e, "workspace allocation");
    if ((e = hipMemsetAsync(ws->ctrl, 0, sizeof(mkag::Ctrl), stream)) != hipSuccess) return hip_fail(e, "memset");
    if ((e = hipMemsetAsync(ws->status, 0, sizeof(mkag::Status), stream)) != hipSuccess) return hip_fail(e, "memset");
  }
  if (ws->flags == nullptr || ws->flags_cap < (size_t)n_flags) {
    if (ws->flags != nullptr) {
      if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
      hipFree(ws->flags);
      ws->flags = nullptr;
    }
    if ((e = hipMalloc(reinterpret_cast<void**>(&ws->flags), (size_t)n_flags * sizeof(uint64_t))) != hipSuccess)
      return hip_fail(e, "workspace allocation");
    if ((e = hipMemsetAsync(ws->flags, 0, (size_t)n_flags * sizeof(uint64_t), stream)) != hipSuccess)
      return hip_fail(e, "memset");
    ws->flags_cap = (size_t)n_flags;
  }
  a.flags = ws->flags;
  a.ctrl = ws->ctrl;
  a.status = ws->status;
  // Unfused phases: the gather stages every chunk with every workgroup and computes
  // nothing; the GEMM stages nothing and consumes the flags the gather just stamped,
  // under the gather's epoch.
  const uint64_t sig[8] = {(uint64_t)(uintptr_t)a.a_shards, (uint64_t)(uintptr_t)a.a_full, (uint64_t)(uintptr_t)a.w,
                           (uint64_t)(uintptr_t)a.c, (uint64_t)n, (uint64_t)m_loc, (uint64_t)k,
                           ((uint64_t)n_out << 32) | (uint32_t)rank};
  if (opts.phase == 1) {
    std::memcpy(ws->gathered_sig, sig, sizeof(sig));
    for (int x = 0; x < a.n_xcd; ++x) a.xcd_ntiles[x] = 0;
    a.n_compute = 0;
    a.split_fixed = 1;
    a.initial_stagers = grid;
    a.epoch = ++ws->epoch;
    ws->gathered_epoch = a.epoch;
  } else if (opts.phase == 2) {
    if (ws->gathered_epoch == 0 || ws->gathered_epoch != ws->epoch ||
        std::memcmp(ws->gathered_sig, sig, sizeof(sig)) != 0)
      return fail(MK_E_INVAL, "opts.phase 2 needs a phase-1 call with the same arguments just before it on this stream");
    a.n_stage_tasks = 0;
    a.split_fixed = 1;
    a.initial_stagers = 0;
    a.epoch = ws->epoch;
    ws->gathered_epoch = 0;
  } else {
    a.epoch = ++ws->epoch;
  }
  if ((e = mkag_kernel_launch(&a, stream)) != hipSuccess) return hip_fail(e, "kernel launch");

  if (stats != nullptr) {
    std::memset(stats, 0, sizeof(*stats));
    mkag::Status ds;
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if ((e = hipMemcpy(&ds, ws->status, sizeof(ds), hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "hipMemcpy");
    stats->status = ds.last_error ? MK_E_TIMEOUT : MK_OK;
    stats->grid_wgs = grid;
    stats->compute_tiles = a.n_compute;
    stats->staging_tasks = a.n_stage_tasks;
    stats->compute_done = ds.compute_done;
    stats->staging_done = ds.stage_done;
    stats->assist_tasks = ds.assist_tasks;
    stats->controller_updates = ds.ctrl_updates;
    stats->max_staging_wgs = ds.max_stage;
    stats->final_target = ds.final_target;
    stats->compute_busy_ticks = ds.compute_ticks;
    stats->compute_wait_ticks = ds.compute_wait_ticks;
    stats->staging_busy_ticks = ds.stage_ticks;
    stats->kernel_ticks = ds.kernel_ticks;
    stats->wg_cycles = ds.wg_cycles;
    stats->wg_ticks = ds.wg_ticks;
  }
  return MK_OK;
}

}  // namespace

// Frees the AllGather+GEMM workspaces (called by mk_release_workspace).
extern "C" __attribute__((visibility("hidden"))) void mkag_release_workspaces(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  for (Workspace* w : g_ws) {
    int cur = 0;
    hipGetDevice(&cur);
    hipSetDevice(w->device);
    hipStreamSynchronize(w->stream);
    hipFree(w->ctrl);
    hipFree(w->status);
    hipFree(w->flags);
    hipSetDevice(cur);
    delete w;
  }
  g_ws.clear();
}

extern "C" {

void mk_ag_gemm_default_opts(mk_ag_gemm_opts* opts) {
  if (opts == nullptr) return;
  std::memset(opts, 0, sizeof(*opts));
  opts->split_mode = MK_SPLIT_ADAPTIVE;
}

mk_status mk_allgather_gemm(const mk_tensor* a_shards, int n_ranks, int rank, const mk_tensor* w, mk_tensor* a_full,
                            mk_tensor* c, hipStream_t stream) {
  return run(a_shards, n_ranks, rank, w, a_full, c, stream, nullptr, nullptr);
}

mk_status mk_allgather_gemm_ex(const mk_tensor* a_shards, int n_ranks, int rank, const mk_tensor* w,
                               mk_tensor* a_full, mk_tensor* c, hipStream_t stream, const mk_ag_gemm_opts* opts,
                               mk_ag_gemm_stats* stats) {
  return run(a_shards, n_ranks, rank, w, a_full, c, stream, opts, stats);
}

mk_status mk_ag_gemm_status(hipStream_t stream) {
  mkra_set_last_error("");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  Workspace* w = find_ws(dev, stream, false);
  if (w == nullptr || w->status == nullptr) return MK_OK;
  uint32_t sticky = 0;
  if ((e = hipMemcpy(&sticky, &w->status->sticky_error, sizeof(sticky), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  if (sticky == 0) return MK_OK;
  const uint32_t zero = 0;
  if ((e = hipMemcpy(&w->status->sticky_error, &zero, sizeof(zero), hipMemcpyHostToDevice)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  return fail(MK_E_TIMEOUT, "a bounded wait of an AllGather+GEMM call expired (status of an earlier call)");
}

}  // extern "C"
