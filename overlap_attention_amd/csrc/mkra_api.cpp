// C-ABI layer of mkra: argument validation (on the host, before anything is
// enqueued), the per-(device, stream) workspace, the decomposition of the problem
// into compute units and staging tasks, the initial staging split, and the launch of
// the persistent kernel. See include/mkra.h for the contract of each entry point.
#include "../../include/mkra.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "mkra_args.h"

extern "C" __attribute__((visibility("hidden"))) hipError_t mkra_kernel_launch(const mkra::KernelArgs* a,
                                                                              hipStream_t stream);
extern "C" __attribute__((visibility("hidden"))) hipError_t mkra_kernel_occupancy(int d, int* blocks_per_cu);
extern "C" __attribute__((visibility("hidden"))) hipError_t mkra_scratch_address(int device, void** ptr);
extern "C" __attribute__((visibility("hidden"))) hipError_t mkra_zero_launch(void* p, uint64_t bytes,
                                                                            hipStream_t stream);

static_assert(mkra::kScratchBytes == MKRA_NOALLOC_SCRATCH_BYTES, "scratch size in the header");

namespace {

using mkra::DevCtrl;
using mkra::DevStatus;
using mkra::TraceRec;

thread_local std::string g_last_error;

mk_status fail(mk_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

mk_status hip_fail(hipError_t e, const char* what) {
  return fail(MK_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

struct Workspace {
  int device = -1;
  hipStream_t stream = nullptr;
  uint64_t epoch = 0;
  DevCtrl* ctrl = nullptr;
  DevStatus* status = nullptr;
  uint32_t* done_count = nullptr;
  size_t done_cap = 0;
  uint64_t* slot_flags = nullptr;
  size_t tiles_cap = 0;
  uint64_t* unit_flags = nullptr;
  size_t units_cap = 0;
  uint8_t* slots = nullptr;
  size_t slot_bytes_cap = 0;
  float* acc = nullptr;
  size_t acc_cap = 0;
  TraceRec* trace = nullptr;
  int trace_cap = 0;
  bool traced_last = false;
  // The unfused baseline: the control block and status of its staging launches (which
  // run beside its compute launches), and one event per step and stream.
  DevCtrl* ctrl_copy = nullptr;
  DevStatus* status_copy = nullptr;
  std::vector<hipEvent_t> ev_staged, ev_computed;
};

std::mutex g_mu;
std::vector<Workspace*> g_ws;

// State of the entry point that allocates nothing, per device: whether its scratch
// array has been set up (status word cleared) and the epoch of its last launch.
struct ScratchState {
  bool ready = false;
  uint64_t epoch = 0;
};
std::vector<ScratchState> g_scratch;

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

struct DeviceInfo {
  int cus = 0;
  int occ[2] = {0, 0};  // blocks per CU for D = 64, 128
};
std::vector<DeviceInfo> g_dev;

template <class T>
hipError_t grow(T** p, size_t* cap, size_t need, hipStream_t s, bool zero) {
  if (need <= *cap && *p != nullptr) return hipSuccess;
  hipError_t e;
  if (*p != nullptr) {
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
    if ((e = hipFree(*p)) != hipSuccess) return e;
    *p = nullptr;
    *cap = 0;
  }
  size_t n = std::max<size_t>(need, 1);
  if ((e = hipMalloc(reinterpret_cast<void**>(p), n * sizeof(T))) != hipSuccess) return e;
  if (zero && (e = hipMemsetAsync(*p, 0, n * sizeof(T), s)) != hipSuccess) return e;
  *cap = n;
  return hipSuccess;
}

void free_ws(Workspace* w) {
  if (w->stream != nullptr || w->device >= 0) {
    int cur = 0;
    hipGetDevice(&cur);
    hipSetDevice(w->device);
    hipStreamSynchronize(w->stream);
    hipFree(w->ctrl);
    hipFree(w->status);
    hipFree(w->done_count);
    hipFree(w->slot_flags);
    hipFree(w->unit_flags);
    hipFree(w->slots);
    hipFree(w->acc);
    hipFree(w->trace);
    hipFree(w->ctrl_copy);
    hipFree(w->status_copy);
    for (hipEvent_t ev : w->ev_staged) hipEventDestroy(ev);
    for (hipEvent_t ev : w->ev_computed) hipEventDestroy(ev);
    hipSetDevice(cur);
  }
  delete w;
}

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

// Contiguous row-major check; strides of extent-1 dimensions are not checked.
bool contiguous(const mk_tensor* t) {
  int64_t expect = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->stride[i] != expect) return false;
    expect *= t->shape[i];
  }
  return true;
}

mk_status check_tensor(const mk_tensor* t, const char* name, int ndim, int dtype) {
  if (t == nullptr) return fail(MK_E_INVAL, std::string(name) + ": null descriptor");
  if (t->ndim != ndim) return fail(MK_E_INVAL, std::string(name) + ": wrong number of dimensions");
  if (t->dtype != dtype) return fail(MK_E_INVAL, std::string(name) + ": wrong dtype");
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

bool overlaps(const mk_tensor* a, int64_t ea, const mk_tensor* b, int64_t eb) {
  if (numel(a) == 0 || numel(b) == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a->data), a1 = a0 + numel(a) * ea;
  uintptr_t b0 = reinterpret_cast<uintptr_t>(b->data), b1 = b0 + numel(b) * eb;
  return a0 < b1 && b0 < a1;
}

// The status a set of device-side error bits reports: a V outside the fp16 range of
// the PV operand first (the launch ended because of it), then an expired wait.
mk_status device_status(uint32_t bits) {
  if (bits & mkra::kErrRange) return MK_E_UNSUPPORTED;
  if (bits & mkra::kErrTimeout) return MK_E_TIMEOUT;
  return bits != 0 ? MK_E_HIP : MK_OK;
}

const char* device_message(uint32_t bits) {
  if (bits & mkra::kErrRange)
    return "a staged V value is outside the fp16 range of the PV operand (|v| >= 65536 or not finite); "
           "the call's outputs are undefined (status of an earlier call on this stream)";
  return "a bounded wait on the GPU expired (status of an earlier call on this stream)";
}

// Same integer Eq. (2) as the kernel's controller.
int eq2_target_host(int64_t b, int64_t rp, int64_t rs, int64_t cp, int64_t cs) {
  if (rs <= 0) return 0;
  uint64_t ws = (uint64_t)rs * (uint64_t)cs;
  uint64_t w = ws + (uint64_t)(rp > 0 ? rp : 0) * (uint64_t)cp;
  int64_t n = (int64_t)((2ull * (uint64_t)b * ws + w) / (2ull * w));
  int64_t hi = std::min<int64_t>(b - 1, rs);
  int64_t lo = hi < 1 ? hi : 1;
  return (int)std::max(lo, std::min(hi, n));
}

// Step groups unless the options say otherwise. A task boundary costs about the same
// whatever the step's size (state store and reload, publish, claim), while a longer
// task leaves workgroups idle longer at the end of the launch. Measured on MI355X
// (same-box A/B): steps of Lk*D < 2^19 key-dims (the 32K-token MHA D=64 workload,
// 1024-token chunks) run best in four-step tasks, 2-9% faster than two-step ones; the
// 64K-token GQA workload (Lk*D = 2^19) runs best in two-step tasks (0.6-0.9% faster
// than four with a tail). Above that it depends on the size with no clear rule: four
// steps with a tail were 0.9% and 1.8% faster at 96K and 128K tokens and 1.5% slower
// at 192K (same box), so two-step tasks stay the default there. A tail of shorter tasks
// (the last kDefaultTailSteps steps in tasks of kDefaultTailStepsPerTask) applies only
// to four-step tasks when the units outnumber the workgroups.
constexpr int kDefaultTailStepsPerTask = 2;
constexpr int kDefaultTailSteps = 4;
int default_steps_per_task(int64_t lk, int64_t d) { return lk * d >= (int64_t(1) << 19) ? 2 : 4; }

// Staging pieces per tile when opts.stage_pieces is 0: two when a step has few tiles
// (at most 8: the first tiles' staging latency is on the critical path of a short
// launch, and two pieces let two workgroups stage a tile at once) or a tile is large
// (>= 1 MB), else one. Measured on the 1K-token MHA workload (8 tiles of 1 MB), the
// 6K-24K-token GQA rings (3-12 tiles of 512 KB) and the 32K-token D = 64 ring (16
// tiles of 2 MB): more pieces than this add per-task costs (the slot check, the
// publish) that outweigh the parallelism.
int default_stage_pieces(int64_t n_tiles, int64_t tile_bytes) {
  return (n_tiles <= 8 || tile_bytes >= (int64_t(1) << 20)) ? 2 : 1;
}


// Largest divisor of g that divides the wave count: query heads per unit.
int heads_per_unit(int g) {
  int best = 1;
  for (int d = 1; d <= mkra::kWaves; ++d)
    if (g % d == 0 && mkra::kWaves % d == 0) best = d;
  return best;
}

mk_status device_info(int dev, DeviceInfo** out) {
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  DeviceInfo& di = g_dev[dev];
  if (di.cus == 0) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    int o64 = 0, o128 = 0;
    if ((e = mkra_kernel_occupancy(64, &o64)) != hipSuccess) return hip_fail(e, "occupancy query");
    if ((e = mkra_kernel_occupancy(128, &o128)) != hipSuccess) return hip_fail(e, "occupancy query");
    di.cus = prop.multiProcessorCount;
    di.occ[0] = std::max(o64, 1);
    di.occ[1] = std::max(o128, 1);
  }
  *out = &di;
  return MK_OK;
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

// The unfused baseline of the mKernel paper's Figure 1(b): two streams, every chunk
// released at a kernel boundary. For each ring step t, the copy stream runs a
// staging-only launch of the ring kernel (copy_wgs workgroups, the step's tiles into
// slot t mod kSlots, after waiting for the compute launch of step t - kSlots that last
// read that slot), and the compute stream, after waiting for that staging launch, runs
// a compute-only launch over every unit's step t (the remaining workgroups; the running
// state goes through the workspace between the steps). Both use the kernel's own device
// code; the staging launches have their own control block, since they run beside the
// compute launches. `a` holds the fused decomposition; all launches share its epoch.
mk_status launch_unfused(const mkra::KernelArgs& a, Workspace* w, hipStream_t stream, hipStream_t copy_stream,
                         int copy_wgs, int64_t n_units) {
  hipError_t e;
  if (w->ctrl_copy == nullptr) {
    if ((e = hipMalloc(reinterpret_cast<void**>(&w->ctrl_copy), sizeof(DevCtrl))) != hipSuccess)
      return hip_fail(e, "workspace allocation");
    if ((e = hipMalloc(reinterpret_cast<void**>(&w->status_copy), sizeof(DevStatus))) != hipSuccess)
      return hip_fail(e, "workspace allocation");
    if ((e = hipMemsetAsync(w->ctrl_copy, 0, sizeof(DevCtrl), stream)) != hipSuccess) return hip_fail(e, "memset");
    if ((e = hipMemsetAsync(w->status_copy, 0, sizeof(DevStatus), stream)) != hipSuccess)
      return hip_fail(e, "memset");
  }
  const int n_steps = a.n_steps;
  while ((int)w->ev_staged.size() < n_steps) {
    hipEvent_t e1, e2;
    if ((e = hipEventCreateWithFlags(&e1, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "event");
    if ((e = hipEventCreateWithFlags(&e2, hipEventDisableTiming)) != hipSuccess) return hip_fail(e, "event");
    w->ev_staged.push_back(e1);
    w->ev_computed.push_back(e2);
  }
  // Workgroups: copy_wgs stage; the rest of the grid computes (both resident at once).
  const int grid_all = a.grid;
  const int n_copy = std::max(1, std::min(copy_wgs, grid_all > 1 ? grid_all - 1 : 1));
  const int n_comp = std::max(1, (int)std::min<int64_t>(grid_all - n_copy, n_units));

  mkra::KernelArgs st = a;  // staging launches
  st.grid = n_copy;
  st.n_xcd = 1;
  for (int x = 0; x <= mkra::kMaxXcd; ++x) st.xcd_unit_begin[x] = 0;
  st.n_groups = 0;  // no compute task
  st.n_stage_tasks = a.stage_per_step;
  st.split_fixed = 1;
  st.initial_stagers = n_copy;
  st.disable_staging = 0;
  st.external_order = 1;
  st.ctrl = w->ctrl_copy;
  st.status = w->status_copy;
  st.trace = nullptr;
  st.trace_cap = 0;

  mkra::KernelArgs cp = a;  // compute launches: one step each
  cp.grid = n_comp;
  cp.n_xcd = std::min(mkra::kMaxXcd, n_comp);
  for (int x = 0; x <= cp.n_xcd; ++x) cp.xcd_unit_begin[x] = (int)((int64_t)x * n_units / cp.n_xcd);
  cp.group = 1;
  cp.tail_group = 1;
  cp.n_big = 1;
  cp.n_groups = 1;
  cp.n_stage_tasks = 0;
  cp.split_fixed = 1;
  cp.initial_stagers = 0;
  cp.disable_staging = 1;
  cp.external_order = 1;
  cp.trace = nullptr;
  cp.trace_cap = 0;

  // The copy stream starts after everything enqueued on the compute stream so far
  // (earlier calls that used the same workspace).
  if ((e = hipEventRecord(w->ev_computed[0], stream)) != hipSuccess) return hip_fail(e, "event record");
  if ((e = hipStreamWaitEvent(copy_stream, w->ev_computed[0], 0)) != hipSuccess) return hip_fail(e, "event wait");
  for (int t = 0; t < n_steps; ++t) {
    if (t >= mkra::kSlots && (e = hipStreamWaitEvent(copy_stream, w->ev_computed[t - mkra::kSlots], 0)) != hipSuccess)
      return hip_fail(e, "event wait");
    st.stage_lo = t * a.stage_per_step;
    if ((e = mkra_kernel_launch(&st, copy_stream)) != hipSuccess) return hip_fail(e, "kernel launch");
    if ((e = hipEventRecord(w->ev_staged[t], copy_stream)) != hipSuccess) return hip_fail(e, "event record");
    if ((e = hipStreamWaitEvent(stream, w->ev_staged[t], 0)) != hipSuccess) return hip_fail(e, "event wait");
    cp.step_lo = t;
    if ((e = mkra_kernel_launch(&cp, stream)) != hipSuccess) return hip_fail(e, "kernel launch");
    if ((e = hipEventRecord(w->ev_computed[t], stream)) != hipSuccess) return hip_fail(e, "event record");
  }
  // The compute stream's last launch follows every staging launch (it waited for the
  // last one), so work enqueued after the call on `stream` sees the whole call done.
  return MK_OK;
}

// no_alloc: take every piece of device state from the fixed scratch array of the
// current device instead of the per-(device, stream) workspace, and call nothing that
// allocates device memory.
// copy_stream != nullptr: the unfused two-stream baseline (staging launches on
// copy_stream with copy_wgs workgroups, one compute launch per step on stream).
mk_status run(const mk_tensor* q, const mk_tensor* kv, int n_chunks, int rank, int causal, int gqa, mk_tensor* out,
              mk_tensor* lse, hipStream_t stream, const mk_ring_attn_opts* user_opts, mk_ring_attn_stats* stats,
              bool no_alloc = false, hipStream_t copy_stream = nullptr, int copy_wgs = 0) {
  g_last_error.clear();
  mk_ring_attn_opts opts;
  mk_ring_attn_default_opts(&opts);
  if (user_opts != nullptr) opts = *user_opts;
  mk_status s;
  if ((s = check_tensor(q, "q", 3, MK_BF16)) != MK_OK) return s;
  if ((s = check_tensor(kv, "kv_chunks", 5, MK_BF16)) != MK_OK) return s;
  if ((s = check_tensor(out, "out", 3, MK_BF16)) != MK_OK) return s;
  if ((s = check_tensor(lse, "lse", 2, MK_F32)) != MK_OK) return s;
  const int64_t lq = q->shape[0], hq = q->shape[1], d = q->shape[2];
  const int64_t nch = kv->shape[0], lk = kv->shape[2], hkv = kv->shape[3];
  if (n_chunks < 1 || nch != n_chunks) return fail(MK_E_INVAL, "kv_chunks.shape[0] must equal n_chunks >= 1");
  if (kv->shape[1] != 2) return fail(MK_E_INVAL, "kv_chunks.shape[1] must be 2 (K, V)");
  if (rank < 0 || rank >= n_chunks) return fail(MK_E_INVAL, "rank must be in [0, n_chunks)");
  if (gqa < 1) return fail(MK_E_INVAL, "gqa_ratio must be >= 1");
  if (kv->shape[4] != d) return fail(MK_E_INVAL, "head_dim of q and kv_chunks differ");
  if (hq != (int64_t)gqa * hkv) return fail(MK_E_INVAL, "Hq must equal gqa_ratio * Hkv");
  if (out->shape[0] != lq || out->shape[1] != hq || out->shape[2] != d)
    return fail(MK_E_INVAL, "out must have the shape of q");
  if (lse->shape[0] != hq || lse->shape[1] != lq) return fail(MK_E_INVAL, "lse must be [Hq, Lq]");
  if (causal != 0 && lq != lk) return fail(MK_E_INVAL, "causal needs Lq == Lk");
  if (overlaps(out, 2, q, 2) || overlaps(out, 2, kv, 2) || overlaps(lse, 4, q, 2) || overlaps(lse, 4, kv, 2) ||
      overlaps(lse, 4, out, 2))
    return fail(MK_E_INVAL, "out/lse overlap an input or each other");
  if (opts.split_mode != MK_SPLIT_ADAPTIVE && opts.split_mode != MK_SPLIT_FIXED &&
      opts.split_mode != MK_SPLIT_ADAPTIVE_PAPER)
    return fail(MK_E_INVAL, "opts.split_mode");
  if (opts.steps_per_task < 0 || opts.steps_per_task > mkra::kMaxGroup)
    return fail(MK_E_INVAL, "opts.steps_per_task must be 0 (default) or 1..4");
  if (opts.tail_steps_per_task < 0 || opts.tail_steps_per_task > mkra::kMaxGroup)
    return fail(MK_E_INVAL, "opts.tail_steps_per_task must be 0 (default) or 1..4");
  if (opts.parallel_steps < -1 || opts.parallel_steps > 1)
    return fail(MK_E_INVAL, "opts.parallel_steps must be -1, 0 or 1");
  if (opts.stage_pieces < 0) return fail(MK_E_INVAL, "opts.stage_pieces must be 0 (default) or positive");
  if (opts.fixed_staging_wgs < 0 || opts.initial_staging_wgs < 0 || opts.grid_wgs < 0 || opts.spin_timeout_us < 0 ||
      opts.controller_period_us < 0 || opts.trace_capacity < 0 || opts.stage_delay_ticks < 0)
    return fail(MK_E_INVAL, "negative option");
  if (lq == 0 || hq == 0) {
    if (stats != nullptr) std::memset(stats, 0, sizeof(*stats));
    return MK_OK;  // nothing to compute
  }
  if (lk == 0) return fail(MK_E_INVAL, "Lk == 0: no keys to attend to");
  if (d != 64 && d != 128) return fail(MK_E_UNSUPPORTED, "head_dim must be 64 or 128");
  const int n_steps = causal ? rank + 1 : n_chunks;
  if (n_steps > (1 << 20) - 2) return fail(MK_E_INVAL, "too many ring steps");
  if (lq > (1 << 30) || lk > (1 << 30) || hq > (1 << 20)) return fail(MK_E_INVAL, "extent too large");

  // Decomposition.
  mkra::KernelArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q->data);
  a.kv = static_cast<const uint16_t*>(kv->data);
  a.out = static_cast<uint16_t*>(out->data);
  a.lse = static_cast<float*>(lse->data);
  a.lq = (int)lq; a.lk = (int)lk; a.hq = (int)hq; a.hkv = (int)hkv; a.d = (int)d; a.gqa = gqa;
  a.n_chunks = n_chunks; a.rank = rank; a.causal = causal ? 1 : 0; a.n_steps = n_steps;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  a.hg = heads_per_unit(gqa);
  a.n_hgroups = gqa / a.hg;
  a.bq = (mkra::kWaves / a.hg) * mkra::kRowsPerWave;
  a.n_qblocks = (int)((lq + a.bq - 1) / a.bq);
  const int64_t n_units = hkv * a.n_hgroups * (int64_t)a.n_qblocks;
  if (n_units > (1 << 26)) return fail(MK_E_INVAL, "too many compute units");
  a.n_units = (int)n_units;
  a.n_tiles = (int)((lk + mkra::kStageRows - 1) / mkra::kStageRows);
  // Blocks per KV head, padded to whole tiles: a tile always stages kStageRows / kBN
  // blocks (keys past Lk as zeros), so a compute phase of two blocks (D = 64) never
  // reaches past its head's blocks.
  a.n_blocks = a.n_tiles * (mkra::kStageRows / mkra::kBN);
  // A tile's KV heads in pieces of piece_heads heads, one staging task and one ready
  // flag each.
  {
    const int64_t tile_bytes = 2 * 2 * std::min<int64_t>(mkra::kStageRows, lk) * hkv * d;
    const int pieces = (int)std::min<int64_t>(
        hkv, opts.stage_pieces > 0 ? opts.stage_pieces : default_stage_pieces(a.n_tiles, tile_bytes));
    a.piece_heads = (int)((hkv + pieces - 1) / pieces);
    a.n_pieces = (int)((hkv + a.piece_heads - 1) / a.piece_heads);
  }
  if ((int64_t)a.n_tiles * a.n_pieces > (int64_t)INT32_MAX / 2) return fail(MK_E_INVAL, "too many staging tasks");
  a.stage_per_step = a.n_tiles * a.n_pieces;
  // Every step's chunk, the local one included, is staged once into the layout the
  // compute role reads.
  const int64_t n_stage_tasks = (int64_t)n_steps * a.stage_per_step;
  if (n_stage_tasks > (int64_t)INT32_MAX - 1) return fail(MK_E_INVAL, "too many staging tasks");
  a.n_stage_tasks = (int)n_stage_tasks;
  a.chunk_elems = 2 * lk * hkv * d;
  const int64_t block_bytes = 2 * (int64_t)mkra::kBN * d * 2;
  a.slot_bytes = hkv * (int64_t)a.n_blocks * block_bytes;

  // Device state.
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if ((s = check_device_pointer(q->data, dev, "q")) != MK_OK) return s;
  if ((s = check_device_pointer(kv->data, dev, "kv_chunks")) != MK_OK) return s;
  if ((s = check_device_pointer(out->data, dev, "out")) != MK_OK) return s;
  if ((s = check_device_pointer(lse->data, dev, "lse")) != MK_OK) return s;

  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo* di = nullptr;
  if ((s = device_info(dev, &di)) != MK_OK) return s;
  const int capacity = di->cus * di->occ[d == 128 ? 1 : 0];
  int grid = opts.grid_wgs > 0 ? std::min(opts.grid_wgs, capacity) : capacity;
  // Parallel step groups: by default when the units fill at most half of the device's
  // workgroup slots, so that a unit's ring steps, run at once and merged, spread the
  // work (the unfused baseline runs one step per launch and keeps the carried state).
  // The choice and the group size depend on the device, not on opts.grid_wgs, so a
  // smaller grid gives the same result bits.
  a.parallel_steps =
      n_steps > 1 && copy_stream == nullptr &&
              (opts.parallel_steps > 0 || (opts.parallel_steps == 0 && n_units * 2 <= (int64_t)capacity))
          ? 1
          : 0;

  // Step groups: `group` steps each, except the last tail_steps steps, which run in
  // groups of tail_group (shorter tasks at the end shorten the launch's tail). With
  // parallel groups the default is a quarter of the steps, 2..4: a task's fixed costs
  // (flags, pipeline fill, the partial's store and merge) weigh about as much as one
  // step of a small problem, so one-step tasks lose to longer ones (measured on the
  // 8K-token and 6K-24K-token workloads).
  const int parallel_group = std::max(2, std::min(mkra::kMaxGroup, n_steps / 4));
  a.group = opts.steps_per_task > 0 ? opts.steps_per_task
            : a.parallel_steps      ? parallel_group
                                    : default_steps_per_task(lk, d);
  a.tail_group = opts.tail_steps_per_task > 0 ? std::min(opts.tail_steps_per_task, a.group)
                                              : std::min(kDefaultTailStepsPerTask, a.group);
  {
    // By default only a sequential launch whose units outnumber its workgroups (several
    // rounds of tasks) has a tail; with fewer units every task starts at once. Parallel
    // groups take no default tail: their grouping sets the merge, and it must not
    // depend on the grid.
    const int tail_default =
        (!a.parallel_steps && a.group > kDefaultTailStepsPerTask && n_units > (int64_t)grid) ? kDefaultTailSteps : 0;
    const int tail_steps = opts.tail_steps > 0 ? opts.tail_steps : opts.tail_steps < 0 ? 0 : tail_default;
    a.n_big = std::max(0, n_steps - tail_steps) / a.group;
    const int rest = n_steps - a.n_big * a.group;
    a.n_groups = a.n_big + (rest + a.tail_group - 1) / a.tail_group;
  }
  // No more workgroups than tasks can use at once.
  const int64_t useful = n_units * (a.parallel_steps ? (int64_t)a.n_groups : 1) + std::min<int64_t>(n_stage_tasks, 16);
  grid = (int)std::max<int64_t>(1, std::min<int64_t>(grid, useful));
  a.grid = grid;
  a.n_xcd = std::min(mkra::kMaxXcd, grid);
  for (int x = 0; x <= a.n_xcd; ++x) a.xcd_unit_begin[x] = (int)((int64_t)x * n_units / a.n_xcd);
  // Staging order. With parallel step groups every group's first step is needed at
  // once, so when no slot is reused (n_steps <= kSlots: staging never waits for a free
  // slot) the steps are staged group-interleaved: every group's first step, then every
  // group's second, and so on. Otherwise step by step, the order slot reuse needs.
  a.stage_interleave = a.parallel_steps && a.n_groups > 1 && n_steps <= mkra::kSlots ? 1 : 0;
  if (a.stage_interleave) {
    auto rel_first = [&](int g) { return g < a.n_big ? g * a.group : a.n_big * a.group + (g - a.n_big) * a.tail_group; };
    int pos = 0;
    for (int r = 0; r < mkra::kMaxGroup; ++r)
      for (int g = 0; g < a.n_groups; ++g) {
        const int t = rel_first(g) + r;
        if (t < std::min(n_steps, rel_first(g + 1))) {
          a.stage_pos[t] = (int8_t)pos;
          a.stage_order[pos++] = (int8_t)t;
        }
      }
    if (pos != n_steps) return fail(MK_E_INVAL, "internal: staging order");
  }
  // Unit-steps that can only follow the last staging task (ADAPTIVE mode's R_p leaves
  // them out): the last staged step's, or with an interleaved order the last step of
  // every group.
  a.rp_tail = n_units * (int64_t)(a.stage_interleave ? a.n_groups : 1);
  // Running-state slots: one per unit, or one per (unit, step group) with parallel groups.
  const int64_t state_slots = n_units * (a.parallel_steps ? (int64_t)a.n_groups : 1);

  // Cost model for the controller's priors and the initial split (Eq. (2) with
  // modelled costs; §3.2: the data dependency sets the initial allocation).
  // Compute: a task's FLOPs at half of one CU's bf16 MFMA peak (4096 FLOP/clk at
  // 2.4 GHz). Staging: a tile's read+write bytes at 40 GB/s per workgroup. Ticks are
  // 100 MHz.
  const double task_flops = 4.0 * d * (a.hg * a.bq) * (double)lk;
  const double cu_rate = 0.5 * 4096.0 * 2.4e9;
  a.cost_compute0 = std::max<int64_t>(1, (int64_t)(task_flops / cu_rate * 1e8));
  const double piece_bytes = 2.0 * 2.0 * 2.0 * (double)std::min<int64_t>(mkra::kStageRows, lk) * a.piece_heads * d;
  a.cost_stage0 = std::max<int64_t>(1, (int64_t)(piece_bytes / 40e9 * 1e8));
  a.split_fixed = opts.split_mode == MK_SPLIT_FIXED ? 1 : 0;
  a.ctrl_paper = opts.split_mode == MK_SPLIT_ADAPTIVE_PAPER ? 1 : 0;
  a.disable_staging = opts.disable_staging ? 1 : 0;
  a.stage_delay_ticks = opts.stage_delay_ticks;
  a.debug_flags = opts.debug_flags;
  int init = 0;
  if (n_stage_tasks > 0 && !a.disable_staging) {
    if (a.split_fixed)
      init = std::min(opts.fixed_staging_wgs, grid - 1 > 0 ? grid - 1 : 0);
    else if (opts.initial_staging_wgs > 0)
      init = std::min(opts.initial_staging_wgs, grid - 1 > 0 ? grid - 1 : 0);
    else if (a.ctrl_paper)
      // Eq. (2) as the paper states it: every compute task remains.
      init = eq2_target_host(grid, n_units * (int64_t)n_steps, n_stage_tasks, a.cost_compute0, a.cost_stage0);
    else {
      // As on the device: R_p without the unit-steps that follow the last staging task
      // whatever the split.
      init = eq2_target_host(grid, std::max<int64_t>(0, n_units * (int64_t)n_steps - a.rp_tail), n_stage_tasks,
                             a.cost_compute0, a.cost_stage0);
      // A short launch whose whole staging fits in one round (no slot reused, at most
      // half of the grid) stages everything at once: a second round would only delay
      // the tiles it stages, and Eq. (2), which balances the roles' total work, does
      // not see that latency. Measured on the 1K-token workload (64 staging tasks, 144
      // workgroups): 0.121 against 0.132 ms with Eq. (2)'s 47.
      if (n_steps <= mkra::kSlots && n_stage_tasks <= grid / 2) init = (int)std::max<int64_t>(init, n_stage_tasks);
    }
  }
  a.initial_stagers = init;
  a.timeout_ticks = (uint64_t)(opts.spin_timeout_us > 0 ? opts.spin_timeout_us : 10000000) * 100ull;
  a.ctrl_period_ticks = (uint64_t)(opts.controller_period_us > 0 ? opts.controller_period_us : 20) * 100ull;

  if (no_alloc) {
    // Layout of the scratch array: [status | control block | done counts | slot flags |
    // unit flags | slot ring + discard block | running state], each part 256-aligned.
    const uint64_t o_ctrl = align256(sizeof(DevStatus));
    const uint64_t o_done = o_ctrl + align256(sizeof(DevCtrl));
    const uint64_t o_sflags = o_done + align256((uint64_t)n_steps * sizeof(uint32_t));
    const uint64_t o_uflags = o_sflags + align256((uint64_t)mkra::kSlots * a.stage_per_step * sizeof(uint64_t));
    const uint64_t o_slots = o_uflags + align256((uint64_t)n_units * sizeof(uint64_t));
    const uint64_t o_acc = o_slots + align256((uint64_t)mkra::kSlots * a.slot_bytes + mkra::kDiscardBytes);
    const uint64_t need =
        o_acc + (n_steps > 1 ? (uint64_t)state_slots * mkra::kWaves * (32 * d + 256) * sizeof(float) : 0);
    if (need > mkra::kScratchBytes)
      return fail(MK_E_UNSUPPORTED, "this problem needs " + std::to_string(need) +
                                        " bytes of device state; the no-allocation entry point holds " +
                                        std::to_string(mkra::kScratchBytes));
    void* base = nullptr;
    if ((e = mkra_scratch_address(dev, &base)) != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    uint8_t* b = static_cast<uint8_t*>(base);
    if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1);
    ScratchState& ss = g_scratch[dev];
    // The status word survives launches (it is cleared by mk_ring_attn_status); the
    // control block, counters and flags start at zero on every call, so a call never
    // sees a flag of an earlier one whatever its epoch.
    if (!ss.ready) {
      if ((e = mkra_zero_launch(b, o_ctrl, stream)) != hipSuccess) return hip_fail(e, "scratch clear");
      ss.ready = true;
    }
    if ((e = mkra_zero_launch(b + o_ctrl, o_slots - o_ctrl, stream)) != hipSuccess)
      return hip_fail(e, "scratch clear");
    a.status = reinterpret_cast<DevStatus*>(b);
    a.ctrl = reinterpret_cast<DevCtrl*>(b + o_ctrl);
    a.done_count = reinterpret_cast<uint32_t*>(b + o_done);
    a.slot_flags = reinterpret_cast<uint64_t*>(b + o_sflags);
    a.unit_flags = reinterpret_cast<uint64_t*>(b + o_uflags);
    a.slots = b + o_slots;
    a.acc = n_steps > 1 ? reinterpret_cast<float*>(b + o_acc) : nullptr;
    a.trace = nullptr;
    a.trace_cap = 0;
    a.epoch = ++ss.epoch;
    if ((e = mkra_kernel_launch(&a, stream)) != hipSuccess) return hip_fail(e, "kernel launch");
    return MK_OK;
  }

  Workspace* w = find_ws(dev, stream, true);
#define GROW(field, cap, need, zero)                                                   \
  if ((e = grow(&w->field, &cap, (size_t)(need), stream, zero)) != hipSuccess) \
    return hip_fail(e, "workspace allocation");
  if (w->ctrl == nullptr) {
    if ((e = hipMalloc(reinterpret_cast<void**>(&w->ctrl), sizeof(DevCtrl))) != hipSuccess)
      return hip_fail(e, "workspace allocation");
    if ((e = hipMalloc(reinterpret_cast<void**>(&w->status), sizeof(DevStatus))) != hipSuccess)
      return hip_fail(e, "workspace allocation");
    if ((e = hipMemsetAsync(w->ctrl, 0, sizeof(DevCtrl), stream)) != hipSuccess) return hip_fail(e, "memset");
    if ((e = hipMemsetAsync(w->status, 0, sizeof(DevStatus), stream)) != hipSuccess) return hip_fail(e, "memset");
  }
  GROW(done_count, w->done_cap, n_steps, true);
  GROW(slot_flags, w->tiles_cap, mkra::kSlots * (size_t)a.stage_per_step, true);
  GROW(unit_flags, w->units_cap, n_units, true);
  // The ring slots, then one block of scratch that the compute role's discarded copies
  // read (its contents are never used).
  GROW(slots, w->slot_bytes_cap, mkra::kSlots * (size_t)a.slot_bytes + mkra::kDiscardBytes, false);
  if (n_steps > 1) GROW(acc, w->acc_cap, (size_t)state_slots * mkra::kWaves * (32 * d + 256), false);
  if (opts.trace) {
    size_t cap = (size_t)(opts.trace_capacity > 0 ? opts.trace_capacity : 262144);
    size_t tc = (size_t)w->trace_cap;
    GROW(trace, tc, cap, false);
    w->trace_cap = (int)std::min<size_t>(tc, INT32_MAX);
  }
#undef GROW
  a.slots = w->slots;
  a.slot_flags = w->slot_flags;
  a.unit_flags = w->unit_flags;
  a.acc = w->acc;
  a.done_count = w->done_count;
  a.ctrl = w->ctrl;
  a.status = w->status;
  a.trace = opts.trace ? w->trace : nullptr;
  a.trace_cap = opts.trace ? w->trace_cap : 0;
  w->traced_last = opts.trace != 0;
  a.epoch = ++w->epoch;

  if (opts.debug_flags & 2) {
    // Debug: every ready flag of the slot ring and every unit flag holds, before the
    // launch, a stamp of the right step but of the previous or the next launch (even
    // and odd entries). The kernel must consume none of them.
    auto stamp = [](uint64_t ep, int step) { return (ep << 20) | (uint64_t)(step + 1); };
    std::vector<uint64_t> sf((size_t)mkra::kSlots * a.stage_per_step), uf((size_t)n_units);
    for (int sl = 0; sl < mkra::kSlots; ++sl)
      for (int j = 0; j < a.stage_per_step; ++j)
        sf[(size_t)sl * a.stage_per_step + j] = stamp(((sl + j) & 1) ? a.epoch + 1 : a.epoch - 1, sl);
    for (int64_t u = 0; u < n_units; ++u)
      uf[(size_t)u] = stamp((u & 1) ? a.epoch + 1 : a.epoch - 1, (int)(u % n_steps));
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if ((e = hipMemcpy(a.slot_flags, sf.data(), sf.size() * sizeof(uint64_t), hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy");
    if ((e = hipMemcpy(a.unit_flags, uf.data(), uf.size() * sizeof(uint64_t), hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy");
  }

  if (copy_stream != nullptr) return launch_unfused(a, w, stream, copy_stream, copy_wgs, n_units);

  if ((e = mkra_kernel_launch(&a, stream)) != hipSuccess) return hip_fail(e, "kernel launch");

  if (stats != nullptr) {
    std::memset(stats, 0, sizeof(*stats));
    DevStatus ds;
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    if ((e = hipMemcpy(&ds, w->status, sizeof(ds), hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "hipMemcpy");
    stats->status = (int32_t)device_status(ds.last_error);
    stats->grid_wgs = grid;
    stats->n_units = a.n_units;
    stats->n_steps = n_steps;
    stats->n_stage_tiles = a.n_tiles;
    stats->n_stage_tasks = a.n_stage_tasks;
    stats->stage_pieces = a.n_pieces;
    stats->compute_tasks_done = ds.compute_done;
    stats->staging_tasks_done = ds.stage_done;
    stats->assist_tasks = ds.assist_tasks;
    stats->initial_target = ds.initial_target;
    stats->final_target = ds.final_target;
    stats->max_staging_wgs = ds.max_stage;
    stats->controller_updates = ds.ctrl_updates;
    stats->role_switches = ds.role_switches;
    stats->compute_busy_ticks = ds.compute_ticks;
    stats->compute_wait_ticks = ds.compute_wait_ticks;
    stats->staging_busy_ticks = ds.stage_ticks;
    stats->staging_wait_ticks = ds.stage_wait_ticks;
    stats->kernel_ticks = ds.kernel_ticks;
    stats->trace_records = ds.trace_records;
    stats->debug_mismatches = ds.debug_mismatch;
    stats->wg_cycles = ds.wg_cycles;
    stats->wg_ticks = ds.wg_ticks;
    stats->steps_per_task = a.group;
    stats->step_groups = a.n_groups;
    stats->parallel_steps = a.parallel_steps;
  }
  return MK_OK;
}

}  // namespace

// The AllGather+GEMM layer (mkag_api.cpp) reports through the same last-error
// message and frees its workspaces with the others.
extern "C" __attribute__((visibility("hidden"))) void mkra_set_last_error(const char* msg) { g_last_error = msg; }
extern "C" __attribute__((visibility("hidden"))) void mkag_release_workspaces(void);

extern "C" {

void mk_ring_attn_default_opts(mk_ring_attn_opts* opts) {
  if (opts == nullptr) return;
  std::memset(opts, 0, sizeof(*opts));
  opts->split_mode = MK_SPLIT_ADAPTIVE;
}

mk_status mk_ring_attn_fwd(const mk_tensor* q, const mk_tensor* kv_chunks, int n_chunks, int rank, int causal,
                           int gqa_ratio, mk_tensor* out, mk_tensor* lse, hipStream_t stream) {
  return run(q, kv_chunks, n_chunks, rank, causal, gqa_ratio, out, lse, stream, nullptr, nullptr);
}

mk_status mk_ring_attn_fwd_ex(const mk_tensor* q, const mk_tensor* kv_chunks, int n_chunks, int rank, int causal,
                              int gqa_ratio, mk_tensor* out, mk_tensor* lse, hipStream_t stream,
                              const mk_ring_attn_opts* opts, mk_ring_attn_stats* stats) {
  return run(q, kv_chunks, n_chunks, rank, causal, gqa_ratio, out, lse, stream, opts, stats);
}

mk_status mk_ring_attn_fwd_noalloc(const mk_tensor* q, const mk_tensor* kv_chunks, int n_chunks, int rank,
                                   int causal, int gqa_ratio, mk_tensor* out, mk_tensor* lse, hipStream_t stream) {
  return run(q, kv_chunks, n_chunks, rank, causal, gqa_ratio, out, lse, stream, nullptr, nullptr, true);
}

mk_status mk_ring_attn_fwd_unfused(const mk_tensor* q, const mk_tensor* kv_chunks, int n_chunks, int rank, int causal,
                                   int gqa_ratio, mk_tensor* out, mk_tensor* lse, hipStream_t stream,
                                   hipStream_t copy_stream, int copy_wgs) {
  g_last_error.clear();
  if (copy_stream == nullptr || copy_stream == stream)
    return fail(MK_E_INVAL, "the unfused baseline needs a copy stream other than the compute stream");
  if (copy_wgs < 1) return fail(MK_E_INVAL, "copy_wgs must be >= 1");
  return run(q, kv_chunks, n_chunks, rank, causal, gqa_ratio, out, lse, stream, nullptr, nullptr, false, copy_stream,
             copy_wgs);
}

mk_status mk_ring_attn_status(hipStream_t stream) {
  g_last_error.clear();
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  // The stream's workspace, and the device's scratch array of the no-allocation entry
  // point if it has been used.
  DevStatus* words[3] = {nullptr, nullptr, nullptr};
  Workspace* w = find_ws(dev, stream, false);
  if (w != nullptr) {
    words[0] = w->status;
    words[2] = w->status_copy;
  }
  if ((int)g_scratch.size() > dev && g_scratch[dev].ready) {
    void* base = nullptr;
    if ((e = mkra_scratch_address(dev, &base)) != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    words[1] = static_cast<DevStatus*>(base);
  }
  uint32_t sticky = 0;
  for (DevStatus* st : words) {
    if (st == nullptr) continue;
    uint32_t v = 0;
    if ((e = hipMemcpy(&v, &st->sticky_error, sizeof(v), hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(e, "hipMemcpy");
    if (v == 0) continue;
    sticky |= v;
    const uint32_t zero = 0;
    if ((e = hipMemcpy(&st->sticky_error, &zero, sizeof(zero), hipMemcpyHostToDevice)) != hipSuccess)
      return hip_fail(e, "hipMemcpy");
  }
  if (sticky == 0) return MK_OK;
  return fail(device_status(sticky), device_message(sticky));
}

mk_status mk_ring_attn_trace(hipStream_t stream, mk_trace_record* records, int64_t capacity, int64_t* n_copied) {
  g_last_error.clear();
  static_assert(sizeof(mk_trace_record) == sizeof(TraceRec), "trace record layout");
  if (n_copied == nullptr || (records == nullptr && capacity > 0) || capacity < 0)
    return fail(MK_E_INVAL, "bad trace buffer");
  *n_copied = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_mu);
  Workspace* w = find_ws(dev, stream, false);
  if (w == nullptr || !w->traced_last || w->trace == nullptr) return fail(MK_E_INVAL, "no traced call on stream");
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int64_t written = 0;
  if ((e = hipMemcpy(&written, &w->status->trace_records, sizeof(written), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  int64_t n = std::min<int64_t>(std::min<int64_t>(written, w->trace_cap), capacity);
  if (n > 0 && (e = hipMemcpy(records, w->trace, (size_t)n * sizeof(TraceRec), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(e, "hipMemcpy");
  *n_copied = n;
  return MK_OK;
}

const char* mk_last_error(void) { return g_last_error.c_str(); }

void mk_release_workspace(void) {
  {
    std::lock_guard<std::mutex> lock(g_mu);
    for (Workspace* w : g_ws) free_ws(w);
    g_ws.clear();
  }
  mkag_release_workspaces();
}

int mk_abi_version(void) { return MKRA_ABI_VERSION; }

}  // extern "C"
