// Persistent AllGather+GEMM for gfx950 (MI355X), one rank's share.
//
// The mKernel paper ("mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", §4 and
// Table 3, AllGather + GEMM row) fuses the gather of the activation shards with the
// GEMM that consumes them: the ranks' shards move in chunks of 128 rows, and the
// GEMM's tiles run as soon as their rows have arrived, the local shard first. Here one
// GPU plays one rank: STAGING workgroups play the gather, copying every shard's
// 128-row chunks from its home (a_shards[s], standing for rank s's memory) into the
// gathered buffer a_full and publishing an epoch-stamped ready flag per chunk; COMPUTE
// workgroups run C = A_full W^T in 128 x 512 output tiles, reading the local shard in
// place and every other chunk from a_full once its flag is set. The staging/compute
// split follows Eq. (2) of §3.2 (remaining tasks of each role times their measured
// costs); a compute workgroup whose tile waits for a chunk nobody has claimed stages
// it first (the stall rule of §3.2).
//
// The product is formed transposed, C^T = W A^T, with v_mfma_f32_32x32x16_bf16 (A
// operand: 32 rows of W, B operand: 32 rows of A, both K-contiguous), so each lane
// ends with four consecutive output columns of one row per 4-element group and stores
// them as one 8-byte write.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mkag_args.h"

namespace mkag {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

enum : int32_t { kOpExit = 0, kOpCompute = 1, kOpStage = 2 };

__device__ __forceinline__ uint64_t ticks() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint32_t ld32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add32(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t add64(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool cas32(uint32_t* p, uint32_t expect, uint32_t desired) {
  return __hip_atomic_compare_exchange_strong(p, &expect, desired, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool cas64(uint64_t* p, uint64_t expect, uint64_t desired) {
  return __hip_atomic_compare_exchange_strong(p, &expect, desired, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ uint64_t stamp(uint64_t epoch) { return (epoch << 20) | 1u; }
__device__ __forceinline__ uint32_t wave_bcast(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ bool has_error(const Args& a) { return ld32(&a.ctrl->error.v) != kErrNone; }
__device__ __forceinline__ void raise_error(const Args& a, uint32_t code) { cas32(&a.ctrl->error.v, kErrNone, code); }

// Shard staged at position o of the staging order: the ring predecessors first (the
// chunks the compute role reads after its own), the local shard (copied into a_full
// only to complete the gathered output) last.
__device__ __forceinline__ int staging_shard(const Args& a, int o) {
  int s = (a.rank - 1 - o) % a.n_ranks;
  return s < 0 ? s + a.n_ranks : s;
}
// Shard the compute role consumes at position p: the local shard first (§4: compute
// tiles ordered by input availability), then the shards in the staging order.
__device__ __forceinline__ int compute_shard(const Args& a, int p) {
  int s = (a.rank - p) % a.n_ranks;
  return s < 0 ? s + a.n_ranks : s;
}

// Bounded wave-wide wait until *p == value; acquire on success. Past timeout_ticks it
// raises kErrTimeout; it returns early once any error is raised.
__device__ __forceinline__ bool wave_wait_stamp(const Args& a, const uint64_t* p, uint64_t value, uint64_t& waited) {
  if (ld64(p) == value) {
    fence_acquire();
    return true;
  }
  const uint64_t t0 = ticks();
  bool ok = true;
  while (ld64(p) != value) {
    if (has_error(a)) { ok = false; break; }
    if (ticks() - t0 > a.timeout_ticks) { raise_error(a, kErrTimeout); ok = false; break; }
    __builtin_amdgcn_s_sleep(4);
  }
  fence_acquire();
  waited += ticks() - t0;
  return ok;
}

// ------------------------------------------------------------------ staging role

// Staging task s: chunk j of the shard at staging position o = s / n_chunks, rows
// [128 j, 128 j + rows) of that shard, copied to its place in a_full; one release of
// the chunk's epoch stamp after every thread's stores (Table 3: 128-row chunks; §4:
// epoch-stamped readiness flags).
__device__ __forceinline__ void stage_chunk(const Args& a, int s, bool assist) {
  const int tid = threadIdx.x;
  const uint64_t t0 = ticks();
  const int o = s / a.n_chunks, j = s % a.n_chunks;
  const int shard = staging_shard(a, o);
  const int r0 = j * kChunkRows;
  const int rows = min(kChunkRows, a.m_loc - r0);
  const int64_t off = ((int64_t)shard * a.m_loc + r0) * a.k;  // same offset in both buffers
  const u32x4* src = reinterpret_cast<const u32x4*>(a.a_shards + off);
  u32x4* dst = reinterpret_cast<u32x4*>(a.a_full + off);
  const int64_t n16 = (int64_t)rows * a.k / 8;  // 16-byte vectors (K is a multiple of 32)
  constexpr int kInFlight = 8;
  int64_t i = tid;
  for (; i + (kInFlight - 1) * kThreads < n16; i += kInFlight * kThreads) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) dst[i + u * kThreads] = v[u];
  }
  for (; i < n16; i += kThreads) dst[i] = __builtin_nontemporal_load(src + i);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (tid == 0) {
    fence_release();
    __hip_atomic_store(&a.flags[s], stamp(a.epoch), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    add64(&a.ctrl->stage_ticks.v, ticks() - t0);
    add32(&a.ctrl->stage_done.v, 1);
    if (assist) add32(&a.ctrl->assist_tasks.v, 1);
  }
}

// ------------------------------------------------------------------ compute role

// LDS: two stages, each an A tile (128 rows x 32 k) and a W tile (512 rows x 32 k),
// rows of 64 bytes whose four 16-byte chunks are swizzled (chunk c of row r at
// c ^ ((r >> 1) & 3)) so the MFMA operand reads of a wave are bank-conflict free.
constexpr int kRowBytes = kBK * 2;
constexpr int kATileBytes = kBM * kRowBytes;  // 8 KB
constexpr int kWTileBytes = kBN * kRowBytes;  // 32 KB
constexpr int kStageBytes = kATileBytes + kWTileBytes;
constexpr int kLdsBytes = 2 * kStageBytes;
__shared__ __attribute__((aligned(16))) uint8_t g_lds[kLdsBytes];
__shared__ int32_t g_cmd[4];

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 3); }

// One output tile: gathered chunk ci (compute order) x column tile nt.
__device__ __forceinline__ void compute_tile(const Args& a, int ci, int nt, uint64_t& waited) {
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int w = (int)wave_bcast((uint32_t)(tid >> 6));
  const int wm = w >> 2, wn = w & 3;  // wave block: rows wm*64.., columns wn*128..
  ci = (int)wave_bcast((uint32_t)ci);
  nt = (int)wave_bcast((uint32_t)nt);
  const int p = ci / a.n_chunks, j = ci % a.n_chunks;
  const int shard = compute_shard(a, p);
  const int r0 = j * kChunkRows;
  const int rows = min(kBM, a.m_loc - r0);
  const int n0 = nt * kBN;
  const int cols = min(kBN, a.n_out - n0);
  const int64_t grow0 = (int64_t)shard * a.m_loc + r0;  // first gathered row of the tile
  // The local shard is read in place; every other chunk from a_full once staged.
  const uint16_t* asrc = (p == 0 ? a.a_shards : a.a_full) + grow0 * a.k;
  bool ok = true;
  if (p > 0) ok = wave_wait_stamp(a, &a.flags[ci - a.n_chunks], stamp(a.epoch), waited);

  // Loads of one K block: thread t moves 16-byte chunk (t & 3) of A row t >> 2 and of W
  // rows (t >> 2) + 128 u, u = 0..3. Rows past the tile's end read a valid row (their
  // results are never stored).
  const int lr = tid >> 2, lc = tid & 3;
  const uint16_t* a_row = asrc + (int64_t)min(lr, rows - 1) * a.k + lc * 8;
  const uint16_t* w_row[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) w_row[u] = a.w + (int64_t)(n0 + min(lr + 128 * u, cols - 1)) * a.k + lc * 8;
  const int a_st = lr * kRowBytes + 16 * swz(lr, lc);
  int w_st[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) w_st[u] = kATileBytes + (lr + 128 * u) * kRowBytes + 16 * swz(lr + 128 * u, lc);
  u32x4 ra, rw[4];
  auto load = [&](int kb) __attribute__((always_inline)) {
    const int k0 = kb * kBK;
    ra = *reinterpret_cast<const u32x4*>(a_row + k0);
#pragma unroll
    for (int u = 0; u < 4; ++u) rw[u] = *reinterpret_cast<const u32x4*>(w_row[u] + k0);
  };
  auto store = [&](int stage) __attribute__((always_inline)) {
    uint8_t* base = g_lds + stage * kStageBytes;
    *reinterpret_cast<u32x4*>(base + a_st) = ra;
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(base + w_st[u]) = rw[u];
  };

  // Operand reads: W rows wn*128 + 32 t + col (t = 0..3) and A rows wm*64 + 32 m + col
  // (m = 0..1), 16-byte chunk 2 kk + hi of the 64-byte row for k-slice kk.
  int w_rd[4][2], a_rd[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = wn * 128 + 32 * t + col;
      w_rd[t][kk] = kATileBytes + r * kRowBytes + 16 * swz(r, 2 * kk + hi);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r = wm * 64 + 32 * m + col;
      a_rd[m][kk] = r * kRowBytes + 16 * swz(r, 2 * kk + hi);
    }
  }
  f32x16 acc[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < 2; ++m) acc[t][m] = f32x16{};

  const int nk = a.k / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const int stage = kb & 1;
    if (kb + 1 < nk) load(kb + 1);  // in flight during the MFMAs below
    const uint8_t* base = g_lds + stage * kStageBytes;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 wf[4], af[2];
#pragma unroll
      for (int t = 0; t < 4; ++t) wf[t] = *reinterpret_cast<const bf16x8*>(base + w_rd[t][kk]);
#pragma unroll
      for (int m = 0; m < 2; ++m) af[m] = *reinterpret_cast<const bf16x8*>(base + a_rd[m][kk]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[t][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t], af[m], acc[t][m], 0, 0, 0);
    }
    if (kb + 1 < nk) store(stage ^ 1);  // the stage read one block ago, freed by the barrier below
    __syncthreads();
  }

  // acc[t][m] element i: output row wm*64 + 32 m + col, column wn*128 + 32 t + 8 (i/4) +
  // 4 hi + (i % 4); four consecutive columns go out as one 8-byte store.
  if (ok) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int r = wm * 64 + 32 * m + col;
      if (r >= rows) continue;
      uint16_t* crow = a.c + (grow0 + r) * a.n_out + n0;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cc = wn * 128 + 32 * t + 8 * g + 4 * hi;
          if (cc >= cols) continue;  // N_out is a multiple of 8: a group is whole or absent
          bf16x4 v;
          v[0] = (__bf16)acc[t][m][4 * g + 0];
          v[1] = (__bf16)acc[t][m][4 * g + 1];
          v[2] = (__bf16)acc[t][m][4 * g + 2];
          v[3] = (__bf16)acc[t][m][4 * g + 3];
          *reinterpret_cast<bf16x4*>(crow + cc) = v;
        }
    }
  }
}

// ------------------------------------------------------------------ scheduling

// Eq. (2) of §3.2 in integers: n = B*Rs*Cs / (Rp*Cp + Rs*Cs), rounded half up, clamped
// to [1, min(B-1, Rs)] while staging remains (0 when B == 1), 0 once it is gone.
__device__ __forceinline__ int eq2_target(int64_t b, int64_t rp, int64_t rs, int64_t cp, int64_t cs) {
  if (rs <= 0) return 0;
  const uint64_t ws = (uint64_t)rs * (uint64_t)cs;
  const uint64_t wt = ws + (uint64_t)(rp > 0 ? rp : 0) * (uint64_t)cp;
  const int64_t n = (int64_t)((2ull * (uint64_t)b * ws + wt) / (2ull * wt));
  const int64_t hi = b - 1 < rs ? b - 1 : rs;
  const int64_t lo = hi < 1 ? hi : 1;
  return (int)(n < lo ? lo : (n > hi ? hi : n));
}

__device__ __forceinline__ int target_of(const Args& a, uint32_t v) { return v == 0 ? a.initial_stagers : (int)v - 1; }

__device__ __forceinline__ int64_t queue_len(const Args& a, int x) {
  return (int64_t)a.n_ranks * a.n_chunks * a.xcd_ntiles[x];
}

struct Sched {
  int32_t role;
  int32_t pending;
  int32_t pend_ci, pend_nt;
};

// Run by lane 0 of wave 0: picks the workgroup's next task and writes (op, x, y).
__device__ __forceinline__ void schedule(const Args& a, Sched* st, int32_t* cmd) {
  int32_t op = kOpExit, x = 0, y = 0;
  if (has_error(a)) {
    cmd[0] = kOpExit;
    return;
  }
  const uint32_t sh = ld32(&a.ctrl->stage_head.v);
  const bool stage_left = (int)sh < a.n_stage_tasks;
  // Controller: rate-limited by a compare-and-swap on the update time.
  if (!a.split_fixed) {
    const uint64_t now = ticks(), last = ld64(&a.ctrl->ctrl_time.v);
    if ((last == 0 || now - last >= a.ctrl_period_ticks) && cas64(&a.ctrl->ctrl_time.v, last, now)) {
      int64_t rp = 0;
      for (int q = 0; q < a.n_xcd; ++q) {
        const int64_t left = queue_len(a, q) - (int64_t)ld32(&a.ctrl->xcd_head[q].v);
        rp += left > 0 ? left : 0;
      }
      const int64_t rs = stage_left ? a.n_stage_tasks - (int64_t)sh : 0;
      const uint64_t cd = ld32(&a.ctrl->compute_done.v), sd = ld32(&a.ctrl->stage_done.v);
      int64_t cp = a.cost_compute0, cs = a.cost_stage0;
      if (a.ctrl_paper) {
        // The paper's inputs: measured busy ticks per finished task.
        if (cd > 0) cp = (int64_t)(ld64(&a.ctrl->compute_ticks.v) / cd);
        if (sd > 0) cs = (int64_t)(ld64(&a.ctrl->stage_ticks.v) / sd);
      } else {
        // Measured ticks averaged with the cost model's priors, weighted as one shard's
        // tasks of each role, so the first (cold) tasks do not swing the split.
        const uint64_t kc = (uint64_t)a.n_chunks * a.n_ntiles, ks = (uint64_t)a.n_chunks;
        cp = (int64_t)((ld64(&a.ctrl->compute_ticks.v) + kc * (uint64_t)a.cost_compute0) / (cd + kc));
        cs = (int64_t)((ld64(&a.ctrl->stage_ticks.v) + ks * (uint64_t)a.cost_stage0) / (sd + ks));
      }
      if (cp < 1) cp = 1;
      if (cs < 1) cs = 1;
      __hip_atomic_store(&a.ctrl->target.v, (uint32_t)(eq2_target(a.grid, rp, rs, cp, cs) + 1), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      add32(&a.ctrl->ctrl_updates.v, 1);
    }
  }
  const int tgt = target_of(a, ld32(&a.ctrl->target.v));
  if (!st->pending) {
    // Role changes at task boundaries (§3.2).
    if (st->role == kRoleStage) {
      const uint32_t ns = ld32(&a.ctrl->n_stage.v);
      if (!stage_left || (!a.split_fixed && (int)ns > tgt && cas32(&a.ctrl->n_stage.v, ns, ns - 1))) {
        if (!stage_left) add32(&a.ctrl->n_stage.v, (uint32_t)-1);
        st->role = kRoleCompute;
      }
    } else if (!a.split_fixed && stage_left) {
      const uint32_t ns = ld32(&a.ctrl->n_stage.v);
      if ((int)ns < tgt && cas32(&a.ctrl->n_stage.v, ns, ns + 1)) {
        st->role = kRoleStage;
        __hip_atomic_fetch_max(&a.ctrl->max_stage.v, ns + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (st->role == kRoleStage) {
      const uint32_t s = add32(&a.ctrl->stage_head.v, 1);
      if ((int)s < a.n_stage_tasks) {
        cmd[0] = kOpStage;
        cmd[1] = (int32_t)s;
        cmd[2] = 0;
        return;
      }
      add32(&a.ctrl->n_stage.v, (uint32_t)-1);
      st->role = kRoleCompute;
    }
    // Claim an output tile: this XCD's queue first, then any queue with tiles left.
    const int own = (int)(blockIdx.x % (unsigned)a.n_xcd);
    for (int i = 0; i < a.n_xcd && !st->pending; ++i) {
      const int q = (own + i) % a.n_xcd;
      const int64_t len = queue_len(a, q);
      if ((int64_t)ld32(&a.ctrl->xcd_head[q].v) >= len) continue;
      const uint32_t h = add32(&a.ctrl->xcd_head[q].v, 1);
      if ((int64_t)h >= len) continue;
      const int nq = a.xcd_ntiles[q];
      st->pend_ci = (int32_t)(h / nq);
      st->pend_nt = q + a.n_xcd * (int32_t)(h % nq);
      st->pending = 1;
    }
    if (!st->pending) {
      // No tile left: help drain the staging, else leave.
      if (stage_left) {
        const uint32_t s = add32(&a.ctrl->stage_head.v, 1);
        if ((int)s < a.n_stage_tasks) {
          cmd[0] = kOpStage;
          cmd[1] = (int32_t)s;
          cmd[2] = 1;
          return;
        }
      }
      cmd[0] = kOpExit;
      return;
    }
  }
  // The stall rule of §3.2: while the chunk the claimed tile reads is unclaimed
  // staging, stage first (claiming the staging head up to that chunk). A failed
  // compare-and-swap returns a larger head, so the loop ends within need - head + 1
  // attempts, either with a claim or with the chunk claimed by someone else (who is
  // staging it: the tile's wait on its flag then ends).
  const int p = st->pend_ci / a.n_chunks;
  if (p > 0) {
    const int need = st->pend_ci - a.n_chunks;  // staging task of the tile's chunk
    uint32_t h = ld32(&a.ctrl->stage_head.v);
    while ((int)h <= need) {
      uint32_t expect = h;
      if (__hip_atomic_compare_exchange_strong(&a.ctrl->stage_head.v, &expect, h + 1, __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        cmd[0] = kOpStage;
        cmd[1] = (int32_t)h;
        cmd[2] = 1;
        return;
      }
      h = expect;
    }
  }
  op = kOpCompute;
  x = st->pend_ci;
  y = st->pend_nt;
  st->pending = 0;
  cmd[0] = op;
  cmd[1] = x;
  cmd[2] = y;
}

__global__ __launch_bounds__(kThreads) void ag_gemm_kernel(Args a) {
  const int tid = threadIdx.x;
  const uint64_t t_start = ticks();
  const uint64_t c_start = __builtin_readcyclecounter();
  __shared__ Sched sched;
  if (tid == 0) {
    __hip_atomic_fetch_max(&a.ctrl->t_first.v, ~t_start, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sched.role = ((int)blockIdx.x < a.initial_stagers) ? kRoleStage : kRoleCompute;
    sched.pending = 0;
    if (sched.role == kRoleStage) {
      const uint32_t n = add32(&a.ctrl->n_stage.v, 1) + 1;
      __hip_atomic_fetch_max(&a.ctrl->max_stage.v, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  while (true) {
    __syncthreads();
    if (tid == 0) schedule(a, &sched, g_cmd);
    __syncthreads();
    const int op = g_cmd[0], x = g_cmd[1], y = g_cmd[2];
    if (op == kOpExit) break;
    if (op == kOpStage) {
      stage_chunk(a, x, y != 0);
    } else {
      const uint64_t t0 = ticks();
      uint64_t waited = 0;
      compute_tile(a, x, y, waited);
      if (tid == 0) {
        add64(&a.ctrl->compute_ticks.v, ticks() - t0 - waited);
        add64(&a.ctrl->compute_wait_ticks.v, waited);
        add32(&a.ctrl->compute_done.v, 1);
      }
    }
  }
  // Exit: the last workgroup out records the statistics and resets the control block.
  __shared__ int last;
  if (tid == 0) {
    const uint64_t t_end = ticks();
    add64(&a.ctrl->wg_cycles.v, __builtin_readcyclecounter() - c_start);
    add64(&a.ctrl->wg_ticks.v, t_end - t_start);
    __hip_atomic_fetch_max(&a.ctrl->t_last.v, t_end, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    fence_release();
    const uint32_t n = __hip_atomic_fetch_add(&a.ctrl->exit_count.v, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = (n == (uint32_t)a.grid - 1);
  }
  __syncthreads();
  if (!last) return;
  fence_acquire();
  if (tid == 0) {
    Ctrl* cb = a.ctrl;
    Status* ds = a.status;
    const uint32_t err = ld32(&cb->error.v);
    ds->sticky_error |= err;
    ds->last_error = err;
    ds->compute_done = (int32_t)ld32(&cb->compute_done.v);
    ds->stage_done = (int32_t)ld32(&cb->stage_done.v);
    ds->assist_tasks = (int32_t)ld32(&cb->assist_tasks.v);
    ds->ctrl_updates = (int32_t)ld32(&cb->ctrl_updates.v);
    ds->max_stage = (int32_t)ld32(&cb->max_stage.v);
    ds->final_target = target_of(a, ld32(&cb->target.v));
    ds->compute_ticks = (int64_t)ld64(&cb->compute_ticks.v);
    ds->compute_wait_ticks = (int64_t)ld64(&cb->compute_wait_ticks.v);
    ds->stage_ticks = (int64_t)ld64(&cb->stage_ticks.v);
    ds->kernel_ticks = (int64_t)(ld64(&cb->t_last.v) - ~ld64(&cb->t_first.v));
    ds->wg_cycles = (int64_t)ld64(&cb->wg_cycles.v);
    ds->wg_ticks = (int64_t)ld64(&cb->wg_ticks.v);
  }
  __syncthreads();
  uint32_t* words = reinterpret_cast<uint32_t*>(a.ctrl);
  for (int i = tid; i < (int)(sizeof(Ctrl) / 4); i += kThreads) words[i] = 0;
}

}  // namespace mkag

extern "C" __attribute__((visibility("hidden"))) hipError_t mkag_kernel_launch(const mkag::Args* a,
                                                                              hipStream_t stream) {
  hipLaunchKernelGGL(mkag::ag_gemm_kernel, dim3((unsigned)a->grid), dim3(mkag::kThreads), 0, stream, *a);
  return hipGetLastError();
}

extern "C" __attribute__((visibility("hidden"))) hipError_t mkag_kernel_occupancy(int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, mkag::ag_gemm_kernel, mkag::kThreads, 0);
}
