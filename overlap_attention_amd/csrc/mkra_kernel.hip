// Persistent ring-attention forward for gfx950 (MI355X).
//
// One launch runs every ring step of one rank (mKernel paper "mKernel: Fast
// Multi-GPU, Multi-Node Fused Kernels", §4 / Table 3, Ring Attention row). Its
// workgroups take roles (§3.2): COMPUTE workgroups run the blockwise
// FlashAttention forward of a (unit, step) task and carry the online-softmax state
// (running max m, running sum l, unnormalised O) from step to step; STAGING
// workgroups play the ring receive on one GPU, copying the chunk of the next step
// into a double buffer in HBM and publishing an epoch-stamped ready flag per
// 128-row tile (Table 3 granularity; epoch-stamped flags per §4). The target
// number of staging workgroups follows Eq. (2) of §3.2, recomputed on the GPU from
// cycle counters; a compute wave stalled on a flag may do a staging task itself.
//
// Compute layout (per wave, 32 query rows of one head): S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q from registers), so each lane
// holds one query column and 16 of every 32 keys; the row max needs one exchange
// with lane^32. O^T = V^T P^T with the same instruction (A = V^T from LDS, stored
// transposed with a key permutation that matches the accumulator layout of S^T,
// B = P^T straight from registers).
#include <hip/hip_runtime.h>

#include "mkra_args.h"

namespace mkra {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Lazy rescale threshold (log2 units): the running max used for exponentials may lag
// the true max by up to this much; P stays <= 2^kTau, exact algebra is unchanged.
constexpr float kTau = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr f16x2 kOnes2 = {(_Float16)1.0f, (_Float16)1.0f};

enum : int32_t { kOpExit = 0, kOpCompute = 1, kOpStage = 2, kOpAssist = 3 };

// ------------------------------------------------------------------ primitives

__device__ __forceinline__ uint64_t ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ uint32_t ld32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64_release(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
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
__device__ __forceinline__ void max32(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void max64(uint64_t* p, uint64_t v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }

// Flags carry (epoch << 20) | (step + 1): a flag of an earlier launch never matches.
__device__ __forceinline__ uint64_t stamp(uint64_t epoch, int step) {
  return (epoch << 20) | (uint64_t)(step + 1);
}

__device__ __forceinline__ uint32_t wave_bcast(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ bool has_error(const KernelArgs& a) { return ld32(&a.ctrl->error.v) != kErrNone; }

__device__ __forceinline__ void raise_error(const KernelArgs& a, uint32_t code) {
  cas32(&a.ctrl->error.v, kErrNone, code);
}

__device__ __forceinline__ int chunk_of_step(const KernelArgs& a, int t) {
  int c = (a.rank - t) % a.n_chunks;
  return c < 0 ? c + a.n_chunks : c;
}

__device__ __noinline__ void trace_rec(const KernelArgs& a, int kind, int64_t v0, int64_t v1, int64_t v2, int64_t v3,
                          int64_t v4, int64_t v5) {
  if (a.trace == nullptr) return;
  uint32_t i = add32(&a.ctrl->trace_head.v, 1);
  if ((int64_t)i >= a.trace_cap) return;
  TraceRec r;
  r.t = ticks();
  r.wg = (int32_t)blockIdx.x;
  r.kind = kind;
  r.v[0] = v0; r.v[1] = v1; r.v[2] = v2; r.v[3] = v3; r.v[4] = v4; r.v[5] = v5;
  a.trace[i] = r;
}

// ------------------------------------------------------------------ controller

// Eq. (2) of §3.2 in integers: n = B*Rs*Cs / (Rp*Cp + Rs*Cs), rounded half up,
// clamped to [1, min(B-1, Rs)] while staging work remains (0 when B == 1, where the
// single workgroup stages only by assisting), and 0 once it is gone.
__device__ __forceinline__ int eq2_target(int64_t b, int64_t rp, int64_t rs, int64_t cp, int64_t cs) {
  if (rs <= 0) return 0;
  uint64_t ws = (uint64_t)rs * (uint64_t)cs;
  uint64_t w = ws + (uint64_t)(rp > 0 ? rp : 0) * (uint64_t)cp;
  int64_t n = (int64_t)((2ull * (uint64_t)b * ws + w) / (2ull * w));
  int64_t hi = b - 1 < rs ? b - 1 : rs;
  int64_t lo = hi < 1 ? hi : 1;
  return (int)(n < lo ? lo : (n > hi ? hi : n));
}

__device__ __forceinline__ int current_target(const KernelArgs& a) {
  uint32_t v = ld32(&a.ctrl->target.v);  // 0 = not yet set by the controller
  return v == 0 ? a.initial_stagers : (int)v - 1;
}

__device__ __forceinline__ int64_t units_in_queue(const KernelArgs& a, int x) {
  return a.xcd_unit_begin[x + 1] - a.xcd_unit_begin[x];
}

__device__ int64_t compute_claimed(const KernelArgs& a) {
  int64_t s = 0;
  for (int x = 0; x < a.n_xcd; ++x) {
    int64_t tot = units_in_queue(a, x) * a.n_steps;
    int64_t h = ld32(&a.ctrl->xcd_head[x].v);
    s += h < tot ? h : tot;
  }
  return s;
}

// Run by one lane. Rate-limited by a compare-and-swap on the update time.
__device__ __noinline__ void maybe_controller(const KernelArgs& a) {
  if (a.split_fixed || a.disable_staging) return;
  uint64_t now = ticks();
  uint64_t last = ld64(&a.ctrl->ctrl_time.v);
  if (last != 0 && now - last < a.ctrl_period_ticks) return;
  if (!cas64(&a.ctrl->ctrl_time.v, last, now)) return;
  int64_t sh = ld32(&a.ctrl->stage_head.v);
  int64_t rs = a.n_stage_tasks - (sh < a.n_stage_tasks ? sh : a.n_stage_tasks);
  int64_t rp = (int64_t)a.n_units * a.n_steps - compute_claimed(a);
  uint64_t cd = ld32(&a.ctrl->compute_done.v), ct = ld64(&a.ctrl->compute_ticks.v);
  uint64_t sd = ld32(&a.ctrl->stage_done.v), stt = ld64(&a.ctrl->stage_ticks.v);
  // A staging workgroup runs kWaves staging tasks at once (one per wave), so its
  // cost per task is the per-wave cost divided by kWaves.
  int64_t cp = cd ? (int64_t)(ct / cd) : a.cost_compute0;
  int64_t cs = sd ? (int64_t)(stt / sd / kWaves) : a.cost_stage0;
  if (cp < 1) cp = 1;
  if (cs < 1) cs = 1;
  int n = eq2_target(a.grid, rp, rs, cp, cs);
  st32(&a.ctrl->target.v, (uint32_t)(n + 1));
  add32(&a.ctrl->ctrl_updates.v, 1);
  trace_rec(a, kTraceController, rp, rs, cp, cs, a.grid, n);
}

// ------------------------------------------------------------------ waits
// All waits are bounded: past timeout_ticks they raise MK_E_TIMEOUT, and every wait
// returns early once any error is raised, so every workgroup reaches its exit.

// Wave-wide wait until *p >= target; acquire on success.
__device__ bool wave_wait_ge32(const KernelArgs& a, uint32_t* p, uint32_t target, uint64_t& waited) {
  if (ld32(p) >= target) {
    fence_acquire();
    return true;
  }
  uint64_t t0 = ticks();
  bool ok = true;
  while (ld32(p) < target) {
    if (has_error(a)) { ok = false; break; }
    if (ticks() - t0 > a.timeout_ticks) { raise_error(a, kErrTimeout); ok = false; break; }
    __builtin_amdgcn_s_sleep(8);
  }
  fence_acquire();
  waited += ticks() - t0;
  return ok;
}


// Wave-wide wait until *p == value (an epoch stamp); acquire on success.
__device__ bool wave_wait_stamp(const KernelArgs& a, const uint64_t* p, uint64_t value, uint64_t& waited) {
  if (ld64(p) == value) {
    fence_acquire();
    return true;
  }
  uint64_t t0 = ticks();
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

// One staging task, run by one wave: part `part` of 128-row tile `j` of the chunk of
// step t, copied from the chunk's home (kv_chunks, standing for the predecessor's
// memory) into slot t % 2. The slot is free once every unit has finished step t-2.
// The wave that completes the last part of the tile publishes its flag.
__device__ __forceinline__ bool stage_task(const KernelArgs& a, uint32_t k, bool assist, uint64_t& waited) {
  const int lane = threadIdx.x & 63;
  const uint64_t t_begin = ticks();
  const int per_step = a.n_tiles * a.parts_per_tile;
  const int t = 1 + (int)k / per_step;
  const int rem = (int)k % per_step;
  const int j = rem / a.parts_per_tile;
  const int part = rem % a.parts_per_tile;
  const int slot = t & 1;
  uint64_t w = 0;
  bool ok = true;
  int64_t dst_off = -1;
  if (t >= 2) ok = wave_wait_ge32(a, &a.done_count[t - 2], (uint32_t)a.n_units, w);

  if (ok) {
    const int c = chunk_of_step(a, t);
    const int r0 = j * kStageRows;
    const int nr = min(kStageRows, a.lk - r0);
    const int64_t row_elems = (int64_t)a.hkv * a.d;
    const int64_t tile_elems = (int64_t)nr * row_elems;
    const int64_t e0 = (int64_t)part * kStagePartElems;
    const int64_t e1 = min(tile_elems, e0 + (int64_t)kStagePartElems);
    const int64_t half = (int64_t)a.lk * row_elems;
    const int64_t off = (int64_t)r0 * row_elems + e0;
    const uint16_t* src = a.kv + (int64_t)c * a.chunk_elems + off;
    uint16_t* dst = a.slots + (int64_t)slot * a.chunk_elems + off;
    const int64_t n16 = e1 > e0 ? (e1 - e0) / 8 : 0;  // 16-byte vectors of K (and of V)
    // K then V, 8 vectors in flight per lane.
    for (int kvsel = 0; kvsel < 2; ++kvsel) {
      const u32x4* s4 = reinterpret_cast<const u32x4*>(src + kvsel * half);
      u32x4* d4 = reinterpret_cast<u32x4*>(dst + kvsel * half);
      for (int64_t i = lane; i < n16; i += 64 * 8) {
        u32x4 r[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          int64_t idx = i + u * 64;
          if (idx < n16) r[u] = __builtin_nontemporal_load(s4 + idx);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          int64_t idx = i + u * 64;
          if (idx < n16) d4[idx] = r[u];
        }
      }
    }
    if (a.debug_flags & 4) {
      // Debug: read back what this wave wrote (after its own stores completed).
      fence_release();
      uint32_t bad = 0;
      for (int kvsel = 0; kvsel < 2; ++kvsel) {
        const u32x4* s4 = reinterpret_cast<const u32x4*>(src + kvsel * half);
        const u32x4* d4 = reinterpret_cast<const u32x4*>(dst + kvsel * half);
        for (int64_t i = lane; i < n16; i += 64) {
          u32x4 x = s4[i], y = d4[i];
          bad += (x[0] != y[0]) | (x[1] != y[1]) | (x[2] != y[2]) | (x[3] != y[3]);
        }
      }
      if (bad) add32(&a.ctrl->debug_mismatch.v, bad << 16);
    }
    dst_off = (int64_t)(dst - a.slots);
    if (a.stage_delay_ticks > 0) {
      uint32_t hsh = (k * 2654435761u) ^ (uint32_t)a.epoch;
      uint64_t until = ticks() + (hsh % (uint32_t)a.stage_delay_ticks);
      while (ticks() < until) __builtin_amdgcn_s_sleep(1);
    }
    fence_release();  // this wave's copies are visible at agent scope
    if (lane == 0) {
      uint32_t* cnt = &a.tile_parts[slot * a.n_tiles + j];
      uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (old == (uint32_t)a.parts_per_tile - 1) {
        st32(cnt, 0);  // reset for step t + 2 before the flag can release anyone
        st64_release(&a.slot_flags[slot * a.n_tiles + j], stamp(a.epoch, t));
      }
    }
  }
  if (lane == 0) {
    uint64_t busy = ticks() - t_begin - w;
    add64(&a.ctrl->stage_ticks.v, busy);
    add32(&a.ctrl->stage_done.v, 1);
    add64(&a.ctrl->stage_wait_ticks.v, w);
    if (assist) add32(&a.ctrl->assist_tasks.v, 1);
    trace_rec(a, kTraceStage, k, t, j, (int64_t)t_begin, assist ? 1 : 0, dst_off);
  }
  waited += w;
  return ok;
}

// ------------------------------------------------------------------ compute role

template <int D>
struct Smem {
  uint16_t k[2][kBN][D + 8];    // K tile rows, bf16 (padded: conflict-free 16-byte reads)
  uint16_t vt[2][D][kBN + 8];   // V tile transposed to fp16, keys permuted within 16
  int32_t cmd[4];
};

// Position of key offset x (0..15) inside its group of 16 in the transposed V tile:
// swaps bits 2 and 3, so each lane's 8 P^T values (keys {0-3,8-11} for lanes 0-31,
// {4-7,12-15} for lanes 32-63, from the 32x32 accumulator layout) meet the 8
// contiguous V^T values it reads.
__device__ __forceinline__ int vt_pos(int key) {
  int x = key & 15;
  return (key & ~15) | (x & 3) | ((x & 4) << 1) | ((x & 8) >> 1);
}

template <int D>
__device__ void compute_task(const KernelArgs& a, Smem<D>& sm, int unit, int t, uint64_t& waited) {
  constexpr int KK = D / 16;                    // k-slices of Q K^T
  constexpr int DB = D / 32;                    // 32-row blocks of O^T
  constexpr int KCH = kBN * D / 8 / kThreads;   // 16-byte K chunks per thread per tile
  constexpr int NVG = (kBN / 4) * (D / 4);      // V groups (4 keys x 4 d) per tile
  constexpr int VSTRIDE = kBN + 8;
  static_assert(KCH >= 1 && NVG <= kThreads, "tile split");

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hi = lane >> 5, col = lane & 31;
  const int p = unit / a.n_qblocks, qb = unit % a.n_qblocks;
  const int kvh = p / a.n_hgroups, hgi = p % a.n_hgroups;
  const int h = kvh * a.gqa + hgi * a.hg + (w % a.hg);
  const int q0w = qb * a.bq + (w / a.hg) * kRowsPerWave;
  const bool wave_rows = q0w < a.lq;
  const int qrow = q0w + col;
  const bool diag = a.causal && t == 0;
  const int c = chunk_of_step(a, t);
  const uint16_t* kbase = (t == 0) ? a.kv + (int64_t)c * a.chunk_elems : a.slots + (int64_t)(t & 1) * a.chunk_elems;
  const int64_t half = (int64_t)a.lk * a.hkv * D;
  const int q_end = min(a.lq, qb * a.bq + a.bq);
  const int kend = diag ? min(a.lk, q_end) : a.lk;
  const int n_kt = (kend + kBN - 1) / kBN;
  const int wkend = diag ? min(a.lk, q0w + kRowsPerWave) : a.lk;
  const int w_kt = wave_rows ? (wkend + kBN - 1) / kBN : 0;
  const float c2 = a.scale_log2;
  bool ok = true;

  // Per-unit step order: the state of step t-1 must be complete.
  if (t > 0) ok &= wave_wait_stamp(a, &a.unit_flags[unit], stamp(a.epoch, t - 1), waited);

  // Ready flags of the staged tiles: one acquire if all are ready already.
  const uint64_t* flags = a.slot_flags + (t & 1) * a.n_tiles;
  const uint64_t st = stamp(a.epoch, t);
  const int n_st = (kend + kStageRows - 1) / kStageRows;
  int ready_upto = n_st;
  if (t > 0) {
    bool mine = true;
    for (int j = lane; j < n_st; j += 64) mine &= (ld64(&flags[j]) == st);
    if (__all(mine)) {
      fence_acquire();
    } else {
      ready_upto = 0;
    }
  }

  // Q: lane holds Q[qrow][h][kk*16 + 8*hi .. +7] for every k-slice.
  bf16x8 qr[KK];
  {
    const bool in = qrow < a.lq;
    const uint16_t* qp = a.q + ((int64_t)(in ? qrow : 0) * a.hq + h) * D + hi * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 v = in ? *reinterpret_cast<const u32x4*>(qp + kk * 16) : u32x4{0, 0, 0, 0};
      qr[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // Running state: O^T blocks, max (log2 units of the scaled score), partial sum.
  f32x16 o[DB];
  float m_run, l_run, lr_run;
  float* accw = a.acc + ((int64_t)unit * kWaves + w) * (32 * D + 256);
  if (t == 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
    lr_run = 0.f;
  } else {
    const f32x4* a4 = reinterpret_cast<const f32x4*>(accw);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = a4[(db * 4 + g) * 64 + lane];
        o[db][g * 4 + 0] = v[0]; o[db][g * 4 + 1] = v[1]; o[db][g * 4 + 2] = v[2]; o[db][g * 4 + 3] = v[3];
      }
    f32x4 ml = reinterpret_cast<const f32x4*>(accw + 32 * D)[lane];
    m_run = ml[0];
    l_run = ml[1];
    lr_run = ml[2];
  }

  // Tile loads: K as 16-byte row chunks; V as 4 keys x 8 d per thread, transposed on
  // the way into LDS.
  u32x4 kreg[KCH];
  u32x2 vreg[4];
  auto wait_tile = [&](int kt) {
    int j = (kt * kBN) / kStageRows;
    if (j >= ready_upto) {
      ok &= wave_wait_stamp(a, &flags[j], st, waited);
      ready_upto = j + 1;
    }
  };
  auto load_tile = [&](int kt) {
    const int k0 = kt * kBN;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int ch = tid + i * kThreads;
      int key = k0 + ch / (D / 8);
      int dd = (ch % (D / 8)) * 8;
      kreg[i] = key < a.lk ? *reinterpret_cast<const u32x4*>(kbase + ((int64_t)key * a.hkv + kvh) * D + dd)
                           : u32x4{0, 0, 0, 0};
    }
    if (tid < NVG) {
      int key4 = k0 + (tid / (D / 4)) * 4;
      int dd = (tid % (D / 4)) * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int key = key4 + r;
        vreg[r] = key < a.lk
                      ? *reinterpret_cast<const u32x2*>(kbase + half + ((int64_t)key * a.hkv + kvh) * D + dd)
                      : u32x2{0, 0};
      }
    }
    if ((a.debug_flags & 1) && t > 0) {
      // Debug: compare what was read from the slot with the chunk's home copy.
      const uint16_t* home = a.kv + (int64_t)c * a.chunk_elems;
      uint32_t bad = 0;
      for (int i = 0; i < KCH; ++i) {
        int ch = tid + i * kThreads;
        int key = k0 + ch / (D / 8);
        int dd = (ch % (D / 8)) * 8;
        if (key < a.lk) {
          u32x4 r = *reinterpret_cast<const u32x4*>(home + ((int64_t)key * a.hkv + kvh) * D + dd);
          bad += (r[0] != kreg[i][0]) | (r[1] != kreg[i][1]) | (r[2] != kreg[i][2]) | (r[3] != kreg[i][3]);
        }
      }
      if (tid < NVG) {
        int key4 = k0 + (tid / (D / 4)) * 4;
        int dd = (tid % (D / 4)) * 4;
        for (int r = 0; r < 4; ++r) {
          int key = key4 + r;
          if (key < a.lk) {
            u32x2 v = *reinterpret_cast<const u32x2*>(home + half + ((int64_t)key * a.hkv + kvh) * D + dd);
            bad += (v[0] != vreg[r][0]) | (v[1] != vreg[r][1]);
          }
        }
      }
      if (bad) add32(&a.ctrl->debug_mismatch.v, bad);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      int ch = tid + i * kThreads;
      int key = ch / (D / 8);
      int dd = (ch % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&sm.k[buf][key][dd]) = kreg[i];
    }
    if (tid < NVG) {
      // vreg[r] holds d = dd..dd+3 of key key4+r as bf16 pairs. Each of the 4 d rows
      // of V^T gets the 4 keys, converted to fp16 (exact for |v| < 65520).
      int key4 = (tid / (D / 4)) * 4;
      int dd = (tid % (D / 4)) * 4;
      int pos = vt_pos(key4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float f[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint32_t wv = vreg[r][e >> 1];
          f[r] = __builtin_bit_cast(float, (e & 1) ? (wv & 0xffff0000u) : (wv << 16));
        }
        f16x2 p01 = {(_Float16)f[0], (_Float16)f[1]};
        f16x2 p23 = {(_Float16)f[2], (_Float16)f[3]};
        *reinterpret_cast<u32x2*>(&sm.vt[buf][dd + e][pos]) =
            u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
      }
    }
  };

  if (n_kt > 0) {
    if (t > 0) wait_tile(0);
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) {
      if (t > 0) wait_tile(kt + 1);
      load_tile(kt + 1);
    }
    if (kt < w_kt) {
      const uint16_t* ks = &sm.k[buf][0][0];
      const uint16_t* vs = &sm.vt[buf][0][0];
      // S^T = K Q^T for 2 blocks of 32 keys.
      f32x16 s[kBN / 32];
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        s[kb] = f32x16{};
        const uint16_t* kr = ks + (kb * 32 + col) * (D + 8) + hi * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          bf16x8 av = *reinterpret_cast<const bf16x8*>(kr + kk * 16);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qr[kk], s[kb], 0, 0, 0);
        }
      }
      // Masks: ragged key tail, and keys after the query on the diagonal step.
      const int k0 = kt * kBN;
      if (k0 + kBN > a.lk || (diag && k0 + kBN - 1 > q0w)) {
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            int key = k0 + kb * 32 + (i >> 2) * 8 + hi * 4 + (i & 3);
            if (key >= a.lk || (diag && key > qrow)) s[kb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mxs = mx * c2;
      // Online-softmax update (FlashAttention-2), rescaling only when the max has
      // grown by more than kTau since the last rescale.
      if (__any(mxs > m_run + kTau)) {
        const float m_new = fmaxf(m_run, mxs);
        const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        l_run *= alpha;
        lr_run *= alpha;
        m_run = m_new;
      }
      const float mref = (m_run == -INFINITY) ? 0.f : m_run;
      f16x8 pb[kBN / 16];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -mref));
          lsum += pv;
          pb[kb * 2 + (i >> 3)][i & 7] = (_Float16)pv;
        }
      l_run += lsum;
      // Two running sums: l (exact P, for the log-sum-exp) and lr, the sum of the
      // fp16-rounded P that the PV product actually weights V with (two per
      // v_dot2c_f32_f16 against (1, 1)). Normalising O by lr makes the applied
      // weights sum to one, so a dominant key's rounding cancels in O / lr.
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int pp = 0; pp < kBN / 16; ++pp) {
        ls0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(pb[pp], pb[pp], 0, 1), kOnes2, ls0, false);
        ls1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(pb[pp], pb[pp], 2, 3), kOnes2, ls1, false);
        ls0 = __builtin_amdgcn_fdot2(__builtin_shufflevector(pb[pp], pb[pp], 4, 5), kOnes2, ls0, false);
        ls1 = __builtin_amdgcn_fdot2(__builtin_shufflevector(pb[pp], pb[pp], 6, 7), kOnes2, ls1, false);
      }
      lr_run += ls0 + ls1;
      // O^T += V^T P^T (fp16 operands, fp32 accumulation).
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vr = vs + (db * 32 + col) * VSTRIDE + hi * 8;
#pragma unroll
        for (int pp = 0; pp < kBN / 16; ++pp) {
          f16x8 av = *reinterpret_cast<const f16x8*>(vr + pp * 16);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[pp], o[db], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (ok && wave_rows) {
    if (t == a.n_steps - 1) {
      // Finalise: out = O / lr, lse = ln(2) * (m + log2 l).
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const float lr_tot = lr_run + __shfl_xor(lr_run, 32);
      if (qrow < a.lq) {
        const float inv = 1.f / lr_tot;
        uint16_t* op = a.out + ((int64_t)qrow * a.hq + h) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 v;
            v[0] = (__bf16)(o[db][g * 4 + 0] * inv);
            v[1] = (__bf16)(o[db][g * 4 + 1] * inv);
            v[2] = (__bf16)(o[db][g * 4 + 2] * inv);
            v[3] = (__bf16)(o[db][g * 4 + 3] * inv);
            *reinterpret_cast<bf16x4*>(op + db * 32 + g * 8 + hi * 4) = v;
          }
        if (hi == 0) a.lse[(int64_t)h * a.lq + qrow] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
      }
    } else {
      f32x4* a4 = reinterpret_cast<f32x4*>(accw);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          a4[(db * 4 + g) * 64 + lane] =
              f32x4{o[db][g * 4 + 0], o[db][g * 4 + 1], o[db][g * 4 + 2], o[db][g * 4 + 3]};
      reinterpret_cast<f32x4*>(accw + 32 * D)[lane] = f32x4{m_run, l_run, lr_run, 0.f};
    }
  }
  // Publish: unit step done (orders the state for step t+1) and slot release.
  fence_release();
  __syncthreads();
  if (tid == 0 && !has_error(a)) {
    st64_release(&a.unit_flags[unit], stamp(a.epoch, t));
    __hip_atomic_fetch_add(&a.done_count[t], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------------ scheduling

// Staging task h exists, belongs to a step <= bound, and its slot is already
// released (every unit has finished step - 2), so running it waits for nothing.
__device__ __forceinline__ bool stage_claimable(const KernelArgs& a, uint32_t h, int bound) {
  if ((int)h >= a.n_stage_tasks) return false;
  const int step = 1 + (int)h / (a.n_tiles * a.parts_per_tile);
  return step <= bound && (step < 2 || ld32(&a.done_count[step - 2]) >= (uint32_t)a.n_units);
}

__device__ __forceinline__ bool assist_claimable(const KernelArgs& a, int bound) {
  return stage_claimable(a, ld32(&a.ctrl->stage_head.v), bound);
}

// Claim the next compute task. Each XCD has a queue of the units of its head groups,
// step-major, so units that read the same KV head share an L2. A workgroup takes
// from its own queue only while that queue is at most one step ahead of the slowest
// queue, else from the slowest queue: every claimed task then needs only staging of
// steps whose slot release depends on tasks already claimed, so the schedule cannot
// deadlock whatever subset of workgroups is resident. Run by one lane.
__device__ __noinline__ bool claim_compute(const KernelArgs& a, int& unit, int& step) {
  const int own = (int)(blockIdx.x % (unsigned)a.n_xcd);
  for (int attempt = 0; attempt < 1 << 20; ++attempt) {
    if (has_error(a)) return false;
    int min_step = a.n_steps, min_x = -1;
    uint32_t heads[kMaxXcd];
    int steps[kMaxXcd];
    for (int x = 0; x < a.n_xcd; ++x) {
      int64_t ux = units_in_queue(a, x);
      heads[x] = ld32(&a.ctrl->xcd_head[x].v);
      steps[x] = (ux == 0 || (int64_t)heads[x] >= ux * a.n_steps) ? a.n_steps : (int)(heads[x] / ux);
      if (steps[x] < min_step) { min_step = steps[x]; min_x = x; }
    }
    if (min_x < 0) return false;  // every queue exhausted
    int x = (steps[own] < a.n_steps && steps[own] <= min_step + 1) ? own : min_x;
    if (cas32(&a.ctrl->xcd_head[x].v, heads[x], heads[x] + 1)) {
      int64_t ux = units_in_queue(a, x);
      step = (int)(heads[x] / ux);
      // Within a step, the queue runs its units from the last: on the causal
      // diagonal step the longest query blocks start first.
      unit = a.xcd_unit_begin[x + 1] - 1 - (int)(heads[x] % ux);
      return true;
    }
  }
  return false;
}

template <int D>
__global__ __launch_bounds__(kThreads) void ring_attn_kernel(KernelArgs a) {
  __shared__ Smem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const uint64_t t_start = ticks();
  uint32_t role = ((int)blockIdx.x < a.initial_stagers) ? kRoleStage : kRoleCompute;
  if (tid == 0) {
    max64(&a.ctrl->t_first.v, ~t_start);  // stores the complement: max of ~t = min t
    if (role == kRoleStage) {
      uint32_t n = add32(&a.ctrl->n_stage.v, 1) + 1;
      max32(&a.ctrl->max_stage.v, n);
    }
  }
  uint64_t waited = 0;
  bool fresh_stager = (role == kRoleStage);
  // A claimed compute task not yet run (thread 0 only).
  bool pending = false;
  int32_t pend_u = 0, pend_t = 0;

  while (true) {
    __syncthreads();
    if (tid == 0) {
      int32_t op = kOpExit, u = 0, s = 0;
      if (!has_error(a)) {
        maybe_controller(a);
        const bool stage_left = (int)ld32(&a.ctrl->stage_head.v) < a.n_stage_tasks;
        if (!pending) {
          if (role == kRoleStage && !fresh_stager) {
            // Back from a staging round: leave the role when staging is done or the
            // target has dropped below the current count.
            uint32_t ns = ld32(&a.ctrl->n_stage.v);
            if (!stage_left ||
                (!a.split_fixed && (int)ns > current_target(a) && cas32(&a.ctrl->n_stage.v, ns, ns - 1))) {
              if (!stage_left) add32(&a.ctrl->n_stage.v, (uint32_t)-1);
              role = kRoleCompute;
              add32(&a.ctrl->role_switches.v, 1);
              trace_rec(a, kTraceRole, 0, ld32(&a.ctrl->n_stage.v), 0, 0, 0, 0);
            }
          }
          fresh_stager = false;
          if (role == kRoleCompute && !a.split_fixed && !a.disable_staging && stage_left) {
            uint32_t ns = ld32(&a.ctrl->n_stage.v);
            if ((int)ns < current_target(a) && cas32(&a.ctrl->n_stage.v, ns, ns + 1)) {
              role = kRoleStage;
              max32(&a.ctrl->max_stage.v, ns + 1);
              add32(&a.ctrl->role_switches.v, 1);
              trace_rec(a, kTraceRole, 1, ns + 1, 0, 0, 0, 0);
            }
          }
          if (role == kRoleStage) {
            op = kOpStage;
          } else if (claim_compute(a, pend_u, pend_t)) {
            pending = true;
          } else if (stage_left && !a.disable_staging) {
            // No compute task left to claim: drain the remaining staging, whatever
            // the target (u = 1 tells the waves to ignore it).
            role = kRoleStage;
            uint32_t n = add32(&a.ctrl->n_stage.v, 1) + 1;
            max32(&a.ctrl->max_stage.v, n);
            op = kOpStage;
            u = 1;
          }
        }
        if (pending) {
          // Stall rule of §3.2: while staging work that its task depends on is still
          // unclaimed (tasks of steps up to its own whose slot is already released),
          // a compute workgroup does that work first; once every such task is
          // claimed, the data its task waits for is in the hands of running waves.
          if (pend_t > 0 && !a.disable_staging && assist_claimable(a, pend_t)) {
            op = kOpAssist;
            s = pend_t;
          } else {
            op = kOpCompute;
            u = pend_u;
            s = pend_t;
            pending = false;
          }
        }
      }
      sm.cmd[0] = op;
      sm.cmd[1] = u;
      sm.cmd[2] = s;
    }
    __syncthreads();
    const int op = sm.cmd[0];
    if (op == kOpExit) break;
    if (op == kOpCompute) {
      const int cu = sm.cmd[1], ct = sm.cmd[2];
      const uint64_t t0 = ticks();
      uint64_t w0 = 0;
      compute_task<D>(a, sm, cu, ct, w0);
      if (tid == 0) {
        const uint64_t busy = ticks() - t0 - w0;
        add64(&a.ctrl->compute_ticks.v, busy);
        add32(&a.ctrl->compute_done.v, 1);
        add64(&a.ctrl->compute_wait_ticks.v, w0);
        trace_rec(a, kTraceCompute, cu, ct, (int64_t)t0, (int64_t)w0, 0, 0);
      }
      waited += w0;
    } else if (op == kOpAssist) {
      // One staging task per wave, claimed only if its slot is already free.
      const int bound = sm.cmd[2];
      uint32_t k = 0xffffffffu;
      if (lane == 0) {
        for (int attempt = 0; attempt < 8 && k == 0xffffffffu; ++attempt) {
          uint32_t h = ld32(&a.ctrl->stage_head.v);
          if (!stage_claimable(a, h, bound)) break;
          if (cas32(&a.ctrl->stage_head.v, h, h + 1)) k = h;
        }
      }
      k = wave_bcast(k);
      if (k != 0xffffffffu) {
        uint64_t w1 = 0;
        stage_task(a, k, true, w1);
      }
    } else {
      // Staging round: every wave claims and runs staging tasks on its own until
      // staging runs out or the controller lowers the target below the count.
      const bool drain = sm.cmd[1] != 0;
      while (true) {
        uint32_t k = 0xffffffffu;
        if (lane == 0) {
          if (!has_error(a)) {
            bool stop = !drain && !a.split_fixed && (int)ld32(&a.ctrl->n_stage.v) > current_target(a);
            if (!stop) {
              uint32_t kk = add32(&a.ctrl->stage_head.v, 1);
              if ((int)kk < a.n_stage_tasks) k = kk;
            }
          }
        }
        k = wave_bcast(k);
        if (k == 0xffffffffu) break;
        uint64_t w1 = 0;
        stage_task(a, k, false, w1);
        if (lane == 0) maybe_controller(a);
        if (a.debug_flags & 2) break;
      }
    }
  }

  // Exit: the last workgroup out snapshots the statistics and resets the control
  // block for the next launch on this workspace.
  __shared__ int last;
  if (tid == 0) {
    max64(&a.ctrl->t_last.v, ticks());
    fence_release();
    uint32_t n = __hip_atomic_fetch_add(&a.ctrl->exit_count.v, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = (n == (uint32_t)a.grid - 1);
  }
  __syncthreads();
  if (!last) return;
  fence_acquire();
  DevCtrl* cb = a.ctrl;
  if (tid == 0) {
    DevStatus* ds = a.status;
    const uint32_t err = ld32(&cb->error.v);
    ds->sticky_error |= err;
    ds->last_error = err;
    ds->initial_target = a.initial_stagers;
    ds->final_target = current_target(a);
    ds->compute_done = (int32_t)ld32(&cb->compute_done.v);
    ds->stage_done = (int32_t)ld32(&cb->stage_done.v);
    ds->assist_tasks = (int32_t)ld32(&cb->assist_tasks.v);
    ds->ctrl_updates = (int32_t)ld32(&cb->ctrl_updates.v);
    ds->role_switches = (int32_t)ld32(&cb->role_switches.v);
    ds->max_stage = (int32_t)ld32(&cb->max_stage.v);
    ds->compute_ticks = (int64_t)ld64(&cb->compute_ticks.v);
    ds->compute_wait_ticks = (int64_t)ld64(&cb->compute_wait_ticks.v);
    ds->stage_ticks = (int64_t)ld64(&cb->stage_ticks.v);
    ds->stage_wait_ticks = (int64_t)ld64(&cb->stage_wait_ticks.v);
    ds->kernel_ticks = (int64_t)(ld64(&cb->t_last.v) - ~ld64(&cb->t_first.v));
    ds->trace_records = (int64_t)ld32(&cb->trace_head.v);
    ds->debug_mismatch = (int64_t)ld32(&cb->debug_mismatch.v);
    sm.cmd[3] = (int32_t)err;
  }
  __syncthreads();
  const bool had_error = sm.cmd[3] != 0;
  uint32_t* words = reinterpret_cast<uint32_t*>(cb);
  for (int i = tid; i < (int)(sizeof(DevCtrl) / 4); i += kThreads) words[i] = 0;
  for (int i = tid; i < a.n_steps; i += kThreads) a.done_count[i] = 0;
  if (had_error)
    for (int i = tid; i < 2 * a.n_tiles; i += kThreads) a.tile_parts[i] = 0;
}

template __global__ void ring_attn_kernel<64>(KernelArgs);
template __global__ void ring_attn_kernel<128>(KernelArgs);

}  // namespace mkra

// Host-side entry points of this translation unit (used by the C-ABI layer).
extern "C" __attribute__((visibility("hidden"))) hipError_t mkra_kernel_launch(const mkra::KernelArgs* a,
                                                                              hipStream_t stream) {
  dim3 grid((unsigned)a->grid), block(mkra::kThreads);
  if (a->d == 128)
    hipLaunchKernelGGL(mkra::ring_attn_kernel<128>, grid, block, 0, stream, *a);
  else
    hipLaunchKernelGGL(mkra::ring_attn_kernel<64>, grid, block, 0, stream, *a);
  return hipGetLastError();
}

extern "C" __attribute__((visibility("hidden"))) hipError_t mkra_kernel_occupancy(int d, int* blocks_per_cu) {
  if (d == 128)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, mkra::ring_attn_kernel<128>, mkra::kThreads,
                                                        0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, mkra::ring_attn_kernel<64>, mkra::kThreads, 0);
}
