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

#include <type_traits>

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

enum : int32_t { kOpExit = 0, kOpCompute = 1, kOpStage = 2 };

// ------------------------------------------------------------------ primitives

__device__ __forceinline__ uint64_t ticks() { return __builtin_amdgcn_s_memrealtime(); }

// The launch arguments where the dispatcher placed them (the kernarg segment, where
// the by-value KernelArgs parameter is the first argument). Out-of-line functions
// read them through this pointer, so the by-value parameter is never address-taken
// and never copied to scratch memory.
__device__ __forceinline__ const KernelArgs* kernel_args() {
  return (const KernelArgs*)__builtin_amdgcn_kernarg_segment_ptr();
}

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

__device__ __noinline__ void trace_rec(const KernelArgs* ap, int kind, int64_t v0, int64_t v1, int64_t v2, int64_t v3,
                          int64_t v4, int64_t v5) {
  const KernelArgs& a = *ap;
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
__device__ __noinline__ void maybe_controller(const KernelArgs* ap) {
  const KernelArgs& a = *ap;
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
  int64_t cp = cd ? (int64_t)(ct / cd) : a.cost_compute0;
  int64_t cs = sd ? (int64_t)(stt / sd) : a.cost_stage0;
  if (cp < 1) cp = 1;
  if (cs < 1) cs = 1;
  int n = eq2_target(a.grid, rp, rs, cp, cs);
  st32(&a.ctrl->target.v, (uint32_t)(n + 1));
  add32(&a.ctrl->ctrl_updates.v, 1);
  trace_rec(ap, kTraceController, rp, rs, cp, cs, a.grid, n);
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

// ------------------------------------------------------------------ LDS

typedef __attribute__((address_space(3))) void lds_void;

// The compute role's LDS ring holds kStages staged KV blocks. Each stage is its own
// object so the compiler can tell a block copy into one stage from reads of another
// (it would otherwise wait for every copy in flight before any LDS read). A staging
// task borrows the same memory as scratch for its transposes.
__shared__ __attribute__((aligned(16))) uint8_t g_stage0[Block<128>::kBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_stage1[Block<128>::kBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_stage2[Block<128>::kBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_stage3[Block<128>::kBytes];
__shared__ int32_t g_cmd[4];

template <int S>
__device__ __forceinline__ uint8_t* stage_buf() {
  static_assert(kStages == 4, "one named buffer per stage");
  if constexpr (S == 0) return g_stage0;
  else if constexpr (S == 1) return g_stage1;
  else if constexpr (S == 2) return g_stage2;
  else return g_stage3;
}

// 16-byte chunk positions inside a staged block (see Block<D>).
template <int D>
__device__ __forceinline__ int swz_k(int row, int chunk) {
  if constexpr (D == 128) return chunk ^ (row & 15);  // 16 chunks per 256-byte row
  else return chunk ^ ((row >> 1) & 7);               // 8 chunks per 128-byte row
}
__device__ __forceinline__ int swz_v(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Position of key offset x (0..15) inside its group of 16 in a V^T row: swaps bits 2
// and 3, so each lane's 8 P^T values (keys {0-3,8-11} for lanes 0-31, {4-7,12-15} for
// lanes 32-63, from the 32x32 accumulator layout) meet 8 contiguous V^T values.
__device__ __forceinline__ int vt_pos(int key) {
  int x = key & 15;
  return (key & ~15) | (x & 3) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Exact bf16 -> fp16 for |v| < 65520 (the fp16 range); two values per 32-bit word.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  f16x2 h = {(_Float16)__builtin_bit_cast(float, w << 16), (_Float16)__builtin_bit_cast(float, w & 0xffff0000u)};
  return __builtin_bit_cast(uint32_t, h);
}

// Waits until at most n vector-memory operations of this wave are outstanding.
__device__ __forceinline__ void wait_vm(int n) {
  // s_waitcnt immediate: vmcnt low bits [3:0], high bits [15:14]; expcnt and lgkmcnt
  // at their maxima (no wait).
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0f70); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0f72); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0f74); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0f76); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0f78); break;
    default: __builtin_amdgcn_s_waitcnt(0x0f70); break;
  }
}

// ------------------------------------------------------------------ staging role

// One staging task, run by the whole workgroup: 128-row tile j of the chunk of step
// t (chunk (rank - t) mod N, read from its home in kv_chunks, which stands for the
// predecessor's memory) becomes staged blocks in slot t % 2: K swizzled, V transposed
// to fp16. The slot is free once every unit has finished step t - 2. One release per
// tile publishes its epoch-stamped flag (paper §4: epoch-stamped readiness flags).
template <int D>
__device__ void stage_tile(const KernelArgs& a, uint32_t k, bool assist) {
  constexpr int CPR = D / 8;                        // 16-byte chunks per K/V row
  constexpr int KCH = kBN * CPR / kThreads;         // K (or V) chunks per thread per block
  constexpr int VPITCH = kBN + 2;                   // fp16 scratch row pitch (breaks bank conflicts)
  constexpr int NB = 4;                             // blocks per batch (one scratch stage each)
  static_assert(KCH >= 1 && kBN * CPR % kThreads == 0, "block split");
  const int tid = threadIdx.x, lane = tid & 63;
  const uint64_t t_begin = ticks();
  const int t = (int)k / a.n_tiles;
  const int j = (int)k % a.n_tiles;
  const int slot = t & 1;
  uint64_t w = 0;
  // Slot release (every wave waits; a timeout leaves the error word set for all).
  if (t >= 2) wave_wait_ge32(a, &a.done_count[t - 2], (uint32_t)a.n_units, w);
  __syncthreads();
  const bool ok = !has_error(a);
  __syncthreads();
  if (ok) {
    const int c = chunk_of_step(a, t);
    const int64_t row_elems = (int64_t)a.hkv * D;
    const uint16_t* kh = a.kv + (int64_t)c * a.chunk_elems;
    const uint16_t* vh = kh + (int64_t)a.lk * row_elems;
    uint8_t* sbase = a.slots + (int64_t)slot * a.slot_bytes;
    const int nb = min(2, a.n_blocks - 2 * j);       // 64-key blocks in this tile
    const int n_pairs = a.hkv * nb;
    for (int p0 = 0; p0 < n_pairs; p0 += NB) {
      u32x4 kr[NB][KCH], vr[NB][KCH];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int p = p0 + b;
        const int g = p / nb, kb = 2 * j + p % nb;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
          const int q = tid + i * kThreads, r = q / CPR, cc = q % CPR, key = kb * kBN + r;
          const bool in = p < n_pairs && key < a.lk;
          const int64_t off = ((int64_t)key * a.hkv + g) * D + 8 * cc;
          kr[b][i] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kh + off)) : u32x4{0, 0, 0, 0};
          vr[b][i] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vh + off)) : u32x4{0, 0, 0, 0};
        }
      }
      uint8_t* scr[NB] = {g_stage0, g_stage1, g_stage2, g_stage3};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int p = p0 + b;
        if (p >= n_pairs) break;
        const int g = p / nb, kb = 2 * j + p % nb;
        uint8_t* blk = sbase + ((int64_t)g * a.n_blocks + kb) * Block<D>::kBytes;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
          const int q = tid + i * kThreads, r = q / CPR, cc = q % CPR;
          *reinterpret_cast<u32x4*>(blk + r * (D * 2) + 16 * swz_k<D>(r, cc)) = kr[b][i];
          // V: 8 consecutive d of key r -> fp16 column vt_pos(r) of 8 scratch rows.
          uint16_t* sc = reinterpret_cast<uint16_t*>(scr[b]);
          const int pos = vt_pos(r);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t h2 = bf16x2_to_f16x2(vr[b][i][e]);
            sc[(8 * cc + 2 * e) * VPITCH + pos] = (uint16_t)(h2 & 0xffffu);
            sc[(8 * cc + 2 * e + 1) * VPITCH + pos] = (uint16_t)(h2 >> 16);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int p = p0 + b;
        if (p >= n_pairs) break;
        const int g = p / nb, kb = 2 * j + p % nb;
        uint8_t* blk = sbase + ((int64_t)g * a.n_blocks + kb) * Block<D>::kBytes + Block<D>::kKBytes;
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(scr[b]);
        for (int q = tid; q < D * 8; q += kThreads) {
          const int d = q / 8, cc = q % 8;
          const uint16_t* row = sc + d * VPITCH + 8 * cc;  // 4-byte aligned (VPITCH even)
          u32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = *reinterpret_cast<const uint32_t*>(row + 2 * e);
          *reinterpret_cast<u32x4*>(blk + d * 128 + 16 * swz_v(d, cc)) = v;
        }
      }
      __syncthreads();
    }
    if (a.debug_flags & 1) {
      // Debug: re-derive the K part of every block of the tile from the chunk's home.
      uint32_t bad = 0;
      for (int p = 0; p < n_pairs; ++p) {
        const int g = p / nb, kb = 2 * j + p % nb;
        const uint8_t* blk = sbase + ((int64_t)g * a.n_blocks + kb) * Block<D>::kBytes;
        for (int q = tid; q < kBN * CPR; q += kThreads) {
          const int r = q / CPR, cc = q % CPR, key = kb * kBN + r;
          u32x4 want = key < a.lk ? *reinterpret_cast<const u32x4*>(kh + ((int64_t)key * a.hkv + g) * D + 8 * cc)
                                  : u32x4{0, 0, 0, 0};
          u32x4 got = *reinterpret_cast<const u32x4*>(blk + r * (D * 2) + 16 * swz_k<D>(r, cc));
          bad += (want[0] != got[0]) | (want[1] != got[1]) | (want[2] != got[2]) | (want[3] != got[3]);
        }
      }
      if (bad) add32(&a.ctrl->debug_mismatch.v, bad);
      __syncthreads();
    }
    if (a.stage_delay_ticks > 0 && tid == 0) {
      uint32_t hsh = (k * 2654435761u) ^ (uint32_t)a.epoch;
      uint64_t until = ticks() + (hsh % (uint32_t)a.stage_delay_ticks);
      while (ticks() < until) __builtin_amdgcn_s_sleep(1);
    }
  }
  // Every wave's stores precede the barrier; one agent-scope release by thread 0
  // then covers the whole tile (workgroup-scope order, then agent scope).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (tid == 0) {
    if (ok) st64_release(&a.slot_flags[slot * a.n_tiles + j], stamp(a.epoch, t));
    const uint64_t busy = ticks() - t_begin - w;
    add64(&a.ctrl->stage_ticks.v, busy);
    add32(&a.ctrl->stage_done.v, 1);
    add64(&a.ctrl->stage_wait_ticks.v, w);
    if (assist) add32(&a.ctrl->assist_tasks.v, 1);
    trace_rec(kernel_args(), kTraceStage, k, t, j, (int64_t)t_begin, assist ? 1 : 0, ok ? 1 : -1);
  }
  (void)lane;
}

// ------------------------------------------------------------------ compute role

// Copies staged block `src` (global) into LDS stage S: each wave moves 1 KB per
// instruction with global_load_lds_dwordx4 (no registers, no VALU).
template <int D, int S>
__device__ __forceinline__ void dma_block(const uint8_t* src) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < Block<D>::kChunksPerThread; ++i) {
    const int ch = i * kThreads + w * 64;
    __builtin_amdgcn_global_load_lds(src + (int64_t)(ch + lane) * 16, (lds_void*)(stage_buf<S>() + ch * 16), 16, 0, 0);
  }
}

template <int D>
__device__ void compute_task(const KernelArgs& a, int unit, int t, uint64_t& waited) {
  constexpr int KK = D / 16;                    // k-slices of Q K^T
  constexpr int DB = D / 32;                    // 32-row blocks of O^T
  constexpr int NI = Block<D>::kChunksPerThread;  // block-copy instructions per wave per tile

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hi = lane >> 5, col = lane & 31;
  const int p = unit / a.n_qblocks, qb = unit % a.n_qblocks;
  const int kvh = p / a.n_hgroups, hgi = p % a.n_hgroups;
  const int h = kvh * a.gqa + hgi * a.hg + (w % a.hg);
  const int q0w = qb * a.bq + (w / a.hg) * kRowsPerWave;
  const bool wave_rows = q0w < a.lq;
  const int qrow = q0w + col;
  const bool diag = a.causal && t == 0;
  const uint8_t* sblk = a.slots + (int64_t)(t & 1) * a.slot_bytes + (int64_t)kvh * a.n_blocks * Block<D>::kBytes;
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
  {
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

  // Running state: O^T blocks, max (log2 units of the scaled score), and two running
  // sums: l of the exact P (for the log-sum-exp) and lr of the fp16-rounded P that the
  // PV product weights V with (for the normalisation, see below).
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

  // Per-lane LDS offsets (the swizzles depend only on the lane).
  const int k_off = col * (D * 2);                // + kb*32*(D*2) + 16*swz
  const int kx = (D == 128) ? (col & 15) : ((col >> 1) & 7);
  const int v_off = Block<D>::kKBytes + col * 128;  // + db*32*128 + 16*swz
  const int vx = (col >> 1) & 7;

  auto issue = [&](int kt, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    const int j = (kt * kBN) / kStageRows;
    if (j >= ready_upto) {
      ok &= wave_wait_stamp(a, &flags[j], st, waited);
      ready_upto = j + 1;
    }
    dma_block<D, S>(sblk + (int64_t)kt * Block<D>::kBytes);
  };

  auto compute_tile = [&](int kt, const uint8_t* sb) {
    // S^T = K Q^T for 2 blocks of 32 keys.
    f32x16 s[kBN / 32];
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
      s[kb] = f32x16{};
      const uint8_t* kr = sb + kb * 32 * (D * 2) + k_off;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        bf16x8 av = *reinterpret_cast<const bf16x8*>(kr + 16 * ((2 * kk + hi) ^ kx));
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
    // Online-softmax update (FlashAttention-2), rescaling only when the max has grown
    // by more than kTau since the last rescale.
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
    // lr sums the fp16-rounded P (two per v_dot2c_f32_f16 against (1, 1)); normalising
    // O by it makes the applied weights sum to one, so a dominant key's rounding
    // cancels in O / lr.
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
      const uint8_t* vr = sb + db * 32 * 128 + v_off;
#pragma unroll
      for (int pp = 0; pp < kBN / 16; ++pp) {
        f16x8 av = *reinterpret_cast<const f16x8*>(vr + 16 * ((2 * pp + hi) ^ vx));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[pp], o[db], 0, 0, 0);
      }
    }
  };

  auto step = [&](int kt, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    if (kt >= n_kt) return;
    // This wave's copies of tile kt are done once at most the newer tiles' copies
    // remain; the barrier makes every wave's part visible and frees stage S-1.
    const int newer = min(kStages - 2, n_kt - 1 - kt);
    wait_vm(newer * NI);
    __builtin_amdgcn_s_barrier();
    // Refill stage S-1 (freed by the barrier) with tile kt+3: now if its staged tile
    // is known to be ready, else after this tile's compute (the wait may block).
    const int kn = kt + kStages - 1;
    const bool early = kn < n_kt && (kn * kBN) / kStageRows < ready_upto;
    if (early) issue(kn, std::integral_constant<int, (S + kStages - 1) % kStages>{});
    if (kt < w_kt) compute_tile(kt, stage_buf<S>());
    if (kn < n_kt && !early) issue(kn, std::integral_constant<int, (S + kStages - 1) % kStages>{});
  };

  // Prologue: kStages-1 blocks in flight, then one per tile.
  if (0 < n_kt) issue(0, std::integral_constant<int, 0>{});
  if (1 < n_kt) issue(1, std::integral_constant<int, 1>{});
  if (2 < n_kt) issue(2, std::integral_constant<int, 2>{});
  for (int kt = 0; kt < n_kt; kt += kStages) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
    step(kt + 2, std::integral_constant<int, 2>{});
    step(kt + 3, std::integral_constant<int, 3>{});
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
  // Publish: unit step done (orders the state for step t+1) and slot release. Every
  // wave's stores precede the barrier; one agent-scope release by thread 0 covers them.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
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
  const int step = (int)h / a.n_tiles;
  return step <= bound && (step < 2 || ld32(&a.done_count[step - 2]) >= (uint32_t)a.n_units);
}

// Claim the next compute task. Each XCD has a queue of the units of its head groups,
// step-major, so units that read the same KV head share an L2. A workgroup takes
// from its own queue only while that queue is at most one step ahead of the slowest
// queue, else from the slowest queue: every claimed task then needs only staging of
// steps whose slot release depends on tasks already claimed, so the schedule cannot
// deadlock whatever subset of workgroups is resident. Run by one lane.
__device__ __noinline__ bool claim_compute(const KernelArgs* ap, int& unit, int& step) {
  const KernelArgs& a = *ap;
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
  const int tid = threadIdx.x;
  const uint64_t t_start = ticks();
  uint32_t role = ((int)blockIdx.x < a.initial_stagers) ? kRoleStage : kRoleCompute;
  if (tid == 0) {
    max64(&a.ctrl->t_first.v, ~t_start);  // stores the complement: max of ~t = min t
    if (role == kRoleStage) {
      uint32_t n = add32(&a.ctrl->n_stage.v, 1) + 1;
      max32(&a.ctrl->max_stage.v, n);
    }
  }
  // A claimed compute task not yet run (thread 0 only).
  bool pending = false;
  int32_t pend_u = 0, pend_t = 0;

  while (true) {
    __syncthreads();
    if (tid == 0) {
      int32_t op = kOpExit, x = 0, y = 0;
      if (!has_error(a)) {
        maybe_controller(kernel_args());
        const bool stage_left = (int)ld32(&a.ctrl->stage_head.v) < a.n_stage_tasks;
        if (!pending) {
          // Role changes happen at task boundaries (§3.2): leave the staging role when
          // staging is done or the target dropped below the count; join it when the
          // count is below the target.
          if (role == kRoleStage) {
            uint32_t ns = ld32(&a.ctrl->n_stage.v);
            if (!stage_left) {
              add32(&a.ctrl->n_stage.v, (uint32_t)-1);
              role = kRoleCompute;
            } else if (!a.split_fixed && (int)ns > current_target(a) && cas32(&a.ctrl->n_stage.v, ns, ns - 1)) {
              role = kRoleCompute;
              add32(&a.ctrl->role_switches.v, 1);
              trace_rec(kernel_args(), kTraceRole, 0, ns - 1, 0, 0, 0, 0);
            }
          } else if (!a.split_fixed && !a.disable_staging && stage_left) {
            uint32_t ns = ld32(&a.ctrl->n_stage.v);
            if ((int)ns < current_target(a) && cas32(&a.ctrl->n_stage.v, ns, ns + 1)) {
              role = kRoleStage;
              max32(&a.ctrl->max_stage.v, ns + 1);
              add32(&a.ctrl->role_switches.v, 1);
              trace_rec(kernel_args(), kTraceRole, 1, ns + 1, 0, 0, 0, 0);
            }
          }
          if (role == kRoleStage) {
            uint32_t kk = add32(&a.ctrl->stage_head.v, 1);
            if ((int)kk < a.n_stage_tasks) {
              op = kOpStage;
              x = (int32_t)kk;
            } else {
              add32(&a.ctrl->n_stage.v, (uint32_t)-1);
              role = kRoleCompute;
            }
          }
          if (op == kOpExit && role == kRoleCompute) {
            if (claim_compute(kernel_args(), pend_u, pend_t)) {
              pending = true;
            } else if (stage_left && !a.disable_staging) {
              // No compute task left to claim: help drain the remaining staging.
              uint32_t kk = add32(&a.ctrl->stage_head.v, 1);
              if ((int)kk < a.n_stage_tasks) {
                op = kOpStage;
                x = (int32_t)kk;
              }
            }
          }
        }
        if (pending) {
          // Stall rule of §3.2: while staging work that the claimed task depends on is
          // unclaimed (tasks of steps up to its own whose slot is already released),
          // the compute workgroup does that work first; once every such task is
          // claimed, the data its task waits for is in the hands of running waves.
          uint32_t h = ld32(&a.ctrl->stage_head.v);
          if (!a.disable_staging && stage_claimable(a, h, pend_t) && cas32(&a.ctrl->stage_head.v, h, h + 1)) {
            op = kOpStage;
            x = (int32_t)h;
            y = 1;
          } else {
            op = kOpCompute;
            x = pend_u;
            y = pend_t;
            pending = false;
          }
        }
      }
      g_cmd[0] = op;
      g_cmd[1] = x;
      g_cmd[2] = y;
    }
    __syncthreads();
    const int op = g_cmd[0], x = g_cmd[1], y = g_cmd[2];
    if (op == kOpExit) break;
    if (op == kOpCompute) {
      const uint64_t t0 = ticks();
      uint64_t w0 = 0;
      compute_task<D>(a, x, y, w0);
      if (tid == 0) {
        const uint64_t busy = ticks() - t0 - w0;
        add64(&a.ctrl->compute_ticks.v, busy);
        add32(&a.ctrl->compute_done.v, 1);
        add64(&a.ctrl->compute_wait_ticks.v, w0);
        trace_rec(kernel_args(), kTraceCompute, x, y, (int64_t)t0, (int64_t)w0, 0, 0);
      }
    } else {
      stage_tile<D>(a, (uint32_t)x, y != 0);
      if (tid == 0) maybe_controller(kernel_args());
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
  }
  __syncthreads();
  uint32_t* words = reinterpret_cast<uint32_t*>(cb);
  for (int i = tid; i < (int)(sizeof(DevCtrl) / 4); i += kThreads) words[i] = 0;
  for (int i = tid; i < a.n_steps; i += kThreads) a.done_count[i] = 0;
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
