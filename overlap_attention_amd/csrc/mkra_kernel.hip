// Persistent ring-attention forward for gfx950 (MI355X).
//
// One launch runs every ring step of one rank (mKernel paper "mKernel: Fast
// Multi-GPU, Multi-Node Fused Kernels", §4 / Table 3, Ring Attention row). Its
// workgroups take roles (§3.2): COMPUTE workgroups run the blockwise
// FlashAttention forward of a (unit, step group) task and carry the online-softmax
// state (running max m, running sum l, unnormalised O) from step to step; STAGING
// workgroups play the ring receive on one GPU, copying the chunk of a coming step
// into a ring of eight slots in HBM and publishing an epoch-stamped ready flag per
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

#include <algorithm>
#include <type_traits>
#include <utility>

#include "mkra_args.h"

// Operand reads in flight ahead of the MFMA that uses the oldest (matrix phase). With
// the matrix phase down to MFMAs and operand reads, 2 was fastest on the 64K-token
// workload (same-box A/B runs: 4 was 2.4 % faster than 6, and 2 0.5 % faster than 4;
// 1 exposes the LDS latency, 22 % slower).
#ifndef MKRA_LDS_AHEAD
#define MKRA_LDS_AHEAD 2
#endif

namespace mkra {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Lazy rescale bound: while each lane's partial sum of a block's P stays at or below
// kSumMax, the running max used for the exponentials is kept (see compute_task).
constexpr float kSumMax = 16384.0f;
constexpr float kLn2 = 0.69314718055994530942f;

enum : int32_t { kOpExit = 0, kOpCompute = 1, kOpStage = 2 };

// ------------------------------------------------------------------ primitives

__device__ __forceinline__ uint64_t ticks() { return __builtin_amdgcn_s_memrealtime(); }

// The launch arguments where the dispatcher placed them (the kernarg segment, where
// the by-value KernelArgs parameter is the first argument). Functions that may be
// called out of line read them through this pointer, so the by-value parameter is
// never address-taken and never copied to scratch memory.
// Valid only in the kernel's own body: in a function the compiler does not inline,
// the intrinsic has no segment and yields a null base, and every argument read
// through it faults. ring_attn_kernel evaluates it once, first thing, and passes the
// pointer down; nothing else may call it (a build test checks that the only call in
// the kernels' code is to trace_rec).
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

// max(a, b, c) in one v_max3_f32 (the library fmaxf would first quiet NaN inputs).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ bool has_error(const KernelArgs& a) { return ld32(&a.ctrl->error.v) != kErrNone; }

__device__ __forceinline__ void raise_error(const KernelArgs& a, uint32_t code) {
  cas32(&a.ctrl->error.v, kErrNone, code);
}

// Ring step staged at staging position pos (the staging tasks of one position are
// consecutive).
__device__ __forceinline__ int stage_step_of(const KernelArgs& a, int pos) {
  return a.stage_interleave ? (int)a.stage_order[pos & (kSlots - 1)] : pos;
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

template <class KA>
__device__ __forceinline__ int target_of(const KA& a, uint32_t v) {
  return v == 0 ? a.initial_stagers : (int)v - 1;  // 0 = not yet set by the controller
}
__device__ __forceinline__ int current_target(const KernelArgs& a) { return target_of(a, ld32(&a.ctrl->target.v)); }

template <class KA>
__device__ __forceinline__ int64_t units_in_queue(const KA& a, int x) {
  return a.xcd_unit_begin[x + 1] - a.xcd_unit_begin[x];
}

// Step groups: the first n_big groups have `group` steps each, the later ones (the
// tail) `tail_group` steps each, the last one possibly fewer. First step of group g,
// and one past its last.
// A launch's step groups start at ring step step_lo (0 unless the launch runs one
// step of the unfused baseline).
template <class KA>
__device__ __forceinline__ int group_rel_first(const KA& a, int g) {
  return g < a.n_big ? g * a.group : a.n_big * a.group + (g - a.n_big) * a.tail_group;
}
template <class KA>
__device__ __forceinline__ int group_first(const KA& a, int g) {
  return a.step_lo + group_rel_first(a, g);
}
template <class KA>
__device__ __forceinline__ int group_end(const KA& a, int g) {
  return min(a.n_steps, group_first(a, g + 1));
}

// Unit-steps covered by the first h tasks of a queue of ux units (tasks are
// group-major).
template <class KA>
__device__ __forceinline__ int64_t steps_claimed(const KA& a, int64_t ux, int64_t h) {
  if (h >= ux * a.n_groups) return ux * (a.n_steps - a.step_lo);
  const int g = (int)(h / ux);
  const int f = group_rel_first(a, g);
  return ux * f + (h % ux) * (group_end(a, g) - a.step_lo - f);
}

// Run by one lane, from a snapshot of the queue heads and the staging head. Compute
// work is counted in unit-steps (R_p remaining, C_p measured per unit-step).
// Rate-limited by a compare-and-swap on the update time.
__device__ __forceinline__ void maybe_controller(const KernelArgs* ap, const uint32_t (&heads)[kMaxXcd],
                                                 uint32_t stage_head, uint64_t last) {
  const KernelArgs& a = *ap;
  if (a.split_fixed || a.disable_staging) return;
  uint64_t now = ticks();
  if (last != 0 && now - last < a.ctrl_period_ticks) return;
  if (!cas64(&a.ctrl->ctrl_time.v, last, now)) return;
  int64_t rs = a.n_stage_tasks - ((int)stage_head < a.n_stage_tasks ? (int)stage_head : a.n_stage_tasks);
  int64_t claimed = 0;
#pragma unroll
  for (int x = 0; x < kMaxXcd; ++x) {
    if (x >= a.n_xcd) break;
    claimed += steps_claimed(a, units_in_queue(a, x), (int64_t)heads[x]);
  }
  int64_t rp = (int64_t)a.n_units * a.n_steps - claimed;
  // Per-task cost of a role. Staging: its busy time plus its waits for a free slot
  // (slots free at the pace of the compute role, so that wait is part of what a
  // staging task costs). Compute: its busy time only. A compute task waits for tiles
  // the staging role has not delivered yet; counted as compute cost, that wait would
  // shift workgroups away from staging exactly when staging lags.
  uint64_t cd = ld32(&a.ctrl->compute_done.v), ct = ld64(&a.ctrl->compute_ticks.v);
  uint64_t sd = ld32(&a.ctrl->stage_done.v),
           stt = ld64(&a.ctrl->stage_ticks.v) + ld64(&a.ctrl->stage_wait_ticks.v);
  // The cost-model priors count as one ring step's tasks of each role (n_units
  // compute unit-steps, stage_per_step staging tasks), so the first few measured tasks
  // (cold caches, no slot waits yet) do not swing the split.
  const uint64_t kc = (uint64_t)a.n_units, ks = (uint64_t)a.stage_per_step;
  int64_t cp, cs, rp2;
  if (a.ctrl_paper) {
    // Eq. (2) with the inputs §3.2 names: every remaining task of each role and the
    // measured busy cost per finished task (the cost model until a role has finished
    // one).
    cp = cd > 0 ? (int64_t)(ct / cd) : a.cost_compute0;
    cs = sd > 0 ? (int64_t)(ld64(&a.ctrl->stage_ticks.v) / sd) : a.cost_stage0;
    rp2 = rp;
  } else {
    cp = (int64_t)((ct + kc * (uint64_t)a.cost_compute0) / (cd + kc));
    cs = (int64_t)((stt + ks * (uint64_t)a.cost_stage0) / (sd + ks));
    // R_p counts the compute work that can overlap the remaining staging: the
    // unit-steps of the last staged ring step (with interleaved parallel step groups,
    // the last step of every group) need tiles staged last, so they follow the last
    // staging task whatever the split, and Eq. (2) balances the rest.
    rp2 = rp > a.rp_tail ? rp - a.rp_tail : 0;
  }
  if (cp < 1) cp = 1;
  if (cs < 1) cs = 1;
  int n = eq2_target(a.grid, rp2, rs, cp, cs);
  st32(&a.ctrl->target.v, (uint32_t)(n + 1));
  add32(&a.ctrl->ctrl_updates.v, 1);
  if (a.trace != nullptr) trace_rec(ap, kTraceController, rp2, rs, cp, cs, a.grid, n);
}
// ------------------------------------------------------------------ waits
// All waits are bounded: past timeout_ticks they raise MK_E_TIMEOUT, and every wait
// returns early once any error is raised, so every workgroup reaches its exit.

// Wave-wide wait until *p >= target; acquire on success.
__device__ __forceinline__ bool wave_wait_ge32(const KernelArgs& a, uint32_t* p, uint32_t target, uint64_t& waited) {
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
__device__ __forceinline__ bool wave_wait_stamp(const KernelArgs& a, const uint64_t* p, uint64_t value, uint64_t& waited) {
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

// A phase of the compute role covers Phase<D>::kBlocks consecutive staged blocks of
// one KV head (1 or 2; the blocks of a 128-row staged tile are adjacent in the slot,
// so a phase is one contiguous copy whose blocks' K parts land side by side in the
// stage's K region, one K matrix of kKeys rows, and their Vᵀ parts side by side in
// its Vᵀ region). Two blocks per phase at D = 64 (32 products per phase, as at
// D = 128) passed the parity tests but ran 8% slower on the 32K-token MHA workload
// than one, so every head size runs one block per phase.
template <int D>
struct Phase {
  static constexpr int kBlocks = 1;
  static constexpr int kKeys = kBlocks * kBN;
  static constexpr int kBytes = kBlocks * Block<D>::kBytes;
  static constexpr int kKBytes = kBlocks * Block<D>::kKBytes;  // K (or Vᵀ) region of a stage
  static constexpr int kChunksPerThread = kBytes / 16 / kThreads;
};
static_assert(Phase<64>::kBytes <= Phase<128>::kBytes, "the LDS ring is sized for D = 128");
static_assert(Phase<64>::kKeys <= kStageRows && kStageRows % Phase<64>::kKeys == 0, "a phase lies in one staged tile");


// The compute role's LDS ring of kStages staged KV blocks: the K parts of stages 0..3
// first, then their Vᵀ parts (stage_k / stage_v byte offsets), so every operand read
// reaches its stage with one per-lane address register and the 16-bit offset field.
// The compute role reads the ring only through ds_read_b128 in inline asm
// (lds_read16) with explicit waits: the compiler cannot tell which stage a block copy
// in flight writes and would otherwise wait for every copy before any LDS read. A
// staging task borrows the same memory as scratch for its transposes (scratch_buf).
constexpr int kLdsBytes = kStages * Phase<128>::kBytes;
__shared__ __attribute__((aligned(16))) uint8_t g_lds[kLdsBytes];
__shared__ int32_t g_cmd[4];
// Waves of the workgroup whose stores of the finished compute task are complete (the
// publish handshake at the end of a compute task).
__shared__ uint32_t g_pub_count;

template <int D, int S>
constexpr int stage_k() { return S * Phase<D>::kKBytes; }
template <int D, int S>
constexpr int stage_v() { return (kStages + S) * Phase<D>::kKBytes; }

template <int B>
__device__ __forceinline__ uint8_t* scratch_buf() {
  static_assert(B >= 0 && B < 4, "scratch");
  return g_lds + B * (kLdsBytes / 4);
}

// LDS byte address of g_lds (the 32-bit offset the ds_* instructions take).
__device__ __forceinline__ uint32_t lds_base() { return (uint32_t)(uintptr_t)((lds_void*)g_lds); }

// 16 bytes from LDS address addr + OFF (OFF < 65536, the instruction's offset field).
// The result may only be used after lgkm_wait with a count that covers it.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536 && OFF % 16 == 0, "ds_read_b128 offset");
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}

// Waits until at most N LDS reads of this wave are outstanding (LDS operations
// complete in order, so every read older than the newest N is done); v, the register
// such a read filled, is tied to the wait so no use of it moves above.
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& v) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
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

// bf16 -> fp16 (round to nearest even), two values per 32-bit word. Exact for
// 2^-14 <= |v| < 2^16 (fp16 normals hold bf16's 8 significant bits); below 2^-14
// the fp16 subnormal spacing 2^-24 rounds the value (absolute error at most 2^-25),
// and |v| >= 2^16 would overflow: the staging role refuses such a V
// (bf16x2_outside_f16) instead of converting it.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  f16x2 h = {(_Float16)__builtin_bit_cast(float, w << 16), (_Float16)__builtin_bit_cast(float, w & 0xffff0000u)};
  return __builtin_bit_cast(uint32_t, h);
}

// True if either bf16 of the word has |v| >= 2^16 or is not finite (exponent field
// >= 127 + 16): a value the fp16 PV operand cannot hold.
__device__ __forceinline__ bool bf16x2_outside_f16(uint32_t w) {
  return (w & 0x7f80u) >= (143u << 7) || (w & 0x7f800000u) >= (143u << 23);
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

// One staging task, run by the whole workgroup: piece pc (KV heads [pc*piece_heads,
// +piece_heads)) of 128-row tile j of the chunk of step t (chunk (rank - t) mod N, read
// from its home in kv_chunks, which stands for the predecessor's memory) becomes
// staged blocks in slot t % kSlots: K swizzled, V transposed to fp16. The slot is free
// once every unit has finished step t - kSlots. One release per piece publishes its
// epoch-stamped flag (paper §4: epoch-stamped readiness flags).
template <int D>
__device__ __forceinline__ void stage_tile(const KernelArgs& a, const KernelArgs* ap, uint32_t k, bool assist) {
  constexpr int CPR = D / 8;                        // 16-byte chunks per K/V row
  constexpr int KCH = kBN * CPR / kThreads;         // K (or V) chunks per thread per block
  constexpr int VPITCH = kBN + 2;                   // fp16 scratch row pitch (breaks bank conflicts)
  constexpr int NB = 4;                             // blocks per batch (one scratch stage each)
  static_assert(KCH >= 1 && kBN * CPR % kThreads == 0, "block split");
  const int tid = threadIdx.x, lane = tid & 63;
  const uint64_t t_begin = ticks();
  const int t = stage_step_of(a, (int)k / a.stage_per_step);
  const int j = ((int)k % a.stage_per_step) / a.n_pieces;
  const int pc = (int)k % a.n_pieces;
  const int g0 = pc * a.piece_heads;               // first KV head of the piece
  const int slot = t % kSlots;
  uint64_t w = 0;
  // Slot release (every wave waits; a timeout leaves the error word set for all).
  if (t >= kSlots && !a.external_order) wave_wait_ge32(a, &a.done_count[t - kSlots], (uint32_t)a.n_units, w);
  // One verdict for the whole workgroup (the barriers below are inside the branch).
  const bool ok = __syncthreads_or(has_error(a) ? 1 : 0) == 0;
  bool v_range = false;  // some V of the tile does not fit the fp16 PV operand
  if (ok) {
    const int c = chunk_of_step(a, t);
    const int64_t row_elems = (int64_t)a.hkv * D;
    const uint16_t* kh = a.kv + (int64_t)c * a.chunk_elems;
    const uint16_t* vh = kh + (int64_t)a.lk * row_elems;
    uint8_t* sbase = a.slots + (int64_t)slot * a.slot_bytes;
    const int nb = min(2, a.n_blocks - 2 * j);       // 64-key blocks in this tile
    const int n_pairs = min(a.piece_heads, a.hkv - g0) * nb;
    for (int p0 = 0; p0 < n_pairs; p0 += NB) {
      u32x4 kr[NB][KCH], vr[NB][KCH];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int p = p0 + b;
        const int g = g0 + p / nb, kb = 2 * j + p % nb;
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
          const int q = tid + i * kThreads, r = q / CPR, cc = q % CPR, key = kb * kBN + r;
          const bool in = p < n_pairs && key < a.lk;
          const int64_t off = ((int64_t)key * a.hkv + g) * D + 8 * cc;
          kr[b][i] = in ? *reinterpret_cast<const u32x4*>(kh + off) : u32x4{0, 0, 0, 0};
          vr[b][i] = in ? *reinterpret_cast<const u32x4*>(vh + off) : u32x4{0, 0, 0, 0};
        }
      }
      uint8_t* scr[NB] = {scratch_buf<0>(), scratch_buf<1>(), scratch_buf<2>(), scratch_buf<3>()};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int p = p0 + b;
        if (p >= n_pairs) break;
        const int g = g0 + p / nb, kb = 2 * j + p % nb;
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
            v_range |= bf16x2_outside_f16(vr[b][i][e]);
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
        const int g = g0 + p / nb, kb = 2 * j + p % nb;
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
    // A V outside the fp16 range ends the launch through the error path (every wait
    // returns once the error word is set) and is reported as unsupported.
    v_range = __syncthreads_or(v_range ? 1 : 0) != 0;
    if (v_range && tid == 0) raise_error(a, kErrRange);
    if (a.debug_flags & 1) {
      // Debug: re-derive the K part of every block of the tile from the chunk's home.
      uint32_t bad = 0;
      for (int p = 0; p < n_pairs; ++p) {
        const int g = g0 + p / nb, kb = 2 * j + p % nb;
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
  // Every wave waits for its own stores to complete (a workgroup-scope fence alone
  // does not: it emits no wait before the barrier), then one agent-scope release by
  // thread 0 covers the whole tile.
  wait_vm(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (tid == 0) {
    if (ok && !v_range) st64_release(&a.slot_flags[(int64_t)slot * a.stage_per_step + (int)k % a.stage_per_step],
                                     stamp(a.epoch, t));
    const uint64_t busy = ticks() - t_begin - w;
    add64(&a.ctrl->stage_ticks.v, busy);
    add32(&a.ctrl->stage_done.v, 1);
    add64(&a.ctrl->stage_wait_ticks.v, w);
    if (assist) add32(&a.ctrl->assist_tasks.v, 1);
    if (a.trace != nullptr) trace_rec(ap, kTraceStage, k, t, j, (int64_t)t_begin, assist ? 1 : 0, ok ? pc : -1);
  }
  (void)lane;
}

// ------------------------------------------------------------------ compute role

// A 64-bit pointer that is the same in every lane, moved to SGPRs.
__device__ __forceinline__ const uint8_t* wave_bcast_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  return (const uint8_t*)(uintptr_t)(((uint64_t)wave_bcast((uint32_t)(v >> 32)) << 32) | wave_bcast((uint32_t)v));
}

// Per-lane byte offsets of a wave's block-copy instructions: instruction I moves the
// 16 bytes at I * kThreads * 16 + 16 * lane of the wave's slice.
template <int D>
struct CopyLanes {
  uint32_t off[Phase<D>::kChunksPerThread];
};

// Copy instruction I of a staged block into LDS stage S: each wave moves 1 KB per
// global_load_lds_dwordx4 (no registers, no VALU); instructions below half the block
// fill the stage's K part (stage_k), the rest its Vᵀ part (stage_v). src_w is the
// block's address plus this wave's 1 KB offset and m0w the LDS address of the same
// offset in stage 0, both wave-uniform; the instruction takes src_w from SGPRs and the
// lane's offset from a
// VGPR computed once per task, so issuing a copy needs no vector ALU work (the matrix
// phase threads these through its MFMAs, and the vector ALU there belongs to the
// other wave's softmax).
template <int D, int S, int I>
__device__ __forceinline__ void dma_one(const uint8_t* src_w, const CopyLanes<D>& cl, uint32_t m0w) {
  // Instruction I moves bytes [I, I+1) * kThreads * 16 of the phase: part x of its
  // block b, a K part or a Vᵀ part (never both).
  constexpr int kSrc = I * kThreads * 16;
  constexpr int b = kSrc / Block<D>::kBytes, x = kSrc % Block<D>::kBytes;
  static_assert(Block<D>::kKBytes % (kThreads * 16) == 0, "one instruction copies K or V, not both");
  constexpr int kDst = x < Block<D>::kKBytes ? stage_k<D, S>() + b * Block<D>::kKBytes + x
                                             : stage_v<D, S>() + b * Block<D>::kKBytes + (x - Block<D>::kKBytes);
  const uint32_t m0 = m0w + (uint32_t)kDst;
  // A memory instruction that reads an SGPR a vector instruction wrote needs 5 wait
  // states first. The compiler keeps that distance for its own loads but not for the
  // SGPR operands of inline asm, and it may set src_w just before with v_readfirstlane
  // or reload it from a spill with v_readlane; s_nop 4 keeps the distance whatever it
  // emits.
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(cl.off[I]), "s"(src_w), "{m0}"(m0) : "memory");
}

// LDS destination of copy instruction I of a block into stage S, relative to the
// wave's slice in stage 0 (see dma_one).
template <int D, int S, int I>
constexpr int dma_dst() {
  constexpr int kSrc = I * kThreads * 16;
  constexpr int b = kSrc / Block<D>::kBytes, x = kSrc % Block<D>::kBytes;
  return x < Block<D>::kKBytes ? stage_k<D, S>() + b * Block<D>::kKBytes + x
                               : stage_v<D, S>() + b * Block<D>::kKBytes + (x - Block<D>::kKBytes);
}

// The whole phase: Phase<D>::kChunksPerThread instructions per wave, as one asm
// statement: one s_nop 4 covers the base's last vector write for all of them (nothing
// can come between), and each m0 write is followed by one wait state before the LDS
// copy that uses it.
template <int D, int S>
__device__ __forceinline__ void dma_block(const uint8_t* src_w, const CopyLanes<D>& cl, uint32_t m0w) {
  constexpr int NI = Phase<D>::kChunksPerThread;
  static_assert(NI == 2 || NI == 4, "two or four copy instructions per block");
  if constexpr (NI == 4) {
    asm volatile(
        "s_nop 4\n\t"
        "s_add_u32 m0, %[m], %[d0]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o0], %[src]\n\t"
        "s_add_u32 m0, %[m], %[d1]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o1], %[src]\n\t"
        "s_add_u32 m0, %[m], %[d2]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o2], %[src]\n\t"
        "s_add_u32 m0, %[m], %[d3]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o3], %[src]"
        :
        : [o0] "v"(cl.off[0]), [o1] "v"(cl.off[1]), [o2] "v"(cl.off[2]), [o3] "v"(cl.off[3]), [src] "s"(src_w),
          [m] "s"(m0w), [d0] "n"(dma_dst<D, S, 0>()), [d1] "n"(dma_dst<D, S, 1>()), [d2] "n"(dma_dst<D, S, 2>()),
          [d3] "n"(dma_dst<D, S, 3>())
        : "memory", "m0", "scc");
  } else {
    asm volatile(
        "s_nop 4\n\t"
        "s_add_u32 m0, %[m], %[d0]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o0], %[src]\n\t"
        "s_add_u32 m0, %[m], %[d1]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[o1], %[src]"
        :
        : [o0] "v"(cl.off[0]), [o1] "v"(cl.off[1]), [src] "s"(src_w), [m] "s"(m0w), [d0] "n"(dma_dst<D, S, 0>()),
          [d1] "n"(dma_dst<D, S, 1>())
        : "memory", "m0", "scc");
  }
}

// Per-lane LDS addresses of the compute role's operand reads (stage 0, block row 0):
// the K read of k-slice kk and the Vᵀ read of Pᵀ slice pp. Stage and block offsets go
// in the instruction's offset field.
template <int D>
struct LaneAddr {
  uint32_t k[D / 16];
  uint32_t v[4];
};

// The matrix-core phase of the compute role for block m in stage S: Oᵀ += Vᵀ Pᵀ for
// block m-1 (stage S-1, when PV) then Sᵀ = K Qᵀ for block m (when QK), as one fixed
// sequence of MFMAs, each fed by a ds_read_b128 issued LA MFMAs ahead, with one block
// copy threaded through it (COPY).
template <int D, int S, bool PV, bool QK, bool COPY = true>
struct MPhase {
  static constexpr int KK = D / 16, DB = D / 32;
  static constexpr int NP = Phase<D>::kKeys / 16;  // Pᵀ slices (16 keys) of a phase
  static constexpr int NS = Phase<D>::kKeys / 32;  // Sᵀ tiles (32 keys) of a phase
  static constexpr int NPV = PV ? DB * NP : 0;
  static constexpr int NQK = QK ? NS * KK : 0;
  static constexpr int N = NPV + NQK;
  static constexpr int LA = MKRA_LDS_AHEAD;  // LDS reads in flight ahead of the MFMA using the oldest
  static constexpr int R = LA + 2;  // operand registers: a read refills the one used two MFMAs ago
  static constexpr int SPV = (S + kStages - 1) % kStages;

  // PV product J: rows 32 pv_db(J) .. of Oᵀ against Pᵀ slice pv_pp(J), which is slice
  // pv_pp(J) % 4 of the phase's block pv_pp(J) / 4. QK product J: Sᵀ tile qk_kb(J)
  // (32 rows of the stage's K matrix) against k-slice qk_kk(J).
  // Order of the products: consecutive MFMAs share their B operand (a Pᵀ slice for
  // the DB row blocks of Oᵀ, a Q k-slice for the NS tiles of Sᵀ), so the matrix
  // cores' B inputs toggle less, which the power limit turns into clock (0.5% on the
  // 64K-token workload). Each accumulator still sums its products in the same order.
  static constexpr int pv_db(int J) { return J % DB; }
  static constexpr int pv_pp(int J) { return J / DB; }
  static constexpr int qk_kb(int J) { return (J - NPV) % NS; }
  static constexpr int qk_kk(int J) { return (J - NPV) / NS; }
  template <int J>
  static constexpr int offset() {
    if constexpr (J < NPV)
      return stage_v<D, SPV>() - stage_v<D, 0>() + (pv_pp(J) / 4) * Block<D>::kKBytes + pv_db(J) * 32 * 128;
    else return stage_k<D, S>() + qk_kb(J) * 32 * (D * 2);
  }
  template <int J>
  static __device__ __forceinline__ void read(u32x4 (&buf)[R], const LaneAddr<D>& la) {
    if constexpr (J < N) {
      if constexpr (J < NPV) buf[J % R] = lds_read16<offset<J>()>(la.v[pv_pp(J) % 4]);
      else buf[J % R] = lds_read16<offset<J>()>(la.k[qk_kk(J)]);
    }
  }
  // The copy into stage S+2 is spread over the sequence: instruction I after MFMA
  // (2I+1) N / (2 NI), so no wave issues several copies at once and waits for the
  // memory pipeline to take them. It is unconditional (a branch here would put vector
  // ALU work for its condition into the stream).
  static constexpr int NI = Phase<D>::kChunksPerThread;
  template <int J>
  static constexpr int dma_at() {
    for (int i = 0; i < NI; ++i)
      if (J == (2 * i + 1) * N / (2 * NI)) return i;
    return -1;
  }
  template <int J>
  static __device__ __forceinline__ void exec(u32x4 (&buf)[R], const LaneAddr<D>& la, f32x16 (&o)[DB],
                                              const f16x8 (&pb)[NP], f32x16 (&s)[NS], const bf16x8 (&qr)[KK],
                                              const uint8_t* dma_src, const CopyLanes<D>& cl, uint32_t m0w) {
    constexpr int newer = (N - 1 - J) < (LA - 1) ? (N - 1 - J) : (LA - 1);
    lgkm_wait<newer>(buf[J % R]);
    if constexpr (J < NPV) {
      constexpr int db = pv_db(J), pp = pv_pp(J);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, buf[J % R]), pb[pp], o[db], 0, 0, 0);
    } else {
      constexpr int kb = qk_kb(J), kk = qk_kk(J);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, buf[J % R]), qr[kk],
                                                      kk == 0 ? f32x16{} : s[kb], 0, 0, 0);
    }
    read<J + LA>(buf, la);
    if constexpr (COPY && dma_at<J>() >= 0) dma_one<D, (S + 2) % kStages, dma_at<J>()>(dma_src, cl, m0w);
    __builtin_amdgcn_sched_barrier(0);
  }
  template <int... J, int... P>
  static __device__ __forceinline__ void seq(std::integer_sequence<int, J...>, std::integer_sequence<int, P...>,
                                             const LaneAddr<D>& la, f32x16 (&o)[DB], const f16x8 (&pb)[NP],
                                             f32x16 (&s)[NS], const bf16x8 (&qr)[KK], const uint8_t* dma_src,
                                             const CopyLanes<D>& cl, uint32_t m0w) {
    u32x4 buf[R];
    __builtin_amdgcn_sched_barrier(0);
    (read<P>(buf, la), ...);
    (exec<J>(buf, la, o, pb, s, qr, dma_src, cl, m0w), ...);
  }
  static __device__ __forceinline__ void run(const LaneAddr<D>& la, f32x16 (&o)[DB], const f16x8 (&pb)[NP],
                                             f32x16 (&s)[NS], const bf16x8 (&qr)[KK], const uint8_t* dma_src,
                                             const CopyLanes<D>& cl, uint32_t m0w) {
    seq(std::make_integer_sequence<int, N>{}, std::make_integer_sequence<int, (LA < N ? LA : N)>{}, la, o, pb, s, qr,
        dma_src, cl, m0w);
  }
  // The phase's first LA operand reads, issued ahead of it by the same wave at the end
  // of its softmax phase. They read the Vᵀ of the previous block, which has been
  // complete and visible since the barrier before the previous matrix phase, so the
  // MFMAs can start right after this phase's barrier instead of one LDS latency
  // later.
  template <int... P>
  static __device__ __forceinline__ void pre(std::integer_sequence<int, P...>, u32x4 (&buf)[R],
                                             const LaneAddr<D>& la) {
    (read<P>(buf, la), ...);
  }
  static __device__ __forceinline__ void prefetch(u32x4 (&buf)[R], const LaneAddr<D>& la) {
    static_assert(PV && LA <= NPV, "the reads issued ahead are PV operands");
    pre(std::make_integer_sequence<int, LA>{}, buf, la);
  }
  template <int... J>
  static __device__ __forceinline__ void seq_pre(std::integer_sequence<int, J...>, u32x4 (&buf)[R],
                                                 const LaneAddr<D>& la, f32x16 (&o)[DB], const f16x8 (&pb)[NP],
                                                 f32x16 (&s)[NS], const bf16x8 (&qr)[KK], const uint8_t* dma_src,
                                                 const CopyLanes<D>& cl, uint32_t m0w) {
    __builtin_amdgcn_sched_barrier(0);
    (exec<J>(buf, la, o, pb, s, qr, dma_src, cl, m0w), ...);
  }
  // The phase after prefetch(buf) was issued for it.
  static __device__ __forceinline__ void run_pre(u32x4 (&buf)[R], const LaneAddr<D>& la, f32x16 (&o)[DB],
                                                 const f16x8 (&pb)[NP], f32x16 (&s)[NS], const bf16x8 (&qr)[KK],
                                                 const uint8_t* dma_src, const CopyLanes<D>& cl, uint32_t m0w) {
    seq_pre(std::make_integer_sequence<int, N>{}, buf, la, o, pb, s, qr, dma_src, cl, m0w);
  }
};

// This wave's slice of the staged blocks of step t for the KV head at head_off (slot of
// step t: t mod kSlots), in scalar registers.
template <int D>
__device__ __forceinline__ const uint8_t* task_slot_ptr(const KernelArgs& a, int t, int64_t head_off) {
  return wave_bcast_ptr(a.slots + (int64_t)((uint32_t)t % (uint32_t)kSlots) * a.slot_bytes + head_off);
}

// The ready flag of piece pc of tile 0 of step t; tile j's is n_pieces * j further.
__device__ __forceinline__ const uint64_t* step_flags(const KernelArgs& a, int t, int pc) {
  return a.slot_flags + ((uint32_t)t % (uint32_t)kSlots) * a.stage_per_step + pc;
}

// Tile gi of a task's tile sequence (the tiles of its steps in order: nt0 of the first
// step starting at t_first, ntf of each later one; at most four steps): the flag of its
// piece pc and the stamp that flag holds once the piece is staged.
__device__ __forceinline__ void task_tile_flag(const KernelArgs& a, int t_first, int nt0, int ntf, int gi, int pc,
                                               const uint64_t*& f, uint64_t& want) {
  static_assert(kMaxGroup <= 4, "three boundaries tell four steps apart");
  const int st = (int)(gi >= nt0) + (int)(gi >= nt0 + ntf) + (int)(gi >= nt0 + 2 * ntf);
  const int t = t_first + st;
  f = step_flags(a, t, pc) + (gi - (st == 0 ? 0 : nt0 + (st - 1) * ntf)) * a.n_pieces;
  want = stamp(a.epoch, t);
}

// Finalise a wave's rows: out = O / l, lse = ln(2) * (m + log2 l), with l summed over
// the two lanes that hold a row's halves.
template <int D>
__device__ __forceinline__ void finalize_rows(const KernelArgs& a, const f32x16 (&o)[D / 32], float m_run,
                                              float l_run, int qrow, int h, int hi) {
  constexpr int DB = D / 32;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < a.lq) {
    const float inv = 1.f / l_tot;
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
}

__shared__ uint32_t g_merge;  // parallel step groups: this workgroup's task merges its unit

// claim_next() picks the workgroup's next task (wave 1); it runs alongside the publish.
template <int D, class ClaimNext>
__device__ __forceinline__ void compute_task(const KernelArgs& a, int unit, int step_group, int grp, uint64_t& waited,
                             ClaimNext&& claim_next) {
  // Where the block copies are issued: at D = 128 from the softmax phase (the matrix
  // phase, 32 MFMAs, is the longer one there, and each copy instruction holds up the
  // wave's issue), at D = 64 from the matrix phase (16 MFMAs; the softmax is longer).
  constexpr bool kCopyInSoftmax = D == 128;
  constexpr int KK = D / 16;                    // k-slices of Q K^T
  constexpr int DB = D / 32;                    // 32-row blocks of O^T
  constexpr int NI = Phase<D>::kChunksPerThread;  // copy instructions per wave per phase
  constexpr int PK = Phase<D>::kKeys;             // keys per phase
  constexpr int NS = PK / 32, NP = PK / 16;       // Sᵀ tiles and Pᵀ slices per phase

  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5, col = lane & 31;
  const int w = (int)wave_bcast((uint32_t)(tid >> 6));  // wave-uniform, kept in SGPRs
  // The task comes through LDS; telling the compiler it is uniform keeps every
  // address derived from it (slot, head, block) in SGPRs.
  unit = (int)wave_bcast((uint32_t)unit);
  step_group = (int)wave_bcast((uint32_t)step_group);
  // The task's ring steps: [t_first, t_end), with the running state in registers
  // from one step to the next.
  const int t_first = group_first(a, step_group), t_end = group_end(a, step_group);
  const int p = unit / a.n_qblocks, qb = unit % a.n_qblocks;
  const int kvh = p / a.n_hgroups, hgi = p % a.n_hgroups;
  const int pc = kvh / a.piece_heads;  // the staging piece that holds this KV head
  const int h = kvh * a.gqa + hgi * a.hg + (w % a.hg);
  const int q0w = qb * a.bq + (w / a.hg) * kRowsPerWave;
  const bool wave_rows = q0w < a.lq;
  const int qrow = q0w + col;
  const int q_end = min(a.lq, qb * a.bq + a.bq);
  const float c2 = a.scale_log2;
  bool ok = true;

  // Q first: it is read-only input, so its loads need no flag and overlap the flag
  // round trip below. Lane holds Q[qrow][h][kk*16 + 8*hi .. +7] for every k-slice.
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

  // Running state: Oᵀ blocks, max (log2 units of the scaled score) and the running sum
  // of P.
  f32x16 o[DB];
  float m_run, l_run;
  // State slot: the unit's (carried from group to group), or with parallel step groups
  // this group's own partial.
  const int64_t slot_of_state = a.parallel_steps ? (int64_t)unit * a.n_groups + step_group : (int64_t)unit;
  float* accw = a.acc + (slot_of_state * kWaves + w) * (32 * D + 256);
  // Per-lane LDS addresses (the swizzles depend only on the lane).
  LaneAddr<D> la;
  {
    const uint32_t b0 = lds_base();
    const int kx = (D == 128) ? (col & 15) : ((col >> 1) & 7);
    const int vx = (col >> 1) & 7;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) la.k[kk] = b0 + col * (D * 2) + 16 * ((2 * kk + hi) ^ kx);
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) la.v[pp] = b0 + stage_v<D, 0>() + col * 128 + 16 * ((2 * pp + hi) ^ vx);
  }

  // Copy addressing: this wave's 1 KB slice of every copy instruction (base in SGPRs,
  // per-lane offsets in VGPRs that the compiler may not recompute inside the matrix
  // phase). The discard block follows the ring slots.
  const uint8_t* const discard_w = wave_bcast_ptr(a.slots + kSlots * a.slot_bytes + w * 64 * 16);
  static_assert(Phase<D>::kBytes <= kDiscardBytes, "discard block");
  CopyLanes<D> cl;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    cl.off[i] = (uint32_t)(i * kThreads * 16 + lane * 16);
    asm volatile("" : "+v"(cl.off[i]));
  }
  const uint32_t m0w_task = lds_base() + (uint32_t)w * 64u * 16u;
  // Sᵀ of the current phase (registers) and Pᵀ of the phase before it (fp16).
  f32x16 s[NS];
  f16x8 pb[NP];

  // The task's KV phases (PK keys each) form one sequence: the n0 phases of step
  // t_first, then nfull phases of each later step of the task (up to kMaxGroup steps).
  // The online softmax does not depend on where one step ends, so one pipeline runs
  // through every step of the task without draining in between. A block is located by
  // its step s within the task (scalar compares against the step boundaries) and its
  // index within that step; tiles likewise count through the task's steps in order
  // (the task's tile sequence), and `ru` is the frontier below which every tile of that
  // sequence is known ready.
  auto kend_of = [&](int t) __attribute__((always_inline)) { return (a.causal && t == 0) ? min(a.lk, q_end) : a.lk; };
  auto n_tiles_of = [&](int t) __attribute__((always_inline)) { return (kend_of(t) + kStageRows - 1) / kStageRows; };
  const int nst = t_end - t_first;                   // steps of the task
  const int nfull = (a.lk + PK - 1) / PK;            // phases of a step after the first
  const int n0 = (kend_of(t_first) + PK - 1) / PK;   // phases of the first step
  const int nb = n0 + (nst - 1) * nfull;
  const int nt0 = n_tiles_of(t_first), ntf = a.n_tiles;
  const int n_task_tiles = nt0 + (nst - 1) * ntf;
  const int64_t head_off = (int64_t)kvh * a.n_blocks * Block<D>::kBytes + w * 64 * 16;
  // This wave's slice of the staged blocks of step st of the task, the ready flags of
  // step t, and tile gi of the task's tile sequence (per lane) with the stamp it must
  // hold: plain functions, not lambdas, so no closure is nested three deep (closures
  // nested that deep kept the compiler from promoting the captured state out of
  // scratch memory).
  auto slot_ptr = [&](int st) __attribute__((always_inline)) { return task_slot_ptr<D>(a, t_first + st, head_off); };

  // Flags, in two loads per lane issued together (one round trip): lanes below 63 read
  // the ready flags of tiles 0..62 of the task's tile sequence and lane 63 the unit's
  // step t_first-1 stamp (that state must be complete); every lane reads the flag of
  // tile 63 + lane. Tiles below the frontier ru are then known ready; later ones are
  // checked when their copy is issued. One acquire covers everything observed.
  int ru;
  {
    bool r0 = true, r1 = true;
    const uint64_t* f;
    uint64_t want;
    if (lane < 63 && lane < n_task_tiles) {
      task_tile_flag(a, t_first, nt0, ntf, lane, pc, f, want);
      r0 = ld64(f) == want;
    } else if (lane == 63 && t_first > 0 && !a.parallel_steps) {
      r0 = ld64(&a.unit_flags[unit]) == stamp(a.epoch, t_first - 1);
    }
    if (63 + lane < n_task_tiles) {
      task_tile_flag(a, t_first, nt0, ntf, 63 + lane, pc, f, want);
      r1 = ld64(f) == want;
    }
    const uint64_t nr0 = __ballot(!r0), nr1 = __ballot(!r1);
    const uint64_t tiles_nr0 = nr0 & ~(1ull << 63);
    ru = (int)wave_bcast(tiles_nr0 ? (uint32_t)__builtin_ctzll(tiles_nr0)
                                   : nr1 ? 63u + (uint32_t)__builtin_ctzll(nr1)
                                         : (uint32_t)min(n_task_tiles, 127));
    if ((nr0 >> 63) & 1) {
      // The unit's previous step is still running: wait for it (acquires on return).
      ok &= wave_wait_stamp(a, &a.unit_flags[unit], stamp(a.epoch, t_first - 1), waited);
    } else {
      fence_acquire();
    }
  }

  if (t_first == 0 || a.parallel_steps) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
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
  }

  // Cursors through the task's block sequence, one for the block the next copy takes
  // and one for the block the next softmax takes. Each is advanced once per phase by
  // scalar integer arithmetic: masks come from arithmetic shifts rather than compares,
  // so no branch and no vector-mask conversion enters the phases. A cursor holds the
  // block's index within its step (b), the block count of that step (nbs) and the
  // step (st); the copy cursor also holds the sequence index (k), the tile in the
  // task's tile sequence and this wave's slice of the block (p).
  constexpr int kBlocksPerTile = kStageRows / PK;
  static_assert((kBlocksPerTile & (kBlocksPerTile - 1)) == 0, "blocks per staged tile");
  int ck = 0, cb = 0, cnbs = n0, cst = 0, ctile = 0;
  const uint8_t* cptr = slot_ptr(0);
  auto cur_advance = [&]() __attribute__((always_inline)) {
    const int nb1 = cb + 1;
    const int cross = (cnbs - nb1 - 1) >> 31;  // -1 when the step ends here, else 0
    ck += 1;
    cb = nb1 & ~cross;
    cnbs ^= (cnbs ^ nfull) & cross;
    cst -= cross;
    ctile += (((cb & (kBlocksPerTile - 1)) - 1) >> 31) & 1;  // a tile starts at its first block
    cptr = cross ? slot_ptr(cst) : cptr + Phase<D>::kBytes;
  };
  int sb = 0, snbs = n0, sst = 0;
  auto sm_advance = [&]() __attribute__((always_inline)) {
    const int nb1 = sb + 1;
    const int cross = (snbs - nb1 - 1) >> 31;
    sb = nb1 & ~cross;
    snbs ^= (snbs ^ nfull) & cross;
    sst -= cross;
  };
  // Copy of the cursor's block into LDS stage S, after making sure its tile is ready.
  auto issue_cur = [&](auto stage_tag) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    if (ctile >= ru) {
      // Wait for this tile's flag (of the piece holding this unit's KV head), then look
      // at the later flags of the task's tile sequence 64 at a time (one load per lane)
      // so the next tiles need no check.
      const int t = t_first + cst;
      ok &= wave_wait_stamp(a, step_flags(a, t, pc) + (cb / kBlocksPerTile) * a.n_pieces, stamp(a.epoch, t), waited);
      int upto = ctile + 1;
      for (int g0 = ctile + 1; g0 < n_task_tiles; g0 += 64) {
        bool ready = false;
        if (g0 + lane < n_task_tiles) {
          const uint64_t* f;
          uint64_t want;
          task_tile_flag(a, t_first, nt0, ntf, g0 + lane, pc, f, want);
          ready = ld64(f) == want;
        }
        const uint64_t notready = __ballot(!ready && g0 + lane < n_task_tiles);
        if (notready) {
          upto = g0 + (int)__builtin_ctzll(notready);
          break;
        }
        upto = min(n_task_tiles, g0 + 64);
      }
      if (upto > ctile + 1) fence_acquire();
      ru = (int)wave_bcast((uint32_t)upto);
    }
    dma_block<D, S>(cptr, cl, m0w_task);
  };

  // Online-softmax update for the softmax cursor's block (FlashAttention-2), producing
  // fp16 Pᵀ.
  auto softmax = [&]() __attribute__((always_inline)) {
    // Masks: ragged key tail, and keys after the query on the diagonal step.
    const bool diag = a.causal && t_first == 0 && sst == 0;
    const int k0 = sb * PK;
    if (k0 + PK > a.lk || (diag && k0 + PK - 1 > q0w)) {
      // Element i of s[kb] holds key k0 + kb*32 + (i/4)*8 + hi*4 + i%4; it is visible iff
      // that key is below lim + k0 + hi*4 (lim is per lane, the offsets constants).
      const int lim = (diag ? min(a.lk, qrow + 1) : a.lk) - k0 - hi * 4;
      // s = min(s, bias) with bias = +inf for a visible key and -inf otherwise, the
      // sign of (offset - lim) picking the sign of the infinity: a compare per element
      // would write a scalar register pair, and with 64 of them in flight the scalar
      // registers of the whole loop spill.
#pragma unroll
      for (int kb = 0; kb < NS; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t neg = (uint32_t)(kb * 32 + (i >> 2) * 8 + (i & 3) - lim) & 0x80000000u;  // set iff visible
          float bias = __builtin_bit_cast(float, 0xff800000u ^ neg);
          asm volatile("" : "+v"(bias));
          s[kb][i] = fminf(s[kb][i], bias);
        }
    }
    // P = exp2(s c2 - m_run) against the running max as it stands, rounded to fp16 for
    // the PV product; l sums the same rounded P, by packed fp16 adds in a tree (15
    // instructions for 32 values, against 31 fp32 adds; the vector ALU is shared with
    // the other wave's softmax), the last level in fp32. The tree's rounding moves a
    // block's sum by about 2^-11 relative per level, independently from block to
    // block. A sum past the fp16 range becomes inf and takes the rescale path below,
    // as any sum above kSumMax does. (A v_dot2c sum would not co-issue with the other
    // wave's MFMAs.)
    float lsum;
    auto exp_block = [&](float mref) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < NS; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pb[kb * 2 + (i >> 3)][i & 7] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -mref));
      static_assert(NP == 4 || NP == 8, "four or eight fp16x8 P vectors");
      f16x8 t8 = (pb[0] + pb[1]) + (pb[2] + pb[3]);
      if constexpr (NP == 8) t8 += (pb[4] + pb[5]) + (pb[6] + pb[7]);
      const f16x4 t4 = __builtin_shufflevector(t8, t8, 0, 1, 2, 3) + __builtin_shufflevector(t8, t8, 4, 5, 6, 7);
      const f16x2 t2 = __builtin_shufflevector(t4, t4, 0, 1) + __builtin_shufflevector(t4, t4, 2, 3);
      lsum = (float)t2[0] + (float)t2[1];
    };
    exp_block(m_run);
    // Only when some P of the block exceeds kSumMax (a lane's partial sum bounds each
    // of its P), or on the first block, is the row max of the block needed: raise
    // m_run to it, rescale O and l, and redo the block. The max the exponentials use
    // may therefore lag the true max, by at most log2(kSumMax); every P stays in the
    // fp16 range and the algebra of the online softmax is unchanged.
    if (__any(!(lsum <= kSumMax))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NS; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = max3(mx, s[kb][i], s[kb][i + 1]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * c2);
      const float alpha = (m_new == m_run || m_run == -INFINITY) ? (m_run == -INFINITY ? 0.f : 1.f)
                                                                 : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      exp_block(m_run == -INFINITY ? 0.f : m_run);
    }
    l_run += lsum;
  };

  // Two-phase schedule. Each wave runs M(0) V(0) M(1) V(1) ... M(nb), where
  // M(m) = PV of block m-1 and QKᵀ of block m (matrix cores) and V(m) = the softmax
  // of block m (vector ALU), one s_barrier before each phase. Waves of group 1 take
  // one extra barrier first and group 0 one at the end, so the two waves sharing a
  // SIMD run opposite phases and keep both the matrix cores and the vector ALU busy.
  // Block m sits in LDS stage m % 4: it is copied during M(m-2) (at D = 128 during
  // V(m-2)), read by QKᵀ in M(m) and by PV in M(m+1), and its stage is refilled in
  // M(m+2) (V(m+2)), after a barrier that both groups pass only once they are done
  // with it. Before every barrier a wave waits for its own copies of the next block it
  // or the other group reads; the barrier then makes every wave's part visible.
  // Every wave runs every block of the unit: on the diagonal step the blocks past a
  // wave's last query are fully masked and add exactly zero. The sequence runs
  // straight from the first step's last block into the second step's first.
  //
  // The compiler may move register-only arithmetic across s_barrier (it orders only
  // memory), which would pull softmax work into the matrix phase or the reverse and
  // undo the ping-pong. Empty volatile asm statements, which keep their order with
  // the barriers, pin each phase's inputs after its barrier and its outputs before
  // the next one.
  auto pin_scores = [&]() __attribute__((always_inline)) {
    if constexpr (NS == 2) asm volatile("" : "+v"(s[0]), "+v"(s[1]));
    else asm volatile("" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]));
  };
  auto pin_acc = [&]() __attribute__((always_inline)) {
    if constexpr (DB == 4) asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
    else asm volatile("" : "+v"(o[0]), "+v"(o[1]));
  };
  auto pin_state = [&]() __attribute__((always_inline)) {
    asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(pb[2]), "+v"(pb[3]), "+v"(m_run), "+v"(l_run));
    if constexpr (NP == 8) asm volatile("" : "+v"(pb[4]), "+v"(pb[5]), "+v"(pb[6]), "+v"(pb[7]));
    pin_acc();
  };
  // Copies: blocks 0 and 1 before the loop, then one block copy per block, into stage
  // (m+2)%4, which holds block m-2 and is dead by then.
  // - D = 64: threaded through every M(m). The copy is block m+2 when it exists and
  //   its staged tile is known to be ready; else it copies the discard block (one
  //   block after the ring slots, always cache-hot, never read), and block m+2, if it
  //   exists, is copied again after the MFMAs once its flag is seen (same wave, same
  //   LDS addresses, completes later).
  // - D = 128: at the start of every V(m), after its barrier: block m+2 (waiting for
  //   its flag there if its tile is not known ready), or past the end the discard
  //   block.
  // Either way every wait below has at least one block copy issued after the one it
  // needs, so waiting until at most NI copy instructions are outstanding is enough
  // before a matrix phase (it may also cover a discarded copy). At D = 128 the wait
  // before a softmax phase drains every copy: the groups run one phase apart, so the
  // copy a wave issued at the start of its previous softmax phase is read by the other
  // group's next matrix phase.
  auto wait_block = [&]() __attribute__((always_inline)) { wait_vm(NI); };
  // M(m): the barrier, the MFMAs, and (D = 64) the copy into stage (S+2)%4. Returns
  // whether the cursor's block still has to be copied (its tile was not known ready),
  // which the caller then does with issue_cur before advancing the cursor: kept out of this
  // lambda, because with it inside, the closures nested here kept the compiler from
  // promoting the captured state out of scratch memory.
  auto mstep = [&](int m, auto stage_tag, auto mfmas) __attribute__((always_inline)) {
    constexpr int S = decltype(stage_tag)::value;
    if (m < nb) wait_block();
    __builtin_amdgcn_s_barrier();
    // The copy cursor is at block m + 2.
    const bool exists = ck < nb;
    const bool ready = exists && ctile < ru;  // from scalars only: stays in SALU
    // Base of this wave's LDS slice, opaque per phase so the compiler adds the stage
    // and instruction offsets here (scalar adds) instead of keeping sixteen of them
    // in SGPRs across the loop.
    uint32_t m0w = wave_bcast(m0w_task);
    asm volatile("" : "+s"(m0w));
    // The wave in its matrix phase issues first: when both waves of the SIMD are ready,
    // its next MFMA or operand read goes ahead of the other wave's softmax instruction
    // (same-box A/B: 0.3 % faster on the 64K-token workload, 1.2 % on the 32K-token
    // D = 64 one; raising it to 3 instead of 1 gained less).
    __builtin_amdgcn_s_setprio(1);
    mfmas(wave_bcast_ptr(ready ? cptr : discard_w), m0w);
    pin_scores();
    pin_acc();
    __builtin_amdgcn_s_setprio(0);
    return exists && !ready;
  };
  // Operand registers of the next matrix phase's first LDS reads, issued at the end of
  // each softmax phase (MPhase::prefetch).
  u32x4 pre[MPhase<D, 0, true, true>::R];
  // V(m) (at D = 128 preceded by the copy of block m+2 into stage SN+1), then the
  // first operand reads of M(m+1), whose stage is SN.
  auto vstep = [&](int m, auto next_stage_tag) __attribute__((always_inline)) {
    constexpr int SN = decltype(next_stage_tag)::value;
    if (m + 1 < nb) {
      if constexpr (kCopyInSoftmax) wait_vm(0);
      else wait_block();
    }
    __builtin_amdgcn_s_barrier();
    if constexpr (kCopyInSoftmax) {
      if (ck < nb) issue_cur(std::integral_constant<int, (SN + 1) % kStages>{});
      else dma_block<D, (SN + 1) % kStages>(discard_w, cl, m0w_task);
      cur_advance();
    }
    pin_scores();
    softmax();
    sm_advance();
    pin_state();
    MPhase<D, SN, true, true>::prefetch(pre, la);
  };
#define MKRA_PVQK(S) \
  [&](const uint8_t* src, uint32_t m0w) __attribute__((always_inline)) {        \
    MPhase<D, S, true, true, !kCopyInSoftmax>::run_pre(pre, la, o, pb, s, qr, src, cl, m0w); \
  }
#define MKRA_PV(S) \
  [&](const uint8_t* src, uint32_t m0w) __attribute__((always_inline)) { \
    MPhase<D, S, true, false, false>::run_pre(pre, la, o, pb, s, qr, src, cl, m0w); \
  }
  // nb >= 1: every unit has keys (Lk >= 1, and the diagonal step covers at least the
  // unit's first query).
  issue_cur(std::integral_constant<int, 0>{});
  cur_advance();
  if (1 < nb) issue_cur(std::integral_constant<int, 1>{});
  else dma_block<D, 1>(discard_w, cl, m0w_task);  // discarded (see the copy rule above)
  cur_advance();
  if (grp) {
    wait_block();
    __builtin_amdgcn_s_barrier();
  }
  // M(m) in stage S, then the copy of the cursor's block if its tile was not known
  // ready, into the stage M(m) left for it, and the cursor's advance.
#define MKRA_M(m, S, MFMAS)                                                         \
  do {                                                                              \
    if (mstep(m, std::integral_constant<int, S>{}, MFMAS) && !kCopyInSoftmax)       \
      issue_cur(std::integral_constant<int, ((S) + 2) % kStages>{});                \
    if (!kCopyInSoftmax) cur_advance();                                             \
  } while (0)
  auto first_qk = [&](const uint8_t* src, uint32_t m0w) __attribute__((always_inline)) {
    MPhase<D, 0, false, true, !kCopyInSoftmax>::run(la, o, pb, s, qr, src, cl, m0w);
  };
  MKRA_M(0, 0, first_qk);
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  vstep(0, S1{});
  int m = 1;
  for (; m + 3 < nb; m += kStages) {
    MKRA_M(m, 1, MKRA_PVQK(1));
    vstep(m, S2{});
    MKRA_M(m + 1, 2, MKRA_PVQK(2));
    vstep(m + 1, S3{});
    MKRA_M(m + 2, 3, MKRA_PVQK(3));
    vstep(m + 2, S0{});
    MKRA_M(m + 3, 0, MKRA_PVQK(0));
    vstep(m + 3, S1{});
  }
  if (m < nb) {
    MKRA_M(m, 1, MKRA_PVQK(1));
    vstep(m, S2{});
    if (++m < nb) {
      MKRA_M(m, 2, MKRA_PVQK(2));
      vstep(m, S3{});
      if (++m < nb) {
        MKRA_M(m, 3, MKRA_PVQK(3));
        vstep(m, S0{});
        ++m;
      }
    }
  }
  // M(nb): PV of the last block only; no wait follows, so it copies nothing (the
  // cursor is past the sequence, so mstep asks for no copy either).
  switch (nb & 3) {
    case 0: mstep(nb, S0{}, MKRA_PV(0)); break;
    case 1: mstep(nb, S1{}, MKRA_PV(1)); break;
    case 2: mstep(nb, S2{}, MKRA_PV(2)); break;
    default: mstep(nb, S3{}, MKRA_PV(3)); break;
  }
#undef MKRA_M
#undef MKRA_PVQK
#undef MKRA_PV
  if (!grp) __builtin_amdgcn_s_barrier();
  // Discarded copies may still be in flight: drain them before this workgroup's next
  // task (or staging task) writes the same LDS.
  wait_vm(0);


  if (ok && wave_rows) {
    if (t_end == a.n_steps && !a.parallel_steps) {
      finalize_rows<D>(a, o, m_run, l_run, qrow, h, hi);
    } else {
      f32x4* a4 = reinterpret_cast<f32x4*>(accw);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          a4[(db * 4 + g) * 64 + lane] =
              f32x4{o[db][g * 4 + 0], o[db][g * 4 + 1], o[db][g * 4 + 2], o[db][g * 4 + 3]};
      reinterpret_cast<f32x4*>(accw + 32 * D)[lane] = f32x4{m_run, l_run, 0.f, 0.f};
    }
  }
  // Publish: unit steps done (orders the state for the next group) and slot release for
  // each step of the task. Each wave waits for its own stores and counts itself in
  // (workgroup-scope release); thread 0 waits for all eight, then one agent-scope
  // release fence covers every wave's stores and the signals after it. Meanwhile
  // wave 1 claims the next task: its few dependent memory round trips overlap the
  // publish instead of delaying it, which matters when a unit's chain of steps is the
  // critical path. (A wave whose wait failed has raised the launch's error; publishing
  // after another workgroup's error is harmless, since every wait ends on it.)
  wait_vm(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane == 0) __hip_atomic_fetch_add(&g_pub_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  claim_next();
  if (tid == 0) {
    // Bounded: every wave counts itself in once its own stores are done.
    while (__hip_atomic_load(&g_pub_count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)kWaves)
      __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __hip_atomic_store(&g_pub_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (tid == 0 && ok) {
    fence_release();
    if (a.parallel_steps) {
      // Count this group in on the unit's epoch-stamped counter (a stamp of an earlier
      // launch counts as zero); the last group in merges.
      uint64_t* f = &a.unit_flags[unit];
      uint64_t v = ld64(f), before;
      while (true) {
        before = (v >> 20) == a.epoch ? (v & 0xfffffull) : 0;
        uint64_t expect = v;
        if (__hip_atomic_compare_exchange_strong(f, &expect, (a.epoch << 20) | (before + 1), __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
          break;
        v = expect;
      }
      g_merge = before + 1 == (uint64_t)a.n_groups;
    } else {
      __hip_atomic_store(&a.unit_flags[unit], stamp(a.epoch, t_end - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int t = t_first; t < t_end; ++t)
      __hip_atomic_fetch_add(&a.done_count[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (tid == 0) {
    g_merge = 0;
  }
  if (a.parallel_steps) {
    // The group that counted in last merges every group's partial in group order (the
    // result does not depend on which group finished last) and finalises.
    __syncthreads();
    if (g_merge && wave_rows) {
      fence_acquire();
      float m_tot = -INFINITY, l_tot = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = f32x16{};
      for (int g = 0; g < a.n_groups; ++g) {
        const float* pw = a.acc + (((int64_t)unit * a.n_groups + g) * kWaves + w) * (32 * D + 256);
        const f32x4 ml = reinterpret_cast<const f32x4*>(pw + 32 * D)[lane];
        const float mn = fmaxf(m_tot, ml[0]);
        // A partial with no keys (-inf max) weighs zero; so does an empty running sum.
        const float sa = m_tot == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_tot - mn);
        const float sb = ml[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[0] - mn);
        const f32x4* a4 = reinterpret_cast<const f32x4*>(pw);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const f32x4 v = a4[(db * 4 + gg) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[db][gg * 4 + e] = fmaf(o[db][gg * 4 + e], sa, v[e] * sb);
          }
        l_tot = fmaf(l_tot, sa, ml[1] * sb);
        m_tot = mn;
      }
      finalize_rows<D>(a, o, m_tot, l_tot, qrow, h, hi);
    }
  }
}

// ------------------------------------------------------------------ scheduling

// Scheduler state of a workgroup (thread 0 only), kept in LDS.
struct Sched {
  int32_t role;     // kRoleCompute / kRoleStage
  int32_t pending;  // a claimed compute task not yet run
  int32_t pend_u, pend_g;  // the pending task: unit and step group
};

// Picks the workgroup's next task and writes (op, x, y) to cmd. Run by thread 0.
//
// Every control word is loaded in one batch first, so a decision costs one memory
// round trip plus, for a compute task, one compare-and-swap (these words are shared
// by all XCDs, so each access goes to memory).
//
// Compute tasks: a task is one unit for the consecutive ring steps of a step group.
// Each XCD has a queue of the units of its head groups, group-major, so units that
// read the same KV head share an L2. A workgroup takes from its own queue only while
// that queue is at most one group ahead of the slowest queue, else from the slowest
// queue. A task of group g needs its unit's group g-1 (claimed earlier, same queue
// order; not with parallel step groups, which need nothing of the unit's other groups)
// and staging of its steps, whose slots are released once every unit is past
// step group_end(g) - 1 - kSlots, which lies in group g-2 or earlier since no group has
// more than kSlots/2 steps; every task of group g-2 is claimed
// when the rule admits group
// g, so the schedule cannot deadlock whatever subset of workgroups is resident. Within
// a group a queue runs its units from the last, so on the causal diagonal step the
// longest query blocks start first.
//
// Roles change at task boundaries (§3.2): a staging workgroup leaves the role when
// staging is done or the controller's target dropped below the count; a compute
// workgroup joins when the count is below the target. The stall rule of §3.2: while
// staging work that a claimed compute task depends on is unclaimed (tasks of steps up
// to its last whose slot is already released), the workgroup does that work first.
__device__ __forceinline__ void schedule(const KernelArgs* ap, Sched* st, int32_t* cmd) {
  const KernelArgs& a = *ap;
  // Wave 0 loads the control words lane-parallel (one instruction, one round trip);
  // lane 0 then decides.
  const int lane = threadIdx.x & 63;
  const uint32_t* src = lane < kMaxXcd ? &a.ctrl->xcd_head[lane].v
                      : lane == 8      ? &a.ctrl->error.v
                      : lane == 9      ? &a.ctrl->stage_head.v
                      : lane == 10     ? &a.ctrl->n_stage.v
                      : lane == 11     ? &a.ctrl->target.v
                      : lane == 12     ? reinterpret_cast<const uint32_t*>(&a.ctrl->ctrl_time.v)
                                       : reinterpret_cast<const uint32_t*>(&a.ctrl->ctrl_time.v) + 1;
  const uint32_t word = lane < 14 ? ld32(src) : 0u;
  uint32_t heads[kMaxXcd];
#pragma unroll
  for (int i = 0; i < kMaxXcd; ++i) heads[i] = i < a.n_xcd ? (uint32_t)__builtin_amdgcn_readlane((int)word, i) : 0u;
  const uint32_t err = (uint32_t)__builtin_amdgcn_readlane((int)word, 8);
  const uint32_t sh = (uint32_t)__builtin_amdgcn_readlane((int)word, 9);
  const uint32_t ns = (uint32_t)__builtin_amdgcn_readlane((int)word, 10);
  const uint32_t tgt = (uint32_t)__builtin_amdgcn_readlane((int)word, 11);
  // The two halves of the update time are read separately: a torn value only makes
  // the controller's compare-and-swap fail once.
  const uint64_t last = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)word, 12) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)word, 13) << 32);
  if (lane != 0) return;
  int32_t op = kOpExit, x = 0, y = 0;
  if (err != kErrNone) {
    cmd[0] = kOpExit;
    return;
  }
  maybe_controller(ap, heads, sh, last);
  const bool stage_left = (int)sh < a.n_stage_tasks;
  if (!st->pending) {
    if (st->role == kRoleStage) {
      if (!stage_left) {
        add32(&a.ctrl->n_stage.v, (uint32_t)-1);
        st->role = kRoleCompute;
      } else if (!a.split_fixed && (int)ns > target_of(a, tgt) && cas32(&a.ctrl->n_stage.v, ns, ns - 1)) {
        st->role = kRoleCompute;
        add32(&a.ctrl->role_switches.v, 1);
        trace_rec(ap, kTraceRole, 0, ns - 1, 0, 0, 0, 0);
      }
    } else if (!a.split_fixed && !a.disable_staging && stage_left) {
      if ((int)ns < target_of(a, tgt) && cas32(&a.ctrl->n_stage.v, ns, ns + 1)) {
        st->role = kRoleStage;
        max32(&a.ctrl->max_stage.v, ns + 1);
        add32(&a.ctrl->role_switches.v, 1);
        trace_rec(ap, kTraceRole, 1, ns + 1, 0, 0, 0, 0);
      }
    }
    if (st->role == kRoleStage) {
      const uint32_t kk = add32(&a.ctrl->stage_head.v, 1);
      if ((int)kk < a.n_stage_tasks) {
        op = kOpStage;
        x = (int32_t)kk;
      } else {
        add32(&a.ctrl->n_stage.v, (uint32_t)-1);
        st->role = kRoleCompute;
      }
    }
    if (op == kOpExit && st->role == kRoleCompute) {
      // Claim a compute task; a failed compare-and-swap returns the queue's head.
      const int own = (int)(blockIdx.x % (unsigned)a.n_xcd);
      bool got = false;
      for (int attempt = 0; attempt < 1 << 16 && !got; ++attempt) {
        int min_step = a.n_groups, min_x = -1, own_step = a.n_groups;
        uint32_t own_head = 0, min_head = 0;
#pragma unroll
        for (int q = 0; q < kMaxXcd; ++q) {
          if (q >= a.n_xcd) break;
          const int64_t ux = units_in_queue(a, q);
          const int sq = (ux == 0 || (int64_t)heads[q] >= ux * a.n_groups) ? a.n_groups : (int)(heads[q] / ux);
          if (q == own) { own_step = sq; own_head = heads[q]; }
          if (sq < min_step) { min_step = sq; min_x = q; min_head = heads[q]; }
        }
        if (min_x < 0) break;  // every queue exhausted
        const bool mine = own_step < a.n_groups && own_step <= min_step + 1;
        const int q = mine ? own : min_x;
        const uint32_t h = mine ? own_head : min_head;
        uint32_t expect = h;
        if (__hip_atomic_compare_exchange_strong(&a.ctrl->xcd_head[q].v, &expect, h + 1, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          const int64_t ux = units_in_queue(a, q);
          st->pend_g = (int32_t)(h / ux);
          st->pend_u = a.xcd_unit_begin[q + 1] - 1 - (int32_t)(h % ux);
          got = true;
        } else {
#pragma unroll
          for (int i = 0; i < kMaxXcd; ++i)
            if (i == q) heads[i] = expect;
          if (ld32(&a.ctrl->error.v) != kErrNone) break;
        }
      }
      if (got) {
        st->pending = 1;
      } else if (stage_left && !a.disable_staging) {
        // No compute task left to claim: help drain the remaining staging.
        const uint32_t kk = add32(&a.ctrl->stage_head.v, 1);
        if ((int)kk < a.n_stage_tasks) {
          op = kOpStage;
          x = (int32_t)kk;
        }
      }
    }
  }
  if (st->pending) {
    // A failed compare-and-swap returns the staging head; retry while the task it
    // names is still one the stall rule allows.
    uint32_t h = sh;
    bool assist = false;
    int released_below = 0;  // steps whose slot is known released
    // The last staging position the task needs: its last step's, or with an
    // interleaved order (no slot is reused, so no staging task waits) the largest
    // position of its steps; every task up to it may be assisted.
    int need_pos = group_end(a, st->pend_g) - 1;
    if (a.stage_interleave) {
      need_pos = 0;
      for (int t = group_first(a, st->pend_g); t < group_end(a, st->pend_g); ++t)
        need_pos = max(need_pos, (int)a.stage_pos[t & (kSlots - 1)]);
    }
    for (int attempt = 0; attempt < 64 && !a.disable_staging && (int)h < a.n_stage_tasks; ++attempt) {
      const int pos = (a.stage_lo + (int)h) / a.stage_per_step;
      if (pos > need_pos) break;
      const int step = stage_step_of(a, pos);
      if (step >= kSlots && step >= released_below) {
        if (ld32(&a.done_count[step - kSlots]) < (uint32_t)a.n_units) break;
        released_below = step + 1;
      }
      uint32_t expect = h;
      if (__hip_atomic_compare_exchange_strong(&a.ctrl->stage_head.v, &expect, h + 1, __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        assist = true;
        break;
      }
      h = expect;
    }
    if (assist) {
      op = kOpStage;
      x = (int32_t)h;
      y = 1;
    } else {
      op = kOpCompute;
      x = st->pend_u;
      y = st->pend_g;
      st->pending = 0;
    }
  }
  cmd[0] = op;
  cmd[1] = x;
  cmd[2] = y;
}

template <int D>
__global__ __launch_bounds__(kThreads) void ring_attn_kernel(KernelArgs a) {
  // The one evaluation of kernel_args(): in the kernel's own body, where it is valid.
  const KernelArgs* const ap = kernel_args();
  const int tid = threadIdx.x;
  const uint64_t t_start = ticks();
  const uint64_t c_start = __builtin_readcyclecounter();  // s_memtime: shader clock
  uint32_t role = ((int)blockIdx.x < a.initial_stagers) ? kRoleStage : kRoleCompute;
  if (tid == 0) {
    max64(&a.ctrl->t_first.v, ~t_start);  // stores the complement: max of ~t = min t
    if (role == kRoleStage) {
      uint32_t n = add32(&a.ctrl->n_stage.v, 1) + 1;
      max32(&a.ctrl->max_stage.v, n);
    }
  }
  // Phase group of this wave (see compute_task): the second wave to land on a SIMD
  // runs the opposite phase of the first. HW_ID bits 5:4 hold the SIMD of the wave.
  __shared__ int32_t simd_of_wave[kWaves];
  int grp;
  {
    const int w = tid >> 6;
    if ((tid & 63) == 0) simd_of_wave[w] = (int32_t)__builtin_amdgcn_s_getreg(4 | (4 << 6) | (1 << 11));
    __syncthreads();
    int before = 0;
    for (int v = 0; v < w; ++v) before += simd_of_wave[v] == simd_of_wave[w];
    grp = before & 1;
  }
  __shared__ Sched sched;
  if (tid == 0) {
    sched.role = (int32_t)role;
    sched.pending = 0;
    g_pub_count = 0;
  }

  bool claimed = false;  // the compute task that just ended already claimed the next one
  while (true) {
    __syncthreads();
    if (!claimed && tid < 64) schedule(ap, &sched, g_cmd);
    claimed = false;
    __syncthreads();
    const int op = g_cmd[0], x = g_cmd[1], y = g_cmd[2];
    if (op == kOpExit) break;
    if (op == kOpCompute) {
      const uint64_t t0 = ticks();
      uint64_t w0 = 0;
      compute_task<D>(a, x, y, grp, w0, [&]() {
        if (tid >= 64 && tid < 128) schedule(ap, &sched, g_cmd);
      });
      claimed = true;
      if (tid == 0) {
        const uint64_t busy = ticks() - t0 - w0;
        const int t_first = group_first(a, y), t_end = group_end(a, y);
        add64(&a.ctrl->compute_ticks.v, busy);
        add32(&a.ctrl->compute_done.v, (uint32_t)(t_end - t_first));  // unit-steps
        add64(&a.ctrl->compute_wait_ticks.v, w0);
        if (a.trace != nullptr)
          for (int t = t_first; t < t_end; ++t)
            trace_rec(ap, kTraceCompute, x, t, (int64_t)t0, (int64_t)w0, 0, 0);
      }
    } else {
      stage_tile<D>(a, ap, (uint32_t)(a.stage_lo + x), y != 0);
    }
  }

  // Exit: the last workgroup out snapshots the statistics and resets the control
  // block for the next launch on this workspace.
  __shared__ int last;
  if (tid == 0) {
    const uint64_t t_end = ticks();
    add64(&a.ctrl->wg_cycles.v, __builtin_readcyclecounter() - c_start);
    add64(&a.ctrl->wg_ticks.v, t_end - t_start);
    max64(&a.ctrl->t_last.v, t_end);
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
    ds->wg_cycles = (int64_t)ld64(&cb->wg_cycles.v);
    ds->wg_ticks = (int64_t)ld64(&cb->wg_ticks.v);
  }
  __syncthreads();
  uint32_t* words = reinterpret_cast<uint32_t*>(cb);
  for (int i = tid; i < (int)(sizeof(DevCtrl) / 4); i += kThreads) words[i] = 0;
  // (A staging-only launch of the unfused baseline leaves the counters to the compute
  // launches that run beside it.)
  if (a.n_groups > 0)
    for (int i = tid; i < a.n_steps; i += kThreads) a.done_count[i] = 0;
}

template __global__ void ring_attn_kernel<64>(KernelArgs);
template __global__ void ring_attn_kernel<128>(KernelArgs);

// ------------------------------------------------------------------ fixed scratch

// Device memory of the entry point that allocates nothing: the control block, the
// flags, the slot ring and the running state of its launches, laid out by the host.
// Each GPU the library runs on holds its own copy until the process ends; every call
// on a GPU shares it. Host code never passes this name to a kernel (on the host it is
// only a stand-in): it uses the address hipGetSymbolAddress returns for the device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Zeroes n 32-bit words (a kernel rather than a memset, so a caller may capture it in
// a graph).
__global__ __launch_bounds__(256) void zero_words(uint32_t* p, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace mkra

// Device address of this device's scratch array, looked up once per device (with that
// device current) and kept. Called with the library lock held.
extern "C" __attribute__((visibility("hidden"))) hipError_t mkra_scratch_address(int device, void** ptr) {
  constexpr int kMaxDevices = 64;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  if (addr[device] == nullptr) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(mkra::scratch));
    if (e != hipSuccess) return e;
    addr[device] = p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

extern "C" __attribute__((visibility("hidden"))) hipError_t mkra_zero_launch(void* p, uint64_t bytes,
                                                                            hipStream_t stream) {
  const uint64_t n = bytes / 4;
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<uint64_t>(1024, (n + 255) / 256);
  hipLaunchKernelGGL(mkra::zero_words, dim3(blocks), dim3(256), 0, stream, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

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
