// Shared between the host launcher and the persistent kernel: launch arguments and
// the layout of the device-side control block. Not part of the public ABI.
#pragma once

#include <stdint.h>

namespace mkra {

// Geometry of a compute workgroup: 8 waves of 64 lanes, each wave owning 32 query
// rows of one query head (the n index of a 32x32x16 bf16 MFMA).
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
// Keys per KV block held in LDS (a ring of kStages blocks).
constexpr int kBN = 64;
// Rows of a staged KV tile: the pages' Table 3 moves Ring Attention's KV in tiles of
// 128 rows. A tile's KV heads may be split into pieces (ranges of heads); one staging
// task and one ready flag per (slot, tile, piece).
constexpr int kStageRows = 128;
// LDS pipeline depth of the compute role: KV blocks in flight per workgroup.
constexpr int kStages = 4;
// Ring slots in HBM: step t is staged into slot t % kSlots, which is free once every
// unit has finished step t - kSlots. Eight slots (C3: 8 x 16.8 MB of the 288 GB) let
// the staging role run up to three step groups ahead of the slowest unit, so a group's
// tiles need not all be staged within one group's compute time.
constexpr int kSlots = 8;
// Ring steps per compute task (KernelArgs::group for the first step groups, tail_group
// for the last ones; at most kMaxGroup): a task runs its group's consecutive steps of
// one unit with the running state in registers, so the state is stored and reloaded,
// and a task claimed, once per group. A task of group g needs
// its steps staged, which needs every unit past step group*(g+1) - 1 - kSlots, i.e.
// group g - kSlots/group complete (g-2 or earlier while kSlots >= 2*group): one group
// of claim look-ahead stays deadlock-free.
constexpr int kMaxGroup = 4;
static_assert(kSlots >= 2 * kMaxGroup, "a group task may depend only on groups <= g-2");
// Bytes after the ring slots that the compute role's discarded block copies read
// (one block of the largest head dim; the contents are never used).
constexpr int kDiscardBytes = 2 * kBN * 128 * 2;
constexpr int kMaxXcd = 8;
// Size of the fixed per-device scratch array of the entry point that allocates
// nothing (mk_ring_attn_fwd_noalloc): its control block, flags, slot ring and running
// state must fit in it.
constexpr uint64_t kScratchBytes = 256ull << 20;

// A staged KV block: the keys [64*kt, 64*kt + 64) of one KV head, laid out as the
// compute role's LDS wants them, so a block moves into LDS as one contiguous copy.
//   K part:   64 rows x D bf16; 16-byte chunk c of row r stored at chunk swz_k(r, c).
//   V^T part: D rows x 64 fp16 (V transposed, keys permuted within each 16 so a lane's
//             eight P^T values meet eight contiguous V^T values); chunk c of row d
//             stored at chunk c ^ ((d >> 1) & 7).
// The swizzles make the compute role's 16-byte LDS reads bank-conflict free.
template <int D>
struct Block {
  static constexpr int kKBytes = kBN * D * 2;
  static constexpr int kBytes = 2 * kKBytes;
  static constexpr int kChunks = kBytes / 16;
  static constexpr int kChunksPerThread = kChunks / kThreads;
};

enum : uint32_t { kRoleCompute = 0, kRoleStage = 1 };
// Device-side errors, one bit each (the host ORs them over launches): a bounded wait
// expired; a V value outside the fp16 range of the PV operand was staged.
enum : uint32_t { kErrNone = 0, kErrTimeout = 4, kErrRange = 8 };
enum : int32_t { kTraceCompute = 1, kTraceStage = 2, kTraceController = 3, kTraceRole = 4 };

// One counter per 64-byte line: the counters are hit by atomics from every CU.
struct alignas(64) Line32 {
  uint32_t v;
  uint32_t pad[15];
};
struct alignas(64) Line64 {
  uint64_t v;
  uint64_t pad[7];
};

// Reset to zero by the last workgroup to leave each launch (and at allocation).
struct DevCtrl {
  Line32 xcd_head[kMaxXcd];   // compute tasks claimed from each XCD's queue
  Line32 stage_head;          // staging tasks claimed
  Line32 n_stage;             // workgroups currently in the staging role
  Line32 target;              // controller's target for n_stage
  Line32 error;               // first device-side error of this launch
  Line32 exit_count;          // workgroups that have left the loop
  Line64 ctrl_time;           // tick of the last controller update
  Line64 compute_ticks;       // busy ticks of finished compute tasks
  Line32 compute_done;
  Line64 stage_ticks;         // busy ticks of finished staging tasks
  Line32 stage_done;
  Line64 compute_wait_ticks;
  Line64 stage_wait_ticks;
  Line32 assist_tasks;
  Line32 ctrl_updates;
  Line32 role_switches;
  Line32 max_stage;
  Line32 trace_head;
  Line32 debug_mismatch;      // debug: staged vectors that differed from their source
  Line64 t_first;             // min start tick (0 = unset)
  Line64 t_last;              // max exit tick
  Line64 wg_cycles;           // shader-clock cycles (s_memtime) summed over workgroups
  Line64 wg_ticks;            // the same spans in 100 MHz ticks
};

// Survives launches: the host reads it after a call.
struct DevStatus {
  uint32_t sticky_error;      // OR of device errors since the host last cleared it
  uint32_t last_error;        // error of the last launch
  int32_t initial_target;
  int32_t final_target;
  int32_t compute_done;
  int32_t stage_done;
  int32_t assist_tasks;
  int32_t ctrl_updates;
  int32_t role_switches;
  int32_t max_stage;
  int64_t compute_ticks;
  int64_t compute_wait_ticks;
  int64_t stage_ticks;
  int64_t stage_wait_ticks;
  int64_t kernel_ticks;
  int64_t trace_records;
  int64_t debug_mismatch;
  int64_t wg_cycles;
  int64_t wg_ticks;
};

struct TraceRec {
  uint64_t t;
  int32_t wg;
  int32_t kind;
  int64_t v[6];
};

struct KernelArgs {
  // Problem (device pointers into caller-owned tensors).
  const uint16_t* q;      // [Lq, Hq, D] bf16
  const uint16_t* kv;     // [N, 2, Lk, Hkv, D] bf16
  uint16_t* out;          // [Lq, Hq, D] bf16
  float* lse;             // [Hq, Lq] fp32
  int lq, lk, hq, hkv, d, gqa;
  int n_chunks, rank, causal, n_steps;
  int group;              // ring steps of each of the first n_big step groups, 1..kMaxGroup
  int n_big;              // step groups of `group` steps
  int tail_group;         // ring steps of each later step group, 1..group
  int n_groups;           // step groups: compute tasks per unit in this launch
  int parallel_steps;     // 1: a unit's step groups run independently from a fresh state,
                          // each storing its partial (O, m, l) in its own state slot; the
                          // group that finishes last merges them in group order
  int step_lo;            // first ring step of this launch's step groups (0 when fused)
  int stage_lo;           // first staging task of this launch (0 when fused)
  int external_order;     // 1: launches ordered by stream events (the unfused two-stream
                          // baseline): staging does not wait for slot release
  float scale_log2;       // log2(e) / sqrt(D)

  // Decomposition into compute units: a unit is (KV head, group of HG query heads
  // sharing it, block of BQ query rows); its 8 waves are HG heads x (BQ/32) row blocks.
  int hg;                 // query heads per unit
  int n_hgroups;          // G / hg
  int bq;                 // query rows per unit
  int n_qblocks;          // ceil(Lq / bq)
  int n_units;
  int n_xcd;              // compute queues (one per XCD)
  int xcd_unit_begin[kMaxXcd + 1];

  // Staging work: tasks = (step 0..S-1) x (128-row tile) x (piece: piece_heads KV
  // heads, the last piece possibly fewer), in that order; each step's chunk is staged
  // into slot step % kSlots as blocks of 64 keys per KV head.
  int n_tiles;            // ceil(Lk / 128)
  int n_blocks;           // 2 * n_tiles: blocks per KV head (keys past Lk staged as zeros)
  int stage_interleave;   // 1: staging position p (of n_steps <= kSlots) stages ring step
                          // stage_order[p] (parallel step groups: every group's first
                          // step, then every group's second, ...); 0: position p is step p
  int8_t stage_order[kSlots];
  int8_t stage_pos[kSlots];   // its inverse: the staging position of ring step t
  int n_pieces;           // ceil(Hkv / piece_heads)
  int piece_heads;        // KV heads per piece
  int stage_per_step;     // n_tiles * n_pieces: staging tasks (and ready flags) per step
  int n_stage_tasks;
  int64_t chunk_elems;    // 2 * Lk * Hkv * D: one chunk in kv_chunks
  int64_t slot_bytes;     // Hkv * n_blocks * block bytes

  // Workspace (library-owned device memory).
  uint8_t* slots;         // [kSlots][Hkv][n_blocks] staged blocks, then kDiscardBytes
  uint64_t* slot_flags;   // [kSlots][n_tiles][n_pieces] epoch-stamped ready flags
  uint64_t* unit_flags;   // [n_units] epoch-stamped "step done" per unit
  float* acc;             // [n_units][kWaves][32*D + 256] running (O, m, l, lr) between steps
  uint32_t* done_count;   // [n_steps] units finished per step (slot release)
  DevCtrl* ctrl;
  DevStatus* status;
  TraceRec* trace;
  int trace_cap;
  uint64_t epoch;         // distinct per launch on this workspace, >= 1

  // Scheduling.
  int grid;
  int split_fixed;        // 1 = FIXED split
  int ctrl_paper;         // 1 = Eq. (2) with the paper's inputs (all remaining tasks, measured costs)
  int initial_stagers;
  int disable_staging;
  int stage_delay_ticks;
  int debug_flags;        // bit 0: a staging workgroup reads back the K it wrote
  int64_t rp_tail;        // ADAPTIVE mode: unit-steps R_p leaves out (those that can only
                          // follow the last staging task)
  int64_t cost_compute0;  // modelled ticks per compute task (controller prior)
  int64_t cost_stage0;    // modelled ticks per staging task (one piece of a tile)
  uint64_t timeout_ticks;
  uint64_t ctrl_period_ticks;
};

}  // namespace mkra
