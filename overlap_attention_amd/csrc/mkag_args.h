// Shared between the host launcher and the persistent AllGather+GEMM kernel: launch
// arguments and the device-side control block. Not part of the public ABI.
#pragma once

#include <stdint.h>

namespace mkag {

// A compute workgroup: 4 waves of 64 lanes, one per SIMD, laid out 2 (rows) x 2
// (columns); each wave owns a 128 x 128 block of the output tile (its accumulators fill
// the accumulation registers, so one workgroup runs per compute unit).
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// Output tile: 256 gathered rows (two staged chunks of one shard) x 256 columns of W;
// K in blocks of 64 (128-byte rows, whole cache lines).
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
// Rows of a staged chunk of A: the pages' Table 3 moves AllGather+GEMM's shards in
// chunks of 128 rows; one staging task and one ready flag per chunk.
constexpr int kChunkRows = 128;
constexpr int kChunksPerTile = kBM / kChunkRows;
// A chunk is staged as kPieces tasks of 64 rows, so two workgroups can copy one chunk
// at once (the chunk's flag counts its pieces in); finer pieces cost more scheduler
// round trips than the shorter start-up waits save.
constexpr int kPieces = 2;
static_assert(kChunkRows % kPieces == 0, "whole-row pieces");
constexpr int kPieceRows = kChunkRows / kPieces;
static_assert(kBM == 2 * kChunkRows, "an output tile reads two staged chunks");
constexpr int kMaxXcd = 8;

enum : uint32_t { kRoleCompute = 0, kRoleStage = 1 };
enum : uint32_t { kErrNone = 0, kErrTimeout = 4 };

struct alignas(64) Line32 {
  uint32_t v;
  uint32_t pad[15];
};
struct alignas(64) Line64 {
  uint64_t v;
  uint64_t pad[7];
};

// Reset to zero by the last workgroup to leave each launch (and at allocation).
struct Ctrl {
  Line32 xcd_head[kMaxXcd];  // compute tiles claimed from each XCD's queue
  Line32 stage_head;         // staging tasks claimed
  Line32 n_stage;            // workgroups in the staging role
  Line32 target;             // controller target + 1 (0 = not set yet)
  Line32 error;
  Line32 exit_count;
  Line64 ctrl_time;
  Line64 compute_ticks;
  Line32 compute_done;
  Line64 stage_ticks;
  Line32 stage_done;
  Line64 compute_wait_ticks;
  Line32 assist_tasks;
  Line32 ctrl_updates;
  Line32 max_stage;
  Line64 t_first;  // complement of the earliest start tick
  Line64 t_last;
  Line64 wg_cycles;
  Line64 wg_ticks;
};

// Survives launches: the host reads it after a call.
struct Status {
  uint32_t sticky_error;
  uint32_t last_error;
  int32_t compute_done;
  int32_t stage_done;
  int32_t assist_tasks;
  int32_t ctrl_updates;
  int32_t max_stage;
  int32_t final_target;
  int64_t compute_ticks;
  int64_t compute_wait_ticks;
  int64_t stage_ticks;
  int64_t kernel_ticks;
  int64_t wg_cycles;
  int64_t wg_ticks;
};

struct Args {
  const uint16_t* a_shards;  // [N, M_loc, K] bf16
  const uint16_t* w;         // [N_out, K] bf16
  uint16_t* a_full;          // [N * M_loc, K] bf16 (written: the gathered activation)
  uint16_t* c;               // [N * M_loc, N_out] bf16 (written)
  int n_ranks, rank, m_loc, k, n_out;
  int n_chunks;              // ceil(M_loc / 128): chunks per shard
  int n_rtiles;              // ceil(M_loc / 256): row tiles per shard (two chunks each)
  int n_ntiles;              // ceil(N_out / 256)
  int n_xcd;                 // compute queues
  int xcd_ntiles[kMaxXcd];   // column tiles of each queue (tile x, x + n_xcd, ...)
  int n_compute;             // compute tiles in total: N * n_rtiles * n_ntiles
  int n_stage_tasks;         // N * n_chunks * kPieces: every shard's chunks, the local one last
  // Device state (library-owned).
  uint64_t* flags;           // [N * n_chunks]: chunk of schedule position o, index j:
                             // (epoch << 20) | pieces staged
  Ctrl* ctrl;
  Status* status;
  uint64_t epoch;
  // Scheduling.
  int grid;
  int split_fixed;
  int ctrl_paper;
  int disable_staging;  // error-path testing: no staging role, no assists
  int initial_stagers;
  int64_t cost_compute0, cost_stage0;  // modelled ticks per task
  uint64_t timeout_ticks;
  uint64_t ctrl_period_ticks;
};

}  // namespace mkag
