/*
 * mkag: one rank's AllGather+GEMM for AMD Instinct MI355X (gfx950), in the same
 * library as the ring-attention forward (libmkra.so) and on the same runtime: one
 * persistent kernel whose workgroups take a staging or a compute role, epoch-stamped
 * ready flags per 128-row chunk, and the on-GPU controller of Eq. (2).
 *
 * Source: the mKernel paper "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels"
 * (arXiv 2609.13585), §4 and Table 3 (AllGather + GEMM row: tensor parallelism,
 * communication feeds computation, shards moved in 128-row chunks, compute tiles
 * ordered by input availability with the local shard first), §3.2 and Eq. (2); the
 * project README's kernel table (AllGather + GEMM row).
 *
 * On one GPU the call plays one rank of an N-rank tensor-parallel group. The staging
 * role plays the gather: it copies each shard's 128-row chunks (as 64-row pieces, so
 * two workgroups can share a chunk) from the shard's home
 * (a_shards[s], standing for rank s's memory) into the gathered activation a_full and
 * publishes a ready flag per chunk. The compute role computes C = A_full W^T in
 * 256 x 256 output tiles (two chunks of one shard each) as their rows arrive, reading
 * the local shard in place.
 *
 * Conventions are those of include/mkra.h: tensor data pointers are device pointers on
 * the current HIP device, everything else host pointers; the caller owns the tensors;
 * the library owns a workspace per (device, stream) (flags, control block, status),
 * grown on demand and freed by mk_release_workspace(); errors are mk_status codes with
 * a message from mk_last_error(); argument errors are found on the host before
 * anything is enqueued.
 */
#ifndef MKAG_H
#define MKAG_H

#include "mkra.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t split_mode;          /* MK_SPLIT_ADAPTIVE (default): Eq. (2) re-targets the
                                  staging-workgroup count from measured per-task costs,
                                  averaged with the cost model's priors (weighted as one
                                  shard's tasks of each role); MK_SPLIT_ADAPTIVE_PAPER:
                                  Eq. (2) with the measured costs alone; MK_SPLIT_FIXED:
                                  workgroups 0..fixed_staging_wgs-1 stage until staging
                                  runs out, then compute. */
  int32_t fixed_staging_wgs;   /* FIXED mode: staging workgroups. */
  int32_t initial_staging_wgs; /* adaptive modes: 0 = from the cost model; >0 = this. */
  int32_t grid_wgs;            /* 0 = one workgroup per resident slot (all CUs). */
  int64_t spin_timeout_us;     /* bound of every on-GPU wait; 0 = 10 s. */
  int32_t controller_period_us;/* minimum time between controller updates; 0 = 20 us. */
  int32_t phase;               /* 0: the fused call. The unfused sequence of the same code
                                  ([P] Fig. 1(b): the gather, then the GEMM, released at
                                  the kernel boundary) for measurement: 1 runs the gather
                                  only (every workgroup stages; a_full and the chunk
                                  flags are written, c is not); 2 runs the GEMM only,
                                  consuming the chunk flags of the phase-1 call just
                                  before it on the same stream, which must have had the
                                  same arguments (MK_E_INVAL if no phase-1 call
                                  precedes it). */
  int32_t disable_staging;     /* DEBUG (testing the error path): nobody stages and no
                                  workgroup assists, so the tiles of remote shards wait
                                  until spin_timeout_us expires and the call reports
                                  MK_E_TIMEOUT through mk_ag_gemm_status. 0 normally. */
  int32_t reserved[3];
} mk_ag_gemm_opts;

/* Filled by mk_allgather_gemm_ex when stats != NULL (the call then synchronises the
 * stream). Ticks are 100 MHz s_memrealtime ticks. */
typedef struct {
  int32_t status;              /* device-side result: MK_OK or MK_E_TIMEOUT */
  int32_t grid_wgs;
  int32_t compute_tiles;       /* output tiles: N * ceil(M_loc/256) * ceil(N_out/256) */
  int32_t staging_tasks;       /* 64-row pieces, 2 per 128-row chunk: N * ceil(M_loc/128)
                                  * 2 (the local shard's too); a chunk's ready flag
                                  counts its pieces in */
  int32_t compute_done;
  int32_t staging_done;
  int32_t assist_tasks;        /* chunks staged by compute workgroups (stall rule) */
  int32_t controller_updates;
  int32_t max_staging_wgs;
  int32_t final_target;
  int64_t compute_busy_ticks;
  int64_t compute_wait_ticks;  /* compute waves waiting for chunk flags */
  int64_t staging_busy_ticks;
  int64_t kernel_ticks;        /* first workgroup start to last exit */
  int64_t wg_cycles;           /* shader-clock cycles of all workgroup lifetimes */
  int64_t wg_ticks;            /* the same lifetimes in 100 MHz ticks */
} mk_ag_gemm_stats;

/* One rank's AllGather+GEMM (paper §4, Table 3, AllGather + GEMM row).
 *
 *  a_shards  [N, M_loc, K]   bf16, device. Every rank's activation shard;
 *                            a_shards[rank] is the local one, the others stand for the
 *                            memory of the other ranks.
 *  n_ranks   N >= 1 (must equal a_shards.shape[0])
 *  rank      0 <= rank < N
 *  w         [N_out, K]      bf16, device. This rank's weight shard (a linear layer's
 *                            layout: row n holds output column n's K weights).
 *  a_full    [N*M_loc, K]    bf16, device, written: the gathered activation, shard s
 *                            at rows s*M_loc .. (s+1)*M_loc - 1.
 *  c         [N*M_loc, N_out] bf16, device, written: C = A_full W^T, accumulated in
 *                            fp32 and rounded to bf16 once.
 *  stream    HIP stream the kernel is enqueued on.
 *
 * K must be a multiple of 64 (at most 2^22) and N_out a multiple of 8 (else
 * MK_E_UNSUPPORTED, MK_E_INVAL past the bound); M_loc
 * may be any size (ragged chunks are masked). M_loc == 0 or N_out == 0 with nothing to
 * gather is a no-op. Data pointers must be 16-byte aligned; a_full and c must not
 * overlap the inputs or each other. Asynchronous; device-side timeouts are reported
 * by mk_ag_gemm_status(). Results are bitwise reproducible across launches, grid sizes
 * and splits (each output element is reduced in a fixed order). */
mk_status mk_allgather_gemm(const mk_tensor* a_shards, int n_ranks, int rank, const mk_tensor* w,
                            mk_tensor* a_full, mk_tensor* c, hipStream_t stream);

/* As mk_allgather_gemm, with options (NULL = defaults) and optional statistics (NULL =
 * none; non-NULL synchronises the stream before returning). */
mk_status mk_allgather_gemm_ex(const mk_tensor* a_shards, int n_ranks, int rank, const mk_tensor* w,
                               mk_tensor* a_full, mk_tensor* c, hipStream_t stream, const mk_ag_gemm_opts* opts,
                               mk_ag_gemm_stats* stats);

/* Fills *opts with the defaults (adaptive split, all CUs, 10 s wait bound). */
void mk_ag_gemm_default_opts(mk_ag_gemm_opts* opts);

/* Synchronises `stream` and returns the device-side status of the AllGather+GEMM calls
 * enqueued on it since the last check: MK_E_TIMEOUT if a bounded wait expired, else
 * MK_OK (MK_E_HIP if the synchronisation fails). Clears the sticky status. */
mk_status mk_ag_gemm_status(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MKAG_H */
