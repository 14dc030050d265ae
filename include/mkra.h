/*
 * mkra — per-rank ring-attention forward for AMD Instinct MI355X (gfx950).
 *
 * One rank of a sequence-parallel ring holds a query chunk; the sequence's KV chunks
 * pass it one ring step at a time, and at each step the rank's FlashAttention
 * consumes the chunk it holds and merges the partial result into its accumulated
 * output with an online softmax (running max, running sum, log-sum-exp).
 * Sources: the mKernel paper "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels"
 * (arXiv 2609.13585), §4 and Table 3 (Ring Attention row), §3.2 with Eq. (2)
 * (adaptive SM partition), §2.2 with Eq. (1) (cost of a fused kernel with S_c
 * communication SMs); the project README's kernel table (Ring Attention row).
 *
 * Everything runs in ONE persistent kernel per call. Its workgroups (one per compute
 * unit) take one of two roles: compute (the attention steps) or staging (the ring
 * receive: copy each step's KV chunk into a ring of eight slots in HBM, 128-row tile
 * by 128-row tile, in the layout the compute role reads, and publish an
 * epoch-stamped ready flag per tile, or per range of a tile's KV heads when the tile
 * is staged in pieces). An on-GPU controller re-targets the number of staging
 * workgroups with Eq. (2).
 *
 * Conventions for every entry point:
 *  - All tensor data pointers are DEVICE pointers on the current HIP device; every
 *    other pointer argument (descriptors, opts, stats, buffers for copies) is a HOST
 *    pointer.
 *  - The caller owns all tensors and must keep them alive until the stream has
 *    passed the call. The library keeps no pointer to them after returning.
 *  - The library owns a workspace per (device, stream): the KV slot ring, ready
 *    flags, counters, the fp32 accumulator carried between ring steps, and an
 *    optional trace buffer. It grows on demand (synchronising that stream first) and
 *    is freed by mk_release_workspace(). Two calls on one stream run one after the
 *    other; calls on different streams use different workspaces.
 *  - Errors are returned as mk_status; nothing is thrown across the ABI. Argument
 *    errors are detected on the host before anything is enqueued. A text message
 *    for the last failing call on the calling thread is kept by mk_last_error().
 */
#ifndef MKRA_H
#define MKRA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MKRA_ABI_VERSION 2

typedef enum {
  MK_OK = 0,
  MK_E_INVAL = 1,        /* bad argument: null pointer, shape, dtype, stride, rank, alignment */
  MK_E_UNSUPPORTED = 2,  /* valid request outside what the kernels implement (head_dim on the
                            host; a V value outside the fp16 range, found on the GPU) */
  MK_E_HIP = 3,          /* a HIP runtime call failed (allocation, launch, copy) */
  MK_E_TIMEOUT = 4       /* a bounded on-GPU wait expired; the kernel exited early */
} mk_status;

typedef enum { MK_BF16 = 1, MK_F32 = 2 } mk_dtype;

/* A strided tensor view. data: device pointer; shape/stride in elements; only the
 * first ndim entries are read. Every tensor passed to mkra must be contiguous in
 * row-major order (strides of dimensions of extent 1 are not checked). */
typedef struct {
  void* data;
  int32_t dtype;   /* mk_dtype */
  int32_t ndim;
  int64_t shape[5];
  int64_t stride[5];
} mk_tensor;

typedef enum { MK_SPLIT_ADAPTIVE = 0, MK_SPLIT_FIXED = 1, MK_SPLIT_ADAPTIVE_PAPER = 2 } mk_split_mode;

typedef struct {
  int32_t split_mode;          /* mk_split_mode. ADAPTIVE (default): the controller of
                                  §3.2 re-targets the staging-workgroup count with
                                  Eq. (2) from measured per-task costs, with two
                                  changes to its inputs: R_p leaves out the compute
                                  of the last staged ring step (it can only follow the
                                  last staging task; with parallel step groups staged
                                  group-interleaved, the last step of every group),
                                  and C_p, C_s are averaged with the
                                  cost model's priors weighted as one ring step (C_s
                                  counting a staging task's waits for a free slot).
                                  ADAPTIVE_PAPER: Eq. (2) as §3.2 states it, R_p all
                                  remaining compute tasks (unit-steps), R_s all
                                  remaining staging tasks, C_p and C_s the measured
                                  busy cycles per finished task of each role (the cost
                                  model only until a role has finished a task). FIXED:
                                  workgroups 0..fixed_staging_wgs-1 stage (by block
                                  index) until staging work runs out, then compute. */
  int32_t fixed_staging_wgs;   /* FIXED mode only: number of staging workgroups. */
  int32_t initial_staging_wgs; /* ADAPTIVE mode: 0 = from the host's cost model of
                                  Eq. (2) with modelled costs, or, for a launch whose
                                  staging fits in one round (at most 8 ring steps and
                                  at most half of the grid's workgroups in staging
                                  tasks), one workgroup per staging task; >0 = start
                                  with this. */
  int32_t grid_wgs;            /* 0 = one workgroup per resident slot (all CUs). */
  int64_t spin_timeout_us;     /* bound of every on-GPU wait; 0 = 10 s. */
  int32_t controller_period_us;/* minimum time between controller updates; 0 = 20 us. */
  int32_t trace;               /* nonzero: record per-task events (mk_ring_attn_trace). */
  int32_t trace_capacity;      /* records kept when tracing; 0 = 262144. */
  int32_t disable_staging;     /* DEBUG: nobody stages, so the first compute task
                                  waits until spin_timeout_us and the call reports
                                  MK_E_TIMEOUT. All workgroups still exit normally. */
  int32_t stage_delay_ticks;   /* DEBUG: before publishing each staged tile, spin a
                                  pseudo-random 0..stage_delay_ticks (100 MHz ticks). */
  int32_t debug_flags;         /* DEBUG bit mask, 0 in normal use. bit 0: a staging
                                  workgroup reads back the K part of every block it
                                  wrote and compares it with the chunk's home copy;
                                  mismatches are counted in
                                  mk_ring_attn_stats.debug_mismatches. bit 1: before
                                  the launch the host synchronises the stream and
                                  writes into every ready flag and unit flag of the
                                  workspace a stamp of the right step but of the
                                  previous or the next launch, which the kernel must
                                  not consume. Other bits are ignored. */
  int32_t steps_per_task;      /* ring steps a compute task runs with the running state
                                  in registers, 1..4; 0 = the library's default (2 for
                                  chunks of Lk*D >= 2^19, else 4). */
  int32_t tail_steps;          /* the last tail_steps ring steps run in tasks of
                                  tail_steps_per_task steps (shorter tasks shorten the
                                  end of the launch); 0 = default (4 when tasks have more than two
                                  steps and the units outnumber the workgroups, else
                                  none), < 0 = none. */
  int32_t tail_steps_per_task; /* 1..steps_per_task (larger values are clamped to it);
                                  0 = default (2). */
  int32_t parallel_steps;      /* 1: a unit's step groups run at once, each from a fresh
                                  online-softmax state, and the group that finishes last
                                  merges the partial (O, m, l) in group order (the
                                  mathematics of the per-chunk LSE merge, in fp32);
                                  -1: never (a unit's groups run in order, the state
                                  carried); 0 = default: on when the units fill at most
                                  half of the device's workgroup slots. With it,
                                  steps_per_task defaults to a quarter of the steps,
                                  clamped to 2..4, and there is no default tail.
                                  Results are reproducible for a given mode and
                                  grouping (the merge runs in group order). */
  int32_t stage_pieces;        /* staging tasks per 128-row tile: its KV heads split
                                  into this many ranges of ceil(Hkv / stage_pieces)
                                  heads (fewer when that divides Hkv into fewer
                                  ranges), each range staged by one task and published
                                  by its own ready flag, which the units of those
                                  heads alone wait for. 1..Hkv (larger values are
                                  clamped to Hkv); 0 = default (set by the library
                                  from the problem's size, see
                                  mk_ring_attn_stats.stage_pieces). Results do not
                                  depend on it. */
} mk_ring_attn_opts;

/* Filled by mk_ring_attn_fwd_ex when stats != NULL (the call then synchronises the
 * stream). Times are in s_memrealtime ticks (100 MHz). */
typedef struct {
  int32_t status;              /* device-side result of the launch (MK_OK, MK_E_TIMEOUT, or
                                  MK_E_UNSUPPORTED for a V outside the fp16 range) */
  int32_t grid_wgs;            /* persistent workgroups launched */
  int32_t n_units;             /* compute units per step (head group x query block) */
  int32_t n_steps;             /* ring steps run */
  int32_t n_stage_tiles;       /* 128-row staged tiles per chunk */
  int32_t n_stage_tasks;       /* staging tasks in total: one per (step, tile, piece);
                                  the local chunk of step 0 is staged too */
  int32_t compute_tasks_done;
  int32_t staging_tasks_done;  /* by staging and by compute workgroups */
  int32_t assist_tasks;        /* staging tasks done by compute workgroups whose input
                                  was not ready (the stall rule of §3.2) */
  int32_t initial_target;      /* staging workgroups at launch */
  int32_t final_target;        /* controller target at exit */
  int32_t max_staging_wgs;     /* largest number of workgroups in the staging role */
  int32_t controller_updates;
  int32_t role_switches;
  int64_t compute_busy_ticks;  /* summed over compute tasks, waits excluded */
  int64_t compute_wait_ticks;  /* compute waves waiting on ready flags / unit order */
  int64_t staging_busy_ticks;  /* summed over staging tasks, waits excluded */
  int64_t staging_wait_ticks;  /* staging workgroups waiting for a slot to be released */
  int64_t kernel_ticks;        /* first workgroup start to last workgroup exit */
  int64_t trace_records;       /* records written (may exceed trace_capacity) */
  int64_t debug_mismatches;    /* see mk_ring_attn_opts.debug_flags */
  int64_t wg_cycles;           /* shader-clock cycles (s_memtime) of every workgroup's
                                  lifetime, summed */
  int64_t wg_ticks;            /* the same lifetimes in 100 MHz ticks: the average
                                  shader clock is wg_cycles / wg_ticks * 100 MHz */
  int32_t steps_per_task;      /* ring steps per compute task in this launch (before
                                  the tail) */
  int32_t step_groups;         /* compute tasks per unit */
  int32_t parallel_steps;      /* 1 if the launch ran its step groups at once (see
                                  mk_ring_attn_opts.parallel_steps) */
  int32_t stage_pieces;        /* staging tasks per tile in this launch (see
                                  mk_ring_attn_opts.stage_pieces) */
} mk_ring_attn_stats;

/* One trace record (64 bytes). kind: 1 compute task (v0 unit, v1 step, v2 start tick,
 * v3 wait ticks), 2 staging task (v0 task, v1 step, v2 tile, v3 start tick, v4 1 if
 * done by a stalled compute workgroup, v5 its piece of the tile, -1 if it did not
 * copy), 3 controller update (v0 R_p as Eq. (2) takes it:
 * unclaimed compute unit-steps, less the last ring step's in ADAPTIVE mode, v1 R_s, v2 C_p,
 * v3 C_s, v4 blocks B, v5 new target), 4 role switch (v0 new role: 0 compute,
 * 1 staging, v1 staging-role count after it). t: tick at which it was written. */
typedef struct {
  uint64_t t;
  int32_t wg;
  int32_t kind;
  int64_t v[6];
} mk_trace_record;

/* Per-rank ring-attention forward (mKernel paper §4, Table 3, Ring Attention row;
 * README kernel table, Ring Attention row; online softmax of FlashAttention-2).
 *
 *  q          [Lq, Hq, D]           bf16, device. This rank's query chunk.
 *  kv_chunks  [N, 2, Lk, Hkv, D]    bf16, device. All N = n_chunks KV chunks of the
 *                                   sequence (index 0 = K, 1 = V). kv_chunks[rank] is
 *                                   the local chunk; the others stand for the memory
 *                                   of the other ranks, from which the staging role
 *                                   copies each step's chunk into the slot ring.
 *  n_chunks   N >= 1 (ring size)
 *  rank       0 <= rank < N
 *  causal     0: every query sees every key. 1: query i sits at global position
 *             rank*Lq + i, key j of chunk c at c*Lk + j, and a query sees a key iff
 *             key position <= query position (needs Lq == Lk); chunks after the rank
 *             are skipped (never read).
 *  gqa_ratio  G >= 1 with Hq == G * Hkv; query head h reads KV head h / G.
 *  out        [Lq, Hq, D]           bf16, device, written: softmax(QK^T/sqrt(D)) V.
 *  lse        [Hq, Lq]              fp32, device, written: natural-log log-sum-exp of
 *                                   the scaled scores of each (head, query).
 *  stream     HIP stream the kernel is enqueued on (0 = null stream).
 *
 * Step t (t = 0..S-1) consumes chunk (rank - t) mod N; S = rank+1 if causal, else N.
 * Precision: QK^T takes Q and K in bf16; the PV product takes V converted to fp16
 * and P rounded to fp16 (fp32 accumulation throughout). V must therefore satisfy
 * |v| < 65536 and be finite in every chunk the call reads (chunks after the rank
 * are not read when causal); a V outside that range is detected by the staging role
 * on the GPU, ends the launch early (every workgroup exits normally; out and lse are
 * then undefined) and is reported as MK_E_UNSUPPORTED by mk_ring_attn_status() and
 * in mk_ring_attn_stats.status. V values below 2^-14 in magnitude are rounded to the
 * fp16 subnormal grid (absolute error at most 2^-25).
 * D must be 64 or 128 (else MK_E_UNSUPPORTED). Lq, Lk, Hq, Hkv may be any size
 * (ragged tiles are masked); Lq == 0 or Hq == 0 is a no-op returning MK_OK; Lk == 0
 * with Lq > 0 is MK_E_INVAL. Data pointers of non-empty tensors must be 16-byte
 * aligned; out and lse must not overlap the inputs or each other.
 * Asynchronous: returns after enqueueing; device-side errors (an expired wait, a V
 * out of range) are reported by mk_ring_attn_status(). Results are bitwise reproducible across launches, grid
 * sizes and staging splits (each output is reduced in a fixed order). */
mk_status mk_ring_attn_fwd(const mk_tensor* q, const mk_tensor* kv_chunks, int n_chunks, int rank, int causal,
                           int gqa_ratio, mk_tensor* out, mk_tensor* lse, hipStream_t stream);

/* As mk_ring_attn_fwd, with options (NULL = defaults) and optional statistics
 * (NULL = none; non-NULL synchronises the stream before returning). */
mk_status mk_ring_attn_fwd_ex(const mk_tensor* q, const mk_tensor* kv_chunks, int n_chunks, int rank, int causal,
                              int gqa_ratio, mk_tensor* out, mk_tensor* lse, hipStream_t stream,
                              const mk_ring_attn_opts* opts, mk_ring_attn_stats* stats);

/* As mk_ring_attn_fwd (default options), for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It calls no hipMalloc, hipFree or other allocating routine. All of its
 * device state (control block, flags, the eight-slot KV ring, the fp32 running state)
 * lives in a fixed array of MKRA_NOALLOC_SCRATCH_BYTES (256 MiB) in the library's
 * code object, one per GPU, held from the library's first use on that GPU until the
 * process ends. A problem whose state does not fit (about 8 staged copies of one KV
 * chunk plus 17 KB of fp32 state per 32 query rows and head, e.g. the 64K-token GQA
 * rank share fits, a 128K-token one does not) returns MK_E_UNSUPPORTED before
 * anything is enqueued. Each call first clears the control block, counters and flags
 * of the array with a small kernel on `stream` (no memset), then launches the ring
 * kernel. Every call on a GPU shares that GPU's array and it keeps the last call's
 * contents: calls that overlap on one GPU (different streams, or different threads
 * without ordering) race and must not be issued. Device-side errors of these calls
 * are reported by mk_ring_attn_status() on any stream of the same device. */
mk_status mk_ring_attn_fwd_noalloc(const mk_tensor* q, const mk_tensor* kv_chunks, int n_chunks, int rank,
                                   int causal, int gqa_ratio, mk_tensor* out, mk_tensor* lse, hipStream_t stream);

#define MKRA_NOALLOC_SCRATCH_BYTES (256ull << 20)

/* The unfused two-stream baseline the fused kernel is measured against (mKernel paper
 * §1, Figure 1(b): a two-stream pipeline that releases each chunk only at a kernel
 * boundary; §5.4 compares the fused Ring Attention with attention kernels followed by
 * a separate collective). A measurement leg, not a second way to compute: same
 * arguments and results as mk_ring_attn_fwd (bitwise equal to mk_ring_attn_fwd_ex with
 * steps_per_task = 1 and tail_steps = -1), computed by the same kernel's device code
 * launched once per ring step:
 *  - copy_stream: for each step t, a staging-only launch with copy_wgs workgroups
 *    copies step t's chunk into slot t mod 8 of the workspace's slot ring, after
 *    waiting (stream event) for the compute launch of step t-8, the last reader of
 *    that slot;
 *  - stream: for each step t, after waiting for that staging launch, a compute-only
 *    launch runs every unit's step t on the rest of the workgroups, carrying the
 *    running state through the workspace from step to step.
 * copy_stream must be a different stream of the same device than `stream`; the call
 * makes copy_stream wait for the work already on `stream`, and the last compute
 * launch on `stream` follows every staging launch, so later work on `stream` sees the
 * whole call done. copy_wgs >= 1 (clamped to leave at least one compute workgroup).
 * The workspace is the one of `stream`; device-side errors of either stream's
 * launches are reported by mk_ring_attn_status(stream). */
mk_status mk_ring_attn_fwd_unfused(const mk_tensor* q, const mk_tensor* kv_chunks, int n_chunks, int rank, int causal,
                                   int gqa_ratio, mk_tensor* out, mk_tensor* lse, hipStream_t stream,
                                   hipStream_t copy_stream, int copy_wgs);

/* Fills *opts with the defaults (adaptive split, all CUs, 10 s wait bound). */
void mk_ring_attn_default_opts(mk_ring_attn_opts* opts);

/* Synchronises `stream` and returns the device-side status of the calls enqueued on
 * it since the last check: MK_E_UNSUPPORTED if any of them staged a V outside the
 * fp16 range (|v| >= 65536 or not finite), else MK_E_TIMEOUT if any hit a wait bound,
 * else MK_OK (MK_E_HIP if the synchronisation itself fails). Clears the sticky
 * status. */
mk_status mk_ring_attn_status(hipStream_t stream);

/* Copies up to `capacity` trace records of the last traced call on `stream` into the
 * host buffer `records` and stores the number copied in *n_copied (host pointer).
 * Synchronises the stream. MK_E_INVAL if no traced call ran on that stream. */
mk_status mk_ring_attn_trace(hipStream_t stream, mk_trace_record* records, int64_t capacity, int64_t* n_copied);

/* Message for the last failing call on this thread ("" if none). Owned by the
 * library; valid until the next call on this thread. */
const char* mk_last_error(void);

/* Frees every workspace after synchronising each owning stream. Later calls
 * allocate again. */
void mk_release_workspace(void);

/* MKRA_ABI_VERSION of the loaded library. */
int mk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MKRA_H */
