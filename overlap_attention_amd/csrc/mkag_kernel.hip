// Persistent AllGather+GEMM for gfx950 (MI355X), one rank's share.
//
// The mKernel paper ("mKernel: Fast Multi-GPU, Multi-Node Fused Kernels", §4 and
// Table 3, AllGather + GEMM row) fuses the gather of the activation shards with the
// GEMM that consumes them: the ranks' shards move in chunks of 128 rows, and the
// GEMM's tiles run as soon as their rows have arrived, the local shard first. Here one
// GPU plays one rank: STAGING workgroups play the gather, copying every shard's
// 128-row chunks from its home (a_shards[s], standing for rank s's memory) into the
// gathered buffer a_full and publishing an epoch-stamped ready flag per chunk; COMPUTE
// workgroups run C = A_full W^T in 256 x 256 output tiles (two chunks each), reading the local shard in
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
#include <utility>

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
// A chunk's flag once all its pieces are staged in launch `epoch`.
__device__ __forceinline__ uint64_t stamp(uint64_t epoch) { return (epoch << 20) | (uint64_t)kPieces; }
__device__ __forceinline__ uint32_t wave_bcast(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Waits until at most N vector-memory operations of this wave are outstanding
// (s_waitcnt: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

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

// Staging task s: piece q = s % kPieces (16 rows) of chunk c = s / kPieces, which is
// chunk j of the shard at staging position o = c / n_chunks: rows
// [128 j + 16 q, 128 j + 16 q + 16) of that shard, copied to its place in a_full. Every
// wave waits for its stores, then thread 0 counts the piece in on the chunk's
// epoch-stamped flag with one agent-scope release (Table 3: 128-row chunks; §4:
// epoch-stamped readiness flags); the chunk is ready when all kPieces are in. Pieces
// past a ragged chunk's end copy nothing and only count in.
__device__ __forceinline__ void stage_piece(const Args& a, int s, bool assist) {
  const int tid = threadIdx.x;
  const uint64_t t0 = ticks();
  const int c = s / kPieces, q = s % kPieces;
  const int o = c / a.n_chunks, j = c % a.n_chunks;
  const int shard = staging_shard(a, o);
  const int r0 = j * kChunkRows + q * kPieceRows;
  const int rows = max(0, min(kPieceRows, a.m_loc - r0));
  const int64_t off = ((int64_t)shard * a.m_loc + r0) * a.k;  // same offset in both buffers
  const u32x4* src = reinterpret_cast<const u32x4*>(a.a_shards + off);
  u32x4* dst = reinterpret_cast<u32x4*>(a.a_full + off);
  const int64_t n16 = (int64_t)rows * a.k / 8;  // 16-byte vectors (K is a multiple of 64)
  constexpr int kInFlight = 16;
  int64_t i = tid;
  for (; i + (kInFlight - 1) * kThreads < n16; i += kInFlight * kThreads) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) dst[i + u * kThreads] = v[u];
  }
  for (; i < n16; i += kThreads) dst[i] = __builtin_nontemporal_load(src + i);
  // Every wave waits for its own stores to complete (a workgroup-scope fence alone does
  // not: it emits no wait before the barrier); thread 0's agent-scope release then
  // covers the whole piece.
  wait_vm<0>();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (tid == 0) {
    fence_release();
    // Count in: a flag stamped by an earlier launch counts as zero pieces.
    uint64_t* f = &a.flags[c];
    uint64_t v = ld64(f);
    while (true) {
      const uint64_t before = (v >> 20) == a.epoch ? (v & 0xfffffull) : 0;
      uint64_t expect = v;
      if (__hip_atomic_compare_exchange_strong(f, &expect, (a.epoch << 20) | (before + 1), __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        break;
      v = expect;
    }
    add64(&a.ctrl->stage_ticks.v, ticks() - t0);
    add32(&a.ctrl->stage_done.v, 1);
    if (assist) add32(&a.ctrl->assist_tasks.v, 1);
  }
}

// ------------------------------------------------------------------ compute role

// LDS: two stages, each an A tile (256 rows x 64 k, 32 KB) and a W tile (256 rows x
// 64 k, 32 KB) in rows of 128 bytes whose eight 16-byte chunks are swizzled (chunk c
// of row r sits at c ^ ((r >> 1) & 7)): any 16 consecutive lanes of an operand read
// (rows r0..r0+15, one chunk index) then cover all 64 banks once.
constexpr int kStages = 2;
constexpr int kRowBytes = kBK * 2;                      // 128
constexpr int kATileBytes = kBM * kRowBytes;            // 32 KB
constexpr int kWTileBytes = kBN * kRowBytes;            // 32 KB
constexpr int kStageBytes = kATileBytes + kWTileBytes;  // 64 KB
constexpr int kLdsBytes = kStages * kStageBytes;        // 128 KB
// A stage is filled by 1 KB block copies (global_load_lds_dwordx4: 64 lanes x 16
// bytes straight into LDS, no registers), 8 rows of 128 bytes each, so every copy
// reads 8 whole cache lines. Copy i of wave w fills block w + kWaves i: blocks 0..31
// hold A rows, 32..63 W rows.
constexpr int kRowsPerCopy = 1024 / kRowBytes;         // 8
constexpr int kCopies = kStageBytes / 1024 / kWaves;   // 16 per wave per stage
constexpr int kCopiesA = kATileBytes / 1024 / kWaves;  // the first 8 of them A
constexpr int kCopiesPerSlice = kCopies / 2;           // issued over one k-slice's MFMAs
static_assert(kStageBytes % (1024 * kWaves) == 0 && kATileBytes % (1024 * kWaves) == 0, "whole copies");
__shared__ __attribute__((aligned(1024))) uint8_t g_lds[kLdsBytes];
__shared__ int32_t g_cmd[4];

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ uint32_t lds_base() { return (uint32_t)(uintptr_t)((lds_void*)g_lds); }

// A 64-bit pointer that is the same in every lane, moved to SGPRs.
__device__ __forceinline__ const uint16_t* wave_bcast_ptr(const uint16_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  return (const uint16_t*)(uintptr_t)(((uint64_t)wave_bcast((uint32_t)(v >> 32)) << 32) | wave_bcast((uint32_t)v));
}

// Workgroup barrier that also orders this wave's LDS reads before it: the copies
// issued after it overwrite a stage the reads came from. The empty asm statements keep
// the compiler from moving LDS accesses across.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Copy i of this wave for the K block whose tile rows start at a_src / w_src
// (wave-uniform), into the stage at LDS address m0s (+ this wave's block).
template <int I>
__device__ __forceinline__ void copy_one(const uint32_t (&voff)[kCopies], const uint16_t* a_src,
                                         const uint16_t* w_src, uint32_t m0s) {
  const uint32_t m0 = m0s + (uint32_t)(I * kWaves * 1024);
  // A memory instruction that reads an SGPR a vector instruction wrote needs 5 wait
  // states first, which the compiler does not keep for inline asm operands. Here the
  // bases are formed once per tile and advanced by scalar adds, and in the compiled
  // code no vector write of a base (nor a branch target) lies within 5 wait states of
  // a copy; the build checks (test_build_isa) hold every build to that, so the copies,
  // one every other MFMA, carry no s_nop (an s_nop 4 each cost 2 % here).
  if constexpr (I < kCopiesA)
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff[I]), "s"(a_src), "{m0}"(m0) : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff[I]), "s"(w_src), "{m0}"(m0) : "memory");
}

template <int... I>
__device__ __forceinline__ void copy_all(std::integer_sequence<int, I...>, const uint32_t (&voff)[kCopies],
                                         const uint16_t* a_src, const uint16_t* w_src, uint32_t m0s) {
  (copy_one<I>(voff, a_src, w_src, m0s), ...);
}

// Operand f of a 16-wide k-slice: f < 4 the wave's W rows 32 f + (lane % 32) of its
// 128, f >= 4 its A rows 32 (f - 4) + (lane % 32); each lane's 8 k values of chunk
// 2 kk + lane / 32 (w_off / a_off carry the wave's rows, kk and the lane's swizzled
// position).
__device__ __forceinline__ bf16x8 read_operand(const uint8_t* sb, int w_off, int a_off, int f) {
  return *reinterpret_cast<const bf16x8*>(sb + (f < 4 ? w_off + 4096 * f : a_off + 4096 * (f - 4)));
}

// The 16 MFMAs of one k-slice on operands f, product q = (A block m = q / 4, W block
// t = q % 4), so consecutive MFMAs share their B operand. After MFMA q: operand q of
// the next slice is read into g (q < 8, READ), and with COPY >= 0 copy COPY + q / 2 is
// issued after every other MFMA, so no wave issues several copies at once and waits for
// the memory pipeline to take them while its matrix core idles. The order is fixed
// (sched_barrier): the compiler may not gather the reads or copies into one burst.
template <bool READ, int COPY>
__device__ __forceinline__ void slice(f32x16 (&acc)[4][4], const bf16x8 (&f)[8], bf16x8 (&g)[8], const uint8_t* gsb,
                                      int w_off, int a_off, const uint32_t (&voff)[kCopies], const uint16_t* a_src,
                                      const uint16_t* w_src, uint32_t m0s) {
  static_assert(COPY < 0 || COPY + kCopiesPerSlice <= kCopies, "copy range");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int m = q >> 2, t = q & 3;
    acc[t][m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[t], f[4 + m], acc[t][m], 0, 0, 0);
    if (READ && q < 8) g[q] = read_operand(gsb, w_off, a_off, q);
    if constexpr (COPY >= 0) {
      if (q % 2 == 0) {
        // q / 2 is a constant after unrolling; dispatch it to the template.
        switch (q / 2) {
          case 0: copy_one<COPY + 0>(voff, a_src, w_src, m0s); break;
          case 1: copy_one<COPY + 1>(voff, a_src, w_src, m0s); break;
          case 2: copy_one<COPY + 2>(voff, a_src, w_src, m0s); break;
          case 3: copy_one<COPY + 3>(voff, a_src, w_src, m0s); break;
          case 4: copy_one<COPY + 4>(voff, a_src, w_src, m0s); break;
          case 5: copy_one<COPY + 5>(voff, a_src, w_src, m0s); break;
          case 6: copy_one<COPY + 6>(voff, a_src, w_src, m0s); break;
          default: copy_one<COPY + 7>(voff, a_src, w_src, m0s); break;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Bounded wait for the ready flag of chunk f (staging order).
__device__ __forceinline__ bool wait_chunk(const Args& a, int f, uint64_t& waited) {
  return wave_wait_stamp(a, &a.flags[f], stamp(a.epoch), waited);
}

// One output tile: row tile rt (compute order) x column tile nt. K blocks of 64 flow
// through the two LDS stages. Block kb + 1 is copied while block kb is consumed: its
// first half once every wave has read block kb - 1 (during the last k-slice of block
// kb - 1), its second half during the first k-slice of block kb; one barrier per block,
// before its last k-slice, after which the next block's first operands are read.
__device__ __forceinline__ void compute_tile(const Args& a, int rt, int nt, uint64_t& waited) {
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hi = lane >> 5;
  const int w = (int)wave_bcast((uint32_t)(tid >> 6));
  const int wm = w >> 1, wn = w & 1;  // wave block: rows wm*128.., columns wn*128..
  rt = (int)wave_bcast((uint32_t)rt);
  nt = (int)wave_bcast((uint32_t)nt);
  const int p = rt / a.n_rtiles, jj = rt % a.n_rtiles;
  const int shard = compute_shard(a, p);
  const int r0 = jj * kBM;
  const int rows = min(kBM, a.m_loc - r0);
  const int n0 = nt * kBN;
  const int cols = min(kBN, a.n_out - n0);
  const int64_t grow0 = (int64_t)shard * a.m_loc + r0;  // first gathered row of the tile
  // The local shard is read in place; every other chunk from a_full once staged.
  const uint16_t* asrc = wave_bcast_ptr((p == 0 ? a.a_shards : a.a_full) + grow0 * a.k);
  const uint16_t* wsrc = wave_bcast_ptr(a.w + (int64_t)n0 * a.k);
  bool ok = true;
  if (p > 0) {
    // Flag of chunk j of the shard at compute position p >= 1: (p - 1) n_chunks + j.
    const int f0 = (p - 1) * a.n_chunks + kChunksPerTile * jj;
    ok = wait_chunk(a, f0, waited);
    if (ok && kChunksPerTile * jj + 1 < a.n_chunks) ok = wait_chunk(a, f0 + 1, waited);
  }
  wait_vm<0>();  // older loads and stores of this wave: the counts below cover copies only

  // Copy lanes: lane l fills LDS chunk l % 8 of row l / 8 of its 1 KB block, which holds
  // k-chunk (l % 8) ^ ((row >> 1) & 7) of that row. Rows past the tile's end read a
  // valid row (their results are never stored).
  const uint32_t row_bytes = (uint32_t)a.k * 2u;
  uint32_t voff[kCopies];
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int b = w + kWaves * i;
    const int r = (i < kCopiesA ? b : b - kBM / kRowsPerCopy) * kRowsPerCopy + (lane >> 3);
    const int rc = i < kCopiesA ? min(r, rows - 1) : min(r, cols - 1);
    voff[i] = (uint32_t)rc * row_bytes + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
  }
  const uint32_t m0w = wave_bcast(lds_base() + (uint32_t)w * 1024u);

  // Operand reads: row r = 32 x + col of a 32-row group, chunk 2 kk + hi, swizzled by
  // (r >> 1) & 7 = (col >> 1) & 7.
  int a_off[4], w_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int lo = col * kRowBytes + 16 * ((2 * kk + hi) ^ ((col >> 1) & 7));
    a_off[kk] = wm * 128 * kRowBytes + lo;
    w_off[kk] = kATileBytes + wn * 128 * kRowBytes + lo;
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[t][m] = f32x16{};

  // Every iteration has the same shape (branches here would split the accumulators'
  // registers): copies past the last block re-read the last block into the stage that
  // is not read again, and the last iteration's reads of the next block's first slice
  // are of valid LDS.
  const int nk = a.k / kBK;
  const auto blk = [&](int x) { return min(x, nk - 1) * kBK; };
  copy_all(std::make_integer_sequence<int, kCopies>{}, voff, asrc, wsrc, m0w);
  copy_all(std::make_integer_sequence<int, kCopiesPerSlice>{}, voff, asrc + blk(1), wsrc + blk(1),
           m0w + (uint32_t)kStageBytes);
  wait_vm<kCopiesPerSlice>();  // block 0
  stage_barrier();
  bf16x8 cur[8], nxt[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) cur[f] = read_operand(g_lds, w_off[0], a_off[0], f);
  for (int kb = 0; kb < nk; ++kb) {
    const int s = kb & 1;
    const uint8_t* sb = g_lds + s * kStageBytes;
    const uint8_t* sb1 = g_lds + (s ^ 1) * kStageBytes;
    const uint32_t m0s = m0w + (uint32_t)(s * kStageBytes), m0s1 = m0w + (uint32_t)((s ^ 1) * kStageBytes);
    const int x1 = blk(kb + 1), x2 = blk(kb + 2);
    // Slice 0 (second half of block kb + 1's copies), slices 1 and 2.
    slice<true, kCopiesPerSlice>(acc, cur, nxt, sb, w_off[1], a_off[1], voff, asrc + x1, wsrc + x1, m0s1);
    slice<true, -1>(acc, nxt, cur, sb, w_off[2], a_off[2], voff, nullptr, nullptr, 0);
    slice<true, -1>(acc, cur, nxt, sb, w_off[3], a_off[3], voff, nullptr, nullptr, 0);
    // Block kb + 1 has landed (this wave's copies; the barrier covers the others') and
    // every wave has read stage s: it takes block kb + 2's first half during slice 3,
    // while block kb + 1's first slice is read.
    wait_vm<0>();
    stage_barrier();
    slice<true, 0>(acc, nxt, cur, sb1, w_off[0], a_off[0], voff, asrc + x2, wsrc + x2, m0s);
  }
  wait_vm<0>();  // the copies past the end, before the next tile fills the stages

  // acc[t][m] element i: output row wm*128 + 32 m + col, column wn*128 + 32 t + 8 (i/4)
  // + 4 hi + (i % 4); four consecutive columns go out as one 8-byte store.
  if (ok) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = wm * 128 + 32 * m + col;
      uint16_t* crow = a.c + (grow0 + r) * a.n_out + n0;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int cc = wn * 128 + 32 * t + 8 * g + 4 * hi;
          // N_out is a multiple of 8: a group of four columns is whole or absent.
          if (r < rows && cc < cols) {
            bf16x4 b;
            b[0] = (__bf16)acc[t][m][4 * g + 0];
            b[1] = (__bf16)acc[t][m][4 * g + 1];
            b[2] = (__bf16)acc[t][m][4 * g + 2];
            b[3] = (__bf16)acc[t][m][4 * g + 3];
            *reinterpret_cast<bf16x4*>(crow + cc) = b;
          }
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

// Queue x: its column tiles of every row tile, in compute order.
__device__ __forceinline__ int64_t queue_len(const Args& a, int x) {
  return (int64_t)a.n_ranks * a.n_rtiles * a.xcd_ntiles[x];
}

struct Sched {
  int32_t role;
  int32_t pending;
  int32_t pend_rt, pend_nt;
};

// Run by wave 0: picks the workgroup's next task and writes (op, x, y). The control
// words are shared by every XCD, so each access is a round trip to memory: the wave
// loads all of them at once, lane-parallel (one round trip), and lane 0 decides from
// that snapshot, with one more round trip to claim a task (and a rate-limited one for
// the controller or a role change).
__device__ __forceinline__ void schedule(const Args& a, Sched* st, int32_t* cmd) {
  const int lane = threadIdx.x & 63;
  const Ctrl* cb = a.ctrl;
  // Lane i < 8: queue head i; then the error word, the staging head, the role count, the
  // target, the update time, the compute and staging tick sums and task counts. 32-bit
  // words are read as the low half of a 64-bit load (each sits at the start of its own
  // 64-byte line).
  const void* src = lane < kMaxXcd ? (const void*)&cb->xcd_head[lane].v
                  : lane == 8      ? (const void*)&cb->error.v
                  : lane == 9      ? (const void*)&cb->stage_head.v
                  : lane == 10     ? (const void*)&cb->n_stage.v
                  : lane == 11     ? (const void*)&cb->target.v
                  : lane == 12     ? (const void*)&cb->ctrl_time.v
                  : lane == 13     ? (const void*)&cb->compute_ticks.v
                  : lane == 14     ? (const void*)&cb->compute_done.v
                  : lane == 15     ? (const void*)&cb->stage_ticks.v
                                   : (const void*)&cb->stage_done.v;
  const uint64_t word = lane < 17 ? ld64(reinterpret_cast<const uint64_t*>(src)) : 0ull;
  auto lane_u32 = [&](int i) { return (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)word, i); };
  auto lane_u64 = [&](int i) {
    return (uint64_t)lane_u32(i) | ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(word >> 32), i) << 32);
  };
  uint32_t heads[kMaxXcd];
#pragma unroll
  for (int i = 0; i < kMaxXcd; ++i) heads[i] = lane_u32(i);
  const uint32_t err = lane_u32(8), sh = lane_u32(9), ns = lane_u32(10), tgt_word = lane_u32(11);
  const uint64_t last = lane_u64(12), c_ticks = lane_u64(13), s_ticks = lane_u64(15);
  const uint32_t cd = lane_u32(14), sd = lane_u32(16);
  if (lane != 0) return;
  int32_t op = kOpExit, x = 0, y = 0;
  if (err != kErrNone) {
    cmd[0] = kOpExit;
    return;
  }
  // With staging disabled (error-path testing) nothing is staged: no role change, no
  // drain, no assist.
  const bool stage_left = !a.disable_staging && (int)sh < a.n_stage_tasks;
  int tgt = target_of(a, tgt_word);
  // Controller: rate-limited by a compare-and-swap on the update time.
  if (!a.split_fixed) {
    const uint64_t now = ticks();
    if ((last == 0 || now - last >= a.ctrl_period_ticks) && cas64(&a.ctrl->ctrl_time.v, last, now)) {
      int64_t rp = 0;
      for (int q = 0; q < a.n_xcd; ++q) {
        const int64_t left = queue_len(a, q) - (int64_t)heads[q];
        rp += left > 0 ? left : 0;
      }
      const int64_t rs = stage_left ? a.n_stage_tasks - (int64_t)sh : 0;
      int64_t cp = a.cost_compute0, cs = a.cost_stage0;
      if (a.ctrl_paper) {
        // The paper's inputs: measured busy ticks per finished task.
        if (cd > 0) cp = (int64_t)(c_ticks / cd);
        if (sd > 0) cs = (int64_t)(s_ticks / sd);
      } else {
        // Measured ticks averaged with the cost model's priors, weighted as one shard's
        // tasks of each role, so the first (cold) tasks do not swing the split.
        const uint64_t kc = (uint64_t)a.n_rtiles * a.n_ntiles, ks = (uint64_t)a.n_chunks * kPieces;
        cp = (int64_t)((c_ticks + kc * (uint64_t)a.cost_compute0) / (cd + kc));
        cs = (int64_t)((s_ticks + ks * (uint64_t)a.cost_stage0) / (sd + ks));
      }
      if (cp < 1) cp = 1;
      if (cs < 1) cs = 1;
      tgt = eq2_target(a.grid, rp, rs, cp, cs);
      __hip_atomic_store(&a.ctrl->target.v, (uint32_t)(tgt + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      add32(&a.ctrl->ctrl_updates.v, 1);
    }
  }
  if (!st->pending) {
    // Role changes at task boundaries (§3.2).
    if (st->role == kRoleStage) {
      if (!stage_left || (!a.split_fixed && (int)ns > tgt && cas32(&a.ctrl->n_stage.v, ns, ns - 1))) {
        if (!stage_left) add32(&a.ctrl->n_stage.v, (uint32_t)-1);
        st->role = kRoleCompute;
      }
    } else if (!a.split_fixed && stage_left) {
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
    // Claim an output tile: this XCD's queue first, then any queue the snapshot shows
    // with tiles left.
    const int own = (int)(blockIdx.x % (unsigned)a.n_xcd);
    for (int i = 0; i < a.n_xcd && !st->pending; ++i) {
      const int q = (own + i) % a.n_xcd;
      const int64_t len = queue_len(a, q);
      uint32_t hq = 0;
#pragma unroll
      for (int j = 0; j < kMaxXcd; ++j)
        if (j == q) hq = heads[j];
      if ((int64_t)hq >= len) continue;
      const uint32_t h = add32(&a.ctrl->xcd_head[q].v, 1);
      if ((int64_t)h >= len) continue;
      const int nq = a.xcd_ntiles[q];
      st->pend_rt = (int32_t)(h / nq);
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
  // The stall rule of §3.2: while a chunk the claimed tile reads is unclaimed staging,
  // stage first (claiming the staging head up to the last piece of the tile's later
  // chunk). A failed
  // compare-and-swap returns a larger head, so the loop ends within need - head + 1
  // attempts, either with a claim or with the chunks claimed by others (who are
  // staging them: the tile's waits on their flags then end).
  const int p = st->pend_rt / a.n_rtiles;
  if (p > 0 && stage_left) {
    const int jj = st->pend_rt % a.n_rtiles;
    const int need =
        ((p - 1) * a.n_chunks + min(kChunksPerTile * jj + kChunksPerTile - 1, a.n_chunks - 1)) * kPieces + kPieces - 1;
    uint32_t h = sh;  // a failed compare-and-swap returns the current head
    while ((int)h <= need && (int)h < a.n_stage_tasks) {
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
  x = st->pend_rt;
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
    if (tid < 64) schedule(a, &sched, g_cmd);
    __syncthreads();
    const int op = g_cmd[0], x = g_cmd[1], y = g_cmd[2];
    if (op == kOpExit) break;
    if (op == kOpStage) {
      stage_piece(a, x, y != 0);
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
