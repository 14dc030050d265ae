// Measurement probes for the ring-attention kernel's bounds on MI355X (gfx950): not part
// of the attention path, built into their own library (libmkra_probes.so).
//
//   mkp_mfma_stream: one workgroup of 8 waves per CU (two per SIMD, as the compute
//     role runs), each wave issuing v_mfma_f32_32x32x16_bf16 back to back, with the A
//     operand taken from registers or read from LDS by one ds_read_b128 per MFMA (the
//     compute role's ratio: 1 KiB of K or Vᵀ per 32x32x16 product), on constant or on
//     random bf16 data, optionally with softmax-like vector work (one exp2 and one FMA
//     per MFMA). Under the chip's power limit the data and the side work set the
//     clock, and so the reachable MFMA rate.
//   mkp_valu_rate: vector-ALU issue rate of v_exp_f32 (the transcendental the softmax
//     needs once per (query, key) pair) and of v_fma_f32, in lane-operations per clock
//     per CU, to compare against the 4·D MFMA FLOPs that accompany each exp.
//   mkp_lds_rate: LDS read bandwidth in bytes per clock per CU, 8 waves per CU issuing
//     ds_read_b128 with no bank conflicts (the compute role reads every MFMA's A
//     operand from LDS, 1 KiB per product, besides the block copies written into LDS).
//   mkp_coexec: the compute role's two-wave pairing on each SIMD, taken apart. The
//     first wave of a SIMD runs the matrix phase's stream (MFMAs on random bf16, each
//     fed by a 1 KiB ds_read_b128), the second the softmax phase's instruction mix
//     (per block: 32 FMAs, 32 exp2, 16 packed fp16 conversions, a 15-add packed fp16
//     tree), alone or both at once, to see how much each slows the other.
//
// Each call allocates its buffers, launches one warm-up and one timed grid of one
// workgroup per CU on the current device, and frees them. Results: ms of the timed
// launch (HIP events), shader clock in GHz (s_memtime cycles over s_memrealtime 100 MHz
// ticks, summed over workgroups), and the rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kThreads = 512;
constexpr int kLdsBytes = 64 * 1024;

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 15;
  x *= 2246822519u;
  x ^= x >> 13;
  return x;
}

// A bf16 with random sign, exponent in [2^-3, 2^1) and random mantissa (about the
// magnitude of unit-normal data).
__device__ __forceinline__ uint32_t rand_bf16(uint32_t x) {
  return (x & 0x8000u) | ((124u + ((x >> 1) & 3u)) << 7) | ((x >> 3) & 0x7fu);
}

__device__ __forceinline__ void stamp(unsigned long long* clk, unsigned long long c0, unsigned long long r0) {
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clk[blockIdx.x * 2] = c1 - c0;
    clk[blockIdx.x * 2 + 1] = r1 - r0;
  }
}

// MODE 0: A from registers (four random sets in turn); 1: A from LDS, constant data;
// 2: A from LDS, random data; 3: as 2 plus one exp2 and one FMA per MFMA.
template <int MODE>
__global__ __launch_bounds__(kThreads) void mfma_stream(float* out, unsigned long long* clk, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr bool kRandom = MODE != 1;
  for (int i = tid; i < kLdsBytes / 16; i += kThreads) {
    u32x4 v;
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = mix((uint32_t)(i * 4 + e) * 2654435761u ^ 0x9e3779b9u);
      v[e] = kRandom ? (rand_bf16(x) | (rand_bf16(x >> 16) << 16)) : (e == 0 ? 0x3c003c00u : 0u);
    }
    reinterpret_cast<u32x4*>(lds)[i] = v;
  }
  __syncthreads();
  // Wave w reads 2 KiB at (w % 4) * 16 KiB: 16 bytes per lane at offsets 0 and 1024.
  const uint32_t base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void*)lds) + (uint32_t)(w & 3) * 16384u + lane * 16u;
  bf16x8 b, ar[4];
  for (int i = 0; i < 8; ++i) {
    b[i] = (__bf16)(kRandom ? ((((lane * 37 + i * 11) % 17) - 8) * 0.21f) : 0.001f * (lane + i));
    for (int k = 0; k < 4; ++k) ar[k][i] = (__bf16)(((((lane + 5 * k) * 29 + i * 13 + k * 7) % 19) - 9) * 0.19f);
  }
  f32x16 c0 = {}, c1 = {};
  float e[8];
  for (int k = 0; k < 8; ++k) e[k] = 0.1f * k + 1e-3f * lane;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
      bf16x8 a0, a1;
      if constexpr (MODE == 0) {
        a0 = ar[(j >> 1) & 3];
        a1 = ar[((j >> 1) + 2) & 3];
      } else {
        u32x4 x0, x1;
        asm volatile("ds_read_b128 %0, %2\n ds_read_b128 %1, %2 offset:1024\n s_waitcnt lgkmcnt(0)"
                     : "=v"(x0), "=v"(x1)
                     : "v"(base));
        a0 = __builtin_bit_cast(bf16x8, x0);
        a1 = __builtin_bit_cast(bf16x8, x1);
      }
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, c1, 0, 0, 0);
      if constexpr (MODE == 3) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          float& v = e[(j + k) & 7];
          v = __builtin_amdgcn_exp2f(-fmaf(v, 0.5f, 0.25f));
        }
      }
    }
  }
  stamp(clk, t0, r0);
  float r = 0.f;
  for (int k = 0; k < 8; ++k) r += e[k];
  for (int i = 0; i < 16; ++i) r += c0[i] + c1[i];
  out[blockIdx.x * kThreads + tid] = r;
}

// MODE 0: v_exp_f32; 1: v_fma_f32. Eight independent chains per lane, 32 operations per
// iteration; the values stay in [0.5, 1].
template <int MODE>
__global__ __launch_bounds__(kThreads) void valu_rate(float* out, unsigned long long* clk, int iters) {
  const int tid = threadIdx.x;
  float x[8];
  for (int k = 0; k < 8; ++k) x[k] = 0.5f + 0.05f * k + 1e-4f * (tid & 63);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if constexpr (MODE == 0) x[k] = __builtin_amdgcn_exp2f(-x[k]);
        else x[k] = fmaf(x[k], 0.999f, 0.0005f);
      }
  }
  stamp(clk, t0, r0);
  float r = 0.f;
  for (int k = 0; k < 8; ++k) r += x[k];
  out[blockIdx.x * kThreads + tid] = r;
}

// Every wave reads its own 8 KiB of LDS as eight ds_read_b128 (lanes at consecutive
// 16-byte addresses, so no bank conflicts), waits for them, and folds one dword of each
// result into a register so the reads stay live: 8 KiB per wave per iteration.
__global__ __launch_bounds__(kThreads) void lds_rate(float* out, unsigned long long* clk, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  static_assert(kLdsBytes == (kThreads / 64) * 8192, "8 KiB of LDS per wave");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kLdsBytes / 4; i += kThreads) reinterpret_cast<uint32_t*>(lds)[i] = mix((uint32_t)i);
  __syncthreads();
  const uint32_t base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void*)lds) + (uint32_t)w * 8192u + lane * 16u;
  uint32_t acc = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    u32x4 x0, x1, x2, x3, x4, x5, x6, x7;
    asm volatile(
        "ds_read_b128 %0, %8\n ds_read_b128 %1, %8 offset:1024\n ds_read_b128 %2, %8 offset:2048\n"
        " ds_read_b128 %3, %8 offset:3072\n ds_read_b128 %4, %8 offset:4096\n ds_read_b128 %5, %8 offset:5120\n"
        " ds_read_b128 %6, %8 offset:6144\n ds_read_b128 %7, %8 offset:7168\n s_waitcnt lgkmcnt(0)"
        : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3), "=v"(x4), "=v"(x5), "=v"(x6), "=v"(x7)
        : "v"(base));
    acc ^= x0[0] ^ x1[1] ^ x2[2] ^ x3[3] ^ x4[0] ^ x5[1] ^ x6[2] ^ x7[3];
  }
  stamp(clk, t0, r0);
  out[blockIdx.x * kThreads + tid] = (float)acc;
}

// MODE 0: only the MFMA waves run; 1: only the softmax waves; 2: both. The first wave
// on a SIMD (by HW_ID) takes the MFMA role, the second the softmax role. Lane 0 of
// each wave writes its role (1 MFMA, 2 softmax, 0 idle) and its s_memtime cycles for
// `iters` iterations: wave_out[2 * (block * 8 + wave) + {0, 1}].
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
template <int MODE>
__global__ __launch_bounds__(kThreads) void coexec(unsigned long long* wave_out, float* sink, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ int32_t simd_of[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kLdsBytes / 16; i += kThreads) {
    u32x4 v;
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = mix((uint32_t)(i * 4 + e) * 2654435761u ^ 0x9e3779b9u);
      v[e] = rand_bf16(x) | (rand_bf16(x >> 16) << 16);
    }
    reinterpret_cast<u32x4*>(lds)[i] = v;
  }
  if (lane == 0) simd_of[w] = (int32_t)__builtin_amdgcn_s_getreg(4 | (4 << 6) | (1 << 11));  // HW_ID bits 5:4
  __syncthreads();
  int before = 0;
  for (int v = 0; v < w; ++v) before += simd_of[v] == simd_of[w];
  const int role = before == 0 ? 1 : before == 1 ? 2 : 0;
  const bool run = role != 0 && (MODE == 2 || MODE == role - 1);
  unsigned long long cyc = 0;
  float r = 0.f;
  if (run && role == 1) {
    // As the compute role issues them: each operand read six MFMAs ahead of its
    // product, with an explicit wait for the oldest read only.
    const uint32_t base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void*)lds) +
                          (uint32_t)(w & 3) * 16384u + lane * 16u;
    uint32_t addr[8];
    for (int k = 0; k < 8; ++k) addr[k] = base + (uint32_t)k * 1024u;
    bf16x8 b;
    for (int i = 0; i < 8; ++i) b[i] = (__bf16)((((lane * 37 + i * 11) % 17) - 8) * 0.21f);
    f32x16 acc[2] = {};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
      u32x4 buf[6];
#pragma unroll
      for (int k = 0; k < 6; ++k) asm volatile("ds_read_b128 %0, %1" : "=v"(buf[k]) : "v"(addr[k]));
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        switch (31 - j < 5 ? 31 - j : 5) {  // reads still in flight after the oldest
          case 5: asm volatile("s_waitcnt lgkmcnt(5)" : "+v"(buf[j % 6])); break;
          case 4: asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(buf[j % 6])); break;
          case 3: asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(buf[j % 6])); break;
          case 2: asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(buf[j % 6])); break;
          case 1: asm volatile("s_waitcnt lgkmcnt(1)" : "+v"(buf[j % 6])); break;
          default: asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(buf[j % 6])); break;
        }
        acc[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, buf[j % 6]), b, acc[j & 1], 0, 0, 0);
        if (j + 6 < 32) asm volatile("ds_read_b128 %0, %1" : "=v"(buf[j % 6]) : "v"(addr[(j + 6) & 7]));
      }
    }
    asm volatile("s_nop 0" ::: "memory");
    for (int i = 0; i < 16; ++i) r += acc[0][i] + acc[1][i];
    cyc = __builtin_amdgcn_s_memtime() - t0;
  } else if (run && role == 2) {
    // One block's softmax per iteration: P = exp2(s c - m) in fp16 pairs, summed by a
    // tree of packed fp16 adds; m follows the sum, so iterations do not overlap.
    float s[32];
    for (int i = 0; i < 32; ++i) s[i] = (((lane * 13 + i * 7) % 23) - 11) * 0.37f;
    float m = 4.f;
    const float c = 1.4426950408889634f * 0.125f;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
      f16x2 p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i][0] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[2 * i], c, -m));
        p[i][1] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[2 * i + 1], c, -m));
      }
#pragma unroll
      for (int k = 8; k >= 1; k >>= 1)
#pragma unroll
        for (int i = 0; i < k; ++i) p[i] = p[i] + p[i + k];
      m = fmaf((float)p[0][0] + (float)p[0][1], 1e-6f, m);
    }
    r = m;
    cyc = __builtin_amdgcn_s_memtime() - t0;
  }
  if (lane == 0) {
    wave_out[2 * (blockIdx.x * (kThreads / 64) + w)] = (unsigned long long)(run ? role : 0);
    wave_out[2 * (blockIdx.x * (kThreads / 64) + w) + 1] = cyc;
  }
  sink[blockIdx.x * kThreads + tid] = r;
}

typedef void (*Kern)(float*, unsigned long long*, int);

// One warm-up launch at iters/10, then a timed launch. res = {ms, GHz, cycles per
// workgroup (mean), CUs}.
int run(Kern k, int iters, double* res) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 1;
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  unsigned long long* h = new unsigned long long[2 * cus];
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  float ms = 0.f;
  if (hipMalloc(&out, sizeof(float) * kThreads * cus) != hipSuccess ||
      hipMalloc(&clk, sizeof(unsigned long long) * 2 * cus) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
      hipEventCreate(&e1) != hipSuccess) {
    rc = 1;
  } else {
    hipLaunchKernelGGL(k, dim3(cus), dim3(kThreads), 0, nullptr, out, clk, iters / 10 > 0 ? iters / 10 : 1);
    rc |= hipDeviceSynchronize() != hipSuccess;
    rc |= hipEventRecord(e0, nullptr) != hipSuccess;
    hipLaunchKernelGGL(k, dim3(cus), dim3(kThreads), 0, nullptr, out, clk, iters);
    rc |= hipEventRecord(e1, nullptr) != hipSuccess;
    rc |= hipEventSynchronize(e1) != hipSuccess;
    rc |= hipGetLastError() != hipSuccess;
    rc |= hipEventElapsedTime(&ms, e0, e1) != hipSuccess;
    rc |= hipMemcpy(h, clk, sizeof(unsigned long long) * 2 * cus, hipMemcpyDeviceToHost) != hipSuccess;
  }
  if (rc == 0) {
    double c = 0, t = 0;
    for (int b = 0; b < cus; ++b) {
      c += (double)h[2 * b];
      t += (double)h[2 * b + 1];
    }
    res[0] = ms;
    res[1] = t > 0 ? c / t * 0.1 : 0.0;
    res[2] = c / cus;
    res[3] = cus;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (clk) (void)hipFree(clk);
  delete[] h;
  return rc;
}

}  // namespace

// mode 0..3 as for mfma_stream above; iters >= 1 (each iteration is 32 MFMAs per
// wave). res[4] = {ms, GHz, TFLOP/s, CUs}. Returns 0, or 1 on a HIP error or a bad
// argument.
extern "C" int mkp_mfma_stream(int mode, int iters, double* res) {
  static const Kern k[4] = {mfma_stream<0>, mfma_stream<1>, mfma_stream<2>, mfma_stream<3>};
  if (mode < 0 || mode > 3 || iters < 1 || !res) return 1;
  double r[4];
  if (run(k[mode], iters, r)) return 1;
  const double flops = r[3] * 8.0 * iters * 32 * (2.0 * 32 * 32 * 16);
  res[0] = r[0];
  res[1] = r[1];
  res[2] = flops / (r[0] * 1e-3) / 1e12;
  res[3] = r[3];
  return 0;
}

// mode 0: v_exp_f32, 1: v_fma_f32; iters >= 1 (32 operations per lane each).
// res[4] = {ms, GHz, lane-operations per clock per CU, CUs}.
extern "C" int mkp_valu_rate(int mode, int iters, double* res) {
  static const Kern k[2] = {valu_rate<0>, valu_rate<1>};
  if (mode < 0 || mode > 1 || iters < 1 || !res) return 1;
  double r[4];
  if (run(k[mode], iters, r)) return 1;
  res[0] = r[0];
  res[1] = r[1];
  res[2] = r[2] > 0 ? (double)kThreads * iters * 32 / r[2] : 0.0;
  res[3] = r[3];
  return 0;
}

// iters >= 1 (8 KiB read per wave each). res[4] = {ms, GHz, bytes per clock per CU, CUs}.
extern "C" int mkp_lds_rate(int iters, double* res) {
  if (iters < 1 || !res) return 1;
  double r[4];
  if (run(lds_rate, iters, r)) return 1;
  res[0] = r[0];
  res[1] = r[1];
  res[2] = r[2] > 0 ? (double)(kThreads / 64) * iters * 8192.0 / r[2] : 0.0;
  res[3] = r[3];
  return 0;
}

// mode 0..2 as for coexec above; iters >= 1 (one iteration: 32 MFMAs for an MFMA wave,
// one block's softmax for a softmax wave). res[4] = {ms, mean cycles per iteration of
// the MFMA waves (0 if none ran), the same for the softmax waves, CUs}.
extern "C" int mkp_coexec(int mode, int iters, double* res) {
  static void (*const k[3])(unsigned long long*, float*, int) = {coexec<0>, coexec<1>, coexec<2>};
  if (mode < 0 || mode > 2 || iters < 1 || !res) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 1;
  const int nw = cus * (kThreads / 64);
  unsigned long long* wo = nullptr;
  float* sink = nullptr;
  unsigned long long* h = new unsigned long long[2 * nw];
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = 0;
  float ms = 0.f;
  if (hipMalloc(&wo, sizeof(unsigned long long) * 2 * nw) != hipSuccess ||
      hipMalloc(&sink, sizeof(float) * kThreads * cus) != hipSuccess || hipEventCreate(&e0) != hipSuccess ||
      hipEventCreate(&e1) != hipSuccess) {
    rc = 1;
  } else {
    hipLaunchKernelGGL(k[mode], dim3(cus), dim3(kThreads), 0, nullptr, wo, sink, iters / 10 > 0 ? iters / 10 : 1);
    rc |= hipDeviceSynchronize() != hipSuccess;
    rc |= hipEventRecord(e0, nullptr) != hipSuccess;
    hipLaunchKernelGGL(k[mode], dim3(cus), dim3(kThreads), 0, nullptr, wo, sink, iters);
    rc |= hipEventRecord(e1, nullptr) != hipSuccess;
    rc |= hipEventSynchronize(e1) != hipSuccess;
    rc |= hipGetLastError() != hipSuccess;
    rc |= hipEventElapsedTime(&ms, e0, e1) != hipSuccess;
    rc |= hipMemcpy(h, wo, sizeof(unsigned long long) * 2 * nw, hipMemcpyDeviceToHost) != hipSuccess;
  }
  if (rc == 0) {
    double cm = 0, cs = 0;
    int nm = 0, ns = 0;
    for (int i = 0; i < nw; ++i) {
      if (h[2 * i] == 1) { cm += (double)h[2 * i + 1]; ++nm; }
      if (h[2 * i] == 2) { cs += (double)h[2 * i + 1]; ++ns; }
    }
    res[0] = ms;
    res[1] = nm ? cm / nm / iters : 0.0;
    res[2] = ns ? cs / ns / iters : 0.0;
    res[3] = cus;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (wo) (void)hipFree(wo);
  if (sink) (void)hipFree(sink);
  delete[] h;
  return rc;
}
