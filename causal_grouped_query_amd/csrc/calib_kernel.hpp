// calib_kernel.hpp -- calibration loops for the roofline of the attention kernel: the
// sustained rate of the matrix core on bf16 operands and of the transcendental unit, at
// the clock the GPU actually holds while it runs them.
//
// The attention kernel's inner loop is v_mfma_f32_32x32x16_bf16 on random bf16 operands
// plus one v_exp_f32 per score; the published MFMA peak assumes the 2.4 GHz peak clock,
// while a board at its power limit runs lower.  These loops measure, with the same
// instructions and one wave per SIMD (the attention kernel's occupancy):
//   KIND 0: eight MFMAs per iteration into four accumulators, the A and B fragments
//           fixed pseudo-random bf16 values (eight of each, so consecutive MFMAs differ
//           in both operands and the datapath toggles as it does on real data), or, with
//           operand_mask 0, all-zero operands (the same instructions with a datapath that
//           does not toggle: the clock difference between the two is the power limit);
//   KIND 1: sixteen independent v_exp_f32 per iteration (x <- 2^-x keeps x in (0, 1]);
//   KIND 2: the KIND 0 loop with a 64 KB LDS reserve, so that two workgroups share a
//           compute unit and every SIMD runs two MFMA waves when the grid has two
//           workgroups per compute unit (a second wave does not raise the matrix core's
//           rate on random operands if the power limit, not the issue, sets it).
// Each wave records the shader-clock counter (s_memtime) and the constant-rate counter
// (s_memrealtime) around its loop (in asm that waits for the values and takes the loop's
// operands, then its results, as inputs, so that nothing moves across a stamp); every
// thread writes one value derived from its results so that the loop cannot be removed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3attn {

constexpr int CALIB_THREADS = 256;             // four waves: one per SIMD of a compute unit
constexpr int CALIB_LDS_BYTES = 96 * 1024;     // over half a CU's LDS: one workgroup per CU
constexpr int CALIB_LDS_BYTES_PAIRED = 64 * 1024;   // two workgroups per CU
constexpr int CALIB_MFMA_PER_ITER = 8;
constexpr int CALIB_EXP_PER_ITER = 16;

// integer mixer (multiply / xor-shift rounds) for the operand bits
__device__ __forceinline__ unsigned calib_mix(unsigned x) {
  x *= 0x9E3779B1u;
  x ^= x >> 15;
  x *= 0x85EBCA77u;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return x;
}

// bf16 bits with random sign and mantissa and a magnitude in [0.25, 4)
__device__ __forceinline__ unsigned short calib_bf16_bits(unsigned h) {
  return (unsigned short)((h & 0x807Fu) | ((125u + ((h >> 8) & 3u)) << 7));
}

template <int KIND>
__global__ __launch_bounds__(CALIB_THREADS, 1) void calib_loop_kernel(uint64_t* stamps,
                                                                     float* sink, int iters,
                                                                     unsigned operand_mask) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  constexpr int LDS_BYTES = KIND == 2 ? CALIB_LDS_BYTES_PAIRED : CALIB_LDS_BYTES;
  __shared__ float reserve[LDS_BYTES / 4];
  constexpr int STRIDE = LDS_BYTES / 4 / CALIB_THREADS;
  const unsigned gid = blockIdx.x * CALIB_THREADS + threadIdx.x;

  // the reserved LDS is used (one word per thread) so that it stays allocated
  reserve[threadIdx.x * STRIDE] = (float)threadIdx.x;
  __syncthreads();

  float result = 0.0f;
  uint64_t t0, t1, r0, r1;
  if constexpr (KIND == 0 || KIND == 2) {
    bf16x8 a[CALIB_MFMA_PER_ITER], b[CALIB_MFMA_PER_ITER];
#pragma unroll
    for (int i = 0; i < CALIB_MFMA_PER_ITER; ++i) {
      u16x8 ua, ub;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ua[e] = calib_bf16_bits(calib_mix(gid * 128u + i * 8u + e)) & operand_mask;
        ub[e] = calib_bf16_bits(calib_mix(gid * 128u + 64u + i * 8u + e)) & operand_mask;
      }
      a[i] = __builtin_bit_cast(bf16x8, ua);
      b[i] = __builtin_bit_cast(bf16x8, ub);
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
    // the operands are inputs of the first stamp, the results of the second: the compiler
    // cannot move either across the loop
    asm volatile("s_memtime %0\n s_memrealtime %1\n s_waitcnt lgkmcnt(0)"
                 : "=s"(t0), "=s"(r0)
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
                   "v"(a[7]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]),
                   "v"(b[6]), "v"(b[7])
                 : "memory");
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < CALIB_MFMA_PER_ITER; ++u)
        acc[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u], acc[u & 3], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) result += acc[j][e];
    asm volatile("s_memtime %0\n s_memrealtime %1\n s_waitcnt lgkmcnt(0)"
                 : "=s"(t1), "=s"(r1) : "v"(result) : "memory");
  } else {
    float x[CALIB_EXP_PER_ITER];
#pragma unroll
    for (int u = 0; u < CALIB_EXP_PER_ITER; ++u)
      x[u] = 0.5f + (float)(calib_mix(gid * 32u + u) >> 9) * 0x1p-24f;   // in [0.5, 1)
    float dep = 0.0f;
#pragma unroll
    for (int u = 0; u < CALIB_EXP_PER_ITER; ++u) dep += x[u];
    asm volatile("s_memtime %0\n s_memrealtime %1\n s_waitcnt lgkmcnt(0)"
                 : "=s"(t0), "=s"(r0) : "v"(dep) : "memory");
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < CALIB_EXP_PER_ITER; ++u) x[u] = __builtin_amdgcn_exp2f(-x[u]);
    }
#pragma unroll
    for (int u = 0; u < CALIB_EXP_PER_ITER; ++u) result += x[u];
    asm volatile("s_memtime %0\n s_memrealtime %1\n s_waitcnt lgkmcnt(0)"
                 : "=s"(t1), "=s"(r1) : "v"(result) : "memory");
  }
  __syncthreads();
  sink[gid] = result + reserve[((threadIdx.x + 1) % CALIB_THREADS) * STRIDE];
  if ((threadIdx.x & 63) == 0) {
    uint64_t* s = stamps + (size_t)(gid / 64) * 4;
    s[0] = t0;
    s[1] = t1;
    s[2] = r0;
    s[3] = r1;
  }
}

}  // namespace h3attn
