// pool_tokens_kernel.hpp -- gfx950 kernel that shortens a token sequence by averaging
// groups of consecutive tokens inside one span (the reference-video tokens).
//
// The second fix direction of the h3.c issue "Qwen text encoder: sequence exceeds Metal
// threadgroup memory with reference video + ref images (>=150 frames)" ("Suggested fix
// directions") pools or down-samples the ~1000 video tokens per second before the text
// encoder.  The operation: x [T, C] bf16; inside [begin, end) every `factor` consecutive
// tokens become their mean (a shorter last group averages what it has); the tokens
// before and after the span are copied.  Output [T - L + ceil(L / factor), C].
//
// HBM-bound: each output row is one workgroup; its threads stream the row's channels
// 8 bf16 (16 bytes) at a time, summing the group's input rows in fp32 and rounding the
// mean to bf16 once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3attn {

struct PoolParams {
  const uint16_t* x;   // [T, C] bf16
  uint16_t* out;       // [T_out, C] bf16
  int T, C, begin, end, factor;
};

constexpr int POOL_THREADS = 256;

__global__ __launch_bounds__(POOL_THREADS) void pool_tokens_kernel(PoolParams p) {
  typedef float f32x8v __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
  typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
  const int row = blockIdx.x;                     // output row
  const int L = p.end - p.begin;
  const int groups = (L + p.factor - 1) / p.factor;
  int first, count;                               // input rows [first, first + count)
  if (row < p.begin) {
    first = row;
    count = 1;
  } else if (row < p.begin + groups) {
    first = p.begin + (row - p.begin) * p.factor;
    count = min(p.factor, p.end - first);
  } else {
    first = p.end + (row - p.begin - groups);
    count = 1;
  }
  const float inv = 1.0f / (float)count;
  for (int c = 8 * threadIdx.x; c < p.C; c += 8 * POOL_THREADS) {
    f32x8v acc = {};
    for (int t = 0; t < count; ++t)
      acc += __builtin_convertvector(
          __builtin_bit_cast(bf16x8v, *(const u32x4v*)(p.x + (size_t)(first + t) * p.C + c)),
          f32x8v);
    if (count > 1) acc *= inv;
    *(u32x4v*)(p.out + (size_t)row * p.C + c) =
        __builtin_bit_cast(u32x4v, __builtin_convertvector(acc, bf16x8v));
  }
}

}  // namespace h3attn
