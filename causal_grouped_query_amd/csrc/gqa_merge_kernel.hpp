// gqa_merge_kernel.hpp -- gfx950 kernel that combines split-KV partials of the causal
// GQA forward into O and LSE.
//
// The first fix direction of the h3.c issue "Qwen text encoder: sequence exceeds Metal
// threadgroup memory with reference video + ref images (>=150 frames)" ("Suggested fix
// directions") computes the score row in several dispatches with intermediate results
// in global memory.  Here the first dispatch (the split instance of the attention
// kernel) leaves, for every query row and every split of its KV range, the attention
// over that split's keys: O_c normalised over those keys and LSE_c their log-sum-exp.
// The softmax over the union of the splits weighs split c by exp(LSE_c) / sum exp(LSE_c'),
// so
//     LSE = m + log(sum_c exp(LSE_c - m)),   O = sum_c exp(LSE_c - LSE) * O_c,
// with m the largest LSE_c of the row.
//
// The work is a stream over the partials (HBM-bound, no data reuse): each (token, head)
// row is handled by D/4 lanes that read 16 bytes of every split's O_c each, in rows of
// consecutive memory, and write 8 bytes of bf16 O each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3attn {

struct MergeParams {
  const float* o_part;    // [num_splits, S, hq, D] fp32
  const float* lse_part;  // [num_splits, hq, S] fp32, -inf where a row saw no key
  uint16_t* o;            // [S, hq, D] bf16
  float* lse;             // [hq, S] fp32, or nullptr
  int seq_len;            // S
  int hq;
  int num_splits;
  int tok_wg;             // query tokens per block of the split kernel
  int bn;                 // keys per KV tile of the split kernel
};

constexpr int MERGE_THREADS = 256;

template <int D>
__global__ __launch_bounds__(MERGE_THREADS) void merge_splits_kernel(MergeParams p) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
  typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
  constexpr int LANES_ROW = D / 4;                    // lanes per (token, head) row
  constexpr int ROWS_BLOCK = MERGE_THREADS / LANES_ROW;
  constexpr float LOG2E = 1.4426950408889634f;
  constexpr float LN2_M = 0.693147180559945309417f;

  const long long row = (long long)blockIdx.x * ROWS_BLOCK + threadIdx.x / LANES_ROW;
  if (row >= (long long)p.seq_len * p.hq) return;     // no barrier in this kernel
  const int d0 = 4 * (threadIdx.x % LANES_ROW);
  const int token = (int)(row / p.hq);
  const int head = (int)(row % p.hq);

  // the splits that hold tiles of this token's query block (same ranges as the split
  // kernel: split_first_tile over the block's causal tile count)
  const int q0 = token / p.tok_wg * p.tok_wg;
  const int n = (min(q0 + p.tok_wg, p.seq_len) + p.bn - 1) / p.bn;
  const int ns = p.num_splits;

  auto holds_tiles = [&](int c) {
    return split_first_tile(n, c, ns) < split_first_tile(n, c + 1, ns);
  };
  float m = -__builtin_inff();
  int c_last = 0;                                     // a split with tiles (the last one)
  for (int c = 0; c < ns; ++c)
    if (holds_tiles(c)) {
      m = fmaxf(m, p.lse_part[((size_t)c * p.hq + head) * p.seq_len + token]);
      c_last = c;
    }

  // Four splits per step, all loads issued before any is used (memory-level parallelism).
  // A slot past num_splits or on a split without tiles reads the c_last split's data
  // (finite, in bounds) and gets weight 0.
  float wsum = 0.0f;
  f32x4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = 0; c0 < ns; c0 += 4) {
    f32x4v oc[4];
    float lc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u;
      const bool ok = c < ns && holds_tiles(c);
      const int cc = ok ? c : c_last;
      lc[u] = p.lse_part[((size_t)cc * p.hq + head) * p.seq_len + token];
      oc[u] = *(const f32x4v*)(p.o_part +
                               (((size_t)cc * p.seq_len + token) * p.hq + head) * D + d0);
      lc[u] = ok ? lc[u] : -__builtin_inff();
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = __builtin_amdgcn_exp2f((lc[u] - m) * LOG2E);   // 0 for -inf
      wsum += w;
      acc += w * oc[u];
    }
  }
  const float inv = 1.0f / wsum;
  const bf16x4v y = __builtin_convertvector(acc * inv, bf16x4v);
  *(u32x2v*)(p.o + ((size_t)token * p.hq + head) * D + d0) = __builtin_bit_cast(u32x2v, y);
  if (p.lse != nullptr && d0 == 0)
    p.lse[(size_t)head * p.seq_len + token] = m + __builtin_amdgcn_logf(wsum) * LN2_M;
}

}  // namespace h3attn
