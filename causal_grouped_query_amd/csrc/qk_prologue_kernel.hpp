// qk_prologue_kernel.hpp -- gfx950 kernel for the step before attention: per-head RMS
// norm of the Q and K rows and the rotary position embedding, in one pass over Q and K.
//
// The h3.c project README ("Checkpoint layout and media pipeline") runs a fused
// QK-normalization / RoPE kernel on the DiT's Q and K rows; its profiling notes fold the
// Q/K normalization and RoPE into the QKV projection.  The pages give no formulas; this
// kernel computes the Qwen-family convention:
//   y_d = x_d / sqrt(mean_d(x_d^2) + eps) * w_d                   (when a weight is given)
//   a_i = p * theta^(-2i/D),  i < D/2, p the token's position
//   z_i = y_i cos a_i - y_{i+D/2} sin a_i,  z_{i+D/2} = y_{i+D/2} cos a_i + y_i sin a_i
// in fp32 with one bf16 rounding at the end; the angles and their cos / sin are computed
// in fp64 (positions reach 10^4-10^5, where fp32 angles would lose ~10^-3 rad).
//
// HBM-bound streaming: one workgroup per TOKENS tokens.  Its threads first compute the
// cos / sin of every (token, pair) of the block into LDS (one fp64 sincos each), then
// each (token, head) row is handled by D/16 lanes; lane l holds the eight elements
// 8l..8l+7 and their rotation partners D/2+8l..D/2+8l+7 (two 16-byte loads), so the
// rotation needs no data exchange and only the row's sum of squares is reduced across
// the row's lanes (butterfly of D/16 lanes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3attn {

struct PrologueParams {
  const uint16_t* q;        // [S, hq, D] bf16
  const uint16_t* k;        // [S, hkv, D] bf16
  uint16_t* q_out;          // [S, hq, D] bf16 (may be q)
  uint16_t* k_out;          // [S, hkv, D] bf16 (may be k)
  const uint16_t* q_weight; // [D] bf16 or nullptr (no norm of Q)
  const uint16_t* k_weight; // [D] bf16 or nullptr (no norm of K)
  const int32_t* positions; // [S] or nullptr (position = token index)
  int seq_len, hq, hkv;
  float eps;
  double theta;
  int rope;                 // 0: no rotary embedding
};

constexpr int PROLOGUE_THREADS = 256;
constexpr int PROLOGUE_TOKENS = 8;

template <int D>
__global__ __launch_bounds__(PROLOGUE_THREADS) void qk_prologue_kernel(PrologueParams p) {
  typedef float f32x8v __attribute__((ext_vector_type(8)));
  typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
  typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
  constexpr int HALF = D / 2;
  constexpr int LANES_ROW = D / 16;                  // lanes per (token, head) row
  constexpr int ROWS_PASS = PROLOGUE_THREADS / LANES_ROW;
  __shared__ float cs[PROLOGUE_TOKENS][HALF][2];     // cos, sin per (token, pair)

  const int t0 = blockIdx.x * PROLOGUE_TOKENS;
  const int ntok = min(PROLOGUE_TOKENS, p.seq_len - t0);

  if (p.rope) {
    for (int e = threadIdx.x; e < PROLOGUE_TOKENS * HALF; e += PROLOGUE_THREADS) {
      const int tt = e / HALF, i = e % HALF;
      if (tt < ntok) {
        const int tok = t0 + tt;
        const double pos = p.positions ? (double)p.positions[tok] : (double)tok;
        const double a = pos * pow(p.theta, -2.0 * (double)i / (double)D);
        double sn, c;
        sincos(a, &sn, &c);
        cs[tt][i][0] = (float)c;
        cs[tt][i][1] = (float)sn;
      }
    }
    __syncthreads();
  }

  const int li = threadIdx.x % LANES_ROW;            // lane within the row
  const int rows_tok = p.hq + p.hkv;
  const int rows = ntok * rows_tok;
  // Each lane group handles RU rows per pass, all loads issued before any arithmetic
  // (memory-level parallelism).  Every lane of a row group runs the same iterations (rows
  // is uniform over the workgroup), so the butterflies below always have all their lanes.
  constexpr int RU = 4;
  for (int r0 = 0; r0 < rows; r0 += ROWS_PASS * RU) {
    f32x8v lo[RU], hi[RU];
    int rr[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int r = r0 + u * ROWS_PASS + threadIdx.x / LANES_ROW;
      rr[u] = r;
      lo[u] = f32x8v{};
      hi[u] = f32x8v{};
      if (r < rows) {
        const int tt = r / rows_tok, h = r % rows_tok, tok = t0 + tt;
        const uint16_t* src = h < p.hq ? p.q + ((size_t)tok * p.hq + h) * D
                                       : p.k + ((size_t)tok * p.hkv + (h - p.hq)) * D;
        lo[u] = __builtin_convertvector(
            __builtin_bit_cast(bf16x8v, *(const u32x4v*)(src + 8 * li)), f32x8v);
        hi[u] = __builtin_convertvector(
            __builtin_bit_cast(bf16x8v, *(const u32x4v*)(src + HALF + 8 * li)), f32x8v);
      }
    }
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const int r = rr[u];
      const bool live = r < rows;
      const int tt = live ? r / rows_tok : 0;
      const int h = live ? r % rows_tok : 0;
      const bool is_q = h < p.hq;
      const int tok = t0 + tt;
      const uint16_t* w = is_q ? p.q_weight : p.k_weight;
      if (w != nullptr) {   // uniform over a row group (depends on is_q only)
        float ss = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) ss += lo[u][t] * lo[u][t] + hi[u][t] * hi[u][t];
#pragma unroll
        for (int m = 1; m < LANES_ROW; m <<= 1) ss += __shfl_xor(ss, m, LANES_ROW);
        const float inv = 1.0f / __builtin_sqrtf(ss / (float)D + p.eps);
        if (live) {
          const f32x8v wl = __builtin_convertvector(
              __builtin_bit_cast(bf16x8v, *(const u32x4v*)(w + 8 * li)), f32x8v);
          const f32x8v wh = __builtin_convertvector(
              __builtin_bit_cast(bf16x8v, *(const u32x4v*)(w + HALF + 8 * li)), f32x8v);
          lo[u] = lo[u] * inv * wl;
          hi[u] = hi[u] * inv * wh;
        }
      }
      if (!live) continue;
      if (p.rope) {
        f32x8v zl, zh;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float c = cs[tt][8 * li + t][0], sn = cs[tt][8 * li + t][1];
          zl[t] = lo[u][t] * c - hi[u][t] * sn;
          zh[t] = hi[u][t] * c + lo[u][t] * sn;
        }
        lo[u] = zl;
        hi[u] = zh;
      }
      uint16_t* dst = is_q ? p.q_out + ((size_t)tok * p.hq + h) * D
                           : p.k_out + ((size_t)tok * p.hkv + (h - p.hq)) * D;
      *(u32x4v*)(dst + 8 * li) =
          __builtin_bit_cast(u32x4v, __builtin_convertvector(lo[u], bf16x8v));
      *(u32x4v*)(dst + HALF + 8 * li) =
          __builtin_bit_cast(u32x4v, __builtin_convertvector(hi[u], bf16x8v));
    }
  }
}

}  // namespace h3attn
