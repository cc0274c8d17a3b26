// gqa_fwd_kernel.hpp -- gfx950 kernel for the bf16 causal grouped-query
// attention forward.
//
// Operation: the text encoder's causal GQA of the h3.c issue "Qwen text
// encoder: sequence exceeds Metal threadgroup memory with reference video +
// ref images (>=150 frames)" (section "Error").  That kernel kept the whole
// causal score row in 32 KB of threadgroup memory and failed past ~7700
// tokens; the issue proposes tiling the scores so on-chip memory holds one
// tile ("Suggested fix directions").  This kernel tiles the keys and keeps a
// running softmax (max and sum per query row, in registers), so the LDS
// footprint is a fixed number of K/V tiles whatever the sequence length, and
// everything runs in one launch without intermediates in global memory.
//
// Mapping onto CDNA4 (gfx950, wave64, 32x32x16 bf16 MFMA):
//
//  * One workgroup = NW waves = one KV head g and a block of TOK_WG
//    consecutive query tokens.  Its 32*NW "query rows" are (token, head)
//    pairs with the G heads of the group adjacent, so all rows of the
//    workgroup read the same K/V: each K/V tile is fetched into LDS once and
//    serves G heads.  Each wave owns 32 rows = 32/G tokens x G heads.
//
//  * Scores are computed transposed, S^T = K * Q^T (keys = MFMA rows, query
//    rows = MFMA columns).  Q^T stays in VGPRs for the whole kernel (the B
//    operand); K comes from LDS (the A operand, 16-byte reads).  The fp32
//    accumulator then holds, per lane, 16 keys of ONE query row, which is
//    exactly the register layout the B operand of O^T = V^T * P^T needs: P
//    goes from the score accumulator to the next MFMA with a bf16 convert
//    and no data movement.  The contraction order over keys inside an MFMA
//    is permuted to match (any consistent permutation of a sum is the sum).
//
//  * V^T fragments are read from a [key][d] LDS tile with the gfx950
//    transposing LDS read (ds_read_b64_tr_b16): 16 lanes read a 4-key x
//    16-d block and each lane receives 4 keys of one d.  K and V therefore
//    share one LDS layout and one fill path.
//
//  * LDS rows are swizzled at 16-byte granularity (chunk ^ f(key)) so the
//    K reads (8 keys, one chunk) and the transposing V reads (4 keys, two
//    chunks) hit distinct banks.
//
//  * Online softmax in the log2 domain (exp2 with scale*log2(e) folded in).
//    The row max is reduced inside the lane (16 keys per key block) and then
//    across the lane pair (l, l^32) with v_permlane32_swap.  The running max
//    is only raised when a row's new max exceeds it by more than
//    RESCALE_SLACK (in log2 units); otherwise the stale max is kept, the
//    weights stay <= 2^RESCALE_SLACK and the O accumulator is not rescaled.
//    The final O = acc / l and LSE use the same max, so the result is the
//    same function; only rounding differs.
//
//  * Causality: KV tiles past the workgroup's last token are never loaded;
//    only tiles that reach past a wave's first token apply the elementwise
//    mask (key > token -> -inf).  Keys past the sequence end are zero-filled
//    in LDS so no row ever reads memory outside its sequence.
//
//  * Two wave groups per workgroup, offset by half a tile.  Waves w and
//    w + NW/2 run on the same SIMD.  Between two barriers, group 0 does the
//    scores, softmax and P.V of tile t; group 1 does the softmax and P.V of
//    tile t-1 and then the scores of tile t.  While one wave of a SIMD issues
//    MFMAs the other issues softmax VALU work, instead of both waves hitting
//    the MFMA pipe and then the VALU together.  The next tile's global loads
//    are issued at the start of the interval and written to LDS at its end;
//    one barrier per tile.  K tiles are double-buffered and V tiles
//    triple-buffered, since group 1 reads a V tile one interval after group 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Kernel arguments (one struct, passed by value).
struct FwdParams {
  const uint16_t* q;           // [T, hq, D]  bf16
  const uint16_t* k;           // [T, hkv, D] bf16
  const uint16_t* v;           // [T, hkv, D] bf16
  uint16_t* o;                 // [T, hq, D]  bf16
  float* lse;                  // [hq, T] fp32, or nullptr
  const int32_t* cu_seqlens;   // [num_seqs + 1] device offsets (packed batches only)
  int seq_len;                 // S (fixed length) or max_seqlen (packed)
  int total_tokens;            // T: rows of the packed tensors, LSE row stride
  int num_seqs;                // 1 for the fixed-length call
  int n_qblk;                  // query blocks per sequence = ceil(seq_len / TOK_WG)
  int hq, hkv;
  float scale_log2;            // softmax_scale * log2(e)
};

// The running max is raised only when a row's tile max exceeds it by more
// than this many log2 units (a factor 2^8 = 256 of headroom in the weights).
constexpr float RESCALE_SLACK = 8.0f;
constexpr float LN2 = 0.693147180559945309417f;

template <int D_, int G_, int NW_, int BN_>
struct FwdConfig {
  static constexpr int D = D_;                 // head dim
  static constexpr int G = G_;                 // query heads per KV head
  static constexpr int NW = NW_;               // waves per workgroup
  static constexpr int BN = BN_;               // keys per KV tile
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROWS_W = 32;            // query rows per wave (one MFMA column block)
  static constexpr int TOK_W = ROWS_W / G;     // tokens per wave
  static constexpr int TOK_WG = TOK_W * NW;    // tokens per workgroup
  static constexpr int CHUNKS_ROW = D / 8;     // 16-byte chunks in one K/V row
  static constexpr int TILE_ELEMS = BN * D;    // bf16 elements of one K (or V) tile
  static constexpr int CHUNKS_PER_THREAD = BN * CHUNKS_ROW / THREADS;
  static constexpr int K_STAGES = 2;
  static constexpr int V_STAGES = 3;
  static constexpr int LDS_BYTES = (K_STAGES + V_STAGES) * TILE_ELEMS * 2;
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  static_assert(BN % 32 == 0, "KV tile is a whole number of 32-key MFMA blocks");
  static_assert(NW % 2 == 0, "two wave groups");
  static_assert((BN * CHUNKS_ROW) % THREADS == 0, "tile fill divides evenly over threads");
};

// Physical 16-byte chunk of logical chunk `chunk` in LDS row `key`.  For 8
// consecutive keys the XOR term takes 8 distinct values (conflict-free
// 16-byte reads of one chunk down 8 keys); for 4 consecutive keys starting at
// a multiple of 4 it takes 4 values spaced by 2 (conflict-free transposing
// reads of two adjacent chunks down 4 keys).
__device__ __forceinline__ int lds_chunk(int key, int chunk) {
  return chunk ^ (((key & 3) << 1) | ((key >> 2) & 1));
}

__device__ __forceinline__ float pair_max(float x) {
  // lanes l and l^32 hold the same query row; v_permlane32_swap returns both halves
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <class C, bool VARLEN>
__global__ __launch_bounds__(C::THREADS, 1) void gqa_causal_fwd_kernel(FwdParams p) {
  constexpr int D = C::D, G = C::G, BN = C::BN;
  constexpr int NKB = BN / 32;   // 32-key blocks per tile
  constexpr int NDS = D / 16;    // 16-wide d steps of the score contraction
  constexpr int NDB = D / 32;    // 32-row d blocks of O^T
  constexpr int NKS = BN / 16;   // 16-key steps of the P.V contraction

  // K tiles double-buffered, V tiles triple-buffered (the lagging wave group reads a V tile
  // one barrier interval after the leading group), all [key][d] with swizzled chunks.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[C::K_STAGES][C::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[C::V_STAGES][C::TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Waves w and w + NW/2 share a SIMD.  Group 0 (the first half) runs each tile as
  // scores -> softmax -> P.V inside one barrier interval; group 1 runs the softmax and P.V
  // of the previous tile first and the scores of the current tile last, so on every SIMD
  // one wave's MFMA work overlaps the other wave's softmax (VALU) work.
  const int group = wave / (C::NW / 2);
  const int half = lane >> 5;    // which 8-wide slice of a 16-wide contraction step
  const int col = lane & 31;     // MFMA column = this lane's query row within the wave

  // ---- work decode: KV head fastest (consecutive workgroups go to consecutive XCDs, so
  // with 8 KV heads each XCD serves one head and keeps its K/V in its own L2), then
  // sequence, then query block from the heaviest (last) one down.
  int bid = blockIdx.x;
  const int g = bid % p.hkv;
  bid /= p.hkv;
  const int seq = bid % p.num_seqs;
  bid /= p.num_seqs;
  const int qblk = p.n_qblk - 1 - bid;

  int start = 0, len = p.seq_len;
  if (VARLEN) {
    int a = p.cu_seqlens[seq];
    int b = p.cu_seqlens[seq + 1];
    a = min(max(a, 0), p.total_tokens);
    b = min(max(b, a), p.total_tokens);
    start = a;
    len = min(b - a, p.seq_len);
  }
  const int q0 = qblk * C::TOK_WG;
  if (q0 >= len) return;                              // uniform over the workgroup
  const int n_tiles = (min(q0 + C::TOK_WG, len) + BN - 1) / BN;

  const int wq0 = q0 + wave * C::TOK_W;               // first token of this wave
  const int w_last = (wq0 < len) ? min(wq0 + C::TOK_W, len) - 1 : -1;
  const int my_tok = wq0 + col / G;                   // this lane's query token
  const int my_head = g * G + col % G;                // and query head
  const bool my_valid = my_tok < len;

  // ---- Q^T fragments (B operand), resident for the whole kernel
  bf16x8 qf[NDS];
  if (my_valid) {
    const uint16_t* qp = p.q + ((size_t)(start + my_tok) * p.hq + my_head) * D + 8 * half;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      qf[ds] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qp + 16 * ds));
  } else {
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
  float m_run = -1e30f;   // running max (log2 units, scaled); finite so exp2(m_run - x) = 0
  float l_run = 0.0f;     // this lane's partial row sum (its 16 keys per block)
  f32x16 s[NKB];          // scores of the tile between its Q.K^T and its softmax

  // ---- K/V tile fill: each thread moves CHUNKS_PER_THREAD 16-byte chunks of K and of V
  const int kv_stride = p.hkv * D;
  const uint16_t* kg = p.k + (size_t)start * kv_stride + g * D;
  const uint16_t* vg = p.v + (size_t)start * kv_stride + g * D;
  u32x4 kreg[C::CHUNKS_PER_THREAD], vreg[C::CHUNKS_PER_THREAD];

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::CHUNKS_PER_THREAD; ++i) {
      const int id = i * C::THREADS + tid;
      const int key = id / C::CHUNKS_ROW;
      const int chunk = id % C::CHUNKS_ROW;
      const int j = kt * BN + key;
      if (j < len) {
        kreg[i] = *(const u32x4*)(kg + j * kv_stride + chunk * 8);
        vreg[i] = *(const u32x4*)(vg + j * kv_stride + chunk * 8);
      } else {
        kreg[i] = u32x4{0, 0, 0, 0};
        vreg[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](uint16_t* kdst, uint16_t* vdst) {
#pragma unroll
    for (int i = 0; i < C::CHUNKS_PER_THREAD; ++i) {
      const int id = i * C::THREADS + tid;
      const int key = id / C::CHUNKS_ROW;
      const int chunk = id % C::CHUNKS_ROW;
      const int off = key * D + lds_chunk(key, chunk) * 8;
      *(u32x4*)&kdst[off] = kreg[i];
      *(u32x4*)&vdst[off] = vreg[i];
    }
  };

  // V^T fragment (transposing read): within each 16-lane group, source lane i reads
  // key kbase + i/4, d = dbase + 4*(i%4) .. +3
  const int grp = lane >> 4;           // 16-lane group
  const int gi = lane & 15;
  const int v_key_in_quad = gi >> 2;   // which of the 4 keys this lane reads
  const int v_d_in_blk = 4 * (gi & 3); // d offset inside the 16-wide block
  const int v_dgrp = 16 * (grp & 1);   // lanes 0-15/32-47 cover d 0-15 of a 32-block, others 16-31
  const int v_ghalf = grp >> 1;        // lanes 32-63 take the second 4-key quads

  // S^T = K Q^T for tile kt (K tile in `ks_lds`)
  auto scores = [&](const uint16_t* ks_lds) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
      const int key = 32 * kb + col;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *(const u32x4*)(ks_lds + key * D + lds_chunk(key, 2 * ds + half) * 8));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], s[kb], 0, 0, 0);
      }
    }
  };

  // mask, online softmax and O^T += V^T P^T for tile kt (V tile in `vs_lds`)
  auto softmax_pv = [&](int kt, const uint16_t* vs_lds) {
    if (kt * BN + BN - 1 > wq0) {   // the tile reaches past the wave's first token
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kt * BN + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (j > my_tok) s[kb][r] = -__builtin_inff();
        }
    }

    // row max over the tile: 16 keys per block in-lane, then the lane pair
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = pair_max(mx);
    const float mx2 = mx * p.scale_log2;

    if (__builtin_amdgcn_ballot_w64(mx2 > m_run + RESCALE_SLACK) != 0) {
      const float m_new = fmaxf(m_run, mx2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m_run = m_new;
    }

    // P = exp2(S * scale*log2e - m) as bf16: the B operand of P.V
    bf16x8 pf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      f32x8 e;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        e[t] = __builtin_amdgcn_exp2f(
            __builtin_fmaf(s[ks >> 1][8 * (ks & 1) + t], p.scale_log2, -m_run));
        l_run += e[t];
      }
      pf[ks] = __builtin_convertvector(e, bf16x8);
    }

#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kq0 = 16 * ks + 4 * v_ghalf + v_key_in_quad;   // key read for slots 0..3
      const int kq1 = kq0 + 8;                                 // and for slots 4..7
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + v_dgrp + v_d_in_blk;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vs_lds + kq0 * D + lds_chunk(kq0, d >> 3) * 8 + (d & 7)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vs_lds + kq1 * D + lds_chunk(kq1, d >> 3) * 8 + (d & 7)));
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], acc[db], 0, 0, 0);
      }
    }
  };

  load_tile(0);
  store_tile(k_lds[0], v_lds[0]);
  __syncthreads();

  int ks_cur = 0, vs_cur = 0, vs_prev = C::V_STAGES - 1;
  for (int kt = 0; kt < n_tiles; ++kt) {
    const bool more = kt + 1 < n_tiles;
    if (more) load_tile(kt + 1);

    if (group == 0) {
      if (kt * BN <= w_last) {
        scores(k_lds[ks_cur]);
        softmax_pv(kt, v_lds[vs_cur]);
      }
    } else {
      if (kt > 0 && (kt - 1) * BN <= w_last) softmax_pv(kt - 1, v_lds[vs_prev]);
      if (kt * BN <= w_last) scores(k_lds[ks_cur]);
    }

    const int ks_next = ks_cur ^ 1;
    const int vs_next = (vs_cur + 1 == C::V_STAGES) ? 0 : vs_cur + 1;
    if (more) store_tile(k_lds[ks_next], v_lds[vs_next]);
    __syncthreads();
    ks_cur = ks_next;
    vs_prev = vs_cur;
    vs_cur = vs_next;
  }
  if (group == 1 && (n_tiles - 1) * BN <= w_last) softmax_pv(n_tiles - 1, v_lds[vs_prev]);

  // ---- epilogue: O = acc / l (bf16), LSE = (m + log2 l) * ln 2
  const float l_tot = pair_sum(l_run);
  if (my_valid) {
    const float inv = 1.0f / l_tot;
    uint16_t* op = p.o + ((size_t)(start + my_tok) * p.hq + my_head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 x;
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = acc[db][4 * r4 + t] * inv;
        const bf16x4 y = __builtin_convertvector(x, bf16x4);
        *(u32x2*)(op + 32 * db + 8 * r4 + 4 * half) = __builtin_bit_cast(u32x2, y);
      }
    if (p.lse != nullptr && half == 0)
      p.lse[(size_t)my_head * p.total_tokens + start + my_tok] =
          (m_run + __builtin_amdgcn_logf(l_tot)) * LN2;
  }
}

}  // namespace h3attn
