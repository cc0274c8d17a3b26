// gqa_fwd_wide_kernel.hpp -- the head-dim-128 attention forward with 64 query rows per
// wave.
//
// Same operation, layouts and work decode as gqa_causal_fwd_kernel (the tiled form of the
// causal GQA of the h3.c issue "Qwen text encoder: sequence exceeds Metal threadgroup memory
// with reference video + ref images (>=150 frames)", sections "Error" and "Suggested fix
// directions"); what changes is how a CU spends its cycles:
//
//  * One workgroup = 4 waves, one per SIMD, and each wave owns two blocks of 32 query rows
//    (64 rows).  Every K fragment and V^T fragment a wave reads from LDS is the A operand of
//    two MFMAs, one per row block, so LDS traffic per MFMA is half that of the 32-row
//    kernel.  On this part, which runs at its power limit under this load, the LDS read
//    energy saved turns into shader clock.  The accumulators of O live in AGPRs (a wave has
//    512 registers), the rest in VGPRs.
//
//  * Keys are walked in 32-key sub-tiles (two per 64-key LDS tile).  The phase of sub-tile
//    j is one instruction stream (tile_phases.inc) in which the softmax of sub-tile j
//    (exp2, bf16 weights, fp32 sums) issues between the score MFMAs of sub-tile j+1 and the
//    P.V MFMAs of sub-tile j-1, so the wave's own VALU work fills the gaps of its MFMAs.
//
//  * The running max of a row starts INIT_HEADROOM above its max over the first sub-tile;
//    later sub-tiles are exponentiated against it, and only when a lane's 16 weights of a
//    sub-tile sum past WIDE_WEIGHT_SUM_LIMIT (or are not finite) does the wave take the max
//    path (C++ after the phase): raise the max of the flagged rows (to MAX_HEADROOM above
//    the sub-tile's max), rescale their O and l, and redo the sub-tile's weights.  Every
//    decision depends on the row's own scores only.
//
//  * K/V tiles go global -> LDS by DMA into a 4-stage ring, each wave loading a quarter of
//    every tile, and the loads are issued from inside the phases, between MFMAs: the phase
//    of sub-tile 2t issues V of tile t+2, that of 2t+1 issues K of tile t+3.  One barrier
//    per 64-key tile: B_t follows the phase of 2t and waits for every load but the newest
//    eight (tile t+2's), so tile t+1 is whole in LDS for the phase of 2t+1; every load goes
//    into a stage whose last reader ran before the previous barrier.
//
//  * A wave whose rows end early runs the remaining phases as fill-only (the skip is a
//    scalar branch inside the phase's assembly, so both paths share one register
//    interface), and every wave leaves the tile loop through the same exit.
//
//  * Q comes in through LDS (ring stages 2 and 3, before tile 2 is requested) and O leaves
//    through an LDS stage (the K half of the ring), so that every Q load and O store
//    instruction moves whole 256-byte rows; both are non-temporal, leaving L2 to K/V.
#pragma once

#include "gqa_fwd_kernel.hpp"
#include "tile_phases.inc"

namespace h3attn {

template <int D_, int G_>
struct WideConfig {
  static constexpr int D = D_;
  static constexpr int G = G_;
  static constexpr int NW = 4;                 // waves per workgroup, one per SIMD
  static constexpr int RB = 2;                 // 32-row blocks per wave
  static constexpr int BN = 64;                // keys per LDS tile
  static constexpr int SUB = 32;               // keys per sub-tile (one phase)
  static constexpr int THREADS = 64 * NW;
  static constexpr int TOK_RB = 32 / G;        // tokens per row block
  static constexpr int TOK_W = RB * TOK_RB;    // tokens per wave
  static constexpr int TOK_WG = TOK_W * NW;    // tokens per workgroup (256 / G, as the 32-row kernel)
  static constexpr int TILE_ELEMS = BN * D;
  static constexpr int TILE_BYTES = TILE_ELEMS * 2;
  static constexpr int SUB_BYTES = SUB * D * 2;
  static constexpr int TILE_PIECES = TILE_BYTES / 1024;
  static constexpr int PIECES_PER_WAVE = TILE_PIECES / NW;
  static constexpr int STAGES = 4;             // K/V tiles resident in LDS
  static constexpr int LDS_BYTES = STAGES * 2 * TILE_BYTES;
  static constexpr int FILLS = 4;              // fill loads a wave issues per phase (half its tile share)
  static_assert(PIECES_PER_WAVE == FILLS, "a phase issues a wave's share of K (or of V) of one tile");
  static_assert(D == 128, "the generated phases are for head dim 128");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  static_assert(TILE_PIECES % NW == 0, "tile fill divides over waves");
};

// The lazy max in log2 units.  The max path is rare but costs a wave ~1000 cycles, and the
// other waves of the workgroup wait for it at the next barrier, so the running max is kept
// well above the scores seen: it starts INIT_HEADROOM above the first sub-tile's max, a
// raise puts it MAX_HEADROOM above the raising sub-tile's max, and a raise is needed only
// once a lane's 16 weights sum past WIDE_WEIGHT_SUM_LIMIT, i.e. once a key scores about
// 84 log2 units above the first sub-tile's max (68 after a raise).  Ranges: a weight is at
// most 2^40; one below 2^-126 (a key more than 78 log2 units under the row's largest
// score) may be flushed to zero, which moves O and l by less than 2^-78 relative; a lane's
// sum l stays below 2^40 per sub-tile, so below 2^53 over 2^13 sub-tiles (262144 keys), and
// O stays finite for |V| < 2^74.  Scaling every weight by a power of two changes neither
// O = acc / l nor LSE = m + log2 l.
constexpr float INIT_HEADROOM = 48.0f;
constexpr float MAX_HEADROOM = 32.0f;
constexpr float WIDE_WEIGHT_SUM_LIMIT = 1099511627776.0f;   // 2^40

// QPRO: the fixed-length causal forward with Q's per-head RMS norm and rotate-half RoPE
// applied to the Q fragments in the kernel (the call h3attn_gqa_causal_qnorm_rope_fwd); its
// LDS adds a cos/sin table of the workgroup's 256/G tokens (G = 4 and 8 fit beside the ring).
template <class C, bool VARLEN, bool CAUSAL, bool QPRO = false>
__global__ __launch_bounds__(C::THREADS, 1) void gqa_fwd_wide_kernel(FwdParams p, QproParams qp) {
  static_assert(!QPRO || (!VARLEN && CAUSAL), "the Q prologue instance is fixed-length causal");
  static_assert(!QPRO || C::LDS_BYTES + C::TOK_WG * (C::D / 2) * 8 <= 160 * 1024, "LDS");
  using namespace wide::d128;
  constexpr int D = C::D, G = C::G, BN = C::BN;
  constexpr int NDS = D / 16, NDB = D / 32;
  constexpr int TB = C::TILE_BYTES, SB = C::SUB_BYTES;

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[C::STAGES][C::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[C::STAGES][C::TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- work decode (as gqa_causal_fwd_kernel): KV head per XCD when the heads divide over
  // the 8 XCDs, query blocks heaviest first, sequences of a packed batch one after another
  int bid = blockIdx.x;
  int g;
  if (p.hkv % kXcds == 0) {
    const int per_head = (int)(gridDim.x / p.hkv);
    const int xcd = bid % kXcds;
    const int j = bid / kXcds;
    g = xcd + kXcds * (j / per_head);
    bid = j % per_head;
  } else {
    g = bid % p.hkv;
    bid /= p.hkv;
  }
  const int seq = bid / p.n_qblk;
  const int qblk = p.n_qblk - 1 - bid % p.n_qblk;
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
  if (q0 >= len) return;                                   // uniform over the workgroup
  const int n_tiles = ((CAUSAL ? min(q0 + C::TOK_WG, len) : len) + BN - 1) / BN;

  const int wq0 = q0 + wave * C::TOK_W;                    // first token of this wave
  const int w_last = (wq0 < len) ? min(wq0 + C::TOK_W, len) - 1 : -1;
  // last 32-key sub-tile this wave needs, -1 if none (wave-uniform)
  const int j_last = __builtin_amdgcn_readfirstlane(
      (w_last < 0) ? -1 : (CAUSAL ? w_last : len - 1) / C::SUB);
  int my_tok[2];
  bool my_valid[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    my_tok[r] = wq0 + r * C::TOK_RB + col / G;
    my_valid[r] = my_tok[r] < len;
  }
  const int my_head = g * G + col % G;

  // ---- Q prologue, part 1: cos / sin of every (token of the block, rotation pair) into LDS.
  // Thread t takes pair i = t mod D/2 and every (THREADS / (D/2))-th token.  theta^(-2i/D) is
  // the host's fp64 theta^(-2/D) raised to i by squaring; the angle pos * theta^(-2i/D) is
  // formed and reduced to [-pi, pi] in fp64 (positions reach 10^4-10^5 rad), then cos / sin
  // are taken in fp32.  Read after the prologue's barrier.
  [[maybe_unused]] float2* qcs = nullptr;
  if constexpr (QPRO) {
    constexpr int HALF = D / 2;
    __shared__ float2 qcs_lds[C::TOK_WG * HALF];
    qcs = qcs_lds;
    if (qp.rope) {
      const int i = tid % HALF;
      double inv_freq = 1.0, power = qp.inv_freq_step;
      for (int b = i; b != 0; b >>= 1) {
        if (b & 1) inv_freq *= power;
        power *= power;
      }
      for (int tt = tid / HALF; tt < C::TOK_WG; tt += C::THREADS / HALF) {
        const int tok = q0 + tt;
        float sn = 0.0f, cs = 1.0f;
        if (tok < len) {
          const double pos = qp.positions ? (double)qp.positions[start + tok] : (double)tok;
          const double a = pos * inv_freq;
          const double r = a - 6.283185307179586476925 * rint(a * 0.159154943091895335768883);
          sincosf((float)r, &sn, &cs);
        }
        qcs[tt * HALF + i] = make_float2(cs, sn);
      }
    }
  }

  // ---- Q^T fragments of both row blocks (B operands), resident for the whole kernel; loaded
  // through LDS in the prologue below
  bf16x8 qf[2][NDS];

  // ---- K/V fill: each lane one 16-byte chunk of each of its wave's 1 KB pieces; rows past
  // the sequence end read as zeros (outside the buffer range)
  const int kv_stride = p.hkv * D;
  const uint16_t* kg = p.k + (size_t)start * kv_stride + g * D;
  const uint16_t* vg = p.v + (size_t)start * kv_stride + g * D;
  unsigned fill_off[C::PIECES_PER_WAVE];
#pragma unroll
  for (int n = 0; n < C::PIECES_PER_WAVE; ++n) {
    const int byte = (n * C::NW + wave) * 1024 + 16 * lane;
    const int row = byte / (2 * D);
    const int phys = (byte % (2 * D)) / 16;
    fill_off[n] = (unsigned)(row * kv_stride * 2 + lds_chunk<D>(row, phys) * 16);
  }
  // In-loop fills (issued inside the phases) step from piece to piece by 16 rows: the swizzle
  // depends on the row only modulo 16, so piece n's offset is piece 0's plus n row steps.
  unsigned fo = fill_off[0];
  const unsigned fs = 16u * kv_stride * 2u;
  auto fill_tile = [&](int kt, uint16_t* kdst, uint16_t* vdst) __attribute__((always_inline)) {
    const int rows = min(len - kt * BN, BN);
    const size_t tile0 = (size_t)kt * BN * kv_stride;
    fill_tile_lds<C>(kg + tile0, vg + tile0, rows * kv_stride * 2, kdst, vdst, wave, fill_off);
  };
  // Buffer resource of tile f's K (or V) rows; a tile past the workgroup's last one gets an
  // empty range, so its loads read zeros and touch no memory (the LDS stage they land in is
  // no longer read).
  auto tile_rsrc = [&](int f, const uint16_t* base) __attribute__((always_inline)) {
    const int rows = __builtin_amdgcn_readfirstlane(f < n_tiles ? min(len - f * BN, BN) : 0);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)f * BN * kv_stride), 0,
                                             rows * kv_stride * 2, BUFFER_RSRC_WORD3);
  };

  // ---- LDS byte addresses of this lane's fragments in stage 0, sub-tile 0 (other stages and
  // sub-tiles are immediate offsets).  K fragment d-step ds: key col, logical chunk 2ds+half.
  // V^T fragment d-block db: two transposing reads (keys key0 + 8h, d = 32db + ...).
  const unsigned kbase = (unsigned)(uintptr_t)(lds_void*)&k_lds[0][0];
  const unsigned vbase = (unsigned)(uintptr_t)(lds_void*)&v_lds[0][0];
  unsigned ka[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) ka[ds] = kbase + 2 * (col * D + lds_chunk<D>(col, 2 * ds + half) * 8);
  unsigned va[NDB][2];
  {
    const int grp = lane >> 4;
    const int gi = lane & 15;
    const int key0 = 4 * (grp >> 1) + (gi >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + 16 * (grp & 1) + 4 * (gi & 3);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = key0 + 8 * h;
        va[db][h] = vbase + 2 * (key * D + lds_chunk<D>(key, d >> 3) * 8 + (d & 7));
      }
    }
  }

  // The phases' fragment buffers and softmax temporaries, v[228:255], held as live values
  // from here to the end so the compiler places nothing of its own there between phases
  // (a queued MFMA of an earlier phase may still read them).
  u32x4 fx[7];
  asm volatile("" : "={v[228:231]}"(fx[0]), "={v[232:235]}"(fx[1]), "={v[236:239]}"(fx[2]),
               "={v[240:243]}"(fx[3]), "={v[244:247]}"(fx[4]), "={v[248:251]}"(fx[5]),
               "={v[252:255]}"(fx[6]));
  // O^T accumulators: AGPRs, touched only through asm operands (tile_phases.inc)
  f32x16 acc[2][NDB];
  o_zero_0(acc);
  o_zero_1(acc);
  float m_run[2] = {0.0f, 0.0f};
  float l_run[2] = {0.0f, 0.0f};
  const float c = p.scale_log2;

  // score and weight buffers: sub-tile j's raw scores in s_[j & 1], its bf16 weights in
  // w_[j & 1]
  f32x16 s_[2][2];
  bf16x8 w_[2][2][2];

  // causal (or sequence-end) mask of sub-tile j's scores in s_[j & 1]
  auto mask = [&](f32x16 (&s)[2], int j) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int rb_first = wq0 + r * C::TOK_RB;
      const bool need = CAUSAL ? (j * C::SUB + C::SUB - 1 > rb_first) : (j * C::SUB + C::SUB > len);
      if (need) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = j * C::SUB + 8 * (e >> 2) + 4 * half + (e & 3);
          if (CAUSAL ? (key > my_tok[r]) : (key >= len)) s[r][e] = -__builtin_inff();
        }
      }
    }
  };

  // Rare path after a phase: rows whose lane weight sums passed the limit get a new max from
  // this sub-tile's scores, O and l rescaled, and the sub-tile's weights recomputed (the same
  // arithmetic and summation order as the phase, so rows not raised get identical values).
  auto max_path = [&](const f32x16 (&s)[2], bf16x8 (&w)[2][2], float (&ls)[2])
      __attribute__((always_inline)) {
    // the phase's last MFMAs (results in O) complete before any VALU reads
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint64_t flagged = __builtin_amdgcn_ballot_w64(!(ls[r] <= WIDE_WEIGHT_SUM_LIMIT));
      if (flagged == 0) continue;
      float mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[r][e]);
      mx = pair_max(mx);
      const bool raise = (((flagged >> col) | (flagged >> (col + 32))) & 1) != 0;
      // a raised max sits MAX_HEADROOM above the sub-tile's max
      const float m_new = raise ? fmaxf(m_run[r], mx * c + MAX_HEADROOM) : m_run[r];
      const float alpha = __builtin_amdgcn_exp2f(m_run[r] - m_new);
      l_run[r] *= alpha;
      if (r == 0)
        o_scale_0(acc, alpha, fx[0]);
      else
        o_scale_1(acc, alpha, fx[0]);
      m_run[r] = m_new;
      float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        f32x8 x;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          x[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r][8 * ks + t], c, -m_run[r]));
        w[r][ks] = __builtin_convertvector(x, bf16x8);
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          if (ks == 0 && t == 0) {
            l0 = x[0];
            l1 = x[1];
          } else {
            l0 += x[t];
            l1 += x[t + 1];
          }
        }
      }
      ls[r] = l0 + l1;
    }
  };

  // Phase of sub-tile j >= 1.  K of sub-tile j+1 sits at byte offset KOFF, V of sub-tile j-1
  // at VOFF (stage * tile + half * sub-tile); f is the tile this phase helps fill, FKV whether
  // it is that tile's V (else K), FST its stage.  For j <= j_last + 1 the whole phase runs:
  // at j = j_last its scores (of a sub-tile this wave does not need) are never read, and at
  // j = j_last + 1 only its P.V counts.  Past that the assembly branches to the fill loads
  // alone.  One register interface for every sub-tile keeps the compiler's allocation of the
  // operands stable.
  auto phase = [&](int j, auto parity, auto koff, auto voff, int f, auto fkv, auto fst)
      __attribute__((always_inline)) {
    constexpr int PAR = decltype(parity)::value;   // j & 1
    constexpr int KOFF = decltype(koff)::value, VOFF = decltype(voff)::value;
    constexpr int FKV = decltype(fkv)::value, FST = decltype(fst)::value;   // fill: K/V, stage
    f32x16 (&sc)[2] = s_[PAR];
    f32x16 (&sn)[2] = s_[PAR ^ 1];
    bf16x8 (&wp)[2][2] = w_[PAR ^ 1];   // weights of sub-tile j-1
    bf16x8 (&wn)[2][2] = w_[PAR];       // weights of sub-tile j
    const __amdgpu_buffer_rsrc_t fr = tile_rsrc(f, FKV ? vg : kg);
    // LDS addresses (M0 values) of this wave's pieces of the target stage
    const unsigned fm = (FKV ? vbase : kbase) + FST * TB + wave * 1024;
    // A wave past its last sub-tile (+1 for the last P.V) only issues its share of the fill;
    // the phase skips its computation inside the asm (one register interface either way).
    const bool live = j <= j_last;      // sub-tile j has keys this wave needs
    if (live) mask(sc, j);
    float lp[2][2];
    // odd j steps the fill offset up through the pieces, even j back down
    if constexpr (PAR == 1)
      phase_step_up<KOFF, VOFF>(acc, wp, va, qf, sn, ka, sc, c, m_run, wn, lp, fr, fm, fo, fs, j,
                                j_last + 1, fx);
    else
      phase_step_down<KOFF, VOFF>(acc, wp, va, qf, sn, ka, sc, c, m_run, wn, lp, fr, fm, fo, fs, j,
                                  j_last + 1, fx);
    if (live) {
      float ls[2] = {lp[0][0] + lp[0][1], lp[1][0] + lp[1][1]};
      if (__builtin_amdgcn_ballot_w64(!(ls[0] <= WIDE_WEIGHT_SUM_LIMIT) ||
                                      !(ls[1] <= WIDE_WEIGHT_SUM_LIMIT)) != 0)
        max_path(sc, wn, ls);
      l_run[0] += ls[0];
      l_run[1] += ls[1];
    }
  };

  // ---- prologue.  Q: the workgroup's 256 rows (token, head of the group) go global -> LDS by
  // DMA into the ring's stages 2 and 3 (free until tile 2 is requested): 16 lanes fetch one
  // whole 256-byte row, so every load instruction covers whole lines and can stream past the
  // caches (non-temporal).  (A lane's MFMA fragments are every other 16 bytes of its row; read
  // straight from global memory, one instruction touches 32 rows' lines 32 bytes each.)  Wave
  // w loads rows 64w .. 64w+63, its own, and reads them back as B fragments; LDS row R keeps
  // its 16-byte chunk c at position c ^ (R & 15), so the fragment reads spread over the banks.
  // Tokens past the sequence end lie outside the buffer range and load as zeros.
  uint16_t* const qstage = wave < 2 ? &k_lds[2][0] : &v_lds[2][0];   // 128 rows per region
  {
    const int ntok = min(len - q0, C::TOK_WG);           // >= 1: the block has a token
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.q + ((size_t)(start + q0) * p.hq + g * G) * D), 0,
        ((ntok - 1) * p.hq + G) * D * 2, BUFFER_RSRC_WORD3);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int row = 64 * wave + 4 * n + (lane >> 4);  // the workgroup's Q row
      const int pos = lane & 15;                        // LDS chunk this lane writes
      const unsigned off = (unsigned)(((row / G) * p.hq + row % G) * D * 2 + ((pos ^ (row & 15)) * 16));
      const unsigned m = __builtin_amdgcn_readfirstlane(
          (unsigned)(uintptr_t)(lds_void*)(qstage + (64 * (wave & 1) + 4 * n) * D));
      // as in fill_tile_lds: one wait state between the M0 write and the load
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                   :: "v"(off), "s"(qr), "s"(m) : "memory", "m0");
#pragma clang diagnostic pop
    }
  }
  // tiles 0 and 1 behind Q; every load the first phases need lands before the barrier.  The
  // wave reads back the rows its own loads wrote, so it needs only its own wait; the barrier
  // then also tells every wave that stages 2 and 3 are read, and tile 2 goes there (it is
  // first read after B_1, which waits for it).
  fill_tile(0, k_lds[0], v_lds[0]);
  if (1 < n_tiles) fill_tile(1, k_lds[1], v_lds[1]);
  // the wait as a compiler barrier too: the LDS reads below must not move above it
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int lrow = 64 * (wave & 1) + 32 * r + col;    // row in this wave's region
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      qf[r][ds] = *(const bf16x8*)(qstage + lrow * D + (((2 * ds + half) ^ (col & 15)) * 8));
  }
  __syncthreads();
  if (2 < n_tiles) fill_tile(2, k_lds[2], v_lds[2]);
  if constexpr (QPRO) {
    // Q prologue, part 2, on this lane's fragments of both row blocks: elements
    // 16*ds + 8*half + 0..7 of the row; element d and its rotation partner d + D/2 sit in
    // fragments ds and ds + NDS/2 of the same lane, and lanes l and l^32 hold the two halves
    // of one row (the norm's sum of squares is one swap across the pair).
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      f32x8 x[NDS];
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) x[ds] = __builtin_convertvector(qf[r][ds], f32x8);
      if (qp.q_weight != nullptr) {
        float ss = 0.0f;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
          for (int t = 0; t < 8; ++t) ss += x[ds][t] * x[ds][t];
        ss = pair_sum(ss);
        const float inv = 1.0f / __builtin_sqrtf(ss / (float)D + qp.q_eps);
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const f32x8 w = __builtin_convertvector(
              __builtin_bit_cast(bf16x8, *(const u32x4*)(qp.q_weight + 16 * ds + 8 * half)),
              f32x8);
          x[ds] = x[ds] * inv * w;
        }
      }
      if (qp.rope) {
        const float2* row = qcs + (wave * C::TOK_W + r * C::TOK_RB + col / G) * (D / 2);
#pragma unroll
        for (int ds = 0; ds < NDS / 2; ++ds)
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float2 cs = row[16 * ds + 8 * half + t];
            const float lo = x[ds][t], hi = x[ds + NDS / 2][t];
            x[ds][t] = lo * cs.x - hi * cs.y;
            x[ds + NDS / 2][t] = hi * cs.x + lo * cs.y;
          }
      }
      if (my_valid[r]) {
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) qf[r][ds] = __builtin_convertvector(x[ds], bf16x8);
      }
    }
  }
  if (0 <= j_last) {
    phase_scores<0, 0>(qf, s_[0], ka, fx);
    mask(s_[0], 0);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s_[0][r][e]);
      m_run[r] = pair_max(mx) * c + INIT_HEADROOM;   // key 0 is visible to every row: finite
    }
    float lp[2][2];
    phase_scores_softmax<SB, 0>(qf, s_[1], ka, s_[0], c, m_run, w_[0], lp, fx);
    l_run[0] = lp[0][0] + lp[0][1];
    l_run[1] = lp[1][0] + lp[1][1];
  }

  // ---- tile loop, unrolled by LDS stage so every fragment offset is an immediate.  Tile t
  // lives in stage t % 4.  The phase of sub-tile 2t+1 issues this wave's share of tile t+3's
  // K, the phase of 2t+2 its share of V, into the stage of tile t-1 (free after B_t); B_t
  // waits for all but the 8 newest loads (those of tile t+2), i.e. for tile t+1.
  auto tile_step = [&](int t, auto stage) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    constexpr int SP = (ST + 3) % 4, SN = (ST + 1) % 4;   // stages of tiles t-1 and t+1
    using I = std::integral_constant<int, 0>;
    if (t > 0) {
      // sub-tile 2t: K of 2t+1 (tile t, upper half), V of 2t-1 (tile t-1, upper half);
      // issues V of tile t+2 into stage (ST + 2) % 4, tile t-2's, last read before B_{t-1}
      phase(2 * t, std::integral_constant<int, 0>{}, std::integral_constant<int, ST * TB + SB>{},
            std::integral_constant<int, SP * TB + SB>{}, t + 2, std::integral_constant<int, 1>{},
            std::integral_constant<int, (ST + 2) % 4>{});
      static_assert(2 * C::FILLS <= 15, "vmcnt field");
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * C::FILLS));   // all but tile t+2's loads
      __syncthreads();    // every wave's share of tile t+1 landed; tile t-1 no longer read
    }
    // sub-tile 2t+1: K of 2t+2 (tile t+1, lower half), V of 2t (tile t, lower half); fills K
    // of tile t+3 into stage SP
    phase(2 * t + 1, std::integral_constant<int, 1>{}, std::integral_constant<int, SN * TB>{},
          std::integral_constant<int, ST * TB>{}, t + 3, I{}, std::integral_constant<int, SP>{});
  };
  // Tile steps 0 .. n_tiles: step n_tiles has no tile of its own; its first phase does the
  // last P.V of a wave whose last sub-tile is the workgroup's last one (a wave that finished
  // earlier, and the second phase, only issue their empty fills).  Every exit leaves the
  // loop in the same state, so there is one epilogue.
  for (int t = 0;; t += 4) {
    tile_step(t, std::integral_constant<int, 0>{});
    if (t + 1 > n_tiles) break;
    tile_step(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 > n_tiles) break;
    tile_step(t + 2, std::integral_constant<int, 2>{});
    if (t + 3 > n_tiles) break;
    tile_step(t + 3, std::integral_constant<int, 3>{});
    if (t + 4 > n_tiles) break;
  }

  // ---- epilogue: O = acc / l (bf16), LSE = (m + log2 l) * ln 2
  // the last P.V MFMAs complete (and have read their operands) before VALU reads of O and
  // before the fixed registers are released
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15"
               : "+{v[228:231]}"(fx[0]), "+{v[232:235]}"(fx[1]), "+{v[236:239]}"(fx[2]),
                 "+{v[240:243]}"(fx[3]), "+{v[244:247]}"(fx[4]), "+{v[248:251]}"(fx[5]),
                 "+{v[252:255]}"(fx[6])
               :
               : "memory");
  // O goes out through LDS so that every store instruction writes whole 256-byte rows.  The
  // K half of the ring (64 KB, no longer read once every wave has passed this barrier) holds
  // a [256 rows][128] bf16 stage, wave w owning rows 64w .. 64w+63; the 16-byte chunk c of
  // row r sits at chunk c ^ (r & 15), so both the row-wise writes and the chunk-wise reads
  // below spread over all LDS banks.  The last phases issued fill loads of tiles past the
  // workgroup's last one (zeros) into K stages; every wave waits for its own before the
  // barrier, so none can land in the stage after O is written there.
  wait_vmem();
  __syncthreads();
  uint8_t* const ostage = reinterpret_cast<uint8_t*>(&k_lds[0][0]) + wave * 64 * 256;
  float l_tot[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    l_tot[r] = pair_sum(l_run[r]);
    const float inv = 1.0f / l_tot[r];
    const int row = 32 * r + col;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x16 ov = o_read(acc[r][db]);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = ov[4 * r4 + e] * inv;
        const bf16x4 y = __builtin_convertvector(x, bf16x4);
        const int chunk = (4 * db + r4) ^ (row & 15);    // d = 32 db + 8 r4 + 4 half + e
        *(u32x2*)(ostage + row * 256 + chunk * 16 + 8 * half) = __builtin_bit_cast(u32x2, y);
      }
    }
  }
  // each lane stores 16 bytes (8 elements, chunk c) of one row; 4 rows per instruction.
  // Non-temporal: O is written once and not read again here.
  {
    const int c = lane & 15;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 4 * i + (lane >> 4);
      const u32x4 val = *(const u32x4*)(ostage + row * 256 + ((c ^ (row & 15)) * 16));
      const int rcol = row & 31;
      const int tok = wq0 + (row >> 5) * C::TOK_RB + rcol / G;
      if (tok < len) {
        const int head = g * G + rcol % G;
        uint16_t* op = p.o + (p.o_head_major ? ((size_t)head * p.total_tokens + start + tok) * D
                                             : ((size_t)(start + tok) * p.hq + head) * D);
        __builtin_nontemporal_store(val, (u32x4*)(op + 8 * c));
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (p.lse != nullptr && half == 0 && my_valid[r])
      p.lse[(size_t)my_head * p.total_tokens + start + my_tok[r]] =
          (m_run[r] + __builtin_amdgcn_logf(l_tot[r])) * LN2;
  }
}

// Host side: one workgroup per (query block, KV head, sequence).  Returns the launch's HIP
// error; hipSuccess without a launch for an empty grid, hipErrorInvalidConfiguration when the
// grid would not fit the 32-bit x dimension.
template <int G, bool VARLEN, bool CAUSAL, bool QPRO = false>
inline hipError_t launch_gqa_fwd_wide(FwdParams p, hipStream_t stream,
                                      const QproParams& qp = QproParams{}) {
  using C = WideConfig<128, G>;
  p.n_qblk = (p.seq_len + C::TOK_WG - 1) / C::TOK_WG;
  const long long blocks = (long long)p.n_qblk * p.hkv * p.num_seqs;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((gqa_fwd_wide_kernel<C, VARLEN, CAUSAL, QPRO>), dim3((unsigned)blocks),
                     dim3(C::THREADS), 0, stream, p, qp);
  return hipGetLastError();
}

}  // namespace h3attn
