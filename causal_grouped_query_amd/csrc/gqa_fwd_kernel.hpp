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
//    K reads (16 keys, one chunk) and the transposing V reads (4 keys, four
//    chunks) hit distinct banks.
//
//  * Online softmax in the log2 domain (exp2 with scale*log2(e) folded in).
//    The running max of a row is its max over the first KV tile; later
//    tiles are exponentiated against it without computing their max.  Each
//    lane sums its fp32 weights of the tile; only when a lane's tile sum
//    exceeds WEIGHT_SUM_LIMIT (or is not finite) does the wave reduce the row
//    maxima (in-lane, then across the lane pair (l, l^32) with
//    v_permlane32_swap), raise the running max of the rows of the flagged
//    lane pairs, rescale their O and l, and redo the tile's exponentials.  A
//    row's decisions depend on its own scores only.
//    The final O = acc / l and LSE use the same max, so the result is the
//    same function whatever the max; only rounding differs.
//
//  * The same kernel also runs without the causal mask (the DiT's attention on
//    the vpipe page and in the h3.c project README): every block then walks
//    all KV tiles and only keys past the sequence end are masked.
//
//  * Causality: KV tiles past the workgroup's last token are never loaded;
//    only tiles that reach past a wave's first token apply the elementwise
//    mask (key > token -> -inf).  Keys past the sequence end are zero-filled
//    in LDS so no row ever reads memory outside its sequence.
//
//  * K/V tiles go to LDS through buffer loads that write LDS directly, into a
//    ring of three stages, two tiles ahead of the scores that read them; one
//    barrier per tile.  The two waves that share a SIMD run the same cycle
//    (softmax -> P.V -> next scores) with their barriers at different points
//    of it, so while one issues MFMAs the other runs its softmax on the VALU.
//
//  * LDS reads are software-pipelined: K fragments are read four MFMAs ahead
//    of use and the first V^T fragments are read before the softmax, so LDS
//    latency hides behind MFMA and VALU work (instruction order pinned with
//    sched_group_barrier).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
typedef __attribute__((address_space(3))) void lds_void;

// Word 3 of a raw buffer resource (no stride swizzle, 32-bit data format) for gfx9-family
// GPUs; loads past num_records return zeros.
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;

// s_waitcnt vmcnt(0): wait until this wave's vector-memory loads, including loads that
// write LDS directly, have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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
  // split-KV partials (split instances only)
  float* o_part;               // [num_splits, T, hq, D] fp32, each normalised over its keys
  float* lse_part;             // [num_splits, hq, T] fp32, -inf where a row has no key
  int num_splits;
  int o_head_major;            // 0: o is [T, hq, D]; 1: o is [hq, T, D]
};

// First KV tile of split `s` of a query block with `n` tiles in `ns` splits: split s
// covers tiles [split_first_tile(n, s, ns), split_first_tile(n, s + 1, ns)), contiguous
// ranges of near-equal length (empty when ns > n).
__host__ __device__ __forceinline__ int split_first_tile(int n, int s, int ns) {
  return (int)(((long long)n * s) / ns);
}

// A lane whose weights over one KV tile (32 keys of its row, each exp2 of the
// score minus the running max) sum to more than this sends its row through
// the max-and-rescale path.  Every weight is then at most 2^16, far inside the
// fp32 / bf16 range, and O and l accumulate without overflow.
constexpr float WEIGHT_SUM_LIMIT = 65536.0f;
constexpr float LN2 = 0.693147180559945309417f;
constexpr int kXcds = 8;   // accelerator complex dies of an MI355X; workgroup i runs on die i % 8

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
  static constexpr int TILE_PIECES = TILE_ELEMS * 2 / 1024;   // 1 KB pieces of one tile
  static constexpr int PIECES_PER_WAVE = TILE_PIECES / NW;
  static constexpr int STAGES = 3;             // K/V tiles resident in LDS
  static constexpr int LDS_BYTES = STAGES * 2 /*K and V*/ * TILE_ELEMS * 2;
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  static_assert(BN % 32 == 0, "KV tile is a whole number of 32-key MFMA blocks");
  static_assert(TILE_PIECES % NW == 0 && PIECES_PER_WAVE >= 1, "tile fill divides over waves");
};

// The instance the library launches for head dim D and group size G: 8 waves per
// workgroup (2 per SIMD, one workgroup per CU), 64 keys per KV tile.
template <int D, int G>
using LaunchConfig = FwdConfig<D, G, 8, 64>;

// Physical 16-byte chunk of logical chunk `chunk` in LDS row `key` (the gfx950 LDS has
// 64 four-byte banks: one 256-byte bank row).  The XOR term is chosen so that
//   * 16-byte reads of one logical chunk down 16 consecutive keys (the K operand: 16
//     lanes per LDS cycle) hit 16 distinct bank quads, and
//   * transposing 8-byte reads of 4 adjacent chunks down 4 consecutive keys (the V^T
//     operand: 32 lanes per LDS cycle) hit 16 distinct bank quads.
// For D = 128 a row is one bank row, so keys k and k+1 must land in different 4-chunk
// groups (bits 2-3 of the term come from key bits 0-1).  For D = 64 two rows share a
// bank row (key parity picks the half), so the term uses key bits 1-3.
template <int D>
__device__ __forceinline__ int lds_chunk(int key, int chunk) {
  if constexpr (D == 128)
    return chunk ^ (((key & 3) << 2) | ((key >> 2) & 3));
  else
    return chunk ^ (((key & 2) << 1) | ((key >> 2) & 3));
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

// Issue one wave's share of a K/V tile fill: PIECES_PER_WAVE 1 KB pieces of K and of V,
// each lane one 16-byte chunk at byte offset fill_off[n] of the tile, written to LDS at
// byte 16*lane of the piece.  Bytes at or past `nbytes` (rows beyond the sequence) read 0.
template <class C>
__device__ __forceinline__ void fill_tile_lds(const uint16_t* ksrc, const uint16_t* vsrc,
                                              int nbytes, uint16_t* kdst, uint16_t* vdst,
                                              int wave, const unsigned* fill_off) {
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)ksrc, 0, nbytes, BUFFER_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc((void*)vsrc, 0, nbytes, BUFFER_RSRC_WORD3);
#pragma unroll
  for (int n = 0; n < C::PIECES_PER_WAVE; ++n) {
    const int piece = (n * C::NW + wave) * 512;       // elements
    const unsigned kl = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_void*)(kdst + piece));
    const unsigned vl = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_void*)(vdst + piece));
    // Issued as inline assembly so that the compiler does not track these LDS writes: it
    // would otherwise wait for them before unrelated LDS reads of other stages.  The
    // kernel orders them itself (wait_vmem, then a workgroup barrier, before any read).
    // The s_nop covers the one wait state between an SALU write of M0 and its use as the
    // LDS address of a buffer load.  M0 is a register the compiler reserves; clang warns
    // that a clobbered reserved register may not be preserved.  Nothing else in these
    // kernels keeps a value in M0: tests/test_abi.py checks the built code object for any
    // other M0 access, so the warning is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(fill_off[n]), "s"(kr), "s"(kl) : "memory", "m0");
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(fill_off[n]), "s"(vr), "s"(vl) : "memory", "m0");
#pragma clang diagnostic pop
  }
}

// VARLEN: packed batch (cu_seqlens).  SPLIT: split-KV partials -- the workgroups of a
// query block each take one contiguous range of its KV tiles and write O and LSE over
// those keys to o_part / lse_part, for the merge kernel to combine.  CAUSAL = false: the
// bidirectional form, every query sees all keys of its sequence (only keys past the end
// of the sequence are masked).
template <class C, bool VARLEN, bool SPLIT = false, bool CAUSAL = true>
__global__ __launch_bounds__(C::THREADS, 1) void gqa_causal_fwd_kernel(FwdParams p) {
  constexpr int D = C::D, G = C::G, BN = C::BN;
  constexpr int NKB = BN / 32;   // 32-key blocks per tile
  constexpr int NDS = D / 16;    // 16-wide d steps of the score contraction
  constexpr int NDB = D / 32;    // 32-row d blocks of O^T
  constexpr int NKS = BN / 16;   // 16-key steps of the P.V contraction

  // K and V tiles, a ring of STAGES, [key][d] with swizzled 16-byte chunks
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[C::STAGES][C::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[C::STAGES][C::TILE_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;    // which 8-wide slice of a 16-wide contraction step
  const int col = lane & 31;     // MFMA column = this lane's query row within the wave

  // ---- work decode.  Consecutive workgroups go to consecutive XCDs (8 of them), each
  // with its own L2.  When the KV heads divide evenly over the XCDs, XCD x serves heads
  // x, x+8, x+16, ... one after the other, so all its concurrent workgroups stream the
  // same head's K/V (with 8 KV heads: one head per XCD for the whole launch); otherwise
  // the KV head is simply the fastest index.  Then split, then query block from the
  // heaviest (last) one down, then sequence: the sequences of a packed batch run one
  // after another, so the workgroups an XCD runs at once stream one sequence's K/V
  // through its L2 (interleaving the sequences multiplies that working set).
  int bid = blockIdx.x;
  int g;
  if (p.hkv % kXcds == 0) {
    const int per_head = (int)(gridDim.x / p.hkv);    // workgroups of one KV head
    const int xcd = bid % kXcds;
    const int j = bid / kXcds;                        // index among this XCD's workgroups
    g = xcd + kXcds * (j / per_head);
    bid = j % per_head;
  } else {
    g = bid % p.hkv;
    bid /= p.hkv;
  }
  int split = 0;
  if constexpr (SPLIT) {
    split = bid % p.num_splits;
    bid /= p.num_splits;
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
  if (q0 >= len) return;                              // uniform over the workgroup
  // KV tiles [t0, t0 + n_tiles): the block's causal range, or this split's part of it
  int t0 = 0;
  int n_tiles = ((CAUSAL ? min(q0 + C::TOK_WG, len) : len) + BN - 1) / BN;
  if constexpr (SPLIT) {
    t0 = split_first_tile(n_tiles, split, p.num_splits);
    n_tiles = split_first_tile(n_tiles, split + 1, p.num_splits) - t0;
    if (n_tiles == 0) return;                         // uniform over the workgroup
  }

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

  // ---- K/V tile fill: buffer loads straight into LDS, no VGPR staging.  A tile is
  // TILE_PIECES pieces of 1 KB; each wave moves PIECES_PER_WAVE pieces of K and as many of
  // V.  Lane i of a piece lands at byte 16*i of it, so the lane fetches the global 16-byte
  // chunk whose swizzled LDS position that is.  Rows past the sequence end fall outside the
  // buffer's range and arrive as zeros.
  const int kv_stride = p.hkv * D;                    // elements between consecutive tokens
  const uint16_t* kg = p.k + (size_t)start * kv_stride + g * D;
  const uint16_t* vg = p.v + (size_t)start * kv_stride + g * D;
  unsigned fill_off[C::PIECES_PER_WAVE];              // byte offset of this lane's chunk in a tile
#pragma unroll
  for (int n = 0; n < C::PIECES_PER_WAVE; ++n) {
    const int byte = (n * C::NW + wave) * 1024 + 16 * lane;
    const int row = byte / (2 * D);
    const int phys = (byte % (2 * D)) / 16;
    const int logical = lds_chunk<D>(row, phys);      // the swizzle is an XOR: its own inverse
    fill_off[n] = (unsigned)(row * kv_stride * 2 + logical * 16);
  }
  auto fill_tile = [&](int kt, uint16_t* kdst, uint16_t* vdst) __attribute__((always_inline)) {
    kt += t0;                                         // local tile -> tile of the sequence
    const int rows = min(len - kt * BN, BN);
    const size_t tile0 = (size_t)kt * BN * kv_stride;
    fill_tile_lds<C>(kg + tile0, vg + tile0, rows * kv_stride * 2, kdst, vdst, wave, fill_off);
  };

  // Per-lane LDS element offsets that do not change from tile to tile.
  // K fragment (key block kb, d step ds): row 32*kb + col, logical chunk 2*ds + half.  The
  // swizzle term depends on key bits 0-3 only, so key blocks differ by a constant.
  int k_off[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) k_off[ds] = col * D + lds_chunk<D>(col, 2 * ds + half) * 8;
  // V^T fragment (16-key step ks, d block db), two transposing reads: within each 16-lane
  // group, source lane i reads key kbase + i/4 and d = dbase + 4*(i%4) .. +3; the first read
  // covers keys 16*ks + 4*(lane/32) + 0..3, the second the same keys + 8.  The swizzle term
  // does not depend on ks, so 16-key steps differ by a constant.
  int v_off[NDB][2];
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
        v_off[db][h] = key * D + lds_chunk<D>(key, d >> 3) * 8 + (d & 7);
      }
    }
  }

  constexpr int NKF = NKB * NDS;   // K fragments (= score MFMAs) per tile
  constexpr int NVF = NKS * NDB;   // V^T fragments (= P.V MFMAs) per tile
  constexpr int KPF = 4;           // K fragments in flight ahead of their MFMA
  constexpr int VPF = 4;           // V^T fragments in flight ahead of their MFMA

  auto k_frag = [&](const uint16_t* ks_lds, int i) __attribute__((always_inline)) {
    const int kb = i % NKB, ds = i / NKB;
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(ks_lds + k_off[ds] + kb * 32 * D));
  };
  auto v_frag = [&](const uint16_t* vs_lds, int i) __attribute__((always_inline)) {
    const int ks = i / NDB, db = i % NDB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(vs_lds + v_off[db][0] + ks * 16 * D));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(vs_lds + v_off[db][1] + ks * 16 * D));
    return __builtin_bit_cast(
        bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                      __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
  };

  f32x16 s[NKB];   // raw scores of the tile whose softmax comes next
  bf16x8 pf[NKS];  // its weights as bf16: the B operands of its P.V MFMAs
  bf16x8 vf[NVF];  // V^T fragments, the first VPF read ahead of the P.V MFMAs

  // S^T = K Q^T for one tile: the two key blocks alternate so consecutive MFMAs are
  // independent; the K fragment reads run KPF MFMAs ahead
  auto scores = [&](const uint16_t* ks_lds) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
    bf16x8 kf[NKF];
#pragma unroll
    for (int i = 0; i < KPF; ++i) kf[i] = k_frag(ks_lds, i);
#pragma unroll
    for (int i = 0; i < NKF; ++i) {
      if (i + KPF < NKF) kf[i + KPF] = k_frag(ks_lds, i + KPF);
      s[i % NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i / NKB], s[i % NKB], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, KPF, 0);
#pragma unroll
    for (int i = 0; i < NKF - KPF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, KPF, 0);
  };

  // causal mask and online softmax of tile kt of the sequence (scores in s) -> pf, l_run,
  // m_run; `first`: the first tile this workgroup processes
  auto softmax = [&](int kt, bool first) __attribute__((always_inline)) {
    if constexpr (CAUSAL) {
      // causal mask, only on tiles that reach past the wave's first token
      if (kt * BN + BN - 1 > wq0) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kt * BN + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
            if (j > my_tok) s[kb][r] = -__builtin_inff();
          }
      }
    } else {
      // bidirectional: only the keys past the sequence end (zero-filled in LDS) are masked
      if (kt * BN + BN > len) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kt * BN + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
            if (j >= len) s[kb][r] = -__builtin_inff();
          }
      }
    }

    // P = exp2(S * scale*log2e - m_run) as bf16 and this lane's fp32 sum of the weights
    // (two chains)
    auto exponentiate = [&]() __attribute__((always_inline)) -> float {
      float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        f32x8 e;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          e[t] = __builtin_amdgcn_exp2f(
              __builtin_fmaf(s[ks >> 1][8 * (ks & 1) + t], p.scale_log2, -m_run));
        pf[ks] = __builtin_convertvector(e, bf16x8);
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          l0 += e[t];
          l1 += e[t + 1];
        }
      }
      return l0 + l1;
    };

    // Common case: weights against the running max as it stands.  The first tile, and
    // any tile where some lane's weights sum past WEIGHT_SUM_LIMIT, take the max path.
    float lsum = 0.0f;
    uint64_t flagged = 0;
    bool max_path = first;
    if (!max_path) {
      lsum = exponentiate();
      flagged = __builtin_amdgcn_ballot_w64(!(lsum <= WEIGHT_SUM_LIMIT));
      max_path = flagged != 0;
    }
    if (max_path) {
      // row max over the tile: 16 keys per block in-lane, then the lane pair
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = pair_max(mx);
      // rows raised: all on the first tile, else those whose lane or partner lane flagged
      const bool raise = first || (((flagged >> col) | (flagged >> (col + 32))) & 1) != 0;
      const float m_new = raise ? fmaxf(m_run, mx * p.scale_log2) : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m_run = m_new;
      lsum = exponentiate();   // rows not raised get the same weights as before
    }
    l_run += lsum;
  };

  // O^T += V^T P^T for one tile; vf[0 .. VPF) already read, the rest run VPF MFMAs ahead
  auto pv = [&](const uint16_t* vs_lds) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NVF; ++i) {
      if (i + VPF < NVF) vf[i + VPF] = v_frag(vs_lds, i + VPF);
      acc[i % NDB] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf[i / NDB], acc[i % NDB], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NVF - VPF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, VPF, 0);
  };

  // ---- tile loop.  Barrier b(j) follows the interval in which this wave's share of tile
  // j+1 was loaded; right after it every wave issues its share of tile j+2.  A tile lives in
  // LDS stage tile % 3: its K is read by the scores before b(tile), its V by the P.V before
  // b(tile + 1), and the stage is refilled (tile + 3) only after b(tile + 1).
  //
  // Each wave runs the cycle  softmax(t) -> P.V(t) -> scores(t+1)  and the two waves that
  // share a SIMD (w and w + NW/2) place their barrier at different points of it: group 0
  // between softmax(t) and P.V(t), group 1 after scores(t+1).  Between two barriers one
  // group therefore issues MFMAs (P.V then scores) while the other runs its softmax on the
  // VALU, and the SIMD's matrix core and VALU work at the same time.
  const int group = wave / (C::NW / 2);
  // last local tile with a key visible to this wave (-1: none in this range)
  const int t_last = (w_last < 0)   ? -1
                     : CAUSAL       ? min(w_last / BN - t0, n_tiles - 1)
                                    : n_tiles - 1;
  auto sync = [&](int j) __attribute__((always_inline)) {
    wait_vmem();        // this wave's share of tile j+1 has landed in LDS ...
    __syncthreads();    // ... and so has every other wave's; b(j) passed
    if (j + 2 < n_tiles) {
      const int st = (j + 2) % 3;
      fill_tile(j + 2, k_lds[st], v_lds[st]);
    }
  };
  // loop step t on LDS stage ST = t % 3 (unrolled by stage so LDS addresses are immediates)
  auto step = [&](int t, auto stage) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage)::value;
    constexpr int SN = (ST + 1) % 3;
    const bool mine = t <= t_last;
    if (mine) {
#pragma unroll
      for (int i = 0; i < VPF; ++i) vf[i] = v_frag(v_lds[ST], i);   // overlap the softmax
      softmax(t0 + t, t == 0);
    }
    if (group == 0) sync(t);
    if (mine) pv(v_lds[ST]);
    if (t + 1 <= t_last) scores(k_lds[SN]);
    if (group == 1 && t + 1 < n_tiles) sync(t + 1);
  };

  fill_tile(0, k_lds[0], v_lds[0]);
  wait_vmem();
  __syncthreads();                                    // b(-1): tile 0 in LDS
  if (1 < n_tiles) fill_tile(1, k_lds[1], v_lds[1]);
  if (0 <= t_last) scores(k_lds[0]);
  if (group == 1) sync(0);
  for (int t = 0; t < n_tiles; t += 3) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_tiles) step(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < n_tiles) step(t + 2, std::integral_constant<int, 2>{});
  }

  // ---- epilogue: O = acc / l (bf16), LSE = (m + log2 l) * ln 2
  const float l_tot = pair_sum(l_run);
  if constexpr (SPLIT) {
    // partial over this split's keys, fp32; a row that saw no key gets O = 0, LSE = -inf
    if (my_valid) {
      const bool empty = !(l_tot > 0.0f);
      const float inv = empty ? 0.0f : 1.0f / l_tot;
      float* op = p.o_part + (((size_t)split * p.total_tokens + start + my_tok) * p.hq + my_head) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 x;
#pragma unroll
          for (int t = 0; t < 4; ++t) x[t] = acc[db][4 * r4 + t] * inv;
          *(f32x4*)(op + 32 * db + 8 * r4 + 4 * half) = x;
        }
      if (half == 0)
        p.lse_part[((size_t)split * p.hq + my_head) * p.total_tokens + start + my_tok] =
            empty ? -__builtin_inff() : (m_run + __builtin_amdgcn_logf(l_tot)) * LN2;
    }
    return;
  }
  if (my_valid) {
    const float inv = 1.0f / l_tot;
    uint16_t* op = p.o + (p.o_head_major
                              ? ((size_t)my_head * p.total_tokens + start + my_tok) * D
                              : ((size_t)(start + my_tok) * p.hq + my_head) * D);
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
