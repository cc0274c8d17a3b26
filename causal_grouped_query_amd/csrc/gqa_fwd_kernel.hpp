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

// The Q prologue the qpro instance applies while it loads Q: per-head RMS norm with weight
// q_weight (nullptr: no norm) and rotate-half RoPE when rope != 0.
struct QproParams {
  const uint16_t* q_weight;    // [D] bf16 or nullptr
  const int32_t* positions;    // [S] token positions, or nullptr (position = token index)
  double inv_freq_step;        // rope_theta^(-2/D): pair i rotates by pos * inv_freq_step^i
  float q_eps;
  int rope;
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
//
// QPRO: before its first scores, every workgroup applies the Q prologue of the h3.c
// project README (per-head RMS norm and rotary position embedding, the computation of
// qk_prologue_kernel.hpp) to the Q fragments it loaded, in fp32 with one bf16 rounding, so
// Q need not make a separate round trip through HBM.  Fixed-length causal calls only.
template <class C, bool VARLEN, bool SPLIT = false, bool CAUSAL = true>
__global__ __launch_bounds__(C::THREADS, 1) void gqa_causal_fwd_kernel(FwdParams p) {
  constexpr bool QPRO = false;
  [[maybe_unused]] const QproParams qp{};
#include "gqa_fwd_body.inc"
}

// The fixed-length causal forward with the Q prologue applied in the kernel.
template <class C>
__global__ __launch_bounds__(C::THREADS, 1) void gqa_causal_qpro_fwd_kernel(FwdParams p,
                                                                             QproParams qp) {
  constexpr bool VARLEN = false, SPLIT = false, CAUSAL = true, QPRO = true;
#include "gqa_fwd_body.inc"
}

}  // namespace h3attn
