// h3attn.hip -- host side of the C ABI declared in include/h3attn.h:
// argument checks, kernel-instance selection, grid planning and launch.
//
// The operation is the causal GQA of the h3.c issue "Qwen text encoder:
// sequence exceeds Metal threadgroup memory with reference video + ref images
// (>=150 frames)" (section "Error"); where that kernel aborted the run when a
// sequence's score row did not fit in threadgroup memory, these entry points
// have no length-dependent capacity check at all: the kernel's LDS use is
// fixed by (D, G).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "calib_kernel.hpp"
#include "gqa_fwd_kernel.hpp"
#include "gqa_fwd_wide_kernel.hpp"
#include "gqa_merge_kernel.hpp"
#include "pool_tokens_kernel.hpp"
#include "qk_prologue_kernel.hpp"
#include "h3attn.h"

namespace {

using h3attn::FwdConfig;
using h3attn::FwdParams;
using h3attn::MergeParams;

template <int D, int G>
using Cfg = h3attn::LaunchConfig<D, G>;

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

bool device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev >= kMaxDevices) return false;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Workspace of h3attn_gqa_causal_splitkv_fwd_noalloc: a fixed array in the code object, one
// copy per GPU the library runs on, held until the process ends.  Host code never uses the
// array's name as an address: each device's copy is looked up once (hipGetSymbolAddress,
// with that device current) and the pointer kept per device.
static_assert(H3ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[H3ATTN_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mutex;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The current device's copy of the scratch array, or nullptr if the lookup fails.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

template <int D, int G, bool VARLEN, bool CAUSAL>
int launch(FwdParams p, hipStream_t stream) {
  using C = Cfg<D, G>;
  p.n_qblk = (p.seq_len + C::TOK_WG - 1) / C::TOK_WG;
  const long long blocks = (long long)p.n_qblk * p.hkv * p.num_seqs;
  if (blocks == 0) return H3ATTN_OK;
  if (blocks > 0x7fffffffLL) return H3ATTN_ERR_SHAPE;
  hipLaunchKernelGGL((h3attn::gqa_causal_fwd_kernel<C, VARLEN, false, CAUSAL>),
                     dim3((unsigned)blocks), dim3(C::THREADS), 0, stream, p);
  return hipGetLastError() == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_LAUNCH;
}

// Head dim 128: the wide kernel (4 waves of 64 query rows, gqa_fwd_wide_kernel.hpp, which
// also fixes its launch shape).
template <int G, bool VARLEN, bool CAUSAL>
int launch_wide(const FwdParams& p, hipStream_t stream) {
  const hipError_t e = h3attn::launch_gqa_fwd_wide<G, VARLEN, CAUSAL>(p, stream);
  if (e == hipErrorInvalidConfiguration) return H3ATTN_ERR_SHAPE;
  return e == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_LAUNCH;
}

template <bool VARLEN, bool CAUSAL = true>
int dispatch(int D, int G, const FwdParams& p, hipStream_t stream) {
  if (D == 128) {
    switch (G) {
      case 1: return launch_wide<1, VARLEN, CAUSAL>(p, stream);
      case 2: return launch_wide<2, VARLEN, CAUSAL>(p, stream);
      case 4: return launch_wide<4, VARLEN, CAUSAL>(p, stream);
      case 8: return launch_wide<8, VARLEN, CAUSAL>(p, stream);
    }
  } else if (D == 64) {
    switch (G) {
      case 1: return launch<64, 1, VARLEN, CAUSAL>(p, stream);
      case 2: return launch<64, 2, VARLEN, CAUSAL>(p, stream);
      case 4: return launch<64, 4, VARLEN, CAUSAL>(p, stream);
      case 8: return launch<64, 8, VARLEN, CAUSAL>(p, stream);
    }
  }
  return H3ATTN_ERR_UNSUPPORTED;
}

// The causal forward with the Q prologue done in the kernel (fixed-length calls only).  Its
// LDS holds the K/V ring plus a cos/sin table of the block's tokens: TOK_WG x D/2 x 8 bytes.
template <int D, int G>
int launch_qpro(const FwdParams& p, const h3attn::QproParams& qp, hipStream_t stream) {
  using C = Cfg<D, G>;
  static_assert(C::LDS_BYTES + C::TOK_WG * (D / 2) * 8 <= 160 * 1024, "LDS");
  FwdParams pp = p;
  pp.n_qblk = (p.seq_len + C::TOK_WG - 1) / C::TOK_WG;
  const long long blocks = (long long)pp.n_qblk * p.hkv;
  if (blocks == 0) return H3ATTN_OK;
  if (blocks > 0x7fffffffLL) return H3ATTN_ERR_SHAPE;
  hipLaunchKernelGGL((h3attn::gqa_causal_qpro_fwd_kernel<C>), dim3((unsigned)blocks),
                     dim3(C::THREADS), 0, stream, pp, qp);
  return hipGetLastError() == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_LAUNCH;
}

template <int G>
int launch_wide_qpro(const FwdParams& p, const h3attn::QproParams& qp, hipStream_t stream) {
  const hipError_t e = h3attn::launch_gqa_fwd_wide<G, false, true, true>(p, stream, qp);
  if (e == hipErrorInvalidConfiguration) return H3ATTN_ERR_SHAPE;
  return e == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_LAUNCH;
}

// (D, G) pairs with a qpro instance: at D = 128 and G = 1 the table (256 tokens) would not
// fit beside the K/V ring.
bool qpro_supported(int D, int G) { return D == 64 || G != 1; }

int dispatch_qpro(int D, int G, const FwdParams& p, const h3attn::QproParams& qp,
                  hipStream_t stream) {
  if (D == 128) {
    switch (G) {
      // G = 4 and 8: the 64-row kernel (its table fits beside the 128 KB ring); G = 2: the
      // 32-row kernel (96 KB ring + a 64 KB table)
      case 2: return launch_qpro<128, 2>(p, qp, stream);
      case 4: return launch_wide_qpro<4>(p, qp, stream);
      case 8: return launch_wide_qpro<8>(p, qp, stream);
    }
  } else if (D == 64) {
    switch (G) {
      case 1: return launch_qpro<64, 1>(p, qp, stream);
      case 2: return launch_qpro<64, 2>(p, qp, stream);
      case 4: return launch_qpro<64, 4>(p, qp, stream);
      case 8: return launch_qpro<64, 8>(p, qp, stream);
    }
  }
  return H3ATTN_ERR_UNSUPPORTED;
}

// Split-KV: the split instance of the attention kernel writes per-split partials to the
// workspace, then the merge kernel combines them into o and lse (same stream, in order).
template <int D, int G>
int launch_split(FwdParams p, hipStream_t stream) {
  using C = Cfg<D, G>;
  p.n_qblk = (p.seq_len + C::TOK_WG - 1) / C::TOK_WG;
  const long long blocks = (long long)p.n_qblk * p.hkv * p.num_splits;
  if (blocks == 0) return H3ATTN_OK;
  if (blocks > 0x7fffffffLL) return H3ATTN_ERR_SHAPE;
  hipLaunchKernelGGL((h3attn::gqa_causal_fwd_kernel<C, false, true>), dim3((unsigned)blocks),
                     dim3(C::THREADS), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return H3ATTN_ERR_LAUNCH;
  MergeParams m{};
  m.o_part = p.o_part;
  m.lse_part = p.lse_part;
  m.o = p.o;
  m.lse = p.lse;
  m.seq_len = p.seq_len;
  m.hq = p.hq;
  m.num_splits = p.num_splits;
  m.tok_wg = C::TOK_WG;
  m.bn = C::BN;
  constexpr int rows_per_block = h3attn::MERGE_THREADS / (D / 4);
  const long long rows = (long long)p.seq_len * p.hq;
  const long long mblocks = (rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((h3attn::merge_splits_kernel<D>), dim3((unsigned)mblocks),
                     dim3(h3attn::MERGE_THREADS), 0, stream, m);
  return hipGetLastError() == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_LAUNCH;
}

int dispatch_split(int D, int G, const FwdParams& p, hipStream_t stream) {
  if (D == 128) {
    switch (G) {
      case 1: return launch_split<128, 1>(p, stream);
      case 2: return launch_split<128, 2>(p, stream);
      case 4: return launch_split<128, 4>(p, stream);
      case 8: return launch_split<128, 8>(p, stream);
    }
  } else if (D == 64) {
    switch (G) {
      case 1: return launch_split<64, 1>(p, stream);
      case 2: return launch_split<64, 2>(p, stream);
      case 4: return launch_split<64, 4>(p, stream);
      case 8: return launch_split<64, 8>(p, stream);
    }
  }
  return H3ATTN_ERR_UNSUPPORTED;
}

// Workspace layout of the split-KV call: partial O (fp32 [num_splits, S, Hq, D]) at
// offset 0, partial LSE (fp32 [num_splits, Hq, S]) at the next 256-byte boundary.
// Returns 0 for invalid sizes.
size_t split_workspace_layout(long long S, long long Hq, long long D, long long ns,
                              size_t* lse_offset) {
  if (S < 0 || Hq <= 0 || D <= 0 || ns < 1 || ns > H3ATTN_MAX_SPLITS) return 0;
  const size_t o_bytes = (size_t)ns * (size_t)S * (size_t)Hq * (size_t)D * sizeof(float);
  const size_t lse_off = (o_bytes + 255) / 256 * 256;
  if (lse_offset) *lse_offset = lse_off;
  return lse_off + (size_t)ns * (size_t)Hq * (size_t)S * sizeof(float);
}

// Checks shared by both entry points; returns a status.
// With zero tokens there is no memory to point at, so NULL tensors are accepted then.
int check_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 long long tokens, int Hq, int Hkv, int D, float scale) {
  if (tokens > 0 && (!q || !k || !v || !o)) return H3ATTN_ERR_NULL;
  if (tokens < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return H3ATTN_ERR_SHAPE;
  if (tokens * (long long)Hq * (long long)D >= (1LL << 31)) return H3ATTN_ERR_SHAPE;
  const int G = Hq / Hkv;
  if ((D != 64 && D != 128) || (G != 1 && G != 2 && G != 4 && G != 8))
    return H3ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
    return H3ATTN_ERR_ALIGN;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return H3ATTN_ERR_SCALE;
  return H3ATTN_OK;
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

namespace {

bool check_cu_seqlens_requested() {
  const char* e = std::getenv("H3ATTN_CHECK_CU_SEQLENS");
  return e != nullptr && std::strcmp(e, "1") == 0;
}

// The debug check of the varlen call: copy the device offsets to the host, in order on the
// caller's stream (after whatever wrote them), wait for the copy, and validate.
int debug_check_cu_seqlens(const int32_t* cu_dev, int num_seqs, int total_tokens,
                           int max_seqlen, hipStream_t stream) {
  std::vector<int32_t> host((size_t)num_seqs + 1);
  if (hipMemcpyAsync(host.data(), cu_dev, host.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return H3ATTN_ERR_LAUNCH;
  return h3attn_check_cu_seqlens(host.data(), num_seqs, total_tokens, max_seqlen);
}

}  // namespace

extern "C" {

int h3attn_gqa_causal_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                          int S, int Hq, int Hkv, int D, float softmax_scale, void* hip_stream) {
  const int rc = check_common(q, k, v, o, lse, S, Hq, Hkv, D, softmax_scale);
  if (rc != H3ATTN_OK) return rc;
  if (S == 0) return H3ATTN_OK;
  if (!device_ok()) return H3ATTN_ERR_DEVICE;
  FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_seqlens = nullptr;
  p.seq_len = S;
  p.total_tokens = S;
  p.num_seqs = 1;
  p.hq = Hq;
  p.hkv = Hkv;
  p.scale_log2 = softmax_scale * kLog2e;
  return dispatch<false>(D, Hq / Hkv, p, static_cast<hipStream_t>(hip_stream));
}

int h3attn_check_cu_seqlens(const int32_t* cu, int num_seqs, int total_tokens, int max_seqlen) {
  if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0) return H3ATTN_ERR_SHAPE;
  if (num_seqs > 0 && !cu) return H3ATTN_ERR_NULL;
  if (num_seqs == 0) return total_tokens == 0 ? H3ATTN_OK : H3ATTN_ERR_SHAPE;
  if (cu[0] != 0 || cu[num_seqs] != total_tokens) return H3ATTN_ERR_SHAPE;
  for (int s = 0; s < num_seqs; ++s) {
    const long long len = (long long)cu[s + 1] - cu[s];
    if (len < 0 || len > max_seqlen) return H3ATTN_ERR_SHAPE;
  }
  return H3ATTN_OK;
}

int h3attn_gqa_causal_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                                 int max_seqlen, int Hq, int Hkv, int D, float softmax_scale,
                                 void* hip_stream) {
  const int rc = check_common(q, k, v, o, lse, total_tokens, Hq, Hkv, D, softmax_scale);
  if (rc != H3ATTN_OK) return rc;
  if (num_seqs < 0 || max_seqlen < 0) return H3ATTN_ERR_SHAPE;
  if (num_seqs == 0) return total_tokens == 0 ? H3ATTN_OK : H3ATTN_ERR_SHAPE;
  if (!cu_seqlens) return H3ATTN_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return H3ATTN_ERR_ALIGN;
  if (total_tokens == 0 || max_seqlen == 0) return H3ATTN_OK;
  if (!device_ok()) return H3ATTN_ERR_DEVICE;
  if (check_cu_seqlens_requested()) {
    const int crc = debug_check_cu_seqlens(cu_seqlens, num_seqs, total_tokens, max_seqlen,
                                           static_cast<hipStream_t>(hip_stream));
    if (crc != H3ATTN_OK) return crc;
  }
  FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.seq_len = max_seqlen < total_tokens ? max_seqlen : total_tokens;
  p.total_tokens = total_tokens;
  p.num_seqs = num_seqs;
  p.hq = Hq;
  p.hkv = Hkv;
  p.scale_log2 = softmax_scale * kLog2e;
  return dispatch<true>(D, Hq / Hkv, p, static_cast<hipStream_t>(hip_stream));
}

int h3attn_gqa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int S,
                   int Hq, int Hkv, int D, float softmax_scale, int flags, void* hip_stream) {
  const int rc = check_common(q, k, v, o, lse, S, Hq, Hkv, D, softmax_scale);
  if (rc != H3ATTN_OK) return rc;
  if ((flags & ~(H3ATTN_NONCAUSAL | H3ATTN_O_HEAD_MAJOR)) != 0) return H3ATTN_ERR_UNSUPPORTED;
  if (S == 0) return H3ATTN_OK;
  if (!device_ok()) return H3ATTN_ERR_DEVICE;
  FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_seqlens = nullptr;
  p.seq_len = S;
  p.total_tokens = S;
  p.num_seqs = 1;
  p.hq = Hq;
  p.hkv = Hkv;
  p.scale_log2 = softmax_scale * kLog2e;
  p.o_head_major = (flags & H3ATTN_O_HEAD_MAJOR) ? 1 : 0;
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  return (flags & H3ATTN_NONCAUSAL) ? dispatch<false, false>(D, Hq / Hkv, p, st)
                                    : dispatch<false, true>(D, Hq / Hkv, p, st);
}

int h3attn_gqa_causal_qnorm_rope_fwd(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int S, int Hq, int Hkv, int D,
                                     float softmax_scale, const void* q_norm_weight, float eps,
                                     float rope_theta, const int32_t* positions, int flags,
                                     void* hip_stream) {
  const int rc = check_common(q, k, v, o, lse, S, Hq, Hkv, D, softmax_scale);
  if (rc != H3ATTN_OK) return rc;
  if ((flags & ~H3ATTN_PROLOGUE_ROPE) != 0 || !qpro_supported(D, Hq / Hkv))
    return H3ATTN_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(q_norm_weight) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(positions) & 3u) != 0)
    return H3ATTN_ERR_ALIGN;
  const bool rope = (flags & H3ATTN_PROLOGUE_ROPE) != 0;
  if (q_norm_weight && (!std::isfinite(eps) || eps < 0.0f)) return H3ATTN_ERR_SCALE;
  if (rope && (!std::isfinite(rope_theta) || !(rope_theta > 0.0f))) return H3ATTN_ERR_SCALE;
  if (S == 0) return H3ATTN_OK;
  if (!device_ok()) return H3ATTN_ERR_DEVICE;
  FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_seqlens = nullptr;
  p.seq_len = S;
  p.total_tokens = S;
  p.num_seqs = 1;
  p.hq = Hq;
  p.hkv = Hkv;
  p.scale_log2 = softmax_scale * kLog2e;
  h3attn::QproParams qp{};
  qp.q_weight = static_cast<const uint16_t*>(q_norm_weight);
  qp.positions = positions;
  qp.inv_freq_step = std::pow((double)rope_theta, -2.0 / (double)D);
  qp.q_eps = eps;
  qp.rope = rope ? 1 : 0;
  return dispatch_qpro(D, Hq / Hkv, p, qp, static_cast<hipStream_t>(hip_stream));
}

int h3attn_qk_norm_rope(const void* q, const void* k, void* q_out, void* k_out, int S, int Hq,
                        int Hkv, int D, const void* q_norm_weight, const void* k_norm_weight,
                        float eps, float rope_theta, const int32_t* positions, int flags,
                        void* hip_stream) {
  if (S > 0 && (!k || !k_out || (Hq > 0 && (!q || !q_out)))) return H3ATTN_ERR_NULL;
  if (S < 0 || Hq < 0 || Hkv <= 0 || D <= 0) return H3ATTN_ERR_SHAPE;
  if ((long long)S * (long long)(Hq > Hkv ? Hq : Hkv) * (long long)D >= (1LL << 31))
    return H3ATTN_ERR_SHAPE;
  if ((D != 64 && D != 128) || (flags & ~H3ATTN_PROLOGUE_ROPE) != 0)
    return H3ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out) ||
      (reinterpret_cast<uintptr_t>(q_norm_weight) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(k_norm_weight) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(positions) & 3u) != 0)
    return H3ATTN_ERR_ALIGN;
  const bool rope = (flags & H3ATTN_PROLOGUE_ROPE) != 0;
  if ((q_norm_weight || k_norm_weight) && (!std::isfinite(eps) || eps < 0.0f))
    return H3ATTN_ERR_SCALE;
  if (rope && (!std::isfinite(rope_theta) || !(rope_theta > 0.0f))) return H3ATTN_ERR_SCALE;
  if (S == 0) return H3ATTN_OK;
  if (!device_ok()) return H3ATTN_ERR_DEVICE;
  h3attn::PrologueParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.q_out = static_cast<uint16_t*>(q_out);
  p.k_out = static_cast<uint16_t*>(k_out);
  p.q_weight = static_cast<const uint16_t*>(q_norm_weight);
  p.k_weight = static_cast<const uint16_t*>(k_norm_weight);
  p.positions = positions;
  p.seq_len = S;
  p.hq = Hq;
  p.hkv = Hkv;
  p.eps = eps;
  p.theta = (double)rope_theta;
  p.rope = rope ? 1 : 0;
  const unsigned blocks = (unsigned)((S + h3attn::PROLOGUE_TOKENS - 1) / h3attn::PROLOGUE_TOKENS);
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (D == 128)
    hipLaunchKernelGGL((h3attn::qk_prologue_kernel<128>), dim3(blocks),
                       dim3(h3attn::PROLOGUE_THREADS), 0, st, p);
  else
    hipLaunchKernelGGL((h3attn::qk_prologue_kernel<64>), dim3(blocks),
                       dim3(h3attn::PROLOGUE_THREADS), 0, st, p);
  return hipGetLastError() == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_LAUNCH;
}

int h3attn_pool_tokens_out_len(int T, int begin, int end, int factor) {
  if (T < 0 || begin < 0 || end < begin || end > T || factor < 1) return -1;
  const int L = end - begin;
  return T - L + (L + factor - 1) / factor;
}

int h3attn_pool_tokens(const void* x, void* out, int T, int C, int begin, int end, int factor,
                       void* hip_stream) {
  const int T_out = h3attn_pool_tokens_out_len(T, begin, end, factor);
  if (T_out < 0 || C <= 0) return H3ATTN_ERR_SHAPE;
  if ((long long)T * (long long)C >= (1LL << 31)) return H3ATTN_ERR_SHAPE;
  if (C % 8 != 0) return H3ATTN_ERR_UNSUPPORTED;
  if (T_out == 0) return H3ATTN_OK;
  if (!x || !out) return H3ATTN_ERR_NULL;
  if (!aligned16(x) || !aligned16(out)) return H3ATTN_ERR_ALIGN;
  if (!device_ok()) return H3ATTN_ERR_DEVICE;
  h3attn::PoolParams p{};
  p.x = static_cast<const uint16_t*>(x);
  p.out = static_cast<uint16_t*>(out);
  p.T = T;
  p.C = C;
  p.begin = begin;
  p.end = end;
  p.factor = factor;
  hipLaunchKernelGGL(h3attn::pool_tokens_kernel, dim3((unsigned)T_out),
                     dim3(h3attn::POOL_THREADS), 0, static_cast<hipStream_t>(hip_stream), p);
  return hipGetLastError() == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_LAUNCH;
}

size_t h3attn_gqa_causal_splitkv_workspace_bytes(int S, int Hq, int D, int num_splits) {
  return split_workspace_layout(S, Hq, D, num_splits, nullptr);
}

int h3attn_gqa_causal_splitkv_fwd(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int S, int Hq, int Hkv, int D,
                                  float softmax_scale, int num_splits, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
  const int rc = check_common(q, k, v, o, lse, S, Hq, Hkv, D, softmax_scale);
  if (rc != H3ATTN_OK) return rc;
  if (num_splits < 1 || num_splits > H3ATTN_MAX_SPLITS) return H3ATTN_ERR_SHAPE;
  if (S == 0) return H3ATTN_OK;
  size_t lse_off = 0;
  const size_t need = split_workspace_layout(S, Hq, D, num_splits, &lse_off);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      workspace_bytes < need)
    return H3ATTN_ERR_WORKSPACE;
  if (!device_ok()) return H3ATTN_ERR_DEVICE;
  FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.cu_seqlens = nullptr;
  p.seq_len = S;
  p.total_tokens = S;
  p.num_seqs = 1;
  p.hq = Hq;
  p.hkv = Hkv;
  p.scale_log2 = softmax_scale * kLog2e;
  p.o_part = static_cast<float*>(workspace);
  p.lse_part = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + lse_off);
  p.num_splits = num_splits;
  return dispatch_split(D, Hq / Hkv, p, static_cast<hipStream_t>(hip_stream));
}

int h3attn_gqa_causal_splitkv_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                          float* lse, int S, int Hq, int Hkv, int D,
                                          float softmax_scale, int num_splits, void* hip_stream) {
  const int rc = check_common(q, k, v, o, lse, S, Hq, Hkv, D, softmax_scale);
  if (rc != H3ATTN_OK) return rc;
  if (num_splits < 1 || num_splits > H3ATTN_MAX_SPLITS) return H3ATTN_ERR_SHAPE;
  if (S == 0) return H3ATTN_OK;
  size_t lse_off = 0;
  if (split_workspace_layout(S, Hq, D, num_splits, &lse_off) > H3ATTN_NOALLOC_SCRATCH_BYTES)
    return H3ATTN_ERR_WORKSPACE;
  if (!device_ok()) return H3ATTN_ERR_DEVICE;
  void* ws = device_scratch();
  if (ws == nullptr) return H3ATTN_ERR_DEVICE;
  return h3attn_gqa_causal_splitkv_fwd(q, k, v, o, lse, S, Hq, Hkv, D, softmax_scale, num_splits,
                                       ws, H3ATTN_NOALLOC_SCRATCH_BYTES, hip_stream);
}

int h3attn_calib_loop(int kind, int n_workgroups, int iters, uint64_t* stamps, float* sink,
                      int* wall_clock_khz, void* hip_stream) {
  if (!stamps || !sink) return H3ATTN_ERR_NULL;
  if (n_workgroups < 1 || n_workgroups > 65535 || iters < 1 || iters > (1 << 24))
    return H3ATTN_ERR_SHAPE;
  if (kind != H3ATTN_CALIB_MFMA && kind != H3ATTN_CALIB_EXP && kind != H3ATTN_CALIB_MFMA_ZERO &&
      kind != H3ATTN_CALIB_MFMA_PAIRED)
    return H3ATTN_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(stamps) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return H3ATTN_ERR_ALIGN;
  if (!device_ok()) return H3ATTN_ERR_DEVICE;
  if (wall_clock_khz) {
    int dev = -1, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      return H3ATTN_ERR_DEVICE;
    *wall_clock_khz = khz;
  }
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (kind == H3ATTN_CALIB_EXP)
    hipLaunchKernelGGL((h3attn::calib_loop_kernel<1>), dim3(n_workgroups),
                       dim3(h3attn::CALIB_THREADS), 0, st, stamps, sink, iters, 0xFFFFu);
  else if (kind == H3ATTN_CALIB_MFMA_PAIRED)
    hipLaunchKernelGGL((h3attn::calib_loop_kernel<2>), dim3(n_workgroups),
                       dim3(h3attn::CALIB_THREADS), 0, st, stamps, sink, iters, 0xFFFFu);
  else   // one instance for both operand sets: the mask is a run-time value
    hipLaunchKernelGGL((h3attn::calib_loop_kernel<0>), dim3(n_workgroups),
                       dim3(h3attn::CALIB_THREADS), 0, st, stamps, sink, iters,
                       kind == H3ATTN_CALIB_MFMA ? 0xFFFFu : 0u);
  return hipGetLastError() == hipSuccess ? H3ATTN_OK : H3ATTN_ERR_LAUNCH;
}

const char* h3attn_status_string(int status) {
  switch (status) {
    case H3ATTN_OK: return "ok";
    case H3ATTN_ERR_NULL: return "a required pointer is NULL";
    case H3ATTN_ERR_SHAPE:
      return "invalid shape: negative size, Hq not a multiple of Hkv, inconsistent offsets, "
             "tokens*Hq*D >= 2^31, or num_splits outside 1..64";
    case H3ATTN_ERR_UNSUPPORTED:
      return "unsupported configuration: head dim must be 64 or 128, Hq/Hkv 1, 2, 4 or 8, "
             "flags known to the entry point, and (token pooling) C a multiple of 8";
    case H3ATTN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case H3ATTN_ERR_SCALE:
      return "softmax_scale must be finite and > 0 (prologue: eps finite and >= 0, rope_theta "
             "finite and > 0)";
    case H3ATTN_ERR_LAUNCH: return "HIP kernel launch failed";
    case H3ATTN_ERR_DEVICE: return "no usable gfx950 device is current";
    case H3ATTN_ERR_WORKSPACE:
      return "workspace is NULL, not 256-byte aligned, or smaller than "
             "h3attn_gqa_causal_splitkv_workspace_bytes() (the allocation-free call: that "
             "size exceeds its fixed scratch, H3ATTN_NOALLOC_SCRATCH_BYTES = 64 MiB)";
    default: return "unknown status";
  }
}

int h3attn_version(void) { return 300; }

int h3attn_lds_bytes(int D, int G) {
  if (D == 128) {   // the wide kernel of the causal / packed / bidirectional calls
    switch (G) {
      case 1: return h3attn::WideConfig<128, 1>::LDS_BYTES;
      case 2: return h3attn::WideConfig<128, 2>::LDS_BYTES;
      case 4: return h3attn::WideConfig<128, 4>::LDS_BYTES;
      case 8: return h3attn::WideConfig<128, 8>::LDS_BYTES;
    }
  } else if (D == 64) {
    switch (G) {
      case 1: return Cfg<64, 1>::LDS_BYTES;
      case 2: return Cfg<64, 2>::LDS_BYTES;
      case 4: return Cfg<64, 4>::LDS_BYTES;
      case 8: return Cfg<64, 8>::LDS_BYTES;
    }
  }
  return -1;
}

}  // extern "C"
