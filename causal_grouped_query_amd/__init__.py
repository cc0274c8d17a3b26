"""Python binding of ``libh3attn.so``: the MI355X causal grouped-query attention forward.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI in ``include/h3attn.h``; PyTorch supplies device
memory and the current HIP stream.  There is no CPU fallback: if the library
is missing or the device is not a gfx950, calls raise.

    o, lse = gqa_causal_fwd(q, k, v)              # q [S,Hq,D], k/v [S,Hkv,D] bf16 on cuda
    o, lse = gqa_causal_varlen_fwd(q, k, v, cu_seqlens, max_seqlen)

The operation is the text encoder's bf16 causal GQA of the h3.c issue "Qwen
text encoder: sequence exceeds Metal threadgroup memory with reference video +
ref images (>=150 frames)" (section "Error"), computed with a tiled kernel
whose on-chip memory does not grow with the sequence ("Suggested fix
directions").
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; H3ATTN_LIBRARY names another build of the same sources (the host-side
# sanitizer test build, for instance).
LIBRARY = os.environ.get("H3ATTN_LIBRARY") or os.path.join(PKG_DIR, "libh3attn.so")

# status codes (include/h3attn.h)
(OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_SCALE, ERR_LAUNCH, ERR_DEVICE,
 ERR_WORKSPACE) = range(9)
MAX_SPLITS = 64
NOALLOC_SCRATCH_BYTES = 64 << 20   # fixed scratch of h3attn_gqa_causal_splitkv_fwd_noalloc

NONCAUSAL, O_HEAD_MAJOR = 1, 2   # flags of h3attn_gqa_fwd
PROLOGUE_ROPE = 1                # flag of h3attn_qk_norm_rope
CALIB_MFMA, CALIB_EXP, CALIB_MFMA_ZERO, CALIB_MFMA_PAIRED = 0, 1, 2, 3   # h3attn_calib_loop kinds

EXPORTED = ("h3attn_gqa_causal_fwd", "h3attn_gqa_fwd", "h3attn_gqa_causal_varlen_fwd",
            "h3attn_gqa_causal_splitkv_fwd", "h3attn_gqa_causal_splitkv_workspace_bytes",
            "h3attn_qk_norm_rope", "h3attn_gqa_causal_qnorm_rope_fwd", "h3attn_pool_tokens",
            "h3attn_pool_tokens_out_len", "h3attn_check_cu_seqlens",
            "h3attn_gqa_causal_splitkv_fwd_noalloc", "h3attn_calib_loop",
            "h3attn_status_string", "h3attn_version",
            "h3attn_lds_bytes")

_lock = threading.Lock()
_lib = None


class H3AttnError(RuntimeError):
    """A nonzero status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"h3attn: {message} (status {status})")
        self.status = status


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load the HIP library (once) and declare the C signatures."""
    global _lib
    # torch ships its own HIP runtime; load it first so that this library binds to the
    # same runtime instance (same device state, streams and allocations) as torch.
    import torch  # noqa: F401

    with _lock:
        if _lib is not None and path == LIBRARY:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"h3attn: HIP library {path} is not built; run "
                "`python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python -m causal_grouped_query_amd.build`")
        lib = ctypes.CDLL(path)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.h3attn_gqa_causal_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp]
        lib.h3attn_gqa_causal_fwd.restype = i32
        lib.h3attn_gqa_causal_varlen_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                     i32, i32, f32, vp]
        lib.h3attn_gqa_causal_varlen_fwd.restype = i32
        lib.h3attn_gqa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp]
        lib.h3attn_gqa_fwd.restype = i32
        lib.h3attn_qk_norm_rope.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, f32, f32,
                                            vp, i32, vp]
        lib.h3attn_qk_norm_rope.restype = i32
        lib.h3attn_gqa_causal_qnorm_rope_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                         f32, vp, f32, f32, vp, i32, vp]
        lib.h3attn_gqa_causal_qnorm_rope_fwd.restype = i32
        lib.h3attn_pool_tokens.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp]
        lib.h3attn_pool_tokens.restype = i32
        lib.h3attn_pool_tokens_out_len.argtypes = [i32, i32, i32, i32]
        lib.h3attn_pool_tokens_out_len.restype = i32
        sz = ctypes.c_size_t
        lib.h3attn_gqa_causal_splitkv_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                      f32, i32, vp, sz, vp]
        lib.h3attn_gqa_causal_splitkv_fwd.restype = i32
        lib.h3attn_gqa_causal_splitkv_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.h3attn_gqa_causal_splitkv_workspace_bytes.restype = sz
        lib.h3attn_status_string.argtypes = [i32]
        lib.h3attn_status_string.restype = ctypes.c_char_p
        lib.h3attn_version.argtypes = []
        lib.h3attn_version.restype = i32
        lib.h3attn_lds_bytes.argtypes = [i32, i32]
        lib.h3attn_lds_bytes.restype = i32
        lib.h3attn_gqa_causal_splitkv_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32,
                                                              i32, f32, i32, vp]
        lib.h3attn_gqa_causal_splitkv_fwd_noalloc.restype = i32
        lib.h3attn_check_cu_seqlens.argtypes = [vp, i32, i32, i32]
        lib.h3attn_check_cu_seqlens.restype = i32
        lib.h3attn_calib_loop.argtypes = [i32, i32, i32, vp, vp, ctypes.POINTER(i32), vp]
        lib.h3attn_calib_loop.restype = i32
        if path == LIBRARY:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().h3attn_status_string(int(status)).decode()


def version() -> int:
    return int(load_library().h3attn_version())


def lds_bytes(head_dim: int, group: int) -> int:
    return int(load_library().h3attn_lds_bytes(int(head_dim), int(group)))


def _check(status: int) -> None:
    if status != OK:
        raise H3AttnError(status, status_string(status))


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensors(q, k, v):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise TypeError(f"h3attn: {name} must be a torch.bfloat16 tensor")
        if t.device.type != "cuda":
            raise ValueError(f"h3attn: {name} must live on a GPU (got {t.device})")
        if not t.is_contiguous():
            raise ValueError(f"h3attn: {name} must be contiguous")
        if t.dim() != 3:
            raise ValueError(f"h3attn: {name} must be [tokens, heads, head_dim]")
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError("h3attn: shapes must be q [T,Hq,D], k and v [T,Hkv,D]")
    if not (q.device == k.device == v.device):
        raise ValueError("h3attn: q, k, v must be on one device")


def _outputs(q, out, lse, return_lse):
    import torch

    T, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("h3attn: out must be a contiguous bf16 tensor shaped like q")
    if lse is None and return_lse:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (Hq, T) or lse.dtype != torch.float32
                              or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("h3attn: lse must be a contiguous float32 tensor [Hq, T]")
    return out, lse


def gqa_causal_fwd(q, k, v, softmax_scale: float | None = None, out=None, lse=None,
                   return_lse: bool = True, stream=None):
    """Causal GQA forward of one sequence.

    q [S, Hq, D], k and v [S, Hkv, D]: contiguous bf16 tensors on the GPU.
    Returns ``(o, lse)``: o [S, Hq, D] bf16 and lse [Hq, S] float32 (natural
    log-sum-exp of the scaled scores; ``None`` if ``return_lse`` is false and
    no ``lse`` buffer is passed).  ``softmax_scale`` defaults to 1/sqrt(D).
    The work is enqueued on ``stream`` (default: torch's current stream).
    """
    _check_tensors(q, k, v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out, lse = _outputs(q, out, lse, return_lse)
    lib = load_library()
    rc = lib.h3attn_gqa_causal_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr() if lse is not None else None, S, Hq, Hkv, D,
                                   scale, _stream_handle(stream, q.device))
    _check(rc)
    return out, lse


def gqa_fwd(q, k, v, causal: bool = True, head_major_out: bool = False,
            softmax_scale: float | None = None, out=None, lse=None, return_lse: bool = True,
            stream=None):
    """GQA forward of one sequence with options (h3attn_gqa_fwd).

    ``causal=False`` is the bidirectional form (every query sees all keys);
    ``head_major_out=True`` returns o as [Hq, S, D] instead of [S, Hq, D].
    lse is [Hq, S] either way.
    """
    import torch

    _check_tensors(q, k, v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if head_major_out:
        if out is None:
            out = torch.empty((Hq, S, D), dtype=torch.bfloat16, device=q.device)
        elif out.shape != (Hq, S, D) or out.dtype != torch.bfloat16 or not out.is_contiguous() \
                or out.device != q.device:
            raise ValueError("h3attn: out must be a contiguous bf16 tensor [Hq, S, D]")
        _, lse = _outputs(q, None, lse, return_lse)
    else:
        out, lse = _outputs(q, out, lse, return_lse)
    flags = (0 if causal else NONCAUSAL) | (O_HEAD_MAJOR if head_major_out else 0)
    lib = load_library()
    rc = lib.h3attn_gqa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr() if lse is not None else None, S, Hq, Hkv, D, scale,
                            flags, _stream_handle(stream, q.device))
    _check(rc)
    return out, lse


def qk_norm_rope(q, k, q_norm_weight=None, k_norm_weight=None, eps: float = 1e-6,
                 rope: bool = True, rope_theta: float = 1e6, positions=None, q_out=None,
                 k_out=None, stream=None):
    """Q/K prologue (h3attn_qk_norm_rope): per-head RMS norm (when a weight is given) and
    rotate-half RoPE.  q [S,Hq,D], k [S,Hkv,D] bf16 on the GPU; weights bf16 [D];
    positions an int32 GPU tensor [S] (default: token index).  Returns (q_out, k_out);
    pass q_out=q, k_out=k to work in place.  q=None transforms K only (q_out is None)."""
    import torch

    for name, t in (("q", q), ("k", k)):
        if name == "q" and t is None:
            continue
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 3 \
                or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"h3attn: {name} must be a contiguous bf16 [S, H, D] GPU tensor")
    S, Hkv, D = k.shape
    Hq = 0
    if q is not None:
        Hq = q.shape[1]
        if q.shape[0] != S or q.shape[2] != D:
            raise ValueError("h3attn: q [S,Hq,D] and k [S,Hkv,D] must agree on S and D")
        q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    pairs = (("k_out", k_out, k),) if q is None else (("q_out", q_out, q), ("k_out", k_out, k))
    for name, t, ref in pairs:
        if t.shape != ref.shape or t.dtype != torch.bfloat16 or not t.is_contiguous() \
                or t.device != ref.device:
            raise ValueError(f"h3attn: {name} must be a contiguous bf16 tensor shaped like its input")
    for name, t in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        if t is not None and (t.dtype != torch.bfloat16 or t.numel() != D or t.device != k.device
                              or not t.is_contiguous()):
            raise ValueError(f"h3attn: {name} must be a contiguous bf16 GPU tensor of D values")
    if positions is not None and (positions.dtype != torch.int32 or positions.numel() != S
                                  or positions.device != k.device
                                  or not positions.is_contiguous()):
        raise ValueError("h3attn: positions must be a contiguous int32 GPU tensor of S values")

    def ptr(t):
        return None if t is None else t.data_ptr()

    rc = load_library().h3attn_qk_norm_rope(
        ptr(q), k.data_ptr(), ptr(q_out), k_out.data_ptr(), S, Hq, Hkv, D,
        ptr(q_norm_weight), ptr(k_norm_weight), float(eps), float(rope_theta), ptr(positions),
        PROLOGUE_ROPE if rope else 0, _stream_handle(stream, k.device))
    _check(rc)
    return q_out, k_out


def gqa_causal_qnorm_rope_fwd(q, k, v, q_norm_weight=None, eps: float = 1e-6, rope: bool = True,
                              rope_theta: float = 1e6, positions=None,
                              softmax_scale: float | None = None, out=None, lse=None,
                              return_lse: bool = True, stream=None):
    """Causal GQA forward with Q's RMS norm and RoPE applied inside the attention kernel
    (h3attn_gqa_causal_qnorm_rope_fwd).  q [S,Hq,D], k and v [S,Hkv,D] bf16 on the GPU; k
    already normalised and rotated (qk_norm_rope(None, k, ...)).  Returns (o, lse)."""
    import torch

    _check_tensors(q, k, v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    if q_norm_weight is not None and (q_norm_weight.dtype != torch.bfloat16
                                      or q_norm_weight.numel() != D
                                      or q_norm_weight.device != q.device
                                      or not q_norm_weight.is_contiguous()):
        raise ValueError("h3attn: q_norm_weight must be a contiguous bf16 GPU tensor of D values")
    if positions is not None and (positions.dtype != torch.int32 or positions.numel() != S
                                  or positions.device != q.device
                                  or not positions.is_contiguous()):
        raise ValueError("h3attn: positions must be a contiguous int32 GPU tensor of S values")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out, lse = _outputs(q, out, lse, return_lse)
    rc = load_library().h3attn_gqa_causal_qnorm_rope_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, S, Hq, Hkv, D, scale,
        None if q_norm_weight is None else q_norm_weight.data_ptr(), float(eps),
        float(rope_theta), None if positions is None else positions.data_ptr(),
        PROLOGUE_ROPE if rope else 0, _stream_handle(stream, q.device))
    _check(rc)
    return out, lse


def check_cu_seqlens(cu_seqlens, total_tokens: int, max_seqlen: int) -> int:
    """Status of the library's host-side check of packed-batch offsets (a host int32
    sequence of num_seqs + 1 values); OK when they are valid for total_tokens / max_seqlen."""
    import numpy as np

    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    ptr = cu.ctypes.data if cu.size else None
    return int(load_library().h3attn_check_cu_seqlens(ptr, int(cu.size) - 1, int(total_tokens),
                                                      int(max_seqlen)))


def calib_loop(kind: int, n_workgroups: int, iters: int, stream=None, device=None,
               stamps=None, sink=None):
    """Enqueue one calibration loop (CALIB_MFMA, CALIB_MFMA_ZERO, CALIB_EXP or
    CALIB_MFMA_PAIRED; see h3attn_calib_loop) and
    return (stamps, wall_clock_khz): stamps is an int64 GPU tensor [n_workgroups * 4, 4]
    (per wave: shader-clock counter before / after its loop, constant-rate counter before /
    after), filled when the stream reaches the launch; wall_clock_khz is the rate of the
    constant-rate counter.  stamps and sink (float32 [n_workgroups * 256]) may be passed in
    to reuse them across calls."""
    import torch

    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    n = int(n_workgroups)
    if stamps is None:
        stamps = torch.zeros((n * 4, 4), dtype=torch.int64, device=device)
    if sink is None:
        sink = torch.empty(n * 256, dtype=torch.float32, device=device)
    if stamps.dtype != torch.int64 or not stamps.is_contiguous() or stamps.numel() < n * 16 \
            or sink.dtype != torch.float32 or not sink.is_contiguous() or sink.numel() < n * 256:
        raise ValueError("h3attn: stamps must be contiguous int64 with n_workgroups * 16 "
                         "elements, sink contiguous float32 with n_workgroups * 256")
    khz = ctypes.c_int(0)
    _check(load_library().h3attn_calib_loop(int(kind), int(n_workgroups), int(iters),
                                            stamps.data_ptr(), sink.data_ptr(),
                                            ctypes.byref(khz), _stream_handle(stream, device)))
    if stream is not None:   # both buffers stay reserved until that stream's work is done
        stamps.record_stream(stream)
        sink.record_stream(stream)
    return stamps, int(khz.value)


def pool_tokens_out_len(T: int, begin: int, end: int, factor: int) -> int:
    """Length of :func:`pool_tokens`'s output (-1 for invalid arguments)."""
    return int(load_library().h3attn_pool_tokens_out_len(int(T), int(begin), int(end),
                                                         int(factor)))


def pool_tokens(x, begin: int, end: int, factor: int, out=None, stream=None):
    """Average-pool groups of ``factor`` tokens inside [begin, end) of x [T, C] (bf16 on the
    GPU); tokens outside the span are copied.  Returns out [T_out, C]."""
    import torch

    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() != 2 \
            or not x.is_contiguous() or x.device.type != "cuda":
        raise ValueError("h3attn: x must be a contiguous bf16 [T, C] GPU tensor")
    T, C = x.shape
    n = pool_tokens_out_len(T, begin, end, factor)
    if n < 0:
        raise H3AttnError(ERR_SHAPE, status_string(ERR_SHAPE))
    if out is None:
        out = torch.empty((n, C), dtype=torch.bfloat16, device=x.device)
    elif out.shape != (n, C) or out.dtype != torch.bfloat16 or not out.is_contiguous() \
            or out.device != x.device:
        raise ValueError("h3attn: out must be a contiguous bf16 tensor [T_out, C]")
    _check(load_library().h3attn_pool_tokens(x.data_ptr(), out.data_ptr(), T, C, int(begin),
                                             int(end), int(factor), _stream_handle(stream, x.device)))
    return out


def gqa_causal_varlen_fwd(q, k, v, cu_seqlens, max_seqlen: int,
                          softmax_scale: float | None = None, out=None, lse=None,
                          return_lse: bool = True, stream=None):
    """Causal GQA forward of a packed batch of independent sequences.

    q [T, Hq, D], k and v [T, Hkv, D] bf16 on the GPU; ``cu_seqlens`` an int32
    tensor [num_seqs + 1] of offsets (cu[0] = 0, cu[-1] = T), on q's device or
    on the host; ``max_seqlen`` bounds every sequence length.  Returns
    ``(o, lse)`` with lse [Hq, T] indexed by packed token.

    Offsets on the device are not read on the host: a table that breaks those
    rules gives unspecified rows (in particular the rows of a sequence past its
    first ``max_seqlen`` tokens are left unwritten), never an out-of-bounds
    access.  Offsets on the host are checked first (``H3AttnError`` with
    ``ERR_SHAPE`` on a bad table) and then copied to q's device; device offsets
    are checked too when ``H3ATTN_CHECK_CU_SEQLENS=1`` is set in the environment
    (the library copies them back, one small synchronous read).
    """
    import torch

    _check_tensors(q, k, v)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device.type == "cpu":
        host = cu_seqlens.to(torch.int32).contiguous()
        _check(check_cu_seqlens(host.numpy(), T, int(max_seqlen)))
        cu_seqlens = host.to(q.device)
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 \
            or cu_seqlens.device != q.device or cu_seqlens.dim() != 1 \
            or not cu_seqlens.is_contiguous():
        raise ValueError("h3attn: cu_seqlens must be a contiguous int32 tensor on q's device "
                         "or on the host")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out, lse = _outputs(q, out, lse, return_lse)
    lib = load_library()
    rc = lib.h3attn_gqa_causal_varlen_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, cu_seqlens.data_ptr(),
        cu_seqlens.numel() - 1, T, int(max_seqlen), Hq, Hkv, D, scale,
        _stream_handle(stream, q.device))
    _check(rc)
    return out, lse


def splitkv_workspace_bytes(seq_len: int, n_q_heads: int, head_dim: int, num_splits: int) -> int:
    """Bytes of device workspace :func:`gqa_causal_splitkv_fwd` needs (0 if invalid)."""
    return int(load_library().h3attn_gqa_causal_splitkv_workspace_bytes(
        int(seq_len), int(n_q_heads), int(head_dim), int(num_splits)))


def gqa_causal_splitkv_fwd(q, k, v, num_splits: int, softmax_scale: float | None = None,
                           out=None, lse=None, workspace=None, return_lse: bool = True,
                           stream=None):
    """Split-KV (two-dispatch) causal GQA forward of one sequence.

    Same inputs and result as :func:`gqa_causal_fwd`; the KV range of every query
    block is cut into ``num_splits`` parts whose partial results go through
    ``workspace`` (a contiguous uint8 CUDA tensor of at least
    :func:`splitkv_workspace_bytes` bytes, 256-byte aligned; allocated here with
    torch when not given) and are merged by a second kernel.
    """
    import torch

    _check_tensors(q, k, v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out, lse = _outputs(q, out, lse, return_lse)
    lib = load_library()
    need = int(lib.h3attn_gqa_causal_splitkv_workspace_bytes(S, Hq, D, int(num_splits)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif (not isinstance(workspace, torch.Tensor) or workspace.device != q.device
          or not workspace.is_contiguous()):
        raise ValueError("h3attn: workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib.h3attn_gqa_causal_splitkv_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, S, Hq, Hkv, D, scale, int(num_splits),
        workspace.data_ptr(), ws_bytes, _stream_handle(stream, q.device))
    _check(rc)
    return out, lse


def gqa_causal_splitkv_fwd_noalloc(q, k, v, num_splits: int, softmax_scale: float | None = None,
                                   out=None, lse=None, return_lse: bool = True, stream=None):
    """:func:`gqa_causal_splitkv_fwd` with the library's fixed scratch array as its workspace
    (for callers that cannot allocate device memory: pass ``out`` and ``lse``).  The
    workspace need must not exceed :data:`NOALLOC_SCRATCH_BYTES`; calls that overlap on
    one GPU race on the shared array."""
    _check_tensors(q, k, v)
    S, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    out, lse = _outputs(q, out, lse, return_lse)
    rc = load_library().h3attn_gqa_causal_splitkv_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, S, Hq, Hkv, D, scale, int(num_splits),
        _stream_handle(stream, q.device))
    _check(rc)
    return out, lse


__all__ = ["gqa_causal_fwd", "gqa_fwd", "gqa_causal_varlen_fwd", "gqa_causal_splitkv_fwd",
           "gqa_causal_splitkv_fwd_noalloc", "NOALLOC_SCRATCH_BYTES",
           "splitkv_workspace_bytes", "status_string", "version", "lds_bytes", "load_library",
           "H3AttnError", "LIBRARY", "EXPORTED", "MAX_SPLITS", "NONCAUSAL", "O_HEAD_MAJOR",
           "qk_norm_rope", "gqa_causal_qnorm_rope_fwd", "PROLOGUE_ROPE", "pool_tokens",
           "pool_tokens_out_len", "calib_loop", "CALIB_MFMA", "CALIB_EXP", "CALIB_MFMA_ZERO",
           "CALIB_MFMA_PAIRED"]
