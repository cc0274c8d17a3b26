"""fp64 CPU oracle for bf16 causal grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library in ``causal_grouped_query_amd`` and imports nothing from
it; the product never imports this package.

The arithmetic lives in ``oracle.c`` (plain C, double precision, each query
row on its own; the rows of the heads that share a KV head are evaluated
together, which reads each key row once for them and changes no sum).  This module only compiles it with gcc, loads it with ctypes
and marshals numpy arrays.  Inputs are bf16 bit patterns: ``numpy.uint16`` /
``int16`` arrays, or CPU ``torch.bfloat16`` tensors.

What the oracle follows: the h3.c issue "Qwen text encoder: sequence exceeds
Metal threadgroup memory with reference video + ref images (>=150 frames)",
sections "Error" (the operation is the text encoder's causal GQA) and
"Suggested fix directions" (the causal attention score row, softmax over it).
"""

from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

# Plain, unreordered IEEE double arithmetic: no fast-math, no FMA contraction.
CFLAGS = ["-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile ``source`` into the shared library ``output`` with gcc."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("oracle: no C compiler (gcc) found")
    tmp = output + ".tmp"
    subprocess.run([cc, *CFLAGS, source, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, output)
    return output


def _as_bits(a, name: str) -> np.ndarray:
    """bf16 tensor/array -> contiguous uint16 numpy array of its bit patterns."""
    if hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch

        a = a.detach().to("cpu").contiguous().view(torch.int16).numpy()
    a = np.asarray(a)
    if a.dtype not in (np.uint16, np.int16):
        raise TypeError(f"oracle: {name} must hold bf16 bit patterns (uint16), got {a.dtype}")
    return np.ascontiguousarray(a).view(np.uint16)


class Oracle:
    """Handle on one compiled oracle library (the default one, or a test build)."""

    def __init__(self, library: str = LIBRARY):
        self.path = library
        lib = ctypes.CDLL(library)
        p_u16 = ctypes.POINTER(ctypes.c_uint16)
        p_i64 = ctypes.POINTER(ctypes.c_int64)
        p_f64 = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_gqa_causal_varlen.argtypes = [p_u16, p_u16, p_u16, p_i64, i64, i64, i64, i64,
                                                 ctypes.c_float, p_i64, i64, p_f64, p_f64,
                                                 ctypes.c_int]
        lib.oracle_gqa_causal_varlen.restype = ctypes.c_int
        lib.oracle_gqa_causal_keyrange.argtypes = [p_u16, p_u16, p_u16, i64, i64, i64, i64,
                                                   ctypes.c_float, i64, i64, p_i64, i64, p_f64,
                                                   p_f64, ctypes.c_int]
        lib.oracle_gqa_causal_keyrange.restype = ctypes.c_int
        lib.oracle_gqa_bidirectional.argtypes = [p_u16, p_u16, p_u16, i64, i64, i64, i64,
                                                 ctypes.c_float, p_i64, i64, p_f64, p_f64,
                                                 ctypes.c_int]
        lib.oracle_gqa_bidirectional.restype = ctypes.c_int
        lib.oracle_qk_norm_rope.argtypes = [p_u16, i64, i64, i64, p_u16, ctypes.c_double,
                                            ctypes.c_int, ctypes.c_double, p_i64, p_f64]
        lib.oracle_qk_norm_rope.restype = ctypes.c_int
        lib.oracle_threads.argtypes = [ctypes.c_int]
        lib.oracle_threads.restype = ctypes.c_int
        self._lib = lib

    def threads(self, requested: int = 0) -> int:
        """Threads a call with ``threads=requested`` uses."""
        return int(self._lib.oracle_threads(int(requested)))

    def gqa_causal_varlen(self, q, k, v, cu_seqlens, scale: float, tokens=None, threads: int = 0):
        """Packed batch: q [T,Hq,D], k/v [T,Hkv,D] bf16 bits; cu_seqlens [n+1].

        Returns ``(o, lse)``: o float64 [ntok, Hq, D], lse float64 [Hq, ntok]
        for the packed query positions ``tokens`` (default: all T).
        """
        q = _as_bits(q, "q")
        k = _as_bits(k, "k")
        v = _as_bits(v, "v")
        if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape:
            raise ValueError("oracle: q must be [T,Hq,D] and k, v [T,Hkv,D]")
        T, Hq, D = q.shape
        if k.shape[0] != T or k.shape[2] != D:
            raise ValueError("oracle: k/v token count or head dim differs from q")
        Hkv = k.shape[1]
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        if cu.ndim != 1 or cu.size < 2 or cu[-1] != T:
            raise ValueError("oracle: cu_seqlens must have n+1 entries ending at T")
        if tokens is None:
            tokens = np.arange(T, dtype=np.int64)
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).reshape(-1))
        n = tokens.size
        o = np.empty((n, Hq, D), dtype=np.float64)
        lse = np.empty((Hq, n), dtype=np.float64)
        if n == 0:
            return o, lse

        def ptr(a, t):
            return a.ctypes.data_as(ctypes.POINTER(t))

        rc = self._lib.oracle_gqa_causal_varlen(
            ptr(q, ctypes.c_uint16), ptr(k, ctypes.c_uint16), ptr(v, ctypes.c_uint16),
            ptr(cu, ctypes.c_int64), cu.size - 1, Hq, Hkv, D, float(np.float32(scale)),
            ptr(tokens, ctypes.c_int64), n, ptr(o, ctypes.c_double), ptr(lse, ctypes.c_double),
            int(threads))
        if rc != 0:
            raise ValueError(f"oracle: invalid arguments (code {rc})")
        return o, lse

    def gqa_causal(self, q, k, v, scale: float, tokens=None, threads: int = 0):
        """One sequence: q [S,Hq,D], k/v [S,Hkv,D] bf16 bits -> (o, lse)."""
        return self.gqa_causal_varlen(q, k, v, [0, int(q.shape[0])], scale, tokens=tokens,
                                      threads=threads)

    def gqa_bidirectional(self, q, k, v, scale: float, tokens=None, threads: int = 0):
        """One sequence, no causal mask: every query sees all S keys -> (o, lse)."""
        q = _as_bits(q, "q")
        k = _as_bits(k, "k")
        v = _as_bits(v, "v")
        if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape or k.shape[0] != q.shape[0] \
                or k.shape[2] != q.shape[2]:
            raise ValueError("oracle: q must be [S,Hq,D] and k, v [S,Hkv,D]")
        S, Hq, D = q.shape
        Hkv = k.shape[1]
        if tokens is None:
            tokens = np.arange(S, dtype=np.int64)
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).reshape(-1))
        n = tokens.size
        o = np.empty((n, Hq, D), dtype=np.float64)
        lse = np.empty((Hq, n), dtype=np.float64)
        if n == 0:
            return o, lse

        def ptr(a, t):
            return a.ctypes.data_as(ctypes.POINTER(t))

        rc = self._lib.oracle_gqa_bidirectional(
            ptr(q, ctypes.c_uint16), ptr(k, ctypes.c_uint16), ptr(v, ctypes.c_uint16), S, Hq,
            Hkv, D, float(np.float32(scale)), ptr(tokens, ctypes.c_int64), n,
            ptr(o, ctypes.c_double), ptr(lse, ctypes.c_double), int(threads))
        if rc != 0:
            raise ValueError(f"oracle: invalid arguments (code {rc})")
        return o, lse

    def qk_norm_rope(self, x, weight=None, eps: float = 1e-6, rope: bool = True,
                     theta: float = 1e6, positions=None):
        """Q/K prologue of one tensor x [S, H, D] (bf16 bits): optional RMS norm with the
        [D] bf16 weight, optional rotate-half RoPE at positions (default: token index).
        Returns float64 [S, H, D]."""
        x = _as_bits(x, "x")
        if x.ndim != 3:
            raise ValueError("oracle: x must be [S, H, D]")
        S, H, D = x.shape
        out = np.empty((S, H, D), dtype=np.float64)
        w = None if weight is None else _as_bits(weight, "weight").reshape(-1)
        if w is not None and w.size != D:
            raise ValueError("oracle: weight must hold D values")
        pos = None
        if positions is not None:
            pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64).reshape(-1))
            if pos.size != S:
                raise ValueError("oracle: positions must hold S values")

        def ptr(a, t):
            return None if a is None else a.ctypes.data_as(ctypes.POINTER(t))

        rc = self._lib.oracle_qk_norm_rope(ptr(x, ctypes.c_uint16), S, H, D,
                                           ptr(w, ctypes.c_uint16), float(eps), int(bool(rope)),
                                           float(theta), ptr(pos, ctypes.c_int64),
                                           ptr(out, ctypes.c_double))
        if rc != 0:
            raise ValueError(f"oracle: invalid arguments (code {rc})")
        return out

    def gqa_causal_keyrange(self, q, k, v, scale: float, key_begin: int, key_end: int,
                            tokens=None, threads: int = 0):
        """One sequence, keys restricted to [key_begin, key_end) (and j <= i).

        Returns ``(o, lse)`` like :meth:`gqa_causal`; rows with no key in range
        get o = 0 and lse = -inf.
        """
        q = _as_bits(q, "q")
        k = _as_bits(k, "k")
        v = _as_bits(v, "v")
        if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape or k.shape[0] != q.shape[0] \
                or k.shape[2] != q.shape[2]:
            raise ValueError("oracle: q must be [S,Hq,D] and k, v [S,Hkv,D]")
        S, Hq, D = q.shape
        Hkv = k.shape[1]
        if tokens is None:
            tokens = np.arange(S, dtype=np.int64)
        tokens = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64).reshape(-1))
        n = tokens.size
        o = np.empty((n, Hq, D), dtype=np.float64)
        lse = np.empty((Hq, n), dtype=np.float64)
        if n == 0:
            return o, lse

        def ptr(a, t):
            return a.ctypes.data_as(ctypes.POINTER(t))

        rc = self._lib.oracle_gqa_causal_keyrange(
            ptr(q, ctypes.c_uint16), ptr(k, ctypes.c_uint16), ptr(v, ctypes.c_uint16), S, Hq,
            Hkv, D, float(np.float32(scale)), int(key_begin), int(key_end),
            ptr(tokens, ctypes.c_int64), n, ptr(o, ctypes.c_double), ptr(lse, ctypes.c_double),
            int(threads))
        if rc != 0:
            raise ValueError(f"oracle: invalid arguments (code {rc})")
        return o, lse


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    """The oracle built from ``oracle.c``; compiled on first use if missing or stale."""
    global _DEFAULT
    if _DEFAULT is None:
        if (not os.path.exists(LIBRARY)
                or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build()
        _DEFAULT = Oracle(LIBRARY)
    return _DEFAULT


def gqa_causal(q, k, v, scale: float, tokens=None, threads: int = 0):
    """Fixed-length causal GQA in fp64; see :meth:`Oracle.gqa_causal`."""
    return default().gqa_causal(q, k, v, scale, tokens=tokens, threads=threads)


def gqa_causal_varlen(q, k, v, cu_seqlens, scale: float, tokens=None, threads: int = 0):
    """Packed-batch causal GQA in fp64; see :meth:`Oracle.gqa_causal_varlen`."""
    return default().gqa_causal_varlen(q, k, v, cu_seqlens, scale, tokens=tokens,
                                       threads=threads)


def gqa_causal_keyrange(q, k, v, scale: float, key_begin: int, key_end: int, tokens=None,
                        threads: int = 0):
    """Attention over a key range; see :meth:`Oracle.gqa_causal_keyrange`."""
    return default().gqa_causal_keyrange(q, k, v, scale, key_begin, key_end, tokens=tokens,
                                         threads=threads)


def gqa_bidirectional(q, k, v, scale: float, tokens=None, threads: int = 0):
    """Non-causal GQA in fp64; see :meth:`Oracle.gqa_bidirectional`."""
    return default().gqa_bidirectional(q, k, v, scale, tokens=tokens, threads=threads)


def qk_norm_rope(x, weight=None, eps: float = 1e-6, rope: bool = True, theta: float = 1e6,
                 positions=None):
    """Q/K RMS norm + RoPE prologue in fp64; see :meth:`Oracle.qk_norm_rope`."""
    return default().qk_norm_rope(x, weight=weight, eps=eps, rope=rope, theta=theta,
                                  positions=positions)


def pool_tokens(x, begin: int, end: int, factor: int):
    """Sequence-axis average pooling of the token span [begin, end) of x [T, C] (bf16 bits).

    The issue "Qwen text encoder: sequence exceeds Metal threadgroup memory with reference
    video + ref images (>=150 frames)", "Suggested fix directions" (second direction),
    shortens the prompt by pooling the reference-video tokens before the encoder.  The
    plainest reading, taken here: consecutive groups of ``factor`` tokens of the span
    are replaced by their mean (the last group may be shorter and averages what it has);
    tokens outside the span are kept.  Written out in float64 with plain loops over the
    output rows.  Returns float64 [T - L + ceil(L / factor), C], L = end - begin.
    """
    x = _as_bits(x, "x")
    if x.ndim != 2:
        raise ValueError("oracle: x must be [T, C]")
    T, C = x.shape
    if not (0 <= begin <= end <= T) or factor < 1:
        raise ValueError("oracle: need 0 <= begin <= end <= T and factor >= 1")
    xf = (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    L = end - begin
    groups = (L + factor - 1) // factor
    out = np.empty((T - L + groups, C), dtype=np.float64)
    row = 0
    for t in range(begin):
        out[row] = xf[t]
        row += 1
    for gi in range(groups):
        a = begin + gi * factor
        b = min(a + factor, end)
        acc = np.zeros(C, dtype=np.float64)
        for t in range(a, b):
            acc += xf[t]
        out[row] = acc / (b - a)
        row += 1
    for t in range(end, T):
        out[row] = xf[t]
        row += 1
    return out


def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint key sets into the result over their union.

    o_parts: [n, ntok, Hq, D], lse_parts: [n, Hq, ntok] (float64; empty parts carry
    lse = -inf).  The softmax over a union of disjoint sets weighs part c by
    exp(lse_c) / sum_c' exp(lse_c'), and the union's log-sum-exp is the log of that
    sum; the largest lse is factored out so that no exponential overflows.  Rows with
    every part empty come out as o = 0, lse = -inf.
    Returns ``(o, lse)`` with shapes [ntok, Hq, D] and [Hq, ntok].
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)                                  # [Hq, ntok]
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_parts - m_safe)                             # exp(-inf) = 0
    total = w.sum(axis=0)                                      # [Hq, ntok]
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(total > 0, m_safe + np.log(total), -np.inf)
        frac = np.where(total > 0, w / np.where(total > 0, total, 1.0), 0.0)   # [n, Hq, ntok]
    # O[t, h, :] = sum_c frac[c, h, t] * o_parts[c, t, h, :]
    o = (frac.transpose(0, 2, 1)[..., None] * o_parts).sum(axis=0)
    return o, lse


def threads(requested: int = 0) -> int:
    return default().threads(requested)
