"""Seeded synthetic inputs for the causal GQA forward.

This module holds no attention arithmetic: it draws random bf16 tensors and
packs sequence offsets.  Both the oracle side (tests, CPU baseline) and the
HIP side (tests, benchmark) take their inputs from here, so the two always see
the same bits.

Where the shapes come from.  The h3.c issue "Qwen text encoder: sequence
exceeds Metal threadgroup memory with reference video + ref images (>=150
frames)" lists, in its table under "Systematic single-variable experiments",
the prompt lengths at which the old kernel failed (8199, 10231, 8184, 8510
tokens) and, under "Trigger condition", the ~7700-token ceiling the 32 KB
threadgroup row imposed.  The real inputs there are Qwen encoder activations of
a prompt + images + video, which need the model's weights and media; seeded
N(0,1) bf16 values stand in for them.  Head counts (64 query / 8 KV heads, head
dim 128) and the stress recipe are this build's choice of a Qwen-style encoder
layer; the pages do not print them.

bf16 values are produced by rounding float32 draws to nearest-even on the bit
pattern, and are handed around as ``numpy.uint16`` bit patterns.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs here are always finite, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim) as the fp32 value both sides use."""
    return float(np.float32(1.0) / np.sqrt(np.float32(head_dim)))


@dataclass(frozen=True)
class Workload:
    """A named synthetic configuration.

    ``seqlens`` has one entry for a fixed-length call and several for a
    packed (varlen) batch.  ``kind`` is ``"normal"`` (Q, K, V ~ N(0,1)) or
    ``"stress"`` (Q, K ~ 4 N(0,1), V ~ U(-1,1), 5% of key rows replaced by one
    shared spike vector, identical across KV heads).
    """

    name: str
    seqlens: tuple
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seed: int
    kind: str = "normal"
    varlen: bool = False
    causal: bool = True
    note: str = field(default="", compare=False)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def scale(self) -> float:
        return default_scale(self.head_dim)

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(np.asarray(self.seqlens, dtype=np.int64))]).astype(
            np.int64)

    def kept_pairs_per_head(self) -> int:
        """(query, key) pairs a query head attends to: key <= query inside each sequence,
        or every pair of the sequence for the bidirectional form."""
        if not self.causal:
            return int(sum(s * s for s in self.seqlens))
        return int(sum(s * (s + 1) // 2 for s in self.seqlens))

    def flop(self) -> int:
        """Algorithmic FLOP: 2*D for Q.K plus 2*D for P.V per kept pair and query head."""
        return 4 * self.head_dim * self.n_q_heads * self.kept_pairs_per_head()

    causal_flop = flop

    def algorithmic_bytes(self) -> int:
        """Q, K, V read once and O (bf16), LSE (fp32) written once."""
        T = self.total_tokens
        return (2 * T * self.n_q_heads * self.head_dim * 2
                + 2 * T * self.n_kv_heads * self.head_dim * 2
                + 4 * T * self.n_q_heads)


# Sequence lengths at which the threadgroup-row kernel failed (issue table).
FAILING_LENGTHS = (8184, 8199, 8510, 10231)

WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_s256_h8kv2_d64", (256,), 8, 2, 64, seed=1,
                 note="small case the oracle finishes in well under a second"),
        Workload("under_cap_s7680", (7680,), 64, 8, 128, seed=2,
                 note="just under the old ~7700-token ceiling"),
        Workload("failing_s10231", (10231,), 64, 8, 128, seed=3,
                 note="the failing prompt length; 10231 is not a multiple of any tile"),
        Workload("varlen_4x_t35124", (8184, 8199, 8510, 10231), 64, 8, 128, seed=4,
                 varlen=True, note="the four failing lengths packed into one batch"),
        Workload("stress_s32768", (32768,), 64, 8, 128, seed=5, kind="stress",
                 note="large logits and tied spike keys at long length"),
    )
}

# Bidirectional (non-causal) attention at the row counts the vpipe issue's logs show for
# the video DiT ("first forward at 19316 rows", "a 34121-row forward").  The pages print no
# head counts for the DiT; 32 heads of dim 128, one KV head per query head (MHA), is this
# build's choice of a DiT layer.
DIT_WORKLOADS = {
    w.name: w
    for w in (
        Workload("dit_s19316_h32_d128", (19316,), 32, 32, 128, seed=7, causal=False,
                 note="bidirectional, the DiT forward's 19316 rows"),
        Workload("dit_s34121_h32_d128", (34121,), 32, 32, 128, seed=8, causal=False,
                 note="bidirectional, the DiT forward's 34121 rows"),
    )
}

# Shapes for the split-KV path only (not the pages' workloads): with a single KV head the
# single-dispatch kernel has one workgroup per query block, 128 at S=4096, too few for
# 256 compute units; splitting each block's KV range multiplies the workgroups.
SPLITKV_WORKLOADS = {
    w.name: w
    for w in (
        Workload("few_heads_s4096_h8kv1", (4096,), 8, 1, 128, seed=6,
                 note="one KV head: too few query blocks to fill the GPU without splits"),
    )
}

ALL_WORKLOADS = {**WORKLOADS, **DIT_WORKLOADS, **SPLITKV_WORKLOADS}

PRIMARY = "failing_s10231"


def normal_inputs(seed: int, T: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                  sigma: float = 1.0):
    """Q [T,Hq,D], K, V [T,Hkv,D] as bf16 bits, i.i.d. sigma*N(0,1), drawn in that order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for heads in (n_q_heads, n_kv_heads, n_kv_heads):
        x = rng.standard_normal((T, heads, head_dim), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out.append(f32_to_bf16_bits(x))
    return tuple(out)


def stress_inputs(seed: int, T: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                  spike_fraction: float = 0.05):
    """Q, K ~ 4 N(0,1); V ~ U(-1,1); floor(spike_fraction*T) key rows = one shared vector.

    The spike vector is 4 N(0,1) rounded to bf16 and written to the chosen token
    positions of every KV head, so the spike keys tie exactly.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = f32_to_bf16_bits(rng.standard_normal((T, n_q_heads, head_dim), dtype=np.float32)
                         * np.float32(4))
    k = f32_to_bf16_bits(rng.standard_normal((T, n_kv_heads, head_dim), dtype=np.float32)
                         * np.float32(4))
    v = f32_to_bf16_bits(rng.random((T, n_kv_heads, head_dim), dtype=np.float32)
                         * np.float32(2) - np.float32(1))
    n_spike = int(np.floor(spike_fraction * T))
    positions = np.sort(rng.permutation(T)[:n_spike])
    spike = f32_to_bf16_bits(rng.standard_normal(head_dim, dtype=np.float32) * np.float32(4))
    k[positions, :, :] = spike[None, None, :]
    return q, k, v, positions


def device_normal_bf16(seed: int, shapes, device="cuda"):
    """bf16 tensors of N(0,1) values drawn on the GPU with torch's seeded generator, one per
    shape in ``shapes`` (in that order).  For sizes where host generation would dominate a
    test (gigabytes); the oracle receives the same values by copying the bits back."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return tuple(torch.randn(tuple(sh), generator=g, device=device, dtype=torch.float32)
                 .to(torch.bfloat16) for sh in shapes)


def generate(w: Workload) -> dict:
    """All inputs of a workload: q, k, v (uint16 bits), cu_seqlens, scale."""
    T = w.total_tokens
    out = {"cu_seqlens": w.cu_seqlens, "scale": w.scale}
    if w.kind == "normal":
        out["q"], out["k"], out["v"] = normal_inputs(w.seed, T, w.n_q_heads, w.n_kv_heads,
                                                     w.head_dim)
    elif w.kind == "stress":
        out["q"], out["k"], out["v"], out["spike_positions"] = stress_inputs(
            w.seed, T, w.n_q_heads, w.n_kv_heads, w.head_dim)
    else:
        raise ValueError(f"unknown workload kind {w.kind!r}")
    return out


def block_tokens(seqlens, block: int = 32) -> np.ndarray:
    """One packed query position per ``block``-token query block of every sequence, its
    offset in the block moving with the block index: local position block*b + (b mod block),
    clamped to the sequence's last token."""
    picks = []
    start = 0
    for s in seqlens:
        for b in range((s + block - 1) // block):
            picks.append(start + min(block * b + b % block, s - 1))
        start += s
    return np.unique(np.asarray(picks, dtype=np.int64))


def sample_tokens(seqlens, n_random: int, seed: int, tile: int = 64) -> np.ndarray:
    """Packed query positions to check at full size.

    Every sequence contributes its first and last two tokens and the tokens on
    either side of each multiple of ``tile`` near its start and end; then
    ``n_random`` positions are drawn uniformly over the whole batch.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    picks = []
    start = 0
    for s in seqlens:
        if s == 0:
            continue
        local = {0, 1, s - 2, s - 1, tile - 1, tile, 2 * tile - 1, 2 * tile,
                 (s // tile) * tile - 1, (s // tile) * tile, s // 2}
        picks.extend(start + t for t in local if 0 <= t < s)
        start += s
    T = start
    if T > 0 and n_random > 0:
        picks.extend(rng.integers(0, T, size=n_random).tolist())
    return np.unique(np.asarray(picks, dtype=np.int64))
