"""Checks that tie the fp64 oracle to facts other than its own formula.

Each ``pin_*`` function takes an :class:`oracle.Oracle` and raises
``AssertionError`` if the oracle disagrees with:

* brute force on tiny inputs (dense float64 matrix products with a masked
  upper triangle),
* a library routine the GQA case reduces to (torch's float64
  ``scaled_dot_product_attention`` with K/V heads repeated per group),
* closed forms (Q = 0 gives the prefix mean of V and LSE = ln(i+1); row 0 is
  V[0] exactly; identical keys give the prefix mean; one overwhelming key
  gives that key's value row exactly; a constant value head gives that
  constant),
* invariants (future tokens never change earlier rows; a packed batch equals
  its sequences run one at a time; GQA equals MHA with K/V repeated),
* the exact result (50-digit mpmath) on sampled rows, including logits large
  enough to overflow exp() without the max shift,
* for the split-KV building blocks: attention over a key range against dense
  masked matrices, a one-key range in closed form, and the merge of partials
  over a partition of the keys against the full result,
* for the bidirectional (non-causal) form: dense matrices, torch's float64
  SDPA without the causal flag, Q = 0 (mean of all values, LSE = ln S), and
  invariance under a permutation of the key/value rows,
* for the Q/K prologue: torch's float64 rms_norm, the mean-square closed form
  and scale invariance of the norm, RoPE on unit vectors (the rotate-half
  convention and the frequency exponent) and RoPE's relative-position and
  length-preserving properties,
* for token pooling: identity at factor 1, equal tokens, numpy's reshape-mean
  on divisible spans, a linear ramp's group midpoints, the output length.

``tests/test_oracle_pins.py`` runs them on the real oracle and
``tests/test_oracle_mutations.py`` checks that each planted mistake in a copy
of ``oracle.c`` trips at least one of them.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from workloads import bf16_bits_to_f32, default_scale, f32_to_bf16_bits, normal_inputs


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def pin_brute_force_dense(orc):
    """Dense masked softmax attention, one matrix per head, on tiny shapes."""
    cases = [  # S, Hq, Hkv, D, seed, sigma
        (1, 1, 1, 8, 10, 1.0),
        (7, 4, 2, 8, 11, 1.0),
        (33, 8, 2, 16, 12, 2.0),
        (64, 8, 8, 16, 13, 1.0),
        (48, 8, 1, 64, 14, 3.0),
    ]
    for S, Hq, Hkv, D, seed, sigma in cases:
        q, k, v = normal_inputs(seed, S, Hq, Hkv, D, sigma=sigma)
        scale = default_scale(D)
        o, lse = orc.gqa_causal(q, k, v, scale)
        Q, K, V = _f64(q), _f64(k), _f64(v)
        G = Hq // Hkv
        above_diagonal = np.triu(np.ones((S, S), dtype=bool), 1)
        for h in range(Hq):
            g = h // G
            X = float(np.float32(scale)) * (Q[:, h, :] @ K[:, g, :].T)
            X[above_diagonal] = -np.inf
            m = X.max(axis=1, keepdims=True)
            P = np.exp(X - m)
            den = P.sum(axis=1, keepdims=True)
            np.testing.assert_allclose(o[:, h, :], (P / den) @ V[:, g, :], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[h], m[:, 0] + np.log(den[:, 0]), rtol=1e-12,
                                       atol=1e-12)


def pin_torch_sdpa_float64(orc):
    """GQA = MHA after repeating each KV head G times; MHA is torch's causal SDPA."""
    import torch
    import torch.nn.functional as F

    cases = [(50, 8, 2, 32, 20), (17, 6, 3, 16, 21), (40, 4, 4, 8, 22), (29, 8, 1, 64, 23)]
    for S, Hq, Hkv, D, seed in cases:
        q, k, v = normal_inputs(seed, S, Hq, Hkv, D)
        scale = default_scale(D)
        o, _ = orc.gqa_causal(q, k, v, scale)
        G = Hq // Hkv
        Q = torch.from_numpy(_f64(q)).permute(1, 0, 2).unsqueeze(0)
        K = torch.from_numpy(_f64(k)).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
        V = torch.from_numpy(_f64(v)).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0)
        ref = F.scaled_dot_product_attention(Q, K, V, is_causal=True,
                                             scale=float(np.float32(scale)))
        np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def pin_zero_query_prefix_mean(orc):
    """Q = 0: every visible score is 0, so O[i] = mean(V[0..i]) and LSE[i] = ln(i+1)."""
    S, Hq, Hkv, D = 70, 8, 2, 16
    _, k, v = normal_inputs(30, S, Hq, Hkv, D)
    q = np.zeros((S, Hq, D), dtype=np.uint16)
    o, lse = orc.gqa_causal(q, k, v, 0.25)
    V = _f64(v)
    prefix_mean = np.cumsum(V, axis=0) / np.arange(1, S + 1)[:, None, None]
    G = Hq // Hkv
    for h in range(Hq):
        np.testing.assert_allclose(o[:, h, :], prefix_mean[:, h // G, :], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[h], np.log(np.arange(1, S + 1)), rtol=0, atol=1e-13)


def pin_row_zero(orc):
    """Row 0 sees only key 0: O[0,h] = V[0,g] exactly and LSE[h,0] = scale * q0.k0."""
    S, Hq, Hkv, D = 5, 8, 2, 64
    q, k, v = normal_inputs(31, S, Hq, Hkv, D, sigma=2.0)
    scale = default_scale(D)
    o, lse = orc.gqa_causal(q, k, v, scale)
    Q, K, V = _f64(q), _f64(k), _f64(v)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        assert np.array_equal(o[0, h, :], V[0, g, :]), f"row 0 of head {h} is not V[0]"
        exact = Fraction(float(np.float32(scale))) * sum(
            Fraction(float(a)) * Fraction(float(b)) for a, b in zip(Q[0, h], K[0, g]))
        assert abs(lse[h, 0] - float(exact)) <= 1e-14 * max(1.0, abs(float(exact)))


def pin_identical_keys_prefix_mean(orc):
    """All keys equal: each visible score is the same, so O[i] = mean(V[0..i])."""
    S, Hq, Hkv, D = 40, 4, 2, 32
    q, k, v = normal_inputs(32, S, Hq, Hkv, D)
    k[:] = k[0:1]  # every token carries token 0's keys
    scale = default_scale(D)
    o, lse = orc.gqa_causal(q, k, v, scale)
    Q, K, V = _f64(q), _f64(k), _f64(v)
    prefix_mean = np.cumsum(V, axis=0) / np.arange(1, S + 1)[:, None, None]
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        np.testing.assert_allclose(o[:, h, :], prefix_mean[:, g, :], rtol=1e-11, atol=1e-13)
        x = float(np.float32(scale)) * (Q[:, h, :] @ K[0, g, :])
        np.testing.assert_allclose(lse[h], x + np.log(np.arange(1, S + 1)), rtol=1e-12,
                                   atol=1e-12)


def pin_overwhelming_key(orc):
    """One key j* scores 1024 above all others: rows i >= j* return V[j*] exactly.

    Rows before j* see only zero scores and return the prefix mean of V.
    """
    S, Hq, Hkv, D, jstar = 24, 2, 1, 8, 9
    q = np.zeros((S, Hq, D), dtype=np.float32)
    q[:, :, 0] = 1.0
    k = np.zeros((S, Hkv, D), dtype=np.float32)
    k[:, :, 1] = 1.0               # ordinary keys: orthogonal to every query
    k[jstar, :, 0] = 1024.0        # the overwhelming key
    rng = np.random.Generator(np.random.PCG64(33))
    v = rng.standard_normal((S, Hkv, D), dtype=np.float32)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    o, lse = orc.gqa_causal(qb, kb, vb, 1.0)
    V = _f64(vb)
    for h in range(Hq):
        for i in range(S):
            if i >= jstar:
                assert np.array_equal(o[i, h], V[jstar, 0]), f"row {i} head {h} not one-hot"
                assert lse[h, i] == 1024.0
            else:
                np.testing.assert_allclose(o[i, h], V[: i + 1, 0].mean(axis=0), rtol=1e-12,
                                           atol=1e-14)
                assert abs(lse[h, i] - np.log(i + 1)) <= 1e-13


def pin_constant_value_heads(orc):
    """V[:, g, :] = c_g: the weights sum to one, so head h returns c_{h // G}."""
    S, Hq, Hkv, D = 45, 8, 4, 16
    q, k, _ = normal_inputs(34, S, Hq, Hkv, D, sigma=2.0)
    consts = np.array([0.5, -1.25, 3.0, 7.5], dtype=np.float32)
    v = _bits(np.broadcast_to(consts[None, :, None], (S, Hkv, D)))
    o, _ = orc.gqa_causal(q, k, v, default_scale(D))
    G = Hq // Hkv
    for h in range(Hq):
        np.testing.assert_allclose(o[:, h, :], consts[h // G], rtol=1e-14, atol=0)


def pin_gqa_equals_repeated_mha(orc):
    """GQA gives bit-identical results to MHA on K/V repeated G times per head."""
    S, Hq, Hkv, D = 37, 8, 2, 16
    q, k, v = normal_inputs(35, S, Hq, Hkv, D)
    G = Hq // Hkv
    scale = default_scale(D)
    o1, l1 = orc.gqa_causal(q, k, v, scale)
    o2, l2 = orc.gqa_causal(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_causality(orc):
    """Changing tokens >= t (Q, K and V) leaves every row < t bit-identical."""
    S, Hq, Hkv, D = 60, 8, 2, 16
    q, k, v = normal_inputs(36, S, Hq, Hkv, D)
    scale = default_scale(D)
    o1, l1 = orc.gqa_causal(q, k, v, scale)
    for t in (1, 17, 59):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        noise = normal_inputs(37 + t, S - t, Hq, Hkv, D, sigma=3.0)
        q2[t:], k2[t:], v2[t:] = noise
        o2, l2 = orc.gqa_causal(q2, k2, v2, scale)
        assert np.array_equal(o1[:t], o2[:t]) and np.array_equal(l1[:, :t], l2[:, :t])
        assert not np.array_equal(o1[t:], o2[t:])


def pin_varlen_is_concatenation(orc):
    """A packed batch equals its sequences run one by one (bit-identical);
    zero-length sequences contribute nothing."""
    lens = [13, 0, 1, 40, 0, 27]
    Hq, Hkv, D = 8, 2, 16
    T = sum(lens)
    q, k, v = normal_inputs(40, T, Hq, Hkv, D)
    scale = default_scale(D)
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, lse = orc.gqa_causal_varlen(q, k, v, cu, scale)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        o1, l1 = orc.gqa_causal(q[a:b], k[a:b], v[a:b], scale)
        assert np.array_equal(o[a:b], o1) and np.array_equal(lse[:, a:b], l1)


def _exact_row(Q, K, V, h, g, i, first, scale, mp):
    """Row i of head h over keys first..i with mpmath at the working precision."""
    s = mp.mpf(float(np.float32(scale)))
    xs = [s * mp.fsum(mp.mpf(float(a)) * mp.mpf(float(b)) for a, b in zip(Q[i, h], K[j, g]))
          for j in range(first, i + 1)]
    m = max(xs)
    w = [mp.exp(x - m) for x in xs]
    den = mp.fsum(w)
    o = [mp.fsum(w[t] * mp.mpf(float(V[first + t, g, d])) for t in range(len(w))) / den
         for d in range(V.shape[2])]
    return o, m + mp.log(den)


def pin_exact_rows_mpmath(orc):
    """50-digit results on sampled rows: the oracle's own error is ~1e-15.

    The second case has logits near +-1000, where exp() overflows in double
    unless the running maximum is subtracted first."""
    import mpmath

    mp = mpmath.mp
    mp.dps = 50
    cases = [  # S, Hq, Hkv, D, seed, sigma, rows
        (96, 4, 2, 64, 50, 1.0, (0, 1, 37, 95)),
        (64, 2, 1, 64, 51, 16.0, (0, 5, 63)),
    ]
    for S, Hq, Hkv, D, seed, sigma, rows in cases:
        q, k, v = normal_inputs(seed, S, Hq, Hkv, D, sigma=sigma)
        v = normal_inputs(seed + 100, S, Hq, Hkv, D)[2]
        scale = default_scale(D)
        o, lse = orc.gqa_causal(q, k, v, scale, tokens=np.array(rows))
        Q, K, V = _f64(q), _f64(k), _f64(v)
        G = Hq // Hkv
        for ri, i in enumerate(rows):
            for h in range(Hq):
                eo, el = _exact_row(Q, K, V, h, h // G, i, 0, scale, mp)
                eo = np.array([float(x) for x in eo])
                assert np.all(np.abs(o[ri, h] - eo) <= 1e-13), (i, h)
                assert abs(lse[h, ri] - float(el)) <= 1e-13 * max(1.0, abs(float(el))), (i, h)


def pin_keyrange_brute_force(orc):
    """Attention over a key range [kb, ke) (and j <= i) against dense masked matrices;
    rows with no key in range give O = 0, LSE = -inf."""
    cases = [  # S, Hq, Hkv, D, seed, kb, ke
        (40, 4, 2, 16, 70, 0, 40),
        (40, 4, 2, 16, 71, 7, 23),
        (33, 8, 1, 8, 72, 32, 33),
        (50, 2, 2, 64, 73, 10, 11),
        (20, 4, 4, 16, 74, 25, 30),     # entirely past the sequence: every row empty
    ]
    for S, Hq, Hkv, D, seed, kb, ke in cases:
        q, k, v = normal_inputs(seed, S, Hq, Hkv, D, sigma=1.5)
        scale = default_scale(D)
        o, lse = orc.gqa_causal_keyrange(q, k, v, scale, kb, ke)
        Q, K, V = _f64(q), _f64(k), _f64(v)
        G = Hq // Hkv
        i_idx, j_idx = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
        visible = (j_idx <= i_idx) & (j_idx >= kb) & (j_idx < ke)
        for h in range(Hq):
            g = h // G
            X = float(np.float32(scale)) * (Q[:, h, :] @ K[:, g, :].T)
            X = np.where(visible, X, -np.inf)
            for i in range(S):
                if not visible[i].any():
                    assert lse[h, i] == -np.inf and np.all(o[i, h] == 0.0), (seed, i, h)
                    continue
                m = X[i].max()
                w = np.exp(X[i] - m)
                assert abs(lse[h, i] - (m + np.log(w.sum()))) <= 1e-12 * max(1.0, abs(m)), (i, h)
                assert np.allclose(o[i, h], (w / w.sum()) @ V[:, g, :], rtol=1e-12, atol=1e-13)


def pin_merge_of_key_partition(orc):
    """Partials over a partition of the keys, merged, equal the full causal result: the
    softmax over a union of disjoint key sets is the exp(LSE)-weighted mix of the
    softmaxes over the parts."""
    cases = [  # S, Hq, Hkv, D, seed, sigma, cut points
        (64, 4, 2, 32, 80, 1.0, (16, 48)),
        (100, 8, 2, 16, 81, 3.0, (1, 2, 50, 99)),
        (37, 2, 1, 64, 82, 8.0, (36,)),       # large logits: merging needs the max shift
        (48, 4, 4, 16, 83, 1.0, (0, 48)),     # empty first and last parts
    ]
    for S, Hq, Hkv, D, seed, sigma, cuts in cases:
        q, k, v = normal_inputs(seed, S, Hq, Hkv, D, sigma=sigma)
        scale = default_scale(D)
        bounds = [0, *cuts, S]
        parts = [orc.gqa_causal_keyrange(q, k, v, scale, a, b) for a, b in zip(bounds, bounds[1:])]
        import oracle as _oracle

        o, lse = _oracle.merge_partials(np.stack([p[0] for p in parts]),
                                        np.stack([p[1] for p in parts]))
        o_ref, lse_ref = orc.gqa_causal(q, k, v, scale)
        assert np.allclose(lse, lse_ref, rtol=1e-13, atol=1e-12), seed
        assert np.allclose(o, o_ref, rtol=1e-12, atol=1e-12), seed


def pin_keyrange_single_key(orc):
    """A one-key range [j, j+1): rows i >= j return V[j] exactly and LSE = scale*q.k_j
    (the dot product exact in rational arithmetic); rows i < j are empty."""
    S, Hq, Hkv, D, j = 24, 4, 2, 16, 9
    q, k, v = normal_inputs(90, S, Hq, Hkv, D)
    scale = default_scale(D)
    o, lse = orc.gqa_causal_keyrange(q, k, v, scale, j, j + 1)
    Q, K, V = _f64(q), _f64(k), _f64(v)
    G = Hq // Hkv
    for i in range(S):
        for h in range(Hq):
            if i < j:
                assert lse[h, i] == -np.inf and np.all(o[i, h] == 0.0)
                continue
            g = h // G
            assert np.all(o[i, h] == V[j, g]), (i, h)
            dot = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(Q[i, h], K[j, g]))
            exact = float(Fraction(float(np.float32(scale))) * dot)
            assert abs(lse[h, i] - exact) <= 1e-14 * max(1.0, abs(exact)), (i, h)


def pin_bidirectional_brute_force(orc):
    """No causal mask: dense float64 matrices per head on tiny shapes."""
    cases = [(1, 2, 1, 8, 300, 1.0), (17, 4, 2, 16, 301, 2.0), (64, 8, 1, 64, 302, 1.0),
             (45, 4, 4, 32, 303, 4.0)]
    for S, Hq, Hkv, D, seed, sigma in cases:
        q, k, v = normal_inputs(seed, S, Hq, Hkv, D, sigma=sigma)
        scale = default_scale(D)
        o, lse = orc.gqa_bidirectional(q, k, v, scale)
        Q, K, V = _f64(q), _f64(k), _f64(v)
        G = Hq // Hkv
        for h in range(Hq):
            g = h // G
            X = float(np.float32(scale)) * (Q[:, h, :] @ K[:, g, :].T)
            m = X.max(axis=1, keepdims=True)
            W = np.exp(X - m)
            assert np.allclose(lse[h], (m[:, 0] + np.log(W.sum(axis=1))), rtol=1e-13, atol=1e-12)
            assert np.allclose(o[:, h, :], (W / W.sum(axis=1, keepdims=True)) @ V[:, g, :],
                               rtol=1e-12, atol=1e-13)


def pin_bidirectional_torch_sdpa(orc):
    """torch float64 scaled_dot_product_attention(is_causal=False), K/V repeated per group."""
    import torch

    S, Hq, Hkv, D = 50, 8, 2, 32
    q, k, v = normal_inputs(310, S, Hq, Hkv, D)
    scale = default_scale(D)
    o, _ = orc.gqa_bidirectional(q, k, v, scale)
    Q, K, V = (torch.from_numpy(_f64(x)).permute(1, 0, 2) for x in (q, k, v))
    K = K.repeat_interleave(Hq // Hkv, dim=0)
    V = V.repeat_interleave(Hq // Hkv, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q, K, V, is_causal=False, scale=float(np.float32(scale))).permute(1, 0, 2).numpy()
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)


def pin_bidirectional_zero_query(orc):
    """Q = 0: every row is the mean of all S value rows and LSE = ln S."""
    S, Hq, Hkv, D = 37, 4, 2, 16
    _, k, v = normal_inputs(320, S, Hq, Hkv, D)
    q = np.zeros((S, Hq, D), dtype=np.uint16)
    o, lse = orc.gqa_bidirectional(q, k, v, 0.25)
    V = _f64(v)
    for h in range(Hq):
        assert np.allclose(o[:, h, :], V[:, h // 2, :].mean(axis=0), rtol=0, atol=1e-14)
    assert np.allclose(lse, np.log(S), rtol=0, atol=1e-14)


def pin_bidirectional_key_permutation(orc):
    """Without a mask the keys form a set: permuting the K/V rows (the same permutation for
    both) changes O and LSE only by summation-order rounding."""
    S, Hq, Hkv, D = 60, 4, 2, 32
    q, k, v = normal_inputs(330, S, Hq, Hkv, D, sigma=2.0)
    scale = default_scale(D)
    o, lse = orc.gqa_bidirectional(q, k, v, scale)
    perm = np.random.Generator(np.random.PCG64(331)).permutation(S)
    o2, lse2 = orc.gqa_bidirectional(q, k[perm], v[perm], scale)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lse2, rtol=1e-13, atol=1e-12)


def pin_rmsnorm_torch(orc):
    """Norm only: torch's float64 rms_norm over the head dim with the same weight and eps."""
    import torch

    S, H, D = 9, 5, 64
    x = normal_inputs(500, S, H, 1, D, sigma=3.0)[0]
    w = _bits(np.random.Generator(np.random.PCG64(501)).uniform(0.5, 1.5, D))
    for eps in (1e-6, 0.5):
        out = orc.qk_norm_rope(x, weight=w, eps=eps, rope=False)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(_f64(x)), (D,),
                                           weight=torch.from_numpy(_f64(w)), eps=eps).numpy()
        assert np.allclose(out, ref, rtol=1e-13, atol=1e-14), eps


def pin_rmsnorm_closed_forms(orc):
    """Unit weight: mean(y^2) = m / (m + eps) with m = mean(x^2); eps = 0: scaling x by a
    power of two (exact in bf16) leaves y unchanged."""
    S, H, D = 4, 3, 128
    x = normal_inputs(510, S, H, 1, D)[0]
    ones = _bits(np.ones(D))
    eps = 0.25
    y = orc.qk_norm_rope(x, weight=ones, eps=eps, rope=False)
    m = (_f64(x) ** 2).mean(axis=2)
    assert np.allclose((y ** 2).mean(axis=2), m / (m + eps), rtol=1e-13)
    y0 = orc.qk_norm_rope(x, weight=ones, eps=0.0, rope=False)
    y1 = orc.qk_norm_rope(_bits(_f64(x) * 8.0), weight=ones, eps=0.0, rope=False)
    assert np.allclose(y0, y1, rtol=1e-14, atol=0)


def pin_rope_unit_vectors(orc):
    """RoPE on unit vectors e_i (i < D/2) at position p: the pair (i, i+D/2) becomes
    (cos a, sin a) with a = p * theta^(-2i/D), everything else stays 0; position 0 is the
    identity."""
    import math

    S, H, D, theta = 6, 1, 16, 10000.0
    half = D // 2
    for i in (0, 1, 5, half - 1):
        x = np.zeros((S, H, D), dtype=np.float32)
        x[:, :, i] = 1.0
        positions = np.array([0, 1, 2, 7, 100, 34120])
        z = orc.qk_norm_rope(_bits(x), rope=True, theta=theta, positions=positions)
        for t, p in enumerate(positions):
            a = p * theta ** (-2.0 * i / D)
            exp = np.zeros(D)
            exp[i], exp[i + half] = math.cos(a), math.sin(a)
            assert np.allclose(z[t, 0], exp, rtol=0, atol=1e-12), (i, p)


def pin_rope_relative_position(orc):
    """<rope(q, m), rope(k, n)> depends on m - n only, and rope keeps each pair's length."""
    S, H, D = 8, 2, 64
    q = normal_inputs(520, S, H, 1, D)[0]
    k = normal_inputs(521, S, H, 1, D)[0]
    base = np.arange(S)
    zq = orc.qk_norm_rope(q, rope=True, theta=1e6, positions=base)
    zk = orc.qk_norm_rope(k, rope=True, theta=1e6, positions=base[::-1].copy())
    zq2 = orc.qk_norm_rope(q, rope=True, theta=1e6, positions=base + 977)
    zk2 = orc.qk_norm_rope(k, rope=True, theta=1e6, positions=base[::-1] + 977)
    d1 = (zq * zk).sum(axis=2)
    d2 = (zq2 * zk2).sum(axis=2)
    assert np.allclose(d1, d2, rtol=1e-10, atol=1e-10)
    Q = _f64(q)
    pair_in = Q[..., : D // 2] ** 2 + Q[..., D // 2:] ** 2
    pair_out = zq[..., : D // 2] ** 2 + zq[..., D // 2:] ** 2
    assert np.allclose(pair_in, pair_out, rtol=1e-13, atol=1e-13)


def pin_pool_tokens(orc):
    """Token pooling: factor 1 is the identity; a span of equal tokens pools to that token;
    a divisible span equals numpy's reshape-mean; a linear ramp pools to the group
    midpoints (closed form); the output length is T - L + ceil(L/f)."""
    import oracle as _oracle

    rng = np.random.Generator(np.random.PCG64(700))
    T, C = 50, 24
    x = _bits(rng.standard_normal((T, C)).astype(np.float32))
    X = _f64(x)
    assert np.array_equal(_oracle.pool_tokens(x, 5, 40, 1), X)
    for begin, end, f in [(10, 34, 4), (0, 50, 5), (7, 7, 3), (3, 50, 7), (20, 29, 2)]:
        out = _oracle.pool_tokens(x, begin, end, f)
        L = end - begin
        assert out.shape == (T - L + -(-L // f), C)
        assert np.array_equal(out[:begin], X[:begin])
        assert np.array_equal(out[out.shape[0] - (T - end):], X[end:])
        if L % f == 0 and L > 0:
            ref = X[begin:end].reshape(L // f, f, C).mean(axis=1)
            assert np.allclose(out[begin:begin + L // f], ref, rtol=1e-15, atol=1e-15)
    same = np.tile(x[:1], (T, 1))
    assert np.array_equal(_oracle.pool_tokens(same, 4, 44, 6)[4:11], np.tile(X[:1], (7, 1)))
    ramp = _bits(np.tile(np.arange(T, dtype=np.float32)[:, None], (1, C)))
    out = _oracle.pool_tokens(ramp, 2, 47, 4)            # groups 2..5, 6..9, ..., 46
    mids = [(a + min(a + 4, 47) - 1) / 2.0 for a in range(2, 47, 4)]
    assert np.allclose(out[2:2 + len(mids), 0], mids, rtol=0, atol=1e-12)


ALL_PINS = [
    pin_brute_force_dense,
    pin_torch_sdpa_float64,
    pin_zero_query_prefix_mean,
    pin_row_zero,
    pin_identical_keys_prefix_mean,
    pin_overwhelming_key,
    pin_constant_value_heads,
    pin_gqa_equals_repeated_mha,
    pin_causality,
    pin_varlen_is_concatenation,
    pin_exact_rows_mpmath,
    pin_keyrange_brute_force,
    pin_merge_of_key_partition,
    pin_keyrange_single_key,
    pin_bidirectional_brute_force,
    pin_bidirectional_torch_sdpa,
    pin_bidirectional_zero_query,
    pin_bidirectional_key_permutation,
    pin_rmsnorm_torch,
    pin_rmsnorm_closed_forms,
    pin_rope_unit_vectors,
    pin_rope_relative_position,
    pin_pool_tokens,
]
