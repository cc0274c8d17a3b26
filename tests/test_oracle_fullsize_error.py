"""The oracle's own error at full size (CPU only).

A few rows of the S=10231 text-encoder workload and of the S=32768 stress workload (one of
them dominated by the tied spike keys) are recomputed independently of oracle.c:

  * each score's dot product from its exact terms: a product of two bf16 values is exact
    in double, and math.fsum returns the correctly rounded sum of the exact terms;
  * the softmax scale (the fp32 value widened), the max, the exponentials, their sum and
    the log in mpmath at 40 significant digits;
  * each output element as math.fsum of weight x value terms, where the weights are the
    40-digit probabilities rounded to double (one rounding per term, 1e-16 relative).

The oracle's O and LSE must agree with these to 1e-12 (absolute), which bounds the error
the oracle brings into every GPU parity comparison far below the tolerances used there.
"""

from __future__ import annotations

import math

import mpmath
import numpy as np
import pytest

import oracle
import workloads

TOL = 1e-12


def _bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _reference_row(q_row, k_rows, v_rows, scale_f32):
    """(O row, LSE, largest weight) of one causal row from its plain definition."""
    qd = _bits_to_f64(q_row)
    kd = _bits_to_f64(k_rows)
    vd = _bits_to_f64(v_rows)
    terms = kd * qd[None, :]                       # exact products
    dots = [math.fsum(r) for r in terms]
    with mpmath.workdps(40):
        scale = mpmath.mpf(float(np.float32(scale_f32)))
        x = [scale * mpmath.mpf(d) for d in dots]
        m = max(x)
        e = [mpmath.exp(xi - m) for xi in x]
        s = mpmath.fsum(e)
        lse = float(m + mpmath.log(s))
        p = np.array([float(ei / s) for ei in e])
    o = np.array([math.fsum(p * vd[:, d]) for d in range(vd.shape[1])])
    return o, lse, float(p.max()), p


def _check(inp, w, token, head):
    g = head // w.group
    o_ref, lse_ref = oracle.gqa_causal(inp["q"], inp["k"], inp["v"], w.scale,
                                       tokens=np.array([token]))
    o, lse, pmax, p = _reference_row(inp["q"][token, head], inp["k"][: token + 1, g],
                                     inp["v"][: token + 1, g], w.scale)
    err_o = float(np.max(np.abs(o_ref[0, head] - o)))
    err_l = abs(float(lse_ref[head, 0]) - lse)
    print(f"[oracle-error] {w.name} token {token} head {head}: max |dO| {err_o:.2e} "
          f"|dLSE| {err_l:.2e} (LSE {lse:.6f}, largest weight {pmax:.3f})", flush=True)
    assert err_o <= TOL and err_l <= TOL
    return p


@pytest.fixture(scope="module")
def text_encoder():
    w = workloads.ALL_WORKLOADS["failing_s10231"]
    return w, workloads.generate(w)


@pytest.fixture(scope="module")
def stress():
    w = workloads.ALL_WORKLOADS["stress_s32768"]
    return w, workloads.generate(w)


@pytest.mark.parametrize("token,head", [(10230, 0), (4097, 37)])
def test_oracle_error_s10231(text_encoder, token, head):
    w, inp = text_encoder
    _check(inp, w, token, head)


def test_oracle_error_stress_last_row(stress):
    w, inp = stress
    _check(inp, w, w.total_tokens - 1, 5)


def test_oracle_error_stress_spike_dominated_row(stress):
    """The late row whose query meets the tied spike keys hardest: their weights carry
    almost all of the softmax."""
    w, inp = stress
    T = w.total_tokens
    spike_rows = np.asarray(inp["spike_positions"])
    spike = _bits_to_f64(inp["k"][spike_rows[0], 0])
    late = np.arange(T - 512, T)
    qd = _bits_to_f64(inp["q"][late].reshape(-1, w.head_dim))     # [512 * Hq, D]
    best = int(np.argmax(qd @ spike))
    token, head = int(late[best // w.n_q_heads]), best % w.n_q_heads
    p = _check(inp, w, token, head)
    visible = spike_rows[spike_rows <= token]
    assert p[visible].sum() > 0.99
