"""Pins of the oracle's attention backward (step 5 of the oracle's description) against
things other than its own formulas: central finite differences of the forward oracle,
a closed form, and an invariance of the softmax."""
import numpy as np
import pytest

import oracle


def _loss(q, rows, sink, scale, d_qk, d_v, dout):
    out, _ = oracle.attention_math(q, rows, sink, scale, d_qk, d_v)
    return float((dout * out).sum())


@pytest.mark.parametrize("d_qk,d_v,with_sink", [(20, 16, False), (20, 16, True), (16, 16, True)],
                         ids=["rope_tail", "rope_tail_sink", "k_equals_v_sink"])
def test_backward_matches_finite_differences_of_the_forward(d_qk, d_v, with_sink):
    rng = np.random.default_rng(d_qk + d_v + with_sink)
    H, n = 3, 7
    q = rng.standard_normal((H, d_qk))
    rows = rng.standard_normal((n, max(d_qk, d_v)))
    sink = np.array([0.7, -np.inf, -1.3]) if with_sink else np.full(H, -np.inf)
    dout = rng.standard_normal((H, d_v))
    scale = 0.37
    dq, drows, dsink = oracle.attention_backward_math(q, rows, sink, scale, d_qk, d_v, dout)
    eps = 1e-5

    def fd(x, i):
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        return xp, xm

    for i in np.ndindex(q.shape):
        qp, qm = fd(q, i)
        g = (_loss(qp, rows, sink, scale, d_qk, d_v, dout) - _loss(qm, rows, sink, scale, d_qk, d_v, dout)) / (2 * eps)
        assert abs(g - dq[i]) <= 1e-7 + 1e-6 * abs(g), (i, g, dq[i])
    for i in np.ndindex(rows.shape):
        rp, rm = fd(rows, i)
        g = (_loss(q, rp, sink, scale, d_qk, d_v, dout) - _loss(q, rm, sink, scale, d_qk, d_v, dout)) / (2 * eps)
        assert abs(g - drows[i]) <= 1e-7 + 1e-6 * abs(g), (i, g, drows[i])
    for h in range(H):
        if not np.isfinite(sink[h]):
            assert dsink[h] == 0.0
            continue
        sp, sm = fd(sink, (h,))
        g = (_loss(q, rows, sp, scale, d_qk, d_v, dout) - _loss(q, rows, sm, scale, d_qk, d_v, dout)) / (2 * eps)
        assert abs(g - dsink[h]) <= 1e-7 + 1e-6 * abs(g), (h, g, dsink[h])


def test_backward_single_row_closed_form():
    """One listed row and no sink: p = 1, out = v, so dq = 0, the key part gets nothing and the
    value part gets dout itself."""
    rng = np.random.default_rng(5)
    H, d_qk, d_v = 4, 12, 8
    q = rng.standard_normal((H, d_qk))
    rows = rng.standard_normal((1, d_qk))
    dout = rng.standard_normal((H, d_v))
    dq, drows, dsink = oracle.attention_backward_math(q, rows, np.full(H, -np.inf), 0.5, d_qk, d_v, dout)
    assert np.allclose(dq, 0.0, atol=1e-14)
    assert np.allclose(drows[0, :d_v], dout.sum(axis=0), atol=1e-14)
    assert np.allclose(drows[0, d_v:], 0.0, atol=1e-14)
    assert np.all(dsink == 0.0)


def test_backward_rope_gradient_sums_to_zero_without_sink():
    """Without a sink the softmax is invariant to adding one vector u to every row's key-only
    columns [d_v, d_qk) (the logits all shift by scale * q . u; the values do not change), so the
    gradients of those columns sum to zero over the listed rows."""
    rng = np.random.default_rng(11)
    H, n, d_qk, d_v = 5, 9, 24, 16
    q = rng.standard_normal((H, d_qk))
    rows = rng.standard_normal((n, d_qk))
    dout = rng.standard_normal((H, d_v))
    _, drows, _ = oracle.attention_backward_math(q, rows, np.full(H, -np.inf), 0.3, d_qk, d_v, dout)
    assert np.abs(drows[:, d_v:].sum(axis=0)).max() < 1e-12
    assert np.abs(drows[:, :d_v].sum(axis=0)).max() > 1e-3      # the value part does not cancel


def _given_case(seed=21):
    rng = np.random.default_rng(seed)
    H, n, d_qk, d_v = 3, 6, 20, 16
    q = rng.standard_normal((H, d_qk))
    rows = rng.standard_normal((n, d_qk))
    sink = np.array([0.4, -np.inf, -0.9])
    dout = rng.standard_normal((H, d_v))
    out, lse = oracle.attention_math(q, rows, sink, 0.45, d_qk, d_v)
    return q, rows, sink, dout, out, lse, 0.45, d_qk, d_v


def test_backward_given_forward_outputs_equal_the_exact_ones():
    q, rows, sink, dout, out, lse, scale, d_qk, d_v = _given_case()
    ref = oracle.attention_backward_math(q, rows, sink, scale, d_qk, d_v, dout)
    got = oracle.attention_backward_math(q, rows, sink, scale, d_qk, d_v, dout, out=out, lse=lse)
    for a, b in zip(ref, got):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_backward_given_out_enters_through_D_only():
    """A perturbed given out (out + delta) changes only D_h by dout_h . delta_h: in closed form
    dsink_h moves by -p_sink_h (dout_h . delta_h), dq_h by -scale (dout_h . delta_h)
    sum_i p_i c_i[:d_qk], and the key part of drows by -scale (dout_h . delta_h) p_i q_h summed
    over h; the value part (p_i dout_h) does not move."""
    q, rows, sink, dout, out, lse, scale, d_qk, d_v = _given_case()
    delta = np.random.default_rng(3).standard_normal(out.shape) * 1e-2
    dq0, dr0, ds0 = oracle.attention_backward_math(q, rows, sink, scale, d_qk, d_v, dout, out=out, lse=lse)
    dq1, dr1, ds1 = oracle.attention_backward_math(q, rows, sink, scale, d_qk, d_v, dout,
                                                   out=out + delta, lse=lse)
    dD = (dout * delta).sum(axis=1)                                     # [H]
    p = np.exp(scale * (q @ rows[:, :d_qk].T) - lse[:, None])           # [H, n]
    p_sink = np.exp(sink - lse)
    assert np.allclose(ds1 - ds0, -p_sink * dD, atol=1e-14)
    assert np.allclose(dq1 - dq0, -scale * dD[:, None] * (p @ rows[:, :d_qk]), atol=1e-13)
    assert np.allclose(dr1[:, :d_qk] - dr0[:, :d_qk], -scale * (p * dD[:, None]).T @ q, atol=1e-13)
    assert np.allclose(dr1[:, d_qk:], dr0[:, d_qk:], atol=0)


def test_backward_given_lse_scales_the_weights():
    """A given lse shifted by eps multiplies every weight p_i and p_sink by e^-eps; with out held,
    dq, the key and value parts of drows and dsink all scale by e^-eps exactly."""
    q, rows, sink, dout, out, lse, scale, d_qk, d_v = _given_case()
    eps = 0.3
    a = oracle.attention_backward_math(q, rows, sink, scale, d_qk, d_v, dout, out=out, lse=lse)
    b = oracle.attention_backward_math(q, rows, sink, scale, d_qk, d_v, dout, out=out, lse=lse + eps)
    for x, y in zip(a, b):
        assert np.allclose(y, np.exp(-eps) * x, rtol=1e-12, atol=1e-15)
