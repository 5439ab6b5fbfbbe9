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
