"""Pins of the parity rules themselves (oracle/compare.py), on the CPU.

Every GPU parity decision goes through scores_ok, topk_ok and attention_ok, so each rule is fed
planted wrong "GPU" outputs that it must reject, beside near-misses on the right side of each
bound that it must accept. The bounds are the ones the layer's statement of correctness fixes:
scores within 1e-3 relative (with a row floor at scores near zero), top-k sets equal except for
candidates within 1e-5 relative of the k-th oracle score, attention within 2e-2 absolute (bf16
cache) or 5e-2 (fp8 caches), and the lse within 1e-3 with -inf exactly on empty rows.
"""
import numpy as np
import pytest

from oracle.compare import attention_ok, scores_ok, topk_ok


# --------------------------------------------------------------------------- scores

def _row(seed=0, n=300):
    rng = np.random.default_rng(seed)
    s = rng.uniform(1.0, 50.0, n)
    s[::7] = 0.0                       # ReLU zeros are common
    return s


def test_scores_accepts_exact_and_near_misses():
    ref = _row()
    assert scores_ok(ref.copy(), ref)[0]
    # 0.9e-3 relative on every nonzero score
    assert scores_ok(ref * (1 + 0.9e-3), ref)[0]
    # at an exact zero the row floor (1e-3 of the row's largest |score|) sets the scale
    g = ref.copy()
    g[0] = 0.9e-3 * 1e-3 * np.abs(ref).max()
    assert scores_ok(g, ref)[0]


@pytest.mark.parametrize("where", [1, 150, 299])
def test_scores_rejects_one_score_off_by_1_1e_3(where):
    ref = _row()
    ref[where] = 40.0                  # well above the row floor
    g = ref.copy()
    g[where] *= 1 + 1.1e-3
    ok, msg = scores_ok(g, ref)
    assert not ok and f"first at {where}" in msg


def test_scores_rejects_zero_above_the_floor_and_nan():
    ref = _row()
    g = ref.copy()
    g[0] = 2e-3 * 1e-3 * np.abs(ref).max()      # twice the floor tolerance at an exact zero
    assert not scores_ok(g, ref)[0]
    g = ref.copy()
    g[5] = np.nan
    assert not scores_ok(g, ref)[0]
    g = ref.copy()
    g[5] = np.inf
    assert not scores_ok(g, ref)[0]


def test_scores_rejects_wrong_shape():
    ref = _row()
    assert not scores_ok(ref[:-1], ref)[0]
    assert not scores_ok(ref[None, :], ref)[0]
    assert not scores_ok(np.zeros(0), ref)[0]
    assert scores_ok(np.zeros(0), np.zeros(0))[0]


# --------------------------------------------------------------------------- top-k rule T

def _scores_with_gap(n=1000, k=100, seed=1):
    """Distinct scores; the k-th (s_k = 10.0) sits at position 500, its neighbours in the order
    are far away except for the two planted near-ties at positions 7 (just inside the window,
    below s_k) and 9 (just outside, below s_k)."""
    rng = np.random.default_rng(seed)
    s = np.empty(n)
    s[:] = rng.uniform(0.0, 5.0, n)              # the bulk: far below s_k
    top = rng.choice(np.setdiff1d(np.arange(n), [7, 9, 500]), k - 1, replace=False)
    s[top] = rng.uniform(20.0, 30.0, k - 1)      # the k - 1 best
    s[500] = 10.0                                # the k-th
    s[7] = 10.0 * (1 - 0.5e-5)                   # inside the 1e-5 window
    s[9] = 10.0 * (1 - 2e-5)                     # outside it
    return s, np.sort(top)


def _gpu_row(sel, k, pad=-1):
    r = np.full(k, pad, np.int64)
    r[:len(sel)] = sel
    return r


def test_topk_accepts_the_oracle_set_in_any_order():
    s, top = _scores_with_gap()
    k = 100
    sel = np.concatenate([top, [500]])
    assert topk_ok(s, k, _gpu_row(sel, k), k)[0]
    assert topk_ok(s, k, _gpu_row(sel[::-1], k), k)[0]


def test_topk_tie_window_edges():
    s, top = _scores_with_gap()
    k = 100
    inside = np.concatenate([top, [7]])          # s_k swapped for a candidate 0.5e-5 below it
    ok, msg = topk_ok(s, k, _gpu_row(inside, k), k)
    assert ok, msg
    outside = np.concatenate([top, [9]])         # ... and for one 2e-5 below it
    ok, msg = topk_ok(s, k, _gpu_row(outside, k), k)
    assert not ok and "position 9" in msg
    far = top.copy()
    far[0] = 3                                   # a top member swapped for a bulk candidate
    ok, _ = topk_ok(s, k, _gpu_row(np.concatenate([far, [500]]), k), k)
    assert not ok


def test_topk_exact_ties_at_s_k_are_accepted():
    """Exact ties straddling the k-th score: any choice among them is correct."""
    s = np.array([5.0, 1.0, 3.0, 3.0, 3.0, 0.5, 4.0])
    k = 3                                        # oracle: 0, 6, then position 2 (ties by position)
    for third in (2, 3, 4):
        assert topk_ok(s, k, np.array([0, 6, third]), k)[0]
    assert not topk_ok(s, k, np.array([0, 6, 1]), k)[0]


def test_topk_rejects_wrong_lens_and_padding():
    s, top = _scores_with_gap()
    k = 100
    sel = np.concatenate([top, [500]])
    row = _gpu_row(sel, k)
    assert not topk_ok(s, k, row, k - 1)[0]                   # lens one short
    assert not topk_ok(s, k, row, k + 1)[0]
    # n <= k: lens = n, then -1 up to k
    small = np.array([3.0, 1.0, 2.0])
    assert topk_ok(small, 5, np.array([2, 0, 1, -1, -1]), 3)[0]
    assert not topk_ok(small, 5, np.array([2, 0, 1, -1, -1]), 5)[0]
    assert not topk_ok(small, 5, np.array([2, 0, 1, 0, -1]), 3)[0]      # tail entry not -1
    assert not topk_ok(small, 5, np.array([2, -1, 1, 0, -1]), 3)[0]     # -1 before lens
    assert not topk_ok(small, 5, np.array([2, 0, 1, -1]), 3)[0]         # row shorter than topk


def test_topk_rejects_duplicates_and_out_of_range():
    s, top = _scores_with_gap()
    k = 100
    sel = np.concatenate([top, [500]])
    dup = sel.copy()
    dup[5] = dup[6]
    assert not topk_ok(s, k, _gpu_row(dup, k), k)[0]
    oor = sel.copy()
    oor[0] = len(s)                              # one past the row's candidates
    assert not topk_ok(s, k, _gpu_row(oor, k), k)[0]
    neg = sel.copy()
    neg[0] = -2
    assert not topk_ok(s, k, _gpu_row(neg, k), k)[0]


def test_topk_rejects_an_incomplete_set_when_n_le_k():
    small = np.array([3.0, 1.0, 2.0, 2.0])
    k = 6
    assert topk_ok(small, k, np.array([0, 1, 2, 3, -1, -1]), 4)[0]
    # right length, distinct, in range, but position 3 missing (0 listed twice is caught too)
    assert not topk_ok(small, k, np.array([0, 1, 2, 0, -1, -1]), 4)[0]
    assert not topk_ok(small, k, np.array([0, 1, 2, -1, -1, -1]), 3)[0]


def test_topk_symmetric_difference_is_walked_in_full():
    """Several swapped-in candidates inside the window and one outside it (position 7, the
    largest of the difference): a checker that stopped at the first element of the difference
    would pass the row."""
    s = np.array([10.0] + [8.0 * (1 - i * 1e-6) for i in range(6)] + [7.0])
    k = 3                                        # oracle {0, 1, 2}; s_k = 8 (1 - 1e-6)
    ok, msg = topk_ok(s, k, np.array([0, 5, 6]), k)       # difference {1, 2, 5, 6}: all inside
    assert ok, msg
    ok, msg = topk_ok(s, k, np.array([0, 6, 7]), k)       # difference {1, 2, 6, 7}: 7 outside
    assert not ok and "position 7" in msg


# --------------------------------------------------------------------------- attention

def _att(H=4, dv=8, seed=2):
    rng = np.random.default_rng(seed)
    out = rng.standard_normal((H, dv)) * 0.3
    lse = rng.standard_normal(H) * 2.0 + 5.0
    return out, lse


@pytest.mark.parametrize("fmt,tol", [("bf16", 2e-2), ("fp8_uniform", 5e-2), ("fp8_ds_mla", 5e-2),
                                     ("fp8_uniform_fnuz", 5e-2)])
def test_attention_output_bound(fmt, tol):
    out, lse = _att()
    g = out.copy()
    g[1, 3] += 0.95 * tol
    assert attention_ok(g, lse, out, lse, fmt)[0]
    g[1, 3] = out[1, 3] + 1.05 * tol
    assert not attention_ok(g, lse, out, lse, fmt)[0]
    g = out.copy()
    g[2, 0] -= 1.05 * tol
    assert not attention_ok(g, lse, out, lse, fmt)[0]


def test_attention_bf16_is_held_to_2e_2_not_the_fp8_bound():
    out, lse = _att()
    g = out.copy()
    g[0, 0] += 2.1e-2
    assert not attention_ok(g, lse, out, lse, "bf16")[0]
    assert attention_ok(g, lse, out, lse, "fp8_ds_mla")[0]
    g[0, 0] = out[0, 0] + 5.1e-2
    assert not attention_ok(g, lse, out, lse, "fp8_ds_mla")[0]
    with pytest.raises(KeyError):
        attention_ok(out, lse, out, lse, "no_such_format")


def test_attention_rejects_lse_errors():
    out, lse = _att()
    g = lse.copy()
    g[3] += 0.9e-3
    assert attention_ok(out, g, out, lse, "bf16")[0]
    g[3] = lse[3] + 1.1e-3
    assert not attention_ok(out, g, out, lse, "bf16")[0]
    ref = lse.copy()
    ref[1] = -np.inf                             # an empty row
    g = ref.copy()
    assert attention_ok(out, g, out, ref, "bf16")[0]
    g[1] = -1e30                                 # finite where the oracle says -inf
    ok, msg = attention_ok(out, g, out, ref, "bf16")
    assert not ok and "-inf" in msg
    g = lse.copy()
    g[0] = -np.inf                               # -inf where the oracle is finite
    assert not attention_ok(out, g, out, lse, "bf16")[0]
    g = lse.copy()
    g[2] = np.nan
    assert not attention_ok(out, g, out, lse, "bf16")[0]


def test_attention_rejects_non_finite_and_wrong_shapes():
    out, lse = _att()
    g = out.copy()
    g[0, 0] = np.nan
    assert not attention_ok(g, lse, out, lse, "bf16")[0]
    g[0, 0] = np.inf
    assert not attention_ok(g, lse, out, lse, "bf16")[0]
    # one head's output broadcast over all heads must not pass for the whole row
    same = np.repeat(out[:1], out.shape[0], axis=0)
    assert not attention_ok(out[:1], lse, same, lse, "bf16")[0]
    assert not attention_ok(out[:, :-1], lse, out, lse, "bf16")[0]
    assert not attention_ok(out, lse[:1], out, lse, "bf16")[0]
    # lse None: only the output is compared
    assert attention_ok(out, None, out, lse, "bf16")[0]
