"""Pins of the oracle's merge on logits (the beam top-k merge with each beam
row's log-softmax folded in): a brute-force reference built from an
independent library routine (scipy's logsumexp) and a full stable sort
(numpy lexsort) on small inputs, the closed form of a constant row, the
normalisation of the log-probabilities it implies, invariance under a
per-row shift of the logits, and the tie rule.  Catches: a row sum without
the max shift or with a dropped term, the lse subtracted with the wrong sign
or not at all, the lse of the wrong row, ranking on the raw logit, the wrong
tie direction, token/parent swapped, an off-by-one cut."""
import itertools

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle


def _brute(x, cum, W):
    R, Win, V = x.shape
    lse = logsumexp(x.astype(np.float64), axis=2)                       # [R, Win]
    toks, pars, scs = [], [], []
    for r in range(R):
        sc = (cum[r].astype(np.float64)[:, None] + (x[r].astype(np.float64) - lse[r][:, None])).reshape(-1)
        f = np.arange(Win * V)
        order = np.lexsort((f, -sc))                                     # score desc, then f asc
        sel = order[:W]
        toks.append(sel % V); pars.append(sel // V); scs.append(sc[sel])
    return np.array(toks, np.int32), np.array(pars, np.int32), np.array(scs), lse


def _check(got, ref, tol=1e-12):
    assert np.array_equal(got[0], ref[0])
    assert np.array_equal(got[1], ref[1])
    np.testing.assert_allclose(got[2], ref[2], rtol=0, atol=tol)
    np.testing.assert_allclose(got[3], ref[3], rtol=0, atol=tol)


def test_random_vs_brute_force():
    rng = np.random.default_rng(21)
    for (R, Win, V) in [(1, 1, 7), (2, 3, 50), (3, 4, 257), (2, 5, 1000)]:
        x = (rng.standard_normal((R, Win, V)) * 3).astype(np.float32)
        cum = (rng.standard_normal((R, Win)) * 2 - 4).astype(np.float32)
        for W in sorted({1, 2, min(7, Win * V), min(33, Win * V), Win * V}):
            _check(oracle.topk_merge_logits(x, cum, W), _brute(x, cum, W))


def test_exhaustive_small_with_ties():
    rng = np.random.default_rng(22)
    for Win, V in itertools.product((1, 2, 3), (1, 2, 5, 8)):
        for trial in range(3):
            x = (rng.integers(-6, 3, size=(2, Win, V)) / 4.0).astype(np.float32)    # many exact ties
            cum = (rng.integers(-3, 1, size=(2, Win)) / 2.0).astype(np.float32)
            for W in range(1, Win * V + 1):
                got = oracle.topk_merge_logits(x, cum, W)
                ref = _brute(x, cum, W)
                # equal fp64 scores: the sort order is decided by the flat index in both
                np.testing.assert_allclose(got[2], ref[2], rtol=0, atol=1e-12)
                np.testing.assert_allclose(got[3], ref[3], rtol=0, atol=1e-12)
                same_score = np.abs(got[2] - ref[2]) <= 1e-12
                assert same_score.all()
                # where two candidates' fp64 scores differ only by rounding of
                # the lse (same logit, same cum, different rows), the brute
                # force and the oracle may order them differently; compare sets
                for r in range(2):
                    g = set(zip(got[1][r].tolist(), got[0][r].tolist()))
                    b = set(zip(ref[1][r].tolist(), ref[0][r].tolist()))
                    if g != b:
                        # only candidates tied (to 1e-12) with the cut may differ
                        cut = ref[2][r][-1]
                        for (pb, tk) in g ^ b:
                            s = float(cum[r, pb]) + (float(x[r, pb, tk]) - ref[3][r, pb])
                            assert abs(s - cut) <= 1e-12


def test_constant_row_closed_form():
    """A row of V equal logits z has lse = z + log V and every candidate of it
    scores cum - log V; with W = Win*V all candidates come out, each row's
    block in flat-index order."""
    V, Win = 37, 3
    x = np.empty((1, Win, V), np.float32)
    x[0, 0, :] = 2.5
    x[0, 1, :] = -7.25
    x[0, 2, :] = 0.0
    cum = np.array([[-1.0, -3.0, -2.0]], np.float32)
    tok, par, sc, lse = oracle.topk_merge_logits(x, cum, Win * V)
    np.testing.assert_allclose(lse[0], np.array([2.5, -7.25, 0.0]) + np.log(V), rtol=0, atol=1e-12)
    assert par[0].tolist() == [0] * V + [2] * V + [1] * V                # cum -1 > -2 > -3
    assert tok[0].tolist() == list(range(V)) * 3
    np.testing.assert_allclose(sc[0], np.repeat(np.array([-1.0, -2.0, -3.0]) - np.log(V), V), rtol=0, atol=1e-12)


def test_log_probs_normalise():
    """With W = Win*V every candidate is output: per row, sum_v exp(score - cum)
    is 1 (the log-probabilities of a distribution)."""
    rng = np.random.default_rng(23)
    R, Win, V = 2, 3, 301
    x = (rng.standard_normal((R, Win, V)) * 4).astype(np.float32)
    x[1, 2, ::3] = -np.inf
    cum = (rng.standard_normal((R, Win)) - 2).astype(np.float32)
    tok, par, sc, lse = oracle.topk_merge_logits(x, cum, Win * V)
    for r in range(R):
        for b in range(Win):
            sel = par[r] == b
            assert sel.sum() == V
            assert abs(np.exp(sc[r][sel] - float(cum[r, b])).sum() - 1.0) < 1e-12


def test_row_shift_invariance():
    """Adding a constant to every logit of a row changes nothing: its lse
    moves by the same constant and the log-probabilities stay."""
    rng = np.random.default_rng(24)
    R, Win, V, W = 2, 6, 500, 40
    x = (np.round(rng.standard_normal((R, Win, V)) * 2048) / 1024).astype(np.float32)   # 2^-10 grid
    cum = (rng.standard_normal((R, Win)) - 3).astype(np.float32)
    shift = np.array([0.0, 8.0, -16.0, 1024.0, -0.5, 64.0], np.float32)  # exact in fp32 for these logits
    xs = (x + shift[None, :, None]).astype(np.float32)
    assert np.array_equal(xs - shift[None, :, None], x)                  # the shift was exact
    a = oracle.topk_merge_logits(x, cum, W)
    b = oracle.topk_merge_logits(xs, cum, W)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    np.testing.assert_allclose(a[2], b[2], rtol=0, atol=1e-9)
    np.testing.assert_allclose(b[3] - a[3], np.broadcast_to(shift, (R, Win)), rtol=0, atol=1e-9)


def test_neg_inf_logits_and_rejects():
    x = np.zeros((1, 2, 4), np.float32)
    x[0, 0, 1:] = -np.inf
    cum = np.zeros((1, 2), np.float32)
    tok, par, sc, lse = oracle.topk_merge_logits(x, cum, 8)
    np.testing.assert_allclose(lse[0], [0.0, np.log(4)], rtol=0, atol=1e-12)
    assert (par[0][:1].tolist(), tok[0][:1].tolist()) == ([0], [0])      # lp 0 beats -log 4
    assert np.isneginf(sc[0][-3:]).all() and par[0][-3:].tolist() == [0, 0, 0]
    assert tok[0][-3:].tolist() == [1, 2, 3]                              # -inf ties: flat order
    bad = np.full((1, 1, 3), -np.inf, np.float32)
    with pytest.raises(ValueError):
        oracle.topk_merge_logits(bad, np.zeros((1, 1), np.float32), 1)
    with pytest.raises(ValueError):
        oracle.topk_merge_logits(np.zeros((1, 1, 3), np.float32), np.zeros((1, 1), np.float32), 4)
