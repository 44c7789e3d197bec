"""Pins of the oracle's beam top-k merge: a full stable sort (numpy lexsort,
an independent library routine) on tiny inputs, exhaustive small cases, tie
stress, fp32-sum semantics and order invariants.  Catches: ranking by the
log-prob instead of the fp32 sum, the sum done in fp64, the wrong tie-break
direction, token/parent swapped, an off-by-one cut."""
import itertools

import numpy as np
import pytest

import oracle
import workloads as wl


def _full_sort(lp, cum, W):
    R, Win, V = lp.shape
    toks, pars, cums = [], [], []
    for r in range(R):
        sc = (cum[r][:, None] + lp[r]).astype(np.float32).reshape(-1)   # one fp32 add each
        f = np.arange(Win * V)
        order = np.lexsort((f, -sc.astype(np.float64)))                  # score desc, then f asc
        sel = order[:W]
        toks.append(sel % V); pars.append(sel // V); cums.append(sc[sel])
    return (np.array(toks, np.int32), np.array(pars, np.int32), np.array(cums, np.float32))


def _check_equal(a, b):
    for x, y in zip(a, b):
        assert np.array_equal(x, y), (x, y)


def test_tiny_workload_vs_full_sort():
    shape = wl.TINY_BEAM
    lp0 = wl.beam_logprobs(shape, 0)
    cum0 = np.zeros((shape.num_requests, 1), np.float32)
    out0 = oracle.topk_merge(lp0, cum0, shape.width)
    _check_equal(out0, _full_sort(lp0, cum0, shape.width))
    assert np.all(out0[1] == 0)
    lp1 = wl.beam_logprobs(shape, 1)
    out1 = oracle.topk_merge(lp1, out0[2], shape.width)
    _check_equal(out1, _full_sort(lp1, out0[2], shape.width))


def test_exhaustive_small():
    rng = np.random.default_rng(1)
    for Win, V in itertools.product((1, 2, 3), (1, 2, 5, 8)):
        for trial in range(3):
            # quantised values force many exact ties
            lp = (rng.integers(-6, 1, size=(2, Win, V)) / 4.0).astype(np.float32)
            cum = (rng.integers(-3, 1, size=(2, Win)) / 2.0).astype(np.float32)
            for W in range(1, Win * V + 1):
                _check_equal(oracle.topk_merge(lp, cum, W), _full_sort(lp, cum, W))


def test_tie_stress_and_neg_inf():
    rng = np.random.default_rng(2)
    lp = (np.round(rng.standard_normal((3, 6, 200)) * 16) / 16 - 5).astype(np.float32)
    lp[:, 2, :] = -np.inf
    lp[1, 4, 50:] = -np.inf
    cum = (np.round(rng.standard_normal((3, 6)) * 4) / 4).astype(np.float32)
    for W in (1, 6, 37, 200, 1000):
        _check_equal(oracle.topk_merge(lp, cum, W), _full_sort(lp, cum, W))
    # W beyond the finite candidates: -inf entries ordered by index
    lpi = np.full((1, 2, 3), -np.inf, np.float32); lpi[0, 1, 2] = -1
    tok, par, co = oracle.topk_merge(lpi, np.zeros((1, 2), np.float32), 4)
    assert tok.tolist() == [[2, 0, 1, 2]] and par.tolist() == [[1, 0, 0, 0]]
    assert co[0, 0] == -1 and np.all(np.isneginf(co[0, 1:]))


def test_fp32_sum_decides_ties():
    # cum = 2^24: fp32 spacing just below is 1, so 2^24-0.5 (a tie, to even)
    # and 2^24-0.25 both round to 2^24.  The two sums are equal in fp32, so
    # the lower flat index must win although its log-prob is smaller; ranking
    # in fp64 (or by log-prob) would pick index 1.
    lp = np.array([[[-0.5, -0.25, -9.0]]], np.float32)
    cum = np.array([[2.0 ** 24]], np.float32)
    assert np.float32(cum[0, 0] + lp[0, 0, 0]) == np.float32(cum[0, 0] + lp[0, 0, 1]) == np.float32(2.0 ** 24)
    tok, par, co = oracle.topk_merge(lp, cum, 1)
    assert tok[0, 0] == 0
    assert co[0, 0] == np.float32(2.0 ** 24)
    tok, par, co = oracle.topk_merge(lp, cum, 2)
    assert tok[0].tolist() == [0, 1]


def test_order_invariants_and_full_permutation():
    rng = np.random.default_rng(4)
    lp = (np.round(rng.standard_normal((2, 4, 30)) * 8) / 8).astype(np.float32)
    cum = rng.standard_normal((2, 4)).astype(np.float32)
    tok, par, co = oracle.topk_merge(lp, cum, 120)
    for r in range(2):
        f = par[r].astype(np.int64) * 30 + tok[r]
        assert sorted(f.tolist()) == list(range(120))          # W = Win*V: a permutation
        assert np.all(np.diff(co[r]) <= 0)                     # scores never increase
        eq = np.diff(co[r]) == 0
        assert np.all(np.diff(f)[eq] > 0)                      # equal scores: index ascends
    tok, par, co = oracle.topk_merge(lp, cum, 10)
    for r in range(2):
        sc = (cum[r][:, None] + lp[r]).astype(np.float32)
        chosen = set((par[r] * 30 + tok[r]).tolist())
        rest = [sc.reshape(-1)[f] for f in range(120) if f not in chosen]
        assert co[r, -1] >= max(rest)


def test_first_step_equivalent_forms():
    # one beam in == W beams in with cum = [0, -inf, ...] (same tokens, parent 0)
    lp0 = wl.logprobs(77, (2, 1, 50))
    W = 6
    a = oracle.topk_merge(lp0, np.zeros((2, 1), np.float32), W)
    lpw = np.repeat(lp0, W, axis=1)
    cum = np.full((2, W), -np.inf, np.float32); cum[:, 0] = 0
    b = oracle.topk_merge(lpw, cum, W)
    _check_equal(a, b)


def test_rejects_bad_width():
    with pytest.raises(ValueError):
        oracle.topk_merge(np.zeros((1, 2, 3), np.float32), np.zeros((1, 2), np.float32), 7)
