"""Pins of the oracle's prefill-only label head: a brute-force reference from
independent library routines (numpy float64 matmul over the rows picked by
cu_seqlens, scipy's softmax, numpy lexsort for the top K), the uniform
distribution of an empty sequence, normalisation, the fixed mapping and the
tie rule.  Catches: the first instead of the last token of a sequence, the
wrong LM-head row for a label, softmax over the vocabulary instead of the
labels, a dropped max shift, the wrong tie direction, an off-by-one cut."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import workloads as wl


def _case(rng, lengths, H, V, L, scale=1.0, quant=None):
    T = int(sum(lengths))
    x = rng.standard_normal((T, H)).astype(np.float32)
    w = (rng.standard_normal((V, H)) * scale).astype(np.float32)
    if quant:
        x = np.round(x * quant) / quant
        w = np.round(w * quant) / quant
    hidden = wl.f32_to_bf16_bits(x.astype(np.float32))
    lm = wl.f32_to_bf16_bits(w.astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    labels = rng.choice(V, size=L, replace=False).astype(np.int32)
    return hidden, lm, cu, labels


def _brute(hidden, lm, cu, labels, K, label_map=None):
    B = len(cu) - 1
    h = wl.bf16_bits_to_f32(hidden).astype(np.float64)
    w = wl.bf16_bits_to_f32(lm).astype(np.float64)[labels]
    last = np.zeros((B, h.shape[1]))
    for b in range(B):
        if cu[b + 1] > cu[b]:
            last[b] = h[cu[b + 1] - 1]
    z = last @ w.T
    p = softmax(z, axis=1)
    idx = np.array([np.lexsort((np.arange(len(labels)), -z[b]))[:K] for b in range(B)], np.int32).reshape(B, K)
    tp = np.take_along_axis(p, idx, axis=1)
    tc = idx if label_map is None else np.asarray(label_map)[idx]
    return z, p, idx, tp, tc


def _check(got, ref, ztol=1e-9):
    np.testing.assert_allclose(got[0], ref[0], rtol=0, atol=ztol)
    np.testing.assert_allclose(got[1], ref[1], rtol=0, atol=1e-12)
    assert np.array_equal(got[2], ref[2])
    np.testing.assert_allclose(got[3], ref[3], rtol=0, atol=1e-12)
    assert np.array_equal(got[4], ref[4])


def test_random_vs_brute_force():
    rng = np.random.default_rng(31)
    for lengths, H, V, L, K in [((3, 1, 7), 64, 100, 5, 2), ((10, 20, 5, 9), 256, 1000, 64, 5),
                                 ((1,) * 12, 128, 300, 33, 33)]:
        hidden, lm, cu, labels = _case(rng, lengths, H, V, L, scale=H ** -0.5)
        _check(oracle.label_head(hidden, cu, lm, labels, K), _brute(hidden, lm, cu, labels, K))


def test_ties_and_map():
    """Quantised values make equal logits: the lower label index ranks first;
    the map turns label indices into classes."""
    rng = np.random.default_rng(32)
    hidden, lm, cu, labels = _case(rng, (4, 6, 2, 8, 3), 16, 50, 20, quant=1)
    lm_bits = lm.copy()
    lm_bits[labels[7]] = lm_bits[labels[2]]          # two labels with the same LM-head row
    label_map = rng.integers(0, 4, size=20).astype(np.int32)
    got = oracle.label_head(hidden, cu, lm_bits, labels, 10, label_map)
    ref = _brute(hidden, lm_bits, cu, labels, 10, label_map)
    _check(got, ref)
    for b in range(len(cu) - 1):
        order = got[2][b].tolist()
        if 2 in order and 7 in order:
            assert order.index(2) < order.index(7)


def test_empty_sequence_is_uniform_and_probs_normalise():
    rng = np.random.default_rng(33)
    hidden, lm, cu, labels = _case(rng, (5, 0, 3, 0), 32, 80, 12, scale=0.2)
    z, p, idx, tp, tc = oracle.label_head(hidden, cu, lm, labels, 4)
    for b in (1, 3):                                  # empty: zero logits, uniform, first K labels
        assert np.all(z[b] == 0.0)
        np.testing.assert_allclose(p[b], np.full(12, 1 / 12), rtol=0, atol=1e-15)
        assert idx[b].tolist() == [0, 1, 2, 3]
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.array_equal(tc, idx)                    # no map: classes are the label indices


def test_rejects():
    rng = np.random.default_rng(34)
    hidden, lm, cu, labels = _case(rng, (2, 3), 8, 20, 4)
    with pytest.raises(ValueError):
        oracle.label_head(hidden, cu, lm, labels, 5)                      # K > L
    bad = labels.copy()
    bad[1] = 20
    with pytest.raises(ValueError):
        oracle.label_head(hidden, cu, lm, bad, 2)                         # label id out of range
