"""GPU parity of the prefill-only label head (through the C ABI) against the
oracle's fp64 definition on the same seeded inputs.

Bound: bf16 x bf16 products are exact in fp32, and an fp32 sum of H terms in
any order is within (H - 1) * 2^-24 * sum|terms| of the exact sum, so each
logit is checked against that bound (doubled), computed per (sequence,
label) from the operands.  Probabilities follow within 2 * max bound + 1e-6.
The top K is checked for validity against the oracle's logits (every label
more than EPS above the oracle's K-th logit is selected, none more than EPS
below it, EPS = twice the row's logit bound) and equal to the oracle's
wherever its top K + 1 logits have no near-tie; top_prob must be the output
probability of the selected label and top_class its mapped class, exactly."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import dev_bf16, note

pytestmark = pytest.mark.gpu


def _run(ctx, hidden, cu, lm, labels, K, label_map=None, probs=True):
    lab = torch.from_numpy(labels).cuda()
    mp = None if label_map is None else torch.from_numpy(label_map).cuda()
    out = ctx.label_head(hidden, cu, lm, lab, K, mp, probs)
    ctx.check()
    return tuple(None if o is None else o.cpu().numpy() for o in out)


def _check(got, hidden_bits, cu, lm_bits, labels, K, label_map=None, what=""):
    rz, rp, ri, rtp, rtc = oracle.label_head(hidden_bits, cu, lm_bits, labels, K, label_map)
    z, p, ti, tp, tc = got
    B, L = rz.shape
    # per-(b, j) summation bound from |a| . |b|
    h = np.abs(wl.bf16_bits_to_f32(hidden_bits).astype(np.float64))
    w = np.abs(wl.bf16_bits_to_f32(lm_bits[labels]).astype(np.float64))
    H = h.shape[1]
    last = np.zeros((B, H))
    for b in range(B):
        if cu[b + 1] > cu[b]:
            last[b] = h[cu[b + 1] - 1]
    bound = 2 * (H - 1) * 2.0 ** -24 * (last @ w.T) + 1e-30
    dz = np.abs(z.astype(np.float64) - rz)
    assert np.all(dz <= bound), "%s: logit off by %.3g (bound %.3g)" % (what, dz.max(), bound[dz > bound].min())
    if p is not None:
        tol = 2 * bound.max() + 1e-6
        dp = np.abs(p.astype(np.float64) - rp)
        assert dp.max() <= tol, "%s: prob off by %.3g" % (what, dp.max())
    exact = 0
    for b in range(B):
        eps = 2 * bound[b].max()
        sel = ti[b]
        assert len(set(sel.tolist())) == K and np.all((sel >= 0) & (sel < L)), what
        # order by the GPU's own logits, ties by index
        zs = z[b][sel]
        assert np.all((zs[:-1] > zs[1:]) | ((zs[:-1] == zs[1:]) & (sel[:-1] < sel[1:]))), what + ": order"
        cut = rz[b][ri[b][-1]]
        assert np.all(rz[b][sel] >= cut - eps), "%s: seq %d selects below the cut" % (what, b)
        must = [j for j in ri[b] if rz[b][j] > cut + eps]
        assert set(must) <= set(sel.tolist()), "%s: seq %d misses %s" % (what, b, set(must) - set(sel.tolist()))
        order = np.lexsort((np.arange(L), -rz[b]))[:K + 1]
        gaps = np.abs(np.diff(rz[b][order]))
        if gaps.size == 0 or gaps.min() > eps:
            assert np.array_equal(sel, ri[b]), "%s: seq %d differs without a near-tie" % (what, b)
            exact += 1
        if p is not None:
            assert np.array_equal(tp[b], p[b][sel]), what + ": top_prob"
        assert np.array_equal(tc[b], sel if label_map is None else label_map[sel]), what + ": top_class"
    return exact


# label counts cover every select variant (logits per lane 1, 4, 16 and 64, up to the 4,096 maximum)
@pytest.mark.parametrize("lengths,H,V,L,K", [((3, 1, 7), 64, 100, 5, 2), ((9, 0, 4, 12, 0, 1), 128, 500, 33, 33),
                                             ((5,) * 40, 256, 1000, 64, 5), ((4,) * 9, 128, 2000, 200, 7),
                                             ((2,) * 70, 1024, 3000, 300, 64), ((1,) * 5, 64, 5000, 1500, 10),
                                             ((2, 3), 64, 8192, 4096, 3)])
def test_shapes(gpu, lengths, H, V, L, K):
    note("label_head B=%d H=%d V=%d L=%d K=%d" % (len(lengths), H, V, L, K))
    rng = np.random.default_rng(sum(lengths) + H + L)
    T = sum(lengths)
    hb = wl.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lb = wl.f32_to_bf16_bits((rng.standard_normal((V, H)) / np.sqrt(H)).astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    labels = rng.choice(V, size=L, replace=False).astype(np.int32)
    label_map = rng.integers(0, 7, size=L).astype(np.int32)
    for mp, probs in ((None, True), (label_map, False)):
        got = _run(gpu, dev_bf16(hb), torch.from_numpy(cu).cuda(), dev_bf16(lb), labels, K, mp, probs)
        _check(got, hb, cu, lb, labels, K, mp, "shapes")


def test_prefill_request_workload(gpu):
    """The prefill-only request (15 packed samples, T=4,395, hidden 1024), 64
    labels from a synthetic 151,936-row LM head, top 5; two launches bitwise
    equal."""
    note("label_head prefill_request workload")
    pr = wl.PREFILL_REQUEST
    hb = wl.prefill_inputs(pr)["hidden"]
    V = 151936
    lm = wl.lm_head_rows(pr.base_seed, V, pr.hidden_dim)
    labels = wl.label_ids(pr.base_seed, V)
    cu = pr.cu_seqlens()
    args = (dev_bf16(hb), torch.from_numpy(cu).cuda(), dev_bf16(lm), labels, wl.LABEL_TOP_K)
    got = _run(gpu, *args)
    again = _run(gpu, *args)
    for a, b in zip(got, again):
        assert np.array_equal(a, b)
    _check(got, hb, cu, lm, labels, wl.LABEL_TOP_K, None, "prefill_request")


def test_bad_label_is_flagged(gpu):
    note("label_head bad label id -> device error flag")
    hb = wl.f32_to_bf16_bits(np.ones((4, 16), np.float32))
    lb = wl.f32_to_bf16_bits(np.ones((10, 16), np.float32))
    cu = torch.tensor([0, 2, 4], dtype=torch.int32).cuda()
    labels = torch.tensor([1, 10, 3], dtype=torch.int32).cuda()        # 10 is outside [0, 10)
    gpu.label_head(dev_bf16(hb), cu, dev_bf16(lb), labels, 2)
    with pytest.raises(Exception, match="label"):
        gpu.check()
    gpu.check()
