"""GPU parity of the merge on logits (through the C ABI) against the oracle's
fp64 definition on the same seeded inputs.

The kernel computes each row's log-sum-exp in fp32 (hardware exp2/log2,
per-lane partial sums of up to ~2.4k terms, combined in a fixed order), so
its lse differs from the exact one by rounding.  Bound used here: per-lane
fp32 accumulation of n <= 2,400 terms has relative error <= n * 2^-24 =
1.4e-4 in the worst case (about 3e-6 typical), the exp2/log2 instructions add
a few 1e-7, so |lse_gpu - lse| <= LSE_TOL = 2e-4.  A score is then off by at
most LSE_TOL plus the two fp32 roundings of cum + (x - lse) (below 1e-5 at
|score| < 64), SCORE_TOL = 2.2e-4.

What is compared: every row's lse (to LSE_TOL); each output score against
the oracle's exact score of the candidate it names (to SCORE_TOL); the
output order (non-increasing scores, ties by flat index); and the selection:
every candidate the oracle ranks clearly inside the top W (above its W-th
score by more than EPS = 2 * SCORE_TOL) is selected, and every selected
candidate is at most EPS below that W-th score.  Where no two of the
oracle's top W + 1 scores are within EPS of each other, tokens and parents
must equal the oracle's exactly.  Two launches must agree bitwise."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import note

pytestmark = pytest.mark.gpu

LSE_TOL = 2e-4
SCORE_TOL = 2.2e-4
EPS = 2 * SCORE_TOL


def _run(ctx, x, cum, W):
    R, Win, _ = x.shape
    lse = torch.empty((R, Win), dtype=torch.float32, device="cuda")
    t, p, c = ctx.beam_topk_merge_logits(x, cum, W, lse_out=lse)
    ctx.check()
    return t.cpu().numpy(), p.cpu().numpy(), c.cpu().numpy(), lse.cpu().numpy()


def _check(got, x, cum, W, what):
    """got: GPU (tokens, parent, cum_out, lse); x, cum host arrays."""
    tok, par, co, lse = got
    rt, rp, rs, rl = oracle.topk_merge_logits(x, cum, W)
    R, Win, V = x.shape
    dl = np.abs(lse.astype(np.float64) - rl)
    assert dl.max() <= LSE_TOL, "%s: lse off by %.3g" % (what, dl.max())
    exact_rows = 0
    for r in range(R):
        assert np.all((par[r] >= 0) & (par[r] < Win) & (tok[r] >= 0) & (tok[r] < V)), what
        f = par[r].astype(np.int64) * V + tok[r]
        assert len(set(f.tolist())) == W, "%s: request %d repeats a candidate" % (what, r)
        # exact scores of the selected candidates
        s = cum[r, par[r]].astype(np.float64) + (x[r, par[r], tok[r]].astype(np.float64) - rl[r, par[r]])
        fin = np.isfinite(s)
        assert np.array_equal(fin, np.isfinite(co[r])), what
        ds = np.abs(co[r][fin].astype(np.float64) - s[fin])
        assert ds.size == 0 or ds.max() <= SCORE_TOL, "%s: score off by %.3g" % (what, ds.max())
        # order: scores non-increasing, equal scores by flat index
        c = co[r].astype(np.float64)
        assert np.all((c[:-1] > c[1:]) | ((c[:-1] == c[1:]) & (f[:-1] < f[1:]))), what + ": order"
        # selection
        cut = rs[r][-1]
        assert np.all(s[fin] >= cut - EPS), "%s: request %d selects a candidate below the cut" % (what, r)
        sel = set(f.tolist())
        rf = rp[r].astype(np.int64) * V + rt[r]
        must = rf[rs[r] > cut + EPS]
        missing = [int(v) for v in must if int(v) not in sel]
        assert not missing, "%s: request %d misses %s" % (what, r, missing[:5])
        # exact where the oracle's ranking has no near-tie
        top = rs[r]
        gaps = np.abs(np.diff(top[np.isfinite(top)]))
        if gaps.size == 0 or gaps.min() > EPS:
            assert np.array_equal(tok[r], rt[r]) and np.array_equal(par[r], rp[r]), \
                "%s: request %d differs without a near-tie" % (what, r)
            exact_rows += 1
    return exact_rows


@pytest.mark.parametrize("R,Win,V,W", [(2, 4, 1000, 4), (3, 5, 1003, 17), (2, 3, 40, 120), (4, 1, 151936, 100),
                                       (1, 64, 4096, 400), (2, 2, 9001, 1), (3, 7, 2048, 512)])
def test_shapes(gpu, R, Win, V, W):
    note("topk_logits R=%d Win=%d V=%d W=%d" % (R, Win, V, W))
    rng = np.random.default_rng(R * 7919 + V + W)
    x = (rng.standard_normal((R, Win, V)) * 3).astype(np.float32)
    x[:, 0, 1::5] = -np.inf
    cum = (rng.standard_normal((R, Win)) * 2 - 5).astype(np.float32)
    got = _run(gpu, torch.from_numpy(x).cuda(), torch.from_numpy(cum).cuda(), W)
    _check(got, x, cum, W, "shapes")


def test_quantised_ties(gpu):
    """Logits on a coarse grid: many equal logits within a row, so equal
    scores are decided by the flat index (rows with one lse share it)."""
    note("topk_logits quantised ties")
    rng = np.random.default_rng(5)
    R, Win, V, W = 2, 6, 3000, 64
    x = (np.round(rng.standard_normal((R, Win, V)) * 4) / 4).astype(np.float32)
    cum = np.zeros((R, Win), np.float32)
    got = _run(gpu, torch.from_numpy(x).cuda(), torch.from_numpy(cum).cuda(), W)
    _check(got, x, cum, W, "ties")
    # within one row equal logits give bitwise-equal scores: their order is by flat index
    tok, par, co, _ = got
    for r in range(R):
        for j in range(W - 1):
            if par[r, j] == par[r, j + 1] and co[r, j] == co[r, j + 1]:
                assert tok[r, j] < tok[r, j + 1]


@pytest.mark.parametrize("R,Win,V,W", [(2, 4, 1000, 4), (3, 5, 1003, 17), (4, 1, 151936, 100), (3, 7, 2048, 512)])
def test_bf16_logits(gpu, R, Win, V, W):
    """bf16 logits: widened exactly, then the same definition (the oracle gets
    the widened values)."""
    note("topk_logits bf16 R=%d Win=%d V=%d W=%d" % (R, Win, V, W))
    rng = np.random.default_rng(R * 31 + V + W)
    bits = wl.f32_to_bf16_bits((rng.standard_normal((R, Win, V)) * 3).astype(np.float32))
    x = wl.bf16_bits_to_f32(bits)
    cum = (rng.standard_normal((R, Win)) * 2 - 5).astype(np.float32)
    xd = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    got = _run(gpu, xd, torch.from_numpy(cum).cuda(), W)
    _check(got, x, cum, W, "bf16")


@pytest.mark.parametrize("shape", [wl.BEAM_SHORT, wl.BEAM_LONG], ids=lambda s: s.name)
def test_full_size(gpu, shape):
    """The merge at the workload's full size (151,936-word vocabulary, the
    launch the bench times), on device-drawn logits copied to the host for
    the oracle; two launches bitwise equal."""
    note("topk_logits %s full size" % shape.name)
    R, W, V = shape.num_requests, shape.width, shape.vocab
    x = wl.torch_logits((R, W, V), (shape.base_seed, wl.TID_LOGITS, 0, 2), "cuda")
    g = torch.Generator().manual_seed(3)
    cum = (torch.randn((R, W), generator=g) * 3 - 10).float()
    got = _run(gpu, x, cum.cuda(), W)
    again = _run(gpu, x, cum.cuda(), W)
    for a, b in zip(got, again):
        assert np.array_equal(a, b), "two launches differ"
    exact = _check(got, x.cpu().numpy(), cum.numpy(), W, shape.name)
    note("topk_logits %s: %d of %d requests exact (the rest have oracle near-ties)" % (shape.name, exact, R))



def test_full_size_bf16(gpu):
    """bf16 logits at the short-prompt shape's full size."""
    shape = wl.BEAM_SHORT
    note("topk_logits %s full size, bf16 logits" % shape.name)
    R, W, V = shape.num_requests, shape.width, shape.vocab
    x = wl.torch_logits((R, W, V), (shape.base_seed, wl.TID_LOGITS, 0, 2), "cuda").to(torch.bfloat16)
    g = torch.Generator().manual_seed(4)
    cum = (torch.randn((R, W), generator=g) * 3 - 10).float()
    got = _run(gpu, x, cum.cuda(), W)
    _check(got, x.float().cpu().numpy(), cum.numpy(), W, "bf16 full size")
