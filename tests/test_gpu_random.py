"""GPU parity on seeded random shapes, beside the hand-picked cases of the
other GPU tests: packed prefill (both forms, plain and planned, with slack
in max_seqlen), beam decode attention (widths, prompts, suffix lengths,
groups, parents) and the top-k merge (widths up to 512, ties), each against
the oracle at the bars of the other tests."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import assert_attn_close, dev_bf16, host_f64, note
from test_gpu_beam import _decode_case, _decode_check, _eq, _topk

pytestmark = pytest.mark.gpu

HEADS = [(4, 2, 64), (16, 8, 128), (14, 2, 64), (12, 4, 128), (8, 8, 64), (6, 2, 128), (16, 2, 64)]


def _prefill_case(i):
    rng = np.random.default_rng(9100 + i)
    Hq, Hkv, D = HEADS[i % len(HEADS)] if i >= 2 else [(14, 2, 64), (16, 8, 128)][i]
    if i < 2:                                   # big enough for the persistent form
        B = int(rng.integers(150, 300))
        lengths = rng.integers(0, 400, B)
    else:
        B = int(rng.integers(1, 25))
        lengths = rng.choice([0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512],
                             B) if i % 3 == 0 else rng.integers(0, 600, B)
    if lengths.sum() == 0:
        lengths[0] = 5
    return wl.PrefillShape("rand%d" % i, 9200 + i, tuple(int(x) for x in lengths), Hq, Hkv, D), rng


@pytest.mark.parametrize("i", range(12))
def test_random_prefill(gpu, i):
    shape, rng = _prefill_case(i)
    T, Hq, Hkv, D = shape.total_tokens, shape.n_heads_q, shape.n_heads_kv, shape.head_dim
    out_dtype = torch.bfloat16 if i % 2 else torch.float32
    ms = min(T, shape.max_seqlen + int(rng.integers(0, 50)))          # any bound >= the longest sequence
    note("random prefill %d: B=%d T=%d Hq=%d Hkv=%d D=%d max_seqlen=%d out=%s" % (
        i, len(shape.lengths), T, Hq, Hkv, D, ms, out_dtype))
    x = wl.prefill_inputs(shape)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    cu = torch.from_numpy(x["cu_seqlens"]).cuda()
    out = gpu.packed_prefill_attn(q, k, v, cu, ms, scale=1 / math.sqrt(D), out_dtype=out_dtype)
    plan = gpu.prefill_plan(cu, ms, T, Hq, Hkv, D)
    out2 = gpu.packed_prefill_attn_planned(plan, q, k, v, cu, ms, scale=1 / math.sqrt(D), out_dtype=out_dtype)
    gpu.check()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "planned run differs from the plain call"
    ref = oracle.prefill_attn(x["q"], x["k"], x["v"], x["cu_seqlens"])
    assert_attn_close(host_f64(out), ref, "random prefill %d" % i)


@pytest.mark.parametrize("i", range(10))
def test_random_decode(gpu, i):
    rng = np.random.default_rng(9300 + i)
    Hq, Hkv = [(14, 2), (4, 4), (8, 2), (6, 3), (16, 8)][i % 5]
    D = 128 if i % 4 == 3 else 64
    NL, R = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    W = int(rng.integers(1, 65))
    P = int(rng.integers(0, 257 if D == 128 else 577))
    hist = int(rng.integers(0, 8))
    S_cap = int(rng.integers(hist + 1, 9))
    out_dtype = torch.bfloat16 if i % 3 == 1 else torch.float32
    note("random decode %d: NL=%d R=%d W=%d P=%d hist=%d S_cap=%d Hq=%d Hkv=%d D=%d out=%s" % (
        i, NL, R, W, P, hist, S_cap, Hq, Hkv, D, out_dtype))
    c = _decode_case(9400 + i, NL, R, W, P, S_cap, hist, Hq, Hkv, D, parent=bool(i % 4))
    _decode_check(gpu, c, "random decode %d" % i, out_dtype)


@pytest.mark.parametrize("i", range(10))
def test_random_topk(gpu, i):
    rng = np.random.default_rng(9500 + i)
    R, Win = int(rng.integers(1, 5)), int(rng.integers(1, 9))
    V = int(rng.integers(1, 6000))
    W = int(rng.integers(1, min(512, Win * V) + 1))
    note("random topk %d: R=%d Win=%d V=%d W=%d" % (i, R, Win, V, W))
    step = [1 / 8, 1 / 1024, 1.0][i % 3]                               # coarse steps make many exact ties
    lp = (np.round(rng.standard_normal((R, Win, V)) * 3 / step) * step - 5).astype(np.float32)
    if i % 4 == 0:
        lp[:, :, ::5] = -np.inf
    cum = (np.round(rng.standard_normal((R, Win)) / step) * step).astype(np.float32)
    _eq(_topk(gpu, lp, cum, W), oracle.topk_merge(lp, cum, W), "random topk %d" % i)
