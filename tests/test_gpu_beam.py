"""GPU parity of the beam path (through the C ABI) against the oracle on the
same seeded inputs: top-k merge (bit-exact tokens, parents, scores), shared-
prompt decode attention (tolerance) with its fused suffix reorder
(bit-exact), the standalone reorder, and the fixed-step sequence."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import assert_attn_close, dev_bf16, host_bits, host_f64, note

pytestmark = pytest.mark.gpu


def _topk(ctx, lp, cum, W):
    t, p, c = ctx.beam_topk_merge(torch.from_numpy(lp).cuda(), torch.from_numpy(cum).cuda(), W)
    return t.cpu().numpy(), p.cpu().numpy(), c.cpu().numpy()


def _eq(got, ref, what):
    for g, r, name in zip(got, ref, ("tokens", "parent", "cum_out")):
        assert np.array_equal(g, r), "%s: %s differ at %s" % (what, name, np.argwhere(g != r)[:5].tolist())


def test_topk_tiny_workload(gpu):
    note("topk tiny_beam first step (Win=1) and step 1 (Win=4)")
    shape = wl.TINY_BEAM
    lp0 = wl.beam_logprobs(shape, 0)
    cum0 = np.zeros((shape.num_requests, 1), np.float32)
    got0 = _topk(gpu, lp0, cum0, shape.width)
    ref0 = oracle.topk_merge(lp0, cum0, shape.width)
    _eq(got0, ref0, "first step")
    lp1 = wl.beam_logprobs(shape, 1)
    _eq(_topk(gpu, lp1, ref0[2], shape.width), oracle.topk_merge(lp1, ref0[2], shape.width), "step 1")


# W = 256 and 257 are the two sides of the switch to the wide form (deeper pipeline, priority rotation)
@pytest.mark.parametrize("R,Win,V,W", [(3, 1, 7, 7), (2, 3, 5, 15), (2, 5, 33, 40), (4, 7, 1003, 512),
                                       (1, 64, 4096, 400), (2, 2, 9001, 1), (3, 9, 3001, 256), (3, 9, 3001, 257)])
def test_topk_shapes_and_ties(gpu, R, Win, V, W):
    note("topk R=%d Win=%d V=%d W=%d tie stress" % (R, Win, V, W))
    rng = np.random.default_rng(R * 1000 + V)
    lp = (np.round(rng.standard_normal((R, Win, V)) * 8) / 8 - 4).astype(np.float32)   # many exact ties
    lp[:, 0, ::3] = -np.inf
    cum = (np.round(rng.standard_normal((R, Win)) * 2) / 2).astype(np.float32)
    _eq(_topk(gpu, lp, cum, W), oracle.topk_merge(lp, cum, W), "ties")
    lpn = rng.standard_normal((R, Win, V)).astype(np.float32)
    _eq(_topk(gpu, lpn, cum, W), oracle.topk_merge(lpn, cum, W), "normal")


@pytest.mark.parametrize("R,Win,V,W", [(32, 16, 100003, 64), (8, 128, 65536, 300), (64, 8, 100000, 300)])
def test_topk_sliced_ranges(gpu, R, Win, V, W):
    # large enough per request that each request's candidates are sliced over
    # its waves (three slices each, at least 4,096 candidates a slice); an odd
    # vocabulary takes the 4-byte load path; exact ties straddle slice bounds
    note("topk sliced R=%d Win=%d V=%d W=%d" % (R, Win, V, W))
    rng = np.random.default_rng(R * 7 + V)
    lp = (np.round(rng.standard_normal((R, Win, V), dtype=np.float32) * 8) / 8 - 12).astype(np.float32)
    cum = -np.sort(-(np.round(rng.standard_normal((R, Win)) * 4) / 4).astype(np.float32), axis=1)   # ranked beams
    _eq(_topk(gpu, lp, cum, W), oracle.topk_merge(lp, cum, W), "sliced")


def test_topk_negative_zero_equals_positive_zero(gpu):
    note("topk -0 vs +0 scores")
    lp = np.array([[[-0.0, 0.0, -1.0, 0.0]]], np.float32)
    cum = np.array([[-0.0]], np.float32)
    _eq(_topk(gpu, lp, cum, 3), oracle.topk_merge(lp, cum, 3), "signed zeros")


@pytest.mark.parametrize("shape", [wl.BEAM_SHORT, wl.BEAM_LONG], ids=lambda s: s.name)
def test_topk_full_size(gpu, shape):
    """The merge at the workload's full size (151,936-word vocabulary), on
    device-drawn log-probs copied to the host for the oracle."""
    note("topk %s full size" % shape.name)
    R, W, V = shape.num_requests, shape.width, shape.vocab
    lp = wl.torch_logprobs((R, W, V), (shape.base_seed, wl.TID_LOGITS, 0, 2), "cuda")
    g = torch.Generator().manual_seed(3)
    cum = (torch.randn((R, W), generator=g) * 3 - 10).float()
    t, p, c = gpu.beam_topk_merge(lp, cum.cuda(), W)
    ref = oracle.topk_merge(lp.cpu().numpy(), cum.numpy(), W)
    _eq((t.cpu().numpy(), p.cpu().numpy(), c.cpu().numpy()), ref, shape.name)


def _decode_case(seed, NL, R, W, P, S_cap, hist, Hq, Hkv, D, parent=True):
    rng = np.random.default_rng(seed)
    bits = lambda *s: wl.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    return dict(q=bits(NL, R, W, Hq, D), pk=bits(NL, R, P, Hkv, D), pv=bits(NL, R, P, Hkv, D),
                sk=bits(NL, R, W, S_cap, Hkv, D), sv=bits(NL, R, W, S_cap, Hkv, D),
                kn=bits(NL, R, W, Hkv, D), vn=bits(NL, R, W, Hkv, D),
                parent=rng.integers(0, W, size=(R, W)).astype(np.int32) if parent else None, hist=hist)


def _decode_gpu(ctx, c, out_dtype=torch.float32):
    S_cap = c["sk"].shape[3]
    sko = torch.zeros(c["sk"].shape, dtype=torch.bfloat16, device="cuda")
    svo = torch.zeros_like(sko)
    par = None if c["parent"] is None else torch.from_numpy(c["parent"]).cuda()
    out = ctx.beam_decode_attn(dev_bf16(c["q"]), dev_bf16(c["pk"]), dev_bf16(c["pv"]), dev_bf16(c["sk"]),
                               dev_bf16(c["sv"]), dev_bf16(c["kn"]), dev_bf16(c["vn"]), par, c["hist"],
                               sko, svo, out_dtype=out_dtype)
    ctx.check()
    return out, sko, svo


def _decode_check(ctx, c, what, out_dtype=torch.float32):
    out, sko, svo = _decode_gpu(ctx, c, out_dtype)
    ref, rk, rv = oracle.beam_decode_attn(c["q"], c["pk"], c["pv"], c["sk"], c["sv"], c["kn"], c["vn"],
                                          c["parent"], c["hist"])
    assert_attn_close(host_f64(out), ref, what)
    n = c["hist"] + 1
    assert np.array_equal(host_bits(sko)[:, :, :, :n], rk[:, :, :, :n]), what + ": suffix K"
    assert np.array_equal(host_bits(svo)[:, :, :, :n], rv[:, :, :, :n]), what + ": suffix V"


@pytest.mark.parametrize("hist", [0, 1, 3])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_decode_tiny_workload(gpu, hist, out_dtype):
    note("decode tiny_beam hist=%d out=%s" % (hist, out_dtype))
    s = wl.TINY_BEAM
    c = _decode_case(11 + hist, s.n_layers, s.num_requests, s.width, s.prompt_len, s.suffix_cap, hist,
                     s.n_heads_q, s.n_heads_kv, s.head_dim)
    _decode_check(gpu, c, "tiny hist=%d" % hist, out_dtype)


@pytest.mark.parametrize("NL,R,W,P,S_cap,hist,Hq,Hkv,D,parent", [
    (1, 1, 1, 0, 1, 0, 2, 1, 64, False),      # no prompt at all, single beam
    (1, 2, 1, 1, 2, 1, 4, 2, 64, True),       # one prompt row
    (2, 1, 5, 64, 3, 2, 14, 2, 64, True),     # exactly one 64-key chunk
    (1, 3, 9, 65, 4, 3, 6, 3, 64, True),      # a 1-key tail chunk
    (1, 2, 7, 200, 8, 7, 8, 2, 128, True),    # head_dim 128, longest suffix
    (3, 2, 33, 130, 5, 4, 14, 2, 64, False),  # identity parent
    (1, 1, 100, 70, 3, 2, 14, 2, 64, True),   # one unit: its 700 rows split over 3 workgroups
])
def test_decode_shapes(gpu, NL, R, W, P, S_cap, hist, Hq, Hkv, D, parent):
    note("decode NL=%d R=%d W=%d P=%d hist=%d Hq=%d Hkv=%d D=%d" % (NL, R, W, P, hist, Hq, Hkv, D))
    c = _decode_case(P * 7 + W, NL, R, W, P, S_cap, hist, Hq, Hkv, D, parent)
    _decode_check(gpu, c, "decode shape")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("NL,R,W,P,hist", [(1, 2, 5, 300, 2), (2, 1, 80, 333, 4)])
def test_decode_long_prompt_forms(gpu, NL, R, W, P, hist, out_dtype):
    """Prompts whose LDS copy leaves room for one workgroup per CU (the
    16-wave form, unstaged output) with a ragged last 64-key chunk; few units
    and many rows, so the rows of a unit are split over several workgroups."""
    note("decode long-prompt form NL=%d R=%d W=%d P=%d hist=%d out=%s" % (NL, R, W, P, hist, out_dtype))
    c = _decode_case(P + W * 3 + hist, NL, R, W, P, hist + 1, hist, 14, 2, 64, True)
    _decode_check(gpu, c, "decode long-prompt form", out_dtype)


@pytest.mark.parametrize("shape", [wl.BEAM_SHORT, wl.BEAM_LONG], ids=lambda s: s.name)
def test_decode_full_size_sampled_layers(gpu, shape):
    """All 24 layers of the last decode step in one launch (the bench's
    launch); two sampled layers checked against the oracle, suffix bit-exact
    for every layer."""
    note("decode %s full size, last step" % shape.name)
    hist = shape.n_steps - 1
    c = _decode_case(shape.base_seed, shape.n_layers, shape.num_requests, shape.width, shape.prompt_len,
                     shape.suffix_cap, hist, shape.n_heads_q, shape.n_heads_kv, shape.head_dim)
    out, sko, svo = _decode_gpu(gpu, c)
    out = host_f64(out)
    for l in (0, shape.n_layers - 1):
        sl = {k: (v[l:l + 1] if isinstance(v, np.ndarray) and k != "parent" else v) for k, v in c.items()}
        ref, rk, rv = oracle.beam_decode_attn(sl["q"], sl["pk"], sl["pv"], sl["sk"], sl["sv"], sl["kn"], sl["vn"],
                                              sl["parent"], hist)
        assert_attn_close(out[l:l + 1], ref, "%s layer %d" % (shape.name, l))
    # suffix: parent's history rows then the new row, every layer
    par = c["parent"]
    r_idx = np.arange(shape.num_requests)[:, None]
    want_k = c["sk"][:, r_idx, par][:, :, :, :hist]
    assert np.array_equal(host_bits(sko)[:, :, :, :hist], want_k)
    assert np.array_equal(host_bits(sko)[:, :, :, hist], c["kn"])
    assert np.array_equal(host_bits(svo)[:, :, :, hist], c["vn"])


def test_reorder_suffix(gpu):
    note("reorder standalone")
    rng = np.random.default_rng(3)
    NL, R, W, S_cap, Hkv, D = 3, 4, 50, 5, 2, 64
    k = wl.f32_to_bf16_bits(rng.standard_normal((NL, R, W, S_cap, Hkv, D)).astype(np.float32))
    v = wl.f32_to_bf16_bits(rng.standard_normal((NL, R, W, S_cap, Hkv, D)).astype(np.float32))
    par = rng.integers(0, W, size=(R, W)).astype(np.int32)
    ko = torch.zeros(k.shape, dtype=torch.bfloat16, device="cuda")
    vo = torch.zeros_like(ko)
    gpu.beam_reorder_suffix(torch.from_numpy(par).cuda(), dev_bf16(k), dev_bf16(v), 4, ko, vo)
    gpu.check()
    rk, rv = oracle.reorder_suffix(par, k, v, 4)
    assert np.array_equal(host_bits(ko)[:, :, :, :4], rk[:, :, :, :4])
    assert np.array_equal(host_bits(vo)[:, :, :, :4], rv[:, :, :, :4])
    assert np.all(host_bits(ko)[:, :, :, 4] == 0)           # rows >= rows untouched


@pytest.mark.parametrize("lengths,W,hist", [((0, 64, 1, 130, 7), 6, 3), ((480, 33, 200), 4, 2)])
def test_decode_ragged_prompts(gpu, lengths, W, hist):
    """Prompts of different lengths packed per layer (offsets prompt_cu): an
    empty prompt, a whole 64-key chunk, one key, ragged tails; the 8-wave and
    the 16-wave forms (longest 130 and 480).  History through the parents,
    suffix bit-exact."""
    NL, Hq, Hkv, D, S_cap = 2, 14, 2, 64, hist + 1
    R = len(lengths)
    note("decode ragged prompts lengths=%s W=%d hist=%d" % (lengths, W, hist))
    rng = np.random.default_rng(sum(lengths) * 3 + W)
    bits = lambda *s: wl.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q, pk, pv = bits(NL, R, W, Hq, D), bits(NL, T, Hkv, D), bits(NL, T, Hkv, D)
    sk, sv = bits(NL, R, W, S_cap, Hkv, D), bits(NL, R, W, S_cap, Hkv, D)
    kn, vn = bits(NL, R, W, Hkv, D), bits(NL, R, W, Hkv, D)
    par = rng.integers(0, W, size=(R, W)).astype(np.int32)
    sko = torch.zeros(sk.shape, dtype=torch.bfloat16, device="cuda")
    svo = torch.zeros_like(sko)
    out = gpu.beam_decode_attn(dev_bf16(q), dev_bf16(pk), dev_bf16(pv), dev_bf16(sk), dev_bf16(sv), dev_bf16(kn),
                               dev_bf16(vn), torch.from_numpy(par).cuda(), hist, sko, svo,
                               prompt_cu=torch.from_numpy(cu).cuda(), prompt_len=max(lengths))
    gpu.check()
    ref, rk, rv = oracle.beam_decode_attn(q, pk, pv, sk, sv, kn, vn, par, hist, prompt_cu=cu)
    assert_attn_close(host_f64(out), ref, "decode ragged prompts")
    n = hist + 1
    assert np.array_equal(host_bits(sko)[:, :, :, :n], rk[:, :, :, :n])
    assert np.array_equal(host_bits(svo)[:, :, :, :n], rv[:, :, :, :n])


def test_decode_bad_prompt_offsets_are_flagged(gpu):
    note("decode bad prompt offsets -> device error flag")
    NL, R, W, Hq, Hkv, D = 1, 2, 2, 4, 2, 64
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 6, 5], dtype=torch.int32, device="cuda")          # decreasing
    gpu.beam_decode_attn(z(NL, R, W, Hq, D), z(NL, 5, Hkv, D), z(NL, 5, Hkv, D), None, None, z(NL, R, W, Hkv, D),
                         z(NL, R, W, Hkv, D), None, 0, z(NL, R, W, 1, Hkv, D), z(NL, R, W, 1, Hkv, D),
                         prompt_cu=cu, prompt_len=6)
    with pytest.raises(Exception, match="cu_seqlens|offset|prompt"):
        gpu.check()


def test_bad_parent_is_flagged(gpu):
    note("reorder bad parent -> device error flag")
    k = torch.zeros((1, 1, 4, 2, 1, 64), dtype=torch.bfloat16, device="cuda")
    par = torch.tensor([[0, 1, 7, 2]], dtype=torch.int32, device="cuda")
    gpu.beam_reorder_suffix(par, k, k.clone(), 2, torch.zeros_like(k), torch.zeros_like(k))
    with pytest.raises(Exception, match="parent"):
        gpu.check()


def run_beam_search_gpu(ctx, shape, step_inputs, prefix_k, prefix_v, logprobs):
    """The fixed-step sequence on the GPU: first merge (one beam in), then per
    step decode attention reading history through the last parents, then the
    merge; finally the standalone reorder by the last parents."""
    R, W, N = shape.num_requests, shape.width, shape.n_steps
    NL, Hkv, D = shape.n_layers, shape.n_heads_kv, shape.head_dim
    pk, pv = dev_bf16(prefix_k), dev_bf16(prefix_v)
    tok, par, cum = ctx.beam_topk_merge(torch.from_numpy(logprobs(0)).cuda(),
                                        torch.zeros((R, 1), dtype=torch.float32, device="cuda"), W)
    res = dict(tokens=[tok.cpu().numpy()], parent=[par.cpu().numpy()], cum=[cum.cpu().numpy()], attn=[],
               suffix_k=[], suffix_v=[])
    sshape = (NL, R, W, shape.suffix_cap, Hkv, D)
    bufs = [(torch.zeros(sshape, dtype=torch.bfloat16, device="cuda"),
             torch.zeros(sshape, dtype=torch.bfloat16, device="cuda")) for _ in range(2)]
    for t in range(1, N + 1):
        x = step_inputs(t)
        (ski, svi), (sko, svo) = bufs[(t + 1) % 2], bufs[t % 2]
        out = ctx.beam_decode_attn(dev_bf16(x["q"]), pk, pv, ski, svi, dev_bf16(x["k_new"]), dev_bf16(x["v_new"]),
                                   par, t - 1, sko, svo)
        res["attn"].append(host_f64(out))
        res["suffix_k"].append(host_bits(sko))
        res["suffix_v"].append(host_bits(svo))
        tok, par, cum = ctx.beam_topk_merge(torch.from_numpy(logprobs(t)).cuda(), cum, W)
        res["tokens"].append(tok.cpu().numpy())
        res["parent"].append(par.cpu().numpy())
        res["cum"].append(cum.cpu().numpy())
    sko, svo = bufs[N % 2]
    fk, fv = torch.zeros(sshape, dtype=torch.bfloat16, device="cuda"), torch.zeros(sshape, dtype=torch.bfloat16,
                                                                                     device="cuda")
    ctx.beam_reorder_suffix(par, sko, svo, N, fk, fv)
    ctx.check()
    res["final_suffix_k"], res["final_suffix_v"] = host_bits(fk), host_bits(fv)
    return res


def test_beam_sequence_tiny(gpu):
    note("beam sequence tiny_beam, 4 steps")
    shape = wl.TINY_BEAM
    st = wl.beam_static_inputs(shape)
    step_inputs = lambda t: wl.beam_step_inputs(shape, t)
    lps = {t: wl.beam_logprobs(shape, t) for t in range(shape.n_steps + 1)}
    got = run_beam_search_gpu(gpu, shape, step_inputs, st["prefix_k"], st["prefix_v"], lps.__getitem__)
    ref = oracle.beam_search(step_inputs, st["prefix_k"], st["prefix_v"], lps.__getitem__, shape.width,
                             shape.n_steps)
    for t in range(shape.n_steps + 1):
        _eq((got["tokens"][t], got["parent"][t], got["cum"][t]), (ref["tokens"][t], ref["parent"][t], ref["cum"][t]),
            "merge %d" % t)
    for t in range(shape.n_steps):
        assert_attn_close(got["attn"][t], ref["attn"][t], "attn step %d" % (t + 1))
        assert np.array_equal(got["suffix_k"][t][:, :, :, :t + 1], ref["suffix_k"][t][:, :, :, :t + 1])
        assert np.array_equal(got["suffix_v"][t][:, :, :, :t + 1], ref["suffix_v"][t][:, :, :, :t + 1])
    assert np.array_equal(got["final_suffix_k"], ref["final_suffix_k"])
    assert np.array_equal(got["final_suffix_v"], ref["final_suffix_v"])


def test_beam_search_driver_tiny(gpu):
    """The one-call driver on the tiny beam shape: every output against the
    oracle's fixed-step sequence (merges bit-exact, attention of each step
    within tolerance, final suffix and backtracked sequences bit-exact)."""
    note("beam search driver tiny_beam, 4 steps")
    shape = wl.TINY_BEAM
    N = shape.n_steps
    st = wl.beam_static_inputs(shape)
    steps = {t: wl.beam_step_inputs(shape, t) for t in range(1, N + 1)}
    lps = [wl.beam_logprobs(shape, t) for t in range(N + 1)]
    state = gpu.beam_search_state(shape.n_layers, shape.num_requests, shape.width, N, shape.n_heads_q,
                                  shape.n_heads_kv, shape.head_dim, attn_per_step=True)
    gpu.beam_search(state, dev_bf16(st["prefix_k"]), dev_bf16(st["prefix_v"]),
                    [torch.from_numpy(lp).cuda() for lp in lps], [dev_bf16(steps[t]["q"]) for t in steps],
                    [dev_bf16(steps[t]["k_new"]) for t in steps], [dev_bf16(steps[t]["v_new"]) for t in steps])
    gpu.check()
    ref = oracle.beam_search(steps.__getitem__, st["prefix_k"], st["prefix_v"], lps.__getitem__, shape.width, N)
    for t in range(N + 1):
        _eq((state["tokens"][t].cpu().numpy(), state["parent"][t].cpu().numpy(), state["cum"][t].cpu().numpy()),
            (ref["tokens"][t], ref["parent"][t], ref["cum"][t]), "merge %d" % t)
    for t in range(N):
        assert_attn_close(host_f64(state["attn_out"][t]), ref["attn"][t], "attn step %d" % (t + 1))
    assert np.array_equal(host_bits(state["final_k"]), ref["final_suffix_k"])
    assert np.array_equal(host_bits(state["final_v"]), ref["final_suffix_v"])
    assert np.array_equal(state["sequences"].cpu().numpy(), ref["sequences"])


@pytest.mark.parametrize("n,R,W", [(1, 3, 5), (5, 2, 100), (6, 8, 400)])
def test_backtrack(gpu, n, R, W):
    note("backtrack n=%d R=%d W=%d" % (n, R, W))
    rng = np.random.default_rng(n * 100 + W)
    tok = rng.integers(0, 151936, size=(n, R, W)).astype(np.int32)
    par = rng.integers(0, W, size=(n, R, W)).astype(np.int32)
    par[0] = 0
    seq = gpu.beam_backtrack(torch.from_numpy(tok).cuda(), torch.from_numpy(par).cuda())
    gpu.check()
    assert np.array_equal(seq.cpu().numpy(), oracle.beam_backtrack(tok, par))


def test_backtrack_bad_parent_is_flagged(gpu):
    note("backtrack bad parent -> device error flag")
    tok = torch.zeros((3, 1, 4), dtype=torch.int32, device="cuda")
    par = torch.zeros((3, 1, 4), dtype=torch.int32, device="cuda")
    par[2, 0, 1] = 9
    gpu.beam_backtrack(tok, par)
    with pytest.raises(Exception, match="parent"):
        gpu.check()
