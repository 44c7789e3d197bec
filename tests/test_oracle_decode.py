"""Pins of the oracle's shared-prompt beam decode attention and suffix
reorder: self-check (b) -- every beam's K/V materialised as prompt + its
parent's history + new row, then torch SDPA in float64 --, a cross-pin with
the prefill oracle's last row, closed forms, and ancestry reconstruction for
the reorder.  Catches: history read without the parent indirection, the new
row dropped or duplicated, prompt not shared per request, GQA mapping, scale."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def _f64(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def _rand_bits(rng, shape):
    return wl.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _case(seed, NL=2, R=3, W=5, P=7, hist=2, S_cap=4, Hq=6, Hkv=2, D=16):
    rng = np.random.default_rng(seed)
    return dict(
        q=_rand_bits(rng, (NL, R, W, Hq, D)),
        pk=_rand_bits(rng, (NL, R, P, Hkv, D)), pv=_rand_bits(rng, (NL, R, P, Hkv, D)),
        sk=_rand_bits(rng, (NL, R, W, S_cap, Hkv, D)), sv=_rand_bits(rng, (NL, R, W, S_cap, Hkv, D)),
        kn=_rand_bits(rng, (NL, R, W, Hkv, D)), vn=_rand_bits(rng, (NL, R, W, Hkv, D)),
        parent=rng.integers(0, W, size=(R, W)).astype(np.int32), hist=hist)


def _materialised_reference(c, scale):
    """Self-check (b): per beam, concat(prompt copy, parent's history, new row),
    then plain attention (torch SDPA, float64, no mask)."""
    q, pk, pv, sk, sv, kn, vn, par, hist = (c[x] for x in ("q", "pk", "pv", "sk", "sv", "kn", "vn", "parent", "hist"))
    NL, R, W, Hq, D = q.shape
    G = Hq // pk.shape[3]
    out = np.zeros(q.shape)
    for l in range(NL):
        for r in range(R):
            for j in range(W):
                src = j if par is None else par[r, j]
                K = np.concatenate([_f64(pk[l, r]), _f64(sk[l, r, src, :hist]), _f64(kn[l, r, j])[None]])
                V = np.concatenate([_f64(pv[l, r]), _f64(sv[l, r, src, :hist]), _f64(vn[l, r, j])[None]])
                qq = torch.from_numpy(_f64(q[l, r, j]))[:, None, :]                  # [Hq,1,D]
                kk = torch.from_numpy(K).transpose(0, 1).repeat_interleave(G, 0)      # [Hq,n,D]
                vv = torch.from_numpy(V).transpose(0, 1).repeat_interleave(G, 0)
                o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
                out[l, r, j] = o[:, 0].numpy()
    return out


@pytest.mark.parametrize("seed,hist,use_parent", [(1, 0, True), (2, 2, True), (3, 3, False)])
def test_vs_materialised(seed, hist, use_parent):
    c = _case(seed, hist=hist)
    if not use_parent:
        c["parent"] = None
    scale = 1 / math.sqrt(16)
    out, sko, svo = oracle.beam_decode_attn(c["q"], c["pk"], c["pv"], c["sk"], c["sv"], c["kn"], c["vn"],
                                            c["parent"], hist, scale)
    np.testing.assert_allclose(out, _materialised_reference(c, scale), rtol=1e-11, atol=1e-12)


def test_suffix_out_carries_parent_history_and_new_row():
    # every row value encodes (layer, request, beam, row, head): a wrong index shows
    NL, R, W, S_cap, Hkv, D = 2, 2, 4, 3, 2, 8
    def code(l, r, j, i, g):
        return float((((l * 7 + r) * 11 + j) * 5 + i) * 3 + g)
    sk = np.zeros((NL, R, W, S_cap, Hkv, D), np.float32)
    for l, r, j, i, g in np.ndindex(NL, R, W, S_cap, Hkv):
        sk[l, r, j, i, g] = code(l, r, j, i, g)
    kn = np.zeros((NL, R, W, Hkv, D), np.float32)
    for l, r, j, g in np.ndindex(NL, R, W, Hkv):
        kn[l, r, j, g] = 1000 + code(l, r, j, 0, g)
    par = np.array([[3, 3, 0, 1], [2, 0, 0, 2]], np.int32)
    rng = np.random.default_rng(0)
    q = _rand_bits(rng, (NL, R, W, 4, D))
    pk = _rand_bits(rng, (NL, R, 5, Hkv, D))
    skb, knb = wl.f32_to_bf16_bits(sk), wl.f32_to_bf16_bits(kn)
    out, sko, svo = oracle.beam_decode_attn(q, pk, pk, skb, skb, knb, knb, par, 2)
    got = wl.bf16_bits_to_f32(sko)
    for l, r, j, g in np.ndindex(NL, R, W, Hkv):
        for i in range(2):
            assert np.all(got[l, r, j, i, g] == wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(
                np.float32(code(l, r, par[r, j], i, g)))))
        assert np.all(got[l, r, j, 2, g] == wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(
            np.float32(1000 + code(l, r, j, 0, g)))))
    assert np.array_equal(sko, svo)


def test_single_beam_equals_prefill_last_row():
    # W=1, identity parent: decode over prompt+history+new == causal prefill's last row
    rng = np.random.default_rng(11)
    P, hist, Hq, Hkv, D = 9, 3, 4, 2, 32
    n = P + hist + 1
    k_seq, v_seq = _rand_bits(rng, (n, Hkv, D)), _rand_bits(rng, (n, Hkv, D))
    q_seq = _rand_bits(rng, (n, Hq, D))
    pre = oracle.prefill_attn(q_seq, k_seq, v_seq, np.array([0, n], np.int32))
    S_cap = 4
    sk = np.zeros((1, 1, 1, S_cap, Hkv, D), np.uint16); sv = np.zeros_like(sk)
    sk[0, 0, 0, :hist], sv[0, 0, 0, :hist] = k_seq[P:P + hist], v_seq[P:P + hist]
    out, _, _ = oracle.beam_decode_attn(q_seq[None, None, None, -1], k_seq[None, None, :P], v_seq[None, None, :P],
                                        sk, sv, k_seq[None, None, None, -1], v_seq[None, None, None, -1], None, hist)
    np.testing.assert_allclose(out[0, 0, 0], pre[-1], rtol=1e-12, atol=1e-13)


def test_zero_query_is_mean_of_values():
    c = _case(5, hist=2)
    c["q"] = np.zeros_like(c["q"])
    out, _, _ = oracle.beam_decode_attn(c["q"], c["pk"], c["pv"], c["sk"], c["sv"], c["kn"], c["vn"], c["parent"], 2)
    NL, R, W, Hq, D = out.shape
    for l, r, j, h in np.ndindex(NL, R, W, Hq):
        g = h // 3
        src = c["parent"][r, j]
        vals = np.concatenate([_f64(c["pv"][l, r, :, g]), _f64(c["sv"][l, r, src, :2, g]), _f64(c["vn"][l, r, j, g])[None]])
        np.testing.assert_allclose(out[l, r, j, h], vals.mean(0), rtol=1e-13, atol=1e-14)


def test_identical_beams_give_identical_outputs():
    c = _case(6, hist=1)
    for key in ("q", "kn", "vn"):
        c[key][:, :, 1:] = c[key][:, :, :1]
    c["parent"][:] = 0
    out, _, _ = oracle.beam_decode_attn(c["q"], c["pk"], c["pv"], c["sk"], c["sv"], c["kn"], c["vn"], c["parent"], 1)
    for j in range(1, out.shape[2]):
        assert np.array_equal(out[:, :, j], out[:, :, 0])


def test_reorder_identity_and_ancestry():
    rng = np.random.default_rng(9)
    NL, R, W, S_cap, Hkv, D = 2, 2, 5, 4, 1, 4
    k = _rand_bits(rng, (NL, R, W, S_cap, Hkv, D))
    ident = np.tile(np.arange(W, dtype=np.int32), (R, 1))
    ko, vo = oracle.reorder_suffix(ident, k, k, 3)
    assert np.array_equal(ko[:, :, :, :3], k[:, :, :, :3])
    # composition over steps == ancestry lookup: row i written at generation i
    # carries the id of the beam that wrote it (small integers: exact in bf16)
    state = np.zeros((NL, R, W, S_cap, Hkv, D), np.uint16)
    parents = [rng.integers(0, W, size=(R, W)).astype(np.int32) for _ in range(S_cap)]
    for i in range(S_cap):
        state, _ = oracle.reorder_suffix(parents[i], state, state, i)
        for r, j in np.ndindex(R, W):
            state[:, r, j, i] = wl.f32_to_bf16_bits(np.float32(10 * i + j))
    for r, j in np.ndindex(R, W):
        anc = j
        for i in range(S_cap - 1, -1, -1):
            assert np.all(wl.bf16_bits_to_f32(state[:, r, j, i]) == 10 * i + anc)
            anc = parents[i][r, anc]


def _ragged_case(seed, lengths, NL=2, W=4, hist=2, S_cap=3, Hq=6, Hkv=2, D=16):
    """Prompts of different lengths packed per layer as [NL, sum(lengths), Hkv, D]."""
    rng = np.random.default_rng(seed)
    R = len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    return dict(
        q=_rand_bits(rng, (NL, R, W, Hq, D)),
        pk=_rand_bits(rng, (NL, T, Hkv, D)), pv=_rand_bits(rng, (NL, T, Hkv, D)),
        sk=_rand_bits(rng, (NL, R, W, S_cap, Hkv, D)), sv=_rand_bits(rng, (NL, R, W, S_cap, Hkv, D)),
        kn=_rand_bits(rng, (NL, R, W, Hkv, D)), vn=_rand_bits(rng, (NL, R, W, Hkv, D)),
        parent=rng.integers(0, W, size=(R, W)).astype(np.int32), hist=hist, cu=cu)


def test_ragged_prompts_vs_materialised():
    """Prompts of lengths 0, 1, 7 and 13 in one packed call: each request's
    result equals the materialised reference of that request alone with its
    own prompt (an empty prompt leaves only the suffix keys)."""
    c = _ragged_case(11, [0, 1, 7, 13])
    scale = 0.3
    out, sko, svo = oracle.beam_decode_attn(c["q"], c["pk"], c["pv"], c["sk"], c["sv"], c["kn"], c["vn"],
                                            c["parent"], c["hist"], scale, prompt_cu=c["cu"])
    cu = c["cu"]
    for r in range(len(cu) - 1):
        one = dict(q=c["q"][:, r:r + 1], pk=c["pk"][:, cu[r]:cu[r + 1]][:, None], pv=c["pv"][:, cu[r]:cu[r + 1]][:, None],
                   sk=c["sk"][:, r:r + 1], sv=c["sv"][:, r:r + 1], kn=c["kn"][:, r:r + 1], vn=c["vn"][:, r:r + 1],
                   parent=c["parent"][r:r + 1], hist=c["hist"])
        np.testing.assert_allclose(out[:, r:r + 1], _materialised_reference(one, scale), rtol=1e-11, atol=1e-12)
    # the suffix reorder does not depend on the prompts
    dense = oracle.beam_decode_attn(c["q"], np.zeros((2, 4, 1, 2, 16), np.uint16), np.zeros((2, 4, 1, 2, 16), np.uint16),
                                    c["sk"], c["sv"], c["kn"], c["vn"], c["parent"], c["hist"], scale)
    assert np.array_equal(sko, dense[1]) and np.array_equal(svo, dense[2])


def test_ragged_equal_lengths_is_the_dense_layout():
    """Equal lengths P packed with offsets r*P are byte for byte the dense
    [NL, R, P, Hkv, D] layout: identical results."""
    c = _case(12, R=3, P=9)
    NL, R, P, Hkv, D = c["pk"].shape
    cu = (np.arange(R + 1) * P).astype(np.int32)
    a = oracle.beam_decode_attn(c["q"], c["pk"], c["pv"], c["sk"], c["sv"], c["kn"], c["vn"], c["parent"], c["hist"])
    b = oracle.beam_decode_attn(c["q"], c["pk"].reshape(NL, R * P, Hkv, D), c["pv"].reshape(NL, R * P, Hkv, D),
                                c["sk"], c["sv"], c["kn"], c["vn"], c["parent"], c["hist"], prompt_cu=cu)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_ragged_rejects_bad_offsets():
    c = _ragged_case(13, [2, 3])
    bad = c["cu"].copy()
    bad[1] = 6                                     # offsets 0, 6, 5: decreasing
    with pytest.raises(ValueError):
        oracle.beam_decode_attn(c["q"], c["pk"], c["pv"], c["sk"], c["sv"], c["kn"], c["vn"], c["parent"], c["hist"],
                                prompt_cu=bad)
