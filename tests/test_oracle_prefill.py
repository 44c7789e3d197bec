"""Pins of the oracle's packed prefill attention and last-token gather
against things other than itself: an independent library routine (torch's
scaled_dot_product_attention in float64), padded-plus-masked dense attention,
closed forms, a hand-worked example and invariances.

Mistakes each pin would catch: dropped or wrong scale (SDPA, hand example),
wrong GQA head mapping (SDPA with repeat_interleave), causal off-by-one (L=1,
hand example, SDPA), attention across sequences (padded/masked, permutation),
transposed operands (SDPA), wrong normalisation (q=0 mean)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def _sdpa_reference(q, k, v, cu, scale):
    """torch SDPA (float64, CPU) per sequence, K/V repeated per GQA group."""
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros((T, Hq, D))
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e == s:
            continue
        qq = torch.from_numpy(_f64(q[s:e])).transpose(0, 1)              # [Hq,L,D]
        kk = torch.from_numpy(_f64(k[s:e])).transpose(0, 1).repeat_interleave(G, 0)
        vv = torch.from_numpy(_f64(v[s:e])).transpose(0, 1).repeat_interleave(G, 0)
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=scale)
        out[s:e] = o.transpose(0, 1).numpy()
    return out


def _padded_masked_reference(q, k, v, cu, scale):
    """Self-check (a): pad every sequence to max length, dense attention with
    -inf for j>i or j>=L, compare on the valid rows only."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    B = len(cu) - 1
    Lmax = int(max(cu[1:] - cu[:-1])) if B else 0
    Qp = np.zeros((B, Lmax, Hq, D)); Kp = np.zeros((B, Lmax, Hkv, D)); Vp = np.zeros((B, Lmax, Hkv, D))
    for b in range(B):
        s, e = int(cu[b]), int(cu[b + 1])
        Qp[b, :e - s], Kp[b, :e - s], Vp[b, :e - s] = _f64(q[s:e]), _f64(k[s:e]), _f64(v[s:e])
    out = np.zeros((T, Hq, D))
    for h in range(Hq):
        g = h // G
        S = np.einsum("bid,bjd->bij", Qp[:, :, h], Kp[:, :, g]) * scale
        i = np.arange(Lmax)[:, None]; j = np.arange(Lmax)[None, :]
        for b in range(B):
            L = int(cu[b + 1] - cu[b])
            mask = (j > i) | (j >= L)
            Sb = np.where(mask, -np.inf, S[b])
            Sb = Sb - Sb.max(axis=1, keepdims=True)
            P = np.exp(Sb)
            O = (P @ Vp[b, :, g]) / P.sum(axis=1, keepdims=True)
            out[int(cu[b]):int(cu[b + 1]), h] = O[:L]
    return out


def test_tiny_workload_vs_sdpa_and_padded():
    x = wl.prefill_inputs(wl.TINY_PREFILL)
    scale = 1 / math.sqrt(64)
    out = oracle.prefill_attn(x["q"], x["k"], x["v"], x["cu_seqlens"], scale)
    ref = _sdpa_reference(x["q"], x["k"], x["v"], x["cu_seqlens"], scale)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    pad = _padded_masked_reference(x["q"], x["k"], x["v"], x["cu_seqlens"], scale)
    np.testing.assert_allclose(out, pad, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 16), (6, 2, 32), (8, 1, 8), (14, 2, 64)])
def test_gqa_shapes_vs_sdpa(Hq, Hkv, D):
    rng = np.random.default_rng(Hq * 100 + Hkv)
    lengths = [1, 5, 0, 17, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, Hq, D)).astype(np.float32))
    k = wl.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    v = wl.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    scale = 0.37
    out = oracle.prefill_attn(q, k, v, cu, scale)
    np.testing.assert_allclose(out, _sdpa_reference(q, k, v, cu, scale), rtol=1e-11, atol=1e-12)


def test_hand_worked_example():
    """tests/golden/prefill_hand_example.json: two tokens, D=2, scale 1,
    worked by hand (row 0 sees only key 0; row 1 weights e^0 and e^2)."""
    ex = json.load(open(os.path.join(GOLDEN, "prefill_hand_example.json")))
    q = wl.f32_to_bf16_bits(np.array(ex["q"], np.float32))
    k = wl.f32_to_bf16_bits(np.array(ex["k"], np.float32))
    v = wl.f32_to_bf16_bits(np.array(ex["v"], np.float32))
    out = oracle.prefill_attn(q, k, v, np.array(ex["cu_seqlens"], np.int32), ex["scale"])
    e2 = math.exp(2.0)
    p0, p1 = 1 / (1 + e2), e2 / (1 + e2)
    expect = np.array([[[1.0, 2.0]], [[p0 * 1 + p1 * 3, p0 * 2 + p1 * -1]]])
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out.reshape(-1), np.array(ex["expected_flat"]), rtol=0, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(3)
    Hq, Hkv, D = 4, 2, 32
    lengths = [1, 9, 30]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    k = wl.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    v = wl.f32_to_bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32))
    # q == 0: uniform weights over keys 0..i -> running mean of v
    q0 = np.zeros((T, Hq, D), np.uint16)
    out = oracle.prefill_attn(q0, k, v, cu, 0.125)
    for b in range(3):
        s, e = cu[b], cu[b + 1]
        vb = _f64(v[s:e])
        csum = np.cumsum(vb, axis=0) / np.arange(1, e - s + 1)[:, None, None]
        for h in range(Hq):
            np.testing.assert_allclose(out[s:e, h], csum[:, h // 2], rtol=1e-13, atol=1e-14)
    # L = 1: the only key is itself -> out = v exactly
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, Hq, D)).astype(np.float32))
    out = oracle.prefill_attn(q, k, v, cu, 0.125)
    for h in range(Hq):
        assert np.array_equal(out[0, h], _f64(v[0, h // 2]))
    # one dominant key: q . k_j* huge for one visible j* -> out ~= v_j*
    kd = np.zeros((T, Hkv, D), np.float32)
    kd[cu[2] + 4, :, 0] = 1.0
    qd = np.zeros((T, Hq, D), np.float32)
    qd[:, :, 0] = 64.0
    out = oracle.prefill_attn(wl.f32_to_bf16_bits(qd), wl.f32_to_bf16_bits(kd), v, cu, 1.0)
    for i in range(4, 30):
        for h in range(Hq):
            np.testing.assert_allclose(out[cu[2] + i, h], _f64(v[cu[2] + 4, h // 2]), atol=1e-20)


def test_packing_invariances():
    x = wl.prefill_inputs(wl.TINY_PREFILL)
    q, k, v, cu = x["q"], x["k"], x["v"], x["cu_seqlens"]
    full = oracle.prefill_attn(q, k, v, cu)
    # permuting the packing order permutes the outputs
    order = [2, 0, 3, 1]
    segs = [slice(int(cu[b]), int(cu[b + 1])) for b in range(4)]
    qp = np.concatenate([q[segs[b]] for b in order]); kp = np.concatenate([k[segs[b]] for b in order])
    vp = np.concatenate([v[segs[b]] for b in order])
    cup = np.concatenate([[0], np.cumsum([cu[b + 1] - cu[b] for b in order])]).astype(np.int32)
    outp = oracle.prefill_attn(qp, kp, vp, cup)
    for n, b in enumerate(order):
        np.testing.assert_array_equal(outp[int(cup[n]):int(cup[n + 1])], full[segs[b]])
    # splitting the pack into two calls changes nothing
    a = oracle.prefill_attn(q[:40], k[:40], v[:40], np.array([0, 7, 40], np.int32))
    bpart = oracle.prefill_attn(q[40:], k[40:], v[40:], np.array([0, 64, 193], np.int32))
    np.testing.assert_array_equal(np.concatenate([a, bpart]), full)
    # rows variant agrees with the full call
    toks = np.array([0, 6, 39, 40, 232, 100], np.int64)
    heads = np.array([0, 3, 1, 2, 3, 0], np.int32)
    rows = oracle.prefill_attn_rows(q, k, v, cu, toks, heads)
    np.testing.assert_array_equal(rows, full[toks, heads])
    # Hkv == Hq with K/V repeated per group equals GQA
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    np.testing.assert_array_equal(oracle.prefill_attn(q, kr, vr, cu), full)


def test_gather_last_row_patterns():
    # row t holds bf16(t mod 251 + column): any index error shows
    lengths = [3, 0, 1, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H = int(cu[-1]), 16
    pattern = lambda t: np.array([(t % 251) + c for c in range(H)], np.float32)
    hidden = wl.f32_to_bf16_bits(np.stack([pattern(t) for t in range(T)]))
    out = oracle.gather_last(hidden, cu)
    assert np.array_equal(out[0], wl.f32_to_bf16_bits(pattern(2)))
    assert np.array_equal(out[1], np.zeros(H, np.uint16))           # empty sequence
    assert np.array_equal(out[2], wl.f32_to_bf16_bits(pattern(3)))
    assert np.array_equal(out[3], wl.f32_to_bf16_bits(pattern(10)))
