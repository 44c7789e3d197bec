"""Beam-search prompt prefill feeding decode without a copy: R prompts of one
length P, packed with cu_seqlens, per layer K/V stored as [R*P, Hkv, D] --
which is byte for byte decode's shared-prompt layout [R, P, Hkv, D] -- go
through packed prefill attention (layer by layer), and the very same buffers
are then the prompt K/V of the first decode step.  Both calls through the C
ABI are checked against the oracle on the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import assert_attn_close, dev_bf16, host_bits, host_f64, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("NL,R,P,W,Hq,Hkv,D", [(2, 3, 33, 5, 14, 2, 64), (1, 4, 128, 7, 8, 2, 128)])
def test_prompt_prefill_then_decode(gpu, NL, R, P, W, Hq, Hkv, D):
    note("prompt prefill NL=%d R=%d P=%d then decode W=%d Hq=%d Hkv=%d D=%d" % (NL, R, P, W, Hq, Hkv, D))
    rng = np.random.default_rng(NL * 100 + R * 10 + P)
    bits = lambda *s: wl.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    pq, pk, pv = bits(NL, R * P, Hq, D), bits(NL, R, P, Hkv, D), bits(NL, R, P, Hkv, D)
    cu = np.arange(R + 1, dtype=np.int32) * P
    k_dev, v_dev = dev_bf16(pk), dev_bf16(pv)                     # [NL, R, P, Hkv, D], decode's layout
    cu_d = torch.from_numpy(cu).cuda()
    for l in range(NL):
        out = gpu.packed_prefill_attn(dev_bf16(pq[l]), k_dev[l].view(R * P, Hkv, D), v_dev[l].view(R * P, Hkv, D),
                                      cu_d, P, scale=1 / math.sqrt(D))
        gpu.check()
        ref = oracle.prefill_attn(pq[l], pk[l].reshape(R * P, Hkv, D), pv[l].reshape(R * P, Hkv, D), cu)
        assert_attn_close(host_f64(out), ref, "prompt prefill layer %d" % l)
    # first decode step: the prompt K/V buffers as they are, no history
    q, kn, vn = bits(NL, R, W, Hq, D), bits(NL, R, W, Hkv, D), bits(NL, R, W, Hkv, D)
    S_cap = 4
    sk = np.zeros((NL, R, W, S_cap, Hkv, D), np.uint16)
    sko = torch.zeros(sk.shape, dtype=torch.bfloat16, device="cuda")
    svo = torch.zeros_like(sko)
    out = gpu.beam_decode_attn(dev_bf16(q), k_dev, v_dev, dev_bf16(sk), dev_bf16(sk), dev_bf16(kn), dev_bf16(vn),
                               None, 0, sko, svo)
    gpu.check()
    ref, rk, rv = oracle.beam_decode_attn(q, pk, pv, sk, sk, kn, vn, None, 0)
    assert_attn_close(host_f64(out), ref, "decode after prompt prefill")
    assert np.array_equal(host_bits(sko)[:, :, :, :1], rk[:, :, :, :1])
    assert np.array_equal(host_bits(svo)[:, :, :, :1], rv[:, :, :, :1])


@pytest.mark.parametrize("lengths,W,D", [((17, 64, 1, 100), 5, 64), ((300, 5, 129), 3, 64), ((40, 0, 77), 4, 128)])
def test_ragged_prompt_prefill_then_decode(gpu, lengths, W, D):
    """Prompts of different lengths packed with cu_seqlens: each layer's K/V
    [sum(lengths), Hkv, D] goes through packed prefill, and the same buffers,
    with the same offsets as prompt_cu, are the prompts of the first decode
    step (no copy, no padding).  Both calls checked against the oracle."""
    NL, Hq, Hkv = 2, 14, 2
    R = len(lengths)
    note("ragged prompt prefill lengths=%s then decode W=%d D=%d" % (lengths, W, D))
    rng = np.random.default_rng(sum(lengths) + W + D)
    bits = lambda *s: wl.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    pq, pk, pv = bits(NL, T, Hq, D), bits(NL, T, Hkv, D), bits(NL, T, Hkv, D)
    k_dev, v_dev = dev_bf16(pk), dev_bf16(pv)
    cu_d = torch.from_numpy(cu).cuda()
    for l in range(NL):
        if T == 0:
            break
        out = gpu.packed_prefill_attn(dev_bf16(pq[l]), k_dev[l], v_dev[l], cu_d, max(lengths), scale=1 / math.sqrt(D))
        gpu.check()
        ref = oracle.prefill_attn(pq[l], pk[l], pv[l], cu)
        assert_attn_close(host_f64(out), ref, "ragged prompt prefill layer %d" % l)
    q, kn, vn = bits(NL, R, W, Hq, D), bits(NL, R, W, Hkv, D), bits(NL, R, W, Hkv, D)
    sk = np.zeros((NL, R, W, 2, Hkv, D), np.uint16)
    sko = torch.zeros(sk.shape, dtype=torch.bfloat16, device="cuda")
    svo = torch.zeros_like(sko)
    out = gpu.beam_decode_attn(dev_bf16(q), k_dev, v_dev, dev_bf16(sk), dev_bf16(sk), dev_bf16(kn), dev_bf16(vn),
                               None, 0, sko, svo, prompt_cu=cu_d, prompt_len=max(lengths))
    gpu.check()
    ref, rk, rv = oracle.beam_decode_attn(q, pk, pv, sk, sk, kn, vn, None, 0, prompt_cu=cu)
    assert_attn_close(host_f64(out), ref, "decode after ragged prompt prefill")
    assert np.array_equal(host_bits(sko)[:, :, :, :1], rk[:, :, :, :1])
    assert np.array_equal(host_bits(svo)[:, :, :, :1], rv[:, :, :, :1])
