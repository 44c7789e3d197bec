"""The seeded input generators: determinism, shapes and bf16 rounding."""
import numpy as np
import torch

import workloads as wl


def test_lengths_match_seeds():
    # lengths uniform on [64,500], seeded; totals are fixed by the seeds
    assert wl.PREFILL_REQUEST.total_tokens == 4395
    assert wl.PREFILL_THROUGHPUT.total_tokens == 269924
    assert len(wl.PREFILL_THROUGHPUT.lengths) == 960
    assert min(wl.PREFILL_THROUGHPUT.lengths) >= 64 and max(wl.PREFILL_THROUGHPUT.lengths) <= 500
    cu = wl.TINY_PREFILL.cu_seqlens()
    assert cu.tolist() == [0, 7, 40, 104, 233]


def test_bf16_rounding_matches_torch():
    # torch's float32 -> bfloat16 conversion rounds to nearest even
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                  65504.0, 1e-30, -0.0, 0.0], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_deterministic():
    a = wl.prefill_inputs(wl.TINY_PREFILL)
    b = wl.prefill_inputs(wl.TINY_PREFILL)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (233, 4, 64) and a["k"].shape == (233, 2, 64)
    lp = wl.beam_logprobs(wl.TINY_BEAM, 1)
    assert lp.shape == (2, 4, 1000) and lp.dtype == np.float32
    # rows are log-probabilities: logsumexp == 0 within fp32 rounding
    lse = np.log(np.exp(lp.astype(np.float64)).sum(-1))
    assert np.abs(lse).max() < 1e-4


def test_torch_generator_seeded():
    a = wl.torch_normal_bf16((4, 8), (1, 2, 3), "cpu")
    b = wl.torch_normal_bf16((4, 8), (1, 2, 3), "cpu")
    c = wl.torch_normal_bf16((4, 8), (1, 2, 4), "cpu")
    assert torch.equal(a, b) and not torch.equal(a, c)
    lp = wl.torch_logprobs((3, 50), (9, 9), "cpu")
    assert torch.allclose(torch.logsumexp(lp.double(), -1), torch.zeros(3, dtype=torch.float64), atol=1e-5)
