"""The packed prefill entry point that allocates nothing
(slm_packed_prefill_attn_noalloc: no context, its scratch memory a static
array of the device) against the context entry point slm_packed_prefill_attn
through the C ABI: bit-for-bit equal outputs on consecutive calls that reuse
the same static array -- a pack large enough for the persistent form (its
work list lives in the array), then a smaller one that also takes it, then a
small pack of the one-workgroup-per-unit form -- plus the capacity refusal
and the caller's error flag.  Runs alone or after the other GPU tests."""
import numpy as np
import pytest
import torch

import bounded_generation_slm_amd as slm
import workloads as wl
from parity_util import dev_bf16, note

pytestmark = pytest.mark.gpu


def _pack(seed, n, Hq, Hkv, D, lo=64, hi=500):
    lengths = tuple(int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, n))
    shape = wl.PrefillShape("noalloc", seed, lengths, Hq, Hkv, D)
    x = wl.prefill_inputs(shape)
    return shape, dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), torch.from_numpy(x["cu_seqlens"]).cuda()


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_context_call(gpu, out_dtype):
    cases = [(2001, 400, 16, 8, 128), (2002, 120, 16, 8, 128), (2003, 6, 14, 2, 64)]
    for seed, n, Hq, Hkv, D in cases:            # second and third calls are smaller than the first
        shape, q, k, v, cu = _pack(seed, n, Hq, Hkv, D)
        persistent = shape.total_tokens * Hq // 128 + 1 >= 8 * 256
        note("noalloc prefill: %d sequences, T=%d, Hq%d/Hkv%d/D%d, %s out, %s form" % (
            n, shape.total_tokens, Hq, Hkv, D, out_dtype, "persistent" if persistent else "per-unit"))
        ref = gpu.packed_prefill_attn(q, k, v, cu, shape.max_seqlen, out_dtype=out_dtype)
        gpu.check()
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = torch.full_like(ref, float("nan"))
        got = slm.slm_packed_prefill_attn_noalloc(q, k, v, cu, shape.max_seqlen, out=out, err_flag=err)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert int(err.item()) == 0
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "differs from the context call"


def test_noalloc_capacity_and_error_flag(gpu):
    note("noalloc prefill: work list beyond the static array; bad cu_seqlens reach the caller's flag")
    T, Hq, Hkv, D = 262144 * 128 // 16, 16, 8, 128     # T * Hq / 128 = 2^18 entries, plus B * Hq = 16 more
    q = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((T, Hkv, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(slm.SlmError) as e:               # refused on the host: nothing is launched
        slm.slm_packed_prefill_attn_noalloc(q, kv, kv, cu, T, out=out)
    assert e.value.status == slm.SLM_ERR_CAPACITY
    del q, kv, out
    x = wl.prefill_inputs(wl.PrefillShape("bad", 5, (10, 10, 10), 4, 2, 64))
    bad = torch.tensor([0, 10, 5, 30], dtype=torch.int32, device="cuda")   # sequence 1 decreasing
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    slm.slm_packed_prefill_attn_noalloc(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), bad, 25, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) != 0
