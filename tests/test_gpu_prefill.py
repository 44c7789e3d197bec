"""GPU parity of packed causal GQA prefill attention and the last-token
gather (through the C ABI) against the fp64 oracle on the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import assert_attn_close, dev_bf16, host_bits, host_f64, note

pytestmark = pytest.mark.gpu


def _run(ctx, x, Hq, Hkv, D, out_dtype=torch.float32, max_seqlen=None):
    cu = x["cu_seqlens"]
    L = np.diff(cu)
    ms = int(L.max()) if len(L) else 0
    ms = ms if max_seqlen is None else max_seqlen
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    cu_d = torch.from_numpy(cu).cuda()
    out = ctx.packed_prefill_attn(q, k, v, cu_d, ms, scale=1 / math.sqrt(D), out_dtype=out_dtype)
    ctx.check()
    return out


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_workload(gpu, out_dtype):
    note("prefill tiny_prefill out=%s" % out_dtype)
    x = wl.prefill_inputs(wl.TINY_PREFILL)
    out = _run(gpu, x, 4, 2, 64, out_dtype)
    ref = oracle.prefill_attn(x["q"], x["k"], x["v"], x["cu_seqlens"])
    assert_attn_close(host_f64(out), ref, "tiny_prefill")


def test_prefill_request_and_gather(gpu):
    shape = wl.PREFILL_REQUEST
    note("prefill prefill_request (15 seqs, T=4395, Hq16/Hkv8/D128) + gather")
    x = wl.prefill_inputs(shape)
    out = _run(gpu, x, 16, 8, 128)
    ref = oracle.prefill_attn(x["q"], x["k"], x["v"], x["cu_seqlens"])
    assert_attn_close(host_f64(out), ref, "prefill_request")
    out_bf = _run(gpu, x, 16, 8, 128, torch.bfloat16)
    assert_attn_close(host_f64(out_bf), ref, "prefill_request bf16 out")
    hidden = dev_bf16(x["hidden"])
    g = gpu.gather_last(hidden, torch.from_numpy(x["cu_seqlens"]).cuda())
    gpu.check()
    assert np.array_equal(host_bits(g), oracle.gather_last(x["hidden"], x["cu_seqlens"]))


CASES = [
    # lengths, Hq, Hkv, D
    ((1, 0, 64, 65, 127, 128, 129, 5), 16, 8, 128),     # tile edges, empty and 1-token sequences
    ((300, 1, 77), 4, 4, 128),                           # G = 1 (one head per workgroup, 128-row tiles)
    ((200, 33, 0, 500), 14, 2, 64),                      # G = 7 (odd group)
    ((96, 250), 8, 2, 64),                               # G = 4
    ((500,), 2, 1, 128),                                 # the longest sequence alone
    ((0, 0, 3), 4, 2, 64),                               # leading empty sequences
]


@pytest.mark.parametrize("lengths,Hq,Hkv,D", CASES)
def test_shapes_and_edges(gpu, lengths, Hq, Hkv, D):
    note("prefill lengths=%s Hq=%d Hkv=%d D=%d" % (lengths, Hq, Hkv, D))
    shape = wl.PrefillShape("edge", 77, tuple(lengths), Hq, Hkv, D)
    x = wl.prefill_inputs(shape)
    ref = oracle.prefill_attn(x["q"], x["k"], x["v"], x["cu_seqlens"])
    out = _run(gpu, x, Hq, Hkv, D)
    assert_attn_close(host_f64(out), ref, "edge %s" % (lengths,))
    # a max_seqlen above the real maximum launches idle tiles only
    out2 = _run(gpu, x, Hq, Hkv, D, max_seqlen=min(shape.total_tokens, max(lengths) + 70))
    assert torch.equal(out, out2)


def test_throughput_workload_sampled_rows(gpu):
    """Full 960-sequence pack (T=269,924, Hq16/Hkv8/D128) in the launch the
    bench times; sampled rows against the oracle, computed one by one, and two
    launches bitwise equal (no atomics feed any reduction)."""
    shape = wl.PREFILL_THROUGHPUT
    note("prefill prefill_throughput full size, sampled rows")
    T, dev = shape.total_tokens, "cuda"
    q = wl.torch_normal_bf16((T, 16, 128), (shape.base_seed, wl.TID_Q, 0, 0), dev)
    k = wl.torch_normal_bf16((T, 8, 128), (shape.base_seed, wl.TID_K, 0, 0), dev)
    v = wl.torch_normal_bf16((T, 8, 128), (shape.base_seed, wl.TID_V, 0, 0), dev)
    cu = shape.cu_seqlens()
    cu_d = torch.from_numpy(cu).cuda()
    out = gpu.packed_prefill_attn(q, k, v, cu_d, shape.max_seqlen)
    out2 = gpu.packed_prefill_attn(q, k, v, cu_d, shape.max_seqlen)
    gpu.check()
    assert torch.equal(out, out2)
    rng = np.random.default_rng(5)
    seqs = rng.choice(len(shape.lengths), 96, replace=False)
    toks, heads = [], []
    for b in seqs:
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for t in (s0, s1 - 1, int(rng.integers(s0, s1)), int(rng.integers(s0, s1))):
            toks.append(t)
            heads.append(int(rng.integers(0, 16)))
    toks, heads = np.array(toks, np.int64), np.array(heads, np.int32)
    ref = oracle.prefill_attn_rows(host_bits(q), host_bits(k), host_bits(v), cu, toks, heads)
    got = host_f64(out[torch.from_numpy(toks).cuda(), torch.from_numpy(heads).long().cuda()])
    assert_attn_close(got, ref, "prefill_throughput sampled")


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 8, 128), (16, 4, 64), (14, 2, 64), (12, 4, 128)])
def test_persistent_many_short_sequences(gpu, Hq, Hkv, D):
    """A pack large enough for the persistent form (at least eight 128-row work
    units per CU; 8, 8, 14 and 12 work units per sequence) made mostly of
    short sequences: single-tile items (whose next item is needed before a
    freshly claimed index is known to have landed), empty sequences and a few
    long ones.  Every row against the oracle, and two launches bitwise equal."""
    rng = np.random.default_rng(11)
    lengths = rng.integers(0, 49, 1600)
    lengths[::97] = 300
    shape = wl.PrefillShape("short_pack", 78, tuple(int(v) for v in lengths), Hq, Hkv, D)
    assert shape.total_tokens * Hq // 128 + 1 >= 8 * 256
    note("prefill persistent short pack T=%d Hq=%d Hkv=%d D=%d" % (shape.total_tokens, Hq, Hkv, D))
    x = wl.prefill_inputs(shape)
    out = _run(gpu, x, Hq, Hkv, D)
    out2 = _run(gpu, x, Hq, Hkv, D)
    assert torch.equal(out, out2)
    ref = oracle.prefill_attn(x["q"], x["k"], x["v"], x["cu_seqlens"])
    assert_attn_close(host_f64(out), ref, "short pack")


def test_bad_cu_seqlens_is_flagged(gpu):
    note("prefill bad cu_seqlens -> device error flag")
    x = wl.prefill_inputs(wl.PrefillShape("bad", 5, (10, 10, 10), 4, 2, 64))
    cu = np.array([0, 10, 5, 30], np.int32)          # decreasing: sequence 1 is invalid
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    gpu.packed_prefill_attn(q, k, v, torch.from_numpy(cu).cuda(), 25)
    with pytest.raises(Exception, match="cu_seqlens"):
        gpu.check()
    gpu.check()                                       # the flag was cleared
