"""GPU: packed prefill over a plan (slm_prefill_plan once, then
slm_packed_prefill_attn_planned for every layer) against the plain call, bit
for bit: in the persistent form, where runs back to back reuse one work list
and each run leaves the list's counters as it found them, and in the
small-pack form; eagerly and as graph replays.  The plain call is checked
against the oracle by the other prefill tests."""
import numpy as np
import pytest
import torch

import bounded_generation_slm_amd as slm
import workloads as wl
from parity_util import dev_bf16, note

pytestmark = pytest.mark.gpu


def _pack(Hq, Hkv, D):
    """The 1,600-sequence short pack: large enough for the persistent form."""
    rng = np.random.default_rng(11)
    lengths = rng.integers(0, 49, 1600)
    lengths[::97] = 300
    shape = wl.PrefillShape("short_pack", 78, tuple(int(v) for v in lengths), Hq, Hkv, D)
    assert shape.total_tokens * Hq // 128 + 1 >= 8 * 256
    x = wl.prefill_inputs(shape)
    cu = x["cu_seqlens"]
    return (dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), torch.from_numpy(cu).cuda(),
            int(np.diff(cu).max()), shape.total_tokens)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv,D", [(16, 8, 128), (14, 2, 64)])
def test_planned_runs_equal_the_plain_call(gpu, Hq, Hkv, D, out_dtype):
    q, k, v, cu, ms, T = _pack(Hq, Hkv, D)
    note("prefill plan: persistent pack T=%d Hq=%d Hkv=%d D=%d out=%s, 5 runs over one plan" % (
        T, Hq, Hkv, D, out_dtype))
    ref = gpu.packed_prefill_attn(q, k, v, cu, ms, out_dtype=out_dtype)
    plan = gpu.prefill_plan(cu, ms, T, Hq, Hkv, D)
    out = torch.empty_like(ref)
    for i in range(5):
        out.fill_(float("nan"))                     # every run must write every element
        if i == 2:
            torch.cuda.synchronize()
            (out * 2).sum()                         # other work on the stream between runs
        gpu.packed_prefill_attn_planned(plan, q, k, v, cu, ms, out=out)
        assert torch.equal(_bits(out), _bits(ref)), "planned run %d differs from the plain call" % i
    gpu.check()


def test_small_pack_planned(gpu):
    """One prefill request (15 sequences): the form without a work list."""
    shape = wl.PREFILL_REQUEST
    note("prefill plan: small pack %s" % shape.name)
    x = wl.prefill_inputs(shape)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    cu = torch.from_numpy(x["cu_seqlens"]).cuda()
    ms = int(np.diff(x["cu_seqlens"]).max())
    ref = gpu.packed_prefill_attn(q, k, v, cu, ms)
    plan = gpu.prefill_plan(cu, ms, shape.total_tokens, shape.n_heads_q, shape.n_heads_kv, shape.head_dim)
    for _ in range(2):
        out = gpu.packed_prefill_attn_planned(plan, q, k, v, cu, ms)
        assert torch.equal(_bits(out), _bits(ref))
    gpu.check()


def test_replaced_plan_is_refused_and_replanning_works(gpu):
    q, k, v, cu, ms, T = _pack(16, 8, 128)
    note("prefill plan: a plain call on another pack replaces the plan")
    ref = gpu.packed_prefill_attn(q, k, v, cu, ms)
    plan = gpu.prefill_plan(cu, ms, T, 16, 8, 128)
    x = wl.prefill_inputs(wl.PREFILL_REQUEST)
    cu2 = torch.from_numpy(x["cu_seqlens"]).cuda()
    gpu.packed_prefill_attn(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), cu2,
                            int(np.diff(x["cu_seqlens"]).max()))
    with pytest.raises(RuntimeError, match="plan"):
        gpu.packed_prefill_attn_planned(plan, q, k, v, cu, ms)
    plan = gpu.prefill_plan(cu, ms, T, 16, 8, 128)
    out = gpu.packed_prefill_attn_planned(plan, q, k, v, cu, ms)
    assert torch.equal(_bits(out), _bits(ref))
    gpu.check()


@pytest.mark.parametrize("with_plan", [False, True], ids=["runs", "plan+runs"])
def test_planned_runs_in_a_graph(gpu, with_plan):
    """Two runs (and, in the second form, the plan before them) captured once
    and replayed three times, with eager runs over the same plan between the
    replays: every output bitwise equal to the plain call's."""
    q, k, v, cu, ms, T = _pack(16, 8, 128)
    note("prefill plan: graph of %s, 3 replays" % ("plan + 2 runs" if with_plan else "2 runs"))
    ref = gpu.packed_prefill_attn(q, k, v, cu, ms)
    outs = [torch.empty_like(ref), torch.empty_like(ref)]

    def body(plan):
        if with_plan:
            plan = gpu.prefill_plan(cu, ms, T, 16, 8, 128)
        for o in outs:
            gpu.packed_prefill_attn_planned(plan, q, k, v, cu, ms, out=o)
        return plan

    plan = gpu.prefill_plan(cu, ms, T, 16, 8, 128)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan = body(plan)                           # warm-up (first launches of each kind) off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan = body(plan)
    torch.cuda.synchronize()
    eager = torch.empty_like(ref)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gpu.check()
        for i, o in enumerate(outs):
            assert torch.equal(_bits(o), _bits(ref)), "replay %d, run %d" % (rep, i)
        eager.fill_(float("nan"))
        gpu.packed_prefill_attn_planned(plan, q, k, v, cu, ms, out=eager)
        torch.cuda.synchronize()
        assert torch.equal(_bits(eager), _bits(ref)), "eager run after replay %d" % rep
    gpu.check()
    del g
