"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times, against the oracle on the same device-drawn inputs copied to the
host:

* the 960-sequence prefill pack (T = 269,924, Hq16/Hkv8/D128): the whole
  output tensor of layer 0 within tolerance, and all 28 layer launches (one
  Q/K/V set), both as plain calls and as runs over one plan (as the bench
  runs them), bitwise equal;
* the two fixed-step beam searches (32 requests x 100 beams, prompt 128, 4
  steps; 8 requests x 400 beams, prompt 480, 5 steps; 24 layers, vocabulary
  151,936) end to end through the one-call driver: every merge's tokens,
  parents and scores bit-exact (the later merges run on the clustered
  cumulative scores of the search itself), every layer of every step's
  attention within tolerance, the suffix K and V rows (history and new row)
  bit-exact after every step, the final suffix and the backtracked sequences
  bit-exact.  The short-prompt search is also captured as one graph and its
  replays are checked against the same oracle results."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import assert_attn_close, assert_attn_close_chunked, host_bits, host_f64, note

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_prefill_throughput_whole_tensor_and_layer_launches(gpu):
    shape = wl.PREFILL_THROUGHPUT
    T, Hq, Hkv, D = shape.total_tokens, shape.n_heads_q, shape.n_heads_kv, shape.head_dim
    note("prefill %s: 28 plain + 28 planned launches bitwise, whole layer-0 tensor vs the oracle (T=%d)" % (shape.name, T))
    q = wl.torch_normal_bf16((T, Hq, D), (shape.base_seed, wl.TID_Q, 0, 0), "cuda")
    k = wl.torch_normal_bf16((T, Hkv, D), (shape.base_seed, wl.TID_K, 0, 0), "cuda")
    v = wl.torch_normal_bf16((T, Hkv, D), (shape.base_seed, wl.TID_V, 0, 0), "cuda")
    cu = shape.cu_seqlens()
    cu_d = torch.from_numpy(cu).cuda()
    out0 = gpu.packed_prefill_attn(q, k, v, cu_d, shape.max_seqlen)
    out = torch.empty_like(out0)
    for layer in range(1, shape.n_layers):
        out.fill_(float("nan"))                 # every launch must rewrite every element
        gpu.packed_prefill_attn(q, k, v, cu_d, shape.max_seqlen, out=out)
        assert torch.equal(out.view(torch.int32), out0.view(torch.int32)), "launch %d differs from launch 0" % layer
    plan = gpu.prefill_plan(cu_d, shape.max_seqlen, T, Hq, Hkv, D)
    for layer in range(shape.n_layers):
        out.fill_(float("nan"))
        gpu.packed_prefill_attn_planned(plan, q, k, v, cu_d, shape.max_seqlen, out=out)
        assert torch.equal(out.view(torch.int32), out0.view(torch.int32)), "planned launch %d differs" % layer
    gpu.check()
    del out
    ref = oracle.prefill_attn(host_bits(q), host_bits(k), host_bits(v), cu)
    rel, mab = assert_attn_close_chunked(out0, ref, "%s layer 0, whole tensor" % shape.name)
    note("prefill whole tensor rel_l2 %.3g max_abs %.3g" % (rel, mab))


def _state(ctx, shape, n_steps, attn_per_step):
    return ctx.beam_search_state(shape.n_layers, shape.num_requests, shape.width, n_steps, shape.n_heads_q,
                                 shape.n_heads_kv, shape.head_dim, suffix_cap=shape.suffix_cap,
                                 attn_per_step=attn_per_step)


def _run(ctx, st, x, n_steps):
    ctx.beam_search(st, x["prefix_k"], x["prefix_v"], x["logprobs"][:n_steps + 1], x["q"][:n_steps],
                    x["k_new"][:n_steps], x["v_new"][:n_steps])


def _captured(ctx, shape, x):
    """The whole search captured once as a graph (after an eager warm-up on
    a side stream) and its state, replayed by the caller."""
    st = _state(ctx, shape, shape.n_steps, True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(ctx, st, x, shape.n_steps)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run(ctx, st, x, shape.n_steps)
    torch.cuda.synchronize()
    return g, st


def _clear(st):
    for key in ("tokens", "parent", "sequences"):
        st[key].fill_(-7)
    st["cum"].zero_()
    for t in st["attn_out"]:
        t.fill_(float("nan"))
    for key in ("final_k", "final_v"):
        st[key].zero_()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("shape", [wl.BEAM_SHORT, wl.BEAM_LONG], ids=lambda s: s.name)
def test_beam_search_end_to_end(gpu, shape):
    NL, R, W, N = shape.n_layers, shape.num_requests, shape.width, shape.n_steps
    graph = shape is wl.BEAM_SHORT
    note("beam search %s end to end vs the oracle%s" % (shape.name, " (eager and graph replays)" if graph else ""))
    x = wl.torch_beam_inputs(shape, "cuda")
    runs = {}
    st = _state(gpu, shape, N, True)
    _run(gpu, st, x, N)
    gpu.check()
    runs["eager"] = st
    if graph:
        g, sg = _captured(gpu, shape, x)
        for rep in range(2):
            _clear(sg)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            gpu.check()
            runs["replay %d" % rep] = {k: (v.clone() if isinstance(v, torch.Tensor) else
                                           [t.clone() for t in v] if isinstance(v, list) else v)
                                       for k, v in sg.items()}
        del g, sg
    # the suffix after step t: the same search stopped after t steps (the
    # driver alternates two suffix buffers, so a full run keeps the last two)
    suffix = {}
    for t in range(1, N + 1):
        s_t = _state(gpu, shape, t, False)
        _run(gpu, s_t, x, t)
        suffix[t] = (s_t["suffix_k"][t % 2].clone(), s_t["suffix_v"][t % 2].clone())
        assert torch.equal(s_t["tokens"], st["tokens"][:t + 1]) and torch.equal(s_t["cum"], st["cum"][:t + 1])
        del s_t
    gpu.check()

    pk, pv = host_bits(x["prefix_k"]), host_bits(x["prefix_v"])

    def step_inputs(t):
        return dict(q=host_bits(x["q"][t - 1]), k_new=host_bits(x["k_new"][t - 1]), v_new=host_bits(x["v_new"][t - 1]))

    def on_step(t, ref):
        worst = 0.0
        for name, run in runs.items():
            out = run["attn_out"][t - 1]
            for l in range(NL):
                rel, _ = assert_attn_close(host_f64(out[l]), ref["attn"][l], "%s %s step %d layer %d" % (
                    shape.name, name, t, l))
                worst = max(worst, rel)
        sk, sv = suffix[t]
        assert np.array_equal(host_bits(sk)[:, :, :, :t], ref["suffix_k"][:, :, :, :t]), "suffix K after step %d" % t
        assert np.array_equal(host_bits(sv)[:, :, :, :t], ref["suffix_v"][:, :, :, :t]), "suffix V after step %d" % t
        note("%s step %d: attention worst rel_l2 %.3g over %d layers; suffix K/V bit-exact" % (shape.name, t, worst, NL))

    ref = oracle.beam_search(step_inputs, pk, pv, lambda t: x["logprobs"][t].cpu().numpy(), W, N,
                             suffix_cap=shape.suffix_cap, on_step=on_step)
    for name, run in runs.items():
        for t in range(N + 1):
            for key in ("tokens", "parent", "cum"):
                got = run[key][t].cpu().numpy()
                assert np.array_equal(got, ref[key][t]), "%s %s: merge %d %s differ at %s" % (
                    shape.name, name, t, key, np.argwhere(got != ref[key][t])[:5].tolist())
        assert np.array_equal(host_bits(run["final_k"]), ref["final_suffix_k"]), name + ": final suffix K"
        assert np.array_equal(host_bits(run["final_v"]), ref["final_suffix_v"]), name + ": final suffix V"
        assert np.array_equal(run["sequences"].cpu().numpy(), ref["sequences"]), name + ": sequences"
