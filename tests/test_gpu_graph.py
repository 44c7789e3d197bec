"""The hot path captured as one HIP graph (the fixed-step beam search as a
single replayable unit, and a packed prefill with its gather): every replay
must reproduce the eager launch sequence bit for bit.  Between replays the
program runs eager work of its own and synchronises; every replay is checked.

The kernels allocate nothing, set no memory by host calls and keep all state
(prefill work-list counters, top-k request state) in the context's workspace,
which they reset themselves, so a captured sequence can be replayed."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import dev_bf16, note

pytestmark = pytest.mark.gpu


def _snapshot(ts):
    return [t.detach().cpu().clone() for t in ts]


def _same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), "%s: output %d differs from the eager run" % (what, i)


def test_graph_replays_match_eager(gpu):
    note("graph capture: prefill pack (persistent form) + gather + 3-step beam search, 3 replays")
    dev = "cuda"
    rng = np.random.default_rng(21)
    lengths = tuple(int(x) for x in rng.integers(64, 501, 100))      # enough for the persistent form
    pf = wl.PrefillShape("graph_pack", 1021, lengths, 16, 8, 128, hidden_dim=256)
    x = wl.prefill_inputs(pf)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    hidden = dev_bf16(x["hidden"])
    cu = torch.from_numpy(x["cu_seqlens"]).to(dev)
    pout = torch.empty((pf.total_tokens, 16, 128), dtype=torch.float32, device=dev)
    gout = torch.empty((len(lengths), 256), dtype=torch.bfloat16, device=dev)

    bs = wl.BeamShape("graph_beam", 1022, num_requests=4, width=50, prompt_len=64, n_steps=3, n_heads_q=14,
                      n_heads_kv=2, head_dim=64, n_layers=2, vocab=4096)
    st = wl.beam_static_inputs(bs)
    pk, pv = dev_bf16(st["prefix_k"]), dev_bf16(st["prefix_v"])
    steps = {t: wl.beam_step_inputs(bs, t) for t in range(1, bs.n_steps + 1)}
    bq = {t: dev_bf16(s["q"]) for t, s in steps.items()}
    kn = {t: dev_bf16(s["k_new"]) for t, s in steps.items()}
    vn = {t: dev_bf16(s["v_new"]) for t, s in steps.items()}
    lps = {t: torch.from_numpy(wl.beam_logprobs(bs, t)).to(dev) for t in range(bs.n_steps + 1)}
    R, W, N = bs.num_requests, bs.width, bs.n_steps
    cum0 = torch.zeros((R, 1), dtype=torch.float32, device=dev)
    toks = [torch.empty((R, W), dtype=torch.int32, device=dev) for _ in range(N + 1)]
    pars = [torch.empty((R, W), dtype=torch.int32, device=dev) for _ in range(N + 1)]
    cums = [torch.empty((R, W), dtype=torch.float32, device=dev) for _ in range(N + 1)]
    sshape = (bs.n_layers, R, W, bs.suffix_cap, bs.n_heads_kv, bs.head_dim)
    suf = [(torch.zeros(sshape, dtype=torch.bfloat16, device=dev), torch.zeros(sshape, dtype=torch.bfloat16,
                                                                                 device=dev)) for _ in range(3)]
    bouts = [torch.empty((bs.n_layers, R, W, bs.n_heads_q, bs.head_dim), dtype=torch.float32, device=dev)
             for _ in range(N + 1)]

    def sequence():
        gpu.packed_prefill_attn(q, k, v, cu, pf.max_seqlen, out=pout)
        gpu.gather_last(hidden, cu, out=gout)
        gpu.beam_topk_merge(lps[0], cum0, W, toks[0], pars[0], cums[0])
        for t in range(1, N + 1):
            (ski, svi), (sko, svo) = suf[(t + 1) % 2], suf[t % 2]
            gpu.beam_decode_attn(bq[t], pk, pv, ski if t > 1 else None, svi if t > 1 else None, kn[t], vn[t],
                                 pars[t - 1], t - 1, sko, svo, out=bouts[t])
            gpu.beam_topk_merge(lps[t], cums[t - 1], W, toks[t], pars[t], cums[t])
        gpu.beam_reorder_suffix(pars[N], suf[N % 2][0], suf[N % 2][1], N, suf[2][0], suf[2][1])

    outs = [pout, gout] + toks + pars + cums + bouts[1:] + [suf[2][0], suf[2][1]]
    sequence()
    gpu.check()
    eager = _snapshot(outs)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sequence()                                  # warm the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        sequence()
    torch.cuda.synchronize()
    scratch = torch.empty_like(pout)
    for rep in range(3):
        for o in outs:                              # replays must rewrite every output
            o.zero_() if o.dtype != torch.int32 else o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gpu.check()
        _same(_snapshot(outs), eager, "replay %d" % rep)
        # the program's own eager work between replays
        gpu.packed_prefill_attn(q, k, v, cu, pf.max_seqlen, out=scratch)
        torch.cuda.synchronize()
        assert torch.equal(scratch.cpu(), eager[0]), "eager call between replays"
