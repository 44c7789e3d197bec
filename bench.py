"""Benchmark of the bounded-generation attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
resident in HBM:
  * prefill-only batch: 64 requests x 15 samples = 960 packed sequences
    (lengths uniform on [64,500], T = 269,924 tokens), 28 layer calls of
    packed causal GQA attention (16 query / 8 KV heads, head_dim 128, fp32
    out) over one seeded Q/K/V set, then the last-valid-token gather of a
    [T,1024] bf16 hidden state;
  * short-prompt beam search: 32 requests x 100 beams, prompt 128, 4 fixed
    decode steps over 24 layers (14 query / 2 KV heads, head_dim 64), vocab
    151,936: first merge (one beam in), then per step the 24-layer decode
    attention (history read through the last parents, suffix written in the
    new order) and the top-k merge; finally the suffix reorder by the last
    parents.

value = prefill tokens per step (T, each through all 28 layers) / step time.
The JSON line also carries the per-part times, the roofline of the dominant
kernel (packed prefill attention) and the oracle timed on a bounded sample.
Outside the timed step, the same calls are timed on two more workloads for
reporting only: one prefill-only request (15 packed samples, one layer, then
the gather) and the long-prompt wide beam search (8 requests x 400 beams,
prompt 480, 5 steps).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed-prefill attn tokens/s & beam-step µs; % of MFMA peak / HBM peak"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the timed oracle sample")
    ap.add_argument("--no-graph", action="store_true", help="skip the captured-graph timing of the step")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the reporting-only prefill-request and long-prompt beam timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration) and exit")
    return ap.parse_args()


def src_sha(name: str) -> str:
    with open(os.path.join(ROOT, "bounded_generation_slm_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def prefill_bytes_flops(lengths, Hq, Hkv, D, out_bytes):
    """Algorithmic bytes (q, k, v read once, out written once) and causal flops."""
    T = sum(lengths)
    byts = T * (Hq * D * 2 + 2 * Hkv * D * 2 + Hq * D * out_bytes)
    flops = 2 * Hq * D * sum(L * (L + 1) for L in lengths)    # QK^T and PV over causal pairs
    return byts, flops


def decode_bytes(s, t):
    """Algorithmic bytes of the 24-layer decode attention at step t (s = t rows)."""
    NL, R, W, P, Hq, Hkv, D = s.n_layers, s.num_requests, s.width, s.prompt_len, s.n_heads_q, s.n_heads_kv, s.head_dim
    q = NL * R * W * Hq * D * 2
    prompt = NL * R * P * Hkv * D * 2 * 2
    suffix = 2 * NL * R * W * t * Hkv * D * 2 * 2          # read t rows (history + new), write t rows
    out = NL * R * W * Hq * D * 4
    return q + prompt + suffix + out


def topk_bytes(R, Win, V, W):
    return R * Win * V * 4 + R * Win * 4 + R * W * 12


def one_thread_times():
    """The oracle with one OpenMP thread on the tiny config's prefill and merge
    and the one-request prefill (15 sequences), in a child process (the thread
    count of a running OpenMP runtime cannot be changed from here)."""
    import subprocess
    code = (
        "import time, numpy as np, oracle, workloads as wl\n"
        "res = {}\n"
        "for name, shp in (('tiny_prefill', wl.TINY_PREFILL), ('prefill_request', wl.PREFILL_REQUEST)):\n"
        "    x = wl.prefill_inputs(shp); t0 = time.perf_counter()\n"
        "    oracle.prefill_attn(x['q'], x['k'], x['v'], x['cu_seqlens']); res[name] = time.perf_counter() - t0\n"
        "s = wl.TINY_BEAM; lp = wl.beam_logprobs(s, 1); t0 = time.perf_counter()\n"
        "oracle.topk_merge(lp, np.zeros((s.num_requests, s.width), np.float32), s.width)\n"
        "res['tiny_merge'] = time.perf_counter() - t0\n"
        "print(repr({k: round(v, 4) for k, v in res.items()}))\n")
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                             timeout=120)
        import ast
        return ast.literal_eval(out.stdout.strip().splitlines()[-1])
    except Exception as e:                                      # reporting only
        return {"error": str(e)[:200]}


def cpu_baseline(pf, bs):
    """The oracle on a bounded sample of the same workload (roughly 10 s on 16
    host threads), scaled to the whole step: one whole prefill layer (all 960
    sequences), one layer of each decode step, and 8 requests of each merge."""
    import numpy as np

    import oracle
    import workloads as wl

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    L = list(pf.lengths)
    sub = L
    shp = wl.PrefillShape("sample", pf.base_seed, tuple(sub), pf.n_heads_q, pf.n_heads_kv, pf.head_dim)
    x = wl.prefill_inputs(shp)
    t0 = time.perf_counter()
    oracle.prefill_attn(x["q"], x["k"], x["v"], x["cu_seqlens"])
    t_pre = time.perf_counter() - t0
    pairs = lambda ls: sum(l * (l + 1) for l in ls)
    est = t_pre * pairs(L) / pairs(sub) * pf.n_layers

    st = wl.beam_static_inputs(bs, layers=[0])
    hist_rng = np.random.default_rng(0)
    t_dec = 0.0
    for t in range(1, bs.n_steps + 1):
        xs = wl.beam_step_inputs(bs, t, layers=[0])
        shp6 = (1, bs.num_requests, bs.width, bs.suffix_cap, bs.n_heads_kv, bs.head_dim)
        sk = wl.f32_to_bf16_bits(hist_rng.standard_normal(shp6).astype(np.float32))
        par = hist_rng.integers(0, bs.width, size=(bs.num_requests, bs.width)).astype(np.int32)
        t0 = time.perf_counter()
        oracle.beam_decode_attn(xs["q"], st["prefix_k"], st["prefix_v"], sk, sk, xs["k_new"], xs["v_new"], par, t - 1)
        t_dec += time.perf_counter() - t0
    est += t_dec * bs.n_layers

    r_s = 8
    t_top = 0.0
    for t in range(0, bs.n_steps + 1):
        win = 1 if t == 0 else bs.width
        lp = wl.logprobs(bs.base_seed, (r_s, win, bs.vocab), t)
        cum = np.zeros((r_s, win), np.float32)
        t0 = time.perf_counter()
        oracle.topk_merge(lp, cum, bs.width)
        t_top += time.perf_counter() - t0
    est += t_top * bs.num_requests / r_s
    sampled = t_pre + t_dec + t_top
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": pf.total_tokens / est,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "host": {"cpu_model": cpu_model, "logical_cpus": os.cpu_count(), "omp_threads": threads,
                 "one_thread_s": one_thread_times()},
        "sample": ("fp64 C oracle, %d threads: prefill layer 0 over %d of 960 sequences (%d tokens), "
                   "decode layer 0 of each of the 4 steps, top-k merge of 8 of 32 requests for the 5 merges; "
                   "%.1f s measured, scaled by causal pairs / layers / requests to one whole step "
                   "(%.0f s estimated)" % (threads, len(sub), sum(sub), sampled, est)),
    }


def traffic_from_counters(kernel_file: str, launch_bytes_key: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source."""
    path = os.path.join(PROFILES, "prefill_attn_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != src_sha(kernel_file):
        return None
    return rec.get(launch_bytes_key)


def extra_workloads(ctx, dev, ev, reps=5):
    """Reporting-only timings outside the timed step (not part of value)."""
    import torch
    import workloads as wl
    res = {}
    # one prefill-only request: 15 packed samples, one layer, then the gather
    pr = wl.PREFILL_REQUEST
    T, Hq, Hkv, D = pr.total_tokens, pr.n_heads_q, pr.n_heads_kv, pr.head_dim
    q = wl.torch_normal_bf16((T, Hq, D), (pr.base_seed, wl.TID_Q, 0, 0), dev)
    k = wl.torch_normal_bf16((T, Hkv, D), (pr.base_seed, wl.TID_K, 0, 0), dev)
    v = wl.torch_normal_bf16((T, Hkv, D), (pr.base_seed, wl.TID_V, 0, 0), dev)
    hidden = wl.torch_normal_bf16((T, pr.hidden_dim), (pr.base_seed, wl.TID_HIDDEN, 0, 0), dev)
    cu = torch.from_numpy(pr.cu_seqlens()).to(dev)
    out = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    g = torch.empty((len(pr.lengths), pr.hidden_dim), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        ctx.packed_prefill_attn(q, k, v, cu, pr.max_seqlen, out=out)
        ctx.gather_last(hidden, cu, out=g)
    times = []
    for _ in range(reps * 4):
        e0 = ev()
        ctx.packed_prefill_attn(q, k, v, cu, pr.max_seqlen, out=out)
        ctx.gather_last(hidden, cu, out=g)
        times.append((e0, ev()))
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in times)[len(times) // 2]
    pbytes, pflops = prefill_bytes_flops(pr.lengths, Hq, Hkv, D, 4)
    res["prefill_request"] = {
        "workload": "15 packed samples U[64,500] (T=%d), Hq16/Hkv8/D128, fp32 out, 1 layer + gather [T,1024]" % T,
        "us_per_request_median": round(us, 1), "tokens_per_s": round(T / (us * 1e-6), 1),
        "hbm_frac": round(pbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(pflops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    # the prefill-only label head after the gather: 64 label rows of a synthetic
    # 151,936-row LM head, top 5, on this request and on the 960-sequence pack
    V = 151936
    g_lm = torch.Generator(device=dev)
    g_lm.manual_seed(29)
    lm = (torch.randn((V, pr.hidden_dim), generator=g_lm, device=dev) * pr.hidden_dim ** -0.5).to(torch.bfloat16)
    labels = torch.from_numpy(wl.label_ids(pr.base_seed, V)).to(dev)
    pf = wl.PREFILL_THROUGHPUT
    hid_pf = wl.torch_normal_bf16((pf.total_tokens, pf.hidden_dim), (pf.base_seed, wl.TID_HIDDEN, 0, 0), dev)
    cu_pf = torch.from_numpy(pf.cu_seqlens()).to(dev)
    for name, hh, cc, nseq in (("label_head_prefill_request", hidden, cu, len(pr.lengths)),
                               ("label_head_prefill_throughput", hid_pf, cu_pf, len(pf.lengths))):
        for _ in range(3):
            ctx.label_head(hh, cc, lm, labels, wl.LABEL_TOP_K)
        times = []
        for _ in range(reps * 4):
            e0 = ev()
            ctx.label_head(hh, cc, lm, labels, wl.LABEL_TOP_K)
            times.append((e0, ev()))
        torch.cuda.synchronize()
        ctx.check()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in times)[len(times) // 2]
        res[name] = {"workload": "%d sequences, hidden %d, %d labels of a %d-row LM head, top %d" % (
            nseq, pr.hidden_dim, wl.LABEL_COUNT, V, wl.LABEL_TOP_K), "us_median": round(us, 1),
            "sequences_per_s": round(nseq / (us * 1e-6), 1)}
    del lm, hid_pf
    del q, k, v, hidden, out
    # the long-prompt wide beam search
    bl = BeamRun(wl.BEAM_LONG, dev)
    bl.run(ctx, [], ev)
    marks = []
    for _ in range(reps):
        bl.run(ctx, marks, ev)
    torch.cuda.synchronize()
    per = {}
    for name, a, b in marks:
        per.setdefault(name, []).append(a.elapsed_time(b) * 1e3)
    res["beam_long_prompt"] = dict(
        {"workload": "R8 x W400, P480, 5 steps, 24 layers, Hq14/Hkv2/D64, V151936"}, **bl.summary(per))
    del bl
    torch.cuda.empty_cache()
    # beam-search prompt prefill: R equal-length prompts packed, K/V kept in
    # the layout decode reads ([R*P, Hkv, D] per layer is [R, P, Hkv, D])
    for bs in (wl.BEAM_SHORT, wl.BEAM_LONG):
        R, P, Hq, Hkv, D, NL = bs.num_requests, bs.prompt_len, bs.n_heads_q, bs.n_heads_kv, bs.head_dim, bs.n_layers
        q = wl.torch_normal_bf16((R * P, Hq, D), (bs.base_seed, wl.TID_Q, 0, 0), dev)
        k = wl.torch_normal_bf16((R * P, Hkv, D), (bs.base_seed, wl.TID_PREFIX_K, 0, 0), dev)
        v = wl.torch_normal_bf16((R * P, Hkv, D), (bs.base_seed, wl.TID_PREFIX_V, 0, 0), dev)
        cu = torch.arange(R + 1, dtype=torch.int32, device=dev) * P
        out = torch.empty((R * P, Hq, D), dtype=torch.float32, device=dev)
        for _ in range(3):
            ctx.packed_prefill_attn(q, k, v, cu, P, out=out)
        times = []
        for _ in range(reps * 4):
            e0 = ev()
            ctx.packed_prefill_attn(q, k, v, cu, P, out=out)
            times.append((e0, ev()))
        torch.cuda.synchronize()
        ctx.check()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in times)[len(times) // 2]
        pbytes, pflops = prefill_bytes_flops([P] * R, Hq, Hkv, D, 4)
        res["prompt_prefill_" + bs.name] = {
            "workload": "%d prompts x %d tokens packed, Hq%d/Hkv%d/D%d, fp32 out; K/V in decode's layout" % (
                R, P, Hq, Hkv, D),
            "us_per_layer_median": round(us, 1), "us_all_%d_layers" % NL: round(us * NL, 1),
            "hbm_frac": round(pbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del q, k, v, out
    # decode (first step) with prompts of different lengths packed with
    # offsets, as a packed prompt prefill leaves them: the short-prompt beam
    # shape with lengths U[64, 192] (mean 128)
    import numpy as np
    bs = wl.BEAM_SHORT
    NL, R, W, Hq, Hkv, D = bs.n_layers, bs.num_requests, bs.width, bs.n_heads_q, bs.n_heads_kv, bs.head_dim
    lengths = np.random.default_rng(bs.base_seed + 77).integers(64, 193, size=R)
    cu_np = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    Tp = int(cu_np[-1])
    cu = torch.from_numpy(cu_np).to(dev)
    q = wl.torch_normal_bf16((NL, R, W, Hq, D), (bs.base_seed, wl.TID_Q, 0, 7), dev)
    pk = wl.torch_normal_bf16((NL, Tp, Hkv, D), (bs.base_seed, wl.TID_PREFIX_K, 0, 7), dev)
    pv = wl.torch_normal_bf16((NL, Tp, Hkv, D), (bs.base_seed, wl.TID_PREFIX_V, 0, 7), dev)
    kn = wl.torch_normal_bf16((NL, R, W, Hkv, D), (bs.base_seed, wl.TID_K_NEW, 0, 7), dev)
    vn = wl.torch_normal_bf16((NL, R, W, Hkv, D), (bs.base_seed, wl.TID_V_NEW, 0, 7), dev)
    sko = torch.empty((NL, R, W, bs.suffix_cap, Hkv, D), dtype=torch.bfloat16, device=dev)
    svo = torch.empty_like(sko)
    out = torch.empty((NL, R, W, Hq, D), dtype=torch.float32, device=dev)
    call = lambda: ctx.beam_decode_attn(q, pk, pv, None, None, kn, vn, None, 0, sko, svo, out=out, prompt_cu=cu,
                                        prompt_len=int(lengths.max()))
    for _ in range(3):
        call()
    times = []
    for _ in range(reps * 4):
        e0 = ev()
        call()
        times.append((e0, ev()))
    torch.cuda.synchronize()
    ctx.check()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in times)[len(times) // 2]
    nbytes = (NL * R * W * Hq * D * 2 + NL * Tp * Hkv * D * 2 * 2 + 2 * NL * R * W * Hkv * D * 2 * 2
              + NL * R * W * Hq * D * 4)
    res["decode_ragged_prompts_" + bs.name] = {
        "workload": "R%d x W%d, prompt lengths U[64,192] packed with offsets (%d rows), first step, %d layers, "
                    "Hq%d/Hkv%d/D%d, fp32 out" % (R, W, Tp, NL, Hq, Hkv, D),
        "us_median": round(us, 1), "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del q, pk, pv, kn, vn, sko, svo, out
    # the merge on logits (log-softmax folded in) at both beam shapes
    for bs in (wl.BEAM_SHORT, wl.BEAM_LONG):
        R, W, V = bs.num_requests, bs.width, bs.vocab
        x = wl.torch_logits((R, W, V), (bs.base_seed, wl.TID_LOGITS, 0, 2), dev)
        gc = torch.Generator(device=dev)
        gc.manual_seed(17)
        cum = torch.randn((R, W), generator=gc, device=dev) * 3 - 10
        outs = [torch.empty((R, W), dtype=torch.int32, device=dev), torch.empty((R, W), dtype=torch.int32, device=dev),
                torch.empty((R, W), dtype=torch.float32, device=dev)]
        for xx, tag, eb in ((x, "", 4), (x.to(torch.bfloat16), "_bf16", 2)):
            for _ in range(3):
                ctx.beam_topk_merge_logits(xx, cum, W, *outs)
            times = []
            for _ in range(reps * 4):
                e0 = ev()
                ctx.beam_topk_merge_logits(xx, cum, W, *outs)
                times.append((e0, ev()))
            torch.cuda.synchronize()
            ctx.check()
            us = sorted(a.elapsed_time(b) * 1e3 for a, b in times)[len(times) // 2]
            nbytes = R * W * V * eb + R * W * 4 + 3 * R * W * 4
            res["merge_on_logits_" + bs.name + tag] = {
                "workload": "R%d x Win%d x V%d %s logits -> top %d (row log-sum-exp folded in)" % (
                    R, W, V, "bf16" if eb == 2 else "fp32", W),
                "us_median": round(us, 1), "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "bytes": nbytes}
            del xx
        del x
    torch.cuda.empty_cache()
    return {"reporting_only": res}


class BeamRun:
    """Device-resident inputs of one fixed-step beam search and its launch
    sequence: first merge (one beam in), then per step the all-layer decode
    attention (history read through the last parents, suffix written in the
    new order) and the merge, finally the suffix reorder by the last parents."""

    def __init__(self, bs, dev):
        import torch
        import workloads as wl
        self.bs = bs
        NL, R, W, P, N, V = bs.n_layers, bs.num_requests, bs.width, bs.prompt_len, bs.n_steps, bs.vocab
        Hq, Hkv, D = bs.n_heads_q, bs.n_heads_kv, bs.head_dim
        self.pk = wl.torch_normal_bf16((NL, R, P, Hkv, D), (bs.base_seed, wl.TID_PREFIX_K, 0, 0), dev)
        self.pv = wl.torch_normal_bf16((NL, R, P, Hkv, D), (bs.base_seed, wl.TID_PREFIX_V, 0, 0), dev)
        steps = range(1, N + 1)
        self.q = [None] + [wl.torch_normal_bf16((NL, R, W, Hq, D), (bs.base_seed, wl.TID_Q, 0, t), dev) for t in steps]
        self.kn = [None] + [wl.torch_normal_bf16((NL, R, W, Hkv, D), (bs.base_seed, wl.TID_K_NEW, 0, t), dev)
                            for t in steps]
        self.vn = [None] + [wl.torch_normal_bf16((NL, R, W, Hkv, D), (bs.base_seed, wl.TID_V_NEW, 0, t), dev)
                            for t in steps]
        self.lps = [wl.torch_logprobs((R, 1 if t == 0 else W, V), (bs.base_seed, wl.TID_LOGITS, 0, t), dev)
                    for t in range(N + 1)]
        self.cum0 = torch.zeros((R, 1), dtype=torch.float32, device=dev)
        self.toks = [torch.empty((R, W), dtype=torch.int32, device=dev) for _ in range(N + 1)]
        self.pars = [torch.empty((R, W), dtype=torch.int32, device=dev) for _ in range(N + 1)]
        self.cums = [torch.empty((R, W), dtype=torch.float32, device=dev) for _ in range(N + 1)]
        sshape = (NL, R, W, bs.suffix_cap, Hkv, D)
        self.suf = [(torch.zeros(sshape, dtype=torch.bfloat16, device=dev),
                     torch.zeros(sshape, dtype=torch.bfloat16, device=dev)) for _ in range(3)]
        self.out = torch.empty((NL, R, W, Hq, D), dtype=torch.float32, device=dev)

    def run(self, ctx, marks, ev):
        bs, N, W = self.bs, self.bs.n_steps, self.bs.width
        e0 = ev()
        ctx.beam_topk_merge(self.lps[0], self.cum0, W, self.toks[0], self.pars[0], self.cums[0])
        marks.append(("merge0", e0, ev()))
        for t in range(1, N + 1):
            (ski, svi), (sko, svo) = self.suf[(t + 1) % 2], self.suf[t % 2]
            e0 = ev()
            ctx.beam_decode_attn(self.q[t], self.pk, self.pv, ski if t > 1 else None, svi if t > 1 else None,
                                 self.kn[t], self.vn[t], self.pars[t - 1], t - 1, sko, svo, out=self.out)
            e1 = ev()
            ctx.beam_topk_merge(self.lps[t], self.cums[t - 1], W, self.toks[t], self.pars[t], self.cums[t])
            e2 = ev()
            marks.append(("decode%d" % t, e0, e1))
            marks.append(("merge%d" % t, e1, e2))
        e0 = ev()
        ctx.beam_reorder_suffix(self.pars[N], self.suf[N % 2][0], self.suf[N % 2][1], N, self.suf[2][0],
                                self.suf[2][1])
        marks.append(("reorder", e0, ev()))

    def summary(self, per):
        """Per-part averages (us) and the beam-step HBM fraction."""
        bs = self.bs
        N, R, W, V = bs.n_steps, bs.num_requests, bs.width, bs.vocab
        avg = {k: sum(v) / len(v) for k, v in per.items()}
        parts = ["merge0"] + ["decode%d" % t for t in range(1, N + 1)] + ["merge%d" % t for t in range(1, N + 1)] \
            + ["reorder"]
        search_us = sum(avg[p] for p in parts)
        step_us = [avg["decode%d" % t] + avg["merge%d" % t] for t in range(1, N + 1)]
        step_bytes = [decode_bytes(bs, t) + topk_bytes(R, W, V, W) for t in range(1, N + 1)]
        return {
            "beam_search_us": round(search_us, 1),
            "beam_step_us": [round(u, 1) for u in step_us],
            "beam_step_us_mean": round(sum(step_us) / N, 1),
            "beam_step_hbm_frac": [round(b / (u * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) for b, u in zip(step_bytes, step_us)],
            "decode_us": [round(avg["decode%d" % t], 1) for t in range(1, N + 1)],
            "decode_hbm_frac": [round(decode_bytes(bs, t) / (avg["decode%d" % t] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                for t in range(1, N + 1)],
            "merge_us": [round(avg["merge%d" % t], 1) for t in range(0, N + 1)],
            "merge_hbm_frac": [round(topk_bytes(R, W, V, W) / (avg["merge%d" % t] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                               for t in range(1, N + 1)],
            "reorder_us": round(avg["reorder"], 1),
            "beam_requests_per_s": round(R / (search_us * 1e-6), 1),
            "beams_steps_per_s": round(R * W * N / (sum(step_us) * 1e-6), 1),
        }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the path shards by sequence / request "
              "with no exchange); --gpus %d is not run" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import bounded_generation_slm_amd as slm
    import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 28                                  # 1 GiB of fp32
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}))
        return

    ctx = slm.Context(0)
    pf, bs = wl.PREFILL_THROUGHPUT, wl.BEAM_SHORT

    # ---- inputs, resident in HBM before timing ----
    T, Hq, Hkv, D = pf.total_tokens, pf.n_heads_q, pf.n_heads_kv, pf.head_dim
    q = wl.torch_normal_bf16((T, Hq, D), (pf.base_seed, wl.TID_Q, 0, 0), dev)
    k = wl.torch_normal_bf16((T, Hkv, D), (pf.base_seed, wl.TID_K, 0, 0), dev)
    v = wl.torch_normal_bf16((T, Hkv, D), (pf.base_seed, wl.TID_V, 0, 0), dev)
    hidden = wl.torch_normal_bf16((T, pf.hidden_dim), (pf.base_seed, wl.TID_HIDDEN, 0, 0), dev)
    cu = torch.from_numpy(pf.cu_seqlens()).to(dev)
    pout = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    gout = torch.empty((len(pf.lengths), pf.hidden_dim), dtype=torch.bfloat16, device=dev)

    beam = BeamRun(bs, dev)
    torch.cuda.synchronize()

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def step(marks):
        """One pass of the whole hot path; marks collects (part, start, end) events."""
        for _ in range(pf.n_layers):
            e0 = ev()
            ctx.packed_prefill_attn(q, k, v, cu, pf.max_seqlen, out=pout)
            marks.append(("prefill", e0, ev()))
        e0 = ev()
        ctx.gather_last(hidden, cu, out=gout)
        marks.append(("gather", e0, ev()))
        beam.run(ctx, marks, ev)

    for _ in range(args.warmup):
        step([])
    ctx.check()
    torch.cuda.synchronize()

    marks = []
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step(marks)
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ctx.check()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps

    # the same step captured as one HIP graph (no per-launch host work)
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step([])
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step([])
        for _ in range(max(1, args.warmup)):
            g.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        ctx.check()
        graph_ms = g0.elapsed_time(g1) / args.steps

    per = {}
    for name, a, b in marks:
        per.setdefault(name, []).append(a.elapsed_time(b) * 1e3)   # us
    prefill_us = sum(per["prefill"]) / len(per["prefill"])
    gather_us = sum(per["gather"]) / len(per["gather"])

    pbytes, pflops = prefill_bytes_flops(pf.lengths, Hq, Hkv, D, 4)
    achieved_gbs = pbytes / (prefill_us * 1e-6) / 1e9
    mfma_tflops = pflops / (prefill_us * 1e-6) / 1e12
    traffic = traffic_from_counters("prefill_attn.hip", "hbm_bytes_per_launch")
    extra = {} if args.no_extra else extra_workloads(ctx, dev, ev)

    value = pf.total_tokens / (ms_step * 1e-3)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill_throughput (960 packed seqs, T=%d, 28 layers, Hq16/Hkv8/D128, fp32 out) + gather "
                        "[T,1024]; beam_short_prompt (R32 x W100, P128, 4 steps, 24 layers, Hq14/Hkv2/D64, V151936)"
                        % T,
            "value_counts": "prefill tokens per step (each through 28 layers) / whole-step time",
        },
        "roofline": {
            "kernel": "prefill_persistent_kernel<128,2,f32> with its prefill_plan_kernel (one prefill call)",
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": pbytes,
            "avg_launch_us": round(prefill_us, 2),          # events around the call: plan + persistent kernel
            "mfma_tflops_causal": round(mfma_tflops, 1),
            "mfma_frac": round(mfma_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_frac_ceiling_at_hbm_peak": round(min(1.0, pflops / pbytes * HBM_PEAK_GBS * 1e9 / 1e12
                                                       / MFMA_BF16_PEAK_TFLOPS), 4),
        },
        "parts": dict({
            "prefill_layer_us": round(prefill_us, 2),
            "prefill_28_layers_ms": round(prefill_us * pf.n_layers / 1e3, 3),
            "prefill_tokens_per_s": round(pf.total_tokens / (prefill_us * pf.n_layers * 1e-6), 1),
            "gather_us": round(gather_us, 2),
        }, **beam.summary(per), host_wall_s=round(t_wall, 3)),
    }
    if graph_ms is not None:
        line["graph_replay"] = {"ms_per_step": round(graph_ms, 4),
                                "tokens_per_s": round(pf.total_tokens / (graph_ms * 1e-3), 1),
                                "what": "the same step captured once as a HIP graph and replayed"}
    line.update(extra)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pf, bs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
