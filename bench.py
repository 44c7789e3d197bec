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
    151,936, as one call of the library's fixed-step driver: first merge (one
    beam in), then per step the 24-layer decode attention (history read
    through the last parents, suffix written in the new order) and the top-k
    merge; finally the suffix reorder by the last parents and the backtrack
    of the parents into each beam's token sequence.

value = prefill tokens per step (T, each through all 28 layers) / step time.
The JSON line also carries the per-part times (medians; the beam-search
breakdown from a pass that issues the same launches one by one with events
between them), the roofline of the dominant kernel (packed prefill
attention, from the mean of its per-launch events over the timed steps) and
the oracle timed per workload on the same arrays.
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
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the timed oracle runs")
    ap.add_argument("--no-graph", action="store_true", help="skip the captured-graph timing of the step")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the reporting-only prefill-request and long-prompt beam timings")
    ap.add_argument("--summarize", nargs="+", metavar=("KIND", "DIR"),
                    help="host only: print a summary of rocprofv3 CSV output and exit. KIND is 'trace' (one "
                         "--kernel-trace dir), 'sq' (--pmc dirs of SQ counters) or 'traffic' (FETCH_SIZE dir, "
                         "WRITE_SIZE dir, and the same two for --copy-calibration; writes the prefill record)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--kernels-only", action="store_true",
                    help="untimed: two launches of every hot-path workload (960-sequence prefill layer, gather, "
                         "short- and long-prompt searches), for counter collection, then exit")
    return ap.parse_args()


PREFILL_SOURCES = ("prefill_attn.hip", "attn_tile.h")


def src_sha(*names: str) -> str:
    """Short hash of kernel sources (csrc/), to tie a counter record to them."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "bounded_generation_slm_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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


def _host(t):
    """A device tensor's contents on the host (bf16 as its 16-bit storage)."""
    import numpy as np
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def oracle_beam_search_time(run):
    """The oracle's whole fixed-step search (oracle.beam_search: every merge,
    every decode step over all layers, the final reorder and backtrack) on
    host copies of the bench's device inputs; seconds."""
    import oracle
    x, bs = run.x, run.bs
    pk, pv = _host(x["prefix_k"]), _host(x["prefix_v"])
    steps = {t: dict(q=_host(x["q"][t - 1]), k_new=_host(x["k_new"][t - 1]), v_new=_host(x["v_new"][t - 1]))
             for t in range(1, bs.n_steps + 1)}
    lps = [_host(lp) for lp in x["logprobs"]]
    t0 = time.perf_counter()
    oracle.beam_search(steps.__getitem__, pk, pv, lps.__getitem__, bs.width, bs.n_steps,
                       on_step=lambda t, r: None)
    return round(time.perf_counter() - t0, 3)


def cpu_baseline(pf, pf_dev, beam, more=None):
    """The oracle on the host cores, per workload on the same arrays the GPU
    reads: the tiny workload (prefill and 4-step search), the one-request
    prefill, layer 0 of the 960-sequence pack (the 28 layer calls of a step
    read one Q/K/V set, so the step's prefill is 28 times that), the whole
    short-prompt search and (in `more`, timed where its arrays live) the whole
    long-prompt search.  value: prefill tokens per second of one whole step
    (28 prefill layers + gather + short-prompt search), like the GPU value."""
    import numpy as np

    import oracle
    import workloads as wl

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    per = {}
    x = wl.prefill_inputs(wl.TINY_PREFILL)
    t0 = time.perf_counter()
    oracle.prefill_attn(x["q"], x["k"], x["v"], x["cu_seqlens"])
    tb = wl.TINY_BEAM
    st = wl.beam_static_inputs(tb)
    oracle.beam_search(lambda t: wl.beam_step_inputs(tb, t), st["prefix_k"], st["prefix_v"],
                       lambda t: wl.beam_logprobs(tb, t), tb.width, tb.n_steps)
    per["tiny (prefill pack of 4 + 4-step search, R2 x W4, V1000)"] = round(time.perf_counter() - t0, 3)
    x = wl.prefill_inputs(wl.PREFILL_REQUEST)
    t0 = time.perf_counter()
    oracle.prefill_attn(x["q"], x["k"], x["v"], x["cu_seqlens"])
    oracle.gather_last(x["hidden"], x["cu_seqlens"])
    per["prefill_request (15 sequences, 1 layer + gather)"] = round(time.perf_counter() - t0, 3)
    q, k, v, hidden = (_host(t) for t in pf_dev)
    cu = pf.cu_seqlens()
    t0 = time.perf_counter()
    oracle.prefill_attn(q, k, v, cu)
    t_layer = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gather_last(hidden, cu)
    t_gather = time.perf_counter() - t0
    del q, k, v, hidden
    per["prefill_throughput layer 0 (960 sequences, T=%d)" % pf.total_tokens] = round(t_layer, 3)
    per["prefill_throughput 28 layers (extrapolated: 28 x layer 0)"] = round(t_layer * pf.n_layers, 3)
    t_search = oracle_beam_search_time(beam)
    per["beam_short_prompt whole search (R32 x W100, 4 steps, 24 layers)"] = t_search
    per.update(more or {})
    step_s = t_layer * pf.n_layers + t_gather + t_search
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
        "value": pf.total_tokens / step_s,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "per_workload_s": per,
        "host": {"cpu_model": cpu_model, "logical_cpus": os.cpu_count(), "omp_threads": threads,
                 "one_thread_s": one_thread_times()},
        "sample": ("fp64 C oracle, %d threads, on the bench's own arrays: prefill layer 0 of the 960-sequence pack "
                   "in full (%.1f s, x28 for the step's 28 layer calls over the same Q/K/V), the gather, and the whole "
                   "short-prompt search in full (%.1f s); one step estimated at %.0f s. The long-prompt search, "
                   "timed in full, is listed per workload (not part of value)" % (
                       threads, t_layer, t_search, step_s)),
    }


def traffic_from_counters(launch_bytes_key: str):
    """HBM bytes per launch from the committed counter record, if it was
    taken on the current prefill kernel sources."""
    path = os.path.join(PROFILES, "prefill_attn_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != src_sha(*PREFILL_SOURCES):
        return None
    return rec.get(launch_bytes_key)


# ---------------------------------------------------------------------------
# rocprofv3 output -> the text summaries kept under profiles/ (runs on the
# host, on the CSV files a profiled run of this script wrote)

N_XCD, N_SIMD = 8, 256 * 4          # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def _kernel_short(name: str) -> str:
    import re
    name = name.replace("void ", "").replace("slm::(anonymous namespace)::", "slm::")
    return re.sub(r"\((slm::)?\w+Params.*\)$", "", name)


def _csv_rows(d: str, suffix: str):
    import csv
    import glob
    out = []
    for path in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(path, newline="") as f:
            out += list(csv.DictReader(f))
    return out


def _dispatch_counters(d: str):
    """{dispatch id: (kernel, grid, duration ns, {counter: value})} of one
    --pmc run (a counter's per-instance rows summed)."""
    disp = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        key = int(r["Dispatch_Id"])
        k = disp.setdefault(key, [r["Kernel_Name"], int(r["Grid_Size"]),
                                  int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), {}])
        k[3][r["Counter_Name"]] = k[3].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return disp


def _groups(disp, only_slm=True):
    """Per (kernel, grid): number of dispatches, mean duration and mean counters."""
    g = {}
    for kern, grid, dur, cs in disp.values():
        if only_slm and "slm::" not in kern:
            continue
        e = g.setdefault((kern, grid), {"n": 0, "dur": 0.0, "c": {}})
        e["n"] += 1
        e["dur"] += dur
        for c, v in cs.items():
            e["c"][c] = e["c"].get(c, 0.0) + v
    for e in g.values():
        e["dur"] /= e["n"]
        e["c"] = {c: v / e["n"] for c, v in e["c"].items()}
    return g


def summarize_kernel_trace(d: str) -> str:
    """Per (kernel, grid) launch statistics from a --kernel-trace run."""
    g = {}
    for r in _csv_rows(d, "kernel_trace.csv"):
        key = (r["Kernel_Name"], int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0))
        g.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    total = sum(sum(v) for v in g.values()) or 1
    lines = ["# calls  avg_us   min_us   max_us   share  grid  kernel"]
    for (kern, grid), v in sorted(g.items(), key=lambda kv: -sum(kv[1])):
        lines.append("%6d %8.1f %8.1f %8.1f %6.2f%% %7d  %s" % (
            len(v), sum(v) / len(v) / 1e3, min(v) / 1e3, max(v) / 1e3, 100.0 * sum(v) / total, grid,
            _kernel_short(kern)[:110]))
    return "\n".join(lines)


def summarize_sq(dirs) -> str:
    """Instruction mix and MFMA use per (kernel, grid) from --pmc runs of SQ
    counters.  Normalisation: GRBM_GUI_ACTIVE is the sum of the 8 XCDs'
    busy-cycle counters (divided by 8 it gives the clock over the dispatch);
    SQ_VALU_MFMA_BUSY_CYCLES is summed over all SIMDs, so the MFMA-busy
    fraction is busy / (cycles x 1024 SIMDs)."""
    merged = {}
    for d in dirs:
        for key, e in _groups(_dispatch_counters(d)).items():
            m = merged.setdefault(key, {"n": e["n"], "dur": e["dur"], "c": {}})
            m["c"].update(e["c"])
    lines = []
    for (kern, grid), e in sorted(merged.items(), key=lambda kv: -kv[1]["dur"] * kv[1]["n"]):
        c = e["c"]
        waves = c.get("SQ_WAVES", 0.0) or 1.0
        mfma = c.get("SQ_INSTS_MFMA", 0.0)
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        row = {"dispatches": e["n"], "grid": grid, "us_profiled": round(e["dur"] / 1e3, 1),
               "clock_GHz": round(cyc / e["dur"], 3) if cyc else None, "waves": int(waves)}
        for name, cnt in (("VALU", "SQ_INSTS_VALU"), ("SALU", "SQ_INSTS_SALU"), ("MFMA", "SQ_INSTS_MFMA"),
                          ("LDS", "SQ_INSTS_LDS"), ("VMEM_RD", "SQ_INSTS_VMEM_RD"), ("SMEM", "SQ_INSTS_SMEM")):
            if cnt in c:
                row[name + "_per_wave"] = round(c[cnt] / waves, 1)
        if mfma:
            row["VALU_per_MFMA"] = round(c.get("SQ_INSTS_VALU", 0.0) / mfma, 2)
            row["SALU_per_MFMA"] = round(c.get("SQ_INSTS_SALU", 0.0) / mfma, 2)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                row["MFMA_busy_cycles_per_inst"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / mfma, 2)
        if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            row["MFMA_busy_frac"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD), 4)
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:         # units of 512 flops
            row["MFMA_bf16_TFLOP_executed"] = round(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e12, 4)
        wc = c.get("SQ_WAVE_CYCLES")
        if wc:
            for name, cnt in (("wait_any", "SQ_WAIT_INST_ANY"), ("active_valu", "SQ_ACTIVE_INST_VALU"),
                              ("active_lds", "SQ_ACTIVE_INST_LDS"), ("active_any", "SQ_ACTIVE_INST_ANY")):
                if cnt in c:
                    row[name + "_per_wave_cycle"] = round(c[cnt] / wc, 3)
        if c.get("SQ_ACTIVE_INST_LDS") and "SQ_LDS_BANK_CONFLICT" in c:
            row["lds_bank_conflict_per_lds_cycle"] = round(c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"], 3)
        lines.append(_kernel_short(kern))
        lines.append("    " + json.dumps(row))
    return "\n".join(lines)


def summarize_traffic(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, record=None) -> str:
    """HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE (KiB) runs,
    each scaled by what the same counter reads for a plain device copy of
    known size (bench.py --copy-calibration).  With `record`, also writes the
    prefill call's bytes (plan + persistent kernel, fp32 out on the
    960-sequence pack) as JSON for the bench's roofline.traffic."""
    copy_bytes = (1 << 28) * 4

    def copy_kib(d, cnt):
        best = 0.0
        for kern, grid, dur, cs in _dispatch_counters(d).values():
            if "slm::" not in kern:
                best = max(best, cs.get(cnt, 0.0))
        return best

    fs = copy_bytes / 1024.0 / copy_kib(cal_fetch_dir, "FETCH_SIZE")
    ws = copy_bytes / 1024.0 / copy_kib(cal_write_dir, "WRITE_SIZE")
    fg, wg = _groups(_dispatch_counters(fetch_dir)), _groups(_dispatch_counters(write_dir))
    lines = ["# copy calibration: %d bytes each way; FETCH_SIZE scale %.4f, WRITE_SIZE scale %.4f" % (
        copy_bytes, fs, ws),
        "# dispatches  grid  FETCH_KiB_raw  WRITE_KiB_raw  read_GB  write_GB  kernel"]
    for key in sorted(set(fg) | set(wg), key=lambda k: -(fg.get(k, {}).get("c", {}).get("FETCH_SIZE", 0.0))):
        f = fg.get(key, {}).get("c", {}).get("FETCH_SIZE", 0.0)
        w = wg.get(key, {}).get("c", {}).get("WRITE_SIZE", 0.0)
        n = fg.get(key, wg.get(key, {})).get("n", 0)
        lines.append("%6d %8d %14.1f %14.1f %8.3f %8.3f  %s" % (
            n, key[1], f, w, f * fs * 1024 / 1e9, w * ws * 1024 / 1e9, _kernel_short(key[0])[:100]))
    if record:
        import workloads as wl
        pf = wl.PREFILL_THROUGHPUT
        per = {"persistent_fetch": 0.0, "persistent_write": 0.0, "plan_fetch": 0.0, "plan_write": 0.0}
        n = 0
        for (kern, grid), e in fg.items():
            if "prefill_persistent_kernel<128, 2, false>" in kern:
                per["persistent_fetch"], n = e["c"].get("FETCH_SIZE", 0.0), e["n"]
            elif "prefill_plan_kernel" in kern:
                per["plan_fetch"] = e["c"].get("FETCH_SIZE", 0.0)
        for (kern, grid), e in wg.items():
            if "prefill_persistent_kernel<128, 2, false>" in kern:
                per["persistent_write"] = e["c"].get("WRITE_SIZE", 0.0)
            elif "prefill_plan_kernel" in kern:
                per["plan_write"] = e["c"].get("WRITE_SIZE", 0.0)
        hbm = per["persistent_fetch"] * fs * 1024 + per["persistent_write"] * ws * 1024   # one layer call
        alg, _ = prefill_bytes_flops(pf.lengths, pf.n_heads_q, pf.n_heads_kv, pf.head_dim, 4)
        rec = {"kernel_source_sha": src_sha(*PREFILL_SOURCES),
               "what": "HBM bytes of one packed-prefill layer call over the step's plan "
                       "(prefill_persistent_kernel<128,2,f32>) on the 960-sequence pack (T=%d, Hq16/Hkv8/D128, "
                       "fp32 out); the plan kernel, once per step, is listed apart" % pf.total_tokens,
               "calibration": {"copy_bytes_each_way": copy_bytes, "fetch_scale": round(fs, 4),
                               "write_scale": round(ws, 4)},
               "per_dispatch_kib": dict({k: round(v, 1) for k, v in per.items()}, dispatches=n),
               "hbm_bytes_per_launch": int(round(hbm)),
               "algorithmic_bytes_per_launch": alg}
        with open(record, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        lines.append("# prefill layer call (persistent kernel): %.4f GB counted vs %.4f GB algorithmic (x%.4f)" % (
            hbm / 1e9, alg / 1e9, hbm / alg))
    return "\n".join(lines)


def extra_workloads(ctx, dev, ev, reps=5, cpu_oracle=True):
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
    bl = BeamRun(ctx, wl.BEAM_LONG, dev)
    bl.run(ctx)
    res["beam_long_prompt"] = dict(
        {"workload": "R8 x W400, P480, 5 steps, 24 layers, Hq14/Hkv2/D64, V151936"}, **time_beam(ctx, bl, ev, 20))
    if cpu_oracle:                  # moved into cpu_baseline by the caller
        res["oracle_long_search_s"] = oracle_beam_search_time(bl)
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
    """Device-resident inputs and preallocated state of one fixed-step beam
    search.  run() is the product's one-call driver (slm_beam_search: first
    merge with one beam in, then per step the all-layer decode attention and
    the merge, finally the suffix reorder by the last parents and the
    backtrack into token sequences); run_parts() issues the same launches one
    by one with events between them, for the per-part breakdown."""

    def __init__(self, ctx, bs, dev):
        import workloads as wl
        self.bs = bs
        self.x = wl.torch_beam_inputs(bs, dev)
        self.st = ctx.beam_search_state(bs.n_layers, bs.num_requests, bs.width, bs.n_steps, bs.n_heads_q,
                                        bs.n_heads_kv, bs.head_dim)

    def run(self, ctx):
        x = self.x
        ctx.beam_search(self.st, x["prefix_k"], x["prefix_v"], x["logprobs"], x["q"], x["k_new"], x["v_new"])

    def run_parts(self, ctx, marks, ev):
        x, st, N, W, R = self.x, self.st, self.bs.n_steps, self.bs.width, self.bs.num_requests
        tok, par, cum = st["tokens"], st["parent"], st["cum"]
        e0 = ev()
        ctx.beam_topk_merge(x["logprobs"][0], st["cum0"].view(R, 1), W, tok[0], par[0], cum[0])
        marks.append(("merge0", e0, ev()))
        for t in range(1, N + 1):
            ski, svi = (st["suffix_k"][(t + 1) % 2], st["suffix_v"][(t + 1) % 2]) if t > 1 else (None, None)
            e0 = ev()
            ctx.beam_decode_attn(x["q"][t - 1], x["prefix_k"], x["prefix_v"], ski, svi, x["k_new"][t - 1],
                                 x["v_new"][t - 1], par[t - 1], t - 1, st["suffix_k"][t % 2], st["suffix_v"][t % 2],
                                 out=st["attn_out"][t - 1])
            e1 = ev()
            ctx.beam_topk_merge(x["logprobs"][t], cum[t - 1], W, tok[t], par[t], cum[t])
            e2 = ev()
            marks.append(("decode%d" % t, e0, e1))
            marks.append(("merge%d" % t, e1, e2))
        e0 = ev()
        ctx.beam_reorder_suffix(par[N], st["suffix_k"][N % 2], st["suffix_v"][N % 2], N, st["final_k"], st["final_v"])
        e1 = ev()
        ctx.beam_backtrack(tok, par, out=st["sequences"])
        marks.append(("reorder", e0, e1))
        marks.append(("backtrack", e1, ev()))

    def summary(self, per, search_us=None):
        """Per-part medians (us) and the beam-step HBM fraction; search_us is
        the one-call driver's time for the whole search, when measured."""
        bs = self.bs
        N, R, W, V = bs.n_steps, bs.num_requests, bs.width, bs.vocab
        med = {k: sorted(v)[len(v) // 2] for k, v in per.items()}
        parts = ["merge0"] + ["decode%d" % t for t in range(1, N + 1)] + ["merge%d" % t for t in range(1, N + 1)] \
            + ["reorder", "backtrack"]
        parts_us = sum(med[p] for p in parts)
        search_us = parts_us if search_us is None else search_us
        step_us = [med["decode%d" % t] + med["merge%d" % t] for t in range(1, N + 1)]
        step_bytes = [decode_bytes(bs, t) + topk_bytes(R, W, V, W) for t in range(1, N + 1)]
        return {
            "beam_search_us": round(search_us, 1),
            "beam_search_parts_sum_us": round(parts_us, 1),
            "beam_step_us": [round(u, 1) for u in step_us],
            "beam_step_us_mean": round(sum(step_us) / N, 1),
            "beam_step_hbm_frac": [round(b / (u * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) for b, u in zip(step_bytes, step_us)],
            "decode_us": [round(med["decode%d" % t], 1) for t in range(1, N + 1)],
            "decode_hbm_frac": [round(decode_bytes(bs, t) / (med["decode%d" % t] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                for t in range(1, N + 1)],
            "merge_us": [round(med["merge%d" % t], 1) for t in range(0, N + 1)],
            "merge_hbm_frac": [round(topk_bytes(R, W, V, W) / (med["merge%d" % t] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                               for t in range(1, N + 1)],
            "reorder_us": round(med["reorder"], 1),
            "backtrack_us": round(med["backtrack"], 1),
            "beam_requests_per_s": round(R / (search_us * 1e-6), 1),
            "beams_steps_per_s": round(R * W * N / (search_us * 1e-6), 1),
            "timing": "per-part medians of per-launch events over the repetitions; beam_search_us: median of the "
                      "one-call driver",
        }


def time_beam(ctx, run, ev, reps):
    """Per-part medians from run_parts and the one-call driver's median time."""
    import torch
    marks, whole = [], []
    for _ in range(reps):
        run.run_parts(ctx, marks, ev)
    for _ in range(reps):
        e0 = ev()
        run.run(ctx)
        whole.append((e0, ev()))
    torch.cuda.synchronize()
    ctx.check()
    per = {}
    for name, a, b in marks:
        per.setdefault(name, []).append(a.elapsed_time(b) * 1e3)
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in whole)[len(whole) // 2]
    return run.summary(per, us)


def main():
    args = parse()
    if args.summarize:
        kind, dirs = args.summarize[0], args.summarize[1:]
        if kind == "trace" and len(dirs) == 1:
            print(summarize_kernel_trace(dirs[0]))
        elif kind == "sq" and dirs:
            print(summarize_sq(dirs))
        elif kind == "traffic" and len(dirs) == 4:
            print(summarize_traffic(*dirs, record=os.path.join(PROFILES, "prefill_attn_traffic.json")))
        else:
            sys.exit("bench.py --summarize: trace DIR | sq DIR... | traffic FETCH WRITE CAL_FETCH CAL_WRITE")
        return
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

    beam = BeamRun(ctx, bs, dev)
    torch.cuda.synchronize()

    if args.kernels_only:
        long_run = BeamRun(ctx, wl.BEAM_LONG, dev)
        for _ in range(2):
            ctx.packed_prefill_attn(q, k, v, cu, pf.max_seqlen, out=pout)
            ctx.gather_last(hidden, cu, out=gout)
            beam.run(ctx)
            long_run.run(ctx)
        torch.cuda.synchronize()
        ctx.check()
        print(json.dumps({"kernels_only": "2 x (prefill layer, gather, short-prompt search, long-prompt search)"}))
        return

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def step(marks):
        """One pass of the whole hot path; marks collects (part, start, end) events.
        The pack's work list is built once and the 28 layer calls run over it."""
        e0 = ev()
        plan = ctx.prefill_plan(cu, pf.max_seqlen, T, Hq, Hkv, D)
        marks.append(("prefill_plan", e0, ev()))
        for _ in range(pf.n_layers):
            e0 = ev()
            ctx.packed_prefill_attn_planned(plan, q, k, v, cu, pf.max_seqlen, out=pout)
            marks.append(("prefill", e0, ev()))
        e0 = ev()
        ctx.gather_last(hidden, cu, out=gout)
        marks.append(("gather", e0, ev()))
        e0 = ev()
        beam.run(ctx)
        marks.append(("beam_search", e0, ev()))

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
        del g

    per = {}
    for name, a, b in marks:
        per.setdefault(name, []).append(a.elapsed_time(b) * 1e3)   # us
    med = lambda xs: sorted(xs)[len(xs) // 2]
    prefill_us = sum(per["prefill"]) / len(per["prefill"])         # mean launch duration (roofline)
    prefill_med = med(per["prefill"])
    plan_us = med(per["prefill_plan"])
    gather_us = med(per["gather"])
    search_us = med(per["beam_search"])
    beam_parts = time_beam(ctx, beam, ev, 20)                        # per-launch breakdown, outside the timed steps
    # the same prefill with bf16 output (half the output bytes), reporting only
    pout_bf = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
    plan = ctx.prefill_plan(cu, pf.max_seqlen, T, Hq, Hkv, D)
    for _ in range(3):
        ctx.packed_prefill_attn_planned(plan, q, k, v, cu, pf.max_seqlen, out=pout_bf)
    bf_ev = []
    for _ in range(pf.n_layers):
        e0 = ev()
        ctx.packed_prefill_attn_planned(plan, q, k, v, cu, pf.max_seqlen, out=pout_bf)
        bf_ev.append((e0, ev()))
    torch.cuda.synchronize()
    ctx.check()
    bf_us = med([a.elapsed_time(b) * 1e3 for a, b in bf_ev])
    del pout_bf

    pbytes, pflops = prefill_bytes_flops(pf.lengths, Hq, Hkv, D, 4)
    achieved_gbs = pbytes / (prefill_us * 1e-6) / 1e9
    mfma_tflops = pflops / (prefill_us * 1e-6) / 1e12
    traffic = traffic_from_counters("hbm_bytes_per_launch")
    extra = {} if args.no_extra else extra_workloads(ctx, dev, ev, cpu_oracle=not args.no_cpu_baseline)
    long_s = extra.get("reporting_only", {}).pop("oracle_long_search_s", None)

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
            "kernel": "prefill_persistent_kernel<128,2,f32> (one layer call over the step's plan)",
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": pbytes,
            "avg_launch_us": round(prefill_us, 2),          # events around the planned call: the persistent kernel
            "mfma_tflops_causal": round(mfma_tflops, 1),
            "mfma_frac": round(mfma_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "mfma_frac_ceiling_at_hbm_peak": round(min(1.0, pflops / pbytes * HBM_PEAK_GBS * 1e9 / 1e12
                                                       / MFMA_BF16_PEAK_TFLOPS), 4),
        },
        "parts": dict({
            "prefill_plan_us": round(plan_us, 2),           # once per step (the pack's work list)
            "prefill_layer_us_median": round(prefill_med, 2),
            "prefill_layer_us_mean": round(prefill_us, 2),
            "prefill_28_layers_ms": round((plan_us + prefill_med * pf.n_layers) / 1e3, 3),
            "prefill_tokens_per_s": round(pf.total_tokens / ((plan_us + prefill_med * pf.n_layers) * 1e-6), 1),
            "gather_us": round(gather_us, 2),
            "beam_search_one_call_us_in_step": round(search_us, 1),
        }, **beam_parts, host_wall_s=round(t_wall, 3)),
    }
    bbytes, _ = prefill_bytes_flops(pf.lengths, Hq, Hkv, D, 2)
    line["prefill_bf16_out"] = {
        "workload": "the same 960-sequence prefill layer with bf16 output (28 launches, median)",
        "us_per_layer_median": round(bf_us, 2),
        "algorithmic_bytes": bbytes,
        "hbm_frac": round(bbytes / (bf_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "mfma_frac": round(pflops / (bf_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "mfma_frac_ceiling_at_hbm_peak": round(min(1.0, pflops / bbytes * HBM_PEAK_GBS * 1e9 / 1e12
                                                   / MFMA_BF16_PEAK_TFLOPS), 4)}
    if graph_ms is not None:
        line["graph_replay"] = {"ms_per_step": round(graph_ms, 4),
                                "tokens_per_s": round(pf.total_tokens / (graph_ms * 1e-3), 1),
                                "what": "the same step captured once as a HIP graph and replayed"}
    line.update(extra)
    if not args.no_cpu_baseline:
        more = {} if long_s is None else {"beam_long_prompt whole search (R8 x W400, 5 steps, 24 layers)": long_s}
        line["cpu_baseline"] = cpu_baseline(pf, (q, k, v, hidden), beam, more)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
