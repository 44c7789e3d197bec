"""The oracle: a plain, slow, fp64 CPU implementation of the attention hot
path, written from the page "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化"
(abstract, §1.1, §1.2).  TEST INFRASTRUCTURE ONLY -- only the tests, the
smoke check and the bench's CPU-baseline leg may use it; it shares no code
with the HIP library and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over independent
rows).  This module compiles it with gcc when no built copy exists and
marshals numpy arrays into it.  Every function returns freshly allocated
numpy arrays.

Parity pins (see tests/test_oracle_*.py): every function here is pinned by
closed forms, brute force or an independent library routine; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP, strict IEEE)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
               "-std=c11", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.orc_prefill_attn.argtypes = [P, P, P, P, i32, i32, i32, i32, f64, P]
        lib.orc_prefill_attn_rows.argtypes = [P, P, P, P, i32, i32, i32, i32, f64, P, P, i64, P]
        lib.orc_gather_last.argtypes = [P, P, i32, i32, P]
        lib.orc_beam_decode_attn.argtypes = [i32] * 9 + [f64] + [P] * 12
        lib.orc_topk_merge.argtypes = [P, P, i32, i32, i32, i32, P, P, P]
        lib.orc_topk_merge_logits.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P]
        lib.orc_label_head.argtypes = [P, P, i32, i32, P, i32, P, i32, i32, P, P, P, P, P, P]
        lib.orc_reorder_suffix.argtypes = [i32] * 7 + [P] * 5
        lib.orc_beam_backtrack.argtypes = [P, P, i32, i32, i32, P]
        for f in ("orc_prefill_attn", "orc_prefill_attn_rows", "orc_gather_last",
                  "orc_beam_decode_attn", "orc_topk_merge", "orc_topk_merge_logits", "orc_label_head",
                  "orc_reorder_suffix", "orc_beam_backtrack"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def prefill_attn(q, k, v, cu_seqlens, scale=None) -> np.ndarray:
    """Packed causal GQA attention.  q [T,Hq,D], k/v [T,Hkv,D] bf16 bits
    (uint16), cu_seqlens [B+1] -> out [T,Hq,D] float64."""
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    cu = _c(cu_seqlens, np.int32)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros((T, Hq, D), np.float64)
    _check(_load().orc_prefill_attn(_p(q), _p(k), _p(v), _p(cu), len(cu) - 1, Hq, Hkv, D,
                                    scale, _p(out)), "prefill_attn")
    return out


def prefill_attn_rows(q, k, v, cu_seqlens, tokens, heads, scale=None) -> np.ndarray:
    """The rows of ``prefill_attn`` at (tokens[i], heads[i]) only -> [n,D]."""
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    cu = _c(cu_seqlens, np.int32)
    tok, hd = _c(tokens, np.int64), _c(heads, np.int32)
    T, Hq, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros((len(tok), D), np.float64)
    _check(_load().orc_prefill_attn_rows(_p(q), _p(k), _p(v), _p(cu), len(cu) - 1, Hq,
                                         k.shape[1], D, scale, _p(tok), _p(hd), len(tok),
                                         _p(out)), "prefill_attn_rows")
    return out


def gather_last(hidden, cu_seqlens) -> np.ndarray:
    """hidden [T,H] 16-bit storage -> [B,H], the last valid row of each sequence."""
    hidden = _c(hidden, np.uint16)
    cu = _c(cu_seqlens, np.int32)
    B, H = len(cu) - 1, hidden.shape[1]
    out = np.empty((B, H), np.uint16)
    _check(_load().orc_gather_last(_p(hidden), _p(cu), B, H, _p(out)), "gather_last")
    return out


def label_head(hidden, cu_seqlens, lm_head, labels, k, label_map=None):
    """Prefill-only label head.  hidden [T,H], lm_head [V,H] 16-bit storage;
    labels [L] token ids; optional label_map [L] int32.  Returns (logits [B,L]
    fp64, probs [B,L] fp64, top_idx [B,K] int32, top_prob [B,K] fp64,
    top_class [B,K] int32 (map[top_idx], or top_idx without a map))."""
    hidden = _c(hidden, np.uint16)
    lm = _c(lm_head, np.uint16)
    cu = _c(cu_seqlens, np.int32)
    lab = _c(labels, np.int32)
    mp = None if label_map is None else _c(label_map, np.int32)
    B, H, V, L, K = len(cu) - 1, hidden.shape[1], lm.shape[0], len(lab), int(k)
    logits = np.empty((B, L), np.float64)
    probs = np.empty((B, L), np.float64)
    ti = np.empty((B, K), np.int32)
    tp = np.empty((B, K), np.float64)
    tc = np.empty((B, K), np.int32)
    _check(_load().orc_label_head(_p(hidden), _p(cu), B, H, _p(lm), V, _p(lab), L, K, _p(mp), _p(logits),
                                  _p(probs), _p(ti), _p(tp), _p(tc)), "label_head")
    return logits, probs, ti, tp, tc


def beam_decode_attn(q, prefix_k, prefix_v, suffix_k_in, suffix_v_in, k_new, v_new,
                     parent, hist_len, scale=None, prompt_cu=None):
    """Shared-prompt + per-beam-suffix decode attention.

    q [NL,R,W,Hq,D]; prefix_k/v [NL,R,P,Hkv,D], or with prompt_cu (R+1
    offsets) prompts of different lengths packed per layer as
    [NL,prompt_cu[R],Hkv,D] (request r: rows prompt_cu[r]..prompt_cu[r+1]);
    suffix_*_in [NL,R,W,S_cap,Hkv,D] (rows < hist_len valid, previous beam
    order); k_new/v_new [NL,R,W,Hkv,D]; parent [R,W] int32 or None (identity).
    Returns (out [NL,R,W,Hq,D] float64, suffix_k_out, suffix_v_out), the
    suffix outputs holding rows 0..hist_len (zeros above)."""
    q = _c(q, np.uint16)
    NL, R, W, Hq, D = q.shape
    pk, pv = _c(prefix_k, np.uint16), _c(prefix_v, np.uint16)
    cu = None
    if prompt_cu is None:
        P, Hkv = pk.shape[2], pk.shape[3]
    else:
        cu = _c(prompt_cu, np.int32)
        if cu.shape != (R + 1,) or pk.shape[:2] != (NL, int(cu[-1])):
            raise ValueError("beam_decode_attn: prompt_cu / packed prompt shape mismatch")
        P, Hkv = int(np.max(np.diff(cu), initial=0)), pk.shape[2]
    sk, sv = _c(suffix_k_in, np.uint16), _c(suffix_v_in, np.uint16)
    S_cap = sk.shape[3]
    kn, vn = _c(k_new, np.uint16), _c(v_new, np.uint16)
    par = None if parent is None else _c(parent, np.int32)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.zeros(q.shape, np.float64)
    sko = np.zeros(sk.shape, np.uint16)
    svo = np.zeros(sv.shape, np.uint16)
    _check(_load().orc_beam_decode_attn(NL, R, W, P, int(hist_len), S_cap, Hq, Hkv, D, scale,
                                        _p(q), _p(pk), _p(pv), _p(sk), _p(sv), _p(kn), _p(vn),
                                        _p(par), _p(cu), _p(out), _p(sko), _p(svo)), "beam_decode_attn")
    return out, sko, svo


def topk_merge(logprobs, cum, width):
    """logprobs [R,Win,V] fp32, cum [R,Win] fp32 -> (tokens, parent, cum_out),
    each [R,W]."""
    lp = _c(logprobs, np.float32)
    cm = _c(cum, np.float32)
    R, Win, V = lp.shape
    W = int(width)
    tok = np.empty((R, W), np.int32)
    par = np.empty((R, W), np.int32)
    co = np.empty((R, W), np.float32)
    _check(_load().orc_topk_merge(_p(lp), _p(cm), R, Win, V, W, _p(tok), _p(par), _p(co)),
           "topk_merge")
    return tok, par, co


def topk_merge_logits(logits, cum, width):
    """logits [R,Win,V] fp32, cum [R,Win] fp32 -> (tokens, parent, score, lse):
    tokens/parent [R,W] int32, score [R,W] fp64 (cum + logit - lse), lse
    [R,Win] fp64 (each row's log-sum-exp).  The merge with the log-softmax of
    each beam row folded in, all in fp64."""
    x = _c(logits, np.float32)
    cm = _c(cum, np.float32)
    R, Win, V = x.shape
    W = int(width)
    tok = np.empty((R, W), np.int32)
    par = np.empty((R, W), np.int32)
    sc = np.empty((R, W), np.float64)
    lse = np.empty((R, Win), np.float64)
    _check(_load().orc_topk_merge_logits(_p(x), _p(cm), R, Win, V, W, _p(tok), _p(par), _p(sc), _p(lse)),
           "topk_merge_logits")
    return tok, par, sc, lse


def reorder_suffix(parent, k_in, v_in, rows):
    """new[l,r,j,i] = old[l,r,parent[r,j],i] for i < rows; other rows zero."""
    k_in, v_in = _c(k_in, np.uint16), _c(v_in, np.uint16)
    NL, R, W, S_cap, Hkv, D = k_in.shape
    par = _c(parent, np.int32)
    ko = np.zeros(k_in.shape, np.uint16)
    vo = np.zeros(v_in.shape, np.uint16)
    _check(_load().orc_reorder_suffix(NL, R, W, int(rows), S_cap, Hkv, D, _p(par), _p(k_in),
                                      _p(v_in), _p(ko), _p(vo)), "reorder_suffix")
    return ko, vo


def beam_backtrack(tokens, parent):
    """tokens, parent [n_merges, R, W] int32 (the merges' outputs, merge 0
    first) -> seq [R, W, n_merges]: the token each final beam's ancestor took
    at every merge, found by following the parents back from the last merge."""
    tok, par = _c(tokens, np.int32), _c(parent, np.int32)
    n, R, W = tok.shape
    if par.shape != tok.shape:
        raise ValueError("beam_backtrack: tokens and parent shapes differ")
    seq = np.empty((R, W, n), np.int32)
    _check(_load().orc_beam_backtrack(_p(tok), _p(par), n, R, W, _p(seq)), "beam_backtrack")
    return seq


def beam_search(step_inputs, prefix_k, prefix_v, logprobs_by_step, width, n_steps,
                suffix_cap=None, scale=None, on_step=None):
    """The fixed-step sequence: merge on the prefill log-probs (one beam in),
    then for t = 1..n_steps: decode attention with s = t suffix rows (history
    read through the last merge's parents), then the merge on step t's
    log-probs; finally the suffix reordered by the last parents and the
    backtrack of the parents into each final beam's token sequence.
    ``step_inputs(t)`` returns dict(q, k_new, v_new) for step t;
    ``logprobs_by_step(t)`` the [R,Win,V] log-probs.

    Returns a dict with per-step outputs: tokens/parent/cum lists (index 0 is
    the first merge), attention outputs and suffix states per step, the final
    suffix reordered by the last merge's parents, and ``sequences`` [R,W,N+1].
    With ``on_step``, each decode step's results are handed to
    ``on_step(t, dict(attn, suffix_k, suffix_v))`` instead of being kept (the
    attention outputs of a full-size search would not fit host memory
    comfortably)."""
    lp0 = logprobs_by_step(0)
    R = lp0.shape[0]
    cum0 = np.zeros((R, lp0.shape[1]), np.float32)
    tok, par, cum = topk_merge(lp0, cum0, width)
    res = dict(tokens=[tok], parent=[par], cum=[cum], attn=[], suffix_k=[], suffix_v=[])
    NL = prefix_k.shape[0]
    Hkv, D = prefix_k.shape[3], prefix_k.shape[4]
    S_cap = n_steps if suffix_cap is None else suffix_cap
    sk = np.zeros((NL, R, width, S_cap, Hkv, D), np.uint16)
    sv = np.zeros_like(sk)
    for t in range(1, n_steps + 1):
        x = step_inputs(t)
        out, sk, sv = beam_decode_attn(x["q"], prefix_k, prefix_v, sk, sv, x["k_new"],
                                       x["v_new"], par, t - 1, scale)
        if on_step is None:
            res["attn"].append(out)
            res["suffix_k"].append(sk)
            res["suffix_v"].append(sv)
        else:
            on_step(t, dict(attn=out, suffix_k=sk, suffix_v=sv))
        del out
        tok, par, cum = topk_merge(logprobs_by_step(t), cum, width)
        res["tokens"].append(tok)
        res["parent"].append(par)
        res["cum"].append(cum)
    fk, fv = reorder_suffix(par, sk, sv, n_steps)
    res["final_suffix_k"], res["final_suffix_v"] = fk, fv
    res["sequences"] = beam_backtrack(np.stack(res["tokens"]), np.stack(res["parent"]))
    return res
