"""Python binding of libslm, the MI355X (gfx950) attention hot path of a
bounded-generation small-language-model engine.

This module only marshals arguments: it checks torch tensors (device, dtype,
contiguity), passes their device pointers and the current HIP stream to the
C ABI declared in ``include/slm.h``, and raises on a non-OK status.  Every
step of the computation runs in the HIP kernels of ``libslm.so``; there is no
CPU or PyTorch fallback, and importing this module fails loudly when the
library has not been built (``python bounded_generation_slm_amd/_build.py``).

The functions carry the C names (``slm_packed_prefill_attn`` and so on) and
take a :class:`Context` first; the same calls are available as methods.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libslm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libslm.so is not built; run `python bounded_generation_slm_amd/_build.py` "
        "(hipcc, gfx950) -- there is no fallback implementation")

_lib = ctypes.CDLL(LIB_PATH)

SLM_OK, SLM_ERR_INVALID_ARG, SLM_ERR_UNSUPPORTED, SLM_ERR_CAPACITY = 0, 1, 2, 3
SLM_ERR_ALIAS, SLM_ERR_DEVICE, SLM_ERR_OOM = 4, 5, 6
SLM_BF16, SLM_F32 = 0, 1

EXPORTED = (
    "slm_abi_version", "slm_status_string", "slm_ctx_create", "slm_ctx_destroy",
    "slm_ctx_set_stream", "slm_ctx_check", "slm_ctx_last_error", "slm_packed_prefill_attn",
    "slm_gather_last", "slm_beam_decode_attn", "slm_beam_topk_merge", "slm_beam_topk_merge_logits",
    "slm_beam_reorder_suffix", "slm_label_head", "slm_beam_backtrack", "slm_beam_search",
    "slm_packed_prefill_attn_noalloc", "slm_prefill_plan", "slm_packed_prefill_attn_planned",
)


class _Caps(ctypes.Structure):
    _fields_ = [("max_requests", ctypes.c_int32), ("max_beams", ctypes.c_int32),
                ("max_vocab", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("max_heads_q", ctypes.c_int32)]


class _BeamAttnArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "num_requests", "width", "prompt_len", "hist_len", "suffix_cap",
        "n_heads_q", "n_heads_kv", "head_dim")] + [("scale", ctypes.c_float)] + [
        (n, ctypes.c_void_p) for n in (
            "q", "prefix_k", "prefix_v", "suffix_k_in", "suffix_v_in", "k_new", "v_new", "parent",
            "suffix_k_out", "suffix_v_out", "out")] + [("out_dtype", ctypes.c_int)] + [
        ("prompt_cu", ctypes.c_void_p), ("prompt_rows", ctypes.c_int32)]


class _BeamSearchArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "num_requests", "width", "prompt_len", "n_steps", "suffix_cap", "n_heads_q", "n_heads_kv",
        "head_dim", "vocab")] + [("scale", ctypes.c_float)] + [
        (n, ctypes.c_void_p) for n in ("prefix_k", "prefix_v", "prompt_cu")] + [("prompt_rows", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in ("cum0", "logprobs", "q", "k_new", "v_new")] + [
        ("suffix_k", ctypes.c_void_p * 2), ("suffix_v", ctypes.c_void_p * 2)] + [
        (n, ctypes.c_void_p) for n in ("final_k", "final_v", "attn_out")] + [("out_dtype", ctypes.c_int)] + [
        (n, ctypes.c_void_p) for n in ("tokens", "parent", "cum", "sequences")]


_P, _I, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
_lib.slm_abi_version.restype = ctypes.c_int
_ABI = 6                                  # the struct layouts above and the symbol set
if _lib.slm_abi_version() != _ABI:
    raise ImportError("%s has ABI version %d, this binding expects %d: rebuild it with "
                      "bounded_generation_slm_amd/_build.py" % (LIB_PATH, _lib.slm_abi_version(), _ABI))
_lib.slm_status_string.restype = ctypes.c_char_p
_lib.slm_status_string.argtypes = [ctypes.c_int]
_lib.slm_ctx_create.argtypes = [ctypes.c_int, ctypes.POINTER(_Caps), ctypes.POINTER(_P)]
_lib.slm_ctx_destroy.argtypes = [_P]
_lib.slm_ctx_destroy.restype = None
_lib.slm_ctx_set_stream.argtypes = [_P, _P]
_lib.slm_ctx_check.argtypes = [_P]
_lib.slm_ctx_last_error.argtypes = [_P]
_lib.slm_ctx_last_error.restype = ctypes.c_char_p
_lib.slm_packed_prefill_attn.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, ctypes.c_int]
_lib.slm_gather_last.argtypes = [_P, _P, _P, _I, _I, _I, ctypes.c_int, _P]
_lib.slm_beam_decode_attn.argtypes = [_P, ctypes.POINTER(_BeamAttnArgs)]
_lib.slm_beam_topk_merge.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P]
_lib.slm_beam_topk_merge_logits.argtypes = [_P, _P, ctypes.c_int, _P, _I, _I, _I, _I, _P, _P, _P, _P]
_lib.slm_label_head.argtypes = [_P, _P, _P, _I, _I, _I, _P, _I, _P, _I, _I, _P, _P, _P, _P, _P, _P]
_lib.slm_beam_reorder_suffix.argtypes = [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]
_lib.slm_beam_backtrack.argtypes = [_P, _P, _P, _I, _I, _I, _P]
_lib.slm_beam_search.argtypes = [_P, ctypes.POINTER(_BeamSearchArgs)]
_lib.slm_packed_prefill_attn_noalloc.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, ctypes.c_int, _P]
_lib.slm_prefill_plan.argtypes = [_P, _P, _I, _I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_uint64)]
_lib.slm_packed_prefill_attn_planned.argtypes = [_P, ctypes.c_uint64, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P,
                                                 ctypes.c_int]
for _name in ("slm_ctx_create", "slm_ctx_set_stream", "slm_ctx_check", "slm_packed_prefill_attn",
              "slm_gather_last", "slm_beam_decode_attn", "slm_beam_topk_merge", "slm_beam_topk_merge_logits",
              "slm_beam_reorder_suffix", "slm_label_head", "slm_beam_backtrack", "slm_beam_search",
              "slm_packed_prefill_attn_noalloc"):
    getattr(_lib, _name).restype = ctypes.c_int


class SlmError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__("%s: %s" % (_lib.slm_status_string(status).decode(), detail))


def abi_version() -> int:
    return _lib.slm_abi_version()


def _ptr(t: Optional[torch.Tensor], name: str, dtypes, device) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s: dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if t.device != device:
        raise ValueError("%s is on %s, the context is on %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16)
_OUT = {torch.float32: SLM_F32, torch.bfloat16: SLM_BF16}


class Context:
    """A libslm context on one GPU: its stream is torch's current stream at
    each call, and its workspace is sized by the caps at creation.

    ``device=-1`` makes a dry-run context: every call runs the library's
    host-side validation on CPU tensors and launches nothing."""

    def __init__(self, device: int = 0, max_requests: int = 64, max_beams: int = 512,
                 max_vocab: int = 262144, max_tokens: int = 1 << 20, max_seqs: int = 8192,
                 max_heads_q: int = 64):
        self.dry_run = device < 0
        if self.dry_run:
            self.device = torch.device("cpu")
        else:
            self.device = torch.device("cuda", device)
            torch.cuda.init()
        caps = _Caps(max_requests, max_beams, max_vocab, max_tokens, max_seqs, max_heads_q)
        handle = _P()
        rc = _lib.slm_ctx_create(device, ctypes.byref(caps), ctypes.byref(handle))
        if rc != SLM_OK:
            raise SlmError(rc, "slm_ctx_create(device=%d)" % device)
        self._h = handle
        self.caps = dict(max_requests=max_requests, max_beams=max_beams, max_vocab=max_vocab,
                         max_tokens=max_tokens, max_seqs=max_seqs, max_heads_q=max_heads_q)

    def close(self):
        if getattr(self, "_h", None):
            _lib.slm_ctx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _stream(self):
        if self.dry_run:
            return
        s = torch.cuda.current_stream(self.device).cuda_stream
        _lib.slm_ctx_set_stream(self._h, _P(s))

    def _raise(self, rc: int, what: str):
        if rc != SLM_OK:
            raise SlmError(rc, "%s: %s" % (what, _lib.slm_ctx_last_error(self._h).decode()))

    def check(self):
        """Synchronise the stream and raise if a kernel flagged bad device-side
        arguments (cu_seqlens, parent)."""
        self._stream()
        self._raise(_lib.slm_ctx_check(self._h), "slm_ctx_check")

    # -- calls (argument marshalling only) --
    def packed_prefill_attn(self, q, k, v, cu_seqlens, max_seqlen: int, scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None, out_dtype=torch.float32):
        return slm_packed_prefill_attn(self, q, k, v, cu_seqlens, max_seqlen, scale, out, out_dtype)

    def prefill_plan(self, cu_seqlens, max_seqlen: int, total_tokens: int, n_heads_q: int, n_heads_kv: int,
                     head_dim: int) -> int:
        return slm_prefill_plan(self, cu_seqlens, max_seqlen, total_tokens, n_heads_q, n_heads_kv, head_dim)

    def packed_prefill_attn_planned(self, plan: int, q, k, v, cu_seqlens, max_seqlen: int,
                                    scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                                    out_dtype=torch.float32):
        return slm_packed_prefill_attn_planned(self, plan, q, k, v, cu_seqlens, max_seqlen, scale, out, out_dtype)

    def gather_last(self, hidden, cu_seqlens, out=None):
        return slm_gather_last(self, hidden, cu_seqlens, out)

    def beam_decode_attn(self, *args, **kw):
        return slm_beam_decode_attn(self, *args, **kw)

    def beam_topk_merge(self, logprobs, cum, width: int, tokens=None, parent=None, cum_out=None):
        return slm_beam_topk_merge(self, logprobs, cum, width, tokens, parent, cum_out)

    def beam_topk_merge_logits(self, logits, cum, width: int, tokens=None, parent=None, cum_out=None,
                               lse_out=None):
        return slm_beam_topk_merge_logits(self, logits, cum, width, tokens, parent, cum_out, lse_out)

    def beam_reorder_suffix(self, parent, k_in, v_in, rows: int, k_out, v_out):
        return slm_beam_reorder_suffix(self, parent, k_in, v_in, rows, k_out, v_out)

    def beam_backtrack(self, tokens, parent, out=None):
        return slm_beam_backtrack(self, tokens, parent, out)

    def beam_search_state(self, n_layers: int, num_requests: int, width: int, n_steps: int, n_heads_q: int,
                          n_heads_kv: int, head_dim: int, suffix_cap: Optional[int] = None,
                          out_dtype=torch.float32, attn_per_step: bool = False) -> dict:
        """Preallocated state of one fixed-step search (the load-time plan):
        the two suffix buffers, the final suffix, the attention output (one
        buffer, or one per step), the merge outputs and the sequences."""
        NL, R, W, N = n_layers, num_requests, width, n_steps
        S = N if suffix_cap is None else suffix_cap
        dev = self.device
        sshape = (NL, R, W, max(S, 1), n_heads_kv, head_dim)
        z = lambda: torch.zeros(sshape, dtype=torch.bfloat16, device=dev)
        one = torch.empty((NL, R, W, n_heads_q, head_dim), dtype=out_dtype, device=dev)
        outs = [one] + [torch.empty_like(one) for _ in range(N - 1)] if attn_per_step else [one] * N
        return dict(suffix_k=[z(), z()], suffix_v=[z(), z()], final_k=z(), final_v=z(), attn_out=outs,
                    tokens=torch.empty((N + 1, R, W), dtype=torch.int32, device=dev),
                    parent=torch.empty((N + 1, R, W), dtype=torch.int32, device=dev),
                    cum=torch.empty((N + 1, R, W), dtype=torch.float32, device=dev),
                    sequences=torch.empty((R, W, N + 1), dtype=torch.int32, device=dev),
                    cum0=torch.zeros((R,), dtype=torch.float32, device=dev))

    def beam_search(self, state: dict, prefix_k, prefix_v, logprobs, q, k_new, v_new, scale=None, prompt_cu=None,
                    prompt_len: Optional[int] = None):
        return slm_beam_search(self, state, prefix_k, prefix_v, logprobs, q, k_new, v_new, scale, prompt_cu,
                               prompt_len)

    def label_head(self, hidden, cu_seqlens, lm_head, labels, k: int, label_map=None, probs: bool = True,
                   out=None):
        return slm_label_head(self, hidden, cu_seqlens, lm_head, labels, k, label_map, probs, out)


def slm_packed_prefill_attn(ctx: Context, q, k, v, cu_seqlens, max_seqlen: int,
                            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                            out_dtype=torch.float32) -> torch.Tensor:
    """q [T,Hq,D], k/v [T,Hkv,D] bf16; cu_seqlens [B+1] int32 (device).
    Returns out [T,Hq,D] (float32 or bfloat16)."""
    return _prefill(ctx, None, q, k, v, cu_seqlens, max_seqlen, scale, out, out_dtype)


def slm_prefill_plan(ctx: Context, cu_seqlens, max_seqlen: int, total_tokens: int, n_heads_q: int,
                     n_heads_kv: int, head_dim: int) -> int:
    """The work list of the pack cu_seqlens [B+1] int32 (device) with these
    sizes, built on the device; returns the plan id for
    slm_packed_prefill_attn_planned (the context's one current plan)."""
    dev = ctx.device
    plan = ctypes.c_uint64(0)
    ctx._stream()
    rc = _lib.slm_prefill_plan(ctx._h, _ptr(cu_seqlens, "cu_seqlens", (torch.int32,), dev), cu_seqlens.numel() - 1,
                               int(total_tokens), int(max_seqlen), int(n_heads_q), int(n_heads_kv), int(head_dim),
                               ctypes.byref(plan))
    ctx._raise(rc, "slm_prefill_plan")
    return plan.value


def slm_packed_prefill_attn_planned(ctx: Context, plan: int, q, k, v, cu_seqlens, max_seqlen: int,
                                    scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                                    out_dtype=torch.float32) -> torch.Tensor:
    """slm_packed_prefill_attn over the plan `plan` (same cu_seqlens and sizes)."""
    return _prefill(ctx, int(plan), q, k, v, cu_seqlens, max_seqlen, scale, out, out_dtype)


def _prefill(ctx: Context, plan, q, k, v, cu_seqlens, max_seqlen, scale, out, out_dtype) -> torch.Tensor:
    dev = ctx.device
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (T, Hkv, D) or v.shape != (T, Hkv, D):
        raise ValueError("k and v must be [T, Hkv, D] matching q")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=out_dtype, device=dev)
    if out.shape != (T, Hq, D) or out.dtype not in _OUT:
        raise ValueError("out must be [T, Hq, D] float32 or bfloat16")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    ctx._stream()
    args = (_ptr(q, "q", _BF16, dev), _ptr(k, "k", _BF16, dev), _ptr(v, "v", _BF16, dev),
            _ptr(cu_seqlens, "cu_seqlens", (torch.int32,), dev), cu_seqlens.numel() - 1, T,
            int(max_seqlen), Hq, Hkv, D, scale, _ptr(out, "out", tuple(_OUT), dev), _OUT[out.dtype])
    if plan is None:
        ctx._raise(_lib.slm_packed_prefill_attn(ctx._h, *args), "slm_packed_prefill_attn")
    else:
        ctx._raise(_lib.slm_packed_prefill_attn_planned(ctx._h, plan, *args), "slm_packed_prefill_attn_planned")
    return out


def slm_gather_last(ctx: Context, hidden, cu_seqlens, out=None) -> torch.Tensor:
    """hidden [T,H] (bf16 or fp32) -> out [B,H], the last valid row of each sequence."""
    dev = ctx.device
    T, H = hidden.shape
    B = cu_seqlens.numel() - 1
    dt = {torch.bfloat16: SLM_BF16, torch.float32: SLM_F32}.get(hidden.dtype)
    if dt is None:
        raise TypeError("hidden must be bfloat16 or float32")
    if out is None:
        out = torch.empty((B, H), dtype=hidden.dtype, device=dev)
    if out.shape != (B, H) or out.dtype != hidden.dtype:
        raise ValueError("out must be [B, H] of hidden's dtype")
    ctx._stream()
    rc = _lib.slm_gather_last(ctx._h, _ptr(hidden, "hidden", (hidden.dtype,), dev),
                              _ptr(cu_seqlens, "cu_seqlens", (torch.int32,), dev), B, T, H, dt,
                              _ptr(out, "out", (hidden.dtype,), dev))
    ctx._raise(rc, "slm_gather_last")
    return out


def slm_beam_decode_attn(ctx: Context, q, prefix_k, prefix_v, suffix_k_in, suffix_v_in, k_new, v_new,
                         parent, hist_len: int, suffix_k_out, suffix_v_out, out=None,
                         scale: Optional[float] = None, out_dtype=torch.float32, prompt_cu=None,
                         prompt_len: Optional[int] = None) -> torch.Tensor:
    """One decode step over all layers.  q [NL,R,W,Hq,D]; prefix_k/v
    [NL,R,P,Hkv,D], or with prompt_cu ([R+1] int32 offsets on the device)
    prompts of different lengths packed per layer as [NL,prompt_cu[R],Hkv,D]
    with prompt_len their longest length (read from prompt_cu when None);
    suffix_*_in/out [NL,R,W,S_cap,Hkv,D]; k_new/v_new [NL,R,W,Hkv,D]; parent
    [R,W] int32 or None.  Returns out [NL,R,W,Hq,D]."""
    dev = ctx.device
    NL, R, W, Hq, D = q.shape
    S_cap = suffix_k_out.shape[3]
    if prompt_cu is None:
        P, Hkv = prefix_k.shape[2], prefix_k.shape[3]
        rows = R * P
        if prefix_k.shape != (NL, R, P, Hkv, D) or prefix_v.shape != prefix_k.shape:
            raise ValueError("prefix_k/v must be [NL,R,P,Hkv,D]")
    else:
        rows, Hkv = prefix_k.shape[1], prefix_k.shape[2]
        if tuple(prompt_cu.shape) != (R + 1,):
            raise ValueError("prompt_cu must be [R+1]")
        if prompt_len is None:
            raise ValueError("prompt_len (the longest prompt) is required with prompt_cu: reading it from the "
                             "device offsets would synchronise the stream")
        P = int(prompt_len)
        if prefix_k.shape != (NL, rows, Hkv, D) or prefix_v.shape != prefix_k.shape:
            raise ValueError("packed prefix_k/v must be [NL,prompt_cu[R],Hkv,D]")
    if k_new.shape != (NL, R, W, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [NL,R,W,Hkv,D]")
    sshape = (NL, R, W, S_cap, Hkv, D)
    for name, t in (("suffix_k_out", suffix_k_out), ("suffix_v_out", suffix_v_out),
                    ("suffix_k_in", suffix_k_in), ("suffix_v_in", suffix_v_in)):
        if t is not None and tuple(t.shape) != sshape:
            raise ValueError("%s must be %s" % (name, sshape))
    if parent is not None and tuple(parent.shape) != (R, W):
        raise ValueError("parent must be [R, W]")
    if out is None:
        out = torch.empty((NL, R, W, Hq, D), dtype=out_dtype, device=dev)
    if tuple(out.shape) != (NL, R, W, Hq, D) or out.dtype not in _OUT:
        raise ValueError("out must be [NL,R,W,Hq,D] float32 or bfloat16")
    a = _BeamAttnArgs()
    a.n_layers, a.num_requests, a.width, a.prompt_len = NL, R, W, P
    a.hist_len, a.suffix_cap, a.n_heads_q, a.n_heads_kv, a.head_dim = int(hist_len), S_cap, Hq, Hkv, D
    a.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    a.q = _ptr(q, "q", _BF16, dev)
    a.prefix_k, a.prefix_v = _ptr(prefix_k, "prefix_k", _BF16, dev), _ptr(prefix_v, "prefix_v", _BF16, dev)
    a.suffix_k_in = _ptr(suffix_k_in, "suffix_k_in", _BF16, dev)
    a.suffix_v_in = _ptr(suffix_v_in, "suffix_v_in", _BF16, dev)
    a.k_new, a.v_new = _ptr(k_new, "k_new", _BF16, dev), _ptr(v_new, "v_new", _BF16, dev)
    a.parent = _ptr(parent, "parent", (torch.int32,), dev)
    a.suffix_k_out = _ptr(suffix_k_out, "suffix_k_out", _BF16, dev)
    a.suffix_v_out = _ptr(suffix_v_out, "suffix_v_out", _BF16, dev)
    a.out, a.out_dtype = _ptr(out, "out", tuple(_OUT), dev), _OUT[out.dtype]
    a.prompt_cu = _ptr(prompt_cu, "prompt_cu", (torch.int32,), dev)
    a.prompt_rows = rows
    ctx._stream()
    ctx._raise(_lib.slm_beam_decode_attn(ctx._h, ctypes.byref(a)), "slm_beam_decode_attn")
    return out


def slm_beam_topk_merge(ctx: Context, logprobs, cum, width: int, tokens=None, parent=None, cum_out=None):
    """logprobs [R,Win,V] fp32, cum [R,Win] fp32 -> (tokens, parent, cum_out), each [R,W]."""
    dev = ctx.device
    R, Win, V = logprobs.shape
    if tuple(cum.shape) != (R, Win):
        raise ValueError("cum must be [R, Win]")
    W = int(width)
    tokens = torch.empty((R, W), dtype=torch.int32, device=dev) if tokens is None else tokens
    parent = torch.empty((R, W), dtype=torch.int32, device=dev) if parent is None else parent
    cum_out = torch.empty((R, W), dtype=torch.float32, device=dev) if cum_out is None else cum_out
    for name, t in (("tokens", tokens), ("parent", parent), ("cum_out", cum_out)):
        if tuple(t.shape) != (R, W):
            raise ValueError("%s must be [R, W]" % name)
    ctx._stream()
    rc = _lib.slm_beam_topk_merge(
        ctx._h, _ptr(logprobs, "logprobs", (torch.float32,), dev), _ptr(cum, "cum", (torch.float32,), dev),
        R, Win, V, W, _ptr(tokens, "tokens", (torch.int32,), dev), _ptr(parent, "parent", (torch.int32,), dev),
        _ptr(cum_out, "cum_out", (torch.float32,), dev))
    ctx._raise(rc, "slm_beam_topk_merge")
    return tokens, parent, cum_out


def slm_beam_topk_merge_logits(ctx: Context, logits, cum, width: int, tokens=None, parent=None, cum_out=None,
                               lse_out=None):
    """logits [R,Win,V] fp32 or bf16, cum [R,Win] fp32 -> (tokens, parent, cum_out) [R,W]; lse_out
    [R,Win] fp32 (optional) receives each row's log-sum-exp."""
    dev = ctx.device
    R, Win, V = logits.shape
    if tuple(cum.shape) != (R, Win):
        raise ValueError("cum must be [R, Win]")
    if lse_out is not None and tuple(lse_out.shape) != (R, Win):
        raise ValueError("lse_out must be [R, Win]")
    W = int(width)
    tokens = torch.empty((R, W), dtype=torch.int32, device=dev) if tokens is None else tokens
    parent = torch.empty((R, W), dtype=torch.int32, device=dev) if parent is None else parent
    cum_out = torch.empty((R, W), dtype=torch.float32, device=dev) if cum_out is None else cum_out
    for name, t in (("tokens", tokens), ("parent", parent), ("cum_out", cum_out)):
        if tuple(t.shape) != (R, W):
            raise ValueError("%s must be [R, W]" % name)
    ctx._stream()
    rc = _lib.slm_beam_topk_merge_logits(
        ctx._h, _ptr(logits, "logits", (torch.float32, torch.bfloat16), dev),
        SLM_BF16 if logits.dtype == torch.bfloat16 else SLM_F32, _ptr(cum, "cum", (torch.float32,), dev),
        R, Win, V, W, _ptr(tokens, "tokens", (torch.int32,), dev), _ptr(parent, "parent", (torch.int32,), dev),
        _ptr(cum_out, "cum_out", (torch.float32,), dev),
        None if lse_out is None else _ptr(lse_out, "lse_out", (torch.float32,), dev))
    ctx._raise(rc, "slm_beam_topk_merge_logits")
    return tokens, parent, cum_out


def slm_beam_reorder_suffix(ctx: Context, parent, k_in, v_in, rows: int, k_out, v_out):
    """k_out[l,r,j,i] = k_in[l,r,parent[r,j],i] for i < rows (and V)."""
    dev = ctx.device
    NL, R, W, S_cap, Hkv, D = k_in.shape
    for name, t in (("v_in", v_in), ("k_out", k_out), ("v_out", v_out)):
        if t.shape != k_in.shape:
            raise ValueError("%s must match k_in's shape" % name)
    if tuple(parent.shape) != (R, W):
        raise ValueError("parent must be [R, W] = %s" % ((R, W),))
    ctx._stream()
    rc = _lib.slm_beam_reorder_suffix(
        ctx._h, NL, R, W, int(rows), S_cap, Hkv, D, _ptr(parent, "parent", (torch.int32,), dev),
        _ptr(k_in, "k_in", _BF16, dev), _ptr(v_in, "v_in", _BF16, dev), _ptr(k_out, "k_out", _BF16, dev),
        _ptr(v_out, "v_out", _BF16, dev))
    ctx._raise(rc, "slm_beam_reorder_suffix")
    return k_out, v_out


def slm_label_head(ctx: Context, hidden, cu_seqlens, lm_head, labels, k: int, label_map=None, probs: bool = True,
                   out=None):
    """hidden [T,H] bf16, cu_seqlens [B+1] int32, lm_head [V,H] bf16, labels [L] int32, optional
    label_map [L] int32 -> (logits [B,L] f32, probs [B,L] f32 or None, top_idx [B,K] int32,
    top_prob [B,K] f32, top_class [B,K] int32).  ``out`` may hold those five tensors."""
    dev = ctx.device
    T, H = hidden.shape
    V = lm_head.shape[0]
    if lm_head.shape[1] != H:
        raise ValueError("lm_head must be [V, H] with the hidden size of hidden")
    B, L, K = cu_seqlens.numel() - 1, labels.numel(), int(k)
    if out is None:
        out = (torch.empty((B, L), dtype=torch.float32, device=dev),
               torch.empty((B, L), dtype=torch.float32, device=dev) if probs else None,
               torch.empty((B, K), dtype=torch.int32, device=dev),
               torch.empty((B, K), dtype=torch.float32, device=dev),
               torch.empty((B, K), dtype=torch.int32, device=dev))
    lg, pr, ti, tp, tc = out
    if label_map is not None and label_map.numel() != L:
        raise ValueError("label_map must hold one class per label (%d)" % L)
    for name, t, shp in (("logits", lg, (B, L)), ("probs", pr, (B, L)), ("top_idx", ti, (B, K)),
                         ("top_prob", tp, (B, K)), ("top_class", tc, (B, K))):
        if t is not None and tuple(t.shape) != shp:
            raise ValueError("%s must be %s" % (name, shp))
    if lg is None or ti is None or tp is None:
        raise ValueError("logits, top_idx and top_prob are required outputs")
    ctx._stream()
    rc = _lib.slm_label_head(
        ctx._h, _ptr(hidden, "hidden", _BF16, dev), _ptr(cu_seqlens, "cu_seqlens", (torch.int32,), dev), B, T, H,
        _ptr(lm_head, "lm_head", _BF16, dev), V, _ptr(labels, "labels", (torch.int32,), dev), L, K,
        _ptr(label_map, "label_map", (torch.int32,), dev), _ptr(lg, "logits", (torch.float32,), dev),
        _ptr(pr, "probs", (torch.float32,), dev), _ptr(ti, "top_idx", (torch.int32,), dev),
        _ptr(tp, "top_prob", (torch.float32,), dev), _ptr(tc, "top_class", (torch.int32,), dev))
    ctx._raise(rc, "slm_label_head")
    return lg, pr, ti, tp, tc


def slm_beam_backtrack(ctx: Context, tokens, parent, out=None) -> torch.Tensor:
    """tokens, parent [n_merges,R,W] int32 (the merges' outputs in order) -> sequences [R,W,n_merges] int32:
    the token each final beam's ancestor took at every merge."""
    dev = ctx.device
    if tokens.dim() != 3 or tuple(parent.shape) != tuple(tokens.shape):
        raise ValueError("tokens and parent must both be [n_merges, R, W]")
    n, R, W = tokens.shape
    out = torch.empty((R, W, n), dtype=torch.int32, device=dev) if out is None else out
    if tuple(out.shape) != (R, W, n):
        raise ValueError("out must be [R, W, n_merges]")
    ctx._stream()
    rc = _lib.slm_beam_backtrack(ctx._h, _ptr(tokens, "tokens", (torch.int32,), dev),
                                 _ptr(parent, "parent", (torch.int32,), dev), n, R, W,
                                 _ptr(out, "out", (torch.int32,), dev))
    ctx._raise(rc, "slm_beam_backtrack")
    return out


def slm_beam_search(ctx: Context, state: dict, prefix_k, prefix_v, logprobs, q, k_new, v_new, scale=None,
                    prompt_cu=None, prompt_len: Optional[int] = None):
    """The whole fixed-step search in one call.  logprobs: n_steps + 1 tensors ([R,1,V], then [R,W,V]);
    q, k_new, v_new: n_steps tensors ([NL,R,W,Hq,D], [NL,R,W,Hkv,D]); prefix_k/v as for
    slm_beam_decode_attn; state: from Context.beam_search_state (written in place).
    Returns (tokens, parent, cum, sequences) of the state."""
    dev = ctx.device
    N = len(q)
    if len(logprobs) != N + 1 or len(k_new) != N or len(v_new) != N or len(state["attn_out"]) != N:
        raise ValueError("need n_steps + 1 log-prob tensors and n_steps q, k_new, v_new and attention outputs")
    tokens, parent, cum, seq, cum0 = (state[k] for k in ("tokens", "parent", "cum", "sequences", "cum0"))
    Np1, R, W = tokens.shape
    if Np1 != N + 1 or tuple(parent.shape) != (Np1, R, W) or tuple(cum.shape) != (Np1, R, W):
        raise ValueError("tokens, parent and cum must be [n_steps + 1, R, W]")
    if seq is not None and tuple(seq.shape) != (R, W, Np1):
        raise ValueError("sequences must be [R, W, n_steps + 1]")
    if tuple(cum0.shape) != (R,):
        raise ValueError("cum0 must be [R]")
    V = logprobs[0].shape[-1]
    for t, lp in enumerate(logprobs):
        if tuple(lp.shape) != (R, 1 if t == 0 else W, V):
            raise ValueError("logprobs[%d] must be [R, %s, V]" % (t, "1" if t == 0 else "W"))
    D = prefix_k.shape[-1]
    Hkv = prefix_k.shape[-2]
    if N:
        NL, _, _, Hq, _ = q[0].shape
    else:
        NL, Hq = prefix_k.shape[0], Hkv
    if prompt_cu is None:
        P = prefix_k.shape[2]
        rows = R * P
        if tuple(prefix_k.shape) != (NL, R, P, Hkv, D) or prefix_v.shape != prefix_k.shape:
            raise ValueError("prefix_k/v must be [NL,R,P,Hkv,D]")
    else:
        if prompt_len is None:
            raise ValueError("prompt_len (the longest prompt) is required with prompt_cu")
        if tuple(prompt_cu.shape) != (R + 1,):
            raise ValueError("prompt_cu must be [R+1]")
        P, rows = int(prompt_len), prefix_k.shape[1]
        if tuple(prefix_k.shape) != (NL, rows, Hkv, D) or prefix_v.shape != prefix_k.shape:
            raise ValueError("packed prefix_k/v must be [NL,prompt_cu[R],Hkv,D]")
    S_cap = state["final_k"].shape[3]
    sshape = (NL, R, W, S_cap, Hkv, D)
    for name in ("final_k", "final_v"):
        if tuple(state[name].shape) != sshape:
            raise ValueError("%s must be %s" % (name, sshape))
    for name in ("suffix_k", "suffix_v"):
        if len(state[name]) != 2 or any(tuple(t.shape) != sshape for t in state[name]):
            raise ValueError("%s must be two %s buffers" % (name, sshape))
    for t in range(N):
        if tuple(q[t].shape) != (NL, R, W, Hq, D):
            raise ValueError("q[%d] must be [NL,R,W,Hq,D]" % t)
        if tuple(k_new[t].shape) != (NL, R, W, Hkv, D) or tuple(v_new[t].shape) != (NL, R, W, Hkv, D):
            raise ValueError("k_new/v_new[%d] must be [NL,R,W,Hkv,D]" % t)
        o = state["attn_out"][t]
        if tuple(o.shape) != (NL, R, W, Hq, D) or o.dtype != state["attn_out"][0].dtype:
            raise ValueError("attn_out[%d] must be [NL,R,W,Hq,D] of one dtype" % t)
    out_dtype = state["attn_out"][0].dtype if N else torch.float32
    if out_dtype not in _OUT:
        raise ValueError("attention output must be float32 or bfloat16")
    arr = lambda ts, name, dt: (ctypes.c_void_p * max(1, len(ts)))(*[_ptr(t, name, dt, dev) for t in ts])
    lp_a = arr(logprobs, "logprobs", (torch.float32,))
    q_a, kn_a, vn_a = arr(q, "q", _BF16), arr(k_new, "k_new", _BF16), arr(v_new, "v_new", _BF16)
    o_a = arr(state["attn_out"], "attn_out", tuple(_OUT))
    a = _BeamSearchArgs()
    a.n_layers, a.num_requests, a.width, a.prompt_len, a.n_steps, a.suffix_cap = NL, R, W, P, N, S_cap
    a.n_heads_q, a.n_heads_kv, a.head_dim, a.vocab = Hq, Hkv, D, V
    a.scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    a.prefix_k, a.prefix_v = _ptr(prefix_k, "prefix_k", _BF16, dev), _ptr(prefix_v, "prefix_v", _BF16, dev)
    a.prompt_cu = _ptr(prompt_cu, "prompt_cu", (torch.int32,), dev)
    a.prompt_rows = rows
    a.cum0 = _ptr(cum0, "cum0", (torch.float32,), dev)
    a.logprobs, a.q, a.k_new, a.v_new, a.attn_out = (ctypes.cast(x, ctypes.c_void_p) for x in (lp_a, q_a, kn_a,
                                                                                               vn_a, o_a))
    for i in range(2):
        a.suffix_k[i] = _ptr(state["suffix_k"][i], "suffix_k", _BF16, dev)
        a.suffix_v[i] = _ptr(state["suffix_v"][i], "suffix_v", _BF16, dev)
    a.final_k, a.final_v = _ptr(state["final_k"], "final_k", _BF16, dev), _ptr(state["final_v"], "final_v", _BF16, dev)
    a.out_dtype = _OUT[out_dtype]
    a.tokens, a.parent = _ptr(tokens, "tokens", (torch.int32,), dev), _ptr(parent, "parent", (torch.int32,), dev)
    a.cum = _ptr(cum, "cum", (torch.float32,), dev)
    a.sequences = _ptr(seq, "sequences", (torch.int32,), dev)
    ctx._stream()
    ctx._raise(_lib.slm_beam_search(ctx._h, ctypes.byref(a)), "slm_beam_search")
    return tokens, parent, cum, seq


def slm_packed_prefill_attn_noalloc(q, k, v, cu_seqlens, max_seqlen: int, scale: Optional[float] = None,
                                    out: Optional[torch.Tensor] = None, out_dtype=torch.float32,
                                    err_flag: Optional[torch.Tensor] = None) -> torch.Tensor:
    """slm_packed_prefill_attn without a context and without any allocation in
    the library (its scratch memory is a static array of the device): on q's
    device and torch's current stream.  Pass ``out`` to allocate nothing at
    all; ``err_flag`` (one int32 on the device, zeroed by the caller) receives
    a nonzero code when cu_seqlens breaks the caller guarantees."""
    if not isinstance(q, torch.Tensor) or q.device.type != "cuda":
        raise ValueError("q must be a device tensor")
    dev = q.device
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (T, Hkv, D) or v.shape != (T, Hkv, D):
        raise ValueError("k and v must be [T, Hkv, D] matching q")
    if out is None:
        out = torch.empty((T, Hq, D), dtype=out_dtype, device=dev)
    if out.shape != (T, Hq, D) or out.dtype not in _OUT:
        raise ValueError("out must be [T, Hq, D] float32 or bfloat16")
    if err_flag is not None and (err_flag.numel() != 1 or err_flag.dtype != torch.int32):
        raise ValueError("err_flag must be one int32")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = _lib.slm_packed_prefill_attn_noalloc(
            _P(stream), _ptr(q, "q", _BF16, dev), _ptr(k, "k", _BF16, dev), _ptr(v, "v", _BF16, dev),
            _ptr(cu_seqlens, "cu_seqlens", (torch.int32,), dev), cu_seqlens.numel() - 1, T, int(max_seqlen), Hq, Hkv,
            D, scale, _ptr(out, "out", tuple(_OUT), dev), _OUT[out.dtype], _ptr(err_flag, "err_flag", (torch.int32,), dev))
    if rc != SLM_OK:
        raise SlmError(rc, "slm_packed_prefill_attn_noalloc (a pack's work list holds T*Hq/128 + B*Hq <= 262144 "
                           "entries)")
    return out
