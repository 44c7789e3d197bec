"""Seeded synthetic inputs for the bounded-generation attention hot path.

This module is shared by the oracle side and the HIP side *only* as a source
of input arrays.  It holds none of the method's arithmetic: it draws random
numbers, rounds them to bf16 storage, and turns normal logits into log-probs
(the upstream model's job, not the hot path's).

Workload shapes follow the page "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化"
(abstract and §1.2): prefill-only requests of 15 samples with inputs under
500 tokens, and beam search with a fixed width (about 100, at most 400) and a
fixed number of decode steps (4 or 5).  Heads and sizes are those of the five
workloads below; the pages name no public dataset, so every tensor is drawn
from a seeded generator.

Two generator backends exist:
  * numpy (``np.random.default_rng([base, tensor_id, layer, step])``, PCG64),
    used for every input that the CPU oracle checks;
  * torch on a device (``torch.Generator(device).manual_seed(...)``, Philox),
    used only for bench-scale inputs that would take minutes to draw on the
    host.  Parity at those sizes copies the same device arrays back to the
    host for the oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

# tensor ids of the seed tuple ``[base_seed, tensor_id, layer, step]``
TID_Q, TID_K, TID_V, TID_HIDDEN = 1, 2, 3, 4
TID_PREFIX_K, TID_PREFIX_V, TID_K_NEW, TID_V_NEW, TID_LOGITS = 5, 6, 7, 8, 9
TID_SUFFIX_K, TID_SUFFIX_V = 10, 11
TID_LM_HEAD, TID_LABELS = 12, 13


@dataclasses.dataclass(frozen=True)
class PrefillShape:
    """A packed prefill workload: ``B`` sequences of lengths ``lengths``."""
    name: str
    base_seed: int
    lengths: tuple
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    n_layers: int = 1
    hidden_dim: int = 0          # 0: no last-token gather in this workload

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def max_seqlen(self) -> int:
        return int(max(self.lengths)) if self.lengths else 0

    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(len(self.lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(np.asarray(self.lengths, dtype=np.int64))
        return cu


@dataclasses.dataclass(frozen=True)
class BeamShape:
    """A fixed-width, fixed-step beam-search workload."""
    name: str
    base_seed: int
    num_requests: int
    width: int
    prompt_len: int
    n_steps: int
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    n_layers: int
    vocab: int

    @property
    def suffix_cap(self) -> int:
        # at decode step t the suffix holds t rows; the cap is the last step's
        return self.n_steps


def uniform_lengths(base_seed: int, n: int, lo: int = 64, hi: int = 500) -> tuple:
    """Sequence lengths uniform on [lo, hi] (inclusive), seeded."""
    rng = np.random.default_rng(base_seed)
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=n))


# -- the five workloads --------------------------------------------------------
TINY_PREFILL = PrefillShape("tiny_prefill", 1001, (7, 33, 64, 129), 4, 2, 64)
# tiny beam step: 4 beams over a 1,000-word vocabulary; R=2 requests, a 33-token
# prompt and 2 layers are this build's choice (the workload fixes only W and V)
TINY_BEAM = BeamShape("tiny_beam", 1001, num_requests=2, width=4, prompt_len=33,
                      n_steps=4, n_heads_q=4, n_heads_kv=2, head_dim=64,
                      n_layers=2, vocab=1000)
PREFILL_REQUEST = PrefillShape("prefill_request", 1002, uniform_lengths(1002, 15),
                               16, 8, 128, n_layers=1, hidden_dim=1024)
PREFILL_THROUGHPUT = PrefillShape("prefill_throughput", 1003, uniform_lengths(1003, 960),
                                  16, 8, 128, n_layers=28, hidden_dim=1024)
BEAM_SHORT = BeamShape("beam_short_prompt", 1004, num_requests=32, width=100,
                       prompt_len=128, n_steps=4, n_heads_q=14, n_heads_kv=2,
                       head_dim=64, n_layers=24, vocab=151936)
BEAM_LONG = BeamShape("beam_long_prompt", 1005, num_requests=8, width=400,
                      prompt_len=480, n_steps=5, n_heads_q=14, n_heads_kv=2,
                      head_dim=64, n_layers=24, vocab=151936)

ALL: Dict[str, object] = {s.name: s for s in (TINY_PREFILL, TINY_BEAM, PREFILL_REQUEST,
                                              PREFILL_THROUGHPUT, BEAM_SHORT, BEAM_LONG)}


# -- numpy backend ------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 storage (round to nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(base: int, tid: int, layer: int = 0, step: int = 0) -> np.random.Generator:
    return np.random.default_rng([base, tid, layer, step])


def normal_bf16(base: int, tid: int, shape: Sequence[int], layer: int = 0,
                step: int = 0) -> np.ndarray:
    """bf16 bits of N(0,1) float32 draws."""
    x = _rng(base, tid, layer, step).standard_normal(tuple(shape), dtype=np.float32)
    return f32_to_bf16_bits(x)


def logits(base: int, shape: Sequence[int], step: int = 0) -> np.ndarray:
    """fp32 N(0,1) logits: the draw the log-probs below are made from."""
    return _rng(base, TID_LOGITS, 0, step).standard_normal(tuple(shape), dtype=np.float32)


def logprobs(base: int, shape: Sequence[int], step: int = 0) -> np.ndarray:
    """fp32 log-probs: N(0,1) fp32 logits, log-softmax over the last axis in
    fp64, one rounding to fp32."""
    z = _rng(base, TID_LOGITS, 0, step).standard_normal(tuple(shape), dtype=np.float32)
    z = z.astype(np.float64)
    m = z.max(axis=-1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True))
    return (z - lse).astype(np.float32)


def prefill_inputs(shape: PrefillShape, layer: int = 0) -> dict:
    """q [T,Hq,D], k/v [T,Hkv,D] as bf16 bits, cu_seqlens [B+1] int32."""
    T, D = shape.total_tokens, shape.head_dim
    out = dict(
        q=normal_bf16(shape.base_seed, TID_Q, (T, shape.n_heads_q, D), layer),
        k=normal_bf16(shape.base_seed, TID_K, (T, shape.n_heads_kv, D), layer),
        v=normal_bf16(shape.base_seed, TID_V, (T, shape.n_heads_kv, D), layer),
        cu_seqlens=shape.cu_seqlens(),
    )
    if shape.hidden_dim:
        out["hidden"] = normal_bf16(shape.base_seed, TID_HIDDEN, (T, shape.hidden_dim), layer)
    return out


def beam_static_inputs(shape: BeamShape, layers: Optional[Sequence[int]] = None) -> dict:
    """Prompt K/V ``[NL,R,P,Hkv,D]`` (bf16 bits) for the listed layers."""
    layers = list(range(shape.n_layers)) if layers is None else list(layers)
    R, P, Hkv, D = shape.num_requests, shape.prompt_len, shape.n_heads_kv, shape.head_dim
    pk = np.stack([normal_bf16(shape.base_seed, TID_PREFIX_K, (R, P, Hkv, D), l) for l in layers])
    pv = np.stack([normal_bf16(shape.base_seed, TID_PREFIX_V, (R, P, Hkv, D), l) for l in layers])
    return dict(prefix_k=pk, prefix_v=pv)


def beam_step_inputs(shape: BeamShape, step: int, layers: Optional[Sequence[int]] = None) -> dict:
    """Per decode step ``step`` (1-based): q ``[NL,R,W,Hq,D]``, k_new/v_new
    ``[NL,R,W,Hkv,D]`` (bf16 bits) and log-probs ``[R,W,V]`` (fp32)."""
    layers = list(range(shape.n_layers)) if layers is None else list(layers)
    R, W, D = shape.num_requests, shape.width, shape.head_dim
    Hq, Hkv = shape.n_heads_q, shape.n_heads_kv
    q = np.stack([normal_bf16(shape.base_seed, TID_Q, (R, W, Hq, D), l, step) for l in layers])
    kn = np.stack([normal_bf16(shape.base_seed, TID_K_NEW, (R, W, Hkv, D), l, step) for l in layers])
    vn = np.stack([normal_bf16(shape.base_seed, TID_V_NEW, (R, W, Hkv, D), l, step) for l in layers])
    return dict(q=q, k_new=kn, v_new=vn)


def beam_logprobs(shape: BeamShape, step: int) -> np.ndarray:
    """Log-probs for the merge after decode step ``step``; step 0 is the
    prefill's, one row per request (``[R,1,V]``), later steps ``[R,W,V]``."""
    win = 1 if step == 0 else shape.width
    return logprobs(shape.base_seed, (shape.num_requests, win, shape.vocab), step)


# -- label head (prefill-only mode): synthetic LM-head rows and label ids -------
LABEL_COUNT, LABEL_TOP_K = 64, 5


def lm_head_rows(base: int, vocab: int, hidden_dim: int) -> np.ndarray:
    """bf16 LM-head rows [V, H]: N(0,1) / sqrt(H), so a unit-variance hidden
    row gives unit-variance logits."""
    x = _rng(base, TID_LM_HEAD).standard_normal((vocab, hidden_dim), dtype=np.float32)
    return f32_to_bf16_bits((x / np.float32(np.sqrt(hidden_dim))).astype(np.float32))


def label_ids(base: int, vocab: int, n: int = LABEL_COUNT) -> np.ndarray:
    """n distinct token ids in [0, vocab)."""
    return _rng(base, TID_LABELS).choice(vocab, size=n, replace=False).astype(np.int32)


# -- torch device backend (bench-scale inputs) -----------------------------------
def torch_normal_bf16(shape, seed_tuple, device):
    """bf16 N(0,1) tensor drawn on ``device`` (Philox), seeded by a tuple."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_fold_seed(seed_tuple))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)   # round to nearest even


def torch_logits(shape, seed_tuple, device):
    """fp32 N(0,1) logits drawn on ``device`` (the draw torch_logprobs normalises)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_fold_seed(seed_tuple))
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)


def torch_logprobs(shape, seed_tuple, device):
    """fp32 log-probs of N(0,1) logits (log-softmax in fp64), drawn on ``device``."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_fold_seed(seed_tuple))
    z = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    out = torch.empty(tuple(shape), device=device, dtype=torch.float32)
    # row blocks keep the fp64 temporary small
    flat_z, flat_o = z.view(-1, shape[-1]), out.view(-1, shape[-1])
    for i in range(0, flat_z.shape[0], 256):
        flat_o[i:i + 256] = torch.log_softmax(flat_z[i:i + 256].double(), dim=-1).float()
    del z
    return out


def torch_beam_inputs(shape: BeamShape, device) -> dict:
    """Device-drawn inputs of one fixed-step search of ``shape``: prompt K/V
    ``[NL,R,P,Hkv,D]``, per decode step t = 1..N the q ``[NL,R,W,Hq,D]`` and
    k_new/v_new ``[NL,R,W,Hkv,D]`` (lists indexed t-1), and the log-probs of
    the N+1 merges (``[R,1,V]``, then ``[R,W,V]``)."""
    NL, R, W, P, N, V = shape.n_layers, shape.num_requests, shape.width, shape.prompt_len, shape.n_steps, shape.vocab
    Hq, Hkv, D, b = shape.n_heads_q, shape.n_heads_kv, shape.head_dim, shape.base_seed
    steps = range(1, N + 1)
    return dict(
        prefix_k=torch_normal_bf16((NL, R, P, Hkv, D), (b, TID_PREFIX_K, 0, 0), device),
        prefix_v=torch_normal_bf16((NL, R, P, Hkv, D), (b, TID_PREFIX_V, 0, 0), device),
        q=[torch_normal_bf16((NL, R, W, Hq, D), (b, TID_Q, 0, t), device) for t in steps],
        k_new=[torch_normal_bf16((NL, R, W, Hkv, D), (b, TID_K_NEW, 0, t), device) for t in steps],
        v_new=[torch_normal_bf16((NL, R, W, Hkv, D), (b, TID_V_NEW, 0, t), device) for t in steps],
        logprobs=[torch_logprobs((R, 1 if t == 0 else W, V), (b, TID_LOGITS, 0, t), device) for t in range(N + 1)])


def _fold_seed(seed_tuple) -> int:
    """Fold a seed tuple into one 63-bit torch seed (SplitMix64 steps)."""
    h = 0x9E3779B97F4A7C15
    for s in seed_tuple:
        h = (h ^ (int(s) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        h = (h + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = h
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        h = z ^ (z >> 31)
    return h & 0x7FFFFFFFFFFFFFFF
