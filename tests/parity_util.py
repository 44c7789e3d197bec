"""Helpers shared by the GPU parity tests: device transfer of bf16 storage and
the attention tolerance (relative L2 <= 5e-3 and max-abs <= 2e-2 against the
fp64 oracle, per call, over the whole compared tensor)."""
import sys

import numpy as np
import torch

REL_L2 = 5e-3
MAX_ABS = 2e-2


def note(msg: str):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(device).view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_attn_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    diff = got - ref
    rel = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30)
    mab = np.abs(diff).max() if diff.size else 0.0
    assert rel <= REL_L2 and mab <= MAX_ABS, "%s: rel_l2 %.3g (<= %g), max_abs %.3g (<= %g)" % (
        what, rel, REL_L2, mab, MAX_ABS)
    return rel, mab


def assert_attn_close_chunked(got, ref: np.ndarray, what: str = "", rows: int = 8192):
    """assert_attn_close over a whole (large) tensor, a block of leading rows
    at a time: got is a device tensor, ref the fp64 oracle array."""
    assert tuple(got.shape) == ref.shape, (tuple(got.shape), ref.shape)
    num = den = 0.0
    mab = 0.0
    for i in range(0, ref.shape[0], rows):
        g = got[i:i + rows].float().cpu().numpy().astype(np.float64)
        r = ref[i:i + rows]
        assert np.all(np.isfinite(g)), what + ": non-finite output"
        d = g - r
        num += float(np.sum(d * d))
        den += float(np.sum(r * r))
        if d.size:
            mab = max(mab, float(np.abs(d).max()))
    rel = (num ** 0.5) / max(den ** 0.5, 1e-30)
    assert rel <= REL_L2 and mab <= MAX_ABS, "%s: rel_l2 %.3g (<= %g), max_abs %.3g (<= %g)" % (
        what, rel, REL_L2, mab, MAX_ABS)
    return rel, mab
