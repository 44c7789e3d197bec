"""Property tests of the C ABI's host-side validation on a dry-run context
(which validates and launches nothing, so no pointer is ever dereferenced):
random sizes (negative, zero, small, huge), random pointers (NULL, aligned,
misaligned, overlapping) and dtypes never crash a call, every call returns a
defined status, and the clearly invalid ones (a negative size, a NULL tensor
that the sizes require) are never accepted."""
import ctypes

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import bounded_generation_slm_amd as slm

L = slm._lib
STATUSES = set(range(7))
SETTINGS = settings(max_examples=150, deadline=None, derandomize=True, database=None,   # same examples every run
                    suppress_health_check=[HealthCheck.function_scoped_fixture])

sizes = st.one_of(st.integers(-3, 3), st.integers(0, 600), st.sampled_from([64, 128, 151936, 1 << 20, 2**31 - 1]))
small = st.integers(-2, 40)
# far-apart aligned regions, a misaligned one, and one inside another region (overlap)
ptrs = st.sampled_from([0, 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x10000004, 0x10000100])
dtypes = st.sampled_from([0, 1, 7])


@pytest.fixture(scope="module")
def h():
    ctx = slm.Context(device=-1)
    yield ctx._h
    del ctx


def _ok(rc):
    assert rc in STATUSES
    return rc == 0


@SETTINGS
@given(p=st.lists(ptrs, min_size=5, max_size=5), B=sizes, T=sizes, ms=sizes, hq=small, hkv=small,
       d=st.sampled_from([0, 64, 96, 128]), scale=st.sampled_from([0.125, 0.0, -1.0, float("nan")]), od=dtypes)
def test_prefill(h, p, B, T, ms, hq, hkv, d, scale, od):
    ok = _ok(L.slm_packed_prefill_attn(h, p[0], p[1], p[2], p[3], B, T, ms, hq, hkv, d, scale, p[4], od))
    if min(B, T, ms) < 0 or hq <= 0 or hkv <= 0:
        assert not ok
    if ok and B > 0 and T > 0:
        assert all(p[i] for i in (0, 1, 2, 3, 4)) and ms > 0
    plan = ctypes.c_uint64(0)
    pok = _ok(L.slm_prefill_plan(h, p[3], B, T, ms, hq, hkv, d, ctypes.byref(plan)))
    if min(B, T, ms) < 0:
        assert not pok
    if pok:
        _ok(L.slm_packed_prefill_attn_planned(h, plan.value, p[0], p[1], p[2], p[3], B, T, ms, hq, hkv, d, scale,
                                              p[4], od))
        assert not _ok(L.slm_packed_prefill_attn_planned(h, plan.value + 1, p[0], p[1], p[2], p[3], B, T, ms, hq,
                                                         hkv, d, scale, p[4], od))


@SETTINGS
@given(p=st.lists(ptrs, min_size=3, max_size=3), B=sizes, T=sizes, H=sizes, dt=dtypes)
def test_gather(h, p, B, T, H, dt):
    ok = _ok(L.slm_gather_last(h, p[0], p[1], B, T, H, dt, p[2]))
    if min(B, T) < 0 or H <= 0:
        assert not ok


@SETTINGS
@given(p=st.lists(ptrs, min_size=5, max_size=5), R=small, Win=small, V=sizes, W=st.integers(-1, 600))
def test_topk(h, p, R, Win, V, W):
    ok = _ok(L.slm_beam_topk_merge(h, p[0], p[1], R, Win, V, W, p[2], p[3], p[4]))
    if R < 0 or min(Win, V, W) <= 0 or W > 512:                      # zero requests: a valid no-op
        assert not ok
    if ok and R > 0:
        assert all(p)
    ok2 = _ok(L.slm_beam_topk_merge_logits(h, p[0], W % 3, p[1], R, Win, V, W, p[2], p[3], p[4], 0))
    if R < 0 or min(Win, V, W) <= 0 or W > 512:
        assert not ok2


@SETTINGS
@given(p=st.lists(ptrs, min_size=5, max_size=5), NL=small, R=small, W=small, rows=small, S=small, hkv=small,
       d=st.sampled_from([0, 8, 64, 100]))
def test_reorder(h, p, NL, R, W, rows, S, hkv, d):
    ok = _ok(L.slm_beam_reorder_suffix(h, NL, R, W, rows, S, hkv, d, p[0], p[1], p[2], p[3], p[4]))
    if min(NL, R, W, S, hkv, d) <= 0 or rows < 0 or rows > S:
        assert not ok


@SETTINGS
@given(p=st.lists(ptrs, min_size=3, max_size=3), n=small, R=small, W=small)
def test_backtrack(h, p, n, R, W):
    ok = _ok(L.slm_beam_backtrack(h, p[0], p[1], n, R, W, p[2]))
    if min(R, W, n) < 0:
        assert not ok


@SETTINGS
@given(p=st.lists(ptrs, min_size=13, max_size=13), v=st.lists(small, min_size=9, max_size=9),
       d=st.sampled_from([0, 64, 128]), od=dtypes)
def test_decode(h, p, v, d, od):
    a = slm._BeamAttnArgs()
    (a.n_layers, a.num_requests, a.width, a.prompt_len, a.hist_len, a.suffix_cap, a.n_heads_q, a.n_heads_kv,
     _) = v
    a.head_dim, a.scale, a.out_dtype = d, 0.125, od
    (a.q, a.prefix_k, a.prefix_v, a.suffix_k_in, a.suffix_v_in, a.k_new, a.v_new, a.parent, a.suffix_k_out,
     a.suffix_v_out, a.out, a.prompt_cu) = [x or None for x in p[:12]]
    a.prompt_rows = v[8]
    ok = _ok(L.slm_beam_decode_attn(h, ctypes.byref(a)))
    if min(v[:3]) <= 0 or v[3] < 0 or v[4] < 0 or v[5] <= 0 or v[4] + 1 > v[5]:
        assert not ok


def _host_array(n, fill):
    """A host array of n device addresses (the per-step pointer arrays are
    read on the host, so they must be real host memory of the documented
    length; the addresses in them are never dereferenced on a dry run)."""
    arr = (ctypes.c_void_p * max(n, 1))(*([fill or None] * max(n, 1)))
    return arr, ctypes.cast(arr, ctypes.c_void_p).value


@SETTINGS
@given(p=st.lists(ptrs, min_size=20, max_size=20), v=st.lists(small, min_size=10, max_size=10), od=dtypes,
       present=st.lists(st.booleans(), min_size=5, max_size=5))
def test_beam_search(h, p, v, od, present):
    a = slm._BeamSearchArgs()
    (a.n_layers, a.num_requests, a.width, a.prompt_len, a.n_steps, a.suffix_cap, a.n_heads_q, a.n_heads_kv,
     a.head_dim, a.vocab) = v
    a.scale, a.out_dtype = 0.125, od
    a.prefix_k, a.prefix_v, a.prompt_cu = (x or None for x in p[0:3])
    a.cum0 = p[3] or None
    keep = []                                   # host arrays: logprobs has n_steps + 1 entries, the rest n_steps
    for name, n, fill, there in zip(("logprobs", "q", "k_new", "v_new"), (v[4] + 1, v[4], v[4], v[4]), p[4:8],
                                    present):
        if there:
            arr, addr = _host_array(n, fill)
            keep.append(arr)
            setattr(a, name, addr)
    a.suffix_k[0], a.suffix_k[1], a.suffix_v[0], a.suffix_v[1] = (x or None for x in p[8:12])
    a.final_k, a.final_v = (x or None for x in p[12:14])
    if present[4]:
        arr, a.attn_out = _host_array(v[4], p[14])
        keep.append(arr)
    a.tokens, a.parent, a.cum, a.sequences = (x or None for x in p[15:19])
    a.prompt_rows = p[19] % 100
    ok = _ok(L.slm_beam_search(h, ctypes.byref(a)))
    if min(a.n_layers, a.num_requests, a.width, a.vocab) <= 0 or a.n_steps < 0:
        assert not ok
