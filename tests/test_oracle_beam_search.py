"""Pins of the oracle's fixed-step beam sequence (first merge on the
prefill log-probs with one beam in, then N x [decode attention, merge]):
score recurrence along parents, the suffix rows carried by the fused
history read, and step count."""
import numpy as np
import pytest

import oracle
import workloads as wl


def test_tiny_beam_sequence_invariants():
    shape = wl.TINY_BEAM
    R, W, N = shape.num_requests, shape.width, shape.n_steps
    st = wl.beam_static_inputs(shape)
    Hkv, D = shape.n_heads_kv, shape.head_dim

    def step_inputs(t):
        x = wl.beam_step_inputs(shape, t)
        # k_new rows encode (step, beam) so the carried suffix can be traced
        kn = np.zeros(x["k_new"].shape, np.float32)
        for j in range(W):
            kn[:, :, j] = 8 * t + j
        x["k_new"] = wl.f32_to_bf16_bits(kn)
        return x

    res = oracle.beam_search(step_inputs, st["prefix_k"], st["prefix_v"],
                             lambda t: wl.beam_logprobs(shape, t), W, N)
    assert len(res["tokens"]) == N + 1 and len(res["attn"]) == N
    assert np.all(res["parent"][0] == 0)
    # cum recurrence: one fp32 add along each chosen (parent, token)
    for t in range(1, N + 1):
        lp = wl.beam_logprobs(shape, t)
        for r in range(R):
            for j in range(W):
                p, tok = res["parent"][t][r, j], res["tokens"][t][r, j]
                assert res["cum"][t][r, j] == np.float32(res["cum"][t - 1][r, p] + lp[r, p, tok])
    # carried suffix rows: after the final reorder, row i of beam j holds the
    # k_new written at step i+1 by its ancestor at that step
    fk = wl.bf16_bits_to_f32(res["final_suffix_k"])
    for r in range(R):
        for j in range(W):
            anc = j
            for t in range(N, 0, -1):
                anc = res["parent"][t][r, anc]          # beam order during step t
                assert np.all(fk[:, r, j, t - 1] == 8 * t + anc)
    # the backtracked sequences agree with the rows the reorder carried: row
    # t-1 names the ancestor beam during step t (merge t-1's order), whose
    # token at merge t-1 is entry t-1 of the sequence; the last entry is the
    # final merge's own token
    seq = res["sequences"]
    assert seq.shape == (R, W, N + 1)
    for r in range(R):
        for j in range(W):
            assert seq[r, j, N] == res["tokens"][N][r, j]
            for t in range(1, N + 1):
                anc = int(fk[0, r, j, t - 1, 0, 0]) - 8 * t
                assert seq[r, j, t - 1] == res["tokens"][t - 1][r, anc]


def _forward_sequences(tokens, parent):
    """Sequences built forward, merge by merge: beam j after merge t extends
    the sequence of its parent after merge t-1 by its own token."""
    n, R, W = tokens.shape
    seqs = [[[int(tokens[0, r, j])] for j in range(W)] for r in range(R)]
    for t in range(1, n):
        seqs = [[seqs[r][int(parent[t, r, j])] + [int(tokens[t, r, j])] for j in range(W)] for r in range(R)]
    return np.array(seqs, np.int32)


def test_backtrack_matches_forward_construction():
    rng = np.random.default_rng(7)
    for n, R, W in ((1, 2, 3), (2, 1, 1), (5, 3, 6), (6, 2, 17)):
        tok = rng.integers(0, 1000, size=(n, R, W)).astype(np.int32)
        par = rng.integers(0, W, size=(n, R, W)).astype(np.int32)
        par[0] = 0
        assert np.array_equal(oracle.beam_backtrack(tok, par), _forward_sequences(tok, par))


def test_backtrack_identity_parents_and_bad_parent():
    n, R, W = 4, 2, 5
    tok = np.arange(n * R * W, dtype=np.int32).reshape(n, R, W)
    par = np.broadcast_to(np.arange(W, dtype=np.int32), (n, R, W)).copy()
    seq = oracle.beam_backtrack(tok, par)
    assert np.array_equal(seq, np.transpose(tok, (1, 2, 0)))      # no reordering: each beam keeps its own column
    par[2, 1, 3] = W                                               # outside [0, W)
    with pytest.raises(ValueError):
        oracle.beam_backtrack(tok, par)
