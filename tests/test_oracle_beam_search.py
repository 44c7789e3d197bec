"""Pins of the oracle's fixed-step beam sequence (first merge on the
prefill log-probs with one beam in, then N x [decode attention, merge]):
score recurrence along parents, the suffix rows carried by the fused
history read, and step count."""
import numpy as np

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
