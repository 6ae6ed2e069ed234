"""Pins of the context-parallel oracle (``oracle.cp``, CPU only).

The summary (M, X) of a segment must reproduce the segment's final state from any start
(the forward is affine in its initial state), and merging the summaries of consecutive
segments must give the states the unsplit sequence has at the segment boundaries.
"""
import numpy as np
import torch

import oracle
from oracle import cp
from chunked_gated_delta_chunk_amd.synth import make_inputs


def test_affine_summary_reproduces_any_start():
    K = V = 8
    inp = make_inputs(2, 20, 2, K, V, seed=71, HV=4)
    M, X = cp.segment_map(inp.q, inp.k, inp.v, inp.g, inp.beta, scale=0.4)
    s0 = np.random.default_rng(2).standard_normal((2, 4, V, K))
    _, S = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, scale=0.4, initial_state=s0)
    np.testing.assert_allclose(S, s0 @ M + X, rtol=1e-11, atol=1e-12)


def test_merged_segments_equal_the_unsplit_sequence():
    """A sequence split at uneven points: the merged entry states equal the unsplit run's states
    at the split points, and the last one its final state."""
    K = V = 8
    T, cuts = 45, [0, 7, 20, 21, 45]
    inp = make_inputs(1, T, 1, K, V, seed=72, HV=2, initial_state=True, gate_mean=1.0)
    cu = torch.tensor(cuts, dtype=torch.int32)
    M, X = cp.segment_map(inp.q, inp.k, inp.v, inp.g, inp.beta, scale=0.3, cu_seqlens=cu)
    s_in = cp.merge(M, X, inp.initial_state[0].double().numpy())
    for r, t in enumerate(cuts[1:], start=1):
        sl = lambda x: x[:, :t].contiguous()  # noqa: E731
        _, S = oracle.recurrent_fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta), scale=0.3,
                                    initial_state=inp.initial_state)
        np.testing.assert_allclose(s_in[r], S[0], rtol=1e-10, atol=1e-12)
