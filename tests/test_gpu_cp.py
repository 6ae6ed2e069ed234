"""Context parallelism on one device: segment summaries and their merge, through the C interface.

A sequence is split into segments as a varlen batch; chunk_dr_segment_map gives each segment's
(M, X), chunk_dr_merge_states the state entering every segment; each segment is then run from
its merged state.  Bar: the state tolerance (1e-3) for M, X and the merged states against the
fp64 oracle (``oracle.cp``), and the forward's bars for the re-run outputs against the unsplit
sequence, compared per token as the page "flash-linear-attention KCP 精度失效根因排查手册"
prescribes.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import cp
import chunked_gated_delta_chunk_amd as cdr
from chunked_gated_delta_chunk_amd.synth import make_inputs

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
S_TOL = 1e-3
DEV = "cuda:0"


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def ratio(x, ref, tol):
    x = np.asarray(x, dtype=np.float64)
    return float(np.max(np.abs(x - ref) / (tol + tol * np.abs(ref)))) if ref.size else 0.0


CASES = [
    # label, cuts, H, HV, C, per_dim, gate_mean, l2n[, spike probability[, strong key dimensions]]
    ("kda_4_segments_C64", [0, 300, 301, 700, 1000], 2, 2, 64, True, 0.0, False),
    ("kda_weak_C128", [0, 256, 640, 900], 1, 2, 128, True, 3.0, True),
    ("gdn_grouped_C64", [0, 128, 500, 512], 1, 2, 64, False, 1.0, False),
    # no forgetting (g = 0, gate_mean None): the segment maps carry everything across segments
    ("kda_g0_C128", [0, 384, 700, 1024], 2, 2, 128, True, None, False),
    ("kda_g0_C64", [0, 130, 600, 1000], 1, 1, 64, True, None, False),
    # isolated g = -40 tokens (1 in 20), with ordinary and with weak gates: wide and narrow tiles
    ("kda_spikes_C64", [0, 200, 450, 700], 2, 2, 64, True, 0.0, False, 0.05),
    ("kda_spikes_weak_C128", [0, 300, 301, 800], 1, 1, 128, True, 3.0, True, 0.02),
    # weak gates (the maps carry) except in a few key dimensions, which forget fast
    # (logsigmoid(N(-6,1))): tiles wide in those dimensions only
    ("kda_weak_strong_dims_C128", [0, 256, 500, 900], 1, 1, 128, True, 3.0, False, 0.0, (0, 77)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_segments_merge_to_the_unsplit_sequence(case):
    label, cuts, H, HV, C, per_dim, gm, l2n = case[:8]
    spikes = case[8] if len(case) > 8 else 0.0
    dims = case[9] if len(case) > 9 else ()
    T = cuts[-1]
    inp = make_inputs(1, T, H, seed=600 + T, per_dim_gate=per_dim, initial_state=True, chunk_size=C,
                      gate="zero" if gm is None else "logsigmoid", gate_mean=gm or 0.0, HV=HV,
                      normalise=not l2n, spike_prob=spikes)
    if dims:
        g = inp.g.clone()
        gen = torch.Generator().manual_seed(610 + T)
        for d in dims:
            g[..., d] = torch.nn.functional.logsigmoid(torch.randn(g.shape[:3], generator=gen) - 6.0)
        inp.g = g
    note(f"[cp] {label} T={T} segments {np.diff(cuts).tolist()} C={C}")
    d = inp.to(DEV)
    cu = torch.tensor(cuts, dtype=torch.int32)
    M, X = cdr.segment_map(d.q, d.k, d.v, d.g, d.beta, cu_seqlens=cu.to(DEV), chunk_size=C,
                           use_qk_l2norm_in_kernel=l2n)
    s_in = cdr.merge_states(M, X, d.initial_state[0])
    torch.cuda.synchronize()
    M_ref, X_ref = cp.segment_map(inp.q, inp.k, inp.v, inp.g, inp.beta, cu_seqlens=cu, use_qk_l2norm=l2n)
    rm, rx = ratio(M.cpu().numpy(), M_ref, S_TOL), ratio(X.cpu().numpy(), X_ref, S_TOL)
    s_ref = cp.merge(M_ref, X_ref, inp.initial_state[0].double().numpy())
    rs = ratio(s_in.cpu().numpy(), s_ref, S_TOL)
    # each segment from its merged state, against the unsplit sequence token by token
    R = len(cuts) - 1
    o_ref, S_ref = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, initial_state=inp.initial_state,
                                        use_qk_l2norm=l2n)
    ro = 0.0
    for r in range(R):
        a, b = cuts[r], cuts[r + 1]
        sl = lambda t: t[:, a:b].contiguous()  # noqa: E731
        o_r, _ = cdr.chunk_dr_fwd(sl(d.q), sl(d.k), sl(d.v), sl(d.g), sl(d.beta),
                                  initial_state=s_in[r:r + 1].contiguous(), chunk_size=C,
                                  use_qk_l2norm_in_kernel=l2n)
        torch.cuda.synchronize()
        ro = max(ro, ratio(o_r.float().cpu().numpy(), o_ref[:, a:b], O_TOL))
    rf = ratio(s_in[R].cpu().numpy(), S_ref[0], S_TOL)
    note(f"[cp] {label}: M {rm:.4f}  X {rx:.4f}  merged {rs:.4f}  final {rf:.4f}  o {ro:.4f} (err/tol)")
    assert max(rm, rx, rs, rf) <= 1.0 and ro <= 1.0


def test_merge_without_initial_state_and_one_segment():
    inp = make_inputs(1, 200, 2, seed=610, chunk_size=64)
    d = inp.to(DEV)
    M, X = cdr.segment_map(d.q, d.k, d.v, d.g, d.beta, chunk_size=64)
    s_in = cdr.merge_states(M, X)
    _, S = cdr.chunk_dr_fwd(d.q, d.k, d.v, d.g, d.beta, chunk_size=64, output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(s_in[0], torch.zeros_like(s_in[0]))
    # one segment from a zero start: the merged final state is X itself
    assert torch.equal(s_in[1], X[0])
    assert ratio(s_in[1].cpu().numpy(), S[0].cpu().double().numpy(), S_TOL) <= 1.0
