"""Parity of the HIP forward with the fp64 oracle, through the C interface.

Bar (page "PyPTO-Gym 的 chunk_kda 算子实战", section 支持的 dtype 与形状约束):
element-wise |x - ref| <= atol + rtol |ref| with rtol = atol = 1e-2 for the bf16
output o and 1e-3 for the fp32 final state S, the reference being the fp64
per-token recurrence on the same bits.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import chunked_gated_delta_chunk_amd as cdr
from chunked_gated_delta_chunk_amd.synth import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
S_TOL = 1e-3
DEV = "cuda:0"


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def run_gpu(inp, output_final_state=True, workspace=None, l2n=False):
    d = inp.to(DEV)
    o, S = cdr.chunk_dr_fwd(d.q, d.k, d.v, d.g, d.beta, initial_state=d.initial_state,
                            cu_seqlens=d.cu_seqlens, chunk_size=inp.chunk_size,
                            output_final_state=output_final_state, workspace=workspace,
                            use_qk_l2norm_in_kernel=l2n)
    torch.cuda.synchronize()
    return o, S


def ratio(x, ref, tol):
    x = np.asarray(x, dtype=np.float64)
    return float(np.max(np.abs(x - ref) / (tol + tol * np.abs(ref)))) if ref.size else 0.0


def check(inp, heads=None, label="", l2n=False):
    """GPU vs oracle; `heads` restricts the oracle (and the comparison) to a head subset."""
    note(f"[parity] {label} q{tuple(inp.q.shape)} v{tuple(inp.v.shape)} C={inp.chunk_size} l2n={l2n}")
    o, S = run_gpu(inp, l2n=l2n)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    sel = slice(None) if heads is None else heads
    sub = lambda t: None if t is None else t[:, :, sel].contiguous()  # noqa: E731
    s0 = None if inp.initial_state is None else inp.initial_state[:, sel].contiguous()
    o_ref, S_ref = oracle.recurrent_fwd(sub(inp.q), sub(inp.k), sub(inp.v), sub(inp.g),
                                        sub(inp.beta), initial_state=s0, cu_seqlens=inp.cu_seqlens,
                                        use_qk_l2norm=l2n)
    ro = ratio(o[:, :, sel].float().cpu().numpy(), o_ref, O_TOL)
    rs = ratio(S[:, sel].cpu().numpy(), S_ref, S_TOL)
    note(f"[parity] {label}: o err/tol {ro:.3f}  S err/tol {rs:.3f}")
    assert ro <= 1.0, f"o out of tolerance ({ro:.3f} x tol)"
    assert rs <= 1.0, f"S out of tolerance ({rs:.3f} x tol)"
    return o, S


# ---------------------------------------------------------------- small shapes, all rows
_L1100 = tuple((7 * i) % 5 for i in range(1100))  # lengths 0..4, empty sequences included
SMALL = [
    # label, B, T, H, C, per_dim, lengths, initial, gate_mean
    ("kda_T64_one_chunk", 1, 64, 2, 64, True, None, False, 0.0),
    ("kda_T37_pure_tail", 1, 37, 2, 64, True, None, True, 0.0),
    ("kda_T1", 1, 1, 1, 64, True, None, True, 0.0),
    ("kda_T200_tail8", 2, 200, 2, 64, True, None, True, 0.0),
    ("kda_T130_C128", 1, 130, 2, 128, True, None, True, 0.0),
    ("kda_T384_C128_weak", 1, 384, 2, 128, True, None, True, 4.0),
    ("kda_T512_C64_weak", 1, 512, 2, 64, True, None, True, 4.0),
    ("gdn_T300_C64", 2, 300, 3, 64, False, None, True, 0.0),
    ("gdn_T256_C128_weak", 1, 256, 2, 128, False, None, True, 4.0),
    ("varlen_64_200_320", 1, 584, 2, 64, True, (64, 200, 320), False, 0.0),
    ("varlen_ragged_empty", 1, 259, 2, 64, True, (1, 0, 63, 65, 130), True, 0.0),
    ("varlen_C128_ragged", 1, 700, 2, 128, True, (127, 129, 1, 443), True, 1.0),
    ("varlen_gdn", 1, 500, 2, 64, False, (100, 0, 400), True, 0.0),
    # equal lengths: the chain order ranks ties by sequence index
    ("varlen_equal_lengths", 1, 390, 2, 64, True, (130, 130, 130), True, 1.0),
    # more packed sequences than the chain ordering handles (1100 > 1024): sequence order
    ("varlen_1100_short", 1, sum(_L1100), 1, 64, True, _L1100, True, 1.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(case):
    label, B, T, H, C, per_dim, lengths, init, gm = case
    inp = make_inputs(B, T, H, seed=100 + T, per_dim_gate=per_dim, lengths=lengths,
                      initial_state=init, chunk_size=C, gate_mean=gm)
    check(inp, label=label)


def test_gate_zero_beta_zero_keeps_state_exactly():
    inp = make_inputs(1, 200, 2, seed=7, gate="zero", beta_mode="zero", initial_state=True,
                      chunk_size=64)
    note("[exact] g=0 beta=0")
    o, S = run_gpu(inp)
    assert torch.equal(S.cpu(), inp.initial_state)


def test_beta_zero_pure_decay():
    inp = make_inputs(1, 256, 2, seed=8, beta_mode="zero", initial_state=True, chunk_size=128,
                      gate_mean=3.0)
    check(inp, label="beta0")


# ---------------------------------------------------------------- invariants of the GPU path
def test_repeat_runs_are_bit_identical_and_workspace_independent():
    inp = make_inputs(1, 1000, 4, seed=9, initial_state=True, chunk_size=128, gate_mean=2.0)
    note("[determinism] two runs, second with a NaN-poisoned workspace")
    o1, S1 = run_gpu(inp)
    d = inp.to(DEV)
    p = cdr.make_problem(1, 1000, 4, 128, 128, 1, True, 128, 128 ** -0.5, True, True, False)
    ws = torch.full((cdr.workspace_bytes(p),), 0xFF, dtype=torch.uint8, device=DEV)
    o2, S2 = run_gpu(inp, workspace=ws)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    del d


def test_single_segment_varlen_equals_fixed_length():
    T = 777
    a = make_inputs(1, T, 2, seed=10, initial_state=True, chunk_size=64)
    b = make_inputs(1, T, 2, seed=10, initial_state=True, chunk_size=64, lengths=(T,))
    note("[varlen==fixed]")
    o1, S1 = run_gpu(a)
    o2, S2 = run_gpu(b)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_continuation_at_chunk_boundary_is_bit_exact():
    T, T1, C = 640, 256, 128
    full = make_inputs(1, T, 2, seed=11, initial_state=True, chunk_size=C, gate_mean=3.0)
    note("[continuation]")
    o, S = run_gpu(full)
    cut = lambda t, a, b: t[:, a:b].contiguous()  # noqa: E731
    fields = lambda a, b: [cut(t, a, b) for t in (full.q, full.k, full.v, full.g, full.beta)]  # noqa: E731
    o_a, S_a = run_gpu(type(full)(*fields(0, T1), full.initial_state, None, C))
    o_b, S_b = run_gpu(type(full)(*fields(T1, T), S_a.cpu(), None, C))
    assert torch.equal(torch.cat([o_a, o_b], dim=1), o)
    assert torch.equal(S_b, S)


def test_chunk_sizes_agree():
    a = make_inputs(1, 512, 2, seed=12, initial_state=True, chunk_size=64, gate_mean=2.0)
    b = make_inputs(1, 512, 2, seed=12, initial_state=True, chunk_size=128, gate_mean=2.0)
    note("[C64 vs C128]")
    o1, S1 = run_gpu(a)
    o2, S2 = run_gpu(b)
    assert ratio(o1.float().cpu().numpy(), o2.double().cpu().numpy(), O_TOL) <= 1.0
    assert ratio(S1.cpu().numpy(), S2.double().cpu().numpy(), S_TOL) <= 1.0


STAGED = [
    ("kda_C128", dict(B=1, T=1000, H=3, chunk_size=128, initial_state=True, gate_mean=2.0)),
    ("kda_C64_varlen", dict(B=1, T=700, H=2, chunk_size=64, initial_state=True, lengths=(100, 0, 333, 267))),
    ("gdn_C64", dict(B=2, T=300, H=2, chunk_size=64, initial_state=True, per_dim_gate=False)),
]


@pytest.mark.parametrize("label,kw", STAGED, ids=[s[0] for s in STAGED])
def test_staged_calls_equal_one_call(label, kw):
    """The three kernels launched one stage per call give the bits of one full call."""
    kw = dict(kw)
    inp = make_inputs(kw.pop("B"), kw.pop("T"), kw.pop("H"), seed=14, **kw)
    note(f"[staged==full] {label}")
    o1, S1 = run_gpu(inp)
    d = inp.to(DEV)
    call = cdr.PreparedForward(d.q, d.k, d.v, d.g, d.beta, initial_state=d.initial_state,
                               cu_seqlens=d.cu_seqlens, chunk_size=inp.chunk_size, output_final_state=True)
    for st in (cdr.STAGE_INTRA, cdr.STAGE_CHAIN, cdr.STAGE_OUTPUT):
        call(st)
    torch.cuda.synchronize()
    assert torch.equal(o1, call.o) and torch.equal(S1, call.S)


# ---------------------------------------------------------------- input variants
VARIANTS = [
    # label, B, T, H, HV, C, per_dim, lengths, normalise on the host, in-kernel l2 norm
    ("kda_gva_C128_tail", 1, 300, 2, 4, 128, True, None, True, False),
    ("gdn_gva_C64_varlen", 1, 400, 1, 3, 64, False, (150, 0, 250), True, False),
    ("kda_l2n_C64", 2, 200, 2, None, 64, True, None, False, True),
    ("kda_l2n_gva_C128_varlen", 1, 500, 2, 4, 128, True, (129, 371), False, True),
    ("gdn_l2n_gva_C128", 1, 260, 2, 4, 128, False, None, False, True),
]


@pytest.mark.parametrize("case", VARIANTS, ids=[c[0] for c in VARIANTS])
def test_input_variants(case):
    label, B, T, H, HV, C, per_dim, lengths, normalise, l2n = case
    inp = make_inputs(B, T, H, seed=21, per_dim_gate=per_dim, lengths=lengths, initial_state=True,
                      chunk_size=C, normalise=normalise, HV=HV, gate_mean=1.0)
    check(inp, label=label, l2n=l2n)


def test_l2norm_switch_changes_the_output():
    """As the page's feature-switch test asks: the normalised run differs from the plain
    one by more than 1e-4 on unnormalised inputs."""
    inp = make_inputs(1, 128, 2, seed=22, chunk_size=64, normalise=False)
    note("[l2n switch]")
    o1, _ = run_gpu(inp, l2n=True)
    o2, _ = run_gpu(inp, l2n=False)
    assert (o1.float() - o2.float()).abs().max().item() > 1e-4


def test_no_final_state_requested():
    inp = make_inputs(1, 128, 2, seed=13, chunk_size=64)
    note("[no final state]")
    o, S = run_gpu(inp, output_final_state=False)
    assert S is None and torch.isfinite(o.float()).all()


# ---------------------------------------------------------------- the five workloads at full size
FULL = [
    ("kda_small", None),
    ("gdn_b2_t2048", None),
    ("kda_t8192", None),
    ("kda_varlen", None),
    ("kda_t65536", [0, 17]),   # the oracle checks two of the 32 heads over all 65536 tokens
]


@pytest.mark.parametrize("name,heads", FULL, ids=[f[0] for f in FULL])
def test_workload_parity(name, heads):
    w = WORKLOADS[name]
    inp = workload_inputs(w, seed=1000 + list(WORKLOADS).index(name) + 1)
    check(inp, heads=heads, label=name)
