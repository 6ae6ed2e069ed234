"""Parity of the HIP per-token (decode) forward with the fp64 oracle, through the C interface.

Same bar as the chunked forward (page "PyPTO-Gym 的 chunk_kda 算子实战", section 支持的 dtype
与形状约束): |x - ref| <= atol + rtol |ref|, rtol = atol = 1e-2 for o (bf16) and 1e-3 for the
fp32 states, against ``oracle.recurrent_fwd`` (separate states) and
``oracle.recurrent_pool_fwd`` (state pool, speculative rows).  Pool slots that a call must not
touch are compared bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import chunked_gated_delta_chunk_amd as cdr
from chunked_gated_delta_chunk_amd.synth import (DECODE_WORKLOADS, decode_workload_inputs,
                                                 make_decode_inputs, make_inputs)

pytestmark = pytest.mark.gpu

O_TOL = 1e-2
S_TOL = 1e-3
DEV = "cuda:0"


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def ratio(x, ref, tol):
    x = np.asarray(x, dtype=np.float64)
    return float(np.max(np.abs(x - ref) / (tol + tol * np.abs(ref)))) if ref.size else 0.0


def run_pool(d, l2n, pool=None):
    g = d.to(DEV)
    pool = g.state_pool.clone() if pool is None else pool
    o, _ = cdr.fused_recurrent_fwd(g.q, g.k, g.v, g.g, g.beta, cu_seqlens=g.cu_seqlens,
                                   use_qk_l2norm_in_kernel=l2n, state_pool=pool,
                                   ssm_state_indices=g.ssm_state_indices,
                                   num_accepted_tokens=g.num_accepted_tokens)
    torch.cuda.synchronize()
    return o, pool


def touched_slots(d):
    idx = d.ssm_state_indices.flatten().tolist()
    return sorted({s for s in idx if 0 <= s < d.state_pool.shape[0]})


def check_pool(d, l2n, label):
    """GPU pool call vs the oracle on a pool compacted to the slots the call may touch;
    every other slot must come back bit-identical."""
    note(f"[decode pool] {label} q{tuple(d.q.shape)} v{tuple(d.v.shape)} "
         f"idx{tuple(d.ssm_state_indices.shape)} pool{tuple(d.state_pool.shape)} l2n={l2n}")
    o, pool = run_pool(d, l2n)
    assert torch.isfinite(o.float()).all() and torch.isfinite(pool).all()
    P = d.state_pool.shape[0]
    used = touched_slots(d)
    remap = torch.full((P + 1,), -1, dtype=torch.int32)
    remap[torch.tensor(used, dtype=torch.long)] = torch.arange(len(used), dtype=torch.int32)
    idx = d.ssm_state_indices.long()
    cidx = torch.where((idx >= 0) & (idx < P), remap[idx.clamp(0, P)], torch.full_like(idx, -1))
    o_ref, pool_ref = oracle.recurrent_pool_fwd(
        d.q, d.k, d.v, d.g, d.beta, d.state_pool[used], cidx.to(torch.int32),
        d.num_accepted_tokens, cu_seqlens=d.cu_seqlens, use_qk_l2norm=l2n)
    ro = ratio(o.float().cpu().numpy(), o_ref, O_TOL)
    host = pool.cpu()
    rs = ratio(host[used].numpy(), pool_ref, S_TOL)
    note(f"[decode pool] {label}: o err/tol {ro:.4f}  pool err/tol {rs:.4f}")
    assert ro <= 1.0 and rs <= 1.0
    rest = torch.ones(P, dtype=torch.bool)
    rest[torch.tensor(used, dtype=torch.long)] = False
    assert torch.equal(host[rest], d.state_pool[rest]), "a slot outside the indices changed"
    return o, pool


# ---------------------------------------------------------------- separate states
SEPARATE = [
    # label, N, T, H, HV, per_dim, lengths, initial, gate_mean, l2n
    ("decode_T1_b8", 8, 1, 2, 2, True, None, True, 0.0, False),
    ("decode_T1_l2n_grouped", 6, 1, 2, 4, True, None, True, 0.0, True),
    ("decode_T5_gdn", 3, 5, 2, 2, False, None, True, 0.0, False),
    ("recurrent_T300_weak", 2, 300, 1, 2, True, None, True, 4.0, True),
    ("recurrent_T64_zero_state", 2, 64, 2, 2, True, None, False, 0.0, False),
    ("varlen_ragged_empty", 4, 0, 2, 2, True, (1, 0, 7, 33), True, 1.0, False),
    ("varlen_gdn_grouped_l2n", 3, 0, 1, 4, False, (5, 1, 12), True, 0.0, True),
]


@pytest.mark.parametrize("case", SEPARATE, ids=[c[0] for c in SEPARATE])
def test_separate_state_parity(case):
    label, N, T, H, HV, per_dim, lengths, init, gm, l2n = case
    if lengths is not None:
        inp = make_inputs(1, sum(lengths), H, seed=300 + len(label), per_dim_gate=per_dim,
                          lengths=lengths, initial_state=init, gate_mean=gm, HV=HV,
                          normalise=not l2n)
    else:
        inp = make_inputs(N, T, H, seed=300 + len(label), per_dim_gate=per_dim,
                          initial_state=init, gate_mean=gm, HV=HV, normalise=not l2n)
    note(f"[decode separate] {label} q{tuple(inp.q.shape)} v{tuple(inp.v.shape)} l2n={l2n}")
    d = inp.to(DEV)
    o, S = cdr.fused_recurrent_fwd(d.q, d.k, d.v, d.g, d.beta, initial_state=d.initial_state,
                                   output_final_state=True, cu_seqlens=d.cu_seqlens,
                                   use_qk_l2norm_in_kernel=l2n)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                        initial_state=inp.initial_state,
                                        cu_seqlens=inp.cu_seqlens, use_qk_l2norm=l2n)
    ro = ratio(o.float().cpu().numpy(), o_ref, O_TOL)
    rs = ratio(S.cpu().numpy(), S_ref, S_TOL)
    note(f"[decode separate] {label}: o err/tol {ro:.4f}  S err/tol {rs:.4f}")
    assert ro <= 1.0 and rs <= 1.0


def test_separate_in_place_equals_out_of_place():
    inp = make_inputs(4, 3, 2, seed=311, initial_state=True, HV=4)
    d = inp.to(DEV)
    o1, S1 = cdr.fused_recurrent_fwd(d.q, d.k, d.v, d.g, d.beta, initial_state=d.initial_state,
                                     output_final_state=True)
    state = d.initial_state.clone()
    o2, S2 = cdr.fused_recurrent_fwd(d.q, d.k, d.v, d.g, d.beta, initial_state=state,
                                     output_final_state=True, final_state_out=state)
    torch.cuda.synchronize()
    assert S2.data_ptr() == state.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, state)


def test_gate_zero_beta_zero_keeps_state_exactly():
    inp = make_inputs(3, 4, 2, seed=312, gate="zero", beta_mode="zero", initial_state=True)
    d = inp.to(DEV)
    _, S = cdr.fused_recurrent_fwd(d.q, d.k, d.v, d.g, d.beta, initial_state=d.initial_state,
                                   output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), inp.initial_state)


# ---------------------------------------------------------------- state pool
POOL = [
    # label, N, T, H, HV, slots, cols, per_dim, lengths, padded, l2n
    ("pool_T1", 16, 1, 2, 2, 64, 0, True, None, (), True),
    ("pool_T3_gdn_grouped", 5, 3, 1, 4, 16, 0, False, None, (), False),
    ("pool_padding", 6, 2, 2, 2, 16, 0, True, None, (1, 4), True),
    ("pool_varlen_empty", 4, 0, 2, 2, 16, 0, True, (2, 0, 1, 5), (), True),
    ("spec_L4", 8, 4, 2, 2, 64, 4, True, None, (), True),
    ("spec_L4_T2_grouped", 8, 2, 2, 4, 64, 4, True, None, (3,), False),
    ("spec_gdn_T6_L4", 4, 6, 1, 2, 32, 4, False, None, (), True),
    ("spec_varlen", 4, 0, 2, 2, 32, 3, True, (3, 0, 1, 2), (), True),
]


@pytest.mark.parametrize("case", POOL, ids=[c[0] for c in POOL])
def test_pool_parity(case):
    label, N, T, H, HV, slots, cols, per_dim, lengths, padded, l2n = case
    d = make_decode_inputs(N, T, H, HV, slots, seed=400 + len(label), index_cols=cols,
                           per_dim_gate=per_dim, normalise=not l2n, lengths=lengths,
                           padded=padded)
    check_pool(d, l2n, label)


def test_spec_bad_accept_counts_and_write_indices():
    """Accepted counts 0 and L + 1 make padding; a -1 and an out-of-range write index skip
    single writes; one sequence starts from a slot it also writes."""
    d = make_decode_inputs(5, 3, 2, 2, 32, seed=420, index_cols=3, normalise=False)
    d.num_accepted_tokens = torch.tensor([0, 4, 2, 3, 1], dtype=torch.int32)
    d.ssm_state_indices[2, 0] = -1
    d.ssm_state_indices[3, 1] = 32
    check_pool(d, True, "spec_bad_indices")


def test_pool_equals_separate_bit_for_bit():
    """The pool path and the separate path run the same arithmetic: a pool call equals a
    separate call on the gathered states, and the states after each draft token of a
    speculative call equal separate calls on the prefixes."""
    d = make_decode_inputs(6, 3, 2, 4, 32, seed=430, index_cols=3, normalise=False)
    o, pool = run_pool(d, True)
    g = d.to(DEV)
    idx = g.ssm_state_indices.long()
    start = idx[torch.arange(6, device=DEV), g.num_accepted_tokens.long() - 1]
    s0 = g.state_pool[start]
    for t in range(3):
        o_t, S_t = cdr.fused_recurrent_fwd(g.q[:, :t + 1].contiguous(), g.k[:, :t + 1].contiguous(),
                                           g.v[:, :t + 1].contiguous(), g.g[:, :t + 1].contiguous(),
                                           g.beta[:, :t + 1].contiguous(), initial_state=s0,
                                           output_final_state=True, use_qk_l2norm_in_kernel=True)
        torch.cuda.synchronize()
        assert torch.equal(pool[idx[:, t]], S_t), f"draft position {t}"
        if t == 2:
            assert torch.equal(o, o_t)


def test_repeat_calls_are_bit_identical():
    d = make_decode_inputs(8, 2, 2, 2, 32, seed=440, index_cols=2, normalise=False)
    o1, p1 = run_pool(d, True)
    o2, p2 = run_pool(d, True)
    assert torch.equal(o1, o2) and torch.equal(p1, p2)


def test_prefill_then_decode():
    """Chunked prefill of 300 tokens, then two decode steps from its final state, against
    one recurrence over all 302 tokens."""
    inp = make_inputs(1, 302, 2, seed=450, initial_state=True, HV=4, normalise=False)
    d = inp.to(DEV)
    o_p, S = cdr.chunk_dr_fwd(d.q[:, :300].contiguous(), d.k[:, :300].contiguous(),
                              d.v[:, :300].contiguous(), d.g[:, :300].contiguous(),
                              d.beta[:, :300].contiguous(), initial_state=d.initial_state,
                              chunk_size=64, output_final_state=True, use_qk_l2norm_in_kernel=True)
    pool = S.clone()
    outs = []
    for t in (300, 301):
        o_t, _ = cdr.fused_recurrent_fwd(d.q[:, t:t + 1].contiguous(), d.k[:, t:t + 1].contiguous(),
                                         d.v[:, t:t + 1].contiguous(), d.g[:, t:t + 1].contiguous(),
                                         d.beta[:, t:t + 1].contiguous(), use_qk_l2norm_in_kernel=True,
                                         state_pool=pool,
                                         ssm_state_indices=torch.zeros(1, dtype=torch.int32, device=DEV))
        outs.append(o_t)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                        initial_state=inp.initial_state, use_qk_l2norm=True)
    o_all = torch.cat([o_p] + outs, dim=1).float().cpu().numpy()
    ro = ratio(o_all, o_ref, O_TOL)
    rs = ratio(pool.cpu().numpy(), S_ref, S_TOL)
    note(f"[prefill+decode] o err/tol {ro:.4f}  S err/tol {rs:.4f}")
    assert ro <= 1.0 and rs <= 1.0


# ---------------------------------------------------------------- full-size decode workloads
@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_decode_workload_parity(name):
    w = DECODE_WORKLOADS[name]
    d = decode_workload_inputs(w, seed=2000 + list(DECODE_WORKLOADS).index(name))
    check_pool(d, w.qk_l2norm, name)
