"""Pins of the decode oracle, ``oracle.recurrent_pool_fwd`` (CPU only).

The decode-side operator of the page "PyPTO-Gym 的 chunk_kda 算子实战" (section 与其他 KDA
算子的关系) keeps the recurrent state in place in a pool (``ssm_state_indices``) and
supports speculative decoding (``num_accepted_tokens``).  These tests tie the oracle's
gather and scatter to facts that do not come from it: closed forms of the recurrence
(beta = 0: pure decay; one token from a zero state: an outer product), the contract
that makes speculative decoding correct (resuming from the slot of the a-th accepted
draft equals having run only the accepted tokens), and the padding rules.
"""
import numpy as np
import torch

import oracle
from chunked_gated_delta_chunk_amd.synth import make_decode_inputs


def _np(t):
    return t.double().numpy()


def _decay_closed_form(d, n, start_state, scale, hv_per_k, t_end=None):
    """beta = 0: the state after token t is S0 * exp(G_t) along K and
    o_t = scale * S0 (q_t * exp(G_t)), G_t = sum of g over tokens 0..t (per value head)."""
    q, g = _np(d.q)[n], _np(d.g)[n]          # [T, H, K], [T, HV, K] or [T, HV]
    T = q.shape[0] if t_end is None else t_end
    HV = start_state.shape[0]
    if g.ndim == 2:
        g = np.repeat(g[:, :, None], q.shape[-1], axis=2)
    G = np.cumsum(g[:T], axis=0)            # [T, HV, K]
    o = np.zeros((T, HV, start_state.shape[1]))
    for t in range(T):
        for hv in range(HV):
            qg = q[t, hv // hv_per_k] * np.exp(G[t, hv])
            o[t, hv] = scale * start_state[hv] @ qg
    states = start_state[None] * np.exp(G)[:, :, None, :]   # [T, HV, V, K]
    return o, states


def test_pool_in_place_beta_zero_closed_form():
    """One slot per sequence, beta = 0, grouped heads (H = 2, HV = 4): every listed slot
    ends decayed by exp(sum g) along K, every other slot is untouched, and o reads the
    listed slot's state."""
    d = make_decode_inputs(3, 5, 2, 4, 12, seed=41, K=16, V=8, beta_mode="zero", normalise=True)
    scale = 0.3
    o, pool = oracle.recurrent_pool_fwd(d.q, d.k, d.v, d.g, d.beta, d.state_pool,
                                        d.ssm_state_indices, scale=scale)
    before = _np(d.state_pool)
    idx = d.ssm_state_indices.tolist()
    for n in range(3):
        o_ref, states = _decay_closed_form(d, n, before[idx[n]], scale, 2)
        np.testing.assert_allclose(o[n], o_ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(pool[idx[n]], states[-1], rtol=1e-12, atol=1e-15)
    untouched = [s for s in range(12) if s not in idx]
    np.testing.assert_array_equal(pool[untouched], before[untouched])


def test_pool_single_token_from_zero_slot_layout():
    """One token from a zero state: the slot becomes beta v k^T laid out [V, K] and
    o = scale beta (q . k) v; with the per-head gate the decay of a zero state is moot."""
    for per_dim in (True, False):
        d = make_decode_inputs(2, 1, 1, 1, 4, seed=42, K=16, V=8, normalise=True,
                               per_dim_gate=per_dim)
        pool0 = torch.zeros_like(d.state_pool)
        o, pool = oracle.recurrent_pool_fwd(d.q, d.k, d.v, d.g, d.beta, pool0,
                                            d.ssm_state_indices, scale=0.5)
        for n, slot in enumerate(d.ssm_state_indices.tolist()):
            q, k, v = _np(d.q)[n, 0, 0], _np(d.k)[n, 0, 0], _np(d.v)[n, 0, 0]
            b = float(d.beta[n, 0, 0])
            np.testing.assert_allclose(pool[slot, 0], b * np.outer(v, k), rtol=1e-14, atol=1e-16)
            np.testing.assert_allclose(o[n, 0, 0], 0.5 * b * (q @ k) * v, rtol=1e-12, atol=1e-15)


def test_spec_positions_hold_state_after_each_token():
    """Speculative rows, beta = 0: slot idx[n, t] holds the start state decayed through
    tokens 0..t, the start is slot idx[n, a - 1], and a sequence may overwrite the slot it
    started from (the start is read first)."""
    d = make_decode_inputs(2, 4, 1, 2, 16, seed=43, K=16, V=8, index_cols=4, beta_mode="zero",
                           normalise=True)
    idx = torch.tensor([[5, 6, 7, 8], [9, 10, 11, 12]], dtype=torch.int32)
    acc = torch.tensor([3, 1], dtype=torch.int32)      # starts: slot 7 (also written), slot 9
    o, pool = oracle.recurrent_pool_fwd(d.q, d.k, d.v, d.g, d.beta, d.state_pool, idx, acc,
                                        scale=0.25)
    before = _np(d.state_pool)
    for n, start in ((0, 7), (1, 9)):
        o_ref, states = _decay_closed_form(d, n, before[start], 0.25, 2)
        np.testing.assert_allclose(o[n], o_ref, rtol=1e-12, atol=1e-14)
        for t in range(4):
            np.testing.assert_allclose(pool[int(idx[n, t])], states[t], rtol=1e-12, atol=1e-15)
    rest = [s for s in range(16) if s not in idx.flatten().tolist()]
    np.testing.assert_array_equal(pool[rest], before[rest])


def test_spec_acceptance_contract():
    """Two speculative steps.  Step A runs 4 drafts per sequence from its slot; step B
    accepts a of them and runs 3 new tokens from slot idx[n, a - 1].  Step B must equal one
    plain recurrence over the a accepted drafts followed by the new tokens, from the state
    step A started from."""
    N, L = 3, 4
    A = make_decode_inputs(N, L, 2, 2, 32, seed=44, K=16, V=8, index_cols=L, normalise=True)
    Bn = make_decode_inputs(N, 3, 2, 2, 32, seed=45, K=16, V=8, index_cols=L, normalise=True)
    idx = A.ssm_state_indices
    start_a = torch.ones(N, dtype=torch.int32)             # step A starts from column 0
    _, pool_a = oracle.recurrent_pool_fwd(A.q, A.k, A.v, A.g, A.beta, A.state_pool, idx,
                                          start_a)
    accepted = torch.tensor([1, 3, 4], dtype=torch.int32)
    # step B writes the same row of slots (a ring of draft positions)
    o_b, pool_b = oracle.recurrent_pool_fwd(Bn.q, Bn.k, Bn.v, Bn.g, Bn.beta,
                                            torch.from_numpy(pool_a), idx, accepted)
    s0 = A.state_pool[idx[:, 0].long()]
    for n in range(N):
        a = int(accepted[n])
        cat = lambda x, y: torch.cat([x[n:n + 1, :a], y[n:n + 1]], dim=1)  # noqa: E731
        o_ref, S_ref = oracle.recurrent_fwd(cat(A.q, Bn.q), cat(A.k, Bn.k), cat(A.v, Bn.v),
                                            cat(A.g, Bn.g), cat(A.beta, Bn.beta),
                                            initial_state=s0[n:n + 1])
        np.testing.assert_allclose(o_b[n], o_ref[0, a:], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(pool_b[int(idx[n, 2])], S_ref[0], rtol=1e-12, atol=1e-14)


def test_padding_entries():
    """A negative or out-of-range start index, or a count of accepted tokens outside
    1..L, makes the sequence padding: zero outputs, no state read or written; the other
    sequences are computed as if the padding were absent.  A negative write index in a
    speculative row skips only that write."""
    d = make_decode_inputs(4, 2, 1, 1, 16, seed=46, K=16, V=8, normalise=True)
    idx = d.ssm_state_indices.clone()
    idx[1] = -1
    idx[2] = 16                                          # == num_slots: out of range
    o, pool = oracle.recurrent_pool_fwd(d.q, d.k, d.v, d.g, d.beta, d.state_pool, idx)
    assert not o[1].any() and not o[2].any()
    for n in (0, 3):
        o1, S1 = oracle.recurrent_fwd(d.q[n:n + 1], d.k[n:n + 1], d.v[n:n + 1], d.g[n:n + 1],
                                      d.beta[n:n + 1],
                                      initial_state=d.state_pool[int(idx[n])][None])
        np.testing.assert_array_equal(o[n], o1[0])
        np.testing.assert_array_equal(pool[int(idx[n])], S1[0])
    before = _np(d.state_pool)
    rest = [s for s in range(16) if s not in (int(idx[0]), int(idx[3]))]
    np.testing.assert_array_equal(pool[rest], before[rest])

    s = make_decode_inputs(3, 3, 1, 1, 16, seed=47, K=16, V=8, index_cols=3, normalise=True)
    idx = s.ssm_state_indices.clone()
    idx[0, 1] = -1                                       # skip one write of sequence 0
    acc = torch.tensor([1, 0, 4], dtype=torch.int32)     # 0 and 4 are outside 1..3: padding
    o, pool = oracle.recurrent_pool_fwd(s.q, s.k, s.v, s.g, s.beta, s.state_pool, idx, acc)
    assert not o[1].any() and not o[2].any()
    before = _np(s.state_pool)
    for n in (1, 2):
        np.testing.assert_array_equal(pool[idx[n].long()], before[idx[n].long()])
    start = s.state_pool[int(idx[0, 0])][None]
    o0, S0 = oracle.recurrent_fwd(s.q[:1], s.k[:1], s.v[:1], s.g[:1], s.beta[:1],
                                  initial_state=start)
    _, S1 = oracle.recurrent_fwd(s.q[:1, :1], s.k[:1, :1], s.v[:1, :1], s.g[:1, :1],
                                 s.beta[:1, :1], initial_state=start)
    np.testing.assert_array_equal(o[0], o0[0])
    np.testing.assert_array_equal(pool[int(idx[0, 0])], S1[0])
    np.testing.assert_array_equal(pool[int(idx[0, 2])], S0[0])


def test_packed_speculative_rows_match_separate_calls():
    """Packed sequences of lengths 2, 0, 3 with speculative rows of 3 slots equal three
    separate calls; the empty sequence writes nothing."""
    lengths = (2, 0, 3)
    d = make_decode_inputs(3, 0, 2, 4, 16, seed=48, K=16, V=8, index_cols=3, lengths=lengths)
    o, pool = oracle.recurrent_pool_fwd(d.q, d.k, d.v, d.g, d.beta, d.state_pool,
                                        d.ssm_state_indices, d.num_accepted_tokens,
                                        cu_seqlens=d.cu_seqlens, use_qk_l2norm=True)
    cu = d.cu_seqlens.tolist()
    before = _np(d.state_pool)
    expect = before.copy()
    for n in range(3):
        s, e = cu[n], cu[n + 1]
        sl = lambda x: x[:, s:e]  # noqa: E731
        o1, p1 = oracle.recurrent_pool_fwd(sl(d.q), sl(d.k), sl(d.v), sl(d.g), sl(d.beta),
                                           d.state_pool, d.ssm_state_indices[n:n + 1],
                                           d.num_accepted_tokens[n:n + 1], use_qk_l2norm=True)
        np.testing.assert_array_equal(o[:, s:e], o1)
        changed = np.flatnonzero(np.any((p1 != before).reshape(16, -1), axis=1))
        expect[changed] = p1[changed]
        if n == 1:
            assert changed.size == 0
    np.testing.assert_array_equal(pool, expect)
