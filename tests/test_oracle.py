"""Pins of the oracle (CPU only).

Each test ties the oracle to something other than itself: a closed form, an
identity of the update rule, a hand-derived example, or the independent chunked
formulation.  The update rule and the chunked algorithm are the ones on the page
"PyPTO-Gym 的 chunk_kda 算子实战" (sections 算子定位与算法背景 and M1-M4).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_chunk_amd.synth import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _f32(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32))


def _widen(t):
    return t.double().numpy()


# ----------------------------------------------------------------------------------------
# hand-derived example
# ----------------------------------------------------------------------------------------

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rest = line.split(":", 1)
            rows = [[float(x) for x in r.split()] for r in rest.split("|")]
            vals[key.strip()] = rows
    return vals


def test_golden_three_tokens():
    gd = _read_golden("three_tokens_k2v2.txt")
    T = 3
    q = _bf16(gd["q"]).reshape(1, T, 1, 2)
    k = _bf16(gd["k"]).reshape(1, T, 1, 2)
    v = _bf16(gd["v"]).reshape(1, T, 1, 2)
    g = _f32(gd["g"]).reshape(1, T, 1, 2)
    beta = _f32(gd["beta"]).reshape(1, T, 1)
    tol = gd["tolerance"][0][0]
    o, S = oracle.recurrent_fwd(q, k, v, g, beta, scale=gd["scale"][0][0])
    np.testing.assert_allclose(o.reshape(T, 2), np.array(gd["o"]), atol=tol, rtol=0)
    np.testing.assert_allclose(S.reshape(2, 2), np.array(gd["S_vk"]), atol=tol, rtol=0)
    o2, S2 = oracle.chunked_fwd(q, k, v, g, beta, scale=gd["scale"][0][0], chunk_size=2)
    np.testing.assert_allclose(o2.reshape(T, 2), np.array(gd["o"]), atol=tol, rtol=0)
    np.testing.assert_allclose(S2.reshape(2, 2), np.array(gd["S_vk"]), atol=tol, rtol=0)


# ----------------------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("per_dim", [True, False])
def test_beta_zero_is_pure_decay(per_dim):
    """beta = 0: the state only decays, S_T = diag(exp(sum g)) S0 along the key axis,
    and o_t = scale * (q_t * exp(sum_{s<=t} g_s))^T S0."""
    B, T, H, K, V = 1, 37, 2, 16, 8
    inp = make_inputs(B, T, H, K, V, seed=11, per_dim_gate=per_dim, initial_state=True,
                      beta_mode="zero", state_std=1.0)
    o, S = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                initial_state=inp.initial_state)
    g = _widen(inp.g)
    if not per_dim:
        g = np.repeat(g[..., None], K, axis=-1)
    G = np.cumsum(g[0], axis=0)                                   # [T, H, K]
    s0 = _widen(inp.initial_state)[0]                             # [H, V, K]
    S_ref = s0 * np.exp(G[-1])[:, None, :]
    np.testing.assert_allclose(S[0], S_ref, rtol=1e-12, atol=1e-300)
    q = _widen(inp.q)[0]
    o_ref = K ** -0.5 * np.einsum("thk,hvk->thv", q * np.exp(G), s0)
    np.testing.assert_allclose(o[0], o_ref, rtol=1e-11, atol=1e-13)


def test_gate_zero_beta_zero_keeps_state_exactly():
    B, T, H, K, V = 1, 20, 3, 8, 8
    inp = make_inputs(B, T, H, K, V, seed=12, gate="zero", beta_mode="zero",
                      initial_state=True, state_std=1.0)
    o, S = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                initial_state=inp.initial_state)
    assert np.array_equal(S, _widen(inp.initial_state))


def test_single_token_outer_product():
    """From a zero state one token gives S = beta k v^T (interface [V, K] holds
    beta v_v k_k) and o = scale beta (q . k) v."""
    K, V = 16, 12
    inp = make_inputs(1, 1, 1, K, V, seed=13)
    o, S = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, scale=0.3)
    q, k, v = (_widen(x).reshape(-1) for x in (inp.q, inp.k, inp.v))
    b = float(inp.beta)
    np.testing.assert_allclose(S.reshape(V, K), b * np.outer(v, k), rtol=1e-14, atol=0)
    np.testing.assert_allclose(o.reshape(V), 0.3 * b * np.dot(q, k) * v, rtol=1e-13, atol=1e-15)


def test_one_hot_keys_give_gated_linear_attention():
    """With one-hot keys on distinct dimensions and a zero start the delta read is
    always zero, so the rule reduces to causal linear attention with per-dimension
    decay: o_t = scale sum_{s<=t} beta_s q_t[d_s] exp(G_t[d_s] - G_s[d_s]) v_s."""
    T, K, V = 24, 32, 8
    rng = np.random.default_rng(5)
    dims = rng.permutation(K)[:T]
    kk = np.zeros((T, K), dtype=np.float32)
    kk[np.arange(T), dims] = 1.0
    base = make_inputs(1, T, 1, K, V, seed=14)
    k = _bf16(kk).reshape(1, T, 1, K)
    o, S = oracle.recurrent_fwd(base.q, k, base.v, base.g, base.beta)
    q = _widen(base.q)[0, :, 0]
    v = _widen(base.v)[0, :, 0]
    beta = _widen(base.beta)[0, :, 0]
    G = np.cumsum(_widen(base.g)[0, :, 0], axis=0)               # [T, K]
    Gd = G[:, dims]                                               # G_t[d_s] -> [t, s]
    decay = np.exp(Gd - np.diag(Gd)[None, :])                     # exp(G_t[d_s] - G_s[d_s])
    scores = q[:, dims] * decay * beta[None, :]
    scores = np.tril(scores)
    o_ref = K ** -0.5 * scores @ v
    np.testing.assert_allclose(o[0, :, 0], o_ref, rtol=1e-11, atol=1e-14)
    S_ref = np.zeros((V, K))
    for s in range(T):
        S_ref[:, dims[s]] = beta[s] * v[s] * np.exp(G[-1, dims[s]] - G[s, dims[s]])
    np.testing.assert_allclose(S[0, 0], S_ref, rtol=1e-11, atol=1e-300)


# ----------------------------------------------------------------------------------------
# identities of the update rule
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("per_dim", [True, False])
def test_delta_rule_is_a_gradient_step(per_dim):
    """One token is one gradient step of the online regression loss
    L(S) = 1/2 ||S^T k - v||^2 taken from the decayed state, with step beta.
    The gradient comes from autograd, not from the update formula."""
    K, V = 12, 10
    inp = make_inputs(1, 1, 1, K, V, seed=15, per_dim_gate=per_dim, initial_state=True,
                      state_std=1.0)
    o, S = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                initial_state=inp.initial_state, scale=0.7)
    s0 = torch.tensor(_widen(inp.initial_state)[0, 0].T)           # K x V
    g = torch.tensor(_widen(inp.g).reshape(-1))
    decay = torch.exp(g) if per_dim else torch.exp(g).expand(K)
    Gs = (decay[:, None] * s0).requires_grad_(True)
    k = torch.tensor(_widen(inp.k).reshape(-1))
    v = torch.tensor(_widen(inp.v).reshape(-1))
    loss = 0.5 * ((Gs.T @ k - v) ** 2).sum()
    (grad,) = torch.autograd.grad(loss, Gs)
    S_ref = (Gs - float(inp.beta) * grad).detach()
    np.testing.assert_allclose(S[0, 0], S_ref.numpy().T, rtol=1e-12, atol=1e-14)
    q = torch.tensor(_widen(inp.q).reshape(-1))
    np.testing.assert_allclose(o.reshape(V), (0.7 * S_ref.T @ q).numpy(), rtol=1e-12, atol=1e-14)


def test_write_invariant_unit_key_beta_one():
    """With beta = 1 and a unit key the update writes v exactly: k^T S = v."""
    K, V = 16, 8
    base = make_inputs(1, 1, 1, K, V, seed=16, initial_state=True, state_std=1.0,
                       beta_mode="one")
    kk = np.zeros(K, dtype=np.float32)
    kk[[1, 4, 9, 13]] = [0.5, -0.5, 0.5, 0.5]                      # exactly unit norm
    k = _bf16(kk).reshape(1, 1, 1, K)
    _, S = oracle.recurrent_fwd(base.q, k, base.v, base.g, base.beta,
                                initial_state=base.initial_state)
    np.testing.assert_allclose(S[0, 0] @ kk, _widen(base.v).reshape(V), rtol=1e-13, atol=1e-14)


def test_per_head_gate_equals_broadcast_per_dim_gate():
    B, T, H, K, V = 2, 33, 2, 16, 16
    inp = make_inputs(B, T, H, K, V, seed=17, per_dim_gate=False, initial_state=True)
    g_full = inp.g[..., None].expand(B, T, H, K).contiguous()
    o1, S1 = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                  initial_state=inp.initial_state)
    o2, S2 = oracle.recurrent_fwd(inp.q, inp.k, inp.v, g_full, inp.beta,
                                  initial_state=inp.initial_state)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_continuation_is_exact():
    """Running T tokens equals running T1 tokens, then the remaining tokens from
    the state the first run returned."""
    B, T, H, K, V, T1 = 1, 50, 2, 16, 16, 21
    inp = make_inputs(B, T, H, K, V, seed=18, initial_state=True)
    o, S = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                initial_state=inp.initial_state)
    sl = lambda x, a, b: x[:, a:b].contiguous()  # noqa: E731
    oa, Sa = oracle.recurrent_fwd(*(sl(x, 0, T1) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta)),
                                  initial_state=inp.initial_state)
    ob, Sb = oracle.recurrent_fwd(*(sl(x, T1, T) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta)),
                                  initial_state=torch.tensor(Sa))
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
    assert np.array_equal(Sb, S)


def test_varlen_equals_separate_sequences_and_empty_sequence():
    lengths = [5, 0, 17, 1, 9]
    H, K, V = 2, 16, 8
    inp = make_inputs(1, sum(lengths), H, K, V, seed=19, lengths=lengths, initial_state=True)
    o, S = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                initial_state=inp.initial_state, cu_seqlens=inp.cu_seqlens)
    cu = inp.cu_seqlens.tolist()
    for n, L in enumerate(lengths):
        a, b = cu[n], cu[n + 1]
        if L == 0:
            assert np.array_equal(S[n], _widen(inp.initial_state[n]))
            continue
        sl = lambda x: x[:, a:b].contiguous()  # noqa: E731
        on, Sn = oracle.recurrent_fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta),
                                      initial_state=inp.initial_state[n:n + 1])
        assert np.array_equal(o[:, a:b], on)
        assert np.array_equal(S[n], Sn[0])


# ----------------------------------------------------------------------------------------
# the two formulations agree
# ----------------------------------------------------------------------------------------

CROSS = [
    # B, T, H, K, V, chunk, per_dim, lengths, initial, gate_mean
    (1, 64, 1, 32, 16, 16, True, None, False, 0.0),
    (2, 45, 2, 16, 24, 16, True, None, True, 0.0),
    (1, 100, 1, 32, 32, 64, True, None, True, 4.0),        # weak gate, ragged tail
    (2, 70, 2, 16, 16, 32, False, None, True, 0.0),        # per-head gate
    (1, 75, 2, 16, 16, 16, True, (7, 0, 40, 28), True, 0.0),  # varlen + empty seq
    (1, 130, 1, 128, 128, 64, True, None, True, 0.0),      # full head dims, tail of 2
    (1, 260, 1, 128, 128, 128, False, None, True, 4.0),
]


@pytest.mark.parametrize("case", CROSS)
def test_chunked_matches_recurrent(case):
    B, T, H, K, V, C, per_dim, lengths, init, gm = case
    inp = make_inputs(B, T, H, K, V, seed=20 + T, per_dim_gate=per_dim, lengths=lengths,
                      initial_state=init, gate_mean=gm)
    o1, S1 = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                  initial_state=inp.initial_state, cu_seqlens=inp.cu_seqlens)
    o2, S2 = oracle.chunked_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                initial_state=inp.initial_state, cu_seqlens=inp.cu_seqlens,
                                chunk_size=C)
    np.testing.assert_allclose(o2, o1, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(S2, S1, rtol=1e-9, atol=1e-11)


def test_chunk_size_does_not_change_the_result():
    inp = make_inputs(1, 96, 1, 16, 16, seed=21, initial_state=True, gate_mean=2.0)
    outs = [oracle.chunked_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta,
                               initial_state=inp.initial_state, chunk_size=c) for c in (1, 7, 32, 96)]
    for o, S in outs[1:]:
        np.testing.assert_allclose(o, outs[0][0], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(S, outs[0][1], rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------------------
# input variants: grouped value heads, in-kernel q/k normalisation
# ----------------------------------------------------------------------------------------

def test_grouped_value_heads_read_key_head_by_group():
    """HV = 6 value heads on H = 2 key heads: value head hv equals a one-head run with key
    head hv // 3 (consecutive value heads share a key head)."""
    inp = make_inputs(1, 40, 2, 16, 12, seed=31, initial_state=True, HV=6)
    o, S = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, scale=0.5,
                                initial_state=inp.initial_state)
    for hv in range(6):
        hk = hv // 3
        one = lambda t, h: t[:, :, h:h + 1].contiguous()  # noqa: E731
        o1, S1 = oracle.recurrent_fwd(one(inp.q, hk), one(inp.k, hk), one(inp.v, hv), one(inp.g, hv),
                                      one(inp.beta, hv), scale=0.5,
                                      initial_state=inp.initial_state[:, hv:hv + 1].contiguous())
        np.testing.assert_array_equal(o[:, :, hv], o1[:, :, 0])
        np.testing.assert_array_equal(S[:, hv], S1[:, 0])
    # and the other grouping (hv % H) would not agree
    o_alt, _ = oracle.recurrent_fwd(inp.q[:, :, 1:2].contiguous(), inp.k[:, :, 1:2].contiguous(),
                                    inp.v[:, :, 1:2].contiguous(), inp.g[:, :, 1:2].contiguous(),
                                    inp.beta[:, :, 1:2].contiguous(), scale=0.5,
                                    initial_state=inp.initial_state[:, 1:2].contiguous())
    assert np.max(np.abs(o_alt[:, :, 0] - o[:, :, 1])) > 1e-3


def test_l2norm_is_per_token_and_scale_invariant():
    """With in-kernel normalisation the result does not change when each token's q and
    k are multiplied by its own power of two (exact in bf16), but does change when the
    switch is off; any other normalisation axis would break the invariance."""
    T, H = 33, 2
    inp = make_inputs(1, T, H, 32, 16, seed=32, initial_state=True, normalise=False)
    gen = torch.Generator("cpu").manual_seed(5)
    f = 2.0 ** torch.randint(-2, 3, (1, T, H, 1), generator=gen).float()
    q2 = (inp.q.float() * f).to(torch.bfloat16)
    k2 = (inp.k.float() * torch.flip(f, dims=[1])).to(torch.bfloat16)
    args = dict(scale=0.25, initial_state=inp.initial_state, use_qk_l2norm=True)
    o1, S1 = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, **args)
    o2, S2 = oracle.recurrent_fwd(q2, k2, inp.v, inp.g, inp.beta, **args)
    # the eps under the square root moves the scales by < 1e-6 relative
    np.testing.assert_allclose(o2, o1, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(S2, S1, rtol=1e-6, atol=1e-7)
    o3, _ = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, scale=0.25,
                                 initial_state=inp.initial_state)
    assert np.max(np.abs(o3 - o1)) > 1e-4


def test_l2norm_single_token_closed_form():
    """One token from zero with normalisation: S = beta k^ v^T, o = scale beta (q^ . k^) v,
    x^ = x / sqrt(|x|^2 + 1e-6)."""
    K, V = 16, 12
    inp = make_inputs(1, 1, 1, K, V, seed=33, normalise=False)
    o, S = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, scale=0.3, use_qk_l2norm=True)
    q, k, v = (_widen(x).reshape(-1) for x in (inp.q, inp.k, inp.v))
    qh, kh = q / np.sqrt(q @ q + 1e-6), k / np.sqrt(k @ k + 1e-6)
    b = float(inp.beta)
    np.testing.assert_allclose(S.reshape(V, K), b * np.outer(v, kh), rtol=1e-13, atol=0)
    np.testing.assert_allclose(o.reshape(V), 0.3 * b * np.dot(qh, kh) * v, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("per_dim", [True, False])
def test_chunked_matches_recurrent_grouped_and_normalised(per_dim):
    """The two formulations agree with grouped value heads and in-kernel normalisation."""
    inp = make_inputs(1, 150, 2, 32, 16, seed=34, initial_state=True, normalise=False, HV=4,
                      per_dim_gate=per_dim, chunk_size=64, gate_mean=1.0)
    a = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, initial_state=inp.initial_state,
                             use_qk_l2norm=True)
    b = oracle.chunked_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, initial_state=inp.initial_state,
                           chunk_size=64, use_qk_l2norm=True)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------- input generators used by the GPU suite
def test_spike_gates_leave_other_inputs_unchanged():
    """spike_prob draws its mask after every other tensor: the rest is the unspiked batch."""
    from chunked_gated_delta_chunk_amd.synth import make_inputs
    a = make_inputs(1, 256, 2, seed=3, spike_prob=0.125, initial_state=True)
    b = make_inputs(1, 256, 2, seed=3, initial_state=True)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.beta, b.beta), (a.initial_state, b.initial_state)):
        assert torch.equal(x, y)
    hit = (a.g == -40.0).all(-1)
    assert 0.05 < hit.float().mean().item() < 0.2
    assert torch.equal(a.g[~hit], b.g[~hit])


def test_teacher_inputs_are_predicted_by_the_initial_state():
    """Values of the cancellation inputs are the initial state's prediction up to the noise and
    the bf16 rounding of v; the keys carry one scale per chunk."""
    from chunked_gated_delta_chunk_amd.synth import make_teacher_inputs
    t = make_teacher_inputs(256, 2, seed=4, chunk_size=64, key_scale=(0.3, 1.2), noise=1e-3)
    pred = torch.einsum("hvk,bthk->bthv", t.initial_state[0], t.k.float())
    err = (t.v.float() - pred).abs()
    assert err.max().item() <= 1e-3 * 6 + 2 ** -8 * pred.abs().max().item()
    norms = t.k.float().norm(dim=-1)[0, :, 0].view(4, 64)
    assert ((norms - norms[:, :1]).abs() < 0.02).all()        # one scale per chunk
    assert norms.min().item() >= 0.29 and norms.max().item() <= 1.21


def test_cancellation_measure_closed_forms():
    """oracle.chunked.cancellation (|v_new| / |u| per chunk, section M4's v_new = u - w S):
    from a zero state the first chunk's v_new is u itself (ratio 1); with one-hot keys, g = 0
    and values that are exactly the state's prediction W k, every v_new is 0 (ratio 0)."""
    from oracle.chunked import cancellation
    gen = torch.Generator().manual_seed(11)
    T, H, K, V = 96, 2, 8, 4
    q = torch.randn(1, T, H, K, generator=gen, dtype=torch.float64)
    k = torch.randn(1, T, H, K, generator=gen, dtype=torch.float64)
    v = torch.randn(1, T, H, V, generator=gen, dtype=torch.float64)
    g = -torch.rand(1, T, H, K, generator=gen, dtype=torch.float64)
    beta = torch.rand(1, T, H, generator=gen, dtype=torch.float64)
    zero = torch.zeros(1, H, V, K, dtype=torch.float64)
    c = cancellation(q, k, v, g, beta, zero, chunk_size=32)
    assert c.shape == (H, 3)
    assert np.allclose(c[:, 0], 1.0, rtol=0, atol=1e-12)
    # linear teacher that the initial state already holds exactly: v_t = W k_t
    W = torch.randint(-8, 9, (H, V, K), generator=gen).double() / 4
    idx = torch.randint(0, K, (T, H), generator=gen)
    k1 = torch.nn.functional.one_hot(idx, K).double().unsqueeze(0)
    v1 = torch.einsum("hvk,bthk->bthv", W, k1)
    c0 = cancellation(q, k1, v1, torch.zeros_like(g), beta, W.unsqueeze(0), chunk_size=32)
    assert np.all(c0 <= 1e-12)
    # a state that does not hold the teacher leaves a visible correction
    c1 = cancellation(q, k1, v1, torch.zeros_like(g), beta, zero, chunk_size=32)
    assert c1[:, 0].min() > 0.5
