"""Pins of the gradient oracle, ``oracle.backward.recurrent_bwd`` (CPU only).

The oracle differentiates the per-token update rule of the page "PyPTO-Gym 的 chunk_kda 算子
实战" (section 算子定位与算法背景) with torch autograd in fp64.  These tests tie it to facts
that do not come from it: central finite differences of the independent chunked fp64
forward (``oracle.chunked_fwd``, numpy, sections M1-M4) in random directions, and closed
forms (one token from a zero state; beta = 0, where the state only decays).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.backward import recurrent_bwd, norm_ratio
from chunked_gated_delta_chunk_amd.synth import make_inputs


def _loss(o, S, do, dht):
    return float(np.sum(o * do) + np.sum(S * dht))


def _fd_check(inp, do, dht, scale, chunk, l2n, rng, eps=1e-6):
    """Directional derivatives of L = <o, do> + <S, dht> by central differences of the
    chunked forward, against the oracle's gradients, for every input."""
    x = {n: getattr(inp, n).double().numpy() for n in ("q", "k", "v", "g", "beta")}
    x["h0"] = inp.initial_state.double().numpy()
    grads = recurrent_bwd(inp.q, inp.k, inp.v, inp.g, inp.beta, torch.from_numpy(do),
                          dht=torch.from_numpy(dht), scale=scale,
                          initial_state=inp.initial_state, cu_seqlens=inp.cu_seqlens,
                          use_qk_l2norm=l2n)
    gname = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}

    def L(y):
        o, S = oracle.chunked_fwd(y["q"], y["k"], y["v"], y["g"], y["beta"], scale=scale,
                                  initial_state=y["h0"], cu_seqlens=inp.cu_seqlens,
                                  chunk_size=chunk, use_qk_l2norm=l2n)
        return _loss(o, S, do, dht)

    for name in x:
        u = rng.standard_normal(x[name].shape)
        yp = dict(x)
        ym = dict(x)
        yp[name] = x[name] + eps * u
        ym[name] = x[name] - eps * u
        fd = (L(yp) - L(ym)) / (2 * eps)
        an = float(np.sum(grads[gname[name]] * u))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}: fd {fd} vs grad {an}"


@pytest.mark.parametrize("per_dim,HV,l2n,lengths", [
    (True, None, False, None),
    (False, None, False, None),
    (True, 4, True, None),
    (True, 2, False, (3, 0, 6)),
])
def test_gradients_match_finite_differences_of_chunked_forward(per_dim, HV, l2n, lengths):
    rng = np.random.default_rng(7)
    H, K, V = 2, 8, 5
    if lengths is None:
        inp = make_inputs(2, 9, H, K, V, seed=61, per_dim_gate=per_dim, initial_state=True,
                          HV=HV, normalise=not l2n, gate_mean=1.0)
        N, B, T = 2, 2, 9
    else:
        inp = make_inputs(1, sum(lengths), H, K, V, seed=62, per_dim_gate=per_dim,
                          initial_state=True, HV=HV, lengths=lengths, normalise=not l2n)
        N, B, T = len(lengths), 1, sum(lengths)
    hv = HV or H
    do = rng.standard_normal((B, T, hv, V))
    dht = rng.standard_normal((N, hv, V, K))
    _fd_check(inp, do, dht, 0.4, 4, l2n, rng)


def test_single_token_from_zero_state_closed_form():
    """o = scale beta (q.k) v: dq = scale beta (v.do) k, dk = scale beta (v.do) q,
    dv = scale beta (q.k) do, dbeta = scale (q.k)(v.do); the decay of a zero state has
    no effect, so dg = 0."""
    inp = make_inputs(1, 1, 1, 8, 6, seed=63)
    rng = np.random.default_rng(3)
    do = rng.standard_normal((1, 1, 1, 6))
    s = 0.7
    gr = recurrent_bwd(inp.q, inp.k, inp.v, inp.g, inp.beta, torch.from_numpy(do), scale=s)
    q, k, v = (getattr(inp, n).double().numpy()[0, 0, 0] for n in ("q", "k", "v"))
    b = float(inp.beta[0, 0, 0])
    d = do[0, 0, 0]
    np.testing.assert_allclose(gr["dq"][0, 0, 0], s * b * (v @ d) * k, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gr["dk"][0, 0, 0], s * b * (v @ d) * q, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gr["dv"][0, 0, 0], s * b * (q @ k) * d, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gr["dbeta"][0, 0, 0], s * (q @ k) * (v @ d), rtol=1e-12, atol=1e-14)
    assert not gr["dg"].any()


def test_beta_zero_closed_form():
    """beta = 0: S_t = S0 * exp(G_t) along K, o_t = scale (q_t * exp(G_t))^T S0.  Then
    dv = 0, dq_t = scale exp(G_t) * (S0 do_t), dh0 = sum_t scale (q_t exp(G_t)) do_t^T +
    exp(G_T) * dht (as [V, K]), and dg_s = sum over t >= s of the per-token decay terms."""
    T, K, V = 6, 5, 4
    inp = make_inputs(1, T, 1, K, V, seed=64, beta_mode="zero", initial_state=True)
    rng = np.random.default_rng(4)
    do = rng.standard_normal((1, T, 1, V))
    dht = rng.standard_normal((1, 1, V, K))
    s = 0.5
    gr = recurrent_bwd(inp.q, inp.k, inp.v, inp.g, inp.beta, torch.from_numpy(do),
                       dht=torch.from_numpy(dht), scale=s, initial_state=inp.initial_state)
    q = inp.q.double().numpy()[0, :, 0]                  # [T, K]
    G = np.cumsum(inp.g.double().numpy()[0, :, 0], axis=0)
    S0 = inp.initial_state.double().numpy()[0, 0].T      # [K, V]
    d = do[0, :, 0]                                      # [T, V]
    dq = s * np.exp(G) * (d @ S0.T)
    dh0 = (s * (q * np.exp(G)).T @ d).T + dht[0, 0] * np.exp(G[-1])[None, :]
    term = s * q * np.exp(G) * (d @ S0.T)                # d o-loss / d G_t
    term[-1] += np.exp(G[-1]) * np.sum(S0 * dht[0, 0].T, axis=1)
    dg = np.cumsum(term[::-1], axis=0)[::-1]
    np.testing.assert_allclose(gr["dq"][0, :, 0], dq, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gr["dh0"][0, 0], dh0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gr["dg"][0, :, 0], dg, rtol=1e-12, atol=1e-14)
    assert not gr["dv"].any()


def test_norm_ratio():
    ref = np.array([3.0, 4.0])
    assert norm_ratio(ref, ref) == 0.0
    assert abs(norm_ratio(ref + np.array([0.03, 0.04]), ref) - 0.01) < 1e-15
    assert norm_ratio(np.zeros(2), np.zeros(2)) == 0.0
