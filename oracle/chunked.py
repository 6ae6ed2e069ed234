"""Oracle, chunked formulation (test infrastructure only), in fp64 numpy.

Written from sections M1-M4 of the page "PyPTO-Gym 的 chunk_kda 算子实战"
(算法原理: chunk 内求逆, chunk 间状态递推), one chunk at a time, with the readings
below where the page's text is garbled or silent:

M1  split the sequence into chunks of ``chunk_size`` tokens (chunks restart at
    every sequence start); multiply q by ``scale``; gamma = inclusive prefix sum
    of g inside the chunk.
M2  A_full[i, j] = sum_d k[i,d] k[j,d] exp(gamma[i,d] - gamma[j,d]); keep the
    strictly lower part and multiply row i by beta[i]; invert (I + A) with a
    triangular solve (the page's golden uses a triangular solve as well).
M3  w = (I + A)^-1 diag(beta) (exp(gamma) * k),  u = (I + A)^-1 diag(beta) v.
    The page writes only "A_inv" here and puts beta on A's rows; the per-token
    rule forces the right-hand sides to carry diag(beta) too (reading 1).
M4  v_new = u - w S;  o = (q * exp(gamma) * scale) S + A2 v_new;
    S <- exp(gamma_last) * S + (exp(gamma_last - gamma) * k)^T v_new, where
    A2[i, j] = scale * sum_d q[i,d] k[j,d] exp(gamma[i,d] - gamma[j,d]) for
    j <= i, diagonal included, because the output reads the state after the
    update (reading 2; the page does not define A2).

With a log-domain forget gate (g <= 0) every exponent evaluated here is <= 0:
gamma itself, gamma_last - gamma, and gamma_i - gamma_j for j <= i (pairs with
j > i are masked before the exponential), so nothing overflows.  Tail chunks
simply have fewer rows, which is what zero-padding the missing rows amounts to.
"""
import numpy as np
from scipy.linalg import solve_triangular


def _as_f64(x):
    if isinstance(x, np.ndarray):
        return x.astype(np.float64)
    return x.detach().cpu().double().numpy()


def _chunk(q, k, v, g, beta, S, scale, detail=False):
    """One chunk of one head. q, k, g: [n, K]; v: [n, V]; beta: [n]; S: [K, V].
    Returns (o, S_next), and also u and v_new when ``detail``."""
    n, K = k.shape
    gam = np.cumsum(g, axis=0)                                   # M1
    diff = gam[:, None, :] - gam[None, :, :]                     # [i, j, d]
    lower_incl = np.tril(np.ones((n, n), dtype=bool))
    decay = np.exp(np.where(lower_incl[:, :, None], diff, -np.inf))
    A = np.einsum("id,jd,ijd->ij", k, k, decay)                  # M2
    A = np.tril(A, -1) * beta[:, None]
    rhs_k = beta[:, None] * (np.exp(gam) * k)
    rhs_v = beta[:, None] * v
    L = np.eye(n) + A
    w = solve_triangular(L, rhs_k, lower=True, unit_diagonal=True)   # M3
    u = solve_triangular(L, rhs_v, lower=True, unit_diagonal=True)
    A2 = scale * np.einsum("id,jd,ijd->ij", q, k, decay)          # inclusive lower
    v_new = u - w @ S                                            # M4
    o = (scale * q * np.exp(gam)) @ S + A2 @ v_new
    g_last = gam[-1]
    S_next = np.exp(g_last)[:, None] * S + (np.exp(g_last[None, :] - gam) * k).T @ v_new
    if detail:
        return o, S_next, u, v_new
    return o, S_next


def chunked_fwd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                chunk_size=64, use_qk_l2norm=False):
    """fp64 chunked forward. Same argument conventions and return values as
    :func:`oracle.recurrent_fwd`: o ``[B,T,H,V]`` and S ``[N,H,V,K]`` (fp64)."""
    q, k, v, g, beta = (_as_f64(x) for x in (q, k, v, g, beta))
    if use_qk_l2norm:   # per token over K, before anything else
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-6)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + 1e-6)
    if v.shape[2] != q.shape[2]:   # grouped value heads: key head h // group for value head h
        grp = v.shape[2] // q.shape[2]
        q, k = np.repeat(q, grp, axis=2), np.repeat(k, grp, axis=2)
    B, T, H, K = q.shape
    V = v.shape[-1]
    if g.ndim == 3:                                   # per-head gate, same for every d
        g = np.broadcast_to(g[..., None], (B, T, H, K))
    if scale is None:
        scale = K ** -0.5
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
                        dtype=np.int64)
        assert B == 1
        bounds = [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    else:
        bounds = [(b, 0, T) for b in range(B)]
    N = len(bounds)
    o = np.zeros((B, T, H, V))
    S_out = np.zeros((N, H, V, K))
    s0 = None if initial_state is None else _as_f64(initial_state)
    for n, (b, bos, eos) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((K, V)) if s0 is None else s0[n, h].T.copy()
            for c0 in range(bos, eos, chunk_size):
                c1 = min(c0 + chunk_size, eos)
                oc, S = _chunk(q[b, c0:c1, h], k[b, c0:c1, h], v[b, c0:c1, h],
                               g[b, c0:c1, h], beta[b, c0:c1, h], S, scale)
                o[b, c0:c1, h] = oc
            S_out[n, h] = S.T
    return o, S_out


def cancellation(q, k, v, g, beta, initial_state, chunk_size=64, scale=None):
    """How much the state's prediction cancels in section M4's v_new = u - w S, per chunk:
    ``|v_new| / |u|`` (Frobenius norms over the chunk), fp64, shape [H, chunks], for one
    fixed-length sequence (B = 1) without grouped heads.  Used to choose adversarial inputs
    (the page's cancellation_stress mode); it defines no expected value."""
    q, k, v, g, beta = (_as_f64(x)[0] for x in (q, k, v, g, beta))
    T, H, K = q.shape
    if scale is None:
        scale = K ** -0.5
    s0 = _as_f64(initial_state)[0]
    out = []
    for h in range(H):
        S = s0[h].T.copy()
        row = []
        for c0 in range(0, T, chunk_size):
            c1 = min(c0 + chunk_size, T)
            _, S, u, vn = _chunk(q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], g[c0:c1, h], beta[c0:c1, h],
                                 S, scale, detail=True)
            row.append(np.linalg.norm(vn) / max(np.linalg.norm(u), 1e-300))
        out.append(row)
    return np.asarray(out)
