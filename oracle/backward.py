"""Oracle for the gradients of the gated delta-rule forward: TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the CPU-baseline leg of the benchmark may use it.

The gradients are those of the per-token update rule of the page "PyPTO-Gym 的 chunk_kda
算子实战" (section 算子定位与算法背景), taken by reverse-mode automatic differentiation of
that rule written out in fp64 torch on the CPU: no hand-derived gradient formula is
involved.  The loss whose gradients are returned is

    L = sum(o * do) + sum(S_final * dht)

so that, for upstream gradients do (of the output) and dht (of the final state), the
results are the vector-Jacobian products a training step needs: dq, dk, dv, dg, dbeta
and dh0 (of the initial state).  The page "flash-linear-attention KCP 精度失效根因排查手册"
(section 验收标准) states the acceptance rule for such gradients against a per-token
reference: the norm ratio |x - ref| / |ref| of every gradient below 5e-3.

Inputs may be bf16 or any float dtype; they are widened to fp64 exactly.  With grouped
value heads (HV value heads on H query/key heads) dq and dk sum over the value heads of
each group, as the forward reads q and k once per value head.
"""
import numpy as np
import torch


def _f64(x):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return torch.from_numpy(np.asarray(x, dtype=np.float64))
    return x.detach().cpu().double()


def recurrent_bwd(q, k, v, g, beta, do, dht=None, scale=None, initial_state=None,
                  cu_seqlens=None, use_qk_l2norm=False):
    """fp64 gradients of the per-token forward.

    q, k ``[B,T,H,K]``; v ``[B,T,HV,V]``; g ``[B,T,HV,K]`` (per-dimension) or ``[B,T,HV]``
    (per-head); beta ``[B,T,HV]``; do ``[B,T,HV,V]``; dht and initial_state ``[N,HV,V,K]``
    or None; cu_seqlens ``[N+1]`` or None (then N = B).  ``scale=None`` means ``K ** -0.5``.
    With ``use_qk_l2norm`` q and k are normalised per token, ``x / sqrt(|x|^2 + 1e-6)``,
    and the gradients are those of the raw inputs.

    Returns a dict of fp64 numpy arrays with the shapes of the inputs: ``dq``, ``dk``,
    ``dv``, ``dg``, ``dbeta`` and ``dh0`` (zeros when there is no initial state).
    """
    q, k, v, g, beta, do = (_f64(t) for t in (q, k, v, g, beta, do))
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    grp = HV // H
    per_dim = g.dim() == 4
    if scale is None:
        scale = K ** -0.5
    if cu_seqlens is not None:
        cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        seqs = [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    else:
        seqs = [(b, 0, T) for b in range(B)]
    N = len(seqs)
    h0 = _f64(initial_state) if initial_state is not None else torch.zeros(N, HV, V, K, dtype=torch.float64)
    dht = _f64(dht) if dht is not None else torch.zeros(N, HV, V, K, dtype=torch.float64)
    leaves = [t.clone().requires_grad_(True) for t in (q, k, v, g, beta, h0)]
    ql, kl, vl, gl, bl, hl = leaves

    loss = torch.zeros((), dtype=torch.float64)
    for n, (b, s, e) in enumerate(seqs):
        S = hl[n].transpose(-1, -2)                    # [HV, K, V]
        for t in range(s, e):
            qt, kt = ql[b, t], kl[b, t]                # [H, K]
            if use_qk_l2norm:
                qt = qt / torch.sqrt((qt * qt).sum(-1, keepdim=True) + 1e-6)
                kt = kt / torch.sqrt((kt * kt).sum(-1, keepdim=True) + 1e-6)
            qt = qt.repeat_interleave(grp, dim=0)      # value head hv reads key head hv // grp
            kt = kt.repeat_interleave(grp, dim=0)
            gt = gl[b, t] if per_dim else gl[b, t][:, None].expand(HV, K)
            S = S * torch.exp(gt)[:, :, None]          # decay along K
            read = torch.einsum("hk,hkv->hv", kt, S)   # on the decayed state
            upd = bl[b, t][:, None] * (vl[b, t] - read)
            S = S + kt[:, :, None] * upd[:, None, :]
            ot = scale * torch.einsum("hk,hkv->hv", qt, S)
            loss = loss + (ot * do[b, t]).sum()
        loss = loss + (S.transpose(-1, -2) * dht[n]).sum()
    grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    out = {}
    for name, gr, leaf in zip(names, grads, leaves):
        out[name] = (torch.zeros_like(leaf) if gr is None else gr).detach().numpy()
    if initial_state is None:
        out["dh0"] = np.zeros_like(out["dh0"])
    return out


def norm_ratio(x, ref):
    """|x - ref| / |ref| over the whole tensor (Frobenius norms); 0 when both are zero."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
