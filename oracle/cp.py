"""Oracle for the segment summaries of context parallelism: TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the CPU-baseline leg of the benchmark may use it.

The page "flash-linear-attention KCP 精度失效根因排查手册" describes splitting a sequence
over ranks: each rank summarises its segment, the summaries are exchanged and merged, and
each rank then knows the state entering its segment.  The per-token rule of the chunk_kda
page is affine in the initial state, so a segment's summary is the pair (M, X) with

    final = initial @ M + X         (states in the [V, K] layout, M [K, K], X [V, K])

X is the final state from a zero start.  Every row of the state evolves on its own, so
with an identity start (V = K rows, row a = e_a) the final state is M + X: that is the
definition used here, two runs of :func:`oracle.recurrent_fwd`.  The merge composes the
summaries of consecutive segments in order.
"""
import numpy as np

from . import recurrent_fwd


def segment_map(q, k, v, g, beta, scale=None, cu_seqlens=None, use_qk_l2norm=False):
    """(M [N,HV,K,K], X [N,HV,V,K]) in fp64 for every sequence of the batch (V must equal K)."""
    HV, V, K = v.shape[2], v.shape[3], q.shape[3]
    if V != K:
        raise ValueError("the identity start needs V == K")
    N = q.shape[0] if cu_seqlens is None else len(cu_seqlens) - 1
    _, X = recurrent_fwd(q, k, v, g, beta, scale=scale, cu_seqlens=cu_seqlens, use_qk_l2norm=use_qk_l2norm)
    eye = np.broadcast_to(np.eye(K), (N, HV, K, K)).copy()
    _, F = recurrent_fwd(q, k, v, g, beta, scale=scale, initial_state=eye, cu_seqlens=cu_seqlens,
                         use_qk_l2norm=use_qk_l2norm)
    return F - X, X


def merge(M, X, initial_state=None):
    """s_in [R+1, HV, V, K]: s_in[0] = initial_state (or 0), s_in[r+1] = s_in[r] @ M[r] + X[r]."""
    M = np.asarray(M, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    R, HV, V, K = X.shape
    out = np.zeros((R + 1, HV, V, K))
    if initial_state is not None:
        out[0] = np.asarray(initial_state, dtype=np.float64)
    for r in range(R):
        out[r + 1] = out[r] @ M[r] + X[r]
    return out
