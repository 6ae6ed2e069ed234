"""Oracle for the per-token forward against a pool of states: TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the CPU-baseline leg of the benchmark may use it.

The page "PyPTO-Gym 的 chunk_kda 算子实战" (section 与其他 KDA 算子的关系) describes the
decode-side companion of the chunked operator: the same per-token recurrence over an
fp32 [H, V, K] state, with the state kept in place in a pool addressed by
``ssm_state_indices`` and speculative decoding steered by ``num_accepted_tokens``.  The
page names these arguments without defining them; this module takes the plainest
reading (stated once more in the project's design notes):

* ``ssm_state_indices`` of shape [N]: sequence n starts from pool slot idx[n] and its
  state after its last token is written back to the same slot.
* ``ssm_state_indices`` of shape [N, L] (speculative decoding): every draft position
  has its own slot.  Sequence n starts from slot idx[n, a_n - 1], a_n =
  ``num_accepted_tokens[n]`` (1 when not given), the state after the a_n-th token that
  the previous step accepted; the state after its own t-th token (t = 0, 1, ...) is
  written to slot idx[n, t] (positions t >= L have no slot and are not stored).
* A slot index outside [0, num_slots) marks a padding entry: a start index outside it
  (or a_n outside 1..L) makes the whole sequence padding, whose outputs are zero and
  which reads and writes no state; a write index outside it skips that write.
* Every start state is read before any state is written, so a sequence may write the
  slot it started from.  Two sequences writing the same slot is not defined.

The recurrence itself is :func:`oracle.recurrent_fwd`, run on each sequence's tokens
(and, for the per-position states of speculative decoding, on each prefix of them:
the state after t + 1 tokens is by definition that of running those t + 1 tokens).
Nothing here reorders or fuses the recurrence; this module only gathers start states
and scatters results.
"""
import numpy as np

from . import recurrent_fwd


def _as_np(x, dtype):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=dtype)


def _sequences(B, T, cu):
    """(batch row, first token, end token) of every sequence."""
    if cu is None:
        return [(b, 0, T) for b in range(B)]
    return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def recurrent_pool_fwd(q, k, v, g, beta, state_pool, ssm_state_indices,
                       num_accepted_tokens=None, scale=None, cu_seqlens=None,
                       use_qk_l2norm=False):
    """fp64 per-token forward against a state pool (readings in the module docstring).

    q, k ``[B,T,H,K]`` bf16; v ``[B,T,HV,V]`` bf16; g ``[B,T,HV,K]`` or ``[B,T,HV]`` fp32;
    beta ``[B,T,HV]`` fp32; state_pool ``[P,HV,V,K]`` (widened to fp64); ssm_state_indices
    int ``[N]`` or ``[N,L]``; num_accepted_tokens int ``[N]`` or None; cu_seqlens ``[N+1]``
    or None (then N = B).

    Returns ``(o, pool)``: o ``[B,T,HV,V]`` fp64 (zero on padding sequences) and the pool
    after the call as a new fp64 array (the input is not modified).
    """
    pool_in = _as_np(state_pool, np.float64)
    pool = pool_in.copy()
    P = pool.shape[0]
    idx = _as_np(ssm_state_indices, np.int64)
    acc = _as_np(num_accepted_tokens, np.int64)
    cu = _as_np(cu_seqlens, np.int64)
    B, T = q.shape[0], q.shape[1]
    HV, V = v.shape[2], v.shape[3]
    seqs = _sequences(B, T, cu)
    if idx.shape[0] != len(seqs):
        raise ValueError("ssm_state_indices needs one row per sequence")
    spec = idx.ndim == 2
    L = idx.shape[1] if spec else 1

    # start slots, read before anything is written
    starts = []
    for n in range(len(seqs)):
        if spec:
            a = 1 if acc is None else int(acc[n])
            r = int(idx[n, a - 1]) if 1 <= a <= L else -1
        else:
            r = int(idx[n])
        starts.append(r if 0 <= r < P else None)
    init = [None if r is None else pool_in[r].copy() for r in starts]

    o = np.zeros((B, T, HV, V), dtype=np.float64)
    writes = []
    for n, (b, s, e) in enumerate(seqs):
        if starts[n] is None:
            continue
        part = lambda x, t1: x[b:b + 1, s:t1]  # noqa: E731
        o_n, S_n = recurrent_fwd(part(q, e), part(k, e), part(v, e), part(g, e), part(beta, e),
                                 scale=scale, initial_state=init[n][None],
                                 use_qk_l2norm=use_qk_l2norm)
        o[b, s:e] = o_n[0]
        if not spec:
            writes.append((starts[n], S_n[0]))
            continue
        for t in range(min(e - s, L)):
            w = int(idx[n, t])
            if not 0 <= w < P:
                continue
            if s + t + 1 == e:
                S_t = S_n[0]
            else:
                _, S_p = recurrent_fwd(part(q, s + t + 1), part(k, s + t + 1), part(v, s + t + 1),
                                       part(g, s + t + 1), part(beta, s + t + 1), scale=scale,
                                       initial_state=init[n][None], use_qk_l2norm=use_qk_l2norm)
                S_t = S_p[0]
            writes.append((w, S_t))
    for w, S in writes:
        pool[w] = S
    return o, pool
