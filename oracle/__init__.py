"""Oracle for the chunked gated delta-rule forward: TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package. The product path (the HIP library and its Python
binding) never calls it and has no CPU fallback.

Two independent fp64 formulations, both written from the page
"PyPTO-Gym 的 chunk_kda 算子实战":

* :func:`recurrent_fwd` -- the per-token update rule (section 算子定位与算法背景),
  in plain C (``recurrent.c``), OpenMP over the independent
  (sequence, head) chains.  This is the reference every GPU result is
  compared with.
* :func:`chunked_fwd` -- the chunked algorithm of sections M1-M4 of the same
  page, in numpy (``chunked.py``).  It is used to cross-check the recurrent
  form and shares no code with it.
* :func:`recurrent_pool_fwd` -- the decode-side use of the same recurrence
  (section 与其他 KDA 算子的关系): start states gathered from a state pool by
  slot index, results scattered back in place, with the per-position states
  of speculative decoding (``decode.py``).

Pins (tests/test_oracle.py) tie both to facts that do not come from either
implementation: closed forms (beta = 0, g = beta = 0, a single token, one-hot
keys), the delta rule as one gradient step (checked with autograd), the
write invariant, varlen and continuation identities, and a hand-derived
three-token example under tests/golden/.
"""
import ctypes
import os

import numpy as np

from . import build as _build
from .chunked import chunked_fwd  # noqa: F401  (re-export)

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        lib.oracle_recurrent_fwd.restype = ctypes.c_int
        lib.oracle_recurrent_fwd.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int,
        ]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the C oracle uses by default (OpenMP max threads)."""
    return _load().oracle_num_threads()


def _bf16_bits(x):
    """Raw bf16 bit patterns (uint16 ndarray) of a torch bf16 tensor or a uint16 ndarray."""
    if isinstance(x, np.ndarray):
        if x.dtype != np.uint16:
            raise TypeError("numpy inputs for bf16 tensors must hold uint16 bit patterns")
        return np.ascontiguousarray(x)
    import torch
    if x.dtype != torch.bfloat16:
        raise TypeError(f"expected a bf16 tensor, got {x.dtype}")
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _f32(x):
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.float32)
    return x.detach().cpu().contiguous().float().numpy()


def _f64(x):
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.float64)
    return x.detach().cpu().contiguous().double().numpy()


def recurrent_fwd(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                  threads=0, use_qk_l2norm=False):
    """fp64 per-token recurrence.

    Shapes follow the page's I/O table: q, k ``[B,T,Hk,K]`` bf16; v ``[B,T,H,V]``
    bf16 with H a multiple of Hk (value head h reads key head ``h // (H // Hk)``); g
    ``[B,T,H,K]`` (per-dimension) or ``[B,T,H]`` (per-head) fp32; beta ``[B,T,H]``
    fp32; initial_state ``[N,H,V,K]`` (any float dtype, widened to fp64) or None;
    cu_seqlens ``[N+1]`` int32 or None (then N = B).  With ``use_qk_l2norm`` q and k
    are normalised per token, ``x / sqrt(|x|^2 + 1e-6)``.

    Returns ``(o, S)`` as fp64 numpy arrays: o ``[B,T,H,V]``, S ``[N,H,V,K]``.
    ``scale=None`` means ``K ** -0.5``.
    """
    qb, kb, vb = _bf16_bits(q), _bf16_bits(k), _bf16_bits(v)
    B, T, Hk, K = qb.shape
    H, V = vb.shape[2], vb.shape[-1]
    if kb.shape != (B, T, Hk, K) or vb.shape[:2] != (B, T) or H % Hk:
        raise ValueError("q/k/v shape mismatch")
    gf = _f32(g)
    if gf.shape == (B, T, H, K):
        per_dim = 1
    elif gf.shape == (B, T, H):
        per_dim = 0
    else:
        raise ValueError(f"bad gate shape {gf.shape}")
    bf = _f32(beta)
    if bf.shape != (B, T, H):
        raise ValueError("bad beta shape")
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu")
                                             else cu_seqlens), dtype=np.int32)
        N = cu.shape[0] - 1
    else:
        cu = None
        N = B
    s0 = None
    if initial_state is not None:
        s0 = _f64(initial_state)
        if s0.shape != (N, H, V, K):
            raise ValueError(f"bad initial_state shape {s0.shape}")
    if scale is None:
        scale = K ** -0.5
    o = np.zeros((B, T, H, V), dtype=np.float64)
    s = np.zeros((N, H, V, K), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    rc = _load().oracle_recurrent_fwd(B, T, Hk, H, K, V, N, per_dim, int(bool(use_qk_l2norm)),
                                      ptr(qb), ptr(kb), ptr(vb),
                                      ptr(gf), ptr(bf), ptr(s0), ptr(cu), float(scale),
                                      ptr(o), ptr(s), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_recurrent_fwd failed with code {rc}")
    return o, s


from .decode import recurrent_pool_fwd  # noqa: E402,F401  (re-export; needs recurrent_fwd above)
