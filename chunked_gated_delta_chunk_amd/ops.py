"""Python binding of the C interface declared in include/chunk_dr.h.

Argument marshalling only: dtype and shape checks, allocation of the outputs and the
workspace with torch, and one call into libchunkdr.so on the current stream.  Every
step of the forward runs in the HIP kernels; there is no fallback of any kind, and
calling without the built library raises.
"""
import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libchunkdr.so")

CDR_OK = 0
_STATUS_EXC = {1: ValueError, 2: ValueError, 3: ValueError, 4: ValueError, 5: RuntimeError,
               6: RuntimeError, 7: ValueError}
GATE_PER_DIM = 0
GATE_PER_HEAD = 1

EXPORTED = ("cdr_check", "cdr_workspace_bytes", "chunk_dr_fwd", "chunk_dr_fwd_stages",
            "chunk_dr_fwd_noalloc",
            "cdr_bwd_workspace_bytes", "chunk_dr_bwd", "chunk_dr_bwd_stages",
            "chunk_dr_segment_map", "chunk_dr_merge_states",
            "cdr_recurrent_check", "chunk_dr_recurrent_fwd", "cdr_check_cu_seqlens", "cdr_status_str",
            "cdr_version")
STATE_SEPARATE, STATE_POOL, STATE_POOL_SPEC = 0, 1, 2
STAGE_INTRA, STAGE_CHAIN, STAGE_OUTPUT, STAGE_ALL = 1, 2, 4, 7
NOALLOC_SCRATCH_BYTES = 256 * 1024 * 1024   # CDR_NOALLOC_SCRATCH_BYTES of chunk_dr.h
BWD_PREP, BWD_CHAINS, BWD_LOCAL, BWD_ALL = 1, 2, 4, 7


class cdr_problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("N", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("scale", ctypes.c_float), ("has_initial_state", ctypes.c_int32),
                ("output_final_state", ctypes.c_int32), ("varlen", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32)]


class cdr_recurrent_problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("HV", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
                ("N", ctypes.c_int32), ("gate", ctypes.c_int32), ("scale", ctypes.c_float),
                ("varlen", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32),
                ("state_mode", ctypes.c_int32), ("has_initial_state", ctypes.c_int32),
                ("output_final_state", ctypes.c_int32), ("num_slots", ctypes.c_int32),
                ("index_cols", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libchunkdr.so (built by chunked_gated_delta_chunk_amd.build); raise if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m chunked_gated_delta_chunk_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(cdr_problem)
    vp = ctypes.c_void_p
    lib.cdr_check.argtypes = [P]
    lib.cdr_check.restype = ctypes.c_int
    lib.cdr_workspace_bytes.argtypes = [P]
    lib.cdr_workspace_bytes.restype = ctypes.c_size_t
    lib.chunk_dr_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.chunk_dr_fwd.restype = ctypes.c_int
    lib.chunk_dr_fwd_stages.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                        ctypes.c_int32, vp]
    lib.chunk_dr_fwd_stages.restype = ctypes.c_int
    lib.chunk_dr_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.chunk_dr_fwd_noalloc.restype = ctypes.c_int
    lib.cdr_bwd_workspace_bytes.argtypes = [P]
    lib.cdr_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.chunk_dr_bwd.argtypes = [P] + [vp] * 16 + [ctypes.c_size_t, vp]
    lib.chunk_dr_bwd.restype = ctypes.c_int
    lib.chunk_dr_bwd_stages.argtypes = [P] + [vp] * 16 + [ctypes.c_size_t, ctypes.c_int32, vp]
    lib.chunk_dr_bwd_stages.restype = ctypes.c_int
    lib.chunk_dr_segment_map.argtypes = [P] + [vp] * 8 + [ctypes.c_size_t, vp]
    lib.chunk_dr_segment_map.restype = ctypes.c_int
    lib.chunk_dr_merge_states.argtypes = [ctypes.c_int32] * 4 + [vp] * 5
    lib.chunk_dr_merge_states.restype = ctypes.c_int
    R = ctypes.POINTER(cdr_recurrent_problem)
    lib.cdr_recurrent_check.argtypes = [R]
    lib.cdr_recurrent_check.restype = ctypes.c_int
    lib.chunk_dr_recurrent_fwd.argtypes = [R] + [vp] * 13
    lib.chunk_dr_recurrent_fwd.restype = ctypes.c_int
    lib.cdr_check_cu_seqlens.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.cdr_check_cu_seqlens.restype = ctypes.c_int
    lib.cdr_status_str.argtypes = [ctypes.c_int]
    lib.cdr_status_str.restype = ctypes.c_char_p
    lib.cdr_version.argtypes = []
    lib.cdr_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _raise(status: int, what: str):
    lib = load_library()
    msg = lib.cdr_status_str(status).decode()
    raise _STATUS_EXC.get(status, RuntimeError)(f"{what}: {msg} (status {status})")


def make_problem(B, T, H, K, V, N, per_dim_gate, chunk_size, scale, has_initial_state,
                 output_final_state, varlen, HV=0, qk_l2norm=False) -> cdr_problem:
    return cdr_problem(int(B), int(T), int(H), int(K), int(V), int(N),
                       GATE_PER_DIM if per_dim_gate else GATE_PER_HEAD, int(chunk_size),
                       float(scale), int(bool(has_initial_state)), int(bool(output_final_state)),
                       int(bool(varlen)), int(HV), int(bool(qk_l2norm)))


def check(p: cdr_problem) -> int:
    """cdr_check: host-only validation status."""
    return load_library().cdr_check(ctypes.byref(p))


def workspace_bytes(p: cdr_problem) -> int:
    return load_library().cdr_workspace_bytes(ctypes.byref(p))


def _need(t, name, dtype, shape=None, dense=False):
    """Type and shape of an argument; `dense` for a buffer the kernels write (an output or the
    workspace), which must be contiguous since the library addresses it row-major."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (the kernels write it row-major)")


def _aligned(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """t as a contiguous tensor whose data is 16-byte aligned (a copy when a view is not)."""
    if t is None:
        return None
    t = t.contiguous()
    return t if t.data_ptr() % 16 == 0 else t.clone()


def _dev_ptr(t: torch.Tensor, device) -> int:
    if t.device != device:
        raise ValueError(f"tensor on {t.device}, expected {device}")
    if t.data_ptr() % 16:
        raise ValueError("tensor data must be 16-byte aligned")
    return t.data_ptr()


class PreparedForward:
    """A validated call of the forward whose arguments are marshalled once.

    Construction takes the same arguments as :func:`chunk_dr_fwd` and allocates the
    outputs and the workspace unless they are given; each call then queues the kernels
    (``stages`` as in chunk_dr_fwd_stages) on the current stream with a single ctypes
    call, so repeated launches carry no per-call host work beyond it.
    """

    def __init__(self, q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                 chunk_size=64, output_final_state=False, workspace=None, out=None,
                 final_state_out=None, use_qk_l2norm_in_kernel=False, noalloc=False):
        lib = load_library()
        _need(q, "q", torch.bfloat16)
        if q.dim() != 4:
            raise ValueError("q must be [B, T, H, K]")
        B, T, H, K = q.shape
        _need(k, "k", torch.bfloat16, (B, T, H, K))
        if v.dim() != 4 or tuple(v.shape[:2]) != (B, T) or v.shape[2] % H:
            raise ValueError("v must be [B, T, HV, V] with HV a multiple of the q/k heads")
        _need(v, "v", torch.bfloat16)
        HV, V = v.shape[2], v.shape[3]
        _need(g, "g", torch.float32)
        if tuple(g.shape) == (B, T, HV, K):
            per_dim = True
        elif tuple(g.shape) == (B, T, HV):
            per_dim = False
        else:
            raise ValueError(f"g must be [B,T,HV,K] or [B,T,HV], got {tuple(g.shape)}")
        _need(beta, "beta", torch.float32, (B, T, HV))
        if cu_seqlens is not None:
            _need(cu_seqlens, "cu_seqlens", torch.int32)
            if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
                raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
            N = cu_seqlens.numel() - 1
        else:
            N = B
        if initial_state is not None:
            _need(initial_state, "initial_state", torch.float32, (N, HV, V, K))
        if scale is None:
            scale = K ** -0.5
        self.problem = make_problem(B, T, H, K, V, N, per_dim, chunk_size, scale,
                                    initial_state is not None, output_final_state,
                                    cu_seqlens is not None, HV, use_qk_l2norm_in_kernel)
        st = lib.cdr_check(ctypes.byref(self.problem))
        if st != CDR_OK:
            _raise(st, "chunk_dr_fwd")
        if out is not None:
            _need(out, "out", torch.bfloat16, (B, T, HV, V), dense=True)
        if output_final_state and final_state_out is not None:
            _need(final_state_out, "final_state_out", torch.float32, (N, HV, V, K), dense=True)
        device = q.device
        if device.type != "cuda":
            raise ValueError("inputs must be on a GPU device")
        self.device = device
        # keep references: the library reads these buffers when the kernels run
        self.inputs = tuple(_aligned(t) for t in (q, k, v, g, beta))
        self.s0 = _aligned(initial_state)
        self.cu = _aligned(cu_seqlens)
        if out is None:
            out = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=device)
        self.o = out
        self.S = None
        if output_final_state:
            if final_state_out is None:
                final_state_out = torch.empty((N, HV, V, K), dtype=torch.float32, device=device)
            self.S = final_state_out
        ptr = lambda t: None if t is None else _dev_ptr(t, device)  # noqa: E731
        qq, kk, vv, gg, bb = self.inputs
        self.noalloc = bool(noalloc)
        if self.noalloc:
            # the library's static workspace (chunk_dr_fwd_noalloc): none is allocated here
            self.workspace = None
            self._args = (ctypes.byref(self.problem), ptr(qq), ptr(kk), ptr(vv), ptr(gg), ptr(bb),
                          ptr(self.s0), ptr(self.cu), ptr(self.o), ptr(self.S))
        else:
            nbytes = lib.cdr_workspace_bytes(ctypes.byref(self.problem))
            if workspace is None:
                workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
            elif workspace.numel() * workspace.element_size() < nbytes:
                raise ValueError("workspace too small")
            elif not workspace.is_contiguous():
                raise ValueError("workspace must be contiguous")
            self.workspace = workspace
            self._args = (ctypes.byref(self.problem), ptr(qq), ptr(kk), ptr(vv), ptr(gg), ptr(bb),
                          ptr(self.s0), ptr(self.cu), ptr(self.o), ptr(self.S), ptr(workspace),
                          workspace.numel() * workspace.element_size())
        self._lib = lib

    def __call__(self, stages: int = STAGE_ALL):
        stream = torch.cuda.current_stream(self.device).cuda_stream
        if self.noalloc:
            if stages != STAGE_ALL:
                raise ValueError("the no-allocation entry point runs all stages")
            st = self._lib.chunk_dr_fwd_noalloc(*self._args, stream)
            if st != CDR_OK:
                _raise(st, "chunk_dr_fwd_noalloc")
            return self.o, self.S
        if stages == STAGE_ALL:
            st = self._lib.chunk_dr_fwd(*self._args, stream)
        else:
            st = self._lib.chunk_dr_fwd_stages(*self._args, int(stages), stream)
        if st != CDR_OK:
            _raise(st, "chunk_dr_fwd")
        return self.o, self.S


def chunk_dr_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                 beta: torch.Tensor, scale: Optional[float] = None,
                 initial_state: Optional[torch.Tensor] = None,
                 cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                 output_final_state: bool = False,
                 workspace: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None,
                 final_state_out: Optional[torch.Tensor] = None,
                 stages: int = STAGE_ALL,
                 use_qk_l2norm_in_kernel: bool = False,
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked gated delta-rule forward on the GPU.

    q, k ``[B,T,H,K]`` bf16; v ``[B,T,HV,V]`` bf16 with HV a multiple of H (value head hv
    uses query/key head ``hv // (HV // H)``); g ``[B,T,HV,K]`` (per-dimension gate) or
    ``[B,T,HV]`` (per-head gate) fp32; beta ``[B,T,HV]`` fp32; initial_state
    ``[N,HV,V,K]`` fp32 or None (zeros); cu_seqlens ``[N+1]`` int32 on the device, or
    None (then N = B). ``scale=None`` means ``K ** -0.5``.  With
    ``use_qk_l2norm_in_kernel`` q and k are normalised over K per token inside the
    kernels (``x / sqrt(|x|^2 + 1e-6)``).  Returns ``(o, S)`` with o ``[B,T,HV,V]`` bf16
    and S ``[N,HV,V,K]`` fp32 (None unless output_final_state).
    ``workspace`` optionally supplies the device scratch buffer (uint8, at least
    :func:`workspace_bytes` bytes); otherwise one is allocated.  ``out`` and
    ``final_state_out`` optionally supply the output buffers.  ``stages`` selects kernel
    stages as chunk_dr_fwd_stages does (default: all).
    """
    call = PreparedForward(q, k, v, g, beta, scale=scale, initial_state=initial_state,
                           cu_seqlens=cu_seqlens, chunk_size=chunk_size,
                           output_final_state=output_final_state, workspace=workspace, out=out,
                           final_state_out=final_state_out,
                           use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel)
    return call(stages)


def chunk_dr_fwd_noalloc(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                         chunk_size=64, output_final_state=False, out=None, final_state_out=None,
                         use_qk_l2norm_in_kernel=False):
    """:func:`chunk_dr_fwd` through the library's no-allocation entry point: the workspace is the
    library's static device array (at most ``NOALLOC_SCRATCH_BYTES``; larger problems raise
    ValueError).  Pass ``out`` (and ``final_state_out``) to allocate nothing in this call either.
    Calls whose kernels overlap in time on one device share that array and race."""
    call = PreparedForward(q, k, v, g, beta, scale=scale, initial_state=initial_state,
                           cu_seqlens=cu_seqlens, chunk_size=chunk_size,
                           output_final_state=output_final_state, out=out,
                           final_state_out=final_state_out,
                           use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, noalloc=True)
    return call()


def segment_map(q, k, v, g, beta, cu_seqlens=None, chunk_size=64, scale=None,
                use_qk_l2norm_in_kernel=False, workspace=None):
    """Affine summary of every sequence (segment): ``final = initial @ M + X``.

    Arguments as :func:`chunk_dr_fwd`.  Returns fp32 ``M [N,HV,K,K]`` and ``X [N,HV,V,K]``.
    """
    lib = load_library()
    B, T, H, K = q.shape
    HV, V = v.shape[2], v.shape[3]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, T, H, K))
    _need(v, "v", torch.bfloat16)
    _need(g, "g", torch.float32)
    _need(beta, "beta", torch.float32, (B, T, HV))
    per_dim = g.dim() == 4
    N = cu_seqlens.numel() - 1 if cu_seqlens is not None else B
    p = make_problem(B, T, H, K, V, N, per_dim, chunk_size, K ** -0.5 if scale is None else scale,
                     False, True, cu_seqlens is not None, HV, use_qk_l2norm_in_kernel)
    st = lib.cdr_check(ctypes.byref(p))
    if st != CDR_OK:
        _raise(st, "chunk_dr_segment_map")
    device = q.device
    if device.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    nbytes = lib.cdr_workspace_bytes(ctypes.byref(p))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    M = torch.empty((N, HV, K, K), dtype=torch.float32, device=device)
    X = torch.empty((N, HV, V, K), dtype=torch.float32, device=device)
    ins = [_aligned(t) for t in (q, k, v, g, beta)]
    cu = _aligned(cu_seqlens)
    ptr = lambda t: None if t is None else _dev_ptr(t, device)  # noqa: E731
    stream = torch.cuda.current_stream(device).cuda_stream
    st = lib.chunk_dr_segment_map(ctypes.byref(p), *(ptr(t) for t in ins), ptr(cu), ptr(M), ptr(X),
                                  ptr(workspace), workspace.numel() * workspace.element_size(), stream)
    if st != CDR_OK:
        _raise(st, "chunk_dr_segment_map")
    return M, X


def merge_states(M, X, initial_state=None):
    """States entering R consecutive segments from their maps: ``s_in[0] = initial_state``,
    ``s_in[r+1] = s_in[r] @ M[r] + X[r]``.  M ``[R,HV,K,K]``, X ``[R,HV,V,K]``, initial_state
    ``[HV,V,K]`` or None (zeros).  Returns ``s_in [R+1,HV,V,K]`` (the last is the final state)."""
    lib = load_library()
    _need(M, "M", torch.float32)
    _need(X, "X", torch.float32)
    R, HV, K, _ = M.shape
    V = X.shape[2]
    if tuple(X.shape) != (R, HV, V, K):
        raise ValueError("X must be [R, HV, V, K]")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (HV, V, K))
    device = M.device
    s_in = torch.empty((R + 1, HV, V, K), dtype=torch.float32, device=device)
    Mc, Xc = _aligned(M), _aligned(X)          # referenced until the call returns
    s0 = _aligned(initial_state)
    ptr = lambda t: None if t is None else _dev_ptr(t, device)  # noqa: E731
    stream = torch.cuda.current_stream(device).cuda_stream
    st = lib.chunk_dr_merge_states(R, HV, K, V, ptr(Mc), ptr(Xc), ptr(s0), ptr(s_in), stream)
    if st != CDR_OK:
        _raise(st, "chunk_dr_merge_states")
    return s_in


def check_cu_seqlens(cu_seqlens, T) -> int:
    """Checks the contents of ``cu_seqlens`` (int32 ``[N+1]`` on a GPU) on the device, which the
    forward does not: 0 when the offsets start at 0, never decrease and end at ``T``, else
    ``i + 1`` for the first offending index ``i``.  Waits for the current stream (a debugging
    aid, not for the hot path)."""
    lib = load_library()
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 >= 2 offsets")
    device = cu_seqlens.device
    cu = _aligned(cu_seqlens)
    result = torch.empty(4, dtype=torch.int32, device=device)   # 16 bytes: the first is the result
    stream = torch.cuda.current_stream(device)
    st = lib.cdr_check_cu_seqlens(_dev_ptr(cu, device), cu.numel() - 1, int(T), _dev_ptr(result, device),
                                  stream.cuda_stream)
    if st != CDR_OK:
        _raise(st, "cdr_check_cu_seqlens")
    stream.synchronize()
    return int(result[0].item())


def bwd_workspace_bytes(p: cdr_problem) -> int:
    return load_library().cdr_bwd_workspace_bytes(ctypes.byref(p))


class PreparedBackward:
    """A validated call of the backward whose arguments are marshalled once.

    Takes the arguments of :func:`chunk_dr_bwd`, allocates the gradients and the workspace
    unless given, and queues the kernels on the current stream at each call, returning
    ``(dq, dk, dv, dg, dbeta, dh0)``.
    """

    def __init__(self, q, k, v, g, beta, do, dht=None, scale=None, initial_state=None,
                 cu_seqlens=None, chunk_size=64, use_qk_l2norm_in_kernel=False, workspace=None):
        lib = load_library()
        _need(q, "q", torch.bfloat16)
        if q.dim() != 4:
            raise ValueError("q must be [B, T, H, K]")
        B, T, H, K = q.shape
        _need(k, "k", torch.bfloat16, (B, T, H, K))
        if v.dim() != 4 or tuple(v.shape[:2]) != (B, T) or v.shape[2] % H:
            raise ValueError("v must be [B, T, HV, V] with HV a multiple of the q/k heads")
        _need(v, "v", torch.bfloat16)
        HV, V = v.shape[2], v.shape[3]
        _need(g, "g", torch.float32)
        if tuple(g.shape) == (B, T, HV, K):
            per_dim = True
        elif tuple(g.shape) == (B, T, HV):
            per_dim = False
        else:
            raise ValueError(f"g must be [B,T,HV,K] or [B,T,HV], got {tuple(g.shape)}")
        _need(beta, "beta", torch.float32, (B, T, HV))
        _need(do, "do", torch.bfloat16, (B, T, HV, V))
        if cu_seqlens is not None:
            _need(cu_seqlens, "cu_seqlens", torch.int32)
            if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
                raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
            N = cu_seqlens.numel() - 1
        else:
            N = B
        if initial_state is not None:
            _need(initial_state, "initial_state", torch.float32, (N, HV, V, K))
        if dht is not None:
            _need(dht, "dht", torch.float32, (N, HV, V, K))
        if scale is None:
            scale = K ** -0.5
        self.problem = make_problem(B, T, H, K, V, N, per_dim, chunk_size, scale,
                                    initial_state is not None, False, cu_seqlens is not None, HV,
                                    use_qk_l2norm_in_kernel)
        st = lib.cdr_check(ctypes.byref(self.problem))
        if st != CDR_OK:
            _raise(st, "chunk_dr_bwd")
        device = q.device
        if device.type != "cuda":
            raise ValueError("inputs must be on a GPU device")
        self.device = device
        self.inputs = tuple(_aligned(t) for t in (q, k, v, g, beta, do))
        self.s0 = _aligned(initial_state)
        self.dht = _aligned(dht)
        self.cu = _aligned(cu_seqlens)
        f32 = dict(dtype=torch.float32, device=device)
        self.grads = (torch.empty((B, T, H, K), **f32), torch.empty((B, T, H, K), **f32),
                      torch.empty((B, T, HV, V), **f32), torch.empty(tuple(g.shape), **f32),
                      torch.empty((B, T, HV), **f32),
                      torch.empty((N, HV, V, K), **f32) if initial_state is not None else None)
        nbytes = lib.cdr_bwd_workspace_bytes(ctypes.byref(self.problem))
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        elif workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        self.workspace = workspace
        ptr = lambda t: None if t is None else _dev_ptr(t, device)  # noqa: E731
        qq, kk, vv, gg, bb, dd = self.inputs
        self._args = (ctypes.byref(self.problem), ptr(qq), ptr(kk), ptr(vv), ptr(gg), ptr(bb),
                      ptr(self.s0), ptr(self.cu), ptr(dd), ptr(self.dht),
                      *(ptr(t) for t in self.grads), ptr(workspace),
                      workspace.numel() * workspace.element_size())
        self._lib = lib

    def __call__(self, stages: int = BWD_ALL):
        stream = torch.cuda.current_stream(self.device).cuda_stream
        if stages == BWD_ALL:
            st = self._lib.chunk_dr_bwd(*self._args, stream)
        else:
            st = self._lib.chunk_dr_bwd_stages(*self._args, int(stages), stream)
        if st != CDR_OK:
            _raise(st, "chunk_dr_bwd")
        return self.grads


def chunk_dr_bwd(q, k, v, g, beta, do, dht=None, scale=None, initial_state=None, cu_seqlens=None,
                 chunk_size=64, use_qk_l2norm_in_kernel=False, workspace=None):
    """Gradients of the chunked forward on the GPU.

    Arguments as :func:`chunk_dr_fwd`, plus ``do`` ``[B,T,HV,V]`` bf16 (gradient of o) and
    ``dht`` ``[N,HV,V,K]`` fp32 or None (gradient of the final state).  Returns fp32
    ``(dq, dk, dv, dg, dbeta, dh0)`` with the shapes of q, k, v, g, beta and initial_state
    (dh0 is None without an initial state); dq and dk sum over grouped value heads.
    """
    return PreparedBackward(q, k, v, g, beta, do, dht=dht, scale=scale, initial_state=initial_state,
                            cu_seqlens=cu_seqlens, chunk_size=chunk_size,
                            use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel, workspace=workspace)()


class PreparedRecurrent:
    """A validated call of the per-token forward whose arguments are marshalled once.

    Takes the arguments of :func:`fused_recurrent_fwd`; each call queues the kernel on the
    current stream with a single ctypes call and returns ``(o, S)``.  In the pool modes every
    call updates the pool in place again.
    """

    def __init__(self, q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False,
                 cu_seqlens=None, use_qk_l2norm_in_kernel=False, state_pool=None,
                 ssm_state_indices=None, num_accepted_tokens=None, out=None, final_state_out=None):
        lib = load_library()
        _need(q, "q", torch.bfloat16)
        if q.dim() != 4:
            raise ValueError("q must be [B, T, H, K]")
        B, T, H, K = q.shape
        _need(k, "k", torch.bfloat16, (B, T, H, K))
        if v.dim() != 4 or tuple(v.shape[:2]) != (B, T) or v.shape[2] % H:
            raise ValueError("v must be [B, T, HV, V] with HV a multiple of the q/k heads")
        _need(v, "v", torch.bfloat16)
        HV, V = v.shape[2], v.shape[3]
        _need(g, "g", torch.float32)
        if tuple(g.shape) == (B, T, HV, K):
            per_dim = True
        elif tuple(g.shape) == (B, T, HV):
            per_dim = False
        else:
            raise ValueError(f"g must be [B,T,HV,K] or [B,T,HV], got {tuple(g.shape)}")
        _need(beta, "beta", torch.float32, (B, T, HV))
        if cu_seqlens is not None:
            _need(cu_seqlens, "cu_seqlens", torch.int32)
            if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
                raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
            N = cu_seqlens.numel() - 1
        else:
            N = B
        if scale is None:
            scale = K ** -0.5
        num_slots, cols = 0, 0
        if state_pool is not None:
            if initial_state is not None or output_final_state:
                raise ValueError("state_pool replaces initial_state and output_final_state")
            _need(state_pool, "state_pool", torch.float32)
            if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (HV, V, K):
                raise ValueError(f"state_pool must be [P, {HV}, {V}, {K}]")
            if not state_pool.is_contiguous():
                raise ValueError("state_pool must be contiguous (it is updated in place)")
            if ssm_state_indices is None:
                raise ValueError("state_pool needs ssm_state_indices")
            _need(ssm_state_indices, "ssm_state_indices", torch.int32)
            num_slots = state_pool.shape[0]
            if ssm_state_indices.dim() == 1 and ssm_state_indices.shape[0] == N:
                mode = STATE_POOL
                if num_accepted_tokens is not None:
                    raise ValueError("num_accepted_tokens needs ssm_state_indices of shape [N, L]")
            elif ssm_state_indices.dim() == 2 and ssm_state_indices.shape[0] == N:
                mode = STATE_POOL_SPEC
                cols = ssm_state_indices.shape[1]
                if num_accepted_tokens is not None:
                    _need(num_accepted_tokens, "num_accepted_tokens", torch.int32, (N,))
            else:
                raise ValueError(f"ssm_state_indices must be [N] or [N, L] with N = {N}")
        else:
            mode = STATE_SEPARATE
            if ssm_state_indices is not None or num_accepted_tokens is not None:
                raise ValueError("ssm_state_indices and num_accepted_tokens need a state_pool")
            if initial_state is not None:
                _need(initial_state, "initial_state", torch.float32, (N, HV, V, K))
        self.problem = cdr_recurrent_problem(
            int(B), int(T), int(H), int(HV), int(K), int(V), int(N),
            GATE_PER_DIM if per_dim else GATE_PER_HEAD, float(scale), int(cu_seqlens is not None),
            int(bool(use_qk_l2norm_in_kernel)), mode, int(initial_state is not None),
            int(bool(output_final_state)), int(num_slots), int(cols))
        st = lib.cdr_recurrent_check(ctypes.byref(self.problem))
        if st != CDR_OK:
            _raise(st, "fused_recurrent_fwd")
        if out is not None:
            _need(out, "out", torch.bfloat16, (B, T, HV, V), dense=True)
        if mode == STATE_SEPARATE and output_final_state and final_state_out is not None:
            _need(final_state_out, "final_state_out", torch.float32, (N, HV, V, K), dense=True)
        device = q.device
        if device.type != "cuda":
            raise ValueError("inputs must be on a GPU device")
        self.device = device
        # keep references: the kernel reads these buffers when it runs
        self.inputs = tuple(_aligned(t) for t in (q, k, v, g, beta))
        self.s0 = _aligned(initial_state)
        self.cu = _aligned(cu_seqlens)
        self.idx = _aligned(ssm_state_indices)
        self.acc = _aligned(num_accepted_tokens)
        self.pool = state_pool
        if out is None:
            out = torch.empty((B, T, HV, V), dtype=torch.bfloat16, device=device)
        self.o = out
        self.S = None
        if mode == STATE_SEPARATE and output_final_state:
            if final_state_out is None:
                final_state_out = torch.empty((N, HV, V, K), dtype=torch.float32, device=device)
            self.S = final_state_out
        ptr = lambda t: None if t is None else _dev_ptr(t, device)  # noqa: E731
        qq, kk, vv, gg, bb = self.inputs
        self._args = (ctypes.byref(self.problem), ptr(qq), ptr(kk), ptr(vv), ptr(gg), ptr(bb),
                      ptr(self.cu), ptr(self.s0), ptr(self.S), ptr(self.pool), ptr(self.idx),
                      ptr(self.acc), ptr(self.o))
        self._lib = lib

    def __call__(self):
        stream = torch.cuda.current_stream(self.device).cuda_stream
        st = self._lib.chunk_dr_recurrent_fwd(*self._args, stream)
        if st != CDR_OK:
            _raise(st, "fused_recurrent_fwd")
        return self.o, self.S


def fused_recurrent_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        beta: torch.Tensor, scale: Optional[float] = None,
                        initial_state: Optional[torch.Tensor] = None,
                        output_final_state: bool = False,
                        cu_seqlens: Optional[torch.Tensor] = None,
                        use_qk_l2norm_in_kernel: bool = False,
                        state_pool: Optional[torch.Tensor] = None,
                        ssm_state_indices: Optional[torch.Tensor] = None,
                        num_accepted_tokens: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None,
                        final_state_out: Optional[torch.Tensor] = None,
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Per-token gated delta-rule forward on the GPU (the decode path).

    q, k, v, g, beta, scale, cu_seqlens and use_qk_l2norm_in_kernel as :func:`chunk_dr_fwd`.

    Without ``state_pool`` the states are separate, as in chunk_dr_fwd: initial_state
    ``[N,HV,V,K]`` fp32 or None (zeros), and the final state is returned when
    output_final_state (``final_state_out`` may be ``initial_state`` itself).

    With ``state_pool`` ``[P,HV,V,K]`` fp32 the states are updated in place in the pool:
    ``ssm_state_indices`` int32 ``[N]`` gives each sequence's slot (read, then written back);
    ``[N,L]`` gives one slot per draft position (speculative decoding), the sequence starting
    from slot ``idx[n, num_accepted_tokens[n] - 1]`` (``num_accepted_tokens`` int32 ``[N]`` or
    None for 1) and writing its state after token t to ``idx[n, t]``.  Slot indices outside
    ``[0, P)`` mark padding (see chunk_dr.h).  Returns ``(o, S)``: S is the final state in the
    separate mode with output_final_state, else None (the pool holds the results).
    """
    return PreparedRecurrent(q, k, v, g, beta, scale=scale, initial_state=initial_state,
                             output_final_state=output_final_state, cu_seqlens=cu_seqlens,
                             use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel,
                             state_pool=state_pool, ssm_state_indices=ssm_state_indices,
                             num_accepted_tokens=num_accepted_tokens, out=out,
                             final_state_out=final_state_out)()
