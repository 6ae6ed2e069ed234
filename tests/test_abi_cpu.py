"""The C interface on the CPU: the library loads, exports what include/chunk_dr.h
declares, and validates problems on the host without touching a device."""
import ctypes
import os
import re

import pytest
import torch

import chunked_gated_delta_chunk_amd as cdr
from chunked_gated_delta_chunk_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "chunk_dr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)) - {"if"}


def test_library_exports_every_declared_function():
    lib = cdr.load_library()
    declared = _declared_functions()
    assert {"chunk_dr_fwd", "cdr_check", "cdr_workspace_bytes", "cdr_status_str",
            "cdr_version"} <= declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in chunk_dr.h but not exported"
    header = open(os.path.join(ROOT, "include", "chunk_dr.h")).read()
    assert lib.cdr_version() == int(re.search(r"#define CDR_VERSION (\d+)", header).group(1))


def test_problem_struct_matches_header():
    """The ctypes mirror lists the C struct's fields in order."""
    text = open(os.path.join(ROOT, "include", "chunk_dr.h")).read()
    body = re.search(r"typedef struct \{([^{}]*)\} cdr_problem;", text).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(?:int32_t|float)\s+(\w+);", body)
    assert fields == [f[0] for f in ops.cdr_problem._fields_]


def test_value_heads_validation_and_workspace():
    lib = cdr.load_library()
    assert cdr.check(_p(H=2, HV=4)) == 0
    assert cdr.check(_p(H=2, HV=3)) == 2      # not whole groups
    assert cdr.check(_p(H=2, HV=-1)) == 2
    assert cdr.check(_p(H=2, HV=0)) == 0      # 0 means HV = H
    a = cdr.workspace_bytes(_p(H=2, HV=2))
    b = cdr.workspace_bytes(_p(H=2, HV=4))
    assert cdr.workspace_bytes(_p(H=2, HV=0)) == a and b > a
    del lib


def _p(**kw):
    base = dict(B=1, T=256, H=2, K=128, V=128, N=1, per_dim_gate=True, chunk_size=64,
                scale=128 ** -0.5, has_initial_state=False, output_final_state=True, varlen=False)
    base.update(kw)
    return cdr.make_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(K=64), 3), (dict(V=256), 3), (dict(chunk_size=32), 3), (dict(chunk_size=256), 3),
    (dict(B=0), 2), (dict(H=0), 2), (dict(T=-1), 2), (dict(N=2), 2),
    (dict(B=2, N=3, varlen=True), 4),
    (dict(B=1, N=5, T=100, varlen=True), 0),
    (dict(T=0), 0),
])
def test_check_status(kw, status):
    assert cdr.check(_p(**kw)) == status


def test_check_rejects_unknown_gate():
    p = _p()
    p.gate = 7
    assert cdr.check(p) == 3


def test_workspace_size_scales_with_chunks():
    a = cdr.workspace_bytes(_p(T=256, chunk_size=64))
    b = cdr.workspace_bytes(_p(T=512, chunk_size=64))
    assert a > 0 and b > a
    assert cdr.workspace_bytes(_p(K=64)) == 0
    # varlen sizes for floor(T/C) + N chunk slots
    v = cdr.workspace_bytes(_p(T=256, N=3, varlen=True))
    assert v > a


def test_fwd_rejects_bad_problem_without_touching_device():
    lib = cdr.load_library()
    p = _p(K=64)
    st = lib.chunk_dr_fwd(ctypes.byref(p), *([None] * 10), 0, None)
    assert st == 3
    p = _p()
    st = lib.chunk_dr_fwd(ctypes.byref(p), *([None] * 10), 0, None)
    assert st == 1  # null tensor pointers
    st = lib.chunk_dr_fwd(ctypes.byref(p), *([1 << 20] * 9), None, 0, None)
    assert st == 5  # no workspace
    assert lib.cdr_status_str(5).decode().startswith("workspace")


def test_binding_type_and_shape_errors():
    B, T, H, K = 1, 8, 2, 128
    q = torch.zeros(B, T, H, K, dtype=torch.bfloat16)
    g = torch.zeros(B, T, H, K)
    beta = torch.zeros(B, T, H)
    with pytest.raises(TypeError):
        cdr.chunk_dr_fwd(q.float(), q, q, g, beta)
    with pytest.raises(TypeError):
        cdr.chunk_dr_fwd(q, q, q, g.double(), beta)
    with pytest.raises(ValueError):
        cdr.chunk_dr_fwd(q, q, q, g[..., :3], beta)
    with pytest.raises(ValueError):
        cdr.chunk_dr_fwd(q, q, q, g, beta, chunk_size=32)
    with pytest.raises(ValueError):  # K != 128
        cdr.chunk_dr_fwd(q[..., :64].contiguous(), q[..., :64].contiguous(), q, g[..., :64], beta)
    with pytest.raises(ValueError):  # varlen needs B == 1
        q2 = torch.zeros(2, T, H, K, dtype=torch.bfloat16)
        cdr.chunk_dr_fwd(q2, q2, q2, torch.zeros(2, T, H, K), torch.zeros(2, T, H),
                         cu_seqlens=torch.tensor([0, 8], dtype=torch.int32))
    with pytest.raises(ValueError):  # host tensors are not accepted: no CPU path exists
        cdr.chunk_dr_fwd(q, q, q, g, beta)
    # caller-supplied outputs are written row-major: a strided view is refused before anything
    # else happens
    o_view = torch.zeros(B, T, K, H, dtype=torch.bfloat16).transpose(2, 3)
    with pytest.raises(ValueError, match="contiguous"):
        cdr.chunk_dr_fwd(q, q, q, g, beta, out=o_view)
    s_view = torch.zeros(B, H, K, K).transpose(2, 3)
    with pytest.raises(ValueError, match="contiguous"):
        cdr.chunk_dr_fwd(q, q, q, g, beta, output_final_state=True, final_state_out=s_view)
    with pytest.raises(ValueError, match="contiguous"):
        cdr.fused_recurrent_fwd(q, q, q, g, beta, out=o_view)


def test_no_cpu_fallback_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(ops, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        ops.load_library(str(tmp_path / "absent.so"))


# ---------------------------------------------------------------------- recurrent entry point

def test_recurrent_struct_matches_header():
    text = open(os.path.join(ROOT, "include", "chunk_dr.h")).read()
    body = re.search(r"typedef struct \{([^{}]*)\} cdr_recurrent_problem;", text).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(?:int32_t|float)\s+(\w+);", body)
    assert fields == [f[0] for f in ops.cdr_recurrent_problem._fields_]


def _rp(**kw):
    base = dict(B=2, T=1, H=2, HV=4, K=128, V=128, N=2, gate=0, scale=0.1, varlen=0,
                qk_l2norm=1, state_mode=ops.STATE_POOL, has_initial_state=0,
                output_final_state=0, num_slots=8, index_cols=0)
    base.update(kw)
    return ops.cdr_recurrent_problem(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    (dict(state_mode=ops.STATE_SEPARATE, num_slots=0), 0),
    (dict(state_mode=ops.STATE_POOL_SPEC, index_cols=4), 0),
    (dict(state_mode=ops.STATE_POOL_SPEC, index_cols=0), 2),   # speculative rows need columns
    (dict(num_slots=0), 2),                                      # a pool needs slots
    (dict(HV=3), 2),                                             # whole groups of value heads
    (dict(K=64), 3),
    (dict(gate=2), 3),
    (dict(state_mode=7), 3),
    (dict(varlen=1), 4),                                         # varlen needs B == 1
    (dict(N=3), 2),                                              # fixed length: N == B
    (dict(B=1, N=3, varlen=1, T=5), 0),
    (dict(T=-1), 2),
])
def test_recurrent_check_status(kw, status):
    lib = cdr.load_library()
    assert lib.cdr_recurrent_check(ctypes.byref(_rp(**kw))) == status


def test_recurrent_rejects_missing_pointers_without_touching_device():
    lib = cdr.load_library()
    p = _rp()
    fake = 1 << 20
    args = [fake] * 5 + [None, None, None, None, None, None, fake, None]
    assert lib.chunk_dr_recurrent_fwd(ctypes.byref(p), *args) == 1   # no pool, no indices
    p = _rp(state_mode=ops.STATE_SEPARATE, has_initial_state=1)
    args = [fake] * 5 + [None] * 7 + [fake, None]
    assert lib.chunk_dr_recurrent_fwd(ctypes.byref(p), *args) == 1   # initial_state missing
    p = _rp(K=64)
    assert lib.chunk_dr_recurrent_fwd(ctypes.byref(p), *([None] * 13)) == 3


def test_recurrent_binding_errors():
    B, T, H, K = 2, 1, 2, 128
    q = torch.zeros(B, T, H, K, dtype=torch.bfloat16)
    v = torch.zeros(B, T, 4, K, dtype=torch.bfloat16)
    g = torch.zeros(B, T, 4, K)
    beta = torch.zeros(B, T, 4)
    pool = torch.zeros(8, 4, K, K)
    idx = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError):  # indices without a pool
        cdr.fused_recurrent_fwd(q, q, v, g, beta, ssm_state_indices=idx)
    with pytest.raises(ValueError):  # a pool without indices
        cdr.fused_recurrent_fwd(q, q, v, g, beta, state_pool=pool)
    with pytest.raises(ValueError):  # pool with the wrong head count
        cdr.fused_recurrent_fwd(q, q, v, g, beta, state_pool=pool[:, :2], ssm_state_indices=idx)
    with pytest.raises(TypeError):   # indices must be int32
        cdr.fused_recurrent_fwd(q, q, v, g, beta, state_pool=pool, ssm_state_indices=idx.long())
    with pytest.raises(ValueError):  # accepted counts need [N, L] indices
        cdr.fused_recurrent_fwd(q, q, v, g, beta, state_pool=pool, ssm_state_indices=idx,
                                num_accepted_tokens=idx)
    with pytest.raises(ValueError):  # the pool replaces initial/final state
        cdr.fused_recurrent_fwd(q, q, v, g, beta, state_pool=pool, ssm_state_indices=idx,
                                output_final_state=True)
    with pytest.raises(ValueError):  # host tensors: no CPU path exists
        cdr.fused_recurrent_fwd(q, q, v, g, beta, state_pool=pool, ssm_state_indices=idx)


def test_noalloc_rejects_a_problem_beyond_its_array_without_touching_device():
    """chunk_dr_fwd_noalloc checks the workspace the problem needs against its static array before
    any device call: kda_t65536 (16384 chunks x heads) does not fit."""
    import chunked_gated_delta_chunk_amd as cdr
    p = cdr.make_problem(1, 65536, 32, 128, 128, 1, True, 128, 128 ** -0.5, False, True, False)
    assert cdr.workspace_bytes(p) > cdr.NOALLOC_SCRATCH_BYTES
    lib = cdr.load_library()
    st = lib.chunk_dr_fwd_noalloc(ctypes.byref(p), *([None] * 9), None)
    assert st == 7 and "static array" in lib.cdr_status_str(st).decode()
    # the workload the limit is stated for fits
    q = cdr.make_problem(1, 8192, 16, 128, 128, 1, True, 128, 128 ** -0.5, True, True, False)
    assert cdr.workspace_bytes(q) <= cdr.NOALLOC_SCRATCH_BYTES


def test_cu_seqlens_check_rejects_bad_arguments_without_touching_device():
    """cdr_check_cu_seqlens validates its arguments on the host before launching anything."""
    lib = cdr.load_library()
    buf = (ctypes.c_int32 * 4)()   # host memory: never handed to a kernel by these calls
    res = (ctypes.c_int32 * 1)()
    assert lib.cdr_check_cu_seqlens(None, 1, 10, ctypes.addressof(res), None) == 1    # NULL array
    assert lib.cdr_check_cu_seqlens(ctypes.addressof(buf), 1, 10, None, None) == 1    # NULL result
    assert lib.cdr_check_cu_seqlens(ctypes.addressof(buf), 0, 10, ctypes.addressof(res), None) == 2
    assert lib.cdr_check_cu_seqlens(ctypes.addressof(buf), 2, -1, ctypes.addressof(res), None) == 2
    with pytest.raises(TypeError):
        cdr.check_cu_seqlens(torch.tensor([0, 4], dtype=torch.int64), 4)
    with pytest.raises(ValueError):
        cdr.check_cu_seqlens(torch.tensor([0], dtype=torch.int32), 0)
