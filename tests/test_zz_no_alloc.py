"""The no-allocation entry point (chunk_dr_fwd_noalloc, for callers that cannot allocate device
memory) against chunk_dr_fwd, through the C interface.

Both run the same kernels on the same inputs, so their results must be bit-identical; the
static workspace is shared by every call on the device, so two calls in a row, the second on a
smaller problem, must each match.
"""
import sys

import pytest
import torch

import chunked_gated_delta_chunk_amd as cdr
from chunked_gated_delta_chunk_amd.synth import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def _both(inp):
    d = inp.to(DEV)
    kw = dict(initial_state=d.initial_state, cu_seqlens=d.cu_seqlens, chunk_size=inp.chunk_size,
              output_final_state=True)
    o_ref, S_ref = cdr.chunk_dr_fwd(d.q, d.k, d.v, d.g, d.beta, **kw)
    nan = float("nan")
    out = torch.full_like(o_ref, nan)
    fs = torch.full_like(S_ref, nan)
    o, S = cdr.chunk_dr_fwd_noalloc(d.q, d.k, d.v, d.g, d.beta, out=out, final_state_out=fs, **kw)
    torch.cuda.synchronize()
    return (o, S), (o_ref, S_ref)


def test_noalloc_equals_fwd_on_two_calls_the_second_smaller():
    big = workload_inputs(WORKLOADS["kda_t8192"], seed=1003)   # the stated limit holds this one
    small = make_inputs(1, 400, 2, seed=31, lengths=(150, 0, 250), initial_state=True, chunk_size=64)
    for label, inp in (("kda_t8192", big), ("varlen 150/0/250 C64", small)):
        note(f"[noalloc] {label}")
        (o, S), (o_ref, S_ref) = _both(inp)
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), label

