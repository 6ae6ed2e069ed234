"""The forward, the backward and a decode step captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed: every replay, with new input contents copied into the captured buffers and eager
GPU work in between, must give the bits of an eager call on the same inputs.  The forward is
covered through both the workspace entry point and the no-allocation one (whose static workspace
is what a capturing caller uses)."""
import pytest
import torch

import chunked_gated_delta_chunk_amd as cdr
from chunked_gated_delta_chunk_amd.synth import make_inputs

pytestmark = pytest.mark.gpu

# label, make_inputs keywords (shapes fixed across replays)
CASES = [
    ("kda_C128_tail", dict(B=1, T=600, H=2, chunk_size=128, initial_state=True)),
    ("kda_C64_varlen", dict(B=1, T=483, H=2, chunk_size=64, lengths=(150, 0, 333), initial_state=True)),
    ("gdn_C64_grouped", dict(B=2, T=200, H=1, HV=2, chunk_size=64, per_dim_gate=False)),
]


def _draw(kw, seed):
    return make_inputs(seed=seed, **kw).to("cuda:0")


def _eager(inp):
    call = cdr.PreparedForward(inp.q, inp.k, inp.v, inp.g, inp.beta, initial_state=inp.initial_state,
                               cu_seqlens=inp.cu_seqlens, chunk_size=inp.chunk_size, output_final_state=True)
    o, S = call()
    torch.cuda.synchronize()
    return o.clone(), S.clone()


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager_calls(case, noalloc):
    label, kw = case
    print(f"[graph] {label} noalloc={noalloc}", flush=True)
    st = _draw(kw, seed=700)   # the captured buffers
    call = cdr.PreparedForward(st.q, st.k, st.v, st.g, st.beta, initial_state=st.initial_state,
                               cu_seqlens=st.cu_seqlens, chunk_size=st.chunk_size, output_final_state=True,
                               noalloc=noalloc)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the capture, as torch recommends
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        new = _draw(kw, seed=701 + r)
        for dst, src in ((st.q, new.q), (st.k, new.k), (st.v, new.v), (st.g, new.g), (st.beta, new.beta),
                         (st.initial_state, new.initial_state)):
            if dst is not None:
                dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        o_ref, S_ref = _eager(new)
        assert torch.equal(call.o, o_ref), f"replay {r}: o differs"
        assert torch.equal(call.S, S_ref), f"replay {r}: final state differs"
        torch.randn(4096, device="cuda:0").abs().sum().item()   # eager work between replays


# ---------------------------------------------------------------- backward
BWD_CASES = [
    ("kda_C128_tail", dict(B=1, T=300, H=2, chunk_size=128, initial_state=True)),
    ("kda_C64_varlen_grouped", dict(B=1, T=260, H=1, HV=2, chunk_size=64, lengths=(100, 0, 160),
                                    initial_state=True)),
]


def _bwd_draw(kw, seed):
    inp = make_inputs(seed=seed, **kw)
    gen = torch.Generator("cpu").manual_seed(seed + 50)
    N = inp.q.shape[0] if inp.cu_seqlens is None else inp.cu_seqlens.numel() - 1
    do = torch.randn(tuple(inp.v.shape), generator=gen).to(torch.bfloat16)
    dht = 0.1 * torch.randn(N, inp.v.shape[2], 128, 128, generator=gen)
    return inp.to("cuda:0"), do.to("cuda:0"), dht.to("cuda:0")


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_graph_replays_match_eager_calls(case):
    """The backward has no allocation or memset inside its calls: captured once, each replay on
    new input contents gives the bits of an eager call."""
    label, kw = case
    print(f"[graph bwd] {label}", flush=True)
    st, do, dht = _bwd_draw(kw, seed=800)
    call = cdr.PreparedBackward(st.q, st.k, st.v, st.g, st.beta, do, dht=dht, initial_state=st.initial_state,
                                cu_seqlens=st.cu_seqlens, chunk_size=st.chunk_size)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        new, do_n, dht_n = _bwd_draw(kw, seed=801 + r)
        for dst, src in ((st.q, new.q), (st.k, new.k), (st.v, new.v), (st.g, new.g), (st.beta, new.beta),
                         (st.initial_state, new.initial_state), (do, do_n), (dht, dht_n)):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        ref = cdr.PreparedBackward(new.q, new.k, new.v, new.g, new.beta, do_n, dht=dht_n,
                                   initial_state=new.initial_state, cu_seqlens=new.cu_seqlens,
                                   chunk_size=new.chunk_size)()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), call.grads, ref):
            assert torch.equal(a, b), f"replay {r}: {name} differs"
        torch.randn(4096, device="cuda:0").abs().sum().item()   # eager work between replays


# ---------------------------------------------------------------- decode on a state pool
DEC_CASES = [
    # label, N, T, H, HV, slots, speculative columns
    ("decode_T1", 16, 1, 2, 2, 48, 0),
    ("spec_L3_grouped", 8, 3, 1, 2, 40, 3),
]


@pytest.mark.parametrize("case", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_decode_graph_replays_match_eager_calls(case):
    """A serving loop captures the decode step once and replays it: new tokens, slot indices,
    accepted counts and pool contents go into the captured buffers before each replay."""
    from chunked_gated_delta_chunk_amd.synth import make_decode_inputs
    label, N, T, H, HV, slots, cols = case
    print(f"[graph decode] {label}", flush=True)
    draw = lambda seed: make_decode_inputs(N, T, H, HV, slots, seed=seed, index_cols=cols,  # noqa: E731
                                           normalise=False).to("cuda:0")
    st = draw(900)
    call = cdr.PreparedRecurrent(st.q, st.k, st.v, st.g, st.beta, use_qk_l2norm_in_kernel=True,
                                 state_pool=st.state_pool, ssm_state_indices=st.ssm_state_indices,
                                 num_accepted_tokens=st.num_accepted_tokens)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        new = draw(901 + r)
        for dst, src in ((st.q, new.q), (st.k, new.k), (st.v, new.v), (st.g, new.g), (st.beta, new.beta),
                         (st.state_pool, new.state_pool), (st.ssm_state_indices, new.ssm_state_indices),
                         (st.num_accepted_tokens, new.num_accepted_tokens)):
            if dst is not None:
                dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        pool_ref = new.state_pool.clone()
        o_ref, _ = cdr.PreparedRecurrent(new.q, new.k, new.v, new.g, new.beta, use_qk_l2norm_in_kernel=True,
                                         state_pool=pool_ref, ssm_state_indices=new.ssm_state_indices,
                                         num_accepted_tokens=new.num_accepted_tokens)()
        torch.cuda.synchronize()
        assert torch.equal(call.o, o_ref), f"replay {r}: o differs"
        assert torch.equal(st.state_pool, pool_ref), f"replay {r}: pool differs"
        torch.randn(4096, device="cuda:0").abs().sum().item()   # eager work between replays
