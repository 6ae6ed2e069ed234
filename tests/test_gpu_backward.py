"""Parity of the HIP backward with the fp64 gradient oracle, through the C interface.

Bar (page "flash-linear-attention KCP 精度失效根因排查手册", section 验收标准): the norm
ratio |x - ref| / |ref| of every gradient below 5e-3, per sequence, against the gradients of
the per-token rule (``oracle.backward.recurrent_bwd``, fp64 autograd) on the same bits.
"""
import sys

import numpy as np
import pytest
import torch

import chunked_gated_delta_chunk_amd as cdr
from chunked_gated_delta_chunk_amd.synth import WORKLOADS, make_inputs, workload_inputs
from oracle.backward import recurrent_bwd, norm_ratio

pytestmark = pytest.mark.gpu

TOL = 5e-3
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def note(msg):
    print(msg, file=sys.stderr, flush=True)


def upstream(inp, seed, dht=True):
    gen = torch.Generator("cpu").manual_seed(seed)
    B, T, HV, V = inp.v.shape
    K = inp.q.shape[-1]
    N = B if inp.cu_seqlens is None else inp.cu_seqlens.numel() - 1
    do = torch.randn(B, T, HV, V, generator=gen).to(torch.bfloat16)
    ht = (0.1 * torch.randn(N, HV, V, K, generator=gen)) if dht else None
    return do, ht


def run_gpu(inp, do, dht, l2n):
    d = inp.to(DEV)
    grads = cdr.chunk_dr_bwd(d.q, d.k, d.v, d.g, d.beta, do.to(DEV),
                             dht=None if dht is None else dht.to(DEV),
                             initial_state=d.initial_state, cu_seqlens=d.cu_seqlens,
                             chunk_size=inp.chunk_size, use_qk_l2norm_in_kernel=l2n)
    torch.cuda.synchronize()
    return dict(zip(NAMES, (None if t is None else t.cpu().numpy() for t in grads)))


def seq_slices(inp):
    if inp.cu_seqlens is None:
        return [(b, slice(None)) for b in range(inp.q.shape[0])]
    cu = inp.cu_seqlens.tolist()
    return [(0, slice(cu[n], cu[n + 1])) for n in range(len(cu) - 1)]


def check(inp, label, l2n=False, dht=True, seed=1, tol=TOL):
    note(f"[bwd] {label} q{tuple(inp.q.shape)} v{tuple(inp.v.shape)} C={inp.chunk_size} l2n={l2n}")
    do, ht = upstream(inp, seed, dht)
    got = run_gpu(inp, do, ht, l2n)
    ref = recurrent_bwd(inp.q, inp.k, inp.v, inp.g, inp.beta, do, dht=ht,
                        initial_state=inp.initial_state, cu_seqlens=inp.cu_seqlens,
                        use_qk_l2norm=l2n)
    worst = {}
    for name in NAMES:
        if name == "dh0":
            if inp.initial_state is None:
                assert got["dh0"] is None
                continue
            for n in range(got["dh0"].shape[0]):
                r = norm_ratio(got["dh0"][n], ref["dh0"][n])
                worst[name] = max(worst.get(name, 0.0), r)
            continue
        assert np.isfinite(got[name]).all(), name
        for b, sl in seq_slices(inp):
            x, y = got[name][b, sl], ref[name][b, sl]
            if y.size == 0:
                continue
            worst[name] = max(worst.get(name, 0.0), norm_ratio(x, y))
    note(f"[bwd] {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    for k, v in worst.items():
        assert v <= tol, f"{k} norm ratio {v:.3e} > {tol}"


SMALL = [
    # label, B, T, H, HV, C, per_dim, lengths, initial, gate_mean, l2n
    ("kda_T64_one_chunk", 1, 64, 2, None, 64, True, None, True, 0.0, False),
    ("kda_T37_tail", 1, 37, 1, None, 64, True, None, True, 0.0, False),
    ("kda_T200_tail8_b2", 2, 200, 2, None, 64, True, None, True, 0.0, False),
    ("kda_T300_C128_weak", 1, 300, 2, None, 128, True, None, True, 4.0, False),
    ("kda_T256_C128_zero_state", 1, 256, 2, None, 128, True, None, False, 0.0, False),
    ("gdn_T300_C64", 2, 300, 2, None, 64, False, None, True, 0.0, False),
    ("gdn_T260_C128_weak", 1, 260, 1, None, 128, False, None, True, 3.0, False),
    ("grouped_l2n_C64", 1, 150, 1, 2, 64, True, None, True, 1.0, True),
    ("grouped_gdn_l2n_C128", 1, 200, 2, 4, 128, False, None, True, 0.0, True),
    ("varlen_ragged_empty", 1, 259, 2, None, 64, True, (1, 0, 63, 65, 130), True, 0.0, False),
    ("varlen_C128", 1, 400, 1, None, 128, True, (127, 129, 144), True, 1.0, True),
]


# Gates far stronger than the workloads' (as in the forward's strong-gate cases): every
# per-token gate near -12, so a 16-token tile spans about 190 in gamma, and isolated tokens
# that forget everything (g = -40 with probability 1/8, or 1/50 so that most tiles stay narrow
# and the two kinds of tile meet in one chunk).  Pair decays inside a tile are then far beyond
# any fp32 pivot factor, and dg is small where the other gradients are not.
STRONG = [
    # label, B, T, H, HV, C, per_dim, lengths, initial, gate_mean, spike_prob
    ("kda_ls_m12_C128", 1, 300, 2, None, 128, True, None, True, -12.0, 0.0),
    ("kda_ls_m12_C64_varlen", 1, 333, 2, None, 64, True, (100, 0, 233), True, -12.0, 0.0),
    ("gdn_ls_m12_C128", 1, 260, 2, None, 128, False, None, True, -12.0, 0.0),
    ("kda_spikes40_C128", 1, 384, 2, None, 128, True, None, True, 0.0, 0.125),
    ("gdn_spikes40_grouped_C64", 1, 200, 1, 2, 64, False, None, True, 0.0, 0.125),
    ("kda_sparse_spikes40_C128", 1, 512, 2, None, 128, True, None, True, 0.0, 0.02),
    ("kda_sparse_spikes40_C64_varlen", 1, 390, 2, None, 64, True, (70, 320), True, 1.0, 0.02),
]


# The state carries over every chunk (g = 0) or nearly (logsigmoid(N(6,1))): the two chains
# multiply -P into their state 32 to 64 times, so its rounding compounds.  With -P kept as hi + lo
# bf16 the norm ratios stay near 1e-5; with one bf16 rounding they were about 1.3e-3, under the
# page's bar but far above the rest.  Checked against 2e-4.
CARRY = [
    ("g0_T2048_C64", 2048, 64, dict(gate="zero")),
    ("g0_T4096_C128", 4096, 128, dict(gate="zero")),
    ("weak6_T2048_C128", 2048, 128, dict(gate_mean=6.0)),
]


@pytest.mark.parametrize("case", CARRY, ids=[c[0] for c in CARRY])
def test_backward_where_the_state_carries(case):
    label, T, C, kw = case
    inp = make_inputs(1, T, 1, seed=77, initial_state=True, chunk_size=C, **kw)
    check(inp, label, tol=2e-4)


@pytest.mark.parametrize("case", STRONG, ids=[c[0] for c in STRONG])
def test_backward_strong_gates(case):
    label, B, T, H, HV, C, per_dim, lengths, init, gm, sp = case
    inp = make_inputs(B, T, H, seed=900 + T, per_dim_gate=per_dim, lengths=lengths, initial_state=init,
                      chunk_size=C, gate_mean=gm, HV=HV, spike_prob=sp)
    check(inp, label)


# Strong gates in a few key dimensions only (logsigmoid(N(-6,1)) there, about -6 per token), in
# every row or in rows 16..47 of each chunk, or as scattered single elements set to -40: a tile
# is then wide through one or a few of its dimensions while the others are narrow, and the
# gradients of the narrow dimensions must not lose precision to the wide ones.
MIXED = [
    # label, T, C, l2n, strong dimensions, rows (None: all), element spike probability
    ("kda_C128_one_strong_dim", 300, 128, False, (0,), None, 0.0),
    ("kda_C64_strong_dims_l2n", 260, 64, True, (5, 64, 127), None, 0.0),
    ("kda_C128_strong_dims_in_some_tiles", 384, 128, False, (3, 70), (16, 48), 0.0),
    ("kda_C128_element_spikes", 256, 128, False, (), None, 1.0 / 64),
]


@pytest.mark.parametrize("case", MIXED, ids=[c[0] for c in MIXED])
def test_backward_strong_gates_in_some_dimensions(case):
    label, T, C, l2n, dims, rows, sp = case
    inp = make_inputs(1, T, 2, seed=960 + T, initial_state=True, chunk_size=C, normalise=not l2n)
    g = inp.g.clone()
    gen = torch.Generator().manual_seed(970 + T)
    if dims:
        strong = torch.nn.functional.logsigmoid(torch.randn(g.shape[:3] + (len(dims),), generator=gen) - 6.0)
        for n, d in enumerate(dims):
            if rows is None:
                g[..., d] = strong[..., n]
            else:
                for c0 in range(0, T, C):
                    g[:, c0 + rows[0]:min(T, c0 + rows[1]), :, d] = strong[:, c0 + rows[0]:min(T, c0 + rows[1]), :, n]
    if sp > 0:
        g = torch.where(torch.rand(g.shape, generator=gen) < sp, torch.full_like(g, -40.0), g)
    inp.g = g
    check(inp, label, l2n=l2n)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_parity(case):
    label, B, T, H, HV, C, per_dim, lengths, init, gm, l2n = case
    inp = make_inputs(B, T, H, seed=500 + T, per_dim_gate=per_dim, lengths=lengths,
                      initial_state=init, chunk_size=C, gate_mean=gm, HV=HV, normalise=not l2n)
    check(inp, label, l2n=l2n)


def test_backward_without_final_state_gradient():
    inp = make_inputs(1, 130, 2, seed=520, initial_state=True, chunk_size=64)
    check(inp, "no_dht", dht=False)


def test_backward_repeat_is_bit_identical():
    inp = make_inputs(1, 260, 2, seed=521, initial_state=True, chunk_size=128, gate_mean=2.0)
    do, ht = upstream(inp, 3)
    a = run_gpu(inp, do, ht, False)
    b = run_gpu(inp, do, ht, False)
    for name in NAMES:
        assert np.array_equal(a[name], b[name]), name


@pytest.mark.parametrize("name", ["kda_t8192"])
def test_backward_workload_one_head(name):
    """The full workload on the GPU; the oracle on the first head (heads are independent)."""
    w = WORKLOADS[name]
    inp = workload_inputs(w, seed=1000 + list(WORKLOADS).index(name) + 1)
    do, ht = upstream(inp, 7)
    note(f"[bwd] {name} full size")
    got = run_gpu(inp, do, ht, False)
    one = lambda t: t[:, :, :1].contiguous()  # noqa: E731
    ref = recurrent_bwd(one(inp.q), one(inp.k), one(inp.v), one(inp.g), one(inp.beta), one(do),
                        dht=ht[:, :1].contiguous(), initial_state=inp.initial_state[:, :1].contiguous())
    worst = {}
    for nm in NAMES:
        x = got[nm][:, :1] if nm == "dh0" else got[nm][:, :, :1]
        worst[nm] = norm_ratio(x, ref[nm])
    note(f"[bwd] {name} head 0: " + "  ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    for k, v in worst.items():
        assert v <= TOL, f"{k} norm ratio {v:.3e} > {TOL}"


def test_backward_single_token_and_no_tokens():
    """One token (a pure-tail chunk), and a varlen batch whose sequences are all empty: then
    the only gradient is dh0 = dht."""
    inp = make_inputs(1, 1, 1, seed=530, initial_state=True, chunk_size=64)
    check(inp, "T1")
    empty = make_inputs(1, 0, 2, seed=531, lengths=(0, 0), initial_state=True, chunk_size=64)
    do, ht = upstream(empty, 4)
    got = run_gpu(empty, do, ht, False)
    assert np.array_equal(got["dh0"], ht.numpy())
