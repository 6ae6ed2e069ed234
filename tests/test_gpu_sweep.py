"""Seeded sweep over mixed configurations, forward and backward, through the C interface.

Each case draws its shape and options from a fixed seed: chunk size, gate kind, head count and
grouping, fixed-length batches or packed sequences (empty ones included), initial state, gate
strength (weak gates that carry the state, ordinary ones, and isolated g = -40 tokens), and
in-kernel q/k normalisation.  The bars are those of the other parity tests: the forward against
the fp64 per-token recurrence element by element (o 1e-2, S 1e-3, page "PyPTO-Gym 的 chunk_kda
算子实战", section 支持的 dtype 与形状约束), the backward by norm ratio against the fp64 gradient
of the same rule (5e-3, page "flash-linear-attention KCP 精度失效根因排查手册", section 验收标准).
"""
import random
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.backward import recurrent_bwd, norm_ratio
import chunked_gated_delta_chunk_amd as cdr
from chunked_gated_delta_chunk_amd.synth import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
O_TOL, S_TOL, G_TOL = 1e-2, 1e-3, 5e-3


def draw(seed, max_T, max_heads):
    rng = random.Random(seed)
    c = dict(C=rng.choice([64, 128]), per_dim=rng.random() < 0.7, H=rng.choice([1, 2, 3]))
    c["HV"] = c["H"] * rng.choice([1, 1, 2])
    if c["HV"] > max_heads:
        c["HV"] = c["H"]
    if rng.random() < 0.4:
        n = rng.randint(1, 6)
        lengths = [rng.choice([0, rng.randint(1, 40), rng.randint(1, max_T // 2)]) for _ in range(n)]
        if sum(lengths) == 0:
            lengths[-1] = 1
        c.update(B=1, lengths=tuple(lengths), T=sum(lengths))
    else:
        c.update(B=rng.choice([1, 2]), lengths=None, T=rng.randint(1, max_T))
    c.update(init=rng.random() < 0.7, gate_mean=rng.choice([-2.0, 0.0, 2.0, 4.0]), l2n=rng.random() < 0.3,
             spikes=rng.choice([0.0, 0.0, 0.05]))
    return c


def inputs(c, seed):
    return make_inputs(c["B"], c["T"], c["H"], seed=seed, per_dim_gate=c["per_dim"], lengths=c["lengths"],
                       initial_state=c["init"], chunk_size=c["C"], gate_mean=c["gate_mean"], HV=c["HV"],
                       normalise=not c["l2n"], spike_prob=c["spikes"])


def local_scale(o_ref, w=8):
    """Largest |o| of each head over the rows within w tokens of each row: [B, T, H]."""
    m = np.abs(o_ref).max(axis=-1)
    out = np.empty_like(m)
    for t in range(m.shape[1]):
        out[:, t] = m[:, max(0, t - w):t + w + 1].max(axis=1)
    return out + 1e-30


def ratio(x, ref, tol):
    x = np.asarray(x, dtype=np.float64)
    return float(np.max(np.abs(x - ref) / (tol + tol * np.abs(ref)))) if ref.size else 0.0


@pytest.mark.parametrize("case", range(24))
def test_forward_sweep(case):
    c = draw(7000 + case, max_T=700, max_heads=6)
    print(f"[sweep fwd {case}] {c}", file=sys.stderr, flush=True)
    inp = inputs(c, 7100 + case)
    d = inp.to(DEV)
    N = d.q.shape[0] if d.cu_seqlens is None else d.cu_seqlens.numel() - 1
    out = torch.full(tuple(d.v.shape), float("nan"), dtype=torch.bfloat16, device=DEV)
    fs = torch.full((N, c["HV"], 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    o, S = cdr.chunk_dr_fwd(d.q, d.k, d.v, d.g, d.beta, initial_state=d.initial_state, cu_seqlens=d.cu_seqlens,
                            chunk_size=c["C"], output_final_state=True, out=out, final_state_out=fs,
                            use_qk_l2norm_in_kernel=c["l2n"])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, initial_state=inp.initial_state,
                                        cu_seqlens=inp.cu_seqlens, use_qk_l2norm=c["l2n"])
    ro = ratio(o.float().cpu().numpy(), o_ref, O_TOL)
    rs = ratio(S.cpu().numpy(), S_ref, S_TOL)
    print(f"[sweep fwd {case}] o err/tol {ro:.3f}  S err/tol {rs:.3f}", file=sys.stderr, flush=True)
    assert ro <= 1.0 and rs <= 1.0


def draw_harsh(seed):
    """Stronger and more varied gates than `draw`: gate means from -8 to 8 and isolated tokens of
    g = -10 .. -80 at up to one in five tokens, which puts wide and narrow tiles side by side."""
    rng = random.Random(seed)
    c = draw(seed, max_T=600, max_heads=4)
    c.update(gate_mean=rng.choice([-8.0, -4.0, -2.0, 0.0, 2.0, 8.0]),
             spikes=rng.choice([0.02, 0.05, 0.1, 0.2]), spike_value=rng.choice([-10.0, -20.0, -40.0, -80.0]))
    return c


@pytest.mark.parametrize("case", range(24))
def test_forward_sweep_harsh_gates(case):
    c = draw_harsh(9000 + case)
    print(f"[sweep harsh {case}] {c}", file=sys.stderr, flush=True)
    inp = make_inputs(c["B"], c["T"], c["H"], seed=9100 + case, per_dim_gate=c["per_dim"], lengths=c["lengths"],
                      initial_state=c["init"], chunk_size=c["C"], gate_mean=c["gate_mean"], HV=c["HV"],
                      normalise=not c["l2n"], spike_prob=c["spikes"], spike_value=c["spike_value"])
    d = inp.to(DEV)
    o, S = cdr.chunk_dr_fwd(d.q, d.k, d.v, d.g, d.beta, initial_state=d.initial_state, cu_seqlens=d.cu_seqlens,
                            chunk_size=c["C"], output_final_state=True, use_qk_l2norm_in_kernel=c["l2n"])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, initial_state=inp.initial_state,
                                        cu_seqlens=inp.cu_seqlens, use_qk_l2norm=c["l2n"])
    og = o.float().cpu().numpy().astype(np.float64)
    ro = ratio(og, o_ref, O_TOL)
    rs = ratio(S.cpu().numpy(), S_ref, S_TOL)
    # the error of each output row against the scale of o around it (the absolute floor of the o
    # tolerance hides heads whose values are all small; a row that cancels to a fraction of its
    # neighbours keeps the neighbours' rounding error, which is not a fault)
    row = (np.abs(og - o_ref).max(axis=-1) / local_scale(o_ref)).max()
    print(f"[sweep harsh {case}] o err/tol {ro:.3f}  S err/tol {rs:.3f}  o row error / local scale {row:.4f}",
          file=sys.stderr, flush=True)
    assert ro <= 1.0 and rs <= 1.0
    assert row <= 0.05


def dimension_gates(g, seed):
    """Per-dimension gate patterns on a per-dimension gate tensor [B, T, H, K]: a random set of 1 to 16
    key dimensions made strong (logsigmoid(N(m, 1)), m from -4 to -10), in all rows or in one
    random row range, and optionally scattered single elements set to -40."""
    rng = random.Random(seed)
    gen = torch.Generator().manual_seed(seed)
    g = g.clone()
    B, T, H, K = g.shape
    dims = rng.sample(range(K), rng.choice([1, 2, 4, 16]))
    m = rng.choice([-4.0, -6.0, -10.0])
    r0, r1 = (0, T) if rng.random() < 0.5 else sorted(rng.sample(range(T + 1), 2))
    strong = torch.nn.functional.logsigmoid(torch.randn(B, T, H, len(dims), generator=gen) + m)
    for n, d in enumerate(dims):
        g[:, r0:r1, :, d] = strong[:, r0:r1, :, n]
    sp = rng.choice([0.0, 1.0 / 256, 1.0 / 32])
    if sp > 0:
        g = torch.where(torch.rand(g.shape, generator=gen) < sp, torch.full_like(g, -40.0), g)
    return g, dict(dims=len(dims), mean=m, rows=(r0, r1), spikes=sp)


@pytest.mark.parametrize("case", range(16))
def test_forward_sweep_dimension_gates(case):
    """Strong gates in some key dimensions only: (tile, dimension) columns take the wide pivots
    and exact diagonal sums beside narrow ones in the same tiles."""
    c = draw(9500 + case, max_T=600, max_heads=4)
    inp = make_inputs(c["B"], c["T"], c["H"], seed=9600 + case, per_dim_gate=True, lengths=c["lengths"],
                      initial_state=c["init"], chunk_size=c["C"], gate_mean=c["gate_mean"], HV=c["HV"],
                      normalise=not c["l2n"])
    inp.g, pat = dimension_gates(inp.g, 9700 + case)
    print(f"[sweep dims {case}] {c} {pat}", file=sys.stderr, flush=True)
    d = inp.to(DEV)
    o, S = cdr.chunk_dr_fwd(d.q, d.k, d.v, d.g, d.beta, initial_state=d.initial_state, cu_seqlens=d.cu_seqlens,
                            chunk_size=c["C"], output_final_state=True, use_qk_l2norm_in_kernel=c["l2n"])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle.recurrent_fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, initial_state=inp.initial_state,
                                        cu_seqlens=inp.cu_seqlens, use_qk_l2norm=c["l2n"])
    og = o.float().cpu().numpy().astype(np.float64)
    ro = ratio(og, o_ref, O_TOL)
    rs = ratio(S.cpu().numpy(), S_ref, S_TOL)
    row = (np.abs(og - o_ref).max(axis=-1) / local_scale(o_ref)).max()
    print(f"[sweep dims {case}] o err/tol {ro:.3f}  S err/tol {rs:.3f}  o row error / local scale {row:.4f}",
          file=sys.stderr, flush=True)
    assert ro <= 1.0 and rs <= 1.0
    assert row <= 0.05


@pytest.mark.parametrize("case", range(20))
def test_backward_sweep(case):
    """Cases 0-9 draw like the forward sweep, 10-19 with the harsh gates."""
    c = draw(8000 + case, max_T=300, max_heads=4) if case < 10 else draw_harsh(8000 + case)
    if case >= 10:
        c["T"] = min(c["T"], 300)
        if c["lengths"] is not None:
            c["lengths"] = tuple(min(x, 100) for x in c["lengths"])
            c["T"] = max(sum(c["lengths"]), 1)
            if sum(c["lengths"]) == 0:
                c["lengths"] = c["lengths"][:-1] + (1,)
    print(f"[sweep bwd {case}] {c}", file=sys.stderr, flush=True)
    inp = make_inputs(c["B"], c["T"], c["H"], seed=8100 + case, per_dim_gate=c["per_dim"], lengths=c["lengths"],
                      initial_state=c["init"], chunk_size=c["C"], gate_mean=c["gate_mean"], HV=c["HV"],
                      normalise=not c["l2n"], spike_prob=c["spikes"], spike_value=c.get("spike_value", -40.0))
    gen = torch.Generator("cpu").manual_seed(8200 + case)
    N = inp.q.shape[0] if inp.cu_seqlens is None else inp.cu_seqlens.numel() - 1
    do = torch.randn(tuple(inp.v.shape), generator=gen).to(torch.bfloat16)
    dht = 0.1 * torch.randn(N, c["HV"], 128, 128, generator=gen)
    d = inp.to(DEV)
    got = cdr.chunk_dr_bwd(d.q, d.k, d.v, d.g, d.beta, do.to(DEV), dht=dht.to(DEV), initial_state=d.initial_state,
                           cu_seqlens=d.cu_seqlens, chunk_size=c["C"], use_qk_l2norm_in_kernel=c["l2n"])
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    got = dict(zip(names, (None if t is None else t.cpu().numpy() for t in got)))
    ref = recurrent_bwd(inp.q, inp.k, inp.v, inp.g, inp.beta, do, dht=dht, initial_state=inp.initial_state,
                        cu_seqlens=inp.cu_seqlens, use_qk_l2norm=c["l2n"])
    worst = {}
    for name in names:
        if got[name] is None:
            assert inp.initial_state is None and name == "dh0"
            continue
        assert np.isfinite(got[name]).all(), name
        worst[name] = norm_ratio(got[name], ref[name])
    print(f"[sweep bwd {case}] " + "  ".join(f"{k} {v:.2e}" for k, v in worst.items()), file=sys.stderr, flush=True)
    for k, v in worst.items():
        assert v <= G_TOL, f"{k} norm ratio {v:.3e}"


@pytest.mark.parametrize("case", range(16))
def test_decode_sweep(case):
    """The per-token kernel on a state pool: sequences, tokens per sequence (packed or not),
    heads and grouping, speculative columns, padding entries, gate kind and strength, in-kernel
    normalisation; checked as the decode tests check a pool call (untouched slots bit for bit)."""
    from test_gpu_decode import check_pool
    from chunked_gated_delta_chunk_amd.synth import make_decode_inputs
    rng = random.Random(9500 + case)
    N = rng.randint(1, 12)
    H = rng.choice([1, 2])
    HV = H * rng.choice([1, 2])
    spec = rng.random() < 0.5
    if rng.random() < 0.3:
        lengths = tuple(rng.randint(0, 4 if spec else 6) for _ in range(N))
        if sum(lengths) == 0:
            lengths = lengths[:-1] + (1,)
        T, cols = 0, (max(lengths) if spec else 0)
    else:
        lengths = None
        T = rng.randint(1, 4 if spec else 6)
        cols = rng.randint(T, 4) if spec else 0
    padded = tuple(i for i in range(N) if rng.random() < 0.15)
    per_dim, l2n = rng.random() < 0.7, rng.random() < 0.5
    gm = rng.choice([-4.0, 0.0, 4.0])
    slots = N * max(cols, 1) + rng.randint(0, 8)
    label = (f"N{N} T{T} lengths{lengths} H{H} HV{HV} cols{cols} padded{padded} per_dim{per_dim} "
             f"l2n{l2n} gm{gm} slots{slots}")
    print(f"[sweep decode {case}] {label}", file=sys.stderr, flush=True)
    d = make_decode_inputs(N, T, H, HV, slots, seed=9600 + case, index_cols=cols, per_dim_gate=per_dim,
                           normalise=not l2n, lengths=lengths, padded=padded, gate_mean=gm)
    check_pool(d, l2n, f"sweep {case}")
