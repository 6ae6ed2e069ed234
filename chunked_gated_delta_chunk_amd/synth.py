"""Seeded synthetic inputs for the chunked gated delta-rule forward.

This module only draws and shapes random inputs; it holds none of the
method's arithmetic, so both the HIP path and the oracle can take their
inputs from it.  Inputs follow the stable-input recipe described on the page
"PyPTO-Gym 的 chunk_kda 算子实战" (sections 使用示例 and test_inputs.py对抗性):
q and k Gaussian and L2-normalised over the key dimension, v Gaussian, a
log-domain gate g = logsigmoid(Gaussian) and beta = sigmoid(Gaussian).

Everything is drawn on the CPU in fp32 from a ``torch.Generator`` seeded with
``seed``, in the fixed order q, k, v, g, beta, initial_state, then cast to the
interface dtypes (bf16 q/k/v, fp32 g/beta/state).  The oracle and the GPU
therefore see identical bits.
"""
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch
import torch.nn.functional as F


@dataclass(frozen=True)
class Workload:
    """One problem shape. ``lengths`` given means a packed varlen batch (B = 1)."""
    name: str
    B: int
    T: int
    H: int
    K: int = 128
    V: int = 128
    chunk_size: int = 64
    per_dim_gate: bool = True
    initial_state: bool = False
    lengths: Optional[Sequence[int]] = None
    description: str = ""

    @property
    def N(self) -> int:
        return len(self.lengths) if self.lengths is not None else self.B

    @property
    def tokens(self) -> int:
        return self.B * self.T


def _varlen(name, lengths, **kw):
    return Workload(name=name, B=1, T=int(sum(lengths)), lengths=tuple(lengths), **kw)


#: The five workloads the forward is specified and measured on.
WORKLOADS = {
    "kda_small": Workload(
        "kda_small", B=1, T=256, H=2, chunk_size=64,
        description="KDA per-dim gate, B=1 T=256 H=2 K=V=128 C=64, zero initial state"),
    "gdn_b2_t2048": Workload(
        "gdn_b2_t2048", B=2, T=2048, H=8, chunk_size=64, per_dim_gate=False,
        description="Gated DeltaNet per-head gate, B=2 T=2048 H=8 K=V=128 C=64, zero initial state"),
    "kda_t8192": Workload(
        "kda_t8192", B=1, T=8192, H=16, chunk_size=128, initial_state=True,
        description="KDA per-dim gate, B=1 T=8192 H=16 K=V=128 C=128, initial state std 0.1"),
    "kda_varlen": _varlen(
        "kda_varlen", (400, 624, 1000, 2048, 4096), H=16, chunk_size=64, initial_state=True,
        description="KDA packed varlen, lengths 400/624/1000/2048/4096 (8168 tokens), H=16 C=64"),
    "kda_t65536": Workload(
        "kda_t65536", B=1, T=65536, H=32, chunk_size=128,
        description="KDA long context, B=1 T=65536 H=32 K=V=128 C=128, zero initial state"),
}


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    chunk_size: int
    extra: dict = field(default_factory=dict)

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return Inputs(mv(self.q), mv(self.k), mv(self.v), mv(self.g), mv(self.beta),
                      mv(self.initial_state), mv(self.cu_seqlens), self.chunk_size,
                      dict(self.extra))


def l2_normalise(x: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """x / max(||x||, eps) over the last dimension, in fp32."""
    return x / x.norm(dim=-1, keepdim=True).clamp_min(eps)


def make_inputs(B: int, T: int, H: int, K: int = 128, V: int = 128, *, seed: int,
                per_dim_gate: bool = True, lengths: Optional[Sequence[int]] = None,
                initial_state: bool = False, chunk_size: int = 64,
                gate_mean: float = 0.0, gate: str = "logsigmoid",
                beta_mode: str = "sigmoid", state_std: float = 0.1,
                normalise: bool = True, HV: Optional[int] = None,
                spike_prob: float = 0.0, spike_value: float = -40.0) -> Inputs:
    """Draw one seeded batch.

    gate: "logsigmoid" -> g = logsigmoid(N(gate_mean, 1)); "zero" -> g = 0.
    beta_mode: "sigmoid" -> sigmoid(N(0, 1)); "zero" -> 0; "one" -> 1.
    With ``lengths`` the batch is packed (B must be 1, T = sum(lengths)) and
    ``cu_seqlens`` is the int32 prefix sum of the lengths.  ``HV`` (a multiple of H)
    gives v, g, beta and the initial state HV value heads while q and k keep H.
    ``spike_prob`` > 0 sets the whole gate of a (token, head) to ``spike_value`` with that
    probability (isolated strong forgetting); the mask is drawn after everything else, so
    the other tensors are those of the same seed without spikes.
    """
    if lengths is not None:
        if B != 1 or T != sum(lengths):
            raise ValueError("packed batches need B == 1 and T == sum(lengths)")
    gen = torch.Generator("cpu").manual_seed(int(seed))
    randn = lambda *shape: torch.randn(*shape, generator=gen, dtype=torch.float32)  # noqa: E731
    Hv = H if HV is None else int(HV)
    if Hv % H:
        raise ValueError("HV must be a multiple of H")
    q = randn(B, T, H, K)
    k = randn(B, T, H, K)
    v = randn(B, T, Hv, V)
    gshape = (B, T, Hv, K) if per_dim_gate else (B, T, Hv)
    g0 = randn(*gshape)
    b0 = randn(B, T, Hv)
    N = len(lengths) if lengths is not None else B
    s0 = randn(N, Hv, V, K) * state_std if initial_state else None
    if normalise:
        q, k = l2_normalise(q), l2_normalise(k)
    if gate == "logsigmoid":
        g = F.logsigmoid(g0 + gate_mean)
    elif gate == "zero":
        g = torch.zeros(gshape, dtype=torch.float32)
    else:
        raise ValueError(gate)
    if beta_mode == "sigmoid":
        beta = torch.sigmoid(b0)
    elif beta_mode == "zero":
        beta = torch.zeros(B, T, Hv)
    elif beta_mode == "one":
        beta = torch.ones(B, T, Hv)
    else:
        raise ValueError(beta_mode)
    if spike_prob > 0:
        hit = torch.rand(B, T, Hv, generator=gen) < spike_prob
        g = torch.where(hit[..., None] if per_dim_gate else hit, torch.tensor(float(spike_value)), g)
    cu = None
    if lengths is not None:
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return Inputs(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16),
                  g.contiguous(), beta.contiguous(),
                  None if s0 is None else s0.contiguous(), cu, chunk_size)


def make_teacher_inputs(T: int, H: int, K: int = 128, V: int = 128, *, seed: int, chunk_size: int = 64,
                        state_scale: float = 1.0, noise: float = 1e-2,
                        key_scale: Sequence[float] = (1.0, 1.0), gate: str = "zero",
                        gate_mean: float = 0.0, beta_mode: str = "sigmoid") -> Inputs:
    """One sequence (B = 1) whose values come from a linear teacher that the initial state
    already holds, the input family of the page's ``cancellation_stress`` mode (section
    test_inputs.py对抗性: inputs aimed at the cancellation in v - w S).

    Drawn in order from one generator seeded with ``seed``: q, k ~ N(0, 1) normalised over K;
    the teacher W = state_scale * N(0, 1) of shape [H, V, K], which is also the initial state;
    per chunk of ``chunk_size`` tokens a key scale drawn log-uniformly from ``key_scale``;
    noise ~ N(0, 1); gates and beta as :func:`make_inputs`.  Then k is scaled per chunk,
    rounded to bf16, and v_t = W k_t + noise * N(0, 1) (in fp32 from the rounded keys) is
    rounded to bf16.  A state that has learnt W predicts every value up to the noise, so the
    correction each chunk applies is a small difference of large terms.
    """
    gen = torch.Generator("cpu").manual_seed(int(seed))
    randn = lambda *shape: torch.randn(*shape, generator=gen, dtype=torch.float32)  # noqa: E731
    q = l2_normalise(randn(1, T, H, K))
    k = l2_normalise(randn(1, T, H, K))
    W = randn(H, V, K) * state_scale
    nch = (T + chunk_size - 1) // chunk_size
    lo, hi = float(key_scale[0]), float(key_scale[1])
    u = torch.rand(nch, generator=gen)
    a = torch.exp(torch.log(torch.tensor(lo)) + u * (torch.log(torch.tensor(hi)) - torch.log(torch.tensor(lo))))
    eps = randn(1, T, H, V)
    g0 = randn(1, T, H, K)
    b0 = randn(1, T, H)
    k = (k * a.repeat_interleave(chunk_size)[:T].view(1, T, 1, 1)).to(torch.bfloat16)
    v = (torch.einsum("hvk,bthk->bthv", W, k.float()) + noise * eps).to(torch.bfloat16)
    if gate == "logsigmoid":
        g = F.logsigmoid(g0 + gate_mean)
    elif gate == "zero":
        g = torch.zeros(1, T, H, K)
    else:
        raise ValueError(gate)
    beta = {"sigmoid": torch.sigmoid(b0), "one": torch.ones(1, T, H)}[beta_mode]
    return Inputs(q.to(torch.bfloat16), k, v, g.contiguous(), beta.contiguous(),
                  W.unsqueeze(0).contiguous(), None, chunk_size)


def workload_inputs(w: Workload, seed: int, **overrides) -> Inputs:
    kw = dict(per_dim_gate=w.per_dim_gate, lengths=w.lengths, initial_state=w.initial_state,
              chunk_size=w.chunk_size)
    kw.update(overrides)
    return make_inputs(w.B, w.T, w.H, w.K, w.V, seed=seed, **kw)


# --------------------------------------------------------------------------- decode

@dataclass(frozen=True)
class DecodeWorkload:
    """One step of batched decoding against a pool of recurrent states.

    N sequences of ``T`` tokens each (or ``lengths``, packed), H query/key heads and HV value
    heads, a state pool of ``num_slots`` entries.  ``index_cols == 0``: one state slot per
    sequence, read and written in place.  ``index_cols > 0``: speculative decoding, a row of
    ``index_cols`` slots per sequence (one per draft position) and a count of accepted tokens
    that selects the slot the step starts from.
    """
    name: str
    N: int
    T: int
    H: int
    HV: int
    num_slots: int
    index_cols: int = 0
    K: int = 128
    V: int = 128
    per_dim_gate: bool = True
    qk_l2norm: bool = True
    lengths: Optional[Sequence[int]] = None
    description: str = ""

    @property
    def tokens(self) -> int:
        return int(sum(self.lengths)) if self.lengths is not None else self.N * self.T


#: Decode workloads: one step of a serving batch with KDA's head shape (H = 16, K = V = 128),
#: raw q/k normalised in the kernel, and a pool larger than the batch.
DECODE_WORKLOADS = {
    "kda_decode_b256": DecodeWorkload(
        "kda_decode_b256", N=256, T=1, H=16, HV=16, num_slots=1024,
        description="KDA decode, 256 sequences x 1 token, H=HV=16 K=V=128, pool of 1024 states"),
    "kda_spec_decode_b64x4": DecodeWorkload(
        "kda_spec_decode_b64x4", N=64, T=4, H=16, HV=16, num_slots=1024, index_cols=4,
        description="KDA speculative decode, 64 sequences x 4 draft tokens, H=HV=16, pool of 1024"),
}


@dataclass
class DecodeInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    cu_seqlens: Optional[torch.Tensor]
    state_pool: torch.Tensor
    ssm_state_indices: torch.Tensor
    num_accepted_tokens: Optional[torch.Tensor]

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return DecodeInputs(mv(self.q), mv(self.k), mv(self.v), mv(self.g), mv(self.beta),
                            mv(self.cu_seqlens), mv(self.state_pool), mv(self.ssm_state_indices),
                            mv(self.num_accepted_tokens))


def make_decode_inputs(N: int, T: int, H: int, HV: int, num_slots: int, *, seed: int,
                       index_cols: int = 0, K: int = 128, V: int = 128,
                       per_dim_gate: bool = True, normalise: bool = False,
                       lengths: Optional[Sequence[int]] = None, padded: Sequence[int] = (),
                       state_std: float = 0.1, gate_mean: float = 0.0,
                       beta_mode: str = "sigmoid", gate: str = "logsigmoid",
                       accepted: Optional[Sequence[int]] = None) -> DecodeInputs:
    """Draw one seeded decode step.

    Token inputs come from :func:`make_inputs` (B = N rows of T tokens, or one packed row of
    ``lengths``) with ``normalise`` applied on the host; a second generator seeded with
    ``seed + 1`` then draws, in order, the pool (``state_std`` x N(0, 1), [num_slots, HV, V, K]),
    a random choice of distinct slots, and the accepted-token counts (uniform in
    1..index_cols) unless ``accepted`` fixes them.  Sequences listed in ``padded`` get slot
    index -1 everywhere (padding entries).
    """
    if lengths is not None:
        inp = make_inputs(1, int(sum(lengths)), H, K, V, seed=seed, per_dim_gate=per_dim_gate,
                          lengths=lengths, normalise=normalise, HV=HV, gate_mean=gate_mean,
                          beta_mode=beta_mode, gate=gate)
        N = len(lengths)
    else:
        inp = make_inputs(N, T, H, K, V, seed=seed, per_dim_gate=per_dim_gate,
                          normalise=normalise, HV=HV, gate_mean=gate_mean,
                          beta_mode=beta_mode, gate=gate)
    gen = torch.Generator("cpu").manual_seed(int(seed) + 1)
    pool = torch.randn(num_slots, HV, V, K, generator=gen, dtype=torch.float32) * state_std
    cols = max(index_cols, 1)
    if N * cols > num_slots:
        raise ValueError("the pool must hold a distinct slot for every index")
    slots = torch.randperm(num_slots, generator=gen)[:N * cols].to(torch.int32).reshape(N, cols)
    acc = None
    if index_cols > 0:
        acc = torch.randint(1, index_cols + 1, (N,), generator=gen, dtype=torch.int32)
        if accepted is not None:
            acc = torch.tensor(list(accepted), dtype=torch.int32)
    else:
        slots = slots[:, 0].contiguous()
    for n in padded:
        slots[n] = -1
    return DecodeInputs(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, pool.contiguous(),
                        slots.contiguous(), acc)


def decode_workload_inputs(w: DecodeWorkload, seed: int, **overrides) -> DecodeInputs:
    kw = dict(index_cols=w.index_cols, K=w.K, V=w.V, per_dim_gate=w.per_dim_gate,
              normalise=not w.qk_l2norm, lengths=w.lengths)
    kw.update(overrides)
    return make_decode_inputs(w.N, w.T, w.H, w.HV, w.num_slots, seed=seed, **kw)
