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
                normalise: bool = True, HV: Optional[int] = None) -> Inputs:
    """Draw one seeded batch.

    gate: "logsigmoid" -> g = logsigmoid(N(gate_mean, 1)); "zero" -> g = 0.
    beta_mode: "sigmoid" -> sigmoid(N(0, 1)); "zero" -> 0; "one" -> 1.
    With ``lengths`` the batch is packed (B must be 1, T = sum(lengths)) and
    ``cu_seqlens`` is the int32 prefix sum of the lengths.  ``HV`` (a multiple of H)
    gives v, g, beta and the initial state HV value heads while q and k keep H.
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
    cu = None
    if lengths is not None:
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return Inputs(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16),
                  g.contiguous(), beta.contiguous(),
                  None if s0 is None else s0.contiguous(), cu, chunk_size)


def workload_inputs(w: Workload, seed: int, **overrides) -> Inputs:
    kw = dict(per_dim_gate=w.per_dim_gate, lengths=w.lengths, initial_state=w.initial_state,
              chunk_size=w.chunk_size)
    kw.update(overrides)
    return make_inputs(w.B, w.T, w.H, w.K, w.V, seed=seed, **kw)
