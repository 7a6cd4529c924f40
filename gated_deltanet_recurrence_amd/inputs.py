"""Seeded synthetic inputs for the Gated Delta Rule token mixer.

This module is shared by the tests, the benchmark and the oracle checks. It
holds sampling recipes only: draws from torch's CPU generator, the
distribution transforms the workloads are defined by, and rounding to the
storage dtype. It does none of the mixer's own arithmetic on its outputs and
it imports neither the HIP binding nor the oracle.

Workloads (all shapes token-major, ``[B, T, H, D]``):

* ``tiny``    - B=1, H=1, T=64, d=16, fp32, zero initial state.
* ``prefill`` - B=4, H=16, T=4096, d=128, bf16 q/k/v, fp32 gates.
* ``decode``  - B=256, H=32, d=128, fp32 state N(0, 0.02) resident on device.
* ``mixer``   - B=8, T=8192, H=16, d=128, raw (pre-conv) bf16 projections.
* ``varlen``  - H=32, d=128, 8 packed sequences, lengths log-uniform in
                [512, 65536], non-zero initial states.
* ``decode_mixer`` - one token of the whole mixer at B=256, H=32, d=128:
                raw projections, a conv cache and the fp32 state.

Conventions shared by every recipe:

* "N(m, s)" means mean m and standard deviation s.
* Unit vectors are sampled as Gaussian vectors divided by their Euclidean
  length (uniform on the sphere), in fp32, then rounded to the storage dtype.
* Decay gates are handed over in log space, ``g = log(alpha)``, as fp32.
* ``beta = sigmoid(N(0,1))`` per (token, head), fp32.
* bf16 rounding is round-to-nearest-even (torch's CPU conversion).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

__all__ = [
    "GDNCase", "MixerCase", "DecodeMixerCase", "unit_gaussian", "log_uniform_lengths",
    "make_tiny", "make_prefill", "make_decode", "make_mixer", "make_varlen",
    "make_decode_mixer", "make_channel_gated", "make_long_memory",
    "make_case", "WORKLOADS",
]


@dataclass
class GDNCase:
    """Inputs of one recurrence call (prefill or decode), on the host.

    q, k: [B, T, H_k, d_k]; v: [B, T, H, d_v] in ``dtype`` (decode: T=1
    folded away by the caller); g, beta: [B, T, H] fp32; s0: [N, H, d_v, d_k]
    fp32 or None; cu_seqlens: int32 [N+1] or None. H counts the value heads,
    H_k (dividing H) the query/key heads.
    """
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    s0: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    scale: float
    dtype: str                      # "f32" or "bf16"
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def T(self) -> int:
        return self.q.shape[1]

    @property
    def H(self) -> int:
        return self.v.shape[2]

    @property
    def Hk(self) -> int:
        return self.q.shape[2]

    @property
    def d_k(self) -> int:
        return self.q.shape[3]

    @property
    def d_v(self) -> int:
        return self.v.shape[3]

    @property
    def N(self) -> int:
        return self.B if self.cu_seqlens is None else self.cu_seqlens.numel() - 1


@dataclass
class MixerCase:
    """Raw (pre-convolution) inputs of the full token mixer, on the host.

    q_raw, k_raw: [B, T, H_k, d_k]; v_raw, z: [B, T, H, d_v]; a, b: [B, T, H];
    conv_w: [2*H_k*d_k + H*d_v, 4] (channel order q, k, v; tap 3 multiplies the
    current token); A: [H] fp32; dt_bias: [H] fp32 or None; norm_w: [d_v]
    fp32 or None (ones).
    """
    name: str
    q_raw: torch.Tensor
    k_raw: torch.Tensor
    v_raw: torch.Tensor
    z: torch.Tensor
    a: torch.Tensor
    b: torch.Tensor
    conv_w: torch.Tensor
    A: torch.Tensor
    dt_bias: Optional[torch.Tensor]
    norm_w: Optional[torch.Tensor]
    scale: float
    eps: float
    dtype: str
    cu_seqlens: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)


_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed: int) -> torch.Generator:
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    return gen


def _normal(gen, shape, std=1.0, mean=0.0):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x


def _uniform(gen, shape, lo, hi):
    return torch.rand(shape, generator=gen, dtype=torch.float32) * (hi - lo) + lo


def unit_gaussian(gen, shape) -> torch.Tensor:
    """Gaussian vectors along the last axis divided by their length (fp32)."""
    x = _normal(gen, shape)
    x.div_(torch.linalg.vector_norm(x, dim=-1, keepdim=True))
    return x


def log_uniform_lengths(gen, n: int, lo: int, hi: int) -> list:
    """``floor(exp(U(ln lo, ln hi)))`` for n sequences."""
    u = torch.rand((n,), generator=gen, dtype=torch.float64)
    lens = torch.floor(torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
    return [int(x) for x in lens.clamp(min=lo, max=hi).tolist()]


def _sigmoid_gaussian(gen, shape) -> torch.Tensor:
    return torch.sigmoid(_normal(gen, shape))


def _mamba_log_decay(a: torch.Tensor, A: torch.Tensor) -> torch.Tensor:
    """Distribution recipe of the decay gate: log(alpha) = -A[h]*softplus(a)."""
    return -(A.view(1, 1, -1) * torch.nn.functional.softplus(a))


def make_tiny(seed: int = 1, T: int = 64, d: int = 16, H: int = 1, B: int = 1,
              dtype: str = "f32") -> GDNCase:
    """B=1, H=1, T=64, d_k=d_v=16, fp32; alpha ~ U(0.9, 1), zero initial state."""
    gen = _gen(seed)
    td = _TORCH_DTYPE[dtype]
    q = unit_gaussian(gen, (B, T, H, d)).to(td)
    k = unit_gaussian(gen, (B, T, H, d)).to(td)
    v = _normal(gen, (B, T, H, d)).to(td)
    alpha = _uniform(gen, (B, T, H), 0.9, 1.0)
    g = torch.log(alpha)
    beta = _sigmoid_gaussian(gen, (B, T, H))
    return GDNCase("tiny", q, k, v, g, beta, None, None, 1.0 / math.sqrt(d), dtype)


def make_prefill(seed: int = 2, B: int = 4, T: int = 4096, H: int = 16, d: int = 128,
                 dtype: str = "bf16", with_state: bool = False,
                 Hk: Optional[int] = None) -> GDNCase:
    """Chunked-prefill workload: q,k unit Gaussian, v ~ N(0,1), log(alpha) =
    -A*softplus(a) with a ~ N(0,1) and A ~ U(0.5, 2) per head, beta =
    sigmoid(N(0,1)), zero initial state unless ``with_state``. ``Hk`` query/key
    heads (default H)."""
    gen = _gen(seed)
    td = _TORCH_DTYPE[dtype]
    Hk = H if Hk is None else Hk
    q = unit_gaussian(gen, (B, T, Hk, d)).to(td)
    k = unit_gaussian(gen, (B, T, Hk, d)).to(td)
    v = _normal(gen, (B, T, H, d)).to(td)
    a = _normal(gen, (B, T, H))
    A = _uniform(gen, (H,), 0.5, 2.0)
    g = _mamba_log_decay(a, A).contiguous()
    beta = _sigmoid_gaussian(gen, (B, T, H))
    s0 = _normal(gen, (B, H, d, d), std=0.02) if with_state else None
    return GDNCase("prefill", q, k, v, g, beta, s0, None, 1.0 / math.sqrt(d), dtype,
                   meta={"A": A})


def make_decode(seed: int = 3, B: int = 256, H: int = 32, d: int = 128,
                dtype: str = "bf16", Hk: Optional[int] = None) -> GDNCase:
    """Single-token decode: fp32 state N(0, 0.02) [B,H,d,d]; q,k unit Gaussian,
    v ~ N(0,1); alpha ~ U(0.8, 1); beta = sigmoid(N(0,1)). Tensors carry a
    T=1 axis: q,k [B,1,Hk,d], v [B,1,H,d], g,beta [B,1,H]."""
    gen = _gen(seed)
    td = _TORCH_DTYPE[dtype]
    Hk = H if Hk is None else Hk
    q = unit_gaussian(gen, (B, 1, Hk, d)).to(td)
    k = unit_gaussian(gen, (B, 1, Hk, d)).to(td)
    v = _normal(gen, (B, 1, H, d)).to(td)
    alpha = _uniform(gen, (B, 1, H), 0.8, 1.0)
    g = torch.log(alpha)
    beta = _sigmoid_gaussian(gen, (B, 1, H))
    s0 = _normal(gen, (B, H, d, d), std=0.02)
    return GDNCase("decode", q, k, v, g, beta, s0, None, 1.0 / math.sqrt(d), dtype)


def make_mixer(seed: int = 4, B: int = 8, T: int = 8192, H: int = 16, d: int = 128,
               dtype: str = "bf16", Hk: Optional[int] = None) -> MixerCase:
    """Full token mixer from pre-projected inputs: q,k,v,z,a,b ~ N(0,1);
    depthwise conv weights N(0, 0.5) with 4 taps; A ~ U(0.5, 2) per head;
    no dt_bias; RMSNorm weight ones, eps 1e-6; scale d^-1/2. ``Hk`` query/key
    heads (default H)."""
    gen = _gen(seed)
    td = _TORCH_DTYPE[dtype]
    Hk = H if Hk is None else Hk
    q = _normal(gen, (B, T, Hk, d)).to(td)
    k = _normal(gen, (B, T, Hk, d)).to(td)
    v = _normal(gen, (B, T, H, d)).to(td)
    z = _normal(gen, (B, T, H, d)).to(td)
    a = _normal(gen, (B, T, H)).to(td)
    b = _normal(gen, (B, T, H)).to(td)
    conv_w = _normal(gen, (2 * Hk * d + H * d, 4), std=0.5).to(td)
    A = _uniform(gen, (H,), 0.5, 2.0)
    return MixerCase("mixer", q, k, v, z, a, b, conv_w, A, None, None,
                     1.0 / math.sqrt(d), 1e-6, dtype)


def make_varlen(seed: int = 5, n_seq: int = 8, H: int = 32, d: int = 128,
                lo: int = 512, hi: int = 65536, dtype: str = "bf16",
                lengths: Optional[list] = None, Hk: Optional[int] = None) -> GDNCase:
    """Packed variable-length prefill: lengths log-uniform in [lo, hi];
    q,k unit Gaussian, v ~ N(0,1); initial states N(0, 0.02); a ~ N(-2, 1),
    A ~ U(0.5, 2) per head, log(alpha) = -A*softplus(a); beta = sigmoid(N(0,1)).
    Shapes: q,k [1, sum(lengths), Hk, d] (Hk defaults to H), v [1, sum(lengths),
    H, d], cu_seqlens int32 [n_seq+1]."""
    gen = _gen(seed)
    td = _TORCH_DTYPE[dtype]
    if lengths is None:
        lengths = log_uniform_lengths(gen, n_seq, lo, hi)
    n_seq = len(lengths)
    total = int(sum(lengths))
    cu = torch.zeros(n_seq + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    Hk = H if Hk is None else Hk
    q = unit_gaussian(gen, (1, total, Hk, d)).to(td)
    k = unit_gaussian(gen, (1, total, Hk, d)).to(td)
    v = _normal(gen, (1, total, H, d)).to(td)
    s0 = _normal(gen, (n_seq, H, d, d), std=0.02)
    a = _normal(gen, (1, total, H), mean=-2.0)
    A = _uniform(gen, (H,), 0.5, 2.0)
    g = _mamba_log_decay(a, A).contiguous()
    beta = _sigmoid_gaussian(gen, (1, total, H))
    return GDNCase("varlen", q, k, v, g, beta, s0, cu, 1.0 / math.sqrt(d), dtype,
                   meta={"lengths": lengths, "A": A})


def make_channel_gated(seed: int = 7, B: int = 2, T: int = 300, H: int = 4, d: int = 128,
                       dtype: str = "bf16", Hk: Optional[int] = None, with_state: bool = True,
                       lengths: Optional[list] = None) -> GDNCase:
    """Per-channel decay (one rate per key channel): q,k unit Gaussian, v ~
    N(0,1), log(alpha)[.., c] = -A[h]*softplus(a[.., c]) with a ~ N(0,1) per
    channel and A ~ U(0.5, 2) per head, beta = sigmoid(N(0,1)), initial states
    N(0, 0.02) when ``with_state``. g is [B, T, H, d]. With ``lengths`` the
    sequences are packed (B = 1, cu_seqlens)."""
    gen = _gen(seed)
    td = _TORCH_DTYPE[dtype]
    Hk = H if Hk is None else Hk
    cu = None
    if lengths is not None:
        B, T = 1, int(sum(lengths))
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    N = B if cu is None else len(lengths)
    q = unit_gaussian(gen, (B, T, Hk, d)).to(td)
    k = unit_gaussian(gen, (B, T, Hk, d)).to(td)
    v = _normal(gen, (B, T, H, d)).to(td)
    a = _normal(gen, (B, T, H, d))
    A = _uniform(gen, (H,), 0.5, 2.0)
    g = -(A.view(1, 1, -1, 1) * torch.nn.functional.softplus(a)).contiguous()
    beta = _sigmoid_gaussian(gen, (B, T, H))
    s0 = _normal(gen, (N, H, d, d), std=0.02) if with_state else None
    return GDNCase("channel_gated", q, k, v, g, beta, s0, cu, 1.0 / math.sqrt(d), dtype,
                   meta={"A": A, "lengths": lengths})


def make_long_memory(seed: int = 200, B: int = 2, T: int = 1024, H: int = 2, d: int = 128,
                     gate: str = "zero", with_state: bool = False, dtype: str = "bf16",
                     per_channel: bool = False, lengths: Optional[list] = None,
                     key_norm: Optional[tuple] = None) -> GDNCase:
    """Long-memory regime: what is written survives many chunks.

    ``gate="zero"``: g = 0 (alpha = 1), the delta rule without forgetting;
    ``gate="near_one"``: alpha ~ U(0.99, 1), g = log(alpha) (per key channel
    when ``per_channel``, g then [B, T, H, d]). q,k unit Gaussian, v ~ N(0,1),
    beta = sigmoid(N(0,1)), initial states N(0, 0.02) when ``with_state``.
    ``lengths``: packed sequences of these lengths instead (B = 1, T their
    sum, cu_seqlens set, one initial state per sequence). ``key_norm=(lo,
    hi)``: each key scaled to a norm ~ U(lo, hi) instead of 1 (drawn after
    everything else, so the other tensors are those of the unit-key case)."""
    gen = _gen(seed)
    td = _TORCH_DTYPE[dtype]
    cu, N = None, B
    if lengths is not None:
        B, T, N = 1, int(sum(lengths)), len(lengths)
        cu = torch.zeros(N + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    q = unit_gaussian(gen, (B, T, H, d)).to(td)
    k32 = unit_gaussian(gen, (B, T, H, d))
    v = _normal(gen, (B, T, H, d)).to(td)
    gshape = (B, T, H, d) if per_channel else (B, T, H)
    if gate == "zero":
        g = torch.zeros(gshape, dtype=torch.float32)
    elif gate == "near_one":
        g = torch.log(_uniform(gen, gshape, 0.99, 1.0))
    else:
        raise ValueError(f"unknown gate recipe {gate!r}")
    beta = _sigmoid_gaussian(gen, (B, T, H))
    s0 = _normal(gen, (N, H, d, d), std=0.02) if with_state else None
    if key_norm is not None:
        k32 = k32 * _uniform(gen, (B, T, H, 1), float(key_norm[0]), float(key_norm[1]))
    k = k32.to(td)
    return GDNCase("long_memory", q, k, v, g.contiguous(), beta, s0, cu, 1.0 / math.sqrt(d),
                   dtype, meta={"gate": gate, "per_channel": per_channel, "lengths": lengths})


@dataclass
class DecodeMixerCase:
    """Inputs of one fused single-token mixer step, on the host.

    q_raw, k_raw: [B, H_k, d_k]; v_raw, z: [B, H, d_v]; a, b: [B, H];
    conv_w: [C, 4], C = 2*H_k*d_k + H*d_v; conv_state: [B, 3, C] (the last
    three raw inputs per channel, oldest first); state: [B, H, d_v, d_k] fp32;
    A: [H] fp32.
    """
    name: str
    q_raw: torch.Tensor
    k_raw: torch.Tensor
    v_raw: torch.Tensor
    z: torch.Tensor
    a: torch.Tensor
    b: torch.Tensor
    conv_w: torch.Tensor
    conv_state: torch.Tensor
    A: torch.Tensor
    state: torch.Tensor
    scale: float
    eps: float
    dtype: str


def make_decode_mixer(seed: int = 6, B: int = 256, H: int = 32, d: int = 128,
                      dtype: str = "bf16", Hk: Optional[int] = None) -> DecodeMixerCase:
    """One token of the mixer at the decode shape: the token's projections
    q,k,v,z,a,b ~ N(0,1); conv weights N(0, 0.5); a conv cache of three earlier
    raw inputs N(0,1) per channel; fp32 state N(0, 0.02); A ~ U(0.5, 2) per
    head; no dt_bias, norm weight ones, eps 1e-6, scale d^-1/2."""
    gen = _gen(seed)
    td = _TORCH_DTYPE[dtype]
    Hk = H if Hk is None else Hk
    C = 2 * Hk * d + H * d
    q = _normal(gen, (B, Hk, d)).to(td)
    k = _normal(gen, (B, Hk, d)).to(td)
    v = _normal(gen, (B, H, d)).to(td)
    z = _normal(gen, (B, H, d)).to(td)
    a = _normal(gen, (B, H)).to(td)
    b = _normal(gen, (B, H)).to(td)
    conv_w = _normal(gen, (C, 4), std=0.5).to(td)
    conv_state = _normal(gen, (B, 3, C)).to(td)
    A = _uniform(gen, (H,), 0.5, 2.0)
    state = _normal(gen, (B, H, d, d), std=0.02)
    return DecodeMixerCase("decode_mixer", q, k, v, z, a, b, conv_w, conv_state, A, state,
                           1.0 / math.sqrt(d), 1e-6, dtype)


WORKLOADS = {
    "tiny": make_tiny,
    "prefill": make_prefill,
    "decode": make_decode,
    "mixer": make_mixer,
    "varlen": make_varlen,
    "decode_mixer": make_decode_mixer,
    "channel_gated": make_channel_gated,
    "long_memory": make_long_memory,
}


def make_case(name: str, **kw):
    return WORKLOADS[name](**kw)
