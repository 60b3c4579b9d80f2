"""Seeded synthetic inputs for the Sparse Delta Memory hot path.

Shared by the CPU oracle's tests and the HIP path's tests and benchmark.  This
module only draws random tensors of the workloads' shapes and distributions;
it holds none of the method's arithmetic (no scoring, selection, weighting or
update).  Tensors are created with torch on the requested device; each tensor
has its own seeded generator, so a workload is reproducible per device.

Workloads (sizes and distributions as specified for the five benchmark
configurations; N(mu, var) names a variance):

* tiny  : B=1 H=1 T=64 d_k=32 n_sub=32 (N=1024) d_v=16 W=R=8, fp32.
          q', k' ~ N(0,1); sub-keys ~ N(0,1/16); v ~ N(0,1);
          alpha = sigmoid(N(3,1)); beta = sigmoid(N(0,1)); M0 = 0.
* mid   : B=4 H=4 T=2048 d_k=128 n_sub=256 (N=65536) d_v=64 W=R=32; q', k',
          v, sub-keys bf16; sub-keys ~ N(0, 1/(d_k/2)); M0 ~ N(0, 0.01) fp32.
* large : B=8 H=8 T=4096 d_k=128 n_sub=1024 (N=2^20) d_v=64 W=R=64; as mid,
          head h's sub-keys scaled by linspace(0.5, 2, H)[h].
* long  : B=1 H=16 T=65536 d_k=256 n_sub=1024 (N=2^20) d_v=128 W=R=128; bf16;
          keys and queries drawn from 4096 recurring Gaussian prototypes per
          head plus N(0, 0.1^2) noise (queries pick prototypes independently).
* gdn   : dense gated-delta baseline, B=16 H=16 T=8192 d_k=d_v=128, fp32;
          k, q = g/|g| with g ~ N(0, I); v ~ N(0,1); gates as tiny; S0 = 0.
* raven : routed slots with selective decay on the same table and scan:
          B=8 H=8 T=4096, M=1024 slots (n_sub=32), K=32 routed slots per
          token and side, rows of d=128 (key and value states side by side);
          router logits zk, zq ~ N(0,1) fp32 [B,H,T,M]; decay
          a = -softplus(N(0,1)); content u ~ N(0,1) bf16 (in v); the scan's
          alpha and beta are 1; S0 ~ N(0, 0.01).
* decode: serving batch of B=32 sequences x H=8 heads at large's per-stream
          shape and distributions, T=64 decoding steps of one token each;
          `decode_layout` gives the step-major, head-major tensors and
          `make_m0(..., head_major=True)` the table as [H,B,N,d_v].
"""
from dataclasses import dataclass, replace
from typing import Optional

import torch

BASE_SEED = 1234

# one id per drawn tensor, so each gets an independent generator
_TENSOR_IDS = {"q": 1, "k": 2, "subkeys": 3, "v": 4, "alpha": 5, "beta": 6, "m0": 7,
               "proto": 8, "proto_k": 9, "proto_q": 10, "noise_k": 11, "noise_q": 12,
               "zk": 13, "zq": 14, "decay": 15}


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # position in the benchmark's configuration list
    B: int
    H: int
    T: int
    d_k: int
    n_sub: int
    d_v: int
    W: int
    R: int
    bf16: bool            # q', k', v, sub-keys in bf16 (else fp32)
    m0_std: float         # 0 -> M0 = 0
    keys: str = "gauss"   # "gauss" or "proto"
    head_scale: Optional[tuple] = None  # per-head sub-key scale range (lo, hi)
    n_proto: int = 4096
    proto_noise: float = 0.1
    dense: bool = False   # the dense gated-delta baseline

    @property
    def N(self) -> int:
        return self.n_sub * self.n_sub

    @property
    def streams(self) -> int:
        return self.B * self.H

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    def table_bytes(self) -> int:
        if self.dense:
            return self.streams * self.d_v * self.d_k * 4
        return self.streams * self.N * self.d_v * 4

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 0, B=1, H=1, T=64, d_k=32, n_sub=32, d_v=16, W=8, R=8,
                     bf16=False, m0_std=0.0),
    "mid": Workload("mid", 1, B=4, H=4, T=2048, d_k=128, n_sub=256, d_v=64, W=32, R=32,
                    bf16=True, m0_std=0.1),
    "large": Workload("large", 2, B=8, H=8, T=4096, d_k=128, n_sub=1024, d_v=64, W=64, R=64,
                      bf16=True, m0_std=0.1, head_scale=(0.5, 2.0)),
    "long": Workload("long", 3, B=1, H=16, T=65536, d_k=256, n_sub=1024, d_v=128, W=128,
                     R=128, bf16=True, m0_std=0.1, keys="proto"),
    "gdn": Workload("gdn", 4, B=16, H=16, T=8192, d_k=128, n_sub=0, d_v=128, W=0, R=0,
                    bf16=False, m0_std=0.0, dense=True),
    "raven": Workload("raven", 6, B=8, H=8, T=4096, d_k=0, n_sub=32, d_v=128, W=32, R=32,
                      bf16=True, m0_std=0.1, keys="route"),
    "decode": Workload("decode", 5, B=32, H=8, T=64, d_k=128, n_sub=1024, d_v=64, W=64, R=64,
                       bf16=True, m0_std=0.1, head_scale=(0.5, 2.0)),
}


def _gen(wl: Workload, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed * 1000 + _TENSOR_IDS[name])
    return g


def _randn(wl, name, shape, device, std=1.0, mean=0.0):
    x = torch.randn(shape, generator=_gen(wl, name, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x


def make_inputs(wl: Workload, device="cpu", with_m0: bool = True) -> dict:
    """Draw every input of one workload on `device`.

    Returns q, k, subkeys, v (bf16 or fp32), alpha, beta (fp32) and, when
    with_m0, m0 (fp32 [B,H,N,d_v]) -- or, for the dense baseline, q, k, v,
    alpha, beta and s0 (zeros [B,H,d_v,d_k])."""
    B, H, T = wl.B, wl.H, wl.T
    out = {}
    out["alpha"] = torch.sigmoid(_randn(wl, "alpha", (B, H, T), device, mean=3.0))
    out["beta"] = torch.sigmoid(_randn(wl, "beta", (B, H, T), device))
    if wl.dense:
        g = _randn(wl, "k", (B, H, T, wl.d_k), device)
        out["k"] = g / g.norm(dim=-1, keepdim=True)
        g = _randn(wl, "q", (B, H, T, wl.d_k), device)
        out["q"] = g / g.norm(dim=-1, keepdim=True)
        out["v"] = _randn(wl, "v", (B, H, T, wl.d_v), device)
        out["s0"] = torch.zeros((B, H, wl.d_v, wl.d_k), device=device, dtype=torch.float32)
        return out

    if wl.keys == "route":
        M = wl.N
        out["zk"] = _randn(wl, "zk", (B, H, T, M), device)
        out["zq"] = _randn(wl, "zq", (B, H, T, M), device)
        out["a"] = -torch.nn.functional.softplus(_randn(wl, "decay", (B, H, T), device))
        out["alpha"] = torch.ones((B, H, T), device=device)
        out["beta"] = torch.ones((B, H, T), device=device)
        out["v"] = _randn(wl, "v", (B, H, T, wl.d_v), device)
        if wl.bf16:
            out["v"] = out["v"].to(torch.bfloat16)
        if with_m0:
            out["m0"] = make_m0(wl, device)
        return out
    dh = wl.d_k // 2
    if wl.keys == "proto":
        proto = _randn(wl, "proto", (H, wl.n_proto, wl.d_k), device)
        for name, pname, nname in (("k", "proto_k", "noise_k"), ("q", "proto_q", "noise_q")):
            pick = torch.randint(0, wl.n_proto, (B, H, T), generator=_gen(wl, pname, device),
                                 device=device)
            hsel = torch.arange(H, device=device).view(1, H, 1).expand(B, H, T)
            x = proto[hsel, pick]
            x.add_(_randn(wl, nname, (B, H, T, wl.d_k), device, std=wl.proto_noise))
            out[name] = x
    else:
        out["q"] = _randn(wl, "q", (B, H, T, wl.d_k), device)
        out["k"] = _randn(wl, "k", (B, H, T, wl.d_k), device)
    C = _randn(wl, "subkeys", (H, 2, wl.n_sub, dh), device, std=dh ** -0.5)
    if wl.head_scale is not None:
        lo, hi = wl.head_scale
        C.mul_(torch.linspace(lo, hi, H, device=device).view(H, 1, 1, 1))
    out["subkeys"] = C
    out["v"] = _randn(wl, "v", (B, H, T, wl.d_v), device)
    if wl.bf16:
        for name in ("q", "k", "subkeys", "v"):
            out[name] = out[name].to(torch.bfloat16)
    if with_m0:
        out["m0"] = make_m0(wl, device)
    return out


def make_m0(wl: Workload, device="cpu", head_major: bool = False) -> torch.Tensor:
    """Initial memory table M0 [B,H,N,d_v] fp32 ([H,B,N,d_v] when head_major)."""
    shape = (wl.H, wl.B, wl.N, wl.d_v) if head_major else (wl.B, wl.H, wl.N, wl.d_v)
    if wl.m0_std == 0.0:
        return torch.zeros(shape, device=device, dtype=torch.float32)
    return _randn(wl, "m0", shape, device, std=wl.m0_std)


def decode_layout(x: dict) -> dict:
    """Per-token inputs of make_inputs rearranged for decoding one token per
    stream per step: q, k [T,H,B,d_k], v [T,H,B,d_v], alpha, beta [T,H,B]
    (step t, head h, sequence b); subkeys unchanged."""
    out = {"subkeys": x["subkeys"]}
    for name in ("q", "k", "v"):
        out[name] = x[name].permute(2, 1, 0, 3).contiguous()
    for name in ("alpha", "beta"):
        out[name] = x[name].permute(2, 1, 0).contiguous()
    return out


def to_numpy(t: torch.Tensor):
    """Host numpy view of a tensor; bf16 becomes its raw uint16 bit pattern."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
