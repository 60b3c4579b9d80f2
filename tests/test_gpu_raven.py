"""Routed slots with selective decay on the GPU against the Raven oracle (run on an MI355X).

Rules:
  * the router's slot lists equal the oracle's exactly (selection is on the
    logits, which both sides read unrounded; ties to the lower slot);
  * gates and write strengths within 1e-5 + 1e-4|ref| (fp32 exp/expm1 on the
    GPU against fp64);
  * the table and the outputs of router + scan within 1e-5 + 1e-4|ref| of the
    oracle's recurrence (fp32 against fp64, a few roundings per token per row).
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import close, np_, say
from oracle import raven as rv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_addressed_linear_amd as sdm
    sdm.lib()
    return torch.device("cuda:0")


def sdm():
    import sparse_addressed_linear_amd as m
    return m


def test_router_vs_oracle_with_ties(dev):
    g = torch.Generator().manual_seed(41)
    for (B, H, T, M, K) in ((1, 2, 33, 64, 8), (2, 1, 17, 1024, 32), (1, 1, 9, 4096, 128),
                            (1, 1, 5, 100, 100),
                            # register form: 256 candidates sorted at once, a ragged M, one slot
                            (1, 2, 7, 1024, 128), (1, 1, 6, 1000, 77), (1, 1, 4, 1, 1)):
        say(f"case: router B={B} H={H} T={T} M={M} K={K}")
        # integer logits: many exact ties
        zk = torch.randint(-4, 5, (B, H, T, M), generator=g).float()
        zq = torch.randn(B, H, T, M, generator=g) * 2
        a = -torch.nn.functional.softplus(torch.randn(B, H, T, generator=g))
        widx, wcoef, ridx, rwt = sdm().route_topk(zk.to(dev), zq.to(dev), a.to(dev), K)
        torch.cuda.synchronize()
        ref = rv.route_tokens(np_(zk), np_(zq), np_(a), K)
        assert np.array_equal(np_(widx), ref["widx"])
        assert np.array_equal(np_(ridx), ref["ridx"])
        assert np.all(close(np_(wcoef), ref["wcoef"]))
        assert np.all(close(np_(rwt), ref["rwt"]))


def run_raven(wl, x):
    widx, wcoef, ridx, rwt = sdm().route_topk(x["zk"], x["zq"], x["a"], wl.W)
    M = x["m0"]
    out = sdm().scan(M, widx, wcoef, ridx, rwt, x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    return M, out


@pytest.mark.parametrize("name,shape,streams", [
    ("small", dict(B=2, H=2, T=300, n_sub=16, d_v=32, W=8, R=8), None),
    ("full size, sampled", {}, ((0, 0), (7, 7))),
])
def test_raven_step_vs_oracle(dev, name, shape, streams):
    wl = synth.WORKLOADS["raven"].with_(**shape)
    say(f"case: raven {name}", wl)
    x = synth.make_inputs(wl, device=dev)
    picks = streams or [(b, h) for b in range(wl.B) for h in range(wl.H)]
    S0 = {p: np_(x["m0"][p]).astype(np.float64) for p in picks}
    M, out = run_raven(wl, x)
    for b, h in picks:
        S = S0[(b, h)]
        u = x["v"][b, h].float().cpu().numpy().astype(np.float64)  # bf16 values, exact
        o = rv.raven_scan_stream(S, np_(x["zk"][b, h]), np_(x["zq"][b, h]), np_(x["a"][b, h]), u,
                                 wl.W)
        assert np.all(close(np_(M[b, h]), S)), f"table of stream ({b},{h})"
        assert np.all(close(np_(out[b, h]), o)), f"outputs of stream ({b},{h})"
