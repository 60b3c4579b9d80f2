"""Empty sequences (T = 0) through every entry point that takes a T axis (run on an MI355X).

Rules: each call returns success, every output with a T axis is empty, and
every state the call owns is left bit for bit as it was (the table and its
gradient for the scans, the dense state for GDN, the sub-key gradient for the
addressing adjoint): with no tokens the recurrence is the identity.
"""
import pytest
import torch

import synth
from gpu_util import say

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


def empty(x):
    """The same tensors cut to T = 0 along axis 2 (sub-keys and tables keep their shape)."""
    keep = ("subkeys", "m0")
    return {k: (v if k in keep else v[:, :, :0].contiguous()) for k, v in x.items()}


@pytest.mark.parametrize("name", ["tiny", "mid"])
def test_addressing_empty(dev, name):
    wl = synth.WORKLOADS[name].with_(B=2, H=2, T=8)
    say(f"case: empty addressing {name}", wl)
    x = empty(synth.make_inputs(wl, device=dev, with_m0=False))
    for packed in (None, sdm().pack_subkeys(x["subkeys"]) if name == "mid" else None):
        widx, wwt, ridx, rwt = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R,
                                                packed=packed)
        torch.cuda.synchronize()
        assert widx.shape == (2, 2, 0, wl.W) and ridx.shape == (2, 2, 0, wl.R)
        assert wwt.numel() == 0 and rwt.numel() == 0
    ds0 = torch.randn(x["subkeys"].shape, device=dev)
    ds = ds0.clone()
    dq, dk, ds = sdm().score_topk_backward(x["q"], x["k"], x["subkeys"], widx, wwt, ridx, rwt,
                                           wwt, rwt, dsubkeys=ds)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and dk.numel() == 0 and torch.equal(ds, ds0)


def test_scans_empty(dev):
    wl = synth.WORKLOADS["tiny"].with_(B=2, H=3, T=8, n_sub=16, d_v=32, W=8, R=8)
    say("case: empty scans", wl)
    x = synth.make_inputs(wl, device=dev)
    B, H, N, d_v = x["m0"].shape
    e = lambda *s, dt=torch.float32: torch.empty((B, H, 0) + s, dtype=dt, device=dev)
    widx, ridx = e(wl.W, dt=torch.int32), e(wl.R, dt=torch.int32)
    wwt, rwt = e(wl.W), e(wl.R)
    v, al, be = e(d_v), e(), e()
    M0 = x["m0"].clone()
    M = M0.clone()
    out = sdm().scan(M, widx, wwt, ridx, rwt, v, al, be, tape=e(wl.W, d_v))
    out_tp = sdm().scan_timeparallel(M, widx, wwt, ridx, rwt, v, al, be)
    dM0 = torch.randn_like(M0)
    dM = dM0.clone()
    g = sdm().scan_backward(M, dM, widx, wwt, ridx, rwt, v, al, be, e(wl.W, d_v), e(d_v))
    torch.cuda.synchronize()
    assert out.shape == (B, H, 0, d_v) and out_tp.shape == (B, H, 0, d_v)
    assert torch.equal(M, M0), "the table moved"
    assert torch.equal(dM, dM0), "the table gradient moved"
    assert all(t.numel() == 0 for t in g.values())


def test_router_and_gdn_empty(dev):
    say("case: empty router and GDN")
    B, H, Mslots, K, d = 2, 2, 64, 8, 128
    z = torch.empty((B, H, 0, Mslots), device=dev)
    a = torch.empty((B, H, 0), device=dev)
    outs = sdm().route_topk(z, z, a, K)
    S0 = torch.randn((B, H, d, d), device=dev)
    S = S0.clone()
    kq = torch.empty((B, H, 0, d), device=dev)
    o = sdm().gdn_scan(S, kq, kq, kq, a, a)
    torch.cuda.synchronize()
    assert all(t.shape == (B, H, 0, K) for t in outs)
    assert o.shape == (B, H, 0, d) and torch.equal(S, S0)
