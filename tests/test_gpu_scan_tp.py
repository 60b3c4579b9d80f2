"""The time-parallel scan (sdm_scan_timeparallel) on an MI355X.

Rules: the table and the outputs are bit-identical to the oracle's scan (each
element goes through the same fp32 operations in the same order: writes in
time order per row, reads summed in rank order).  At full size the table is
also bit-identical to the sequential GPU scan's.  Slot lists come from seeded
generators or from the oracle's own addressing, never from the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import np_, say

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


def scan_case(dev, B, H, T, n_sub, d_v, W, R, seed, v_bf16=False, hot=None):
    g = torch.Generator().manual_seed(seed)
    N = n_sub * n_sub
    span = N if hot is None else hot
    widx = torch.stack([torch.randperm(span, generator=g)[:W] for _ in range(B * H * T)])
    ridx = torch.stack([torch.randperm(span, generator=g)[:R] for _ in range(B * H * T)])
    d = dict(widx=widx.view(B, H, T, W).int(),
             wwt=torch.softmax(torch.randn(B * H * T, W, generator=g), -1).view(B, H, T, W),
             ridx=ridx.view(B, H, T, R).int(),
             rwt=torch.softmax(torch.randn(B * H * T, R, generator=g), -1).view(B, H, T, R),
             v=torch.randn(B, H, T, d_v, generator=g),
             alpha=torch.sigmoid(torch.randn(B, H, T, generator=g) + 3),
             beta=torch.sigmoid(torch.randn(B, H, T, generator=g)),
             M0=torch.randn(B, H, N, d_v, generator=g) * 0.1)
    if v_bf16:
        d["v"] = d["v"].to(torch.bfloat16)
    return {k: t.contiguous().to(dev) for k, t in d.items()}


@pytest.mark.parametrize("label,args", [
    ("small d_v=16", dict(B=1, H=2, T=50, n_sub=16, d_v=16, W=8, R=8, seed=1)),
    ("d_v=64", dict(B=2, H=2, T=129, n_sub=64, d_v=64, W=32, R=32, seed=2)),
    ("bf16 v, ragged T", dict(B=1, H=3, T=77, n_sub=32, d_v=32, W=16, R=24, seed=3,
                              v_bf16=True)),
    ("hot slots, deep chains", dict(B=2, H=1, T=200, n_sub=32, d_v=32, W=16, R=16, seed=4,
                                    hot=48)),
    ("hot W=1", dict(B=1, H=1, T=300, n_sub=8, d_v=32, W=1, R=3, seed=5, hot=4)),
    ("W=R=128, d_v=256", dict(B=2, H=2, T=40, n_sub=32, d_v=256, W=128, R=128, seed=6,
                              hot=300)),
    ("T=1", dict(B=1, H=1, T=1, n_sub=8, d_v=32, W=4, R=4, seed=7)),
    # N = 1089 needs 11 slot bits: two passes of 6-bit digits
    ("N=33^2, two 6-bit passes", dict(B=2, H=2, T=90, n_sub=33, d_v=64, W=24, R=40, seed=8)),
    # N = 16: one 4-bit pass, every slot hot
    ("N=16", dict(B=1, H=3, T=64, n_sub=4, d_v=16, W=5, R=7, seed=9)),
])
def test_timeparallel_equals_oracle_bitwise(dev, label, args):
    say(f"case: time-parallel scan {label}", args)
    d = scan_case(dev, **args)
    M = d["M0"].clone()
    out = sdm().scan_timeparallel(M, d["widx"], d["wwt"], d["ridx"], d["rwt"], d["v"],
                                  d["alpha"], d["beta"])
    torch.cuda.synchronize()
    M_ref = np_(d["M0"]).copy()
    out_ref = oracle.scan(M_ref, np_(d["widx"]), np_(d["wwt"]), np_(d["ridx"]), np_(d["rwt"]),
                          np_(d["v"]), np_(d["alpha"]), np_(d["beta"]))
    assert np.array_equal(np_(M).view(np.uint32), M_ref.view(np.uint32)), "table differs"
    assert np.array_equal(np_(out).view(np.uint32), out_ref.view(np.uint32)), "outputs differ"


def test_timeparallel_large_full_size(dev):
    """N = 2^20, 64 streams: the table equals the sequential scan's bit for bit;
    two streams run on the oracle's own addressing and match the oracle's
    table and outputs bit for bit."""
    wl = synth.WORKLOADS["large"]
    say("case: time-parallel scan, large", wl)
    x = synth.make_inputs(wl, device=dev)
    g = [t.clone() for t in sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)]
    picks = ((0, 0), (wl.B - 1, wl.H - 1))
    refs = {}
    for b, h in picks:
        sl = (slice(b, b + 1), slice(h, h + 1))
        r = oracle.score_topk(np_(x["q"][sl]), np_(x["k"][sl]), np_(x["subkeys"][h:h + 1]),
                              wl.W, wl.R)
        for j, key in enumerate(("widx", "wwt", "ridx", "rwt")):
            g[j][b, h] = torch.from_numpy(r[key][0, 0]).to(dev)
        M_ref = np_(x["m0"][sl]).copy()
        o_ref = oracle.scan(M_ref, r["widx"], r["wwt"], r["ridx"], r["rwt"], np_(x["v"][sl]),
                            np_(x["alpha"][sl]), np_(x["beta"][sl]))
        refs[(b, h)] = (M_ref[0, 0], o_ref[0, 0])
    M_seq = x["m0"].clone()
    sdm().scan(M_seq, *g, x["v"], x["alpha"], x["beta"])
    M = x["m0"]
    out = sdm().scan_timeparallel(M, *g, x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    assert torch.equal(M, M_seq), "table differs from the sequential scan's"
    del M_seq
    for b, h in picks:
        assert np.array_equal(np_(M[b, h]), refs[(b, h)][0])
        assert np.array_equal(np_(out[b, h]), refs[(b, h)][1])
