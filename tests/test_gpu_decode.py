"""Decoding: one token per stream per call, many streams at once (run on an MI355X).

A decode step is the same two calls as a sequence (addressing, then the scan)
with T = 1, laid out head-major so that the tokens of one head score together.
Rules:
  * stepping T tokens one call at a time gives the same bits as one call over
    the whole sequence: slot lists, weights, outputs and the final table;
  * sampled streams match the oracle by the rules of the sequence tests: slot
    sets modulo the gap rule, weights within 1e-5 + 1e-4|ref|, and end to end
    (the oracle's own addressing and scan) table and outputs within
    1e-5 + 1e-4|ref| for streams with no flagged token.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import close, compare_topk, np_, say

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


def run_decode(wl, xd, M, packed):
    """Steps 0..T-1; returns per-step slot lists [T,H,B,k] and outputs [T,H,B,d_v]."""
    bufs = {}
    idx = [[], [], [], []]
    outs = []
    for t in range(wl.T):
        o = sdm().decode_step(M, xd["q"][t], xd["k"][t], xd["subkeys"], xd["v"][t],
                              xd["alpha"][t], xd["beta"][t], wl.W, wl.R, packed=packed,
                              bufs=bufs)
        outs.append(o.clone())
        for j in range(4):
            idx[j].append(bufs["idx"][j][0].clone())
    torch.cuda.synchronize()
    return [torch.stack(a) for a in idx], torch.stack(outs)


@pytest.mark.parametrize("use_packed", [True, False])
def test_decode_steps_equal_sequence_call(dev, use_packed):
    wl = synth.WORKLOADS["decode"].with_(B=12, H=3, T=9, n_sub=256, W=32, R=24)
    say(f"case: decode vs sequence, packed={use_packed}", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    xd = synth.decode_layout(x)
    M_dec = synth.make_m0(wl, dev, head_major=True)
    M_seq = M_dec.transpose(0, 1).contiguous()
    M0_host = np_(M_seq)
    g = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    out_seq = sdm().scan(M_seq, *g, x["v"], x["alpha"], x["beta"])
    packed = sdm().pack_subkeys(x["subkeys"]) if use_packed else None
    idx, outs = run_decode(wl, xd, M_dec, packed)
    # [T,H,B,*] -> [B,H,T,*]
    for j in range(4):
        assert torch.equal(idx[j].permute(2, 1, 0, 3), g[j]), f"slot list {j} differs"
    assert torch.equal(outs.permute(2, 1, 0, 3), out_seq)
    assert torch.equal(M_dec.transpose(0, 1), M_seq)
    # two sampled streams against the oracle's own addressing and scan, end to
    # end from M0 (a stream holding a token flagged by the gap rule is skipped)
    for b, h in ((0, 0), (wl.B - 1, wl.H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.score_topk(np_(x["q"][sl]), np_(x["k"][sl]), np_(x["subkeys"][h:h + 1]),
                                wl.W, wl.R)
        flags = 0
        for j, (ri, rw, gp) in enumerate(((ref["widx"], ref["wwt"], ref["wgap"]),
                                           (ref["ridx"], ref["rwt"], ref["rgap"]))):
            n, flagged, bad = compare_topk(np_(g[2 * j][sl]), np_(g[2 * j + 1][sl]), ri, rw, gp,
                                           wl.N)
            assert bad == 0
            flags += flagged
        M_ref = np.ascontiguousarray(M0_host[b:b + 1, h:h + 1])
        o_ref = oracle.scan(M_ref, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"],
                            np_(x["v"][sl]), np_(x["alpha"][sl]), np_(x["beta"][sl]))
        if flags:
            say(f"  stream ({b},{h}) holds a flagged token; end to end not compared")
            continue
        assert np.all(close(np_(M_dec[h, b]), M_ref[0, 0]))
        assert np.all(close(np_(outs[:, h, b]), o_ref[0, 0]))


def test_decode_full_size_sampled(dev):
    """The serving batch at N = 2^20 (32 sequences x 8 heads, 68.7 GB table):
    three steps, sampled streams checked against the oracle from M0."""
    wl = synth.WORKLOADS["decode"].with_(T=3)
    say("case: decode full size, 3 steps", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    xd = synth.decode_layout(x)
    M = synth.make_m0(wl, dev, head_major=True)
    picks = ((0, 0), (17, 3), (wl.B - 1, wl.H - 1))
    M0 = {p: np_(M[p[1], p[0]]) for p in picks}
    packed = sdm().pack_subkeys(x["subkeys"])
    idx, outs = run_decode(wl, xd, M, packed)
    for b, h in picks:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.score_topk(np_(x["q"][sl]), np_(x["k"][sl]), np_(x["subkeys"][h:h + 1]),
                                wl.W, wl.R)
        gi = [np_(idx[j][:, h, b])[None, None] for j in range(4)]
        flags = 0
        for j, (ri, rw, gp) in enumerate(((ref["widx"], ref["wwt"], ref["wgap"]),
                                           (ref["ridx"], ref["rwt"], ref["rgap"]))):
            n, flagged, bad = compare_topk(gi[2 * j], gi[2 * j + 1], ri, rw, gp, wl.N)
            say(f"  stream ({b},{h}) {'WR'[j]}: {n} tokens, {flagged} flagged, {bad} mismatched")
            assert bad == 0
            flags += flagged
        # end to end against the oracle's own addressing and scan
        M_ref = np.ascontiguousarray(M0[(b, h)][None, None])
        o_ref = oracle.scan(M_ref, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"],
                            np_(x["v"][sl]), np_(x["alpha"][sl]), np_(x["beta"][sl]))
        if flags:
            continue
        assert np.all(close(np_(M[h, b]), M_ref[0, 0]))
        assert np.all(close(np_(outs[:, h, b]), o_ref[0, 0]))
    del M
    torch.cuda.empty_cache()


def test_decode_graph_replays_match_eager(dev):
    """Decode steps captured in a HIP graph: every replay, with eager steps and
    synchronisations in between, gives the eager path's bits."""
    wl = synth.WORKLOADS["decode"].with_(B=8, H=2, T=4, n_sub=128, W=16, R=16)
    say("case: decode graph replays", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    xd = synth.decode_layout(x)
    MA = synth.make_m0(wl, dev, head_major=True)
    MB = MA.clone()
    packed = sdm().pack_subkeys(x["subkeys"])
    bA, bB = {}, {}

    def step(M, bufs, t):
        return sdm().decode_step(M, xd["q"][t], xd["k"][t], xd["subkeys"], xd["v"][t],
                                 xd["alpha"][t], xd["beta"][t], wl.W, wl.R, packed=packed,
                                 bufs=bufs)
    step(MA, bA, 0)
    step(MB, bB, 0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for t in range(1, wl.T):
                step(MB, bB, t)
    torch.cuda.synchronize()
    for r in range(3):
        for t in range(1, wl.T):
            step(MA, bA, t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(MA, MB), f"replay {r}: tables differ"
        assert torch.equal(bA["out"], bB["out"]), f"replay {r}: outputs differ"
        for j in range(4):
            assert torch.equal(bA["idx"][j], bB["idx"][j]), f"replay {r}: slot list {j} differs"
