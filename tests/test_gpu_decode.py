"""Decoding: one token per stream per call, many streams at once (run on an MI355X).

A decode step is the same two calls as a sequence (addressing, then the scan)
with T = 1, laid out head-major so that the tokens of one head score together.
Rules:
  * stepping T tokens one call at a time gives the same bits as one call over
    the whole sequence: slot lists, weights, outputs and the final table;
  * streams match the oracle by the rules of the sequence tests: slot sets
    modulo valid near-tie swaps, weights within 1e-5 + 1e-4|ref|, and end to
    end (the oracle's own addressing and scan) table and outputs within
    1e-5 + 1e-4|ref| outside the positions a valid swap taints.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import E2ETally, close, e2e_stream, np_, say

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
    # every stream against the oracle's own addressing and scan, end to end from M0
    tot = E2ETally()
    for b in range(wl.B):
        for h in range(wl.H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            ref = oracle.score_topk(np_(x["q"][sl]), np_(x["k"][sl]),
                                    np_(x["subkeys"][h:h + 1]), wl.W, wl.R)
            M_ref = np.ascontiguousarray(M0_host[b:b + 1, h:h + 1])
            o_ref = oracle.scan(M_ref, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"],
                                np_(x["v"][sl]), np_(x["alpha"][sl]), np_(x["beta"][sl]))
            gl = [np_(idx[j][:, h, b]) for j in range(4)]
            tot.add(e2e_stream(gl, ref, np_(x["k"][b, h]), np_(x["q"][b, h]),
                               np_(x["subkeys"][h:h + 1]), np_(M_dec[h, b]), M_ref[0, 0],
                               np_(outs[:, h, b]), o_ref[0, 0], msg=f"decode ({b},{h})"))
    say(tot.line("decode vs oracle"))
    assert tot.outs_compared >= 0.95 * tot.outs


def test_decode_full_size_sampled(dev):
    """The serving batch at N = 2^20 (32 sequences x 8 heads, 68.7 GB table):
    three steps; 16 streams spread over the batch and the heads checked end to
    end against the oracle from M0 (each needs its 268 MB initial table on the
    host)."""
    wl = synth.WORKLOADS["decode"].with_(T=3)
    say("case: decode full size, 3 steps", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    xd = synth.decode_layout(x)
    M = synth.make_m0(wl, dev, head_major=True)
    picks = tuple((2 * i + i // 8, i % wl.H) for i in range(15)) + ((wl.B - 1, wl.H - 1),)
    M0 = {p: np_(M[p[1], p[0]]) for p in picks}
    packed = sdm().pack_subkeys(x["subkeys"])
    idx, outs = run_decode(wl, xd, M, packed)
    tot = E2ETally()
    for b, h in picks:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.score_topk(np_(x["q"][sl]), np_(x["k"][sl]), np_(x["subkeys"][h:h + 1]),
                                wl.W, wl.R)
        # end to end against the oracle's own addressing and scan
        M_ref = np.ascontiguousarray(M0[(b, h)][None, None])
        o_ref = oracle.scan(M_ref, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"],
                            np_(x["v"][sl]), np_(x["alpha"][sl]), np_(x["beta"][sl]))
        gl = [np_(idx[j][:, h, b]) for j in range(4)]
        tot.add(e2e_stream(gl, ref, np_(x["k"][b, h]), np_(x["q"][b, h]),
                           np_(x["subkeys"][h:h + 1]), np_(M[h, b]), M_ref[0, 0],
                           np_(outs[:, h, b]), o_ref[0, 0], msg=f"decode ({b},{h})"))
    say(tot.line("decode full size"))
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


def test_fused_decode_step_equals_two_calls(dev):
    """sdm_decode_step (one launch) against decode_step (addressing, then the
    scan), step by step on the same inputs: slot lists and weights
    bit-identical (the same addressing), tables bit-identical (the same write
    in the same roundings), outputs within 1e-5 + 1e-4|ref| (the read is
    summed in another order).  10 sequences per head: a ragged last tile."""
    wl = synth.WORKLOADS["decode"].with_(B=10, H=3, T=5, n_sub=256, W=32, R=24)
    say("case: fused decode vs two calls", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    xd = synth.decode_layout(x)
    M_a = synth.make_m0(wl, dev, head_major=True)
    M_b = M_a.clone()
    packed = sdm().pack_subkeys(x["subkeys"])
    ba, bb = {}, {}
    for t in range(wl.T):
        args = (xd["q"][t], xd["k"][t], xd["subkeys"], xd["v"][t], xd["alpha"][t],
                xd["beta"][t], wl.W, wl.R)
        oa = sdm().decode_step(M_a, *args, packed=packed, bufs=ba)
        ob = sdm().decode_step_fused(M_b, *args, packed=packed, bufs=bb)
        torch.cuda.synchronize()
        for j in range(4):
            assert torch.equal(ba["idx"][j], bb["idx"][j]), f"step {t}: slot list {j} differs"
        assert np.all(close(np_(ob), np_(oa))), f"step {t}: outputs differ"
    assert torch.equal(M_a, M_b), "tables differ"
    # without pre-packed tables the binding packs them on every call
    ob2 = sdm().decode_step_fused(M_b.clone(), *args, bufs={})
    torch.cuda.synchronize()
    assert ob2.shape == ob.shape
    # buffers kept for other sizes, or a packed buffer that is too small, are
    # refused before any launch
    with pytest.raises(ValueError):
        sdm().decode_step_fused(M_b, *args[:-2], wl.W + 8, wl.R, packed=packed, bufs=bb)
    with pytest.raises(ValueError):
        sdm().decode_step_fused(M_b, *args, packed=packed[: packed.numel() // 2], bufs=bb)


def test_fused_decode_step_fp32_against_oracle(dev):
    """fp32 inputs are scored in the oracle's order, so every slot equals the
    oracle's; weights, tables and outputs are then within 1e-5 + 1e-4|ref| of
    the oracle's own addressing and scan (the weights' exponentials round
    differently, and the writes use them).  d_v = 16, W = R = 8, a random
    initial table, 6 sequences per head (a ragged second tile), three steps."""
    wl = synth.WORKLOADS["tiny"].with_(B=6, H=2, T=3)
    say("case: fused decode fp32 vs oracle", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    xd = synth.decode_layout(x)
    g = torch.Generator().manual_seed(41)
    M = (torch.randn(wl.H, wl.B, wl.N, wl.d_v, generator=g) * 0.1).to(dev)
    M0 = np_(M).copy()
    bufs = {}
    outs, idx = [], [[], [], [], []]
    for t in range(wl.T):
        o = sdm().decode_step_fused(M, xd["q"][t], xd["k"][t], xd["subkeys"], xd["v"][t],
                                    xd["alpha"][t], xd["beta"][t], wl.W, wl.R, bufs=bufs)
        outs.append(np_(o).copy())
        for j in range(4):
            idx[j].append(np_(bufs["idx"][j][0]).copy())
    torch.cuda.synchronize()
    Mg = np_(M)
    for b in range(wl.B):
        for h in range(wl.H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            ref = oracle.score_topk(np_(x["q"][sl]), np_(x["k"][sl]),
                                    np_(x["subkeys"][h:h + 1]), wl.W, wl.R)
            for j, key in enumerate(("widx", "wwt", "ridx", "rwt")):
                got = np.stack([idx[j][t][h, b] for t in range(wl.T)])
                if key.endswith("idx"):
                    assert np.array_equal(got, ref[key][0, 0]), (b, h, key)
                else:
                    assert np.all(close(got, ref[key][0, 0])), (b, h, key)
            M_ref = np.ascontiguousarray(M0[h, b][None, None])
            o_ref = oracle.scan(M_ref, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"],
                                np_(x["v"][sl]), np_(x["alpha"][sl]), np_(x["beta"][sl]))
            assert np.all(close(Mg[h, b], M_ref[0, 0])), (b, h)
            untouched = np.ones(wl.N, bool)
            untouched[ref["widx"][0, 0].ravel()] = False
            assert np.array_equal(Mg[h, b][untouched], M0[h, b][untouched]), (b, h)
            got = np.stack([outs[t][h, b] for t in range(wl.T)])
            assert np.all(close(got, o_ref[0, 0])), (b, h)
