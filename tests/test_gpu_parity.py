"""GPU parity of the HIP path against the CPU oracle (run on an MI355X).

Rules (fixed before any kernel was written):
  * slot sets per token equal the oracle's, except where the oracle's relative
    gap between the k-th and (k+1)-th candidate sum is below 1e-5 (counted);
  * weights, outputs and tables within 1e-5 absolute + 1e-4 relative;
  * the GPU scan fed the oracle's own indices and weights gives the oracle's
    memory table bit for bit (both evaluate the write as the same sequence of
    fp32 roundings) and outputs within tolerance (read sums are added in a
    different order);
  * end to end (GPU addressing + GPU scan against the oracle's addressing +
    the oracle's scan) tables and outputs are within tolerance, except in
    streams holding a token that the gap rule flags;
  * nothing the GPU computes is ever an input to the oracle.
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


def run_gpu(wl, x, M=None):
    M = x["m0"].clone() if M is None else M
    widx, wwt, ridx, rwt = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    out = sdm().scan(M, widx, wwt, ridx, rwt, x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    return M, out, (widx, wwt, ridx, rwt)


def oracle_stream(x, wl, b, h, m0_host):
    """The oracle's own addressing and scan of stream (b,h) from m0_host;
    returns (addressing dict, M, out)."""
    sl = (slice(b, b + 1), slice(h, h + 1))
    ref = oracle.score_topk(np_(x["q"][sl]), np_(x["k"][sl]), np_(x["subkeys"][h:h + 1]),
                            wl.W, wl.R)
    M = np.ascontiguousarray(m0_host)
    out = oracle.scan(M, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"], np_(x["v"][sl]),
                      np_(x["alpha"][sl]), np_(x["beta"][sl]))
    return ref, M, out


def inject(g, b, h, ref, dev):
    """Replace stream (b,h)'s slot lists and weights by the oracle's."""
    for j, key in enumerate(("widx", "wwt", "ridx", "rwt")):
        g[j][b, h] = torch.from_numpy(ref[key][0, 0]).to(dev)


def flagged_stream(g, ref, b, h, N):
    """Whether any token of stream (b,h) has a slot set that differs from the
    oracle's within the gap rule (one flipped slot changes what follows)."""
    flags = 0
    for j, (ri, rw, gp) in enumerate(((ref["widx"], ref["wwt"], ref["wgap"]),
                                       (ref["ridx"], ref["rwt"], ref["rgap"]))):
        n, f, bad = compare_topk(np_(g[2 * j][b, h])[None, None], np_(g[2 * j + 1][b, h])[None, None],
                                 ri, rw, gp, N)
        assert bad == 0
        flags += f
    return flags > 0


# ------------------------------------------------------------------ tiny ---

def test_tiny_end_to_end(dev):
    wl = synth.WORKLOADS["tiny"]
    say("case: tiny end to end", wl)
    x = synth.make_inputs(wl, device=dev)
    M, out, g = run_gpu(wl, x)
    h = {k: np_(v) for k, v in x.items()}
    ref = oracle.score_topk(h["q"], h["k"], h["subkeys"], wl.W, wl.R)
    for gi, gw, ri, rw, gp in ((g[0], g[1], ref["widx"], ref["wwt"], ref["wgap"]),
                               (g[2], g[3], ref["ridx"], ref["rwt"], ref["rgap"])):
        n, flagged, bad = compare_topk(np_(gi), np_(gw), ri, rw, gp, wl.N)
        say(f"tiny topk: {n} tokens, {flagged} flagged, {bad} mismatched")
        assert bad == 0
    # fp32 scores are computed in the oracle's order: indices match exactly
    assert np.array_equal(np_(g[0]), ref["widx"]) and np.array_equal(np_(g[2]), ref["ridx"])
    # the GPU scan fed the oracle's own addressing: bit-identical table
    g2 = [t.clone() for t in g]
    inject(g2, 0, 0, ref, dev)
    M_inj = x["m0"].clone()
    out_inj = sdm().scan(M_inj, *g2, x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    M_ref = h["m0"].copy()
    out_ref = oracle.scan(M_ref, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"], h["v"],
                          h["alpha"], h["beta"])
    assert np.array_equal(np_(M_inj), M_ref)
    assert np.all(close(np_(out_inj), out_ref))
    # end to end against the oracle's own addressing
    M2 = h["m0"].copy()
    out2 = oracle.scan(M2, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"], h["v"], h["alpha"],
                       h["beta"])
    assert np.all(close(np_(M), M2)) and np.all(close(np_(out), out2))


# ------------------------------------------------------------ addressing ---

def test_score_topk_integer_ties(dev):
    """Small-integer bf16 inputs: every score is exact on both sides, with many
    exact ties, so indices must match the oracle exactly (lowest index wins)."""
    say("case: integer ties")
    g = torch.Generator().manual_seed(7)
    for (B, H, T, d_k, n_sub, W, R) in ((1, 2, 40, 32, 64, 16, 12), (2, 1, 33, 64, 32, 32, 5),
                                        (1, 1, 17, 32, 128, 128, 128),
                                        # sub-key halves of 80 and 96: K padded to 128
                                        (2, 1, 19, 160, 32, 32, 20), (1, 2, 29, 192, 128, 128, 97),
                                        # largest shape the call takes: halves of 256, 1024
                                        # sub-keys, W = R = 128
                                        (1, 1, 9, 512, 1024, 128, 128),
                                        # smallest table, every sub-key in the stage-1 lists
                                        (1, 2, 11, 32, 16, 16, 16)):
        q = torch.randint(-2, 3, (B, H, T, d_k), generator=g).float()
        k = torch.randint(-2, 3, (B, H, T, d_k), generator=g).float()
        C = torch.randint(-1, 2, (H, 2, n_sub, d_k // 2), generator=g).float()
        qb, kb, Cb = (t.to(torch.bfloat16).to(dev) for t in (q, k, C))
        say(f"  B={B} H={H} T={T} d_k={d_k} n_sub={n_sub} W={W} R={R}")
        widx, wwt, ridx, rwt = sdm().score_topk(qb, kb, Cb, W, R)
        torch.cuda.synchronize()
        ref = oracle.score_topk(np_(qb), np_(kb), np_(Cb), W, R)
        assert np.array_equal(np_(widx), ref["widx"])
        assert np.array_equal(np_(ridx), ref["ridx"])
        assert np.all(close(np_(wwt), ref["wwt"])) and np.all(close(np_(rwt), ref["rwt"]))


def test_score_topk_ragged_and_fp32(dev):
    """T not a multiple of the token tile, fp32 inputs, W != R."""
    say("case: ragged fp32 addressing")
    wl = synth.WORKLOADS["tiny"].with_(B=2, H=3, T=37, W=5, R=11)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    widx, wwt, ridx, rwt = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    torch.cuda.synchronize()
    ref = oracle.score_topk(np_(x["q"]), np_(x["k"]), np_(x["subkeys"]), wl.W, wl.R)
    assert np.array_equal(np_(widx), ref["widx"]) and np.array_equal(np_(ridx), ref["ridx"])
    assert np.all(close(np_(wwt), ref["wwt"])) and np.all(close(np_(rwt), ref["rwt"]))


def test_score_topk_mid_all_tokens(dev):
    wl = synth.WORKLOADS["mid"]
    say("case: mid addressing, all tokens", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    g = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    torch.cuda.synchronize()
    ref = oracle.score_topk(np_(x["q"]), np_(x["k"]), np_(x["subkeys"]), wl.W, wl.R)
    tot = [0, 0, 0]
    for gi, gw, ri, rw, gp in ((g[0], g[1], ref["widx"], ref["wwt"], ref["wgap"]),
                               (g[2], g[3], ref["ridx"], ref["rwt"], ref["rgap"])):
        r = compare_topk(np_(gi), np_(gw), ri, rw, gp, wl.N)
        tot = [a + b for a, b in zip(tot, r)]
    say(f"mid topk: {tot[0]} token-sets, {tot[1]} flagged (gap < 1e-5), {tot[2]} mismatched")
    assert tot[2] == 0


@pytest.mark.parametrize("name,per_stream", [("large", 8), ("long", 24)])
def test_score_topk_full_size_sampled(dev, name, per_stream):
    """Full-size addressing on the GPU; the oracle recomputes a seeded sample
    of tokens of every stream (tokens are independent)."""
    wl = synth.WORKLOADS[name]
    say(f"case: {name} addressing, full size, sampled", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    g = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    g2 = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    torch.cuda.synchronize()
    # a second call gives the same bits, and every slot is a row of the table
    for a, b2 in zip(g, g2):
        assert torch.equal(a, b2)
    for ix in (g[0], g[2]):
        assert int(ix.min()) >= 0 and int(ix.max()) < wl.N
    rng = np.random.default_rng(wl.seed)
    tot = [0, 0, 0]
    for b in range(wl.B):
        for h in range(wl.H):
            ts = np.sort(rng.choice(wl.T, per_stream, replace=False))
            ts[0], ts[-1] = 0, wl.T - 1
            tt = torch.from_numpy(ts).to(dev)
            q = np_(x["q"][b:b + 1, h:h + 1].index_select(2, tt))
            k = np_(x["k"][b:b + 1, h:h + 1].index_select(2, tt))
            ref = oracle.score_topk(q, k, np_(x["subkeys"][h:h + 1]), wl.W, wl.R)
            for j, (ri, rw, gp) in enumerate(((ref["widx"], ref["wwt"], ref["wgap"]),
                                               (ref["ridx"], ref["rwt"], ref["rgap"]))):
                gi = np_(g[2 * j][b, h].index_select(0, tt))
                gw = np_(g[2 * j + 1][b, h].index_select(0, tt))
                r = compare_topk(gi, gw, ri, rw, gp, wl.N)
                tot = [a + c for a, c in zip(tot, r)]
    say(f"{name} topk sample: {tot[0]} token-sets, {tot[1]} flagged, {tot[2]} mismatched")
    assert tot[2] == 0


# ------------------------------------------------------------------ scan ---

def scan_case(dev, B, H, T, n_sub, d_v, W, R, seed, v_bf16=False, hot=None):
    """Random scan inputs; `hot` restricts slots to the first `hot` rows to
    force many in-block collisions."""
    g = torch.Generator().manual_seed(seed)
    N = n_sub * n_sub
    span = N if hot is None else hot
    widx = torch.stack([torch.randperm(span, generator=g)[:W] for _ in range(B * H * T)])
    ridx = torch.stack([torch.randperm(span, generator=g)[:R] for _ in range(B * H * T)])
    wwt = torch.softmax(torch.randn(B * H * T, W, generator=g), -1)
    rwt = torch.softmax(torch.randn(B * H * T, R, generator=g), -1)
    v = torch.randn(B, H, T, d_v, generator=g)
    if v_bf16:
        v = v.to(torch.bfloat16)
    alpha = torch.sigmoid(torch.randn(B, H, T, generator=g) + 3)
    beta = torch.sigmoid(torch.randn(B, H, T, generator=g))
    M0 = torch.randn(B, H, N, d_v, generator=g) * 0.1
    d = dict(widx=widx.view(B, H, T, W).int(), wwt=wwt.view(B, H, T, W),
             ridx=ridx.view(B, H, T, R).int(), rwt=rwt.view(B, H, T, R), v=v, alpha=alpha,
             beta=beta, M0=M0)
    return {k: t.contiguous().to(dev) for k, t in d.items()}


def check_scan(d, label):
    say(f"case: scan {label}")
    M = d["M0"].clone()
    out = sdm().scan(M, d["widx"], d["wwt"], d["ridx"], d["rwt"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    M_ref = np_(d["M0"]).copy()
    out_ref = oracle.scan(M_ref, np_(d["widx"]), np_(d["wwt"]), np_(d["ridx"]), np_(d["rwt"]),
                          np_(d["v"]), np_(d["alpha"]), np_(d["beta"]))
    Mg = np_(M)
    diff = np.count_nonzero(Mg.view(np.uint32) != M_ref.view(np.uint32))
    assert diff == 0, f"{label}: {diff} table entries differ"
    assert np.all(close(np_(out), out_ref)), f"{label}: outputs differ"
    return M, out


# Small tables (n_sub <= 32) and large ones with the same events: "hot"
# confines the slots to [0, hot), so a large table can still have long
# dependence chains inside a block of tokens, and W = R = 128 with hot slots
# drives the overflow path.
@pytest.mark.parametrize("label,args", [
    ("small d_v=16", dict(B=1, H=2, T=50, n_sub=16, d_v=16, W=8, R=8, seed=1)),
    ("d_v=64 partitions", dict(B=2, H=2, T=129, n_sub=64, d_v=64, W=32, R=32, seed=2)),
    ("bf16 v, ragged T", dict(B=1, H=3, T=77, n_sub=32, d_v=32, W=16, R=24, seed=3,
                                       v_bf16=True)),
    ("hot slots, deep chains", dict(B=2, H=1, T=200, n_sub=64, d_v=32, W=16, R=16, seed=4,
                                    hot=48)),
    ("small table, hot slots", dict(B=2, H=1, T=200, n_sub=32, d_v=32, W=16, R=16, seed=4,
                                hot=48)),
    ("hot slots W=1", dict(B=1, H=1, T=300, n_sub=64, d_v=32, W=1, R=3, seed=5, hot=4)),
    ("small table, W=1", dict(B=1, H=1, T=300, n_sub=8, d_v=32, W=1, R=3, seed=5, hot=4)),
    ("overflow path", dict(B=4, H=4, T=40, n_sub=64, d_v=512, W=128, R=128, seed=6,
                           hot=300)),
    ("small table, d_v=512, W=R=128", dict(B=2, H=2, T=40, n_sub=32, d_v=512, W=128, R=128,
                                       seed=6, hot=300)),
    ("W=256, R=200", dict(B=1, H=2, T=20, n_sub=32, d_v=32, W=256, R=200, seed=8)),
    ("T=1", dict(B=1, H=1, T=1, n_sub=64, d_v=32, W=4, R=4, seed=7)),
    ("small table, T=1", dict(B=1, H=1, T=1, n_sub=8, d_v=32, W=4, R=4, seed=7)),
])
def test_scan_vs_oracle(dev, label, args):
    check_scan(scan_case(dev, **args), label)


def test_table_size_does_not_change_results(dev):
    """The same events on a 1024-slot table and on a 4096-slot table whose
    extra rows nothing touches (one slot partition at 160 streams either way):
    the touched rows and the outputs are identical bit for bit, and the extra
    rows keep their values."""
    say("case: scan on a small and a large table")
    small = scan_case(dev, B=10, H=16, T=40, n_sub=32, d_v=32, W=16, R=16, seed=12, hot=900)
    big = dict(small)
    M0b = torch.zeros((10, 16, 64 * 64, 32), device=dev)
    M0b[:, :, :1024] = small["M0"]
    big["M0"] = M0b
    Ms, Mb = small["M0"].clone(), big["M0"].clone()
    args = lambda d: (d["widx"], d["wwt"], d["ridx"], d["rwt"], d["v"], d["alpha"], d["beta"])
    out_s = sdm().scan(Ms, *args(small))
    out_b = sdm().scan(Mb, *args(big))
    torch.cuda.synchronize()
    assert torch.equal(Ms, Mb[:, :, :1024]) and torch.equal(out_s, out_b)
    assert torch.equal(Mb[:, :, 1024:], M0b[:, :, 1024:])


def test_scan_empty_sequence(dev):
    d = scan_case(dev, B=1, H=1, T=1, n_sub=8, d_v=32, W=4, R=4, seed=8)
    d = {k: (v[:, :, :0].contiguous() if k != "M0" else v) for k, v in d.items()}
    M = d["M0"].clone()
    out = sdm().scan(M, d["widx"], d["wwt"], d["ridx"], d["rwt"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    assert out.shape[2] == 0 and torch.equal(M, d["M0"])


def test_scan_resume_and_determinism(dev):
    say("case: scan chunked resume + determinism")
    d = scan_case(dev, B=2, H=2, T=96, n_sub=32, d_v=64, W=32, R=32, seed=9, hot=200)
    M1 = d["M0"].clone()
    out1 = sdm().scan(M1, d["widx"], d["wwt"], d["ridx"], d["rwt"], d["v"], d["alpha"],
                      d["beta"])
    M2 = d["M0"].clone()
    outs = []
    for lo, hi in ((0, 37), (37, 96)):
        p = {k: (v[:, :, lo:hi].contiguous() if k != "M0" else v) for k, v in d.items()}
        outs.append(sdm().scan(M2, p["widx"], p["wwt"], p["ridx"], p["rwt"], p["v"],
                               p["alpha"], p["beta"]))
    M3 = d["M0"].clone()
    out3 = sdm().scan(M3, d["widx"], d["wwt"], d["ridx"], d["rwt"], d["v"], d["alpha"],
                      d["beta"])
    torch.cuda.synchronize()
    assert torch.equal(M1, M2) and torch.equal(out1, torch.cat(outs, 2))
    assert torch.equal(M1, M3) and torch.equal(out1, out3)


def test_mid_end_to_end(dev):
    """All 16 streams: the GPU's addressing + scan against the oracle's, end to
    end (streams with a token flagged by the gap rule are counted, not
    compared); then the GPU scan fed the oracle's addressing gives the
    oracle's table bit for bit."""
    wl = synth.WORKLOADS["mid"]
    say("case: mid end to end", wl)
    x = synth.make_inputs(wl, device=dev)
    m0 = np_(x["m0"])
    M, out, g = run_gpu(wl, x, M=x["m0"].clone())
    Mg, og = np_(M), np_(out)
    g2 = [t.clone() for t in g]
    refs, skipped = {}, 0
    for b in range(wl.B):
        for h in range(wl.H):
            ref, M_ref, out_ref = oracle_stream(x, wl, b, h, m0[b:b + 1, h:h + 1].copy())
            refs[(b, h)] = (M_ref, out_ref)
            inject(g2, b, h, ref, dev)
            if flagged_stream(g, ref, b, h, wl.N):
                skipped += 1
                continue
            assert np.all(close(Mg[b:b + 1, h:h + 1], M_ref)), (b, h)
            assert np.all(close(og[b:b + 1, h:h + 1], out_ref)), (b, h)
    say(f"mid end to end: {skipped} of {wl.streams} streams hold a flagged token")
    M2 = x["m0"].clone()
    out2 = sdm().scan(M2, *g2, x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    for (b, h), (M_ref, out_ref) in refs.items():
        assert np.array_equal(np_(M2[b:b + 1, h:h + 1]), M_ref), (b, h)
        assert np.all(close(np_(out2[b:b + 1, h:h + 1]), out_ref)), (b, h)


@pytest.mark.parametrize("name,streams", [("large", ((0, 0), (7, 7), (3, 5))),
                                          ("long", ((0, 0), (0, 15)))])
def test_scan_full_size_sampled(dev, name, streams):
    """Full-size scan (N = 2^20) on the GPU in the benchmark's launch
    configuration.  Sampled streams run on the oracle's own addressing (their
    lists are replaced by the oracle's before the scan) and must give the
    oracle's table bit for bit; the other streams keep the GPU's lists."""
    wl = synth.WORKLOADS[name]
    say(f"case: {name} scan, full size", wl)
    x = synth.make_inputs(wl, device=dev)
    g = [t.clone() for t in sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)]
    refs = {}
    for (b, h) in streams:
        say(f"  oracle of stream ({b},{h})")
        ref, M_ref, out_ref = oracle_stream(x, wl, b, h, np_(x["m0"][b, h])[None, None].copy())
        inject(g, b, h, ref, dev)
        refs[(b, h)] = (M_ref, out_ref)
    M = x["m0"]  # in place: the table is large
    out = sdm().scan(M, *g, x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    for (b, h), (M_ref, out_ref) in refs.items():
        assert np.array_equal(np_(M[b, h])[None, None], M_ref), (b, h)
        assert np.all(close(np_(out[b, h])[None, None], out_ref)), (b, h)


# ------------------------------------------------------------------- gdn ---

def test_gdn_small(dev):
    say("case: gdn small")
    wl = synth.WORKLOADS["gdn"].with_(B=2, H=2, T=70)
    x = synth.make_inputs(wl, device=dev)
    S0 = torch.randn(wl.B, wl.H, wl.d_v, wl.d_k, device=dev) * 0.1
    S = S0.clone()
    out = sdm().gdn_scan(S, x["k"], x["q"], x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    S_ref = np_(S0).copy()
    out_ref = oracle.gdn_scan(S_ref, np_(x["k"]), np_(x["q"]), np_(x["v"]), np_(x["alpha"]),
                              np_(x["beta"]))
    assert np.all(close(np_(out), out_ref)) and np.all(close(np_(S), S_ref))


def test_gdn_full_size_sampled(dev):
    wl = synth.WORKLOADS["gdn"]
    say("case: gdn full size", wl)
    x = synth.make_inputs(wl, device=dev)
    S = x["s0"].clone()
    out = sdm().gdn_scan(S, x["k"], x["q"], x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (15, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        S_ref = np.zeros((1, 1, wl.d_v, wl.d_k), np.float32)
        out_ref = oracle.gdn_scan(S_ref, np_(x["k"][sl]), np_(x["q"][sl]), np_(x["v"][sl]),
                                  np_(x["alpha"][sl]), np_(x["beta"][sl]))
        assert np.all(close(np_(out[sl]), out_ref)), (b, h)
        assert np.all(close(np_(S[sl]), S_ref)), (b, h)
