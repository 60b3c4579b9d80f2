"""GPU parity of the gradient path against the fp64 gradient oracle (run on an MI355X).

Rules:
  * the tape the recorded forward stores is bit-identical to the rows the C
    oracle's scan holds before each token (the tables are bit-identical);
  * after the reverse sweep the table is M0 again, bit for bit;
  * every gradient (dM0, dv, dalpha, dbeta, dwwt, drwt, dq, dk, dsubkeys) is
    within |g - ref| <= 2e-4 * (|ref| + rms(ref)) of the fp64 oracle.  fp32
    roundings along the reverse recurrence compound at most once per token
    that touches a row; at T = 4096 that bounds the relative error by about
    T * 2^-24 = 2.4e-4 and typically sqrt(T) * 2^-24;
  * slot lists and weights fed to both sides come from seeded generators or
    from the oracle's own addressing, never from the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import backward as ob
from gpu_util import ignored_events, np_, say, thread_map, workers

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


def grad_close(g, r, what, rtol=2e-4):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    scale = np.sqrt(np.mean(r * r)) if r.size else 0.0
    bad = np.abs(g - r) > rtol * (np.abs(r) + scale)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"worst |g-r| = {np.abs(g - r).max():.3e}, rms(ref) = {scale:.3e}")


def scan_inputs(B, H, T, n_sub, d_v, W, R, seed, hot=None, v_bf16=False, repeat_reads=False):
    """Random scan inputs and gradients; `repeat_reads` makes tokens read
    slots more than once (positions 1 and 3 repeat position 0, and every
    fifth token reads one slot R times)."""
    g = torch.Generator().manual_seed(seed)
    N = n_sub * n_sub
    span = N if hot is None else hot
    n = B * H * T
    widx = torch.stack([torch.randperm(span, generator=g)[:W] for _ in range(n)])
    ridx = torch.stack([torch.randperm(span, generator=g)[:R] for _ in range(n)])
    if repeat_reads:
        ridx[:, 1] = ridx[:, 0]
        ridx[:, 3] = ridx[:, 0]
        ridx[::5] = ridx[::5, 2:3]
    d = dict(widx=widx.view(B, H, T, W).int(),
             wwt=torch.softmax(torch.randn(n, W, generator=g), -1).view(B, H, T, W),
             ridx=ridx.view(B, H, T, R).int(),
             rwt=torch.softmax(torch.randn(n, R, generator=g), -1).view(B, H, T, R),
             v=torch.randn(B, H, T, d_v, generator=g),
             alpha=torch.sigmoid(torch.randn(B, H, T, generator=g) + 3),
             beta=torch.sigmoid(torch.randn(B, H, T, generator=g)),
             M0=torch.randn(B, H, N, d_v, generator=g) * 0.3,
             dout=torch.randn(B, H, T, d_v, generator=g),
             dMT=torch.randn(B, H, N, d_v, generator=g))
    if v_bf16:
        d["v"] = d["v"].to(torch.bfloat16)
    return d


def run_gpu_scan_grads(d, dev):
    x = {k: t.contiguous().to(dev) for k, t in d.items()}
    B, H, T, W = x["widx"].shape
    d_v = x["M0"].shape[-1]
    M = x["M0"].clone()
    tape = torch.empty((B, H, T, W, d_v), device=dev)
    out = sdm().scan(M, x["widx"], x["wwt"], x["ridx"], x["rwt"], x["v"], x["alpha"], x["beta"],
                     tape=tape)
    dM = x["dMT"].clone()
    g = sdm().scan_backward(M, dM, x["widx"], x["wwt"], x["ridx"], x["rwt"], x["v"], x["alpha"],
                            x["beta"], tape, x["dout"])
    torch.cuda.synchronize()
    return x, M, dM, g, tape, out


def oracle_tape(d, b, h):
    """Rows before each token's write, from the fp32 C oracle stepped token by token."""
    M = np_(d["M0"][b:b + 1, h:h + 1]).copy()
    T, W = d["widx"].shape[2], d["widx"].shape[3]
    rows = np.empty((T, W, M.shape[-1]), np.float32)
    for t in range(T):
        sl = (slice(b, b + 1), slice(h, h + 1), slice(t, t + 1))
        rows[t] = M[0, 0][np_(d["widx"][b, h, t])]
        oracle.scan(M, np_(d["widx"][sl]), np_(d["wwt"][sl]), np_(d["ridx"][sl]),
                    np_(d["rwt"][sl]), np_(d["v"][sl]), np_(d["alpha"][sl]), np_(d["beta"][sl]))
    return rows


def check_stream(d, g, dM, b, h, label):
    sl = (b, h)
    ref = ob.scan_backward_stream(np_(d["M0"][sl]), np_(d["widx"][sl]), np_(d["wwt"][sl]),
                                  np_(d["ridx"][sl]), np_(d["rwt"][sl]), np_(d["v"][sl]),
                                  np_(d["alpha"][sl]), np_(d["beta"][sl]), np_(d["dout"][sl]),
                                  np_(d["dMT"][sl]))
    grad_close(np_(dM[sl]), ref["dM0"], f"{label} dM0")
    for key in ("dv", "dalpha", "dbeta", "dwwt", "drwt"):
        grad_close(np_(g[key][sl]), ref[key], f"{label} {key}")


@pytest.mark.parametrize("label,args", [
    ("tiny d_v=16", dict(B=1, H=1, T=40, n_sub=16, d_v=16, W=8, R=8, seed=21)),
    ("partitions d_v=64", dict(B=2, H=2, T=97, n_sub=64, d_v=64, W=32, R=32, seed=22)),
    ("bf16 v d_v=128", dict(B=1, H=3, T=45, n_sub=32, d_v=128, W=16, R=24, seed=23,
                            v_bf16=True)),
    ("hot slots, deep chains", dict(B=2, H=1, T=120, n_sub=32, d_v=32, W=16, R=16, seed=24,
                                    hot=40)),
    ("hot W=1", dict(B=1, H=1, T=150, n_sub=8, d_v=32, W=1, R=3, seed=25, hot=4)),
    ("serial path", dict(B=2, H=2, T=30, n_sub=32, d_v=256, W=128, R=128, seed=26, hot=300)),
    ("T=1", dict(B=1, H=1, T=1, n_sub=8, d_v=32, W=4, R=4, seed=27)),
    ("256 B slice forward, 16 streams", dict(B=4, H=4, T=24, n_sub=32, d_v=128, W=128, R=128,
                                           seed=32, hot=600)),
    ("repeated read slots", dict(B=1, H=2, T=33, n_sub=16, d_v=32, W=8, R=8, seed=28, hot=40,
                                 repeat_reads=True)),
    ("repeated read slots, partitions", dict(B=2, H=2, T=41, n_sub=64, d_v=64, W=32, R=32,
                                             seed=29, repeat_reads=True)),
])
def test_scan_backward_vs_oracle(dev, label, args):
    say(f"case: scan backward {label}", args)
    d = scan_inputs(**args)
    x, M, dM, g, tape, out = run_gpu_scan_grads(d, dev)
    assert torch.equal(M, x["M0"]), "table not restored to M0"
    B, H = args["B"], args["H"]
    for b, h in {(0, 0), (B - 1, H - 1)}:
        assert np.array_equal(np_(tape[b, h]), oracle_tape(d, b, h)), "tape differs"
        check_stream(d, g, dM, b, h, label)


def test_scan_backward_ignores_slots_outside_the_table(dev):
    """Events whose slot lies outside [0, N) are skipped by the recorded
    forward and by the reverse sweep, and their weight gradients are 0.
    Oracle: those writes go to sink rows [200, 256) and those reads get
    weight 0, with dL/dM_T zero on the sink rows, so every gradient is the
    same; only the oracle's drwt of the weight-0 reads (row . dO) is not
    compared (the GPU's is 0)."""
    N, sink0 = 256, 200
    d = scan_inputs(B=2, H=2, T=57, n_sub=16, d_v=64, W=16, R=16, seed=30, hot=sink0)
    d["dMT"][:, :, sink0:] = 0.0
    gpu_l, ref_l, masks = ignored_events(d, N, sink0, seed=31)
    assert masks["widx"].any() and masks["ridx"].any()
    dg = dict(d, **{k: gpu_l[k] for k in ("widx", "ridx")})
    x, M, dM, g, tape, out = run_gpu_scan_grads(dg, dev)
    assert torch.equal(M, x["M0"]), "table not restored to M0"
    dr = dict(d, **ref_l)
    for b, h in ((0, 0), (1, 1)):
        sl = (b, h)
        ref = ob.scan_backward_stream(np_(dr["M0"][sl]), np_(dr["widx"][sl]), np_(dr["wwt"][sl]),
                                      np_(dr["ridx"][sl]), np_(dr["rwt"][sl]), np_(dr["v"][sl]),
                                      np_(dr["alpha"][sl]), np_(dr["beta"][sl]),
                                      np_(dr["dout"][sl]), np_(dr["dMT"][sl]))
        label = f"ignored slots stream {b},{h}"
        grad_close(np_(dM[sl]), ref["dM0"], f"{label} dM0")
        for key in ("dv", "dalpha", "dbeta", "dwwt"):
            grad_close(np_(g[key][sl]), ref[key], f"{label} {key}")
        mr = masks["ridx"][sl].numpy()
        assert np.all(np_(g["drwt"][sl])[mr] == 0.0), f"{label}: ignored reads' drwt not 0"
        assert np.all(np_(g["dwwt"][sl])[masks["widx"][sl].numpy()] == 0.0)
        grad_close(np_(g["drwt"][sl])[~mr], ref["drwt"][~mr], f"{label} drwt")


def test_score_backward_vs_oracle(dev):
    """Addressing adjoint on the oracle's own selections, bf16 and fp32 inputs."""
    for bf16, (B, H, T, d_k, n_sub, W, R) in ((True, (2, 3, 37, 128, 64, 32, 24)),
                                               (False, (1, 2, 20, 32, 32, 16, 8)),
                                               (True, (1, 1, 9, 192, 128, 128, 100)),
                                               # the largest shape the call takes
                                               (True, (1, 1, 6, 512, 1024, 128, 128))):
        say(f"case: score backward bf16={bf16} B={B} H={H} T={T} d_k={d_k} n_sub={n_sub}")
        gen = torch.Generator().manual_seed(31 + T)
        q = torch.randn(B, H, T, d_k, generator=gen)
        k = torch.randn(B, H, T, d_k, generator=gen)
        C = torch.randn(H, 2, n_sub, d_k // 2, generator=gen) * (d_k // 2) ** -0.5
        if bf16:
            q, k, C = q.bfloat16(), k.bfloat16(), C.bfloat16()
        ref_fw = oracle.score_topk(np_(q), np_(k), np_(C), W, R)
        dw = torch.randn(B, H, T, W, generator=gen)
        dr = torch.randn(B, H, T, R, generator=gen)
        ref = ob.score_backward(np_(q), np_(k), np_(C), ref_fw["widx"], ref_fw["ridx"], np_(dw),
                                np_(dr))
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        dq, dk, dC = sdm().score_topk_backward(q.to(dev), k.to(dev), C.to(dev), t(ref_fw["widx"]),
                                               t(ref_fw["wwt"]), t(ref_fw["ridx"]),
                                               t(ref_fw["rwt"]), dw.to(dev), dr.to(dev))
        torch.cuda.synchronize()
        grad_close(np_(dq), ref["dq"], "dq")
        grad_close(np_(dk), ref["dk"], "dk")
        grad_close(np_(dC), ref["dsubkeys"], "dsubkeys")


def test_score_backward_is_deterministic(dev):
    """Every output of the addressing adjoint, the sub-key gradient included,
    is the same bit for bit on repeated calls (each sum has a fixed order),
    and a second call adds the same gradient again."""
    wl = synth.WORKLOADS["mid"].with_(B=2, H=2, T=300)
    say("case: score backward determinism", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    g = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    gen = torch.Generator(device=dev).manual_seed(5)
    dw = torch.randn(g[1].shape, generator=gen, device=dev)
    dr = torch.randn(g[3].shape, generator=gen, device=dev)
    runs = [sdm().score_topk_backward(x["q"], x["k"], x["subkeys"], *g, dw, dr) for _ in range(3)]
    acc = torch.zeros(x["subkeys"].shape, device=dev)
    for _ in range(2):
        sdm().score_topk_backward(x["q"], x["k"], x["subkeys"], *g, dw, dr, dsubkeys=acc)
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert all(torch.equal(a, b) for a, b in zip(runs[0], r))
    assert torch.equal(acc, runs[0][2] + runs[0][2])


def test_training_step_large_sampled(dev):
    """The large workload's forward with tape and both backward calls at full
    size (N = 2^20, 64 streams).  Every stream of the last head, and stream
    (0, 0), run on the oracle's own addressing (their slots and weights are
    overwritten with the oracle's before the scan) and are checked against the
    gradient oracle: the scan's gradients and dq', dk' per stream, and the
    last head's sub-key gradient, which sums over all of that head's streams."""
    wl = synth.WORKLOADS["large"]
    say("case: large training step, sampled", wl)
    x = synth.make_inputs(wl, device=dev)
    B, H, T = wl.B, wl.H, wl.T
    g = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    widx, wwt, ridx, rwt = (t.clone() for t in g)
    hl = H - 1
    picks = [(b, hl) for b in range(B)] + [(0, 0)]

    def addr(p):
        b, h = p
        sl = (slice(b, b + 1), slice(h, h + 1))
        return oracle.score_topk(np_(x["q"][sl]), np_(x["k"][sl]), np_(x["subkeys"][h:h + 1]),
                                 wl.W, wl.R)

    refs = dict(zip(picks, thread_map(addr, picks)))
    for (b, h), r in refs.items():
        for dst, key in ((widx, "widx"), (wwt, "wwt"), (ridx, "ridx"), (rwt, "rwt")):
            dst[b, h] = torch.from_numpy(r[key][0, 0]).to(dev)
    gen = torch.Generator(device=dev).manual_seed(77)
    dout = torch.randn((B, H, T, wl.d_v), generator=gen, device=dev)
    M0 = {p: np_(x["m0"][p]) for p in picks}
    M = x["m0"]
    tape = torch.empty((B, H, T, wl.W, wl.d_v), device=dev)
    sdm().scan(M, widx, wwt, ridx, rwt, x["v"], x["alpha"], x["beta"], tape=tape)
    dM = torch.zeros_like(M)
    gs = sdm().scan_backward(M, dM, widx, wwt, ridx, rwt, x["v"], x["alpha"], x["beta"], tape,
                             dout)
    dq, dk, dC = sdm().score_topk_backward(x["q"], x["k"], x["subkeys"], widx, wwt, ridx, rwt,
                                           gs["dwwt"], gs["drwt"])
    torch.cuda.synchronize()
    del tape
    assert torch.isfinite(dC).all()
    for p in picks:
        assert np.array_equal(np_(M[p]), M0[p]), f"table of stream {p} not restored to M0"
    host = {p: {n: np_(x[n][p]) for n in ("v", "alpha", "beta")} | {"dout": np_(dout[p])}
            for p in picks}

    def rev(p):
        r = refs[p]
        return ob.scan_backward_stream(M0[p], r["widx"][0, 0], r["wwt"][0, 0], r["ridx"][0, 0],
                                       r["rwt"][0, 0], host[p]["v"], host[p]["alpha"],
                                       host[p]["beta"], host[p]["dout"])

    grads = dict(zip(picks, thread_map(rev, picks, n=min(workers(), 8))))
    for p in picks:
        ref = grads[p]
        grad_close(np_(dM[p]), ref["dM0"], f"large dM0 {p}")
        for key in ("dv", "dalpha", "dbeta", "dwwt", "drwt"):
            grad_close(np_(gs[key][p]), ref[key], f"large {key} {p}")
    # the addressing adjoint: dq', dk' of stream (0, 0); dq', dk' of every
    # stream of the last head and that head's sub-key gradient
    for hh, bs in ((0, [0]), (hl, list(range(B)))):
        sel = (slice(bs[0], bs[-1] + 1), slice(hh, hh + 1))
        stack = lambda key: np.stack([refs[(b, hh)][key][0] for b in bs])
        dstack = lambda key: np.stack([grads[(b, hh)][key][None] for b in bs])
        sref = ob.score_backward(np_(x["q"][sel]), np_(x["k"][sel]), np_(x["subkeys"][hh:hh + 1]),
                                 stack("widx"), stack("ridx"), dstack("dwwt"), dstack("drwt"))
        grad_close(np_(dq[sel]), sref["dq"], f"large dq, head {hh}")
        grad_close(np_(dk[sel]), sref["dk"], f"large dk, head {hh}")
        if hh == hl:
            grad_close(np_(dC[hl]), sref["dsubkeys"][0], f"large dsubkeys, head {hl}")
