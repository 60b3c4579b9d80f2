"""Pins of the gradient oracle (oracle/backward.py) -- CPU only.

Each pin ties the hand-written adjoints to something other than themselves:
  * autograd of the forward written out in torch ops (an independent
    derivation), on streams whose slots collide across tokens and between a
    token's reads and writes;
  * central finite differences of the forward, along random directions;
  * the fp64 forward itself against the fp32 C oracle (so the gradients are
    of the function the rest of the suite checks);
  * closed forms worked by hand: one token with one slot; alpha = 1, beta = 0
    (the table is then only read); a weight gradient constant over the slots
    (softmax is shift-invariant, so nothing flows into the scores).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob


def stream_case(seed, T=12, n_sub=8, d_k=16, d_v=8, W=4, R=3, hot=None):
    """One stream of random inputs; slots drawn from the first `hot` rows to
    force collisions (writes of different tokens, and reads of written slots)."""
    rng = np.random.default_rng(seed)
    N = n_sub * n_sub
    span = N if hot is None else hot
    widx = np.stack([rng.choice(span, W, replace=False) for _ in range(T)])
    ridx = np.stack([rng.choice(span, R, replace=False) for _ in range(T)])
    return dict(q=rng.normal(size=(T, d_k)), k=rng.normal(size=(T, d_k)),
                C=rng.normal(size=(2, n_sub, d_k // 2)) * (d_k // 2) ** -0.5,
                M0=rng.normal(size=(N, d_v)) * 0.3, widx=widx, ridx=ridx,
                v=rng.normal(size=(T, d_v)), alpha=1 / (1 + np.exp(-rng.normal(3, 1, T))),
                beta=1 / (1 + np.exp(-rng.normal(0, 1, T))), dout=rng.normal(size=(T, d_v)),
                dMT=rng.normal(size=(N, d_v)))


def explicit_path_grads(c):
    """The hand-written adjoints composed: scan, then the addressing."""
    wwt = ob.slot_weights(c["k"], c["C"], c["widx"])
    rwt = ob.slot_weights(c["q"], c["C"], c["ridx"])
    s = ob.scan_backward_stream(c["M0"], c["widx"], wwt, c["ridx"], rwt, c["v"], c["alpha"],
                                c["beta"], c["dout"], c["dMT"])
    sc = ob.score_backward(c["q"][None, None], c["k"][None, None], c["C"][None],
                           c["widx"][None, None], c["ridx"][None, None],
                           s["dwwt"][None, None], s["drwt"][None, None])
    return dict(q=sc["dq"][0, 0], k=sc["dk"][0, 0], C=sc["dsubkeys"][0], M0=s["dM0"],
                v=s["dv"], alpha=s["dalpha"], beta=s["dbeta"]), s, wwt, rwt


@pytest.mark.parametrize("seed,hot", [(1, None), (2, 10), (3, 6)])
def test_scan_adjoint_equals_autograd(seed, hot):
    c = stream_case(seed, hot=hot)
    wwt = ob.slot_weights(c["k"], c["C"], c["widx"])
    rwt = ob.slot_weights(c["q"], c["C"], c["ridx"])
    s = ob.scan_backward_stream(c["M0"], c["widx"], wwt, c["ridx"], rwt, c["v"], c["alpha"],
                                c["beta"], c["dout"], c["dMT"])
    a = ob.scan_grads_autograd(c["M0"], c["widx"], wwt, c["ridx"], rwt, c["v"], c["alpha"],
                               c["beta"], c["dout"], c["dMT"])
    for mine, ref in (("dM0", "M0"), ("dwwt", "wwt"), ("drwt", "rwt"), ("dv", "v"),
                      ("dalpha", "alpha"), ("dbeta", "beta")):
        np.testing.assert_allclose(s[mine], a[ref], rtol=1e-11, atol=1e-11, err_msg=mine)


def test_scan_adjoint_with_repeated_read_slots_equals_autograd():
    """A token may read one slot more than once (the scan's contract asks only
    write slots to be distinct): each read adds its own share of the output's
    gradient to that row.  Weights are free inputs here (rows of a softmax)."""
    c = stream_case(11, T=10, W=3, R=5, hot=7)
    rng = np.random.default_rng(12)
    # repeat slots inside reads: positions 1 and 3 copy position 0, and one
    # token reads a single slot five times
    c["ridx"][:, 1] = c["ridx"][:, 0]
    c["ridx"][:, 3] = c["ridx"][:, 0]
    c["ridx"][4, :] = c["ridx"][4, 2]
    wwt = rng.dirichlet(np.ones(3), size=10)
    rwt = rng.dirichlet(np.ones(5), size=10)
    s = ob.scan_backward_stream(c["M0"], c["widx"], wwt, c["ridx"], rwt, c["v"], c["alpha"],
                                c["beta"], c["dout"], c["dMT"])
    a = ob.scan_grads_autograd(c["M0"], c["widx"], wwt, c["ridx"], rwt, c["v"], c["alpha"],
                               c["beta"], c["dout"], c["dMT"])
    for mine, ref in (("dM0", "M0"), ("dwwt", "wwt"), ("drwt", "rwt"), ("dv", "v"),
                      ("dalpha", "alpha"), ("dbeta", "beta")):
        np.testing.assert_allclose(s[mine], a[ref], rtol=1e-10, atol=1e-12, err_msg=mine)


@pytest.mark.parametrize("seed,hot", [(4, None), (5, 8)])
def test_composed_adjoints_equal_autograd_of_whole_path(seed, hot):
    c = stream_case(seed, hot=hot)
    mine, *_ = explicit_path_grads(c)
    ref = ob.path_grads_autograd(c["q"], c["k"], c["C"], c["M0"], c["widx"], c["ridx"], c["v"],
                                 c["alpha"], c["beta"], c["dout"], c["dMT"])
    for key in ref:
        np.testing.assert_allclose(mine[key], ref[key], rtol=1e-10, atol=1e-11, err_msg=key)


def test_finite_differences_of_the_forward():
    c = stream_case(6, T=8, hot=9)
    mine, *_ = explicit_path_grads(c)
    rng = np.random.default_rng(60)
    t64 = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    ti = lambda a: torch.tensor(np.asarray(a), dtype=torch.int64)

    def L(x):
        with torch.no_grad():
            return float(ob.loss_t(t64(x["q"]), t64(x["k"]), t64(x["C"]), t64(x["M0"]),
                                   ti(x["widx"]), ti(x["ridx"]), t64(x["v"]), t64(x["alpha"]),
                                   t64(x["beta"]), t64(x["dout"]), t64(x["dMT"])))
    eps = 1e-6
    for key in ("q", "k", "C", "M0", "v", "alpha", "beta"):
        u = rng.normal(size=np.shape(c[key]))
        xp, xm = dict(c), dict(c)
        xp[key] = c[key] + eps * u
        xm[key] = c[key] - eps * u
        fd = (L(xp) - L(xm)) / (2 * eps)
        an = float((mine[key] * u).sum())
        assert abs(fd - an) <= 1e-6 * (1 + abs(an)), (key, fd, an)


def test_fp64_forward_is_the_c_oracles_function():
    c = stream_case(7, T=10, hot=12)
    f32 = lambda a: np.asarray(a, np.float32)
    # weights: the C oracle's own selection, recomputed here in fp64
    ref = oracle.score_topk(f32(c["q"])[None, None], f32(c["k"])[None, None], f32(c["C"])[None],
                            4, 3)
    w64 = ob.slot_weights(f32(c["k"]), f32(c["C"]), ref["widx"][0, 0])
    r64 = ob.slot_weights(f32(c["q"]), f32(c["C"]), ref["ridx"][0, 0])
    np.testing.assert_allclose(w64, ref["wwt"][0, 0], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(r64, ref["rwt"][0, 0], rtol=1e-5, atol=1e-6)
    # the scan, fed the same slots and weights
    M = f32(c["M0"])[None, None].copy()
    out = oracle.scan(M, c["widx"][None, None].astype(np.int32), f32(w64)[None, None],
                      c["ridx"][None, None].astype(np.int32), f32(r64)[None, None],
                      f32(c["v"])[None, None], f32(c["alpha"])[None, None],
                      f32(c["beta"])[None, None])
    t64 = lambda a: torch.tensor(np.asarray(a, np.float32).astype(np.float64))
    ti = lambda a: torch.tensor(np.asarray(a), dtype=torch.int64)
    o64, M64 = ob.scan_forward_t(t64(c["M0"]), ti(c["widx"]), t64(w64), ti(c["ridx"]),
                                 t64(r64), t64(c["v"]), t64(c["alpha"]), t64(c["beta"]))
    np.testing.assert_allclose(out[0, 0], o64.numpy(), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(M[0, 0], M64.numpy(), rtol=1e-5, atol=1e-6)


def test_closed_form_one_token_one_slot():
    """T = 1, W = R = 1, the read slot is the written one: w = r = 1, c = beta,
    M1[s] = (1-beta) alpha M0[s] + beta v, o = M1[s].  With G = dMT[s] + dO:
    dv = beta G, dalpha = (1-beta) <G, M0[s]>, dbeta = <G, v - alpha M0[s]>,
    dM0[s] = (1-beta) alpha G, other rows dMT, dr = <dO, M1[s]>, dw = beta dbeta."""
    rng = np.random.default_rng(8)
    N, d_v, s = 16, 5, 11
    M0 = rng.normal(size=(N, d_v))
    v, dO, dMT = rng.normal(size=d_v), rng.normal(size=d_v), rng.normal(size=(N, d_v))
    al, be = 0.9, 0.3
    g = ob.scan_backward_stream(M0, np.array([[s]]), np.ones((1, 1)), np.array([[s]]),
                                np.ones((1, 1)), v[None], np.array([al]), np.array([be]),
                                dO[None], dMT)
    G = dMT[s] + dO
    M1s = (1 - be) * al * M0[s] + be * v
    np.testing.assert_allclose(g["dv"][0], be * G, rtol=1e-14)
    np.testing.assert_allclose(g["dalpha"][0], (1 - be) * G @ M0[s], rtol=1e-13)
    np.testing.assert_allclose(g["dbeta"][0], G @ (v - al * M0[s]), rtol=1e-13)
    np.testing.assert_allclose(g["dwwt"][0, 0], be * (G @ (v - al * M0[s])), rtol=1e-13)
    np.testing.assert_allclose(g["drwt"][0, 0], dO @ M1s, rtol=1e-13)
    expect = dMT.copy()
    expect[s] = (1 - be) * al * G
    np.testing.assert_allclose(g["dM0"], expect, rtol=1e-14)


def test_closed_form_read_only_table():
    """alpha = 1, beta = 0: every write leaves its row as it was, so
    dM0 = dMT + sum_t sum_r r_r dO_t at row ridx_r and dv = 0."""
    c = stream_case(9, T=10, hot=7)
    T = c["widx"].shape[0]
    rwt = ob.slot_weights(c["q"], c["C"], c["ridx"])
    wwt = ob.slot_weights(c["k"], c["C"], c["widx"])
    g = ob.scan_backward_stream(c["M0"], c["widx"], wwt, c["ridx"], rwt, c["v"], np.ones(T),
                                np.zeros(T), c["dout"], c["dMT"])
    expect = c["dMT"].copy()
    for t in range(T):
        for r in range(c["ridx"].shape[1]):
            expect[c["ridx"][t, r]] += rwt[t, r] * c["dout"][t]
    np.testing.assert_allclose(g["dM0"], expect, rtol=1e-13, atol=1e-14)
    assert np.all(g["dv"] == 0)
    np.testing.assert_allclose(g["drwt"], np.einsum("trd,td->tr", c["M0"][c["ridx"]], c["dout"]),
                               rtol=1e-13)


def test_closed_form_shift_invariant_weight_gradient():
    """A weight gradient equal over a token's slots moves no score: softmax
    weights sum to one, so dq, dk and dC vanish."""
    c = stream_case(10, T=6)
    T = c["widx"].shape[0]
    dw = np.repeat(np.random.default_rng(1).normal(size=(T, 1)), 4, 1)
    dr = np.repeat(np.random.default_rng(2).normal(size=(T, 1)), 3, 1)
    sc = ob.score_backward(c["q"][None, None], c["k"][None, None], c["C"][None],
                           c["widx"][None, None], c["ridx"][None, None], dw[None, None],
                           dr[None, None])
    for key in ("dq", "dk", "dsubkeys"):
        assert np.abs(sc[key]).max() < 1e-14, key


def test_score_adjoint_equals_autograd_on_bf16_inputs():
    """bf16 inputs are read as their exact fp32 values (uint16 bit patterns)."""
    rng = np.random.default_rng(11)
    T, n_sub, d_k, W = 9, 16, 32, 5
    f = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = f(rng.normal(size=(T, d_k)))
    C = f(rng.normal(size=(2, n_sub, d_k // 2)) * 0.25)
    idx = np.stack([rng.choice(n_sub * n_sub, W, replace=False) for _ in range(T)])
    dw = rng.normal(size=(T, W))
    sc = ob.score_backward(x[None, None], x[None, None], C[None], idx[None, None],
                           idx[None, None], dw[None, None], np.zeros((1, 1, T, W)))
    gx, gC = ob.score_grads_autograd(ob.as_f64(x), ob.as_f64(C), idx, dw)
    np.testing.assert_allclose(sc["dk"][0, 0], gx, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sc["dsubkeys"][0], gC, rtol=1e-11, atol=1e-12)
    assert np.all(sc["dq"] == 0)
