"""Pins of the CPU oracle against things other than itself (CPU only).

Each test cites the passage of the "Sparse Delta Memory" summary pages
(gist.science paper 2607.07386; ES = Spanish page, FR = French page) or the
mathematical fact it pins.  Kinds of pin: hand-worked fixtures (tests/golden),
brute force, an independent library routine (numpy sort / fp64 matmul),
closed forms, special cases and invariants.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U32 = 2.0 ** -24  # unit roundoff of binary32


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------- fixtures ---

def test_topk_handworked(orc):
    """ES 'Mecanismo Central' item 2: top-k over the outer sum of half scores."""
    g = load("topk_handworked.json")
    s1 = np.array(g["s1"], np.float32)
    s2 = np.array(g["s2"], np.float32)
    for case in g["cases"]:
        k = case["k"]
        for fn in (orc.two_stage_topk, orc.topk_bruteforce):
            res = fn(s1, s2, k)
            assert res[0].tolist() == case["idx"], (fn.__name__, k)
            assert res[1].tolist() == case["score"]
        gap = orc.two_stage_topk(s1, s2, k)[2]
        if case["gap"] == "inf":
            assert gap == np.inf
        else:
            assert np.float32(gap) == np.float32(case["gap"])


def test_scan_handworked(orc):
    """ES 'Mecanismo Central' items 3-4: gated delta write, then sparse read."""
    g = load("scan_handworked.json")
    M = np.array(g["m0"], np.float32).reshape(1, 1, 4, 2).copy()
    toks = g["tokens"]
    T = len(toks)
    f = lambda key, dt=np.float32: np.array([t[key] for t in toks], dt).reshape(1, 1, T, -1)
    out = orc.scan(M, f("widx", np.int32), f("wwt"), f("ridx", np.int32), f("rwt"), f("v"),
                   f("alpha").reshape(1, 1, T), f("beta").reshape(1, 1, T))
    assert out.reshape(T, 2).tolist() == [t["out"] for t in toks]
    assert M.reshape(4, 2).tolist() == g["m_final"]


def test_gdn_handworked(orc):
    """Dense gated-delta baseline, worked by hand."""
    g = load("gdn_handworked.json")
    toks = g["tokens"]
    T = len(toks)
    f = lambda key: np.array([t[key] for t in toks], np.float32).reshape(1, 1, T, -1)
    S = np.zeros((1, 1, 2, 2), np.float32)
    out = orc.gdn_scan(S, f("k"), f("q"), f("v"), f("alpha").reshape(1, 1, T),
                       f("beta").reshape(1, 1, T))
    assert out.reshape(T, 2).tolist() == [t["out"] for t in toks]
    assert S.reshape(2, 2).tolist() == g["s_final"]


# -------------------------------------------------------- half scores ---

def test_half_scores_fp64_bound(orc):
    """s[i] = <x, C_i>: within the recursive-summation error bound of an fp64
    matmul (a dropped term or a transposed table fails this)."""
    rng = np.random.default_rng(0)
    for dh, n_sub in ((16, 32), (64, 256), (7, 5)):
        x = rng.standard_normal(dh).astype(np.float32)
        C = (rng.standard_normal((n_sub, dh)) / np.sqrt(dh)).astype(np.float32)
        s = orc.half_scores(x, C)
        ref = C.astype(np.float64) @ x.astype(np.float64)
        bound = (dh + 1) * U32 * (np.abs(C.astype(np.float64)) @ np.abs(x.astype(np.float64)))
        assert np.all(np.abs(s - ref) <= 1.01 * bound + 1e-30)


def test_half_scores_exact_integers(orc):
    """Small-integer inputs: every product and partial sum is exact in fp32,
    so the result equals the int64 matmul exactly."""
    rng = np.random.default_rng(1)
    x = rng.integers(-8, 9, 64)
    C = rng.integers(-8, 9, (256, 64))
    s = orc.half_scores(x.astype(np.float32), C.astype(np.float32))
    assert np.array_equal(s.astype(np.int64), C @ x)


def test_half_scores_identity_subkeys(orc):
    """Special case C = I (n_sub = d_k/2): the half scores are the half itself,
    the literal reading of 'the halves' outer sum gives the N scores'."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal(16).astype(np.float32)
    assert np.array_equal(orc.half_scores(x, np.eye(16, dtype=np.float32)), x)


# ------------------------------------------------------------ top-k ---

def numpy_topk(s1, s2, k):
    """Top-k of all n_sub^2 fp32 outer sums via numpy's lexsort (independent
    library routine): order by score desc, then slot asc."""
    sums = (s1[:, None] + s2[None, :]).astype(np.float32).ravel()  # fp32 rounding, like C
    slots = np.arange(sums.size)
    order = np.lexsort((slots, -sums.astype(np.float64)))
    return order[:k].astype(np.int32), sums[order[:k]]


@pytest.mark.parametrize("kind", ["int", "gauss"])
def test_bruteforce_vs_numpy(orc, kind):
    rng = np.random.default_rng(3)
    for _ in range(60):
        n_sub = int(rng.integers(1, 24))
        N = n_sub * n_sub
        k = int(rng.integers(1, N + 1))
        if kind == "int":
            s1 = rng.integers(-3, 4, n_sub).astype(np.float32)
            s2 = rng.integers(-3, 4, n_sub).astype(np.float32)
        else:
            s1 = rng.standard_normal(n_sub).astype(np.float32)
            s2 = rng.standard_normal(n_sub).astype(np.float32)
        idx, sc = orc.topk_bruteforce(s1, s2, k)
        ridx, rsc = numpy_topk(s1, s2, k)
        assert np.array_equal(idx, ridx)
        assert np.array_equal(sc, rsc)


def test_two_stage_equals_bruteforce_with_ties(orc):
    """ES item 2: topk(s1 (+) s2) = topk(topk(s1) (+) topk(s2)).  With
    small-integer scores every sum is exact, so the identity must hold exactly
    even under heavy ties (lowest index wins at both stages)."""
    rng = np.random.default_rng(4)
    for _ in range(1500):
        n_sub = int(rng.integers(1, 20))
        N = n_sub * n_sub
        k = int(rng.integers(1, N + 1))
        s1 = rng.integers(-2, 3, n_sub).astype(np.float32)
        s2 = rng.integers(-2, 3, n_sub).astype(np.float32)
        a = orc.two_stage_topk(s1, s2, k)
        b = orc.topk_bruteforce(s1, s2, k)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), (n_sub, k, s1, s2)


def test_two_stage_equals_bruteforce_continuous(orc):
    """Same identity on Gaussian scores.  In fp32 two different half scores can
    round to the same sum; only such rounding ties may reorder slots, and the
    score sequence must still agree exactly."""
    rng = np.random.default_rng(5)
    exceptions = 0
    for _ in range(1500):
        n_sub = int(rng.integers(2, 40))
        k = int(rng.integers(1, min(n_sub * n_sub, 80) + 1))
        s1 = rng.standard_normal(n_sub).astype(np.float32)
        s2 = rng.standard_normal(n_sub).astype(np.float32)
        a = orc.two_stage_topk(s1, s2, k)
        b = orc.topk_bruteforce(s1, s2, k)
        assert np.array_equal(a[1], b[1])
        if not np.array_equal(a[0], b[0]):
            exceptions += 1
            diff = np.nonzero(a[0] != b[0])[0]
            # every differing position sits inside a run of equal scores
            for p in diff:
                assert np.sum(b[1] == b[1][p]) > 1
    assert exceptions <= 3


def test_two_stage_gap(orc):
    """Relative gap between the k-th and (k+1)-th candidate: compared with the
    brute-force ranking of all N sums."""
    rng = np.random.default_rng(6)
    for _ in range(300):
        n_sub = int(rng.integers(2, 16))
        N = n_sub * n_sub
        k = int(rng.integers(1, N + 1))
        s1 = rng.standard_normal(n_sub).astype(np.float32)
        s2 = rng.standard_normal(n_sub).astype(np.float32)
        gap = orc.two_stage_topk(s1, s2, k)[2]
        if k == N:
            assert gap == np.inf
            continue
        _, sc = numpy_topk(s1, s2, k + 1)
        a, b = np.float64(sc[k - 1]), np.float64(sc[k])
        ref = 0.0 if a == b else (a - b) / max(abs(a), abs(b))
        assert abs(gap - ref) <= 1e-6 * max(1.0, ref)


# ---------------------------------------------------------- softmax ---

def test_softmax(orc):
    """Write/read weights: softmax over the selected scores (reading of the
    undefined per-slot factor k_t^(i), ES item 3)."""
    rng = np.random.default_rng(7)
    for k in (1, 2, 8, 64, 128):
        s = np.sort(rng.standard_normal(k).astype(np.float32) * 3)[::-1].copy()
        w = orc.softmax(s)
        e = np.exp(s.astype(np.float64) - s.max())
        ref = e / e.sum()
        assert np.all(np.abs(w - ref) <= 2e-7 + 4e-6 * ref)
        assert np.all(w > 0)
        assert np.all(np.diff(w) <= 0)
        assert abs(float(w.astype(np.float64).sum()) - 1.0) <= k * U32 * 4


def test_softmax_equal_scores_exact(orc):
    """Equal scores: every weight is exactly 1/k for k a power of two."""
    for k in (1, 2, 4, 64):
        w = orc.softmax(np.full(k, 0.37, np.float32))
        assert np.all(w == np.float32(1.0 / k))


# ------------------------------------------------- full addressing ---

def test_score_topk_vs_fp64_bruteforce(orc):
    """The selected slots are the top-W (top-R) of ALL N fp64 outer sums of
    the half scores, up to fp32 rounding; weights are the fp64 softmax of the
    selected sums.  Half 1 = first d_k/2 elements, scored against table 0 of
    the head (reading of 'split into two halves')."""
    rng = np.random.default_rng(8)
    B, H, T, d_k, n_sub, W, R = 1, 2, 6, 32, 32, 8, 5
    dh = d_k // 2
    q = rng.standard_normal((B, H, T, d_k)).astype(np.float32)
    k = rng.standard_normal((B, H, T, d_k)).astype(np.float32)
    C = (rng.standard_normal((H, 2, n_sub, dh)) * 0.25).astype(np.float32)
    res = orc.score_topk(q, k, C, W, R)
    for h in range(H):
        for t in range(T):
            for x, kk, idx, wt, gap in ((k, W, res["widx"], res["wwt"], res["wgap"]),
                                        (q, R, res["ridx"], res["rwt"], res["rgap"])):
                xv = x[0, h, t].astype(np.float64)
                s1 = C[h, 0].astype(np.float64) @ xv[:dh]
                s2 = C[h, 1].astype(np.float64) @ xv[dh:]
                full = (s1[:, None] + s2[None, :]).ravel()
                sel = idx[0, h, t]
                assert len(set(sel.tolist())) == kk
                tol = 1e-5 * (np.abs(full).max() + 1)
                rest = np.delete(full, sel)
                assert full[sel].min() >= rest.max() - tol
                sc = full[sel]
                assert np.all(np.diff(sc) <= tol)  # rank order
                e = np.exp(sc - sc.max())
                assert np.allclose(wt[0, h, t], e / e.sum(), rtol=1e-4, atol=1e-6)
                ranked = np.sort(full)[::-1]
                ref_gap = (ranked[kk - 1] - ranked[kk]) / max(abs(ranked[kk - 1]), abs(ranked[kk]))
                assert abs(gap[0, h, t] - ref_gap) <= 1e-4 + 1e-3 * ref_gap


def test_score_topk_bf16_matches_fp32_of_same_bits(orc):
    """bf16 inputs are widened exactly: feeding the bf16 bit patterns gives
    the same result as feeding their fp32 values."""
    import torch
    rng = np.random.default_rng(9)
    B, H, T, d_k, n_sub = 1, 1, 5, 16, 8
    mk = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(torch.bfloat16)
    q, k, C = mk(B, H, T, d_k), mk(B, H, T, d_k), mk(H, 2, n_sub, d_k // 2)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    a = orc.score_topk(bits(q), bits(k), bits(C), 4, 3)
    b = orc.score_topk(q.float().numpy(), k.float().numpy(), C.float().numpy(), 4, 3)
    for key in a:
        assert np.array_equal(a[key], b[key])


# -------------------------------------------------------------- scan ---

def rand_scan_inputs(rng, B=1, H=1, T=20, n_sub=6, d_v=8, W=3, R=4, m0_std=1.0):
    N = n_sub * n_sub
    widx = np.stack([rng.permutation(N)[:W] for _ in range(B * H * T)]).reshape(B, H, T, W)
    ridx = np.stack([rng.permutation(N)[:R] for _ in range(B * H * T)]).reshape(B, H, T, R)
    wwt = rng.dirichlet(np.ones(W), (B, H, T)).astype(np.float32)
    rwt = rng.dirichlet(np.ones(R), (B, H, T)).astype(np.float32)
    v = rng.standard_normal((B, H, T, d_v)).astype(np.float32)
    alpha = (1 / (1 + np.exp(-rng.normal(3, 1, (B, H, T))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.normal(0, 1, (B, H, T))))).astype(np.float32)
    M0 = (rng.standard_normal((B, H, N, d_v)) * m0_std).astype(np.float32)
    return dict(M0=M0, widx=widx.astype(np.int32), wwt=wwt, ridx=ridx.astype(np.int32), rwt=rwt,
                v=v, alpha=alpha, beta=beta)


def run_scan(orc, d, M=None):
    M = d["M0"].copy() if M is None else M
    out = orc.scan(M, d["widx"], d["wwt"], d["ridx"], d["rwt"], d["v"], d["alpha"], d["beta"])
    return M, out


def test_scan_literal_form_fp64(orc):
    """The oracle's (1-c) m~ + c v equals the page's m~ + beta w (v - m~) (ES
    item 3) evaluated literally in fp64, over many tokens with repeated slots."""
    rng = np.random.default_rng(10)
    d = rand_scan_inputs(rng, B=2, H=2, T=200, n_sub=5, d_v=6, W=4, R=3)
    M, out = run_scan(orc, d)
    M64 = d["M0"].astype(np.float64).copy()
    out64 = np.zeros(out.shape)
    for b in range(2):
        for h in range(2):
            for t in range(200):
                a, be = float(d["alpha"][b, h, t]), float(d["beta"][b, h, t])
                v = d["v"][b, h, t].astype(np.float64)
                for s, w in zip(d["widx"][b, h, t], d["wwt"][b, h, t]):
                    mt = a * M64[b, h, s]
                    M64[b, h, s] = mt + be * float(w) * (v - mt)
                rows = M64[b, h, d["ridx"][b, h, t]]
                out64[b, h, t] = d["rwt"][b, h, t].astype(np.float64) @ rows
    assert np.all(np.abs(M - M64) <= 1e-5 + 1e-4 * np.abs(M64))
    assert np.all(np.abs(out - out64) <= 1e-5 + 1e-4 * np.abs(out64))


def test_scan_unselected_rows_untouched(orc):
    """ES item 3: 'unselected slots remain unchanged' -- bitwise."""
    rng = np.random.default_rng(11)
    d = rand_scan_inputs(rng, T=15, n_sub=8, W=3)
    M, _ = run_scan(orc, d)
    written = np.zeros(64, bool)
    written[d["widx"].ravel()] = True
    assert np.array_equal(M[0, 0, ~written].view(np.uint32), d["M0"][0, 0, ~written].view(np.uint32))
    assert not np.array_equal(M[0, 0, written], d["M0"][0, 0, written])


def test_scan_identity_gates(orc):
    """alpha = 1, beta = 0: M is bitwise unchanged and o = sum r M0[ridx]."""
    rng = np.random.default_rng(12)
    d = rand_scan_inputs(rng, T=10)
    d["alpha"][:] = 1.0
    d["beta"][:] = 0.0
    M, out = run_scan(orc, d)
    assert np.array_equal(M.view(np.uint32), d["M0"].view(np.uint32))
    ref = np.einsum("tr,trd->td", d["rwt"][0, 0].astype(np.float64),
                    d["M0"][0, 0].astype(np.float64)[d["ridx"][0, 0]])
    assert np.all(np.abs(out[0, 0] - ref) <= 1e-6 + 1e-5 * np.abs(ref))


def test_scan_full_strength_write_stores_v(orc):
    """W = 1 gives w = 1; with beta = 1 the write strength c = beta*w = 1 and the
    slot becomes exactly v_t; reading it back alone (R = 1) returns v_t exactly."""
    rng = np.random.default_rng(13)
    d = rand_scan_inputs(rng, T=12, W=1, R=1)
    d["wwt"][:] = 1.0
    d["rwt"][:] = 1.0
    d["beta"][:] = 1.0
    d["ridx"][:] = d["widx"]
    M, out = run_scan(orc, d)
    assert np.array_equal(out, d["v"])
    last = {}
    for t in range(12):
        last[int(d["widx"][0, 0, t, 0])] = t
    for s, t in last.items():
        assert np.array_equal(M[0, 0, s], d["v"][0, 0, t])


def test_scan_dense_limit(orc):
    """W = N (no sparsity): every row gets the dense gated row update
    M <- a M + b w_i (v - a M), with w the softmax over all N outer sums;
    checked with a vectorised fp64 expression over all rows at once, driven
    by addressing computed independently in numpy."""
    rng = np.random.default_rng(14)
    n_sub, d_k, d_v, T = 4, 8, 5, 6
    N = n_sub * n_sub
    q = rng.standard_normal((1, 1, T, d_k)).astype(np.float32)
    k = rng.standard_normal((1, 1, T, d_k)).astype(np.float32)
    C = (rng.standard_normal((1, 2, n_sub, d_k // 2)) * 0.5).astype(np.float32)
    v = rng.standard_normal((1, 1, T, d_v)).astype(np.float32)
    alpha = rng.uniform(0.5, 1, (1, 1, T)).astype(np.float32)
    beta = rng.uniform(0, 1, (1, 1, T)).astype(np.float32)
    M0 = rng.standard_normal((1, 1, N, d_v)).astype(np.float32)
    a = orc.score_topk(q, k, C, N, N)
    M = M0.copy()
    out = orc.scan(M, a["widx"], a["wwt"], a["ridx"], a["rwt"], v, alpha, beta)
    M64 = M0[0, 0].astype(np.float64)
    for t in range(T):
        def dense_w(x):
            s1 = C[0, 0].astype(np.float64) @ x[: d_k // 2].astype(np.float64)
            s2 = C[0, 1].astype(np.float64) @ x[d_k // 2:].astype(np.float64)
            s = (s1[:, None] + s2[None, :]).ravel()
            e = np.exp(s - s.max())
            return e / e.sum()
        wk, wq = dense_w(k[0, 0, t]), dense_w(q[0, 0, t])
        aM = alpha[0, 0, t] * M64
        M64 = aM + beta[0, 0, t] * wk[:, None] * (v[0, 0, t][None, :] - aM)
        o64 = wq @ M64
        assert np.all(np.abs(out[0, 0, t] - o64) <= 1e-5 + 1e-4 * np.abs(o64))
    assert np.all(np.abs(M[0, 0] - M64) <= 1e-5 + 1e-4 * np.abs(M64))


def test_scan_chunked_resume_and_stream_independence(orc):
    """The table is the whole recurrent state: scanning [0,T1) then [T1,T)
    equals one scan bitwise; streams are independent (permuting them permutes
    the results)."""
    rng = np.random.default_rng(15)
    d = rand_scan_inputs(rng, B=2, H=3, T=30, n_sub=4, W=2, R=3)
    M_full, out_full = run_scan(orc, d)
    M = d["M0"].copy()
    outs = []
    for lo, hi in ((0, 11), (11, 30)):
        part = {key: (val[:, :, lo:hi] if key != "M0" else val) for key, val in d.items()}
        outs.append(orc.scan(M, part["widx"], part["wwt"], part["ridx"], part["rwt"], part["v"],
                             part["alpha"], part["beta"]))
    assert np.array_equal(np.concatenate(outs, axis=2), out_full)
    assert np.array_equal(M, M_full)
    perm = rng.permutation(6)
    flat = {key: val.reshape((6,) + val.shape[2:])[perm].reshape(val.shape) for key, val in d.items()}
    M_p, out_p = run_scan(orc, flat)
    assert np.array_equal(out_p.reshape(6, -1), out_full.reshape(6, -1)[perm])
    assert np.array_equal(M_p.reshape(6, -1), M_full.reshape(6, -1)[perm])


def test_scan_bounded(orc):
    """Each write is a convex combination of alpha*M and v, and each read a
    convex combination of rows, so |M| and |o| never exceed
    max(|M0|, max|v|) (up to rounding)."""
    rng = np.random.default_rng(16)
    d = rand_scan_inputs(rng, T=300, n_sub=4, W=3, R=3, m0_std=3.0)
    M, out = run_scan(orc, d)
    bound = max(np.abs(d["M0"]).max(), np.abs(d["v"]).max()) * (1 + 1e-6)
    assert np.abs(M).max() <= bound
    assert np.abs(out).max() <= bound


def test_scan_rejects_bad_index(orc):
    rng = np.random.default_rng(17)
    d = rand_scan_inputs(rng, T=3)
    d["widx"][0, 0, 1, 0] = 36
    M = d["M0"].copy()
    with pytest.raises(orc.OracleError):
        orc.scan(M, d["widx"], d["wwt"], d["ridx"], d["rwt"], d["v"], d["alpha"], d["beta"])
    assert np.array_equal(M, d["M0"])


# --------------------------------------------------------------- GDN ---

def test_gdn_decay_only(orc):
    """beta = 0: S_t = alpha_t S_{t-1} bitwise (sequential fp32 products)."""
    rng = np.random.default_rng(20)
    B, H, T, dk, dv = 1, 2, 9, 6, 5
    S0 = rng.standard_normal((B, H, dv, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    alpha = rng.uniform(0.5, 1, (B, H, T)).astype(np.float32)
    S = S0.copy()
    orc.gdn_scan(S, k, k, rng.standard_normal((B, H, T, dv)).astype(np.float32), alpha,
                 np.zeros((B, H, T), np.float32))
    ref = S0.copy()
    for t in range(T):
        ref = (alpha[:, :, t, None, None] * ref).astype(np.float32)
    assert np.array_equal(S, ref)


def test_gdn_first_step_closed_form(orc):
    """From S = 0, one step: S_1 = beta v k^T and o = beta (k.q) v."""
    rng = np.random.default_rng(21)
    dk, dv = 16, 12
    k = rng.standard_normal((1, 1, 1, dk)).astype(np.float32)
    q = rng.standard_normal((1, 1, 1, dk)).astype(np.float32)
    v = rng.standard_normal((1, 1, 1, dv)).astype(np.float32)
    alpha = np.array([[[0.9]]], np.float32)
    beta = np.array([[[0.3]]], np.float32)
    S = np.zeros((1, 1, dv, dk), np.float32)
    out = orc.gdn_scan(S, k, q, v, alpha, beta)
    b = float(beta.ravel()[0])
    S_ref = b * np.outer(v.ravel().astype(np.float64), k.ravel().astype(np.float64))
    o_ref = b * float(k.ravel().astype(np.float64) @ q.ravel().astype(np.float64)) * v.ravel()
    assert np.allclose(S[0, 0], S_ref, rtol=1e-6, atol=1e-7)
    assert np.allclose(out.ravel(), o_ref, rtol=1e-5, atol=1e-6)


def test_gdn_delta_rule_recalls_last_write(orc):
    """Delta-rule property: with beta_t = 1 and unit-norm k_t, S_t k_t = v_t for
    any alpha_t (the update fits the new association exactly), so reading with
    q_t = k_t returns v_t."""
    rng = np.random.default_rng(22)
    B, H, T, dk, dv = 1, 3, 40, 32, 16
    g = rng.standard_normal((B, H, T, dk))
    k = (g / np.linalg.norm(g, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    alpha = rng.uniform(0.6, 1, (B, H, T)).astype(np.float32)
    S = np.zeros((B, H, dv, dk), np.float32)
    out = orc.gdn_scan(S, k, k, v, alpha, np.ones((B, H, T), np.float32))
    assert np.all(np.abs(out - v) <= 2e-5 * (1 + np.abs(v)))


def test_gdn_matches_sdm_one_hot(orc):
    """Cross-oracle special case: SDM with W = R = 1 (so w = r = 1) and alpha = 1
    on N slots is GDN with one-hot keys k = e_widx, queries q = e_ridx and
    S = M^T.  The two oracles use different but algebraically equal update
    forms, so they agree to a few ulps."""
    rng = np.random.default_rng(23)
    n_sub, dv, T = 3, 4, 25
    N = n_sub * n_sub
    d = rand_scan_inputs(rng, T=T, n_sub=n_sub, d_v=dv, W=1, R=1)
    d["wwt"][:] = 1.0
    d["rwt"][:] = 1.0
    d["alpha"][:] = 1.0
    M, out = run_scan(orc, d)
    eye = np.eye(N, dtype=np.float32)
    k = eye[d["widx"][..., 0]]
    q = eye[d["ridx"][..., 0]]
    S = np.ascontiguousarray(d["M0"].transpose(0, 1, 3, 2))
    out_g = orc.gdn_scan(S, k, q, d["v"], d["alpha"], d["beta"])
    assert np.allclose(out_g, out, rtol=1e-6, atol=1e-6)
    assert np.allclose(S.transpose(0, 1, 3, 2), M, rtol=1e-6, atol=1e-6)


def test_gdn_bounded(orc):
    """|alpha (I - beta k k^T)| <= alpha < 1 for unit k: the state stays bounded."""
    rng = np.random.default_rng(24)
    B, H, T, dk, dv = 1, 1, 500, 16, 8
    g = rng.standard_normal((B, H, T, dk))
    k = (g / np.linalg.norm(g, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    alpha = (1 / (1 + np.exp(-rng.normal(3, 1, (B, H, T))))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.normal(0, 1, (B, H, T))))).astype(np.float32)
    S = np.zeros((B, H, dv, dk), np.float32)
    orc.gdn_scan(S, k, k, v, alpha, beta)
    assert np.isfinite(S).all()
    assert np.linalg.norm(S[0, 0], 2) <= np.abs(v).max() * np.sqrt(dv) / (1 - alpha.max()) + 1
