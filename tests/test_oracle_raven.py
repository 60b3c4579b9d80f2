"""Pins of the Raven-style routed-slot oracle (oracle/raven.py) -- CPU only.

  * the router's top-K equals a brute-force count (how many entries beat each
    entry, ties to the lower index), on integer logits full of ties;
  * gates are positive, non-increasing in rank and sum to one;
  * a = 0 freezes every slot bit for bit; slots never routed keep their rows
    bit for bit whatever a is;
  * K = 1 (gate 1) and a -> -inf (gamma = 0) have closed forms;
  * a two-token example worked by hand;
  * cross-oracle: the SDM oracle's scan (plain fp32 C) with alpha = beta = 1
    and write weights 1 - exp(a r) is the same recurrence, so it must agree
    with this one to fp32 rounding.
"""
import numpy as np

import oracle
from oracle import raven as rv


def brute_topk(z, K):
    """Rank of entry i = #{j: z_j > z_i or (z_j == z_i and j < i)}."""
    z = list(z)
    rank = [sum(1 for j in range(len(z)) if z[j] > z[i] or (z[j] == z[i] and j < i))
            for i in range(len(z))]
    out = [0] * K
    for i, rk in enumerate(rank):
        if rk < K:
            out[rk] = i
    return np.array(out)


def stream(seed, T=20, M=64, d=6, K=5, a_scale=1.0):
    rng = np.random.default_rng(seed)
    return dict(S0=rng.normal(size=(M, d)), zk=rng.normal(size=(T, M)), zq=rng.normal(size=(T, M)),
                a=-a_scale * np.log1p(np.exp(rng.normal(size=T))), u=rng.normal(size=(T, d)), K=K)


def test_topk_equals_brute_force_with_ties():
    rng = np.random.default_rng(1)
    for M, K in ((16, 5), (50, 50), (64, 1), (33, 17)):
        for _ in range(20):
            z = rng.integers(-3, 4, size=M).astype(np.float64)
            assert np.array_equal(rv.topk_desc(z, K), brute_topk(z, K))


def test_gates_are_a_distribution_in_rank_order():
    rng = np.random.default_rng(2)
    for _ in range(50):
        i, r = rv.route(rng.normal(size=100) * 3, 16)
        assert np.all(r > 0) and abs(r.sum() - 1) < 1e-14
        assert np.all(np.diff(r) <= 0)
        assert len(set(i.tolist())) == 16


def test_zero_decay_freezes_everything():
    c = stream(3)
    S = c["S0"].copy()
    o = rv.raven_scan_stream(S, c["zk"], c["zq"], np.zeros(len(c["a"])), c["u"], c["K"])
    assert np.array_equal(S, c["S0"])
    for t in range(len(o)):
        j, rq = rv.route(c["zq"][t], c["K"])
        assert np.allclose(o[t], rq @ c["S0"][j], rtol=1e-14, atol=0)


def test_unrouted_slots_keep_their_rows():
    c = stream(4, T=15, M=128, K=4, a_scale=3.0)
    S = c["S0"].copy()
    rv.raven_scan_stream(S, c["zk"], c["zq"], c["a"], c["u"], c["K"])
    touched = set()
    for t in range(15):
        touched.update(rv.topk_desc(c["zk"][t], c["K"]).tolist())
    frozen = np.array(sorted(set(range(128)) - touched))
    assert len(frozen) > 0 and np.array_equal(S[frozen], c["S0"][frozen])
    assert not np.array_equal(S[sorted(touched)], c["S0"][sorted(touched)])


def test_closed_forms_one_slot_and_full_decay():
    c = stream(5, T=1, K=1)
    S = c["S0"].copy()
    rv.raven_scan_stream(S, c["zk"], c["zq"], c["a"], c["u"], 1)
    s = int(np.argmax(c["zk"][0]))
    g = np.exp(c["a"][0])  # the one routed slot gets gate 1
    assert np.allclose(S[s], g * c["S0"][s] + (1 - g) * c["u"][0], rtol=1e-14)
    # a -> -inf: every routed slot becomes u_t exactly
    c = stream(6, T=3, K=7)
    S = c["S0"].copy()
    rv.raven_scan_stream(S, c["zk"], c["zq"], np.full(3, -1e4), c["u"], 7)
    last = rv.topk_desc(c["zk"][2], 7)
    assert np.array_equal(S[last], np.repeat(c["u"][2][None], 7, 0))


def test_hand_worked_two_tokens():
    """M = 4 slots, K = 2, d = 1, S0 = [1, 2, 3, 4], a = ln(1/2) on both tokens.
    Token 0: zk = [0, 5, 5, -1] routes slots 1, 2 (tie -> lower first) with
    equal gates 1/2, so gamma = 2^-1/2 on both; u = 10.
    Token 1: zk = [9, 0, 0, 0] routes slots 0, 1 (1 wins the tie of zeros),
    gates proportional to sigmoid(9), sigmoid(0); u = -2."""
    S = np.array([[1.0], [2.0], [3.0], [4.0]])
    zk = np.array([[0, 5, 5, -1], [9, 0, 0, 0]], np.float64)
    zq = np.array([[0, 0, 0, 7], [0, 8, 0, 0]], np.float64)
    a = np.full(2, np.log(0.5))
    u = np.array([[10.0], [-2.0]])
    o = rv.raven_scan_stream(S, zk, zq, a, u, 2)
    g = 0.5 ** 0.5
    s1 = g * 2 + (1 - g) * 10
    s2 = g * 3 + (1 - g) * 10
    # token 0 read: slots 3 (z=7) and 0 (first of the zeros), gates sigmoid(7), 1/2
    m3, m0 = 1 / (1 + np.exp(-7.0)), 0.5
    assert np.isclose(o[0, 0], (m3 * 4 + m0 * 1) / (m3 + m0), rtol=1e-14)
    m9 = 1 / (1 + np.exp(-9.0))
    r0, r1 = m9 / (m9 + 0.5), 0.5 / (m9 + 0.5)
    g0, g1 = 0.5 ** r0, 0.5 ** r1
    s0 = g0 * 1 + (1 - g0) * -2
    s1b = g1 * s1 + (1 - g1) * -2
    assert np.allclose(S[:, 0], [s0, s1b, s2, 4.0], rtol=1e-14)
    # token 1 read: slot 1 (z=8) then slot 0 (first of the zeros)
    m8 = 1 / (1 + np.exp(-8.0))
    assert np.isclose(o[1, 0], (m8 * s1b + 0.5 * s0) / (m8 + 0.5), rtol=1e-14)


def test_same_recurrence_as_the_sdm_scan_oracle():
    """alpha = beta = 1 and w = 1 - exp(a r) turn the SDM write
    (1 - c)(alpha M) + c v into gamma M + (1 - gamma) u."""
    B, H, T, M, d, K = 1, 2, 30, 64, 8, 6
    rng = np.random.default_rng(7)
    zk = rng.normal(size=(B, H, T, M))
    zq = rng.normal(size=(B, H, T, M))
    a = -np.log1p(np.exp(rng.normal(size=(B, H, T))))
    u = rng.normal(size=(B, H, T, d)).astype(np.float32)
    S0 = rng.normal(size=(B, H, M, d)).astype(np.float32)
    rt = rv.route_tokens(zk, zq, a, K)
    Mtab = S0.copy()
    out = oracle.scan(Mtab, rt["widx"], rt["wcoef"].astype(np.float32), rt["ridx"],
                      rt["rwt"].astype(np.float32), u, np.ones((B, H, T), np.float32),
                      np.ones((B, H, T), np.float32))
    for h in range(H):
        S = S0[0, h].astype(np.float64)
        o = rv.raven_scan_stream(S, zk[0, h], zq[0, h], a[0, h], u[0, h], K)
        np.testing.assert_allclose(Mtab[0, h], S, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(out[0, h], o, rtol=1e-5, atol=1e-6)
