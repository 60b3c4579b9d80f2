"""The parity checker itself, on the CPU (no GPU): the rules the GPU tests apply.

compare_topk must accept a slot set that differs from the oracle's only by a
swap of exactly tied slots, and reject a swap for a slot that scores lower, a
set that differs where the oracle's gap is large, duplicate slots, and weights
that are not the softmax of the chosen slots.  taint must mark exactly the rows
a flipped write touched and the outputs that read them from that token on.
Every "GPU" list here is built by hand from the oracle's own output.
"""
import numpy as np
import pytest

import oracle
from gpu_util import compare_topk, e2e_stream, slot_scores64, taint


def tie_case():
    """One token whose k' ties two slots exactly at the write boundary:
    sub-keys are unit vectors, so half-scores are the halves themselves."""
    n_sub, dh = 4, 4
    C = np.zeros((1, 2, n_sub, dh), np.float32)
    for c in range(2):
        C[0, c, :, :] = np.eye(n_sub, dh)
    # half 1 scores [3, 2, 1, 0], half 2 scores [3, 2, 2, 0]:
    # slot sums: (0,0)=6, (0,1)=5, (0,2)=5, (1,0)=5, (0,3)=3, (1,1)=4, (1,2)=4 ...
    k = np.array([3, 2, 1, 0, 3, 2, 2, 0], np.float32).reshape(1, 1, 1, 8)
    q = k.copy()
    return n_sub, C, q, k


def test_exact_tie_swap_is_flagged_and_valid(orc):
    n_sub, C, q, k = tie_case()
    W = 3  # ranks: 6 (slot 0), 5 (slot 1), 5 (slot 2); then 5 (slot 4) ties the 3rd
    ref = orc.score_topk(q, k, C, W, W)
    assert ref["widx"][0, 0, 0].tolist() == [0, 1, 2]
    assert ref["wgap"][0, 0, 0] == 0.0
    # a "GPU" set that took slot 4 (sum 5, tied) instead of slot 2
    g_idx = np.array([[[[0, 1, 4]]]], np.int32)
    s = slot_scores64(k[0, 0, 0].astype(np.float64), C[0].astype(np.float64), [0, 1, 4], n_sub)
    e = np.exp(s - s.max())
    g_wt = (e / e.sum()).astype(np.float32)[None, None, None]
    t = compare_topk(g_idx, g_wt, ref["widx"], ref["wwt"], ref["wgap"], k, C)
    assert (t.tokens, t.flagged, t.bad) == (1, 1, 0) and t.flagged_at == [0]


def test_swap_for_a_lower_slot_is_rejected(orc):
    n_sub, C, q, k = tie_case()
    ref = orc.score_topk(q, k, C, 3, 3)
    # slot 5 = (1,1) sums to 4, below the boundary: not a near-tie
    g_idx = np.array([[[[0, 1, 5]]]], np.int32)
    t = compare_topk(g_idx, ref["wwt"], ref["widx"], ref["wwt"], ref["wgap"], k, C)
    assert t.bad == 1 and t.flagged == 0


def test_wrong_weights_on_a_valid_swap_are_rejected(orc):
    n_sub, C, q, k = tie_case()
    ref = orc.score_topk(q, k, C, 3, 3)
    g_idx = np.array([[[[0, 1, 4]]]], np.int32)
    g_wt = np.array([[[[0.5, 0.3, 0.2]]]], np.float32)  # rank-ordered, sums to 1, wrong
    t = compare_topk(g_idx, g_wt, ref["widx"], ref["wwt"], ref["wgap"], k, C)
    assert t.bad == 1


def test_difference_with_a_large_gap_is_rejected(orc):
    rng = np.random.default_rng(3)
    C = rng.standard_normal((1, 2, 16, 8)).astype(np.float32)
    k = rng.standard_normal((1, 1, 32, 16)).astype(np.float32)
    ref = orc.score_topk(k, k, C, 4, 4)
    big = ref["wgap"][0, 0] >= 1e-5
    t0 = int(np.nonzero(big)[0][0])
    g_idx = ref["widx"].copy()
    # replace the last slot of a well-separated token by its (k+1)-th best
    s_all = np.add.outer(*(C[0, c].astype(np.float64) @ k[0, 0, t0, 8 * c:8 * c + 8]
                           .astype(np.float64) for c in range(2))).ravel()
    order = np.lexsort((np.arange(256), -s_all))
    g_idx[0, 0, t0, -1] = order[4]
    t = compare_topk(g_idx, ref["wwt"], ref["widx"], ref["wwt"], ref["wgap"], k, C)
    assert t.bad == 1


def test_duplicate_slots_are_rejected(orc):
    n_sub, C, q, k = tie_case()
    ref = orc.score_topk(q, k, C, 3, 3)
    g_idx = np.array([[[[0, 1, 1]]]], np.int32)
    with pytest.raises(AssertionError):
        compare_topk(g_idx, ref["wwt"], ref["widx"], ref["wwt"], ref["wgap"], k, C)


def test_taint_marks_flipped_rows_and_later_reads():
    T, N = 6, 32
    r_w = np.array([[0, 1], [2, 3], [4, 5], [6, 7], [8, 9], [10, 11]])
    g_w = r_w.copy()
    g_w[2] = [4, 20]            # token 2 wrote 20 instead of 5
    r_r = np.array([[12, 13], [5, 14], [15, 16], [20, 17], [18, 19], [21, 5]])
    g_r = r_r.copy()
    g_r[4] = [18, 22]           # token 4's read set flipped
    row_ok, out_ok = taint(N, T, g_w, r_w, [2], g_r, r_r, [4])
    assert set(np.nonzero(~row_ok)[0].tolist()) == {5, 20}
    # token 1 read row 5 before the flip (ok); token 3 reads 20, token 5 reads 5
    assert out_ok.tolist() == [True, True, True, False, False, False]


def test_e2e_stream_on_oracle_lists_compares_everything(orc):
    """The oracle against itself: nothing flagged, every output and row compared."""
    rng = np.random.default_rng(5)
    n_sub, dh, T, d_v, W = 8, 8, 20, 4, 3
    C = rng.standard_normal((1, 2, n_sub, dh)).astype(np.float32)
    q = rng.standard_normal((1, 1, T, 2 * dh)).astype(np.float32)
    k = rng.standard_normal((1, 1, T, 2 * dh)).astype(np.float32)
    v = rng.standard_normal((1, 1, T, d_v)).astype(np.float32)
    al = np.full((1, 1, T), 0.9, np.float32)
    be = np.full((1, 1, T), 0.5, np.float32)
    ref = orc.score_topk(q, k, C, W, W)
    M = np.zeros((1, 1, n_sub * n_sub, d_v), np.float32)
    o = orc.scan(M, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"], v, al, be)
    gl = [ref[key][0, 0] for key in ("widx", "wwt", "ridx", "rwt")]
    t = e2e_stream(gl, ref, k[0, 0], q[0, 0], C, M[0, 0], M[0, 0], o[0, 0], o[0, 0])
    assert t.outs_compared == T and t.rows_compared == n_sub * n_sub
    # a perturbed output outside any tainted position fails
    o2 = o[0, 0].copy()
    o2[7, 1] += 1e-3
    with pytest.raises(AssertionError):
        e2e_stream(gl, ref, k[0, 0], q[0, 0], C, M[0, 0], M[0, 0], o2, o[0, 0])
