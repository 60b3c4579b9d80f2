"""Helpers for the GPU parity tests (comparison rules against the CPU oracle)."""
import numpy as np
import torch

import synth

GAP_TOL = 1e-5     # oracle relative gap below which a slot-set flip is allowed
ATOL, RTOL = 1e-5, 1e-4


def say(*a):
    print(*a, flush=True)


def np_(t):
    return synth.to_numpy(t)


def close(g, r, atol=ATOL, rtol=RTOL):
    return np.abs(g.astype(np.float64) - r.astype(np.float64)) <= atol + rtol * np.abs(r)


def compare_topk(g_idx, g_wt, r_idx, r_wt, r_gap, N):
    """Slot sets must match per token except where the oracle's gap between the
    k-th and (k+1)-th candidate is below GAP_TOL; on matching sets the weight of
    every slot must agree.  Returns (#tokens, #flagged, #mismatched)."""
    k = g_idx.shape[-1]
    g_idx = g_idx.reshape(-1, k)
    r_idx = r_idx.reshape(-1, k)
    g_wt = g_wt.reshape(-1, k)
    r_wt = r_wt.reshape(-1, k)
    gap = r_gap.reshape(-1)
    assert g_idx.min() >= 0 and g_idx.max() < N
    # distinct slots per token, weights in rank order and summing to one
    gs = np.sort(g_idx, -1)
    assert np.all(np.diff(gs, axis=-1) > 0), "duplicate slots in a token"
    assert np.all(np.diff(g_wt, axis=-1) <= 1e-6), "weights not in rank order"
    assert np.allclose(g_wt.sum(-1), 1.0, atol=1e-5)
    rs = np.sort(r_idx, -1)
    same = np.all(gs == rs, -1)
    flagged = ~same & (gap < GAP_TOL)
    bad = ~same & ~flagged
    # weights by slot on matching sets
    go = np.argsort(g_idx, -1)
    ro = np.argsort(r_idx, -1)
    gw = np.take_along_axis(g_wt, go, -1)[same]
    rw = np.take_along_axis(r_wt, ro, -1)[same]
    assert np.all(close(gw, rw)), "weights differ on matching slot sets"
    return int(same.size), int(flagged.sum()), int(bad.sum())


def oracle_inputs_for(x, b, h, ts=None):
    """Host copies (numpy, bf16 as uint16) of one stream's addressing inputs."""
    sl = (slice(b, b + 1), slice(h, h + 1)) + ((ts,) if ts is not None else ())
    q = np_(x["q"][sl])
    k = np_(x["k"][sl])
    if ts is not None and q.ndim == 3:
        q, k = q[:, :, None, :], k[:, :, None, :]
    return q, k, np_(x["subkeys"][h:h + 1])


def make_torch_inputs(wl, dev, with_m0=True):
    return synth.make_inputs(wl, device=dev, with_m0=with_m0)
