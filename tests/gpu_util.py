"""Helpers for the GPU parity tests (comparison rules against the CPU oracle).

Slot sets.  Per token, the GPU's slot set must equal the oracle's.  A different
set is accepted only where the oracle's relative gap between its k-th and
(k+1)-th candidate sum is below GAP_TOL, and only if the difference is a swap
of near-equal slots: every slot the GPU chose that the oracle did not, and
every slot the oracle chose that the GPU did not, is scored in fp64 from the
inputs (q' or k' and the sub-key tables, never from anything the GPU
computed), and the best excluded slot may beat the worst included one by at
most GAP_TOL relative.  On such a token the GPU's weights must also be the
fp64 softmax of its own slots' fp64 scores.  Such tokens are counted.

End to end.  One flipped write slot changes two rows of the table (the slot
the oracle wrote and the one the GPU wrote instead), and from then on every
read of those rows.  Rows never interact, so `taint` marks exactly those rows
(from the token of the flip on) and the outputs that read them or whose own
read set flipped; everything else is compared.
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

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


def as_f64(a):
    """Host array of fp32 values or bf16 bit patterns (uint16) as float64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def workers():
    """Host threads for oracle runs: the CPUs this process may use, at most 16
    (the oracle is single-threaded C and releases the GIL)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def thread_map(fn, items, n=None):
    """fn over items on a thread pool, results in item order."""
    with ThreadPoolExecutor(max_workers=n or workers()) as ex:
        return list(ex.map(fn, items))


def slot_scores64(x64, C64, slots, n_sub):
    """fp64 scores of `slots` for one token: x64 [d_k] (the token's k' or q'),
    C64 [2][n_sub][d_k/2] (its head's sub-keys); slot = i*n_sub + j scores
    <x[:d/2], C[0][i]> + <x[d/2:], C[1][j]>."""
    dh = x64.shape[0] // 2
    slots = np.asarray(slots, np.int64)
    i, j = slots // n_sub, slots % n_sub
    return C64[0][i] @ x64[:dh] + C64[1][j] @ x64[dh:]


@dataclass
class TopkTally:
    tokens: int = 0          # token sets compared
    flagged: int = 0         # sets that differ within the gap rule (valid swaps)
    bad: int = 0             # sets that differ outside it, or invalid swaps
    flagged_at: list = field(default_factory=list)  # flat token positions of flagged sets

    def add(self, o):
        self.tokens += o.tokens
        self.flagged += o.flagged
        self.bad += o.bad
        return self


def compare_topk(g_idx, g_wt, r_idx, r_wt, r_gap, x, C, msg=""):
    """Compare one side (writes or reads) of the addressing.

    g_idx, g_wt: the GPU's [..., T, k] lists; r_idx, r_wt, r_gap: the oracle's;
    x: the side's inputs [..., T, d_k] (k' for writes, q' for reads; fp32 or
    bf16 bits) with the same leading shape; C: sub-keys [H, 2, n_sub, d_k/2]
    (fp32 or bf16 bits), where the head of a token is its second-to-last
    leading index (inputs are [B, H, T, ...]) or 0 when there is only one
    leading axis.  Returns a TopkTally.
    """
    k = g_idx.shape[-1]
    lead = g_idx.shape[:-1]
    n_sub = C.shape[2]
    N = n_sub * n_sub
    g_idx = g_idx.reshape(-1, k)
    r_idx = r_idx.reshape(-1, k)
    g_wt = g_wt.reshape(-1, k)
    r_wt = r_wt.reshape(-1, k)
    gap = r_gap.reshape(-1)
    assert g_idx.min() >= 0 and g_idx.max() < N, f"{msg}: slot outside [0, N)"
    # distinct slots per token, weights in rank order and summing to one
    gs = np.sort(g_idx, -1)
    assert np.all(np.diff(gs, axis=-1) > 0), f"{msg}: duplicate slots in a token"
    assert np.all(np.diff(g_wt, axis=-1) <= 1e-6), f"{msg}: weights not in rank order"
    assert np.allclose(g_wt.sum(-1), 1.0, atol=1e-5), f"{msg}: weights do not sum to one"
    rs = np.sort(r_idx, -1)
    same = np.all(gs == rs, -1)
    # weights by slot on matching sets
    go = np.argsort(g_idx, -1)
    ro = np.argsort(r_idx, -1)
    gw = np.take_along_axis(g_wt, go, -1)[same]
    rw = np.take_along_axis(r_wt, ro, -1)[same]
    assert np.all(close(gw, rw)), f"{msg}: weights differ on matching slot sets"
    tally = TopkTally(tokens=int(same.size))
    diff = np.nonzero(~same)[0]
    if diff.size == 0:
        return tally
    xf = x.reshape(-1, x.shape[-1])
    T = lead[-1]
    nlead = len(lead)
    for pos in diff:
        if not gap[pos] < GAP_TOL:
            tally.bad += 1
            continue
        head = (pos // T) % C.shape[0] if nlead >= 2 else 0
        x64 = as_f64(xf[pos])
        C64 = as_f64(C[head])
        gset, rset = set(g_idx[pos].tolist()), set(r_idx[pos].tolist())
        only_g = sorted(gset - rset)
        only_r = sorted(rset - gset)
        sg = slot_scores64(x64, C64, only_g, n_sub)
        sr = slot_scores64(x64, C64, only_r, n_sub)
        kth = slot_scores64(x64, C64, r_idx[pos], n_sub).min()
        den = max(abs(kth), abs(sr.max()), abs(sg.min()), 1e-30)
        ok = (sr.max() - sg.min()) <= GAP_TOL * den
        # the GPU's weights are the softmax of its own slots' scores
        s_all = slot_scores64(x64, C64, g_idx[pos], n_sub)
        e = np.exp(s_all - s_all.max())
        ok = ok and bool(np.all(close(g_wt[pos], e / e.sum())))
        if ok:
            tally.flagged += 1
            tally.flagged_at.append(int(pos))
        else:
            tally.bad += 1
    return tally


def taint(N, T, g_widx, r_widx, flag_w, g_ridx, r_ridx, flag_r):
    """Positions one stream's end-to-end comparison must skip.

    g_widx/r_widx [T, W] and g_ridx/r_ridx [T, R]: the GPU's and the oracle's
    slot lists; flag_w / flag_r: tokens whose write / read sets differ (valid
    swaps).  Returns (row_ok [N] bool: rows that no flipped write touched,
    out_ok [T] bool: outputs whose read set did not flip and that read no row
    touched by a flipped write at or before their token)."""
    INF = np.iinfo(np.int64).max
    t_row = np.full(N, INF, np.int64)
    for t in sorted(flag_w):
        rows = np.setxor1d(g_widx[t], r_widx[t])
        t_row[rows] = np.minimum(t_row[rows], t)
    out_ok = np.ones(T, bool)
    out_ok[list(flag_r)] = False
    if flag_w:
        tt = np.arange(T)[:, None]
        hit = (t_row[g_ridx] <= tt).any(1) | (t_row[r_ridx] <= tt).any(1)
        out_ok &= ~hit
    return t_row == INF, out_ok


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


def device_sync():
    torch.cuda.synchronize()


@dataclass
class E2ETally:
    """End-to-end comparison counts over streams."""
    streams: int = 0
    w: TopkTally = field(default_factory=TopkTally)
    r: TopkTally = field(default_factory=TopkTally)
    flagged_streams: int = 0
    outs: int = 0            # outputs (tokens) in the compared streams
    outs_compared: int = 0
    rows: int = 0
    rows_compared: int = 0

    def add(self, o):
        self.streams += o.streams
        self.w.add(o.w)
        self.r.add(o.r)
        self.flagged_streams += o.flagged_streams
        self.outs += o.outs
        self.outs_compared += o.outs_compared
        self.rows += o.rows
        self.rows_compared += o.rows_compared
        return self

    def line(self, label):
        return (f"{label}: {self.streams} streams; flagged (valid near-tie swaps) write sets "
                f"{self.w.flagged} and read sets {self.r.flagged} of {self.w.tokens} tokens each, "
                f"in {self.flagged_streams} streams; mismatched {self.w.bad + self.r.bad}; "
                f"outputs compared {self.outs_compared} of {self.outs}; "
                f"table rows compared {self.rows_compared} of {self.rows}")


def e2e_stream(g_lists, ref, xk, xq, C, Mg, M_ref, og, o_ref, msg=""):
    """One stream end to end: the GPU's addressing + scan against the oracle's
    own addressing + scan.

    g_lists: the GPU's (widx, wwt, ridx, rwt), each [T, k]; ref: the oracle's
    score_topk dict for the stream ([1,1,T,...] arrays); xk, xq: the stream's
    k', q' [T, d_k]; C: its head's sub-keys [1, 2, n_sub, d_k/2]; Mg / M_ref:
    final tables [N, d_v]; og / o_ref: outputs [T, d_v].  Asserts and returns
    an E2ETally for the stream."""
    gw, gww, gr, grw = g_lists
    T = gw.shape[0]
    N = C.shape[2] * C.shape[2]
    tw = compare_topk(gw, gww, ref["widx"][0, 0], ref["wwt"][0, 0], ref["wgap"][0, 0], xk, C,
                      msg=f"{msg} writes")
    tr = compare_topk(gr, grw, ref["ridx"][0, 0], ref["rwt"][0, 0], ref["rgap"][0, 0], xq, C,
                      msg=f"{msg} reads")
    assert tw.bad == 0 and tr.bad == 0, f"{msg}: {tw.bad} write and {tr.bad} read sets mismatched"
    row_ok, out_ok = taint(N, T, gw, ref["widx"][0, 0], tw.flagged_at, gr, ref["ridx"][0, 0],
                           tr.flagged_at)
    assert np.all(close(Mg[row_ok], M_ref[row_ok])), f"{msg}: table rows differ"
    assert np.all(close(og[out_ok], o_ref[out_ok])), f"{msg}: outputs differ"
    return E2ETally(streams=1, w=tw, r=tr, flagged_streams=int(bool(tw.flagged or tr.flagged)),
                    outs=T, outs_compared=int(out_ok.sum()), rows=N,
                    rows_compared=int(row_ok.sum()))


def ignored_events(lists, N, sink0, seed, frac=0.1):
    """Slot lists with about `frac` of the events given a slot outside
    [0, N) (-1, -2^31, 2^31 - 1, N or N + 7), which the scans ignore, and the
    oracle's equivalent: those writes write the distinct sink slots
    sink0 + rank and those reads read slot sink0 with weight 0, which
    changes rows [sink0, N) only.  Every valid slot must be below sink0 and
    N - sink0 >= W.  `lists` maps widx, wwt, ridx, rwt to CPU tensors;
    returns (gpu_lists, oracle_lists, {"widx": mask, "ridx": mask})."""
    import torch
    g = torch.Generator().manual_seed(seed)
    bad_vals = torch.tensor([-1, -(1 << 31), (1 << 31) - 1, N, N + 7], dtype=torch.int32)
    gpu, ref, masks = dict(lists), dict(lists), {}
    for key, wkey in (("widx", "wwt"), ("ridx", "rwt")):
        idx = lists[key]
        assert int(idx.max()) < sink0
        mask = torch.rand(idx.shape, generator=g) < frac
        bad = bad_vals[torch.randint(0, len(bad_vals), idx.shape, generator=g)]
        gpu[key] = torch.where(mask, bad, idx).contiguous()
        if key == "widx":
            k = idx.shape[-1]
            assert N - sink0 >= k
            sink = (sink0 + torch.arange(k, dtype=torch.int32)).expand(idx.shape)
            ref[key] = torch.where(mask, sink, idx).contiguous()
        else:
            ref[key] = torch.where(mask, torch.full_like(idx, sink0), idx).contiguous()
            ref[wkey] = torch.where(mask, torch.zeros_like(lists[wkey]), lists[wkey]).contiguous()
        masks[key] = mask
    return gpu, ref, masks
