"""GPU parity of the HIP path against the CPU oracle (run on an MI355X).

Rules (fixed before any kernel was written):
  * slot sets per token equal the oracle's, except where the oracle's relative
    gap between the k-th and (k+1)-th candidate sum is below 1e-5 (counted);
  * weights, outputs and tables within 1e-5 absolute + 1e-4 relative;
  * the GPU scan fed the oracle's own indices and weights gives the oracle's
    memory table bit for bit (both evaluate the write as the same sequence of
    fp32 roundings) and outputs within tolerance (read sums are added in a
    different order);
  * a slot-set flip is valid only as a swap of near-equal slots, checked in
    fp64 from q', k' and the sub-keys (gpu_util.compare_topk);
  * end to end (GPU addressing + GPU scan against the oracle's addressing +
    the oracle's scan) tables and outputs are within tolerance everywhere
    except the rows a valid write flip touched and the outputs that read them
    (gpu_util.taint); a floor on the compared share keeps this from passing
    vacuously;
  * every stream of every workload is checked, full size included (host
    threads run one single-threaded oracle per stream);
  * nothing the GPU computes is ever an input to the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (E2ETally, close, compare_topk, e2e_stream, ignored_events, np_, say,
                      thread_map)

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


def inject(g, b, h, ref, dev):
    """Replace stream (b,h)'s slot lists and weights by the oracle's."""
    for j, key in enumerate(("widx", "wwt", "ridx", "rwt")):
        g[j][b, h] = torch.from_numpy(ref[key][0, 0]).to(dev)


# ------------------------------------------------------------------ tiny ---

def test_tiny_end_to_end(dev):
    wl = synth.WORKLOADS["tiny"]
    say("case: tiny end to end", wl)
    x = synth.make_inputs(wl, device=dev)
    M, out, g = run_gpu(wl, x)
    h = {k: np_(v) for k, v in x.items()}
    ref = oracle.score_topk(h["q"], h["k"], h["subkeys"], wl.W, wl.R)
    for gi, gw, ri, rw, gp, xs in ((g[0], g[1], ref["widx"], ref["wwt"], ref["wgap"], h["k"]),
                                   (g[2], g[3], ref["ridx"], ref["rwt"], ref["rgap"], h["q"])):
        t = compare_topk(np_(gi), np_(gw), ri, rw, gp, xs, h["subkeys"], msg="tiny")
        say(f"tiny topk: {t.tokens} tokens, {t.flagged} flagged, {t.bad} mismatched")
        assert t.bad == 0 and t.flagged == 0
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

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_score_topk_integer_ties(dev, dtype):
    """Small-integer inputs: every score is exact on both sides, with many
    exact ties, so indices must match the oracle exactly (lowest index wins).
    In fp32 the ties also reach the stage-1 lists' rank-k entries, which then
    send stage 2 to the full (k+1) x (k+1) grid."""
    say(f"case: integer ties, {dtype}")
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
        qb, kb, Cb = (t.to(dtype).to(dev) for t in (q, k, C))
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


@pytest.mark.parametrize("W,R", [(8, 5), (96, 80)], ids=["small grid", "large grid"])
def test_score_topk_tile_groups_with_ragged_ends(dev, W, R):
    """Workgroups take groups of token tiles (8 for pruned grids of at most 5
    keys a lane, 16 for larger ones, while at least 2048 workgroups remain):
    here 16 streams of 16405 tokens, 2051 tiles of 8, so the last group holds 3
    tiles and the last tile 5 tokens.  fp32 inputs are scored in the oracle's
    order: every slot equals the oracle's."""
    wl = synth.WORKLOADS["tiny"].with_(B=2, H=8, T=16405, n_sub=256, W=W, R=R)
    say("case: tile groups with ragged ends", wl)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    widx, wwt, ridx, rwt = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    torch.cuda.synchronize()
    q, k, C = np_(x["q"]), np_(x["k"]), np_(x["subkeys"])
    streams = [(b, h) for b in range(wl.B) for h in range(wl.H)]

    def ref(p):
        b, h = p
        sl = (slice(b, b + 1), slice(h, h + 1))
        return oracle.score_topk(q[sl], k[sl], C[h:h + 1], wl.W, wl.R)

    for (b, h), r in zip(streams, thread_map(ref, streams)):
        assert np.array_equal(np_(widx[b, h]), r["widx"][0, 0]), f"write slots of {(b, h)}"
        assert np.array_equal(np_(ridx[b, h]), r["ridx"][0, 0]), f"read slots of {(b, h)}"
        assert np.all(close(np_(wwt[b, h]), r["wwt"][0, 0])), f"write weights of {(b, h)}"
        assert np.all(close(np_(rwt[b, h]), r["rwt"][0, 0])), f"read weights of {(b, h)}"


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
    ("d_v=128, partitions", dict(B=2, H=2, T=97, n_sub=64, d_v=128, W=64, R=64, seed=10)),
    ("d_v=256, hot, bf16 v", dict(B=1, H=2, T=60, n_sub=32, d_v=256, W=32, R=48, seed=11,
                                  hot=120, v_bf16=True)),
    # 16 streams of d_v = 128 with W = R = 128 take 256 B slices in 8 partitions
    ("256 B slices, 16 streams", dict(B=4, H=4, T=40, n_sub=32, d_v=128, W=128, R=128, seed=18,
                                      hot=600)),
    ("256 B slices, 16 streams, bf16 v, T=1", dict(B=4, H=4, T=1, n_sub=32, d_v=128, W=128,
                                                   R=128, seed=19, v_bf16=True)),
    ("N=33^2, not a power of two", dict(B=2, H=3, T=75, n_sub=33, d_v=64, W=24, R=40, seed=22)),
    ("T=1", dict(B=1, H=1, T=1, n_sub=64, d_v=32, W=4, R=4, seed=7)),
    ("small table, T=1", dict(B=1, H=1, T=1, n_sub=8, d_v=32, W=4, R=4, seed=7)),
])
def test_scan_vs_oracle(dev, label, args):
    check_scan(scan_case(dev, **args), label)


def _partition_hash(x):
    """The scan's slot-partition hash (lowbias32), used here only to build an
    input that piles every event into one partition."""
    x ^= x >> 16
    x = (x * 0x7FEB352D) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 0x846CA68B) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def test_scan_overflow_with_256b_slices(dev):
    """64 streams of d_v = 64 with W = R = 64 take whole 256 B rows in 4
    partitions, 48 register slots per token and partition.  Every slot here
    falls in partition 0, so each token's 128 events overflow the registers
    and every block takes the overflow path: table bit-identical, outputs
    close."""
    import ctypes
    import sparse_addressed_linear_amd as m
    dims = m.Dims(8, 8, 24, 2, 32, 64, 64, 64)
    assert m.lib().sdm_scan_workspace_size(ctypes.byref(dims)) == 4 * 64 * 24 * 64 * 4
    pool = torch.tensor([s for s in range(1024) if ((_partition_hash(s) >> 16) & 3) == 0][:80],
                        dtype=torch.int32)
    d = scan_case(dev, B=8, H=8, T=24, n_sub=32, d_v=64, W=64, R=64, seed=20)
    g = torch.Generator().manual_seed(21)
    n = 8 * 8 * 24
    for key in ("widx", "ridx"):
        pick = torch.stack([pool[torch.randperm(80, generator=g)[:64]] for _ in range(n)])
        d[key] = pick.view(8, 8, 24, 64).contiguous().to(dev)
    check_scan(d, "overflow with 256 B slices")


def test_scans_ignore_slots_outside_the_table(dev):
    """Events whose slot lies outside [0, N) are neither read nor written by
    the sequential or the time-parallel scan.  Against the oracle run with
    those writes sent to sink rows [960, 1024) and those reads given weight
    0: rows [0, 960) bit-identical, the sink rows untouched (still M0),
    outputs close (sequential) or equal (time-parallel)."""
    N, sink0 = 1024, 960
    d = scan_case(dev, B=2, H=2, T=70, n_sub=32, d_v=64, W=16, R=16, seed=16, hot=sink0)
    cpu = {k: d[k].cpu() for k in ("widx", "wwt", "ridx", "rwt")}
    gpu_l, ref_l, masks = ignored_events(cpu, N, sink0, seed=17)
    assert masks["widx"].any() and masks["ridx"].any()
    M_ref = np_(d["M0"]).copy()
    out_ref = oracle.scan(M_ref, *(np_(ref_l[k]) for k in ("widx", "wwt", "ridx", "rwt")),
                          np_(d["v"]), np_(d["alpha"]), np_(d["beta"]))
    g = [gpu_l[k].to(dev) for k in ("widx", "wwt", "ridx", "rwt")]
    M0 = np_(d["M0"])
    for name, fn in (("sequential", sdm().scan), ("time-parallel", sdm().scan_timeparallel)):
        say(f"case: {name} scan with slots outside the table")
        M = d["M0"].clone()
        out = fn(M, *g, d["v"], d["alpha"], d["beta"])
        torch.cuda.synchronize()
        Mg = np_(M)
        assert np.array_equal(Mg[:, :, :sink0].view(np.uint32),
                              M_ref[:, :, :sink0].view(np.uint32)), f"{name}: table differs"
        assert np.array_equal(Mg[:, :, sink0:].view(np.uint32),
                              M0[:, :, sink0:].view(np.uint32)), f"{name}: sink rows touched"
        if name == "sequential":
            assert np.all(close(np_(out), out_ref)), f"{name}: outputs differ"
        else:
            assert np.array_equal(np_(out), out_ref), f"{name}: outputs differ"


def test_scan_table_over_2gib_per_stream(dev):
    """A stream's table past 2^31 bytes (N = 1025^2, d_v = 512: 2.15 GB) is
    scanned with plain 64-bit row addresses instead of 32-bit buffer offsets.
    Half of every token's slots lie in the table's last 4096 rows, past the
    2^31-byte mark; table bit-identical to the oracle's, outputs close."""
    d = scan_case(dev, B=1, H=1, T=24, n_sub=1025, d_v=512, W=32, R=32, seed=13, hot=64)
    N = 1025 * 1025
    g = torch.Generator().manual_seed(14)
    for key, k in (("widx", 32), ("ridx", 32)):
        top = torch.stack([torch.randperm(4096, generator=g)[:k // 2] for _ in range(24)])
        idx = d[key].cpu().clone()
        idx[0, 0, :, : k // 2] = (N - 4096 + top).int()  # the rest stays in [0, 64)
        d[key] = idx.to(dev)
    assert int(d["widx"].max()) * 512 * 4 >= 1 << 31
    check_scan(d, "table over 2 GiB per stream")


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


def full_end_to_end(wl, dev, x, out_floor, label):
    """Every stream of a workload, end to end, at its full size and in the
    benchmark's launch configuration.

    1. The GPU's addressing (twice: identical bits) against the oracle's, every
       token of every stream, both sides.
    2. The GPU scan fed the oracle's own addressing (every stream's lists
       replaced by the oracle's): the oracle's table bit for bit, outputs
       within tolerance.
    3. The GPU's addressing + scan against the oracle's addressing + scan:
       tables and outputs within tolerance outside the positions a valid
       near-tie flip taints; at least `out_floor` of all outputs compared.
    The oracle runs one stream per host thread."""
    S, H = wl.streams, wl.H
    host = {n: np_(x[n]) for n in ("q", "k", "subkeys", "v", "alpha", "beta")}
    g = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    g2 = sdm().score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    torch.cuda.synchronize()
    for a, b2 in zip(g, g2):
        assert torch.equal(a, b2), "addressing is not deterministic"
    del g2
    for ix in (g[0], g[2]):
        assert int(ix.min()) >= 0 and int(ix.max()) < wl.N

    def stream_in(s):
        b, h = divmod(s, H)
        return (slice(b, b + 1), slice(h, h + 1)), b, h

    def addressing(s):
        sl, b, h = stream_in(s)
        return oracle.score_topk(host["q"][sl], host["k"][sl], host["subkeys"][h:h + 1], wl.W,
                                 wl.R)
    say(f"  oracle addressing of {S} streams")
    refs = thread_map(addressing, range(S))
    inj = [torch.from_numpy(np.concatenate([r[key] for r in refs], 0)
                            .reshape(wl.B, wl.H, wl.T, -1)).to(dev)
           for key in ("widx", "wwt", "ridx", "rwt")]
    say("  GPU scans: own addressing, then the oracle's")
    M_e2e = x["m0"].clone()
    out_e2e = sdm().scan(M_e2e, *g, x["v"], x["alpha"], x["beta"])
    M_inj = x["m0"].clone()
    out_inj = sdm().scan(M_inj, *inj, x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    del inj

    def check(s):
        sl, b, h = stream_in(s)
        ref = refs[s]
        M_ref = np_(x["m0"][b, h]).copy()[None, None]
        o_ref = oracle.scan(M_ref, ref["widx"], ref["wwt"], ref["ridx"], ref["rwt"],
                            host["v"][sl], host["alpha"][sl], host["beta"][sl])
        M_ref, o_ref = M_ref[0, 0], o_ref[0, 0]
        Mi = np_(M_inj[b, h])
        ndiff = np.count_nonzero(Mi.view(np.uint32) != M_ref.view(np.uint32))
        assert ndiff == 0, f"{label} ({b},{h}): oracle addressing, {ndiff} table entries differ"
        del Mi
        assert np.all(close(np_(out_inj[b, h]), o_ref)), \
            f"{label} ({b},{h}): oracle addressing, outputs differ"
        gl = [np_(t[b, h]) for t in g]
        return e2e_stream(gl, ref, host["k"][b, h], host["q"][b, h], host["subkeys"][h:h + 1],
                          np_(M_e2e[b, h]), M_ref, np_(out_e2e[b, h]), o_ref,
                          msg=f"{label} ({b},{h})")
    say(f"  oracle scans and comparisons of {S} streams")
    tot = E2ETally()
    for t in thread_map(check, range(S)):
        tot.add(t)
    say(tot.line(f"{label} end to end"))
    assert tot.streams == S
    assert tot.outs_compared >= out_floor * tot.outs, "too few outputs compared"
    assert tot.rows_compared >= 0.99 * tot.rows, "too few table rows compared"
    return tot


def test_mid_end_to_end(dev):
    """All 16 streams of the mid workload, every token."""
    wl = synth.WORKLOADS["mid"]
    say("case: mid end to end", wl)
    x = synth.make_inputs(wl, device=dev)
    full_end_to_end(wl, dev, x, 0.95, "mid")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["large", "long"])
def test_full_size_end_to_end(dev, name):
    """All streams of the N = 2^20 workloads (Large: 64 streams x 4096 tokens,
    Long: 16 x 65536), every token, at full size."""
    wl = synth.WORKLOADS[name]
    say(f"case: {name} end to end, full size", wl)
    x = synth.make_inputs(wl, device=dev)
    full_end_to_end(wl, dev, x, 0.90, name)
    del x
    torch.cuda.empty_cache()


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


@pytest.mark.timeout(900)
def test_gdn_full_size(dev):
    """All 256 streams x 8192 tokens of the dense baseline (one oracle stream
    per host thread)."""
    wl = synth.WORKLOADS["gdn"]
    say("case: gdn full size, all streams", wl)
    x = synth.make_inputs(wl, device=dev)
    S = x["s0"].clone()
    out = sdm().gdn_scan(S, x["k"], x["q"], x["v"], x["alpha"], x["beta"])
    torch.cuda.synchronize()
    host = {n: np_(x[n]) for n in ("k", "q", "v", "alpha", "beta")}
    og, Sg = np_(out), np_(S)

    def check(s):
        b, h = divmod(s, wl.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        S_ref = np.zeros((1, 1, wl.d_v, wl.d_k), np.float32)
        out_ref = oracle.gdn_scan(S_ref, *(host[n][sl] for n in ("k", "q", "v", "alpha", "beta")))
        assert np.all(close(og[sl], out_ref)), (b, h)
        assert np.all(close(Sg[sl], S_ref)), (b, h)
        return 1
    assert sum(thread_map(check, range(wl.streams))) == wl.streams
    say(f"gdn full size: {wl.streams} streams x {wl.T} tokens compared")
