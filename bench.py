"""Throughput of the Sparse Delta Memory hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
product-key addressing (sdm_score_topk) for every token of every (b,h) stream,
then the sparse gated-delta scan (sdm_scan) over the same tokens.  The memory
table is carried from step to step (each step continues the recurrence, like
the next chunk of a long sequence; the work per step is identical).

Default workload: the large N = 2^20 configuration (B=8, H=8, T=4096,
d_k=128, n_sub=1024, d_v=64, W=R=64, bf16 projections, fp32 table of 17 GB).

Prints ONE JSON line with the throughput in stream-tokens/s (tokens of all
B*H streams per second), a roofline object for the dominant kernel (the scan)
and a CPU baseline (the oracle on a bounded sample of the same workload).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config large]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SDM tokens/sec (all B·H streams) at N=2^20; scan HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak


def scan_bytes_per_token(wl):
    """Algorithmic scan bytes per stream-token: W rows read and written, R rows
    read, d_v fp32 each."""
    return (2 * wl.W + wl.R) * wl.d_v * 4


def score_bytes_per_token(wl):
    """Algorithmic addressing/stream bytes per stream-token: q', k' read,
    (idx, weight) of W + R slots written by the addressing and read by the
    scan, v and the two gates read, the output row written."""
    e = 2 if wl.bf16 else 4
    return 2 * wl.d_k * e + 2 * (wl.W + wl.R) * 8 + wl.d_v * e + 8 + wl.d_v * 4


def measured_scan_traffic(wl):
    """HBM bytes per scan launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters (copy-calibrated), or None when they were taken on
    another workload or the scan sources have changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"scan_{wl.name}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    csrc = os.path.join(ROOT, "sparse_addressed_linear_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read()
                   for f in ("scan.hip", "scan_kernel.h", "scan_buf.hip", "scan_common.h",
                             "sdm_internal.h"))
    if rec.get("scan_source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec["hbm_bytes_per_launch"]


def host_threads():
    """Host threads for the all-core oracle leg: the CPUs this process may use,
    at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_stream(wl, host, m0, s):
    """The oracle's addressing + scan of stream s from its initial table m0;
    returns (addressing dict, seconds)."""
    import oracle
    b, h = divmod(s, wl.H)
    sl = (slice(b, b + 1), slice(h, h + 1))
    M = m0[None, None].copy()
    t0 = time.perf_counter()
    r = oracle.score_topk(host["q"][sl], host["k"][sl], host["subkeys"][h:h + 1], wl.W, wl.R)
    oracle.scan(M, r["widx"], r["wwt"], r["ridx"], r["rwt"], host["v"][sl], host["alpha"][sl],
                host["beta"][sl])
    return r, time.perf_counter() - t0


def cpu_baseline(wl, host, m0s, n_one, gpu_idx=None):
    """The oracle timed on the host: single-threaded on the first n_one
    streams, then all streams with one single-threaded oracle per stream on a
    pool of host threads (the C oracle releases the GIL, so they run in
    parallel).  With gpu_idx (the GPU's (widx, ridx) as host arrays) it also
    counts the tokens whose slot sets differ from the oracle's."""
    from concurrent.futures import ThreadPoolExecutor
    t_one, tok_one = 0.0, 0
    for s in range(n_one):
        _, dt = _oracle_stream(wl, host, m0s[s], s)
        t_one += dt
        tok_one += wl.T
    n = host_threads()
    S = len(m0s)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as ex:
        res = list(ex.map(lambda s: _oracle_stream(wl, host, m0s[s], s)[0], range(S)))
    wall = time.perf_counter() - t0
    out = {"value": S * wl.T / wall, "unit": "tokens/s", "cores": n, "kind": "oracle",
           "sample": f"all {S} streams x {wl.T} tokens ({S * wl.T} stream-tokens), addressing + "
                     f"scan, one single-threaded fp32 C oracle per stream on {n} host threads",
           "one_core": {"value": tok_one / t_one if t_one else None, "unit": "tokens/s",
                        "cores": 1,
                        "sample": f"{n_one} of {S} streams x all {wl.T} tokens ({tok_one} "
                                  "stream-tokens), single-threaded"}}
    flags = None
    if gpu_idx is not None:
        flags = gap_flag_counts(wl, res, gpu_idx)
    return out, flags


def gap_flag_counts(wl, refs, gpu_idx, gap_tol=1e-5):
    """Tokens whose GPU slot set differs from the oracle's: 'flagged' where the
    oracle's relative gap between the k-th and (k+1)-th candidate is below
    gap_tol (allowed), 'mismatched' otherwise (a failure)."""
    import numpy as np
    cnt = {"tokens_per_side": 0, "write_flagged": 0, "read_flagged": 0, "streams_flagged": 0,
           "mismatched": 0, "streams": len(refs), "gap_tol": gap_tol}
    for s, r in enumerate(refs):
        b, h = divmod(s, wl.H)
        any_flag = False
        for side, key, gkey in (("write", "widx", "wgap"), ("read", "ridx", "rgap")):
            g = np.sort(gpu_idx[key][b, h], -1)
            o = np.sort(r[key][0, 0], -1)
            diff = ~np.all(g == o, -1)
            small = r[gkey][0, 0] < gap_tol
            cnt[f"{side}_flagged"] += int((diff & small).sum())
            cnt["mismatched"] += int((diff & ~small).sum())
            any_flag |= bool((diff & small).any())
        cnt["tokens_per_side"] += wl.T
        cnt["streams_flagged"] += int(any_flag)
    return cnt


def cpu_baseline_gdn(wl, x, n_one):
    """The GDN oracle: single-threaded on n_one streams, then all streams on a
    pool of host threads (one single-threaded oracle per stream)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle
    import synth
    host = {n: synth.to_numpy(x[n]) for n in ("k", "q", "v", "alpha", "beta")}

    def one(s):
        b, h = divmod(s, wl.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        S = np.zeros((1, 1, wl.d_v, wl.d_k), np.float32)
        t0 = time.perf_counter()
        oracle.gdn_scan(S, *(host[n][sl] for n in ("k", "q", "v", "alpha", "beta")))
        return time.perf_counter() - t0
    t_one = sum(one(s) for s in range(n_one))
    n = host_threads()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(one, range(wl.streams)))
    wall = time.perf_counter() - t0
    return {"value": wl.streams * wl.T / wall, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"all {wl.streams} streams x {wl.T} tokens, one single-threaded fp32 C "
                      f"oracle per stream on {n} host threads",
            "one_core": {"value": n_one * wl.T / t_one if t_one else None, "unit": "tokens/s",
                         "cores": 1, "sample": f"{n_one} of {wl.streams} streams x all {wl.T} "
                                               "tokens, single-threaded"}}


def cpu_baseline_decode(wl, x, m0_cpu, n_streams):
    """Oracle (single thread) decoding the same tokens of the first n_streams
    streams: addressing + scan of every step's token."""
    import oracle
    import synth
    tok, t_total = 0, 0.0
    for s in range(n_streams):
        b, h = divmod(s, wl.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        M = synth.to_numpy(m0_cpu[s])[None, None].copy()
        hq, hk, hv, ha, hb = (synth.to_numpy(x[n][sl]) for n in ("q", "k", "v", "alpha", "beta"))
        hc = synth.to_numpy(x["subkeys"][h:h + 1])
        t0 = time.perf_counter()
        for t in range(wl.T):
            ts = slice(t, t + 1)
            r = oracle.score_topk(hq[:, :, ts], hk[:, :, ts], hc, wl.W, wl.R)
            oracle.scan(M, r["widx"], r["wwt"], r["ridx"], r["rwt"], hv[:, :, ts], ha[:, :, ts],
                        hb[:, :, ts])
        t_total += time.perf_counter() - t0
        tok += wl.T
    return {"value": tok / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_streams} of {wl.streams} streams x {wl.T} decoding steps "
                      f"({tok} stream-tokens), addressing + scan per step, single-threaded fp32 C"}


def bench_decode(args, wl, dev):
    """Decoding: each step scores and scans ONE new token of every stream
    (head-major layouts, sub-keys packed once).  The timed K steps are captured
    in one HIP graph, each step reading its own token's inputs, and the graph
    is replayed once: the time is the device time of K back-to-back steps,
    without host launch overhead.  The eager per-step wall time (host launch
    overhead included) is reported beside it."""
    import torch

    import sparse_addressed_linear_amd as sdm
    import synth
    K, Wm = args.steps, args.warmup
    wl = wl.with_(T=max(wl.T, 2 * Wm + 2 * K))
    print(f"[bench] workload {wl.name}: generating inputs on the device", file=sys.stderr,
          flush=True)
    x = synth.make_inputs(wl, device=dev, with_m0=False)
    xd = synth.decode_layout(x)
    M = synth.make_m0(wl, dev, head_major=True)
    n_cpu = min(args.cpu_streams if args.cpu_streams is not None else 8, wl.streams)
    m0_cpu = [M[s % wl.H, s // wl.H].cpu() for s in range(n_cpu)]
    packed = sdm.pack_subkeys(x["subkeys"])
    bufs = {}
    H, B = wl.H, wl.B
    stream = torch.cuda.current_stream()

    def step(t, ev=None):
        if ev:
            ev[0].record(stream)
        idx = sdm.score_topk(xd["q"][t].view(1, H, B, wl.d_k), xd["k"][t].view(1, H, B, wl.d_k),
                             xd["subkeys"], wl.W, wl.R, out=bufs.get("idx"), packed=packed)
        bufs["idx"] = idx
        if ev:
            ev[1].record(stream)
        v = [t_.view(H, B, 1, -1) for t_ in idx]
        bufs["out"] = sdm.scan(M, *v, xd["v"][t].view(H, B, 1, wl.d_v),
                               xd["alpha"][t].view(H, B, 1), xd["beta"][t].view(H, B, 1),
                               out=bufs.get("out"), workspace=bufs.get("ws"))
        if ev:
            ev[2].record(stream)

    need = sdm.scan_workspace_size(H, B, 1, wl.N, wl.d_v, wl.W, wl.R)
    bufs["ws"] = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    t = 0
    for _ in range(Wm):
        step(t)
        t += 1
    torch.cuda.synchronize()
    # eager: per-step events and wall time
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        step(t, evs[i])
        t += 1
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / K
    ms_score = sum(e[0].elapsed_time(e[1]) for e in evs) / K
    ms_scan = sum(e[1].elapsed_time(e[2]) for e in evs) / K
    # graph of K steps (tokens t .. t+K-1), replayed once
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(K):
                step(t + i)
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {K} decoding steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K
    # the same steps fused into one launch each (sdm_decode_step), timed the same way
    fbufs = {}

    def fstep(tk):
        sdm.decode_step_fused(M, xd["q"][tk], xd["k"][tk], xd["subkeys"], xd["v"][tk],
                              xd["alpha"][tk], xd["beta"][tk], wl.W, wl.R, packed=packed,
                              bufs=fbufs)

    fstep(Wm)
    torch.cuda.synchronize()
    gf = torch.cuda.CUDAGraph()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(gf, stream=cap):
            for i in range(K):
                fstep(Wm + i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gf.replay()
    torch.cuda.synchronize()
    ms_fused = (time.perf_counter() - t0) * 1e3 / K
    value = wl.streams / (ms_step * 1e-3)
    sbytes = wl.streams * scan_bytes_per_token(wl)
    achieved = sbytes / (ms_scan * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": "sdm_scan (one token per stream)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "ms": round(ms_scan, 4), "bytes_per_launch": sbytes}
    cpu = None
    if n_cpu:
        print(f"[bench] CPU baseline: oracle on {n_cpu} streams", file=sys.stderr, flush=True)
        cpu = cpu_baseline_decode(wl.with_(T=K), x, m0_cpu, n_cpu)
    cfg = {"workload": wl.name, "B": wl.B, "H": wl.H, "tokens_per_step": 1, "d_k": wl.d_k,
           "d_v": wl.d_v, "n_sub": wl.n_sub, "N": wl.N, "W": wl.W, "R": wl.R, "inputs": "bf16",
           "table": "fp32", "table_GB": round(wl.table_bytes() / 1e9, 2),
           "timing": f"{K} steps in one HIP graph, replayed once"}
    line = {"metric": "SDM decoding: stream-tokens/sec (one token per stream per step) at N=2^20",
            "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
            "warmup": Wm, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": cfg, "roofline": roof, "cpu_baseline": cpu,
            "kernels": {"score_topk_ms": round(ms_score, 5), "scan_ms": round(ms_scan, 5),
                        "eager_wall_ms_per_step": round(eager_ms, 5),
                        "fused_ms_per_step": round(ms_fused, 5),
                        "fused_tokens_per_s": round(wl.streams / (ms_fused * 1e-3), 1)}}
    print(json.dumps(line), flush=True)


def scan_bwd_bytes_per_token(wl):
    """Algorithmic bytes of the reverse scan per stream-token: each read row
    is read from M and read-modified-written in dM (3 row transfers), each
    write row read-modified-written in dM, its tape row read and its M row
    restored (4 row transfers)."""
    return (3 * wl.R + 4 * wl.W) * wl.d_v * 4


def cpu_baseline_train(wl, x, dout, n_streams):
    """Oracle (single thread) training step on the first n_streams streams:
    the C oracle's addressing, then the fp64 gradient oracle's scan forward
    and reverse sweep and its addressing adjoint."""
    import oracle
    import synth
    from oracle import backward as ob
    tok, t_total = 0, 0.0
    for s in range(n_streams):
        b, h = divmod(s, wl.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        m0 = synth.to_numpy(x["m0_cpu"][s])
        hq, hk, hv, ha, hb = (synth.to_numpy(x[n][sl]) for n in ("q", "k", "v", "alpha", "beta"))
        hc = synth.to_numpy(x["subkeys"][h:h + 1])
        hd = synth.to_numpy(dout[sl])
        t0 = time.perf_counter()
        r = oracle.score_topk(hq, hk, hc, wl.W, wl.R)
        g = ob.scan_backward_stream(m0, r["widx"][0, 0], r["wwt"][0, 0], r["ridx"][0, 0],
                                    r["rwt"][0, 0], hv[0, 0], ha[0, 0], hb[0, 0], hd[0, 0])
        ob.score_backward(hq, hk, hc, r["widx"], r["ridx"], g["dwwt"][None, None],
                          g["drwt"][None, None])
        t_total += time.perf_counter() - t0
        tok += wl.T
    return {"value": tok / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_streams} of {wl.streams} streams x all {wl.T} tokens ({tok} "
                      "stream-tokens): C oracle addressing, fp64 numpy scan forward, reverse "
                      "sweep and addressing adjoint, single-threaded"}


def bench_train(args, wl, dev):
    """Training step: addressing, the scan recording its tape, the reverse scan
    (which walks the table back to M0, so every step starts from the same
    table) and the addressing adjoint.  The gradient of M0 and of the sub-keys
    accumulate over the steps, as gradient buffers do; clearing them is the
    optimiser's work and is not timed."""
    import torch

    import sparse_addressed_linear_amd as sdm
    import synth
    print(f"[bench] workload {wl.name} (training step): generating inputs on the device",
          file=sys.stderr, flush=True)
    x = synth.make_inputs(wl, device=dev)
    B, H, T = wl.B, wl.H, wl.T
    n_cpu = args.cpu_streams if args.cpu_streams is not None else \
        {"tiny": 1, "mid": 4, "large": 2, "long": 1}[wl.name]
    n_cpu = min(n_cpu, wl.streams)
    x["m0_cpu"] = [x["m0"][s // H, s % H].cpu() for s in range(n_cpu)]
    gen = torch.Generator(device=dev).manual_seed(wl.seed * 1000 + 99)
    dout = torch.randn((B, H, T, wl.d_v), generator=gen, device=dev)
    M = x["m0"]
    dM = torch.zeros_like(M)
    dC = torch.zeros(x["subkeys"].shape, dtype=torch.float32, device=dev)
    tape = torch.empty((B, H, T, wl.W, wl.d_v), device=dev)
    idx = (torch.empty((B, H, T, wl.W), dtype=torch.int32, device=dev),
           torch.empty((B, H, T, wl.W), device=dev),
           torch.empty((B, H, T, wl.R), dtype=torch.int32, device=dev),
           torch.empty((B, H, T, wl.R), device=dev))
    out = torch.empty((B, H, T, wl.d_v), device=dev)
    need = sdm.scan_workspace_size(B, H, T, wl.N, wl.d_v, wl.W, wl.R)
    work = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    sneed = sdm.score_topk_backward_workspace_size(B, H, T, wl.d_k, wl.n_sub, wl.W, wl.R)
    swork = torch.empty(max(sneed, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev else (lambda i: None)
        rec(0)
        sdm.score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R, out=idx)
        rec(1)
        sdm.scan(M, *idx, x["v"], x["alpha"], x["beta"], out=out, workspace=work, tape=tape)
        rec(2)
        g = sdm.scan_backward(M, dM, *idx, x["v"], x["alpha"], x["beta"], tape, dout)
        rec(3)
        sdm.score_topk_backward(x["q"], x["k"], x["subkeys"], *idx, g["dwwt"], g["drwt"],
                                dsubkeys=dC, workspace=swork)
        rec(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} training steps", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_wall = (time.perf_counter() - t0) * 1e3 / args.steps
    part = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j in range(4)]
    stream_tokens = wl.streams * T
    bbytes = stream_tokens * scan_bwd_bytes_per_token(wl)
    achieved = bbytes / (part[2] * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": "sdm_scan_bwd (sdm_scan_bwd_kernel + sdm_bwd_sum_kernel)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "ms": round(part[2], 4), "bytes_per_launch": bbytes}
    del tape
    cpu = None
    if n_cpu:
        print(f"[bench] CPU baseline: oracle on {n_cpu} streams", file=sys.stderr, flush=True)
        cpu = cpu_baseline_train(wl, x, dout, n_cpu)
    fwd_bytes = stream_tokens * (scan_bytes_per_token(wl) + wl.W * wl.d_v * 4)
    cfg = {"workload": wl.name, "B": B, "H": H, "T": T, "d_k": wl.d_k, "d_v": wl.d_v,
           "n_sub": wl.n_sub, "N": wl.N, "W": wl.W, "R": wl.R,
           "inputs": "bf16" if wl.bf16 else "fp32", "table": "fp32",
           "step": "addressing + recorded scan + reverse scan + addressing adjoint"}
    line = {"metric": "SDM training step (forward + backward) stream-tokens/sec at N=2^20",
            "value": round(stream_tokens / (ms_wall * 1e-3), 1), "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_wall, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": cfg,
            "roofline": roof, "cpu_baseline": cpu,
            "kernels": {"score_topk_ms": round(part[0], 4),
                        "scan_record_ms": round(part[1], 4),
                        "scan_record_GBps": round(fwd_bytes / (part[1] * 1e-3) / 1e9, 1),
                        "scan_backward_ms": round(part[2], 4),
                        "score_topk_backward_ms": round(part[3], 4)}}
    print(json.dumps(line), flush=True)


def bench_raven(args, wl, dev):
    """Routed slots with selective decay: one step is the router of every
    token (write and read sides) and the scan that applies the decaying
    writes and reads on the same table."""
    import torch

    import sparse_addressed_linear_amd as sdm
    import synth
    print(f"[bench] workload {wl.name}: generating inputs on the device", file=sys.stderr,
          flush=True)
    x = synth.make_inputs(wl, device=dev)
    B, H, T = wl.B, wl.H, wl.T
    n_cpu = min(args.cpu_streams if args.cpu_streams is not None else 2, wl.streams)
    m0_cpu = [x["m0"][s // H, s % H].cpu() for s in range(n_cpu)]
    out = torch.empty((B, H, T, wl.d_v), device=dev)
    if args.timeparallel:
        import ctypes
        d = sdm.Dims(B, H, T, 2, wl.n_sub, wl.d_v, wl.W, wl.R)
        need = int(sdm.lib().sdm_scan_timeparallel_workspace_size(ctypes.byref(d)))
        scan_fn = sdm.scan_timeparallel
    else:
        need = sdm.scan_workspace_size(B, H, T, wl.N, wl.d_v, wl.W, wl.R)
        scan_fn = sdm.scan
    work = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        r = sdm.route_topk(x["zk"], x["zq"], x["a"], wl.W)
        if ev:
            ev[1].record(stream)
        scan_fn(x["m0"], *r, x["v"], x["alpha"], x["beta"], out=out, workspace=work)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_wall = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_route = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    ms_scan = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    st = wl.streams * T
    sbytes = st * scan_bytes_per_token(wl)
    rbytes = st * (2 * wl.N * 4 + 4 + 4 * wl.W * 4)  # logits, decay, two (slot, value) lists
    achieved = sbytes / (ms_scan * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": "sdm_scan (sdm_scan_kernel + sdm_partial_sum_kernel)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "ms": round(ms_scan, 4), "bytes_per_launch": sbytes}
    cpu = None
    if n_cpu:
        import numpy as np
        from oracle import raven as rv
        print(f"[bench] CPU baseline: oracle on {n_cpu} streams", file=sys.stderr, flush=True)
        tok, tt = 0, 0.0
        for s_ in range(n_cpu):
            b, h = divmod(s_, H)
            S = synth.to_numpy(m0_cpu[s_]).astype(np.float64)
            zk, zq, a_ = (synth.to_numpy(x[n][b, h]) for n in ("zk", "zq", "a"))
            u = x["v"][b, h].float().cpu().numpy().astype(np.float64)
            t0 = time.perf_counter()
            rv.raven_scan_stream(S, zk, zq, a_, u, wl.W)
            tt += time.perf_counter() - t0
            tok += T
        cpu = {"value": tok / tt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_cpu} of {wl.streams} streams x all {T} tokens ({tok} "
                         "stream-tokens), router + decaying writes + reads, fp64 numpy"}
    cfg = {"workload": wl.name, "B": B, "H": H, "T": T, "M": wl.N, "K": wl.W, "d": wl.d_v,
           "content": "bf16" if wl.bf16 else "fp32", "table": "fp32",
           "table_GB": round(wl.table_bytes() / 1e9, 2)}
    if args.timeparallel:
        cfg["scan"] = "time-parallel"
        roof["kernel"] = "sdm_scan_timeparallel (slot sort, slot segments, read sums)"
    line = {"metric": "Routed selective-decay slots: stream-tokens/sec (router + scan)",
            "value": round(st / (ms_wall * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_wall, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu,
            "kernels": {"route_ms": round(ms_route, 4),
                        "route_GBps": round(rbytes / (ms_route * 1e-3) / 1e9, 1),
                        "scan_ms": round(ms_scan, 4)}}
    print(json.dumps(line), flush=True)


def copy_bandwidth(gib=4.0, reps=5):
    """Context for the scan's fraction of peak: read + write GB/s of a plain
    device-to-device copy of `gib` GiB on this GPU (best of `reps`)."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * n * 4 / (best * 1e-3) / 1e9, 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="large",
                    choices=["tiny", "mid", "large", "long", "gdn", "decode", "raven"])
    ap.add_argument("--timeparallel", action="store_true",
                    help="run the scan in its time-parallel form (sdm_scan_timeparallel)")
    ap.add_argument("--train", action="store_true",
                    help="time a training step (forward with tape + both backward calls)")
    ap.add_argument("--streams", default=None, metavar="B,H",
                    help="override the workload's batch and head counts (e.g. 1,1: one "
                         "stream of its per-stream shape)")
    ap.add_argument("--tokens", type=int, default=None, metavar="T",
                    help="override the workload's tokens per stream")
    ap.add_argument("--cpu-streams", type=int, default=None,
                    help="streams in the oracle CPU-baseline sample (0 = skip)")
    ap.add_argument("--copy-probe", type=float, default=None, metavar="GIB",
                    help="only run 3 plain device copies of GIB GiB (calibrates the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); streams (b,h) "
              "are independent, so more GPUs would each run their share of them.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_addressed_linear_amd as sdm
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe is not None:
        n = int(args.copy_probe * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                          "launches": 3}), flush=True)
        return
    sdm.lib()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.config]
    if args.streams:
        b_, h_ = (int(v) for v in args.streams.split(","))
        wl = wl.with_(B=b_, H=h_)
    if args.tokens:
        wl = wl.with_(T=args.tokens)
    if wl.name == "decode":
        bench_decode(args, wl, dev)
        return
    if wl.keys == "route":
        bench_raven(args, wl, dev)
        return
    if args.train:
        if wl.dense:
            print("bench.py: --train covers the sparse path only", file=sys.stderr)
            sys.exit(2)
        bench_train(args, wl, dev)
        return

    print(f"[bench] workload {wl.name}: generating inputs on the device", file=sys.stderr,
          flush=True)
    x = synth.make_inputs(wl, device=dev)
    dense = wl.dense
    # single-threaded oracle sample sized for roughly 10-20 s of CPU work; the
    # all-core leg then runs every stream
    default_cpu = {"tiny": 1, "mid": 16, "large": 24, "long": 1, "gdn": 16}[wl.name]
    if args.streams or args.tokens:
        default_cpu = 0  # a resized workload: no oracle baseline unless asked
    n_cpu = args.cpu_streams if args.cpu_streams is not None else default_cpu
    n_cpu = min(n_cpu, wl.streams)
    host, m0s = None, None
    if not dense and n_cpu:
        # host copies of every stream's inputs and initial table, taken before
        # the GPU steps modify M
        host = {n: synth.to_numpy(x[n]) for n in ("q", "k", "subkeys", "v", "alpha", "beta")}
        m0s = [synth.to_numpy(x["m0"][s // wl.H, s % wl.H]) for s in range(wl.streams)]

    stream = torch.cuda.current_stream()
    if dense:
        S = x["s0"]
        out = torch.empty((wl.B, wl.H, wl.T, wl.d_v), device=dev)

        def step(ev=None):
            if ev:
                ev[0].record(stream)
            sdm.gdn_scan(S, x["k"], x["q"], x["v"], x["alpha"], x["beta"], out=out)
            if ev:
                ev[1].record(stream)
    else:
        M = x["m0"]
        B, H, T = wl.B, wl.H, wl.T
        idx_bufs = (torch.empty((B, H, T, wl.W), dtype=torch.int32, device=dev),
                    torch.empty((B, H, T, wl.W), device=dev),
                    torch.empty((B, H, T, wl.R), dtype=torch.int32, device=dev),
                    torch.empty((B, H, T, wl.R), device=dev))
        out = torch.empty((B, H, T, wl.d_v), device=dev)
        if args.timeparallel:
            import ctypes
            d = sdm.Dims(B, H, T, 2, wl.n_sub, wl.d_v, wl.W, wl.R)
            need = int(sdm.lib().sdm_scan_timeparallel_workspace_size(ctypes.byref(d)))
            scan_fn = sdm.scan_timeparallel
        else:
            need = sdm.scan_workspace_size(B, H, T, wl.N, wl.d_v, wl.W, wl.R)
            scan_fn = sdm.scan
        work = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

        def step(ev=None):
            if ev:
                ev[0].record(stream)
            sdm.score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R, out=idx_bufs)
            if ev:
                ev[1].record(stream)
            scan_fn(M, *idx_bufs, x["v"], x["alpha"], x["beta"], out=out, workspace=work)
            if ev:
                ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)

    nev = 2 if dense else 3
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = sum(e[0].elapsed_time(e[-1]) for e in evs) / args.steps
    ms_wall = wall * 1e3 / args.steps
    stream_tokens = wl.streams * wl.T
    value = stream_tokens / (ms_wall * 1e-3)

    if dense:
        ms_k = ms_step
        flops = wl.streams * wl.T * (4 * wl.d_v * wl.d_k * 2)  # 4 d_v d_k FMA per token
        achieved = flops / (ms_k * 1e-3) / 1e12
        roof = {"bound": "alu", "kernel": "sdm_gdn_kernel", "achieved": round(achieved, 2),
                "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP32_VALU_PEAK_TFLOPS, 4), "traffic": None,
                "ms": round(ms_k, 4), "work_per_launch": flops}
        kernels = {"gdn_ms": round(ms_k, 4)}
    else:
        ms_score = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
        ms_scan = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
        sbytes = stream_tokens * scan_bytes_per_token(wl)
        achieved = sbytes / (ms_scan * 1e-3) / 1e9
        kname = ("sdm_scan_timeparallel (slot sort, slot segments, read sums)"
                 if args.timeparallel else "sdm_scan (sdm_scan_kernel + sdm_partial_sum_kernel)")
        roof = {"bound": "hbm", "kernel": kname,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": (None if args.timeparallel or args.streams or args.tokens
                            else measured_scan_traffic(wl)),
                "ms": round(ms_scan, 4), "bytes_per_launch": sbytes}
        allb = stream_tokens * (scan_bytes_per_token(wl) + score_bytes_per_token(wl))
        kernels = {"score_topk_ms": round(ms_score, 4), "scan_ms": round(ms_scan, 4),
                   "step_GBps_all_traffic": round(allb / (ms_step * 1e-3) / 1e9, 1),
                   "model_tokens_per_s": round(wl.B * wl.T / (ms_wall * 1e-3), 1),
                   "copy_GBps_measured": copy_bandwidth()}

    cpu, flags = None, None
    if n_cpu:
        print(f"[bench] CPU baseline: oracle on {n_cpu} streams single-threaded, then all "
              f"{wl.streams} streams on {host_threads()} threads", file=sys.stderr, flush=True)
        if dense:
            cpu = cpu_baseline_gdn(wl, x, n_cpu)
        else:
            gidx = {"widx": synth.to_numpy(idx_bufs[0]), "ridx": synth.to_numpy(idx_bufs[2])}
            cpu, flags = cpu_baseline(wl, host, m0s, n_cpu, gidx)

    cfg = {"workload": wl.name, "B": wl.B, "H": wl.H, "T": wl.T, "d_k": wl.d_k, "d_v": wl.d_v}
    if args.timeparallel:
        cfg["scan"] = "time-parallel"
    if not dense:
        cfg.update({"n_sub": wl.n_sub, "N": wl.N, "W": wl.W, "R": wl.R,
                    "inputs": "bf16" if wl.bf16 else "fp32", "table": "fp32",
                    "table_GB": round(wl.table_bytes() / 1e9, 2)})
    line = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_wall, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu,
            "kernels": kernels, "ms_per_step_events": round(ms_step, 4)}
    if flags is not None:
        line["gap_flagged"] = flags
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
