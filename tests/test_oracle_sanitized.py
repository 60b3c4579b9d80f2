"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle is rebuilt with gcc's -fsanitize=address,undefined into a temporary
directory and driven from a child Python process with the sanitizer runtimes
preloaded: addressing (both input types), the scan with repeated and hot
slots, and the dense baseline, on small inputs.  Any report fails the test
(-fno-sanitize-recover makes the child exit non-zero)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import numpy as np
import oracle
import synth
for name in ("tiny", "mid"):
    wl = synth.WORKLOADS[name].with_(B=1, H=2, T=9)
    x = {k: synth.to_numpy(v) for k, v in synth.make_inputs(wl, device="cpu").items()}
    r = oracle.score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
    M = x["m0"].copy()
    oracle.scan(M, r["widx"], r["wwt"], r["ridx"], r["rwt"], x["v"], x["alpha"], x["beta"])
    hot = r["ridx"] % 7  # repeated read slots within a token
    oracle.scan(M, r["widx"], r["wwt"], hot, r["rwt"], x["v"], x["alpha"], x["beta"])
g = synth.WORKLOADS["gdn"].with_(B=1, H=1, T=5)
x = {k: synth.to_numpy(v) for k, v in synth.make_inputs(g, device="cpu").items()}
S = x["s0"].copy()
oracle.gdn_scan(S, x["k"], x["q"], x["v"], x["alpha"], x["beta"])
print("sanitized oracle ok")
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    from oracle import build as ob
    lib = ob.build(force=True, out=str(tmp_path / "libsdm_oracle_san.so"),
                   extra_flags=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                "-fno-omit-frame-pointer", "-g"))
    env = dict(os.environ, SDM_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0", PYTHONPATH=ROOT, CUDA_VISIBLE_DEVICES="",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0 and "sanitized oracle ok" in r.stdout, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
