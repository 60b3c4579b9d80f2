"""sdm_score_topk_noalloc (no workspace, the library's static scratch) against
sdm_score_topk (caller workspace), through the C ABI (run on an MI355X).

Both run the same kernels, so the slot lists and weights must be identical bit
for bit.  Two calls in a row on one device, the second smaller than the first,
check that the scratch left by one call does not leak into the next; an fp32
call needs no scratch at all.
"""
import ctypes

import pytest
import torch

import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_addressed_linear_amd as sdm
    sdm.lib()
    return torch.device("cuda:0")


def outputs(B, H, T, W, R, dev):
    return (torch.full((B, H, T, W), -1, dtype=torch.int32, device=dev),
            torch.full((B, H, T, W), float("nan"), device=dev),
            torch.full((B, H, T, R), -1, dtype=torch.int32, device=dev),
            torch.full((B, H, T, R), float("nan"), device=dev))


def noalloc_call(x, W, R, out):
    """sdm_score_topk_noalloc called directly through ctypes."""
    import sparse_addressed_linear_amd as sdm
    B, H, T, d_k = x["q"].shape
    n_sub = x["subkeys"].shape[2]
    d = sdm.Dims(B, H, T, d_k, n_sub, 1, W, R)
    dt = 1 if x["q"].dtype == torch.bfloat16 else 0
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = sdm.lib().sdm_score_topk_noalloc(
        ctypes.byref(d), dt, p(x["q"]), p(x["k"]), p(x["subkeys"]), *(p(t) for t in out),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, sdm.lib().sdm_status_str(rc).decode()


@pytest.mark.parametrize("cases", [
    # (workload, overrides): the second call of each pair is smaller
    (("long", dict(B=1, H=16, T=37)), ("large", dict(B=2, H=3, T=29))),
    (("large", dict(B=2, H=8, T=70)), ("mid", dict(B=1, H=2, T=19))),
    (("tiny", dict(B=2, H=2, T=21)), ("tiny", dict(B=1, H=1, T=5))),
])
def test_noalloc_equals_workspace_call(dev, cases):
    import sparse_addressed_linear_amd as sdm
    for name, kw in cases:
        wl = synth.WORKLOADS[name].with_(**kw)
        say(f"case: score_topk_noalloc {name} {kw} d_k={wl.d_k} n_sub={wl.n_sub} W={wl.W}")
        x = synth.make_inputs(wl, device=dev, with_m0=False)
        ref = sdm.score_topk(x["q"], x["k"], x["subkeys"], wl.W, wl.R)
        out = outputs(wl.B, wl.H, wl.T, wl.W, wl.R, dev)
        noalloc_call(x, wl.W, wl.R, out)
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b)
        # and through the binding of the same name
        out2 = outputs(wl.B, wl.H, wl.T, wl.W, wl.R, dev)
        sdm.score_topk_noalloc(x["q"], x["k"], x["subkeys"], wl.W, wl.R, out=out2)
        torch.cuda.synchronize()
        for a, b in zip(out2, ref):
            assert torch.equal(a, b)
