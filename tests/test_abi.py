"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before touching HIP."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")


@pytest.fixture(scope="module")
def L():
    import sparse_addressed_linear_amd as sdm
    if not os.path.exists(sdm.LIB_PATH):
        pytest.skip("libsdm.so not built")
    return sdm.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(
        ["sdm_score_topk", "sdm_score_topk_workspace_size", "sdm_pack_subkeys",
         "sdm_score_topk_packed", "sdm_score_topk_noalloc", "sdm_decode_step", "sdm_scan",
         "sdm_scan_workspace_size", "sdm_scan_record",
         "sdm_scan_backward", "sdm_scan_backward_workspace_size", "sdm_score_topk_backward",
         "sdm_score_topk_backward_workspace_size",
         "sdm_route_topk", "sdm_scan_timeparallel", "sdm_scan_timeparallel_workspace_size",
         "sdm_gdn_scan", "sdm_status_str", "sdm_version"])


def test_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.sdm_version().decode().count(".") == 2
    for code in range(9):
        assert L.sdm_status_str(code) != b"unknown status"
    assert L.sdm_status_str(99) == b"unknown status"


def dims(**kw):
    import sparse_addressed_linear_amd as sdm
    base = dict(B=1, H=1, T=4, d_k=32, n_sub=32, d_v=16, W=8, R=8)
    base.update(kw)
    return sdm.Dims(**base)


P = ctypes.c_void_p(4096)  # aligned, never dereferenced: validation fails first


def score(L, d, dt=1, ptr=P, null_at=None, ws=1 << 30, wsp=P):
    args = [ptr] * 7
    if null_at is not None:
        args[null_at] = ctypes.c_void_p(0)
    return L.sdm_score_topk(ctypes.byref(d), dt, *args, wsp, ctypes.c_size_t(ws), None)


def test_score_topk_rejects(L):
    for i in range(7):
        assert score(L, dims(), null_at=i) == 1
    assert L.sdm_score_topk(None, 1, *([P] * 7), P, ctypes.c_size_t(1 << 30), None) == 1
    assert score(L, dims(d_k=31)) == 2          # odd d_k
    assert score(L, dims(W=0)) == 2
    assert score(L, dims(W=1025)) == 2          # W > N
    assert score(L, dims(n_sub=50000)) == 2     # N >= 2^31
    assert score(L, dims(), dt=7) == 3
    assert score(L, dims(n_sub=2048, W=8)) == 4  # kernel limits
    assert score(L, dims(n_sub=40, W=8)) == 4    # n_sub not a multiple of 16
    assert score(L, dims(d_k=40)) == 4          # half not a multiple of 16
    assert score(L, dims(W=33)) == 4            # W > n_sub
    assert score(L, dims(n_sub=256, W=129, R=8)) == 4
    assert score(L, dims(), ptr=ctypes.c_void_p(4100)) == 5


def test_score_topk_workspace_contract(L):
    import sparse_addressed_linear_amd as sdm
    d = dims(B=2, H=8, T=4096, d_k=128, n_sub=1024, W=64, R=64)
    need = L.sdm_score_topk_workspace_size(ctypes.byref(d), 1)
    # bf16: the packed sub-key fragments, 8 heads x 2 halves x 64 tiles x 2 K steps x 1 KB
    assert need == 8 * 2 * 64 * 2 * 1024
    assert L.sdm_score_topk_workspace_size(ctypes.byref(d), 0) == 0  # fp32 needs none
    assert score(L, d, ws=need - 1) == 7
    assert score(L, d, ws=need, wsp=ctypes.c_void_p(0)) == 7
    assert score(L, d, ws=need, wsp=ctypes.c_void_p(4104)) == 5
    assert sdm.score_topk_workspace_size(2, 8, 4096, 128, 1024, 64, 64) == need


def test_pack_and_packed_score_reject_before_any_launch(L):
    d = dims(B=2, H=8, T=64, d_k=128, n_sub=1024, W=64, R=64)
    need = L.sdm_score_topk_workspace_size(ctypes.byref(d), 1)
    pack = lambda d, dt=1, sk=P, ws=need, wsp=P: L.sdm_pack_subkeys(
        ctypes.byref(d), dt, sk, wsp, ctypes.c_size_t(ws), None)
    assert L.sdm_pack_subkeys(None, 1, P, P, ctypes.c_size_t(need), None) == 1
    assert pack(d, sk=ctypes.c_void_p(0)) == 1
    assert pack(d, dt=4) == 3
    assert pack(dims(d_k=40)) == 4
    assert pack(d, sk=ctypes.c_void_p(4100)) == 5
    assert pack(d, ws=need - 1) == 7
    assert pack(d, wsp=ctypes.c_void_p(0)) == 7
    assert pack(d, wsp=ctypes.c_void_p(4104)) == 5
    # fp32 tables need no packing: accepted with no workspace and no launch
    assert pack(d, dt=0, ws=0, wsp=ctypes.c_void_p(0)) == 0

    def packed(d, ws=need, wsp=P, null_at=None):
        args = [P] * 7
        if null_at is not None:
            args[null_at] = ctypes.c_void_p(0)
        return L.sdm_score_topk_packed(ctypes.byref(d), 1, *args, wsp, ctypes.c_size_t(ws), None)
    for i in range(7):
        assert packed(d, null_at=i) == 1
    assert packed(dims(W=33)) == 4
    assert packed(d, ws=need - 1) == 7
    assert packed(d, wsp=ctypes.c_void_p(0)) == 7
    assert packed(d, wsp=ctypes.c_void_p(4104)) == 5


def scan(L, d, dt=0, ptr=P, ws=0, null_at=None):
    args = [ptr] * 9
    if null_at is not None:
        args[null_at] = ctypes.c_void_p(0)
    return L.sdm_scan(ctypes.byref(d), dt, *args, ptr, ctypes.c_size_t(ws), None)


def test_empty_sequence_accepts_null_token_tensors(L):
    z = ctypes.c_void_p(0)
    d = dims(T=0)
    assert L.sdm_score_topk(ctypes.byref(d), 1, z, z, P, z, z, z, z, z, ctypes.c_size_t(0), None) == 0
    assert L.sdm_scan(ctypes.byref(d), 0, P, *([z] * 8), z, ctypes.c_size_t(0), None) == 0
    assert L.sdm_gdn_scan(1, 1, 0, 128, 128, 0, P, *([z] * 6), None) == 0
    assert L.sdm_scan(ctypes.byref(d), 0, z, *([z] * 8), z, ctypes.c_size_t(0), None) == 1


def test_scan_rejects(L):
    for i in range(9):
        assert scan(L, dims(), null_at=i) == 1
    assert scan(L, dims(R=0)) == 2
    assert scan(L, dims(), dt=5) == 3
    assert scan(L, dims(d_v=20)) == 4
    assert scan(L, dims(n_sub=64, W=300)) == 4
    assert scan(L, dims(), ptr=ctypes.c_void_p(4104), ws=1 << 30) == 5


def test_scan_workspace_contract(L):
    import sparse_addressed_linear_amd as sdm
    # a large multi-stream problem spreads each stream over slot partitions
    d = dims(B=8, H=8, T=4096, d_k=128, n_sub=1024, d_v=64, W=64, R=64)
    need = L.sdm_scan_workspace_size(ctypes.byref(d))
    assert need > 0 and need % (8 * 8 * 4096 * 64 * 4) == 0
    assert scan(L, d, ws=need - 1) == 7
    assert sdm.scan_workspace_size(8, 8, 4096, 1 << 20, 64, 64, 64) == need
    assert L.sdm_scan_workspace_size(ctypes.byref(dims(W=0))) == 0


def test_gdn_rejects(L):
    args = [P] * 7
    assert L.sdm_gdn_scan(1, 1, 4, 128, 128, 0, ctypes.c_void_p(0), *args[1:], None) == 1
    assert L.sdm_gdn_scan(0, 1, 4, 128, 128, 0, *args, None) == 2
    assert L.sdm_gdn_scan(1, 1, 4, 128, 128, 9, *args, None) == 3
    assert L.sdm_gdn_scan(1, 1, 4, 64, 128, 0, *args, None) == 4
    assert L.sdm_gdn_scan(1, 1, 4, 128, 128, 0, ctypes.c_void_p(4097), *args[1:], None) == 5


def test_python_binding_requires_device_tensors():
    import torch
    import sparse_addressed_linear_amd as sdm
    if not os.path.exists(sdm.LIB_PATH):
        pytest.skip("libsdm.so not built")
    x = torch.zeros(1, 1, 4, 32)
    C = torch.zeros(1, 2, 32, 16)
    with pytest.raises(ValueError, match="device tensor"):
        sdm.score_topk(x, x, C, 8, 8)


def test_gradient_entry_points_reject_before_any_launch(L):
    d = dims(B=2, H=4, T=64, d_k=128, n_sub=256, d_v=64, W=32, R=32)
    # sdm_scan_record: sdm_scan's checks plus the tape
    rec = lambda d, tape=P, ws=1 << 30: L.sdm_scan_record(
        ctypes.byref(d), 0, *([P] * 9), tape, P, ctypes.c_size_t(ws), None)
    assert rec(d, tape=ctypes.c_void_p(0)) == 1
    assert rec(d, tape=ctypes.c_void_p(4100)) == 5
    assert rec(dims(d_v=20)) == 4
    # sdm_scan_backward: 17 pointers
    need = L.sdm_scan_backward_workspace_size(ctypes.byref(d))
    assert need > 0  # 8 streams spread over slot partitions

    def bwd(d, null_at=None, dt=0, ws=need, wsp=P, ptr=P):
        args = [ptr] * 16
        if null_at is not None:
            args[null_at] = ctypes.c_void_p(0)
        return L.sdm_scan_backward(ctypes.byref(d), dt, *args, wsp, ctypes.c_size_t(ws), None)
    for i in range(16):
        assert bwd(d, null_at=i) == 1, i
    assert bwd(d, dt=3) == 3
    assert bwd(dims(d_v=48)) == 4          # rows must be a power of two
    assert bwd(dims(d_v=512)) == 4
    assert bwd(d, ws=need - 1) == 7
    assert bwd(d, wsp=ctypes.c_void_p(0)) == 7
    assert bwd(d, ptr=ctypes.c_void_p(4100)) == 5
    assert L.sdm_scan_backward_workspace_size(ctypes.byref(dims(d_v=48))) == 0
    z = ctypes.c_void_p(0)
    assert L.sdm_scan_backward(ctypes.byref(dims(T=0)), 0, P, P, *([z] * 14), z,
                               ctypes.c_size_t(0), None) == 0

    # sdm_score_topk_backward: 12 pointers, then the workspace
    sneed = L.sdm_score_topk_backward_workspace_size(ctypes.byref(d))
    assert sneed > 0

    def sbwd(d, null_at=None, dt=1, ptr_at=None, ws=None, wsp=P):
        args = [P] * 12
        if null_at is not None:
            args[null_at] = ctypes.c_void_p(0)
        if ptr_at is not None:
            args[ptr_at] = ctypes.c_void_p(4100)
        return L.sdm_score_topk_backward(ctypes.byref(d), dt, *args, wsp,
                                         ctypes.c_size_t(sneed if ws is None else ws), None)
    for i in range(12):
        assert sbwd(d, null_at=i) == 1, i
    assert sbwd(d, dt=2) == 3
    assert sbwd(dims(n_sub=2048, W=8)) == 4
    assert sbwd(dims(n_sub=256, W=129, R=8)) == 4
    assert sbwd(dims(d_k=31)) == 2
    assert sbwd(dims(d_k=40)) == 4           # halves of 20: not a multiple of 16
    for i in (0, 1, 2, 9, 10, 11):           # read or written 16 bytes a lane
        assert sbwd(d, ptr_at=i) == 5, i
    assert sbwd(d, ws=sneed - 1) == 7
    assert sbwd(d, wsp=ctypes.c_void_p(0)) == 7
    assert sbwd(d, wsp=ctypes.c_void_p(4096 + 16)) == 5   # the workspace is 256-byte aligned
    assert L.sdm_score_topk_backward_workspace_size(ctypes.byref(dims(d_k=40))) == 0
    assert L.sdm_score_topk_backward_workspace_size(ctypes.byref(dims(T=0))) == 0


def test_route_topk_rejects_before_any_launch(L):
    route = lambda B=1, H=1, T=4, M=64, K=8, null_at=None: L.sdm_route_topk(
        B, H, T, M, K, *[ctypes.c_void_p(0) if i == null_at else P for i in range(7)], None)
    for i in range(7):
        assert route(null_at=i) == 1
    assert route(K=65) == 2          # K > M
    assert route(K=0) == 2
    assert route(T=-1) == 2
    assert route(M=16384, K=8) == 4
    assert route(M=256, K=129) == 4
    z = ctypes.c_void_p(0)
    assert L.sdm_route_topk(1, 1, 0, 64, 8, *([z] * 7), None) == 0


def test_scan_timeparallel_rejects_before_any_launch(L):
    d = dims(B=2, H=4, T=64, d_k=128, n_sub=256, d_v=64, W=32, R=32)
    need = L.sdm_scan_timeparallel_workspace_size(ctypes.byref(d))
    # two slot and position buffers (16 bytes per event), one digit count per
    # 4096-event tile and digit (8-bit digits for N = 2^16), the read buffer
    ev = 2 * 4 * 64 * 64
    assert need >= ev * 16 + 2 * 4 * 256 * 4 + 2 * 4 * 64 * 32 * 64 * 4

    def tp(d, null_at=None, dt=0, ws=need, wsp=ctypes.c_void_p(4096), ptr=P):
        args = [ptr] * 9
        if null_at is not None:
            args[null_at] = ctypes.c_void_p(0)
        return L.sdm_scan_timeparallel(ctypes.byref(d), dt, *args, wsp, ctypes.c_size_t(ws), None)
    for i in range(9):
        assert tp(d, null_at=i) == 1, i
    assert tp(d, dt=2) == 3
    assert tp(dims(d_v=48)) == 4
    assert tp(dims(d_v=512)) == 4
    assert tp(d, ws=need - 1) == 7
    assert tp(d, wsp=ctypes.c_void_p(0)) == 7
    assert tp(d, wsp=ctypes.c_void_p(4112)) == 5   # not 256-byte aligned
    assert L.sdm_scan_timeparallel_workspace_size(ctypes.byref(dims(d_v=48))) == 0
    # 2^31 events: places no longer fit int32
    big = dims(B=1, H=1, T=1 << 24, d_k=128, n_sub=256, d_v=64, W=64, R=64)
    assert L.sdm_scan_timeparallel_workspace_size(ctypes.byref(big)) == 0
    assert tp(big) == 4
    ok = dims(B=1, H=1, T=(1 << 24) - 1, d_k=128, n_sub=256, d_v=64, W=64, R=64)
    assert L.sdm_scan_timeparallel_workspace_size(ctypes.byref(ok)) > 0


def test_score_topk_noalloc_rejects_on_the_host(L):
    """Validation before any launch: bad arguments as sdm_score_topk's, and
    sizes whose packed sub-key tables exceed the 16 MiB static scratch."""
    noalloc = lambda d, dt=1, null_at=None: L.sdm_score_topk_noalloc(
        ctypes.byref(d), dt, *[ctypes.c_void_p(0) if i == null_at else P for i in range(7)], None)
    for i in range(7):
        assert noalloc(dims(), null_at=i) == 1
    assert noalloc(dims(d_k=31)) == 2
    assert noalloc(dims(), dt=7) == 3
    assert noalloc(dims(n_sub=2048, W=8)) == 4
    # bf16: 2 KiB per 16 sub-keys per half per 32 elements of a half; 32 heads
    # of 1024 sub-keys with halves of 256 need 32 MiB
    assert noalloc(dims(H=32, d_k=512, n_sub=1024, W=64, R=64)) == 8
    assert L.sdm_score_topk_workspace_size(ctypes.byref(dims(H=32, d_k=512, n_sub=1024, W=64,
                                                              R=64)), 1) == 32 << 20
    # 16 heads of that size fit exactly
    assert L.sdm_score_topk_workspace_size(ctypes.byref(dims(H=16, d_k=512, n_sub=1024, W=64,
                                                              R=64)), 1) == 16 << 20


def test_decode_step_rejects_on_the_host(L):
    """Validation before any launch: addressing arguments as sdm_score_topk's,
    the scan's tensors, v's type, d_v a power of two in [16, 256], the packed
    sub-keys as workspace for bf16 inputs, 16-byte alignment."""
    def step(d, dt=1, vdt=1, null_at=None, ws=P, wsb=1 << 30, m=P):
        args = [P] * 15
        args[6] = m
        if null_at is not None:
            args[null_at] = ctypes.c_void_p(0)
        q, k, sk = args[0:3]
        M, v, al, be, wi, ww, ri, rw, out = args[6:15]
        return L.sdm_decode_step(ctypes.byref(d), dt, q, k, sk, vdt, M, v, al, be, wi, ww, ri,
                                 rw, out, ws, ctypes.c_size_t(wsb), None)
    d = dims(d_v=64)
    for i in (0, 1, 2, 6, 7, 8, 9, 10, 11, 12, 13, 14):
        assert step(d, null_at=i) == 1, i
    assert step(d, dt=5) == 3
    assert step(d, vdt=5) == 3
    assert step(dims(d_v=48)) == 4
    assert step(dims(d_v=512)) == 4
    assert step(d, ws=ctypes.c_void_p(0)) == 7
    assert step(d, wsb=16) == 7
    assert step(d, m=ctypes.c_void_p(4100)) == 5
    # fp32 inputs need no packed tables
    assert step(d, dt=0, ws=ctypes.c_void_p(0), wsb=0, m=ctypes.c_void_p(4100)) == 5
    assert step(dims(d_v=64, T=0), null_at=6) == 0


def test_scan_plan_partitions(L):
    """The scan's slot partitions, read off its workspace (P partial read sums
    of B*H*T*d_v floats when P > 1): 256 B row slices at Large (whole rows,
    P = 4), for Long's 16 streams (P = 8) and for 8 streams of Long's shape
    (P = 16, within (2W+R)/24 partitions); 128 B slices where 256 B ones
    cannot fill the GPU (4 streams of Long's shape, Mid) and for decoding
    (a token's 128 events of one partition would not fit a wave of 256 B
    slices)."""
    def parts(**kw):
        d = dims(**kw)
        return L.sdm_scan_workspace_size(ctypes.byref(d)) / (d.B * d.H * d.T * d.d_v * 4)
    assert parts(B=8, H=8, T=4096, d_k=128, n_sub=1024, d_v=64, W=64, R=64) == 4
    assert parts(B=1, H=16, T=65536, d_k=256, n_sub=1024, d_v=128, W=128, R=128) == 8
    assert parts(B=1, H=8, T=65536, d_k=256, n_sub=1024, d_v=128, W=128, R=128) == 16
    assert parts(B=1, H=4, T=65536, d_k=256, n_sub=1024, d_v=128, W=128, R=128) == 16
    assert parts(B=4, H=4, T=2048, d_k=128, n_sub=256, d_v=64, W=32, R=32) == 8
    assert parts(B=256, H=1, T=1, d_k=128, n_sub=1024, d_v=64, W=64, R=64) == 0
    assert parts(B=4, H=4, T=40, d_k=32, n_sub=32, d_v=128, W=128, R=128) == 8
