"""Sparse Delta Memory hot path on MI355X (gfx950).

Thin Python binding over ``libsdm.so`` (the C ABI declared in
``include/sdm.h``): argument marshalling only.  Every step of the path runs in
the library's HIP kernels; torch supplies device memory and the current HIP
stream.  There is no fallback: if the library is missing, every call raises.

    widx, wwt, ridx, rwt = score_topk(qp, kp, subkeys, W, R)
    out = scan(M, widx, wwt, ridx, rwt, v, alpha, beta)      # M updated in place
    out = gdn_scan(S, k, q, v, alpha, beta)                  # S updated in place
"""
import ctypes
import os

import torch

__all__ = ["lib", "score_topk", "score_topk_workspace_size", "scan", "gdn_scan",
           "scan_workspace_size", "SdmError", "LIB_PATH", "Dims"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdm.so")

SDM_F32, SDM_BF16 = 0, 1
STATUS = {0: "SDM_OK", 1: "SDM_ERR_NULL", 2: "SDM_ERR_SHAPE", 3: "SDM_ERR_DTYPE",
          4: "SDM_ERR_UNSUPPORTED", 5: "SDM_ERR_ALIGN", 6: "SDM_ERR_HIP",
          7: "SDM_ERR_WORKSPACE", 8: "SDM_ERR_SCRATCH"}
EXPORTS = ("sdm_score_topk", "sdm_score_topk_workspace_size", "sdm_pack_subkeys",
           "sdm_score_topk_packed", "sdm_score_topk_noalloc", "sdm_decode_step", "sdm_scan",
           "sdm_scan_workspace_size", "sdm_scan_record",
           "sdm_scan_backward", "sdm_scan_backward_workspace_size", "sdm_score_topk_backward",
           "sdm_score_topk_backward_workspace_size",
           "sdm_route_topk", "sdm_scan_timeparallel", "sdm_scan_timeparallel_workspace_size",
           "sdm_gdn_scan", "sdm_status_str", "sdm_version")


class SdmError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} "
                         f"({lib().sdm_status_str(code).decode()})")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "T", "d_k", "n_sub", "d_v", "W", "R")]


_lib = None


def lib():
    """Load libsdm.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        PD = ctypes.POINTER(Dims)
        L.sdm_score_topk.argtypes = [PD, I32, P, P, P, P, P, P, P, P, SZ, P]
        L.sdm_score_topk.restype = ctypes.c_int
        L.sdm_pack_subkeys.argtypes = [PD, I32, P, P, SZ, P]
        L.sdm_pack_subkeys.restype = ctypes.c_int
        L.sdm_score_topk_packed.argtypes = [PD, I32, P, P, P, P, P, P, P, P, SZ, P]
        L.sdm_score_topk_packed.restype = ctypes.c_int
        L.sdm_decode_step.argtypes = [PD, I32, P, P, P, I32, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.sdm_decode_step.restype = ctypes.c_int
        L.sdm_score_topk_noalloc.argtypes = [PD, I32, P, P, P, P, P, P, P, P]
        L.sdm_score_topk_noalloc.restype = ctypes.c_int
        L.sdm_score_topk_workspace_size.argtypes = [PD, I32]
        L.sdm_score_topk_workspace_size.restype = SZ
        L.sdm_scan.argtypes = [PD, I32, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.sdm_scan.restype = ctypes.c_int
        L.sdm_scan_record.argtypes = [PD, I32] + [P] * 11 + [SZ, P]
        L.sdm_scan_record.restype = ctypes.c_int
        L.sdm_scan_backward.argtypes = [PD, I32] + [P] * 17 + [SZ, P]
        L.sdm_scan_backward.restype = ctypes.c_int
        L.sdm_scan_backward_workspace_size.argtypes = [PD]
        L.sdm_scan_backward_workspace_size.restype = SZ
        L.sdm_score_topk_backward.argtypes = [PD, I32] + [P] * 13 + [SZ, P]
        L.sdm_score_topk_backward.restype = ctypes.c_int
        L.sdm_score_topk_backward_workspace_size.argtypes = [PD]
        L.sdm_score_topk_backward_workspace_size.restype = SZ
        L.sdm_scan_timeparallel.argtypes = [PD, I32] + [P] * 10 + [SZ, P]
        L.sdm_scan_timeparallel.restype = ctypes.c_int
        L.sdm_scan_timeparallel_workspace_size.argtypes = [PD]
        L.sdm_scan_timeparallel_workspace_size.restype = SZ
        L.sdm_route_topk.argtypes = [I32] * 5 + [P] * 8
        L.sdm_route_topk.restype = ctypes.c_int
        L.sdm_scan_workspace_size.argtypes = [PD]
        L.sdm_scan_workspace_size.restype = SZ
        L.sdm_gdn_scan.argtypes = [I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P]
        L.sdm_gdn_scan.restype = ctypes.c_int
        L.sdm_status_str.argtypes = [ctypes.c_int]
        L.sdm_status_str.restype = ctypes.c_char_p
        L.sdm_version.argtypes = []
        L.sdm_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _dtype_code(*ts):
    dt = {t.dtype for t in ts}
    if len(dt) != 1:
        raise TypeError(f"tensors must share one element type, got {dt}")
    dt = dt.pop()
    if dt == torch.float32:
        return SDM_F32
    if dt == torch.bfloat16:
        return SDM_BF16
    raise TypeError(f"unsupported element type {dt}")


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _want(t, shape, name, dtype=None):
    """Check a caller-provided tensor's shape (and dtype) before a kernel
    writes or reads it through a raw pointer."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _scratch(nbytes, device, stream=None, have=None):
    """Device scratch of at least nbytes: `have` when big enough, else a new
    uint8 tensor.  A tensor allocated here and used on a stream other than
    the current one is recorded on that stream, so the caching allocator does
    not hand its memory out again before the kernels that use it are done."""
    if have is not None and have.numel() * have.element_size() >= nbytes:
        return have
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)
    return t


def _check(fn, rc):
    if rc != 0:
        raise SdmError(fn, rc)


def pack_subkeys(subkeys, workspace=None, stream=None):
    """Matrix-core copy of the sub-key tables [H,2,n_sub,d_k/2] for
    ``score_topk(..., packed=...)``: a uint8 device tensor, or None for fp32
    tables (nothing to pack)."""
    H, two, n_sub, dh = subkeys.shape
    if two != 2:
        raise ValueError("subkeys must be [H,2,n_sub,d_k/2]")
    dt = _dtype_code(subkeys)
    d = Dims(1, H, 1, 2 * dh, n_sub, 1, 1, 1)
    need = int(lib().sdm_score_topk_workspace_size(ctypes.byref(d), dt))
    if need == 0:
        return None
    workspace = _scratch(need, subkeys.device, stream, workspace)
    rc = lib().sdm_pack_subkeys(ctypes.byref(d), dt, _dev(subkeys, "subkeys"),
                                _dev(workspace, "workspace"), ctypes.c_size_t(need),
                                _stream(stream))
    _check("sdm_pack_subkeys", rc)
    return workspace


def score_topk(qp, kp, subkeys, W, R, out=None, workspace=None, stream=None, packed=None):
    """Product-key addressing.  qp, kp: [B,H,T,d_k]; subkeys: [H,2,n_sub,d_k/2]
    (all fp32 or all bf16).  Returns (widx, wwt, ridx, rwt): [B,H,T,W] int32,
    fp32 and [B,H,T,R] int32, fp32, in rank order.  ``workspace`` (uint8 device
    tensor) is allocated here when not given or too small.  ``packed``, from
    ``pack_subkeys(subkeys)``, skips repacking the sub-key tables."""
    B, H, T, d_k = qp.shape
    if kp.shape != qp.shape or subkeys.dim() != 4 or subkeys.shape[0] != H or \
            subkeys.shape[1] != 2 or subkeys.shape[3] * 2 != d_k:
        raise ValueError("shape mismatch between qp, kp and subkeys")
    n_sub = subkeys.shape[2]
    dt = _dtype_code(qp, kp, subkeys)
    dev = qp.device
    if out is None:
        out = (torch.empty((B, H, T, W), dtype=torch.int32, device=dev),
               torch.empty((B, H, T, W), dtype=torch.float32, device=dev),
               torch.empty((B, H, T, R), dtype=torch.int32, device=dev),
               torch.empty((B, H, T, R), dtype=torch.float32, device=dev))
    widx, wwt, ridx, rwt = out
    _want(widx, (B, H, T, W), "widx")
    _want(wwt, (B, H, T, W), "wwt")
    _want(ridx, (B, H, T, R), "ridx")
    _want(rwt, (B, H, T, R), "rwt")
    d = Dims(B, H, T, d_k, n_sub, 1, W, R)
    need = int(lib().sdm_score_topk_workspace_size(ctypes.byref(d), dt))
    fn = "sdm_score_topk"
    if packed is not None and need:
        if packed.numel() * packed.element_size() < need:
            raise ValueError("packed sub-keys are smaller than these sizes need")
        workspace, fn = packed, "sdm_score_topk_packed"
    elif need:
        workspace = _scratch(need, dev, stream, workspace)
    wsp = _dev(workspace, "workspace") if need else ctypes.c_void_p(0)
    rc = getattr(lib(), fn)(ctypes.byref(d), dt, _dev(qp, "qp"), _dev(kp, "kp"),
                            _dev(subkeys, "subkeys"), _dev(widx, "widx", torch.int32),
                            _dev(wwt, "wwt", torch.float32), _dev(ridx, "ridx", torch.int32),
                            _dev(rwt, "rwt", torch.float32), wsp, ctypes.c_size_t(need),
                            _stream(stream))
    _check(fn, rc)
    return widx, wwt, ridx, rwt


def score_topk_noalloc(qp, kp, subkeys, W, R, out, stream=None):
    """``score_topk`` through sdm_score_topk_noalloc: no workspace, no device
    allocation (the library's static scratch holds the packed sub-keys).
    ``out`` = (widx, wwt, ridx, rwt) must be given, so nothing is allocated
    here either.  Overlapping calls on one device race on that scratch."""
    B, H, T, d_k = qp.shape
    if kp.shape != qp.shape or subkeys.dim() != 4 or subkeys.shape[0] != H or \
            subkeys.shape[1] != 2 or subkeys.shape[3] * 2 != d_k:
        raise ValueError("shape mismatch between qp, kp and subkeys")
    n_sub = subkeys.shape[2]
    dt = _dtype_code(qp, kp, subkeys)
    widx, wwt, ridx, rwt = out
    _want(widx, (B, H, T, W), "widx")
    _want(wwt, (B, H, T, W), "wwt")
    _want(ridx, (B, H, T, R), "ridx")
    _want(rwt, (B, H, T, R), "rwt")
    d = Dims(B, H, T, d_k, n_sub, 1, W, R)
    rc = lib().sdm_score_topk_noalloc(
        ctypes.byref(d), dt, _dev(qp, "qp"), _dev(kp, "kp"), _dev(subkeys, "subkeys"),
        _dev(widx, "widx", torch.int32), _dev(wwt, "wwt", torch.float32),
        _dev(ridx, "ridx", torch.int32), _dev(rwt, "rwt", torch.float32), _stream(stream))
    _check("sdm_score_topk_noalloc", rc)
    return widx, wwt, ridx, rwt


def score_topk_workspace_size(B, H, T, d_k, n_sub, W, R, bf16=True):
    d = Dims(B, H, T, d_k, n_sub, 1, W, R)
    return int(lib().sdm_score_topk_workspace_size(ctypes.byref(d), SDM_BF16 if bf16 else SDM_F32))


def scan_workspace_size(B, H, T, N, d_v, W, R):
    n_sub = int(round(N ** 0.5))
    d = Dims(B, H, T, 2, n_sub, d_v, W, R)
    return int(lib().sdm_scan_workspace_size(ctypes.byref(d)))


def score_topk_backward_workspace_size(B, H, T, d_k, n_sub, W, R):
    d = Dims(B, H, T, d_k, n_sub, 1, W, R)
    return int(lib().sdm_score_topk_backward_workspace_size(ctypes.byref(d)))


def scan(M, widx, wwt, ridx, rwt, v, alpha, beta, out=None, workspace=None, stream=None,
         tape=None):
    """Sparse gated-delta scan; M [B,H,N,d_v] fp32 is updated in place.
    Returns out [B,H,T,d_v] fp32.  With ``tape`` (fp32 [B,H,T,W,d_v]) the
    pre-write row of every write event is recorded there (sdm_scan_record),
    for scan_backward."""
    B, H, N, d_v = M.shape
    n_sub = int(round(N ** 0.5))
    if n_sub * n_sub != N:
        raise ValueError("N must be n_sub^2")
    T, W = widx.shape[2], widx.shape[3]
    R = ridx.shape[3]
    if widx.shape[:2] != (B, H) or ridx.shape[:3] != (B, H, T) or v.shape != (B, H, T, d_v) \
            or alpha.shape != (B, H, T) or beta.shape != (B, H, T) or \
            wwt.shape != widx.shape or rwt.shape != ridx.shape:
        raise ValueError("shape mismatch in scan arguments")
    dt = _dtype_code(v)
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=torch.float32, device=M.device)
    _want(out, (B, H, T, d_v), "out")
    d = Dims(B, H, T, 2, n_sub, d_v, W, R)
    need = int(lib().sdm_scan_workspace_size(ctypes.byref(d)))
    if need:
        workspace = _scratch(need, M.device, stream, workspace)
    wsp = _dev(workspace, "workspace") if need else ctypes.c_void_p(0)
    args = [_dev(M, "M", torch.float32), _dev(widx, "widx", torch.int32),
            _dev(wwt, "wwt", torch.float32), _dev(ridx, "ridx", torch.int32),
            _dev(rwt, "rwt", torch.float32), _dev(v, "v"), _dev(alpha, "alpha", torch.float32),
            _dev(beta, "beta", torch.float32), _dev(out, "out", torch.float32)]
    if tape is None:
        rc = lib().sdm_scan(ctypes.byref(d), dt, *args, wsp, ctypes.c_size_t(need),
                            _stream(stream))
        _check("sdm_scan", rc)
    else:
        if tape.shape != (B, H, T, W, d_v):
            raise ValueError("tape must be [B,H,T,W,d_v]")
        rc = lib().sdm_scan_record(ctypes.byref(d), dt, *args, _dev(tape, "tape", torch.float32),
                                   wsp, ctypes.c_size_t(need), _stream(stream))
        _check("sdm_scan_record", rc)
    return out


def scan_timeparallel(M, widx, wwt, ridx, rwt, v, alpha, beta, out=None, workspace=None,
                      stream=None):
    """The scan evaluated slot by slot (sdm_scan_timeparallel): same arguments
    and results as ``scan``; ``workspace`` (uint8, 256-byte aligned) is
    allocated here when not given or too small."""
    B, H, N, d_v = M.shape
    n_sub = int(round(N ** 0.5))
    T, W = widx.shape[2], widx.shape[3]
    R = ridx.shape[3]
    if widx.shape[:2] != (B, H) or ridx.shape[:3] != (B, H, T) or v.shape != (B, H, T, d_v) \
            or alpha.shape != (B, H, T) or beta.shape != (B, H, T) or \
            wwt.shape != widx.shape or rwt.shape != ridx.shape:
        raise ValueError("shape mismatch in scan_timeparallel arguments")
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=torch.float32, device=M.device)
    _want(out, (B, H, T, d_v), "out")
    d = Dims(B, H, T, 2, n_sub, d_v, W, R)
    need = int(lib().sdm_scan_timeparallel_workspace_size(ctypes.byref(d)))
    workspace = _scratch(max(need, 256), M.device, stream, workspace)
    f32 = torch.float32
    rc = lib().sdm_scan_timeparallel(
        ctypes.byref(d), _dtype_code(v), _dev(M, "M", f32), _dev(widx, "widx", torch.int32),
        _dev(wwt, "wwt", f32), _dev(ridx, "ridx", torch.int32), _dev(rwt, "rwt", f32),
        _dev(v, "v"), _dev(alpha, "alpha", f32), _dev(beta, "beta", f32), _dev(out, "out", f32),
        _dev(workspace, "workspace"), ctypes.c_size_t(need), _stream(stream))
    _check("sdm_scan_timeparallel", rc)
    return out


def scan_backward(M, dM, widx, wwt, ridx, rwt, v, alpha, beta, tape, dout, workspace=None,
                  stream=None):
    """Reverse sweep of the scan.  M: the table the recorded forward left
    (restored to M0 in place); dM: dL/dM_T on entry, dL/dM0 on return (in
    place).  Returns dict dv, dalpha, dbeta, dwwt, drwt (fp32)."""
    B, H, N, d_v = M.shape
    n_sub = int(round(N ** 0.5))
    T, W = widx.shape[2], widx.shape[3]
    R = ridx.shape[3]
    if dM.shape != M.shape or tape.shape != (B, H, T, W, d_v) or dout.shape != (B, H, T, d_v) \
            or widx.shape[:2] != (B, H) or ridx.shape[:3] != (B, H, T) or wwt.shape != widx.shape \
            or rwt.shape != ridx.shape or v.shape != (B, H, T, d_v) or alpha.shape != (B, H, T) \
            or beta.shape != (B, H, T):
        raise ValueError("shape mismatch in scan_backward arguments")
    dev = M.device
    g = dict(dv=torch.empty((B, H, T, d_v), device=dev), dalpha=torch.empty((B, H, T), device=dev),
             dbeta=torch.empty((B, H, T), device=dev), dwwt=torch.empty((B, H, T, W), device=dev),
             drwt=torch.empty((B, H, T, R), device=dev))
    d = Dims(B, H, T, 2, n_sub, d_v, W, R)
    need = int(lib().sdm_scan_backward_workspace_size(ctypes.byref(d)))
    if need:
        workspace = _scratch(need, dev, stream, workspace)
    wsp = _dev(workspace, "workspace") if need else ctypes.c_void_p(0)
    f32 = torch.float32
    rc = lib().sdm_scan_backward(
        ctypes.byref(d), _dtype_code(v), _dev(M, "M", f32), _dev(dM, "dM", f32),
        _dev(widx, "widx", torch.int32), _dev(wwt, "wwt", f32), _dev(ridx, "ridx", torch.int32),
        _dev(rwt, "rwt", f32), _dev(v, "v"), _dev(alpha, "alpha", f32), _dev(beta, "beta", f32),
        _dev(tape, "tape", f32), _dev(dout, "dout", f32), _dev(g["dv"], "dv"),
        _dev(g["dalpha"], "dalpha"), _dev(g["dbeta"], "dbeta"), _dev(g["dwwt"], "dwwt"),
        _dev(g["drwt"], "drwt"), wsp, ctypes.c_size_t(need), _stream(stream))
    _check("sdm_scan_backward", rc)
    return g


def score_topk_backward(qp, kp, subkeys, widx, wwt, ridx, rwt, dwwt, drwt, dsubkeys=None,
                        workspace=None, stream=None):
    """Adjoint of the addressing.  Returns (dq, dk, dsubkeys), fp32; the
    sub-key gradient is added into ``dsubkeys`` when given (else a zeroed one)."""
    B, H, T, d_k = qp.shape
    if kp.shape != qp.shape or subkeys.dim() != 4 or subkeys.shape[0] != H or \
            subkeys.shape[1] != 2 or subkeys.shape[3] * 2 != d_k:
        raise ValueError("shape mismatch between qp, kp and subkeys")
    n_sub = subkeys.shape[2]
    W, R = widx.shape[3], ridx.shape[3]
    for t, shape, name in ((widx, (B, H, T, W), "widx"), (wwt, (B, H, T, W), "wwt"),
                           (dwwt, (B, H, T, W), "dwwt"), (ridx, (B, H, T, R), "ridx"),
                           (rwt, (B, H, T, R), "rwt"), (drwt, (B, H, T, R), "drwt")):
        _want(t, shape, name)
    dt = _dtype_code(qp, kp, subkeys)
    dev = qp.device
    dq = torch.empty((B, H, T, d_k), device=dev)
    dk = torch.empty((B, H, T, d_k), device=dev)
    if dsubkeys is None:
        dsubkeys = torch.zeros(subkeys.shape, dtype=torch.float32, device=dev)
    _want(dsubkeys, subkeys.shape, "dsubkeys", torch.float32)
    d = Dims(B, H, T, d_k, n_sub, 1, W, R)
    f32 = torch.float32
    need = int(lib().sdm_score_topk_backward_workspace_size(ctypes.byref(d)))
    if need:
        workspace = _scratch(need, dev, stream, workspace)
    wsp = _dev(workspace, "workspace") if need else ctypes.c_void_p(0)
    rc = lib().sdm_score_topk_backward(
        ctypes.byref(d), dt, _dev(qp, "qp"), _dev(kp, "kp"), _dev(subkeys, "subkeys"),
        _dev(widx, "widx", torch.int32), _dev(wwt, "wwt", f32), _dev(ridx, "ridx", torch.int32),
        _dev(rwt, "rwt", f32), _dev(dwwt, "dwwt", f32), _dev(drwt, "drwt", f32),
        _dev(dq, "dq", f32), _dev(dk, "dk", f32), _dev(dsubkeys, "dsubkeys", f32), wsp,
        ctypes.c_size_t(need), _stream(stream))
    _check("sdm_score_topk_backward", rc)
    return dq, dk, dsubkeys


def decode_step(M, qp, kp, subkeys, v, alpha, beta, W, R, packed=None, bufs=None,
                stream=None):
    """One decoding step: one new token for every stream, addressing then scan.

    Head-major layouts, so that the tokens of one head (which share its
    sub-key tables) are scored together:  M [H,B,N,d_v] fp32 (updated in
    place), qp, kp [H,B,d_k], v [H,B,d_v], alpha, beta [H,B], subkeys
    [H,2,n_sub,d_k/2].  Stream (b,h) of the sequence layout is row (h,b) here.
    ``packed`` is ``pack_subkeys(subkeys)``; ``bufs`` (a dict, filled on
    first use) keeps the slot lists, output and scan workspace between steps.
    Returns out [H,B,d_v] fp32."""
    H, B, N, d_v = M.shape
    d_k = qp.shape[-1]
    if qp.shape != (H, B, d_k) or kp.shape != qp.shape or v.shape != (H, B, d_v) or \
            alpha.shape != (H, B) or beta.shape != (H, B):
        raise ValueError("shape mismatch in decode_step arguments")
    bufs = {} if bufs is None else bufs
    dev = M.device
    if "idx" not in bufs:
        bufs["idx"] = (torch.empty((1, H, B, W), dtype=torch.int32, device=dev),
                       torch.empty((1, H, B, W), dtype=torch.float32, device=dev),
                       torch.empty((1, H, B, R), dtype=torch.int32, device=dev),
                       torch.empty((1, H, B, R), dtype=torch.float32, device=dev))
        bufs["out"] = torch.empty((H, B, 1, d_v), dtype=torch.float32, device=dev)
        need = scan_workspace_size(H, B, 1, N, d_v, W, R)
        bufs["scan_ws"] = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        need = 0 if packed is not None else score_topk_workspace_size(
            1, H, B, d_k, subkeys.shape[2], W, R, bf16=subkeys.dtype == torch.bfloat16)
        bufs["score_ws"] = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    widx, wwt, ridx, rwt = score_topk(qp.view(1, H, B, d_k), kp.view(1, H, B, d_k), subkeys, W, R,
                                      out=bufs["idx"], workspace=bufs.get("score_ws"),
                                      stream=stream, packed=packed)
    out = scan(M, widx.view(H, B, 1, W), wwt.view(H, B, 1, W), ridx.view(H, B, 1, R),
               rwt.view(H, B, 1, R), v.view(H, B, 1, d_v), alpha.view(H, B, 1),
               beta.view(H, B, 1), out=bufs["out"], workspace=bufs.get("scan_ws"), stream=stream)
    return out.view(H, B, d_v)


def decode_step_fused(M, qp, kp, subkeys, v, alpha, beta, W, R, packed=None, bufs=None,
                      stream=None):
    """decode_step in one launch (sdm_decode_step): the same layouts and
    arguments; tables bit-identical to decode_step's, outputs equal to fp32
    rounding.  ``packed`` is ``pack_subkeys(subkeys)`` (packed here on every
    call when None and the sub-keys are bf16).  Returns out [H,B,d_v] fp32."""
    H, B, N, d_v = M.shape
    d_k = qp.shape[-1]
    n_sub = int(round(N ** 0.5))
    if n_sub * n_sub != N:
        raise ValueError("N must be n_sub^2")
    if qp.shape != (H, B, d_k) or kp.shape != qp.shape or v.shape != (H, B, d_v) or \
            alpha.shape != (H, B) or beta.shape != (H, B) or subkeys.shape != (H, 2, n_sub, d_k // 2):
        raise ValueError("shape mismatch in decode_step_fused arguments")
    bufs = {} if bufs is None else bufs
    dev = M.device
    if "idx" not in bufs:
        bufs["idx"] = (torch.empty((1, H, B, W), dtype=torch.int32, device=dev),
                       torch.empty((1, H, B, W), dtype=torch.float32, device=dev),
                       torch.empty((1, H, B, R), dtype=torch.int32, device=dev),
                       torch.empty((1, H, B, R), dtype=torch.float32, device=dev))
        bufs["out"] = torch.empty((H, B, d_v), dtype=torch.float32, device=dev)
    if packed is None and subkeys.dtype == torch.bfloat16:
        packed = pack_subkeys(subkeys, stream=stream)
    dt = _dtype_code(qp)
    if _dtype_code(kp) != dt or _dtype_code(subkeys) != dt:
        raise ValueError("qp, kp and subkeys must share one dtype")
    d = Dims(1, H, B, d_k, n_sub, d_v, W, R)
    need = int(lib().sdm_score_topk_workspace_size(ctypes.byref(d), dt))
    wsp = _dev(packed, "packed") if need else ctypes.c_void_p(0)
    if need and packed.numel() * packed.element_size() < need:
        raise ValueError("packed sub-keys are smaller than these sizes need")
    widx, wwt, ridx, rwt = bufs["idx"]
    out = bufs["out"]
    # buffers kept from an earlier call must still fit this call's sizes
    _want(widx, (1, H, B, W), "bufs['idx'] write slots")
    _want(wwt, (1, H, B, W), "bufs['idx'] write weights")
    _want(ridx, (1, H, B, R), "bufs['idx'] read slots")
    _want(rwt, (1, H, B, R), "bufs['idx'] read weights")
    _want(out, (H, B, d_v), "bufs['out']")
    rc = lib().sdm_decode_step(
        ctypes.byref(d), dt, _dev(qp, "qp"), _dev(kp, "kp"), _dev(subkeys, "subkeys"),
        _dtype_code(v), _dev(M, "M", torch.float32), _dev(v, "v"),
        _dev(alpha, "alpha", torch.float32), _dev(beta, "beta", torch.float32),
        _dev(widx, "widx", torch.int32), _dev(wwt, "wwt", torch.float32),
        _dev(ridx, "ridx", torch.int32), _dev(rwt, "rwt", torch.float32),
        _dev(out, "out", torch.float32), wsp, ctypes.c_size_t(need), _stream(stream))
    _check("sdm_decode_step", rc)
    return out


def route_topk(zk, zq, a, K, stream=None):
    """Router of routed-slot writes: zk, zq [B,H,T,M] fp32 logits, a [B,H,T]
    fp32 decay.  Returns (widx, wcoef, ridx, rwt), [B,H,T,K] each, for
    ``scan(M, widx, wcoef, ridx, rwt, u, ones, ones)``."""
    B, H, T, M = zk.shape
    if zq.shape != zk.shape or a.shape != (B, H, T):
        raise ValueError("shape mismatch in route_topk arguments")
    dev = zk.device
    widx = torch.empty((B, H, T, K), dtype=torch.int32, device=dev)
    ridx = torch.empty((B, H, T, K), dtype=torch.int32, device=dev)
    wcoef = torch.empty((B, H, T, K), dtype=torch.float32, device=dev)
    rwt = torch.empty((B, H, T, K), dtype=torch.float32, device=dev)
    f32 = torch.float32
    rc = lib().sdm_route_topk(B, H, T, M, K, _dev(zk, "zk", f32), _dev(zq, "zq", f32),
                              _dev(a, "a", f32), _dev(widx, "widx", torch.int32),
                              _dev(wcoef, "wcoef", f32), _dev(ridx, "ridx", torch.int32),
                              _dev(rwt, "rwt", f32), _stream(stream))
    _check("sdm_route_topk", rc)
    return widx, wcoef, ridx, rwt


def gdn_scan(S, k, q, v, alpha, beta, out=None, stream=None):
    """Dense gated-delta scan; S [B,H,d_v,d_k] fp32 is updated in place.
    Returns out [B,H,T,d_v] fp32."""
    B, H, d_v, d_k = S.shape
    T = k.shape[2]
    if k.shape != (B, H, T, d_k) or q.shape != k.shape or v.shape != (B, H, T, d_v) or \
            alpha.shape != (B, H, T) or beta.shape != (B, H, T):
        raise ValueError("shape mismatch in gdn_scan arguments")
    dt = _dtype_code(k, q, v)
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=torch.float32, device=S.device)
    _want(out, (B, H, T, d_v), "out")
    rc = lib().sdm_gdn_scan(B, H, T, d_k, d_v, dt, _dev(S, "S", torch.float32), _dev(k, "k"),
                            _dev(q, "q"), _dev(v, "v"), _dev(alpha, "alpha", torch.float32),
                            _dev(beta, "beta", torch.float32), _dev(out, "out", torch.float32),
                            _stream(stream))
    _check("sdm_gdn_scan", rc)
    return out
