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
          7: "SDM_ERR_WORKSPACE"}
EXPORTS = ("sdm_score_topk", "sdm_score_topk_workspace_size", "sdm_scan",
           "sdm_scan_workspace_size", "sdm_gdn_scan", "sdm_status_str", "sdm_version")


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
        L.sdm_score_topk_workspace_size.argtypes = [PD, I32]
        L.sdm_score_topk_workspace_size.restype = SZ
        L.sdm_scan.argtypes = [PD, I32, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.sdm_scan.restype = ctypes.c_int
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


def _check(fn, rc):
    if rc != 0:
        raise SdmError(fn, rc)


def score_topk(qp, kp, subkeys, W, R, out=None, workspace=None, stream=None):
    """Product-key addressing.  qp, kp: [B,H,T,d_k]; subkeys: [H,2,n_sub,d_k/2]
    (all fp32 or all bf16).  Returns (widx, wwt, ridx, rwt): [B,H,T,W] int32,
    fp32 and [B,H,T,R] int32, fp32, in rank order.  ``workspace`` (uint8 device
    tensor) is allocated here when not given or too small."""
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
    d = Dims(B, H, T, d_k, n_sub, 1, W, R)
    need = int(lib().sdm_score_topk_workspace_size(ctypes.byref(d), dt))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wsp = _dev(workspace, "workspace") if need else ctypes.c_void_p(0)
    rc = lib().sdm_score_topk(ctypes.byref(d), dt, _dev(qp, "qp"), _dev(kp, "kp"),
                              _dev(subkeys, "subkeys"), _dev(widx, "widx", torch.int32),
                              _dev(wwt, "wwt", torch.float32), _dev(ridx, "ridx", torch.int32),
                              _dev(rwt, "rwt", torch.float32), wsp, ctypes.c_size_t(need),
                              _stream(stream))
    _check("sdm_score_topk", rc)
    return widx, wwt, ridx, rwt


def score_topk_workspace_size(B, H, T, d_k, n_sub, W, R, bf16=True):
    d = Dims(B, H, T, d_k, n_sub, 1, W, R)
    return int(lib().sdm_score_topk_workspace_size(ctypes.byref(d), SDM_BF16 if bf16 else SDM_F32))


def scan_workspace_size(B, H, T, N, d_v, W, R):
    n_sub = int(round(N ** 0.5))
    d = Dims(B, H, T, 2, n_sub, d_v, W, R)
    return int(lib().sdm_scan_workspace_size(ctypes.byref(d)))


def scan(M, widx, wwt, ridx, rwt, v, alpha, beta, out=None, workspace=None, stream=None):
    """Sparse gated-delta scan; M [B,H,N,d_v] fp32 is updated in place.
    Returns out [B,H,T,d_v] fp32."""
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
    d = Dims(B, H, T, 2, n_sub, d_v, W, R)
    need = int(lib().sdm_scan_workspace_size(ctypes.byref(d)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=M.device)
    wsp = _dev(workspace, "workspace") if need else ctypes.c_void_p(0)
    rc = lib().sdm_scan(ctypes.byref(d), dt, _dev(M, "M", torch.float32),
                        _dev(widx, "widx", torch.int32), _dev(wwt, "wwt", torch.float32),
                        _dev(ridx, "ridx", torch.int32), _dev(rwt, "rwt", torch.float32),
                        _dev(v, "v"), _dev(alpha, "alpha", torch.float32),
                        _dev(beta, "beta", torch.float32), _dev(out, "out", torch.float32),
                        wsp, ctypes.c_size_t(need), _stream(stream))
    _check("sdm_scan", rc)
    return out


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
    rc = lib().sdm_gdn_scan(B, H, T, d_k, d_v, dt, _dev(S, "S", torch.float32), _dev(k, "k"),
                            _dev(q, "q"), _dev(v, "v"), _dev(alpha, "alpha", torch.float32),
                            _dev(beta, "beta", torch.float32), _dev(out, "out", torch.float32),
                            _stream(stream))
    _check("sdm_gdn_scan", rc)
    return out
