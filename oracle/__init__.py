"""CPU oracle for Sparse Delta Memory -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never touches it, and it shares no
code with the HIP path.

This module is argument marshalling over ``libsdm_oracle.so`` (plain fp32 C,
single-threaded, ``-ffp-contract=off``).  Arrays are numpy; bf16 tensors are
passed as their raw ``uint16`` bit patterns.  Every function here follows the
"Sparse Delta Memory" summary pages (Spanish and French pages, section
"Mecanismo Central" / "Mecanisme Central"): see ``sdm_oracle.c`` for the
statement of each step and of the readings taken where the pages are silent.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

F32, BF16 = 0, 1


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "T", "d_k", "n_sub", "d_v", "W", "R")]


def lib():
    """Load (building first if needed) the oracle library, or the build named
    by SDM_ORACLE_LIB (an instrumented one, for the sanitizer test)."""
    global _lib
    if _lib is None:
        path = os.environ.get("SDM_ORACLE_LIB") or _build.build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        L.sdm_ref_half_scores.argtypes = [P, P, i32, i32, P]
        L.sdm_ref_topk_bruteforce.argtypes = [P, P, i32, i32, P, P]
        L.sdm_ref_two_stage_topk.argtypes = [P, P, i32, i32, P, P, P]
        L.sdm_ref_softmax.argtypes = [P, i32, P]
        L.sdm_ref_score_topk.argtypes = [ctypes.POINTER(Dims), i32, P, P, P, P, P, P, P, P, P]
        L.sdm_ref_scan.argtypes = [ctypes.POINTER(Dims), i32, P, P, P, P, P, P, P, P, P]
        L.sdm_ref_gdn_scan.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P]
        for f in ("sdm_ref_half_scores", "sdm_ref_topk_bruteforce", "sdm_ref_two_stage_topk",
                  "sdm_ref_softmax", "sdm_ref_score_topk", "sdm_ref_scan", "sdm_ref_gdn_scan"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} returned {rc}")


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    """C-contiguous array of the given dtype (no copy when already so)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _elem(a):
    """(array, dtype code) for an element tensor given as float32 or bf16 bits."""
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a), BF16
    return _c(a, np.float32), F32


def half_scores(x, C):
    x = _c(x, np.float32)
    C = _c(C, np.float32)
    n_sub, dh = C.shape
    assert x.shape == (dh,)
    s = np.empty(n_sub, np.float32)
    _check(lib().sdm_ref_half_scores(_p(x), _p(C), n_sub, dh, _p(s)), "half_scores")
    return s


def topk_bruteforce(s1, s2, k):
    s1 = _c(s1, np.float32)
    s2 = _c(s2, np.float32)
    idx = np.empty(k, np.int32)
    sc = np.empty(k, np.float32)
    _check(lib().sdm_ref_topk_bruteforce(_p(s1), _p(s2), s1.size, k, _p(idx), _p(sc)),
           "topk_bruteforce")
    return idx, sc


def two_stage_topk(s1, s2, k):
    s1 = _c(s1, np.float32)
    s2 = _c(s2, np.float32)
    idx = np.empty(k, np.int32)
    sc = np.empty(k, np.float32)
    gap = np.empty(1, np.float32)
    _check(lib().sdm_ref_two_stage_topk(_p(s1), _p(s2), s1.size, k, _p(idx), _p(sc), _p(gap)),
           "two_stage_topk")
    return idx, sc, float(gap[0])


def softmax(score):
    score = _c(score, np.float32)
    w = np.empty_like(score)
    _check(lib().sdm_ref_softmax(_p(score), score.size, _p(w)), "softmax")
    return w


def score_topk(qp, kp, subkeys, W, R):
    """qp, kp: [B,H,T,d_k]; subkeys: [H,2,n_sub,d_k/2] (float32 or bf16 bits).

    Returns dict of widx, wwt, wgap, ridx, rwt, rgap."""
    qp, dt = _elem(qp)
    kp, dt2 = _elem(kp)
    subkeys, dt3 = _elem(subkeys)
    if not (dt == dt2 == dt3):
        raise ValueError("q', k' and sub-keys must share one element type")
    B, H, T, d_k = qp.shape
    assert kp.shape == qp.shape
    n_sub = subkeys.shape[2]
    assert subkeys.shape == (H, 2, n_sub, d_k // 2)
    d = Dims(B, H, T, d_k, n_sub, 1, W, R)
    out = dict(widx=np.empty((B, H, T, W), np.int32), wwt=np.empty((B, H, T, W), np.float32),
               wgap=np.empty((B, H, T), np.float32), ridx=np.empty((B, H, T, R), np.int32),
               rwt=np.empty((B, H, T, R), np.float32), rgap=np.empty((B, H, T), np.float32))
    _check(lib().sdm_ref_score_topk(ctypes.byref(d), dt, _p(qp), _p(kp), _p(subkeys),
                                    _p(out["widx"]), _p(out["wwt"]), _p(out["wgap"]),
                                    _p(out["ridx"]), _p(out["rwt"]), _p(out["rgap"])),
           "score_topk")
    return out


def scan(M, widx, wwt, ridx, rwt, v, alpha, beta):
    """In-place sparse gated-delta scan.  M: float32 [B,H,N,d_v] C-contiguous
    (modified in place); returns out [B,H,T,d_v]."""
    if not (M.dtype == np.float32 and M.flags.c_contiguous):
        raise ValueError("M must be a C-contiguous float32 array (updated in place)")
    B, H, N, d_v = M.shape
    n_sub = int(round(N ** 0.5))
    if n_sub * n_sub != N:
        raise ValueError("N must be a perfect square")
    widx = _c(widx, np.int32)
    ridx = _c(ridx, np.int32)
    wwt = _c(wwt, np.float32)
    rwt = _c(rwt, np.float32)
    v, vdt = _elem(v)
    alpha = _c(alpha, np.float32)
    beta = _c(beta, np.float32)
    T, W = widx.shape[2], widx.shape[3]
    R = ridx.shape[3]
    assert widx.shape == (B, H, T, W) and ridx.shape == (B, H, T, R)
    assert v.shape == (B, H, T, d_v) and alpha.shape == (B, H, T) and beta.shape == (B, H, T)
    out = np.empty((B, H, T, d_v), np.float32)
    d = Dims(B, H, T, 2, n_sub, d_v, W, R)
    _check(lib().sdm_ref_scan(ctypes.byref(d), vdt, _p(M), _p(widx), _p(wwt), _p(ridx), _p(rwt),
                              _p(v), _p(alpha), _p(beta), _p(out)), "scan")
    return out


def gdn_scan(S, k, q, v, alpha, beta):
    """In-place dense gated-delta scan.  S: float32 [B,H,d_v,d_k]; returns out."""
    if not (S.dtype == np.float32 and S.flags.c_contiguous):
        raise ValueError("S must be a C-contiguous float32 array (updated in place)")
    B, H, d_v, d_k = S.shape
    k, dt = _elem(k)
    q, dt2 = _elem(q)
    v, dt3 = _elem(v)
    if not (dt == dt2 == dt3):
        raise ValueError("k, q and v must share one element type")
    T = k.shape[2]
    assert k.shape == (B, H, T, d_k) and q.shape == k.shape and v.shape == (B, H, T, d_v)
    alpha = _c(alpha, np.float32)
    beta = _c(beta, np.float32)
    out = np.empty((B, H, T, d_v), np.float32)
    _check(lib().sdm_ref_gdn_scan(B, H, T, d_k, d_v, dt, _p(S), _p(k), _p(q), _p(v), _p(alpha),
                                  _p(beta), _p(out)), "gdn_scan")
    return out
