"""Raven-style routed slots with selective decay -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product library never touches it and shares no code
with it.  numpy, fp64 unless stated.

Follows the Spanish page "Resumen Tecnico: Raven", section 2.2 ("La
Arquitectura Raven"), on a table of M slots (rows of width d):

  router   m = sigmoid(z_t) over the M slots; keep the K largest, zero the rest;
           normalise the kept ones so that they sum to one: r_i = m_i / sum m
  decay    only on routed slots: gamma_i = exp(a_t * r_i)  (a_t <= 0),
           S_t[i] = gamma_i * S_{t-1}[i] + (1 - gamma_i) * u_t,
           every other slot keeps its row exactly
  read     the same router form on the query side: o_t = sum_i rq_i * S_t[i]
           over the K slots the query routes to, after the write.

Readings where the page is silent or loose:
  * sigmoid is strictly increasing, so the K largest sigmoid scores are the
    K largest logits; ties go to the lower slot index (as everywhere in this
    repository).  Selecting on the logits keeps the choice exact.
  * "normalised" is read as division by the sum of the kept scores (the
    top-K sigmoid-gate normalisation of the MoE router the page cites).
  * the key and value states decay with the same gates (the page writes the
    key state; the value state is its twin), so they are one row [k ; v] and
    u_t = [k_t ; v_t].
  * the page gives no read; the query side is read through the same router.
"""
import numpy as np


def topk_desc(z, K):
    """Indices of the K largest entries of z, largest first, ties to the
    lower index (stable sort on -z)."""
    return np.argsort(-np.asarray(z, np.float64), kind="stable")[:K]


def route(z, K):
    """Router of one token: (slots [K] by rank, normalised gates r [K])."""
    idx = topk_desc(z, K)
    m = 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)[idx]))
    return idx, m / m.sum()


def route_tokens(zk, zq, a, K):
    """Router of every token: zk, zq [B,H,T,M] logits, a [B,H,T] decay.
    Returns widx [B,H,T,K] int32, wcoef = 1 - exp(a*r) [B,H,T,K] (the write
    strength of each routed slot), ridx [B,H,T,K] int32, rwt [B,H,T,K]."""
    B, H, T, M = zk.shape
    out = dict(widx=np.empty((B, H, T, K), np.int32), wcoef=np.empty((B, H, T, K)),
               ridx=np.empty((B, H, T, K), np.int32), rwt=np.empty((B, H, T, K)))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                i, r = route(zk[b, h, t], K)
                out["widx"][b, h, t] = i
                out["wcoef"][b, h, t] = -np.expm1(float(a[b, h, t]) * r)
                i, r = route(zq[b, h, t], K)
                out["ridx"][b, h, t] = i
                out["rwt"][b, h, t] = r
    return out


def raven_scan_stream(S, zk, zq, a, u, K):
    """One stream, in place on S [M,d] (float64 copy taken by the caller):
    zk, zq [T,M]; a [T]; u [T,d].  Returns o [T,d]."""
    T = zk.shape[0]
    o = np.empty((T, S.shape[1]))
    for t in range(T):
        i, r = route(zk[t], K)
        g = np.exp(float(a[t]) * r)[:, None]
        S[i] = g * S[i] + (1.0 - g) * np.asarray(u[t], np.float64)[None, :]
        j, rq = route(zq[t], K)
        o[t] = rq @ S[j]
    return o
