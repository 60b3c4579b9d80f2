"""Gradients of the Sparse Delta Memory path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product library never touches it and shares no code
with it.  Everything here is fp64 on the CPU.

The forward it differentiates is the one of the "Sparse Delta Memory" summary
pages (Spanish page "Mecanismo Central", items 2-4; French page "Mecanisme
Central"), in the readings the C oracle takes:

  sigma_r = s1[i_r] + s2[j_r],  s_c[i] = <x_c, C[c][i]>,  slot = i*n_sub + j
  w = softmax(sigma) over the W write slots, r = softmax(rho) over the R reads
  write:  c = beta*w_r,  M_t[s_r] = (1 - c) * (alpha * M_{t-1}[s_r]) + c * v_t
  read:   o_t = sum_r r_r * M_t[ridx_r]           (after the write)

and the initial table M0 is a parameter (Spanish page "Estado Inicial
Aprendido"), so it has a gradient too.  The slot selections are piecewise
constant: the gradient is that of the path with the selected slots held fixed,
so slot lists are inputs here.

Two independent statements of the same gradients:

* ``*_autograd``: the forward written out in torch CPU ops and differentiated
  by autograd -- the definition; small sizes only.
* ``scan_backward`` and ``score_backward``: the adjoint recurrences written out
  by hand in numpy (reverse over time for the scan), usable at full size.  The
  tests pin them to the autograd versions and to finite differences of the
  forward.

Adjoint of one token t (reverse order: the read, then the write):
  read:   dr_r = <dO_t, M_t[ridx_r]>,  dM[ridx_r] += r_r * dO_t
  write:  G_r = dM[s_r];  old_r = M_{t-1}[s_r]
          dc_r = <G_r, v_t - alpha*old_r>,  dw_r = beta*dc_r
          dbeta_t = sum_r w_r*dc_r,  dalpha_t = sum_r (1 - c_r) <G_r, old_r>
          dv_t = sum_r c_r*G_r,  dM[s_r] = (1 - c_r)*alpha*G_r
Adjoint of the softmax and the scores:
  dsigma = w * (dw - <w, dw>);  dx_1 = sum_r dsigma_r C[1][i_r],
  dx_2 = sum_r dsigma_r C[2][j_r];  dC[1][i_r] += dsigma_r x_1, dC[2][j_r] += dsigma_r x_2.
"""
import numpy as np
import torch


def as_f64(a) -> np.ndarray:
    """float64 copy of a numpy array; uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ------------------------------------------------------------ definitions ---

def slot_weights_t(x, C, idx):
    """Softmax weights of selected slots, torch fp64.  x [..., d_k] of one head,
    C [2, n_sub, d_k/2] that head's sub-keys, idx [..., k] slots."""
    n_sub, dh = C.shape[1], C.shape[2]
    s1 = x[..., :dh] @ C[0].T
    s2 = x[..., dh:] @ C[1].T
    sig = torch.gather(s1, -1, idx // n_sub) + torch.gather(s2, -1, idx % n_sub)
    return torch.softmax(sig, -1)


def scan_forward_t(M0, widx, wwt, ridx, rwt, v, alpha, beta):
    """One stream, torch fp64: M0 [N,d_v]; widx/wwt [T,W]; ridx/rwt [T,R]; v [T,d_v];
    alpha, beta [T].  Returns (outputs [T,d_v], final table)."""
    M = M0.clone()
    outs = []
    for t in range(widx.shape[0]):
        s = widx[t]
        c = (beta[t] * wwt[t])[:, None]
        M.index_put_((s,), (1 - c) * (alpha[t] * M[s]) + c * v[t][None, :])
        outs.append((rwt[t][:, None] * M[ridx[t]]).sum(0))
    return torch.stack(outs), M


def loss_t(q, k, C, M0, widx, ridx, v, alpha, beta, dout, dMT):
    """Scalar <o, dout> + <M_T, dMT> of the whole path for one stream (b,h)
    of head C: q, k [T,d_k]; the pairing that the gradients below are of."""
    wwt = slot_weights_t(k, C, widx)
    rwt = slot_weights_t(q, C, ridx)
    out, MT = scan_forward_t(M0, widx, wwt, ridx, rwt, v, alpha, beta)
    return (out * dout).sum() + (MT * dMT).sum()


def path_grads_autograd(q, k, C, M0, widx, ridx, v, alpha, beta, dout, dMT):
    """Gradients of loss_t with respect to q, k, C, M0, v, alpha, beta (numpy
    fp64 in, numpy fp64 out; one stream, small sizes)."""
    T = lambda a: torch.tensor(as_f64(a), dtype=torch.float64, requires_grad=True)
    I = lambda a: torch.tensor(np.asarray(a), dtype=torch.int64)
    xs = [T(a) for a in (q, k, C, M0, v, alpha, beta)]
    L = loss_t(xs[0], xs[1], xs[2], xs[3], I(widx), I(ridx), xs[4], xs[5], xs[6],
               torch.tensor(as_f64(dout)), torch.tensor(as_f64(dMT)))
    g = torch.autograd.grad(L, xs)
    return dict(zip(("q", "k", "C", "M0", "v", "alpha", "beta"), (a.numpy() for a in g)))


def scan_grads_autograd(M0, widx, wwt, ridx, rwt, v, alpha, beta, dout, dMT):
    """Gradients of <o, dout> + <M_T, dMT> of the scan alone (weights as
    inputs) with respect to M0, wwt, rwt, v, alpha, beta; one stream."""
    T = lambda a: torch.tensor(as_f64(a), dtype=torch.float64, requires_grad=True)
    I = lambda a: torch.tensor(np.asarray(a), dtype=torch.int64)
    xs = [T(a) for a in (M0, wwt, rwt, v, alpha, beta)]
    out, MT = scan_forward_t(xs[0], I(widx), xs[1], I(ridx), xs[2], xs[3], xs[4], xs[5])
    L = (out * torch.tensor(as_f64(dout))).sum() + (MT * torch.tensor(as_f64(dMT))).sum()
    g = torch.autograd.grad(L, xs)
    return dict(zip(("M0", "wwt", "rwt", "v", "alpha", "beta"), (a.numpy() for a in g)))


def score_grads_autograd(x, C, idx, dw):
    """Gradients of <softmax weights, dw> with respect to x [T,d_k] and C
    [2,n_sub,d_k/2] of one head; idx [T,k]."""
    xt = torch.tensor(as_f64(x), requires_grad=True)
    Ct = torch.tensor(as_f64(C), requires_grad=True)
    w = slot_weights_t(xt, Ct, torch.tensor(np.asarray(idx), dtype=torch.int64))
    gx, gC = torch.autograd.grad((w * torch.tensor(as_f64(dw))).sum(), [xt, Ct])
    return gx.numpy(), gC.numpy()


# ------------------------------------------------------- adjoint by hand ---

def scan_backward(M0, widx, wwt, ridx, rwt, v, alpha, beta, dout, dMT):
    """Adjoint of the scan for every stream.  Shapes as the scan's ([B,H,...]);
    dout [B,H,T,d_v], dMT [B,H,N,d_v] (or None for zero).  Returns a dict of
    fp64 arrays: dM0 [B,H,N,d_v], dwwt [B,H,T,W], drwt [B,H,T,R], dv [B,H,T,d_v],
    dalpha, dbeta [B,H,T]."""
    B, H, N, d_v = M0.shape
    T, W = widx.shape[2], widx.shape[3]
    R = ridx.shape[3]
    res = dict(dM0=np.empty((B, H, N, d_v)), dwwt=np.empty((B, H, T, W)),
               drwt=np.empty((B, H, T, R)), dv=np.empty((B, H, T, d_v)),
               dalpha=np.empty((B, H, T)), dbeta=np.empty((B, H, T)))
    for b in range(B):
        for h in range(H):
            g = scan_backward_stream(M0[b, h], widx[b, h], wwt[b, h], ridx[b, h], rwt[b, h],
                                     v[b, h], alpha[b, h], beta[b, h], dout[b, h],
                                     None if dMT is None else dMT[b, h])
            for key, val in g.items():
                res[key][b, h] = val
    return res


def scan_backward_stream(M0, widx, wwt, ridx, rwt, v, alpha, beta, dout, dMT=None):
    """One stream: the forward in fp64 keeping each token's pre-write rows
    and post-write read rows, then the reverse sweep."""
    M = as_f64(M0).copy()
    wwt, rwt, v = as_f64(wwt), as_f64(rwt), as_f64(v)
    alpha, beta, dout = as_f64(alpha), as_f64(beta), as_f64(dout)
    T = widx.shape[0]
    old_rows, read_rows = [], []
    for t in range(T):
        s = widx[t]
        old = M[s].copy()
        c = (beta[t] * wwt[t])[:, None]
        M[s] = (1 - c) * (alpha[t] * old) + c * v[t][None, :]
        old_rows.append(old)
        read_rows.append(M[ridx[t]].copy())
    dM = np.zeros_like(M) if dMT is None else as_f64(dMT).copy()
    dwwt = np.empty(wwt.shape)
    drwt = np.empty(rwt.shape)
    dv = np.empty(v.shape)
    dalpha = np.empty(T)
    dbeta = np.empty(T)
    for t in range(T - 1, -1, -1):
        # read of token t (it came after the write)
        r = ridx[t]
        drwt[t] = read_rows[t] @ dout[t]
        # a slot read more than once by one token takes every read's share
        np.add.at(dM, r, rwt[t][:, None] * dout[t][None, :])
        # write of token t
        s = widx[t]
        G = dM[s].copy()
        old = old_rows[t]
        c = beta[t] * wwt[t]
        dc = (G * (v[t][None, :] - alpha[t] * old)).sum(1)
        dwwt[t] = beta[t] * dc
        dbeta[t] = (wwt[t] * dc).sum()
        dalpha[t] = ((1 - c) * (G * old).sum(1)).sum()
        dv[t] = (c[:, None] * G).sum(0)
        dM[s] = ((1 - c) * alpha[t])[:, None] * G
    return dict(dM0=dM, dwwt=dwwt, drwt=drwt, dv=dv, dalpha=dalpha, dbeta=dbeta)


def slot_weights(x, C, idx):
    """Softmax weights of selected slots in numpy fp64 (for score_backward):
    x [..., d_k], C [2,n_sub,d_k/2], idx [..., k]."""
    n_sub, dh = C.shape[1], C.shape[2]
    x, C = as_f64(x), as_f64(C)
    i, j = idx // n_sub, idx % n_sub
    sig = np.einsum("...d,...kd->...k", x[..., :dh], C[0][i]) + \
        np.einsum("...d,...kd->...k", x[..., dh:], C[1][j])
    e = np.exp(sig - sig.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def score_backward(qp, kp, subkeys, widx, ridx, dwwt, drwt, chunk=256):
    """Adjoint of the addressing for every stream: weight gradients dwwt
    [B,H,T,W], drwt [B,H,T,R] to dq, dk [B,H,T,d_k] and dsubkeys [H,2,n_sub,d_k/2]
    (summed over batches, tokens, and the key and query sides).  Weights are
    recomputed in fp64 from the inputs."""
    B, H, T, d_k = qp.shape
    n_sub, dh = subkeys.shape[2], subkeys.shape[3]
    dq = np.empty((B, H, T, d_k))
    dk = np.empty((B, H, T, d_k))
    dC = np.zeros((H, 2, n_sub, dh))
    for h in range(H):
        C = as_f64(subkeys[h])
        for b in range(B):
            for t0 in range(0, T, chunk):
                ts = slice(t0, min(T, t0 + chunk))
                for x_in, idx, dw, dx in ((kp, widx, dwwt, dk), (qp, ridx, drwt, dq)):
                    x = as_f64(x_in[b, h, ts])
                    ix = np.asarray(idx[b, h, ts], dtype=np.int64)
                    w = slot_weights(x, C, ix)
                    g = as_f64(dw[b, h, ts])
                    ds = w * (g - (w * g).sum(-1, keepdims=True))
                    i, j = ix // n_sub, ix % n_sub
                    dx[b, h, ts, :dh] = np.einsum("tk,tkd->td", ds, C[0][i])
                    dx[b, h, ts, dh:] = np.einsum("tk,tkd->td", ds, C[1][j])
                    np.add.at(dC[h, 0], i.reshape(-1),
                              (ds[..., None] * x[:, None, :dh]).reshape(-1, dh))
                    np.add.at(dC[h, 1], j.reshape(-1),
                              (ds[..., None] * x[:, None, dh:]).reshape(-1, dh))
    return dict(dq=dq, dk=dk, dsubkeys=dC)
