"""Backward pass of the token recurrence (reverse mode), fp64. TEST INFRASTRUCTURE, like the
rest of this package; nothing in the HIP library computes it yet.

The forward is the recurrence of ``recurrent`` (the Muir abstract's order: decay the state,
predict for the incoming key, erase the prediction under the value-channel gate, write, then
the matched-filter read of the openai-hub page's readout section). For one (batch, head),
with q_hat = r * g * q and b = w * v:

    S- = Diag(a_t) S,   p_t = S-^T k_t,   u_t = b_t - e_t * p_t,   S = S- + k_t u_t^T,
    o_t = S^T q_hat_t.

The loss whose gradients are returned is L = sum(o * do) + sum(S_T * dS_T) for given upstream
gradients do [B,T,H,dv] and dS_T [B,H,dk,dv]. Three forms, each a function of the same
arguments returning the same dictionary of gradients (q, k, v, a, g, e, w, r, s0, and the
log-decay gradient la = a * dL/da):

  * ``grads_autograd``  the definition: torch autograd through a plain fp64 torch version of
                        the forward (small inputs);
  * ``grads_adjoint``   the reverse recurrence written out token by token (numpy), from the
                        adjoint lambda_t = dL/dS_t:
                            mu = lambda + q_hat_t do_t^T            (the read of token t)
                            du_t = mu^T k_t                          (gradient of u_t)
                            dp_t = -e_t * du_t,   de_t = -p_t * du_t,   db_t = du_t
                            dk_t = mu u_t + S-_t dp_t,   dq_hat_t = S_t do_t
                            da_t = rowsum(S_{t-1} * (mu + k_t dp_t^T))
                            lambda <- Diag(a_t) (mu + k_t dp_t^T)
  * ``grads_chunked``   the same gradients from chunk-level products (numpy): per chunk, in
                        reverse, the transposed triangular system per value column,
                            (I + M^T Diag(e_j)) dU_j = (K*beta) lambda_C + P^T dO,
                        the adjoint carry lambda_0 = Diag(gamma_C) lambda_C + (Qh*gamma)^T dO
                        + (K*gamma)^T dP, the decayed key and query products for dq_hat and
                        dk, and the log-decay gradient from the identity
                            la_tau = sum_{t >= tau} [q_hat * dq_hat + k * dk_read - k * dk_write]_t
                                     + rowsum(S_C * lambda_C).
                        Decays here are plain products inside the chunk (fp64, test sizes).

Chunk notation as in the forward: gamma_t = product of a from the chunk start through t,
Gamma_{t,s} = product over s < tau <= t, beta_t = product over t < tau <= chunk end,
M_{ts} = sum_i k_ti Gamma_tsi k_si (s < t), P_{ts} = sum_i q_hat_ti Gamma_tsi k_si (s <= t).
"""
from __future__ import annotations

import numpy as np

NAMES = ("q", "k", "v", "a", "g", "e", "w")

__all__ = ["grads_autograd", "grads_adjoint", "grads_chunked", "grads_c", "loss"]


def _heads(x, b, h):
    return np.asarray(x, dtype=np.float64)[b, :, h, :]


def loss(q, k, v, a, g, e, w, r, s0, do, dS):
    """L = sum(o * do) + sum(S_T * dS), from the forward recurrence in numpy (fp64)."""
    B, T, H, dk = np.shape(q)
    total = 0.0
    for b in range(B):
        for h in range(H):
            o, S = _forward_head(*[_heads(x, b, h) for x in (q, k, v, a, g, e, w)],
                                 np.asarray(r, np.float64)[h],
                                 np.zeros((dk, np.shape(v)[-1])) if s0 is None else np.asarray(s0, np.float64)[b, h])
            total += float(np.sum(o * _heads(do, b, h))) + float(np.sum(S * np.asarray(dS, np.float64)[b, h]))
    return total


def _forward_head(q, k, v, a, g, e, w, r, s0, keep=False):
    """One head's forward: o [T,dv] and S_T; with keep, also every S_{t-1}, p_t and u_t."""
    T = q.shape[0]
    qh, bv = r * g * q, w * v
    S = s0.copy()
    o = np.zeros((T, v.shape[1]))
    prev, ps, us = [], [], []
    for t in range(T):
        prev.append(S)
        Sm = a[t][:, None] * S
        p = Sm.T @ k[t]
        u = bv[t] - e[t] * p
        S = Sm + np.outer(k[t], u)
        o[t] = S.T @ qh[t]
        ps.append(p)
        us.append(u)
    if keep:
        return o, S, prev, np.array(ps), np.array(us)
    return o, S


def _empty(q, v, r, s0):
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    out = {n: np.zeros((B, T, H, dk if n in ("q", "k", "a", "g") else dv)) for n in NAMES}
    out["la"] = np.zeros((B, T, H, dk))
    out["r"] = np.zeros((H, dk))
    out["s0"] = np.zeros((B, H, dk, dv))
    return out


def _finish(out, b, h, q, g, r, dqh):
    """q_hat = r * g * q: its gradient into dq, dg and dr."""
    out["q"][b, :, h] = r * g * dqh
    out["g"][b, :, h] = r * q * dqh
    out["r"][h] += np.sum(g * q * dqh, axis=0)


def grads_autograd(q, k, v, a, g, e, w, r, s0, do, dS):
    """Gradients by torch autograd through the fp64 forward (plain PyTorch CPU ops)."""
    import torch
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    out = _empty(q, v, r, s0)
    for b in range(B):
        for h in range(H):
            xs = {n: torch.tensor(_heads(x, b, h), requires_grad=True)
                  for n, x in zip(NAMES, (q, k, v, a, g, e, w))}
            rh = torch.tensor(np.asarray(r, np.float64)[h], requires_grad=True)
            S = torch.tensor(np.zeros((dk, dv)) if s0 is None else np.asarray(s0, np.float64)[b, h],
                             requires_grad=True)
            S_init = S
            qh = rh * xs["g"] * xs["q"]
            bv = xs["w"] * xs["v"]
            L = torch.zeros((), dtype=torch.float64)
            dot = torch.tensor(_heads(do, b, h))
            for t in range(T):
                Sm = xs["a"][t][:, None] * S
                p = Sm.T @ xs["k"][t]
                u = bv[t] - xs["e"][t] * p
                S = Sm + torch.outer(xs["k"][t], u)
                L = L + torch.dot(S.T @ qh[t], dot[t])
            L = L + torch.sum(S * torch.tensor(np.asarray(dS, np.float64)[b, h]))
            gr = torch.autograd.grad(L, [xs[n] for n in NAMES] + [rh, S_init])
            for n, gn in zip(NAMES, gr[:7]):
                out[n][b, :, h] = gn.numpy()
            out["r"][h] += gr[7].numpy()
            out["s0"][b, h] = gr[8].numpy()
            out["la"][b, :, h] = out["a"][b, :, h] * _heads(a, b, h)
    return out


def grads_adjoint(q, k, v, a, g, e, w, r, s0, do, dS):
    """Gradients by the token-by-token reverse recurrence (see the module docstring)."""
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    out = _empty(q, v, r, s0)
    for b in range(B):
        for h in range(H):
            qb, kb, vb, ab, gb, eb, wb = [_heads(x, b, h) for x in (q, k, v, a, g, e, w)]
            rh = np.asarray(r, np.float64)[h]
            S0 = np.zeros((dk, dv)) if s0 is None else np.asarray(s0, np.float64)[b, h]
            o, S_T, prev, ps, us = _forward_head(qb, kb, vb, ab, gb, eb, wb, rh, S0, keep=True)
            qh = rh * gb * qb
            dob = _heads(do, b, h)
            lam = np.asarray(dS, np.float64)[b, h].copy()
            dqh = np.zeros((T, dk))
            for t in range(T - 1, -1, -1):
                Sm = ab[t][:, None] * prev[t]
                St = Sm + np.outer(kb[t], us[t])
                mu = lam + np.outer(qh[t], dob[t])
                du = mu.T @ kb[t]
                dp = -eb[t] * du
                out["v"][b, t, h] = wb[t] * du
                out["w"][b, t, h] = vb[t] * du
                out["e"][b, t, h] = -ps[t] * du
                out["k"][b, t, h] = mu @ us[t] + Sm @ dp
                dqh[t] = St @ dob[t]
                dSm = mu + np.outer(kb[t], dp)
                out["a"][b, t, h] = np.sum(prev[t] * dSm, axis=1)
                out["la"][b, t, h] = ab[t] * out["a"][b, t, h]
                lam = ab[t][:, None] * dSm
            out["s0"][b, h] = lam
            _finish(out, b, h, qb, gb, rh, dqh)
    return out


def grads_c(q, k, v, a, g, e, w, r, s0, do, dS, *, threads=None):
    """The token adjoint of ``grads_adjoint`` in C (``oracle_grads_f64`` in recurrence.c),
    fp64, OpenMP over (b, h), with the forward's states checkpointed every 128 tokens and
    recomputed per segment, so long sequences fit in memory. Same arguments and result."""
    import ctypes
    from . import load, max_threads
    lib = load()
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    f = lambda x: None if x is None else np.ascontiguousarray(x, dtype=np.float64)
    ins = [f(x) for x in (q, k, v, a, g, e, w, r, s0, do, dS)]
    out = _empty(q, v, r, s0)
    ptr = lambda x: None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    outs = [out[n] for n in ("q", "k", "v", "a", "la", "g", "e", "w", "r", "s0")]
    nthreads = max_threads() if threads is None else int(threads)
    rc = lib.oracle_grads_f64(B, T, H, dk, dv, *[ptr(x) for x in ins], *[ptr(x) for x in outs],
                              nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle backward failed with code {rc}")
    return out


def grads_chunked(q, k, v, a, g, e, w, r, s0, do, dS, *, chunk):
    """Gradients from chunk-level products (see the module docstring). The forward's chunk
    start states and u come from the token forward; everything of the backward is formed
    per chunk. The decay gradient comes out as la (= a * dL/da); "a" holds la / a where
    a > 0 and NaN where a token's decay is exactly zero."""
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    out = _empty(q, v, r, s0)
    for b in range(B):
        for h in range(H):
            qb, kb, vb, ab, gb, eb, wb = [_heads(x, b, h) for x in (q, k, v, a, g, e, w)]
            rh = np.asarray(r, np.float64)[h]
            S0 = np.zeros((dk, dv)) if s0 is None else np.asarray(s0, np.float64)[b, h]
            _, S_T, prev, _, us = _forward_head(qb, kb, vb, ab, gb, eb, wb, rh, S0, keep=True)
            qh = rh * gb * qb
            dob = _heads(do, b, h)
            lam = np.asarray(dS, np.float64)[b, h].copy()
            dqh = np.zeros((T, dk))
            starts = list(range(0, T, chunk))
            for c0 in reversed(starts):
                c1 = min(c0 + chunk, T)
                n = c1 - c0
                K, Q, U, E, A, dO = kb[c0:c1], qh[c0:c1], us[c0:c1], eb[c0:c1], ab[c0:c1], dob[c0:c1]
                Sc0 = prev[c0]
                S_C = prev[c1] if c1 < T else S_T
                gam = np.cumprod(A, axis=0)                       # gamma_t
                gamC = gam[-1]
                # Gamma_{t,s} = prod over s < tau <= t (1 for s = t, 0 for s > t).
                Gam = np.zeros((n, n, dk))
                for t in range(n):
                    run = np.ones(dk)
                    Gam[t, t] = run
                    for s in range(t - 1, -1, -1):
                        run = run * A[s + 1]
                        Gam[t, s] = run
                beta = np.array([np.prod(A[t + 1:], axis=0) for t in range(n)])
                Mx = np.einsum("ti,tsi,si->ts", K, Gam, K) * np.tri(n, k=-1)
                Px = np.einsum("ti,tsi,si->ts", Q, Gam, K)
                # Transposed triangular system per value column.
                rhs = (K * beta) @ lam + Px.T @ dO
                dU = np.zeros((n, dv))
                for j in range(dv):
                    dU[:, j] = np.linalg.solve(np.eye(n) + Mx.T * E[:, j][None, :], rhs[:, j])
                Pred = (K * gam) @ Sc0 + Mx @ U                     # p_t, the prediction
                dP = -E * dU
                out["v"][b, c0:c1, h] = wb[c0:c1] * dU
                out["w"][b, c0:c1, h] = vb[c0:c1] * dU
                out["e"][b, c0:c1, h] = -Pred * dU
                # Decayed key and query products.
                OU = dO @ U.T                                       # [t, s] = do_t . u_s
                PU = dP @ U.T                                       # [t, s] = dp_t . u_s
                dq_c = gam * (dO @ Sc0.T) + np.einsum("ts,tsi,si->ti", OU * np.tri(n), Gam, K)
                dkr = gam * (dP @ Sc0.T) + np.einsum("ts,tsi,si->ti", PU * np.tri(n, k=-1), Gam, K)
                dkw = (beta * (U @ lam.T)
                       + np.einsum("ts,tsi,ti->si", OU * np.tri(n), Gam, Q)
                       + np.einsum("ts,tsi,ti->si", PU * np.tri(n, k=-1), Gam, K))
                dqh[c0:c1] = dq_c
                out["k"][b, c0:c1, h] = dkr + dkw
                terms = Q * dq_c + K * dkr - K * dkw
                la = np.cumsum(terms[::-1], axis=0)[::-1] + np.sum(S_C * lam, axis=1)[None, :]
                out["la"][b, c0:c1, h] = la
                with np.errstate(divide="ignore", invalid="ignore"):
                    out["a"][b, c0:c1, h] = np.where(A > 0, la / np.where(A > 0, A, 1.0), np.nan)
                lam = gamC[:, None] * lam + (Q * gam).T @ dO + (K * gam).T @ dP
            out["s0"][b, h] = lam
            _finish(out, b, h, qb, gb, rh, dqh)
    return out
