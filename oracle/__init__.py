"""CPU oracle for the chunkwise gated delta rule with matched-filter readout.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
CPU-baseline leg may import or call anything in this package. It shares no code with
the HIP library (``gated_delta_rule_06_amd``), and neither imports the other.

What it computes is defined by the plain token recurrence (``recurrent``): per head,
a dk x dv state is decayed per row, the decayed state's prediction for the incoming
key is erased under a value-channel erase gate, the gated value is written, and the
state is read through a static row scale times a dynamic query gate. Sources: the
Muir abstract ("Full text" on the Astral Feed page "Muir: Linear Attention with
Sensitivity-Allocated Gating and Matched-Filter Readout") for the update order, the
openai-hub news page (section on matched-filter readout) and the liuch.name summary
(first bullet) for the readout.

Forms provided here:
  * ``recurrent``          the token recurrence in plain C (fp64 for parity, fp32 for
                           the timed CPU baseline), OpenMP over (b, h, column block);
  * ``recurrent_np``       the same definition in numpy (fp64), small cases only;
  * ``chunked_np``         the chunkwise form the pages describe for training: chunk
                           products pivoted at block boundaries (every factor in (0,1],
                           no division) and a recursive block-Neumann triangular solve
                           applied per value column (liuch.name summary, third bullet;
                           openai-hub page, section on the TPU chunkwise algorithm);
  * ``bruteforce_np``      the recurrence unrolled into explicit per-column transition
                           products (tiny sizes);
  * ``naive_unpivoted_nonfinite`` the unpivoted fp32 scheme that divides by cumulative
                           decays, kept only as a negative control (same two passages);
  * ``lowrank_gates``      (``gates.py``) the four gates from the rank-512 gate projection.
  * ``output_gate``        (``gates.py``) the output gate from the same projection.
  * ``backward``           (``backward.py``) every input's gradient, by autograd, by the
                           token adjoint and by chunk products (no GPU counterpart yet).

Every form is pinned by tests that do not reuse its own formula: closed forms that
reduce to textbook linear attention or gated linear attention, the last-write-only
case, exact erasure, brute force, linearity, column independence and a norm bound.
Absolute values on realistic inputs are pinned only through those invariants: the
pages print no worked example.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

from .gates import lowrank_gates, output_gate  # noqa: E402  (the low-rank gate definition)

__all__ = [
    "recurrent", "recurrent_np", "chunked_np", "bruteforce_np",
    "naive_unpivoted_nonfinite", "pivot_factors", "max_threads", "load", "lowrank_gates", "output_gate",
]

_LIB = None


def load():
    """Load (building if needed) the C oracle library."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        for name, ctype in (("oracle_recurrent_f64", ctypes.c_double),
                            ("oracle_recurrent_f32", ctypes.c_float)):
            fn = getattr(lib, name)
            ptr = ctypes.POINTER(ctype)
            fn.argtypes = [ctypes.c_int] * 5 + [ptr] * 11 + [ctypes.c_int]
            fn.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_grads_f64.argtypes = [ctypes.c_int] * 5 + [dp] * 21 + [ctypes.c_int]
        lib.oracle_grads_f64.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def max_threads() -> int:
    return int(load().oracle_max_threads())


def recurrent(q, k, v, a, g, e, w, r, s0=None, *, precision="f64", threads=None):
    """Token recurrence in C. Inputs [B,T,H,d] (r [H,dk], s0 [B,H,dk,dv] or None).

    Returns (o [B,T,H,dv], s_out [B,H,dk,dv]) as numpy arrays of the chosen precision.
    Inputs are converted exactly to that precision (bf16-valued float32 inputs are
    exact in both).
    """
    lib = load()
    dt = {"f64": np.float64, "f32": np.float32}[precision]
    ct = {"f64": ctypes.c_double, "f32": ctypes.c_float}[precision]
    fn = lib.oracle_recurrent_f64 if precision == "f64" else lib.oracle_recurrent_f32
    B, T, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    arrs = [np.ascontiguousarray(x, dtype=dt) for x in (q, k, v, a, g, e, w, r)]
    s0a = None if s0 is None else np.ascontiguousarray(s0, dtype=dt)
    o = np.empty((B, T, H, dv), dtype=dt)
    s_out = np.empty((B, H, dk, dv), dtype=dt)
    p = lambda x: None if x is None else x.ctypes.data_as(ctypes.POINTER(ct))
    nthreads = max_threads() if threads is None else int(threads)
    rc = fn(B, T, H, dk, dv, *[p(x) for x in arrs], p(s0a), p(o), p(s_out), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle recurrence failed with code {rc}")
    return o, s_out


def _prep(q, k, v, a, g, e, w, r):
    f = lambda x: np.asarray(x, dtype=np.float64)
    q, k, v, a, g, e, w, r = map(f, (q, k, v, a, g, e, w, r))
    qh = r[None, None] * g * q            # matched-filter query r * g_t * q_t
    b = w * v                             # gated write value w_t * v_t
    return qh, k, b, a, e


def recurrent_np(q, k, v, a, g, e, w, r, s0=None):
    """The token recurrence in numpy (fp64), vectorised over (b, h). Small inputs only."""
    qh, k, b, a, e = _prep(q, k, v, a, g, e, w, r)
    B, T, H, dk = k.shape
    dv = b.shape[-1]
    S = np.zeros((B, H, dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        S = a[:, t, :, :, None] * S                                  # decay
        p = np.einsum("bhij,bhi->bhj", S, k[:, t])                   # prediction
        S = S - k[:, t, :, :, None] * (e[:, t] * p)[:, :, None, :]   # erase
        S = S + k[:, t, :, :, None] * b[:, t][:, :, None, :]         # write
        o[:, t] = np.einsum("bhij,bhi->bhj", S, qh[:, t])            # read
    return o, S


def pivot_factors(a_blk: np.ndarray, m: int):
    """Boundary-pivoted factors for a split of a token range at local index ``m``.

    ``a_blk`` holds the decays of tokens lo..hi-1 (rows) for each channel (columns).
    Returns (F, R): F[t-m] = prod_{m<=tau<=t} a_tau for the right part t in [m, hi),
    R[s] = prod_{s<tau<m} a_tau for the left part s in [lo, m). Each is a running
    product of factors in (0, 1]: there is no division and no logarithm, so nothing
    overflows and an underflow only ever rounds a genuinely tiny decay to zero. For
    s < m <= t the pairwise decay prod_{s<tau<=t} a_tau equals F[t-m] * R[s].
    """
    a_blk = np.asarray(a_blk, dtype=np.float64)
    F = np.cumprod(a_blk[m:], axis=0)
    n_left = m
    R = np.ones((n_left,) + a_blk.shape[1:])
    for s in range(n_left - 2, -1, -1):
        R[s] = R[s + 1] * a_blk[s + 1]
    return F, R


def _split(lo, hi, leaf):
    nleaves = -(-(hi - lo) // leaf)
    return lo + leaf * ((nleaves + 1) // 2)


def chunked_np(q, k, v, a, g, e, w, r, s0=None, *, chunk=64, leaf=16,
               solve="neumann"):
    """The chunkwise form (fp64): pivoted chunk products, per-column triangular solve.

    Per chunk of C tokens with start state S0 (gamma_t = prod_{tau<=t} a_tau from the
    chunk start, beta_s = prod_{s<tau<=C} a_tau to the chunk end):
      H = (K * gamma) S0                                   prediction from S0
      (I + Diag(E[:, j]) M) U[:, j] = B[:, j] - E[:, j] * H[:, j]   for every column j
      O = (Qh * gamma) S0 + P U
      S_C = Diag(gamma_C) S0 + (K * beta)^T U
    with M[t,s] = sum_i k_ti Gamma_tsi k_si (s < t) and P[t,s] = sum_i qh_ti Gamma_tsi
    k_si (s <= t), Gamma_ts = prod_{s<tau<=t} a_tau. M and P are filled by recursive
    halving: the off-diagonal block of a split at m is one product
    (K_right * F)(K_left * R)^T of pivoted factors; blocks of at most ``leaf`` tokens
    use running products. ``solve='neumann'`` applies the recursive block-Neumann
    inverse of the unit lower-triangular system to each right-hand side (solve the
    left half, subtract E * (M_21 X_1) from the right half, solve the right half);
    ``solve='substitution'`` uses plain forward substitution.
    """
    qh, k, b, a, e = _prep(q, k, v, a, g, e, w, r)
    B_, T, H, dk = k.shape
    dv = b.shape[-1]
    S_all = np.zeros((B_, H, dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((B_, T, H, dv))
    for bi in range(B_):
        for h in range(H):
            S = S_all[bi, h]
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                n = c1 - c0
                K = k[bi, c0:c1, h]
                Q = qh[bi, c0:c1, h]
                A = a[bi, c0:c1, h]
                E = e[bi, c0:c1, h]
                Bv = b[bi, c0:c1, h]
                gamma = np.cumprod(A, axis=0)
                beta = np.ones_like(A)
                for s in range(n - 2, -1, -1):
                    beta[s] = beta[s + 1] * A[s + 1]
                M = np.zeros((n, n))
                P = np.zeros((n, n))

                def gram(lo, hi):
                    if hi - lo <= leaf:
                        for s in range(lo, hi):
                            run = np.ones(dk)
                            P[s, s] = np.dot(Q[s], K[s])
                            for t in range(s + 1, hi):
                                run = run * A[t]
                                M[t, s] = np.dot(K[t] * run, K[s])
                                P[t, s] = np.dot(Q[t] * run, K[s])
                        return
                    m = _split(lo, hi, leaf)
                    F, R = pivot_factors(A[lo:hi], m - lo)
                    left = K[lo:m] * R
                    M[m:hi, lo:m] = (K[m:hi] * F) @ left.T
                    P[m:hi, lo:m] = (Q[m:hi] * F) @ left.T
                    gram(lo, m)
                    gram(m, hi)

                gram(0, n)
                Hs = (K * gamma) @ S
                rhs = Bv - E * Hs
                if solve == "substitution":
                    U = np.zeros((n, dv))
                    for t in range(n):
                        U[t] = rhs[t] - E[t] * (M[t, :t] @ U[:t])
                elif solve == "neumann":
                    U = rhs.copy()

                    def nsolve(lo, hi):
                        if hi - lo <= leaf:
                            for t in range(lo, hi):
                                U[t] = U[t] - E[t] * (M[t, lo:t] @ U[lo:t])
                            return
                        m = _split(lo, hi, leaf)
                        nsolve(lo, m)
                        U[m:hi] -= E[m:hi] * (M[m:hi, lo:m] @ U[lo:m])
                        nsolve(m, hi)

                    nsolve(0, n)
                else:
                    raise ValueError(solve)
                o[bi, c0:c1, h] = (Q * gamma) @ S + P @ U
                S = gamma[-1][:, None] * S + (K * beta).T @ U
            S_all[bi, h] = S
    return o, S_all


def bruteforce_np(q, k, v, a, g, e, w, r, s0=None):
    """The recurrence unrolled into explicit transition products (fp64, tiny sizes).

    Per value column j, token t applies the dk x dk transition
    A_t = (I - e_tj k_t k_t^T) Diag(a_t), then adds k_t b_tj. Unrolled:
    S_t[:, j] = Phi_{t,0} S0[:, j] + sum_{s<=t} Phi_{t,s} k_s b_sj with
    Phi_{t,s} = A_t A_{t-1} ... A_{s+1}; o_tj = qh_t . S_t[:, j].
    """
    qh, k, b, a, e = _prep(q, k, v, a, g, e, w, r)
    B_, T, H, dk = k.shape
    dv = b.shape[-1]
    S0 = np.zeros((B_, H, dk, dv)) if s0 is None else np.asarray(s0, dtype=np.float64)
    o = np.zeros((B_, T, H, dv))
    S_T = np.zeros((B_, H, dk, dv))
    I = np.eye(dk)
    for bi in range(B_):
        for h in range(H):
            for j in range(dv):
                trans = [(I - e[bi, t, h, j] * np.outer(k[bi, t, h], k[bi, t, h]))
                         @ np.diag(a[bi, t, h]) for t in range(T)]
                for t in range(T):
                    phi = np.eye(dk)
                    for tau in range(t, -1, -1):
                        phi = phi @ trans[tau]
                    col = phi @ S0[bi, h, :, j]
                    for s in range(t + 1):
                        phi_ts = np.eye(dk)
                        for tau in range(t, s, -1):
                            phi_ts = phi_ts @ trans[tau]
                        col = col + phi_ts @ k[bi, s, h] * b[bi, s, h, j]
                    o[bi, t, h, j] = qh[bi, t, h] @ col
                    if t == T - 1:
                        S_T[bi, h, :, j] = col
    return o, S_T


def naive_unpivoted_nonfinite(a, k, chunk):
    """Negative control: which heads the unpivoted fp32 chunk scheme breaks.

    The traditional chunkwise algorithm forms (K * gamma)(K / gamma)^T with gamma the
    cumulative decay from the chunk start, i.e. it divides by cumulative decays. In
    fp32 gamma underflows on fast rows over a long chunk, 1/gamma overflows, and the
    product turns non-finite. Returns a boolean per head [H]: True when any chunk of
    any batch row produces a non-finite entry. ``a``, ``k``: [B,T,H,d] float32.
    """
    B_, T, H, d = a.shape
    bad = np.zeros(H, dtype=bool)
    with np.errstate(over="ignore", under="ignore", divide="ignore", invalid="ignore"):
        for c0 in range(0, T, chunk):
            c1 = min(T, c0 + chunk)
            gamma = np.cumprod(np.asarray(a[:, c0:c1], dtype=np.float32), axis=1,
                               dtype=np.float32)
            inv = np.float32(1.0) / gamma
            kk = np.asarray(k[:, c0:c1], dtype=np.float32)
            lhs = kk * gamma
            rhs = kk * inv
            # (K*gamma)(K/gamma)^T per (b, h); check finiteness of the operands and of
            # the products without forming every C x C matrix when one is enough.
            fin = np.isfinite(rhs).all(axis=(1, 3)) & np.isfinite(lhs).all(axis=(1, 3))
            for bi in range(B_):
                for h in range(H):
                    if bad[h] or not fin[bi, h]:
                        bad[h] = True
                        continue
                    prod = lhs[bi, :, h] @ rhs[bi, :, h].T
                    if not np.isfinite(prod).all():
                        bad[h] = True
    return bad
