"""Pins of the backward oracle (reverse mode of the token recurrence, fp64).

The three forms in ``oracle.backward`` (autograd, token adjoint, chunk products) are
checked against each other, and against facts that none of them reuses:
  * central finite differences of the loss computed by the C forward recurrence, along
    random directions in every input at once and along each input on its own;
  * textbook causal linear attention (decay 1, no erase, unit gates): o = tril(Q K^T) V,
    whose gradients are dV = tril(Q K^T)^T dO, dQ = tril(dO V^T) K, dK = tril(dO V^T)^T Q;
  * full forgetting (decay 0): each token sees only its own write, so o_t = (q_hat_t . k_t) b_t,
    and the decay gradient has a short closed form derived by hand from one token's update;
  * no erase (gated linear attention): the initial state's gradient is
    sum_t (gamma_t * q_hat_t) do_t^T + Diag(gamma_T) dS_T, gamma_t the decay product through t.
A dropped term (the erase's path into the keys, the read of the current write), a wrong sign,
a transposed operand or an off-by-one decay fails at least one of these.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as bw

GRADS = ("q", "k", "v", "a", "g", "e", "w", "r", "s0")


def _inputs(rng, B=1, T=11, H=2, dk=5, dv=3, s0=True):
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return dict(
        q=rng.standard_normal((B, T, H, dk)), k=k, v=rng.standard_normal((B, T, H, dv)),
        a=rng.uniform(0.3, 1.0, (B, T, H, dk)), g=rng.uniform(0.0, 1.0, (B, T, H, dk)),
        e=rng.uniform(0.0, 1.0, (B, T, H, dv)), w=rng.uniform(0.0, 1.0, (B, T, H, dv)),
        r=rng.uniform(0.5, 1.5, (H, dk)),
        s0=rng.standard_normal((B, H, dk, dv)) if s0 else None,
        do=rng.standard_normal((B, T, H, dv)), dS=rng.standard_normal((B, H, dk, dv)))


def _args(x):
    return tuple(x[n] for n in ("q", "k", "v", "a", "g", "e", "w", "r", "s0", "do", "dS"))


def _loss_c(x):
    """The loss from the C forward recurrence, which shares no code with oracle.backward."""
    o, s = oracle.recurrent(x["q"], x["k"], x["v"], x["a"], x["g"], x["e"], x["w"], x["r"],
                            s0=x["s0"])
    return float(np.sum(o * x["do"]) + np.sum(s * x["dS"]))


def _close(got, want, tol):
    scale = max(1.0, float(np.max(np.abs(want))))
    assert np.max(np.abs(got - want)) <= tol * scale, np.max(np.abs(got - want))


@pytest.mark.parametrize("chunk", [1, 3, 4, 11, 16])
def test_three_forms_agree(chunk):
    x = _inputs(np.random.default_rng(1), B=2)
    A = bw.grads_autograd(*_args(x))
    D = bw.grads_adjoint(*_args(x))
    C = bw.grads_chunked(*_args(x), chunk=chunk)
    for n in GRADS + ("la",):
        _close(D[n], A[n], 1e-12)
        _close(C[n], A[n], 1e-12)


def test_la_is_a_times_da():
    x = _inputs(np.random.default_rng(2))
    A = bw.grads_adjoint(*_args(x))
    _close(A["la"], x["a"] * A["a"], 1e-15)


def test_finite_differences_along_random_directions():
    rng = np.random.default_rng(3)
    x = _inputs(rng, T=9)
    G = bw.grads_adjoint(*_args(x))
    C = bw.grads_chunked(*_args(x), chunk=4)
    h = 1e-5
    for trial in range(3):
        dirs = {n: rng.standard_normal(np.shape(x[n])) for n in GRADS}
        plus = dict(x, **{n: x[n] + h * dirs[n] for n in GRADS})
        minus = dict(x, **{n: x[n] - h * dirs[n] for n in GRADS})
        fd = (_loss_c(plus) - _loss_c(minus)) / (2 * h)
        for grads in (G, C):
            an = sum(float(np.sum(grads[n] * dirs[n])) for n in GRADS)
            assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (trial, an, fd)


@pytest.mark.parametrize("name", GRADS)
def test_finite_differences_per_input(name):
    rng = np.random.default_rng(4)
    x = _inputs(rng, T=7, H=1)
    G = bw.grads_adjoint(*_args(x))
    d = rng.standard_normal(np.shape(x[name]))
    h = 1e-5
    fd = (_loss_c(dict(x, **{name: x[name] + h * d})) -
          _loss_c(dict(x, **{name: x[name] - h * d}))) / (2 * h)
    an = float(np.sum(G[name] * d))
    assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (an, fd)


def test_linear_attention_closed_form():
    rng = np.random.default_rng(5)
    T, d = 10, 4
    x = _inputs(rng, T=T, H=1, dk=d, dv=d, s0=False)
    x.update(a=np.ones((1, T, 1, d)), e=np.zeros((1, T, 1, d)), g=np.ones((1, T, 1, d)),
             w=np.ones((1, T, 1, d)), r=np.ones((1, d)), dS=np.zeros((1, 1, d, d)))
    Q, K, V, dO = (x[n][0, :, 0] for n in ("q", "k", "v", "do"))
    want = {"v": np.tril(Q @ K.T).T @ dO, "q": np.tril(dO @ V.T) @ K, "k": np.tril(dO @ V.T).T @ Q}
    for form in (bw.grads_adjoint(*_args(x)), bw.grads_chunked(*_args(x), chunk=4),
                 bw.grads_autograd(*_args(x))):
        for n, W in want.items():
            _close(form[n][0, :, 0], W, 1e-12)
        # With unit gates the gate gradients are the products with the gated operand.
        _close(form["w"][0, :, 0], V * want["v"], 1e-12)
        _close(form["g"][0, :, 0], Q * want["q"], 1e-12)
        _close(form["r"][0], np.sum(Q * want["q"], axis=0), 1e-12)


def test_full_forgetting_closed_form():
    rng = np.random.default_rng(6)
    T, dk, dv = 6, 4, 3
    x = _inputs(rng, T=T, H=1, dk=dk, dv=dv)
    x["a"] = np.zeros((1, T, 1, dk))
    qh = (x["r"][0] * x["g"] * x["q"])[0, :, 0]
    K, E, dO = x["k"][0, :, 0], x["e"][0, :, 0], x["do"][0, :, 0]
    b = (x["w"] * x["v"])[0, :, 0]
    dS = x["dS"][0, 0]
    s = np.sum(qh * K, axis=1)                              # q_hat_t . k_t
    db = s[:, None] * dO
    db[-1] += dS.T @ K[-1]                                  # the final state is k_T b_T^T
    dqh = K * np.sum(b * dO, axis=1)[:, None]
    dkey = qh * np.sum(b * dO, axis=1)[:, None]
    dkey[-1] += dS @ b[-1]
    # Decay gradient: perturbing a_t's channel i brings back row i of the previous state,
    # once directly and once through the prediction that the erase removes.
    prev = np.concatenate([x["s0"][0, 0][None], np.einsum("ti,tj->tij", K[:-1], b[:-1])])
    da = np.zeros((T, dk))
    for t in range(T):
        for i in range(dk):
            row = prev[t][i]
            dsrow = qh[t, i] * row - s[t] * K[t, i] * E[t] * row
            da[t, i] = dsrow @ dO[t]
            if t == T - 1:
                dstate_i = np.zeros((dk, dv))
                dstate_i[i] = row
                dstate_i -= np.outer(K[t], K[t, i] * E[t] * row)
                da[t, i] += np.sum(dS * dstate_i)
    for form in (bw.grads_adjoint(*_args(x)), bw.grads_autograd(*_args(x))):
        _close(form["v"][0, :, 0], x["w"][0, :, 0] * db, 1e-12)
        _close(form["w"][0, :, 0], x["v"][0, :, 0] * db, 1e-12)
        _close(form["q"][0, :, 0], x["r"][0] * x["g"][0, :, 0] * dqh, 1e-12)
        _close(form["k"][0, :, 0], dkey, 1e-12)
        _close(form["e"][0, :, 0], np.zeros((T, dv)), 1e-15)
        _close(form["s0"][0, 0], np.zeros((dk, dv)), 1e-15)
        _close(form["a"][0, :, 0], da, 1e-12)
    C = bw.grads_chunked(*_args(x), chunk=4)
    _close(C["la"][0, :, 0], np.zeros((T, dk)), 1e-15)
    assert np.all(np.isnan(C["a"]))


def test_no_erase_initial_state_gradient():
    rng = np.random.default_rng(7)
    x = _inputs(rng, T=9, H=1)
    x["e"] = np.zeros_like(x["e"])
    gam = np.cumprod(x["a"][0, :, 0], axis=0)
    qh = (x["r"][0] * x["g"] * x["q"])[0, :, 0]
    want = (gam * qh).T @ x["do"][0, :, 0] + gam[-1][:, None] * x["dS"][0, 0]
    for form in (bw.grads_adjoint(*_args(x)), bw.grads_chunked(*_args(x), chunk=4)):
        _close(form["s0"][0, 0], want, 1e-12)


def test_some_tokens_forget_everything():
    """Exact zeros in the decay: the chunk form's log-decay identity still gives a * da."""
    rng = np.random.default_rng(8)
    x = _inputs(rng, T=13)
    x["a"][0, 5, 0] = 0.0
    x["a"][0, 9, 1, :2] = 0.0
    A = bw.grads_autograd(*_args(x))
    C = bw.grads_chunked(*_args(x), chunk=4)
    for n in GRADS:
        if n != "a":
            _close(C[n], A[n], 1e-12)
    _close(C["la"], A["la"], 1e-12)


def test_c_adjoint_matches_autograd_across_segments():
    """The C token adjoint (checkpointed every 128 tokens, segments recomputed) against the
    definition, torch autograd through the fp64 forward: several segments and a ragged last
    one, an initial state and a final-state cotangent, two batch rows sharing dr."""
    x = _inputs(np.random.default_rng(11), B=2, T=290, H=2, dk=4, dv=3)
    A = bw.grads_autograd(*_args(x))
    G = bw.grads_c(*_args(x))
    for n in GRADS + ("la",):
        _close(G[n], A[n], 1e-12)


def test_c_adjoint_finite_differences_and_absent_state():
    """Central differences of the C forward's loss along random directions, with s0 and dS
    absent (zeros), and with decays of exactly 0 (la finite, equal to a * da)."""
    rng = np.random.default_rng(12)
    x = _inputs(rng, T=9, s0=False)
    x["dS"] = None
    x["a"][0, 4, 1, :3] = 0.0
    G = bw.grads_c(*_args(x))
    assert all(np.isfinite(G[n]).all() for n in G)
    _close(G["la"], x["a"] * G["a"], 1e-15)
    h = 1e-5
    names = [n for n in GRADS if n != "s0"]
    base = dict(x, s0=None, dS=np.zeros((1, 2, 5, 3)))
    for trial in range(3):
        dirs = {n: rng.standard_normal(np.shape(x[n])) for n in names}
        plus = dict(base, **{n: x[n] + h * dirs[n] for n in names})
        minus = dict(base, **{n: x[n] - h * dirs[n] for n in names})
        fd = (_loss_c(plus) - _loss_c(minus)) / (2 * h)
        an = sum(float(np.sum(G[n] * dirs[n])) for n in names)
        assert abs(an - fd) <= 1e-6 * max(1.0, abs(fd)), (trial, an, fd)


def test_loss_matches_the_c_forward_and_linear_attention():
    """oracle.backward.loss (numpy forward) against the C forward recurrence on random
    inputs, and against causal linear attention written with a library matmul
    (L = <tril(Q K^T) V, dO> + <K^T V, dS> at unit gates, no decay, no erase)."""
    x = _inputs(np.random.default_rng(13), B=2, T=10)
    assert abs(bw.loss(*_args(x)) - _loss_c(x)) <= 1e-12 * max(1.0, abs(_loss_c(x)))
    T, d = 8, 4
    y = _inputs(np.random.default_rng(14), T=T, H=1, dk=d, dv=d, s0=False)
    y.update(a=np.ones((1, T, 1, d)), e=np.zeros((1, T, 1, d)), g=np.ones((1, T, 1, d)),
             w=np.ones((1, T, 1, d)), r=np.ones((1, d)))
    Q, K, V, dO = (y[n][0, :, 0] for n in ("q", "k", "v", "do"))
    want = float(np.sum((np.tril(Q @ K.T) @ V) * dO) + np.sum((K.T @ V) * y["dS"][0, 0]))
    assert abs(bw.loss(*_args(y)) - want) <= 1e-12 * max(1.0, abs(want))
