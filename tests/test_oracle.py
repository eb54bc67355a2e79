"""Pins of the CPU oracle against facts fixed outside its own code.

Each test checks the oracle (C token recurrence, numpy token recurrence, chunked form,
brute force) against something it does not reuse: a hand-derived worked example,
closed forms that reduce to textbook causal linear attention or gated linear
attention, the last-write-only and exact-erase special cases, the unrolled transition
products, linearity, column independence and a norm bound. A plausible mistake (a
dropped term, a wrong sign, reading before the write, decaying columns instead of
rows, a transposed operand) fails at least one of them.
"""
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NAMES = "q k v a g e w r".split()


def _rand_inputs(rng, B, T, H, d, unit_keys=True, s0=True):
    """Generic fp64 inputs in the method's ranges (keys unit-norm unless told not)."""
    k = rng.standard_normal((B, T, H, d))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((B, T, H, d))
    v = rng.standard_normal((B, T, H, d))
    a = rng.uniform(0.2, 1.0, (B, T, H, d))
    g = rng.uniform(0.0, 1.0, (B, T, H, d))
    e = rng.uniform(0.0, 1.0, (B, T, H, d))
    w = rng.uniform(0.0, 1.0, (B, T, H, d))
    r = rng.uniform(0.5, 1.5, (H, d))
    S0 = rng.standard_normal((B, H, d, d)) if s0 else None
    return [q, k, v, a, g, e, w, r], S0


def _all_forms(args, s0, chunk=4, leaf=4):
    out = {"c_f64": oracle.recurrent(*args, s0=s0),
           "numpy": oracle.recurrent_np(*args, s0=s0),
           "chunked": oracle.chunked_np(*args, s0=s0, chunk=chunk, leaf=leaf)}
    return out


def _load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *nums = line.split()
            vals[key] = np.array([float(x) for x in nums])
    return vals


def test_hand_derived_example_2x2():
    g = _load_golden("hand_example_2x2.txt")
    T, d = 2, 2
    shp = (1, T, 1, d)
    args = [g[n].reshape(shp) if n != "r" else g[n].reshape(1, d) for n in NAMES]
    for name, (o, S) in _all_forms(args, None, chunk=2, leaf=1).items():
        np.testing.assert_allclose(o.reshape(T, d), g["o"].reshape(T, d), rtol=0, atol=1e-12,
                                   err_msg=name)
        np.testing.assert_allclose(S.reshape(d, d), g["S_T"].reshape(d, d), rtol=0, atol=1e-12,
                                   err_msg=name)


def test_reduces_to_causal_linear_attention():
    """a = 1, e = 0, g = w = r = 1: O = tril(Q K^T) V (inclusive), S_T = K^T V."""
    rng = np.random.default_rng(11)
    B, T, H, d = 2, 13, 2, 5
    (q, k, v, a, g, e, w, r), _ = _rand_inputs(rng, B, T, H, d, unit_keys=False)
    a[:] = 1.0
    e[:] = 0.0
    g[:] = 1.0
    w[:] = 1.0
    r[:] = 1.0
    args = [q, k, v, a, g, e, w, r]
    for bi in range(B):
        for h in range(H):
            Q, K, V = q[bi, :, h], k[bi, :, h], v[bi, :, h]
            O_ref = np.tril(Q @ K.T) @ V
            S_ref = K.T @ V
            for name, (o, S) in _all_forms(args, None).items():
                np.testing.assert_allclose(o[bi, :, h], O_ref, atol=1e-11, err_msg=name)
                np.testing.assert_allclose(S[bi, h], S_ref, atol=1e-11, err_msg=name)


def test_zero_decay_keeps_only_last_write():
    """a = 0: S_t = k_t (w_t * v_t)^T and o_t = (k_t . qh_t)(w_t * v_t)."""
    rng = np.random.default_rng(12)
    B, T, H, d = 1, 9, 3, 6
    (q, k, v, a, g, e, w, r), S0 = _rand_inputs(rng, B, T, H, d)
    a[:] = 0.0
    args = [q, k, v, a, g, e, w, r]
    qh = r[None, None] * g * q
    o_ref = np.sum(k * qh, axis=-1, keepdims=True) * (w * v)
    S_ref = k[:, -1, :, :, None] * (w * v)[:, -1, :, None, :]
    for name, (o, S) in _all_forms(args, S0).items():
        np.testing.assert_allclose(o, o_ref, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(S, S_ref, atol=1e-12, err_msg=name)


def test_full_erase_stores_value_exactly():
    """e = 1 with unit keys: after token t the state maps k_t exactly to w_t * v_t."""
    rng = np.random.default_rng(13)
    B, H, d = 2, 2, 7
    for T in (1, 2, 5, 8):
        (q, k, v, a, g, e, w, r), S0 = _rand_inputs(rng, B, T, H, d)
        e[:] = 1.0
        _, S = oracle.recurrent(q, k, v, a, g, e, w, r, s0=S0)
        pred = np.einsum("bhij,bhi->bhj", S, k[:, -1])
        np.testing.assert_allclose(pred, (w * v)[:, -1], atol=1e-12)


def test_no_erase_is_gated_linear_attention():
    """e = 0: o_t = sum_{s<=t} sum_i qh_ti Gamma_tsi k_si b_s + (qh_t * gamma_t)^T S0."""
    rng = np.random.default_rng(14)
    B, T, H, d = 1, 11, 2, 4
    (q, k, v, a, g, e, w, r), S0 = _rand_inputs(rng, B, T, H, d)
    e[:] = 0.0
    args = [q, k, v, a, g, e, w, r]
    qh = r[None, None] * g * q
    b = w * v
    o_ref = np.zeros((B, T, H, d))
    for h in range(H):
        for t in range(T):
            gam_t = np.prod(a[0, : t + 1, h], axis=0)
            acc = (qh[0, t, h] * gam_t) @ S0[0, h]
            for s in range(t + 1):
                Gam = np.prod(a[0, s + 1 : t + 1, h], axis=0)  # empty product = 1
                acc = acc + np.sum(qh[0, t, h] * Gam * k[0, s, h]) * b[0, s, h]
            o_ref[0, t, h] = acc
    for name, (o, _) in _all_forms(args, S0).items():
        np.testing.assert_allclose(o, o_ref, atol=1e-12, err_msg=name)


def test_bruteforce_transition_products():
    rng = np.random.default_rng(15)
    B, T, H, d = 1, 6, 2, 3
    args, S0 = _rand_inputs(rng, B, T, H, d)
    o_bf, S_bf = oracle.bruteforce_np(*args, s0=S0)
    for name, (o, S) in _all_forms(args, S0, chunk=4, leaf=2).items():
        np.testing.assert_allclose(o, o_bf, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(S, S_bf, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("chunk,leaf", [(1, 16), (3, 16), (16, 4), (20, 4), (20, 16),
                                        (37, 4), (64, 16)])
@pytest.mark.parametrize("solve", ["neumann", "substitution"])
def test_chunked_form_equals_token_form(chunk, leaf, solve):
    inp = workloads.chunk_inputs(0, B=2, T=37, H=2, d=8)
    args = [inp[n] for n in NAMES]
    S0 = np.random.default_rng(16).standard_normal((2, 2, 8, 8))
    o_ref, S_ref = oracle.recurrent(*args, s0=S0)
    o, S = oracle.chunked_np(*args, s0=S0, chunk=chunk, leaf=leaf, solve=solve)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, atol=1e-12)


def test_pivot_factors_in_unit_interval_and_exact():
    rng = np.random.default_rng(17)
    n, d = 24, 5
    a = rng.uniform(0.0, 1.0, (n, d))
    a[3, 1] = 0.0   # a hard reset
    a[7, :] = 1.0
    for m in (1, 5, 12, 23):
        F, R = oracle.pivot_factors(a, m)
        assert np.all((F >= 0) & (F <= 1)) and np.all((R >= 0) & (R <= 1))
        assert np.all(np.isfinite(F)) and np.all(np.isfinite(R))
        for t in range(m, n):
            for s in range(m):
                direct = np.prod(a[s + 1 : t + 1], axis=0)
                np.testing.assert_allclose(F[t - m] * R[s], direct, rtol=1e-14, atol=0)


def test_linear_in_state_and_values():
    rng = np.random.default_rng(18)
    B, T, H, d = 1, 10, 2, 6
    (q, k, v1, a, g, e, w, r), S1 = _rand_inputs(rng, B, T, H, d)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    al, be = 0.7, -1.3
    o1, s1 = oracle.recurrent(q, k, v1, a, g, e, w, r, s0=S1)
    o2, s2 = oracle.recurrent(q, k, v2, a, g, e, w, r, s0=S2)
    o3, s3 = oracle.recurrent(q, k, al * v1 + be * v2, a, g, e, w, r, s0=al * S1 + be * S2)
    np.testing.assert_allclose(o3, al * o1 + be * o2, atol=1e-12)
    np.testing.assert_allclose(s3, al * s1 + be * s2, atol=1e-12)


def test_value_columns_are_independent():
    rng = np.random.default_rng(19)
    B, T, H, d = 1, 12, 2, 20
    (q, k, v, a, g, e, w, r), S0 = _rand_inputs(rng, B, T, H, d)
    o, S = oracle.recurrent(q, k, v, a, g, e, w, r, s0=S0)
    jp = 5
    v2, e2, w2, S02 = v.copy(), e.copy(), w.copy(), S0.copy()
    v2[..., jp] += 1.0
    e2[..., jp] = 1.0 - e2[..., jp]
    w2[..., jp] *= 0.5
    S02[..., jp] -= 2.0
    o2, Sb = oracle.recurrent(q, k, v2, a, g, e2, w2, r, s0=S02)
    others = [j for j in range(d) if j != jp]
    assert np.array_equal(o[..., others], o2[..., others])
    assert np.array_equal(S[..., others], Sb[..., others])
    assert not np.allclose(o[..., jp], o2[..., jp])


def test_column_norm_bound():
    """With unit keys, e in [0,1] and a <= 1 each per-column transition has norm <= 1:
    ||S_t[:, j]|| <= ||S_{t-1}[:, j]|| + |w_tj v_tj|."""
    rng = np.random.default_rng(20)
    B, T, H, d = 2, 40, 2, 8
    (q, k, v, a, g, e, w, r), S = _rand_inputs(rng, B, T, H, d)
    v *= 10.0
    for t in range(T):
        sl = slice(t, t + 1)
        _, S_next = oracle.recurrent(q[:, sl], k[:, sl], v[:, sl], a[:, sl], g[:, sl],
                                     e[:, sl], w[:, sl], r, s0=S)
        bound = np.linalg.norm(S, axis=2) + np.abs(w[:, t] * v[:, t])
        assert np.all(np.linalg.norm(S_next, axis=2) <= bound + 1e-12)
        S = S_next


def test_split_sequence_resumes_from_state():
    inp = workloads.chunk_inputs(0, B=1, T=50, H=2, d=8)
    args = [inp[n] for n in NAMES]
    o, S = oracle.recurrent(*args)
    first = [x[:, :23] if x.ndim == 4 else x for x in args]
    second = [x[:, 23:] if x.ndim == 4 else x for x in args]
    o1, S1 = oracle.recurrent(*first)
    o2, S2 = oracle.recurrent(*second, s0=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, atol=1e-13)
    np.testing.assert_allclose(S2, S, atol=1e-13)


def test_f32_instantiation_tracks_f64():
    inp = workloads.chunk_inputs(0)
    args = [inp[n] for n in NAMES]
    o64, S64 = oracle.recurrent(*args)
    o32, S32 = oracle.recurrent(*args, precision="f32")
    assert o32.dtype == np.float32
    assert np.abs(o32 - o64).max() / np.abs(o64).max() < 1e-5
    assert np.abs(S32 - S64).max() / np.abs(S64).max() < 1e-5


def test_stress_decays_stay_finite_in_pivoted_form():
    """a in {0, 1e-30, 1} and U(1e-3, 0.05): the pivoted chunk form never divides."""
    rng = np.random.default_rng(21)
    B, T, H, d = 1, 40, 1, 6
    (q, k, v, a, g, e, w, r), S0 = _rand_inputs(rng, B, T, H, d)
    a[:] = rng.uniform(1e-3, 0.05, a.shape)
    a[0, 5, 0, 0] = 0.0
    a[0, 9, 0, 1] = 1e-30
    a[0, 12, 0, :] = 1.0
    o_ref, S_ref = oracle.recurrent(q, k, v, a, g, e, w, r, s0=S0)
    o, S = oracle.chunked_np(q, k, v, a, g, e, w, r, s0=S0, chunk=32, leaf=8)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, atol=1e-12)


def test_negative_control_unpivoted_division_breaks_stress_heads():
    """The traditional scheme divides by cumulative decays: in fp32 it turns
    non-finite on the stress heads already at chunk 64, and on more heads as the chunk
    grows (all 16 at chunk 256) -- the failure the pivoted scheme removes."""
    inp = workloads.chunk_inputs(3)
    a, k = inp["a"], inp["k"]
    stress = set(inp["stress_heads"])
    assert stress == {0, 4, 8, 12}
    bad = {C: set(np.flatnonzero(oracle.naive_unpivoted_nonfinite(a, k, C)))
           for C in (64, 128, 256)}
    assert bad[64] == stress
    assert bad[64] <= bad[128] <= bad[256]
    assert bad[256] == set(range(16))
