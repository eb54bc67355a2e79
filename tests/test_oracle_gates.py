"""Pins of the oracle's low-rank gate generation (oracle/gates.py) against closed forms:
zero up-projections, one-hot ranks (which select one up-projection column, and so pin the
rank slices and the weight index order), additivity of the pre-activation, the slice of
the output gate feeding none of the four gates, and the output gate itself reading its
slice only."""
import math

import numpy as np
import pytest

import oracle
from oracle import gates as G

pytestmark = []


def weights(rng, H, d, scale=0.5):
    U = {n: rng.standard_normal((H, d, G.RANKS[n])) * scale for n in ("decay", "erase", "write", "read")}
    c = {n: rng.standard_normal((H, d)) for n in ("decay", "erase", "write", "read")}
    return U, c


def call(z, U, c):
    return oracle.lowrank_gates(z, U["decay"], U["erase"], U["write"], U["read"],
                                c["decay"], c["erase"], c["write"], c["read"])


def sig(y):
    return 1.0 / (1.0 + math.exp(-y))


def test_rank_slices_follow_the_gate_table():
    assert [G.RANKS[n] for n in ("decay", "erase", "output", "write", "read")] == [64, 64, 128, 128, 128]
    assert G.RANK == 512
    assert (G.SLICES["decay"].start, G.SLICES["erase"].start, G.SLICES["output"].start,
            G.SLICES["write"].start, G.SLICES["read"].start) == (0, 64, 128, 256, 384)


def test_zero_up_projection_gives_the_activated_offsets():
    rng = np.random.default_rng(1)
    H, d = 2, 3
    U, c = weights(rng, H, d)
    U = {n: np.zeros_like(u) for n, u in U.items()}
    z = rng.standard_normal((1, 4, 512))
    a, e, w, g = call(z, U, c)
    for h in range(H):
        for i in range(d):
            assert a[0, 2, h, i] == pytest.approx(math.exp(-math.exp(c["decay"][h, i])), rel=1e-14)
            assert e[0, 1, h, i] == pytest.approx(sig(c["erase"][h, i]), rel=1e-14)
            assert w[0, 3, h, i] == pytest.approx(sig(c["write"][h, i]), rel=1e-14)
            assert g[0, 0, h, i] == pytest.approx(sig(c["read"][h, i]), rel=1e-14)


@pytest.mark.parametrize("k", [0, 63, 64, 127, 128, 255, 256, 383, 384, 511])
def test_one_hot_rank_selects_one_weight_column(k):
    rng = np.random.default_rng(2 + k)
    H, d = 2, 4
    U, c = weights(rng, H, d)
    z = np.zeros((1, 1, 512))
    z[0, 0, k] = 1.0
    out = dict(zip(("decay", "erase", "write", "read"), call(z, U, c)))
    act = {"decay": lambda y: math.exp(-math.exp(y)), "erase": sig, "write": sig, "read": sig}
    for n in ("decay", "erase", "write", "read"):
        sl = G.SLICES[n]
        for h in range(H):
            for i in range(d):
                y = c[n][h, i] + (U[n][h, i, k - sl.start] if sl.start <= k < sl.stop else 0.0)
                assert out[n][0, 0, h, i] == pytest.approx(act[n](y), rel=1e-13)


def test_preactivation_is_affine_in_z():
    rng = np.random.default_rng(3)
    U, c = weights(rng, 2, 5)
    z1, z2 = rng.standard_normal((2, 1, 3, 512))
    for n in ("decay", "erase", "write", "read"):
        y12 = G.preactivation(z1 + z2, U[n], c[n], n)
        y1 = G.preactivation(z1, U[n], c[n], n)
        y2 = G.preactivation(z2, U[n], c[n], n)
        np.testing.assert_allclose(y12, y1 + y2 - c[n][None, None], rtol=1e-12, atol=1e-12)


def test_output_gate_slice_feeds_none_of_the_four_gates():
    rng = np.random.default_rng(4)
    U, c = weights(rng, 2, 3)
    z = rng.standard_normal((1, 5, 512))
    base = call(z, U, c)
    z[..., G.SLICES["output"]] = rng.standard_normal((1, 5, 128)) * 10
    for x, y in zip(base, call(z, U, c)):
        assert np.array_equal(x, y)


def test_ranges():
    rng = np.random.default_rng(5)
    U, c = weights(rng, 3, 8, scale=0.1)
    a, e, w, g = call(rng.standard_normal((2, 7, 512)), U, c)
    assert ((a > 0) & (a <= 1)).all()
    for x in (e, w, g):
        assert ((x > 0) & (x < 1)).all()


def test_output_gate_zero_up_projection_and_one_hot_ranks():
    rng = np.random.default_rng(6)
    H, d = 2, 3
    Uo = rng.standard_normal((H, d, 128)) * 0.5
    co = rng.standard_normal((H, d))
    og = oracle.output_gate(rng.standard_normal((1, 2, 512)), np.zeros_like(Uo), co)
    for h in range(H):
        for i in range(d):
            assert og[0, 1, h, i] == pytest.approx(sig(co[h, i]), rel=1e-14)
    for k in (0, 127, 128, 200, 255, 256, 511):
        z = np.zeros((1, 1, 512))
        z[0, 0, k] = 1.0
        og = oracle.output_gate(z, Uo, co)
        for h in range(H):
            for i in range(d):
                y = co[h, i] + (Uo[h, i, k - 128] if 128 <= k < 256 else 0.0)
                assert og[0, 0, h, i] == pytest.approx(sig(y), rel=1e-13)


def test_output_gate_reads_its_slice_only():
    rng = np.random.default_rng(7)
    Uo = rng.standard_normal((2, 4, 128)) * 0.5
    co = rng.standard_normal((2, 4))
    z = rng.standard_normal((1, 6, 512))
    og = oracle.output_gate(z, Uo, co)
    z2 = rng.standard_normal((1, 6, 512)) * 10
    z2[..., G.SLICES["output"]] = z[..., G.SLICES["output"]]
    assert np.array_equal(og, oracle.output_gate(z2, Uo, co))
    assert ((og > 0) & (og < 1)).all()
    # The pre-activation is the slice times the up-projection, written out.
    b, t, h, i = 0, 3, 1, 2
    y = co[h, i] + sum(z[b, t, 128 + r] * Uo[h, i, r] for r in range(128))
    assert og[b, t, h, i] == pytest.approx(sig(y), rel=1e-13)
