"""Flop accounting of the chunk forward against the pages' figure: 98% of the chunkwise
flops on the matrix units (liuch.name summary, third bullet). This is a consistency check of
how the kernels split the work, not a measurement (the measured split comes from the
rocprofv3 instruction counters)."""
import bench


def test_matrix_cores_carry_at_least_95_percent_at_c256_d128():
    t = bench.flop_tally(256, 128)
    print(f"C=256 d=128: MFMA {t['mfma_flops']:.0f}, VALU {t['valu_flops']:.0f} flops per "
          f"token-head, MFMA share {t['mfma_share']:.4f}")
    assert t["mfma_share"] >= 0.95


def test_tally_matches_the_closed_form_of_the_products():
    """The matrix-core part is 6 d^2 (three state products) plus 2 C d for M and P plus
    C d + d for the solve's and the readout's triangular products (strictly lower between
    leaves and inclusive P U), which the per-term sums must reproduce exactly."""
    for C, d in ((64, 64), (128, 128), (256, 128)):
        t = bench.flop_tally(C, d)
        leaf, nb = 16, C // 16
        gram = (nb * (nb - 1) // 2 * 2 * leaf * leaf + nb * (leaf * leaf)) * 2 * d / C
        assert abs(t["mfma"]["gram_between_leaves"] + t["mfma"]["gram_inside_leaves"] - gram) < 1e-9
        assert abs(gram - 2 * C * d) < 1e-9                    # M and P: C^2 entries in all
        assert t["mfma"]["state_products"] == 6 * d * d
        pu = (C + 1) * d
        assert abs(t["mfma"]["readout_PU"] - pu) < 1e-9


def test_share_grows_with_chunk_size():
    """Larger chunks put more of the work into the matrix-core products (the pages' reason
    for large chunks); the share never falls below 90% at the configurations run here."""
    shares = [bench.flop_tally(C, 128)["mfma_share"] for C in (64, 128, 256)]
    assert shares == sorted(shares)
    assert min(shares + [bench.flop_tally(64, 64)["mfma_share"]]) >= 0.90
