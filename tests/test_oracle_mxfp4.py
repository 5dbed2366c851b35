"""Pins of the oracle's microscaling FP4 (MXFP4) reading, CPU only.

The reading (oracle.c, "Microscaling FP4"): blocks of 32 elements along the
contraction axis share a power-of-two scale X = 2^(floor(log2 amax) - 2); elements are
E2M1 (+-{0, .5, 1, 1.5, 2, 3, 4, 6}) rounded to nearest, ties to even, saturating.
Q and smoothed K are blocked along the channels, V along the tokens, P along 32
consecutive keys.  The pins below come from that definition and from closed forms,
not from the oracle's own code.
"""
import numpy as np
import pytest

import oracle

MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# fp32(sm_scale) * fp32(log2 e) == 1.0 exactly for this sm_scale: scores are in log2 units
UNIT_SM = 0.6931471824645996


def _nearest_e2m1(x: float) -> float:
    """Brute force: the closest E2M1 magnitude, ties to the one with an even index
    (mantissa bit 0), values past 6 clamp to 6."""
    a = abs(x)
    if a >= 6.0:
        r = 6.0
    else:
        d = np.abs(MAGS - a)
        best = np.flatnonzero(d == d.min())
        r = MAGS[best[0]] if len(best) == 1 else MAGS[[i for i in best if i % 2 == 0][0]]
    return -r if np.signbit(x) else r


def test_e2m1_rounding_vs_brute_force():
    grid = np.concatenate([np.arange(-640, 641) / 64.0, np.random.default_rng(0).uniform(-12, 12, 2000),
                           [1e9, -1e9, 1e-30, -1e-30, -0.0, 0.0]])
    got = oracle.round_to(grid, oracle.E2M1, sat=True)
    want = np.array([_nearest_e2m1(float(x)) for x in grid])
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(want))


def test_e2m1_ties_go_to_even():
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for x, want in ties.items():
        assert oracle.round_to(np.array([x]), oracle.E2M1, sat=True)[0] == want, x
        assert oracle.round_to(np.array([-x]), oracle.E2M1, sat=True)[0] == -want, -x


def test_e2m1_codes_round_trip():
    for c in range(16):
        v = float(oracle.e2m1_decode(c))
        assert oracle.lib().orc_e2m1_code(v) == c, c
    assert oracle.lib().orc_e2m1_code(-0.0) == 8
    np.testing.assert_array_equal(oracle.e2m1_decode(np.arange(8)), MAGS)


def test_mx_exponent_definition():
    for e in range(-20, 20):
        for f in (1.0, 1.25, 1.999):
            assert oracle.mx_exp(f * 2.0 ** e) == e - 2
    assert oracle.mx_exp(0.0) == -126
    assert oracle.mx_exp(2.0 ** -140) == -126
    assert oracle.mx_exp(3.0e38) == 125


def _blocks(x):
    """(rows, D) -> list of (row, slice) blocks of 32 channels"""
    R, D = x.shape
    return [(r, slice(c, min(c + 32, D))) for r in range(R) for c in range(0, D, 32)]


def test_block_quantizer_invariants():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((1, 3, 50, 72)) * np.exp(rng.uniform(-8, 8, (1, 3, 50, 1)))).astype(np.float32)
    x[0, 1, 7, 32:64] = 0.0  # an all-zero block
    code, E = oracle.quant_mxfp4_rows(x)
    xd = oracle.mx_dequant(code, E)
    flat, fd, fe = x.reshape(-1, 72).astype(np.float64), xd.reshape(-1, 72), E.reshape(-1, 3)
    for r, sl in _blocks(flat):
        blk, deq = flat[r, sl], fd[r, sl]
        X = 2.0 ** fe[r, sl.start // 32]
        amax = np.abs(blk).max()
        if amax == 0:
            assert fe[r, sl.start // 32] == -126 and not deq.any()
            continue
        assert 4 * X <= amax < 8 * X  # the largest element lands in [4, 8) before clipping
        y = np.abs(blk) / X
        spacing = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
        err = np.abs(blk - deq)
        inside = y <= 6
        assert (err[inside] <= spacing[inside] / 2 * X).all()
        assert (np.abs(deq[~inside]) == 6 * X).all() and (err[~inside] < 2 * X).all()
        assert np.abs(deq).max() >= 4 * X  # the block maximum keeps its top code


def test_partial_block_uses_only_real_channels():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 2, 9, 40)).astype(np.float32)
    pad = np.zeros((1, 2, 9, 64), np.float32)
    pad[..., :40] = x
    c1, e1 = oracle.quant_mxfp4_rows(x)
    c2, e2 = oracle.quant_mxfp4_rows(pad)
    np.testing.assert_array_equal(c1, c2[..., :40])
    np.testing.assert_array_equal(e1, e2)
    assert not c2[..., 40:].any()


def test_smoothing_subtracts_the_mean_in_fp32():
    rng = np.random.default_rng(3)
    k = (rng.standard_normal((1, 2, 70, 64)) + 5).astype(np.float32)
    mu = oracle.k_mean(k)
    c1, e1 = oracle.quant_mxfp4_rows(k, mu)
    c2, e2 = oracle.quant_mxfp4_rows((k - mu[:, :, None, :]).astype(np.float32))
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(e1, e2)


def test_token_blocks_are_the_row_blocks_of_the_transpose():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((2, 2, 77, 24)).astype(np.float32)
    c, e = oracle.quant_mxfp4_tokens(v)
    ct, et = oracle.quant_mxfp4_rows(np.ascontiguousarray(v.transpose(0, 1, 3, 2)))
    np.testing.assert_array_equal(c, ct)
    np.testing.assert_array_equal(e, et)


def test_emulate_p_quantisation_closed_form():
    """Two 32-key half blocks with scores (log2 units) chosen so every step is known:
    keys 0, 2..31 at t = -1/8, key 1 at t = 0 (the row maximum), key 32 at t = -1/4.
    Half block 0: X = 2^-2, p = 2^-1/8 -> 3.668 -> 4 (p^ = 1), p = 1 -> 4 (p^ = 1).
    Half block 1: pmax = 2^-1/4 = 0.841, X = 2^-3, 6.73 clips to 6 (p^ = 0.75).
    l sums the unquantised p."""
    N, D = 33, 32
    q = np.zeros((1, 1, 1, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, N, D), np.float32)
    k[0, 0, 1, 0] = 0.125     # S = +1/8 : the maximum
    k[0, 0, 32, 0] = -0.125   # S = -1/8
    # channel 0 mean over keys is 0 (+1/8 and -1/8), so smoothing changes nothing
    v = np.zeros((1, 1, N, D), np.float32)
    v[0, 0, 0, 0], v[0, 0, 1, 0], v[0, 0, 32, 0] = 1.0, 0.5, 0.75
    v[0, 0, 0, 1], v[0, 0, 1, 1], v[0, 0, 32, 1] = -3.0, 2.0, 1.5
    Q = oracle.quantize_mxfp4(q, k, v)
    np.testing.assert_array_equal(oracle.mx_dequant(Q.v_code, Q.v_exp)[0, 0].T, v[0, 0])  # V lossless
    o = oracle.attn_emulate_mxfp4(Q, False, UNIT_SM, np.array([[0, 0, 0]]))[0]
    p_a, p_c = float(np.float32(2.0 ** -0.125)), float(np.float32(2.0 ** -0.25))
    l = 31 * p_a + 1.0 + p_c
    want0 = (1.0 * 1.0 + 1.0 * 0.5 + 0.75 * 0.75) / l
    want1 = (1.0 * -3.0 + 1.0 * 2.0 + 0.75 * 1.5) / l
    assert o[0] == pytest.approx(want0, rel=1e-12) and o[1] == pytest.approx(want1, rel=1e-12)
    assert not o[2:].any()


def test_emulate_p_rounding_between_codes():
    """One key at t = -1/2 beside the maximum: p = 2^-1/2 = 0.7071 -> 2.83 X -> 3 X (0.75)."""
    D = 32
    q = np.zeros((1, 1, 1, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 2, D), np.float32)
    k[0, 0, 0, 0], k[0, 0, 1, 0] = 0.25, -0.25
    v = np.zeros((1, 1, 2, D), np.float32)
    v[0, 0, 0, 3], v[0, 0, 1, 3] = 1.0, 0.5
    Q = oracle.quantize_mxfp4(q, k, v)
    o = oracle.attn_emulate_mxfp4(Q, False, UNIT_SM, np.array([[0, 0, 0]]))[0]
    l = 1.0 + float(np.float32(2.0 ** -0.5))
    assert o[3] == pytest.approx((1.0 + 0.75 * 0.5) / l, rel=1e-12)


def test_emulate_special_cases():
    rng = np.random.default_rng(5)
    D = 64
    # one key: p = 1 exactly, so o is the dequantised V row
    q = rng.standard_normal((1, 2, 5, D)).astype(np.float32)
    k = rng.standard_normal((1, 2, 1, D)).astype(np.float32)
    v = rng.standard_normal((1, 2, 1, D)).astype(np.float32)
    Q = oracle.quantize_mxfp4(q, k, v)
    rows = oracle.all_rows(1, 2, 5)
    o = oracle.attn_emulate_mxfp4(Q, False, 0.125, rows)
    vd = oracle.mx_dequant(Q.v_code, Q.v_exp)[..., 0]  # (B, H, D)
    np.testing.assert_array_equal(o, vd[rows[:, 0], rows[:, 1]])
    # Q = 0: every p = 1, so o is the mean of the dequantised V rows
    q0 = np.zeros((1, 1, 3, D), np.float32)
    k = rng.standard_normal((1, 1, 100, D)).astype(np.float32)
    v = rng.standard_normal((1, 1, 100, D)).astype(np.float32)
    Q = oracle.quantize_mxfp4(q0, k, v)
    o = oracle.attn_emulate_mxfp4(Q, False, 0.125, oracle.all_rows(1, 1, 3))
    mean = oracle.mx_dequant(Q.v_code, Q.v_exp)[0, 0].mean(axis=1)
    np.testing.assert_allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-12)
    # causal row 0 sees key 0 only
    q = rng.standard_normal((1, 1, 70, D)).astype(np.float32)
    Q = oracle.quantize_mxfp4(q, k[:, :, :70], v[:, :, :70])
    o = oracle.attn_emulate_mxfp4(Q, True, 0.125, np.array([[0, 0, 0]]))
    np.testing.assert_array_equal(o[0], oracle.mx_dequant(Q.v_code, Q.v_exp)[0, 0, :, 0])


def test_emulate_gqa_equals_repeated_heads():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 4, 40, 64)).astype(np.float32)
    k = rng.standard_normal((1, 2, 90, 64)).astype(np.float32)
    v = rng.standard_normal((1, 2, 90, 64)).astype(np.float32)
    rows = oracle.all_rows(1, 4, 40)
    a = oracle.attn_emulate_mxfp4(oracle.quantize_mxfp4(q, k, v), True, 0.125, rows)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    b = oracle.attn_emulate_mxfp4(oracle.quantize_mxfp4(q, kr, vr), True, 0.125, rows)
    np.testing.assert_array_equal(a, b)


def test_emulate_within_the_schemes_error_envelope():
    """End to end against exact attention on random inputs.  FP4 keeps one mantissa
    bit, so the envelope is wide: the measured error of this reading on N(0,1)
    inputs is rel-L1 ~0.25, cosine ~0.97 (Q/K, V and P each contribute)."""
    rng = np.random.default_rng(7)
    for D, N, causal in ((64, 300, False), (128, 700, True), (96, 200, False)):
        q = rng.standard_normal((1, 2, N, D)).astype(np.float32)
        k = (rng.standard_normal((1, 2, N, D)) + rng.normal(0, 2, (1, 2, 1, D))).astype(np.float32)
        v = rng.standard_normal((1, 2, N, D)).astype(np.float32)
        rows = oracle.sample_rows(1, 2, N, 24, seed=1)
        em = oracle.attn_emulate_mxfp4(oracle.quantize_mxfp4(q, k, v), causal, D ** -0.5, rows)
        ex = oracle.attn_exact(q, k, v, causal, D ** -0.5, rows)
        rel = np.abs(em - ex).sum() / np.abs(ex).sum()
        cos = (em * ex).sum() / np.linalg.norm(em) / np.linalg.norm(ex)
        assert rel < 0.35 and cos > 0.94, (D, N, rel, cos)


def test_emulate_ambiguity_is_zero_for_exact_powers():
    """The row maximum's block has p = 1 exactly (t = 0): no exponent ambiguity."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 8, 64)).astype(np.float32)
    k = rng.standard_normal((1, 1, 1, 64)).astype(np.float32)
    v = rng.standard_normal((1, 1, 1, 64)).astype(np.float32)
    _, amb = oracle.attn_emulate_mxfp4(oracle.quantize_mxfp4(q, k, v), False, 0.125, oracle.all_rows(1, 1, 8),
                                       with_ambiguity=True)
    assert not amb.any()
