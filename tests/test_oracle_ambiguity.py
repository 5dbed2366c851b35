"""Pins of the oracle's tie allowance (CPU only).

A rounding of p to FP16 / e4m3 (or E2M1 with its block exponent) is a decision taken
on an fp32 value; a p within a relative 2^-14 of a rounding tie may round either way
in another correct fp32 evaluation, and the oracle reports, per output element, the
change that flipping such a decision makes: |code_hi - code_lo| * |v^| / l.  The
margin is a fixed constant and holds while the scores that matter stay below 2^10 in
magnitude; beyond that the oracle refuses to give it.

The pins build P values at known distances from a tie (the distance measured here
against the neighbouring representable values, taken from tables of every fp16 and
e4m3fn code decoded by numpy / torch) and check the flag, the exact allowance, its
rescaling across key blocks, and the range guard.
"""
import numpy as np
import pytest
import torch

import oracle

AMB = 2.0 ** -14
# fp32(sm_scale) * fp32(log2 e) == 1.0 exactly for this sm_scale: scores are in log2 units
UNIT_SM = 0.6931471824645996


def _table(fmt) -> np.ndarray:
    """Every non-negative finite value of the format, sorted (from the library's decoding)."""
    if fmt == oracle.FP16:
        v = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    else:
        v = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    v = v[np.isfinite(v) & (v >= 0)]
    return np.unique(v)


TABLES = {oracle.FP16: _table(oracle.FP16), oracle.E4M3: _table(oracle.E4M3)}


def _neighbours(x: float, fmt) -> tuple:
    """(lo, hi): the representable values with lo <= x < hi."""
    t = TABLES[fmt]
    i = int(np.searchsorted(t, x, side="right"))
    return float(t[i - 1]), float(t[i])


def _rel_to_tie(x: float, fmt) -> tuple:
    """(relative distance of x from the midpoint of its two neighbouring codes, their spacing)."""
    lo, hi = _neighbours(x, fmt)
    return abs(x - 0.5 * (lo + hi)) / x, hi - lo


def test_unit_sm_scale_is_exact():
    assert np.float32(UNIT_SM) * np.float32(1.4426950408889634) == np.float32(1.0)


# ----------------------------------------------------------------------------- the per-P term

@pytest.mark.parametrize("fmt,mid,q", [
    (oracle.FP16, 1 + 2.0 ** -11, 2.0 ** -10),        # between 1 and 1 + 2^-10
    (oracle.FP16, 1 - 2.0 ** -12, 2.0 ** -11),        # between 1 - 2^-11 and 1
    (oracle.FP16, 1.5 * 2.0 ** -24, 2.0 ** -24),      # subnormal: between 2^-24 and 2^-23
    (oracle.FP16, 0.5 * 2.0 ** -24, 2.0 ** -24),      # between 0 and the smallest subnormal
    (oracle.E4M3, 1.0625, 0.125),                     # between 1 and 1.125
    (oracle.E4M3, 432.0, 32.0),                       # between 416 and 448
    (oracle.E4M3, 1.5 * 2.0 ** -9, 2.0 ** -9),        # subnormal
    (oracle.E2M1, 5.0, 2.0),                          # between 4 and 6
    (oracle.E2M1, 0.25, 0.5),                         # between 0 and 0.5
])
def test_tie_flip_at_known_distances(fmt, mid, q):
    """Exactly at a tie, and at 0.5x / 0.9x the margin on either side: flagged with the
    code spacing; at 1.2x and 4x the margin: not flagged."""
    for f in (0.0, 0.5, 0.9, -0.5, -0.9):
        assert oracle.tie_flip(mid * (1 + f * AMB), fmt) == q, f
    for f in (1.2, 4.0, -1.2, -4.0):
        assert oracle.tie_flip(mid * (1 + f * AMB), fmt) == 0.0, f


@pytest.mark.parametrize("fmt", [oracle.FP16, oracle.E4M3])
def test_tie_flip_spacing_matches_the_code_tables(fmt):
    """At the midpoint of every pair of neighbouring codes in a wide range the flag is
    their spacing; a little way off (3x the margin) it is zero."""
    t = TABLES[fmt]
    t = t[(t >= 2.0 ** -20) & (t < (60000.0 if fmt == oracle.FP16 else 448.0))]
    for lo, hi in zip(t[:-1], t[1:]):
        mid = 0.5 * (lo + hi)
        assert oracle.tie_flip(mid, fmt) == hi - lo, (lo, hi)
        assert oracle.tie_flip(mid * (1 + 3 * AMB), fmt) == 0.0
        assert oracle.tie_flip(mid * (1 - 3 * AMB), fmt) == 0.0


# ----------------------------------------------------------------------------- in the emulation

def _codes(S: int) -> tuple:
    """int8 codes (a, b) with a + 127 b = S (the score against q codes (1, 127))."""
    b = int(np.clip(round(S / 127), -127, 127))
    a = S - 127 * b
    assert -127 <= a <= 127
    return a, b


def _p_of(n: int, k: int) -> float:
    """fp32(2^t) for t = -n 2^-k (exact in fp32), correctly rounded."""
    return float(np.float32(np.exp2(np.float64(-n * 2.0 ** -k))))


def _pair_case(n: int, k: int, pv_fp8: bool):
    """One query against two keys with exact integer scores: q codes (1, 127), key 0
    scoring 16256 (the maximum), key 1 scoring 16256 - n; scales 1 and 2^-k and the
    unit sm_scale make c = 2^-k, so t = -n 2^-k exactly and p1 = fp32(2^t)."""
    q8 = np.array([[[[1, 127]]]], np.int8)
    k8 = np.array([[[_codes(16256), _codes(16256 - n)]]], np.int8)
    if pv_fp8:
        vh = np.array([[[[448.0, 0.0], [224.0, -448.0]]]], np.float32)
        vs = np.array([[[0.5 / 224.0, 2.0 / 448.0]]], np.float32)
    else:
        vh = np.array([[[[1.0, 0.0], [0.5, -2.0]]]], np.float32)
        vs = None
    return oracle.Quantized(q8, np.ones((1, 1, 1), np.float32), k8, np.full((1, 1, 1), 2.0 ** -k, np.float32),
                            np.zeros((1, 1, 2), np.float32), vh, vs, pv_fp8, 1, 1)


def _find_n(k: int, fmt, lo_rel: float, hi_rel: float, start: int = 200, count: int = 1):
    """The first n whose P (p, or fp32(448 p) for e4m3) lies between lo_rel and hi_rel
    (relative) from a tie."""
    out = []
    for n in range(start, 16000):
        p = _p_of(n, k)
        x = float(np.float32(np.float32(p) * np.float32(448.0))) if fmt == oracle.E4M3 else p
        d, sp = _rel_to_tie(x, fmt)
        if lo_rel <= d < hi_rel:
            out.append((n, p, sp))
            if len(out) == count:
                return out
    raise AssertionError("no such n")


@pytest.mark.parametrize("pv_fp8", [False, True])
def test_emulation_allowance_is_the_exact_flip(pv_fp8):
    """A p1 within 2^-16 of a tie gets amb = spacing * |v^| / l per channel (times
    v_scale / 448 with FP8); one between 2^-13 and 2^-12 away gets amb = 0; the row
    maximum (p = 1 exactly) never contributes."""
    fmt = oracle.E4M3 if pv_fp8 else oracle.FP16
    [(n, p1, sp)] = _find_n(14, fmt, 0.0, 2.0 ** -16)
    Q = _pair_case(n, 14, pv_fp8)
    out, amb = oracle.attn_emulate(Q, False, UNIT_SM, np.array([[0, 0, 0]]), with_ambiguity=True)
    want = sp * np.abs(Q.v_hat[0, 0, 1].astype(np.float64)) / (1.0 + p1)
    if pv_fp8:
        want = want * Q.v_scale[0, 0].astype(np.float64) / 448.0
    np.testing.assert_allclose(amb[0], want, rtol=1e-15, atol=0)
    assert amb[0].min() > 0
    [(n, _, _)] = _find_n(14, fmt, 2.0 ** -13, 2.0 ** -12)
    _, amb = oracle.attn_emulate(_pair_case(n, 14, pv_fp8), False, UNIT_SM, np.array([[0, 0, 0]]),
                                 with_ambiguity=True)
    assert (amb == 0).all()


def test_emulation_allowance_sums_over_blocks_with_the_rescale():
    """Block 0: 63 keys at score A (p = 1) and key 1 at A - n1 (a tie); block 1: key 64
    at A + d (the new maximum) and key 65 at A + d - n2 (a tie).  The allowance is
    (alpha * s1 |v1| + s2 |v65|) / l with alpha = 2^(-d 2^-14), l = alpha (63 + p1) +
    1 + p2, exactly as the output itself is rescaled and normalised."""
    k, A, d = 14, 16000, 256
    (n1, p1, s1), (n2, p2, s2) = _find_n(k, oracle.FP16, 0.0, 2.0 ** -16, count=2)
    Nkv = 66
    k8 = np.zeros((1, 1, Nkv, 2), np.int8)
    k8[0, 0, :64] = _codes(A)
    k8[0, 0, 1] = _codes(A - n1)
    k8[0, 0, 64] = _codes(A + d)
    k8[0, 0, 65] = _codes(A + d - n2)
    vh = np.zeros((1, 1, Nkv, 2), np.float32)
    vh[0, 0, 1] = (1.0, -0.5)
    vh[0, 0, 65] = (0.25, 2.0)
    Q = oracle.Quantized(np.array([[[[1, 127]]]], np.int8), np.ones((1, 1, 1), np.float32), k8,
                         np.full((1, 1, 2), 2.0 ** -k, np.float32), np.zeros((1, 1, 2), np.float32), vh, None,
                         False, 1, 1)
    _, amb = oracle.attn_emulate(Q, False, UNIT_SM, np.array([[0, 0, 0]]), with_ambiguity=True)
    alpha = np.exp2(-d * 2.0 ** -k)
    l = alpha * (63.0 + p1) + (1.0 + p2)
    want = (alpha * s1 * np.abs(vh[0, 0, 1].astype(np.float64)) + s2 * np.abs(vh[0, 0, 65].astype(np.float64))) / l
    np.testing.assert_allclose(amb[0], want, rtol=1e-13)


# ----------------------------------------------------------------------------- the range guard

def _guard_case(k: int, second):
    q8 = np.array([[[[1, 127]]]], np.int8)
    k8 = np.array([[[[127, 127], list(second)]]], np.int8)
    vh = np.array([[[[1.0, 0.0], [0.0, 1.0]]]], np.float32)
    return oracle.Quantized(q8, np.ones((1, 1, 1), np.float32), k8, np.full((1, 1, 1), 2.0 ** -k, np.float32),
                            np.zeros((1, 1, 2), np.float32), vh, None, False, 1, 1)


def test_score_range_guard():
    """Scores of 2^10 or more in log2 units leave the range in which the margin is
    defined: the emulation still runs, but asking for the allowance raises."""
    rows = np.array([[0, 0, 0]])
    oracle.attn_emulate(_guard_case(4, (0, 120)), False, UNIT_SM, rows, with_ambiguity=True)  # max 1016
    oracle.attn_emulate(_guard_case(3, (0, 120)), False, UNIT_SM, rows)                       # max 2032, no amb
    with pytest.raises(oracle.ScoreRangeError):
        oracle.attn_emulate(_guard_case(3, (0, 120)), False, UNIT_SM, rows, with_ambiguity=True)


def test_score_range_guard_ignores_keys_that_round_to_zero():
    """A key whose p is below 2^-32 cannot produce a nonzero code, so its magnitude does
    not matter: scores 1016 and -2032 (c = 2^-3 ... -16256 * 2^-3) pass."""
    q8 = np.array([[[[1, 127]]]], np.int8)
    k8 = np.array([[[[127, 63], [-127, -127]]]], np.int8)  # scores 8128 and -16256
    vh = np.array([[[[1.0, 0.0], [0.0, 1.0]]]], np.float32)
    Q = oracle.Quantized(q8, np.ones((1, 1, 1), np.float32), k8, np.full((1, 1, 1), 2.0 ** -3, np.float32),
                         np.zeros((1, 1, 2), np.float32), vh, None, False, 1, 1)
    oracle.attn_emulate(Q, False, UNIT_SM, np.array([[0, 0, 0]]), with_ambiguity=True)


# ----------------------------------------------------------------------------- microscaling P blocks

def test_mx_p_block_row_maximum_is_exact():
    """Block maximum from an integer t (p = 1): X = 2^-2, no alternative exponent; p =
    2^-0.5 -> 2.83 X -> 3 X; no element near an E2M1 tie, so no allowance."""
    p = np.array([1.0, 2 ** -0.5, 0.3])
    t = np.log2(p).astype(np.float32)
    t[0] = 0.0
    ph, flip = oracle.mx_p_block(p, t)
    np.testing.assert_array_equal(ph, [1.0, 0.75, 0.25])
    np.testing.assert_array_equal(flip, [0.0, 0.0, 0.0])


def test_mx_p_block_maximum_just_below_a_power_of_two():
    """Maximum 2^-1e-5 (non-integer t, within 2^-14 below 1): exponent -3 (X = 1/8,
    the maximum clips from 7.9999 X to 6 X); the alternative exponent -2 gives 4 X' = 1,
    so the allowance there is 1 - 0.75; 0.5 rounds alike under both (0), 0.9 does not
    (7.2 X -> 6 X = 0.75 against 3.6 X' -> 4 X' = 1)."""
    p = np.array([2.0 ** -1e-5, 0.5, 0.9])
    t = np.log2(p).astype(np.float32)
    ph, flip = oracle.mx_p_block(p, t)
    np.testing.assert_array_equal(ph, [0.75, 0.5, 0.75])
    np.testing.assert_array_equal(flip, [0.25, 0.0, 0.25])


def test_mx_p_block_maximum_just_above_a_power_of_two():
    """Maximum 0.5 * 2^1e-5 (within 2^-14 above 1/2): exponent -3 gives 4 X = 0.5; the
    alternative -4 saturates at 6 X' = 0.375: allowance 0.125.  0.2 = 1.6 X -> 1.5 X,
    and 3.2 X' -> 3 X', the same 0.1875: no allowance."""
    p = np.array([0.5 * 2.0 ** 1e-5, 0.2])
    t = np.log2(p).astype(np.float32)
    ph, flip = oracle.mx_p_block(p, t)
    np.testing.assert_array_equal(ph, [0.5, 0.1875])
    np.testing.assert_array_equal(flip, [0.125, 0.0])


def test_mx_p_block_maximum_far_from_a_power_of_two():
    """Maximum 0.75 (t non-integer, far from a power of two): no alternative exponent."""
    p = np.array([0.75, 0.9 * 0.75])
    t = np.log2(p).astype(np.float32)
    ph, flip = oracle.mx_p_block(p, t)
    # X = 2^(floor(log2 0.75) - 2) = 1/8: 6 X = 0.75; 0.675 = 5.4 X -> 6 X
    np.testing.assert_array_equal(ph, [0.75, 0.75])
    np.testing.assert_array_equal(flip, [0.0, 0.0])


def test_mx_p_block_element_at_an_e2m1_tie():
    """p = 0.875 in a block whose maximum is 1 (X = 1/4): 3.5 X is the midpoint of 3 X
    and 4 X, rounds to the even code 4 X, and the allowance is the spacing X."""
    p = np.array([1.0, 0.875, 0.875 * (1 + 4 * AMB)])
    t = np.log2(p).astype(np.float32)
    t[0] = 0.0
    ph, flip = oracle.mx_p_block(p, t)
    np.testing.assert_array_equal(ph, [1.0, 1.0, 1.0])
    np.testing.assert_array_equal(flip, [0.0, 0.25, 0.0])


def test_mx_score_range_guard():
    """An MXFP4 row whose scores reach 2^10 (32 channels of 6 * 2^e against 6 * 2^e:
    S = 1152 * 4^e in log2 units): the allowance is refused at e = 0, given at e = -1."""
    D = 32
    qc = np.full((1, 1, 1, D), 7, np.uint8)  # code 7: magnitude 6
    kc = np.full((1, 1, 2, D), 7, np.uint8)
    vc = np.zeros((1, 1, D, 2), np.uint8)

    def M(e):
        return oracle.MXQuantized(qc, np.full((1, 1, 1, 1), e, np.int32), kc, np.full((1, 1, 2, 1), e, np.int32),
                                  np.zeros((1, 1, D), np.float32), vc, np.zeros((1, 1, D, 1), np.int32), 1, 1)
    rows = np.array([[0, 0, 0]])
    oracle.attn_emulate_mxfp4(M(-1), False, UNIT_SM, rows, with_ambiguity=True)
    with pytest.raises(oracle.ScoreRangeError):
        oracle.attn_emulate_mxfp4(M(0), False, UNIT_SM, rows, with_ambiguity=True)
