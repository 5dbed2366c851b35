"""Pins for the CPU oracle: every check compares it with something other than
itself -- a library routine, a closed form, brute force on tiny inputs, or an
invariant of the mathematics -- so that a dropped term, a wrong sign or index,
or a transposed operand in ``oracle/oracle.c`` fails at least one test.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth_inputs as si

LOG2E = 1.4426950408889634

rng = np.random.default_rng(1234)


def _bf16_vals(shape, scale=1.0, seed=0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16).float().numpy()


def _fp16_vals(shape, scale=1.0, seed=0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.float16).float().numpy()


# ----------------------------------------------------------------------------- rounding

def _all_finite_fp16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    return vals[np.isfinite(vals)]


def test_round_e4m3_matches_torch_exhaustive():
    """Saturating RNE to OCP e4m3fn vs torch's float8_e4m3fn cast (library)."""
    base = _all_finite_fp16()
    xs = np.concatenate([base * s for s in (1.0, 0.37, 3.1, 1 / 448.0, 448.0 / 7.0)])
    xs = np.clip(xs, -448.0, 448.0).astype(np.float32).astype(np.float64)
    mine = oracle.round_to(xs, oracle.E4M3, sat=True)
    ref = torch.from_numpy(xs.astype(np.float32)).to(torch.float8_e4m3fn).float().double().numpy()
    np.testing.assert_array_equal(mine, ref)


def test_round_e4m3_special_points():
    # ties to even, saturation and overflow (OCP e4m3fn: max 448, no infinities)
    r = lambda x, sat=True: float(oracle.lib().orc_round(x, oracle.E4M3, int(sat)))
    assert r(1.0625) == 1.0          # halfway between 1.0 and 1.125 -> even mantissa
    assert r(1.1875) == 1.25         # halfway between 1.125 and 1.25 -> even mantissa
    assert r(460.0) == 448.0         # below the 464 midpoint: rounds down
    assert r(500.0) == 448.0         # saturates
    assert math.isnan(r(500.0, sat=False))
    assert r(2.0 ** -10) == 0.0      # half of the smallest subnormal 2^-9 -> even (0)
    assert r(2.0 ** -10 * 1.001) == 2.0 ** -9
    assert r(-3 * 2.0 ** -10) == -(2.0 ** -8)  # tie between 1 and 2 subnormal quanta -> 2


def test_round_fp16_matches_numpy():
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 5, 200000),
        _all_finite_fp16() + 0.0,
        (_all_finite_fp16()[:-1] + _all_finite_fp16()[1:]) / 2,  # exact midpoints (ties)
    ])
    x = x[np.abs(x) < 65504]
    np.testing.assert_array_equal(oracle.round_to(x, oracle.FP16), x.astype(np.float16).astype(np.float64))
    # saturation beyond the largest finite value
    assert oracle.round_to(np.array([70000.0, -1e9]), oracle.FP16, sat=True).tolist() == [65504.0, -65504.0]
    assert np.isinf(oracle.round_to(np.array([65520.0]), oracle.FP16)).all()


def test_round_bf16_matches_torch():
    x32 = np.concatenate([
        (rng.standard_normal(300000) * 10.0 ** rng.integers(-30, 30, 300000)).astype(np.float32),
        # exact ties: bf16 value + half a bf16 ulp
        (np.arange(1, 60000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    x32 = x32[np.isfinite(x32)]
    ref = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_to(x32.astype(np.float64), oracle.BF16), ref)


# ----------------------------------------------------------------------------- K mean

def test_k_mean_fp16_exact_any_order():
    k = _fp16_vals((2, 3, 200, 40), scale=3.0, seed=5)  # ragged: 200 = 3*64 + 8
    mine = oracle.k_mean(k)
    ref = (k.astype(np.float64).sum(axis=2) / 200).astype(np.float32)  # numpy pairwise order
    np.testing.assert_array_equal(mine, ref)


def test_k_mean_bf16_close_to_other_order():
    k = _bf16_vals((2, 2, 1000, 16), scale=1e3, seed=6)
    k[0, 0, 7, 3] = 3e30  # huge dynamic range makes summation order visible
    k[0, 0, 900, 3] = -3e30
    mine = oracle.k_mean(k).astype(np.float64)
    ref = np.sort(k.astype(np.float64), axis=2).sum(axis=2) / 1000
    ok = np.isclose(mine, ref, rtol=2 ** -23, atol=0)
    ok[0, 0, 3] = True  # catastrophic-cancellation channel checked below
    assert ok.all()


def test_k_mean_block_order_is_the_contract():
    """Blockwise fp64 order: within a 64-token block first, then across blocks.
    Block 0 = [2^60, 1 x 63], block 1 = [-2^60, 0 x 63]: the ones vanish inside
    block 0 (ulp(2^60) = 256), so the mean is exactly 0, not 63/128."""
    k = np.zeros((1, 1, 128, 1), np.float32)
    k[0, 0, 0, 0] = 2.0 ** 60
    k[0, 0, 1:64, 0] = 1.0
    k[0, 0, 64, 0] = -(2.0 ** 60)
    assert oracle.k_mean(k)[0, 0, 0] == 0.0
    k2 = k.copy()
    k2[0, 0, 64:, 0] = k[0, 0, :64, 0]
    k2[0, 0, :64, 0] = 0
    k2[0, 0, 0, 0] = -(2.0 ** 60)
    assert oracle.k_mean(k2)[0, 0, 0] == 0.0


def test_k_mean_constant():
    k = np.full((1, 2, 77, 8), 0.3125, np.float32)
    assert (oracle.k_mean(k) == np.float32(0.3125)).all()


# ----------------------------------------------------------------------------- INT8 block quantisation

def test_quant_rne_and_scale_worked_example():
    # amax = 127 -> scale = 1 and inv = 1 exactly, so q = rne(x): ties go to even
    x = np.zeros((1, 1, 64, 8), np.float32)
    x[0, 0, 0, :8] = [127, -127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.49999997]
    q, s = oracle.quant_blocks(x)
    assert s[0, 0, 0] == 1.0
    assert q[0, 0, 0, :8].tolist() == [127, -127, 2, 4, -2, 0, 2, 0]


def test_quant_invariants():
    x = _bf16_vals((2, 3, 300, 72), scale=2.0, seed=7)  # ragged tail of 44 tokens
    x[1, 2, 64:128] = 0.0  # an all-zero block
    mu = oracle.k_mean(x)
    for mean in (None, mu):
        q, s = oracle.quant_blocks(x, mean)
        y = x - (mean[:, :, None, :] if mean is not None else 0)  # fp32 subtract
        assert np.abs(q.astype(np.int32)).max() <= 127
        for b in range(2):
            for h in range(3):
                for j in range(5):
                    blk = y[b, h, 64 * j:64 * j + 64].astype(np.float64)
                    qb = q[b, h, 64 * j:64 * j + 64].astype(np.float64)
                    amax = np.abs(blk).max()
                    sc = float(s[b, h, j])
                    if amax == 0:
                        assert sc == 0 and (qb == 0).all()
                        continue
                    assert abs(sc * 127 - amax) <= amax * 2 ** -23
                    assert np.abs(qb[np.abs(blk) == amax]).min() == 127
                    # rounding error + the gap between x*fl(127/amax) and x/fl(amax/127)
                    assert (np.abs(blk - qb * sc) <= sc * (0.5 + 2 ** -15)).all()
    # the zero block
    q, s = oracle.quant_blocks(x)
    assert s[1, 2, 1] == 0 and (q[1, 2, 64:128] == 0).all()


def test_quant_ragged_tail_uses_only_real_tokens():
    x = _fp16_vals((1, 1, 100, 16), seed=8)
    q, s = oracle.quant_blocks(x)
    q2, s2 = oracle.quant_blocks(np.ascontiguousarray(x[:, :, 64:]))
    assert s[0, 0, 1] == s2[0, 0, 0]
    np.testing.assert_array_equal(q[:, :, 64:], q2)


def test_quant_mean_subtraction_is_fp32():
    x = _bf16_vals((1, 2, 130, 24), scale=5.0, seed=9)
    mu = oracle.k_mean(x)
    q_a, s_a = oracle.quant_blocks(x, mu)
    q_b, s_b = oracle.quant_blocks(np.ascontiguousarray(x - mu[:, :, None, :]))
    np.testing.assert_array_equal(q_a, q_b)
    np.testing.assert_array_equal(s_a, s_b)


# ----------------------------------------------------------------------------- V operand

def test_quant_v_fp16():
    v = _bf16_vals((1, 2, 70, 8), seed=10)
    v[0, 0, 3, 1] = 1e6  # beyond fp16 range: saturates
    vh, vs = oracle.quant_v(v, pv_fp8=False)
    assert vs is None
    ref = v.astype(np.float64)
    ref[0, 0, 3, 1] = 65504.0
    ref = ref.astype(np.float16).astype(np.float64)
    np.testing.assert_array_equal(vh.astype(np.float64), ref)


def test_quant_v_fp8_per_channel():
    v = _bf16_vals((2, 2, 150, 12), scale=3.0, seed=11)
    v[1, 1, :, 5] = 0.0  # all-zero channel
    vh, vs = oracle.quant_v(v, pv_fp8=True)
    amax = np.abs(v).max(axis=2)
    assert vs[1, 1, 5] == 0 and (vh[1, 1, :, 5] == 0).all()
    nz = amax > 0
    assert np.all(np.abs(vs[nz].astype(np.float64) * 448 - amax[nz]) <= amax[nz] * 2 ** -23)
    # the per-channel amax element maps to +-448
    for b in range(2):
        for h in range(2):
            for c in range(12):
                if amax[b, h, c] == 0:
                    continue
                i = np.argmax(np.abs(v[b, h, :, c]))
                assert abs(vh[b, h, i, c]) == 448.0
    # codes are e4m3 values; relative error bound of 3 mantissa bits (+ subnormal floor)
    assert np.array_equal(torch.from_numpy(vh).to(torch.float8_e4m3fn).float().numpy(), vh)
    recon = vh.astype(np.float64) * (vs[:, :, None, :].astype(np.float64))
    err = np.abs(recon - v)
    assert np.all(err <= np.abs(v) * 2 ** -4 + 2 ** -10 * vs[:, :, None, :] + 1e-30)


# ----------------------------------------------------------------------------- INT32 scores

def test_scores_i32_vs_numpy_matmul():
    q = _fp16_vals((2, 4, 150, 40), seed=12)
    k = _fp16_vals((2, 2, 130, 40), seed=13)
    v = _fp16_vals((2, 2, 130, 40), seed=14)
    Q = oracle.quantize(q, k, v, pv_fp8=False)
    tiles = [(0, 0, 0, 0), (1, 3, 2, 2), (0, 1, 2, 0), (1, 2, 1, 2), (0, 3, 0, 1)]
    got = oracle.scores_i32(Q, tiles)
    qp = np.zeros((2, 4, 192, 40), np.int64)
    kp = np.zeros((2, 2, 192, 40), np.int64)
    qp[:, :, :150] = Q.q_i8
    kp[:, :, :130] = Q.k_i8
    for t, (b, h, qb, kb) in enumerate(tiles):
        ref = qp[b, h, 64 * qb:64 * qb + 64] @ kp[b, h // 2, 64 * kb:64 * kb + 64].T
        np.testing.assert_array_equal(got[t], ref)


# ----------------------------------------------------------------------------- exact attention

def _sdpa64(q, k, v, causal, scale):
    t = lambda a: torch.from_numpy(a.astype(np.float64))
    return F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal, scale=scale,
                                          enable_gqa=q.shape[1] != k.shape[1]).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (6, 3)])
def test_exact_vs_torch_sdpa(causal, hq, hkv):
    q = _bf16_vals((2, hq, 70, 24), seed=20)
    k = _bf16_vals((2, hkv, 70, 24), seed=21)
    v = _bf16_vals((2, hkv, 70, 24), seed=22)
    sc = float(np.float32(1 / math.sqrt(24)))
    rows = oracle.all_rows(2, hq, 70)
    got = oracle.attn_exact(q, k, v, causal, sc, rows).reshape(2, hq, 70, 24)
    np.testing.assert_allclose(got, _sdpa64(q, k, v, causal, sc), rtol=0, atol=1e-12)


def test_exact_vs_brute_force_dense():
    q = _fp16_vals((1, 1, 9, 5), seed=23)
    k = _fp16_vals((1, 1, 13, 5), seed=24)
    v = _fp16_vals((1, 1, 13, 5), seed=25)
    s = 0.7 * (q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T)
    w = np.exp(s) / np.exp(s).sum(axis=1, keepdims=True)
    ref = w @ v[0, 0].astype(np.float64)
    got = oracle.attn_exact(q, k, v, False, 0.7, oracle.all_rows(1, 1, 9))
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_exact_softmax_invariance_to_key_offset():
    q = _bf16_vals((1, 2, 40, 16), seed=26)
    # keys on a 1/64 grid so that adding the offset is exact in fp32
    k = np.round(_bf16_vals((1, 2, 40, 16), seed=27) * 64).astype(np.float32) / 64
    v = _bf16_vals((1, 2, 40, 16), seed=28)
    c = (np.arange(16, dtype=np.float32) - 7.5) * 0.75
    rows = oracle.all_rows(1, 2, 40)
    for causal in (False, True):
        a = oracle.attn_exact(q, k, v, causal, 0.25, rows)
        b = oracle.attn_exact(q, k + c, v, causal, 0.25, rows)
        m = oracle.attn_exact(q, k - oracle.k_mean(k)[:, :, None, :], v, causal, 0.25, rows)
        np.testing.assert_allclose(a, b, atol=1e-12)
        np.testing.assert_allclose(a, m, atol=1e-6)  # the fp32 subtraction rounds per element


# ----------------------------------------------------------------------------- emulation

def test_emulate_hand_worked_example():
    """One query, two keys, D = 4, FP16 PV.  q = (127,0,0,0) and k = (177,0,0,0),
    (-77,0,0,0): the K mean is 50, so the smoothed keys are +-127, every scale
    is exactly 1 and the int8 codes are (127,...), (+-127,...).  With
    sm_scale = 2^-14 the two scores are +-16129/16384; softmax weights are
    1 and w = exp(-2*16129/16384); P is rounded to fp16 while l is not.  Worked in
    fp32 as the scheme is: c = 2^-14 * fp32(log2 e) (a power-of-two scaling, exact),
    S2 = +-fp32(16129 c), t = -2 fp32(16129 c) (exact), w = fp32(2^t)."""
    q = np.zeros((1, 1, 1, 4), np.float32)
    q[0, 0, 0, 0] = 127
    k = np.zeros((1, 1, 2, 4), np.float32)
    k[0, 0, :, 0] = [177, -77]
    v = np.zeros((1, 1, 2, 4), np.float32)
    v[0, 0, 0, 0] = 1.0
    v[0, 0, 1, 1] = 1.0
    Q = oracle.quantize(q, k, v, pv_fp8=False)
    assert Q.k_mean[0, 0, 0] == 50 and Q.q_scale.item() == 1 and Q.k_scale.item() == 1
    assert Q.k_i8[0, 0, :, 0].tolist() == [127, -127]
    c = np.float32(2.0 ** -14) * np.float32(LOG2E)
    t = np.float32(-2) * (np.float32(16129) * c)
    w = float(np.float32(np.exp2(np.float64(t))))
    assert abs(w - math.exp(-2 * 16129 / 16384)) < 1e-7
    l = 1 + w
    w16 = float(np.float16(w))
    out = oracle.attn_emulate(Q, False, 2.0 ** -14, np.array([[0, 0, 0]]))[0]
    np.testing.assert_allclose(out, [1 / l, w16 / l, 0, 0], rtol=1e-14)
    # FP8 PV: the V scale is amax/448 = 1/448 per used channel, P is coded as e4m3(448 p)
    Q8 = oracle.quantize(q, k, v, pv_fp8=True)
    assert Q8.v_scale[0, 0, 0] == np.float32(1 / 448) and Q8.v_hat[0, 0, 0, 0] == 448
    out8 = oracle.attn_emulate(Q8, False, 2.0 ** -14, np.array([[0, 0, 0]]))[0]
    p8 = float(torch.tensor(np.float32(448) * np.float32(w), dtype=torch.float32).to(torch.float8_e4m3fn).float())
    vs = float(np.float32(1 / 448))
    np.testing.assert_allclose(out8, [448 * 448 * vs / 448 / l, p8 * 448 * vs / 448 / l, 0, 0], rtol=1e-14)


@pytest.mark.parametrize("pv_fp8", [False, True])
def test_emulate_single_block_equals_one_shot_softmax(pv_fp8):
    """With one key block the online softmax is a one-shot softmax in base 2:
    m = max S2, p = 2^(S2 - m), l = sum p, o = sum p^ v^ / l."""
    q = _bf16_vals((1, 2, 50, 32), seed=30)
    k = _bf16_vals((1, 2, 60, 32), scale=2.0, seed=31) + 0.5
    v = _bf16_vals((1, 2, 60, 32), seed=32)
    Q = oracle.quantize(q, k, v, pv_fp8)
    sc = 0.3
    for h in range(2):
        s32 = Q.q_i8[0, h].astype(np.int64) @ Q.k_i8[0, h].astype(np.int64).T
        s2 = s32 * Q.q_scale[0, h, 0].astype(np.float64) * Q.k_scale[0, h, 0].astype(np.float64) * sc * LOG2E
        p = np.exp2(s2 - s2.max(axis=1, keepdims=True))
        if pv_fp8:
            ph = torch.from_numpy((p * 448).astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
        else:
            ph = p.astype(np.float16).astype(np.float64)
        ref = ph @ Q.v_hat[0, h].astype(np.float64) / p.sum(axis=1, keepdims=True)
        if pv_fp8:
            ref = ref * Q.v_scale[0, h].astype(np.float64) / 448
        rows = np.array([[0, h, i] for i in range(50)])
        got, amb = oracle.attn_emulate(Q, False, sc, rows, with_ambiguity=True)
        # p is formed in fp32 in the oracle (relative 1e-7 from this fp64 reference): only P
        # roundings that sit within 2^-14 of a tie may differ, and amb bounds their effect
        assert (np.abs(got - ref) <= 1e-6 * np.abs(ref) + amb + 1e-12).all()
        # the allowance is rare and small: a 2^-14 band around ties flags about 2^-14 /
        # (spacing / p) of the P values (1/4 for fp16 near 1, 1/512 for e4m3)
        assert amb.max() < (1e-3 if not pv_fp8 else 2e-2)


def test_emulate_multiblock_with_fixed_max():
    """If every row's maximum score sits in key block 0, alpha = 1 in all later
    blocks and the online result equals the one-shot softmax over all keys."""
    D = 16
    q = np.abs(_fp16_vals((1, 1, 64, D), seed=33)) + 0.5
    k = _fp16_vals((1, 1, 300, D), scale=0.2, seed=34)
    k[0, 0, 0] = 8.0  # key 0 dominates every (positive) query
    v = _fp16_vals((1, 1, 300, D), seed=35)
    Q = oracle.quantize(q, k, v, pv_fp8=False)
    kq = Q.k_i8[0, 0].astype(np.int64)
    nkb = 5
    sk = np.repeat(Q.k_scale[0, 0].astype(np.float64), 64)[:300]
    s32 = Q.q_i8[0, 0].astype(np.int64) @ kq.T
    s2 = s32 * Q.q_scale[0, 0, 0].astype(np.float64) * sk[None, :] * 0.5 * LOG2E
    assert (s2.argmax(axis=1) == 0).all() and nkb == Q.k_scale.shape[2]
    p = np.exp2(s2 - s2[:, :1])
    ref = p.astype(np.float16).astype(np.float64) @ Q.v_hat[0, 0].astype(np.float64) / p.sum(1, keepdims=True)
    got = oracle.attn_emulate(Q, False, 0.5, oracle.all_rows(1, 1, 64))
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-12)  # p in fp32


def test_emulate_online_rescale_tracks_one_shot():
    """When the maximum moves to later blocks, P is rounded relative to the
    running maximum; the result still matches the one-shot softmax to within
    fp16 rounding of P (a missing or wrong rescale factor is far outside)."""
    q = _bf16_vals((1, 1, 32, 32), seed=36)
    k = _bf16_vals((1, 1, 512, 32), seed=37) * np.linspace(0.2, 3.0, 512)[None, None, :, None].astype(np.float32)
    v = _bf16_vals((1, 1, 512, 32), seed=38)
    Q = oracle.quantize(q, k, v, pv_fp8=False)
    sk = np.repeat(Q.k_scale[0, 0].astype(np.float64), 64)
    s2 = (Q.q_i8[0, 0].astype(np.int64) @ Q.k_i8[0, 0].astype(np.int64).T) * \
        Q.q_scale[0, 0, 0].astype(np.float64) * sk[None, :] * 0.4 * LOG2E
    assert (s2.argmax(axis=1) >= 64).mean() > 0.9  # the max really moves
    p = np.exp2(s2 - s2.max(1, keepdims=True))
    ref = p @ Q.v_hat[0, 0].astype(np.float64) / p.sum(1, keepdims=True)
    got = oracle.attn_emulate(Q, False, 0.4, oracle.all_rows(1, 1, 32))
    np.testing.assert_allclose(got, ref, atol=2e-3)


def test_emulate_special_cases():
    D = 24
    v = _bf16_vals((1, 1, 90, D), seed=40)
    k = _bf16_vals((1, 1, 90, D), seed=41)
    q = _bf16_vals((1, 1, 90, D), seed=42)
    # Nkv = 1: output is the V^ row
    Q = oracle.quantize(q, k[:, :, :1].copy(), v[:, :, :1].copy(), pv_fp8=False)
    np.testing.assert_array_equal(oracle.attn_emulate(Q, False, 0.2, oracle.all_rows(1, 1, 90)),
                                  np.repeat(Q.v_hat[0, 0, :1].astype(np.float64), 90, 0))
    # causal row 0 sees key 0 only
    Q = oracle.quantize(q, k, v, pv_fp8=False)
    np.testing.assert_array_equal(oracle.attn_emulate(Q, True, 0.2, np.array([[0, 0, 0]]))[0],
                                  Q.v_hat[0, 0, 0].astype(np.float64))
    # FP8: Nkv = 1 -> v^ * vscale
    Q8 = oracle.quantize(q, k[:, :, :1].copy(), v[:, :, :1].copy(), pv_fp8=True)
    np.testing.assert_allclose(oracle.attn_emulate(Q8, False, 0.2, np.array([[0, 0, 5]]))[0],
                               Q8.v_hat[0, 0, 0].astype(np.float64) * Q8.v_scale[0, 0].astype(np.float64),
                               rtol=1e-15)
    # Q = 0: every score is 0, p = 1, o = mean of the V^ rows
    Qz = oracle.quantize(np.zeros_like(q), k, v, pv_fp8=False)
    np.testing.assert_allclose(oracle.attn_emulate(Qz, False, 0.2, np.array([[0, 0, 3]]))[0],
                               Qz.v_hat[0, 0].astype(np.float64).mean(0), rtol=1e-13)
    # constant V: output is that row (P^ sum / l differs only by fp16 rounding of P)
    vc = np.broadcast_to(v[:, :, :1], v.shape).copy()
    Qc = oracle.quantize(q, k, vc, pv_fp8=False)
    np.testing.assert_allclose(oracle.attn_emulate(Qc, False, 0.2, oracle.all_rows(1, 1, 90)),
                               np.repeat(Qc.v_hat[0, 0, :1].astype(np.float64), 90, 0), rtol=2e-3)


@pytest.mark.parametrize("pv_fp8", [False, True])
def test_emulate_gqa_equals_repeated_heads(pv_fp8):
    q = _bf16_vals((2, 6, 80, 16), seed=43)
    k = _bf16_vals((2, 2, 80, 16), seed=44)
    v = _bf16_vals((2, 2, 80, 16), seed=45)
    rows = oracle.all_rows(2, 6, 80)
    a = oracle.attn_emulate(oracle.quantize(q, k, v, pv_fp8), True, 0.25, rows)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)   # head h uses kv head h // 3
    b = oracle.attn_emulate(oracle.quantize(q, kr, vr, pv_fp8), True, 0.25, rows)
    np.testing.assert_array_equal(a, b)
    # and the exact mode agrees with torch's GQA convention
    e = oracle.attn_exact(q, k, v, True, 0.25, rows).reshape(2, 6, 80, 16)
    np.testing.assert_allclose(e, _sdpa64(q, k, v, True, 0.25), atol=1e-12)


@pytest.mark.parametrize("pv_fp8", [False, True])
def test_emulate_head_dim_padding_invariance(pv_fp8):
    q = _bf16_vals((1, 2, 100, 96), seed=46)
    k = _bf16_vals((1, 2, 100, 96), seed=47)
    v = _bf16_vals((1, 2, 100, 96), seed=48)
    pad = lambda a: np.concatenate([a, np.zeros(a.shape[:3] + (32,), np.float32)], axis=3)
    rows = oracle.all_rows(1, 2, 100)
    a = oracle.attn_emulate(oracle.quantize(q, k, v, pv_fp8), False, 0.1, rows)
    Qp = oracle.quantize(pad(q), pad(k), pad(v), pv_fp8)
    b = oracle.attn_emulate(Qp, False, 0.1, rows)
    np.testing.assert_array_equal(b[:, 96:], 0)
    np.testing.assert_array_equal(a, b[:, :96])


def test_layouts_are_the_same_tensor():
    w = si.workload("tiny", layout="NHD")
    q, k, v = si.make_qkv(w)
    qh, kh, vh = si.make_qkv(w.with_(layout="HND"))
    np.testing.assert_array_equal(oracle.to_hnd_f32(q, "NHD"), oracle.to_hnd_f32(qh, "HND"))
    np.testing.assert_array_equal(oracle.to_hnd_f32(v, "NHD"), oracle.to_hnd_f32(vh, "HND"))


# ----------------------------------------------------------------------------- the scheme vs exact

def _metrics(a, b):
    a = a.ravel()
    b = b.ravel()
    cos = float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
    rel_l1 = float(np.abs(a - b).sum() / np.abs(b).sum())
    return cos, rel_l1


@pytest.mark.parametrize("name,over", [
    ("tiny", {}),
    ("llm_prefill", {}),
    ("llm_prefill", {"causal": True}),
    ("video_dit", {}),
    ("gqa", {"Nq": 1024, "Nkv": 1024}),
    ("gqa", {"Nq": 1024, "Nkv": 1024, "D": 96}),
    ("seq_sweep", {"B": 1, "Hq": 4, "Hkv": 4, "Nq": 2048, "Nkv": 2048}),
])
def test_emulation_within_exact_tolerance(name, over):
    """The quantisation scheme itself meets cosine >= 0.999 against fp64 exact
    attention on the workload shapes; relative L1 <= 3e-2 with FP16 P.V.  With
    FP8-e4m3 P.V the 3-bit mantissa of P and V alone costs about 4 % relative
    L1 on these near-uniform N(0,1) attention maps, so the bound there is 5e-2."""
    w = si.workload(name, **over)
    q, k, v = si.make_qkv(w)
    qf, kf, vf = (oracle.to_hnd_f32(t, w.layout) for t in (q, k, v))
    rows = oracle.sample_rows(w.B, w.Hq, w.Nq, per_head=16, seed=1)
    sc = float(np.float32(1 / math.sqrt(w.D)))
    Q = oracle.quantize(qf, kf, vf, w.pv == "fp8")
    em = oracle.attn_emulate(Q, w.causal, sc, rows)
    ex = oracle.attn_exact(qf, kf, vf, w.causal, sc, rows)
    cos, rl1 = _metrics(em, ex)
    assert cos >= 0.999 and rl1 <= (5e-2 if w.pv == "fp8" else 3e-2), (cos, rl1)


def test_smoothing_matters_on_offset_keys():
    """On keys with a large shared per-channel offset, quantising K without the
    mean subtraction doubles the score error and clearly worsens the output
    (FP16 P.V, so that the P.V rounding does not mask the QK^T error)."""
    w = si.workload("video_dit", Nq=2048, Nkv=2048, Hq=2, Hkv=2)
    q, k, v = si.make_qkv(w)
    qf, kf, vf = (oracle.to_hnd_f32(t, w.layout) for t in (q, k, v))
    rows = oracle.sample_rows(w.B, w.Hq, w.Nq, per_head=32, seed=2)
    Q = oracle.quantize(qf, kf, vf, False)
    ex = oracle.attn_exact(qf, kf, vf, False, 0.125, rows)
    good = _metrics(oracle.attn_emulate(Q, False, 0.125, rows), ex)
    k8, sk = oracle.quant_blocks(kf)  # no smoothing
    Qbad = oracle.Quantized(Q.q_i8, Q.q_scale, k8, sk, Q.k_mean, Q.v_hat, Q.v_scale, False, 2, 2)
    bad = _metrics(oracle.attn_emulate(Qbad, False, 0.125, rows), ex)
    assert good[1] < 0.75 * bad[1], (good, bad)
    q64 = qf[0, 0].astype(np.float64)
    rep = lambda a: np.repeat(a.astype(np.float64), 64)

    def score_rms_err(k8_, sk_, k_used):
        approx = (Q.q_i8[0, 0].astype(np.int64) @ k8_[0, 0].astype(np.int64).T) * \
            rep(Q.q_scale[0, 0])[:, None] * rep(sk_[0, 0])[None, :]
        return np.sqrt(((approx - q64 @ k_used.T) ** 2).mean())

    k_smooth = kf[0, 0].astype(np.float64) - Q.k_mean[0, 0].astype(np.float64)
    assert score_rms_err(Q.k_i8, Q.k_scale, k_smooth) < 0.6 * score_rms_err(k8, sk, kf[0, 0].astype(np.float64))


def test_emulation_error_bound_on_scores():
    """|S2_emulated - S2_exact| <= sm_scale*log2e * sum_d(|q_d| s_k/2 + |k~_d| s_q/2 + s_q s_k/4)
    (plus the small reciprocal gap), per score."""
    q = _bf16_vals((1, 1, 64, 32), seed=50)
    k = _bf16_vals((1, 1, 64, 32), seed=51) + 1.0
    v = _bf16_vals((1, 1, 64, 32), seed=52)
    Q = oracle.quantize(q, k, v, False)
    sq = float(Q.q_scale[0, 0, 0])
    sk = float(Q.k_scale[0, 0, 0])
    kt = (k - Q.k_mean[:, :, None, :])[0, 0].astype(np.float64)
    qq = q[0, 0].astype(np.float64)
    exact = qq @ kt.T
    emul = (Q.q_i8[0, 0].astype(np.int64) @ Q.k_i8[0, 0].astype(np.int64).T) * sq * sk
    eq, ek = sq * (0.5 + 2 ** -15), sk * (0.5 + 2 ** -15)
    bound = np.abs(qq).sum(1)[:, None] * ek + np.abs(kt).sum(1)[None, :] * eq + 32 * eq * ek
    assert (np.abs(emul - exact) <= bound).all()


# ----------------------------------------------------------------------------- causal with Nq != Nkv, varlen

@pytest.mark.parametrize("nq,nkv", [(5, 9), (9, 5), (64, 130), (70, 70)])
def test_exact_causal_bottom_right_vs_sdpa_mask(nq, nkv):
    """Causal with Nq != Nkv: key j visible to query i iff j <= i + Nkv - Nq.  Checked
    against torch SDPA (fp64) given that boolean mask explicitly; rows that see no key
    are zeros in the oracle (SDPA leaves them undefined)."""
    q = _bf16_vals((1, 2, nq, 16), seed=60)
    k = _bf16_vals((1, 2, nkv, 16), seed=61)
    v = _bf16_vals((1, 2, nkv, 16), seed=62)
    sc = 0.25
    got = oracle.attn_exact(q, k, v, True, sc, oracle.all_rows(1, 2, nq)).reshape(1, 2, nq, 16)
    mask = torch.ones(nq, nkv, dtype=torch.bool).tril(diagonal=nkv - nq)
    t = lambda a: torch.from_numpy(a.astype(np.float64))
    ref = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask, scale=sc).numpy()
    seen = mask.any(dim=1).numpy()
    np.testing.assert_allclose(got[:, :, seen], ref[:, :, seen], rtol=0, atol=1e-12)
    assert (got[:, :, ~seen] == 0).all()


def test_emulate_causal_offset_is_the_tail_of_the_square_problem():
    """With Nkv - Nq a multiple of 64 the short query set's 64-token blocks coincide
    with the last blocks of the full one, so its causal (bottom-right) emulation must
    equal, bit for bit, the last Nq rows of the square causal problem."""
    n, nq = 200, 72  # offset 128
    q = _bf16_vals((1, 2, n, 32), seed=63)
    k = _bf16_vals((1, 2, n, 32), seed=64) + 0.5
    v = _bf16_vals((1, 2, n, 32), seed=65)
    for pv_fp8 in (False, True):
        full = oracle.quantize(q, k, v, pv_fp8)
        short = oracle.quantize(np.ascontiguousarray(q[:, :, n - nq:]), k, v, pv_fp8)
        np.testing.assert_array_equal(short.q_i8, full.q_i8[:, :, n - nq:])
        rows_full = np.array([(0, h, n - nq + i) for h in range(2) for i in range(nq)], np.int64)
        rows_short = np.array([(0, h, i) for h in range(2) for i in range(nq)], np.int64)
        a = oracle.attn_emulate(full, True, 0.2, rows_full)
        b = oracle.attn_emulate(short, True, 0.2, rows_short)
        np.testing.assert_array_equal(a, b)


def test_rows_without_visible_keys_are_zero():
    q = _bf16_vals((1, 1, 10, 8), seed=66)
    k = _bf16_vals((1, 1, 4, 8), seed=67)
    v = _bf16_vals((1, 1, 4, 8), seed=68)
    rows = oracle.all_rows(1, 1, 10)
    Q = oracle.quantize(q, k, v, False)
    em = oracle.attn_emulate(Q, True, 0.3, rows)
    ex = oracle.attn_exact(q, k, v, True, 0.3, rows)
    # offset 4 - 10 = -6: queries 0..5 see no key, query 6 sees key 0 only
    assert (em[:6] == 0).all() and (ex[:6] == 0).all()
    np.testing.assert_allclose(ex[6], v[0, 0, 0], rtol=1e-15)
    assert np.abs(em[6:]).sum() > 0


def test_varlen_oracle_is_the_dense_oracle_per_sequence():
    """The packed (total, H, D) helpers slice each sequence back to (1, H, n, D) and
    call the dense functions: check the slicing against dense calls made directly."""
    lens_q, lens_k = [3, 70, 1], [5, 66, 2]
    cu_q, cu_k = np.cumsum([0] + lens_q), np.cumsum([0] + lens_k)
    H, D = 2, 16
    q = _bf16_vals((cu_q[-1], H, D), seed=69)
    k = _bf16_vals((cu_k[-1], H, D), seed=70)
    v = _bf16_vals((cu_k[-1], H, D), seed=71)
    Qs = oracle.quantize_varlen(q, k, v, cu_q, cu_k, True)
    rows = np.array([(b, h, i) for b in range(3) for h in range(H) for i in range(lens_q[b])], np.int64)
    got = oracle.attn_emulate_varlen(Qs, True, 0.25, rows, D)
    ex = oracle.attn_exact_varlen(q, k, v, cu_q, cu_k, True, 0.25, rows)
    for b in range(3):
        qs = q[cu_q[b]:cu_q[b + 1]].transpose(1, 0, 2)[None].copy()
        ks = k[cu_k[b]:cu_k[b + 1]].transpose(1, 0, 2)[None].copy()
        vs = v[cu_k[b]:cu_k[b + 1]].transpose(1, 0, 2)[None].copy()
        Qd = oracle.quantize(qs, ks, vs, True)
        np.testing.assert_array_equal(Qd.k_i8, Qs[b].k_i8)
        r = oracle.all_rows(1, H, lens_q[b])
        sel = rows[:, 0] == b
        np.testing.assert_array_equal(got[sel], oracle.attn_emulate(Qd, True, 0.25, r))
        np.testing.assert_array_equal(ex[sel], oracle.attn_exact(qs, ks, vs, True, 0.25, r))


# ----------------------------------------------------------------------------- finer granularity
# "per-thread" quantisation (SageAttention project README, "Project Updates" v2.0.1 and
# "Current Features"): one Q scale per token, one K scale per 32 keys.

def _equal_amax(shape, A, seed, group_axis_len):
    """bf16 values in (-A, A) with |x| = A reached once in every group of
    `group_axis_len` tokens (every token when 1): every group has amax A."""
    x = np.clip(_bf16_vals(shape, scale=0.3 * A, seed=seed), -0.9 * A, 0.9 * A)
    B, H, N, D = shape
    g = torch.Generator().manual_seed(seed + 1)
    for t0 in range(0, N, group_axis_len):
        t = t0 + int(torch.randint(0, min(group_axis_len, N - t0), (1,), generator=g))
        c = int(torch.randint(0, D, (1,), generator=g))
        x[:, :, t, c] = A if (t + c) % 2 else -A
    return np.ascontiguousarray(x.astype(np.float32))


def test_quant_groups_of_64_are_the_blocks():
    x = _bf16_vals((2, 2, 150, 40), seed=60)
    for mean in (None, oracle.k_mean(x)):
        a = oracle.quant_blocks(x, mean)
        b = oracle.quant_groups(x, 64, mean)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("G", [1, 32])
def test_quant_groups_equal_amax_reduce_to_blocks(G):
    """When every group of G tokens has the block's amax, the group scales equal the
    block scale and the codes equal the block codes (ragged tail included)."""
    x = _equal_amax((1, 2, 150, 24), 3.0, 61, G)
    qb, sb = oracle.quant_blocks(x)
    qg, sg = oracle.quant_groups(x, G)
    np.testing.assert_array_equal(qg, qb)
    assert sg.shape == (1, 2, (150 + G - 1) // G)
    assert (sg == sb[0, 0, 0]).all()


@pytest.mark.parametrize("G", [1, 32])
def test_quant_groups_invariants(G):
    """Per group: max|code| = 127 where the group is non-zero, scale = amax / 127 and
    |y - code * scale| <= scale / 2 (plus the inv rounding), zeros for a zero group."""
    x = _bf16_vals((1, 2, 100, 48), seed=62) * np.exp(_bf16_vals((1, 2, 100, 1), scale=1.5, seed=63))
    x = np.ascontiguousarray(x.astype(np.float32))
    x[0, 1, 40:72] = 0.0
    mu = oracle.k_mean(x)
    for mean in (None, mu):
        q, s = oracle.quant_groups(x, G, mean)
        y = x - (mean[:, :, None, :] if mean is not None else 0)
        for h in range(2):
            for j in range(s.shape[2]):
                blk = y[0, h, G * j:G * j + G].astype(np.float64)
                qb = q[0, h, G * j:G * j + G].astype(np.float64)
                amax, sc = np.abs(blk).max(), float(s[0, h, j])
                if amax == 0:
                    assert sc == 0 and (qb == 0).all()
                    continue
                assert abs(sc * 127 - amax) <= amax * 2 ** -23
                assert np.abs(qb).max() == 127
                assert (np.abs(blk - qb * sc) <= sc * (0.5 + 2 ** -15)).all()


def test_per_token_q_scales_shrink_error_on_outlier_tokens():
    """Tokens 50x larger than their neighbours: per-token scales keep the small
    tokens' relative error at the INT8 level, one scale per 64 tokens does not."""
    x = _bf16_vals((1, 1, 128, 64), seed=64).astype(np.float32)
    x[0, 0, ::16] *= 50.0
    small = np.ones(128, bool)
    small[::16] = False
    errs = {}
    for G in (64, 1):
        q, s = oracle.quant_groups(np.ascontiguousarray(x), G)
        sc = np.repeat(s[0, 0], G)[:128][:, None]
        deq = q[0, 0].astype(np.float64) * sc
        errs[G] = np.abs(deq - x[0, 0])[small].mean() / np.abs(x[0, 0])[small].mean()
    assert errs[1] < 0.01 and errs[64] > 5 * errs[1], errs


@pytest.mark.parametrize("pv_fp8", [False, True])
def test_emulate_thread_granularity_equal_scales_is_block(pv_fp8):
    """With every Q token and every 32-key group at the block amax (and K's mean 0:
    each channel holds +x and -x), the finer scales equal the block scales and the
    emulation gives the block result exactly."""
    q = _equal_amax((1, 2, 100, 32), 2.0, 65, 1)
    kh = _equal_amax((1, 2, 75, 32), 1.5, 66, 32)
    k = np.ascontiguousarray(np.concatenate([kh, -kh], axis=2))  # channel sums exactly 0
    v = _bf16_vals((1, 2, 150, 32), seed=67)
    Qb = oracle.quantize(q, k, v, pv_fp8, "block")
    Qt = oracle.quantize(q, k, v, pv_fp8, "thread")
    assert (Qt.k_mean == 0).all()
    np.testing.assert_array_equal(Qb.q_i8, Qt.q_i8)
    np.testing.assert_array_equal(Qb.k_i8, Qt.k_i8)
    rows = oracle.all_rows(1, 2, 100)
    for causal in (False, True):
        np.testing.assert_array_equal(oracle.attn_emulate(Qb, causal, 0.2, rows),
                                      oracle.attn_emulate(Qt, causal, 0.2, rows))


@pytest.mark.parametrize("causal", [False, True])
def test_emulate_thread_granularity_is_softmax_of_dequantised_scores(causal):
    """FP16 P.V: the emulation equals fp64 softmax(sm_scale * Qd Kd^T) V^ with Qd, Kd
    the codes times their own token / 32-key scales (V^ = fp16(v)), up to the fp16
    rounding of P.  Scales spread over 100x between groups, so a score dequantised
    with another group's scale would be far off."""
    q = _bf16_vals((1, 2, 70, 32), seed=68) * np.exp(_bf16_vals((1, 2, 70, 1), scale=1.2, seed=69))
    k = _bf16_vals((1, 2, 150, 32), seed=70) * np.exp(_bf16_vals((1, 2, 150, 1), scale=1.2, seed=71)) + 0.3
    v = _bf16_vals((1, 2, 150, 32), seed=72)
    q, k = (np.ascontiguousarray(a.astype(np.float32)) for a in (q, k))
    Q = oracle.quantize(q, k, v, False, "thread")
    assert Q.q_scale.shape == (1, 2, 70) and Q.k_scale.shape == (1, 2, 5)
    sm = 0.25
    rows = oracle.all_rows(1, 2, 70)
    got = oracle.attn_emulate(Q, causal, sm, rows)
    for h in range(2):
        qd = Q.q_i8[0, h].astype(np.float64) * Q.q_scale[0, h][:, None].astype(np.float64)
        kd = Q.k_i8[0, h].astype(np.float64) * np.repeat(Q.k_scale[0, h], 32)[:150, None].astype(np.float64)
        s = sm * qd @ kd.T
        if causal:
            s = np.where(np.arange(150)[None, :] <= np.arange(70)[:, None] + 80, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        ref = p @ Q.v_hat[0, h].astype(np.float64) / p.sum(axis=1, keepdims=True)
        err = np.abs(got[h * 70:(h + 1) * 70] - ref).max()
        assert err <= 2e-3 * np.abs(ref).max(), err


# ----------------------------------------------------------------------------- error breakdown

@pytest.mark.parametrize("pv_fp8,causal", [(False, False), (True, True)])
def test_breakdown_extremes(pv_fp8, causal):
    """No approximation on: exact attention.  All on: the emulation (whose fp32 softmax
    steps move p by ~1e-7; P roundings within 2^-14 of a tie may differ, as amb says)."""
    q = _bf16_vals((1, 2, 150, 48), seed=60)
    k = _bf16_vals((1, 2, 150, 48), seed=61) + 0.7
    v = _bf16_vals((1, 2, 150, 48), seed=62)
    Q = oracle.quantize(q, k, v, pv_fp8)
    rows = oracle.all_rows(1, 2, 150)
    ex = oracle.attn_exact(q, k, v, causal, 0.2, rows)
    np.testing.assert_allclose(oracle.attn_breakdown(q, k, v, Q, causal, 0.2, rows, 0), ex, rtol=0, atol=1e-12)
    em, amb = oracle.attn_emulate(Q, causal, 0.2, rows, with_ambiguity=True)
    full = oracle.attn_breakdown(q, k, v, Q, causal, 0.2, rows, 7)
    # fp32 against fp64 p: relative ~1e-7 on each weight, so absolute 1e-6 of the output scale
    assert (np.abs(full - em) <= 1e-6 * np.abs(em).max() + amb).all()


def test_breakdown_single_parts_closed_forms():
    """Each approximation alone, against its closed form on one key block (one-shot
    base-2 softmax): INT8 scores -> softmax of the dequantised code products; P only ->
    fp16-rounded weights over the unrounded sum; V only -> the exact weights on the
    fp16 V (fp16 inputs: V unchanged, so equal to exact attention)."""
    q = _fp16_vals((1, 1, 40, 32), seed=63)
    k = _fp16_vals((1, 1, 60, 32), seed=64)
    v = _fp16_vals((1, 1, 60, 32), seed=65)
    Q = oracle.quantize(q, k, v, pv_fp8=False)
    rows = oracle.all_rows(1, 1, 40)
    sc = 0.3
    s_ex = q[0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T * sc * LOG2E
    s_q = (Q.q_i8[0, 0].astype(np.int64) @ Q.k_i8[0, 0].astype(np.int64).T) * \
        Q.q_scale[0, 0, 0].astype(np.float64) * Q.k_scale[0, 0, 0].astype(np.float64) * sc * LOG2E
    V = v[0, 0].astype(np.float64)

    def soft(s, rnd=False):
        p = np.exp2(s - s.max(1, keepdims=True))
        w = p.astype(np.float16).astype(np.float64) if rnd else p
        return w @ V / p.sum(1, keepdims=True)
    np.testing.assert_allclose(oracle.attn_breakdown(q, k, v, Q, False, sc, rows, oracle.PART_QK), soft(s_q),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.attn_breakdown(q, k, v, Q, False, sc, rows, oracle.PART_P), soft(s_ex, True),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.attn_breakdown(q, k, v, Q, False, sc, rows, oracle.PART_V), soft(s_ex),
                               rtol=1e-12, atol=1e-14)
