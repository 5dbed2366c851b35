"""GPU parity for packed variable-length batches (sageattn_varlen) through the C ABI.

By definition a packed batch is the dense scheme applied to every sequence on its
own, so the oracle runs each sequence separately: the K mean, INT8 codes, block
scales, V^ codes and V scales of every sequence must match bit for bit at their
documented rows and slots, and the outputs must meet the dense acceptance test.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_attention_04_amd as qa
import synth_inputs as si
from gpu_helpers import compare_rows, note, sm_scale_of

pytestmark = pytest.mark.gpu

VW = si.VarlenWorkload

CASES = [
    VW("mixed_fp16", (1, 64, 100, 1000, 257), (1, 64, 100, 1000, 257), 4, 2, 128, seed=30),
    VW("mixed_fp8_causal", (1, 64, 100, 1000, 257), (1, 64, 100, 1000, 257), 4, 2, 128, causal=True, pv="fp8",
       seed=31),
    VW("q_ne_k_causal_d96", (10, 300, 64, 5), (100, 300, 30, 64), 4, 4, 96, dtype="fp16", causal=True, seed=32),
    VW("q_ne_k_fp8_d64_offset", (70, 3, 129), (200, 65, 129), 2, 1, 64, pv="fp8", seed=33, k_offset_sigma=2.0),
    VW("empty_sequences", (0, 50, 20, 7), (10, 0, 80, 7), 2, 2, 64, pv="fp8", causal=True, seed=34),
    VW("d256_fp8_causal", (100, 300, 65), (100, 300, 130), 4, 2, 256, pv="fp8", causal=True, seed=37),
]


class VCase:
    def __init__(self, w: si.VarlenWorkload):
        self.w = w
        note(f"[varlen case] {w}")
        self.q, self.k, self.v, self.cu_q, self.cu_k = si.make_varlen(w)
        self.qf, self.kf, self.vf = (x.float().numpy() for x in (self.q, self.k, self.v))
        self.cq, self.ck = self.cu_q.numpy().astype(np.int64), self.cu_k.numpy().astype(np.int64)
        self.Qs = oracle.quantize_varlen(self.qf, self.kf, self.vf, self.cq, self.ck, w.pv == "fp8")

    def gpu(self, accum=None, fused=False):
        w, dev = self.w, "cuda:0"
        note(f"[gpu] varlen {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} D{w.D} pv={w.pv} causal={w.causal} fused={fused}")
        q, k, v, cq, ck = (x.to(dev) for x in (self.q, self.k, self.v, self.cu_q, self.cu_k))
        if fused:
            qk, vq = qa.quant_qkv_varlen(q, k, v, cq, ck, max(w.lens_q + (1,)), max(w.lens_k + (1,)), w.pv)
        else:
            qk = qa.quant_qk_varlen(q, k, cq, ck, max(w.lens_q + (1,)), max(w.lens_k + (1,)))
            vq = qa.quant_v_varlen(v, ck, max(w.lens_k + (1,)), w.pv)
        out = qa.attn_fwd_varlen(qk, vq, w.torch_dtype, w.causal, sm_scale_of(w.D), accum or w.accum)
        torch.cuda.synchronize()
        return qk, vq, out


def _rows_slots(cu, b):
    R = int(cu[b]) + 64 * b
    return R, R // 64


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "fused"])
@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_varlen_quantization_bit_exact(w, fused):
    c = VCase(w)
    qk, vq, _ = c.gpu(fused=fused)
    Dp = qa.padded_dim(w.D)
    q8, qs = qk.q_i8.cpu().numpy(), qk.q_scale.cpu().numpy()
    k8, ks, km = qk.k_i8.cpu().numpy(), qk.k_scale.cpu().numpy(), qk.k_mean.cpu().numpy()
    raw = vq.v_hat.cpu()
    vh = raw.numpy() if w.pv == "fp8" else raw.view(torch.int16).numpy().view(np.uint16)
    for b in range(w.B):
        nq, nk = w.lens_q[b], w.lens_k[b]
        if nq:
            ref_q8, ref_qs = oracle.quant_blocks(oracle._seq(c.qf, c.cq, b))
            R, S = _rows_slots(c.cq, b)
            nb = qa.num_blocks(nq)
            np.testing.assert_array_equal(q8[:, R:R + nq, :w.D], ref_q8[0], err_msg=f"q_i8 seq {b}")
            assert not q8[:, R + nq:R + 64 * nb].any() and not q8[:, R:R + nq, w.D:].any()
            np.testing.assert_array_equal(qs[:, S:S + nb], ref_qs[0], err_msg=f"q_scale seq {b}")
        if nk:
            o = c.Qs[b]
            R, S = _rows_slots(c.ck, b)
            nb = qa.num_blocks(nk)
            np.testing.assert_array_equal(km[b], o.k_mean[0], err_msg=f"k_mean seq {b}")
            np.testing.assert_array_equal(k8[:, R:R + nk, :w.D], o.k_i8[0], err_msg=f"k_i8 seq {b}")
            assert not k8[:, R + nk:R + 64 * nb].any() and not k8[:, R:R + nk, w.D:].any()
            np.testing.assert_array_equal(ks[:, S:S + nb], o.k_scale[0], err_msg=f"k_scale seq {b}")
            # V^ blocks at slots S .. S+nb-1, channel-major [Dp][64]
            blocks = vh[:, S:S + nb].reshape(w.Hkv, nb, Dp, 64)
            tok = blocks.transpose(0, 1, 3, 2).reshape(w.Hkv, nb * 64, Dp)
            np.testing.assert_array_equal(tok[:, :nk, :w.D], oracle.v_hat_bits(o.v_hat[0], w.pv == "fp8"),
                                          err_msg=f"v_hat seq {b}")
            assert not tok[:, nk:].any() and not tok[:, :, w.D:].any()
            if w.pv == "fp8":
                np.testing.assert_array_equal(vq.v_scale.cpu().numpy()[b, :, :w.D], o.v_scale[0],
                                              err_msg=f"v_scale seq {b}")


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_varlen_output_matches_oracle(w):
    c = VCase(w)
    fmt = oracle.BF16 if w.dtype == "bf16" else oracle.FP16
    rows = np.array([(b, h, i) for b in range(w.B) for h in range(w.Hq) for i in range(w.lens_q[b])], np.int64)
    sm = sm_scale_of(w.D)
    em, amb = oracle.attn_emulate_varlen(c.Qs, w.causal, sm, rows, w.D, with_ambiguity=True)
    ex = oracle.attn_exact_varlen(c.qf, c.kf, c.vf, c.cq, c.ck, w.causal, sm, rows)
    for acc in ("fp32", "fp16+fp32"):
        _, _, out = c.gpu(acc)
        o = out.float().cpu().numpy()
        got = o[c.cq[rows[:, 0]] + rows[:, 2], rows[:, 1]].astype(np.float64)
        compare_rows(got, em, amb, ex if acc == w.accum else None, fmt, w.pv)
        # sequences without keys: zeros
        for b in range(w.B):
            if w.lens_k[b] == 0 and w.lens_q[b]:
                assert not out[int(c.cq[b]):int(c.cq[b + 1])].any()


def test_varlen_equals_dense_per_sequence():
    """A packed batch and per-sequence dense calls run the same arithmetic on the same
    tiles: the outputs must be identical bit for bit."""
    w = VW("dense_equiv", (300, 64, 1000), (300, 64, 1000), 4, 2, 128, causal=True, pv="fp8", seed=35)
    c = VCase(w)
    _, _, out = c.gpu()
    for b in range(w.B):
        q = c.q[c.cq[b]:c.cq[b + 1]][None].to("cuda:0")
        k = c.k[c.ck[b]:c.ck[b + 1]][None].to("cuda:0")
        v = c.v[c.ck[b]:c.ck[b + 1]][None].to("cuda:0")
        dense = qa.sageattn(q, k, v, "NHD", True, sm_scale_of(w.D), pv="fp8")
        assert torch.equal(dense[0], out[int(c.cq[b]):int(c.cq[b + 1])]), f"sequence {b}"


def test_varlen_large_sampled_rows():
    """A realistic packed batch (mixed lengths up to 8K, GQA, FP8 P.V, causal) on
    sampled rows of every sequence."""
    w = VW("large", (8192, 1500, 4096, 333, 2048), (8192, 1500, 4096, 333, 2048), 16, 4, 128, causal=True,
           pv="fp8", accum="fp16+fp32", seed=36)
    c = VCase(w)
    _, _, out = c.gpu()
    rows = []
    rng = np.random.default_rng(9)
    for b in range(w.B):
        for h in range(0, w.Hq, 3):
            for i in sorted(set([0, w.lens_q[b] - 1] + list(rng.integers(0, w.lens_q[b], 6)))):
                rows.append((b, h, int(i)))
    rows = np.array(rows, np.int64)
    sm = sm_scale_of(w.D)
    em, amb = oracle.attn_emulate_varlen(c.Qs, True, sm, rows, w.D, with_ambiguity=True)
    ex = oracle.attn_exact_varlen(c.qf, c.kf, c.vf, c.cq, c.ck, True, sm, rows)
    o = out.float().cpu().numpy()
    got = o[c.cq[rows[:, 0]] + rows[:, 2], rows[:, 1]].astype(np.float64)
    compare_rows(got, em, amb, ex, oracle.BF16, "fp8")


# ----------------------------------------------------------------------------- Q quantised in the attention kernel

@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_varlen_fused_q_equals_separate(w):
    """quant_kv_varlen + attn_fwd_varlen_fused_q against quant_qkv_varlen + attn_fwd_varlen:
    K/V operands, the Q codes and scales the kernel formed (padding rows included) and
    the outputs, bit for bit."""
    c = VCase(w)
    qk, vq, ref = c.gpu(fused=True)
    dev = "cuda:0"
    q, k, v, cq, ck = (x.to(dev) for x in (c.q, c.k, c.v, c.cu_q, c.cu_k))
    mq, mk = max(w.lens_q + (1,)), max(w.lens_k + (1,))
    kq, vq2 = qa.quant_kv_varlen(k, v, ck, mk, w.pv)
    qi = torch.full_like(qk.q_i8, 0x55)
    qs = torch.full_like(qk.q_scale, -1.0)
    out = qa.attn_fwd_varlen_fused_q(q, cq, mq, kq, vq2, w.causal, sm_scale_of(w.D), w.accum, q_codes=(qi, qs))
    torch.cuda.synchronize()
    # the documented rows and slots of every sequence (rows between sequences are never written)
    assert torch.equal(kq.k_mean, qk.k_mean)
    for b in range(w.B):
        if w.pv == "fp8" and w.lens_k[b] > 0:  # a sequence without keys has no V scale written
            assert torch.equal(vq2.v_scale[b], vq.v_scale[b]), f"V scales of sequence {b}"
        R, S = _rows_slots(c.ck, b)
        nb = (w.lens_k[b] + 63) // 64
        assert torch.equal(kq.k_i8[:, R:R + 64 * nb], qk.k_i8[:, R:R + 64 * nb]), f"K codes of sequence {b}"
        assert torch.equal(kq.k_scale[:, S:S + nb], qk.k_scale[:, S:S + nb]), f"K scales of sequence {b}"
        assert torch.equal(vq2.v_hat[:, S:S + nb], vq.v_hat[:, S:S + nb]), f"V codes of sequence {b}"
        R, S = _rows_slots(c.cq, b)
        nb = (w.lens_q[b] + 63) // 64
        assert torch.equal(qi[:, R:R + 64 * nb], qk.q_i8[:, R:R + 64 * nb]), f"Q codes of sequence {b}"
        assert torch.equal(qs[:, S:S + nb], qk.q_scale[:, S:S + nb]), f"Q scales of sequence {b}"
    assert torch.equal(out, ref)
    # and sageattn_varlen takes this schedule by default
    o2 = qa.sageattn_varlen(q, k, v, cq, ck, mq, mk, w.causal, sm_scale_of(w.D), w.pv, w.accum)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref)
