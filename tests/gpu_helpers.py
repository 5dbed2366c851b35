"""Shared helpers for the GPU parity tests: run the HIP path and the CPU oracle on
the same seeded inputs and compare them."""
from __future__ import annotations

import math
import sys
from typing import Dict, Optional

import numpy as np
import torch

import oracle
import quantized_attention_04_amd as qa
import synth_inputs as si

FP8_REL_L1 = 5e-2   # exact-mode bound with FP8 P.V (the scheme itself sits near 4e-2, above the 3e-2 target)
FP16_REL_L1 = 3e-2
AMB_CAP = 1e-2      # per-element cap on the tie allowance added to the emulation tolerance


def note(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def sm_scale_of(D: int) -> float:
    return float(np.float32(1.0 / math.sqrt(D)))


class Case:
    """Inputs (host + device), the GPU quantisation and the oracle quantisation."""

    def __init__(self, w: si.Workload, dev: str = "cuda:0", gran: str = "block"):
        self.w = w
        self.gran = gran
        note(f"[case] {w} gran={gran}")
        self.q, self.k, self.v = si.make_qkv(w)
        self.dq, self.dk, self.dv = (t.to(dev) for t in (self.q, self.k, self.v))
        self.qf, self.kf, self.vf = (oracle.to_hnd_f32(t, w.layout) for t in (self.q, self.k, self.v))
        self._oq: Optional[oracle.Quantized] = None

    def with_pv(self, pv: str) -> "Case":
        """The same inputs with the other P.V mode (no regeneration)."""
        c = object.__new__(Case)
        c.__dict__.update(self.__dict__)
        c.w = self.w.with_(pv=pv)
        c._oq = None
        return c

    @property
    def oq(self) -> oracle.Quantized:
        if self._oq is None:
            self._oq = oracle.quantize(self.qf, self.kf, self.vf, self.w.pv == "fp8", self.gran)
        return self._oq

    def gpu_quant(self, fused: bool = False):
        note(f"[gpu] {'quant_qkv' if fused else 'quant_qk/quant_v'} {self.w.name} B{self.w.B} Hq{self.w.Hq} "
             f"Hkv{self.w.Hkv} Nq{self.w.Nq} Nkv{self.w.Nkv} D{self.w.D} {self.w.layout} pv={self.w.pv}")
        if fused or self.gran != "block":
            qk, vq = qa.quant_qkv(self.dq, self.dk, self.dv, self.w.layout, self.w.pv, gran=self.gran)
        else:
            qk = qa.quant_qk(self.dq, self.dk, self.w.layout)
            vq = qa.quant_v(self.dv, self.w.layout, self.w.pv)
        torch.cuda.synchronize()
        return qk, vq

    def gpu_attn(self, qk, vq, accum: Optional[str] = None, causal: Optional[bool] = None) -> torch.Tensor:
        w = self.w
        c = w.causal if causal is None else causal
        note(f"[gpu] attn_fwd {w.name} causal={c} accum={accum or w.accum}")
        out = qa.attn_fwd(qk, vq, w.torch_dtype, w.layout, c, sm_scale_of(w.D), accum or w.accum)
        torch.cuda.synchronize()
        return out


def check_quant_bit_exact(case: Case, qk, vq) -> None:
    w, o = case.w, case.oq
    Dp = qa.padded_dim(w.D)
    np.testing.assert_array_equal(qk.k_mean.cpu().numpy(), o.k_mean, err_msg="k_mean")
    for name, g, ref, N in (("q", qk.q_i8, o.q_i8, w.Nq), ("k", qk.k_i8, o.k_i8, w.Nkv)):
        g = g.cpu().numpy()
        np.testing.assert_array_equal(g[:, :, :N, :w.D], ref, err_msg=f"{name}_i8")
        assert not g[:, :, N:, :].any() and not g[:, :, :, w.D:].any(), f"{name}_i8 padding not zero"
    if case.gran == "block":
        np.testing.assert_array_equal(qk.q_scale.cpu().numpy(), o.q_scale, err_msg="q_scale")
        np.testing.assert_array_equal(qk.k_scale.cpu().numpy(), o.k_scale, err_msg="k_scale")
    else:
        # per token [B, Hq, N_pad] (padding rows 0); per 32 keys [B, Hkv, NB, 2]
        qs = qk.q_scale.cpu().numpy()
        np.testing.assert_array_equal(qs[:, :, :w.Nq], o.q_scale, err_msg="q_scale (per token)")
        assert not qs[:, :, w.Nq:].any()
        ks = qk.k_scale.cpu().numpy().reshape(w.B, w.Hkv, -1)
        ng = o.k_scale.shape[2]
        np.testing.assert_array_equal(ks[:, :, :ng], o.k_scale, err_msg="k_scale (per 32 keys)")
        assert not ks[:, :, ng:].any()
    # V^: [B, H, NB, Dp, 64] channel-major blocks -> [B, H, N_pad, Dp]
    B, H, NB = w.B, w.Hkv, qa.num_blocks(w.Nkv)
    raw = vq.v_hat.cpu()
    if w.pv == "fp8":
        bits = raw.numpy().reshape(B, H, NB, Dp, 64)
    else:
        bits = raw.view(torch.int16).numpy().view(np.uint16).reshape(B, H, NB, Dp, 64)
    tok = bits.transpose(0, 1, 2, 4, 3).reshape(B, H, NB * 64, Dp)
    ref_bits = oracle.v_hat_bits(o.v_hat, w.pv == "fp8")
    np.testing.assert_array_equal(tok[:, :, :w.Nkv, :w.D], ref_bits, err_msg="v_hat")
    assert not tok[:, :, w.Nkv:, :].any() and not tok[:, :, :, w.D:].any(), "v_hat padding not zero"
    if w.pv == "fp8":
        vs = vq.v_scale.cpu().numpy()
        np.testing.assert_array_equal(vs[:, :, :w.D], o.v_scale, err_msg="v_scale")
        assert not vs[:, :, w.D:].any()


def gather_rows(out: torch.Tensor, rows: np.ndarray, layout: str) -> np.ndarray:
    t = out.float()
    if layout == "NHD":
        t = t.transpose(1, 2)
    r = torch.from_numpy(rows).to(out.device)
    return t[r[:, 0], r[:, 1], r[:, 2]].double().cpu().numpy()


def metrics(a: np.ndarray, b: np.ndarray) -> Dict[str, float]:
    a = a.ravel()
    b = b.ravel()
    return {
        "max_abs": float(np.abs(a - b).max()),
        "cos": float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b))),
        "rel_l1": float(np.abs(a - b).sum() / np.abs(b).sum()),
    }


def compare_rows(got: np.ndarray, em_raw: np.ndarray, amb: np.ndarray, ex: Optional[np.ndarray], fmt: int,
                 pv: str) -> Dict[str, Dict[str, float]]:
    """The output acceptance test on gathered rows [R, D]: against the emulation,
    max-abs <= 1e-2 (one output ulp where that is wider) plus the ambiguity allowance
    and cosine >= 0.9999; against exact attention (if given) cosine >= 0.999 and
    relative L1 <= 3e-2 (FP16 P.V) / 5e-2 (FP8 P.V)."""
    assert np.isfinite(got).all()
    # the emulation's output is its fp64 result rounded to the output dtype
    em = oracle.round_to(em_raw, fmt)
    res = {"emulate": metrics(got, em)}
    res["emulate"]["ambiguity_max"] = float(amb.max())
    # max-abs <= 1e-2, except where one output ulp is wider than that (bf16 |o| >= 2):
    # both sides round independently computed values, so one ulp apart is allowed there;
    # plus the effect of P roundings that sit within 2^-14 of a tie (either side is right),
    # capped per element so that the allowance can never carry a large error
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(em), 1e-30))).astype(int) - (7 if fmt == oracle.BF16 else 10))
    base = np.maximum(1e-2, ulp)
    err = np.abs(got - em)
    res["emulate"]["worst_excess"] = float((err - base - np.minimum(amb, AMB_CAP)).max())
    res["emulate"]["needed_allowance"] = int((err > base).sum())   # elements inside only because of it
    res["emulate"]["elements"] = int(err.size)
    assert res["emulate"]["worst_excess"] <= 0 and res["emulate"]["cos"] >= 0.9999, res
    if ex is not None:
        res["exact"] = metrics(got, ex)
        bound = FP8_REL_L1 if pv == "fp8" else FP16_REL_L1
        assert res["exact"]["cos"] >= 0.999 and res["exact"]["rel_l1"] <= bound, res
    note(f"[metrics] {res}")
    return res


def check_output(case: Case, out: torch.Tensor, rows: np.ndarray, causal: Optional[bool] = None,
                 exact: bool = True) -> Dict[str, Dict[str, float]]:
    w = case.w
    c = w.causal if causal is None else causal
    got = gather_rows(out, rows, w.layout)
    assert np.isfinite(got).all()
    note(f"[oracle] emulate {len(rows)} rows")
    fmt = oracle.BF16 if w.dtype == "bf16" else oracle.FP16
    em_raw, amb = oracle.attn_emulate(case.oq, c, sm_scale_of(w.D), rows, with_ambiguity=True)
    ex = None
    if exact:
        note(f"[oracle] exact {len(rows)} rows")
        ex = oracle.attn_exact(case.qf, case.kf, case.vf, c, sm_scale_of(w.D), rows)
    return compare_rows(got, em_raw, amb, ex, fmt, w.pv)


def tile_sample(w: si.Workload, per_head_random: int = 8, heads: int = 4, seed: int = 0) -> np.ndarray:
    """(b, h, q_block, k_block): first, last, diagonal and random tiles of a few heads."""
    rng = np.random.default_rng(seed)
    nbq, nbk = qa.num_blocks(w.Nq), qa.num_blocks(w.Nkv)
    out = []
    pairs = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    pick = [pairs[i] for i in sorted(rng.choice(len(pairs), size=min(heads, len(pairs)), replace=False))]
    for b, h in pick:
        out += [(b, h, 0, 0), (b, h, nbq - 1, nbk - 1), (b, h, nbq - 1, 0), (b, h, 0, nbk - 1)]
        for d in range(0, min(nbq, nbk), max(1, min(nbq, nbk) // 4)):
            out.append((b, h, d, d))
        for _ in range(per_head_random):
            out.append((b, h, int(rng.integers(nbq)), int(rng.integers(nbk))))
    return np.asarray(out, dtype=np.int64)
