"""CPU oracle for SageAttention-style quantized attention (TEST INFRASTRUCTURE).

Only ``tests/``, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  It shares no code with the HIP path; its arithmetic
lives in ``oracle.c`` (see the header there for the passages each step
follows), and this wrapper only marshals numpy arrays.

Variable-length batches (``*_varlen``): the tokens of B sequences packed along one
axis, delimited by prefix sums cu_seqlens; the batch is, by definition here, the
dense scheme applied to every sequence on its own (its own K mean, block scales and
V scales; causal aligned per sequence).

Two modes:
  * ``attn_emulate``: the quantisation scheme replayed step by step (K mean
    smoothing, per-64-token INT8 Q/K, exact int32 scores, online exp2 softmax,
    P rounded to FP16 or FP8-e4m3, fp64 accumulation);
  * ``attn_exact``: softmax(sm_scale * Q K^T + mask) V in fp64.
Both work on a caller-chosen subset of query rows, given as (b, h, i) triples.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FP16, BF16, E4M3, E2M1 = 0, 1, 2, 3
BLK = 64

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_L = ctypes.c_long


def lib() -> ctypes.CDLL:
    """Load liboracle.so, building it with gcc first if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    L = ctypes.CDLL(_LIB_PATH)
    L.orc_version.restype = ctypes.c_int
    L.orc_threads.restype = ctypes.c_int
    L.orc_round.restype = ctypes.c_double
    L.orc_round.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_int]
    L.orc_round_array.argtypes = [_f64p, _L, ctypes.c_int, ctypes.c_int, _f64p]
    L.orc_k_mean.argtypes = [_f32p, _L, _L, _L, _L, _f32p]
    L.orc_quant_blocks.argtypes = [_f32p, ctypes.c_void_p, _L, _L, _L, _L, _i8p, _f32p]
    L.orc_quant_groups.argtypes = [_f32p, ctypes.c_void_p, _L, _L, _L, _L, _L, _i8p, _f32p]
    L.orc_quant_v.argtypes = [_f32p, _L, _L, _L, _L, ctypes.c_int, _f32p, _f32p]
    L.orc_scores_i32.argtypes = [_i8p, _i8p, _L, _L, _L, _L, _L, _L, _i64p, _L, _i32p]
    L.orc_attn_emulate.restype = _L
    L.orc_attn_emulate.argtypes = [_i8p, _f32p, _i8p, _f32p, _f32p, _f32p, ctypes.c_int, _L, _L, _L, _L, _L,
                                   _L, ctypes.c_int, ctypes.c_double, _i64p, _L, _f64p, ctypes.c_void_p]
    L.orc_attn_emulate_g.restype = _L
    L.orc_attn_emulate_g.argtypes = [_i8p, _f32p, _i8p, _f32p, _f32p, _f32p, ctypes.c_int, _L, _L, _L, _L, _L,
                                     _L, _L, _L, ctypes.c_int, ctypes.c_double, _i64p, _L, _f64p, ctypes.c_void_p]
    L.orc_attn_breakdown.argtypes = [_f32p, _f32p, _f32p, _i8p, _f32p, _i8p, _f32p, _f32p, _f32p, ctypes.c_int, _L,
                                     _L, _L, _L, _L, _L, ctypes.c_int, ctypes.c_double, _i64p, _L, ctypes.c_int,
                                     _f64p]
    L.orc_tie_flip.restype = ctypes.c_double
    L.orc_tie_flip.argtypes = [ctypes.c_double, ctypes.c_int]
    L.orc_mx_p_block.argtypes = [_f64p, _f32p, _i32p, _L, _f64p, _f64p]
    L.orc_attn_exact.argtypes = [_f32p, _f32p, _f32p, _L, _L, _L, _L, _L, _L, ctypes.c_int, ctypes.c_double,
                                 _i64p, _L, _f64p]
    L.orc_mx_exp.restype = ctypes.c_int
    L.orc_mx_exp.argtypes = [ctypes.c_double]
    L.orc_e2m1_value.restype = ctypes.c_double
    L.orc_e2m1_value.argtypes = [ctypes.c_int]
    L.orc_e2m1_code.restype = ctypes.c_int
    L.orc_e2m1_code.argtypes = [ctypes.c_double]
    L.orc_quant_mxfp4_rows.argtypes = [_f32p, ctypes.c_void_p, _L, _L, _L, _L, _u8p, _i32p]
    L.orc_quant_mxfp4_tokens.argtypes = [_f32p, _L, _L, _L, _L, _u8p, _i32p]
    L.orc_attn_emulate_mxfp4.restype = _L
    L.orc_attn_emulate_mxfp4.argtypes = [_u8p, _i32p, _u8p, _i32p, _u8p, _i32p, _L, _L, _L, _L, _L, _L,
                                         ctypes.c_int, ctypes.c_double, _i64p, _L, _f64p, ctypes.c_void_p]
    _lib = L
    return L


def threads() -> int:
    return int(lib().orc_threads())


# ----------------------------------------------------------------------------- helpers

def to_hnd_f32(x, layout: str) -> np.ndarray:
    """fp16/bf16 torch tensor in HND or NHD -> float32 numpy (B, H, N, D) (exact upcast)."""
    a = x.float().cpu().numpy()
    if layout == "NHD":
        a = a.transpose(0, 2, 1, 3)
    elif layout != "HND":
        raise ValueError(layout)
    return np.ascontiguousarray(a, dtype=np.float32)


def round_to(x: np.ndarray, fmt: int, sat: bool = False) -> np.ndarray:
    """Round reals to fp16 / bf16 / e4m3fn values (RNE); returns float64 values."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    lib().orc_round_array(x.reshape(-1), x.size, int(fmt), int(bool(sat)), out.reshape(-1))
    return out


def all_rows(B: int, H: int, N: int) -> np.ndarray:
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    return np.ascontiguousarray(np.stack([b.ravel(), h.ravel(), i.ravel()], 1).astype(np.int64))


def sample_rows(B: int, H: int, N: int, per_head: int = 64, seed: int = 0) -> np.ndarray:
    """Per (b, h): first and last row of 8 evenly spaced 64-row blocks, the last
    row of the sequence, plus seeded random rows, ``per_head`` rows in total."""
    rng = np.random.default_rng(seed)
    nblk = (N + BLK - 1) // BLK
    out = []
    for b in range(B):
        for h in range(H):
            sel = set()
            for t in np.linspace(0, nblk - 1, num=min(8, nblk)).astype(int):
                sel.add(int(t) * BLK)
                sel.add(min(int(t) * BLK + BLK - 1, N - 1))
            sel.add(N - 1)
            while len(sel) < min(per_head, N):
                sel.add(int(rng.integers(0, N)))
            out.extend((b, h, i) for i in sorted(sel))
    return np.asarray(out, dtype=np.int64)


# ----------------------------------------------------------------------------- quantisation

def k_mean(k: np.ndarray) -> np.ndarray:
    B, H, N, D = k.shape
    out = np.empty((B, H, D), np.float32)
    lib().orc_k_mean(np.ascontiguousarray(k, np.float32), B, H, N, D, out)
    return out


def quant_blocks(x: np.ndarray, mean: Optional[np.ndarray] = None):
    """Per-64-token INT8 quantisation; returns (int8 [B,H,N,D], scale [B,H,NB])."""
    B, H, N, D = x.shape
    nb = (N + BLK - 1) // BLK
    xq = np.empty((B, H, N, D), np.int8)
    sc = np.empty((B, H, nb), np.float32)
    mp = None
    if mean is not None:
        mean = np.ascontiguousarray(mean, np.float32)
        assert mean.shape == (B, H, D)
        mp = mean.ctypes.data_as(ctypes.c_void_p)
    lib().orc_quant_blocks(np.ascontiguousarray(x, np.float32), mp, B, H, N, D, xq, sc)
    return xq, sc


def quant_groups(x: np.ndarray, G: int, mean: Optional[np.ndarray] = None):
    """INT8 quantisation with one scale per G consecutive tokens (G = 64: quant_blocks);
    returns (int8 [B,H,N,D], scale [B,H,ceil(N/G)])."""
    B, H, N, D = x.shape
    ng = (N + G - 1) // G
    xq = np.empty((B, H, N, D), np.int8)
    sc = np.empty((B, H, ng), np.float32)
    mp = None
    if mean is not None:
        mean = np.ascontiguousarray(mean, np.float32)
        assert mean.shape == (B, H, D)
        mp = mean.ctypes.data_as(ctypes.c_void_p)
    lib().orc_quant_groups(np.ascontiguousarray(x, np.float32), mp, B, H, N, D, int(G), xq, sc)
    return xq, sc


# Quantisation granularities: tokens per Q scale and per K scale.  "thread" is the
# gfx950 reading of the README's per-thread quantisation (one scale per query row,
# one per 32 keys: the groups one lane / one half-wave owns in the score MFMA).
GRANULARITY = {"block": (64, 64), "thread": (1, 32)}


def quant_v(v: np.ndarray, pv_fp8: bool):
    """V operand: (values float32 [B,H,N,D], vscale float32 [B,H,D] or None)."""
    B, H, N, D = v.shape
    vh = np.empty((B, H, N, D), np.float32)
    vs = np.zeros((B, H, D), np.float32)
    lib().orc_quant_v(np.ascontiguousarray(v, np.float32), B, H, N, D, int(bool(pv_fp8)), vh, vs)
    return vh, (vs if pv_fp8 else None)


@dataclasses.dataclass
class Quantized:
    q_i8: np.ndarray
    q_scale: np.ndarray
    k_i8: np.ndarray
    k_scale: np.ndarray
    k_mean: np.ndarray
    v_hat: np.ndarray            # exact values of the fp16 / e4m3 codes, float32
    v_scale: Optional[np.ndarray]
    pv_fp8: bool
    Hq: int
    Hkv: int
    qg: int = 64   # tokens per Q scale
    kg: int = 64   # tokens per K scale


def quantize(q: np.ndarray, k: np.ndarray, v: np.ndarray, pv_fp8: bool, gran: str = "block") -> Quantized:
    """q, k, v: float32 (B, H, N, D) arrays holding the exact fp16/bf16 inputs."""
    qg, kg = GRANULARITY[gran]
    mu = k_mean(k)
    q8, sq = quant_groups(q, qg)
    k8, sk = quant_groups(k, kg, mu)
    vh, vs = quant_v(v, pv_fp8)
    return Quantized(q8, sq, k8, sk, mu, vh, vs, bool(pv_fp8), q.shape[1], k.shape[1], qg, kg)


def v_hat_bits(vals: np.ndarray, pv_fp8: bool) -> np.ndarray:
    """Storage bits (uint8 e4m3fn or uint16 fp16) of exactly representable values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(vals, np.float32))
    if pv_fp8:
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------- scores / attention

def scores_i32(Q: Quantized, tiles: Sequence[Sequence[int]]) -> np.ndarray:
    """INT32 score tiles [T, 64, 64] for (b, h, q_block, k_block) quadruples."""
    B, Hq, Nq, D = Q.q_i8.shape
    Nkv = Q.k_i8.shape[2]
    t = np.ascontiguousarray(np.asarray(tiles, np.int64).reshape(-1, 4))
    out = np.empty((t.shape[0], BLK, BLK), np.int32)
    lib().orc_scores_i32(Q.q_i8, Q.k_i8, B, Hq, Q.Hkv, Nq, Nkv, D, t, t.shape[0], out)
    return out


AMB_REL = 2.0 ** -14    # relative distance from a rounding tie within which either code is correct
SCORE_RANGE = 1024.0    # |S2| below which that margin covers every fp32 evaluation of p


class ScoreRangeError(ValueError):
    """The tie margin was asked for on rows whose scores leave the range in which it holds."""


def _range_check(bad: int, with_ambiguity: bool) -> None:
    if with_ambiguity and bad:
        raise ScoreRangeError(f"{bad} row(s) have a score or running max with |S2| >= {SCORE_RANGE:g} (log2 "
                              f"units) where p can still round to a nonzero code: the 2^-14 tie margin is not "
                              f"defined there")


def tie_flip(x: float, fmt: int) -> float:
    """|code_hi - code_lo| when x (> 0) lies within a relative 2^-14 of a rounding tie of
    format fmt, else 0 (the per-P term of the ambiguity allowance)."""
    return float(lib().orc_tie_flip(float(x), int(fmt)))


def attn_emulate(Q: Quantized, causal: bool, sm_scale: float, rows: np.ndarray, with_ambiguity: bool = False):
    """Emulation-mode rows [R, D] (fp64).  With with_ambiguity, also the per-element
    effect of flipping the P roundings that lie within 2^-14 (relative) of a tie; that
    margin holds while the scores that matter stay below 2^10 in magnitude, and
    ScoreRangeError is raised for rows beyond it."""
    B, Hq, Nq, D = Q.q_i8.shape
    Nkv = Q.k_i8.shape[2]
    rows = np.ascontiguousarray(rows, np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], D), np.float64)
    amb = np.empty((rows.shape[0], D), np.float64) if with_ambiguity else None
    vs = Q.v_scale if Q.v_scale is not None else np.zeros((B, Q.Hkv, D), np.float32)
    bad = lib().orc_attn_emulate_g(Q.q_i8, Q.q_scale, Q.k_i8, Q.k_scale, Q.v_hat, vs, int(Q.pv_fp8), B, Hq, Q.Hkv,
                                   Nq, Nkv, D, int(Q.qg), int(Q.kg), int(bool(causal)), float(sm_scale), rows,
                                   rows.shape[0], out, None if amb is None else amb.ctypes.data_as(ctypes.c_void_p))
    _range_check(bad, with_ambiguity)
    return (out, amb) if with_ambiguity else out


# approximations of the scheme that attn_breakdown can switch on one at a time
PART_QK, PART_P, PART_V = 1, 2, 4


def attn_breakdown(q: np.ndarray, k: np.ndarray, v: np.ndarray, Q: Quantized, causal: bool, sm_scale: float,
                   rows: np.ndarray, parts: int) -> np.ndarray:
    """Rows [R, D] (fp64) of attention with the chosen approximations of the scheme on
    (PART_QK: INT8 scores, PART_P: P rounded to its P.V format, PART_V: V quantised) and
    the others exact; parts = 0 is exact attention.  Block granularity."""
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    rows = np.ascontiguousarray(rows, np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], D), np.float64)
    vs = Q.v_scale if Q.v_scale is not None else np.zeros((B, Hkv, D), np.float32)
    lib().orc_attn_breakdown(np.ascontiguousarray(q, np.float32), np.ascontiguousarray(k, np.float32),
                             np.ascontiguousarray(v, np.float32), Q.q_i8, Q.q_scale, Q.k_i8, Q.k_scale, Q.v_hat, vs,
                             int(Q.pv_fp8), B, Hq, Hkv, Nq, Nkv, D, int(bool(causal)), float(sm_scale), rows,
                             rows.shape[0], int(parts), out)
    return out


def attn_exact(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, sm_scale: float,
               rows: np.ndarray) -> np.ndarray:
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    rows = np.ascontiguousarray(rows, np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], D), np.float64)
    lib().orc_attn_exact(np.ascontiguousarray(q, np.float32), np.ascontiguousarray(k, np.float32),
                         np.ascontiguousarray(v, np.float32), B, Hq, Hkv, Nq, Nkv, D, int(bool(causal)),
                         float(sm_scale), rows, rows.shape[0], out)
    return out


# ----------------------------------------------------------------------------- variable-length batches
# sageattn_varlen (SageAttention project README, "Available APIs" and "Project Updates"):
# several sequences of different lengths in one call.  Inputs are packed THD arrays
# (total_tokens, H, D) with int prefix sums cu (cu[0] = 0, cu[B] = total).

def _seq(x: np.ndarray, cu, b: int) -> np.ndarray:
    """Sequence b of a packed (total, H, D) array as a (1, H, n, D) float32 array."""
    return np.ascontiguousarray(x[int(cu[b]):int(cu[b + 1])].transpose(1, 0, 2)[None], dtype=np.float32)


def quantize_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, pv_fp8: bool, gran: str = "block"):
    """Per-sequence Quantized (None where the sequence has no key)."""
    out = []
    for b in range(len(cu_q) - 1):
        if int(cu_k[b + 1]) == int(cu_k[b]):
            out.append(None)
            continue
        out.append(quantize(_seq(q, cu_q, b), _seq(k, cu_k, b), _seq(v, cu_k, b), pv_fp8, gran))
    return out


def _per_sequence(rows: np.ndarray, D: int, fn):
    """rows (b, h, i) with i local to sequence b; fn(b, local_rows) -> [n, D] (or None = zeros)."""
    rows = np.asarray(rows, np.int64).reshape(-1, 3)
    out = np.zeros((rows.shape[0], D), np.float64)
    for b in np.unique(rows[:, 0]):
        sel = np.nonzero(rows[:, 0] == b)[0]
        local = rows[sel].copy()
        local[:, 0] = 0
        res = fn(int(b), np.ascontiguousarray(local))
        if res is not None:
            out[sel] = res
    return out


def attn_emulate_varlen(Qs, causal: bool, sm_scale: float, rows: np.ndarray, D: int, with_ambiguity: bool = False):
    """Emulation rows of a varlen batch; a sequence without keys outputs zeros."""
    amb_parts = {}

    def fn(b, local):
        if Qs[b] is None:
            return None
        o, a = attn_emulate(Qs[b], causal, sm_scale, local, with_ambiguity=True)
        amb_parts[b] = a
        return o

    out = _per_sequence(rows, D, fn)
    if not with_ambiguity:
        return out
    amb = _per_sequence(rows, D, lambda b, local: amb_parts.get(b))
    return out, amb


def attn_exact_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, causal: bool, sm_scale: float,
                      rows: np.ndarray) -> np.ndarray:
    D = q.shape[2]

    def fn(b, local):
        if int(cu_k[b + 1]) == int(cu_k[b]):
            return None
        return attn_exact(_seq(q, cu_q, b), _seq(k, cu_k, b), _seq(v, cu_k, b), causal, sm_scale, local)

    return _per_sequence(rows, D, fn)


# ----------------------------------------------------------------------------- microscaling FP4

MX_BLOCK = 32
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def mx_exp(amax: float) -> int:
    """Shared exponent of an MX block: floor(log2 amax) - 2, held to [-126, 127]."""
    return int(lib().orc_mx_exp(float(amax)))


def e2m1_decode(code) -> np.ndarray:
    """Values of 4-bit E2M1 codes (sign bit 8)."""
    c = np.asarray(code, np.int64)
    mag = np.asarray(E2M1_VALUES)[c & 7]
    return np.where(c & 8, -mag, mag)


def quant_mxfp4_rows(x: np.ndarray, mean: Optional[np.ndarray] = None):
    """Q or K (B, H, N, D) -> (codes uint8 [B,H,N,D], exponents int32 [B,H,N,ceil(D/32)]),
    blocks of 32 channels per token; ``mean`` (B, H, D) is subtracted first (fp32)."""
    B, H, N, D = x.shape
    code = np.empty((B, H, N, D), np.uint8)
    E = np.empty((B, H, N, (D + 31) // 32), np.int32)
    mp = None
    if mean is not None:
        mean = np.ascontiguousarray(mean, np.float32)
        assert mean.shape == (B, H, D)
        mp = mean.ctypes.data_as(ctypes.c_void_p)
    lib().orc_quant_mxfp4_rows(np.ascontiguousarray(x, np.float32), mp, B, H, N, D, code, E)
    return code, E


def quant_mxfp4_tokens(v: np.ndarray):
    """V (B, H, N, D) -> (codes uint8 [B,H,D,N] channel-major, exponents int32
    [B,H,D,ceil(N/32)]), blocks of 32 tokens per channel."""
    B, H, N, D = v.shape
    code = np.empty((B, H, D, N), np.uint8)
    E = np.empty((B, H, D, (N + 31) // 32), np.int32)
    lib().orc_quant_mxfp4_tokens(np.ascontiguousarray(v, np.float32), B, H, N, D, code, E)
    return code, E


def mx_dequant(code: np.ndarray, E: np.ndarray) -> np.ndarray:
    """Dequantised values (float64) of codes whose last axis is blocked by 32."""
    n = code.shape[-1]
    scale = np.repeat(np.ldexp(1.0, E.astype(np.int64)), MX_BLOCK, axis=-1)[..., :n]
    return e2m1_decode(code) * scale


@dataclasses.dataclass
class MXQuantized:
    q_code: np.ndarray   # [B, Hq, Nq, D]
    q_exp: np.ndarray    # [B, Hq, Nq, ceil(D/32)]
    k_code: np.ndarray   # [B, Hkv, Nkv, D] (smoothed K)
    k_exp: np.ndarray
    k_mean: np.ndarray   # [B, Hkv, D]
    v_code: np.ndarray   # [B, Hkv, D, Nkv]
    v_exp: np.ndarray    # [B, Hkv, D, ceil(Nkv/32)]
    Hq: int
    Hkv: int


def quantize_mxfp4(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> MXQuantized:
    """q, k, v: float32 (B, H, N, D) arrays holding the exact fp16/bf16 inputs."""
    mu = k_mean(k)
    qc, qe = quant_mxfp4_rows(q)
    kc, ke = quant_mxfp4_rows(k, mu)
    vc, ve = quant_mxfp4_tokens(v)
    return MXQuantized(qc, qe, kc, ke, mu, vc, ve, q.shape[1], k.shape[1])


def attn_emulate_mxfp4(Q: MXQuantized, causal: bool, sm_scale: float, rows: np.ndarray,
                       with_ambiguity: bool = False):
    """Emulation of the microscaling FP4 scheme for rows (b, h, i); [R, D] float64
    (and the per-element ambiguity allowance when asked)."""
    B, Hq, Nq, D = Q.q_code.shape
    Nkv = Q.k_code.shape[2]
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((len(rows), D), np.float64)
    amb = np.empty((len(rows), D), np.float64) if with_ambiguity else None
    bad = lib().orc_attn_emulate_mxfp4(Q.q_code, Q.q_exp, Q.k_code, Q.k_exp, Q.v_code, Q.v_exp, B, Hq, Q.Hkv, Nq,
                                       Nkv, D, int(bool(causal)), float(sm_scale), rows, len(rows), out,
                                       amb.ctypes.data_as(ctypes.c_void_p) if amb is not None else None)
    _range_check(bad, with_ambiguity)
    return (out, amb) if with_ambiguity else out


def mx_p_block(p: np.ndarray, t: np.ndarray, vis: Optional[np.ndarray] = None):
    """One 32-key block of P in the microscaling scheme: (dequantised values, ambiguity
    per element) for p = 2^t (float64 p, float32 t)."""
    p = np.ascontiguousarray(p, np.float64)
    t = np.ascontiguousarray(t, np.float32)
    vis = np.ones(p.shape, np.int32) if vis is None else np.ascontiguousarray(vis, np.int32)
    ph = np.empty_like(p)
    flip = np.empty_like(p)
    lib().orc_mx_p_block(p, t, vis, p.size, ph, flip)
    return ph, flip


def quantize_mxfp4_varlen(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k):
    """Per-sequence MXQuantized of a packed batch (None where the sequence has no key)."""
    out = []
    for b in range(len(cu_q) - 1):
        if int(cu_k[b + 1]) == int(cu_k[b]):
            out.append(None)
            continue
        out.append(quantize_mxfp4(_seq(q, cu_q, b), _seq(k, cu_k, b), _seq(v, cu_k, b)))
    return out


def attn_emulate_mxfp4_varlen(Qs, causal: bool, sm_scale: float, rows: np.ndarray, D: int,
                              with_ambiguity: bool = False):
    """MXFP4 emulation rows of a packed batch; a sequence without keys outputs zeros."""
    amb_parts = {}

    def fn(b, local):
        if Qs[b] is None:
            return None
        o, a = attn_emulate_mxfp4(Qs[b], causal, sm_scale, local, with_ambiguity=True)
        amb_parts[b] = a
        return o

    out = _per_sequence(rows, D, fn)
    if not with_ambiguity:
        return out
    amb = _per_sequence(rows, D, lambda b, local: amb_parts.get(b))
    return out, amb
