"""MI355X (gfx950) SageAttention-style quantized attention forward.

Thin Python binding over the C-ABI library ``libsage.so`` (include/sage.h).  The
binding only marshals arguments: every step of the computation runs in the HIP
kernels.  PyTorch provides device memory and the current stream.

Low level (same names as the C ABI; raw device pointers as ints):
    sage_quant_qk, sage_quant_v, sage_attn_fwd, sage_debug_qk_int32, ...
Tensor level:
    quant_qk(q, k, layout) -> QKQuant
    quant_v(v, layout, pv) -> VQuant
    attn_fwd(qk, vq, ...) -> out
    debug_qk_int32(qk, tiles, pv) -> int32 [T, 64, 64]
    sageattn(q, k, v, tensor_layout="HND", is_causal=False, sm_scale=None,
             pv="fp8", accum="fp32")   -- the composition of the three calls
Microscaling FP4 (OCP MXFP4 blocks of 32 on both products, head dim <= 256):
    quant_mxfp4(q, k, v, layout) -> MXQuant
    attn_fwd_mxfp4(mq, out_dtype, layout, is_causal, sm_scale) -> out
    sageattn_mxfp4(q, k, v, tensor_layout="HND", is_causal=False, sm_scale=None)
    quant_mxfp4_varlen, attn_fwd_mxfp4_varlen, sageattn_mxfp4_varlen (packed batches)
Packed variable-length batches (q (total_q, H, D), cu_seqlens prefix sums):
    quant_qk_varlen, quant_v_varlen, attn_fwd_varlen,
    sageattn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    is_causal=False, sm_scale=None, pv="fp16", accum="fp32")
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

__all__ = [
    "SageError", "lib", "library_path", "QKQuant", "VQuant", "quant_qk", "quant_v", "attn_fwd", "debug_qk_int32",
    "quant_qkv", "sageattn", "QKQuantVarlen", "VQuantVarlen", "quant_qk_varlen", "quant_v_varlen",
    "quant_qkv_varlen", "attn_fwd_varlen", "MXQuant", "quant_mxfp4", "attn_fwd_mxfp4", "sageattn_mxfp4",
    "MXQuantVarlen", "quant_mxfp4_varlen", "attn_fwd_mxfp4_varlen", "sageattn_mxfp4_varlen",
    "sageattn_varlen", "varlen_rows", "varlen_slots", "padded_dim", "num_blocks", "SAGE_OK", "SAGE_ERR_INVALID_ARG", "SAGE_ERR_UNSUPPORTED",
    "SAGE_ERR_WORKSPACE", "SAGE_ERR_DEVICE", "SAGE_ERR_HIP",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libsage.so")

SAGE_OK, SAGE_ERR_INVALID_ARG, SAGE_ERR_UNSUPPORTED, SAGE_ERR_WORKSPACE, SAGE_ERR_DEVICE, SAGE_ERR_HIP = range(6)
SAGE_FP16, SAGE_BF16 = 0, 1
SAGE_HND, SAGE_NHD = 0, 1
SAGE_PV_FP16, SAGE_PV_FP8 = 0, 1
SAGE_ACC_FP32, SAGE_ACC_FP16_FP32, SAGE_ACC_FP16, SAGE_ACC_FP16_FP32_SPLIT = 0, 1, 2, 3
SAGE_GRAN_BLOCK, SAGE_GRAN_THREAD = 0, 1

_EXPORTS = {
    # name: (restype, argtypes)
    "sage_abi_version": (ctypes.c_int, []),
    "sage_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sage_last_error_detail": (ctypes.c_char_p, []),
    "sage_padded_dim": (ctypes.c_int, [ctypes.c_int]),
    "sage_num_blocks": (ctypes.c_int, [ctypes.c_int]),
    "sage_quant_qk_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "sage_quant_qk": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_int] * 6
                      + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sage_quant_v_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "sage_quant_v": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_int] * 5
                     + [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sage_attn_fwd": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int, ctypes.c_int] + [ctypes.c_int] * 7
                      + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "sage_debug_qk_int32": (ctypes.c_int, [ctypes.c_void_p] * 2 + [ctypes.c_int] * 7
                            + [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "sage_varlen_rows": (ctypes.c_int64, [ctypes.c_int] * 2),
    "sage_varlen_slots": (ctypes.c_int64, [ctypes.c_int] * 2),
    "sage_quant_qk_varlen_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "sage_quant_qk_varlen": (ctypes.c_int, [ctypes.c_void_p] * 2 + [ctypes.c_int] + [ctypes.c_void_p] * 2
                             + [ctypes.c_int] * 8 + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sage_quant_v_varlen": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p] + [ctypes.c_int] * 6
                            + [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sage_attn_fwd_varlen": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] + [ctypes.c_void_p] * 2
                             + [ctypes.c_int] * 9 + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "sage_quant_qkv_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "sage_quant_qkv": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 2 + [ctypes.c_int] * 8
                       + [ctypes.c_void_p] * 8 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sage_quant_qkv_varlen_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "sage_quant_qkv_varlen": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] + [ctypes.c_void_p] * 2
                              + [ctypes.c_int] * 10 + [ctypes.c_void_p] * 8 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sage_attn_fwd_g": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int, ctypes.c_int] + [ctypes.c_int] * 7
                        + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "sage_quant_mxfp4_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "sage_quant_mxfp4": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 2 + [ctypes.c_int] * 6
                         + [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "sage_attn_fwd_mxfp4": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 2 + [ctypes.c_int] * 7
                            + [ctypes.c_float, ctypes.c_void_p]),
    "sage_quant_mxfp4_kv": (ctypes.c_int, [ctypes.c_void_p] * 2 + [ctypes.c_int] * 6 + [ctypes.c_void_p] * 6
                            + [ctypes.c_size_t, ctypes.c_void_p]),
    "sage_attn_fwd_mxfp4_fused_q": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 5
                                    + [ctypes.c_int] * 7 + [ctypes.c_float] + [ctypes.c_void_p] * 3),
    "sage_quant_mxfp4_varlen_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 4),
    "sage_quant_mxfp4_varlen": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] + [ctypes.c_void_p] * 2
                                + [ctypes.c_int] * 8 + [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_size_t,
                                                                                ctypes.c_void_p]),
    "sage_attn_fwd_mxfp4_varlen": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] + [ctypes.c_void_p] * 2
                                   + [ctypes.c_int] * 9 + [ctypes.c_float, ctypes.c_void_p]),
    "sage_attn_fwd_split_choice": (ctypes.c_int, [ctypes.c_int] * 6 + [ctypes.c_int]),
    "sage_attn_fwd_split_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "sage_attn_fwd_split": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] * 9
                            + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                               ctypes.c_size_t, ctypes.c_void_p]),
    "sage_quant_qkv_noalloc_max_bytes": (ctypes.c_size_t, []),
    "sage_quant_qkv_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 3 + [ctypes.c_int] * 10
                               + [ctypes.c_void_p] * 8),
    "sage_quant_kv_varlen": (ctypes.c_int, [ctypes.c_void_p] * 2 + [ctypes.c_int, ctypes.c_void_p] + [ctypes.c_int] * 6
                             + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]),
    "sage_attn_fwd_varlen_fused_q": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 7
                                     + [ctypes.c_int] * 9 + [ctypes.c_float, ctypes.c_int, ctypes.c_int]
                                     + [ctypes.c_void_p] * 3),
    "sage_quant_kv": (ctypes.c_int, [ctypes.c_void_p] * 2 + [ctypes.c_int] * 7 + [ctypes.c_void_p] * 6
                      + [ctypes.c_size_t, ctypes.c_void_p]),
    "sage_attn_fwd_fused_q": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 5
                              + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int, ctypes.c_int]
                              + [ctypes.c_void_p] * 3),
    "sage_attn_fwd_varlen_g": (ctypes.c_int, [ctypes.c_void_p] * 7 + [ctypes.c_int] + [ctypes.c_void_p] * 2
                               + [ctypes.c_int] * 9 + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                       ctypes.c_void_p]),
}

_lib = None


class SageError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{_status_string(status)} -- {detail}")


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libsage.so.  Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m quantized_attention_04_amd.build` "
                          "(the HIP library is the only implementation)")
    L = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _EXPORTS.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if L.sage_abi_version() != 6:
        raise ImportError("libsage ABI version mismatch")
    _lib = L
    return L


def _status_string(s: int) -> str:
    try:
        return lib().sage_status_string(s).decode()
    except Exception:  # pragma: no cover
        return f"status {s}"


def _check(status: int) -> None:
    if status != SAGE_OK:
        raise SageError(status, lib().sage_last_error_detail().decode())


def padded_dim(D: int) -> int:
    return int(lib().sage_padded_dim(D))


def num_blocks(N: int) -> int:
    return int(lib().sage_num_blocks(N))


# ----------------------------------------------------------------------------- tensor helpers

_DT = {torch.float16: SAGE_FP16, torch.bfloat16: SAGE_BF16}
_GRAN = {"block": SAGE_GRAN_BLOCK, "thread": SAGE_GRAN_THREAD}
_LAYOUT = {"HND": SAGE_HND, "NHD": SAGE_NHD}
_PV = {"fp16": SAGE_PV_FP16, "fp8": SAGE_PV_FP8}
# "fp16+fp32" runs the fp32 single-level accumulation (gfx950 matrix cores accumulate in fp32);
# "fp16+fp32-split": the literal two-level form (a fresh fp32 partial per 64-key tile plus a
# vector add), within one output ulp of it
_ACC = {"fp32": SAGE_ACC_FP32, "fp16+fp32": SAGE_ACC_FP16_FP32, "fp32+fp16": SAGE_ACC_FP16_FP32,
        "fp16": SAGE_ACC_FP16, "fp16+fp32-split": SAGE_ACC_FP16_FP32_SPLIT}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _dims(x: torch.Tensor, layout: str):
    if x.dim() != 4:
        raise ValueError(f"expected a 4-D tensor, got shape {tuple(x.shape)}")
    if layout == "HND":
        B, H, N, D = x.shape
    elif layout == "NHD":
        B, N, H, D = x.shape
    else:
        raise ValueError(f"tensor_layout must be 'HND' or 'NHD', got {layout!r}")
    return B, H, N, D


def _check_input(x: torch.Tensor, name: str) -> None:
    if x.dtype not in _DT:
        raise ValueError(f"{name}: dtype must be float16 or bfloat16, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


@dataclasses.dataclass
class QKQuant:
    q_i8: torch.Tensor      # int8 [B, Hq, N_pad(Nq), Dp]
    q_scale: torch.Tensor   # f32  [B, Hq, NB(Nq)]
    k_i8: torch.Tensor      # int8 [B, Hkv, N_pad(Nkv), Dp]
    k_scale: torch.Tensor   # f32  [B, Hkv, NB(Nkv)]
    k_mean: torch.Tensor    # f32  [B, Hkv, D]
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    gran: str = "block"     # "thread": q_scale [B, Hq, N_pad(Nq)] per token, k_scale [B, Hkv, NB(Nkv), 2]


@dataclasses.dataclass
class VQuant:
    v_hat: torch.Tensor               # uint8 [B, Hkv, NB, Dp, 64*elt] (fp16 or e4m3 bytes)
    v_scale: Optional[torch.Tensor]   # f32 [B, Hkv, Dp] (FP8 only)
    pv: str


def quant_qk(q: torch.Tensor, k: torch.Tensor, layout: str = "HND", workspace: Optional[torch.Tensor] = None,
             out: Optional[QKQuant] = None) -> QKQuant:
    _check_input(q, "q")
    _check_input(k, "k")
    if q.dtype != k.dtype or q.device != k.device:
        raise ValueError("q and k must share dtype and device")
    B, Hq, Nq, D = _dims(q, layout)
    Bk, Hkv, Nkv, Dk = _dims(k, layout)
    if Bk != B or Dk != D:
        raise ValueError("q and k disagree on batch or head_dim")
    L = lib()
    Dp, nbq, nbk = padded_dim(D), num_blocks(Nq), num_blocks(Nkv)
    dev = q.device
    if out is None:
        out = QKQuant(torch.empty(B, Hq, nbq * 64, max(Dp, 1), dtype=torch.int8, device=dev),
                      torch.empty(B, Hq, nbq, dtype=torch.float32, device=dev),
                      torch.empty(B, Hkv, nbk * 64, max(Dp, 1), dtype=torch.int8, device=dev),
                      torch.empty(B, Hkv, nbk, dtype=torch.float32, device=dev),
                      torch.empty(B, Hkv, D, dtype=torch.float32, device=dev), B, Hq, Hkv, Nq, Nkv, D)
    need = L.sage_quant_qk_workspace_bytes(B, Hkv, Nkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    _check(L.sage_quant_qk(q.data_ptr(), k.data_ptr(), _DT[q.dtype], _LAYOUT[layout], B, Hq, Hkv, Nq, Nkv, D,
                           out.q_i8.data_ptr(), out.q_scale.data_ptr(), out.k_i8.data_ptr(), out.k_scale.data_ptr(),
                           out.k_mean.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(dev)))
    return out


def quant_v(v: torch.Tensor, layout: str = "HND", pv: str = "fp8", workspace: Optional[torch.Tensor] = None,
            out: Optional[VQuant] = None) -> VQuant:
    _check_input(v, "v")
    if pv not in _PV:
        raise ValueError(f"pv must be 'fp16' or 'fp8', got {pv!r}")
    B, Hkv, Nkv, D = _dims(v, layout)
    L = lib()
    Dp, nb = padded_dim(D), num_blocks(Nkv)
    dev = v.device
    elt = 1 if pv == "fp8" else 2
    if out is None:
        out = VQuant(torch.empty(B, Hkv, nb, max(Dp, 1), 64 * elt, dtype=torch.uint8, device=dev),
                     torch.empty(B, Hkv, max(Dp, 1), dtype=torch.float32, device=dev) if pv == "fp8" else None, pv)
    need = L.sage_quant_v_workspace_bytes(B, Hkv, D, _PV[pv])
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(L.sage_quant_v(v.data_ptr(), _DT[v.dtype], _LAYOUT[layout], B, Hkv, Nkv, D, _PV[pv], out.v_hat.data_ptr(),
                          _ptr(out.v_scale), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                          _stream(dev)))
    return out


def split_choice(qk: QKQuant, pv: str, is_causal: bool = False) -> int:
    """The library's key-range split count for this launch (1: no split)."""
    return int(lib().sage_attn_fwd_split_choice(qk.B, qk.Hq, qk.Nq, qk.Nkv, qk.D, int(bool(is_causal)), _PV[pv]))


def split_workspace_bytes(qk: QKQuant, splits: int) -> int:
    return int(lib().sage_attn_fwd_split_workspace_bytes(qk.B, qk.Hq, qk.Nq, qk.D, int(splits)))


def attn_fwd(qk: QKQuant, vq: VQuant, out_dtype: torch.dtype, layout: str = "HND", is_causal: bool = False,
             sm_scale: Optional[float] = None, accum: str = "fp32", out: Optional[torch.Tensor] = None,
             splits=1, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sage_attn_fwd (or sage_attn_fwd_g).  splits: key-range splits of every query tile
    (sage_attn_fwd_split; FP16 P.V, block granularity), an int or "auto" for the
    library's choice; workspace: the splits' fp32 state (allocated here if None)."""
    if out_dtype not in _DT:
        raise ValueError("out_dtype must be float16 or bfloat16")
    if accum not in _ACC:
        raise ValueError(f"accum must be one of {sorted(_ACC)}, got {accum!r}")
    B, Hq, Hkv, Nq, Nkv, D = qk.B, qk.Hq, qk.Hkv, qk.Nq, qk.Nkv, qk.D
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dev = qk.q_i8.device
    if out is None:
        shape = (B, Hq, Nq, D) if layout == "HND" else (B, Nq, Hq, D)
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    args = (qk.q_i8.data_ptr(), qk.q_scale.data_ptr(), qk.k_i8.data_ptr(), qk.k_scale.data_ptr(), vq.v_hat.data_ptr(),
            _ptr(vq.v_scale), out.data_ptr(), _DT[out_dtype], _LAYOUT[layout], B, Hq, Hkv, Nq, Nkv, D,
            int(bool(is_causal)), float(sm_scale), _PV[vq.pv], _ACC[accum])
    if splits == "auto":
        splits = split_choice(qk, vq.pv, is_causal) if qk.gran == "block" and accum != "fp16+fp32-split" else 1
    splits = int(splits)
    if splits > 1:
        need = split_workspace_bytes(qk, splits)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        _check(lib().sage_attn_fwd_split(*args, splits, workspace.data_ptr(), workspace.numel(), _stream(dev)))
    elif qk.gran == "block":
        _check(lib().sage_attn_fwd(*args, _stream(dev)))
    else:
        _check(lib().sage_attn_fwd_g(*args, _GRAN[qk.gran], _stream(dev)))
    return out


def debug_qk_int32(qk: QKQuant, tiles: torch.Tensor, pv: str = "fp8") -> torch.Tensor:
    """INT32 score tiles through the attention kernel's operand path; tiles int32 [T, 4] on the GPU."""
    tiles = tiles.to(torch.int32).contiguous()
    T = tiles.shape[0]
    out = torch.empty(T, 64, 64, dtype=torch.int32, device=qk.q_i8.device)
    _check(lib().sage_debug_qk_int32(qk.q_i8.data_ptr(), qk.k_i8.data_ptr(), qk.B, qk.Hq, qk.Hkv, qk.Nq, qk.Nkv, qk.D,
                                     _PV[pv], tiles.data_ptr(), T, out.data_ptr(), _stream(qk.q_i8.device)))
    return out


def quant_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: str = "HND", pv: str = "fp8",
              workspace: Optional[torch.Tensor] = None, out_qk: Optional[QKQuant] = None,
              out_v: Optional[VQuant] = None, gran: str = "block", noalloc: bool = False):
    """quant_qk and quant_v in one library call (same outputs, fewer kernel launches).
    gran="thread": one Q scale per token and one K scale per 32 keys.
    noalloc=True: sage_quant_qkv_noalloc, whose workspace is the library's static device
    scratch (nothing is allocated for the call once out_qk and out_v are given)."""
    if gran not in _GRAN:
        raise ValueError(f"gran must be 'block' or 'thread', got {gran!r}")
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_input(x, name)
    if not (q.dtype == k.dtype == v.dtype) or not (q.device == k.device == v.device):
        raise ValueError("q, k and v must share dtype and device")
    if pv not in _PV:
        raise ValueError(f"pv must be 'fp16' or 'fp8', got {pv!r}")
    B, Hq, Nq, D = _dims(q, layout)
    Bk, Hkv, Nkv, Dk = _dims(k, layout)
    if Bk != B or Dk != D or _dims(v, layout) != (B, Hkv, Nkv, D):
        raise ValueError("q, k and v disagree on batch, heads, length or head_dim")
    L = lib()
    Dp, nbq, nbk = padded_dim(D), num_blocks(Nq), num_blocks(Nkv)
    dev = q.device
    if out_qk is None:
        thr = gran == "thread"
        out_qk = QKQuant(torch.empty(B, Hq, nbq * 64, max(Dp, 1), dtype=torch.int8, device=dev),
                         torch.empty(B, Hq, nbq * 64 if thr else nbq, dtype=torch.float32, device=dev),
                         torch.empty(B, Hkv, nbk * 64, max(Dp, 1), dtype=torch.int8, device=dev),
                         torch.empty((B, Hkv, nbk, 2) if thr else (B, Hkv, nbk), dtype=torch.float32, device=dev),
                         torch.empty(B, Hkv, D, dtype=torch.float32, device=dev), B, Hq, Hkv, Nq, Nkv, D, gran)
    elif out_qk.gran != gran:
        raise ValueError("out_qk was allocated for another granularity")
    if out_v is None:
        elt = 1 if pv == "fp8" else 2
        out_v = VQuant(torch.empty(B, Hkv, nbk, max(Dp, 1), 64 * elt, dtype=torch.uint8, device=dev),
                       torch.empty(B, Hkv, max(Dp, 1), dtype=torch.float32, device=dev) if pv == "fp8" else None, pv)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        _check(L.sage_quant_qkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DT[q.dtype], _LAYOUT[layout], B,
                                        Hq, Hkv, Nq, Nkv, D, _PV[pv], _GRAN[gran], out_qk.q_i8.data_ptr(),
                                        out_qk.q_scale.data_ptr(), out_qk.k_i8.data_ptr(), out_qk.k_scale.data_ptr(),
                                        out_qk.k_mean.data_ptr(), out_v.v_hat.data_ptr(), _ptr(out_v.v_scale),
                                        _stream(dev)))
        return out_qk, out_v
    need = L.sage_quant_qkv_workspace_bytes(B, Hkv, Nkv, D, _PV[pv])
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    _check(L.sage_quant_qkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DT[q.dtype], _LAYOUT[layout], B, Hq, Hkv, Nq,
                            Nkv, D, _PV[pv], _GRAN[gran], out_qk.q_i8.data_ptr(), out_qk.q_scale.data_ptr(),
                            out_qk.k_i8.data_ptr(), out_qk.k_scale.data_ptr(), out_qk.k_mean.data_ptr(),
                            out_v.v_hat.data_ptr(), _ptr(out_v.v_scale), workspace.data_ptr(), workspace.numel(),
                            _stream(dev)))
    return out_qk, out_v


@dataclasses.dataclass
class MXQuant:
    """Outputs of sage_quant_mxfp4 (layouts in include/sage.h, "Microscaling FP4")."""
    q4: torch.Tensor       # uint8 [B, Hq, N_pad(Nq), Dp/2]   E2M1 codes, two per byte
    q4_exp: torch.Tensor   # uint8 [B, Hq, N_pad(Nq), Dp/32]  E8M0 block exponents
    k4: torch.Tensor       # uint8 [B, Hkv, N_pad(Nkv), Dp/2] (smoothed K)
    k4_exp: torch.Tensor   # uint8 [B, Hkv, N_pad(Nkv), Dp/32]
    k_mean: torch.Tensor   # f32   [B, Hkv, D]
    v4: torch.Tensor       # uint8 [B, Hkv, NB(Nkv), Dp, 32]
    v4_exp: torch.Tensor   # uint8 [B, Hkv, NB(Nkv), 2, 32, Dp/32]
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int


def quant_mxfp4(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, layout: str = "HND",
                workspace: Optional[torch.Tensor] = None, out: Optional[MXQuant] = None) -> MXQuant:
    """K mean, then MXFP4 codes and block exponents of Q, smoothed K and V in one call."""
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_input(x, name)
    if not (q.dtype == k.dtype == v.dtype) or not (q.device == k.device == v.device):
        raise ValueError("q, k and v must share dtype and device")
    B, Hq, Nq, D = _dims(q, layout)
    Bk, Hkv, Nkv, Dk = _dims(k, layout)
    if Bk != B or Dk != D or _dims(v, layout) != (B, Hkv, Nkv, D):
        raise ValueError("q, k and v disagree on batch, heads, length or head_dim")
    L = lib()
    Dp, nbq, nbk = padded_dim(D), num_blocks(Nq), num_blocks(Nkv)
    Dp = max(Dp, 64)
    dev = q.device
    if out is None:
        u8 = dict(dtype=torch.uint8, device=dev)
        out = MXQuant(torch.empty(B, Hq, nbq * 64, Dp // 2, **u8), torch.empty(B, Hq, nbq * 64, Dp // 32, **u8),
                      torch.empty(B, Hkv, nbk * 64, Dp // 2, **u8), torch.empty(B, Hkv, nbk * 64, Dp // 32, **u8),
                      torch.empty(B, Hkv, D, dtype=torch.float32, device=dev),
                      torch.empty(B, Hkv, nbk, Dp, 32, **u8), torch.empty(B, Hkv, nbk, 2, 32, Dp // 32, **u8),
                      B, Hq, Hkv, Nq, Nkv, D)
    need = L.sage_quant_mxfp4_workspace_bytes(B, Hkv, Nkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    _check(L.sage_quant_mxfp4(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DT[q.dtype], _LAYOUT[layout], B, Hq, Hkv, Nq,
                              Nkv, D, out.q4.data_ptr(), out.q4_exp.data_ptr(), out.k4.data_ptr(),
                              out.k4_exp.data_ptr(), out.k_mean.data_ptr(), out.v4.data_ptr(), out.v4_exp.data_ptr(),
                              workspace.data_ptr(), workspace.numel(), _stream(dev)))
    return out


def attn_fwd_mxfp4(mq: MXQuant, out_dtype: torch.dtype, layout: str = "HND", is_causal: bool = False,
                   sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out_dtype not in _DT:
        raise ValueError("out_dtype must be float16 or bfloat16")
    if layout not in _LAYOUT:
        raise ValueError(f"layout must be 'HND' or 'NHD', got {layout!r}")
    B, Hq, Hkv, Nq, Nkv, D = mq.B, mq.Hq, mq.Hkv, mq.Nq, mq.Nkv, mq.D
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    dev = mq.q4.device
    if out is None:
        shape = (B, Hq, Nq, D) if layout == "HND" else (B, Nq, Hq, D)
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    _check(lib().sage_attn_fwd_mxfp4(mq.q4.data_ptr(), mq.q4_exp.data_ptr(), mq.k4.data_ptr(), mq.k4_exp.data_ptr(),
                                     mq.v4.data_ptr(), mq.v4_exp.data_ptr(), out.data_ptr(), _DT[out_dtype],
                                     _LAYOUT[layout], B, Hq, Hkv, Nq, Nkv, D, int(bool(is_causal)), float(sm_scale),
                                     _stream(dev)))
    return out


@dataclasses.dataclass
class MXKQuant:
    """Outputs of sage_quant_mxfp4_kv: MXQuant's K and V parts."""
    k4: torch.Tensor
    k4_exp: torch.Tensor
    k_mean: torch.Tensor
    v4: torch.Tensor
    v4_exp: torch.Tensor
    B: int
    Hkv: int
    Nkv: int
    D: int


def quant_mxfp4_kv(k: torch.Tensor, v: torch.Tensor, layout: str = "HND", workspace: Optional[torch.Tensor] = None,
                   out: Optional[MXKQuant] = None) -> MXKQuant:
    """sage_quant_mxfp4_kv: the K mean and the MXFP4 codes and exponents of smoothed K and of V
    (for attn_fwd_mxfp4_fused_q, which quantises Q itself)."""
    for name, x in (("k", k), ("v", v)):
        _check_input(x, name)
    if k.dtype != v.dtype or k.device != v.device:
        raise ValueError("k and v must share dtype and device")
    B, Hkv, Nkv, D = _dims(k, layout)
    if _dims(v, layout) != (B, Hkv, Nkv, D):
        raise ValueError("k and v disagree on batch, heads, length or head_dim")
    L = lib()
    Dp, nbk = max(padded_dim(D), 64), num_blocks(Nkv)
    dev = k.device
    if out is None:
        u8 = dict(dtype=torch.uint8, device=dev)
        out = MXKQuant(torch.empty(B, Hkv, nbk * 64, Dp // 2, **u8), torch.empty(B, Hkv, nbk * 64, Dp // 32, **u8),
                       torch.empty(B, Hkv, D, dtype=torch.float32, device=dev),
                       torch.empty(B, Hkv, nbk, Dp, 32, **u8), torch.empty(B, Hkv, nbk, 2, 32, Dp // 32, **u8),
                       B, Hkv, Nkv, D)
    need = L.sage_quant_mxfp4_workspace_bytes(B, Hkv, Nkv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    _check(L.sage_quant_mxfp4_kv(k.data_ptr(), v.data_ptr(), _DT[k.dtype], _LAYOUT[layout], B, Hkv, Nkv, D,
                                 out.k4.data_ptr(), out.k4_exp.data_ptr(), out.k_mean.data_ptr(), out.v4.data_ptr(),
                                 out.v4_exp.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(dev)))
    return out


def attn_fwd_mxfp4_fused_q(q: torch.Tensor, mk: MXKQuant, layout: str = "HND", is_causal: bool = False,
                           sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                           q_codes: Optional[tuple] = None) -> torch.Tensor:
    """sage_attn_fwd_mxfp4_fused_q: MXFP4 attention that quantises Q (fp16 / bf16, dense) in
    its own prologue; output in q's dtype and layout.  q_codes: optional (q4, q4_exp)
    tensors, shaped as MXQuant's, that receive the codes and exponent bytes."""
    _check_input(q, "q")
    B, Hq, Nq, D = _dims(q, layout)
    if (mk.B, mk.D) != (B, D):
        raise ValueError("q and the K operand disagree on batch or head_dim")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    qc, qe = (None, None) if q_codes is None else q_codes
    _check(lib().sage_attn_fwd_mxfp4_fused_q(q.data_ptr(), _DT[q.dtype], _LAYOUT[layout], mk.k4.data_ptr(),
                                             mk.k4_exp.data_ptr(), mk.v4.data_ptr(), mk.v4_exp.data_ptr(),
                                             out.data_ptr(), B, Hq, mk.Hkv, Nq, mk.Nkv, D, int(bool(is_causal)),
                                             float(sm_scale), _ptr(qc), _ptr(qe), _stream(q.device)))
    return out


def sageattn_mxfp4(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tensor_layout: str = "HND",
                   is_causal: bool = False, sm_scale: Optional[float] = None) -> torch.Tensor:
    """The microscaling FP4 variant (output in q's dtype and layout): quant_mxfp4_kv, then
    attn_fwd_mxfp4_fused_q, which quantises Q in its prologue -- the same codes and output
    as quant_mxfp4 followed by attn_fwd_mxfp4."""
    _check_input(q, "q")
    if q.dtype != k.dtype or q.device != k.device:
        raise ValueError("q, k and v must share dtype and device")
    mk = quant_mxfp4_kv(k, v, tensor_layout)
    return attn_fwd_mxfp4_fused_q(q, mk, tensor_layout, is_causal, sm_scale)


def sageattn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, tensor_layout: str = "HND", is_causal: bool = False,
             sm_scale: Optional[float] = None, pv: str = "fp8", accum: str = "fp32",
             qk_gran: str = "block") -> torch.Tensor:
    """softmax(sm_scale * q k^T [causal]) v with INT8 QK^T and FP8/FP16 PV; returns q's dtype and layout.
    qk_gran: "block" (one scale per 64 tokens) or "thread" (per query token, per 32 keys).
    Launches too small to fill the GPU take the library's key-range splits (FP16 P.V);
    otherwise, at block granularity, Q is quantised inside the attention kernel
    (sage_quant_kv + sage_attn_fwd_fused_q: the same codes and output, no Q codes in HBM)."""
    if pv not in _PV:
        raise ValueError(f"pv must be 'fp16' or 'fp8', got {pv!r}")
    B, Hq, Nq, D = _dims(q, tensor_layout)
    _, _, Nkv, _ = _dims(k, tensor_layout)
    if qk_gran == "block" and accum != "fp16+fp32-split" and \
            lib().sage_attn_fwd_split_choice(B, Hq, Nq, Nkv, D, int(bool(is_causal)), _PV[pv]) == 1:
        _check_input(q, "q")
        if q.dtype != k.dtype or q.device != k.device:
            raise ValueError("q, k and v must share dtype and device")
        kq, vq = quant_kv(k, v, tensor_layout, pv)
        return attn_fwd_fused_q(q, kq, vq, tensor_layout, is_causal, sm_scale, accum)
    qk, vq = quant_qkv(q, k, v, tensor_layout, pv, gran=qk_gran)
    return attn_fwd(qk, vq, q.dtype, tensor_layout, is_causal, sm_scale, accum, splits="auto")


# ----------------------------------------------------------------------------- variable-length batches
# sageattn_varlen (SageAttention project README, "Available APIs"): the tokens of B
# sequences packed along one axis, q (total_q, Hq, D) and k, v (total_kv, Hkv, D),
# delimited by int32 prefix sums cu_seqlens [B + 1] on the GPU.

def varlen_rows(total: int, B: int) -> int:
    return int(lib().sage_varlen_rows(total, B))


def varlen_slots(total: int, B: int) -> int:
    return int(lib().sage_varlen_slots(total, B))


@dataclasses.dataclass
class QKQuantVarlen:
    q_i8: torch.Tensor      # int8 [Hq, rows(total_q), Dp]
    q_scale: torch.Tensor   # f32  [Hq, slots(total_q)]
    k_i8: torch.Tensor      # int8 [Hkv, rows(total_kv), Dp]
    k_scale: torch.Tensor   # f32  [Hkv, slots(total_kv)]
    k_mean: torch.Tensor    # f32  [B, Hkv, D]
    cu_q: torch.Tensor
    cu_k: torch.Tensor
    B: int
    Hq: int
    Hkv: int
    total_q: int
    total_kv: int
    max_q: int
    max_k: int
    D: int
    gran: str = "block"     # "thread": q_scale [Hq, rows(total_q)], k_scale [Hkv, slots(total_kv), 2]


@dataclasses.dataclass
class VQuantVarlen:
    v_hat: torch.Tensor               # uint8 [Hkv, slots(total_kv), Dp, 64*elt]
    v_scale: Optional[torch.Tensor]   # f32 [B, Hkv, Dp] (FP8 only)
    pv: str


def _packed_dims(x: torch.Tensor, name: str):
    if x.dim() != 3:
        raise ValueError(f"{name}: expected a packed (total_tokens, heads, head_dim) tensor, got {tuple(x.shape)}")
    return x.shape


def _cu(cu: torch.Tensor, dev: torch.device, name: str) -> torch.Tensor:
    if cu.dim() != 1 or cu.numel() < 2:
        raise ValueError(f"{name}: expected a 1-D tensor of B + 1 prefix sums")
    if cu.device != dev:
        raise ValueError(f"{name}: must live on {dev}")
    return cu.to(torch.int32).contiguous()


def quant_qk_varlen(q: torch.Tensor, k: torch.Tensor, cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                    max_seqlen_q: int, max_seqlen_k: int, workspace: Optional[torch.Tensor] = None,
                    out: Optional[QKQuantVarlen] = None) -> QKQuantVarlen:
    _check_input(q, "q")
    _check_input(k, "k")
    if q.dtype != k.dtype or q.device != k.device:
        raise ValueError("q and k must share dtype and device")
    total_q, Hq, D = _packed_dims(q, "q")
    total_k, Hkv, Dk = _packed_dims(k, "k")
    if Dk != D:
        raise ValueError("q and k disagree on head_dim")
    dev = q.device
    cq, ck = _cu(cu_seqlens_q, dev, "cu_seqlens_q"), _cu(cu_seqlens_k, dev, "cu_seqlens_k")
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must describe the same number of sequences")
    B = cq.numel() - 1
    L = lib()
    Dp = padded_dim(D)
    if out is None:
        rq, sq, rk, sk = varlen_rows(total_q, B), varlen_slots(total_q, B), varlen_rows(total_k, B), varlen_slots(total_k, B)
        out = QKQuantVarlen(torch.empty(Hq, rq, max(Dp, 1), dtype=torch.int8, device=dev),
                            torch.empty(Hq, sq, dtype=torch.float32, device=dev),
                            torch.empty(Hkv, rk, max(Dp, 1), dtype=torch.int8, device=dev),
                            torch.empty(Hkv, sk, dtype=torch.float32, device=dev),
                            torch.empty(B, Hkv, D, dtype=torch.float32, device=dev), cq, ck, B, Hq, Hkv, total_q,
                            total_k, int(max_seqlen_q), int(max_seqlen_k), D)
    need = L.sage_quant_qk_varlen_workspace_bytes(B, Hkv, total_k, D)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    _check(L.sage_quant_qk_varlen(q.data_ptr(), k.data_ptr(), _DT[q.dtype], cq.data_ptr(), ck.data_ptr(), B, Hq, Hkv,
                                  total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D, out.q_i8.data_ptr(),
                                  out.q_scale.data_ptr(), out.k_i8.data_ptr(), out.k_scale.data_ptr(),
                                  out.k_mean.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(dev)))
    return out


def quant_v_varlen(v: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_k: int, pv: str = "fp16",
                   workspace: Optional[torch.Tensor] = None, out: Optional[VQuantVarlen] = None) -> VQuantVarlen:
    _check_input(v, "v")
    if pv not in _PV:
        raise ValueError(f"pv must be 'fp16' or 'fp8', got {pv!r}")
    total_k, Hkv, D = _packed_dims(v, "v")
    dev = v.device
    ck = _cu(cu_seqlens_k, dev, "cu_seqlens_k")
    B = ck.numel() - 1
    L = lib()
    Dp = padded_dim(D)
    elt = 1 if pv == "fp8" else 2
    if out is None:
        out = VQuantVarlen(torch.empty(Hkv, varlen_slots(total_k, B), max(Dp, 1), 64 * elt, dtype=torch.uint8,
                                       device=dev),
                           torch.empty(B, Hkv, max(Dp, 1), dtype=torch.float32, device=dev) if pv == "fp8" else None,
                           pv)
    need = L.sage_quant_v_workspace_bytes(B, Hkv, D, _PV[pv])
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(L.sage_quant_v_varlen(v.data_ptr(), _DT[v.dtype], ck.data_ptr(), B, Hkv, total_k, int(max_seqlen_k), D,
                                 _PV[pv], out.v_hat.data_ptr(), _ptr(out.v_scale), _ptr(workspace),
                                 0 if workspace is None else workspace.numel(), _stream(dev)))
    return out


@dataclasses.dataclass
class KQuant:
    k_i8: torch.Tensor      # int8 [B, Hkv, N_pad(Nkv), Dp]
    k_scale: torch.Tensor   # f32  [B, Hkv, NB(Nkv)]
    k_mean: torch.Tensor    # f32  [B, Hkv, D]
    B: int
    Hkv: int
    Nkv: int
    D: int


def quant_kv(k: torch.Tensor, v: torch.Tensor, layout: str = "HND", pv: str = "fp8",
             workspace: Optional[torch.Tensor] = None, out_k: Optional[KQuant] = None,
             out_v: Optional[VQuant] = None):
    """sage_quant_kv: the K and V part of quant_qkv (for attn_fwd_fused_q, which
    quantises Q itself); block granularity."""
    for name, x in (("k", k), ("v", v)):
        _check_input(x, name)
    if k.dtype != v.dtype or k.device != v.device:
        raise ValueError("k and v must share dtype and device")
    if pv not in _PV:
        raise ValueError(f"pv must be 'fp16' or 'fp8', got {pv!r}")
    B, Hkv, Nkv, D = _dims(k, layout)
    if _dims(v, layout) != (B, Hkv, Nkv, D):
        raise ValueError("k and v disagree on batch, heads, length or head_dim")
    L = lib()
    Dp, nbk = padded_dim(D), num_blocks(Nkv)
    dev = k.device
    if out_k is None:
        out_k = KQuant(torch.empty(B, Hkv, nbk * 64, max(Dp, 1), dtype=torch.int8, device=dev),
                       torch.empty(B, Hkv, nbk, dtype=torch.float32, device=dev),
                       torch.empty(B, Hkv, D, dtype=torch.float32, device=dev), B, Hkv, Nkv, D)
    if out_v is None:
        elt = 1 if pv == "fp8" else 2
        out_v = VQuant(torch.empty(B, Hkv, nbk, max(Dp, 1), 64 * elt, dtype=torch.uint8, device=dev),
                       torch.empty(B, Hkv, max(Dp, 1), dtype=torch.float32, device=dev) if pv == "fp8" else None, pv)
    need = L.sage_quant_qkv_workspace_bytes(B, Hkv, Nkv, D, _PV[pv])
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    _check(L.sage_quant_kv(k.data_ptr(), v.data_ptr(), _DT[k.dtype], _LAYOUT[layout], B, Hkv, Nkv, D, _PV[pv],
                           out_k.k_i8.data_ptr(), out_k.k_scale.data_ptr(), out_k.k_mean.data_ptr(),
                           out_v.v_hat.data_ptr(), _ptr(out_v.v_scale), workspace.data_ptr(), workspace.numel(),
                           _stream(dev)))
    return out_k, out_v


def attn_fwd_fused_q(q: torch.Tensor, kq: KQuant, vq: VQuant, layout: str = "HND", is_causal: bool = False,
                     sm_scale: Optional[float] = None, accum: str = "fp32", out: Optional[torch.Tensor] = None,
                     q_codes: Optional[tuple] = None) -> torch.Tensor:
    """sage_attn_fwd_fused_q: attention that quantises Q (fp16 / bf16, dense) in its own
    prologue; output in q's dtype and layout.  q_codes: optional (q_i8, q_scale) tensors,
    shaped as QKQuant's, that receive the codes and block scales the kernel formed."""
    _check_input(q, "q")
    if accum not in _ACC:
        raise ValueError(f"accum must be one of {sorted(_ACC)}, got {accum!r}")
    B, Hq, Nq, D = _dims(q, layout)
    if (kq.B, kq.D) != (B, D):
        raise ValueError("q and the K operand disagree on batch or head_dim")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    qi, qs = (None, None) if q_codes is None else q_codes
    _check(lib().sage_attn_fwd_fused_q(q.data_ptr(), _DT[q.dtype], _LAYOUT[layout], kq.k_i8.data_ptr(),
                                       kq.k_scale.data_ptr(), vq.v_hat.data_ptr(), _ptr(vq.v_scale), out.data_ptr(),
                                       B, Hq, kq.Hkv, Nq, kq.Nkv, D, int(bool(is_causal)), float(sm_scale),
                                       _PV[vq.pv], _ACC[accum], _ptr(qi), _ptr(qs), _stream(q.device)))
    return out


def quant_qkv_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                     cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, pv: str = "fp16",
                     workspace: Optional[torch.Tensor] = None, out_qk: Optional[QKQuantVarlen] = None,
                     out_v: Optional[VQuantVarlen] = None, gran: str = "block"):
    """quant_qk_varlen and quant_v_varlen in one library call (same outputs)."""
    if gran not in _GRAN:
        raise ValueError(f"gran must be 'block' or 'thread', got {gran!r}")
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_input(x, name)
    if not (q.dtype == k.dtype == v.dtype) or not (q.device == k.device == v.device):
        raise ValueError("q, k and v must share dtype and device")
    if pv not in _PV:
        raise ValueError(f"pv must be 'fp16' or 'fp8', got {pv!r}")
    total_q, Hq, D = _packed_dims(q, "q")
    total_k, Hkv, Dk = _packed_dims(k, "k")
    if Dk != D or tuple(v.shape) != (total_k, Hkv, D):
        raise ValueError("q, k and v disagree on heads, tokens or head_dim")
    dev = q.device
    cq, ck = _cu(cu_seqlens_q, dev, "cu_seqlens_q"), _cu(cu_seqlens_k, dev, "cu_seqlens_k")
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must describe the same number of sequences")
    B = cq.numel() - 1
    L = lib()
    Dp = padded_dim(D)
    rq, sq, rk, sk = varlen_rows(total_q, B), varlen_slots(total_q, B), varlen_rows(total_k, B), varlen_slots(total_k, B)
    qk = out_qk
    if qk is None:
        thr = gran == "thread"
        qk = QKQuantVarlen(torch.empty(Hq, rq, max(Dp, 1), dtype=torch.int8, device=dev),
                           torch.empty(Hq, rq if thr else sq, dtype=torch.float32, device=dev),
                           torch.empty(Hkv, rk, max(Dp, 1), dtype=torch.int8, device=dev),
                           torch.empty((Hkv, sk, 2) if thr else (Hkv, sk), dtype=torch.float32, device=dev),
                           torch.empty(B, Hkv, D, dtype=torch.float32, device=dev), cq, ck, B, Hq, Hkv, total_q,
                           total_k, int(max_seqlen_q), int(max_seqlen_k), D, gran)
    elif qk.gran != gran:
        raise ValueError("out_qk was allocated for another granularity")
    vq = out_v
    if vq is None:
        elt = 1 if pv == "fp8" else 2
        vq = VQuantVarlen(torch.empty(Hkv, sk, max(Dp, 1), 64 * elt, dtype=torch.uint8, device=dev),
                          torch.empty(B, Hkv, max(Dp, 1), dtype=torch.float32, device=dev) if pv == "fp8" else None,
                          pv)
    need = L.sage_quant_qkv_varlen_workspace_bytes(B, Hkv, total_k, D, _PV[pv])
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    _check(L.sage_quant_qkv_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DT[q.dtype], cq.data_ptr(),
                                   ck.data_ptr(), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D,
                                   _PV[pv], _GRAN[gran], qk.q_i8.data_ptr(), qk.q_scale.data_ptr(), qk.k_i8.data_ptr(),
                                   qk.k_scale.data_ptr(), qk.k_mean.data_ptr(), vq.v_hat.data_ptr(),
                                   _ptr(vq.v_scale), workspace.data_ptr(), workspace.numel(), _stream(dev)))
    return qk, vq


def attn_fwd_varlen(qk: QKQuantVarlen, vq: VQuantVarlen, out_dtype: torch.dtype, is_causal: bool = False,
                    sm_scale: Optional[float] = None, accum: str = "fp32",
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out_dtype not in _DT:
        raise ValueError("out_dtype must be float16 or bfloat16")
    if accum not in _ACC:
        raise ValueError(f"accum must be one of {sorted(_ACC)}, got {accum!r}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(qk.D)
    dev = qk.q_i8.device
    if out is None:
        out = torch.empty(qk.total_q, qk.Hq, qk.D, dtype=out_dtype, device=dev)
    args = (qk.q_i8.data_ptr(), qk.q_scale.data_ptr(), qk.k_i8.data_ptr(), qk.k_scale.data_ptr(), vq.v_hat.data_ptr(),
            _ptr(vq.v_scale), out.data_ptr(), _DT[out_dtype], qk.cu_q.data_ptr(), qk.cu_k.data_ptr(), qk.B, qk.Hq,
            qk.Hkv, qk.total_q, qk.total_kv, qk.max_q, qk.max_k, qk.D, int(bool(is_causal)), float(sm_scale),
            _PV[vq.pv], _ACC[accum])
    if qk.gran == "block":
        _check(lib().sage_attn_fwd_varlen(*args, _stream(dev)))
    else:
        _check(lib().sage_attn_fwd_varlen_g(*args, _GRAN[qk.gran], _stream(dev)))
    return out


def quant_kv_varlen(k: torch.Tensor, v: torch.Tensor, cu_seqlens_k: torch.Tensor, max_seqlen_k: int,
                    pv: str = "fp16", workspace: Optional[torch.Tensor] = None, out_k=None, out_v=None):
    """sage_quant_kv_varlen: the K and V part of quant_qkv_varlen (block granularity);
    returns (QKQuantVarlen with the K fields set and Q's left None, VQuantVarlen)."""
    for name, x in (("k", k), ("v", v)):
        _check_input(x, name)
    if k.dtype != v.dtype or k.device != v.device:
        raise ValueError("k and v must share dtype and device")
    if pv not in _PV:
        raise ValueError(f"pv must be 'fp16' or 'fp8', got {pv!r}")
    total_k, Hkv, D = _packed_dims(k, "k")
    if tuple(v.shape) != (total_k, Hkv, D):
        raise ValueError("k and v disagree on heads, tokens or head_dim")
    dev = k.device
    ck = _cu(cu_seqlens_k, dev, "cu_seqlens_k")
    B = ck.numel() - 1
    L = lib()
    Dp = padded_dim(D)
    rk, sk = varlen_rows(total_k, B), varlen_slots(total_k, B)
    elt = 1 if pv == "fp8" else 2
    kq = out_k
    if kq is None:
        kq = QKQuantVarlen(None, None, torch.empty(Hkv, rk, max(Dp, 1), dtype=torch.int8, device=dev),
                           torch.empty(Hkv, sk, dtype=torch.float32, device=dev),
                           torch.empty(B, Hkv, D, dtype=torch.float32, device=dev), None, ck, B, None, Hkv, None,
                           total_k, None, int(max_seqlen_k), D)
    vq = out_v
    if vq is None:
        vq = VQuantVarlen(torch.empty(Hkv, sk, max(Dp, 1), 64 * elt, dtype=torch.uint8, device=dev),
                          torch.empty(B, Hkv, max(Dp, 1), dtype=torch.float32, device=dev) if pv == "fp8" else None, pv)
    need = L.sage_quant_qkv_varlen_workspace_bytes(B, Hkv, total_k, D, _PV[pv])
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    _check(L.sage_quant_kv_varlen(k.data_ptr(), v.data_ptr(), _DT[k.dtype], ck.data_ptr(), B, Hkv, total_k,
                                  int(max_seqlen_k), D, _PV[pv], kq.k_i8.data_ptr(), kq.k_scale.data_ptr(),
                                  kq.k_mean.data_ptr(), vq.v_hat.data_ptr(), _ptr(vq.v_scale), workspace.data_ptr(),
                                  workspace.numel(), _stream(dev)))
    return kq, vq


def attn_fwd_varlen_fused_q(q: torch.Tensor, cu_seqlens_q: torch.Tensor, max_seqlen_q: int, kq, vq,
                            is_causal: bool = False, sm_scale: Optional[float] = None, accum: str = "fp32",
                            out: Optional[torch.Tensor] = None, q_codes: Optional[tuple] = None) -> torch.Tensor:
    """sage_attn_fwd_varlen_fused_q: packed attention that quantises each sequence's Q in
    its own prologue; kq, vq from quant_kv_varlen; output (total_q, Hq, D) in q's dtype.
    q_codes: optional (q_i8, q_scale) tensors shaped as QKQuantVarlen's."""
    _check_input(q, "q")
    if accum not in _ACC:
        raise ValueError(f"accum must be one of {sorted(_ACC)}, got {accum!r}")
    total_q, Hq, D = _packed_dims(q, "q")
    if D != kq.D:
        raise ValueError("q and the K operand disagree on head_dim")
    cq = _cu(cu_seqlens_q, q.device, "cu_seqlens_q")
    if cq.numel() != kq.cu_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must describe the same number of sequences")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    qi, qs = (None, None) if q_codes is None else q_codes
    _check(lib().sage_attn_fwd_varlen_fused_q(q.data_ptr(), _DT[q.dtype], cq.data_ptr(), kq.cu_k.data_ptr(),
                                              kq.k_i8.data_ptr(), kq.k_scale.data_ptr(), vq.v_hat.data_ptr(),
                                              _ptr(vq.v_scale), out.data_ptr(), kq.B, Hq, kq.Hkv, total_q,
                                              kq.total_kv, int(max_seqlen_q), kq.max_k, D, int(bool(is_causal)),
                                              float(sm_scale), _PV[vq.pv], _ACC[accum], _ptr(qi), _ptr(qs),
                                              _stream(q.device)))
    return out


def sageattn_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                    cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, is_causal: bool = False,
                    sm_scale: Optional[float] = None, pv: str = "fp16", accum: str = "fp32",
                    qk_gran: str = "block") -> torch.Tensor:
    """Attention over a packed batch of sequences of different lengths (each sequence
    attends only to its own keys); returns q's dtype, shape (total_q, Hq, D).  At block
    granularity Q is quantised inside the attention kernel (quant_kv_varlen +
    attn_fwd_varlen_fused_q: the same codes and output as the separate calls)."""
    if qk_gran == "block" and accum != "fp16+fp32-split":
        _check_input(q, "q")
        if q.dtype != k.dtype or q.device != k.device:
            raise ValueError("q, k and v must share dtype and device")
        kq, vq = quant_kv_varlen(k, v, cu_seqlens_k, max_seqlen_k, pv)
        return attn_fwd_varlen_fused_q(q, cu_seqlens_q, max_seqlen_q, kq, vq, is_causal, sm_scale, accum)
    qk, vq = quant_qkv_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, pv, gran=qk_gran)
    return attn_fwd_varlen(qk, vq, q.dtype, is_causal, sm_scale, accum)


@dataclasses.dataclass
class MXQuantVarlen:
    """Outputs of sage_quant_mxfp4_varlen (packed rows and slots per head)."""
    q4: torch.Tensor       # uint8 [Hq, rows(total_q), Dp/2]
    q4_exp: torch.Tensor   # uint8 [Hq, rows(total_q), Dp/32]
    k4: torch.Tensor       # uint8 [Hkv, rows(total_kv), Dp/2]
    k4_exp: torch.Tensor   # uint8 [Hkv, rows(total_kv), Dp/32]
    k_mean: torch.Tensor   # f32   [B, Hkv, D]
    v4: torch.Tensor       # uint8 [Hkv, slots(total_kv), Dp, 32]
    v4_exp: torch.Tensor   # uint8 [Hkv, slots(total_kv), 2, 32, Dp/32]
    cu_q: torch.Tensor
    cu_k: torch.Tensor
    B: int
    Hq: int
    Hkv: int
    total_q: int
    total_k: int
    max_q: int
    max_k: int
    D: int


def quant_mxfp4_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                       cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                       workspace: Optional[torch.Tensor] = None, out: Optional[MXQuantVarlen] = None) -> MXQuantVarlen:
    """quant_mxfp4 on a packed batch: each sequence quantised on its own."""
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_input(x, name)
    if not (q.dtype == k.dtype == v.dtype) or not (q.device == k.device == v.device):
        raise ValueError("q, k and v must share dtype and device")
    total_q, Hq, D = _packed_dims(q, "q")
    total_k, Hkv, Dk = _packed_dims(k, "k")
    if Dk != D or tuple(v.shape) != (total_k, Hkv, D):
        raise ValueError("q, k and v disagree on heads, tokens or head_dim")
    dev = q.device
    cq, ck = _cu(cu_seqlens_q, dev, "cu_seqlens_q"), _cu(cu_seqlens_k, dev, "cu_seqlens_k")
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must describe the same number of sequences")
    B = cq.numel() - 1
    L = lib()
    Dp = max(padded_dim(D), 64)
    rq, rk, sk = varlen_rows(total_q, B), varlen_rows(total_k, B), varlen_slots(total_k, B)
    if out is None:
        u8 = dict(dtype=torch.uint8, device=dev)
        out = MXQuantVarlen(torch.empty(Hq, rq, Dp // 2, **u8), torch.empty(Hq, rq, Dp // 32, **u8),
                            torch.empty(Hkv, rk, Dp // 2, **u8), torch.empty(Hkv, rk, Dp // 32, **u8),
                            torch.empty(B, Hkv, D, dtype=torch.float32, device=dev),
                            torch.empty(Hkv, sk, Dp, 32, **u8), torch.empty(Hkv, sk, 2, 32, Dp // 32, **u8),
                            cq, ck, B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D)
    need = L.sage_quant_mxfp4_varlen_workspace_bytes(B, Hkv, total_k, D)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=dev)
    _check(L.sage_quant_mxfp4_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DT[q.dtype], cq.data_ptr(),
                                     ck.data_ptr(), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q),
                                     int(max_seqlen_k), D, out.q4.data_ptr(), out.q4_exp.data_ptr(),
                                     out.k4.data_ptr(), out.k4_exp.data_ptr(), out.k_mean.data_ptr(),
                                     out.v4.data_ptr(), out.v4_exp.data_ptr(), workspace.data_ptr(),
                                     workspace.numel(), _stream(dev)))
    return out


def attn_fwd_mxfp4_varlen(mq: MXQuantVarlen, out_dtype: torch.dtype, is_causal: bool = False,
                          sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out_dtype not in _DT:
        raise ValueError("out_dtype must be float16 or bfloat16")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(mq.D)
    dev = mq.q4.device
    if out is None:
        out = torch.empty(mq.total_q, mq.Hq, mq.D, dtype=out_dtype, device=dev)
    _check(lib().sage_attn_fwd_mxfp4_varlen(mq.q4.data_ptr(), mq.q4_exp.data_ptr(), mq.k4.data_ptr(),
                                            mq.k4_exp.data_ptr(), mq.v4.data_ptr(), mq.v4_exp.data_ptr(),
                                            out.data_ptr(), _DT[out_dtype], mq.cu_q.data_ptr(), mq.cu_k.data_ptr(),
                                            mq.B, mq.Hq, mq.Hkv, mq.total_q, mq.total_k, mq.max_q, mq.max_k, mq.D,
                                            int(bool(is_causal)), float(sm_scale), _stream(dev)))
    return out


def sageattn_mxfp4_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                          cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, is_causal: bool = False,
                          sm_scale: Optional[float] = None) -> torch.Tensor:
    """The microscaling FP4 variant on a packed batch (output (total_q, H_qo, D) in q's dtype)."""
    mq = quant_mxfp4_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    return attn_fwd_mxfp4_varlen(mq, q.dtype, is_causal, sm_scale)
