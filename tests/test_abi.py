"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import pytest
import torch

import quantized_attention_04_amd as qa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")

# A fake, 256-byte aligned device address: every call below fails validation before
# any pointer is dereferenced or any HIP call is made.
FAKE = 0x7F0000000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = qa.lib()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    # and the binding declares a signature for each of them
    assert set(names) <= set(qa._EXPORTS)


def test_abi_version_and_strings():
    L = qa.lib()
    assert L.sage_abi_version() == 6
    for s in range(6):
        assert L.sage_status_string(s).decode().startswith("SAGE_")
    assert qa.padded_dim(1) == 64 and qa.padded_dim(64) == 64 and qa.padded_dim(65) == 128
    assert qa.padded_dim(128) == 128 and qa.padded_dim(129) == 256 and qa.padded_dim(256) == 256
    assert qa.padded_dim(257) == 0 and qa.padded_dim(0) == 0
    assert qa.num_blocks(1) == 1 and qa.num_blocks(64) == 1 and qa.num_blocks(65) == 2 and qa.num_blocks(17776) == 278


def test_workspace_sizes():
    L = qa.lib()
    assert L.sage_quant_qk_workspace_bytes(2, 8, 8192, 128) == 2 * 8 * 128 * 128 * 8
    assert L.sage_quant_qk_workspace_bytes(1, 1, 100, 96) == 2 * 96 * 8
    assert L.sage_quant_qk_workspace_bytes(1, 1, 100, 129) == 2 * 129 * 8
    assert L.sage_quant_qk_workspace_bytes(1, 1, 100, 257) == 0
    assert L.sage_quant_v_workspace_bytes(2, 8, 96, qa.SAGE_PV_FP8) == 2 * 8 * 128 * 4
    assert L.sage_quant_v_workspace_bytes(2, 8, 96, qa.SAGE_PV_FP16) == 0


def _qk(**kw):
    a = dict(q=FAKE, k=FAKE, dtype=0, layout=0, B=1, Hq=2, Hkv=2, Nq=128, Nkv=128, D=64, q_i8=FAKE, q_scale=FAKE,
             k_i8=FAKE, k_scale=FAKE, k_mean=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return qa.lib().sage_quant_qk(a["q"], a["k"], a["dtype"], a["layout"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                                  a["Nkv"], a["D"], a["q_i8"], a["q_scale"], a["k_i8"], a["k_scale"], a["k_mean"],
                                  a["ws"], a["ws_bytes"], a["stream"])


def _attn(**kw):
    a = dict(q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, v_hat=FAKE, v_scale=FAKE, out=FAKE, odt=0, olay=0,
             B=1, Hq=2, Hkv=2, Nq=128, Nkv=128, D=64, causal=0, sm=0.125, pv=1, acc=0, stream=None)
    a.update(kw)
    return qa.lib().sage_attn_fwd(a["q_i8"], a["q_scale"], a["k_i8"], a["k_scale"], a["v_hat"], a["v_scale"],
                                  a["out"], a["odt"], a["olay"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["D"],
                                  a["causal"], a["sm"], a["pv"], a["acc"], a["stream"])


def _v(**kw):
    a = dict(v=FAKE, dtype=1, layout=1, B=1, Hkv=2, Nkv=100, D=96, pv=1, v_hat=FAKE, v_scale=FAKE, ws=FAKE,
             ws_bytes=1 << 16, stream=None)
    a.update(kw)
    return qa.lib().sage_quant_v(a["v"], a["dtype"], a["layout"], a["B"], a["Hkv"], a["Nkv"], a["D"], a["pv"],
                                 a["v_hat"], a["v_scale"], a["ws"], a["ws_bytes"], a["stream"])


def _detail():
    return qa.lib().sage_last_error_detail().decode()


def _fused(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, layout=0, B=1, Hq=4, Hkv=2, Nq=128, Nkv=100, D=96, pv=1, gran=0, q_i8=FAKE,
             q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, k_mean=FAKE, v_hat=FAKE, v_scale=FAKE, ws=FAKE, ws_bytes=1 << 20,
             stream=None)
    a.update(kw)
    return qa.lib().sage_quant_qkv(a["q"], a["k"], a["v"], a["dtype"], a["layout"], a["B"], a["Hq"], a["Hkv"],
                                   a["Nq"], a["Nkv"], a["D"], a["pv"], a["gran"], a["q_i8"], a["q_scale"], a["k_i8"],
                                   a["k_scale"], a["k_mean"], a["v_hat"], a["v_scale"], a["ws"], a["ws_bytes"],
                                   a["stream"])


def test_fused_quant_workspace_sizes():
    L = qa.lib()
    fp8, fp16 = qa.SAGE_PV_FP8, qa.SAGE_PV_FP16
    slots = 2 * 8 * 128  # B * H_kv * NB(8192)
    assert L.sage_quant_qkv_workspace_bytes(2, 8, 8192, 128, fp16) == slots * 128 * 8
    assert L.sage_quant_qkv_workspace_bytes(2, 8, 8192, 128, fp8) == slots * 128 * 8 + slots * 128 * 4 + 2 * 8 * 128 * 4
    # D = 96: K sums over the 96 real channels, V maxima over Dp = 128
    assert L.sage_quant_qkv_workspace_bytes(1, 2, 100, 96, fp8) == 4 * 96 * 8 + 4 * 128 * 4 + 2 * 128 * 4
    assert L.sage_quant_qkv_workspace_bytes(1, 2, 100, 257, fp8) == 0
    assert L.sage_quant_qkv_workspace_bytes(1, 2, 100, 96, 3) == 0
    # packed: H_kv * ceil((total + 64 B) / 64) slots
    s = 2 * ((1000 + 64 * 3 + 63) // 64)
    assert L.sage_quant_qkv_varlen_workspace_bytes(3, 2, 1000, 96, fp16) == s * 96 * 8
    assert L.sage_quant_qkv_varlen_workspace_bytes(3, 2, 1000, 96, fp8) == s * 96 * 8 + s * 128 * 4 + 3 * 2 * 128 * 4


@pytest.mark.parametrize("kw,code", [
    ({"v": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"k_mean": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"pv": 2}, qa.SAGE_ERR_INVALID_ARG),
    ({"v_scale": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"dtype": 3}, qa.SAGE_ERR_INVALID_ARG),
    ({"layout": 2}, qa.SAGE_ERR_INVALID_ARG),
    ({"Hq": 3}, qa.SAGE_ERR_INVALID_ARG),
    ({"D": 257}, qa.SAGE_ERR_UNSUPPORTED),
    ({"v": FAKE + 4}, qa.SAGE_ERR_INVALID_ARG),
    ({"ws": None}, qa.SAGE_ERR_WORKSPACE),
    ({"ws_bytes": 4 * 96 * 8 + 4 * 128 * 4 + 2 * 128 * 4 - 1}, qa.SAGE_ERR_WORKSPACE),
    ({"ws": FAKE + 4}, qa.SAGE_ERR_WORKSPACE),
    ({"gran": 2}, qa.SAGE_ERR_INVALID_ARG),
])
def test_fused_quant_rejects(kw, code):
    assert _fused(**kw) == code
    assert _detail()


def test_fused_quant_fp16_takes_no_scale():
    if torch.cuda.is_available():
        pytest.skip("would launch kernels on fake pointers")
    assert _fused(pv=0, v_scale=None, ws_bytes=4 * 96 * 8) == qa.SAGE_ERR_DEVICE
    assert _fused() == qa.SAGE_ERR_DEVICE
    assert _fused(gran=1) == qa.SAGE_ERR_DEVICE


def test_quant_qkv_noalloc_limits():
    """The allocation-free fused quantisation refuses sizes whose workspace exceeds its
    static scratch before any HIP call, and otherwise validates like sage_quant_qkv."""
    L = qa.lib()
    cap = L.sage_quant_qkv_noalloc_max_bytes()
    assert cap == 32 << 20

    def call(B, Hkv, N, D, pv=1, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, layout=0, B=B, Hq=Hkv, Hkv=Hkv, Nq=N, Nkv=N, D=D, pv=pv, gran=0)
        a.update(kw)
        return L.sage_quant_qkv_noalloc(a["q"], a["k"], a["v"], a["dtype"], a["layout"], a["B"], a["Hq"], a["Hkv"],
                                        a["Nq"], a["Nkv"], a["D"], a["pv"], a["gran"], *([FAKE] * 7), None)
    assert L.sage_quant_qkv_workspace_bytes(4, 32, 10880, 128, 1) <= cap < L.sage_quant_qkv_workspace_bytes(
        4, 32, 10944, 128, 1)
    assert call(4, 32, 10944, 128) == qa.SAGE_ERR_UNSUPPORTED and "static scratch" in _detail()
    assert call(1, 2, 100, 64, gran=5) == qa.SAGE_ERR_INVALID_ARG
    assert call(1, 2, 100, 64, q=None) == qa.SAGE_ERR_INVALID_ARG
    assert call(1, 2, 100, 300) == qa.SAGE_ERR_UNSUPPORTED
    if not torch.cuda.is_available():
        assert call(4, 32, 10880, 128) == qa.SAGE_ERR_DEVICE


def test_attn_fwd_split_limits():
    """Key-range splits: FP16 P.V only, a workspace of the stated size, 1..64 splits; the
    library's choice splits only under-filled FP16 P.V launches."""
    L = qa.lib()
    ws = L.sage_attn_fwd_split_workspace_bytes(1, 8, 2048, 128, 6)
    assert ws == 8 * 2048 * 6 * (128 * 2 + 8)
    assert L.sage_attn_fwd_split_workspace_bytes(1, 8, 2048, 128, 1) == 0
    assert L.sage_attn_fwd_split_workspace_bytes(1, 8, 2048, 300, 4) == 0
    assert L.sage_attn_fwd_split_choice(1, 8, 2048, 2048, 128, 0, 0) > 1          # LLM prefill, FP16 P.V
    assert L.sage_attn_fwd_split_choice(1, 8, 2048, 2048, 128, 0, 1) == 1         # FP8 P.V: never
    assert L.sage_attn_fwd_split_choice(4, 32, 8192, 8192, 128, 0, 0) == 1        # fills the GPU
    assert L.sage_attn_fwd_split_choice(1, 8, 2048, 256, 128, 0, 0) == 1          # too few key tiles
    for B, H, N in ((1, 8, 2048), (1, 2, 256), (2, 3, 700)):
        S = L.sage_attn_fwd_split_choice(B, H, N, N, 64, 1, 0)
        if S > 1:  # balanced ranges of at least four tiles
            tps = -(-qa.num_blocks(N) // S)
            assert tps >= 4 and -(-qa.num_blocks(N) // tps) == S
    ws = L.sage_attn_fwd_split_workspace_bytes(1, 8, 2048, 128, 4)

    def call(**kw):
        a = dict(pv=0, acc=0, splits=4, ws=FAKE, wsb=ws, D=128)
        a.update(kw)
        return L.sage_attn_fwd_split(*([FAKE] * 7), 0, 0, 1, 8, 8, 2048, 2048, a["D"], 0, 0.088, a["pv"], a["acc"],
                                     a["splits"], a["ws"], a["wsb"], None)
    assert call(pv=1) == qa.SAGE_ERR_UNSUPPORTED and "FP16" in _detail()
    assert call(acc=qa.SAGE_ACC_FP16_FP32_SPLIT) == qa.SAGE_ERR_UNSUPPORTED
    assert call(splits=0) == qa.SAGE_ERR_INVALID_ARG
    assert call(splits=65) == qa.SAGE_ERR_INVALID_ARG
    assert call(wsb=ws - 1) == qa.SAGE_ERR_WORKSPACE
    assert call(ws=None) == qa.SAGE_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == qa.SAGE_ERR_WORKSPACE
    if not torch.cuda.is_available():
        assert call() == qa.SAGE_ERR_DEVICE
        assert call(splits=1, ws=None) == qa.SAGE_ERR_DEVICE  # one split: plain sage_attn_fwd


def test_attn_fwd_g_checks_granularity_first():
    L = qa.lib()
    args = [FAKE] * 7 + [0, 0, 1, 2, 2, 128, 128, 64, 0, 0.125, 1, 0]
    assert L.sage_attn_fwd_g(*args, 5, None) == qa.SAGE_ERR_INVALID_ARG and "granularity" in _detail()
    assert L.sage_attn_fwd_g(*args[:6], None, *args[7:], 1, None) == qa.SAGE_ERR_INVALID_ARG
    if not torch.cuda.is_available():
        assert L.sage_attn_fwd_g(*args, 1, None) == qa.SAGE_ERR_DEVICE
    vargs = [FAKE] * 7 + [0, FAKE, FAKE, 2, 2, 2, 100, 100, 60, 60, 64, 0, 0.125, 1, 0]
    assert L.sage_attn_fwd_varlen_g(*vargs, -1, None) == qa.SAGE_ERR_INVALID_ARG
    # the explicit two-level accumulation is offered with block granularity only
    split = args[:-1] + [qa.SAGE_ACC_FP16_FP32_SPLIT]
    assert L.sage_attn_fwd_g(*split, 1, None) == qa.SAGE_ERR_UNSUPPORTED and "SPLIT" in _detail()
    assert L.sage_attn_fwd_varlen_g(*(vargs[:-1] + [qa.SAGE_ACC_FP16_FP32_SPLIT]), 1, None) == qa.SAGE_ERR_UNSUPPORTED
    if not torch.cuda.is_available():
        assert L.sage_attn_fwd_g(*split, 0, None) == qa.SAGE_ERR_DEVICE


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"k_mean": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"dtype": 2}, qa.SAGE_ERR_INVALID_ARG),
    ({"layout": 7}, qa.SAGE_ERR_INVALID_ARG),
    ({"B": 0}, qa.SAGE_ERR_INVALID_ARG),
    ({"Nkv": -1}, qa.SAGE_ERR_INVALID_ARG),
    ({"Hq": 6, "Hkv": 4}, qa.SAGE_ERR_INVALID_ARG),
    ({"D": 257}, qa.SAGE_ERR_UNSUPPORTED),
    ({"D": 512}, qa.SAGE_ERR_UNSUPPORTED),
    ({"q": FAKE + 2}, qa.SAGE_ERR_INVALID_ARG),
    ({"ws": None}, qa.SAGE_ERR_WORKSPACE),
    ({"ws_bytes": 2 * 64 * 8 - 1}, qa.SAGE_ERR_WORKSPACE),
])
def test_quant_qk_rejects(kw, code):
    assert _qk(**kw) == code
    assert _detail()


@pytest.mark.parametrize("kw,code", [
    ({"v": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"pv": 5}, qa.SAGE_ERR_INVALID_ARG),
    ({"v_scale": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"ws": None}, qa.SAGE_ERR_WORKSPACE),
    ({"ws_bytes": 2 * 128 * 4 - 4}, qa.SAGE_ERR_WORKSPACE),
    ({"D": 300}, qa.SAGE_ERR_UNSUPPORTED),
    ({"v_hat": FAKE + 8}, qa.SAGE_ERR_INVALID_ARG),
])
def test_quant_v_rejects(kw, code):
    assert _v(**kw) == code


@pytest.mark.parametrize("kw,code", [
    ({"out": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"sm": 0.0}, qa.SAGE_ERR_INVALID_ARG),
    ({"sm": -1.0}, qa.SAGE_ERR_INVALID_ARG),
    ({"sm": float("inf")}, qa.SAGE_ERR_INVALID_ARG),
    ({"sm": float("nan")}, qa.SAGE_ERR_INVALID_ARG),
    ({"pv": 2}, qa.SAGE_ERR_INVALID_ARG),
    ({"acc": 4}, qa.SAGE_ERR_INVALID_ARG),
    ({"causal": 2}, qa.SAGE_ERR_INVALID_ARG),
    ({"acc": qa.SAGE_ACC_FP16}, qa.SAGE_ERR_UNSUPPORTED),
    ({"v_scale": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"Hq": 32, "Hkv": 6}, qa.SAGE_ERR_INVALID_ARG),
    ({"out": FAKE + 2}, qa.SAGE_ERR_INVALID_ARG),
])
def test_attn_fwd_rejects(kw, code):
    assert _attn(**kw) == code
    assert _detail()


def test_fp16_pv_needs_no_scale_or_workspace_validation_order():
    # FP16 mode ignores v_scale; without a GPU the call reaches the device check.
    if torch.cuda.is_available():
        pytest.skip("would launch kernels on fake pointers")
    assert _attn(pv=0, v_scale=None) == qa.SAGE_ERR_DEVICE
    assert _v(pv=0, v_scale=None, ws=None, ws_bytes=0) == qa.SAGE_ERR_DEVICE
    assert "device" in _detail()


def test_valid_arguments_reach_the_device_check_only():
    if torch.cuda.is_available():
        pytest.skip("would launch kernels on fake pointers")
    assert _qk() == qa.SAGE_ERR_DEVICE
    assert _attn() == qa.SAGE_ERR_DEVICE
    assert _v() == qa.SAGE_ERR_DEVICE
    assert _attn(causal=1, Nkv=256) == qa.SAGE_ERR_DEVICE  # causal with Nq != Nkv is accepted
    assert _qkv() == qa.SAGE_ERR_DEVICE
    assert _vv() == qa.SAGE_ERR_DEVICE
    assert _attnv() == qa.SAGE_ERR_DEVICE


def test_python_layer_rejects_fp32_and_cpu_tensors():
    x = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError, match="float16 or bfloat16"):
        qa.sageattn(x, x, x)
    h = x.half()
    with pytest.raises(ValueError, match="GPU"):
        qa.sageattn(h, h, h)


# ----------------------------------------------------------------------------- packed (varlen) batches

def test_varlen_sizes():
    L = qa.lib()
    assert L.sage_varlen_rows(1000, 3) == 1000 + 192
    assert L.sage_varlen_slots(1000, 3) == (1192 + 63) // 64
    assert L.sage_varlen_rows(0, 3) == 0 and L.sage_varlen_slots(10, 0) == 0
    assert L.sage_quant_qk_varlen_workspace_bytes(3, 2, 1000, 96) == 2 * ((1192 + 63) // 64) * 96 * 8
    assert L.sage_quant_qk_varlen_workspace_bytes(3, 2, 1000, 257) == 0


def _qkv(**kw):
    a = dict(q=FAKE, k=FAKE, dtype=0, cuq=FAKE, cuk=FAKE, B=3, Hq=2, Hkv=2, tq=300, tk=400, mq=200, mk=200, D=64,
             q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, k_mean=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return qa.lib().sage_quant_qk_varlen(a["q"], a["k"], a["dtype"], a["cuq"], a["cuk"], a["B"], a["Hq"], a["Hkv"],
                                         a["tq"], a["tk"], a["mq"], a["mk"], a["D"], a["q_i8"], a["q_scale"],
                                         a["k_i8"], a["k_scale"], a["k_mean"], a["ws"], a["ws_bytes"], a["stream"])


def _vv(**kw):
    a = dict(v=FAKE, dtype=1, cuk=FAKE, B=3, Hkv=2, tk=400, mk=200, D=128, pv=1, v_hat=FAKE, v_scale=FAKE, ws=FAKE,
             ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return qa.lib().sage_quant_v_varlen(a["v"], a["dtype"], a["cuk"], a["B"], a["Hkv"], a["tk"], a["mk"], a["D"],
                                        a["pv"], a["v_hat"], a["v_scale"], a["ws"], a["ws_bytes"], a["stream"])


def _attnv(**kw):
    a = dict(q_i8=FAKE, q_scale=FAKE, k_i8=FAKE, k_scale=FAKE, v_hat=FAKE, v_scale=FAKE, out=FAKE, odt=1, cuq=FAKE,
             cuk=FAKE, B=3, Hq=4, Hkv=2, tq=300, tk=400, mq=200, mk=200, D=128, causal=1, sm=0.1, pv=1, acc=0,
             stream=None)
    a.update(kw)
    return qa.lib().sage_attn_fwd_varlen(a["q_i8"], a["q_scale"], a["k_i8"], a["k_scale"], a["v_hat"], a["v_scale"],
                                         a["out"], a["odt"], a["cuq"], a["cuk"], a["B"], a["Hq"], a["Hkv"], a["tq"],
                                         a["tk"], a["mq"], a["mk"], a["D"], a["causal"], a["sm"], a["pv"], a["acc"],
                                         a["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"cuq": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"cuk": FAKE + 2}, qa.SAGE_ERR_INVALID_ARG),
    ({"tq": 0}, qa.SAGE_ERR_INVALID_ARG),
    ({"mk": 0}, qa.SAGE_ERR_INVALID_ARG),
    ({"B": 0}, qa.SAGE_ERR_INVALID_ARG),
    ({"Hq": 3}, qa.SAGE_ERR_INVALID_ARG),
    ({"D": 260}, qa.SAGE_ERR_UNSUPPORTED),
    ({"tq": 2 ** 31 - 100}, qa.SAGE_ERR_UNSUPPORTED),
    ({"ws_bytes": 16}, qa.SAGE_ERR_WORKSPACE),
    ({"q_i8": FAKE + 4}, qa.SAGE_ERR_INVALID_ARG),
])
def test_quant_qk_varlen_rejects(kw, code):
    assert _qkv(**kw) == code
    assert _detail()


@pytest.mark.parametrize("kw,code", [
    ({"cuk": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"pv": 3}, qa.SAGE_ERR_INVALID_ARG),
    ({"v_scale": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"ws": None}, qa.SAGE_ERR_WORKSPACE),
    ({"tk": -1}, qa.SAGE_ERR_INVALID_ARG),
])
def test_quant_v_varlen_rejects(kw, code):
    assert _vv(**kw) == code


@pytest.mark.parametrize("kw,code", [
    ({"cuq": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"out": None}, qa.SAGE_ERR_INVALID_ARG),
    ({"sm": float("nan")}, qa.SAGE_ERR_INVALID_ARG),
    ({"acc": qa.SAGE_ACC_FP16}, qa.SAGE_ERR_UNSUPPORTED),
    ({"Hq": 5}, qa.SAGE_ERR_INVALID_ARG),
    ({"mq": -3}, qa.SAGE_ERR_INVALID_ARG),
])
def test_attn_fwd_varlen_rejects(kw, code):
    assert _attnv(**kw) == code
    assert _detail()


def test_python_varlen_layer_rejects_bad_shapes():
    x = torch.zeros(2, 1, 64, 64, dtype=torch.float16)
    cu = torch.tensor([0, 64], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        qa.sageattn_varlen(x, x, x, cu, cu, 64, 64)


# ---- microscaling FP4 entry points

def _mxq(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, layout=0, B=1, Hq=2, Hkv=2, Nq=128, Nkv=128, D=64, q4=FAKE, q4e=FAKE,
             k4=FAKE, k4e=FAKE, km=FAKE, v4=FAKE, v4e=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return qa.lib().sage_quant_mxfp4(a["q"], a["k"], a["v"], a["dtype"], a["layout"], a["B"], a["Hq"], a["Hkv"],
                                     a["Nq"], a["Nkv"], a["D"], a["q4"], a["q4e"], a["k4"], a["k4e"], a["km"], a["v4"],
                                     a["v4e"], a["ws"], a["ws_bytes"], a["stream"])


def _mxa(**kw):
    a = dict(q4=FAKE, q4e=FAKE, k4=FAKE, k4e=FAKE, v4=FAKE, v4e=FAKE, out=FAKE, odt=1, olay=0, B=1, Hq=2, Hkv=2,
             Nq=128, Nkv=128, D=64, causal=0, sm=0.125, stream=None)
    a.update(kw)
    return qa.lib().sage_attn_fwd_mxfp4(a["q4"], a["q4e"], a["k4"], a["k4e"], a["v4"], a["v4e"], a["out"], a["odt"],
                                        a["olay"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["D"], a["causal"],
                                        a["sm"], a["stream"])


def test_mxfp4_workspace_sizes():
    L = qa.lib()
    assert L.sage_quant_mxfp4_workspace_bytes(4, 32, 8192, 128) == 4 * 32 * 128 * 128 * 8
    assert L.sage_quant_mxfp4_workspace_bytes(1, 1, 100, 72) == 2 * 72 * 8
    assert L.sage_quant_mxfp4_workspace_bytes(1, 1, 100, 200) == 2 * 200 * 8
    assert L.sage_quant_mxfp4_workspace_bytes(1, 1, 100, 257) == 0
    assert L.sage_quant_mxfp4_workspace_bytes(0, 1, 100, 64) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), qa.SAGE_ERR_INVALID_ARG), (dict(v4e=None), qa.SAGE_ERR_INVALID_ARG),
    (dict(km=None), qa.SAGE_ERR_INVALID_ARG), (dict(dtype=2), qa.SAGE_ERR_INVALID_ARG),
    (dict(layout=2), qa.SAGE_ERR_INVALID_ARG), (dict(q4=FAKE + 8), qa.SAGE_ERR_INVALID_ARG),
    (dict(Hq=3), qa.SAGE_ERR_INVALID_ARG), (dict(Nkv=0), qa.SAGE_ERR_INVALID_ARG),
    (dict(D=300), qa.SAGE_ERR_UNSUPPORTED), (dict(ws=None), qa.SAGE_ERR_WORKSPACE),
    (dict(ws_bytes=2 * 64 * 8 - 1), qa.SAGE_ERR_WORKSPACE), (dict(ws=FAKE + 4), qa.SAGE_ERR_WORKSPACE),
])
def test_quant_mxfp4_rejects(kw, code):
    assert _mxq(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q4=None), qa.SAGE_ERR_INVALID_ARG), (dict(out=None), qa.SAGE_ERR_INVALID_ARG),
    (dict(odt=5), qa.SAGE_ERR_INVALID_ARG), (dict(olay=3), qa.SAGE_ERR_INVALID_ARG),
    (dict(causal=2), qa.SAGE_ERR_INVALID_ARG), (dict(sm=0.0), qa.SAGE_ERR_INVALID_ARG),
    (dict(sm=float("nan")), qa.SAGE_ERR_INVALID_ARG), (dict(k4=FAKE + 1), qa.SAGE_ERR_INVALID_ARG),
    (dict(Hkv=4), qa.SAGE_ERR_INVALID_ARG), (dict(D=257), qa.SAGE_ERR_UNSUPPORTED),
    (dict(D=0), qa.SAGE_ERR_INVALID_ARG),
])
def test_attn_fwd_mxfp4_rejects(kw, code):
    assert _mxa(**kw) == code


def test_mxfp4_valid_arguments_reach_the_device_check_only():
    if torch.cuda.is_available():
        pytest.skip("would launch kernels on fake pointers")
    assert _mxq() == qa.SAGE_ERR_DEVICE
    assert _mxa() == qa.SAGE_ERR_DEVICE


def _mxqv(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, cq=FAKE, ck=FAKE, B=2, Hq=2, Hkv=2, tq=100, tk=100, mq=64, mk=64, D=64,
             q4=FAKE, q4e=FAKE, k4=FAKE, k4e=FAKE, km=FAKE, v4=FAKE, v4e=FAKE, ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return qa.lib().sage_quant_mxfp4_varlen(a["q"], a["k"], a["v"], a["dtype"], a["cq"], a["ck"], a["B"], a["Hq"],
                                            a["Hkv"], a["tq"], a["tk"], a["mq"], a["mk"], a["D"], a["q4"], a["q4e"],
                                            a["k4"], a["k4e"], a["km"], a["v4"], a["v4e"], a["ws"], a["ws_bytes"],
                                            a["stream"])


def _mxav(**kw):
    a = dict(q4=FAKE, q4e=FAKE, k4=FAKE, k4e=FAKE, v4=FAKE, v4e=FAKE, out=FAKE, odt=1, cq=FAKE, ck=FAKE, B=2, Hq=2,
             Hkv=2, tq=100, tk=100, mq=64, mk=64, D=64, causal=0, sm=0.125, stream=None)
    a.update(kw)
    return qa.lib().sage_attn_fwd_mxfp4_varlen(a["q4"], a["q4e"], a["k4"], a["k4e"], a["v4"], a["v4e"], a["out"],
                                               a["odt"], a["cq"], a["ck"], a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"],
                                               a["mq"], a["mk"], a["D"], a["causal"], a["sm"], a["stream"])


def test_mxfp4_varlen_workspace_sizes():
    L = qa.lib()
    assert L.sage_quant_mxfp4_varlen_workspace_bytes(3, 2, 500, 64) == 2 * qa.varlen_slots(500, 3) * 64 * 8
    assert L.sage_quant_mxfp4_varlen_workspace_bytes(3, 2, 500, 257) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(v=None), qa.SAGE_ERR_INVALID_ARG), (dict(cq=None), qa.SAGE_ERR_INVALID_ARG),
    (dict(ck=FAKE + 2), qa.SAGE_ERR_INVALID_ARG), (dict(dtype=7), qa.SAGE_ERR_INVALID_ARG),
    (dict(tq=0), qa.SAGE_ERR_INVALID_ARG), (dict(Hq=3), qa.SAGE_ERR_INVALID_ARG),
    (dict(D=300), qa.SAGE_ERR_UNSUPPORTED), (dict(ws=None), qa.SAGE_ERR_WORKSPACE),
    (dict(ws_bytes=8), qa.SAGE_ERR_WORKSPACE),
])
def test_quant_mxfp4_varlen_rejects(kw, code):
    assert _mxqv(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), qa.SAGE_ERR_INVALID_ARG), (dict(cq=None), qa.SAGE_ERR_INVALID_ARG),
    (dict(odt=3), qa.SAGE_ERR_INVALID_ARG), (dict(causal=5), qa.SAGE_ERR_INVALID_ARG),
    (dict(sm=-1.0), qa.SAGE_ERR_INVALID_ARG), (dict(tk=0), qa.SAGE_ERR_INVALID_ARG),
    (dict(D=300), qa.SAGE_ERR_UNSUPPORTED),
])
def test_attn_fwd_mxfp4_varlen_rejects(kw, code):
    assert _mxav(**kw) == code


def test_mxfp4_varlen_valid_arguments_reach_the_device_check_only():
    if torch.cuda.is_available():
        pytest.skip("would launch kernels on fake pointers")
    assert _mxqv() == qa.SAGE_ERR_DEVICE
    assert _mxav() == qa.SAGE_ERR_DEVICE


def test_fused_q_entry_points_validate_first():
    """sage_quant_kv and sage_attn_fwd_fused_q: bad arguments are refused before any HIP
    call (then, with no GPU, the device check fails)."""
    L = qa.lib()
    need = L.sage_quant_qkv_workspace_bytes(2, 4, 1000, 128, 1)

    def kv(**kw):
        a = dict(k=FAKE, dtype=1, layout=0, H=4, N=1000, D=128, pv=1, vs=FAKE, ws=FAKE, wsb=need)
        a.update(kw)
        return L.sage_quant_kv(a["k"], FAKE, a["dtype"], a["layout"], 2, a["H"], a["N"], a["D"], a["pv"], FAKE, FAKE,
                               FAKE, FAKE, a["vs"], a["ws"], a["wsb"], None)
    assert kv(k=None) == qa.SAGE_ERR_INVALID_ARG
    assert kv(dtype=7) == qa.SAGE_ERR_INVALID_ARG
    assert kv(vs=None) == qa.SAGE_ERR_INVALID_ARG and "v_scale" in _detail()
    assert kv(layout=3) == qa.SAGE_ERR_INVALID_ARG
    assert kv(D=300) == qa.SAGE_ERR_UNSUPPORTED
    assert kv(wsb=need - 1) == qa.SAGE_ERR_WORKSPACE
    assert kv(k=FAKE + 8) == qa.SAGE_ERR_INVALID_ARG  # misaligned
    if not torch.cuda.is_available():
        assert kv() == qa.SAGE_ERR_DEVICE
        assert kv(pv=0, vs=None) == qa.SAGE_ERR_DEVICE  # FP16 V needs no v_scale

    def fq(**kw):
        a = dict(q=FAKE, dtype=1, layout=0, Hq=8, Hkv=2, acc=0, qi=None, causal=0, sm=0.088)
        a.update(kw)
        return L.sage_attn_fwd_fused_q(a["q"], a["dtype"], a["layout"], FAKE, FAKE, FAKE, FAKE, FAKE, 2, a["Hq"],
                                       a["Hkv"], 1000, 1000, 128, a["causal"], a["sm"], 1, a["acc"], a["qi"], None,
                                       None)
    assert fq(q=None) == qa.SAGE_ERR_INVALID_ARG
    assert fq(dtype=5) == qa.SAGE_ERR_INVALID_ARG
    assert fq(q=FAKE + 2) == qa.SAGE_ERR_INVALID_ARG
    assert fq(qi=FAKE + 4) == qa.SAGE_ERR_INVALID_ARG
    assert fq(acc=qa.SAGE_ACC_FP16_FP32_SPLIT) == qa.SAGE_ERR_UNSUPPORTED
    assert fq(acc=qa.SAGE_ACC_FP16) == qa.SAGE_ERR_UNSUPPORTED
    assert fq(Hq=7) == qa.SAGE_ERR_INVALID_ARG  # not a multiple of H_kv
    assert fq(causal=2) == qa.SAGE_ERR_INVALID_ARG
    assert fq(sm=-1.0) == qa.SAGE_ERR_INVALID_ARG
    if not torch.cuda.is_available():
        assert fq() == qa.SAGE_ERR_DEVICE


def test_mxfp4_fused_q_entry_points_validate_first():
    L = qa.lib()
    need = L.sage_quant_mxfp4_workspace_bytes(1, 2, 500, 128)

    def kv(**kw):
        a = dict(k=FAKE, dtype=1, layout=0, D=128, wsb=need, km=FAKE)
        a.update(kw)
        return L.sage_quant_mxfp4_kv(a["k"], FAKE, a["dtype"], a["layout"], 1, 2, 500, a["D"], FAKE, FAKE, a["km"],
                                     FAKE, FAKE, FAKE, a["wsb"], None)
    assert kv(k=None) == qa.SAGE_ERR_INVALID_ARG
    assert kv(km=None) == qa.SAGE_ERR_INVALID_ARG
    assert kv(dtype=4) == qa.SAGE_ERR_INVALID_ARG
    assert kv(layout=2) == qa.SAGE_ERR_INVALID_ARG
    assert kv(k=FAKE + 4) == qa.SAGE_ERR_INVALID_ARG
    assert kv(D=257) == qa.SAGE_ERR_UNSUPPORTED
    assert kv(wsb=need - 8) == qa.SAGE_ERR_WORKSPACE
    if not torch.cuda.is_available():
        assert kv() == qa.SAGE_ERR_DEVICE

    def fq(**kw):
        a = dict(q=FAKE, dtype=0, causal=1, sm=0.1, Hq=4, qc=None)
        a.update(kw)
        return L.sage_attn_fwd_mxfp4_fused_q(a["q"], a["dtype"], 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1, a["Hq"], 2, 300,
                                             500, 128, a["causal"], a["sm"], a["qc"], None, None)
    assert fq(q=None) == qa.SAGE_ERR_INVALID_ARG
    assert fq(dtype=9) == qa.SAGE_ERR_INVALID_ARG
    assert fq(causal=3) == qa.SAGE_ERR_INVALID_ARG
    assert fq(sm=float("inf")) == qa.SAGE_ERR_INVALID_ARG
    assert fq(q=FAKE + 2) == qa.SAGE_ERR_INVALID_ARG
    assert fq(qc=FAKE + 1) == qa.SAGE_ERR_INVALID_ARG
    assert fq(Hq=3) == qa.SAGE_ERR_INVALID_ARG
    if not torch.cuda.is_available():
        assert fq() == qa.SAGE_ERR_DEVICE


def test_varlen_fused_q_entry_points_validate_first():
    L = qa.lib()
    need = L.sage_quant_qkv_varlen_workspace_bytes(3, 2, 500, 64, 0)

    def kv(**kw):
        a = dict(k=FAKE, cu=FAKE, pv=0, vs=None, wsb=need)
        a.update(kw)
        return L.sage_quant_kv_varlen(a["k"], FAKE, 0, a["cu"], 3, 2, 500, 300, 64, a["pv"], FAKE, FAKE, FAKE, FAKE,
                                      a["vs"], FAKE, a["wsb"], None)
    assert kv(k=None) == qa.SAGE_ERR_INVALID_ARG
    assert kv(cu=None) == qa.SAGE_ERR_INVALID_ARG
    assert kv(pv=1) == qa.SAGE_ERR_INVALID_ARG  # FP8 without v_scale
    assert kv(wsb=need - 8) == qa.SAGE_ERR_WORKSPACE
    if not torch.cuda.is_available():
        assert kv() == qa.SAGE_ERR_DEVICE

    def fq(**kw):
        a = dict(q=FAKE, acc=0, causal=1, cu=FAKE)
        a.update(kw)
        return L.sage_attn_fwd_varlen_fused_q(a["q"], 1, a["cu"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 4, 2, 600, 500,
                                              300, 300, 64, a["causal"], 0.125, 1, a["acc"], None, None, None)
    assert fq(q=None) == qa.SAGE_ERR_INVALID_ARG
    assert fq(q=FAKE + 2) == qa.SAGE_ERR_INVALID_ARG
    assert fq(cu=None) == qa.SAGE_ERR_INVALID_ARG
    assert fq(causal=5) == qa.SAGE_ERR_INVALID_ARG
    assert fq(acc=qa.SAGE_ACC_FP16_FP32_SPLIT) == qa.SAGE_ERR_UNSUPPORTED
    if not torch.cuda.is_available():
        assert fq() == qa.SAGE_ERR_DEVICE
