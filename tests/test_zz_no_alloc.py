"""The allocation-free fused quantisation (sage_quant_qkv_noalloc, for callers that cannot
allocate) against sage_quant_qkv with a caller workspace, through the C ABI: every output
bit for bit, on two calls in a row, the second with a smaller input (the static scratch
keeps the first call's contents)."""
import ctypes

import pytest
import torch

import quantized_attention_04_amd as qa
import synth_inputs as si

pytestmark = pytest.mark.gpu

W = si.workload


def _outputs(w, gran):
    B, Hq, Hkv, Nq, Nkv, D = w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D
    Dp, nbq, nbk = qa.padded_dim(D), qa.num_blocks(Nq), qa.num_blocks(Nkv)
    thr = gran == "thread"
    dev = "cuda:0"
    t = dict(q_i8=torch.full((B, Hq, nbq * 64, Dp), 77, dtype=torch.int8, device=dev),
             q_scale=torch.full((B, Hq, nbq * 64 if thr else nbq), 7.0, device=dev),
             k_i8=torch.full((B, Hkv, nbk * 64, Dp), 77, dtype=torch.int8, device=dev),
             k_scale=torch.full((B, Hkv, nbk, 2) if thr else (B, Hkv, nbk), 7.0, device=dev),
             k_mean=torch.full((B, Hkv, D), 7.0, device=dev),
             v_hat=torch.full((B, Hkv, nbk, Dp, 64 * (1 if w.pv == "fp8" else 2)), 77, dtype=torch.uint8, device=dev),
             v_scale=torch.full((B, Hkv, Dp), 7.0, device=dev))
    return t


def _call(L, w, q, k, v, o, gran, ws=None):
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), 1 if w.dtype == "bf16" else 0, 1 if w.layout == "NHD" else 0,
            w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, 1 if w.pv == "fp8" else 0, 1 if gran == "thread" else 0,
            o["q_i8"].data_ptr(), o["q_scale"].data_ptr(), o["k_i8"].data_ptr(), o["k_scale"].data_ptr(),
            o["k_mean"].data_ptr(), o["v_hat"].data_ptr(), o["v_scale"].data_ptr()]
    stream = torch.cuda.current_stream().cuda_stream
    if ws is None:
        return L.sage_quant_qkv_noalloc(*args, stream)
    return L.sage_quant_qkv(*args, ws.data_ptr(), ws.numel(), stream)


CASES = [
    # first call: the largest the scratch holds at B4 H32 D128 FP8 takes most of it
    (W("seq_sweep", Nq=10880, Nkv=10880), "block"),
    # second call: smaller, another dtype, layout, head dim and P.V mode
    (W("llm_prefill", Hq=8, Hkv=2, Nq=700, Nkv=900, D=96, layout="NHD"), "block"),
    (W("video_dit", Hq=4, Hkv=4, Nq=300, Nkv=333, D=64), "thread"),
]


def test_noalloc_matches_workspace_call():
    L = qa.lib()
    assert L.sage_quant_qkv_noalloc_max_bytes() == 32 << 20
    for w, gran in CASES:
        print(f"[case] noalloc {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} Nq{w.Nq} Nkv{w.Nkv} D{w.D} {w.layout} {w.pv} {gran}",
              flush=True)
        need = L.sage_quant_qkv_workspace_bytes(w.B, w.Hkv, w.Nkv, w.D, 1 if w.pv == "fp8" else 0)
        assert 0 < need <= 32 << 20
        g = torch.Generator(device="cuda:0").manual_seed(w.seed)
        shp = lambda H, N: (w.B, H, N, w.D) if w.layout == "HND" else (w.B, N, H, w.D)
        q = torch.randn(*shp(w.Hq, w.Nq), generator=g, device="cuda:0").to(w.torch_dtype)
        k = (torch.randn(*shp(w.Hkv, w.Nkv), generator=g, device="cuda:0") + 1.5).to(w.torch_dtype)
        v = torch.randn(*shp(w.Hkv, w.Nkv), generator=g, device="cuda:0").to(w.torch_dtype)
        ref, got = _outputs(w, gran), _outputs(w, gran)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        assert _call(L, w, q, k, v, ref, gran, ws) == 0
        assert _call(L, w, q, k, v, got, gran) == 0, ctypes.string_at(L.sage_last_error_detail()).decode()
        torch.cuda.synchronize()
        for name in ref:
            if name == "v_scale" and w.pv != "fp8":
                continue
            assert torch.equal(ref[name], got[name]), name


def test_noalloc_rejects_sizes_beyond_the_scratch():
    L = qa.lib()
    w = W("seq_sweep", Nq=16384, Nkv=16384)
    o = _outputs(w.with_(Nq=64, Nkv=64), "block")  # never written: the call is refused first
    z = torch.zeros(1, dtype=torch.bfloat16, device="cuda:0")
    assert _call(L, w, z, z, z, o, "block") == qa.SAGE_ERR_UNSUPPORTED
    assert b"static scratch" in ctypes.string_at(L.sage_last_error_detail())
