"""HIP graph capture.  The library only enqueues kernels (no allocation, no memset, no
host synchronisation), so a whole step -- quantisation and attention -- can be captured
into a graph and replayed.  Each case captures one step, then replays it three times
with new inputs written eagerly between the replays; every replay must equal the eager
step on the same inputs bit for bit."""
import pytest
import torch

import quantized_attention_04_amd as qa

pytestmark = pytest.mark.gpu

B, H, HKV, N, D = 2, 4, 2, 700, 128  # GQA, ragged last block


def _inputs(dev, gen):
    return [torch.randn(B, h, N, D, device=dev, generator=gen).to(torch.bfloat16) for h in (H, HKV, HKV)]


def _step_fn(kind, q, k, v, causal):
    """Preallocate every buffer once; return a function that runs one step into them."""
    L = qa.lib()
    dev = q.device
    if kind == "mxfp4":
        ws = torch.empty(max(8, L.sage_quant_mxfp4_workspace_bytes(B, HKV, N, D)), dtype=torch.uint8, device=dev)
        mq = qa.quant_mxfp4(q, k, v, workspace=ws)
        out = qa.attn_fwd_mxfp4(mq, torch.bfloat16, "HND", causal)

        def step():
            qa.quant_mxfp4(q, k, v, workspace=ws, out=mq)
            qa.attn_fwd_mxfp4(mq, torch.bfloat16, "HND", causal, out=out)
        return step, out
    pv = "fp16" if kind in ("int8_fp16", "int8_fp16_split") else "fp8"
    if kind == "int8_fused_q":  # sage_quant_kv + sage_attn_fwd_fused_q (Q quantised in the attention prologue)
        ws = torch.empty(max(8, L.sage_quant_qkv_workspace_bytes(B, HKV, N, D, 1)), dtype=torch.uint8, device=dev)
        kq, vq = qa.quant_kv(k, v, "HND", pv, workspace=ws)
        out = qa.attn_fwd_fused_q(q, kq, vq, "HND", causal)

        def step():
            qa.quant_kv(k, v, "HND", pv, workspace=ws, out_k=kq, out_v=vq)
            qa.attn_fwd_fused_q(q, kq, vq, "HND", causal, out=out)
        return step, out
    if kind == "int8_separate":  # sage_quant_qk + sage_quant_v (its FP8 path clears a buffer with a kernel)
        wk = torch.empty(max(8, L.sage_quant_qk_workspace_bytes(B, HKV, N, D)), dtype=torch.uint8, device=dev)
        wv = torch.empty(max(8, L.sage_quant_v_workspace_bytes(B, HKV, D, 1)), dtype=torch.uint8, device=dev)
        qk = qa.quant_qk(q, k, "HND", workspace=wk)
        vq = qa.quant_v(v, "HND", pv, workspace=wv)

        def quant():
            qa.quant_qk(q, k, "HND", workspace=wk, out=qk)
            qa.quant_v(v, "HND", pv, workspace=wv, out=vq)
    else:
        ws = torch.empty(max(8, L.sage_quant_qkv_workspace_bytes(B, HKV, N, D, 1 if pv == "fp8" else 0)),
                         dtype=torch.uint8, device=dev)
        qk, vq = qa.quant_qkv(q, k, v, "HND", pv, workspace=ws)

        def quant():
            qa.quant_qkv(q, k, v, "HND", pv, workspace=ws, out_qk=qk, out_v=vq)
    # key-range splits (split kernel, then the merge): one workspace for every call
    splits = 3 if kind == "int8_fp16_split" else 1
    aws = torch.empty(max(16, qa.split_workspace_bytes(qk, splits)), dtype=torch.uint8, device=dev) \
        if splits > 1 else None
    out = qa.attn_fwd(qk, vq, torch.bfloat16, "HND", causal, splits=splits, workspace=aws)

    def step():
        quant()
        qa.attn_fwd(qk, vq, torch.bfloat16, "HND", causal, out=out, splits=splits, workspace=aws)
    return step, out


@pytest.mark.parametrize("kind,causal", [("int8_fp8", False), ("int8_fp16", True), ("int8_separate", True),
                                         ("mxfp4", True), ("int8_fp16_split", False), ("int8_fp16_split", True),
                                         ("int8_fused_q", True)])
def test_graph_replays_equal_eager_steps(kind, causal):
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(41)
    q, k, v = _inputs(dev, gen)
    step, out = _step_fn(kind, q, k, v, causal)
    # warm up on a side stream, then capture one step
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    print(f"[graph] {kind} causal={causal} captured", flush=True)
    for rep in range(3):
        for t, n in zip((q, k, v), _inputs(dev, gen)):
            t.copy_(n)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        out.zero_()
        step()
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, out), f"replay {rep} differs from the eager step"
