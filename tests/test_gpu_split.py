"""Key-range splits of under-filled launches (sage_attn_fwd_split, FP16 P.V): every split
runs the online softmax over its own key range and a merge combines the fp32 states.
Each output is held to the oracle's bar (emulation and exact attention), and to within
an output rounding or two of the unsplit kernel."""
import numpy as np
import pytest
import torch

import oracle
import quantized_attention_04_amd as qa
import synth_inputs as si
from gpu_helpers import Case, check_output, note, sm_scale_of

pytestmark = pytest.mark.gpu

W = si.workload

CASES = [
    ("llm_prefill", W("llm_prefill"), "auto", "all"),
    ("llm_prefill_causal", W("llm_prefill", causal=True), "auto", "all"),
    ("llm_prefill_3", W("llm_prefill", Nq=1000, Nkv=1000, seed=70), 3, "all"),
    ("ragged_d40_7", W("tiny", B=2, Hq=3, Hkv=3, Nq=333, Nkv=700, D=40, seed=71), 7, "all"),
    ("gqa_d96_nhd_causal_chunk", W("gqa", B=1, Hq=8, Hkv=2, Nq=300, Nkv=1500, D=96, seed=72), 5, "all"),
    ("causal_nq_gt_nkv", W("llm_prefill", Hq=4, Hkv=2, Nq=700, Nkv=600, causal=True, seed=73), 4, "all"),
    ("one_query", W("llm_prefill", Nq=1, Nkv=3000, seed=74), 6, "all"),
    ("d256_causal", W("llm_prefill", Hq=2, Hkv=2, Nq=900, Nkv=900, D=256, causal=True, seed=75), 4, "all"),
    ("d64_bf16", W("tiny", B=1, Hq=4, Hkv=4, Nq=2048, Nkv=2048, dtype="bf16", seed=76), "auto", 64),
]


@pytest.mark.parametrize("cid,w,splits,rows", CASES, ids=[c[0] for c in CASES])
def test_split_output_matches_oracle(cid, w, splits, rows):
    assert w.pv == "fp16"
    case = Case(w)
    qk, vq = case.gpu_quant()
    sm = sm_scale_of(w.D)
    n = qa.split_choice(qk, w.pv, w.causal) if splits == "auto" else splits
    note(f"[gpu] attn_fwd_split {cid} splits={n}")
    assert n > 1
    out = qa.attn_fwd(qk, vq, w.torch_dtype, w.layout, w.causal, sm, "fp32", splits=n)
    plain = qa.attn_fwd(qk, vq, w.torch_dtype, w.layout, w.causal, sm, "fp32")
    torch.cuda.synchronize()
    r = oracle.all_rows(w.B, w.Hq, w.Nq) if rows == "all" else oracle.sample_rows(w.B, w.Hq, w.Nq, rows, seed=2)
    check_output(case, out, r)
    # against the unsplit kernel: the same P up to one fp16 rounding each, merged in fp32
    # (outputs of order 1: a few 1e-4 apart at most; near-zero outputs differ relatively more)
    worst = float((out.float() - plain.float()).abs().max())
    note(f"[split] {cid}: largest difference from the unsplit kernel {worst:g}")
    assert worst <= 2e-3
    if w.causal and w.Nq > w.Nkv:  # queries that see no key
        dead = w.Nq - w.Nkv
        t = out if w.layout == "HND" else out.transpose(1, 2)
        assert not t[:, :, :dead].any()


def test_split_choice_and_determinism():
    w = W("llm_prefill")
    case = Case(w)
    qk, vq = case.gpu_quant()
    n = qa.split_choice(qk, "fp16")
    assert 2 <= n <= 8
    assert qa.split_choice(qk, "fp8") == 1
    ws = torch.empty(qa.split_workspace_bytes(qk, n), dtype=torch.uint8, device="cuda:0")
    o1 = qa.attn_fwd(qk, vq, w.torch_dtype, w.layout, False, None, "fp32", splits=n, workspace=ws)
    ws.fill_(0xFF)  # stale workspace contents play no part
    o2 = qa.attn_fwd(qk, vq, w.torch_dtype, w.layout, False, None, "fp32", splits=n, workspace=ws)
    assert torch.equal(o1, o2)
    # sageattn takes the split itself
    o3 = qa.sageattn(case.dq, case.dk, case.dv, w.layout, False, pv="fp16")
    assert torch.equal(o1, o3)
