"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: K mean, INT8 Q/K codes and block scales, V^ codes and V scales, INT32
score tiles.  Output: max-abs <= 1e-2 and cosine >= 0.9999 against the emulation;
cosine >= 0.999 and relative L1 <= 3e-2 (FP16 P.V) / 5e-2 (FP8 P.V) against fp64
exact attention.  Big workloads compare sampled query rows.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_attention_04_amd as qa
import synth_inputs as si
from gpu_helpers import Case, check_output, check_quant_bit_exact, note, sm_scale_of, tile_sample

pytestmark = pytest.mark.gpu

W = si.workload

# (id, workload) -- the five workload families at their sizes plus ragged / odd shapes
QUANT_CASES = [
    ("tiny", W("tiny")),
    ("llm_prefill", W("llm_prefill")),
    ("video_dit", W("video_dit")),
    ("sweep_1k", W("seq_sweep", Nq=1024, Nkv=1024)),
    ("sweep_32k", W("seq_sweep", Nq=32768, Nkv=32768)),
    ("gqa_d128", W("gqa")),
    ("gqa_d96", W("gqa", D=96)),
    ("ragged_fp16_d40", W("tiny", B=2, Hq=3, Hkv=3, Nq=100, Nkv=100, D=40, seed=11)),
    ("ragged_bf16_nhd_d72_fp8", W("video_dit", B=2, Hq=4, Hkv=2, Nq=70, Nkv=200, D=72, seed=12)),
    ("one_token_d8", W("tiny", Nq=1, Nkv=1, D=8, seed=13)),
    ("d100_fp8", W("seq_sweep", B=1, Hq=2, Hkv=2, Nq=300, Nkv=300, D=100, seed=14)),
    ("d256_fp8", W("seq_sweep", B=1, Hq=4, Hkv=2, Nq=300, Nkv=300, D=256, seed=22)),
    ("d200_fp16_nhd", W("gqa", B=1, Hq=4, Hkv=2, Nq=200, Nkv=250, D=200, seed=23)),
]


@pytest.mark.parametrize("cid,w", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_quantization_bit_exact(cid, w):
    case = Case(w)
    qk, vq = case.gpu_quant()
    check_quant_bit_exact(case, qk, vq)
    # the other P.V mode of the same V
    other = "fp16" if w.pv == "fp8" else "fp8"
    case2 = case.with_pv(other)
    vq2 = qa.quant_v(case2.dv, w.layout, other)
    torch.cuda.synchronize()
    check_quant_bit_exact(case2, qk, vq2)


@pytest.mark.parametrize("cid,w", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_fused_quantization_bit_exact(cid, w):
    """sage_quant_qkv (one call, three or four launches) against the oracle, in both P.V modes."""
    case = Case(w)
    qk, vq = case.gpu_quant(fused=True)
    check_quant_bit_exact(case, qk, vq)
    case2 = case.with_pv("fp16" if w.pv == "fp8" else "fp8")
    qk2, vq2 = case2.gpu_quant(fused=True)
    check_quant_bit_exact(case2, qk2, vq2)


TILE_CASES = [
    ("tiny", W("tiny")),
    ("llm_prefill", W("llm_prefill")),
    ("video_dit_small", W("video_dit", Nq=1000, Nkv=1000, Hq=2, Hkv=2)),
    ("gqa_d96", W("gqa", Nq=700, Nkv=700, B=1)),
    ("ragged_d40", W("tiny", B=2, Hq=4, Hkv=2, Nq=100, Nkv=150, D=40, seed=11)),
    ("d256", W("seq_sweep", B=1, Hq=2, Hkv=2, Nq=200, Nkv=200, D=256, seed=22)),
    ("d200", W("gqa", B=1, Hq=4, Hkv=2, Nq=130, Nkv=190, D=200, seed=23)),
]


@pytest.mark.parametrize("pv", ["fp16", "fp8"])
@pytest.mark.parametrize("cid,w", TILE_CASES, ids=[c[0] for c in TILE_CASES])
def test_int32_score_tiles_bit_exact(cid, w, pv):
    case = Case(w)
    qk, _ = case.gpu_quant()
    tiles = tile_sample(w)
    note(f"[gpu] debug_qk_int32 {len(tiles)} tiles pv={pv}")
    got = qa.debug_qk_int32(qk, torch.from_numpy(tiles).to("cuda:0"), pv).cpu().numpy()
    ref = oracle.scores_i32(case.oq, tiles)
    np.testing.assert_array_equal(got, ref)


OUT_CASES = [
    ("tiny", W("tiny"), "all"),
    ("llm_prefill", W("llm_prefill"), "all"),
    ("llm_prefill_causal", W("llm_prefill", causal=True), "all"),
    ("video_dit", W("video_dit"), 48),
    ("sweep_1k", W("seq_sweep", Nq=1024, Nkv=1024), 64),
    ("sweep_1k_causal", W("seq_sweep", Nq=1024, Nkv=1024, causal=True), 64),
    ("sweep_8k", W("seq_sweep"), 16),
    ("sweep_8k_causal", W("seq_sweep", causal=True), 16),
    ("gqa_d128", W("gqa"), 24),
    ("gqa_d96", W("gqa", D=96), 24),
    ("ragged_fp16_d40", W("tiny", B=2, Hq=3, Hkv=3, Nq=100, Nkv=100, D=40, seed=11), "all"),
    ("ragged_causal_fp8", W("seq_sweep", B=2, Hq=4, Hkv=2, Nq=333, Nkv=333, D=128, causal=True, seed=15), "all"),
    ("nq_ne_nkv_fp8", W("video_dit", B=2, Hq=4, Hkv=2, Nq=70, Nkv=200, D=72, seed=12), "all"),
    ("d100_fp8", W("seq_sweep", B=1, Hq=2, Hkv=2, Nq=300, Nkv=300, D=100, seed=14), "all"),
    ("one_key", W("tiny", Nq=130, Nkv=1, seed=16), "all"),
    ("one_query", W("llm_prefill", Nq=1, Nkv=500, seed=17), "all"),
    # causal with Nq != Nkv: the diagonal aligned to the bottom-right corner
    ("causal_nq_lt_nkv_fp8", W("seq_sweep", B=2, Hq=4, Hkv=2, Nq=130, Nkv=333, causal=True, seed=18), "all"),
    ("causal_nq_gt_nkv_fp16", W("llm_prefill", Hq=4, Hkv=2, Nq=300, Nkv=100, causal=True, seed=19), "all"),
    ("causal_decode_d64_fp8", W("video_dit", Hq=2, Hkv=2, Nq=1, Nkv=1000, causal=True, seed=20), "all"),
    ("causal_chunk_d96", W("gqa", B=1, Nq=200, Nkv=1500, D=96, causal=True, seed=21), "all"),
    # six kv heads in causal groups of four: a full group, then a partial one
    ("causal_head_groups_4_2", W("seq_sweep", B=3, Hq=4, Hkv=2, Nq=260, Nkv=260, causal=True, seed=27), "all"),
    # groups of more than four kv heads, where a group fits one XCD's share of the grid:
    # 68 kv heads (B34, H_kv 2, G 2, two query tiles: 4 workgroups per kv head, 272 in
    # all, 34 per XCD) make groups of eight -- eight full ones, then a partial one of four
    ("causal_head_groups_8_4", W("seq_sweep", B=34, Hq=4, Hkv=2, Nq=200, Nkv=200, causal=True, seed=127), 16),
    # head dims above 128: Dp = 256
    ("d256_fp8", W("seq_sweep", B=1, Hq=4, Hkv=2, Nq=300, Nkv=300, D=256, seed=22), "all"),
    ("d256_causal_fp16", W("llm_prefill", Hq=2, Hkv=2, Nq=300, Nkv=300, D=256, causal=True, seed=24), "all"),
    ("d200_gqa_nhd", W("gqa", B=1, Hq=8, Hkv=2, Nq=500, Nkv=500, D=200, seed=25), "all"),
    ("d256_4k", W("seq_sweep", B=1, Hq=8, Hkv=8, Nq=4096, Nkv=4096, D=256, seed=26), 16),
]


@pytest.mark.parametrize("cid,w,rows", OUT_CASES, ids=[c[0] for c in OUT_CASES])
def test_output_matches_oracle(cid, w, rows):
    case = Case(w)
    qk, vq = case.gpu_quant()
    r = oracle.all_rows(w.B, w.Hq, w.Nq) if rows == "all" else oracle.sample_rows(w.B, w.Hq, w.Nq, rows, seed=3)
    accums = ["fp32", "fp16+fp32"]
    for acc in accums:
        out = case.gpu_attn(qk, vq, accum=acc)
        check_output(case, out, r, exact=(acc == w.accum))


def test_sweep_32k_sampled_rows():
    """The largest sweep point at full size, in the launch configuration the benchmark times."""
    w = W("seq_sweep", Nq=32768, Nkv=32768)
    case = Case(w)
    qk, vq = case.gpu_quant()
    out = case.gpu_attn(qk, vq)
    rows = oracle.sample_rows(w.B, w.Hq, w.Nq, per_head=4, seed=5)
    check_output(case, out, rows, exact=True)


def test_sweep_16k_causal_sampled_rows():
    """Causal at 16K, where the launch interleaves the query tiles of kv-head pairs."""
    w = W("seq_sweep", Nq=16384, Nkv=16384, causal=True)
    case = Case(w)
    qk, vq = case.gpu_quant()
    out = case.gpu_attn(qk, vq)
    rows = oracle.sample_rows(w.B, w.Hq, w.Nq, per_head=4, seed=6)
    check_output(case, out, rows, exact=True)


# The rest of the sequence sweep (1K and 8K are in OUT_CASES, 32K non-causal and 16K causal
# above), in the launch configuration the benchmark times.  At 32K causal each kv head's
# K^ + V^ take 8 MiB, so the causal order runs one head at a time (group of one).
SWEEP_CASES = [
    ("sweep_2k", W("seq_sweep", Nq=2048, Nkv=2048), 8),
    ("sweep_2k_causal", W("seq_sweep", Nq=2048, Nkv=2048, causal=True), 8),
    ("sweep_4k", W("seq_sweep", Nq=4096, Nkv=4096), 8),
    ("sweep_4k_causal", W("seq_sweep", Nq=4096, Nkv=4096, causal=True), 8),
    ("sweep_16k", W("seq_sweep", Nq=16384, Nkv=16384), 4),
    ("sweep_32k_causal", W("seq_sweep", Nq=32768, Nkv=32768, causal=True), 4),
]


@pytest.mark.parametrize("cid,w,per_head", SWEEP_CASES, ids=[c[0] for c in SWEEP_CASES])
def test_sweep_points_sampled_rows(cid, w, per_head):
    case = Case(w)
    qk, vq = case.gpu_quant(fused=True)
    out = case.gpu_attn(qk, vq)
    rows = oracle.sample_rows(w.B, w.Hq, w.Nq, per_head=per_head, seed=7)
    check_output(case, out, rows, exact=True)


def test_layouts_give_identical_outputs():
    w = W("gqa", B=1, Nq=500, Nkv=500, D=96)
    a = Case(w.with_(layout="HND"))
    b = Case(w.with_(layout="NHD"))
    oa = a.gpu_attn(*a.gpu_quant())
    ob = b.gpu_attn(*b.gpu_quant())
    assert torch.equal(oa, ob.transpose(1, 2).contiguous())


def test_gqa_equals_repeated_kv_heads_on_gpu():
    w = W("gqa", B=1, Nq=600, Nkv=600)
    c = Case(w)
    out = c.gpu_attn(*c.gpu_quant())
    k_rep = c.dk.repeat_interleave(w.Hq // w.Hkv, dim=2).contiguous()   # NHD: heads on dim 2
    v_rep = c.dv.repeat_interleave(w.Hq // w.Hkv, dim=2).contiguous()
    qk = qa.quant_qk(c.dq, k_rep, "NHD")
    vq = qa.quant_v(v_rep, "NHD", w.pv)
    out2 = qa.attn_fwd(qk, vq, w.torch_dtype, "NHD", True, sm_scale_of(w.D), w.accum)
    assert torch.equal(out, out2)


def test_deterministic():
    w = W("seq_sweep", B=1, Hq=4, Hkv=4, Nq=2048, Nkv=2048)
    c = Case(w)
    qk, vq = c.gpu_quant()
    o1 = c.gpu_attn(qk, vq)
    qk2, vq2 = c.gpu_quant()
    o2 = c.gpu_attn(qk2, vq2)
    assert torch.equal(o1, o2)


def test_sageattn_composition():
    w = W("llm_prefill", Nq=640, Nkv=640, causal=True)
    c = Case(w)
    out = qa.sageattn(c.dq, c.dk, c.dv, "HND", True, pv="fp16", accum="fp32")
    check_output(c, out, oracle.all_rows(w.B, w.Hq, w.Nq), causal=True)
    # default sm_scale is 1/sqrt(D)
    out2 = qa.sageattn(c.dq, c.dk, c.dv, "HND", True, sm_scale=1 / np.sqrt(128), pv="fp16")
    assert torch.equal(out, out2)


def test_zero_query_block_gives_mean_of_values():
    """An all-zero Q block has scale 0: every score is 0, so each output row is the
    mean of the V^ rows (within the P rounding)."""
    w = W("tiny", Nq=128, Nkv=200, seed=18)
    c = Case(w)
    c.dq[:, :, :64] = 0
    c.q[:, :, :64] = 0
    c.qf[:, :, :64] = 0
    qk, vq = c.gpu_quant()
    assert float(qk.q_scale[0, 0, 0]) == 0.0
    out = c.gpu_attn(qk, vq)
    check_output(c, out, oracle.all_rows(w.B, w.Hq, w.Nq))


@pytest.mark.parametrize("D,pv", [(128, "fp8"), (128, "fp16"), (64, "fp8"), (120, "fp8")])
def test_extreme_scores(D, pv):
    """Every INT8 score at its extreme, +-D * 127^2 (2064512 at D = 128): Q constant (codes
    127, or -127 in the second head) against K rows of alternating sign per token (channel
    mean 0, codes +-127).  Half the keys then score about +16 in log2 units and half about
    -16; the output is the mean of the V^ rows of the winning keys."""
    w = W("tiny", B=1, Hq=2, Hkv=2, Nq=128, Nkv=192, D=D, pv=pv, seed=31)
    c = Case(w)
    sign = torch.tensor([1.0, -1.0], dtype=torch.float32).view(1, 2, 1, 1)
    q = (torch.ones(1, 2, w.Nq, D) * sign).to(c.q.dtype)
    tok = torch.where(torch.arange(w.Nkv) % 2 == 0, 1.0, -1.0).view(1, 1, w.Nkv, 1)
    k = (torch.ones(1, 2, w.Nkv, D) * tok).to(c.k.dtype)
    c.q, c.k = q, k
    c.dq, c.dk = q.to(c.dq.device), k.to(c.dk.device)
    c.qf, c.kf = (oracle.to_hnd_f32(t, w.layout) for t in (q, k))
    qk, vq = c.gpu_quant()
    check_quant_bit_exact(c, qk, vq)
    assert int(qk.q_i8[0, 0, 0, 0]) == 127 and int(qk.q_i8[0, 1, 0, 0]) == -127
    assert int(qk.k_i8[0, 0, 0, 0]) == 127 and int(qk.k_i8[0, 0, 1, 0]) == -127
    for causal in (False, True):
        out = c.gpu_attn(qk, vq, causal=causal)
        check_output(c, out, oracle.all_rows(w.B, w.Hq, w.Nq), causal=causal)
