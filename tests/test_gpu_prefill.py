"""Causal GQA prefill on the GPU (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows, stepped_scores, to_np

pytestmark = pytest.mark.gpu


def _run(inp, **kw):
    import mha_mla_kv_amd as attn
    out = attn.attn_prefill_gqa_causal(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), **kw)
    torch.cuda.synchronize()
    return out


CASES = [
    # name, B, S, Hq, Hkv, D
    ("gqa4_s300", 2, 300, 8, 2, 128),      # several q/k tiles and a ragged tail
    ("gqa4_s256", 1, 256, 32, 8, 128),
    ("mqa_s200", 1, 200, 8, 1, 128),
    ("mha_s130", 2, 130, 4, 4, 128),
    ("s1", 2, 1, 8, 2, 128),
    ("s63", 1, 63, 4, 2, 128),
    ("d64_s200", 2, 200, 8, 2, 64),
    ("minimind768_d96_s300", 2, 300, 8, 4, 96),  # the MiniMind-768 GQA heads (2*4*96 cached per token)
    ("d96_mqa_s200", 1, 200, 8, 1, 96),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(case):
    name, B, S, Hq, Hkv, D = case
    inp = synth.gqa_prefill_inputs(B, S, Hq, Hkv, D, seed=31)
    print(f"[case] {name}", flush=True)
    out = _run(inp)
    ref = oracle.gqa_prefill_causal(inp["q"], inp["k"], inp["v"])
    assert_close_rows(out, ref, TOL_BF16, name)


def test_prefill_fp32_output_and_scale():
    inp = synth.gqa_prefill_inputs(1, 150, 8, 2, 128, seed=7)
    out = _run(inp, out_dtype=torch.float32, softmax_scale=0.05)
    assert out.dtype == torch.float32
    ref = oracle.gqa_prefill_causal(inp["q"], inp["k"], inp["v"], softmax_scale=0.05)
    assert_close_rows(out, ref, TOL_BF16, "fp32 out, scale 0.05")


def test_prefill_first_row_is_v0_and_deterministic():
    inp = synth.gqa_prefill_inputs(2, 200, 8, 2, 128, seed=3)
    a = to_np(_run(inp, out_dtype=torch.float32))
    b = to_np(_run(inp, out_dtype=torch.float32))
    assert np.array_equal(a, b)
    v = inp["v"].float().numpy()
    for h in range(8):
        # query 0 sees only key 0, so its output is V[0]: the kernel subtracts the
        # row's max from its one visible score, p = 1; the 1e-6 slack covers the
        # normalisation (a leak of any other key would show at the 1e-2 level)
        np.testing.assert_allclose(a[:, 0, h], v[:, 0, h // 4], rtol=1e-6, atol=1e-6)


def test_prefill_full_size_sampled_rows():
    """Llama-3-8B prefill shape (B 4, S 4096, Hq 32, Hkv 8) in the benchmark's launch
    configuration; sampled query positions (incl. tile edges and the last row) vs the oracle."""
    inp = synth.make("llama3_8b_gqa_prefill")
    out = to_np(_run(inp))
    rows = [0, 1, 127, 128, 2047, 2048, 4000, 4095]
    ref = oracle.gqa_prefill_causal(inp["q"], inp["k"], inp["v"], rows=rows)
    assert_close_rows(out[:, rows], ref[:, rows], TOL_BF16, "prefill full size sampled rows")


def test_prefill_moving_max_matches_oracle():
    """Scores that climb tile after tile (stepped_scores): the path where a tile's max exceeds
    the reference by more than the slack, on every tile after the first."""
    inp = synth.gqa_prefill_inputs(2, 330, 8, 2, 128, seed=37)  # 6 key tiles
    inp["q"], inp["k"] = stepped_scores(inp["q"], inp["k"], 4)
    out = _run(inp)
    ref = oracle.gqa_prefill_causal(inp["q"], inp["k"], inp["v"])
    assert_close_rows(out, ref, TOL_BF16, "moving max")
