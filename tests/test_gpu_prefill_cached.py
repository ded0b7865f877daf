"""Causal GQA prefill after a cached prefix on the GPU (through the C ABI) against the fp64 oracle.

Inputs poison (NaN) the q rows past q_lens[b] and the cache rows past start_pos[b] + q_lens[b],
so a kernel that reads either shows NaN in a checked row."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows, stepped_scores, to_np

pytestmark = pytest.mark.gpu


def _run(inp, q_lens=True, **kw):
    import mha_mla_kv_amd as attn
    ql = inp["q_lens"].cuda() if q_lens else None
    out = attn.attn_prefill_gqa_cached(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["start_pos"].cuda(),
                                       ql, **kw)
    torch.cuda.synchronize()
    return out


def _ref(inp, q_lens=True, **kw):
    return oracle.gqa_prefill_cached(inp["q"], inp["k"], inp["v"], inp["start_pos"],
                                     inp["q_lens"] if q_lens else None, **kw)


CASES = [
    # name, B, S, Hq, Hkv, D, T_max, start_pos, q_lens
    ("gqa4_ragged", 3, 300, 8, 2, 128, 1000, [0, 517, 130], [300, 77, 1]),
    ("gqa4_llama_heads", 2, 256, 32, 8, 128, 900, [640, 37], [256, 200]),
    ("mqa", 2, 200, 8, 1, 128, 700, [333, 64], [200, 150]),
    ("mha", 2, 130, 4, 4, 128, 400, [100, 270], [130, 130]),
    ("gqa16", 1, 150, 32, 2, 128, 500, [311], [150]),
    ("empty_chunk", 2, 100, 8, 2, 128, 300, [10, 50], [0, 100]),
    ("prefix_fills_cache", 2, 64, 8, 2, 128, 256, [256, 251], [64, 64]),
    ("negative_start_clamps", 1, 70, 8, 2, 128, 128, [-5], [70]),
    ("d64", 2, 200, 8, 2, 64, 600, [64, 399], [200, 199]),
    ("minimind768_d96", 2, 300, 8, 4, 96, 1000, [0, 517], [300, 77]),
    ("d96_mqa", 2, 150, 8, 1, 96, 500, [201, 33], [150, 90]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cached_prefill_matches_oracle(case):
    name, B, S, Hq, Hkv, D, T, sp, ql = case
    inp = synth.gqa_prefill_cached_inputs(B, S, Hq, Hkv, D, T, sp, ql, seed=41)
    print(f"[case] {name}", flush=True)
    out = _run(inp)
    assert_close_rows(out, _ref(inp), TOL_BF16, name)


def test_cached_prefill_all_rows_and_fp32_scale():
    """q_lens NULL (every row new), fp32 output and an explicit scale."""
    inp = synth.gqa_prefill_cached_inputs(2, 190, 8, 2, 128, 800, [450, 3], None, seed=43)
    out = _run(inp, q_lens=False, out_dtype=torch.float32, softmax_scale=0.06)
    assert out.dtype == torch.float32
    assert_close_rows(out, _ref(inp, q_lens=False, softmax_scale=0.06), TOL_BF16, "q_lens NULL, fp32, scale")


def test_zero_prefix_is_causal_prefill_bitwise():
    """start_pos 0 over a cache of exactly S rows runs the causal prefill arithmetic unchanged."""
    import mha_mla_kv_amd as attn
    inp = synth.gqa_prefill_inputs(2, 333, 8, 2, 128, seed=44)
    q, k, v = inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda()
    a = attn.attn_prefill_gqa_causal(q, k, v, out_dtype=torch.float32)
    b = attn.attn_prefill_gqa_cached(q, k, v, torch.zeros(2, dtype=torch.int32, device="cuda"),
                                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_cached_row_is_decode_at_its_position():
    """New token i equals a decode of the same query over the first start_pos + i + 1 cache rows
    (both through the library; same tolerance as against the oracle)."""
    import mha_mla_kv_amd as attn
    inp = synth.gqa_prefill_cached_inputs(1, 96, 8, 2, 128, 600, [389], [96], seed=45)
    pre = to_np(_run(inp, out_dtype=torch.float32))
    for i in (0, 31, 63, 95):
        q = inp["q"][:, i].contiguous().cuda()
        lens = torch.tensor([389 + i + 1], dtype=torch.int32, device="cuda")
        dec = attn.attn_decode_gqa(q, inp["k"].cuda(), inp["v"].cuda(), lens, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close_rows(pre[:, i], dec, TOL_BF16, f"row {i} vs decode")


def test_chunked_prefill_full_size_sampled_rows():
    """Llama-3-8B heads (Hq 32, Hkv 8, head_dim 128), 4 sequences, a 512-token chunk after a
    3584-token prefix, in the benchmark's launch configuration; sampled rows vs the oracle."""
    inp = synth.make("llama3_8b_gqa_chunked_prefill")
    out = to_np(_run(inp))
    assert np.all(np.isfinite(out))
    rows = [0, 1, 63, 64, 127, 128, 300, 511]
    # row i alone: a one-token chunk at position start_pos + i over the same cache
    ref = np.concatenate([oracle.gqa_prefill_cached(inp["q"][:, i:i + 1], inp["k"], inp["v"], inp["start_pos"] + i,
                                                    None) for i in rows], axis=1)
    assert_close_rows(out[:, rows], ref, TOL_BF16, "chunked prefill full size sampled rows")


def test_cached_prefill_moving_max_matches_oracle():
    """Scores that climb tile after tile over the cached prefix and the chunk (the reference max
    moves on every tile after the first)."""
    inp = synth.gqa_prefill_cached_inputs(2, 200, 8, 2, 128, 400, [200, 64], [200, 141], seed=39)  # 7 key tiles
    inp["q"], inp["k"] = stepped_scores(inp["q"], inp["k"], 4)
    assert_close_rows(_run(inp), _ref(inp), TOL_BF16, "cached, moving max")
