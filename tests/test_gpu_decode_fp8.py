"""GQA decode over FP8 E4M3 caches (attn_decode_gqa_fp8kv) on the GPU, through the C ABI, against
the fp64 oracle decode over the caches' values (codes decoded from the format's definition,
times the scales).  Codes past each length are NaN."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows, row_rel_err, to_np

pytestmark = pytest.mark.gpu


def _values(inp, name, sl=slice(None)):
    codes = inp[name][sl].contiguous().view(torch.uint8).numpy()
    return oracle.e4m3_to_float(codes, inp[name + "_scale"]).astype(np.float32)


def _run(inp, **kw):
    import mha_mla_kv_amd as attn
    out = attn.attn_decode_gqa_fp8kv(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["k_scale"],
                                     inp["v_scale"], inp["cache_lens"].cuda(), **kw)
    torch.cuda.synchronize()
    return out


def _ref(inp, sl=slice(None)):
    return oracle.gqa_decode(inp["q"][sl], _values(inp, "k", sl), _values(inp, "v", sl), inp["cache_lens"][sl])


CASES = [
    # name, B, Hq, Hkv, T_max, lens, split
    ("gqa4_ragged", 4, 32, 8, 1500, [0, 1, 700, 1500], 0),
    ("gqa4_split64", 3, 32, 8, 900, [899, 64, 65], 64),
    ("mqa_n32", 2, 32, 1, 3000, [2999, 1234], 0),
    ("mha", 2, 8, 8, 700, [700, 33], 0),
    ("gqa16", 2, 32, 2, 600, [599, 300], 0),
    ("n_rep64", 1, 64, 1, 500, [500], 0),
    ("one_chunk", 3, 8, 2, 64, [64, 0, 17], 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_decode_matches_oracle(case):
    name, B, Hq, Hkv, T, lens, split = case
    print(f"[case] {name}", flush=True)
    inp = synth.gqa_decode_fp8_inputs(B, Hq, Hkv, 128, T, lens, seed=81)
    assert_close_rows(_run(inp, split_tokens=split), _ref(inp), TOL_BF16, name)


def test_fp8_decode_bf16_output_and_scale():
    inp = synth.gqa_decode_fp8_inputs(3, 16, 4, 128, 800, [800, 5, 444], seed=82)
    out = _run(inp, out_dtype=torch.bfloat16, softmax_scale=0.05)
    assert out.dtype == torch.bfloat16
    ref = oracle.gqa_decode(inp["q"], _values(inp, "k"), _values(inp, "v"), inp["cache_lens"], softmax_scale=0.05)
    assert_close_rows(out, ref, TOL_BF16, "bf16 out, scale 0.05")


def test_fp8_decode_fixed_schedule_large_batch():
    print("[case] B=1100 fixed schedule", flush=True)
    inp = synth.gqa_decode_fp8_inputs(1100, 8, 2, 128, 130, (0, 130), seed=83)
    assert_close_rows(_run(inp), _ref(inp), TOL_BF16, "fixed schedule")


def test_fp8_decode_full_size_sampled_rows():
    """The Llama-3-8B decode shape (B 32, Hq 32, Hkv 8, T_max 8192, lengths U[1024, 8192]) with fp8
    caches, in the benchmark's launch configuration; every head of sampled sequences."""
    inp = synth.gqa_decode_fp8_inputs(32, 32, 8, 128, 8192, (1024, 8192), seed=2)
    out = to_np(_run(inp))
    for b in (0, 15, 31):
        sl = slice(b, b + 1)
        assert_close_rows(out[sl], _ref(inp, sl), TOL_BF16, f"fp8 full size b={b}")


@pytest.mark.parametrize("B,Hq,Hkv,T,lens", [(4, 32, 8, 1500, [0, 1, 700, 1500]), (2, 32, 1, 3000, [2999, 1234]),
                                             (3, 8, 2, 640, [640, 639, 5]), (2, 16, 4, 8192, [8192, 4097])])
def test_fp8_default_chunk_fits_the_decode_workspace(B, Hq, Hkv, T, lens):
    """split_tokens = 0 picks a longer chunk for FP8 caches than attn_decode_gqa does; a workspace
    of exactly attn_decode_gqa_workspace_bytes(..., 0) is enough for it, and the output matches the
    oracle and the same call with 64-position chunks (up to fp32 rounding)."""
    import mha_mla_kv_amd as attn
    inp = synth.gqa_decode_fp8_inputs(B, Hq, Hkv, 128, T, lens, seed=19)
    n = attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, 128, T, 0)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = _run(inp, workspace=ws)
    assert_close_rows(out, _ref(inp), TOL_BF16, f"fp8 default chunk B={B} Hq={Hq} Hkv={Hkv} T={T}")
    # different chunks round the bf16 probabilities against different running maxima: about 2^-9
    assert row_rel_err(out, _run(inp, split_tokens=64)) <= 5e-3
