"""GQA decode over int4 caches (attn_decode_gqa_int4kv) on the GPU, through the C ABI, against the
fp64 oracle decode over the caches' values (oracle.int4_to_float: codes times their rows' scales).
The scales of rows past each length are NaN, so reading them shows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows, to_np

pytestmark = pytest.mark.gpu


def _values(inp, name, sl=slice(None)):
    """The cache's values in the [B,T_max,Hkv,128] layout the oracle decode takes (the int4 caches
    are head-major)."""
    x = oracle.int4_to_float(inp[name][sl].numpy(), inp[name + "_scale"][sl].numpy())
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3)).astype(np.float32)


def _run(inp, **kw):
    import mha_mla_kv_amd as attn
    out = attn.attn_decode_gqa_int4kv(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["k_scale"].cuda(),
                                      inp["v_scale"].cuda(), inp["cache_lens"].cuda(), **kw)
    torch.cuda.synchronize()
    return out


def _ref(inp, sl=slice(None), **kw):
    return oracle.gqa_decode(inp["q"][sl], _values(inp, "k", sl), _values(inp, "v", sl), inp["cache_lens"][sl], **kw)


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
def test_int4_decode_matches_oracle(case):
    name, B, Hq, Hkv, T, lens, split = case
    print(f"[case] {name}", flush=True)
    inp = synth.gqa_decode_int4_inputs(B, Hq, Hkv, 128, T, lens, seed=91)
    assert_close_rows(_run(inp, split_tokens=split), _ref(inp), TOL_BF16, name)


def test_int4_decode_bf16_output_and_scale():
    inp = synth.gqa_decode_int4_inputs(3, 16, 4, 128, 800, [800, 5, 444], seed=92)
    out = _run(inp, out_dtype=torch.bfloat16, softmax_scale=0.05)
    assert out.dtype == torch.bfloat16
    assert_close_rows(out, _ref(inp, softmax_scale=0.05), TOL_BF16, "bf16 out, scale 0.05")


def test_int4_decode_extreme_codes():
    """Every element of every cached row at -8 or at 7 (the codes' extremes, where the offset of
    the widening is largest relative to the value), with unit scales."""
    import mha_mla_kv_amd as attn
    inp = synth.gqa_decode_int4_inputs(2, 16, 4, 128, 300, [300, 129], seed=93)
    g = torch.Generator().manual_seed(93)
    hi = torch.randint(0, 2, inp["k"].shape, generator=g, dtype=torch.uint8)
    inp["k"] = torch.where(hi.bool(), torch.tensor(0x77, dtype=torch.uint8), torch.tensor(0x88, dtype=torch.uint8))
    inp["v"] = torch.where(hi.flip(-1).bool(), torch.tensor(0x87, dtype=torch.uint8), torch.tensor(0x78, dtype=torch.uint8))
    L = inp["cache_lens"].numpy()
    for name in ("k_scale", "v_scale"):
        sc = torch.full_like(inp[name], 0.125)
        for b in range(2):
            sc[b, :, L[b]:] = float("nan")
        inp[name] = sc
    assert_close_rows(_run(inp), _ref(inp), TOL_BF16, "extreme codes")


def test_int4_decode_fixed_schedule_large_batch():
    print("[case] B=1100 fixed schedule", flush=True)
    inp = synth.gqa_decode_int4_inputs(1100, 8, 2, 128, 130, (0, 130), seed=94)
    assert_close_rows(_run(inp), _ref(inp), TOL_BF16, "fixed schedule")


def test_int4_decode_full_size_sampled_rows():
    """The Llama-3-8B decode shape (B 32, Hq 32, Hkv 8, T_max 8192, lengths U[1024, 8192]) with int4
    caches, in the benchmark's launch configuration; every head of sampled sequences."""
    inp = synth.gqa_decode_int4_inputs(32, 32, 8, 128, 8192, (1024, 8192), seed=2)
    out = to_np(_run(inp))
    for b in (0, 15, 31):
        sl = slice(b, b + 1)
        assert_close_rows(out[sl], _ref(inp, sl), TOL_BF16, f"int4 full size b={b}")
