"""MLA decode over an FP8 E4M3 latent cache (attn_decode_mla_fp8kv) on the GPU, through the C ABI,
against the fp64 oracle's absorbed decode over the cache's values (oracle.e4m3_to_float: codes
times the cache scale; k_rope bf16).  The latent rows past each length are NaN codes, so reading
them shows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows, to_np

pytestmark = pytest.mark.gpu


def _fp8_case(B, H, dn, dR, dv, r, T, lens, seed):
    inp = synth.mla_decode_inputs(B, H, dn, dR, dv, r, T, lens, seed=seed)
    c = inp["c_kv"].float()
    scale = float(torch.nan_to_num(c, nan=0.0).abs().max()) / 448.0
    inp["c_codes"] = (c / scale).to(torch.float8_e4m3fn)
    inp["c_scale"] = scale
    return inp


def _values(inp):
    return oracle.e4m3_to_float(inp["c_codes"].view(torch.uint8).numpy(), inp["c_scale"])


def _run(inp, **kw):
    import mha_mla_kv_amd as attn
    d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    out = attn.attn_decode_mla_fp8kv(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["c_codes"], inp["c_scale"],
                                     d["k_rope"], d["cache_lens"], **kw)
    torch.cuda.synchronize()
    return out


def _ref(inp, sl=slice(None), **kw):
    return oracle.mla_decode_absorbed(inp["q_nope"][sl], inp["q_rope"][sl], inp["w_uk"], inp["w_uv"], _values(inp)[sl],
                                      inp["k_rope"][sl], inp["cache_lens"][sl], **kw)


CASES = [
    # name, B, H, dn, dR, dv, r, T, lens, split
    ("minimind_small", 3, 8, 96, 48, 96, 128, 300, [300, 1, 77], 64),
    ("minimind_auto", 2, 8, 96, 48, 96, 128, 700, [700, 333], 0),
    ("h1_r64_dr16", 2, 1, 32, 16, 48, 64, 200, [200, 33], 64),
    ("h16_r256_dr64", 2, 16, 128, 64, 128, 256, 260, [260, 129], 128),
    ("h5_r128_dr32", 2, 5, 64, 32, 80, 128, 150, [150, 64], 64),
    ("many_chunks", 2, 2, 32, 16, 48, 64, 5000, [5000, 4097], 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_latent_mla_matches_oracle(case):
    name, B, H, dn, dR, dv, r, T, lens, split = case
    print(f"[case] {name}", flush=True)
    inp = _fp8_case(B, H, dn, dR, dv, r, T, lens, seed=61)
    assert_close_rows(_run(inp, split_tokens=split), _ref(inp), TOL_BF16, name)


def test_fp8_latent_mla_empty_sequences_bf16_out_scale():
    inp = _fp8_case(3, 8, 96, 48, 96, 128, 100, [0, 100, 0], seed=62)
    out = _run(inp, split_tokens=64, out_dtype=torch.bfloat16, softmax_scale=0.07)
    o = to_np(out)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert_close_rows(out, _ref(inp, softmax_scale=0.07), TOL_BF16, "fp8 mla empty, bf16 out, scale")


def test_fp8_latent_mla_full_size_minimind():
    """The MiniMind-768 MLA decode shape (B 64, H 8, cache 4096, lengths U[1024, 4096]) with an
    FP8 latent cache, in the default launch configuration; every head of sampled sequences."""
    inp = _fp8_case(64, 8, 96, 48, 96, 128, 4096, (1024, 4096), seed=5)
    out = to_np(_run(inp))
    for b in (0, 31, 63):
        sl = slice(b, b + 1)
        assert_close_rows(out[sl], _ref(inp, sl), TOL_BF16, f"fp8 mla full size b={b}")
