"""MLA causal prefill on the GPU (through the C ABI) against the fp64 oracle (keys and values
rebuilt from the latent).

Inputs poison (NaN) the query rows past q_lens[b] and the cache rows past
start_pos[b] + q_lens[b], so a kernel that reads either shows NaN in a checked row."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows, to_np

pytestmark = pytest.mark.gpu

KEYS = ("q_nope", "q_rope", "w_uk", "w_uv", "c_kv", "k_rope")
DIMS = (96, 48, 96, 128)  # nope, rope, v, kv_lora_rank (MiniMind-768)


def _run(inp, start=True, lens=True, **kw):
    import mha_mla_kv_amd as attn
    out = attn.attn_prefill_mla_causal(*(inp[k].cuda() for k in KEYS),
                                       start_pos=inp["start_pos"].cuda() if start else None,
                                       q_lens=inp["q_lens"].cuda() if lens else None, **kw)
    torch.cuda.synchronize()
    return out


def _ref(inp, start=True, lens=True, **kw):
    return oracle.mla_prefill_causal(*(inp[k] for k in KEYS), inp["start_pos"] if start else None,
                                     inp["q_lens"] if lens else None, **kw)


CASES = [
    # name, B, S, H, T_max, start_pos, q_lens
    ("no_prefix_s300", 2, 300, 8, 300, [0, 0], [300, 300]),
    ("no_prefix_ragged", 2, 200, 8, 200, [0, 0], [200, 77]),
    ("prefix_ragged", 3, 150, 8, 700, [0, 517, 130], [150, 64, 1]),
    ("h16", 1, 130, 16, 400, [200], [130]),
    ("h1", 2, 100, 1, 300, [37, 150], [100, 100]),
    ("empty_chunk", 2, 90, 8, 300, [10, 40], [0, 90]),
    ("prefix_fills_cache", 2, 64, 8, 256, [256, 250], [64, 64]),
    ("b8_xcd_mapping", 8, 140, 8, 400, [0, 13, 64, 100, 0, 255, 7, 1], [140, 140, 99, 140, 1, 140, 64, 128]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mla_prefill_matches_oracle(case):
    name, B, S, H, T, sp, ql = case
    inp = synth.mla_prefill_inputs(B, S, H, *DIMS, T, sp, ql, seed=51)
    print(f"[case] {name}", flush=True)
    out = _run(inp)
    assert_close_rows(out, _ref(inp), TOL_BF16, name)


def test_mla_prefill_defaults_fp32_and_scale():
    """start_pos and q_lens NULL (the listing's whole-sequence prefill), fp32 output, explicit scale."""
    inp = synth.mla_prefill_inputs(2, 260, 8, *DIMS, 260, 0, None, seed=52)
    out = _run(inp, start=False, lens=False, out_dtype=torch.float32, softmax_scale=0.07)
    assert out.dtype == torch.float32
    assert_close_rows(out, _ref(inp, start=False, lens=False, softmax_scale=0.07), TOL_BF16, "defaults, fp32, scale")


def test_mla_prefill_rows_are_mla_decodes():
    """New token i equals the library's MLA decode of the same query over the cache up to its
    position (same tolerance as against the oracle)."""
    import mha_mla_kv_amd as attn
    inp = synth.mla_prefill_inputs(1, 70, 8, *DIMS, 500, [301], [70], seed=53)
    pre = to_np(_run(inp, out_dtype=torch.float32))
    for i in (0, 31, 64, 69):
        q = [inp["q_nope"][:, i].contiguous().cuda(), inp["q_rope"][:, i].contiguous().cuda()]
        lens = torch.tensor([301 + i + 1], dtype=torch.int32, device="cuda")
        dec = attn.attn_decode_mla_absorbed(*q, *(inp[k].cuda() for k in KEYS[2:]), lens, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close_rows(pre[:, i], dec, TOL_BF16, f"row {i} vs MLA decode")


def test_mla_prefill_deterministic():
    inp = synth.mla_prefill_inputs(1, 200, 8, *DIMS, 200, 0, None, seed=54)
    a = _run(inp, out_dtype=torch.float32)
    b = _run(inp, out_dtype=torch.float32)
    assert torch.equal(a, b)


def test_mla_prefill_full_size_sampled_rows():
    """MiniMind-768 MLA widths, 4 sequences of 4096 tokens, in the benchmark's launch configuration;
    sampled rows vs the oracle, each as a one-token chunk at its own position."""
    inp = synth.make("minimind768_mla_prefill")
    out = to_np(_run(inp))
    assert np.all(np.isfinite(out))
    rows = [0, 1, 127, 128, 2047, 4095]
    ref = np.concatenate([oracle.mla_prefill_causal(inp["q_nope"][:, i:i + 1], inp["q_rope"][:, i:i + 1],
                                                    *(inp[k] for k in KEYS[2:]), inp["start_pos"] + i, None)
                          for i in rows], axis=1)
    assert_close_rows(out[:, rows], ref, TOL_BF16, "MLA prefill full size sampled rows")


def test_mla_prefill_moving_max_matches_oracle():
    """Scores that climb by about 8.4 (log2 units) from one 64-key tile to the next through the
    shared rotated key: q_rope along one direction per sequence, k_rope along it times
    0.5 + 1.45 * (position // 64), plus noise; the latent part scaled down to a small
    perturbation.  The reference max moves on most tiles after the first; six key tiles keep the
    scores below about 50, where the bf16-rounded scaled q_rope moves the weights by about 1%.
    NaN poison stays in place."""
    inp = synth.mla_prefill_inputs(2, 300, 8, *DIMS, 384, [0, 84], [300, 300], seed=53)
    g = torch.Generator().manual_seed(9)
    B, S, H, dR = inp["q_rope"].shape
    T = inp["k_rope"].shape[1]
    u = torch.randn(B, 1, 1, dR, generator=g)
    qr = u + 0.1 * torch.randn(B, S, H, dR, generator=g)
    mag = 0.5 + 1.45 * (torch.arange(T) // 64).float()
    kr = mag[None, :, None] * (u[:, :, 0] + 0.1 * torch.randn(B, T, dR, generator=g))
    inp["q_rope"] = (inp["q_rope"].float() * 0 + qr).to(torch.bfloat16)
    inp["k_rope"] = (inp["k_rope"].float() * 0 + kr).to(torch.bfloat16)
    inp["q_nope"] = (inp["q_nope"].float() * 0.3).to(torch.bfloat16)
    inp["c_kv"] = (inp["c_kv"].float() * 0.3).to(torch.bfloat16)
    assert_close_rows(_run(inp), _ref(inp), TOL_BF16, "mla, moving max")
