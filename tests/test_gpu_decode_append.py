"""Decode step with the new token's K/V (attn_decode_gqa_append) on the GPU, through the C ABI:
the output against the fp64 oracle decode over the cache with the new row in place, and the
cache afterwards against the oracle's append, bit for bit.  Cache rows past each length are NaN
before the call, so a read of the row being written (or beyond) would show."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, TOL_FP32, assert_close_rows

pytestmark = pytest.mark.gpu


def _step(B, Hq, Hkv, D, T, lens, dtype="bf16", split=0, seed=71):
    import mha_mla_kv_amd as attn
    inp = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, lens, dtype=dtype, seed=seed)  # NaN past each length
    g = torch.Generator().manual_seed(seed)
    tdt = inp["q"].dtype
    k_new = torch.randn(B, Hkv, D, generator=g).to(tdt)
    v_new = torch.randn(B, Hkv, D, generator=g).to(tdt)
    kc, vc = inp["k"].cuda(), inp["v"].cuda()
    out = attn.attn_decode_gqa_append(inp["q"].cuda(), k_new.cuda(), v_new.cuda(), kc, vc,
                                      inp["cache_lens"].cuda(), split_tokens=split)
    torch.cuda.synchronize()
    L = np.clip(inp["cache_lens"].numpy(), 0, T)
    # reference: the cache extended by one row, the new token at row L_b, decode over L_b + 1 rows
    f = lambda t: t.float().numpy()
    ext_k = np.concatenate([f(inp["k"]), np.zeros((B, 1, Hkv, D), np.float32)], axis=1)
    ext_v = np.concatenate([f(inp["v"]), np.zeros((B, 1, Hkv, D), np.float32)], axis=1)
    for b in range(B):
        ext_k[b, L[b]] = f(k_new[b])
        ext_v[b, L[b]] = f(v_new[b])
    ref = oracle.gqa_decode(f(inp["q"]), ext_k, ext_v, (L + 1).astype(np.int32))
    bits = lambda t: t.cpu().view(torch.int16 if tdt == torch.bfloat16 else torch.int32).numpy()
    kb = oracle.cache_append(bits(inp["k"]), bits(k_new)[:, None], L, np.ones(B, np.int32))
    vb = oracle.cache_append(bits(inp["v"]), bits(v_new)[:, None], L, np.ones(B, np.int32))
    assert np.array_equal(bits(kc), kb) and np.array_equal(bits(vc), vb), "cache after the step"
    return out, ref


CASES = [
    # name, B, Hq, Hkv, D, T_max, lens, dtype, split
    ("gqa4_ragged", 4, 32, 8, 128, 1500, [0, 1, 700, 1499], "bf16", 0),
    ("gqa4_full_cache", 3, 32, 8, 128, 600, [600, 599, 300], "bf16", 0),
    ("one_chunk", 3, 8, 2, 128, 200, [200, 0, 57], "bf16", 0),
    ("mqa", 2, 32, 1, 128, 3000, [2999, 1234], "bf16", 0),
    ("mha", 2, 8, 8, 128, 900, [899, 100], "bf16", 64),
    ("d64", 3, 16, 4, 64, 700, [0, 333, 700], "bf16", 0),
    ("d96_fp32", 2, 8, 4, 96, 512, [511, 40], "f32", 0),
    ("single_chunk_split", 3, 8, 2, 128, 200, [200, 0, 57], "bf16", 256),  # one chunk: merge still runs
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_append_matches_oracle(case):
    name, B, Hq, Hkv, D, T, lens, dtype, split = case
    print(f"[case] {name}", flush=True)
    out, ref = _step(B, Hq, Hkv, D, T, lens, dtype, split)
    assert_close_rows(out, ref, TOL_BF16 if dtype == "bf16" else TOL_FP32, name)


def test_decode_append_fixed_schedule_large_batch():
    """More sequences than the queue schedule plans for: one workgroup per unit."""
    print("[case] B=1100 fixed schedule", flush=True)
    out, ref = _step(1100, 8, 2, 128, 130, (0, 130), seed=72)
    assert_close_rows(out, ref, TOL_BF16, "fixed schedule")


def test_decode_append_equals_append_then_decode():
    import mha_mla_kv_amd as attn
    B, Hq, Hkv, D, T = 8, 32, 8, 128, 4096
    inp = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, (1, 4000), seed=73)
    g = torch.Generator().manual_seed(73)
    k_new, v_new = (torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16).cuda() for _ in range(2))
    q, lens = inp["q"].cuda(), inp["cache_lens"].cuda()
    k1, v1 = inp["k"].cuda(), inp["v"].cuda()
    fused = attn.attn_decode_gqa_append(q, k_new, v_new, k1, v1, lens)
    k2, v2 = inp["k"].cuda(), inp["v"].cuda()
    attn.attn_cache_append(k_new[:, None].contiguous(), k2, v_new[:, None].contiguous(), v2, lens)
    plain = attn.attn_decode_gqa(q, k2, v2, lens + 1)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16)) and torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    assert_close_rows(fused, plain.double().cpu().numpy(), TOL_BF16, "fused vs append + decode")
