"""Causal GQA prefill after a cached prefix that appends the new rows in the same launch
(attn_prefill_gqa_cached_append), on the GPU through the C ABI.

The expected output is the fp64 oracle's cached prefill over the caches holding the new rows; the
expected caches are the oracle's cache append, compared bit for bit.  Before the call the cache rows
at and past start_pos[b] are NaN and the new rows past q_lens[b] are NaN, so a kernel that read the
cache where the new rows go, or new rows past the chunk, shows NaN in a checked row."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows, stepped_scores

pytestmark = pytest.mark.gpu


def _split(inp):
    """k_new / v_new [B,S,Hkv,D] taken from the cache rows start_pos[b].. of the inputs (NaN past
    each chunk's clamped length), and caches with NaN at and past start_pos[b]."""
    k, v = inp["k"], inp["v"]
    B, T = k.shape[0], k.shape[1]
    S = inp["q"].shape[1]
    sp = np.clip(inp["start_pos"].numpy(), 0, T)
    ql = np.clip(inp["q_lens"].numpy(), 0, S)
    n = np.minimum(ql, T - sp)
    nan = torch.tensor(float("nan"), dtype=k.dtype)
    k_new = torch.full((B, S) + tuple(k.shape[2:]), float("nan"), dtype=k.dtype)
    v_new = k_new.clone()
    kc, vc = k.clone(), v.clone()
    for b in range(B):
        k_new[b, :n[b]] = k[b, sp[b]:sp[b] + n[b]]
        v_new[b, :n[b]] = v[b, sp[b]:sp[b] + n[b]]
        kc[b, sp[b]:] = nan
        vc[b, sp[b]:] = nan
    return k_new, v_new, kc, vc


def _bits(t):
    return t.cpu().view(torch.int16).numpy()


def _check(inp, q_lens=True, out_dtype=torch.bfloat16, softmax_scale=0.0, what=""):
    import mha_mla_kv_amd as attn
    k_new, v_new, kc, vc = _split(inp)
    ql = inp["q_lens"] if q_lens else None
    dk, dv = kc.cuda(), vc.cuda()
    out = attn.attn_prefill_gqa_cached_append(inp["q"].cuda(), k_new.cuda(), v_new.cuda(), dk, dv,
                                              inp["start_pos"].cuda(), None if ql is None else ql.cuda(),
                                              out_dtype=out_dtype, softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    ref = oracle.gqa_prefill_cached(inp["q"], inp["k"], inp["v"], inp["start_pos"], ql, softmax_scale=softmax_scale)
    assert_close_rows(out, ref, TOL_BF16, what)
    sp = inp["start_pos"].numpy()
    n = None if ql is None else ql.numpy()
    assert np.array_equal(_bits(dk), oracle.cache_append(_bits(kc), _bits(k_new), sp, n)), f"{what}: k cache"
    assert np.array_equal(_bits(dv), oracle.cache_append(_bits(vc), _bits(v_new), sp, n)), f"{what}: v cache"
    return out


CASES = [
    # name, B, S, Hq, Hkv, D, T_max, start_pos, q_lens
    ("gqa4_ragged", 3, 300, 8, 2, 128, 1000, [0, 517, 130], [300, 77, 1]),
    ("gqa4_llama_heads", 2, 256, 32, 8, 128, 900, [640, 37], [256, 200]),
    ("aligned_prefix", 2, 192, 8, 2, 128, 700, [128, 64], [192, 150]),
    ("mqa", 2, 200, 8, 1, 128, 700, [333, 64], [200, 150]),
    ("mha", 2, 130, 4, 4, 128, 400, [100, 270], [130, 130]),
    ("empty_chunk", 2, 100, 8, 2, 128, 300, [10, 50], [0, 100]),
    ("prefix_fills_cache", 2, 64, 8, 2, 128, 256, [256, 251], [64, 64]),
    ("negative_start_clamps", 1, 70, 8, 2, 128, 128, [-5], [70]),
    ("d64", 2, 200, 8, 2, 64, 600, [64, 399], [200, 199]),
    ("minimind768_d96", 2, 300, 8, 4, 96, 1000, [0, 517], [300, 77]),
    ("d96_mqa", 2, 150, 8, 1, 96, 500, [201, 33], [150, 90]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cached_append_prefill_matches_oracle(case):
    name, B, S, Hq, Hkv, D, T, sp, ql = case
    print(f"[case] {name}", flush=True)
    inp = synth.gqa_prefill_cached_inputs(B, S, Hq, Hkv, D, T, sp, ql, seed=61)
    _check(inp, what=name)


def test_cached_append_all_rows_fp32_scale():
    """q_lens NULL (every row new), fp32 output and an explicit scale."""
    inp = synth.gqa_prefill_cached_inputs(2, 190, 8, 2, 128, 800, [450, 3], None, seed=63)
    out = _check(inp, q_lens=False, out_dtype=torch.float32, softmax_scale=0.06, what="q_lens NULL, fp32, scale")
    assert out.dtype == torch.float32


def test_cached_append_matches_append_then_cached_prefill():
    """The one launch equals attn_cache_append then attn_prefill_gqa_cached, up to fp32 rounding."""
    import mha_mla_kv_amd as attn
    inp = synth.gqa_prefill_cached_inputs(2, 256, 32, 8, 128, 2000, [1000, 1531], [256, 201], seed=65)
    k_new, v_new, kc, vc = _split(inp)
    q, sp, ql = inp["q"].cuda(), inp["start_pos"].cuda(), inp["q_lens"].cuda()
    k1, v1 = kc.cuda(), vc.cuda()
    fused = attn.attn_prefill_gqa_cached_append(q, k_new.cuda(), v_new.cuda(), k1, v1, sp, ql,
                                                out_dtype=torch.float32)
    k2, v2 = kc.cuda(), vc.cuda()
    attn.attn_cache_append(k_new.cuda(), k2, v_new.cuda(), v2, sp, ql)
    two = attn.attn_prefill_gqa_cached(q, k2, v2, sp, ql, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    assert_close_rows(fused, two, 1e-2, "fused vs append + cached prefill")


def test_cached_append_moving_max():
    """Scores that climb tile after tile over the cached prefix (cut at P - 1) and the chunk's
    own tiles: the reference max moves on every tile after the first."""
    inp = synth.gqa_prefill_cached_inputs(2, 200, 8, 2, 128, 400, [200, 97], [200, 141], seed=67)
    inp["q"], inp["k"] = stepped_scores(inp["q"], inp["k"], 4)
    _check(inp, what="cached append, moving max")
