"""Causal GQA prefill after a cached prefix over a paged cache (attn_prefill_gqa_paged) on the GPU,
through the C ABI.

Each case draws the contiguous chunked-prefill inputs (q rows past q_lens and cache rows past
start_pos + q_lens NaN), scatters the caches' pages over pools in a seeded order with spare NaN
pages, and checks the paged prefill against the fp64 oracle over the contiguous caches, and bit for
bit against attn_prefill_gqa_cached over them (the paging only changes where each 64-key tile is
read from)."""
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows

pytestmark = pytest.mark.gpu


def _scatter(cache, used, page_size, spare=2, seed=0):
    """cache [B, T, Hkv, D] -> (pages [n_pages, page_size, Hkv, D], block_table [B, T / page_size])."""
    B, T = cache.shape[:2]
    n_pages = sum(used) + spare
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(seed))
    pages = torch.full((n_pages, page_size) + tuple(cache.shape[2:]), float("nan"), dtype=cache.dtype)
    table = torch.full((B, T // page_size), -3, dtype=torch.int32)  # unused entries: anything
    nxt = 0
    for b in range(B):
        for p in range(used[b]):
            page = int(perm[nxt])
            nxt += 1
            table[b, p] = page
            pages[page] = cache[b, p * page_size:(p + 1) * page_size]
    return pages, table


def _paged(inp, page_size, seed):
    T = inp["k"].shape[1]
    sp = inp["start_pos"].clamp(0, T)
    ql = inp["q_lens"] if inp.get("q_lens") is not None else torch.full_like(sp, inp["q"].shape[1])
    ends = torch.minimum(sp + ql.clamp(min=0), torch.full_like(sp, T))
    used = [(int(e) + page_size - 1) // page_size for e in ends]
    kp, table = _scatter(inp["k"], used, page_size, seed=seed)
    vp, table2 = _scatter(inp["v"], used, page_size, seed=seed)
    assert torch.equal(table, table2)
    return kp, vp, table


def _run_paged(inp, kp, vp, table, **kw):
    import mha_mla_kv_amd as attn
    out = attn.attn_prefill_gqa_paged(inp["q"].cuda(), kp.cuda(), vp.cuda(), table.cuda(), inp["start_pos"].cuda(),
                                      inp["q_lens"].cuda(), **kw)
    torch.cuda.synchronize()
    return out


def _run_contiguous(inp, **kw):
    import mha_mla_kv_amd as attn
    out = attn.attn_prefill_gqa_cached(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["start_pos"].cuda(),
                                       inp["q_lens"].cuda(), **kw)
    torch.cuda.synchronize()
    return out


CASES = [
    # name, B, S, Hq, Hkv, D, page_size, max_pages, start_pos, q_lens
    ("gqa4_ps64_ragged", 3, 300, 8, 2, 128, 64, 16, [0, 517, 130], [300, 77, 1]),
    ("llama_heads_ps128", 2, 256, 32, 8, 128, 128, 8, [640, 37], [256, 200]),
    ("mqa_ps256", 2, 200, 8, 1, 128, 256, 3, [333, 64], [200, 150]),
    ("empty_chunk_ps64", 2, 100, 8, 2, 128, 64, 5, [10, 50], [0, 100]),
    ("prefix_fills_cache_ps64", 2, 64, 8, 2, 128, 64, 4, [256, 251], [64, 64]),
    ("d64_ps64", 2, 200, 8, 2, 64, 64, 10, [64, 399], [200, 199]),
    ("d96_ps192", 2, 300, 8, 4, 96, 192, 6, [0, 517], [300, 77]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_prefill_matches_oracle_and_contiguous(case):
    name, B, S, Hq, Hkv, D, ps, mp, sp, ql = case
    print(f"[case] {name}", flush=True)
    inp = synth.gqa_prefill_cached_inputs(B, S, Hq, Hkv, D, ps * mp, sp, ql, seed=51)
    kp, vp, table = _paged(inp, ps, seed=len(name))
    out = _run_paged(inp, kp, vp, table)
    ref = oracle.gqa_prefill_cached(inp["q"], inp["k"], inp["v"], inp["start_pos"], inp["q_lens"])
    assert_close_rows(out, ref, TOL_BF16, name)
    assert torch.equal(out, _run_contiguous(inp)), f"{name}: paged and contiguous prefills differ"


def test_paged_prefill_llama3_chunk_shape_bitwise():
    """The Llama-3-8B chunked-prefill shape (B 4, 512 new tokens after 3584 cached, Hq 32, Hkv 8,
    head_dim 128) over 64-position pages: bit for bit the contiguous cached prefill, fp32 output."""
    inp = synth.gqa_prefill_cached_inputs(4, 512, 32, 8, 128, 4096, [3584] * 4, [512] * 4, seed=6, poison=False)
    kp, vp, table = _paged(inp, 64, seed=3)
    out = _run_paged(inp, kp, vp, table, out_dtype=torch.float32)
    assert torch.equal(out, _run_contiguous(inp, out_dtype=torch.float32))
