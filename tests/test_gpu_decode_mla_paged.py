"""MLA decode over paged latent caches (attn_decode_mla_paged) on the GPU, through the C ABI.

Each case draws contiguous caches (rows past each length NaN), scatters their pages over a pool in
a seeded order with spare NaN pages, and checks the paged decode against the fp64 oracle's
absorbed decode over the contiguous caches, and bit for bit against attn_decode_mla_absorbed over
them (T_max = page_size * max_pages_per_seq, so both plan the same chunks: the paging only
changes where each 16-row slice is read from).  The oracle's gather_pages is pinned to the same
block-table reading on the CPU."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows, to_np

pytestmark = pytest.mark.gpu


def _scatter(cache, lens, page_size, spare=3, seed=0):
    """cache [B, T, w] -> (pages [n_pages, page_size, w], block_table [B, T / page_size])."""
    B, T, w = cache.shape
    mp = T // page_size
    used = [(min(max(int(L), 0), T) + page_size - 1) // page_size for L in lens]
    n_pages = sum(used) + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)
    pages = torch.full((n_pages, page_size, w), float("nan"), dtype=cache.dtype)
    table = torch.full((B, mp), -7, dtype=torch.int32)  # unused entries: anything
    nxt = 0
    for b in range(B):
        for p in range(used[b]):
            page = int(perm[nxt])
            nxt += 1
            table[b, p] = page
            pages[page] = cache[b, p * page_size:(p + 1) * page_size]
    return pages, table


def _paged(inp, page_size, seed=0):
    L = inp["cache_lens"].numpy()
    cp, table = _scatter(inp["c_kv"], L, page_size, seed=seed)
    kp, table2 = _scatter(inp["k_rope"], L, page_size, seed=seed)
    assert torch.equal(table, table2)
    return cp, kp, table


def _run_paged(inp, cp, kp, table, **kw):
    import mha_mla_kv_amd as attn
    d = {k: v.cuda() for k, v in inp.items()}
    out = attn.attn_decode_mla_paged(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], cp.cuda(), kp.cuda(),
                                     table.cuda(), d["cache_lens"], **kw)
    torch.cuda.synchronize()
    return out


def _run_contiguous(inp, **kw):
    import mha_mla_kv_amd as attn
    d = {k: v.cuda() for k, v in inp.items()}
    out = attn.attn_decode_mla_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["c_kv"], d["k_rope"],
                                        d["cache_lens"], **kw)
    torch.cuda.synchronize()
    return out


def _oracle(inp, bh=None):
    return oracle.mla_decode_absorbed(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["w_uv"], inp["c_kv"],
                                      inp["k_rope"], inp["cache_lens"], bh=bh)


CASES = [
    # name, B, H, dn, dR, dv, r, page_size, max_pages, lens, split
    ("minimind_ps16", 3, 8, 96, 48, 96, 128, 16, 40, [640, 1, 77], 64),
    ("minimind_ps48_auto_split", 2, 8, 96, 48, 96, 128, 48, 15, [700, 333], 0),  # 256-position chunks start mid-page
    ("h16_r256_dr64_ps64", 2, 16, 128, 64, 128, 256, 64, 5, [260, 129], 128),
    ("h1_r64_dr16_ps32", 2, 1, 32, 16, 48, 64, 32, 7, [200, 33], 64),
    ("h5_r128_dr32_ps16_split192", 2, 5, 64, 32, 80, 128, 16, 24, [384, 250], 192),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_mla_matches_oracle_and_contiguous(case):
    name, B, H, dn, dR, dv, r, ps, mp, lens, split = case
    print(f"[case] {name}", flush=True)
    inp = synth.mla_decode_inputs(B, H, dn, dR, dv, r, ps * mp, lens, seed=31)
    cp, kp, table = _paged(inp, ps, seed=len(name))
    out = _run_paged(inp, cp, kp, table, split_tokens=split)
    assert_close_rows(out, _oracle(inp), TOL_BF16, name)
    ref = _run_contiguous(inp, split_tokens=split)
    assert torch.equal(out, ref), f"{name}: paged and contiguous decodes differ"


def test_paged_mla_empty_sequences_bf16_out():
    inp = synth.mla_decode_inputs(3, 8, 96, 48, 96, 128, 160, [0, 100, 0], seed=32)
    cp, kp, table = _paged(inp, 16, seed=5)
    out = _run_paged(inp, cp, kp, table, split_tokens=64, out_dtype=torch.bfloat16)
    o = to_np(out)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert_close_rows(out, _oracle(inp), TOL_BF16, "paged mla empty")


def test_paged_mla_full_size_minimind():
    """The MiniMind-768 MLA decode shape (B 64, H 8, cache 4096, lengths U[1024, 4096]) over
    16-position pages in the default launch configuration; every head of sampled sequences
    against the oracle, and the whole output bit for bit against the contiguous decode."""
    inp = synth.mla_decode_inputs(64, 8, 96, 48, 96, 128, 4096, (1024, 4096), seed=5)
    cp, kp, table = _paged(inp, 16, seed=9)
    out = _run_paged(inp, cp, kp, table)
    ref = _run_contiguous(inp)
    assert torch.equal(out, ref), "paged and contiguous MiniMind decodes differ"
    o = to_np(out)
    for b in (0, 31, 63):
        sl = {k: (v[b:b + 1] if k not in ("w_uk", "w_uv") else v) for k, v in inp.items()}
        assert_close_rows(o[b:b + 1], _oracle(sl), TOL_BF16, f"paged mla full size b={b}")
