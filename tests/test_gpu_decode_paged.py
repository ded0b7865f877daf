"""GQA decode over paged caches (attn_decode_gqa_paged) on the GPU, through the C ABI.

The expected output is the fp64 oracle's decode over the caches gathered out of the page pool
(oracle.gather_pages, the block-table layout written out).  Pages that no sequence uses and rows
past each length are NaN, so reading them shows.  Against attn_decode_gqa on the gathered caches
the result must be bit for bit the same: the paging only changes where each 32-position tile is
read from."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL_BF16, assert_close_rows

pytestmark = pytest.mark.gpu


def _paged_case(B, Hq, Hkv, D, page_size, max_pages, lens, spare_pages=3, seed=0):
    """A pool with every sequence's pages in a shuffled order, plus spare NaN pages."""
    g = torch.Generator().manual_seed(seed)
    T = page_size * max_pages
    lens = torch.tensor(lens, dtype=torch.int32)
    used = [int((min(max(int(L), 0), T) + page_size - 1) // page_size) for L in lens]
    n_pages = sum(used) + spare_pages
    perm = torch.randperm(n_pages, generator=g)
    table = torch.full((B, max_pages), -7, dtype=torch.int32)  # unused entries: anything
    k_pages = torch.full((n_pages, page_size, Hkv, D), float("nan"), dtype=torch.bfloat16)
    v_pages = k_pages.clone()
    nxt = 0
    for b in range(B):
        for p in range(used[b]):
            page = int(perm[nxt])
            nxt += 1
            table[b, p] = page
            rows = min(page_size, int(lens[b]) - p * page_size)
            k_pages[page, :rows] = torch.randn(rows, Hkv, D, generator=g).to(torch.bfloat16)
            v_pages[page, :rows] = torch.randn(rows, Hkv, D, generator=g).to(torch.bfloat16)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    return q, k_pages, v_pages, table, lens


def _run(q, kp, vp, table, lens, **kw):
    import mha_mla_kv_amd as attn
    out = attn.attn_decode_gqa_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(), lens.cuda(), **kw)
    torch.cuda.synchronize()
    return out


def _gathered(kp, vp, table, lens):
    f = lambda t: t.float().numpy()
    return oracle.gather_pages(f(kp), table.numpy(), lens.numpy()), oracle.gather_pages(f(vp), table.numpy(),
                                                                                        lens.numpy())


CASES = [
    # name, B, Hq, Hkv, D, page_size, max_pages, lens, split
    ("gqa4_ps64_ragged", 4, 32, 8, 128, 64, 20, [1280, 0, 77, 1000], 0),
    ("gqa4_ps32_chunks", 3, 32, 8, 128, 32, 40, [1280, 640, 33], 128),
    ("ps256_big_units", 2, 32, 8, 128, 256, 16, [4096, 2500], 0),
    ("mqa_ps128", 2, 32, 1, 128, 128, 16, [2048, 1111], 256),
    ("mha_d64", 3, 8, 8, 64, 64, 8, [512, 1, 300], 0),
    ("d96_minimind_heads", 2, 8, 4, 96, 32, 16, [512, 200], 64),
    ("one_chunk_fixed_schedule", 5, 16, 4, 128, 32, 2, [64, 10, 0, 33, 64], 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_decode_matches_oracle(case):
    name, B, Hq, Hkv, D, ps, mp, lens, split = case
    print(f"[case] {name}", flush=True)
    q, kp, vp, table, L = _paged_case(B, Hq, Hkv, D, ps, mp, lens, seed=len(name))
    out = _run(q, kp, vp, table, L, split_tokens=split)
    k, v = _gathered(kp, vp, table, L)
    ref = oracle.gqa_decode(q, k.astype(np.float32), v.astype(np.float32), L)
    assert_close_rows(out, ref, TOL_BF16, name)


@pytest.mark.parametrize("case", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_paged_equals_contiguous_bitwise(case):
    import mha_mla_kv_amd as attn
    name, B, Hq, Hkv, D, ps, mp, lens, split = case
    q, kp, vp, table, L = _paged_case(B, Hq, Hkv, D, ps, mp, lens, seed=len(name))
    k, v = _gathered(kp, vp, table, L)
    kc = torch.from_numpy(k).to(torch.bfloat16).cuda()
    vc = torch.from_numpy(v).to(torch.bfloat16).cuda()
    paged = _run(q, kp, vp, table, L, split_tokens=split)
    contig = attn.attn_decode_gqa(q.cuda(), kc, vc, L.cuda(), split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(paged, contig)


def test_paged_llama3_shape_sampled_and_clamped_entries():
    """Llama-3-8B decode shape (B 32, Hq 32, Hkv 8, cache up to 8192) in 64-position pages in a
    shuffled pool, checked bit for bit against the contiguous decode and on sampled rows against
    the oracle; one sequence's table holds a page number past the pool, which reads the last page
    (the stated clamp), as the oracle's gather does."""
    import mha_mla_kv_amd as attn
    g = torch.Generator().manual_seed(90)
    B, Hq, Hkv, D, ps, mp = 32, 32, 8, 128, 64, 128
    lens = torch.randint(1024, 8193, (B,), generator=g, dtype=torch.int32)
    q, kp, vp, table, L = _paged_case(B, Hq, Hkv, D, ps, mp, lens.tolist(), spare_pages=1, seed=91)
    table[5, 0] = kp.shape[0] + 40  # clamped to the last page of the pool
    # the last page is a spare (NaN) page unless it was handed out: give it values
    last = kp.shape[0] - 1
    kp[last] = torch.randn(ps, Hkv, D, generator=g).to(torch.bfloat16)
    vp[last] = torch.randn(ps, Hkv, D, generator=g).to(torch.bfloat16)
    paged = _run(q, kp, vp, table, L)
    k, v = _gathered(kp, vp, table, L)
    kc = torch.from_numpy(k).to(torch.bfloat16).cuda()
    vc = torch.from_numpy(v).to(torch.bfloat16).cuda()
    contig = attn.attn_decode_gqa(q.cuda(), kc, vc, L.cuda())
    torch.cuda.synchronize()
    assert torch.equal(paged, contig)
    seqs = [0, 5, 17, B - 1]  # sampled sequences, every head
    ref = oracle.gqa_decode(q[seqs], k[seqs].astype(np.float32), v[seqs].astype(np.float32), L[seqs])
    assert_close_rows(paged[seqs], ref, TOL_BF16, "llama3 paged sampled sequences")
