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


def _paged_case(B, Hq, Hkv, D, page_size, max_pages, lens, spare_pages=3, seed=0, extra=0):
    """A pool with every sequence's pages in a shuffled order, plus spare NaN pages.  extra = 1
    also hands out the page of position L (a decode step's new row), its rows left NaN."""
    g = torch.Generator().manual_seed(seed)
    T = page_size * max_pages
    lens = torch.tensor(lens, dtype=torch.int32)
    used = [int((min(max(int(L), 0) + extra, T) + page_size - 1) // page_size) for L in lens]
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
            rows = max(0, min(page_size, int(lens[b]) - p * page_size))
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


# ---- decode step with the new token over paged caches (attn_decode_gqa_paged_append)

def _paged_step(B, Hq, Hkv, D, ps, mp, lens, split=0, seed=0, seqs=None):
    """Runs attn_decode_gqa_paged_append; checks the pools afterwards bit for bit against the
    oracle's paged append and returns (out, oracle reference for the sequences seqs (default
    all), inputs)."""
    import mha_mla_kv_amd as attn
    q, kp, vp, table, L = _paged_case(B, Hq, Hkv, D, ps, mp, lens, seed=seed, extra=1)
    g = torch.Generator().manual_seed(seed + 1)
    k_new = torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16)
    v_new = torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16)
    kpd, vpd = kp.cuda(), vp.cuda()
    out = attn.attn_decode_gqa_paged_append(q.cuda(), k_new.cuda(), v_new.cuda(), kpd, vpd, table.cuda(), L.cuda(),
                                            split_tokens=split)
    torch.cuda.synchronize()
    T = ps * mp
    Lc = np.clip(L.numpy(), 0, T)
    bits = lambda t: t.cpu().view(torch.int16).numpy()
    assert np.array_equal(bits(kpd), oracle.append_pages(bits(kp), table.numpy(), bits(k_new)[:, None], Lc)), "k pool"
    assert np.array_equal(bits(vpd), oracle.append_pages(bits(vp), table.numpy(), bits(v_new)[:, None], Lc)), "v pool"
    # reference: the gathered caches extended by one row, the new token at row L_b
    sq = list(range(B)) if seqs is None else list(seqs)
    k, v = _gathered(kp, vp, table[sq], L[sq])
    ext_k = np.concatenate([k, np.zeros((len(sq), 1, Hkv, D), np.float32)], axis=1)
    ext_v = np.concatenate([v, np.zeros((len(sq), 1, Hkv, D), np.float32)], axis=1)
    for i, b in enumerate(sq):
        ext_k[i, Lc[b]] = k_new[b].float().numpy()
        ext_v[i, Lc[b]] = v_new[b].float().numpy()
    ref = oracle.gqa_decode(q[sq], ext_k, ext_v, (Lc[sq] + 1).astype(np.int32))
    return out, ref, (q, k_new, v_new, kp, vp, table, L)


APPEND_CASES = [
    # name, B, Hq, Hkv, D, page_size, max_pages, lens, split
    ("gqa4_ps64_ragged", 4, 32, 8, 128, 64, 20, [1279, 0, 77, 1000], 0),     # last row, row 0, mid-page
    ("gqa4_ps32_page_starts", 3, 32, 8, 128, 32, 40, [640, 32, 31], 128),   # new rows opening / ending pages
    ("full_cache_not_stored", 2, 16, 4, 128, 64, 4, [256, 255], 0),         # L = T: attended, not stored
    ("mqa_ps128", 2, 32, 1, 128, 128, 16, [2047, 1111], 256),
    ("mha_d64", 3, 8, 8, 64, 64, 8, [511, 1, 300], 0),
    ("d96_minimind_heads", 2, 8, 4, 96, 32, 16, [511, 200], 64),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_paged_decode_step_matches_oracle(case):
    name, B, Hq, Hkv, D, ps, mp, lens, split = case
    print(f"[case] paged step {name}", flush=True)
    out, ref, _ = _paged_step(B, Hq, Hkv, D, ps, mp, lens, split, seed=len(name) + 100)
    assert_close_rows(out, ref, TOL_BF16, name)


@pytest.mark.parametrize("case", APPEND_CASES[:4], ids=[c[0] for c in APPEND_CASES[:4]])
def test_paged_decode_step_equals_contiguous_bitwise(case):
    """Against attn_decode_gqa_append over the gathered caches: the same output bits, and the
    contiguous cache gets the same new rows."""
    import mha_mla_kv_amd as attn
    name, B, Hq, Hkv, D, ps, mp, lens, split = case
    print(f"[case] paged step bitwise {name}", flush=True)
    out, _, (q, k_new, v_new, kp, vp, table, L) = _paged_step(B, Hq, Hkv, D, ps, mp, lens, split,
                                                               seed=len(name) + 200)
    k, v = _gathered(kp, vp, table, L)
    kc = torch.from_numpy(k).to(torch.bfloat16).cuda()
    vc = torch.from_numpy(v).to(torch.bfloat16).cuda()
    contig = attn.attn_decode_gqa_append(q.cuda(), k_new.cuda(), v_new.cuda(), kc, vc, L.cuda(), split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(out, contig)


def test_paged_decode_step_llama3_shape_sampled():
    """The Llama-3-8B decode shape in 64-position pages: the pools bit for bit against the
    oracle's paged append, the output bit for bit against the contiguous decode step and on
    sampled sequences against the oracle."""
    import mha_mla_kv_amd as attn
    g = torch.Generator().manual_seed(92)
    B, Hq, Hkv, D, ps, mp = 32, 32, 8, 128, 64, 128
    lens = torch.randint(1024, 8192, (B,), generator=g, dtype=torch.int32).tolist()
    seqs = [0, 9, B - 1]
    print("[case] paged step llama3", flush=True)
    out, ref, (q, k_new, v_new, kp, vp, table, L) = _paged_step(B, Hq, Hkv, D, ps, mp, lens, seed=93, seqs=seqs)
    k, v = _gathered(kp, vp, table, L)
    kc = torch.from_numpy(k).to(torch.bfloat16).cuda()
    vc = torch.from_numpy(v).to(torch.bfloat16).cuda()
    contig = attn.attn_decode_gqa_append(q.cuda(), k_new.cuda(), v_new.cuda(), kc, vc, L.cuda())
    torch.cuda.synchronize()
    assert torch.equal(out, contig)
    assert_close_rows(out[seqs], ref, TOL_BF16, "llama3 paged step sampled sequences")
