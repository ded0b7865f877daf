"""MLA decode over a paged FP8 latent cache (attn_decode_mla_paged_fp8kv) on the GPU, through the
C ABI.

Each case encodes a latent cache as E4M3 codes (rows past each length NaN codes), scatters the
code pages and the bf16 k_rope pages over pools in one seeded order with spare NaN pages, and
checks the paged decode against the fp64 oracle's absorbed decode over the codes' values, and bit
for bit against attn_decode_mla_fp8kv over the contiguous codes (T_max = page_size *
max_pages_per_seq, so both plan the same chunks: the paging only changes where each 16-row
slice is read from)."""
import pytest
import torch

from tests.parity import TOL_BF16, assert_close_rows
from tests.test_gpu_decode_mla_fp8 import _fp8_case, _ref

pytestmark = pytest.mark.gpu

NAN_CODE = 0x7F  # E4M3 NaN


def _scatter(cache, lens, page_size, fill, seed):
    """cache [B, T, w] -> (pages [n_pages, page_size, w] holding each sequence's pages in a seeded
    order plus three spare pages of `fill`, block_table [B, T / page_size])."""
    B, T, w = cache.shape
    mp = T // page_size
    used = [(min(max(int(L), 0), T) + page_size - 1) // page_size for L in lens]
    n_pages = sum(used) + 3
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(seed))
    pages = torch.full((n_pages, page_size, w), fill, dtype=cache.dtype)
    table = torch.full((B, mp), -7, dtype=torch.int32)  # unused entries: anything
    nxt = 0
    for b in range(B):
        for p in range(used[b]):
            page = int(perm[nxt])
            nxt += 1
            table[b, p] = page
            pages[page] = cache[b, p * page_size:(p + 1) * page_size]
    return pages, table


def _run_paged(inp, ps, seed, **kw):
    import mha_mla_kv_amd as attn
    L = inp["cache_lens"].numpy()
    cp, table = _scatter(inp["c_codes"].view(torch.uint8), L, ps, NAN_CODE, seed)
    kp, table2 = _scatter(inp["k_rope"], L, ps, float("nan"), seed)
    assert torch.equal(table, table2)
    d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    out = attn.attn_decode_mla_paged_fp8kv(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                           cp.view(torch.float8_e4m3fn).cuda(), inp["c_scale"], kp.cuda(),
                                           table.cuda(), d["cache_lens"], **kw)
    torch.cuda.synchronize()
    return out


CASES = [
    # name, B, H, dn, dR, dv, r, T, lens, page_size, split
    ("minimind_ps16", 3, 8, 96, 48, 96, 128, 320, [300, 1, 77], 16, 64),
    ("minimind_ps64_auto", 2, 8, 96, 48, 96, 128, 704, [700, 333], 64, 0),
    ("h1_r64_dr16_ps32", 2, 1, 32, 16, 48, 64, 224, [200, 33], 32, 64),
    ("h5_r128_dr32_ps16", 2, 5, 64, 32, 80, 128, 160, [150, 64], 16, 64),
    ("h16_r256_dr64_ps32", 2, 16, 128, 64, 128, 256, 288, [260, 129], 32, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_fp8_latent_mla_matches_oracle(case):
    name, B, H, dn, dR, dv, r, T, lens, ps, split = case
    print(f"[case] {name}", flush=True)
    inp = _fp8_case(B, H, dn, dR, dv, r, T, lens, seed=71)
    assert_close_rows(_run_paged(inp, ps, seed=len(name), split_tokens=split), _ref(inp), TOL_BF16, name)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_fp8_latent_equals_contiguous_bitwise(case):
    import mha_mla_kv_amd as attn
    name, B, H, dn, dR, dv, r, T, lens, ps, split = case
    inp = _fp8_case(B, H, dn, dR, dv, r, T, lens, seed=71)
    paged = _run_paged(inp, ps, seed=len(name), split_tokens=split)
    d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    contig = attn.attn_decode_mla_fp8kv(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["c_codes"], inp["c_scale"],
                                        d["k_rope"], d["cache_lens"], split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(paged, contig)


def test_minimind_shape_paged_fp8_latent():
    """MiniMind-768 MLA decode shape (B 64, cache 4096) in 16-position pages: bit for bit the
    contiguous FP8-latent decode, sampled sequences against the oracle."""
    import mha_mla_kv_amd as attn
    inp = _fp8_case(64, 8, 96, 48, 96, 128, 4096, [4096] * 60 + [1, 17, 4000, 2049], seed=73)
    paged = _run_paged(inp, 16, seed=5)
    d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}
    contig = attn.attn_decode_mla_fp8kv(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["c_codes"], inp["c_scale"],
                                        d["k_rope"], d["cache_lens"])
    torch.cuda.synchronize()
    assert torch.equal(paged, contig)
    rows = [0, 60, 61, 63]
    assert_close_rows(paged[rows], _ref(inp, sl=rows), TOL_BF16, "minimind paged fp8 latent, sampled rows")
