"""GQA decode over paged FP8 caches (attn_decode_gqa_paged_fp8kv) on the GPU, through the C ABI.

The pools hold OCP FP8 E4M3 codes of N(0,1) data divided by the scale (pages no sequence uses and
rows past each length are NaN codes).  The expected output is the fp64 oracle's decode over the
codes gathered out of the pool (oracle.gather_pages on the bytes), decoded from the format's
definition (oracle.e4m3_to_float) and scaled.  Against attn_decode_gqa_fp8kv on the gathered
codes the result must be bit for bit the same: the paging only changes where each 32-position
tile is read from."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL_BF16, assert_close_rows, row_rel_err
from tests.test_gpu_decode_paged import _paged_case

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 4.5 / 448.0, 3.0 / 448.0


def _fp8(pages_bf16, scale):
    return (pages_bf16.float() / scale).clamp(-448, 448).to(torch.float8_e4m3fn)  # NaN stays NaN


def _case(B, Hq, Hkv, ps, mp, lens, seed, spare_pages=3):
    q, kp, vp, table, L = _paged_case(B, Hq, Hkv, 128, ps, mp, lens, spare_pages=spare_pages, seed=seed)
    return q, _fp8(kp, K_SCALE), _fp8(vp, V_SCALE), table, L


def _run(q, kp, vp, table, lens, **kw):
    import mha_mla_kv_amd as attn
    out = attn.attn_decode_gqa_paged_fp8kv(q.cuda(), kp.cuda(), vp.cuda(), K_SCALE, V_SCALE, table.cuda(),
                                           lens.cuda(), **kw)
    torch.cuda.synchronize()
    return out


def _gathered_codes(pool, table, lens):
    """[B, T, Hkv, 128] codes (uint8) of the caches the block table describes."""
    return oracle.gather_pages(pool.view(torch.uint8).numpy(), table.numpy(), lens.numpy())


def _ref(q, kp, vp, table, lens, rows=None):
    kc, vc = _gathered_codes(kp, table, lens), _gathered_codes(vp, table, lens)
    sl = slice(None) if rows is None else rows
    k = oracle.e4m3_to_float(kc[sl], K_SCALE).astype(np.float32)
    v = oracle.e4m3_to_float(vc[sl], V_SCALE).astype(np.float32)
    return oracle.gqa_decode(q[sl], k, v, lens[sl])


CASES = [
    # name, B, Hq, Hkv, page_size, max_pages, lens, split
    ("gqa4_ps64_ragged", 4, 32, 8, 64, 20, [1280, 0, 77, 1000], 0),
    ("gqa4_ps32_chunks", 3, 32, 8, 32, 40, [1280, 640, 33], 128),
    ("ps256_big_units", 2, 32, 8, 256, 16, [4096, 2500], 0),
    ("mqa_ps128", 2, 32, 1, 128, 16, [2048, 1111], 0),
    ("mha", 3, 8, 8, 64, 8, [512, 1, 300], 64),
    ("one_chunk_fixed_schedule", 5, 16, 4, 32, 2, [64, 10, 0, 33, 64], 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_fp8_decode_matches_oracle(case):
    name, B, Hq, Hkv, ps, mp, lens, split = case
    print(f"[case] {name}", flush=True)
    q, kp, vp, table, L = _case(B, Hq, Hkv, ps, mp, lens, seed=len(name) + 100)
    out = _run(q, kp, vp, table, L, split_tokens=split)
    assert_close_rows(out, _ref(q, kp, vp, table, L), TOL_BF16, name)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_fp8_equals_contiguous_fp8_bitwise(case):
    import mha_mla_kv_amd as attn
    name, B, Hq, Hkv, ps, mp, lens, split = case
    q, kp, vp, table, L = _case(B, Hq, Hkv, ps, mp, lens, seed=len(name) + 100)
    kc = torch.from_numpy(_gathered_codes(kp, table, L)).view(torch.float8_e4m3fn).cuda()
    vc = torch.from_numpy(_gathered_codes(vp, table, L)).view(torch.float8_e4m3fn).cuda()
    paged = _run(q, kp, vp, table, L, split_tokens=split)
    contig = attn.attn_decode_gqa_fp8kv(q.cuda(), kc, vc, K_SCALE, V_SCALE, L.cuda(), split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(paged, contig)


def test_paged_fp8_llama3_heads_sampled_rows():
    """Llama-3-8B heads (Hq 32, Hkv 8) in 64-position pages of a shuffled pool, 8 sequences of
    up to 8192 positions: bit for bit the contiguous FP8 decode, sampled sequences against the
    oracle, and a table entry past the pool reads the pool's last page (the stated clamp)."""
    import mha_mla_kv_amd as attn
    g = torch.Generator().manual_seed(93)
    B, Hq, Hkv, ps, mp = 8, 32, 8, 64, 128
    lens = torch.randint(1024, 8193, (B,), generator=g, dtype=torch.int32)
    q, kp, vp, table, L = _case(B, Hq, Hkv, ps, mp, lens.tolist(), seed=94, spare_pages=1)
    table[3, 0] = kp.shape[0] + 40
    last = kp.shape[0] - 1
    kp[last] = _fp8(torch.randn(ps, Hkv, 128, generator=g), K_SCALE)
    vp[last] = _fp8(torch.randn(ps, Hkv, 128, generator=g), V_SCALE)
    paged = _run(q, kp, vp, table, L)
    kc = torch.from_numpy(_gathered_codes(kp, table, L)).view(torch.float8_e4m3fn).cuda()
    vc = torch.from_numpy(_gathered_codes(vp, table, L)).view(torch.float8_e4m3fn).cuda()
    contig = attn.attn_decode_gqa_fp8kv(q.cuda(), kc, vc, K_SCALE, V_SCALE, L.cuda())
    torch.cuda.synchronize()
    assert torch.equal(paged, contig)
    rows = [0, 3, 7]
    assert row_rel_err(paged[rows], _ref(q, kp, vp, table, L, rows=rows)) <= TOL_BF16
