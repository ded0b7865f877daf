"""MLA absorbed decode on the GPU (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows, to_np

pytestmark = pytest.mark.gpu


def _run(inp, **kw):
    import mha_mla_kv_amd as attn
    d = {k: v.to("cuda") for k, v in inp.items()}
    out = attn.attn_decode_mla_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["c_kv"], d["k_rope"],
                                        d["cache_lens"], **kw)
    torch.cuda.synchronize()
    return out


def _oracle(inp, bh=None, decompressed=False):
    fn = oracle.mla_decode_decompressed if decompressed else oracle.mla_decode_absorbed
    return fn(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["w_uv"], inp["c_kv"], inp["k_rope"],
              inp["cache_lens"], bh=bh)


CASES = [
    # name, B, H, dn, dR, dv, r, T, lens, split
    ("minimind_small", 3, 8, 96, 48, 96, 128, 300, [300, 1, 77], 64),
    ("minimind_auto", 2, 8, 96, 48, 96, 128, 700, [700, 333], 0),
    ("h1_r64_dr16", 2, 1, 32, 16, 48, 64, 200, [200, 33], 64),
    ("h16_r256_dr64", 2, 16, 128, 64, 128, 256, 260, [260, 129], 128),
    ("h5_r128_dr32", 2, 5, 64, 32, 80, 128, 150, [150, 64], 64),
    ("many_chunks", 2, 2, 32, 16, 48, 64, 5000, [5000, 4097], 64),  # more than 64 chunks to merge
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mla_matches_decompressed_oracle(case):
    name, B, H, dn, dR, dv, r, T, lens, split = case
    inp = synth.mla_decode_inputs(B, H, dn, dR, dv, r, T, lens, seed=21)
    print(f"[case] {name}", flush=True)
    out = _run(inp, split_tokens=split)
    assert_close_rows(out, _oracle(inp, decompressed=True), TOL_BF16, name)


def test_mla_empty_sequences_and_bf16_out():
    inp = synth.mla_decode_inputs(3, 8, 96, 48, 96, 128, 100, [0, 100, 0], seed=2)
    out = _run(inp, split_tokens=64, out_dtype=torch.bfloat16)
    o = to_np(out)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert_close_rows(out, _oracle(inp), TOL_BF16, "mla empty")


def test_mla_split_invariance_nan_poison_determinism():
    args = (2, 8, 96, 48, 96, 128, 900, [900, 455])
    poisoned = synth.mla_decode_inputs(*args, seed=8, poison=True)
    clean = synth.mla_decode_inputs(*args, seed=8, poison=False)
    outs = [to_np(_run(poisoned, split_tokens=s)) for s in (64, 256, 1024, 0)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) / np.max(np.abs(outs[0])) < 2e-3
    assert np.array_equal(to_np(_run(clean, split_tokens=64)), outs[0])
    assert np.array_equal(to_np(_run(poisoned, split_tokens=64)), outs[0])


def test_mla_selection_is_bit_exact():
    """0/1 selection weights and a saturating score: the output is an exact copy of latent
    coordinates of the selected token."""
    B, H, dn, dR, dv, r, T = 2, 8, 96, 48, 96, 128, 300
    lens = torch.tensor([300, 130], dtype=torch.int32)
    w_uk = torch.zeros(H, dn, r)
    w_uv = torch.zeros(H, dv, r)
    for h in range(H):
        w_uk[h, 0, h] = 1.0
        for i in range(dv):
            w_uv[h, i, (i + 2 * h) % r] = 1.0
    g = torch.Generator().manual_seed(4)
    q_nope = torch.zeros(B, H, dn)
    q_nope[:, :, 0] = 64.0
    q_rope = torch.zeros(B, H, dR)
    k_rope = torch.randn(B, T, dR, generator=g)
    for t_star in (0, 31, 64, 129):
        c = torch.randn(B, T, r, generator=g)
        c[:, :, :H] = 0.0
        c[:, t_star, :H] = 64.0
        inp = {"q_nope": q_nope, "q_rope": q_rope, "w_uk": w_uk, "w_uv": w_uv, "c_kv": c, "k_rope": k_rope,
               "cache_lens": lens}
        inp = {k: (v.to(torch.bfloat16) if v.dtype == torch.float32 else v) for k, v in inp.items()}
        out = to_np(_run(inp, split_tokens=64))
        cb = inp["c_kv"].float().numpy()
        for b in range(B):
            for h in range(H):
                want = np.array([cb[b, t_star, (i + 2 * h) % r] for i in range(dv)])
                assert np.array_equal(out[b, h], want), (t_star, b, h)


def test_full_size_minimind_mla():
    """MiniMind-768 MLA shape (B 64, H 8, cache 4096) in the benchmark's launch configuration:
    every row against the absorbed oracle, sampled rows against the decompressed oracle."""
    inp = synth.make("minimind768_mla_decode")
    out = _run(inp)
    assert_close_rows(out, _oracle(inp), TOL_BF16, "mla full vs absorbed oracle")
    bh = [0, 7, 8 * 31 + 3, 8 * 63 + 7]
    ref = _oracle(inp, bh=bh, decompressed=True).reshape(-1, 96)[bh]
    assert_close_rows(to_np(out).reshape(-1, 96)[bh], ref, TOL_BF16, "mla full vs decompressed oracle")


def test_mla_moving_max_matches_oracle():
    """Scores that climb along the cache through the shared rotated key: q_rope along one
    direction per sequence, k_rope along it times 1 + 0.4 * (position // 16), plus noise, the
    latent part scaled down to a small perturbation.  Each streaming wave's next 16-row slice
    (four slices on) beats its running max by about 9 (log2 units), more than the 2^8 slack, so
    the reference moves slice after slice and the chunks merge across very different maxima."""
    B, H, dn, dR, dv, r, T = 2, 8, 96, 48, 96, 128, 300
    inp = synth.mla_decode_inputs(B, H, dn, dR, dv, r, T, [300, 217], seed=23)
    g = torch.Generator().manual_seed(7)
    u = torch.randn(B, 1, dR, generator=g)
    qr = u + 0.1 * torch.randn(B, H, dR, generator=g)
    mag = 1.0 + 0.4 * (torch.arange(T) // 16).float()
    kr = mag[None, :, None] * (u + 0.1 * torch.randn(B, T, dR, generator=g))
    inp["q_rope"] = qr.to(torch.bfloat16)
    inp["k_rope"] = (inp["k_rope"].float() * 0 + kr).to(torch.bfloat16)
    inp["q_nope"] = (inp["q_nope"].float() * 0.3).to(torch.bfloat16)
    inp["c_kv"] = (inp["c_kv"].float() * 0.3).to(torch.bfloat16)
    ref = _oracle(inp, decompressed=True)
    for split in (64, 0):
        assert_close_rows(_run(inp, split_tokens=split), ref, TOL_BF16, f"mla moving max split {split}")
