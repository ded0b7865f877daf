"""MLA decode step with the new token (attn_decode_mla_append) on the GPU, through the C ABI: the
output against the fp64 oracle (decompressed form) over the caches with the new rows in place, and
the caches afterwards against the oracle's append, bit for bit.  Cache rows past each length are NaN
before the call, so a read of the row being written (or beyond) would show."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, assert_close_rows

pytestmark = pytest.mark.gpu

KEYS = ("q_nope", "q_rope", "w_uk", "w_uv", "c_kv", "k_rope", "cache_lens")


def _step(B, H, dn, dR, dv, r, T, lens, split=0, seed=81, out_dtype=torch.float32):
    import mha_mla_kv_amd as attn
    inp = synth.mla_decode_inputs(B, H, dn, dR, dv, r, T, lens, seed=seed)  # NaN past each length
    g = torch.Generator().manual_seed(seed)
    c_new = torch.randn(B, r, generator=g).to(torch.bfloat16)
    kr_new = torch.randn(B, dR, generator=g).to(torch.bfloat16)
    d = {k: v.cuda() for k, v in inp.items()}
    out = attn.attn_decode_mla_append(d["q_nope"], d["q_rope"], c_new.cuda(), kr_new.cuda(), d["w_uk"], d["w_uv"],
                                      d["c_kv"], d["k_rope"], d["cache_lens"], split_tokens=split, out_dtype=out_dtype)
    torch.cuda.synchronize()
    L = np.clip(inp["cache_lens"].numpy(), 0, T)
    f = lambda t: t.float().numpy()
    ext_c = np.concatenate([f(inp["c_kv"]), np.zeros((B, 1, r), np.float32)], axis=1)
    ext_r = np.concatenate([f(inp["k_rope"]), np.zeros((B, 1, dR), np.float32)], axis=1)
    for b in range(B):
        ext_c[b, L[b]] = f(c_new[b])
        ext_r[b, L[b]] = f(kr_new[b])
    ref = oracle.mla_decode_decompressed(inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["w_uv"], ext_c, ext_r,
                                         (L + 1).astype(np.int32))
    bits = lambda t: t.cpu().view(torch.int16).numpy()
    cb = oracle.cache_append(bits(inp["c_kv"]), bits(c_new)[:, None], L, np.ones(B, np.int32))
    rb = oracle.cache_append(bits(inp["k_rope"]), bits(kr_new)[:, None], L, np.ones(B, np.int32))
    assert np.array_equal(bits(d["c_kv"]), cb) and np.array_equal(bits(d["k_rope"]), rb), "caches after the step"
    return out, ref, inp, c_new, kr_new


CASES = [
    # name, B, H, dn, dR, dv, r, T, lens, split
    ("minimind_ragged", 4, 8, 96, 48, 96, 128, 300, [299, 0, 77, 300], 0),   # empty and full caches
    ("minimind_chunks", 3, 8, 96, 48, 96, 128, 900, [899, 64, 455], 64),     # several chunks: last-arriver merge
    ("h16_r256_dr64", 2, 16, 128, 64, 128, 256, 260, [200, 129], 128),
    ("h1_r64_dr16", 2, 1, 32, 16, 48, 64, 200, [0, 33], 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mla_decode_step(case):
    name, B, H, dn, dR, dv, r, T, lens, split = case
    print(f"[case] {name}", flush=True)
    out, ref, *_ = _step(B, H, dn, dR, dv, r, T, lens, split)
    assert_close_rows(out, ref, TOL_BF16, name)


def test_mla_decode_step_matches_append_then_decode():
    """The fused step equals attn_cache_append of the two rows then attn_decode_mla_absorbed over
    cache_lens + 1 rows (up to fp32 rounding: the new token is merged as one more partial)."""
    import mha_mla_kv_amd as attn
    B, H, dn, dR, dv, r, T = 3, 8, 96, 48, 96, 128, 600
    out, ref, inp, c_new, kr_new = _step(B, H, dn, dR, dv, r, T, [599, 130, 1], split=0, seed=83,
                                         out_dtype=torch.bfloat16)
    d = {k: v.cuda() for k, v in inp.items()}
    attn.attn_cache_append(c_new.cuda()[:, None], d["c_kv"], kr_new.cuda()[:, None], d["k_rope"], d["cache_lens"])
    lens1 = (d["cache_lens"] + 1).to(torch.int32)
    two = attn.attn_decode_mla_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], d["c_kv"], d["k_rope"], lens1,
                                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_close_rows(out, two, 1e-2, "fused step vs append + decode")
    assert_close_rows(out, ref, TOL_BF16, "fused step vs oracle")
