"""Cache append on the GPU (through the C ABI) against the oracle's plain slice assignment,
bit for bit (raw 16-bit patterns)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy()


def _rand(g, *shape, dtype=torch.bfloat16):
    return torch.randn(*shape, generator=g).to(dtype)


CASES = [
    # name, B, S, T_max, start_pos, n_new, row shape a, row shape b
    ("kv_decode_step", 32, 1, 300, [0, 17, 299] + [5] * 29, None, (8, 128), (8, 128)),
    ("kv_chunk_ragged", 3, 130, 700, [0, 517, 130], [130, 77, 1], (2, 128), (2, 128)),
    ("kv_clamped", 3, 64, 256, [250, 256, -7], [64, 64, 64], (4, 64), (4, 64)),
    ("kv_empty", 2, 40, 100, [10, 20], [0, 40], (1, 128), (1, 128)),
    ("mla_latent_rope", 4, 50, 400, [0, 100, 333, 399], [50, 50, 50, 50], (128,), (48,)),
    ("single_pair", 2, 70, 300, [3, 200], [70, 33], (8, 96), None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cache_append_bit_exact(case):
    import mha_mla_kv_amd as attn
    name, B, S, T, sp, nn, ra, rb = case
    print(f"[case] {name}", flush=True)
    g = torch.Generator().manual_seed(61)
    new_a, cache_a = _rand(g, B, S, *ra), _rand(g, B, T, *ra)
    spt = torch.tensor(sp, dtype=torch.int32)
    nnt = None if nn is None else torch.tensor(nn, dtype=torch.int32)
    ca = cache_a.cuda()
    if rb is not None:
        new_b, cache_b = _rand(g, B, S, *rb), _rand(g, B, T, *rb)
        cb = cache_b.cuda()
        attn.attn_cache_append(new_a.cuda(), ca, new_b.cuda(), cb, spt.cuda(), None if nnt is None else nnt.cuda())
    else:
        attn.attn_cache_append(new_a.cuda(), ca, start_pos=spt.cuda(), n_new=None if nnt is None else nnt.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_bits(ca), oracle.cache_append(_bits(cache_a), _bits(new_a), sp, nn))
    if rb is not None:
        assert np.array_equal(_bits(cb), oracle.cache_append(_bits(cache_b), _bits(new_b), sp, nn))


def test_append_then_decode_sees_the_new_token():
    """A decode step as the page runs it: write the new token's K/V at position L, then attend to
    L + 1 positions; equals the oracle decode over the appended cache."""
    import mha_mla_kv_amd as attn
    from tests.parity import TOL_BF16, assert_close_rows
    g = torch.Generator().manual_seed(62)
    B, Hq, Hkv, D, T = 4, 32, 8, 128, 600
    lens = torch.tensor([0, 100, 377, 599], dtype=torch.int32)
    k, v = _rand(g, B, T, Hkv, D), _rand(g, B, T, Hkv, D)
    kn, vn, q = _rand(g, B, 1, Hkv, D), _rand(g, B, 1, Hkv, D), _rand(g, B, Hq, D)
    kc, vc = k.cuda(), v.cuda()
    attn.attn_cache_append(kn.cuda(), kc, vn.cuda(), vc, lens.cuda())
    out = attn.attn_decode_gqa(q.cuda(), kc, vc, (lens + 1).cuda())
    torch.cuda.synchronize()
    k2 = oracle.cache_append(k.float().numpy(), kn.float().numpy(), lens.numpy())
    v2 = oracle.cache_append(v.float().numpy(), vn.float().numpy(), lens.numpy())
    ref = oracle.gqa_decode(q.float().numpy(), k2, v2, (lens + 1).numpy())
    assert_close_rows(out, ref, TOL_BF16, "append + decode")
