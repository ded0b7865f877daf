"""Rotary position embedding fused with the cache write (attn_rope_append) on the GPU, through the
C ABI, against the fp64 oracle's rotation (oracle.rope / oracle.rope_append).

Rotated values are checked element by element: a bf16 result may differ from the exact value by
its own rounding (2^-8 relative, with margin) plus the fp32 arithmetic (1e-6 of the head vector's
largest element); an fp32 result by 1e-6 of the head vector's largest element.  Everything the call
must not touch (rows past n_new, cache rows off the written positions, which are NaN-poisoned) and
the unrotated stream x are compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import TOL_BF16, assert_close_rows

pytestmark = pytest.mark.gpu


def _bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def _check_rotated(gpu, ref, what):
    """gpu [..., d] torch, ref [..., d] float64 numpy: element bound per head vector."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if g.size == 0:
        return
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    bound = (2.0 ** -8 * np.abs(ref) + 1e-6 * scale) if gpu.dtype == torch.bfloat16 else 1e-6 * scale
    err = np.abs(g - ref)
    bad = ~(err <= bound)
    print(f"[rope] {what}: worst error / bound {np.max(err / np.maximum(bound, 1e-300)):.3f}", flush=True)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, first at {np.argwhere(bad)[0]}"


def _rand(g, shape, dtype):
    return torch.randn(*shape, generator=g).to(dtype)


def _nan_like(t):
    return torch.full_like(t, float("nan"))


def _run_case(B, S, Hq, Hk, d, T, start, n_new, dtype, base=10000.0, seed=0, x_bytes=256, three_d_k=False):
    import mha_mla_kv_amd as attn
    g = torch.Generator().manual_seed(seed)
    q = _rand(g, (B, S, Hq, d), dtype)
    kshape = (B, S, d) if three_d_k else (B, S, Hk, d)
    k = _rand(g, kshape, dtype)
    x = torch.randint(-30000, 30000, (B, S, x_bytes // 2), generator=g, dtype=torch.int16)
    kc = _nan_like(torch.zeros((B, T) + kshape[2:], dtype=dtype))
    xc = torch.randint(-30000, 30000, (B, T, x_bytes // 2), generator=g, dtype=torch.int16)
    sp = torch.tensor(start, dtype=torch.int32)
    nn = None if n_new is None else torch.tensor(n_new, dtype=torch.int32)
    dq, dk, dkc, dxc = q.cuda(), k.cuda(), kc.cuda(), xc.cuda()
    attn.attn_rope_append(dk, dkc, dq, sp.cuda(), None if nn is None else nn.cuda(), x.cuda(), dxc, rope_base=base)
    torch.cuda.synchronize()
    k4 = k if not three_d_k else k[:, :, None]
    kc4 = kc if not three_d_k else kc[:, :, None]
    ref = oracle.rope_append(k4, kc4, q, sp.numpy(), None if nn is None else nn.numpy(),
                             x.numpy(), xc.numpy(), base=base)
    P = np.maximum(sp.numpy(), 0)
    n = np.full(B, S) if nn is None else np.clip(nn.numpy(), 0, S)
    got_kc = dkc if not three_d_k else dkc[:, :, None]
    for b in range(B):
        _check_rotated(dq[b, :n[b]], ref["q"][b, :n[b]], f"q rows of sequence {b}")
        assert np.array_equal(_bits(dq[b, n[b]:]), _bits(q[b, n[b]:])), "q rows past n_new"
        lo, hi = min(P[b], T), min(P[b] + n[b], T)
        _check_rotated(got_kc[b, lo:hi], ref["k_cache"][b, lo:hi], f"cache rows of sequence {b}")
        kb = _bits(got_kc[b])
        assert np.array_equal(np.delete(kb, np.arange(lo, hi), axis=0),
                              np.delete(_bits(kc4[b]), np.arange(lo, hi), axis=0)), "cache rows off the positions"
    assert np.array_equal(dxc.cpu().numpy(), ref["x_cache"]), "x cache bytes"
    assert np.array_equal(_bits(dk), _bits(k)), "k_new must not change when k_cache is given"
    return dq, dkc


CASES = [
    # name, B, S, Hq, Hk, d, T_max, start_pos, n_new, dtype
    ("gqa_chunk_bf16", 2, 300, 8, 2, 128, 1000, [0, 517], [300, 77], torch.bfloat16),
    ("gqa_decode_step_bf16", 16, 1, 32, 8, 128, 4096, list(range(0, 4096, 256)), None, torch.bfloat16),
    ("gqa_fp32_d96", 2, 70, 8, 4, 96, 300, [5, 250], [70, 70], torch.float32),
    ("overruns_cache", 2, 40, 4, 2, 64, 100, [90, -7], [40, 12], torch.bfloat16),
    ("empty_and_far_positions", 3, 20, 4, 1, 64, 50, [1000000, 3, 2 ** 30], [20, 0, 5], torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rope_append_matches_oracle(case):
    name, B, S, Hq, Hk, d, T, sp, nn, dtype = case
    print(f"[case] {name}", flush=True)
    _run_case(B, S, Hq, Hk, d, T, sp, nn, dtype, seed=len(name), x_bytes=Hk * d * (2 if dtype == torch.bfloat16 else 4))


def test_rope_append_mla_shapes_and_base():
    """MLA: q_rope [B,S,H,48], the shared k_rope [B,S,48] (3-D, one head), the latent rows as x;
    a MiniMind-style base of 1e6."""
    print("[case] mla rope_dim 48, base 1e6", flush=True)
    _run_case(4, 33, 8, 1, 48, 200, [0, 100, 167, 199], [33, 33, 33, 2], torch.bfloat16, base=1e6, seed=3,
              x_bytes=256, three_d_k=True)


def test_rope_in_place_and_chunking_is_bitwise():
    """k_cache NULL rotates k_new in place; one sequence appended in two chunks writes exactly the
    caches of one call over the whole sequence (each token's rotation depends on its position only)."""
    import mha_mla_kv_amd as attn
    g = torch.Generator().manual_seed(9)
    B, S, Hq, Hk, d, T = 2, 96, 8, 2, 128, 256
    q, k = _rand(g, (B, S, Hq, d), torch.bfloat16).cuda(), _rand(g, (B, S, Hk, d), torch.bfloat16).cuda()
    sp0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    q1, k1 = q.clone(), k.clone()
    attn.attn_rope_append(k1, None, q1, sp0)  # in place
    torch.cuda.synchronize()
    ref = oracle.rope_append(k.cpu(), None, q.cpu())
    _check_rotated(q1, ref["q"], "q in place")
    _check_rotated(k1, ref["k"], "k in place")
    one = torch.zeros(B, T, Hk, d, dtype=torch.bfloat16, device="cuda")
    attn.attn_rope_append(k.clone(), one, q.clone(), sp0)
    two = torch.zeros_like(one)
    P = 40
    attn.attn_rope_append(k[:, :P].contiguous(), two, q[:, :P].contiguous(), sp0)
    attn.attn_rope_append(k[:, P:].contiguous(), two, q[:, P:].contiguous(), sp0 + P)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))
    assert torch.equal(one[:, :S].view(torch.int16), k1.view(torch.int16)), "cache rows = rows rotated in place"


def test_decode_step_with_rope_matches_oracle():
    """A GQA decode step from unrotated projections: attn_rope_append (q in place, K to the cache
    at cache_lens, V copied) then attn_decode_gqa over cache_lens + 1, against the oracle's rotation,
    append and decode."""
    import mha_mla_kv_amd as attn
    import synth
    B, Hq, Hkv, D, T = 4, 32, 8, 128, 2000
    inp = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, [1999, 0, 700, 64], seed=17)
    g = torch.Generator().manual_seed(17)
    q = _rand(g, (B, 1, Hq, D), torch.bfloat16)
    k_new, v_new = _rand(g, (B, 1, Hkv, D), torch.bfloat16), _rand(g, (B, 1, Hkv, D), torch.bfloat16)
    lens = inp["cache_lens"]
    dq, dk, dv = q.cuda(), inp["k"].cuda(), inp["v"].cuda()
    attn.attn_rope_append(k_new.cuda(), dk, dq, lens.cuda(), None, v_new.cuda(), dv)
    out = attn.attn_decode_gqa(dq[:, 0].contiguous(), dk, dv, (lens + 1).cuda())
    torch.cuda.synchronize()
    r = oracle.rope_append(k_new, inp["k"], q, lens.numpy())
    vc = oracle.cache_append(inp["v"].float().numpy(), v_new.float().numpy(), lens.numpy())
    ref = oracle.gqa_decode(r["q"][:, 0].astype(np.float32), r["k_cache"].astype(np.float32), vc.astype(np.float32),
                            (lens + 1).numpy())
    assert_close_rows(out, ref, TOL_BF16, "rope + append + decode")
