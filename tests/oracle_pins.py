"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function takes an oracle library handle (``oracle.load()`` or a
deliberately broken build of oracle.c) and raises AssertionError when the
oracle disagrees with:
  * a library routine: torch's CPU float64 ``scaled_dot_product_attention``, with
    K/V expanded to one head per query head by ``repeat_interleave`` along the
    head axis (the expansion the "MQA & GQA 调研" page's repeat_kv docstring
    names), and, for MLA, keys/values rebuilt with ``torch.nn.functional.linear``
    from the up-projection weights exactly as the MultiHeadLatentAttention
    listing on the qqstock DeepSeek MLA article builds them;
  * closed forms: one cached token returns its V row; a zero query returns the
    mean of the V rows; two tokens weight V by logistic functions of the score
    gap; a saturating one-hot key selects one V row bit-exactly;
  * invariants: a joint permutation of cached tokens, a constant added to every
    score, per-head MHA, MQA = every head reading KV head 0, GQA = MHA on K/V
    expanded by the contiguous head-to-group map h -> h // n_rep, MLA absorbed =
    decompressed;
  * cached-prefix prefill: torch SDPA with an explicit position mask, an empty
    prefix reducing to causal prefill, and each new row equal to a decode at its
    own position;
  * MLA prefill: the listing's own scaled_dot_product_attention(is_causal=True) over
    keys and values rebuilt with F.linear, and each new row equal to an MLA decode
    at its position;
  * the empty cache giving zeros (a reading; the pages are silent).
The tests run them on the real oracle; tests/test_oracle_mutants.py runs them on
broken copies and requires that each planted mistake trips at least one pin.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle

TOL = 1e-12


def _rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def _close(a, b, tol=TOL, what=""):
    r = _rel(a, b)
    assert np.all(np.isfinite(a)), f"{what}: non-finite oracle output"
    assert r <= tol, f"{what}: relative error {r:.3e} > {tol:.1e}"


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _rand(rng, *shape):
    return rng.standard_normal(size=shape).astype(np.float32)


# ----------------------------------------------------------------------------- library routine

def sdpa_decode_ref(q, k, v, lens, scale=None):
    """torch float64 SDPA, one sequence at a time, K/V expanded per query head."""
    B, Hq, D = q.shape
    Hkv = k.shape[2]
    n_rep = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        qb = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]          # [1,Hq,1,D]
        kb = torch.from_numpy(k[b, :L].astype(np.float64)).repeat_interleave(n_rep, dim=1)
        vb = torch.from_numpy(v[b, :L].astype(np.float64)).repeat_interleave(n_rep, dim=1)
        kb = kb.permute(1, 0, 2)[None]                                              # [1,Hq,L,D]
        vb = vb.permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(qb, kb, vb, scale=scale)
        out[b] = o[0, :, 0, :].numpy()
    return out


def sdpa_prefill_ref(q, k, v, scale=None):
    B, S, Hq, D = q.shape
    n_rep = Hq // k.shape[2]
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(n_rep, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(n_rep, dim=2).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def sdpa_mla_ref(q_nope, q_rope, w_uk, w_uv, c_kv, k_rope, lens, scale=None):
    """Keys [W_UK c , k_rope] and values W_UV c rebuilt with F.linear from the per-head weights
    viewed as the up-projection Linear weights ([H*dn, r] and [H*dv, r]); k_rope is broadcast to
    every head; the new token's query sees the whole cache (no causal cut inside the cache)."""
    B, H, dn = q_nope.shape
    dR = q_rope.shape[2]
    dv, r = w_uv.shape[1], w_uv.shape[2]
    Wk = torch.from_numpy(w_uk.astype(np.float64)).reshape(H * dn, r)
    Wv = torch.from_numpy(w_uv.astype(np.float64)).reshape(H * dv, r)
    out = np.zeros((B, H, dv))
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        c = torch.from_numpy(c_kv[b, :L].astype(np.float64))                       # [L, r]
        k_nope = F.linear(c, Wk).view(L, H, dn).permute(1, 0, 2)                     # [H, L, dn]
        value = F.linear(c, Wv).view(L, H, dv).permute(1, 0, 2)                      # [H, L, dv]
        kr = torch.from_numpy(k_rope[b, :L].astype(np.float64))[None].expand(H, L, dR)
        k_rec = torch.cat([k_nope, kr], dim=-1)[None]                                # [1,H,L,dn+dR]
        q_rec = torch.cat([torch.from_numpy(q_nope[b].astype(np.float64)),
                           torch.from_numpy(q_rope[b].astype(np.float64))], dim=-1)[None, :, None, :]
        o = F.scaled_dot_product_attention(q_rec, k_rec, value[None], scale=scale)
        out[b] = o[0, :, 0, :].numpy()
    return out


# ----------------------------------------------------------------------------- GQA decode pins

DECODE_SHAPES = [
    # B, Hq, Hkv, D, T_max, lens
    (2, 8, 2, 16, 12, [12, 5]),
    (3, 4, 4, 8, 9, [1, 9, 4]),       # MHA
    (2, 6, 1, 8, 7, [7, 3]),          # MQA
    (1, 8, 4, 96, 33, [33]),
    (2, 32, 8, 128, 20, [17, 20]),
]


def pin_decode_vs_sdpa(lib):
    for i, (B, Hq, Hkv, D, T, lens) in enumerate(DECODE_SHAPES):
        rng = _rng(100 + i)
        q, k, v = _rand(rng, B, Hq, D), _rand(rng, B, T, Hkv, D), _rand(rng, B, T, Hkv, D)
        lens = np.array(lens, dtype=np.int32)
        _close(oracle.gqa_decode(q, k, v, lens, lib=lib), sdpa_decode_ref(q, k, v, lens),
               what=f"decode default scale {B,Hq,Hkv,D}")
        s = 0.37
        _close(oracle.gqa_decode(q, k, v, lens, softmax_scale=s, lib=lib),
               sdpa_decode_ref(q, k, v, lens, scale=s), what="decode explicit scale")


def pin_decode_closed_forms(lib):
    rng = _rng(7)
    B, Hq, Hkv, D, T = 2, 4, 2, 8, 6
    q, k, v = _rand(rng, B, Hq, D), _rand(rng, B, T, Hkv, D), _rand(rng, B, T, Hkv, D)
    n_rep = Hq // Hkv
    # one cached token: the output is that token's V row, exactly
    out = oracle.gqa_decode(q, k, v, np.array([1, 1], np.int32), lib=lib)
    for b in range(B):
        for h in range(Hq):
            assert np.array_equal(out[b, h], v[b, 0, h // n_rep].astype(np.float64)), "L=1 != V0"
    # zero query: uniform weights, the mean of the visible V rows
    lens = np.array([6, 3], np.int32)
    out = oracle.gqa_decode(np.zeros_like(q), k, v, lens, lib=lib)
    for b in range(B):
        for h in range(Hq):
            _close(out[b, h], v[b, :lens[b], h // n_rep].astype(np.float64).mean(axis=0), 1e-14,
                   "q=0 mean")
    # two tokens: weights sigma(s0-s1), sigma(s1-s0)
    scale = 1.0 / math.sqrt(D)
    out = oracle.gqa_decode(q, k, v, np.array([2, 2], np.int32), lib=lib)
    for b in range(B):
        for h in range(Hq):
            g = h // n_rep
            s0 = scale * float(np.dot(q[b, h].astype(np.float64), k[b, 0, g]))
            s1 = scale * float(np.dot(q[b, h].astype(np.float64), k[b, 1, g]))
            w0 = 1.0 / (1.0 + math.exp(s1 - s0))
            want = w0 * v[b, 0, g].astype(np.float64) + (1.0 - w0) * v[b, 1, g].astype(np.float64)
            _close(out[b, h], want, 1e-14, "two-token sigmoid")
    # saturating one-hot selection: q = 8*1, K[t*] = 8*1, other K = 0 -> exactly V[t*]
    T2 = 40
    q1 = np.full((1, Hq, D), 8.0, np.float32)
    k1 = np.zeros((1, T2, Hkv, D), np.float32)
    v1 = _rand(rng, 1, T2, Hkv, D)
    for t_star in (0, 17, 39):
        k1[:] = 0.0
        k1[0, t_star] = 8.0
        out = oracle.gqa_decode(q1, k1, v1, np.array([T2], np.int32), lib=lib)
        for h in range(Hq):
            assert np.array_equal(out[0, h], v1[0, t_star, h // n_rep].astype(np.float64)), "one-hot"


def pin_decode_invariants(lib):
    rng = _rng(11)
    B, Hq, Hkv, D, T = 2, 8, 2, 16, 10
    q, k, v = _rand(rng, B, Hq, D), _rand(rng, B, T, Hkv, D), _rand(rng, B, T, Hkv, D)
    lens = np.array([10, 10], np.int32)
    base = oracle.gqa_decode(q, k, v, lens, lib=lib)
    perm = rng.permutation(T)
    _close(oracle.gqa_decode(q, k[:, perm], v[:, perm], lens, lib=lib), base, 1e-13, "permutation")
    # each output coordinate lies between the min and max of the V rows it read
    n_rep = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            vv = v[b, :, h // n_rep].astype(np.float64)
            assert np.all(base[b, h] <= vv.max(0) + 1e-12) and np.all(base[b, h] >= vv.min(0) - 1e-12)
    # a constant added to every score changes nothing: single head, K' = K + c q/|q|^2
    q1, k1, v1 = _rand(rng, 1, 1, D), _rand(rng, 1, T, 1, D), _rand(rng, 1, T, 1, D)
    L1 = np.array([T], np.int32)
    qq = q1[0, 0].astype(np.float64)
    shift = (3.0 * qq / np.dot(qq, qq)).astype(np.float64)
    k_shift = (k1.astype(np.float64) + shift[None, None, None, :])
    a = oracle.gqa_decode(q1, k1, v1, L1, lib=lib)
    b_ = oracle.gqa_decode(q1, k_shift.astype(np.float32), v1, L1, lib=lib)
    assert _rel(a, b_) < 1e-5, "score shift"  # k_shift is rounded to float32 once
    # an empty cache gives zeros; lengths beyond T_max are clamped
    z = oracle.gqa_decode(q, k, v, np.array([0, 10], np.int32), lib=lib)
    assert np.all(z[0] == 0.0) and np.all(np.isfinite(z))
    _close(oracle.gqa_decode(q, k, v, np.array([999, 10], np.int32), lib=lib), base, 0.0, "clamp")


def pin_decode_head_structure(lib):
    rng = _rng(13)
    B, Hq, D, T = 2, 8, 16, 9
    lens = np.array([9, 4], np.int32)
    # MHA (Hkv = Hq) equals single-head attention run independently per head
    q, k, v = _rand(rng, B, Hq, D), _rand(rng, B, T, Hq, D), _rand(rng, B, T, Hq, D)
    mha = oracle.gqa_decode(q, k, v, lens, lib=lib)
    for h in range(Hq):
        one = oracle.gqa_decode(np.ascontiguousarray(q[:, h:h + 1]), np.ascontiguousarray(k[:, :, h:h + 1]),
                                np.ascontiguousarray(v[:, :, h:h + 1]), lens, lib=lib)
        _close(mha[:, h:h + 1], one, 0.0, "MHA per head")
    # MQA (Hkv = 1) equals MHA with the single K/V head copied to every head
    k1, v1 = _rand(rng, B, T, 1, D), _rand(rng, B, T, 1, D)
    mqa = oracle.gqa_decode(q, k1, v1, lens, lib=lib)
    _close(mqa, oracle.gqa_decode(q, np.repeat(k1, Hq, axis=2), np.repeat(v1, Hq, axis=2), lens, lib=lib),
           0.0, "MQA")
    # GQA equals MHA on K/V expanded to one head per query head, built from the grouping
    # definition itself: query head h reads KV head h // n_rep (the contiguous grouping)
    for Hkv in (2, 4):
        n_rep = Hq // Hkv
        kg, vg = _rand(rng, B, T, Hkv, D), _rand(rng, B, T, Hkv, D)
        src = np.arange(Hq) // n_rep
        ke, ve = kg[:, :, src], vg[:, :, src]
        assert np.array_equal(ke, np.repeat(kg, n_rep, axis=2))  # the same expansion as repeat_interleave
        _close(oracle.gqa_decode(q, kg, vg, lens, lib=lib),
               oracle.gqa_decode(q, np.ascontiguousarray(ke), np.ascontiguousarray(ve), lens, lib=lib),
               0.0, f"expanded K/V n_rep={n_rep}")


# ----------------------------------------------------------------------------- prefill pins

PREFILL_SHAPES = [(2, 7, 8, 2, 16), (1, 5, 4, 4, 8), (1, 6, 4, 1, 8), (1, 33, 8, 2, 128)]


def pin_prefill_vs_sdpa(lib):
    for i, (B, S, Hq, Hkv, D) in enumerate(PREFILL_SHAPES):
        rng = _rng(200 + i)
        q, k, v = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
        _close(oracle.gqa_prefill_causal(q, k, v, lib=lib), sdpa_prefill_ref(q, k, v), what="prefill")
        _close(oracle.gqa_prefill_causal(q, k, v, softmax_scale=0.2, lib=lib),
               sdpa_prefill_ref(q, k, v, scale=0.2), what="prefill scale")


def pin_prefill_rows(lib):
    rng = _rng(17)
    B, S, Hq, Hkv, D = 2, 9, 8, 2, 16
    q, k, v = _rand(rng, B, S, Hq, D), _rand(rng, B, S, Hkv, D), _rand(rng, B, S, Hkv, D)
    full = oracle.gqa_prefill_causal(q, k, v, lib=lib)
    n_rep = Hq // Hkv
    for b in range(B):  # the first query sees only key 0
        for h in range(Hq):
            assert np.array_equal(full[b, 0, h], v[b, 0, h // n_rep].astype(np.float64)), "row 0"
    sub = oracle.gqa_prefill_causal(q, k, v, rows=[8, 3], lib=lib)
    _close(sub[:, [3, 8]], full[:, [3, 8]], 0.0, "row subset")
    for i in (3, 8):  # causal row i = decode of query i against the first i+1 cached tokens
        dec = oracle.gqa_decode(np.ascontiguousarray(q[:, i]), k, v, np.full(B, i + 1, np.int32), lib=lib)
        _close(full[:, i], dec, 1e-14, f"row {i} vs decode")


# ----------------------------------------------------------------------------- cached-prefix prefill pins

CACHED_SHAPES = [
    # B, S, Hq, Hkv, D, T_max, start_pos, q_lens
    (2, 5, 8, 2, 16, 12, [4, 7], [5, 3]),
    (3, 4, 4, 4, 8, 9, [0, 5, 2], [4, 4, 1]),     # MHA, one sequence with an empty prefix
    (2, 6, 6, 1, 8, 10, [3, 4], [6, 6]),          # MQA
    (1, 9, 8, 2, 128, 30, [21], [9]),
]


def sdpa_cached_ref(q, k, v, start_pos, q_lens, scale=None):
    """torch float64 SDPA per sequence with an explicit boolean mask: new token i, at position
    P + i, may attend cache positions j <= P + i, out of the first P + n positions."""
    B, S, Hq, D = q.shape
    n_rep = Hq // k.shape[2]
    out = np.zeros((B, S, Hq, D))
    for b in range(B):
        P, n = int(start_pos[b]), int(q_lens[b])
        if n == 0:
            continue
        L = P + n
        qt = torch.from_numpy(q[b, :n].astype(np.float64)).permute(1, 0, 2)[None]            # [1,Hq,n,D]
        kt = torch.from_numpy(k[b, :L].astype(np.float64)).repeat_interleave(n_rep, dim=1).permute(1, 0, 2)[None]
        vt = torch.from_numpy(v[b, :L].astype(np.float64)).repeat_interleave(n_rep, dim=1).permute(1, 0, 2)[None]
        mask = torch.arange(L)[None, :] <= (P + torch.arange(n))[:, None]                     # [n, L]
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        out[b, :n] = o[0].permute(1, 0, 2).numpy()
    return out


def pin_cached_vs_sdpa(lib):
    for i, (B, S, Hq, Hkv, D, T, sp, ql) in enumerate(CACHED_SHAPES):
        rng = _rng(400 + i)
        q, k, v = _rand(rng, B, S, Hq, D), _rand(rng, B, T, Hkv, D), _rand(rng, B, T, Hkv, D)
        sp, ql = np.array(sp, np.int32), np.array(ql, np.int32)
        got = oracle.gqa_prefill_cached(q, k, v, sp, ql, lib=lib)
        _close(got, sdpa_cached_ref(q, k, v, sp, ql), what=f"cached prefill {B,S,Hq,Hkv,D}")
        for b in range(B):  # rows past the new-token count are zero
            assert not np.any(got[b, ql[b]:]), "rows past q_lens"
        _close(oracle.gqa_prefill_cached(q, k, v, sp, ql, softmax_scale=0.3, lib=lib),
               sdpa_cached_ref(q, k, v, sp, ql, scale=0.3), what="cached prefill scale")


def pin_cached_reductions(lib):
    """An empty prefix is causal prefill over the new tokens; each new row is a decode of that
    query against the cache up to its own position; a cache whose keys are all equal makes every
    row the mean of the visible V rows."""
    rng = _rng(29)
    B, S, Hq, Hkv, D, T = 2, 6, 8, 2, 16, 15
    q, k, v = _rand(rng, B, S, Hq, D), _rand(rng, B, T, Hkv, D), _rand(rng, B, T, Hkv, D)
    zero = oracle.gqa_prefill_cached(q, k, v, np.zeros(B, np.int32), None, lib=lib)
    causal = oracle.gqa_prefill_causal(q, np.ascontiguousarray(k[:, :S]), np.ascontiguousarray(v[:, :S]), lib=lib)
    _close(zero, causal, 1e-14, "empty prefix vs causal prefill")
    sp = np.array([9, 3], np.int32)
    got = oracle.gqa_prefill_cached(q, k, v, sp, None, lib=lib)
    for i in range(S):
        dec = oracle.gqa_decode(np.ascontiguousarray(q[:, i]), k, v, sp + i + 1, lib=lib)
        _close(got[:, i], dec, 1e-14, f"cached row {i} vs decode")
    kc = np.broadcast_to(k[:, :1], k.shape).copy()
    got = oracle.gqa_prefill_cached(q, kc, v, sp, None, lib=lib)
    n_rep = Hq // Hkv
    for b in range(B):
        for i in range(S):
            L = sp[b] + i + 1
            want = v[b, :L].astype(np.float64).mean(axis=0)          # [Hkv, D]
            for h in range(Hq):
                _close(got[b, i, h], want[h // n_rep], 1e-13, "equal keys -> mean of V")
    # the prefix fills the cache: the new-token count is clamped to the room left
    got = oracle.gqa_prefill_cached(q, k, v, np.array([T - 2, T], np.int32), None, lib=lib)
    assert not np.any(got[0, 2:]) and not np.any(got[1]), "clamp at T_max"


# ----------------------------------------------------------------------------- MLA pins

MLA_SHAPES = [
    # B, H, dn, dR, dv, r, T, lens
    (2, 4, 8, 4, 6, 16, 7, [7, 3]),
    (1, 8, 96, 48, 96, 128, 12, [12]),
    (2, 2, 5, 3, 7, 9, 5, [5, 1]),
]


def _mla_inputs(rng, B, H, dn, dR, dv, r, T):
    return (_rand(rng, B, H, dn), _rand(rng, B, H, dR), _rand(rng, H, dn, r) / np.float32(math.sqrt(r)),
            _rand(rng, H, dv, r) / np.float32(math.sqrt(r)), _rand(rng, B, T, r), _rand(rng, B, T, dR))


def pin_mla_vs_sdpa(lib):
    for i, (B, H, dn, dR, dv, r, T, lens) in enumerate(MLA_SHAPES):
        rng = _rng(300 + i)
        args = _mla_inputs(rng, B, H, dn, dR, dv, r, T)
        lens = np.array(lens, np.int32)
        ref = sdpa_mla_ref(*args, lens)
        _close(oracle.mla_decode_decompressed(*args, lens, lib=lib), ref, what="MLA decompressed")
        _close(oracle.mla_decode_absorbed(*args, lens, lib=lib), ref, what="MLA absorbed")
        ref_s = sdpa_mla_ref(*args, lens, scale=0.11)
        _close(oracle.mla_decode_absorbed(*args, lens, softmax_scale=0.11, lib=lib), ref_s, what="MLA scale")


def pin_mla_absorbed_equals_decompressed(lib):
    rng = _rng(19)
    B, H, dn, dR, dv, r, T = 3, 8, 96, 48, 96, 128, 20
    args = _mla_inputs(rng, B, H, dn, dR, dv, r, T)
    lens = np.array([20, 1, 13], np.int32)
    a = oracle.mla_decode_absorbed(*args, lens, lib=lib)
    d = oracle.mla_decode_decompressed(*args, lens, lib=lib)
    _close(a, d, TOL, "absorbed vs decompressed")
    sub = oracle.mla_decode_absorbed(*args, lens, bh=[5, 17], lib=lib)
    flat, fsub = a.reshape(B * H, dv), sub.reshape(B * H, dv)
    _close(fsub[[5, 17]], flat[[5, 17]], 0.0, "bh subset")


def pin_mla_selection(lib):
    """0/1 selection weights and a saturating score make the output an exact copy of chosen
    latent coordinates."""
    H, dn, dR, dv, r, T = 2, 4, 4, 3, 8, 6
    w_uk = np.zeros((H, dn, r), np.float32)
    w_uv = np.zeros((H, dv, r), np.float32)
    for h in range(H):
        w_uk[h, 0, h] = 1.0              # k_nope[h][0] = c[h]
        for i in range(dv):
            w_uv[h, i, (i + 2 * h) % r] = 1.0  # v[h][i] = c[(i + 2h) % r]
    rng = _rng(23)
    c = _rand(rng, 1, T, r)
    t_star = 4
    for h in range(H):
        c[0, :, h] = 0.0
        c[0, t_star, h] = 50.0
    q_nope = np.zeros((1, H, dn), np.float32)
    q_nope[0, :, 0] = 50.0
    q_rope = np.zeros((1, H, dR), np.float32)
    k_rope = _rand(rng, 1, T, dR)
    for fn in (oracle.mla_decode_absorbed, oracle.mla_decode_decompressed):
        out = fn(q_nope, q_rope, w_uk, w_uv, c, k_rope, np.array([T], np.int32), lib=lib)
        for h in range(H):
            want = np.array([c[0, t_star, (i + 2 * h) % r] for i in range(dv)], np.float64)
            assert np.array_equal(out[0, h], want), "MLA selection"


def sdpa_mla_prefill_ref(q_nope, q_rope, w_uk, w_uv, c_kv, k_rope, start_pos, q_lens, scale=None):
    """The listing's prefill: keys [F.linear(c, W_UK) , k_rope broadcast to every head], values
    F.linear(c, W_UV), torch SDPA per sequence; is_causal=True when there is no prefix, else an
    explicit mask letting new token i (position P + i) see cache rows j <= P + i."""
    B, S, H, dn = q_nope.shape
    dR = q_rope.shape[3]
    dv, r = w_uv.shape[1], w_uv.shape[2]
    Wk = torch.from_numpy(w_uk.astype(np.float64)).reshape(H * dn, r)
    Wv = torch.from_numpy(w_uv.astype(np.float64)).reshape(H * dv, r)
    out = np.zeros((B, S, H, dv))
    for b in range(B):
        P, n = int(start_pos[b]), int(q_lens[b])
        if n == 0:
            continue
        L = P + n
        c = torch.from_numpy(c_kv[b, :L].astype(np.float64))
        k_nope = F.linear(c, Wk).view(L, H, dn).permute(1, 0, 2)
        value = F.linear(c, Wv).view(L, H, dv).permute(1, 0, 2)
        kr = torch.from_numpy(k_rope[b, :L].astype(np.float64))[None].expand(H, L, dR)
        k_rec = torch.cat([k_nope, kr], dim=-1)[None]
        q_rec = torch.cat([torch.from_numpy(q_nope[b, :n].astype(np.float64)),
                           torch.from_numpy(q_rope[b, :n].astype(np.float64))], dim=-1).permute(1, 0, 2)[None]
        if P == 0:
            o = F.scaled_dot_product_attention(q_rec, k_rec, value[None], is_causal=True, scale=scale)
        else:
            mask = torch.arange(L)[None, :] <= (P + torch.arange(n))[:, None]
            o = F.scaled_dot_product_attention(q_rec, k_rec, value[None], attn_mask=mask, scale=scale)
        out[b, :n] = o[0].permute(1, 0, 2).numpy()
    return out


MLA_PREFILL_SHAPES = [
    # B, S, H, dn, dR, dv, r, T_max, start_pos, q_lens
    (2, 6, 4, 8, 4, 6, 16, 6, [0, 0], [6, 6]),
    (2, 5, 3, 8, 4, 6, 16, 14, [7, 2], [5, 3]),
    (1, 7, 8, 96, 48, 96, 128, 12, [5], [7]),
]


def pin_mla_prefill_vs_sdpa(lib):
    for i, (B, S, H, dn, dR, dv, r, T, sp, ql) in enumerate(MLA_PREFILL_SHAPES):
        rng = _rng(500 + i)
        qn, qr = _rand(rng, B, S, H, dn), _rand(rng, B, S, H, dR)
        w_uk = _rand(rng, H, dn, r) / np.float32(math.sqrt(r))
        w_uv = _rand(rng, H, dv, r) / np.float32(math.sqrt(r))
        c, kr = _rand(rng, B, T, r), _rand(rng, B, T, dR)
        sp, ql = np.array(sp, np.int32), np.array(ql, np.int32)
        got = oracle.mla_prefill_causal(qn, qr, w_uk, w_uv, c, kr, sp, ql, lib=lib)
        _close(got, sdpa_mla_prefill_ref(qn, qr, w_uk, w_uv, c, kr, sp, ql), what=f"MLA prefill {i}")
        for b in range(B):
            assert not np.any(got[b, ql[b]:]), "MLA prefill rows past q_lens"
        _close(oracle.mla_prefill_causal(qn, qr, w_uk, w_uv, c, kr, sp, ql, softmax_scale=0.09, lib=lib),
               sdpa_mla_prefill_ref(qn, qr, w_uk, w_uv, c, kr, sp, ql, scale=0.09), what="MLA prefill scale")


def pin_mla_prefill_rows_are_decodes(lib):
    """New token i of an MLA prefill equals an MLA decode of its query over the cache up to its
    own position (the decode is pinned on its own), in both the decompressed and absorbed forms."""
    rng = _rng(31)
    B, S, H, dn, dR, dv, r, T = 2, 5, 4, 16, 8, 12, 32, 20
    qn, qr = _rand(rng, B, S, H, dn), _rand(rng, B, S, H, dR)
    w_uk = _rand(rng, H, dn, r) / np.float32(math.sqrt(r))
    w_uv = _rand(rng, H, dv, r) / np.float32(math.sqrt(r))
    c, kr = _rand(rng, B, T, r), _rand(rng, B, T, dR)
    sp = np.array([11, 0], np.int32)
    got = oracle.mla_prefill_causal(qn, qr, w_uk, w_uv, c, kr, sp, None, lib=lib)
    for i in range(S):
        args = (np.ascontiguousarray(qn[:, i]), np.ascontiguousarray(qr[:, i]), w_uk, w_uv, c, kr, sp + i + 1)
        _close(got[:, i], oracle.mla_decode_decompressed(*args, lib=lib), 1e-13, f"MLA prefill row {i}")
        _close(got[:, i], oracle.mla_decode_absorbed(*args, lib=lib), 1e-12, f"MLA prefill row {i} absorbed")
    # no prefix and no q_lens is the same as start_pos 0 and q_lens S
    _close(oracle.mla_prefill_causal(qn, qr, w_uk, w_uv, c, kr, None, None, lib=lib),
           oracle.mla_prefill_causal(qn, qr, w_uk, w_uv, c, kr, np.zeros(B, np.int32), np.full(B, S, np.int32),
                                     lib=lib), 0.0, "MLA prefill defaults")


def pin_cache_append(lib):
    """Appending a chunk after a prefix and running the cached-prefix prefill over the cache gives
    the causal prefill of the concatenated sequence at the chunk's rows; the prefix and the rows
    after the chunk stay as they were; a chunk that overruns the cache is cut at T_max."""
    rng = _rng(37)
    B, P, n, Hq, Hkv, D, T = 2, 9, 5, 4, 2, 8, 20
    prefix_k, prefix_v = _rand(rng, B, P, Hkv, D), _rand(rng, B, P, Hkv, D)
    new_k, new_v, q = _rand(rng, B, n, Hkv, D), _rand(rng, B, n, Hkv, D), _rand(rng, B, n, Hq, D)
    cache_k, cache_v = _rand(rng, B, T, Hkv, D), _rand(rng, B, T, Hkv, D)
    cache_k[:, :P], cache_v[:, :P] = prefix_k, prefix_v
    sp = np.full(B, P, np.int32)
    k2, v2 = oracle.cache_append(cache_k, new_k, sp), oracle.cache_append(cache_v, new_v, sp)
    assert np.array_equal(k2[:, :P], prefix_k) and np.array_equal(k2[:, P + n:], cache_k[:, P + n:]), "untouched"
    got = oracle.gqa_prefill_cached(q, k2, v2, sp, None, lib=lib)
    full_q = np.concatenate([_rand(rng, B, P, Hq, D), q], axis=1)
    ref = oracle.gqa_prefill_causal(full_q, np.concatenate([prefix_k, new_k], 1), np.concatenate([prefix_v, new_v], 1),
                                    lib=lib)
    _close(got, ref[:, P:], 1e-14, "append + cached prefill vs causal prefill of the concatenation")
    k3 = oracle.cache_append(cache_k, new_k, np.array([T - 2, -3], np.int32), np.array([5, 2], np.int32))
    assert np.array_equal(k3[0, T - 2:], new_k[0, :2]) and np.array_equal(k3[0, :T - 2], cache_k[0, :T - 2])
    assert np.array_equal(k3[1, :2], new_k[1, :2]) and np.array_equal(k3[1, 2:], cache_k[1, 2:])


def pin_e4m3_decoding(lib):
    """Every FP8 E4M3 code against torch's float8_e4m3fn conversion (a library routine), plus
    the format's landmarks: 1.0, the largest finite 448, the smallest subnormal 2^-9, NaN."""
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_float(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isnan(got), ~fin), "NaN codes"
    assert np.array_equal(got[fin], ref[fin]), "E4M3 values"
    assert oracle.e4m3_to_float([0x38])[0] == 1.0 and oracle.e4m3_to_float([0x7E])[0] == 448.0
    assert oracle.e4m3_to_float([0x01])[0] == 2.0 ** -9 and oracle.e4m3_to_float([0xB8], 0.5)[0] == -0.5


def pin_rope_quarter_turns(lib):
    """Closed forms that fix which elements pair up, the turning direction and the frequency
    exponent 2j/d.  With d = 4 and base = (2/pi)^2 the second pair turns by base^(-1/2) = pi/2 per
    position: (x2, x3) = (0.25, -0.5) becomes (0.5, 0.25), (-0.25, 0.5), (-0.5, -0.25) and back at
    positions 1..4, while the first pair turns by 1 radian per position, taking (1, 0) to
    (cos m, sin m).  With d = 6 and base = (2/pi)^(3/2) the third pair turns by base^(-2/3) = pi/2."""
    base4 = (2.0 / math.pi) ** 2
    x = np.array([[[1.0, 0.0, 0.25, -0.5]]], np.float32)  # one token, one head, d = 4
    quarter = {1: (0.5, 0.25), 2: (-0.25, 0.5), 3: (-0.5, -0.25), 4: (0.25, -0.5)}
    for m, (a, b) in quarter.items():
        got = oracle.rope(x, [m], base4, lib=lib)[0, 0]
        _close(got, [math.cos(m), math.sin(m), a, b], 1e-14, f"d=4 position {m}")
    base6 = (2.0 / math.pi) ** 1.5
    y = np.array([[[0.0, 0.0, 0.0, 0.0, 1.0, 2.0]]], np.float32)
    _close(oracle.rope(y, [1], base6, lib=lib)[0, 0, 4:], [-2.0, 1.0], 1e-14, "d=6 third pair, position 1")
    # a lone second element of the first pair stays in the first pair: (0, 1) -> (-sin m, cos m)
    z = np.array([[[0.0, 1.0, 0.0, 0.0]]], np.float32)
    _close(oracle.rope(z, [2], base4, lib=lib)[0, 0], [-math.sin(2.0), math.cos(2.0), 0.0, 0.0], 1e-14,
           "first pair holds elements 0 and 1")


def pin_rope_invariants(lib):
    """Position 0 is the identity; every pair keeps its length; the score between a rotated query
    at position m and a rotated key at position n depends on n - m only (checked for shifts up to
    10^5 and the LLaMA base 10000)."""
    rng = _rng(41)
    x = _rand(rng, 3, 4, 16)
    assert np.array_equal(oracle.rope(x, [0, 0, 0], lib=lib), x.astype(np.float64)), "position 0"
    r = oracle.rope(x, [5, 77, 4096], lib=lib)
    n0 = np.hypot(x[..., 0::2].astype(np.float64), x[..., 1::2].astype(np.float64))
    _close(np.hypot(r[..., 0::2], r[..., 1::2]), n0, 1e-13, "pair lengths")
    q, k = _rand(rng, 1, 1, 64), _rand(rng, 1, 1, 64)
    for m, n in ((0, 0), (3, 17), (200, 9), (4095, 4096)):
        ref = float(np.sum(oracle.rope(q, [m], lib=lib) * oracle.rope(k, [n], lib=lib)))
        for sft in (1, 31, 1000, 100000):
            got = float(np.sum(oracle.rope(q, [m + sft], lib=lib) * oracle.rope(k, [n + sft], lib=lib)))
            assert abs(got - ref) <= 1e-9 * max(1.0, abs(ref)), f"score at ({m}, {n}) shifted by {sft}"


def pin_rope_append(lib):
    """The rotate-and-append step: appending a sequence in two chunks (the second at start_pos =
    the first's length) writes the same caches as appending it in one; each new row is the
    rotation at its absolute position; rows past n_new are neither rotated nor written, rows past
    T_max are rotated but not stored; and a decode over the rotated caches does not change when
    every position is shifted by the same amount (the relative-position property in use)."""
    rng = _rng(43)
    B, T, Hq, Hk, d = 2, 24, 4, 2, 8
    q, k = _rand(rng, B, T, Hq, d), _rand(rng, B, T, Hk, d)
    v = _rand(rng, B, T, Hk, d)
    cache_k, cache_v = np.zeros((B, T, Hk, d), np.float32), np.zeros((B, T, Hk, d), np.float32)
    one = oracle.rope_append(k, cache_k, q, None, None, v, cache_v, lib=lib)
    P = 10
    first = oracle.rope_append(k[:, :P], cache_k, q[:, :P], None, None, v[:, :P], cache_v, lib=lib)
    second = oracle.rope_append(k[:, P:], first["k_cache"], q[:, P:], np.full(B, P), None,
                                v[:, P:], first["x_cache"], lib=lib)
    assert np.array_equal(second["k_cache"], one["k_cache"]) and np.array_equal(second["x_cache"], one["x_cache"])
    assert np.array_equal(np.concatenate([first["q"], second["q"]], 1), one["q"]), "queries in two chunks"
    pos = np.broadcast_to(np.arange(T), (B, T))
    _close(one["k"], oracle.rope(k, pos, lib=lib), 0.0, "rows rotated at their positions")
    # n_new and T_max cuts: sequence 0 starts at T - 3 with 5 new rows (3 stored), sequence 1 has 2 of 5
    part = oracle.rope_append(k[:, :5], cache_k, q[:, :5], np.array([T - 3, 4]), np.array([5, 2]), lib=lib)
    _close(part["q"][0], oracle.rope(q[0, :5], np.arange(T - 3, T + 2), lib=lib), 0.0, "rotated past T_max")
    assert np.array_equal(part["q"][1, 2:], q[1, 2:5].astype(np.float64)), "rows past n_new untouched"
    assert np.array_equal(part["k_cache"][0, T - 3:], part["k"][0, :3]) and not part["k_cache"][0, :T - 3].any()
    assert np.array_equal(part["k_cache"][1, 4:6], part["k"][1, :2]) and not part["k_cache"][1, 6:].any()
    # decode of the last query over all T rotated keys (rows in order): a common shift of 500
    # positions changes nothing
    lens = np.full(B, T, np.int32)
    outs = []
    for start in (0, 500):
        r = oracle.rope_append(k, None, q, np.full(B, start), None, lib=lib)
        outs.append(oracle.gqa_decode(r["q"][:, -1].astype(np.float32), r["k"].astype(np.float32), v, lens, lib=lib))
    _close(outs[1], outs[0], 2e-6, "decode under a common position shift (float32 rounding of the rotated rows)")


def pin_gather_pages(lib):
    """The block-table layout: a pool holding a contiguous cache page by page in order, with the
    identity table, gives that cache back (and zeros past each length); shuffling the pool's pages
    and renumbering the table to match changes nothing; pages no table entry below the length
    points at, and table entries past it, are never read; a decode over the gathered caches equals
    the decode over the original ones."""
    rng = _rng(47)
    B, ps, mp, Hkv, D = 3, 4, 5, 2, 8
    cache = _rand(rng, B, mp * ps, Hkv, D)
    lens = np.array([20, 7, 0], np.int32)
    pool = cache.reshape(B * mp, ps, Hkv, D)
    ident = np.arange(B * mp, dtype=np.int32).reshape(B, mp)
    got = oracle.gather_pages(pool, ident, lens)
    for b in range(B):
        assert np.array_equal(got[b, :lens[b]], cache[b, :lens[b]]) and not got[b, lens[b]:].any(), "identity"
    perm = rng.permutation(B * mp)
    shuffled = np.empty_like(pool)
    shuffled[perm] = pool  # old page i is now page perm[i]
    table = perm[ident].astype(np.int32)
    table[1, 2:] = -99  # entries past sequence 1's length (7 positions: pages 0, 1)
    assert np.array_equal(oracle.gather_pages(shuffled, table, lens), got), "shuffled pool"
    spare = np.concatenate([shuffled, np.full((2, ps, Hkv, D), np.nan, np.float32)])
    assert np.array_equal(oracle.gather_pages(spare, table, lens), got), "unreferenced pages"
    q = _rand(rng, B, 4, D)
    _close(oracle.gqa_decode(q, got, oracle.gather_pages(shuffled, table, lens), lens, lib=lib),
           oracle.gqa_decode(q, cache, cache, lens, lib=lib), 0.0, "decode over gathered caches")


def pin_append_pages(lib):
    """The paged cache write against the contiguous one it stands for: appending rows into a
    shuffled pool and gathering the pages back equals cache_append on the gathered cache (pinned
    by pin_cache_append), over lengths that start mid-page, end a page and fill the cache; rows of
    the pool outside the written positions, spare pages included, keep their bits; an append
    past the cache is cut at T, as cache_append's is."""
    rng = _rng(53)
    B, ps, mp, Hkv, D = 3, 4, 5, 2, 8
    T = mp * ps
    cache = _rand(rng, B, T, Hkv, D)
    pool = cache.reshape(B * mp, ps, Hkv, D)
    perm = rng.permutation(B * mp)
    shuffled = np.concatenate([np.empty_like(pool), np.full((2, ps, Hkv, D), np.nan, np.float32)])
    shuffled[perm] = pool
    table = perm[np.arange(B * mp).reshape(B, mp)].astype(np.int32)
    new = _rand(rng, B, 3, Hkv, D)
    for start, n in (([5, 8, 0], None), ([3, 19, 20], [2, 3, 1]), ([0, 0, 18], [0, 1, 3])):
        start = np.array(start, np.int32)
        got = oracle.append_pages(shuffled, table, new, start, None if n is None else np.array(n, np.int32))
        full = np.full(B, T, np.int32)
        want = oracle.cache_append(oracle.gather_pages(shuffled, table, full), new, start,
                                   None if n is None else np.array(n, np.int32))
        assert np.array_equal(oracle.gather_pages(got, table, full), want), ("paged append", start, n)
        changed = ~np.all((got == shuffled) | (np.isnan(got) & np.isnan(shuffled)), axis=(2, 3))
        written = set()
        for b in range(B):
            m = 3 if n is None else n[b]
            for t in range(start[b], min(start[b] + m, T)):
                written.add((int(table[b, t // ps]), t % ps))
        assert {tuple(x) for x in np.argwhere(changed)} <= written, "rows outside the written positions"
        assert np.isnan(got[B * mp:]).all(), "spare pages"


def pin_int4_decoding(lib):
    """Every one of the 256 bytes against the two's-complement reading of each nibble computed by
    integer arithmetic (low nibble first), plus landmarks: 0x07 -> (7, 0), 0x80 -> (0, -8),
    0xF1 -> (1, -1), 0xFF -> (-1, -1); a row scale multiplies every code of its row."""
    allb = np.arange(256, dtype=np.uint8)[:, None]
    got = oracle.int4_to_float(allb)
    for v in range(256):
        lo, hi = v % 16, v // 16
        want = (lo - 16 if lo > 7 else lo, hi - 16 if hi > 7 else hi)
        assert tuple(got[v]) == want, (v, got[v], want)
    assert tuple(oracle.int4_to_float(np.array([0x07, 0x80, 0xF1, 0xFF], np.uint8))) == (7, 0, 0, -8, 1, -1, -1, -1)
    rows = np.array([[0x21, 0x43], [0x21, 0x43]], np.uint8)
    scaled = oracle.int4_to_float(rows, np.array([0.5, -2.0]))
    assert np.array_equal(scaled, [[0.5, 1.0, 1.5, 2.0], [-2.0, -4.0, -6.0, -8.0]]), scaled


ALL_PINS = [pin_decode_vs_sdpa, pin_decode_closed_forms, pin_decode_invariants, pin_decode_head_structure,
            pin_prefill_vs_sdpa, pin_prefill_rows, pin_cached_vs_sdpa, pin_cached_reductions, pin_mla_vs_sdpa, pin_mla_absorbed_equals_decompressed,
            pin_mla_selection, pin_mla_prefill_vs_sdpa, pin_mla_prefill_rows_are_decodes, pin_cache_append,
            pin_e4m3_decoding, pin_rope_quarter_turns, pin_rope_invariants, pin_rope_append,
            pin_gather_pages, pin_append_pages, pin_int4_decoding]
