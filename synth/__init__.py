"""Seeded synthetic inputs shared by the HIP library's tests/benchmark and the oracle.

This module holds no attention arithmetic: it only draws numbers.  Every tensor
comes from ``numpy.random.Generator(PCG64(seed))`` as float32 i.i.d. N(0, 1)
(weights N(0, 1/fan_in)), in a fixed draw order, and is then rounded
to-nearest-even to bfloat16 when the workload is bf16.  The same rounded values
feed both sides, so the oracle widens exactly what the GPU reads.

Cache slots at or beyond a sequence's length are filled with NaN ("poison") by
default: a kernel that reads past ``cache_lens[b]`` then produces NaN instead
of a plausible number.

Returned tensors are CPU ``torch`` tensors (torch is the device-memory plumbing of
the library); the oracle converts them to float32 numpy itself.
"""
from __future__ import annotations

import numpy as np
import torch

_DT = {"f32": torch.float32, "fp32": torch.float32, "bf16": torch.bfloat16}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _as(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    return t if _DT[dtype] == torch.float32 else t.to(_DT[dtype])


def _lengths(rng: np.random.Generator, B: int, T_max: int, lens) -> np.ndarray:
    """``lens``: int (same length for every sequence), (lo, hi) drawn uniformly with both ends
    included, or an explicit sequence of B ints."""
    if isinstance(lens, (int, np.integer)):
        return np.full(B, int(lens), dtype=np.int32)
    if isinstance(lens, tuple) and len(lens) == 2:
        lo, hi = lens
        return rng.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)
    arr = np.asarray(lens, dtype=np.int32)
    assert arr.shape == (B,)
    return arr


def _poison_tail(x: torch.Tensor, lens: np.ndarray) -> None:
    """Fill cache slots t >= lens[b] (axis 1) with NaN, in place."""
    for b, L in enumerate(lens.tolist()):
        L = max(0, min(int(L), x.shape[1]))
        if L < x.shape[1]:
            x[b, L:] = float("nan")


def gqa_decode_inputs(B: int, Hq: int, Hkv: int, D: int, T_max: int, lens, dtype: str = "bf16",
                      seed: int = 0, poison: bool = True) -> dict:
    """q [B,Hq,D], k/v caches [B,T_max,Hkv,D], cache_lens [B] int32.  Draw order q, k, v, lens."""
    rng = _rng(seed)
    q = _as(_normal(rng, (B, Hq, D)), dtype)
    k = _as(_normal(rng, (B, T_max, Hkv, D)), dtype)
    v = _as(_normal(rng, (B, T_max, Hkv, D)), dtype)
    L = _lengths(rng, B, T_max, lens)
    if poison:
        _poison_tail(k, L)
        _poison_tail(v, L)
    return {"q": q, "k": k, "v": v, "cache_lens": torch.from_numpy(L.copy())}


def gqa_decode_fp8_inputs(B: int, Hq: int, Hkv: int, D: int, T_max: int, lens, seed: int = 0,
                          poison: bool = True) -> dict:
    """q [B,Hq,D] bf16 and K/V caches [B,T_max,Hkv,D] stored as FP8 E4M3 (torch.float8_e4m3fn)
    with one scale per cache: each cache is drawn N(0, 1) in float32 and divided by
    scale = max|x| / 448 before the cast (round to nearest even), so the largest code is 448.
    Draw order q, k, v, lens.  With poison, codes past each length are NaN (0x7F)."""
    rng = _rng(seed)
    q = _as(_normal(rng, (B, Hq, D)), "bf16")
    k = _normal(rng, (B, T_max, Hkv, D))
    v = _normal(rng, (B, T_max, Hkv, D))
    L = _lengths(rng, B, T_max, lens)
    out = {"q": q, "cache_lens": torch.from_numpy(L.copy())}
    for name, x in (("k", k), ("v", v)):
        scale = float(np.abs(x).max()) / 448.0
        codes = torch.from_numpy(x / np.float32(scale)).to(torch.float8_e4m3fn)
        if poison:
            raw = codes.view(torch.uint8)
            for b, n in enumerate(L.tolist()):
                raw[b, max(0, min(int(n), T_max)):] = 0x7F
        out[name] = codes
        out[name + "_scale"] = scale
    return out


def gqa_decode_int4_inputs(B: int, Hq: int, Hkv: int, D: int, T_max: int, lens, seed: int = 0,
                           poison: bool = True) -> dict:
    """q [B,Hq,D] bf16 and K/V caches stored as packed signed 4-bit codes with one fp32 scale per
    cached row, head-major: k [B,Hkv,T_max,D/2] uint8 (code 2i in the low nibble of byte i, two's
    complement), k_scale [B,Hkv,T_max] float32, the same for v.  Each row is drawn N(0, 1) in
    float32 (drawn as [B,T_max,Hkv,D], then stored head-major), its scale is max|x| / 7 and its
    codes round(x / scale) clamped to [-8, 7] (round half to even).  Draw order q, k, v, lens.
    With poison, the scales of rows past each length are NaN."""
    rng = _rng(seed)
    q = _as(_normal(rng, (B, Hq, D)), "bf16")
    k = _normal(rng, (B, T_max, Hkv, D))
    v = _normal(rng, (B, T_max, Hkv, D))
    L = _lengths(rng, B, T_max, lens)
    out = {"q": q, "cache_lens": torch.from_numpy(L.copy())}
    for name, x in (("k", k), ("v", v)):
        x = x.transpose(0, 2, 1, 3)  # head-major
        scale = (np.abs(x).max(axis=-1) / np.float32(7.0)).astype(np.float32)
        scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
        codes = np.clip(np.rint(x / scale[..., None]), -8, 7).astype(np.int64)
        nib = (codes & 0xF).astype(np.uint8)
        packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
        if poison:
            for b, n in enumerate(L.tolist()):
                scale[b, :, max(0, min(int(n), T_max)):] = np.nan
        out[name] = torch.from_numpy(np.ascontiguousarray(packed))
        out[name + "_scale"] = torch.from_numpy(np.ascontiguousarray(scale))
    return out


def gqa_prefill_inputs(B: int, S: int, Hq: int, Hkv: int, D: int, dtype: str = "bf16",
                       seed: int = 0) -> dict:
    """q [B,S,Hq,D], k/v [B,S,Hkv,D].  Draw order q, k, v."""
    rng = _rng(seed)
    q = _as(_normal(rng, (B, S, Hq, D)), dtype)
    k = _as(_normal(rng, (B, S, Hkv, D)), dtype)
    v = _as(_normal(rng, (B, S, Hkv, D)), dtype)
    return {"q": q, "k": k, "v": v}


def gqa_prefill_cached_inputs(B: int, S: int, Hq: int, Hkv: int, D: int, T_max: int, start_pos,
                              q_lens=None, dtype: str = "bf16", seed: int = 0, poison: bool = True) -> dict:
    """Chunked prefill after a cached prefix: q [B,S,Hq,D] (the new tokens, padded to S), k/v
    caches [B,T_max,Hkv,D] already holding the new tokens' rows at start_pos[b]..,
    start_pos [B] and q_lens [B] int32 (``_lengths`` forms; q_lens None: S each).  Draw order q,
    k, v, start_pos, q_lens.  With poison, q rows past q_lens[b] and cache rows past
    start_pos[b] + q_lens[b] are NaN."""
    rng = _rng(seed)
    q = _as(_normal(rng, (B, S, Hq, D)), dtype)
    k = _as(_normal(rng, (B, T_max, Hkv, D)), dtype)
    v = _as(_normal(rng, (B, T_max, Hkv, D)), dtype)
    sp = _lengths(rng, B, T_max, start_pos)
    ql = _lengths(rng, B, S, S if q_lens is None else q_lens)
    if poison:
        _poison_tail(q, ql)
        end = np.minimum(np.maximum(sp.astype(np.int64), 0) + np.maximum(ql, 0), T_max).astype(np.int32)
        _poison_tail(k, end)
        _poison_tail(v, end)
    return {"q": q, "k": k, "v": v, "start_pos": torch.from_numpy(sp.copy()),
            "q_lens": torch.from_numpy(ql.copy())}


def mla_decode_inputs(B: int, H: int, nope_head_dim: int, rope_dim: int, v_head_dim: int,
                      kv_lora_rank: int, T_max: int, lens, dtype: str = "bf16", seed: int = 0,
                      poison: bool = True) -> dict:
    """q_nope [B,H,dn], q_rope [B,H,dR], w_uk [H,dn,r], w_uv [H,dv,r], c_kv [B,T_max,r],
    k_rope [B,T_max,dR], cache_lens [B].

    w_uk / w_uv are the k-nope and value up-projection weights, drawn N(0, 1/r) (r, the latent
    width, is the fan-in of both) and viewed per head.  Draw order: q_nope, q_rope, w_uk, w_uv,
    c_kv, k_rope, lens."""
    rng = _rng(seed)
    dn, dR, dv, r = nope_head_dim, rope_dim, v_head_dim, kv_lora_rank
    q_nope = _as(_normal(rng, (B, H, dn)), dtype)
    q_rope = _as(_normal(rng, (B, H, dR)), dtype)
    w_uk = _as(_normal(rng, (H, dn, r), std=float(1.0 / np.sqrt(r))), dtype)
    w_uv = _as(_normal(rng, (H, dv, r), std=float(1.0 / np.sqrt(r))), dtype)
    c_kv = _as(_normal(rng, (B, T_max, r)), dtype)
    k_rope = _as(_normal(rng, (B, T_max, dR)), dtype)
    L = _lengths(rng, B, T_max, lens)
    if poison:
        _poison_tail(c_kv, L)
        _poison_tail(k_rope, L)
    return {"q_nope": q_nope, "q_rope": q_rope, "w_uk": w_uk, "w_uv": w_uv, "c_kv": c_kv,
            "k_rope": k_rope, "cache_lens": torch.from_numpy(L.copy())}


def mla_prefill_inputs(B: int, S: int, H: int, nope_head_dim: int, rope_dim: int, v_head_dim: int,
                       kv_lora_rank: int, T_max: int, start_pos=0, q_lens=None, dtype: str = "bf16",
                       seed: int = 0, poison: bool = True) -> dict:
    """MLA prefill: q_nope [B,S,H,dn], q_rope [B,S,H,dR] (the new tokens, padded to S), w_uk
    [H,dn,r], w_uv [H,dv,r] (N(0, 1/r)), c_kv [B,T_max,r], k_rope [B,T_max,dR] (holding the new
    rows at start_pos[b]..), start_pos and q_lens [B] int32 (``_lengths`` forms; q_lens None: S).
    Draw order as named.  With poison, q rows past q_lens[b] and cache rows past
    start_pos[b] + q_lens[b] are NaN."""
    rng = _rng(seed)
    dn, dR, dv, r = nope_head_dim, rope_dim, v_head_dim, kv_lora_rank
    q_nope = _as(_normal(rng, (B, S, H, dn)), dtype)
    q_rope = _as(_normal(rng, (B, S, H, dR)), dtype)
    w_uk = _as(_normal(rng, (H, dn, r), std=float(1.0 / np.sqrt(r))), dtype)
    w_uv = _as(_normal(rng, (H, dv, r), std=float(1.0 / np.sqrt(r))), dtype)
    c_kv = _as(_normal(rng, (B, T_max, r)), dtype)
    k_rope = _as(_normal(rng, (B, T_max, dR)), dtype)
    sp = _lengths(rng, B, T_max, start_pos)
    ql = _lengths(rng, B, S, S if q_lens is None else q_lens)
    if poison:
        _poison_tail(q_nope, ql)
        _poison_tail(q_rope, ql)
        end = np.minimum(np.maximum(sp.astype(np.int64), 0) + np.maximum(ql, 0), T_max).astype(np.int32)
        _poison_tail(c_kv, end)
        _poison_tail(k_rope, end)
    return {"q_nope": q_nope, "q_rope": q_rope, "w_uk": w_uk, "w_uv": w_uv, "c_kv": c_kv, "k_rope": k_rope,
            "start_pos": torch.from_numpy(sp.copy()), "q_lens": torch.from_numpy(ql.copy())}


# The workloads the pages' shapes give (name -> generator kwargs).  Seeds are fixed per workload.
WORKLOADS = {
    "minimind768_gqa_decode": dict(kind="gqa_decode", B=1, Hq=8, Hkv=4, D=96, T_max=512, lens=512,
                                   dtype="f32", seed=1),
    "llama3_8b_gqa_decode": dict(kind="gqa_decode", B=32, Hq=32, Hkv=8, D=128, T_max=8192,
                                 lens=(1024, 8192), dtype="bf16", seed=2),
    "kv_sweep_mha": dict(kind="gqa_decode", B=16, Hq=32, Hkv=32, D=128, T_max=8192, lens=8192,
                         dtype="bf16", seed=3),
    "kv_sweep_gqa8": dict(kind="gqa_decode", B=16, Hq=32, Hkv=8, D=128, T_max=8192, lens=8192,
                          dtype="bf16", seed=3),
    "kv_sweep_mqa": dict(kind="gqa_decode", B=16, Hq=32, Hkv=1, D=128, T_max=8192, lens=8192,
                         dtype="bf16", seed=3),
    "llama3_8b_gqa_prefill": dict(kind="gqa_prefill", B=4, S=4096, Hq=32, Hkv=8, D=128,
                                  dtype="bf16", seed=4),
    "llama3_8b_gqa_chunked_prefill": dict(kind="gqa_prefill_cached", B=4, S=512, Hq=32, Hkv=8, D=128,
                                          T_max=4096, start_pos=3584, q_lens=512, dtype="bf16", seed=6),
    "minimind768_mla_prefill": dict(kind="mla_prefill", B=4, S=4096, H=8, nope_head_dim=96, rope_dim=48,
                                    v_head_dim=96, kv_lora_rank=128, T_max=4096, start_pos=0, dtype="bf16", seed=7),
    "minimind768_mla_decode": dict(kind="mla_decode", B=64, H=8, nope_head_dim=96, rope_dim=48,
                                   v_head_dim=96, kv_lora_rank=128, T_max=4096, lens=4096,
                                   dtype="bf16", seed=5),
}


def make(name_or_spec, **overrides) -> dict:
    """Generate a named workload (optionally with some fields overridden)."""
    spec = dict(WORKLOADS[name_or_spec]) if isinstance(name_or_spec, str) else dict(name_or_spec)
    spec.update(overrides)
    kind = spec.pop("kind")
    if kind == "gqa_decode":
        return gqa_decode_inputs(**spec)
    if kind == "gqa_prefill":
        return gqa_prefill_inputs(**spec)
    if kind == "gqa_prefill_cached":
        return gqa_prefill_cached_inputs(**spec)
    if kind == "mla_prefill":
        return mla_prefill_inputs(**spec)
    if kind == "mla_decode":
        return mla_decode_inputs(**spec)
    raise ValueError(kind)
