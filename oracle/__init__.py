"""Plain fp64 CPU oracle for GQA / MQA / MHA / MLA attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It never imports the
HIP library (``mha_mla_kv_amd``) and shares no code with it; the two meet only
through the seeded inputs of ``synth``.

The arithmetic lives in ``oracle.c`` (plain loops, double accumulation, OpenMP
over independent output rows).  This module compiles it with gcc, marshals
arrays through ctypes and returns float64 numpy arrays.  ``accounting`` holds
the KV-cache byte and parameter closed forms.

What each routine computes, and the passage it follows, is stated at the top of
``oracle.c``.  Parity of every routine is pinned by ``tests/test_oracle_*.py``
against library routines, closed forms, invariants and the numbers the pages
print; none is left unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _SO) -> str:
    """Compile ``src`` (default: oracle.c) into a shared library at ``out``."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _declare(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_threads.restype = I
    lib.oracle_threads.argtypes = []
    lib.oracle_gqa_decode.restype = None
    lib.oracle_gqa_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, D]
    lib.oracle_gqa_prefill_causal.restype = None
    lib.oracle_gqa_prefill_causal.argtypes = [P, P, P, P, I, I, I, I, I, D, P, I]
    lib.oracle_mla_prefill_causal.restype = None
    lib.oracle_mla_prefill_causal.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, D]
    lib.oracle_gqa_prefill_cached.restype = None
    lib.oracle_gqa_prefill_cached.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, D]
    lib.oracle_rope.restype = None
    lib.oracle_rope.argtypes = [P, P, I, I, I, D, P]
    for name in ("oracle_mla_decode_decompressed", "oracle_mla_decode_absorbed"):
        fn = getattr(lib, name)
        fn.restype = None
        fn.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, I]
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it first when it is missing or stale)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            build(force=False)
            _lib = _declare(ctypes.CDLL(_SO))
    return _lib


def _f32(x) -> np.ndarray:
    """Any CPU array-like (numpy, or a torch tensor of any float dtype) -> contiguous float32.

    bf16 and fp32 values are exactly representable in float32, so nothing is rounded."""
    if hasattr(x, "detach"):  # torch tensor, without importing torch here
        x = x.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check_groups(Hq: int, Hkv: int) -> None:
    if Hkv <= 0 or Hq <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hkv={Hkv} must divide Hq={Hq}")


def gqa_decode(q, k, v, cache_lens, softmax_scale: float = 0.0, lib=None) -> np.ndarray:
    """q [B,Hq,D], k/v [B,T_max,Hkv,D], cache_lens [B] -> out [B,Hq,D] float64."""
    q, k, v, lens = _f32(q), _f32(k), _f32(v), _i32(cache_lens)
    B, Hq, D = q.shape
    _, T_max, Hkv, _ = k.shape
    _check_groups(Hq, Hkv)
    assert k.shape == (B, T_max, Hkv, D) and v.shape == k.shape and lens.shape == (B,)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    (lib or load()).oracle_gqa_decode(_p(q), _p(k), _p(v), _p(lens), _p(out), B, Hq, Hkv, D, T_max,
                                      float(softmax_scale))
    return out


def gqa_prefill_causal(q, k, v, softmax_scale: float = 0.0, rows=None, lib=None) -> np.ndarray:
    """q [B,S,Hq,D], k/v [B,S,Hkv,D] -> out [B,S,Hq,D] float64.

    ``rows``: optional list of query positions to compute (others stay NaN)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    _check_groups(Hq, Hkv)
    assert k.shape == (B, S, Hkv, D) and v.shape == k.shape
    out = np.full((B, S, Hq, D), np.nan, dtype=np.float64)
    r = None if rows is None else _i32(rows)
    (lib or load()).oracle_gqa_prefill_causal(_p(q), _p(k), _p(v), _p(out), B, S, Hq, Hkv, D,
                                              float(softmax_scale), _p(r),
                                              0 if r is None else int(r.size))
    return out


def gqa_prefill_cached(q, k_cache, v_cache, start_pos, q_lens=None, softmax_scale: float = 0.0,
                       lib=None) -> np.ndarray:
    """Causal prefill after a cached prefix: q [B,S,Hq,D] (new tokens), k/v caches
    [B,T_max,Hkv,D] holding the new rows at start_pos[b] .., start_pos [B], q_lens [B] or None
    -> out [B,S,Hq,D] float64 (rows past q_lens[b] zero)."""
    q, k, v, sp = _f32(q), _f32(k_cache), _f32(v_cache), _i32(start_pos)
    B, S, Hq, D = q.shape
    _, T_max, Hkv, _ = k.shape
    _check_groups(Hq, Hkv)
    assert k.shape == (B, T_max, Hkv, D) and v.shape == k.shape and sp.shape == (B,)
    ql = None if q_lens is None else _i32(q_lens)
    assert ql is None or ql.shape == (B,)
    out = np.zeros((B, S, Hq, D), dtype=np.float64)
    (lib or load()).oracle_gqa_prefill_cached(_p(q), _p(k), _p(v), _p(sp), _p(ql), _p(out), B, S, Hq, Hkv, D,
                                              T_max, float(softmax_scale))
    return out


def _mla(fn_name, q_nope, q_rope, w_uk, w_uv, c_kv, k_rope, cache_lens, softmax_scale, bh, lib):
    q_nope, q_rope, w_uk, w_uv = _f32(q_nope), _f32(q_rope), _f32(w_uk), _f32(w_uv)
    c_kv, k_rope, lens = _f32(c_kv), _f32(k_rope), _i32(cache_lens)
    B, H, dn = q_nope.shape
    dR = q_rope.shape[2]
    _, dv, r = w_uv.shape
    T_max = c_kv.shape[1]
    assert q_rope.shape == (B, H, dR) and w_uk.shape == (H, dn, r) and w_uv.shape == (H, dv, r)
    assert c_kv.shape == (B, T_max, r) and k_rope.shape == (B, T_max, dR) and lens.shape == (B,)
    out = np.full((B, H, dv), np.nan, dtype=np.float64)
    bhl = None if bh is None else _i32(bh)
    getattr(lib or load(), fn_name)(_p(q_nope), _p(q_rope), _p(w_uk), _p(w_uv), _p(c_kv), _p(k_rope),
                                    _p(lens), _p(out), B, H, dn, dR, dv, r, T_max,
                                    float(softmax_scale), _p(bhl), 0 if bhl is None else int(bhl.size))
    return out


def mla_decode_decompressed(q_nope, q_rope, w_uk, w_uv, c_kv, k_rope, cache_lens,
                            softmax_scale: float = 0.0, bh=None, lib=None) -> np.ndarray:
    """MLA decode with keys/values rebuilt from the latent.  w_uk [H,dn,r], w_uv [H,dv,r].

    ``bh``: optional flattened (b*H + h) rows to compute (others stay NaN)."""
    return _mla("oracle_mla_decode_decompressed", q_nope, q_rope, w_uk, w_uv, c_kv, k_rope,
                cache_lens, softmax_scale, bh, lib)


def mla_decode_absorbed(q_nope, q_rope, w_uk, w_uv, c_kv, k_rope, cache_lens,
                        softmax_scale: float = 0.0, bh=None, lib=None) -> np.ndarray:
    """MLA decode with W_UK folded into the query and W_UV applied after the weighted sum."""
    return _mla("oracle_mla_decode_absorbed", q_nope, q_rope, w_uk, w_uv, c_kv, k_rope,
                cache_lens, softmax_scale, bh, lib)


def mla_prefill_causal(q_nope, q_rope, w_uk, w_uv, c_kv, k_rope, start_pos=None, q_lens=None,
                       softmax_scale: float = 0.0, lib=None) -> np.ndarray:
    """MLA causal prefill (keys/values rebuilt from the latent): q_nope [B,S,H,dn], q_rope
    [B,S,H,dR], w_uk [H,dn,r], w_uv [H,dv,r], c_kv [B,T_max,r], k_rope [B,T_max,dR] holding the
    new rows at start_pos[b].. (None: 0), q_lens [B] or None (S) -> out [B,S,H,dv] float64."""
    q_nope, q_rope, w_uk, w_uv = _f32(q_nope), _f32(q_rope), _f32(w_uk), _f32(w_uv)
    c_kv, k_rope = _f32(c_kv), _f32(k_rope)
    B, S, H, dn = q_nope.shape
    dR = q_rope.shape[3]
    _, dv, r = w_uv.shape
    T_max = c_kv.shape[1]
    assert q_rope.shape == (B, S, H, dR) and w_uk.shape == (H, dn, r) and w_uv.shape == (H, dv, r)
    assert c_kv.shape == (B, T_max, r) and k_rope.shape == (B, T_max, dR)
    sp = None if start_pos is None else _i32(start_pos)
    ql = None if q_lens is None else _i32(q_lens)
    assert sp is None or sp.shape == (B,)
    assert ql is None or ql.shape == (B,)
    out = np.zeros((B, S, H, dv), dtype=np.float64)
    (lib or load()).oracle_mla_prefill_causal(_p(q_nope), _p(q_rope), _p(w_uk), _p(w_uv), _p(c_kv), _p(k_rope),
                                              _p(sp), _p(ql), _p(out), B, S, H, dn, dR, dv, r, T_max,
                                              float(softmax_scale))
    return out


def cache_append(cache, new, start_pos=None, n_new=None) -> np.ndarray:
    """The cache write of Attention.forward on the MQA & GQA survey page (code section):
    cache[b, P : P + n] = new[b, :n] with P = start_pos[b] clamped to [0, T_max] and n = n_new[b]
    clamped to [0, min(S, T_max - P)].  Returns a new array; the arguments are not modified.
    Works on any dtype (bf16 tensors are compared as raw 16-bit patterns by the tests)."""
    out = np.array(cache, copy=True)
    new = np.asarray(new)
    B, S = new.shape[0], new.shape[1]
    T_max = out.shape[1]
    for b in range(B):
        P = 0 if start_pos is None else min(max(int(start_pos[b]), 0), T_max)
        n = S if n_new is None else int(n_new[b])
        n = max(0, min(n, S, T_max - P))
        out[b, P:P + n] = new[b, :n]
    return out


def gather_pages(pages, block_table, cache_lens, page_size: int | None = None) -> np.ndarray:
    """A paged cache written out as a contiguous one: pages [n_pages, page_size, ...] and
    block_table [B, max_pages] give cache [B, max_pages * page_size, ...] with
    cache[b, t] = pages[block_table[b, t // page_size], t % page_size] for t < cache_lens[b]
    (clamped to [0, max_pages * page_size]) and zeros elsewhere.  The block-table layout is the
    reading of paging taken here (the pages only mention paging as a serving cost); page numbers
    are clamped to [0, n_pages).  Works on any dtype."""
    pages = np.asarray(pages)
    table = np.asarray(block_table, dtype=np.int64)
    ps = pages.shape[1] if page_size is None else int(page_size)
    B, max_pages = table.shape
    T = max_pages * ps
    out = np.zeros((B, T) + pages.shape[2:], dtype=pages.dtype)
    for b in range(B):
        L = min(max(int(cache_lens[b]), 0), T)
        for p in range((L + ps - 1) // ps):  # logical page p holds positions p * ps ..
            page = min(max(int(table[b, p]), 0), pages.shape[0] - 1)
            rows = min(ps, L - p * ps)
            out[b, p * ps:p * ps + rows] = pages[page, :rows]
    return out


def append_pages(pages, block_table, new, start_pos, n_new=None) -> np.ndarray:
    """cache_append over a paged cache: new[b, i] goes to position P + i of sequence b, i.e. row
    (P + i) % page_size of page block_table[b, (P + i) // page_size] (clamped to [0, n_pages)),
    with P = start_pos[b] clamped to [0, T] and n = n_new[b] (default S) clamped to
    [0, min(S, T - P)], T = max_pages * page_size: the block-table layout of gather_pages, read
    in the writing direction.  Returns a new pool; the arguments are not modified.  Any dtype."""
    out = np.array(pages, copy=True)
    new = np.asarray(new)
    table = np.asarray(block_table, dtype=np.int64)
    ps = out.shape[1]
    B, S = new.shape[0], new.shape[1]
    T = table.shape[1] * ps
    for b in range(B):
        P = min(max(int(start_pos[b]), 0), T)
        n = S if n_new is None else int(n_new[b])
        n = max(0, min(n, S, T - P))
        for i in range(n):
            t = P + i
            page = min(max(int(table[b, t // ps]), 0), out.shape[0] - 1)
            out[page, t % ps] = new[b, i]
    return out


def rope(x, positions, base: float = 10000.0, lib=None) -> np.ndarray:
    """Rotary position embedding (oracle_rope in oracle.c): x [..., H, d] with d even, positions
    [...] (one absolute position per token, the leading dimensions of x) -> float64 [..., H, d].
    Pair (x[2j], x[2j+1]) is turned by the angle m * base^(-2j/d)."""
    x = _f32(x)
    H, d = x.shape[-2], x.shape[-1]
    assert d % 2 == 0, "rope width must be even"
    pos = _i32(np.broadcast_to(np.asarray(positions), x.shape[:-2]))
    N = int(np.prod(x.shape[:-2], dtype=np.int64))
    out = np.zeros(x.shape, dtype=np.float64)
    (lib or load()).oracle_rope(_p(x), _p(pos), N, H, d, float(base), _p(out))
    return out


def rope_append(k_new, k_cache=None, q=None, start_pos=None, n_new=None, x_new=None, x_cache=None,
                base: float = 10000.0, lib=None) -> dict:
    """The decode / prefill step before attention in Attention.forward on the MQA & GQA survey page
    (code section): rotate the new tokens' queries and keys (``rope``) at their absolute positions,
    then write the rotated keys (and the second stream x, as given) into the caches at start_pos.

    k_new [B,S,Hk,d], q [B,S,Hq,d] or None, k_cache [B,T_max,Hk,d] or None (then the rotated k_new
    is returned instead), x_new [B,S,...] / x_cache [B,T_max,...] or None.  Token i of sequence b
    sits at position P + i with P = max(start_pos[b], 0) (None: 0); rows i < n = n_new[b] clamped
    to [0, S] (None: S) are rotated, the others are returned unchanged.  The cache writes are
    ``cache_append`` at P with n rows (rows that do not fit in T_max are not stored).
    Returns float64 arrays: "q" (rotated q), "k" (rotated k_new) and, when given, "k_cache" and
    "x_cache" (x_cache keeps the input dtype)."""
    B, S = k_new.shape[0], k_new.shape[1]
    P = np.zeros(B, np.int64) if start_pos is None else np.maximum(np.asarray(start_pos, np.int64), 0)
    n = np.full(B, S, np.int64) if n_new is None else np.clip(np.asarray(n_new, np.int64), 0, S)
    pos = P[:, None] + np.arange(S)[None, :]
    live = np.arange(S)[None, :] < n[:, None]                          # [B, S] rows that are rotated

    def rotate(t):
        t64 = _f32(t).astype(np.float64)
        r = rope(t, pos, base, lib)
        return np.where(live[:, :, None, None], r, t64)

    out = {"k": rotate(k_new)}
    if q is not None:
        out["q"] = rotate(q)
    if k_cache is not None:
        kc = _f32(k_cache) if hasattr(k_cache, "detach") else k_cache  # float64 caches are kept as they are
        out["k_cache"] = cache_append(np.asarray(kc, dtype=np.float64), out["k"], P, n)
    if x_cache is not None:
        out["x_cache"] = cache_append(x_cache, x_new, P, n)
    return out


def int4_to_float(packed, scales=None) -> np.ndarray:
    """Values of packed signed 4-bit codes: packed [..., n] uint8 holds 2n codes, code 2i in the
    low nibble (bits 3..0) of byte i and code 2i + 1 in the high nibble, each a two's-complement
    integer in [-8, 7]; scales (broadcast over the last axis of the result, e.g. one per cached
    row) multiply them.  Returns float64 [..., 2n].  The int4 cache reading: the "MHA, MQA và GQA"
    e-book counts an int4 number as half a byte and gives no layout; this is the plainest one."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    lo, hi = b & 0xF, (b >> 4) & 0xF
    codes = np.stack([lo, hi], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))
    vals = np.where(codes >= 8, codes - 16, codes).astype(np.float64)
    if scales is not None:
        vals = vals * np.asarray(scales, dtype=np.float64)[..., None]
    return vals


def e4m3_to_float(codes, scale: float = 1.0) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (uint8 array) times scale, as float64: sign bit 7,
    exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 is subnormal
    (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN (there is no infinity).  Written from the
    format's definition; the low-precision cache reading of the MHA, MQA and GQA e-book
    (fp8: one byte per cached number) takes this format with one scale per cache."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val * float(scale)


def threads(lib=None) -> int:
    """OpenMP threads the oracle runs with."""
    return int((lib or load()).oracle_threads())
