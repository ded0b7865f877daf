"""Python binding of libattn_mi355x.so: GQA/MQA/MHA decode, causal GQA prefill (also after a
cached prefix), MLA absorbed decode and MLA causal prefill on AMD MI355X (gfx950).

The functions carry the C entry points' names and do argument marshalling only: they check
that the torch tensors are CUDA (HIP) tensors of the right dtype, shape and layout, allocate
the output and workspace with torch when the caller passes none, and call the C ABI on
torch's current stream.  Every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or fails to load, importing the functions
raises.

Build the library with ``python -m mha_mla_kv_amd.build`` (hipcc, gfx950).
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "attn_mi355x.h")

ATTN_F32, ATTN_BF16 = 0, 1
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_GROUPS",
          4: "ATTN_ERR_UNSUPPORTED", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_HIP"}

_lock = threading.Lock()
_lib = None


class AttnError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{fn}: {self.name}: {detail}")


def _declare(lib):
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_abi_version.restype = I
    lib.attn_abi_version.argtypes = []
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [I]
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_decode_gqa_workspace_bytes.restype = Z
    lib.attn_decode_gqa_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.attn_decode_gqa.restype = I
    lib.attn_decode_gqa.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, Z, P]
    lib.attn_prefill_gqa_causal.restype = I
    lib.attn_prefill_gqa_causal.argtypes = [P, P, P, P, I, I, I, I, I, F, I, I, P]
    lib.attn_decode_gqa_paged.restype = I
    lib.attn_decode_gqa_paged.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, I, P, Z, P]
    lib.attn_decode_gqa_paged_append.restype = I
    lib.attn_decode_gqa_paged_append.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, I, P, Z, P]
    lib.attn_decode_gqa_noalloc.restype = I
    lib.attn_decode_gqa_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, I, P]
    lib.attn_decode_gqa_int4kv.restype = I
    lib.attn_decode_gqa_int4kv.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P, Z, P]
    lib.attn_decode_gqa_paged_fp8kv.restype = I
    lib.attn_decode_gqa_paged_fp8kv.argtypes = [P, P, P, F, F, P, P, P, I, I, I, I, I, I, I, F, I, I, P, Z, P]
    lib.attn_decode_gqa_fp8kv.restype = I
    lib.attn_decode_gqa_fp8kv.argtypes = [P, P, P, F, F, P, P, I, I, I, I, I, F, I, I, P, ctypes.c_size_t, P]
    lib.attn_decode_gqa_append_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode_gqa_append_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.attn_decode_gqa_append.restype = I
    lib.attn_decode_gqa_append.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, I, P, ctypes.c_size_t, P]
    lib.attn_rope_append.restype = I
    lib.attn_rope_append.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.attn_cache_append.restype = I
    lib.attn_cache_append.argtypes = [P, P, I, P, P, I, P, P, I, I, I, P]
    lib.attn_prefill_mla_causal.restype = I
    lib.attn_prefill_mla_causal.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, P]
    lib.attn_prefill_gqa_cached.restype = I
    lib.attn_prefill_gqa_cached.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P]
    lib.attn_prefill_gqa_paged.restype = I
    lib.attn_prefill_gqa_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, I, P]
    lib.attn_prefill_gqa_cached_append.restype = I
    lib.attn_prefill_gqa_cached_append.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, P]
    lib.attn_decode_mla_workspace_bytes.restype = Z
    lib.attn_decode_mla_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.attn_decode_mla_supported.restype = I
    lib.attn_decode_mla_supported.argtypes = [I, I, I, I]
    lib.attn_decode_mla_append.restype = I
    lib.attn_decode_mla_append.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, I, P, Z, P]
    lib.attn_decode_mla_absorbed.restype = I
    lib.attn_decode_mla_absorbed.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, I,
                                             P, Z, P]
    lib.attn_decode_mla_fp8kv.restype = I
    lib.attn_decode_mla_fp8kv.argtypes = [P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, I, F, I, I, P, Z, P]
    lib.attn_decode_mla_paged_fp8kv.restype = I
    lib.attn_decode_mla_paged_fp8kv.argtypes = [P, P, P, P, P, F, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, I, P,
                                                Z, P]
    lib.attn_decode_mla_paged.restype = I
    lib.attn_decode_mla_paged.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, I, I,
                                          P, Z, P]
    return lib


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mha_mla_kv_amd.build`")
            _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/attn_mi355x.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, shape=None, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _raise_if(status: int, fn: str):
    if status != 0:
        raise AttnError(status, fn, lib().attn_last_error().decode())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_ws_cache: dict = {}


def _workspace(nbytes: int, device, kind: str) -> torch.Tensor:
    """A zero-filled workspace cached per (device, current stream, entry point), grown as needed.

    The GQA decode leaves its queue counter (the first 4 bytes) zero after every call and
    the MLA decode needs no initialisation, so a cached workspace stays valid for later
    calls of any shape.  Calls on one stream are ordered, so they never use it concurrently."""
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream, kind)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=torch.device("cuda", idx))
        _ws_cache[key] = buf
    return buf


def attn_decode_gqa_workspace_bytes(B: int, Hq: int, Hkv: int, head_dim: int, T_max: int,
                                    split_tokens: int = 0) -> int:
    return int(lib().attn_decode_gqa_workspace_bytes(B, Hq, Hkv, head_dim, T_max, split_tokens))


def attn_decode_gqa(q, k_cache, v_cache, cache_lens, out=None, softmax_scale: float = 0.0,
                    out_dtype=torch.float32, split_tokens: int = 0, workspace=None):
    """out[b,h] = softmax_t(scale q[b,h].k[b,t,g]) v[b,t,g], t < cache_lens[b], g = h // (Hq/Hkv).

    q [B,Hq,D], k_cache/v_cache [B,T_max,Hkv,D] (same dtype, fp32 or bf16), cache_lens [B] int32,
    out [B,Hq,D] of out_dtype.  A caller-provided workspace (uint8) must have been zero-filled
    before its first use (its first 4 bytes are the work-queue counter); calls leave it so.
    Returns out."""
    _check(q, "q")
    B, Hq, D = q.shape
    _check(k_cache, "k_cache", dtype=q.dtype)
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError(f"k_cache must be [B={B}, T_max, Hkv, {D}] (got {tuple(k_cache.shape)})")
    T_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(v_cache, "v_cache", shape=k_cache.shape, dtype=q.dtype)
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, Hq, D))
    need = attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T_max, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q.device, "gqa")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_gqa(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens), _ptr(out), B, Hq,
                               Hkv, D, T_max, float(softmax_scale), _dt(q), _dt(out), int(split_tokens),
                               _ptr(workspace), workspace.numel(), _stream(q.device))
    _raise_if(st, "attn_decode_gqa")
    return out


def attn_decode_gqa_int4kv(q, k_codes, v_codes, k_scales, v_scales, cache_lens, out=None,
                           softmax_scale: float = 0.0, out_dtype=torch.float32, split_tokens: int = 0,
                           workspace=None):
    """attn_decode_gqa over caches of packed signed 4-bit codes with one fp32 scale per row: element
    2i of a row is the low nibble of byte i, 2i + 1 the high nibble, each times the row's scale.

    q [B,Hq,128] bf16, k_codes/v_codes [B,Hkv,T_max,64] uint8 and k_scales/v_scales [B,Hkv,T_max]
    float32 (head-major), cache_lens [B] int32.  Returns out [B,Hq,128] of out_dtype."""
    _check(q, "q", dtype=torch.bfloat16)
    B, Hq, D = q.shape
    _check(k_codes, "k_codes", dtype=torch.uint8)
    if k_codes.dim() != 4 or k_codes.shape[0] != B or k_codes.shape[3] * 2 != D:
        raise ValueError(f"k_codes must be [B={B}, Hkv, T_max, {D // 2}] (got {tuple(k_codes.shape)})")
    Hkv, T_max = k_codes.shape[1], k_codes.shape[2]
    _check(v_codes, "v_codes", shape=k_codes.shape, dtype=torch.uint8)
    _check(k_scales, "k_scales", shape=(B, Hkv, T_max), dtype=torch.float32)
    _check(v_scales, "v_scales", shape=(B, Hkv, T_max), dtype=torch.float32)
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, Hq, D))
    need = attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T_max, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q.device, "gqa")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_gqa_int4kv(_ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scales), _ptr(v_scales),
                                      _ptr(cache_lens), _ptr(out), B, Hq, Hkv, D, T_max, float(softmax_scale),
                                      _dt(out), int(split_tokens), _ptr(workspace), workspace.numel(),
                                      _stream(q.device))
    _raise_if(st, "attn_decode_gqa_int4kv")
    return out


def attn_decode_gqa_paged(q, k_pages, v_pages, block_table, cache_lens, out=None, softmax_scale: float = 0.0,
                          out_dtype=torch.float32, split_tokens: int = 0, workspace=None):
    """attn_decode_gqa over paged caches: position t of sequence b is row t % page_size of page
    block_table[b, t // page_size] of the pools.

    q [B,Hq,D] bf16, k_pages/v_pages [n_pages, page_size, Hkv, D] bf16, block_table
    [B, max_pages_per_seq] int32, cache_lens [B] int32 (clamped to page_size * max_pages_per_seq).
    Returns out [B,Hq,D] of out_dtype."""
    _check(q, "q")
    B, Hq, D = q.shape
    _check(k_pages, "k_pages", dtype=q.dtype)
    if k_pages.dim() != 4 or k_pages.shape[3] != D:
        raise ValueError(f"k_pages must be [n_pages, page_size, Hkv, {D}] (got {tuple(k_pages.shape)})")
    n_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _check(v_pages, "v_pages", shape=k_pages.shape, dtype=q.dtype)
    _check(block_table, "block_table", dtype=torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages_per_seq] (got {tuple(block_table.shape)})")
    max_pages = block_table.shape[1]
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, Hq, D))
    need = attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, page_size * max_pages, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q.device, "gqa")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_gqa_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(cache_lens),
                                     _ptr(out), B, Hq, Hkv, D, page_size, n_pages, max_pages, float(softmax_scale),
                                     _dt(q), _dt(out), int(split_tokens), _ptr(workspace), workspace.numel(),
                                     _stream(q.device))
    _raise_if(st, "attn_decode_gqa_paged")
    return out


def attn_decode_gqa_paged_append(q, k_new, v_new, k_pages, v_pages, block_table, cache_lens, out=None,
                                 softmax_scale: float = 0.0, out_dtype=torch.float32, split_tokens: int = 0,
                                 workspace=None):
    """One decode step with the new token over paged caches: writes k_new/v_new [B,Hkv,D] at
    position cache_lens[b] (row cache_lens[b] % page_size of page block_table[b, cache_lens[b] //
    page_size]) and attends q [B,Hq,D] to the cache_lens[b] cached positions plus the new one.
    Pools and table as attn_decode_gqa_paged; cache_lens is not changed.  Returns out [B,Hq,D]."""
    _check(q, "q")
    B, Hq, D = q.shape
    _check(k_pages, "k_pages", dtype=q.dtype)
    if k_pages.dim() != 4 or k_pages.shape[3] != D:
        raise ValueError(f"k_pages must be [n_pages, page_size, Hkv, {D}] (got {tuple(k_pages.shape)})")
    n_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _check(v_pages, "v_pages", shape=k_pages.shape, dtype=q.dtype)
    _check(k_new, "k_new", shape=(B, Hkv, D), dtype=q.dtype)
    _check(v_new, "v_new", shape=(B, Hkv, D), dtype=q.dtype)
    _check(block_table, "block_table", dtype=torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages_per_seq] (got {tuple(block_table.shape)})")
    max_pages = block_table.shape[1]
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, Hq, D))
    need = attn_decode_gqa_append_workspace_bytes(B, Hq, Hkv, D, page_size * max_pages, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q.device, "gqa_append")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_gqa_paged_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
                                            _ptr(block_table), _ptr(cache_lens), _ptr(out), B, Hq, Hkv, D, page_size,
                                            n_pages, max_pages, float(softmax_scale), _dt(q), _dt(out),
                                            int(split_tokens), _ptr(workspace), workspace.numel(), _stream(q.device))
    _raise_if(st, "attn_decode_gqa_paged_append")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_NOALLOC_SCRATCH_BYTES


def attn_decode_gqa_noalloc(q, k_cache, v_cache, cache_lens, out, softmax_scale: float = 0.0,
                            split_tokens: int = 0):
    """attn_decode_gqa without a workspace: the library's per-device scratch holds the partial
    results (sizes needing more than NOALLOC_SCRATCH_BYTES are rejected).  The caller passes
    out [B,Hq,D] (fp32 or bf16); nothing is allocated.  Calls that overlap on one device race.
    Returns out."""
    _check(q, "q")
    B, Hq, D = q.shape
    _check(k_cache, "k_cache", dtype=q.dtype)
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError(f"k_cache must be [B={B}, T_max, Hkv, {D}] (got {tuple(k_cache.shape)})")
    T_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(v_cache, "v_cache", shape=k_cache.shape, dtype=q.dtype)
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    _check(out, "out", shape=(B, Hq, D))
    st = lib().attn_decode_gqa_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_lens), _ptr(out), B, Hq,
                                       Hkv, D, T_max, float(softmax_scale), _dt(q), _dt(out), int(split_tokens),
                                       _stream(q.device))
    _raise_if(st, "attn_decode_gqa_noalloc")
    return out


def attn_decode_gqa_fp8kv(q, k_cache, v_cache, k_scale: float, v_scale: float, cache_lens, out=None,
                          softmax_scale: float = 0.0, out_dtype=torch.float32, split_tokens: int = 0, workspace=None):
    """GQA decode over FP8 E4M3 caches (torch.float8_e4m3fn, [B,T_max,Hkv,128]) holding K/k_scale
    and V/v_scale; q [B,Hq,128] bf16.  Returns out [B,Hq,128]."""
    _check(q, "q", dtype=torch.bfloat16)
    B, Hq, D = q.shape
    _check(k_cache, "k_cache", dtype=torch.float8_e4m3fn)
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError(f"k_cache must be [B={B}, T_max, Hkv, {D}] (got {tuple(k_cache.shape)})")
    T_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(v_cache, "v_cache", shape=k_cache.shape, dtype=torch.float8_e4m3fn)
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, Hq, D))
    need = attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T_max, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q.device, "gqa")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_gqa_fp8kv(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale), float(v_scale),
                                     _ptr(cache_lens), _ptr(out), B, Hq, Hkv, D, T_max, float(softmax_scale),
                                     _dt(out), int(split_tokens), _ptr(workspace), workspace.numel(),
                                     _stream(q.device))
    _raise_if(st, "attn_decode_gqa_fp8kv")
    return out


def attn_decode_gqa_paged_fp8kv(q, k_pages, v_pages, k_scale: float, v_scale: float, block_table, cache_lens,
                                out=None, softmax_scale: float = 0.0, out_dtype=torch.float32, split_tokens: int = 0,
                                workspace=None):
    """attn_decode_gqa_fp8kv over paged FP8 caches: k_pages/v_pages [n_pages, page_size, Hkv, 128]
    torch.float8_e4m3fn holding K/k_scale and V/v_scale, block_table [B, max_pages_per_seq]
    int32 as attn_decode_gqa_paged; q [B,Hq,128] bf16.  Returns out [B,Hq,128]."""
    _check(q, "q", dtype=torch.bfloat16)
    B, Hq, D = q.shape
    _check(k_pages, "k_pages", dtype=torch.float8_e4m3fn)
    if k_pages.dim() != 4 or k_pages.shape[3] != D:
        raise ValueError(f"k_pages must be [n_pages, page_size, Hkv, {D}] (got {tuple(k_pages.shape)})")
    n_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _check(v_pages, "v_pages", shape=k_pages.shape, dtype=torch.float8_e4m3fn)
    _check(block_table, "block_table", dtype=torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages_per_seq] (got {tuple(block_table.shape)})")
    max_pages = block_table.shape[1]
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, Hq, D))
    need = attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, page_size * max_pages, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q.device, "gqa")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_gqa_paged_fp8kv(_ptr(q), _ptr(k_pages), _ptr(v_pages), float(k_scale), float(v_scale),
                                           _ptr(block_table), _ptr(cache_lens), _ptr(out), B, Hq, Hkv, D, page_size,
                                           n_pages, max_pages, float(softmax_scale), _dt(out), int(split_tokens),
                                           _ptr(workspace), workspace.numel(), _stream(q.device))
    _raise_if(st, "attn_decode_gqa_paged_fp8kv")
    return out


def attn_decode_gqa_append_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, T_max: int,
                                           split_tokens: int = 0) -> int:
    return int(lib().attn_decode_gqa_append_workspace_bytes(B, Hq, Hkv, D, T_max, split_tokens))


def attn_decode_gqa_append(q, k_new, v_new, k_cache, v_cache, cache_lens, out=None, softmax_scale: float = 0.0,
                           out_dtype=torch.float32, split_tokens: int = 0, workspace=None):
    """One decode step with the new token: writes k_new/v_new [B,Hkv,D] into the caches at row
    cache_lens[b] and attends q [B,Hq,D] to the cache_lens[b] cached rows plus the new one.
    cache_lens is not changed.  Returns out [B,Hq,D]."""
    _check(q, "q")
    B, Hq, D = q.shape
    _check(k_cache, "k_cache", dtype=q.dtype)
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError(f"k_cache must be [B={B}, T_max, Hkv, {D}] (got {tuple(k_cache.shape)})")
    T_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(v_cache, "v_cache", shape=k_cache.shape, dtype=q.dtype)
    _check(k_new, "k_new", shape=(B, Hkv, D), dtype=q.dtype)
    _check(v_new, "v_new", shape=(B, Hkv, D), dtype=q.dtype)
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, Hq, D))
    need = attn_decode_gqa_append_workspace_bytes(B, Hq, Hkv, D, T_max, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q.device, "gqa_append")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_gqa_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(cache_lens), _ptr(out), B, Hq, Hkv, D, T_max, float(softmax_scale), _dt(q),
                                      _dt(out), int(split_tokens), _ptr(workspace), workspace.numel(),
                                      _stream(q.device))
    _raise_if(st, "attn_decode_gqa_append")
    return out


def attn_prefill_gqa_causal(q, k, v, out=None, softmax_scale: float = 0.0, out_dtype=torch.bfloat16):
    """Causal prefill: out[b,i,h] = softmax_{j<=i}(scale q[b,i,h].k[b,j,g]) v[b,j,g].

    q [B,S,Hq,D], k/v [B,S,Hkv,D] bf16; out [B,S,Hq,D] of out_dtype.  Returns out."""
    _check(q, "q")
    B, S, Hq, D = q.shape
    _check(k, "k", dtype=q.dtype)
    if k.dim() != 4 or k.shape[0] != B or k.shape[1] != S or k.shape[3] != D:
        raise ValueError(f"k must be [B={B}, S={S}, Hkv, {D}] (got {tuple(k.shape)})")
    Hkv = k.shape[2]
    _check(v, "v", shape=k.shape, dtype=q.dtype)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, S, Hq, D))
    st = lib().attn_prefill_gqa_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, Hq, Hkv, D,
                                       float(softmax_scale), _dt(q), _dt(out), _stream(q.device))
    _raise_if(st, "attn_prefill_gqa_causal")
    return out


def attn_prefill_gqa_cached(q, k_cache, v_cache, start_pos, q_lens=None, out=None, softmax_scale: float = 0.0,
                            out_dtype=torch.bfloat16):
    """Causal prefill after a cached prefix: new token i of sequence b sits at position
    start_pos[b] + i and attends cache rows j <= start_pos[b] + i; rows i >= q_lens[b] are zeros.

    q [B,S,Hq,D] bf16 (new tokens), k_cache/v_cache [B,T_max,Hkv,D] bf16 already holding the new
    rows at start_pos[b]..; start_pos, q_lens [B] int32 (q_lens None: S).  Returns out."""
    _check(q, "q")
    B, S, Hq, D = q.shape
    _check(k_cache, "k_cache", dtype=q.dtype)
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError(f"k_cache must be [B={B}, T_max, Hkv, {D}] (got {tuple(k_cache.shape)})")
    T_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(v_cache, "v_cache", shape=k_cache.shape, dtype=q.dtype)
    _check(start_pos, "start_pos", shape=(B,), dtype=torch.int32)
    if q_lens is not None:
        _check(q_lens, "q_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, S, Hq, D))
    st = lib().attn_prefill_gqa_cached(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(start_pos),
                                       _ptr(q_lens), _ptr(out), B, S, Hq, Hkv, D,
                                       T_max, float(softmax_scale), _dt(q), _dt(out), _stream(q.device))
    _raise_if(st, "attn_prefill_gqa_cached")
    return out


def attn_prefill_gqa_paged(q, k_pages, v_pages, block_table, start_pos, q_lens=None, out=None,
                           softmax_scale: float = 0.0, out_dtype=torch.bfloat16):
    """attn_prefill_gqa_cached over a paged cache: position t of sequence b is row t % page_size
    of page block_table[b, t // page_size] of the pools (which already hold the new rows).

    q [B,S,Hq,D] bf16, k_pages/v_pages [n_pages, page_size, Hkv, D] bf16, block_table
    [B, max_pages_per_seq] int32, start_pos, q_lens [B] int32 (q_lens None: S).  Returns out."""
    _check(q, "q")
    B, S, Hq, D = q.shape
    _check(k_pages, "k_pages", dtype=q.dtype)
    if k_pages.dim() != 4 or k_pages.shape[3] != D:
        raise ValueError(f"k_pages must be [n_pages, page_size, Hkv, {D}] (got {tuple(k_pages.shape)})")
    n_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    _check(v_pages, "v_pages", shape=k_pages.shape, dtype=q.dtype)
    _check(block_table, "block_table", dtype=torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages_per_seq] (got {tuple(block_table.shape)})")
    max_pages = block_table.shape[1]
    _check(start_pos, "start_pos", shape=(B,), dtype=torch.int32)
    if q_lens is not None:
        _check(q_lens, "q_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, S, Hq, D))
    st = lib().attn_prefill_gqa_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(start_pos),
                                      _ptr(q_lens), _ptr(out), B, S, Hq, Hkv, D, page_size, n_pages, max_pages,
                                      float(softmax_scale), _dt(q), _dt(out), _stream(q.device))
    _raise_if(st, "attn_prefill_gqa_paged")
    return out


def attn_prefill_gqa_cached_append(q, k_new, v_new, k_cache, v_cache, start_pos, q_lens=None, out=None,
                                   softmax_scale: float = 0.0, out_dtype=torch.bfloat16):
    """Causal prefill after a cached prefix that also appends the new rows, in one launch: new token
    i of sequence b attends cache rows j < start_pos[b] and new rows j <= i, and k_new / v_new rows
    i < q_lens[b] are written into the caches at start_pos[b] + i.

    q [B,S,Hq,D] bf16, k_new/v_new [B,S,Hkv,D] bf16, k_cache/v_cache [B,T_max,Hkv,D] bf16 (updated in
    place), start_pos, q_lens [B] int32 (q_lens None: S).  Returns out."""
    _check(q, "q")
    B, S, Hq, D = q.shape
    _check(k_cache, "k_cache", dtype=q.dtype)
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError(f"k_cache must be [B={B}, T_max, Hkv, {D}] (got {tuple(k_cache.shape)})")
    T_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    _check(v_cache, "v_cache", shape=k_cache.shape, dtype=q.dtype)
    _check(k_new, "k_new", shape=(B, S, Hkv, D), dtype=q.dtype)
    _check(v_new, "v_new", shape=(B, S, Hkv, D), dtype=q.dtype)
    _check(start_pos, "start_pos", shape=(B,), dtype=torch.int32)
    if q_lens is not None:
        _check(q_lens, "q_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, S, Hq, D), dtype=out_dtype, device=q.device)
    _check(out, "out", shape=(B, S, Hq, D))
    st = lib().attn_prefill_gqa_cached_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                              _ptr(start_pos), _ptr(q_lens), _ptr(out), B, S, Hq, Hkv, D, T_max,
                                              float(softmax_scale), _dt(q), _dt(out), _stream(q.device))
    _raise_if(st, "attn_prefill_gqa_cached_append")
    return out


def attn_prefill_mla_causal(q_nope, q_rope, w_uk, w_uv, c_kv, k_rope, start_pos=None, q_lens=None, out=None,
                            softmax_scale: float = 0.0, out_dtype=torch.bfloat16):
    """MLA causal prefill over the latent cache: new token i of sequence b (position start_pos[b] + i)
    attends cache rows j <= start_pos[b] + i with keys [W_UK c, k_rope] and values W_UV c.

    q_nope [B,S,H,dn], q_rope [B,S,H,dR], w_uk [H,dn,r], w_uv [H,dv,r], c_kv [B,T_max,r],
    k_rope [B,T_max,dR] bf16 (the new rows already in the cache); start_pos, q_lens [B] int32 or
    None.  Returns out [B,S,H,dv]."""
    _check(q_nope, "q_nope")
    B, S, H, dn = q_nope.shape
    _check(q_rope, "q_rope", dtype=q_nope.dtype)
    if q_rope.dim() != 4 or tuple(q_rope.shape[:3]) != (B, S, H):
        raise ValueError(f"q_rope must be [B={B}, S={S}, H={H}, rope_dim] (got {tuple(q_rope.shape)})")
    dR = q_rope.shape[3]
    _check(w_uk, "w_uk", dtype=q_nope.dtype)
    if w_uk.dim() != 3 or w_uk.shape[0] != H or w_uk.shape[1] != dn:
        raise ValueError(f"w_uk must be [H={H}, {dn}, kv_lora_rank] (got {tuple(w_uk.shape)})")
    r = w_uk.shape[2]
    _check(w_uv, "w_uv", dtype=q_nope.dtype)
    if w_uv.dim() != 3 or w_uv.shape[0] != H or w_uv.shape[2] != r:
        raise ValueError(f"w_uv must be [H={H}, v_head_dim, {r}] (got {tuple(w_uv.shape)})")
    dv = w_uv.shape[1]
    _check(c_kv, "c_kv", dtype=q_nope.dtype)
    if c_kv.dim() != 3 or c_kv.shape[0] != B or c_kv.shape[2] != r:
        raise ValueError(f"c_kv must be [B={B}, T_max, {r}] (got {tuple(c_kv.shape)})")
    T_max = c_kv.shape[1]
    _check(k_rope, "k_rope", shape=(B, T_max, dR), dtype=q_nope.dtype)
    if start_pos is not None:
        _check(start_pos, "start_pos", shape=(B,), dtype=torch.int32)
    if q_lens is not None:
        _check(q_lens, "q_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, S, H, dv), dtype=out_dtype, device=q_nope.device)
    _check(out, "out", shape=(B, S, H, dv))
    st = lib().attn_prefill_mla_causal(_ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(c_kv), _ptr(k_rope),
                                       _ptr(start_pos), _ptr(q_lens), _ptr(out), B, S, H, dn, dR, dv, r, T_max,
                                       float(softmax_scale), _dt(q_nope), _dt(out), _stream(q_nope.device))
    _raise_if(st, "attn_prefill_mla_causal")
    return out


def attn_rope_append(k_new, k_cache=None, q=None, start_pos=None, n_new=None, x_new=None, x_cache=None,
                     rope_base: float = 10000.0):
    """Rotary position embedding of the new tokens fused with the cache write, in one launch: token
    i of sequence b sits at position max(start_pos[b], 0) + i; q (in place) and k_new are rotated
    pair by pair (angle m * rope_base^(-2j/d)); the rotated keys go to k_cache and the x_new rows,
    as given, to x_cache at those positions (rows past T_max are not stored).  k_cache None: k_new
    is rotated in place.  Rows i >= n_new[b] are left alone.

    k_new [B,S,Hk,d] (or [B,S,d]: Hk = 1), q [B,S,Hq,d] or None, k_cache [B,T_max,Hk,d] (or
    [B,T_max,d]) or None, all bf16 or all fp32; x_new [B,S,...] and x_cache [B,T_max,...] of any
    dtype with equal row sizes, or None; start_pos, n_new [B] int32 or None.  Returns None."""
    _check(k_new, "k_new")
    if k_new.dim() not in (3, 4):
        raise ValueError(f"k_new must be [B, S, Hk, d] or [B, S, d] (got {tuple(k_new.shape)})")
    B, S, d = k_new.shape[0], k_new.shape[1], k_new.shape[-1]
    Hk = k_new.shape[2] if k_new.dim() == 4 else 1
    Hq, T_max, xb = 0, 0, 0
    if q is not None:
        _check(q, "q", dtype=k_new.dtype)
        if q.dim() != 4 or tuple(q.shape[:2]) != (B, S) or q.shape[3] != d:
            raise ValueError(f"q must be [B={B}, S={S}, Hq, {d}] (got {tuple(q.shape)})")
        Hq = q.shape[2]
    if k_cache is not None:
        _check(k_cache, "k_cache", dtype=k_new.dtype)
        if k_cache.dim() != k_new.dim() or k_cache.shape[0] != B or tuple(k_cache.shape[2:]) != tuple(k_new.shape[2:]):
            raise ValueError(f"k_cache must be [B, T_max] + {tuple(k_new.shape[2:])} (got {tuple(k_cache.shape)})")
        T_max = k_cache.shape[1]
    if (x_new is None) != (x_cache is None):
        raise ValueError("x_new and x_cache go together")
    if x_new is not None:
        _check(x_new, "x_new", dtype=x_new.dtype)
        _check(x_cache, "x_cache", dtype=x_new.dtype)
        if k_cache is None or tuple(x_new.shape[:2]) != (B, S) or x_cache.shape[0] != B or \
                x_cache.shape[1] != T_max or tuple(x_cache.shape[2:]) != tuple(x_new.shape[2:]):
            raise ValueError("x_new must be [B, S, ...] and x_cache [B, T_max, ...] (with k_cache)")
        xb = x_new[0, 0].numel() * x_new.element_size()
    for t, name in ((start_pos, "start_pos"), (n_new, "n_new")):
        if t is not None:
            _check(t, name, shape=(B,), dtype=torch.int32)
    st = lib().attn_rope_append(_ptr(q), _ptr(k_new), _ptr(k_cache), _ptr(x_new), _ptr(x_cache), _ptr(start_pos),
                                _ptr(n_new), B, S, Hq, Hk, d, xb, T_max, float(rope_base), _dt(k_new),
                                _stream(k_new.device))
    _raise_if(st, "attn_rope_append")


def attn_cache_append(new_a, cache_a, new_b=None, cache_b=None, start_pos=None, n_new=None):
    """cache_a[b, start_pos[b] + i] = new_a[b, i] for i < n_new[b] (and the same for the b pair):
    K and V caches [B, T_max, Hkv, D] with new rows [B, S, Hkv, D], or the MLA caches c_kv
    [B, T_max, r] and k_rope [B, T_max, dR].  start_pos, n_new [B] int32 or None (0, S)."""
    _check(new_a, "new_a")
    B, S = new_a.shape[0], new_a.shape[1]
    _check(cache_a, "cache_a", dtype=new_a.dtype)
    if cache_a.dim() != new_a.dim() or cache_a.shape[0] != B or tuple(cache_a.shape[2:]) != tuple(new_a.shape[2:]):
        raise ValueError(f"cache_a must be [B={B}, T_max, {tuple(new_a.shape[2:])}] (got {tuple(cache_a.shape)})")
    T_max = cache_a.shape[1]
    rb_a = new_a[0, 0].numel() * new_a.element_size()
    rb_b = 0
    if new_b is not None:
        _check(new_b, "new_b")
        _check(cache_b, "cache_b", dtype=new_b.dtype)
        if new_b.shape[0] != B or new_b.shape[1] != S or cache_b.shape[0] != B or cache_b.shape[1] != T_max or \
                tuple(cache_b.shape[2:]) != tuple(new_b.shape[2:]):
            raise ValueError("new_b / cache_b must be [B, S, ...] / [B, T_max, ...] like the a pair")
        rb_b = new_b[0, 0].numel() * new_b.element_size()
    if start_pos is not None:
        _check(start_pos, "start_pos", shape=(B,), dtype=torch.int32)
    if n_new is not None:
        _check(n_new, "n_new", shape=(B,), dtype=torch.int32)
    st = lib().attn_cache_append(_ptr(new_a), _ptr(cache_a), rb_a, _ptr(new_b), _ptr(cache_b), rb_b, _ptr(start_pos),
                                 _ptr(n_new), B, S, T_max, _stream(new_a.device))
    _raise_if(st, "attn_cache_append")


def attn_decode_mla_workspace_bytes(B: int, H: int, kv_lora_rank: int, rope_dim: int, T_max: int,
                                    split_tokens: int = 0) -> int:
    return int(lib().attn_decode_mla_workspace_bytes(B, H, kv_lora_rank, rope_dim, T_max, split_tokens))


def attn_decode_mla_supported(H: int, kv_lora_rank: int, rope_dim: int, dtype=torch.bfloat16) -> bool:
    return bool(lib().attn_decode_mla_supported(H, kv_lora_rank, rope_dim,
                                                ATTN_BF16 if dtype == torch.bfloat16 else ATTN_F32))


def attn_decode_mla_absorbed(q_nope, q_rope, w_uk, w_uv, c_kv, k_rope, cache_lens, out=None,
                             softmax_scale: float = 0.0, out_dtype=torch.float32, split_tokens: int = 0,
                             workspace=None):
    """MLA decode with W_UK absorbed into the query and W_UV applied after the weighted sum.

    q_nope [B,H,dn], q_rope [B,H,dR], w_uk [H,dn,r], w_uv [H,dv,r], c_kv [B,T_max,r],
    k_rope [B,T_max,dR] (all bf16), cache_lens [B] int32 -> out [B,H,dv] of out_dtype."""
    _check(q_nope, "q_nope")
    B, H, dn = q_nope.shape
    dt = q_nope.dtype
    _check(q_rope, "q_rope", dtype=dt)
    if q_rope.dim() != 3 or q_rope.shape[:2] != (B, H):
        raise ValueError(f"q_rope must be [B={B}, H={H}, rope_dim] (got {tuple(q_rope.shape)})")
    dR = q_rope.shape[2]
    _check(w_uk, "w_uk", dtype=dt)
    if w_uk.dim() != 3 or w_uk.shape[:2] != (H, dn):
        raise ValueError(f"w_uk must be [H={H}, nope_head_dim={dn}, kv_lora_rank] (got {tuple(w_uk.shape)})")
    r = w_uk.shape[2]
    _check(w_uv, "w_uv", dtype=dt)
    if w_uv.dim() != 3 or w_uv.shape[0] != H or w_uv.shape[2] != r:
        raise ValueError(f"w_uv must be [H={H}, v_head_dim, kv_lora_rank={r}] (got {tuple(w_uv.shape)})")
    dv = w_uv.shape[1]
    _check(c_kv, "c_kv", dtype=dt)
    if c_kv.dim() != 3 or c_kv.shape[0] != B or c_kv.shape[2] != r:
        raise ValueError(f"c_kv must be [B={B}, T_max, kv_lora_rank={r}] (got {tuple(c_kv.shape)})")
    T_max = c_kv.shape[1]
    _check(k_rope, "k_rope", shape=(B, T_max, dR), dtype=dt)
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, H, dv), dtype=out_dtype, device=q_nope.device)
    _check(out, "out", shape=(B, H, dv))
    need = attn_decode_mla_workspace_bytes(B, H, r, dR, T_max, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q_nope.device, "mla")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_mla_absorbed(_ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(c_kv),
                                        _ptr(k_rope), _ptr(cache_lens), _ptr(out), B, H, dn, dR, dv, r, T_max,
                                        float(softmax_scale), _dt(q_nope), _dt(out), int(split_tokens),
                                        _ptr(workspace), workspace.numel(), _stream(q_nope.device))
    _raise_if(st, "attn_decode_mla_absorbed")
    return out


def attn_decode_mla_fp8kv(q_nope, q_rope, w_uk, w_uv, c_kv, c_scale: float, k_rope, cache_lens, out=None,
                          softmax_scale: float = 0.0, out_dtype=torch.float32, split_tokens: int = 0,
                          workspace=None):
    """attn_decode_mla_absorbed over a latent cache of OCP FP8 E4M3 codes: c_kv [B,T_max,r]
    (torch.float8_e4m3fn or uint8 codes) times c_scale; k_rope [B,T_max,dR] bf16; q_nope [B,H,dn],
    q_rope [B,H,dR], w_uk [H,dn,r], w_uv [H,dv,r] bf16; cache_lens [B] int32 -> out [B,H,dv]."""
    _check(q_nope, "q_nope", dtype=torch.bfloat16)
    B, H, dn = q_nope.shape
    _check(q_rope, "q_rope", dtype=torch.bfloat16)
    if q_rope.dim() != 3 or q_rope.shape[:2] != (B, H):
        raise ValueError(f"q_rope must be [B={B}, H={H}, rope_dim] (got {tuple(q_rope.shape)})")
    dR = q_rope.shape[2]
    _check(w_uk, "w_uk", dtype=torch.bfloat16)
    if w_uk.dim() != 3 or w_uk.shape[:2] != (H, dn):
        raise ValueError(f"w_uk must be [H={H}, nope_head_dim={dn}, kv_lora_rank] (got {tuple(w_uk.shape)})")
    r = w_uk.shape[2]
    _check(w_uv, "w_uv", dtype=torch.bfloat16)
    if w_uv.dim() != 3 or w_uv.shape[0] != H or w_uv.shape[2] != r:
        raise ValueError(f"w_uv must be [H={H}, v_head_dim, kv_lora_rank={r}] (got {tuple(w_uv.shape)})")
    dv = w_uv.shape[1]
    _check(c_kv, "c_kv")
    if c_kv.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise ValueError(f"c_kv must hold E4M3 codes (float8_e4m3fn or uint8), got {c_kv.dtype}")
    if c_kv.dim() != 3 or c_kv.shape[0] != B or c_kv.shape[2] != r:
        raise ValueError(f"c_kv must be [B={B}, T_max, kv_lora_rank={r}] (got {tuple(c_kv.shape)})")
    T_max = c_kv.shape[1]
    _check(k_rope, "k_rope", shape=(B, T_max, dR), dtype=torch.bfloat16)
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, H, dv), dtype=out_dtype, device=q_nope.device)
    _check(out, "out", shape=(B, H, dv))
    need = attn_decode_mla_workspace_bytes(B, H, r, dR, T_max, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q_nope.device, "mla")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_mla_fp8kv(_ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(c_kv),
                                     float(c_scale), _ptr(k_rope), _ptr(cache_lens), _ptr(out), B, H, dn, dR, dv, r,
                                     T_max, float(softmax_scale), _dt(out), int(split_tokens), _ptr(workspace),
                                     workspace.numel(), _stream(q_nope.device))
    _raise_if(st, "attn_decode_mla_fp8kv")
    return out


def attn_decode_mla_paged_fp8kv(q_nope, q_rope, w_uk, w_uv, c_pages, c_scale: float, k_rope_pages, block_table,
                                cache_lens, out=None, softmax_scale: float = 0.0, out_dtype=torch.float32,
                                split_tokens: int = 0, workspace=None):
    """attn_decode_mla_fp8kv over paged latent caches: c_pages [n_pages, page_size, r] of E4M3 codes
    (torch.float8_e4m3fn or uint8) times c_scale, k_rope_pages [n_pages, page_size, dR] bf16,
    block_table [B, max_pages_per_seq] int32 as attn_decode_mla_paged; q_nope [B,H,dn], q_rope
    [B,H,dR], w_uk [H,dn,r], w_uv [H,dv,r] bf16; cache_lens [B] int32 -> out [B,H,dv]."""
    _check(q_nope, "q_nope", dtype=torch.bfloat16)
    B, H, dn = q_nope.shape
    _check(q_rope, "q_rope", dtype=torch.bfloat16)
    if q_rope.dim() != 3 or q_rope.shape[:2] != (B, H):
        raise ValueError(f"q_rope must be [B={B}, H={H}, rope_dim] (got {tuple(q_rope.shape)})")
    dR = q_rope.shape[2]
    _check(w_uk, "w_uk", dtype=torch.bfloat16)
    if w_uk.dim() != 3 or w_uk.shape[:2] != (H, dn):
        raise ValueError(f"w_uk must be [H={H}, nope_head_dim={dn}, kv_lora_rank] (got {tuple(w_uk.shape)})")
    r = w_uk.shape[2]
    _check(w_uv, "w_uv", dtype=torch.bfloat16)
    if w_uv.dim() != 3 or w_uv.shape[0] != H or w_uv.shape[2] != r:
        raise ValueError(f"w_uv must be [H={H}, v_head_dim, kv_lora_rank={r}] (got {tuple(w_uv.shape)})")
    dv = w_uv.shape[1]
    _check(c_pages, "c_pages")
    if c_pages.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise ValueError(f"c_pages must hold E4M3 codes (float8_e4m3fn or uint8), got {c_pages.dtype}")
    if c_pages.dim() != 3 or c_pages.shape[2] != r:
        raise ValueError(f"c_pages must be [n_pages, page_size, kv_lora_rank={r}] (got {tuple(c_pages.shape)})")
    n_pages, page_size = c_pages.shape[0], c_pages.shape[1]
    _check(k_rope_pages, "k_rope_pages", shape=(n_pages, page_size, dR), dtype=torch.bfloat16)
    _check(block_table, "block_table", dtype=torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages_per_seq] (got {tuple(block_table.shape)})")
    max_pages = block_table.shape[1]
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, H, dv), dtype=out_dtype, device=q_nope.device)
    _check(out, "out", shape=(B, H, dv))
    need = attn_decode_mla_workspace_bytes(B, H, r, dR, page_size * max_pages, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q_nope.device, "mla")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_mla_paged_fp8kv(_ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(c_pages),
                                           float(c_scale), _ptr(k_rope_pages), _ptr(block_table), _ptr(cache_lens),
                                           _ptr(out), B, H, dn, dR, dv, r, page_size, n_pages, max_pages,
                                           float(softmax_scale), _dt(out), int(split_tokens), _ptr(workspace),
                                           workspace.numel(), _stream(q_nope.device))
    _raise_if(st, "attn_decode_mla_paged_fp8kv")
    return out


def attn_decode_mla_paged(q_nope, q_rope, w_uk, w_uv, c_pages, k_rope_pages, block_table, cache_lens, out=None,
                          softmax_scale: float = 0.0, out_dtype=torch.float32, split_tokens: int = 0,
                          workspace=None):
    """attn_decode_mla_absorbed over paged latent caches: position t of sequence b is row
    t % page_size of page block_table[b, t // page_size] of the pools.

    q_nope [B,H,dn], q_rope [B,H,dR], w_uk [H,dn,r], w_uv [H,dv,r], c_pages [n_pages, page_size, r],
    k_rope_pages [n_pages, page_size, dR] (all bf16), block_table [B, max_pages_per_seq] int32,
    cache_lens [B] int32 (clamped to page_size * max_pages_per_seq) -> out [B,H,dv] of out_dtype."""
    _check(q_nope, "q_nope")
    B, H, dn = q_nope.shape
    dt = q_nope.dtype
    _check(q_rope, "q_rope", dtype=dt)
    if q_rope.dim() != 3 or q_rope.shape[:2] != (B, H):
        raise ValueError(f"q_rope must be [B={B}, H={H}, rope_dim] (got {tuple(q_rope.shape)})")
    dR = q_rope.shape[2]
    _check(w_uk, "w_uk", dtype=dt)
    if w_uk.dim() != 3 or w_uk.shape[:2] != (H, dn):
        raise ValueError(f"w_uk must be [H={H}, nope_head_dim={dn}, kv_lora_rank] (got {tuple(w_uk.shape)})")
    r = w_uk.shape[2]
    _check(w_uv, "w_uv", dtype=dt)
    if w_uv.dim() != 3 or w_uv.shape[0] != H or w_uv.shape[2] != r:
        raise ValueError(f"w_uv must be [H={H}, v_head_dim, kv_lora_rank={r}] (got {tuple(w_uv.shape)})")
    dv = w_uv.shape[1]
    _check(c_pages, "c_pages", dtype=dt)
    if c_pages.dim() != 3 or c_pages.shape[2] != r:
        raise ValueError(f"c_pages must be [n_pages, page_size, kv_lora_rank={r}] (got {tuple(c_pages.shape)})")
    n_pages, page_size = c_pages.shape[0], c_pages.shape[1]
    _check(k_rope_pages, "k_rope_pages", shape=(n_pages, page_size, dR), dtype=dt)
    _check(block_table, "block_table", dtype=torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}, max_pages_per_seq] (got {tuple(block_table.shape)})")
    max_pages = block_table.shape[1]
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, H, dv), dtype=out_dtype, device=q_nope.device)
    _check(out, "out", shape=(B, H, dv))
    need = attn_decode_mla_workspace_bytes(B, H, r, dR, page_size * max_pages, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q_nope.device, "mla")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_mla_paged(_ptr(q_nope), _ptr(q_rope), _ptr(w_uk), _ptr(w_uv), _ptr(c_pages),
                                     _ptr(k_rope_pages), _ptr(block_table), _ptr(cache_lens), _ptr(out), B, H, dn,
                                     dR, dv, r, page_size, n_pages, max_pages, float(softmax_scale), _dt(q_nope),
                                     _dt(out), int(split_tokens), _ptr(workspace), workspace.numel(),
                                     _stream(q_nope.device))
    _raise_if(st, "attn_decode_mla_paged")
    return out


def attn_decode_mla_append(q_nope, q_rope, c_new, k_rope_new, w_uk, w_uv, c_kv, k_rope, cache_lens, out=None,
                           softmax_scale: float = 0.0, out_dtype=torch.float32, split_tokens: int = 0, workspace=None):
    """One MLA decode step with the new token: writes c_new [B,r] and k_rope_new [B,dR] into the
    caches at row cache_lens[b] and attends to the cache_lens[b] cached rows plus the new one.
    Other arguments as attn_decode_mla_absorbed; cache_lens is not changed.  Returns out [B,H,dv]."""
    _check(q_nope, "q_nope")
    B, H, dn = q_nope.shape
    dt = q_nope.dtype
    _check(c_kv, "c_kv", dtype=dt)
    if c_kv.dim() != 3 or c_kv.shape[0] != B:
        raise ValueError(f"c_kv must be [B={B}, T_max, kv_lora_rank] (got {tuple(c_kv.shape)})")
    T_max, r = c_kv.shape[1], c_kv.shape[2]
    _check(k_rope, "k_rope", dtype=dt)
    if k_rope.dim() != 3 or k_rope.shape[:2] != (B, T_max):
        raise ValueError(f"k_rope must be [B={B}, T_max={T_max}, rope_dim] (got {tuple(k_rope.shape)})")
    dR = k_rope.shape[2]
    _check(q_rope, "q_rope", shape=(B, H, dR), dtype=dt)
    _check(c_new, "c_new", shape=(B, r), dtype=dt)
    _check(k_rope_new, "k_rope_new", shape=(B, dR), dtype=dt)
    _check(w_uk, "w_uk", shape=(H, dn, r), dtype=dt)
    _check(w_uv, "w_uv", dtype=dt)
    if w_uv.dim() != 3 or w_uv.shape[0] != H or w_uv.shape[2] != r:
        raise ValueError(f"w_uv must be [H={H}, v_head_dim, kv_lora_rank={r}] (got {tuple(w_uv.shape)})")
    dv = w_uv.shape[1]
    _check(cache_lens, "cache_lens", shape=(B,), dtype=torch.int32)
    if out is None:
        out = torch.empty((B, H, dv), dtype=out_dtype, device=q_nope.device)
    _check(out, "out", shape=(B, H, dv))
    need = attn_decode_mla_workspace_bytes(B, H, r, dR, T_max, split_tokens)
    if workspace is None:
        workspace = _workspace(need, q_nope.device, "mla")
    _check(workspace, "workspace", dtype=torch.uint8)
    st = lib().attn_decode_mla_append(_ptr(q_nope), _ptr(q_rope), _ptr(c_new), _ptr(k_rope_new), _ptr(w_uk),
                                      _ptr(w_uv), _ptr(c_kv), _ptr(k_rope), _ptr(cache_lens), _ptr(out), B, H, dn, dR,
                                      dv, r, T_max, float(softmax_scale), _dt(q_nope), _dt(out), int(split_tokens),
                                      _ptr(workspace), workspace.numel(), _stream(q_nope.device))
    _raise_if(st, "attn_decode_mla_append")
    return out


__all__ = ["attn_decode_gqa", "attn_decode_gqa_paged", "attn_decode_gqa_paged_fp8kv", "attn_decode_gqa_paged_append", "attn_decode_mla_paged", "attn_decode_mla_fp8kv", "attn_decode_mla_paged_fp8kv", "attn_prefill_gqa_paged", "attn_decode_gqa_int4kv", "attn_decode_gqa_workspace_bytes", "attn_decode_gqa_noalloc", "NOALLOC_SCRATCH_BYTES", "attn_decode_gqa_append", "attn_decode_gqa_fp8kv",
           "attn_decode_gqa_append_workspace_bytes", "attn_prefill_gqa_causal", "attn_prefill_gqa_cached", "attn_prefill_gqa_cached_append",
           "attn_prefill_mla_causal", "attn_cache_append", "attn_rope_append",
           "attn_decode_mla_absorbed", "attn_decode_mla_append", "attn_decode_mla_workspace_bytes", "attn_decode_mla_supported",
           "AttnError", "lib", "header_functions", "LIB_PATH", "ATTN_F32", "ATTN_BF16"]
