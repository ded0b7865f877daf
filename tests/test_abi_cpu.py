"""The C-ABI library loads, exports every declared symbol, and rejects invalid arguments on the host.

Validation runs before any HIP call, so every error status is reachable without a GPU.  The
calls below pass fake (never dereferenced) device pointers and are each built to fail
validation; they are skipped where a GPU is visible so that a validation bug can never turn one
of them into a real launch."""
import ctypes

import pytest
import torch

import mha_mla_kv_amd as attn

OK, NULL, SHAPE, GROUPS, UNSUP, WS, HIP = range(7)
F32, BF16 = attn.ATTN_F32, attn.ATTN_BF16
FAKE = ctypes.c_void_p(0x100000)      # 256-byte aligned, never dereferenced
FAKE_MIS = ctypes.c_void_p(0x100008)  # 8-byte aligned only

no_gpu_only = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer validation runs without a GPU")


def test_library_loads_and_exports_every_declared_symbol():
    lib = attn.lib()
    names = attn.header_functions()
    for required in ("attn_decode_gqa", "attn_prefill_gqa_causal", "attn_prefill_gqa_cached",
                     "attn_decode_mla_absorbed", "attn_prefill_mla_causal", "attn_cache_append",
                     "attn_decode_gqa_append", "attn_decode_gqa_fp8kv"):
        assert required in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/attn_mi355x.h but not exported"
    assert lib.attn_abi_version() == 1


def test_status_strings():
    lib = attn.lib()
    for s in range(7):
        assert lib.attn_status_string(s)
    assert lib.attn_status_string(3) == b"KV head count does not divide query head count"


def test_workspace_sizes():
    al = lambda x: (x + 255) // 256 * 256
    # chunks of 512 at the Llama-3-8B decode shape: queue counter (256 bytes), lse [slots*n_rep],
    # partials [slots*n_rep*D] fp32 with slots = B*Hkv*ceil(T/512), each piece 256-byte aligned
    B, Hq, Hkv, D, T = 32, 32, 8, 128, 8192
    slots = B * Hkv * (T // 512)
    n = attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T, 512)
    assert n == 256 + al(slots * 4 * 4) + al(slots * 4 * D * 4)
    # split 0: the library picks B*Hkv*T/4096 = 512 positions per block here
    slots = B * Hkv * (T // 512)
    assert attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T, 0) == 256 + al(slots * 4 * 4) + al(slots * 4 * D * 4)
    # a single chunk per sequence needs no partials
    assert attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, 512, 512) == 256
    assert attn.attn_decode_gqa_workspace_bytes(0, 32, 8, 128, 8192, 0) == 0
    assert attn.attn_decode_gqa_workspace_bytes(1, 32, 8, 128, 8192, 100) == 0  # split not a multiple of 64
    assert attn.attn_decode_mla_workspace_bytes(64, 8, 128, 48, 4096, 0) > 0
    # MLA with fixed chunks of 512: per-sequence done counters [B] uint32, lse
    # [B*n_splits*H] fp32, partials [B*n_splits*H, r] fp32
    B, H, r, dR, T = 64, 8, 128, 48, 4096
    rows = B * H * (T // 512)
    assert attn.attn_decode_mla_workspace_bytes(B, H, r, dR, T, 512) == al(B * 4) + al(rows * 4) + al(rows * r * 4)
    # split 0: chunks of at least 256 positions, about one per compute unit of a
    # 256-unit device over B * T (1024 here), whatever device is current
    rows = B * H * (T // 1024)
    assert attn.attn_decode_mla_workspace_bytes(B, H, r, dR, T, 0) == al(B * 4) + al(rows * 4) + al(rows * r * 4)
    assert attn.attn_decode_mla_supported(8, 128, 48)
    assert not attn.attn_decode_mla_supported(8, 100, 48)
    assert not attn.attn_decode_mla_supported(8, 128, 48, torch.float32)


def _gqa(lib, q=FAKE, k=FAKE, v=FAKE, lens=FAKE, out=FAKE, B=2, Hq=8, Hkv=2, D=128, T=64, scale=0.0,
         ind=BF16, outd=F32, split=0, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = 1 << 30
    return lib.attn_decode_gqa(q, k, v, lens, out, B, Hq, Hkv, D, T, scale, ind, outd, split, ws, wsb, None)


@no_gpu_only
def test_decode_gqa_validation():
    lib = attn.lib()
    assert _gqa(lib, q=None) == NULL
    assert _gqa(lib, lens=None) == NULL
    assert _gqa(lib, B=0) == SHAPE
    assert _gqa(lib, T=-1) == SHAPE
    assert _gqa(lib, B=70000) == SHAPE
    assert _gqa(lib, Hq=32, Hkv=3) == GROUPS      # 32 heads into 3 groups: an error, not rounded
    assert b"remainder 2" in lib.attn_last_error()
    assert _gqa(lib, Hq=32, Hkv=6) == GROUPS
    assert _gqa(lib, split=100) == SHAPE
    assert _gqa(lib, B=1025, T=64 * 70000, split=64) == SHAPE  # one workgroup per unit: > 65535 chunks
    assert _gqa(lib, ind=7) == UNSUP
    assert _gqa(lib, D=80) == UNSUP
    assert _gqa(lib, Hq=128, Hkv=1) == UNSUP     # n_rep 128 not built
    assert _gqa(lib, ind=F32, Hq=64, Hkv=2) == UNSUP  # fp32 path: n_rep <= 16
    assert _gqa(lib, q=FAKE_MIS) == UNSUP
    assert _gqa(lib, ws=None) == WS
    assert _gqa(lib, wsb=16) == WS
    assert b"workspace" in lib.attn_last_error()
    assert _gqa(lib, ws=FAKE_MIS) == WS


@no_gpu_only
def test_decode_append_validation():
    lib = attn.lib()

    def f(**kw):
        return lib.attn_decode_gqa_append(FAKE, kw.get("kn", FAKE), kw.get("vn", FAKE), FAKE, FAKE, FAKE, FAKE,
                                          kw.get("B", 2), 8, 2, 128, kw.get("T", 64), 0.0, BF16, F32, 0,
                                          kw.get("ws", FAKE), kw.get("wsb", 1 << 30), None)
    assert f(kn=None) == NULL
    assert f(vn=FAKE_MIS) == UNSUP
    assert f(B=0) == SHAPE
    assert f(ws=None) == WS
    assert f(wsb=300) == WS   # partials are needed even for a single chunk
    # a single chunk per sequence still needs partial slots in the fused step
    plain = attn.attn_decode_gqa_workspace_bytes(2, 8, 2, 128, 64, 0)
    assert plain == 256 and attn.attn_decode_gqa_append_workspace_bytes(2, 8, 2, 128, 64, 0) > plain


@no_gpu_only
def test_fp8_decode_validation():
    lib = attn.lib()

    def f(**kw):
        return lib.attn_decode_gqa_fp8kv(FAKE, FAKE, FAKE, kw.get("ks", 0.01), kw.get("vs", 0.01), FAKE, FAKE, 2, 8, 2,
                                         kw.get("D", 128), 64, 0.0, F32, 0, FAKE, 1 << 30, None)
    assert f(ks=0.0) == SHAPE
    assert f(vs=float("inf")) == SHAPE
    assert f(vs=float("nan")) == SHAPE
    assert f(D=64) == UNSUP


@no_gpu_only
def test_prefill_validation():
    lib = attn.lib()
    f = lambda **kw: lib.attn_prefill_gqa_causal(kw.get("q", FAKE), FAKE, FAKE, kw.get("out", FAKE), kw.get("B", 1),
                                                 kw.get("S", 16), kw.get("Hq", 8), kw.get("Hkv", 2), kw.get("D", 128),
                                                 0.0, kw.get("ind", BF16), BF16, None)
    assert f(q=None) == NULL
    assert f(S=0) == SHAPE
    assert f(Hq=8, Hkv=3) == GROUPS
    assert f(ind=F32) == UNSUP
    assert f(D=80) == UNSUP
    assert f(out=FAKE_MIS) == UNSUP


@no_gpu_only
def test_cached_prefill_validation():
    lib = attn.lib()

    def f(**kw):
        return lib.attn_prefill_gqa_cached(kw.get("q", FAKE), FAKE, FAKE, kw.get("sp", FAKE), kw.get("ql", FAKE),
                                           FAKE, kw.get("B", 2), kw.get("S", 16), kw.get("Hq", 8), kw.get("Hkv", 2),
                                           kw.get("D", 128), kw.get("T", 64), 0.0, kw.get("ind", BF16), BF16, None)
    assert f(sp=None) == NULL
    assert f(q=None) == NULL
    assert f(T=0) == SHAPE
    assert f(S=0) == SHAPE
    assert f(Hq=8, Hkv=3) == GROUPS
    assert f(ind=F32) == UNSUP
    assert f(D=80) == UNSUP
    assert f(q=FAKE_MIS) == UNSUP


@no_gpu_only
def test_cached_append_prefill_validation():
    lib = attn.lib()

    def f(**kw):
        return lib.attn_prefill_gqa_cached_append(FAKE, kw.get("kn", FAKE), kw.get("vn", FAKE), FAKE, FAKE,
                                                  kw.get("sp", FAKE), None, FAKE, kw.get("B", 2), 16, 8, 2,
                                                  kw.get("D", 128), kw.get("T", 64), 0.0, BF16, BF16, None)
    assert f(sp=None) == NULL
    assert f(kn=None) == NULL
    assert f(vn=None) == NULL
    assert f(T=0) == SHAPE
    assert f(B=0) == SHAPE
    assert f(D=80) == UNSUP
    assert f(vn=FAKE_MIS) == UNSUP


@no_gpu_only
def test_mla_prefill_validation():
    lib = attn.lib()

    def f(**kw):
        return lib.attn_prefill_mla_causal(kw.get("qn", FAKE), FAKE, FAKE, FAKE, kw.get("c", FAKE), FAKE, None, None,
                                           FAKE, kw.get("B", 2), kw.get("S", 16), kw.get("H", 8), kw.get("dn", 96),
                                           kw.get("dR", 48), kw.get("dv", 96), kw.get("r", 128), kw.get("T", 64), 0.0,
                                           kw.get("ind", BF16), BF16, None)
    assert f(qn=None) == NULL
    assert f(T=0) == SHAPE
    assert f(S=0) == SHAPE
    assert f(r=256) == UNSUP
    assert f(dR=64) == UNSUP
    assert f(dn=128) == UNSUP
    assert f(ind=F32) == UNSUP
    assert f(c=FAKE_MIS) == UNSUP
    assert b"not built" in lib.attn_last_error() or b"aligned" in lib.attn_last_error()


@no_gpu_only
def test_cache_append_validation():
    lib = attn.lib()

    def f(**kw):
        return lib.attn_cache_append(kw.get("na", FAKE), kw.get("ca", FAKE), kw.get("ra", 256), kw.get("nb", FAKE),
                                     kw.get("cb", FAKE), kw.get("rb", 256), None, None, kw.get("B", 2), kw.get("S", 4),
                                     kw.get("T", 64), None)
    assert f(na=None) == NULL
    assert f(nb=None) == NULL
    assert f(B=0) == SHAPE
    assert f(T=0) == SHAPE
    assert f(ra=0) == SHAPE
    assert f(ra=100) == UNSUP
    assert f(rb=8) == UNSUP
    assert f(ca=FAKE_MIS) == UNSUP


@no_gpu_only
def test_mla_validation():
    lib = attn.lib()

    def f(**kw):
        return lib.attn_decode_mla_absorbed(kw.get("qn", FAKE), FAKE, FAKE, FAKE, kw.get("c", FAKE), FAKE, FAKE, FAKE,
                                            kw.get("B", 2), kw.get("H", 8), kw.get("dn", 96), kw.get("dR", 48),
                                            kw.get("dv", 96), kw.get("r", 128), kw.get("T", 64), 0.0,
                                            kw.get("ind", BF16), F32, kw.get("split", 0), kw.get("ws", FAKE),
                                            kw.get("wsb", 1 << 30), None)
    assert f(qn=None) == NULL
    assert f(T=0) == SHAPE
    assert f(split=65) == SHAPE
    assert f(H=17) == UNSUP
    assert f(r=100) == UNSUP
    assert f(dR=40) == UNSUP
    assert f(ind=F32) == UNSUP
    assert f(dn=300) == UNSUP
    assert f(dn=100) == UNSUP   # nope_head_dim: a multiple of 8
    assert f(dv=90) == UNSUP    # v_head_dim: a multiple of 16
    assert f(c=FAKE_MIS) == UNSUP
    assert f(ws=None) == WS
    assert f(wsb=10) == WS


def test_python_binding_rejects_cpu_tensors():
    q = torch.zeros(1, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 16, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.attn_decode_gqa(q, k, k, torch.zeros(1, dtype=torch.int32))


@no_gpu_only
def test_noalloc_decode_validation():
    lib = attn.lib()

    def f(q=FAKE, B=2, Hq=8, Hkv=2, D=128, T=64, split=0):
        return lib.attn_decode_gqa_noalloc(q, FAKE, FAKE, FAKE, FAKE, B, Hq, Hkv, D, T, 0.0, BF16, F32, split, None)
    assert f(q=None) == NULL
    assert f(B=0) == SHAPE
    assert f(Hq=32, Hkv=3) == GROUPS
    assert f(D=80) == UNSUP
    assert f(split=100) == SHAPE
    # sizes whose workspace exceeds the built-in scratch are rejected before anything runs
    B, Hq, Hkv, D, T = 64, 64, 64, 128, 65536
    assert attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T, 0) > attn.NOALLOC_SCRATCH_BYTES
    assert f(B=B, Hq=Hq, Hkv=Hkv, D=D, T=T) == WS
    assert b"scratch" in lib.attn_last_error()
    # the Llama-3-8B decode shape fits
    assert attn.attn_decode_gqa_workspace_bytes(32, 32, 8, 128, 8192, 0) <= attn.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_header():
    import re
    text = open(attn.HEADER_PATH).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == attn.NOALLOC_SCRATCH_BYTES


@no_gpu_only
def test_mla_append_validation():
    lib = attn.lib()

    def f(cn=FAKE, kn=FAKE, **kw):
        return lib.attn_decode_mla_append(FAKE, FAKE, cn, kn, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("B", 2), 8, 96,
                                          48, kw.get("dv", 96), 128, 64, 0.0, BF16, F32, 0, kw.get("ws", FAKE),
                                          kw.get("wsb", 1 << 30), None)
    assert f(cn=None) == NULL
    assert f(kn=None) == NULL
    assert f(kn=FAKE_MIS) == UNSUP
    assert f(B=0) == SHAPE
    assert f(dv=90) == UNSUP
    assert f(ws=None) == WS


@no_gpu_only
def test_rope_append_validation():
    lib = attn.lib()

    def f(k=FAKE, kc=FAKE, x=FAKE, xc=FAKE, **kw):
        return lib.attn_rope_append(kw.get("q", FAKE), k, kc, x, xc, None, None, kw.get("B", 2), 4, 8, 2,
                                    kw.get("d", 128), kw.get("xb", 512), kw.get("T", 64), kw.get("base", 10000.0),
                                    BF16, None)
    assert f(k=None) == NULL
    assert f(x=None) == NULL
    assert f(kc=None) == NULL          # x goes only with a key cache
    assert f(kc=None, xb=0, T=0) == HIP       # valid: reaches the launch, which fails without a GPU
    assert f(B=0) == SHAPE
    assert f(T=0) == SHAPE
    assert f(base=0.0) == SHAPE
    assert f(base=float("inf")) == SHAPE
    assert f(d=12) == UNSUP
    assert f(d=2048) == UNSUP
    assert f(xb=24) == UNSUP
    assert f(q=FAKE_MIS) == UNSUP


@no_gpu_only
def test_paged_decode_validation():
    lib = attn.lib()

    def f(tb=FAKE, **kw):
        return lib.attn_decode_gqa_paged(FAKE, FAKE, FAKE, tb, FAKE, FAKE, 2, 32, 8, kw.get("D", 128),
                                         kw.get("ps", 64), kw.get("np", 100), kw.get("mp", 16), 0.0,
                                         kw.get("ind", BF16), F32, kw.get("split", 0), FAKE, 1 << 30, None)
    assert f(tb=None) == NULL
    assert f(ps=0) == SHAPE
    assert f(np=0) == SHAPE
    assert f(mp=0) == SHAPE
    assert f(ps=48) == UNSUP
    assert f(ind=F32) == UNSUP
    assert f(split=2048) == UNSUP
    assert f(D=80) == UNSUP


@no_gpu_only
def test_paged_fp8_decode_validation():
    lib = attn.lib()

    def f(tb=FAKE, **kw):
        return lib.attn_decode_gqa_paged_fp8kv(FAKE, FAKE, FAKE, kw.get("ks", 0.01), kw.get("vs", 0.01), tb, FAKE, FAKE,
                                               2, 32, 8, kw.get("D", 128), kw.get("ps", 64), kw.get("np", 100),
                                               kw.get("mp", 16), 0.0, F32, kw.get("split", 0), FAKE, 1 << 30, None)
    assert f(tb=None) == NULL
    assert f(ks=0.0) == SHAPE
    assert f(vs=float("nan")) == SHAPE
    assert f(ps=0) == SHAPE
    assert f(ps=48) == UNSUP
    assert f(split=2048) == UNSUP
    assert f(D=96) == UNSUP          # fp8 caches: head_dim 128 only


@no_gpu_only
def test_paged_decode_step_validation():
    lib = attn.lib()

    def f(tb=FAKE, kn=FAKE, vn=FAKE, **kw):
        return lib.attn_decode_gqa_paged_append(FAKE, kn, vn, FAKE, FAKE, tb, FAKE, FAKE, 2, 32, 8, kw.get("D", 128),
                                                kw.get("ps", 64), kw.get("np", 100), kw.get("mp", 16), 0.0,
                                                kw.get("ind", BF16), F32, kw.get("split", 0), FAKE, 1 << 30, None)
    assert f(tb=None) == NULL
    assert f(kn=None) == NULL
    assert f(vn=None) == NULL
    assert f(kn=FAKE_MIS) == UNSUP  # new rows not 16-byte aligned
    assert f(ps=0) == SHAPE
    assert f(np=0) == SHAPE
    assert f(mp=0) == SHAPE
    assert f(ps=48) == UNSUP
    assert f(ind=F32) == UNSUP
    assert f(split=2048) == UNSUP
    assert f(D=80) == UNSUP


@no_gpu_only
def test_mla_paged_decode_validation():
    lib = attn.lib()

    def f(tb=FAKE, **kw):
        return lib.attn_decode_mla_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, tb, FAKE, FAKE, 2, 8, 96, 48, 96, 128,
                                         kw.get("ps", 16), kw.get("np", 100), kw.get("mp", 64), 0.0, BF16, F32,
                                         kw.get("split", 0), FAKE, 1 << 30, None)
    assert f(tb=None) == NULL
    assert f(ps=0) == SHAPE
    assert f(np=0) == SHAPE
    assert f(mp=0) == SHAPE
    assert f(ps=24) == UNSUP
    assert f(split=4096) == UNSUP  # 4096 / 16 + 2 pages per chunk, more than 128
    assert f(split=2048) == UNSUP  # 130
    assert f(ps=32, split=4096) == UNSUP


@no_gpu_only
def test_mla_paged_fp8_decode_validation():
    lib = attn.lib()

    def f(tb=FAKE, **kw):
        return lib.attn_decode_mla_paged_fp8kv(FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("cs", 0.01), FAKE, tb, FAKE, FAKE,
                                               2, 8, 96, 48, 96, 128, kw.get("ps", 16), kw.get("np", 100),
                                               kw.get("mp", 64), 0.0, F32, kw.get("split", 0), FAKE, 1 << 30, None)
    assert f(tb=None) == NULL
    assert f(cs=0.0) == SHAPE
    assert f(cs=float("inf")) == SHAPE
    assert f(ps=0) == SHAPE
    assert f(ps=24) == UNSUP
    assert f(split=2048) == UNSUP  # 2048 / 16 + 2 pages per chunk, more than 128


@no_gpu_only
def test_paged_prefill_validation():
    lib = attn.lib()

    def f(tb=FAKE, sp=FAKE, **kw):
        return lib.attn_prefill_gqa_paged(FAKE, FAKE, FAKE, tb, sp, None, FAKE, 2, 64, 8, 2, kw.get("D", 128),
                                          kw.get("ps", 64), kw.get("np", 10), kw.get("mp", 8), 0.0, BF16, BF16, None)
    assert f(tb=None) == NULL
    assert f(sp=None) == NULL
    assert f(ps=0) == SHAPE
    assert f(np=0) == SHAPE
    assert f(mp=0) == SHAPE
    assert f(ps=32) == UNSUP
    assert f(ps=96) == UNSUP
    assert f(D=80) == UNSUP


@no_gpu_only
def test_mla_fp8_decode_validation():
    lib = attn.lib()

    def f(cs=0.01, **kw):
        return lib.attn_decode_mla_fp8kv(FAKE, FAKE, FAKE, FAKE, kw.get("c", FAKE), cs, FAKE, FAKE, FAKE, 2, 8, 96, 48,
                                         96, kw.get("r", 128), 256, 0.0, F32, 0, FAKE, 1 << 30, None)
    assert f(cs=0.0) == SHAPE
    assert f(cs=-1.0) == SHAPE
    assert f(cs=float("nan")) == SHAPE
    assert f(cs=float("inf")) == SHAPE
    assert f(c=None) == NULL
    assert f(c=FAKE_MIS) == UNSUP
    assert f(r=96) == UNSUP


@no_gpu_only
def test_int4_decode_validation():
    lib = attn.lib()

    def f(ks=FAKE, vs=FAKE, **kw):
        return lib.attn_decode_gqa_int4kv(FAKE, kw.get("kc", FAKE), FAKE, ks, vs, FAKE, FAKE, 2, 32, 8,
                                          kw.get("D", 128), 64, 0.0, F32, 0, FAKE, 1 << 30, None)
    assert f(ks=None) == NULL
    assert f(vs=None) == NULL
    assert f(D=96) == UNSUP
    assert f(ks=ctypes.c_void_p(0x100002)) == UNSUP
    assert f(kc=FAKE_MIS) == UNSUP
