"""The compute entry points captured in a HIP graph (torch.cuda.graph) and replayed.

Each call is launched with a caller-provided workspace, so it allocates nothing; the GQA
decode's work-queue counter is returned to zero by the call itself, so every replay starts
from the same state.  Replays are interleaved with unrelated eager work and synchronisations,
and every replay must reproduce the eager result bit for bit (the result of a call does not
depend on which workgroup takes which unit)."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _graph_matches_eager(call, out, replays=4):
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as capture requires
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    scratch = torch.ones(1 << 20, device="cuda")
    for i in range(replays):
        out.fill_(float("nan"))
        scratch.mul_(1.5).add_(i)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
    return eager


def test_gqa_decode_graph_replay():
    import mha_mla_kv_amd as attn
    B, Hq, Hkv, D, T = 4, 32, 8, 128, 3000
    inp = {k: v.cuda() for k, v in synth.gqa_decode_inputs(B, Hq, Hkv, D, T, [3000, 17, 2048, 0], seed=7).items()}
    print(f"[case] gqa decode graph B={B} Hq={Hq} Hkv={Hkv} D={D} T={T}", flush=True)
    ws = torch.zeros(attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, D, device="cuda")
    eager = _graph_matches_eager(
        lambda: attn.attn_decode_gqa(inp["q"], inp["k"], inp["v"], inp["cache_lens"], out=out, workspace=ws), out)
    assert torch.isfinite(eager).all()
    assert int(ws[:4].view(torch.int32)[0]) == 0  # the queue counter is back to zero


def test_mla_decode_graph_replay():
    import mha_mla_kv_amd as attn
    B, H, dn, dR, dv, r, T = 3, 8, 96, 48, 96, 128, 1500
    inp = {k: v.cuda() for k, v in synth.mla_decode_inputs(B, H, dn, dR, dv, r, T, [1500, 1, 700], seed=8).items()}
    print(f"[case] mla decode graph B={B} H={H} r={r} dR={dR} T={T}", flush=True)
    ws = torch.zeros(attn.attn_decode_mla_workspace_bytes(B, H, r, dR, T, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, H, dv, device="cuda")
    keys = ("q_nope", "q_rope", "w_uk", "w_uv", "c_kv", "k_rope", "cache_lens")
    eager = _graph_matches_eager(
        lambda: attn.attn_decode_mla_absorbed(*(inp[k] for k in keys), out=out, workspace=ws), out)
    assert torch.isfinite(eager).all()


def test_prefill_graph_replay():
    import mha_mla_kv_amd as attn
    B, S, Hq, Hkv, D = 1, 700, 16, 4, 128
    inp = {k: v.cuda() for k, v in synth.gqa_prefill_inputs(B, S, Hq, Hkv, D, seed=9).items()}
    print(f"[case] prefill graph B={B} S={S} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
    out = torch.empty_like(inp["q"])
    eager = _graph_matches_eager(lambda: attn.attn_prefill_gqa_causal(inp["q"], inp["k"], inp["v"], out=out), out)
    assert torch.isfinite(eager.float()).all()


def test_cached_prefill_graph_replay():
    import mha_mla_kv_amd as attn
    B, S, Hq, Hkv, D, T = 2, 300, 16, 4, 128, 1200
    inp = {k: v.cuda() for k, v in synth.gqa_prefill_cached_inputs(B, S, Hq, Hkv, D, T, [700, 64], [300, 111],
                                                                   seed=10).items()}
    print(f"[case] cached prefill graph B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} T={T}", flush=True)
    out = torch.empty_like(inp["q"])
    eager = _graph_matches_eager(lambda: attn.attn_prefill_gqa_cached(inp["q"], inp["k"], inp["v"], inp["start_pos"],
                                                                      inp["q_lens"], out=out), out)
    assert torch.isfinite(eager.float()).all()
    assert not eager[1, 111:].any()  # rows past the chunk are zeros


def test_mla_prefill_graph_replay():
    import mha_mla_kv_amd as attn
    B, S, H, T = 2, 200, 8, 600
    inp = {k: v.cuda() for k, v in synth.mla_prefill_inputs(B, S, H, 96, 48, 96, 128, T, [300, 0], [200, 77],
                                                            seed=11).items()}
    print(f"[case] mla prefill graph B={B} S={S} H={H} T={T}", flush=True)
    out = torch.empty(B, S, H, 96, dtype=torch.bfloat16, device="cuda")
    keys = ("q_nope", "q_rope", "w_uk", "w_uv", "c_kv", "k_rope")
    eager = _graph_matches_eager(lambda: attn.attn_prefill_mla_causal(*(inp[k] for k in keys), inp["start_pos"],
                                                                      inp["q_lens"], out=out), out)
    assert torch.isfinite(eager.float()).all()
    assert not eager[1, 77:].any()


def test_decode_step_and_fp8_decode_graph_replay():
    """The decode step with the new token (its cache write repeats the same bytes on every replay)
    and the decode over FP8 caches, captured and replayed."""
    import mha_mla_kv_amd as attn
    B, Hq, Hkv, D, T = 4, 32, 8, 128, 2000
    inp = {k: v.cuda() for k, v in synth.gqa_decode_inputs(B, Hq, Hkv, D, T, [1999, 0, 700, 64], seed=12).items()}
    g = torch.Generator().manual_seed(12)
    k_new, v_new = (torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16).cuda() for _ in range(2))
    print(f"[case] decode step graph B={B} Hq={Hq} Hkv={Hkv} T={T}", flush=True)
    ws = torch.zeros(attn.attn_decode_gqa_append_workspace_bytes(B, Hq, Hkv, D, T, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, D, device="cuda")
    eager = _graph_matches_eager(lambda: attn.attn_decode_gqa_append(inp["q"], k_new, v_new, inp["k"], inp["v"],
                                                                     inp["cache_lens"], out=out, workspace=ws), out)
    assert torch.isfinite(eager).all()
    f8 = synth.gqa_decode_fp8_inputs(B, Hq, Hkv, D, T, [1999, 0, 700, 64], seed=13)
    fk, fv, fl, fq = f8["k"].cuda(), f8["v"].cuda(), f8["cache_lens"].cuda(), f8["q"].cuda()
    print("[case] fp8 decode graph", flush=True)
    ws8 = torch.zeros(attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T, 0), dtype=torch.uint8, device="cuda")
    out8 = torch.empty(B, Hq, D, device="cuda")
    eager8 = _graph_matches_eager(lambda: attn.attn_decode_gqa_fp8kv(fq, fk, fv, f8["k_scale"], f8["v_scale"], fl,
                                                                     out=out8, workspace=ws8), out8)
    assert torch.isfinite(eager8).all()


def test_mla_step_and_cached_append_prefill_graph_replay():
    """The MLA decode step with the new token and the cached prefill that appends its rows, captured
    and replayed (their cache writes repeat the same bytes on every replay)."""
    import mha_mla_kv_amd as attn
    B, H, dn, dR, dv, r, T = 3, 8, 96, 48, 96, 128, 1500
    inp = {k: v.cuda() for k, v in synth.mla_decode_inputs(B, H, dn, dR, dv, r, T, [1499, 0, 700], seed=14).items()}
    g = torch.Generator().manual_seed(14)
    c_new = torch.randn(B, r, generator=g).to(torch.bfloat16).cuda()
    kr_new = torch.randn(B, dR, generator=g).to(torch.bfloat16).cuda()
    print(f"[case] mla decode step graph B={B} H={H} T={T}", flush=True)
    ws = torch.zeros(attn.attn_decode_mla_workspace_bytes(B, H, r, dR, T, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, H, dv, device="cuda")
    eager = _graph_matches_eager(lambda: attn.attn_decode_mla_append(
        inp["q_nope"], inp["q_rope"], c_new, kr_new, inp["w_uk"], inp["w_uv"], inp["c_kv"], inp["k_rope"],
        inp["cache_lens"], out=out, workspace=ws), out)
    assert torch.isfinite(eager).all()
    assert not ws[:4 * B].any()  # the per-sequence chunk counters are back to zero

    Bp, S, Hq, Hkv, D, Tp = 2, 300, 16, 4, 128, 1200
    pin = {k: v.cuda() for k, v in synth.gqa_prefill_cached_inputs(Bp, S, Hq, Hkv, D, Tp, [700, 64], [300, 111],
                                                                   seed=15).items()}
    k_new = torch.stack([pin["k"][b, p:p + S] for b, p in enumerate([700, 64])]).contiguous()
    v_new = torch.stack([pin["v"][b, p:p + S] for b, p in enumerate([700, 64])]).contiguous()
    print(f"[case] cached append prefill graph B={Bp} S={S} Hq={Hq} Hkv={Hkv} T={Tp}", flush=True)
    pout = torch.empty_like(pin["q"])
    peager = _graph_matches_eager(lambda: attn.attn_prefill_gqa_cached_append(
        pin["q"], k_new, v_new, pin["k"], pin["v"], pin["start_pos"], pin["q_lens"], out=pout), pout)
    assert torch.isfinite(peager.float()).all()
    assert not peager[1, 111:].any()


def test_paged_and_low_precision_paths_graph_replay():
    """The paged GQA and MLA decodes, the FP8-latent MLA decode, the int4 GQA decode and the paged
    chunked prefill, each captured and replayed (their queue and chunk counters go back to zero
    inside the launch)."""
    import mha_mla_kv_amd as attn
    B, H, dn, dR, dv, r, T = 3, 8, 96, 48, 96, 128, 1024
    inp = {k: v.cuda() for k, v in synth.mla_decode_inputs(B, H, dn, dR, dv, r, T, [1024, 1, 500], seed=16,
                                                           poison=False).items()}
    ws = torch.zeros(attn.attn_decode_mla_workspace_bytes(B, H, r, dR, T, 0), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, H, dv, device="cuda")
    cpool = inp["c_kv"].view(B * T // 16, 16, r).flip(0).contiguous()
    rpool = inp["k_rope"].view(B * T // 16, 16, dR).flip(0).contiguous()
    n_pages = B * T // 16
    table = (n_pages - 1 - torch.arange(n_pages, dtype=torch.int32, device="cuda")).view(B, T // 16).contiguous()
    print(f"[case] paged mla graph B={B} T={T}", flush=True)
    e1 = _graph_matches_eager(lambda: attn.attn_decode_mla_paged(
        inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["w_uv"], cpool, rpool, table, inp["cache_lens"], out=out,
        workspace=ws), out)
    assert torch.isfinite(e1).all() and not ws[:4 * B].any()
    c8s = float(inp["c_kv"].float().abs().max()) / 448.0
    c8 = (inp["c_kv"].float() / c8s).to(torch.float8_e4m3fn)
    assert not torch.isnan(c8.float()).any()
    print(f"[case] fp8 latent mla graph B={B} T={T}", flush=True)
    e2 = _graph_matches_eager(lambda: attn.attn_decode_mla_fp8kv(
        inp["q_nope"], inp["q_rope"], inp["w_uk"], inp["w_uv"], c8, c8s, inp["k_rope"], inp["cache_lens"],
        out=out, workspace=ws), out)
    assert torch.isfinite(e2).all() and not ws[:4 * B].any()

    i4 = {k: v.cuda() for k, v in synth.gqa_decode_int4_inputs(4, 32, 8, 128, 1500, [1500, 3, 700, 0],
                                                              seed=17).items()}
    gws = torch.zeros(attn.attn_decode_gqa_workspace_bytes(4, 32, 8, 128, 1500, 0), dtype=torch.uint8,
                      device="cuda")
    gout = torch.empty(4, 32, 128, device="cuda")
    print("[case] int4 decode graph", flush=True)
    e3 = _graph_matches_eager(lambda: attn.attn_decode_gqa_int4kv(
        i4["q"], i4["k"], i4["v"], i4["k_scale"], i4["v_scale"], i4["cache_lens"], out=gout, workspace=gws), gout)
    assert torch.isfinite(e3).all() and not gws[:4].any()

    Bp, S, Hq, Hkv, D, Tp = 2, 200, 16, 4, 128, 1024
    pin = {k: v.cuda() for k, v in synth.gqa_prefill_cached_inputs(Bp, S, Hq, Hkv, D, Tp, [700, 64], [200, 111],
                                                                   seed=18, poison=False).items()}
    kp = pin["k"].view(Bp * Tp // 64, 64, Hkv, D)
    vp = pin["v"].view(Bp * Tp // 64, 64, Hkv, D)
    ptable = torch.arange(Bp * Tp // 64, dtype=torch.int32, device="cuda").view(Bp, Tp // 64).contiguous()
    pout = torch.empty_like(pin["q"])
    print(f"[case] paged prefill graph B={Bp} S={S}", flush=True)
    e4 = _graph_matches_eager(lambda: attn.attn_prefill_gqa_paged(
        pin["q"], kp, vp, ptable, pin["start_pos"], pin["q_lens"], out=pout), pout)
    assert torch.isfinite(e4.float()).all()
