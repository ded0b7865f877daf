#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass over the C-ABI compute entry points, each on its own synthetic workload
(shapes from the pages' configurations, i.i.d. N(0,1) inputs from fixed seeds):

  * attn_prefill_gqa_causal   Llama-3-8B-shaped causal prefill: B 4, S 4096, Hq 32, Hkv 8,
                              head_dim 128, bf16 in / out
  * attn_prefill_gqa_cached   the same heads, a 512-token chunk after a 3584-token cached
                              prefix in each of 4 sequences (chunked prefill), bf16 in / out
  * attn_prefill_mla_causal   MiniMind-768 MLA causal prefill: B 4, S 4096, 8 heads, nope 96,
                              rope 48, v 96, kv_lora_rank 128, bf16 in / out
  * attn_decode_mla_absorbed  MiniMind-768 MLA decode: B 64, 8 heads, nope 96, rope 48, v 96,
                              kv_lora_rank 128, cache 4096, bf16 (six cache copies used in turn)
  * attn_cache_append         the decode step's K/V write: each of the 32 Llama-3 sequences'
                              newest K and V rows written at position cache_lens - 1 (the rows
                              it already holds, so the decode inputs do not change)
  * attn_decode_gqa           Llama-3-8B-shaped GQA decode: B 32, Hq 32, Hkv 8, head_dim 128,
                              cache lengths uniform in [1024, 8192] (T_max 8192), bf16 in, fp32 out
  * attn_decode_gqa_append    the same write and the decode in one call (cache_lens - 1 cached
                              rows plus the new one: the same attention as attn_decode_gqa)
  * attn_decode_gqa_fp8kv     the Llama-3 decode shape and lengths over FP8 E4M3 caches (one
                              byte per element, one scale per cache)
  * attn_decode_gqa           KV-group sweep: Hq 32, head_dim 128, B 16, cache 8192, bf16, with
                              Hkv 32 (MHA), 8 (GQA-8) and 1 (MQA); 1, 2 and 8 cache copies used in
                              turn, so each setting's copies total at least 1 GiB
  * attn_decode_gqa           MiniMind-768 GQA decode: Hq 8, Hkv 4, head_dim 96, B 1, cache 512,
                              fp32 in / out (1.5 MiB of K/V: latency-bound by size)

Cache copies used in turn keep every decode part reading from HBM rather than from the
256 MB Infinity Cache when a part is timed on its own; inside a step the other parts'
traffic (several GB) separates two calls of one part in any case.

The printed `value` is the Llama-3 GQA decode's KV-cache read rate (algorithmic bytes: every
cached K and V row read once per KV head, 2*Hkv*head_dim*2 bytes per cached position) divided
by the time of one attn_decode_gqa call (its streaming kernel and the small kernel that merges
the partial results), measured with HIP events around the call on the stream the library
launches on.  Every other part is reported under "parts" with its own algorithmic unit.
Inputs are resident in HBM before the timed region.  `cpu_baseline` times the fp64 CPU oracle
(the tests' checker, not tuned) on a bounded sample of each configuration on this host.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GQA/MLA decode KV-cache GB/s (% HBM peak) + causal prefill TFLOP/s, 1 MI355X"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published (no sparsity)
# dense bf16 MFMA flop per compute unit and clock on CDNA4: 4 matrix cores of 1024 flop/clock
# each (twice CDNA3's rate); times the device's compute units and peak engine clock
BF16_FLOP_PER_CU_CLK = 4096
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gqa_decode_llama3_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=3.0, help="target CPU oracle time per configuration")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy per step (for counter calibration)")
    ap.add_argument("--parts", default="", help="comma-separated subset of parts to run (default: all)")
    ap.add_argument("--fixed-cost", action="store_true",
                    help="instead of the step: time the MQA, Llama-3-head and MLA decodes over a range of cache "
                         "lengths and fit time = fixed + bytes / stream rate (one JSON line)")
    return ap.parse_args()


def fixed_cost(attn, torch, synth, dev, dev_normal):
    """Per-call time of three decode families against their cache bytes, to separate a call's
    fixed cost (launch, first loads, epilogue, merge) from its streaming rate.  Every length runs
    over rotating cache copies of at least 512 MiB in all (twice the Infinity Cache), each time
    the median of 5 repeats of 10 back-to-back calls; the fit is least squares over the four
    largest lengths, where every compute unit has work."""
    import numpy as np

    def timed(fn, n_copies):
        for i in range(2):
            fn(i % n_copies)
        reps = []
        c = 0
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                fn(c % n_copies)
                c += 1
            e1.record()
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) / 10 * 1000)
        return float(np.median(reps))

    def copies_for(nbytes):
        return max(2, -(-(512 << 20) // nbytes))

    res = {}
    # GQA decode: MQA (the sweep's B 16, Hq 32, Hkv 1) and the Llama-3-8B heads (B 32, Hq 32, Hkv 8)
    for fam, B, Hq, Hkv, lengths in (("mqa_b16", 16, 32, 1, (1024, 2048, 4096, 8192, 16384, 32768)),
                                     ("llama3_heads_b32", 32, 32, 8, (512, 1024, 2048, 4096, 8192))):
        D = 128
        pts = []
        q = dev_normal((B, Hq, D))
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
        for L in lengths:
            nbytes = 2 * B * L * Hkv * D * 2
            nc = copies_for(nbytes)
            kv = [(dev_normal((B, L, Hkv, D)), dev_normal((B, L, Hkv, D))) for _ in range(nc)]
            lens = torch.full((B,), L, dtype=torch.int32, device=dev)
            ws = torch.zeros(attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, L, 0), dtype=torch.uint8, device=dev)
            us = timed(lambda i: attn.attn_decode_gqa(q, kv[i][0], kv[i][1], lens, out=out, workspace=ws), nc)
            pts.append((L, nbytes, us))
            del kv
            torch.cuda.empty_cache()
        res[fam] = pts
    # MLA decode at the MiniMind-768 widths (B 64, H 8, r 128, dR 48)
    mla = {k: v.to(dev) for k, v in synth.make("minimind768_mla_decode").items()}
    MB, H, dn = mla["q_nope"].shape
    dR, dv, r = mla["q_rope"].shape[2], mla["w_uv"].shape[1], mla["w_uv"].shape[2]
    out = torch.empty(MB, H, dv, dtype=torch.float32, device=dev)
    pts = []
    for L in (512, 1024, 2048, 4096, 8192, 16384):
        nbytes = MB * L * (r + dR) * 2
        nc = copies_for(nbytes)
        cc = [(dev_normal((MB, L, r)), dev_normal((MB, L, dR))) for _ in range(nc)]
        lens = torch.full((MB,), L, dtype=torch.int32, device=dev)
        ws = torch.zeros(attn.attn_decode_mla_workspace_bytes(MB, H, r, dR, L, 0), dtype=torch.uint8, device=dev)
        us = timed(lambda i: attn.attn_decode_mla_absorbed(mla["q_nope"], mla["q_rope"], mla["w_uk"], mla["w_uv"],
                                                           cc[i][0], cc[i][1], lens, out=out, workspace=ws), nc)
        pts.append((L, nbytes, us))
        del cc
        torch.cuda.empty_cache()
    res["mla_minimind768_b64"] = pts

    report = {}
    for fam, pts in res.items():
        x = np.array([p[1] for p in pts[-4:]], dtype=np.float64)
        y = np.array([p[2] for p in pts[-4:]], dtype=np.float64)
        slope, icept = np.polyfit(x, y, 1)  # us per byte, us
        report[fam] = {"points": [{"L": L, "bytes": b, "us": round(t, 2), "TB/s": round(b / t / 1e6, 3)}
                                  for L, b, t in pts],
                       "fit_over_L": [p[0] for p in pts[-4:]],
                       "fixed_us": round(float(icept), 2), "stream_TB/s": round(1.0 / float(slope) / 1e6, 3)}
    print(json.dumps({"fixed_cost": report, "hbm_peak_TB/s": 8.0,
                      "note": "per-call time = fixed_us + bytes / stream rate, fitted over the four largest lengths"}))


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mha_mla_kv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when they were
    taken on another version of the kernel's source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_clock_ghz(index: int):
    """Peak engine clock of device `index` in GHz from hipDeviceGetAttribute, or None.

    torch's device properties carry no clock on ROCm.  The HIP runtime is the one torch has
    loaded already (same soname, so dlopen returns that copy rather than a second runtime)."""
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
    except OSError:
        return None
    clock_rate_khz = 5  # hipDeviceAttributeClockRate: sixth entry of hipDeviceAttribute_t
    v = ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(v), clock_rate_khz, index) != 0 or v.value <= 0:
        return None
    return v.value / 1e6


def gqa_decode_bytes(Hkv, D, elem_bytes, sum_len):
    """Algorithmic K/V bytes of a decode: every cached K and V row read once per KV head."""
    return 2 * Hkv * D * elem_bytes * sum_len


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): the library is a "
              "single-GPU kernel set; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mha_mla_kv_amd as attn
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (HIP device)", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    attn.lib()  # fail loudly now if the library is missing
    props = torch.cuda.get_device_properties(dev)
    want = set(p for p in args.parts.split(",") if p)

    t_gen = time.time()
    gen = torch.Generator(device=dev).manual_seed(8)

    def dev_normal(shape, dtype=torch.bfloat16, scale=1.0):
        x = torch.randn(*shape, device=dev, generator=gen)
        if scale != 1.0:
            x *= scale
        return x.to(dtype)

    if args.fixed_cost:
        fixed_cost(attn, torch, synth, dev, dev_normal)
        return

    # ---- Llama-3-8B GQA decode (the headline), its append / fused step, FP8 caches ----
    dspec = synth.WORKLOADS["llama3_8b_gqa_decode"]
    dec_cpu = synth.make("llama3_8b_gqa_decode")
    dec = {k: v.to(dev) for k, v in dec_cpu.items()}
    B, Hq, D = dec["q"].shape
    T_max, Hkv = dec["k"].shape[1], dec["k"].shape[2]
    sum_len = int(dec_cpu["cache_lens"].clamp(0, T_max).sum())
    dec_bytes = gqa_decode_bytes(Hkv, D, 2, sum_len)
    dec_flops = 4 * Hq * D * sum_len                           # QK^T and PV
    dec_out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    dec_ws = torch.zeros(attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T_max, 0), dtype=torch.uint8,
                         device=dev)
    last = (dec_cpu["cache_lens"].clamp(1, T_max) - 1).to(dev)
    app_pos = last.to(torch.int32)
    app_k = dec["k"][torch.arange(B, device=dev), last.long()].unsqueeze(1).contiguous()  # [B, 1, Hkv, D]
    app_v = dec["v"][torch.arange(B, device=dev), last.long()].unsqueeze(1).contiguous()
    app_bytes = 2 * 2 * B * Hkv * D * 2                       # K and V rows, read once and written once
    app_new_k, app_new_v = app_k[:, 0].contiguous(), app_v[:, 0].contiguous()  # [B, Hkv, D]
    step_out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    f8_scale = 4.5 / 448.0
    # (clamped to E4M3's largest finite value: torch turns values past it into NaN codes)
    f8_k = (torch.randn(B, T_max, Hkv, D, device=dev, generator=gen) / f8_scale).clamp(-448, 448).to(torch.float8_e4m3fn)
    f8_v = (torch.randn(B, T_max, Hkv, D, device=dev, generator=gen) / f8_scale).clamp(-448, 448).to(torch.float8_e4m3fn)
    f8_bytes = dec_bytes // 2                                 # one byte per cached element
    f8_out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    # int4 caches: random code bytes and per-row scales in [0.25, 0.75), drawn on the device, three
    # copies used in turn (152 MB each, so a call does not find its rows in the Infinity Cache)
    # (head-major: [B, Hkv, T_max, D/2] codes, [B, Hkv, T_max] scales)
    i4 = [(torch.randint(0, 256, (B, Hkv, T_max, D // 2), device=dev, generator=gen, dtype=torch.uint8),
           torch.randint(0, 256, (B, Hkv, T_max, D // 2), device=dev, generator=gen, dtype=torch.uint8),
           torch.rand(B, Hkv, T_max, device=dev, generator=gen) * 0.5 + 0.25,
           torch.rand(B, Hkv, T_max, device=dev, generator=gen) * 0.5 + 0.25) for _ in range(3)]
    i4_bytes = 2 * Hkv * (D // 2 + 4) * sum_len              # codes and row scales of K and V
    i4_out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    # paged view of the same caches: 64-position pages, every sequence's pages scattered over the
    # whole pool by a seeded permutation (the pool is the contiguous cache, seen as pages)
    pg_size = 64
    pg_max = T_max // pg_size
    pg_k = dec["k"].view(B * pg_max, pg_size, Hkv, D)
    pg_v = dec["v"].view(B * pg_max, pg_size, Hkv, D)
    pg_table = torch.randperm(B * pg_max, generator=torch.Generator().manual_seed(11)).to(torch.int32)
    pg_table = pg_table.view(B, pg_max).to(dev)
    pg_out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    # paged decode step: the newest row of every sequence in the paged view (through its page) is the
    # new token, written back at the same place, so every call rewrites rows with their own values
    pgs_page = pg_table[torch.arange(B, device=dev), (app_pos // pg_size).long()].long()
    pgs_row = (app_pos % pg_size).long()
    pgs_new_k, pgs_new_v = pg_k[pgs_page, pgs_row].contiguous(), pg_v[pgs_page, pgs_row].contiguous()  # [B, Hkv, D]
    pgs_out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    step_ws = torch.zeros(attn.attn_decode_gqa_append_workspace_bytes(B, Hq, Hkv, D, T_max, 0), dtype=torch.uint8,
                          device=dev)

    # ---- KV-group sweep (MHA / GQA-8 / MQA): caches drawn on the device, copies used in turn ----
    sweep = {}
    for name, copies in (("kv_sweep_mha", 1), ("kv_sweep_gqa8", 2), ("kv_sweep_mqa", 8)):
        if want and name not in want:
            continue
        sp = synth.WORKLOADS[name]
        SB, SHq, SHkv, SD, ST = sp["B"], sp["Hq"], sp["Hkv"], sp["D"], sp["T_max"]
        lens = torch.full((SB,), sp["lens"], dtype=torch.int32, device=dev)
        kv = [(dev_normal((SB, ST, SHkv, SD)), dev_normal((SB, ST, SHkv, SD))) for _ in range(copies)]
        sweep[name] = {
            "q": dev_normal((SB, SHq, SD)), "kv": kv, "lens": lens,
            "out": torch.empty(SB, SHq, SD, dtype=torch.float32, device=dev),
            "ws": torch.zeros(attn.attn_decode_gqa_workspace_bytes(SB, SHq, SHkv, SD, ST, 0), dtype=torch.uint8,
                              device=dev),
            "bytes": gqa_decode_bytes(SHkv, SD, 2, SB * sp["lens"]), "flops": 4 * SHq * SD * SB * sp["lens"],
            "tokens": SB, "copies": copies,
            "workload": f"{name}: B={SB} Hq={SHq} Hkv={SHkv} head_dim={SD} cache={sp['lens']} bf16 in, fp32 out; "
                        f"N(0,1) caches drawn on the device (seed 8), {copies} cache cop{'y' if copies == 1 else 'ies'} "
                        "used in turn",
        }

    # ---- MiniMind-768 GQA decode, fp32 ----
    mm_cpu = synth.make("minimind768_gqa_decode")
    mm = {k: v.to(dev) for k, v in mm_cpu.items()}
    MMB, MMHq, MMD = mm["q"].shape
    MMT, MMHkv = mm["k"].shape[1], mm["k"].shape[2]
    mm_len = int(mm_cpu["cache_lens"].clamp(0, MMT).sum())
    mm_bytes = gqa_decode_bytes(MMHkv, MMD, 4, mm_len)
    mm_out = torch.empty(MMB, MMHq, MMD, dtype=torch.float32, device=dev)
    mm_ws = torch.zeros(attn.attn_decode_gqa_workspace_bytes(MMB, MMHq, MMHkv, MMD, MMT, 0), dtype=torch.uint8,
                        device=dev)

    # ---- MiniMind-768 MLA decode: the seeded workload plus five device-drawn cache copies ----
    mspec = synth.WORKLOADS["minimind768_mla_decode"]
    mla_cpu = synth.make("minimind768_mla_decode")
    mla = {k: v.to(dev) for k, v in mla_cpu.items()}
    MB, H, dn = mla["q_nope"].shape
    dR = mla["q_rope"].shape[2]
    dv, r = mla["w_uv"].shape[1], mla["w_uv"].shape[2]
    MT = mla["c_kv"].shape[1]
    mla_copies = [(mla["c_kv"], mla["k_rope"])] + [(dev_normal((MB, MT, r)), dev_normal((MB, MT, dR)))
                                                   for _ in range(5)]
    mla_len = int(mla_cpu["cache_lens"].clamp(0, MT).sum())
    mla_bytes = (r + dR) * 2 * mla_len                          # one [c_kv, k_rope] row per position
    mla_flops = H * (2 * (r + dR) + 2 * r) * mla_len
    mla_out = torch.empty(MB, H, dv, dtype=torch.float32, device=dev)
    mla_ws = torch.zeros(attn.attn_decode_mla_workspace_bytes(MB, H, r, dR, MT, 0), dtype=torch.uint8, device=dev)
    # decode step with the new token: the row at cache_lens - 1 of each cache copy is appended again
    # at that position, so every step rewrites a row with its own value and the caches stay the same
    mla_last = (mla_cpu["cache_lens"].clamp(1, MT) - 1).to(dev)
    mla_step_pos = mla_last.to(torch.int32)
    mla_step_new = [(c[torch.arange(MB, device=dev), mla_last.long()].contiguous(),             # [B, r]
                     kr[torch.arange(MB, device=dev), mla_last.long()].contiguous())            # [B, dR]
                    for c, kr in mla_copies]
    mla_step_out = torch.empty(MB, H, dv, dtype=torch.float32, device=dev)
    # paged view of the same caches: 16-position pages, every sequence's pages scattered over the
    # whole pool by a seeded permutation (each cache copy is a pool, read through the same table)
    mpg_size = 16
    mpg_max = MT // mpg_size
    mpg_table = torch.randperm(MB * mpg_max, generator=torch.Generator().manual_seed(12)).to(torch.int32)
    mpg_table = mpg_table.view(MB, mpg_max).to(dev)
    mpg_out = torch.empty(MB, H, dv, dtype=torch.float32, device=dev)
    # FP8 E4M3 latent: each copy's c_kv as codes with one scale (N(0,1) data, scale 4.5 / 448),
    # k_rope bf16
    mf8_scale = 4.5 / 448.0
    mf8_copies = [((c.float() / mf8_scale).clamp(-448, 448).to(torch.float8_e4m3fn), kr) for c, kr in mla_copies]
    mf8_bytes = (r + 2 * dR) * mla_len                          # one fp8 latent + bf16 rope row per position
    mf8_out = torch.empty(MB, H, dv, dtype=torch.float32, device=dev)
    mla_step_ws = torch.zeros(attn.attn_decode_mla_workspace_bytes(MB, H, r, dR, MT, 0), dtype=torch.uint8,
                              device=dev)

    # ---- prefills ----
    pspec = synth.WORKLOADS["llama3_8b_gqa_prefill"]
    pre = {k: v.to(dev) for k, v in synth.make("llama3_8b_gqa_prefill").items()}
    PB, S, PHq, PD = pre["q"].shape
    pre_flops = 4 * PB * PHq * PD * S * (S + 1) // 2           # unmasked (i, j <= i) pairs only
    pre_out = torch.empty_like(pre["q"])
    cspec = synth.WORKLOADS["llama3_8b_gqa_chunked_prefill"]
    chk_cpu = synth.make("llama3_8b_gqa_chunked_prefill")
    chk = {k: v.to(dev) for k, v in chk_cpu.items()}
    CB, CS, CHq, CD = chk["q"].shape
    CT = chk["k"].shape[1]
    chk_flops = 0
    for P, n in zip(chk_cpu["start_pos"].tolist(), chk_cpu["q_lens"].tolist()):
        P = max(0, min(P, CT))
        n = max(0, min(n, CS, CT - P))
        chk_flops += 4 * CHq * CD * (n * P + n * (n + 1) // 2)   # new token i sees P + i + 1 keys
    chk_tokens = int(chk_cpu["q_lens"].sum())
    chk_out = torch.empty_like(chk["q"])
    # the same chunk over a paged view of the caches: 64-position pages, every sequence's pages
    # scattered over the pool by a seeded permutation
    cpg_size = 64
    cpg_max = CT // cpg_size
    cpg_table = torch.randperm(CB * cpg_max, generator=torch.Generator().manual_seed(13)).to(torch.int32)
    cpg_table = cpg_table.view(CB, cpg_max).to(dev)
    cpg_k = chk["k"].view(CB * cpg_max, cpg_size, chk["k"].shape[2], CD)
    cpg_v = chk["v"].view(CB * cpg_max, cpg_size, chk["v"].shape[2], CD)
    cpg_out = torch.empty_like(chk["q"])
    # the same chunk through the one-launch append + prefill: the new rows are the cache rows at
    # start_pos.., written back unchanged every step
    chk_sp = chk_cpu["start_pos"].clamp(0, CT)
    chk_rows = torch.stack([torch.arange(CS) + int(p) for p in chk_sp]).clamp(max=CT - 1)      # [B, S]
    chk_k_new = torch.stack([chk_cpu["k"][b, chk_rows[b]] for b in range(CB)]).to(dev)
    chk_v_new = torch.stack([chk_cpu["v"][b, chk_rows[b]] for b in range(CB)]).to(dev)
    chk_app_out = torch.empty_like(chk["q"])
    # rotary embedding + cache write of the same chunk: q rotated in place (a copy, so the prefill
    # parts keep their inputs), K rotated into the cache at start_pos.., V copied
    rope_q = chk["q"].clone()
    chk_sp_dev = chk["start_pos"]
    rope_chunk_bytes = 2 * (CB * CS * CHq * CD * 2) + 2 * 2 * (CB * CS * chk["k"].shape[2] * CD * 2)
    rope_dec_q = dec["q"].clone().unsqueeze(1)                       # [B, 1, Hq, D]
    rope_dec_bytes = 2 * (B * Hq * D * 2) + 2 * 2 * (B * Hkv * D * 2)

    mpspec = synth.WORKLOADS["minimind768_mla_prefill"]
    mlp = {k: v.to(dev) for k, v in synth.make("minimind768_mla_prefill").items()}
    MPB, MPS, MPH, MPdn = mlp["q_nope"].shape
    MPdR = mlp["q_rope"].shape[3]
    MPdv, MPr = mlp["w_uv"].shape[1], mlp["w_uv"].shape[2]
    mlp_pairs = MPB * MPH * MPS * (MPS + 1) // 2
    # MFMA work of the absorbed form: 2(r + dR) + 2r per unmasked (query, key) pair and head, plus
    # the query absorption (2 dn r) and the value up-projection (2 dv r) per new token and head
    mlp_flops = mlp_pairs * (2 * (MPr + MPdR) + 2 * MPr) + MPB * MPS * MPH * 2 * MPr * (MPdn + MPdv)
    # the listing's decompressed SDPA: 2 (dn + dR) + 2 dv per pair and head (K and V rebuilt first)
    mlp_flops_sdpa = mlp_pairs * (2 * (MPdn + MPdR) + 2 * MPdv)
    mlp_out = torch.empty(MPB, MPS, MPH, MPdv, dtype=torch.bfloat16, device=dev)
    copy_src = copy_dst = None
    if args.copy_calibration:
        copy_src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        copy_dst = torch.empty_like(copy_src)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    stream = torch.cuda.current_stream(dev)

    def run_decode(i):
        attn.attn_decode_gqa(dec["q"], dec["k"], dec["v"], dec["cache_lens"], out=dec_out, workspace=dec_ws)

    def run_mla(i):
        c, kr = mla_copies[i % len(mla_copies)]
        attn.attn_decode_mla_absorbed(mla["q_nope"], mla["q_rope"], mla["w_uk"], mla["w_uv"], c, kr,
                                      mla["cache_lens"], out=mla_out, workspace=mla_ws)

    def run_mla_paged(i):
        c, kr = mla_copies[i % len(mla_copies)]
        attn.attn_decode_mla_paged(mla["q_nope"], mla["q_rope"], mla["w_uk"], mla["w_uv"],
                                   c.view(MB * mpg_max, mpg_size, r), kr.view(MB * mpg_max, mpg_size, dR), mpg_table,
                                   mla["cache_lens"], out=mpg_out, workspace=mla_ws)

    def run_mla_fp8(i):
        c8, kr = mf8_copies[i % len(mf8_copies)]
        attn.attn_decode_mla_fp8kv(mla["q_nope"], mla["q_rope"], mla["w_uk"], mla["w_uv"], c8, mf8_scale, kr,
                                   mla["cache_lens"], out=mf8_out, workspace=mla_ws)

    def run_mla_paged_fp8(i):  # the FP8 latent copies as pools of 16-position pages, read through one table
        c8, kr = mf8_copies[i % len(mf8_copies)]
        attn.attn_decode_mla_paged_fp8kv(mla["q_nope"], mla["q_rope"], mla["w_uk"], mla["w_uv"],
                                         c8.view(MB * mpg_max, mpg_size, r), mf8_scale,
                                         kr.view(MB * mpg_max, mpg_size, dR), mpg_table, mla["cache_lens"],
                                         out=mf8_out, workspace=mla_ws)

    def run_prefill(i):
        attn.attn_prefill_gqa_causal(pre["q"], pre["k"], pre["v"], out=pre_out)

    def run_append(i):
        attn.attn_cache_append(app_k, dec["k"], app_v, dec["v"], app_pos)

    def run_step(i):
        attn.attn_decode_gqa_append(dec["q"], app_new_k, app_new_v, dec["k"], dec["v"], app_pos, out=step_out,
                                    workspace=step_ws)

    def run_int4(i):
        kc, vc, ks, vs = i4[i % len(i4)]
        attn.attn_decode_gqa_int4kv(dec["q"], kc, vc, ks, vs, dec["cache_lens"], out=i4_out, workspace=dec_ws)

    def run_paged(i):
        attn.attn_decode_gqa_paged(dec["q"], pg_k, pg_v, pg_table, dec["cache_lens"], out=pg_out, workspace=dec_ws)

    def run_paged_fp8(i):  # the FP8 caches seen as pools of 64-position pages, read through the same table
        attn.attn_decode_gqa_paged_fp8kv(dec["q"], f8_k.view(B * pg_max, pg_size, Hkv, D),
                                         f8_v.view(B * pg_max, pg_size, Hkv, D), f8_scale, f8_scale, pg_table,
                                         dec["cache_lens"], out=f8_out, workspace=dec_ws)

    def run_paged_step(i):
        attn.attn_decode_gqa_paged_append(dec["q"], pgs_new_k, pgs_new_v, pg_k, pg_v, pg_table, app_pos, out=pgs_out,
                                          workspace=step_ws)

    def run_fp8(i):
        attn.attn_decode_gqa_fp8kv(dec["q"], f8_k, f8_v, f8_scale, f8_scale, dec["cache_lens"], out=f8_out,
                                   workspace=dec_ws)

    def run_mla_prefill(i):
        attn.attn_prefill_mla_causal(mlp["q_nope"], mlp["q_rope"], mlp["w_uk"], mlp["w_uv"], mlp["c_kv"], mlp["k_rope"],
                                     out=mlp_out)

    def run_chunked(i):
        attn.attn_prefill_gqa_cached(chk["q"], chk["k"], chk["v"], chk["start_pos"], chk["q_lens"], out=chk_out)

    def run_chunked_paged(i):
        attn.attn_prefill_gqa_paged(chk["q"], cpg_k, cpg_v, cpg_table, chk["start_pos"], chk["q_lens"], out=cpg_out)

    def run_chunked_append(i):
        attn.attn_prefill_gqa_cached_append(chk["q"], chk_k_new, chk_v_new, chk["k"], chk["v"], chk["start_pos"],
                                            chk["q_lens"], out=chk_app_out)

    def run_rope_chunk(i):
        attn.attn_rope_append(chk_k_new, chk["k"], rope_q, chk_sp_dev, chk["q_lens"], chk_v_new, chk["v"])

    def run_rope_decode(i):
        attn.attn_rope_append(app_k, dec["k"], rope_dec_q, app_pos, None, app_v, dec["v"])

    def run_mla_step(i):  # a different cache copy from the one mla_decode read just before
        j = (i + 3) % len(mla_copies)
        (c, kr), (cn, krn) = mla_copies[j], mla_step_new[j]
        attn.attn_decode_mla_append(mla["q_nope"], mla["q_rope"], cn, krn, mla["w_uk"], mla["w_uv"], c, kr,
                                    mla_step_pos, out=mla_step_out, workspace=mla_step_ws)

    def run_sweep(name):
        w = sweep[name]

        def fn(i):
            k, v = w["kv"][i % w["copies"]]
            attn.attn_decode_gqa(w["q"], k, v, w["lens"], out=w["out"], workspace=w["ws"])
        return fn

    def run_minimind(i):
        attn.attn_decode_gqa(mm["q"], mm["k"], mm["v"], mm["cache_lens"], out=mm_out, workspace=mm_ws)

    # prefill for new requests, then the decode steps of running ones (the order a serving
    # step takes), then the sweep settings; each part is timed on its own
    parts = [("prefill", run_prefill), ("chunked_prefill", run_chunked), ("chunked_prefill_append", run_chunked_append),
             ("chunked_prefill_paged", run_chunked_paged),
             ("mla_prefill", run_mla_prefill), ("mla_decode", run_mla), ("mla_decode_step", run_mla_step),
             ("mla_decode_paged", run_mla_paged), ("mla_decode_fp8", run_mla_fp8),
             ("mla_decode_paged_fp8", run_mla_paged_fp8),
             ("kv_append", run_append), ("rope_append_decode", run_rope_decode), ("rope_append_chunk", run_rope_chunk),
             ("gqa_decode", run_decode), ("gqa_decode_paged", run_paged), ("gqa_decode_step", run_step),
             ("gqa_decode_paged_step", run_paged_step), ("gqa_decode_fp8", run_fp8),
             ("gqa_decode_paged_fp8", run_paged_fp8), ("gqa_decode_int4", run_int4)]
    parts += [(name, run_sweep(name)) for name in sweep]
    parts.append(("minimind768_gqa_decode", run_minimind))
    if want:
        parts = [p for p in parts if p[0] in want or p[0] == "gqa_decode"]
    if args.copy_calibration:
        parts.append(("copy_1GiB", lambda i: copy_dst.copy_(copy_src)))

    for i in range(args.warmup):
        for _, fn in parts:
            fn(i)
    torch.cuda.synchronize()

    # The K steps are timed part by part: each part's K calls run back to back between one pair
    # of events on the library's stream, as a serving loop calls them, so that an event pair
    # around every single call (a few microseconds each) does not count as kernel time.  The
    # step's total work is unchanged (every part K times); the parts with long kernels come
    # first, so the host has queued the short ones before the GPU reaches them.
    K = args.steps
    ev = {name: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for name, _ in parts}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for name, fn in parts:
        e0, e1 = ev[name]
        e0.record(stream)
        for i in range(K):
            fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {name: e0.elapsed_time(e1) / K for name, (e0, e1) in ev.items()}

    def rate(nbytes, name):
        return nbytes / (ms[name] * 1e-3) / 1e9

    dec_gbs = rate(dec_bytes, "gqa_decode")
    dec_hash = source_hash("decode_gqa.hip", "attn_internal.h")
    # HBM bytes of the call's two launches (decode + merge), from the committed counter runs
    t_main = measured_traffic("gqa_decode_bf16<128, 1, true, false, false, false>", dec_hash)
    t_merge = measured_traffic("gqa_decode_merge", dec_hash)
    traffic = round(t_main + t_merge) if t_main is not None and t_merge is not None else None
    clk_ghz = device_clock_ghz(torch.cuda.current_device())
    derived_peak = (props.multi_processor_count * BF16_FLOP_PER_CU_CLK * clk_ghz * 1e9 / 1e12) if clk_ghz else None

    result = {
        "metric": METRIC,
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"llama3_8b_gqa_decode: B={B} Hq={Hq} Hkv={Hkv} head_dim={D} T_max={T_max} "
                         f"cache_lens~U[{dspec['lens'][0]},{dspec['lens'][1]}] (sum {sum_len}) seed={dspec['seed']}, "
                         "bf16 in, fp32 out, default schedule (device-wide unit queue, library-chosen blocks)"),
            "step": ", ".join(name for name, _ in parts) + ": one call each; timed part by part, each "
                    "part's K calls back to back between one event pair, in this order",
            "tokens_per_step": {"gqa_decode": B, "mla_decode": MB, "mla_decode_step": MB, "mla_decode_paged": MB, "mla_decode_fp8": MB, "prefill": PB * S,
                                "chunked_prefill": chk_tokens, "chunked_prefill_append": chk_tokens,
                                "chunked_prefill_paged": chk_tokens,
                                "mla_prefill": MPB * MPS},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("gqa_decode_bf16<128, 1, true, false, false, false> + gqa_decode_merge: one attn_decode_gqa call "
                       "(two launches), K calls back to back between one event pair"),
            "achieved": round(dec_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dec_bytes,
            "avg_launch_ms": round(ms["gqa_decode"], 5),
        },
        "peaks": {"hbm_GB/s": HBM_PEAK_GBS, "bf16_dense_TFLOP/s_published": BF16_DENSE_PEAK_TFLOPS,
                  "bf16_dense_TFLOP/s_from_device": round(derived_peak, 1) if derived_peak else None,
                  "device": {"name": props.name, "compute_units": props.multi_processor_count,
                             "max_clock_GHz": clk_ghz}},
        "parts": {},
        "input_generation_s": round(t_gen, 2),
    }
    P = result["parts"]

    def decode_part(name, nbytes, tokens, flops=None, workload=None, extra=None):
        gbs = rate(nbytes, name)
        e = {"ms": round(ms[name], 5), "GB/s": round(gbs, 1),
             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": nbytes,
             "tokens_per_s": round(tokens / (ms[name] * 1e-3), 1)}
        if flops is not None:
            e["TFLOP/s"] = round(flops / (ms[name] * 1e-3) / 1e12, 2)
        if workload:
            e["workload"] = workload
        if extra:
            e.update(extra)
        P[name] = e

    def prefill_part(name, flops, tokens, workload, extra=None):
        tfs = flops / (ms[name] * 1e-3) / 1e12
        e = {"ms": round(ms[name], 5), "TFLOP/s": round(tfs, 1),
             "mfma_frac": round(tfs / BF16_DENSE_PEAK_TFLOPS, 4), "algorithmic_flops_per_launch": flops,
             "tokens_per_s": round(tokens / (ms[name] * 1e-3), 1), "workload": workload}
        if extra:
            e.update(extra)
        P[name] = e

    decode_part("gqa_decode", dec_bytes, B, dec_flops)
    if "mla_decode" in ms:
        decode_part("mla_decode", mla_bytes, MB, mla_flops,
                    f"minimind768_mla_decode: B={MB} H={H} nope={dn} rope={dR} v={dv} r={r} cache={MT} "
                    f"seed={mspec['seed']} (+5 device-drawn cache copies, used in turn)")
    if "prefill" in ms:
        prefill_part("prefill", pre_flops, PB * S,
                     f"llama3_8b_gqa_prefill: B={PB} S={S} Hq={PHq} Hkv={pre['k'].shape[2]} head_dim={PD} "
                     f"seed={pspec['seed']} bf16 causal")
    if "chunked_prefill" in ms:
        prefill_part("chunked_prefill", chk_flops, chk_tokens,
                     f"llama3_8b_gqa_chunked_prefill: B={CB} chunk={CS} start_pos={cspec['start_pos']} T_max={CT} "
                     f"Hq={CHq} Hkv={chk['k'].shape[2]} head_dim={CD} seed={cspec['seed']} bf16")
    if "chunked_prefill_append" in ms:
        prefill_part("chunked_prefill_append", chk_flops, chk_tokens,
                     "llama3_8b_gqa_chunked_prefill through attn_prefill_gqa_cached_append: the chunk's K/V rows "
                     "come in their own arrays and are written into the caches by the same launch")
    if "chunked_prefill_paged" in ms:
        prefill_part("chunked_prefill_paged", chk_flops, chk_tokens,
                     f"llama3_8b_gqa_chunked_prefill over a paged cache: {cpg_size}-position pages, each sequence's "
                     "pages scattered over the pool by a seeded permutation (attn_prefill_gqa_paged)")
    if "mla_decode_step" in ms:
        decode_part("mla_decode_step", mla_bytes, MB, mla_flops,
                    "minimind768_mla_decode with the newest rows as the new token (attn_decode_mla_append: "
                    "decode over cache_lens - 1 rows plus the new row, which is written at cache_lens - 1)")
    if "mla_decode_paged" in ms:
        decode_part("mla_decode_paged", mla_bytes, MB, mla_flops,
                    f"minimind768_mla_decode shape and lengths over paged latent caches: {mpg_size}-position pages, "
                    "each sequence's pages scattered over the pool by a seeded permutation (attn_decode_mla_paged)")
    if "mla_decode_fp8" in ms:
        decode_part("mla_decode_fp8", mf8_bytes, MB, mla_flops,
                    "minimind768_mla_decode shape and lengths with the latent c_kv as FP8 E4M3 codes (one scale, "
                    "N(0,1)/scale drawn on the device; k_rope bf16): 224 bytes per position (attn_decode_mla_fp8kv)")
    if "mla_decode_paged_fp8" in ms:
        decode_part("mla_decode_paged_fp8", mf8_bytes, MB, mla_flops,
                    f"the FP8-latent caches of mla_decode_fp8 as pools of {mpg_size}-position pages, each sequence's "
                    "pages scattered over the pool by the seeded permutation of mla_decode_paged "
                    "(attn_decode_mla_paged_fp8kv)")
    if "mla_prefill" in ms:
        prefill_part("mla_prefill", mlp_flops, MPB * MPS,
                     f"minimind768_mla_prefill: B={MPB} S={MPS} H={MPH} nope={MPdn} rope={MPdR} v={MPdv} "
                     f"r={MPr} seed={mpspec['seed']} bf16 causal",
                     {"flop_count": "absorbed form: 2(r+dR)+2r per unmasked pair and head + 2r(dn+dv) per token "
                                    "and head",
                      "TFLOP/s_sdpa_count": round(mlp_flops_sdpa / (ms["mla_prefill"] * 1e-3) / 1e12, 1),
                      "mfma_frac_sdpa_count": round(mlp_flops_sdpa / (ms["mla_prefill"] * 1e-3) / 1e12
                                                    / BF16_DENSE_PEAK_TFLOPS, 4),
                      "algorithmic_flops_sdpa_count": mlp_flops_sdpa})
    if "gqa_decode_fp8" in ms:
        decode_part("gqa_decode_fp8", f8_bytes, B, None,
                    "llama3_8b_gqa_decode shape and lengths, K/V as FP8 E4M3 codes of N(0,1)/scale "
                    "(device-drawn, seed 8), scale 4.5/448")
    if "gqa_decode_paged_fp8" in ms:
        decode_part("gqa_decode_paged_fp8", f8_bytes, B, None,
                    f"the FP8 caches of gqa_decode_fp8 as pools of {pg_size}-position pages, each sequence's pages "
                    "scattered over the pool by the seeded permutation of gqa_decode_paged (attn_decode_gqa_paged_fp8kv)")
    if "gqa_decode_paged" in ms:
        decode_part("gqa_decode_paged", dec_bytes, B, None,
                    f"llama3_8b_gqa_decode shape and lengths over paged caches: {pg_size}-position pages, each "
                    "sequence's pages scattered over the pool by a seeded permutation (attn_decode_gqa_paged)")
    if "gqa_decode_int4" in ms:
        decode_part("gqa_decode_int4", i4_bytes, B, None,
                    "llama3_8b_gqa_decode shape and lengths, K/V as packed signed 4-bit codes with one fp32 scale "
                    "per row (random bytes, scales U[0.25, 0.75), device-drawn, 3 copies used in turn)")
    if "gqa_decode_step" in ms:
        decode_part("gqa_decode_step", dec_bytes, B, None,
                    "llama3_8b_gqa_decode with the newest rows as the new token "
                    "(attn_decode_gqa_append: write + decode in one call)")
    if "gqa_decode_paged_step" in ms:
        decode_part("gqa_decode_paged_step", dec_bytes, B, None,
                    f"llama3_8b_gqa_decode step over the paged caches of gqa_decode_paged ({pg_size}-position pages "
                    "scattered over the pool), the newest row of each sequence as the new token "
                    "(attn_decode_gqa_paged_append: write + decode in one call)")
    if "kv_append" in ms:
        P["kv_append"] = {"ms": round(ms["kv_append"], 5), "bytes_per_launch": app_bytes,
                          "GB/s": round(rate(app_bytes, "kv_append"), 1),
                          "workload": f"llama3_8b_gqa_decode step write: B={B} rows of Hkv={Hkv} x {D} for K and V"}
    if "rope_append_chunk" in ms:
        P["rope_append_chunk"] = {
            "ms": round(ms["rope_append_chunk"], 5), "bytes_per_launch": rope_chunk_bytes,
            "GB/s": round(rate(rope_chunk_bytes, "rope_append_chunk"), 1),
            "hbm_frac": round(rate(rope_chunk_bytes, "rope_append_chunk") / HBM_PEAK_GBS, 4),
            "workload": f"llama3_8b_gqa_chunked_prefill chunk through attn_rope_append: q [{CB},{CS},{CHq},{CD}] "
                        f"rotated in place, K rotated into the cache and V copied at start_pos (bf16, base 10000)"}
    if "rope_append_decode" in ms:
        P["rope_append_decode"] = {
            "ms": round(ms["rope_append_decode"], 5), "bytes_per_launch": rope_dec_bytes,
            "GB/s": round(rate(rope_dec_bytes, "rope_append_decode"), 1),
            "workload": f"llama3_8b_gqa_decode step through attn_rope_append: q [{B},1,{Hq},{D}] rotated in place, "
                        f"one K row rotated into the cache and one V row copied per sequence"}
    for name, w in sweep.items():
        decode_part(name, w["bytes"], w["tokens"], w["flops"], w["workload"])
    if "minimind768_gqa_decode" in ms:
        decode_part("minimind768_gqa_decode", mm_bytes, MMB, 4 * MMHq * MMD * mm_len,
                    f"minimind768_gqa_decode: B={MMB} Hq={MMHq} Hkv={MMHkv} head_dim={MMD} cache={MMT} fp32 in/out "
                    f"seed={synth.WORKLOADS['minimind768_gqa_decode']['seed']} (1.5 MiB of K/V: cache-resident and "
                    "launch-bound by size; the HBM bar does not apply)")
    if args.copy_calibration:
        P["copy_1GiB"] = {"ms": round(ms["copy_1GiB"], 5),
                          "GB/s_read+write": round(2 * (1 << 30) / (ms["copy_1GiB"] * 1e-3) / 1e9, 1)}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, dec_cpu, dec_bytes, mm_cpu, mm_bytes, synth, np)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def cpu_baseline(args, dec_cpu, dec_bytes, mm_cpu, mm_bytes, synth, np):
    """The fp64 C oracle, as it stands, on a bounded sample of each configuration (about
    --cpu-seconds each), on this host's cores.  `value` is the Llama-3 decode sample's rate in
    the headline unit; `per_config` holds every configuration's sample, time and rate."""
    import oracle

    def timed(fn):
        reps, t = 0, 0.0
        t_begin = time.perf_counter()
        while True:
            t1 = time.perf_counter()
            fn()
            t += time.perf_counter() - t1
            reps += 1
            if time.perf_counter() - t_begin >= args.cpu_seconds or reps >= 50:
                return reps, t

    per = {}
    reps, t = timed(lambda: oracle.gqa_decode(dec_cpu["q"], dec_cpu["k"], dec_cpu["v"], dec_cpu["cache_lens"]))
    per["llama3_8b_gqa_decode"] = {"sample": f"all {dec_cpu['q'].shape[0]} sequences", "runs": reps,
                                   "s_per_run": round(t / reps, 4), "GB/s": round(dec_bytes * reps / t / 1e9, 3)}
    headline = per["llama3_8b_gqa_decode"]["GB/s"]
    reps, t = timed(lambda: oracle.gqa_decode(mm_cpu["q"], mm_cpu["k"], mm_cpu["v"], mm_cpu["cache_lens"]))
    per["minimind768_gqa_decode"] = {"sample": "the whole workload", "runs": reps, "s_per_run": round(t / reps, 5),
                                     "GB/s": round(mm_bytes * reps / t / 1e9, 3)}
    for name in ("kv_sweep_mha", "kv_sweep_gqa8", "kv_sweep_mqa"):
        w = synth.make(name, B=2)
        nb = gqa_decode_bytes(w["k"].shape[2], w["k"].shape[3], 2, int(w["cache_lens"].sum()))
        reps, t = timed(lambda: oracle.gqa_decode(w["q"], w["k"], w["v"], w["cache_lens"]))
        per[name] = {"sample": "2 of the 16 sequences", "runs": reps, "s_per_run": round(t / reps, 4),
                     "GB/s": round(nb * reps / t / 1e9, 3)}
    pw = synth.make("llama3_8b_gqa_prefill", B=1, Hq=4, Hkv=1)
    S = pw["q"].shape[1]
    rows = list(range(S - 1, -1, -64))  # 64 query rows spread over the sequence
    fl = sum(4 * 4 * 128 * (i + 1) for i in rows)
    reps, t = timed(lambda: oracle.gqa_prefill_causal(pw["q"], pw["k"], pw["v"], rows=rows))
    per["llama3_8b_gqa_prefill"] = {"sample": "1 sequence, 1 KV group (4 query heads), 64 of the 4096 query rows",
                                    "runs": reps, "s_per_run": round(t / reps, 4),
                                    "TFLOP/s": round(fl * reps / t / 1e12, 5)}
    mw = synth.make("minimind768_mla_decode", B=4)
    mb = (mw["c_kv"].shape[2] + mw["k_rope"].shape[2]) * 2 * int(mw["cache_lens"].sum())
    keys = ("q_nope", "q_rope", "w_uk", "w_uv", "c_kv", "k_rope", "cache_lens")
    reps, t = timed(lambda: oracle.mla_decode_decompressed(*(mw[k] for k in keys)))
    per["minimind768_mla_decode"] = {"sample": "4 of the 64 sequences, decompressed form (keys and values rebuilt)",
                                     "runs": reps, "s_per_run": round(t / reps, 4),
                                     "GB/s": round(mb * reps / t / 1e9, 4)}
    return {
        "value": headline,
        "unit": "GB/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": ("fp64 C oracle (oracle/oracle.c, OpenMP over output rows) on the full llama3_8b_gqa_decode "
                   "workload (float32 copies of the bf16 inputs; conversion included); per_config lists a "
                   "bounded sample of every configuration"),
        "per_config": per,
    }


if __name__ == "__main__":
    main()
