#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass over the C-ABI compute entry points, each on its own synthetic workload
(shapes from the pages' configurations, i.i.d. N(0,1) inputs from fixed seeds):

  * attn_decode_gqa           Llama-3-8B-shaped GQA decode: B 32, Hq 32, Hkv 8, head_dim 128,
                              cache lengths uniform in [1024, 8192] (T_max 8192), bf16 in, fp32 out
  * attn_decode_mla_absorbed  MiniMind-768 MLA decode: B 64, 8 heads, nope 96, rope 48, v 96,
                              kv_lora_rank 128, cache 4096, bf16
  * attn_prefill_gqa_causal   Llama-3-8B-shaped causal prefill: B 4, S 4096, Hq 32, Hkv 8,
                              head_dim 128, bf16 in / out
  * attn_prefill_gqa_cached   the same heads, a 512-token chunk after a 3584-token cached
                              prefix in each of 4 sequences (chunked prefill), bf16 in / out
  * attn_prefill_mla_causal   MiniMind-768 MLA causal prefill: B 4, S 4096, 8 heads, nope 96,
                              rope 48, v 96, kv_lora_rank 128, bf16 in / out
  * attn_cache_append         the decode step's K/V write: each of the 32 Llama-3 sequences'
                              newest K and V rows written at position cache_lens - 1 (the rows
                              it already holds, so the decode inputs do not change)
  * attn_decode_gqa_append    the same write and the decode in one call (cache_lens - 1 cached
                              rows plus the new one: the same attention as attn_decode_gqa)
  * attn_decode_gqa_fp8kv     the Llama-3 decode shape and lengths over FP8 E4M3 caches (one
                              byte per element, one scale per cache)

The printed `value` is the GQA decode's KV-cache read rate (algorithmic bytes: every cached
K and V row read once per KV head, 2*Hkv*head_dim*2 bytes per cached position) divided by
the time of one attn_decode_gqa call (its streaming kernel and the small kernel that merges
the partial results), measured with HIP events around the call on the stream the library
launches on.  The other two entry points are reported under "parts".  Inputs are resident in
HBM before the timed region.  `cpu_baseline` times the fp64 CPU oracle (tests' checker, not
tuned) on the same decode workload on this host.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gqa_decode_llama3_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU oracle time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy per step (for counter calibration)")
    return ap.parse_args()


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

    t_gen = time.time()
    # ---- workloads (generated on the host from fixed seeds, then moved to HBM) ----
    dspec = synth.WORKLOADS["llama3_8b_gqa_decode"]
    dec_cpu = synth.make("llama3_8b_gqa_decode")
    dec = {k: v.to(dev) for k, v in dec_cpu.items()}
    B, Hq, D = dec["q"].shape
    T_max, Hkv = dec["k"].shape[1], dec["k"].shape[2]
    sum_len = int(dec_cpu["cache_lens"].clamp(0, T_max).sum())
    dec_bytes = 2 * Hkv * D * 2 * sum_len                      # K and V rows, bf16, once per KV head
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
    gen = torch.Generator(device=dev).manual_seed(8)
    f8_scale = 4.5 / 448.0
    f8_k = (torch.randn(B, T_max, Hkv, D, device=dev, generator=gen) / f8_scale).to(torch.float8_e4m3fn)
    f8_v = (torch.randn(B, T_max, Hkv, D, device=dev, generator=gen) / f8_scale).to(torch.float8_e4m3fn)
    f8_bytes = dec_bytes // 2                                 # one byte per cached element
    f8_out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    step_ws = torch.zeros(attn.attn_decode_gqa_append_workspace_bytes(B, Hq, Hkv, D, T_max, 0), dtype=torch.uint8,
                          device=dev)

    mspec = synth.WORKLOADS["minimind768_mla_decode"]
    mla_cpu = synth.make("minimind768_mla_decode")
    mla = {k: v.to(dev) for k, v in mla_cpu.items()}
    MB, H, dn = mla["q_nope"].shape
    dR = mla["q_rope"].shape[2]
    dv, r = mla["w_uv"].shape[1], mla["w_uv"].shape[2]
    MT = mla["c_kv"].shape[1]
    mla_len = int(mla_cpu["cache_lens"].clamp(0, MT).sum())
    mla_bytes = (r + dR) * 2 * mla_len                          # one [c_kv, k_rope] row per position
    mla_flops = H * (2 * (r + dR) + 2 * r) * mla_len
    mla_out = torch.empty(MB, H, dv, dtype=torch.float32, device=dev)
    mla_ws = torch.zeros(attn.attn_decode_mla_workspace_bytes(MB, H, r, dR, MT, 0), dtype=torch.uint8, device=dev)

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

    mpspec = synth.WORKLOADS["minimind768_mla_prefill"]
    mlp = {k: v.to(dev) for k, v in synth.make("minimind768_mla_prefill").items()}
    MPB, MPS, MPH, MPdn = mlp["q_nope"].shape
    MPdR = mlp["q_rope"].shape[3]
    MPdv, MPr = mlp["w_uv"].shape[1], mlp["w_uv"].shape[2]
    # MFMA work of the absorbed form: 2(r + dR) + 2r per unmasked (query, key) pair and head, plus
    # the query absorption (2 dn r) and the value up-projection (2 dv r) per new token and head
    mlp_flops = (MPB * MPH * MPS * (MPS + 1) // 2 * (2 * (MPr + MPdR) + 2 * MPr)
                 + MPB * MPS * MPH * 2 * MPr * (MPdn + MPdv))
    mlp_out = torch.empty(MPB, MPS, MPH, MPdv, dtype=torch.bfloat16, device=dev)
    copy_src = copy_dst = None
    if args.copy_calibration:
        copy_src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        copy_dst = torch.empty_like(copy_src)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    stream = torch.cuda.current_stream(dev)

    def run_decode():
        attn.attn_decode_gqa(dec["q"], dec["k"], dec["v"], dec["cache_lens"], out=dec_out, workspace=dec_ws)

    def run_mla():
        attn.attn_decode_mla_absorbed(mla["q_nope"], mla["q_rope"], mla["w_uk"], mla["w_uv"], mla["c_kv"],
                                      mla["k_rope"], mla["cache_lens"], out=mla_out, workspace=mla_ws)

    def run_prefill():
        attn.attn_prefill_gqa_causal(pre["q"], pre["k"], pre["v"], out=pre_out)

    def run_append():
        attn.attn_cache_append(app_k, dec["k"], app_v, dec["v"], app_pos)

    def run_step():
        attn.attn_decode_gqa_append(dec["q"], app_new_k, app_new_v, dec["k"], dec["v"], app_pos, out=step_out,
                                    workspace=step_ws)

    def run_fp8():
        attn.attn_decode_gqa_fp8kv(dec["q"], f8_k, f8_v, f8_scale, f8_scale, dec["cache_lens"], out=f8_out,
                                   workspace=dec_ws)

    def run_mla_prefill():
        attn.attn_prefill_mla_causal(mlp["q_nope"], mlp["q_rope"], mlp["w_uk"], mlp["w_uv"], mlp["c_kv"], mlp["k_rope"],
                                     out=mlp_out)

    def run_chunked():
        attn.attn_prefill_gqa_cached(chk["q"], chk["k"], chk["v"], chk["start_pos"], chk["q_lens"], out=chk_out)

    # prefill for new requests, then the decode steps of running ones (the order a serving
    # step takes); each part is timed on its own
    parts = [("prefill", run_prefill), ("chunked_prefill", run_chunked), ("mla_prefill", run_mla_prefill),
             ("mla_decode", run_mla), ("kv_append", run_append), ("gqa_decode", run_decode),
             ("gqa_decode_step", run_step), ("gqa_decode_fp8", run_fp8)]
    if args.copy_calibration:
        parts.append(("copy_1GiB", lambda: copy_dst.copy_(copy_src)))

    for _ in range(args.warmup):
        for _, fn in parts:
            fn()
    torch.cuda.synchronize()

    K = args.steps
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for name, _ in parts}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        for name, fn in parts:
            e0, e1 = ev[name][i]
            e0.record(stream)
            fn()
            e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {name: float(np.mean([a.elapsed_time(b) for a, b in ev[name]])) for name, _ in parts}

    dec_gbs = dec_bytes / (ms["gqa_decode"] * 1e-3) / 1e9
    mla_gbs = mla_bytes / (ms["mla_decode"] * 1e-3) / 1e9
    pre_tfs = pre_flops / (ms["prefill"] * 1e-3) / 1e12
    chk_tfs = chk_flops / (ms["chunked_prefill"] * 1e-3) / 1e12
    mlp_tfs = mlp_flops / (ms["mla_prefill"] * 1e-3) / 1e12

    dec_hash = source_hash("decode_gqa.hip", "attn_internal.h")
    traffic = measured_traffic("gqa_decode_bf16<128, 1, true, false>", dec_hash)

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
            "step": ("attn_prefill_gqa_causal, attn_prefill_gqa_cached, attn_prefill_mla_causal, "
                     "attn_decode_mla_absorbed, attn_cache_append, attn_decode_gqa, attn_decode_gqa_append, "
                     "attn_decode_gqa_fp8kv: one call each, in this order"),
            "tokens_per_step": {"gqa_decode": B, "mla_decode": MB, "prefill": PB * S, "chunked_prefill": chk_tokens,
                                "mla_prefill": MPB * MPS},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("gqa_decode_bf16<128, 1, true, false> + gqa_decode_merge: one attn_decode_gqa call "
                       "(two launches), timed together"),
            "achieved": round(dec_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dec_bytes,
            "avg_launch_ms": round(ms["gqa_decode"], 5),
        },
        "parts": {
            "gqa_decode": {"ms": round(ms["gqa_decode"], 5), "GB/s": round(dec_gbs, 1),
                           "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4), "TFLOP/s": round(dec_flops / (ms["gqa_decode"] * 1e-3) / 1e12, 2),
                           "tokens_per_s": round(B / (ms["gqa_decode"] * 1e-3), 1)},
            "mla_decode": {"ms": round(ms["mla_decode"], 5), "GB/s": round(mla_gbs, 1),
                           "hbm_frac": round(mla_gbs / HBM_PEAK_GBS, 4),
                           "algorithmic_bytes_per_launch": mla_bytes,
                           "TFLOP/s": round(mla_flops / (ms["mla_decode"] * 1e-3) / 1e12, 2),
                           "tokens_per_s": round(MB / (ms["mla_decode"] * 1e-3), 1),
                           "workload": f"minimind768_mla_decode: B={MB} H={H} nope={dn} rope={dR} v={dv} r={r} "
                                       f"cache={MT} seed={mspec['seed']}"},
            "prefill": {"ms": round(ms["prefill"], 5), "TFLOP/s": round(pre_tfs, 1),
                        "mfma_frac": round(pre_tfs / BF16_DENSE_PEAK_TFLOPS, 4),
                        "algorithmic_flops_per_launch": pre_flops,
                        "tokens_per_s": round(PB * S / (ms["prefill"] * 1e-3), 1),
                        "workload": f"llama3_8b_gqa_prefill: B={PB} S={S} Hq={PHq} Hkv={pre['k'].shape[2]} "
                                    f"head_dim={PD} seed={pspec['seed']} bf16 causal"},
            "chunked_prefill": {"ms": round(ms["chunked_prefill"], 5), "TFLOP/s": round(chk_tfs, 1),
                                "mfma_frac": round(chk_tfs / BF16_DENSE_PEAK_TFLOPS, 4),
                                "algorithmic_flops_per_launch": chk_flops,
                                "tokens_per_s": round(chk_tokens / (ms["chunked_prefill"] * 1e-3), 1),
                                "workload": f"llama3_8b_gqa_chunked_prefill: B={CB} chunk={CS} "
                                            f"start_pos={cspec['start_pos']} T_max={CT} Hq={CHq} "
                                            f"Hkv={chk['k'].shape[2]} head_dim={CD} seed={cspec['seed']} bf16"},
            "gqa_decode_fp8": {"ms": round(ms["gqa_decode_fp8"], 5),
                               "GB/s": round(f8_bytes / (ms["gqa_decode_fp8"] * 1e-3) / 1e9, 1),
                               "hbm_frac": round(f8_bytes / (ms["gqa_decode_fp8"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "algorithmic_bytes_per_launch": f8_bytes,
                               "tokens_per_s": round(B / (ms["gqa_decode_fp8"] * 1e-3), 1),
                               "workload": "llama3_8b_gqa_decode shape and lengths, K/V as FP8 E4M3 codes of "
                                           "N(0,1)/scale (device-generated, seed 8), scale 4.5/448"},
            "gqa_decode_step": {"ms": round(ms["gqa_decode_step"], 5),
                                "GB/s": round(dec_bytes / (ms["gqa_decode_step"] * 1e-3) / 1e9, 1),
                                "workload": "llama3_8b_gqa_decode with the newest rows as the new token "
                                            "(attn_decode_gqa_append: write + decode in one call)"},
            "kv_append": {"ms": round(ms["kv_append"], 5), "bytes_per_launch": app_bytes,
                          "GB/s": round(app_bytes / (ms["kv_append"] * 1e-3) / 1e9, 1),
                          "workload": f"llama3_8b_gqa_decode step write: B={B} rows of Hkv={Hkv} x {D} for K and V"},
            "mla_prefill": {"ms": round(ms["mla_prefill"], 5), "TFLOP/s": round(mlp_tfs, 1),
                            "mfma_frac": round(mlp_tfs / BF16_DENSE_PEAK_TFLOPS, 4),
                            "algorithmic_flops_per_launch": mlp_flops,
                            "tokens_per_s": round(MPB * MPS / (ms["mla_prefill"] * 1e-3), 1),
                            "workload": f"minimind768_mla_prefill: B={MPB} S={MPS} H={MPH} nope={MPdn} rope={MPdR} "
                                        f"v={MPdv} r={MPr} seed={mpspec['seed']} bf16 causal"},
        },
        "input_generation_s": round(t_gen, 2),
    }
    if args.copy_calibration:
        result["parts"]["copy_1GiB"] = {"ms": round(ms["copy_1GiB"], 5),
                                        "GB/s_read+write": round(2 * (1 << 30) / (ms["copy_1GiB"] * 1e-3) / 1e9, 1)}

    if not args.no_cpu_baseline:
        import oracle
        # the oracle as it stands, on the same decode workload (all 32 sequences), repeated until
        # about --cpu-seconds of host time
        reps, t_cpu = 0, 0.0
        t_begin = time.perf_counter()
        while True:
            t1 = time.perf_counter()
            oracle.gqa_decode(dec_cpu["q"], dec_cpu["k"], dec_cpu["v"], dec_cpu["cache_lens"])
            t_cpu += time.perf_counter() - t1
            reps += 1
            if time.perf_counter() - t_begin >= args.cpu_seconds or reps >= 50:
                break
        result["cpu_baseline"] = {
            "value": round(dec_bytes * reps / t_cpu / 1e9, 3),
            "unit": "GB/s",
            "cores": oracle.threads(),
            "kind": "oracle",
            "sample": (f"fp64 C oracle (oracle/oracle.c, OpenMP over (sequence, head) rows) on the full "
                       f"llama3_8b_gqa_decode workload, {reps} run(s) in {t_cpu:.2f} s (float32 copies of the "
                       f"bf16 inputs; conversion included)"),
        }
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
