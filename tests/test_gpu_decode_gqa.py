"""GQA / MQA / MHA decode on the GPU (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL_BF16, TOL_FP32, assert_close_rows, to_np

pytestmark = pytest.mark.gpu


def _attn():
    import mha_mla_kv_amd as attn
    return attn


def _run(inp, dev="cuda", **kw):
    attn = _attn()
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    lens = inp["cache_lens"].to(dev)
    out = attn.attn_decode_gqa(q, k, v, lens, **kw)
    torch.cuda.synchronize()
    return out


CASES = [
    # name, B, Hq, Hkv, D, T_max, lens, dtype, split
    ("minimind768_f32", 1, 8, 4, 96, 512, 512, "f32", 0),
    ("gqa4_bf16_ragged", 3, 32, 8, 128, 700, [700, 1, 333], "bf16", 128),
    ("gqa4_bf16_ragged_auto", 3, 32, 8, 128, 700, [700, 5, 333], "bf16", 0),
    ("mqa_bf16", 2, 32, 1, 128, 600, [600, 257], "bf16", 192),
    ("mha_bf16", 2, 8, 8, 128, 300, [300, 31], "bf16", 64),
    ("nrep64_bf16", 2, 64, 1, 128, 200, [200, 65], "bf16", 64),
    ("nrep2_d64_bf16", 2, 8, 4, 64, 260, [260, 100], "bf16", 64),
    ("nrep8_d96_bf16", 2, 16, 2, 96, 300, [299, 300], "bf16", 128),
    ("nrep3_bf16", 2, 12, 4, 128, 150, [150, 17], "bf16", 64),
    ("f32_nrep1_d128", 2, 4, 4, 128, 200, [200, 7], "f32", 64),
    ("f32_nrep4_d64", 2, 16, 4, 64, 300, [300, 129], "f32", 128),
    ("f32_nrep8_d128", 1, 16, 2, 128, 257, [257], "f32", 64),
    ("f32_nrep16_d96", 1, 16, 1, 96, 100, [100], "f32", 64),
    ("f32_nrep5_d96", 2, 10, 2, 96, 90, [90, 64], "f32", 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(case):
    name, B, Hq, Hkv, D, T, lens, dt, split = case
    inp = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, lens, dtype=dt, seed=11)
    print(f"[case] {name} B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} lens={lens} {dt} split={split}", flush=True)
    out = _run(inp, split_tokens=split)
    ref = oracle.gqa_decode(inp["q"], inp["k"], inp["v"], inp["cache_lens"])
    assert_close_rows(out, ref, TOL_FP32 if dt == "f32" else TOL_BF16, name)


def test_empty_and_clamped_lengths():
    B, Hq, Hkv, D, T = 4, 8, 2, 128, 100
    inp = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, [0, 100, 37, 0], seed=3)
    out = _run(inp, split_tokens=64)
    o = to_np(out)
    assert np.all(o[0] == 0) and np.all(o[3] == 0)
    ref = oracle.gqa_decode(inp["q"], inp["k"], inp["v"], inp["cache_lens"])
    assert_close_rows(out, ref, TOL_BF16, "empty rows")
    # lengths above T_max are clamped to T_max; negative lengths to 0
    inp2 = dict(inp)
    inp2["cache_lens"] = torch.tensor([-5, 1000, 37, 0], dtype=torch.int32)
    inp2["k"] = inp["k"].clone()
    inp2["v"] = inp["v"].clone()
    inp2["k"][1] = torch.randn_like(inp2["k"][1].float()).to(inp2["k"].dtype)
    inp2["v"][1] = torch.randn_like(inp2["v"][1].float()).to(inp2["v"].dtype)
    out2 = _run(inp2, split_tokens=64)
    ref2 = oracle.gqa_decode(inp2["q"], inp2["k"], inp2["v"], inp2["cache_lens"])
    assert np.all(to_np(out2)[0] == 0)
    assert_close_rows(out2, ref2, TOL_BF16, "clamped lengths")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_split_invariance_and_determinism(dt):
    B, Hq, Hkv, D, T = 2, 16, 4, 128, 1000
    inp = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, [1000, 613], dtype=dt, seed=5)
    outs = [to_np(_run(inp, split_tokens=s)) for s in (64, 128, 448, 1024, 0)]
    for o in outs[1:]:
        err = np.max(np.abs(o - outs[0])) / np.max(np.abs(outs[0]))
        assert err < (2e-6 if dt == "f32" else 2e-3), err
    again = to_np(_run(inp, split_tokens=128))
    assert np.array_equal(again, outs[1]), "not bitwise reproducible"


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_nan_poison_beyond_length_is_never_read(dt):
    B, Hq, Hkv, D, T = 2, 8, 2, 128, 300
    poisoned = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, [200, 77], dtype=dt, seed=9, poison=True)
    clean = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, [200, 77], dtype=dt, seed=9, poison=False)
    assert torch.isnan(poisoned["k"][0, 200:].float()).all()
    a = to_np(_run(poisoned, split_tokens=64))
    b = to_np(_run(clean, split_tokens=64))
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("bf16", 96), ("f32", 128), ("f32", 96)])
def test_saturating_selection_is_bit_exact(dt, D):
    """q = 8*1 and K[t*] = 8*1 with every other K = 0: the softmax weight of every other token
    underflows to exactly 0 in fp32, so the output must equal V[b, t*, h // n_rep] bitwise."""
    B, Hq, Hkv, T = 2, 16, 4, 640
    n_rep = Hq // Hkv
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    lens = torch.tensor([640, 300], dtype=torch.int32)
    q = torch.full((B, Hq, D), 8.0, dtype=dtype)
    v = torch.randn(B, T, Hkv, D, generator=torch.Generator().manual_seed(1)).to(dtype)
    for t_star in (0, 63, 64, 127, 128, 299, 639):
        k = torch.zeros(B, T, Hkv, D, dtype=dtype)
        for b in range(B):
            ts = min(t_star, int(lens[b]) - 1)
            k[b, ts] = 8.0
        out = to_np(_run({"q": q, "k": k, "v": v, "cache_lens": lens}, split_tokens=64))
        for b in range(B):
            ts = min(t_star, int(lens[b]) - 1)
            want = v[b, ts].float().numpy()  # [Hkv, D]
            for h in range(Hq):
                assert np.array_equal(out[b, h], want[h // n_rep]), (t_star, b, h)


def test_bf16_output():
    inp = synth.gqa_decode_inputs(2, 32, 8, 128, 300, [300, 100], seed=4)
    out = _run(inp, out_dtype=torch.bfloat16)
    assert out.dtype == torch.bfloat16
    ref = oracle.gqa_decode(inp["q"], inp["k"], inp["v"], inp["cache_lens"])
    assert_close_rows(out, ref, TOL_BF16, "bf16 out")


FULL = ["llama3_8b_gqa_decode", "kv_sweep_mha", "kv_sweep_gqa8", "kv_sweep_mqa", "minimind768_gqa_decode"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    """Full-size workloads in the launch configuration the benchmark times (default split);
    the oracle recomputes every head of a few sampled sequences."""
    spec = dict(synth.WORKLOADS[name])
    inp = synth.make(name)
    print(f"[case] {name} {spec}", flush=True)
    out = to_np(_run(inp))
    B = inp["q"].shape[0]
    picks = sorted(set([0, B - 1, B // 2]))
    for b in picks:
        sl = slice(b, b + 1)
        ref = oracle.gqa_decode(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["cache_lens"][sl])
        tol = TOL_FP32 if spec["dtype"] == "f32" else TOL_BF16
        assert_close_rows(out[sl], ref, tol, f"{name} b={b} L={int(inp['cache_lens'][b])}")


def test_workspace_reuse_across_calls_keeps_queue_counter_zero():
    """Calls that share one zero-filled workspace stay correct, also when the lengths and the
    sizes change between calls, and leave the work-queue counter (first 4 bytes) zero."""
    import mha_mla_kv_amd as attn
    B, Hq, Hkv, D, T = 6, 16, 4, 128, 3000
    ws = torch.zeros(attn.attn_decode_gqa_workspace_bytes(B, Hq, Hkv, D, T, 64), dtype=torch.uint8, device="cuda")
    runs = ((1, B, [3000, 1, 2999, 1500, 64, 0], 0), (2, B, [17, 3000, 3000, 2048, 1000, 999], 64),
            (3, B, [0, 0, 5, 3000, 2, 1], 0), (4, 3, [2500, 700, 3000], 128))
    for seed, b, lens, split in runs:
        inp = synth.gqa_decode_inputs(b, Hq, Hkv, D, T, lens, seed=seed)
        out = attn.attn_decode_gqa(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["cache_lens"].cuda(),
                                   split_tokens=split, workspace=ws)
        torch.cuda.synchronize()
        assert_close_rows(out, oracle.gqa_decode(inp["q"], inp["k"], inp["v"], inp["cache_lens"]), TOL_BF16,
                          f"reuse seed {seed}")
        assert int(ws[:4].view(torch.int32)[0]) == 0


@pytest.mark.parametrize("B", [1024, 1025])
def test_batch_limit_of_the_queue_schedule(B):
    """1024 sequences is the largest batch the device-side queue plans for; 1025 launches one
    workgroup per unit.  Both, with ragged and empty lengths over several chunks, match the oracle."""
    Hq, Hkv, D, T = 8, 2, 64, 300
    rng = np.random.default_rng(B)
    lens = rng.integers(0, T + 1, size=B).tolist()
    lens[0], lens[-1] = 0, T
    inp = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, lens, seed=B)
    print(f"[case] B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} split=64", flush=True)
    out = _run(inp, split_tokens=64)
    ref = oracle.gqa_decode(inp["q"], inp["k"], inp["v"], inp["cache_lens"])
    assert_close_rows(out, ref, TOL_BF16, f"B={B}")


@pytest.mark.parametrize("Hq,Hkv,B,T", [(32, 8, 16, 2048), (32, 1, 64, 4096)], ids=["gqa4", "mqa"])
def test_four_block_units_every_row(Hq, Hkv, B, T):
    """Problems with at least 16 blocks per compute unit run the queue with units of four
    blocks first; every output row (ragged lengths, some shorter than one block, one empty,
    one full) matches the oracle.  The MQA case also covers two 16-head blocks per unit."""
    D = 128
    rng = np.random.default_rng(B + Hkv)
    lens = rng.integers(1, T + 1, size=B).tolist()
    lens[0], lens[1], lens[-1] = 0, 40, T
    inp = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, lens, seed=11 + Hkv)
    print(f"[case] four-block units B={B} Hq={Hq} Hkv={Hkv} D={D} T={T} split=64", flush=True)
    out = _run(inp, split_tokens=64)
    ref = oracle.gqa_decode(inp["q"], inp["k"], inp["v"], inp["cache_lens"])
    assert_close_rows(out, ref, TOL_BF16, f"four-block units Hkv={Hkv}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_moving_max_matches_oracle(dt):
    """Scores that climb along the cache: every key of KV head g points along the group's query
    direction u_g, times 1 + 0.15 * (position // 32), plus 10% noise, so each wave's next
    32-position tile (four tiles on) beats its running max by about 10 (log2 units) -- more than
    the kernels' 2^8 slack -- and the reference moves with a rescale factor strictly between 0
    and 1, tile after tile; the units' partials then merge across very different maxima.  Keys
    of one tile stay close, so rows are smooth averages of V."""
    B, Hq, Hkv, D, T = 2, 16, 4, 128, 700
    inp = synth.gqa_decode_inputs(B, Hq, Hkv, D, T, [700, 513], dtype=dt, seed=13)
    g = torch.Generator().manual_seed(6)
    u = torch.randn(B, 1, Hkv, D, generator=g)
    q = u[:, 0].repeat_interleave(Hq // Hkv, dim=1) + 0.1 * torch.randn(B, Hq, D, generator=g)
    mag = 1.0 + 0.15 * (torch.arange(T) // 32).float()
    k = mag[None, :, None, None] * (u + 0.1 * torch.randn(B, T, Hkv, D, generator=g))
    dtype = inp["q"].dtype
    inp["q"] = q.to(dtype)
    inp["k"] = (inp["k"].float() * 0 + k).to(dtype)  # NaN poison past the lengths stays
    ref = oracle.gqa_decode(inp["q"], inp["k"], inp["v"], inp["cache_lens"])
    for split in (64, 256, 0):
        out = _run(inp, split_tokens=split)
        assert_close_rows(out, ref, TOL_FP32 if dt == "f32" else TOL_BF16, f"moving max {dt} split {split}")
