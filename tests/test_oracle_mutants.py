"""Plant plausible mistakes in a copy of the oracle (on the CPU) and require the pins to catch each.

Every mutation edits one spot of oracle.c in a temporary copy, builds it with gcc and runs the full
pin battery of oracle_pins.py against it; at least one pin must fail.  This shows the pins are not
the oracle's formulas typed twice."""
import os
import shutil

import pytest

import oracle
from tests import oracle_pins as pins

MUTATIONS = {
    # wrong head -> KV-group map (interleaved instead of contiguous groups)
    "group_index_mod": ("const int g = h / n_rep;", "const int g = h % Hkv;"),
    # wrong default scale (1/D instead of 1/sqrt(D))
    "scale_no_sqrt": ("scale = 1.0 / sqrt((double)D);", "scale = 1.0 / (double)D;"),
    # sign error inside the softmax
    "softmax_sign": ("denom += exp(s[t] - m);\n  for (int t = 0; t < n; ++t) {\n    double p = exp(s[t] - m) / denom;",
                     "denom += exp(m - s[t]);\n  for (int t = 0; t < n; ++t) {\n    double p = exp(m - s[t]) / denom;"),
    # causal window off by one (strictly earlier keys only)
    "causal_off_by_one": ("const int n = i + 1; /* keys 0..i */", "const int n = (i > 0) ? i : 1;"),
    # MLA: rope term dropped from the absorbed score
    "mla_drop_rope": ("      for (int j = 0; j < r; ++j) dot += q_abs[j] * (double)c[j];\n      for (int e = 0; e < dR; ++e) dot += (double)qr[e] * (double)kr[e];",
                      "      for (int j = 0; j < r; ++j) dot += q_abs[j] * (double)c[j];"),
    # MLA: W_UK read transposed when absorbing
    "mla_wuk_transposed": ("for (int i = 0; i < dn; ++i) a += (double)Wk[(long)i * r + j] * (double)qn[i];",
                           "for (int i = 0; i < dn; ++i) a += (double)Wk[((long)j * dn + i) % ((long)dn * r)] * (double)qn[i];"),
    # MLA: wrong default scale (latent width instead of nope+rope)
    "mla_scale_latent_width": ("if (scale <= 0.0) scale = 1.0 / sqrt((double)(dn + dR));\n  const int N = bh_list ? n_bh : B * H;\n#pragma omp parallel for schedule(dynamic)\n  for (int idx = 0; idx < N; ++idx) {\n    const int bh = bh_list ? bh_list[idx] : idx;\n    const int b = bh / H, h = bh % H;\n    if (b < 0 || b >= B) continue;\n    const int L = clamp_len(cache_lens[b], T_max);\n    double* q_abs",
                               "if (scale <= 0.0) scale = 1.0 / sqrt((double)(r + dR));\n  const int N = bh_list ? n_bh : B * H;\n#pragma omp parallel for schedule(dynamic)\n  for (int idx = 0; idx < N; ++idx) {\n    const int bh = bh_list ? bh_list[idx] : idx;\n    const int b = bh / H, h = bh % H;\n    if (b < 0 || b >= B) continue;\n    const int L = clamp_len(cache_lens[b], T_max);\n    double* q_abs"),
    # decode reads one token past the cache length
    "decode_reads_past_len": ("const int L = clamp_len(cache_lens[b], T_max);\n      double* s", "const int L = clamp_len(cache_lens[b] + 1, T_max);\n      double* s"),
    # cached prefill aligned top-left (new token i sees keys 0..i, ignoring the prefix)
    "cached_top_left": ("const int n = P + i + 1; /* keys 0 .. P + i */", "const int n = i + 1;"),
    # cached prefill attends the whole new chunk (no causal cut among the new tokens)
    "cached_no_causal_cut": ("const int n = P + i + 1; /* keys 0 .. P + i */", "const int n = P + nq;"),
    # MLA prefill: rope term dropped from the score
    "mla_prefill_drop_rope": ("          for (int e = 0; e < dR; ++e) dot += (double)qr[e] * (double)kr[e];\n          sc[t] = scale * dot;",
                              "          sc[t] = scale * dot;"),
    # MLA prefill: the causal cut ignores the prefix
    "mla_prefill_top_left": ("const int n = P + i + 1; /* keys 0 .. P + i */\n        for (int t = 0; t < n; ++t) {\n          const float* kr",
                             "const int n = i + 1;\n        for (int t = 0; t < n; ++t) {\n          const float* kr"),
    # RoPE: pairs taken as (x[j], x[j + d/2]) instead of consecutive elements
    "rope_half_split_pairs": ("const double re = (double)xr[2 * j], im = (double)xr[2 * j + 1];\n        o[2 * j] = re * cos(a) - im * sin(a);\n        o[2 * j + 1] = re * sin(a) + im * cos(a);",
                              "const double re = (double)xr[j], im = (double)xr[j + d / 2];\n        o[j] = re * cos(a) - im * sin(a);\n        o[j + d / 2] = re * sin(a) + im * cos(a);"),
    # RoPE: turned the other way
    "rope_direction": ("o[2 * j] = re * cos(a) - im * sin(a);\n        o[2 * j + 1] = re * sin(a) + im * cos(a);",
                       "o[2 * j] = re * cos(a) + im * sin(a);\n        o[2 * j + 1] = -re * sin(a) + im * cos(a);"),
    # RoPE: frequency exponent j/d instead of 2j/d
    "rope_exponent": ("pow(base, -2.0 * (double)j / (double)d)", "pow(base, -1.0 * (double)j / (double)d)"),
    # RoPE: a reflection instead of a rotation (sign slip in the second component)
    "rope_reflection": ("o[2 * j + 1] = re * sin(a) + im * cos(a);", "o[2 * j + 1] = re * sin(a) - im * cos(a);"),
    # value row taken from the wrong KV head (always head 0)
    "value_head_zero": ("const float* vbase = v + ((long)b * T_max * Hkv + g) * D;", "const float* vbase = v + ((long)b * T_max * Hkv + 0) * D;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    so = oracle.build(force=True, src=str(path), out=str(tmp_path / "libmutant.so"))
    lib = oracle.load(so)
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError as e:
            failures.append(pin.__name__)
    assert failures, f"mutation {name} was not caught by any pin"
