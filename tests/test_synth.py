"""Pins of the seeded input generator (shared by the oracle and the GPU path)."""
import json
import math
import os

import numpy as np
import pytest
import torch


def test_splitmix64_published_vector(syn):
    """First outputs of SplitMix64 seeded with 1234567, as printed with the generator's reference C code
    (Steele, Lea, Flood, OOPSLA 2014; the splitmix64.c that accompanies the xoshiro generators)."""
    L = syn.lib()
    got = [L.synth_splitmix64_at(1234567, i) for i in range(5)]
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]


def test_box_muller_pairs(syn):
    """n0^2 + n1^2 = -2 ln u1 for each pair, and the sample moments of N(0,1)."""
    L = syn.lib()
    s = (7 << 32) + 3
    for pair in range(50):
        n0, n1 = L.synth_normal_at(s, 2 * pair), L.synth_normal_at(s, 2 * pair + 1)
        u1 = ((L.synth_splitmix64_at(s, 2 * pair) >> 11) + 1) * 2.0**-53
        assert n0 * n0 + n1 * n1 == pytest.approx(-2 * math.log(u1), rel=1e-12)
    a = syn.normal_f32(7, 3, 1.0, (1 << 20,)).astype(np.float64)
    assert abs(a.mean()) < 5e-3 and abs(a.std() - 1) < 5e-3
    b = syn.bf16_to_f32(syn.normal_bf16(7, 3, 0.02, (1 << 20,))).astype(np.float64)
    assert abs(b.std() - 0.02) < 1e-4


def test_bf16_rounding_is_rne_like_torch(syn):
    rng = np.random.default_rng(0)
    f = rng.normal(size=4096).astype(np.float32)
    bits = f.view(np.uint32)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7FFFFF, 0x00008000], np.uint32).view(np.float32)
    f = np.concatenate([f, ties, np.array([np.inf, -np.inf, 0.0, -0.0], np.float32)])
    ours = np.array([syn.lib().synth_f32_to_bf16(float(v)) for v in f], np.uint16)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_fill_is_rounded_f32_fill(syn):
    f = syn.normal_f32(3, 5, 0.02, (4096,))
    b = syn.normal_bf16(3, 5, 0.02, (4096,))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_zipf_bias_probabilities(syn):
    b = syn.zipf_logit_bias(16, 1.2)
    p = np.exp(b.astype(np.float64))
    assert p.sum() == pytest.approx(1.0, rel=1e-6)
    assert np.all(np.diff(p) < 0)
    assert p[0] == pytest.approx(1 / sum(r**-1.2 for r in range(1, 17)), rel=1e-6)
    assert p[0] + p[1] > 0.5


def test_skewed_layer_routes_majority_to_few_experts(orc, syn):
    """The skewed Phi-3.5-shaped layer reproduces the hot-expert property: a few experts take more than
    half the tokens (HARMOEny article, section 2)."""
    figs = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
    sp = syn.spec("c3")
    L = syn.make_layer(sp, with_weights=False)
    idx, _ = orc.topk(orc.router_logits(L["x"], L["wg"], L["bias"]), sp.k)
    counts = np.bincount(idx.reshape(-1), minlength=sp.E)
    top3 = np.sort(counts)[::-1][:3].sum() / counts.sum()
    assert top3 > figs["hot_expert_share"]["value"]
    assert counts.max() > 4 * counts.sum() / sp.E


def test_config_table_shapes(syn):
    c = syn.CONFIGS
    assert (c["c1"].T, c["c1"].m, c["c1"].p, c["c1"].E, c["c1"].k) == (32, 256, 512, 8, 2)
    assert (c["c2"].T, c["c2"].m, c["c2"].p, c["c2"].E) == (16, 4096, 14336, 8)
    assert (c["c3"].T, c["c3"].p, c["c3"].E, c["c3"].zipf_s) == (256, 6400, 16, 1.2)
    assert (c["c4"].T, c["c4"].kind, c["c4"].w_dtype) == (8192, "swiglu", "bf16")
    assert (c["c5"].T, c["c5"].w_dtype, c["c5"].x_dtype) == (64, "i8", "bf16")
    assert [c[f"c{i}"].seed for i in range(1, 6)] == [0, 1, 2, 3, 4]
