"""The seeded input generator: bit-exact against an exact integer model of SplitMix64, and the
recipe's value ranges. (Generator only: no MoE arithmetic is tested here.)"""
import numpy as np
import torch

import synth
from synth import rng


def test_hash_words_match_python_integers():
    key = rng.derive_key(1, 2, 3)
    got = rng.hash_words(key, 5, 64, "cpu").numpy().view(np.uint64)
    gamma = 0x9E3779B97F4A7C15
    ref = [rng.mix64_int((key + (5 + i + 1) * gamma) & ((1 << 64) - 1)) for i in range(64)]
    assert [int(v) for v in got] == ref


def test_fill_bytes_chunk_independent():
    a = torch.empty(1000, dtype=torch.uint8)
    rng.fill_bytes(a, 77)
    words = rng.hash_words(77, 0, 125, "cpu").view(torch.uint8)
    assert torch.equal(a, words[:1000])


def test_recipe_ranges():
    st = synth.make_workload(synth.TINY)
    s = st.w13_scales.float()
    assert float(s.min()) >= 0.0049 and float(s.max()) <= 0.0201
    assert torch.equal(st.w13_biases.float(), -8.0 * s)
    assert abs(float(st.router.std()) - 0.02) < 0.002
    x = synth.make_x(synth.TINY.shape, 64, 1)
    assert abs(float(x.float().std()) - 1.0) < 0.05
    nib = torch.cat([st.w13_codes & 0xF, st.w13_codes >> 4]).float()
    assert abs(float(nib.mean()) - 7.5) < 0.1
    st8 = synth.make_stack(synth.MoeShape(128, 4, 2, 64, 64, 8), 1, 3)
    assert torch.equal(st8.w2_biases.float(), -128.0 * st8.w2_scales.float())


def test_layers_depend_only_on_seed_and_index():
    a = synth.make_stack(synth.TINY.shape, 2, 5)
    b = synth.make_stack(synth.TINY.shape, 1, 5)
    for name, t in b.tensors().items():
        assert torch.equal(t[0], a.tensors()[name][0]), name


def test_zipf_bias_is_log_rank():
    st = synth.make_stack(synth.TINY.shape, 1, 5, zipf_s=1.1)
    b = st.router_bias[0].double()
    ranks = torch.exp(-b / 1.1).round()
    assert sorted(ranks.long().tolist()) == list(range(1, 17))


def test_affine_bias_recipe():
    """affine_bias draws the biases independently of the scales: both signs, within [-0.25, 0.25],
    mostly far from the zero point -zp * scale; scales and codes are those of the default recipe."""
    base = synth.make_stack(synth.TINY.shape, 1, 9)
    st = synth.make_stack(synth.TINY.shape, 1, 9, affine_bias=True)
    assert torch.equal(st.w13_scales, base.w13_scales) and torch.equal(st.w13_codes, base.w13_codes)
    for b, s in ((st.w13_biases, st.w13_scales), (st.w2_biases, st.w2_scales), (st.s2_biases, st.s2_scales)):
        bf = b.float()
        assert float(bf.min()) >= -0.25 and float(bf.max()) <= 0.25
        assert float((bf > 0).float().mean()) > 0.4 and float((bf < 0).float().mean()) > 0.4
        far = (bf + 8.0 * s.float()).abs() > 0.05
        assert float(far.float().mean()) > 0.7
