"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than its own formula: brute force,
closed forms, hand-derived fixtures, exact special cases and invariances. Chosen so that a
dropped term, a wrong sign or index, swapped gate/up, a transposed operand or a wrong tie
rule each fail at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

from tests.golden.fixtures import load_dequant_fixture
from tests.helpers import bf16_bits, host_layer

pytestmark = pytest.mark.usefixtures("oracle_lib")


# ---------------------------------------------------------------- routing: top-k selection

def brute_force_topk(l, K):
    """Subset of size K with the largest logit sum; equal sums -> lexicographically smallest
    index tuple (itertools yields tuples in lexicographic order, so keep the first maximum).
    Sums are exact (math.fsum), then ordered by (logit desc, index asc)."""
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(l)), K):
        s = math.fsum(l[i] for i in comb)
        if best_sum is None or s > best_sum:
            best, best_sum = comb, s
    return sorted(best, key=lambda i: (-l[i], i))


@pytest.mark.parametrize("E,K,seed", [(16, 2, 0), (16, 2, 1), (8, 3, 2), (10, 4, 3), (12, 1, 4),
                                      (9, 9, 5), (7, 6, 6)])
def test_topk_matches_brute_force_random(oracle_lib, E, K, seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        l = rng.normal(size=E)
        assert list(oracle_lib.topk(l, K)) == brute_force_topk(list(l), K)


@pytest.mark.parametrize("E,K", [(16, 2), (8, 3), (10, 5)])
def test_topk_brute_force_with_ties(oracle_lib, E, K):
    # integer-valued logits drawn from a tiny range force many ties, including across the
    # K-th boundary; brute force with exact sums decides them by the lowest index
    rng = np.random.default_rng(E * 100 + K)
    for _ in range(50):
        l = rng.integers(-2, 3, size=E).astype(np.float64)
        assert list(oracle_lib.topk(l, K)) == brute_force_topk(list(l), K)


def test_topk_adversarial(oracle_lib):
    assert list(oracle_lib.topk(np.zeros(16), 4)) == [0, 1, 2, 3]  # all equal -> lowest indices
    l = np.array([-0.0, 0.0, -1.0, 0.0])
    assert list(oracle_lib.topk(l, 1)) == [0]  # +0 == -0: the lower index wins
    assert list(oracle_lib.topk(l, 3)) == [0, 1, 3]
    l = np.array([1.0, 3.0, 2.0, 3.0, 2.0])  # duplicates straddling the K=3 boundary
    assert list(oracle_lib.topk(l, 3)) == [1, 3, 2]
    assert list(oracle_lib.topk(np.array([5.0, -np.inf, 7.0]), 2)) == [2, 0]


# ---------------------------------------------------------------- routing: weights

def test_route_weights_closed_forms(oracle_lib):
    rng = np.random.default_rng(7)
    for _ in range(20):
        E = int(rng.integers(2, 40))
        l = rng.normal(scale=2.0, size=E)
        # K = 1: a single expert gets weight exactly 1
        idx = oracle_lib.topk(l, 1)
        assert oracle_lib.route_weights(l, idx)[0] == 1.0
        # K = 2: w0 = 1 / (1 + exp(l1 - l0))
        idx = oracle_lib.topk(l, 2)
        w = oracle_lib.route_weights(l, idx)
        w0 = 1.0 / (1.0 + math.exp(l[idx[1]] - l[idx[0]]))
        assert abs(w[0] - w0) < 1e-15 and abs(w[1] - (1.0 - w0)) < 1e-15
        # K = E: renormalisation is the identity, so w is the library softmax, in selection order
        idx = oracle_lib.topk(l, E)
        w = oracle_lib.route_weights(l, idx)
        ref = scipy.special.softmax(l)[idx]
        np.testing.assert_allclose(w, ref, rtol=1e-14, atol=1e-16)
        # any K: weights are positive, sum to 1, and are invariant to a shift of all logits
        K = int(rng.integers(1, E + 1))
        idx = oracle_lib.topk(l, K)
        w = oracle_lib.route_weights(l, idx)
        assert np.all(w > 0) and abs(w.sum() - 1.0) < 1e-14
        assert np.all(np.diff(w) <= 0)  # ordered by logit, so weights are non-increasing
        w_shift = oracle_lib.route_weights(l + 123.25, idx)
        np.testing.assert_allclose(w_shift, w, rtol=1e-12)


def test_router_logits_one_hot_and_bias(oracle_lib):
    rng = np.random.default_rng(8)
    E, H = 6, 10
    R = rng.normal(size=(E, H)).astype(np.float32)
    bias = rng.normal(size=E).astype(np.float32)
    for j in range(H):
        x = np.zeros(H)
        x[j] = 1.0
        # one-hot input selects column j of the [E, H] router exactly (catches a transposed R)
        np.testing.assert_array_equal(oracle_lib.router_logits(x, R), R[:, j].astype(np.float64))
        np.testing.assert_array_equal(oracle_lib.router_logits(x, R, bias),
                                      R[:, j].astype(np.float64) + bias.astype(np.float64))


# ---------------------------------------------------------------- dequantisation (golden)

@pytest.mark.parametrize("name", ["dequant_4bit.txt", "dequant_8bit.txt"])
def test_dequant_golden(oracle_lib, name):
    fx = load_dequant_fixture(name)
    for (r, g), v in np.ndenumerate(fx["scale_values"]):
        assert oracle_lib.bf16_to_double(int(fx["scales"][r, g])) == v
    for (r, g), v in np.ndenumerate(fx["bias_values"]):
        assert oracle_lib.bf16_to_double(int(fx["biases"][r, g])) == v
    rows = [oracle_lib.dequant_row(fx["codes"], fx["scales"], fx["biases"], fx["cols"], fx["bits"],
                                   fx["group"], r) for r in range(fx["rows"])]
    assert fx["expect"], "fixture lists no expected values"
    for r, c, v in fx["expect"]:
        assert rows[r][c] == v, (name, r, c, rows[r][c], v)


def test_bf16_rounding_pins(oracle_lib):
    # ties to even at 8 significant bits
    assert oracle_lib.double_to_bf16(1.0) == 0x3F80
    assert oracle_lib.double_to_bf16(1.0 + 2 ** -8) == 0x3F80  # tie -> even (1.0)
    assert oracle_lib.double_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82  # tie -> even (1 + 2^-6)
    assert oracle_lib.double_to_bf16(1.0 + 2 ** -8 + 2 ** -30) == 0x3F81  # above the tie
    assert oracle_lib.double_to_bf16(-2.0) == 0xC000
    assert oracle_lib.double_to_bf16(0.0) == 0x0000
    # against the library conversion (float32 -> bf16 is round-to-nearest-even in torch)
    rng = np.random.default_rng(9)
    v = (rng.normal(size=4000) * np.exp(rng.uniform(-20, 20, size=4000))).astype(np.float32)
    ref = bf16_bits(torch.from_numpy(v).to(torch.bfloat16))
    got = np.array([oracle_lib.double_to_bf16(float(a)) for a in v], np.uint16)
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------- whole layer

def _tiny(E=16, K=2, H=256, I=128, Is=128, bits=4, seed=11, zipf=None):
    import synth
    shape = synth.MoeShape(H, E, K, I, Is, bits)
    return synth.make_stack(shape, 1, seed, "cpu", zipf_s=zipf)


def test_zero_point_codes_give_exactly_zero_output(oracle_lib):
    """Every code at the zero point (8 for 4-bit, 128 for 8-bit, bias = -zp*scale) dequantises to
    exactly 0, so every expert and the shared expert output exactly 0."""
    import oracle
    import synth
    for bits, zp_byte in ((4, 0x88), (8, 0x80)):
        st = _tiny(bits=bits)
        for name in ("w13_codes", "w2_codes", "s13_codes", "s2_codes"):
            st.tensors()[name].fill_(zp_byte)
        x = synth.make_x(st.shape, 3, 5)
        out = oracle.layer_forward(host_layer(st, 0), bf16_bits(x))
        assert np.all(out["y"] == 0.0)
        assert np.all(np.abs(out["w"].sum(1) - 1.0) < 1e-14)


def test_shared_gate_zero_gives_half(oracle_lib):
    import oracle
    import synth
    st = _tiny()
    st.shared_gate.zero_()
    out = oracle.layer_forward(host_layer(st, 0), bf16_bits(synth.make_x(st.shape, 2, 1)))
    assert np.all(out["gamma"] == 0.5)


def _closed_form_layer():
    """H = G = 64, E = 4, K = 2, I = Is = 64, scale 1 and bias -8 everywhere (w = q - 8, integers).
    Input x = e_0, so g_r and u_r are the codes of input column 0 of each gate/up row, router logits
    are column 0 of R, and each down row r has a single weight 1 at column (r mod I)."""
    import synth
    H, E, K, I = 64, 4, 2, 64
    shape = synth.MoeShape(H, E, K, I, I, 4)
    st = synth.make_stack(shape, 1, 3, "cpu")
    rng = np.random.default_rng(12)
    one = torch.tensor(1.0, dtype=torch.bfloat16)
    for sc, bi in ((st.w13_scales, st.w13_biases), (st.w2_scales, st.w2_biases),
                   (st.s13_scales, st.s13_biases), (st.s2_scales, st.s2_biases)):
        sc.fill_(one)
        bi.fill_(-8.0)
    n_exp = E + 1  # routed experts, then the shared expert
    a = rng.integers(-4, 5, size=(n_exp, I))  # gate values at input column 0
    b = rng.integers(-4, 5, size=(n_exp, I))  # up values at input column 0
    c1 = rng.integers(0, 16, size=(n_exp, 2 * I))  # codes of column 1 (high nibble of byte 0)
    for e in range(n_exp):
        w13 = st.w13_codes[0, e] if e < E else st.s13_codes[0, 0]
        w2 = st.w2_codes[0, e] if e < E else st.s2_codes[0, 0]
        w13.random_(0, 256, generator=torch.Generator().manual_seed(e))  # columns >= 2: anything
        for r in range(2 * I):
            q0 = int((a[e, r] if r < I else b[e, r - I]) + 8)
            w13[r, 0] = q0 | (int(c1[e, r]) << 4)
        w2.fill_(0x88)  # all zero weights
        for r in range(H):
            j = r % I
            byte = w2[r, j // 2].item()
            w2[r, j // 2] = (byte & 0xF0) | 9 if j % 2 == 0 else (byte & 0x0F) | (9 << 4)
    st.router.zero_()
    logit0 = np.array([0.5, -0.25, 1.0, 0.0], np.float32)
    st.router[0, :, 0] = torch.from_numpy(logit0)
    st.router[0, :, 1:] = torch.randn(E, H - 1)  # ignored by the one-hot input
    st.shared_gate.zero_()
    st.shared_gate[0, 0] = 0.3
    st.shared_gate[0, 1:] = 5.0
    x = torch.zeros(1, H, dtype=torch.bfloat16)
    x[0, 0] = 1.0
    return st, x, a, b, logit0


def test_closed_form_layer(oracle_lib):
    import oracle
    st, x, a, b, logit0 = _closed_form_layer()
    out = oracle.layer_forward(host_layer(st, 0), bf16_bits(x))
    sig = lambda v: 1.0 / (1.0 + math.exp(-v))
    # routing: logits 0.5, -0.25, 1.0, 0.0 -> top-2 = experts 2 then 0
    assert list(out["idx"][0]) == [2, 0]
    w2_ = 1.0 / (1.0 + math.exp(float(logit0[0]) - float(logit0[2])))
    assert abs(out["w"][0, 0] - w2_) < 1e-15
    gamma = sig(float(np.float32(0.3)))  # the gate vector is fp32
    assert abs(out["gamma"][0] - gamma) < 1e-15
    I = a.shape[1]
    h = lambda e, j: a[e, j] * sig(a[e, j]) * b[e, j]  # silu(gate) * up
    y_ref = np.array([w2_ * h(2, r % I) + (1 - w2_) * h(0, r % I) + gamma * h(4, r % I)
                      for r in range(st.shape.hidden)])
    np.testing.assert_allclose(out["y"][0], y_ref, rtol=1e-13, atol=1e-13)


def test_one_hot_input_reads_one_column(oracle_lib):
    """g and u of an expert for x = e_j are column j of the dequantised gate and up rows."""
    import oracle
    st = _tiny(H=128, I=64, Is=64, E=4)
    L = host_layer(st, 0).arrays
    H, I = 128, 64
    for j in (0, 1, 2, 63, 64, 127):
        x = np.zeros(H)
        x[j] = 1.0
        g, u = oracle.gate_up(L["w13_codes"][1], L["w13_scales"][1], L["w13_biases"][1], H, I, 4, 64, x)
        col = np.array([oracle.dequant_row(L["w13_codes"][1], L["w13_scales"][1], L["w13_biases"][1],
                                           H, 4, 64, r)[j] for r in range(2 * I)])
        np.testing.assert_array_equal(g, col[:I])
        np.testing.assert_array_equal(u, col[I:])


def _torch_dequant(codes, scales, biases, bits, group):
    """Independent unpacker in torch bit ops (pinned separately by the golden fixtures)."""
    c = torch.from_numpy(codes.astype(np.int64))
    if bits == 4:
        q = torch.stack([c & 0xF, c >> 4], dim=-1).reshape(c.shape[0], -1)
    else:
        q = c
    s = torch.from_numpy(scales.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    b = torch.from_numpy(biases.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    return q.to(torch.float64) * s.repeat_interleave(group, 1) + b.repeat_interleave(group, 1)


@pytest.mark.parametrize("bits", [4, 8])
def test_single_expert_is_textbook_swiglu_mlp(oracle_lib, bits):
    """E = K = 1 with no shared expert reduces to the SwiGLU MLP W2 (silu(W_gate x) * W_up x),
    evaluated here with torch's own linear and silu in float64."""
    import oracle
    import synth
    shape = synth.MoeShape(192, 1, 1, 128, 0, bits)
    st = synth.make_stack(shape, 1, 21, "cpu")
    x = synth.make_x(shape, 3, 2)
    L = host_layer(st, 0).arrays
    out = oracle.layer_forward(host_layer(st, 0), bf16_bits(x))
    w13 = _torch_dequant(L["w13_codes"][0], L["w13_scales"][0], L["w13_biases"][0], bits, 64)
    w2 = _torch_dequant(L["w2_codes"][0], L["w2_scales"][0], L["w2_biases"][0], bits, 64)
    xd = x.to(torch.float64)
    gate, up = torch.nn.functional.linear(xd, w13).split(128, dim=-1)
    ref = torch.nn.functional.linear(torch.nn.functional.silu(gate) * up, w2).numpy()
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.all(out["w"] == 1.0)


def test_layer_matches_library_dense_mixture(oracle_lib):
    """The full tiny layer equals a dense mixture built from library routines: torch.topk on the
    logits (no ties here), torch.softmax over the selected logits (renormalised softmax equals the
    softmax of the kept logits), torch linear/silu for every expert, torch.sigmoid for the gate."""
    import oracle
    import synth
    st = _tiny(seed=31)
    x = synth.make_x(st.shape, 4, 9)
    sh = st.shape
    out = oracle.layer_forward(host_layer(st, 0), bf16_bits(x))
    L = host_layer(st, 0).arrays
    xd = x.to(torch.float64)
    logits = xd @ torch.from_numpy(L["router"].astype(np.float64)).T
    vals, idx = torch.topk(logits, sh.top_k, dim=-1)
    w = torch.softmax(vals, dim=-1)

    def mlp(c13, s13, b13, c2, s2, b2, I):
        w13 = _torch_dequant(c13, s13, b13, sh.bits, 64)
        w2 = _torch_dequant(c2, s2, b2, sh.bits, 64)
        g, u = torch.nn.functional.linear(xd, w13).split(I, dim=-1)
        return torch.nn.functional.linear(torch.nn.functional.silu(g) * u, w2)

    dense = torch.stack([mlp(L["w13_codes"][e], L["w13_scales"][e], L["w13_biases"][e], L["w2_codes"][e],
                             L["w2_scales"][e], L["w2_biases"][e], sh.inter) for e in range(sh.num_experts)],
                        dim=1)  # [T, E, H]
    ref = (w.unsqueeze(-1) * torch.gather(dense, 1, idx.unsqueeze(-1).expand(-1, -1, sh.hidden))).sum(1)
    gamma = torch.sigmoid(xd @ torch.from_numpy(L["shared_gate"].astype(np.float64)))
    ref = ref + gamma.unsqueeze(-1) * mlp(L["s13_codes"], L["s13_scales"], L["s13_biases"],
                                          L["s2_codes"], L["s2_scales"], L["s2_biases"], sh.shared_inter)
    np.testing.assert_array_equal(out["idx"], idx.numpy())
    np.testing.assert_allclose(out["w"], w.numpy(), rtol=1e-13)
    np.testing.assert_allclose(out["y"], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_expert_permutation_invariance(oracle_lib):
    import oracle
    import synth
    st = _tiny(seed=41, zipf=1.1)
    x = synth.make_x(st.shape, 4, 3)
    base = oracle.layer_forward(host_layer(st, 0), bf16_bits(x))
    perm = torch.from_numpy(np.random.default_rng(3).permutation(st.shape.num_experts))
    for name in ("router", "router_bias", "w13_codes", "w13_scales", "w13_biases", "w2_codes",
                 "w2_scales", "w2_biases"):
        t = st.tensors()[name]
        t[0] = t[0][perm].clone()
    got = oracle.layer_forward(host_layer(st, 0), bf16_bits(x))
    np.testing.assert_array_equal(perm.numpy()[got["idx"]], base["idx"])
    # the softmax denominator is summed in expert-index order, so only rounding may differ
    np.testing.assert_allclose(got["y"], base["y"], rtol=1e-13, atol=1e-15)


def test_token_independence(oracle_lib):
    import oracle
    import synth
    st = _tiny(seed=51)
    x = synth.make_x(st.shape, 5, 4)
    L = host_layer(st, 0)
    full = oracle.layer_forward(L, bf16_bits(x))
    for t in range(5):
        one = oracle.layer_forward(L, bf16_bits(x[t:t + 1]))
        np.testing.assert_array_equal(one["y"][0], full["y"][t])
        np.testing.assert_array_equal(one["idx"][0], full["idx"][t])


def test_given_logits_mode(oracle_lib):
    """Selection from given fp32 logits follows those logits exactly (used to make both sides
    decide routing from identical logits)."""
    import oracle
    import synth
    st = _tiny(seed=61)
    x = synth.make_x(st.shape, 3, 4)
    L = host_layer(st, 0)
    given = np.zeros((3, 16), np.float32)
    given[0, [5, 9]] = [2.0, 1.0]
    given[1, :] = 1.0  # all tied -> experts 0, 1
    given[2, [3, 7]] = [-0.0, 0.0]
    given[2, [0, 1, 2, 4, 5, 6] + list(range(8, 16))] = -1.0
    out = oracle.layer_forward(L, bf16_bits(x), logits_in=given)
    assert [list(r) for r in out["idx"]] == [[5, 9], [0, 1], [3, 7]]
    assert abs(out["w"][1, 0] - 0.5) < 1e-16 and abs(out["w"][2, 1] - 0.5) < 1e-16


def test_rms_glue(oracle_lib):
    import oracle
    y = np.full(64, -3.0)
    assert np.all(oracle.rms_glue(y, 0.0) == 0xBF80)  # -3 / 3 = -1 exactly
    rng = np.random.default_rng(5)
    y = rng.normal(size=2048) * 7.0
    got = oracle.rms_glue(y, 1e-6)
    ref = bf16_bits(torch.from_numpy((y / np.sqrt(np.mean(y * y) + 1e-6)).astype(np.float32))
                    .to(torch.bfloat16))
    # fp64 vs fp32 quotient may straddle a rounding boundary: at most 1 ulp apart
    assert np.max(np.abs(got.astype(np.int32) - ref.astype(np.int32))) <= 1


@pytest.mark.parametrize("T,K,E,seed", [(1, 1, 1, 0), (4, 2, 16, 1), (33, 8, 256, 2), (130, 10, 512, 3), (7, 4, 4, 4)])
def test_group_pairs_properties(oracle_lib, T, K, E, seed):
    """The grouping is pinned by properties that determine it uniquely, checked with plain loops
    (no sort): counts are the histogram, offsets its exclusive prefix, perm a permutation whose
    segment e holds exactly the pairs selecting e in increasing pair order, pos its inverse."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, pos = oracle_lib.group_pairs(idx, E)
    flat = idx.reshape(-1)
    hist = [0] * E
    for e in flat:
        hist[int(e)] += 1
    assert list(counts) == hist
    run = 0
    for e in range(E):
        assert offsets[e] == run
        run += hist[e]
    assert offsets[E] == T * K
    assert sorted(perm.tolist()) == list(range(T * K))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]].tolist()
        assert all(flat[q] == e for q in seg)
        assert all(a < b for a, b in zip(seg, seg[1:]))
    for q in range(T * K):
        assert perm[pos[q]] == q


def test_group_pairs_planted_order_mistake(oracle_lib):
    """A grouping that is not stable (pairs of one expert out of pair order) violates the
    segment-order property the test above checks."""
    idx = np.array([[0, 1], [1, 0], [0, 1]], dtype=np.int32)
    counts, offsets, perm, pos = oracle_lib.group_pairs(idx, 2)
    assert perm[offsets[0]:offsets[1]].tolist() == [0, 3, 4]
    assert perm[offsets[1]:offsets[2]].tolist() == [1, 2, 5]
