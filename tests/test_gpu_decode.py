"""GPU parity of the router and the decode path against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_common import (bf16_bits, check_routing_against_oracle, check_y, host_layer, need_gpu,
                              oracle_layer)

pytestmark = pytest.mark.gpu


def _moe():
    import quantized_moe_decode_router_amd as moe
    return moe


def run_decode(shape, layer, x, T, dev):
    moe = _moe()
    y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    idx = torch.empty(T, shape.top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, shape.top_k, dtype=torch.float32, device=dev)
    lg = torch.empty(T, shape.num_experts, dtype=torch.float32, device=dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_DECODE, dev)
    moe.moe_layer_decode(shape, layer, x, T, y, idx, w, lg, workspace=ws)
    assert moe.moe_read_status(ws) == 0
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


# ------------------------------------------------------------------------------ router

ROUTE_SHAPES = {
    "tiny": synth.TINY.shape,
    "35b": synth.QWEN35B_4BIT.shape,
    "80b": synth.QWEN80B_4BIT.shape,
}


@pytest.mark.parametrize("name,T", [("tiny", 4), ("35b", 1), ("35b", 33), ("80b", 7)])
def test_route_given_logits_bit_exact(name, T):
    """With identical fp32 logits (made by the oracle), the GPU's indices equal the oracle's
    exactly and its weights agree to 1e-6."""
    import oracle
    dev = need_gpu()
    moe = _moe()
    shape = ROUTE_SHAPES[name]
    st = synth.make_stack(shape, 1, 100 + T, "cpu")
    x = synth.make_x(shape, T, 7)
    Lh = host_layer(st, 0)
    ref = oracle.layer_forward(Lh, bf16_bits(x))
    lg32 = ref["logits"].astype(np.float32)
    logits = torch.from_numpy(lg32).to(dev)
    idx = torch.empty(T, shape.top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, shape.top_k, dtype=torch.float32, device=dev)
    moe.moe_route(shape, None, None, T, logits, idx, w, flags=moe.MOE_ROUTE_LOGITS_IN)
    torch.cuda.synchronize()
    for t in range(T):
        want = oracle.topk(lg32[t].astype(np.float64), shape.top_k)
        assert list(idx[t].cpu().numpy()) == list(want)
        np.testing.assert_allclose(w[t].cpu().numpy(), oracle.route_weights(lg32[t].astype(np.float64), want),
                                   rtol=0, atol=1e-6)


def test_route_adversarial_logits():
    """Ties, +-0, duplicates across the K-th boundary and all-equal rows decide exactly as the
    oracle's (logit desc, index asc) rule."""
    import oracle
    dev = need_gpu()
    moe = _moe()
    shape = synth.MoeShape(256, 16, 4, 128, 128, 4)
    rows = [np.zeros(16), np.full(16, -3.5),
            np.array([1, 3, 2, 3, 2, 2, 0, 0, 3, 1, 1, 1, 2, 2, 0, 0], float),
            np.array([-0.0, 0.0] * 8), np.array([0.0, -0.0] * 8)]
    rng = np.random.default_rng(4)
    rows += [rng.integers(-2, 3, size=16).astype(float) for _ in range(27)]
    lg = np.stack(rows).astype(np.float32)
    T = lg.shape[0]
    idx = torch.empty(T, 4, dtype=torch.int32, device=dev)
    w = torch.empty(T, 4, dtype=torch.float32, device=dev)
    moe.moe_route(shape, None, None, T, torch.from_numpy(lg).to(dev), idx, w, flags=moe.MOE_ROUTE_LOGITS_IN)
    torch.cuda.synchronize()
    for t in range(T):
        assert list(idx[t].cpu().numpy()) == list(oracle.topk(lg[t].astype(np.float64), 4)), t


@pytest.mark.parametrize("name,T", [("tiny", 4), ("35b", 2), ("80b", 3)])
def test_route_own_logits(name, T):
    import oracle
    dev = need_gpu()
    moe = _moe()
    shape = ROUTE_SHAPES[name]
    st = synth.make_stack(shape, 1, 200 + T, "cpu", zipf_s=1.1)
    x = synth.make_x(shape, T, 9)
    Lh = host_layer(st, 0)
    ref = oracle.layer_forward(Lh, bf16_bits(x))
    sd = st.to(dev).layer(0)
    logits = torch.empty(T, shape.num_experts, dtype=torch.float32, device=dev)
    idx = torch.empty(T, shape.top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, shape.top_k, dtype=torch.float32, device=dev)
    gamma = torch.empty(T, dtype=torch.float32, device=dev)
    moe.moe_route(shape, sd, x.to(dev), T, logits, idx, w, gamma)
    torch.cuda.synchronize()
    amb = check_routing_against_oracle(idx.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy(), ref,
                                       bf16_bits(x), Lh, shape.top_k)
    assert amb == 0
    np.testing.assert_allclose(gamma.cpu().numpy(), ref["gamma"], rtol=0, atol=1e-6)


# ------------------------------------------------------------------------------ one layer

DECODE_CASES = [
    ("tiny_T4", synth.TINY.shape, 4, 1),
    ("tiny_T1", synth.TINY.shape, 1, 2),
    ("35b_4bit_T1", synth.QWEN35B_4BIT.shape, 1, 3),
    ("35b_4bit_T8", synth.QWEN35B_4BIT.shape, 8, 4),
    ("80b_4bit_T1", synth.QWEN80B_4BIT.shape, 1, 5),
    ("35b_8bit_T1", synth.QWEN35B_8BIT.shape, 1, 6),
    ("35b_8bit_T3", synth.QWEN35B_8BIT.shape, 3, 7),
    ("k1_no_shared", synth.MoeShape(512, 8, 1, 256, 0, 4), 5, 8),
    ("k_eq_e", synth.MoeShape(256, 4, 4, 64, 64, 8), 2, 9),
    ("wide_inter", synth.MoeShape(1024, 32, 6, 1024, 256, 4), 3, 10),
]


@pytest.mark.parametrize("name,shape,T,seed", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_layer_decode_parity(name, shape, T, seed):
    dev = need_gpu()
    st = synth.make_stack(shape, 1, 1000 + seed, dev, zipf_s=None)
    x = synth.make_x(shape, T, seed, device=dev)
    Lh = host_layer(st, 0)
    ref = oracle_layer(st, 0, bf16_bits(x))
    y, idx, w, lg = run_decode(shape, st.layer(0), x, T, dev)
    amb = check_routing_against_oracle(idx, w, lg, ref, bf16_bits(x), Lh, shape.top_k)
    assert amb == 0, "seed gives a near-tie in routing; pick another"
    err = check_y(y, ref["y"])
    print(f"{name}: max|err|/RMS = {err:.2e}")


def test_decode_edge_values():
    """All codes at the zero point -> y exactly 0; run twice -> bitwise identical output."""
    dev = need_gpu()
    shape = synth.QWEN35B_4BIT.shape
    st = synth.make_stack(shape, 1, 77, dev)
    x = synth.make_x(shape, 2, 3, device=dev)
    y1 = run_decode(shape, st.layer(0), x, 2, dev)[0]
    y2 = run_decode(shape, st.layer(0), x, 2, dev)[0]
    assert np.array_equal(y1, y2)
    for t in (st.w13_codes, st.w2_codes, st.s13_codes, st.s2_codes):
        t.fill_(0x88)
    y0 = run_decode(shape, st.layer(0), x, 2, dev)[0]
    assert np.all(y0 == 0.0)


def test_decode_tokens_are_independent():
    """Row t of a T=8 call equals a T=1 call on token t (bitwise: each token's work is the same)."""
    dev = need_gpu()
    shape = synth.QWEN35B_4BIT.shape
    st = synth.make_stack(shape, 1, 78, dev)
    x = synth.make_x(shape, 8, 4, device=dev)
    y8 = run_decode(shape, st.layer(0), x, 8, dev)[0]
    for t in (0, 5, 7):
        y1 = run_decode(shape, st.layer(0), x[t:t + 1].contiguous(), 1, dev)[0]
        assert np.array_equal(y1[0], y8[t])


# ------------------------------------------------------------------------------ stacks

def _stack_run(shape, st, n_layers, x, T, dev, phased=False):
    moe = _moe()
    H, K, E = shape.hidden, shape.top_k, shape.num_experts
    out = dict(y=torch.empty(T, H, dtype=torch.float32, device=dev),
               x_all=torch.empty(n_layers, T, H, dtype=torch.bfloat16, device=dev),
               y_all=torch.empty(n_layers, T, H, dtype=torch.float32, device=dev),
               idx_all=torch.empty(n_layers, T, K, dtype=torch.int32, device=dev),
               w_all=torch.empty(n_layers, T, K, dtype=torch.float32, device=dev),
               logits_all=torch.empty(n_layers, T, E, dtype=torch.float32, device=dev))
    ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev)
    fn = moe.moe_stack_decode_phased if phased else moe.moe_stack_decode
    fn(shape, st, n_layers, x, T, out["y"], out["x_all"], out["y_all"], out["idx_all"], out["w_all"],
       out["logits_all"], workspace=ws)
    assert moe.moe_read_status(ws) == 0
    return out


def test_stack_phased_equals_persistent():
    dev = need_gpu()
    shape = synth.QWEN35B_4BIT.shape
    st = synth.make_stack(shape, 3, 5, dev)
    x = synth.make_x(shape, 2, 1, device=dev)
    a = _stack_run(shape, st, 3, x, 2, dev)
    b = _stack_run(shape, st, 3, x, 2, dev, phased=True)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def _glue_ref(y):
    """The inter-layer RMS glue evaluated in fp32 by numpy (x_next = bf16(y / sqrt(mean y^2 + eps)))."""
    y = y.astype(np.float32)
    inv = np.float32(1.0) / np.sqrt(np.mean(y * y, dtype=np.float32) + np.float32(1e-6))
    return bf16_bits(torch.from_numpy(y * inv).to(torch.bfloat16))


def _stack_layer_check(l, gx, xo, out, ref, Lh, K):
    """One layer of the chained comparison. The two chains' inputs may differ by one bf16 ulp in
    a few elements (fp32 vs fp64 glue); that difference is added to the logit bound and loosens
    the weight tolerance. Returns False when the routing is legitimately ambiguous and differs."""
    from tests.gpu_common import W_TOL, logit_bound, topk_margin
    from tests.helpers import bits_to_f32
    xg = bits_to_f32(gx[0]).astype(np.float64)
    xr = bits_to_f32(xo[0]).astype(np.float64)
    R = Lh.arrays["router"].astype(np.float64)
    bnd = logit_bound(xr, Lh.arrays["router"], Lh.arrays.get("router_bias")).max()
    bnd += float((np.abs(R) @ np.abs(xg - xr)).max())
    idx = out["idx_all"][l].cpu().numpy()[0]
    w = out["w_all"][l].cpu().numpy()[0]
    if topk_margin(ref["logits"][0], K) > 2 * bnd:
        assert list(idx) == list(ref["idx"][0]), f"layer {l}: {idx} vs {ref['idx'][0]}"
    elif list(idx) != list(ref["idx"][0]):
        return False
    tol = W_TOL if np.array_equal(gx, xo) else 2.0 * bnd
    np.testing.assert_allclose(w, ref["w"][0], rtol=0, atol=tol)
    assert abs(float(w.astype(np.float64).sum()) - 1.0) <= 1e-6
    return True


@pytest.mark.parametrize("wl", [synth.QWEN35B_4BIT, synth.QWEN80B_4BIT, synth.QWEN35B_8BIT],
                         ids=["35b_4bit", "80b_4bit", "35b_8bit"])
def test_full_stack_against_chained_oracle(wl):
    """The full stack in the configuration the benchmark times (T = 1, every layer chained by the
    glue) against the oracle run layer by layer on its own chain (its own fp64 glue; no GPU value
    feeds the oracle). Every layer's input, routing and output are compared; the comparison stops
    at the first layer whose routing is legitimately ambiguous between the two chains."""
    import oracle
    dev = need_gpu()
    shape = wl.shape
    st = synth.make_workload(wl, dev)
    x = synth.make_x(shape, 1, 0, device=dev)
    out = _stack_run(shape, st, wl.n_layers, x, 1, dev)
    xo = bf16_bits(x)
    compared, worst, ndiff = 0, 0.0, 0
    for l in range(wl.n_layers):
        Lh = host_layer(st, l)
        ref = oracle.layer_forward(Lh, xo)
        gx = bf16_bits(out["x_all"][l])
        d = np.abs(gx.astype(np.int32) - xo.astype(np.int32))
        assert d.max() <= 1, f"layer {l}: inputs differ by more than one bf16 ulp"
        ndiff += int((d > 0).sum())
        if not _stack_layer_check(l, gx, xo, out, ref, Lh, shape.top_k):
            print(f"layer {l}: routing legitimately ambiguous between the chains; stopping")
            break
        worst = max(worst, check_y(out["y_all"][l].cpu().numpy(), ref["y"]))
        if l + 1 < wl.n_layers:  # the GPU glue itself, against numpy fp32, to one ulp
            g = _glue_ref(out["y_all"][l].cpu().numpy()[0])
            nx = bf16_bits(out["x_all"][l + 1])[0]
            assert np.max(np.abs(g.astype(np.int32) - nx.astype(np.int32))) <= 1
        xo = oracle.rms_glue(ref["y"][0], 1e-6)[None, :]
        compared += 1
    print(f"{wl.name}: {compared}/{wl.n_layers} layers compared, worst max|err|/RMS {worst:.2e}, "
          f"{ndiff} input elements 1 ulp apart")
    assert compared >= wl.n_layers // 2
    assert torch.equal(out["y"], out["y_all"][-1])
