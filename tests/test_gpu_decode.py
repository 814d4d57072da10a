"""GPU parity of the router and the decode path against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_common import (Guarded, bf16_bits, check_routing_against_oracle, check_y, host_layer, need_gpu,
                              oracle_layer)

pytestmark = pytest.mark.gpu


def _moe():
    import quantized_moe_decode_router_amd as moe
    return moe


def run_decode(shape, layer, x, T, dev):
    """One decode call with every output inside canary guard bands (checked after the call)."""
    moe = _moe()
    g = Guarded(dev)
    y = g.empty(T, shape.hidden)
    idx = g.empty(T, shape.top_k, dtype=torch.int32)
    w = g.empty(T, shape.top_k)
    lg = g.empty(T, shape.num_experts)
    ws = moe.workspace(shape, T, moe.MOE_WS_DECODE, dev)
    moe.moe_layer_decode(shape, layer, x, T, y, idx, w, lg, workspace=ws)
    assert moe.moe_read_status(ws) == 0
    g.check()
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


@pytest.mark.parametrize("E,K", [(128, 8), (256, 8), (512, 10), (1024, 16)])
def test_route_adversarial_logits_wide(E, K):
    """Several keys per lane (E > 64): few distinct logit values, so a lane often holds equal
    keys in several of its slots and several lanes tie at the maximum; +-0 rows; the selection is
    the oracle's (logit desc, index asc) order exactly."""
    import oracle
    dev = need_gpu()
    moe = _moe()
    shape = synth.MoeShape(256, E, K, 128, 128, 4)
    rng = np.random.default_rng(E + K)
    rows = [np.zeros(E), np.where(np.arange(E) % 3 == 0, -0.0, 0.0)]
    rows += [rng.integers(-2, 3, size=E).astype(float) for _ in range(20)]
    rows += [np.where(rng.random(E) < 0.02, 1.0, 0.0) for _ in range(6)]
    rows += [rng.standard_normal(E) for _ in range(4)]
    lg = np.stack(rows).astype(np.float32)
    T = lg.shape[0]
    idx = torch.empty(T, K, dtype=torch.int32, device=dev)
    w = torch.empty(T, K, dtype=torch.float32, device=dev)
    moe.moe_route(shape, None, None, T, torch.from_numpy(lg).to(dev), idx, w, flags=moe.MOE_ROUTE_LOGITS_IN)
    torch.cuda.synchronize()
    for t in range(T):
        want = oracle.topk(lg[t].astype(np.float64), K)
        assert list(idx[t].cpu().numpy()) == list(want), t
        np.testing.assert_allclose(w[t].cpu().numpy(), oracle.route_weights(lg[t].astype(np.float64), want),
                                   rtol=0, atol=1e-6)


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
    differ = check_routing_against_oracle(idx.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy(), ref,
                                          bf16_bits(x), Lh, shape.top_k)
    assert not differ
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
    ("k_eq_e", synth.MoeShape(256, 4, 4, 128, 128, 8), 2, 9),
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
    differ = check_routing_against_oracle(idx, w, lg, ref, bf16_bits(x), Lh, shape.top_k)
    keep = [t for t in range(T) if t not in differ]
    assert keep, "every token's routing is legitimately ambiguous; pick another seed"
    err = check_y(y[keep], ref["y"][keep])
    print(f"{name}: max|err|/RMS = {err:.2e} over {len(keep)}/{T} tokens")


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

def _stack_run(shape, st, n_layers, x, T, dev, flags=0):
    moe = _moe()
    H, K, E = shape.hidden, shape.top_k, shape.num_experts
    out = dict(y=torch.empty(T, H, dtype=torch.float32, device=dev),
               x_all=torch.empty(n_layers, T, H, dtype=torch.bfloat16, device=dev),
               y_all=torch.empty(n_layers, T, H, dtype=torch.float32, device=dev),
               idx_all=torch.empty(n_layers, T, K, dtype=torch.int32, device=dev),
               w_all=torch.empty(n_layers, T, K, dtype=torch.float32, device=dev),
               logits_all=torch.empty(n_layers, T, E, dtype=torch.float32, device=dev))
    ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=n_layers)
    moe.moe_stack_decode(shape, st, n_layers, x, T, out["y"], out["x_all"], out["y_all"], out["idx_all"],
                         out["w_all"], out["logits_all"], workspace=ws, flags=flags)
    assert moe.moe_read_status(ws) == 0
    return out


def test_stack_layers_equal_single_layer_calls():
    """An unchained stack computes, for every layer, exactly what a one-layer call computes."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.QWEN35B_4BIT.shape
    st = synth.make_stack(shape, 3, 5, dev)
    x = synth.make_x(shape, 2, 1, device=dev)
    out = _stack_run(shape, st, 3, x, 2, dev, flags=moe.MOE_STACK_INDEPENDENT)
    for l in range(3):
        y, idx, w, lg = run_decode(shape, st.layer(l), x, 2, dev)
        assert np.array_equal(out["y_all"][l].cpu().numpy(), y), l
        assert np.array_equal(out["idx_all"][l].cpu().numpy(), idx), l
        assert torch.equal(out["x_all"][l], x)
    assert torch.equal(out["y"], out["y_all"][2])


def test_repeated_calls_reuse_the_workspace():
    """Back-to-back calls on one workspace (the call counter advances) give identical results."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.QWEN35B_4BIT.shape
    st = synth.make_stack(shape, 4, 6, dev)
    x = synth.make_x(shape, 1, 2, device=dev)
    ws = moe.workspace(shape, 1, moe.MOE_WS_STACK, dev, n_layers=4)
    ys = []
    for _ in range(5):
        y = torch.empty(1, shape.hidden, dtype=torch.float32, device=dev)
        moe.moe_stack_decode(shape, st, 4, x, 1, y, workspace=ws)
        ys.append(y)
    assert moe.moe_read_status(ws) == 0
    for y in ys[1:]:
        assert torch.equal(y, ys[0])


def _glue_ref(y):
    """The inter-layer RMS glue evaluated in fp32 by numpy (x_next = bf16(y / sqrt(mean y^2 + eps)))."""
    y = y.astype(np.float32)
    inv = np.float32(1.0) / np.sqrt(np.mean(y * y, dtype=np.float32) + np.float32(1e-6))
    return bf16_bits(torch.from_numpy(y * inv).to(torch.bfloat16))


STACKS = [synth.QWEN35B_4BIT, synth.QWEN80B_4BIT, synth.QWEN35B_8BIT]
STACK_IDS = ["35b_4bit", "80b_4bit", "35b_8bit"]


@pytest.mark.parametrize("wl", STACKS, ids=STACK_IDS)
def test_full_stack_every_layer(wl):
    """The full stack in one launch with every layer taking the same input (unchained): every
    layer's routing and output against the oracle on identical inputs."""
    import oracle
    dev = need_gpu()
    moe = _moe()
    shape = wl.shape
    st = synth.make_workload(wl, dev)
    x = synth.make_x(shape, 1, 0, device=dev)
    out = _stack_run(shape, st, wl.n_layers, x, 1, dev, flags=moe.MOE_STACK_INDEPENDENT)
    xo = bf16_bits(x)
    worst = 0.0
    for l in range(wl.n_layers):
        Lh = host_layer(st, l)
        ref = oracle.layer_forward(Lh, xo)
        differ = check_routing_against_oracle(out["idx_all"][l].cpu().numpy(), out["w_all"][l].cpu().numpy(),
                                              out["logits_all"][l].cpu().numpy(), ref, xo, Lh, shape.top_k)
        if not differ:
            worst = max(worst, check_y(out["y_all"][l].cpu().numpy(), ref["y"]))
    print(f"{wl.name}: {wl.n_layers} layers, worst max|err|/RMS {worst:.2e}")


@pytest.mark.parametrize("wl", STACKS, ids=STACK_IDS)
def test_full_stack_chained(wl):
    """The chained stack exactly as the benchmark runs it (T = 1, layers joined by the glue)
    against the oracle run on its own chain with its own fp64 glue (no GPU value feeds the
    oracle). While the two chains' layer inputs are bitwise identical each layer is held to the
    layer tolerance; rounding can later make the chains' bf16 inputs differ, after which a
    per-layer tolerance no longer bounds the difference, so from there on only the GPU's own glue
    (against numpy fp32, to one bf16 ulp) and finiteness are checked."""
    import oracle
    dev = need_gpu()
    shape = wl.shape
    st = synth.make_workload(wl, dev)
    x = synth.make_x(shape, 1, 0, device=dev)
    out = _stack_run(shape, st, wl.n_layers, x, 1, dev)
    xo = bf16_bits(x)
    strict = 0
    for l in range(wl.n_layers):
        gx = bf16_bits(out["x_all"][l])
        if not np.array_equal(gx, xo):
            break
        Lh = host_layer(st, l)
        ref = oracle.layer_forward(Lh, xo)
        differ = check_routing_against_oracle(out["idx_all"][l].cpu().numpy(), out["w_all"][l].cpu().numpy(),
                                              out["logits_all"][l].cpu().numpy(), ref, xo, Lh, shape.top_k)
        if differ:
            break
        check_y(out["y_all"][l].cpu().numpy(), ref["y"])
        xo = oracle.rms_glue(ref["y"][0], 1e-6)[None, :]
        strict += 1
    y_all = out["y_all"].cpu().numpy()
    assert np.all(np.isfinite(y_all))
    for l in range(wl.n_layers - 1):
        g = _glue_ref(y_all[l][0])
        nx = bf16_bits(out["x_all"][l + 1])[0]
        assert np.max(np.abs(g.astype(np.int32) - nx.astype(np.int32))) <= 1, f"glue after layer {l}"
    assert torch.equal(out["y"], out["y_all"][-1])
    print(f"{wl.name}: {strict}/{wl.n_layers} chained layers on bitwise-identical inputs")
    assert strict >= 1


# ------------------------------------------------------------------------------ the largest shapes

# E = 1024 experts and top-16 are the library's limits. The decode kernel holds a token's h (K I + Is
# words), the router rows and the routed rows of its share in LDS, so not every such shape fits it:
# the candidates run from the largest down. A shape it cannot hold must be refused with
# MOE_ERR_UNSUPPORTED (before any launch) and routed to the batched path, which computes it; the
# largest shape it does take must match the oracle.
MAX_CANDIDATES = [
    (synth.MoeShape(2048, 1024, 16, 512, 512, 4), 8),
    (synth.MoeShape(2048, 1024, 16, 512, 512, 4), 4),
    (synth.MoeShape(2048, 1024, 16, 512, 512, 4), 1),
    (synth.MoeShape(2048, 1024, 16, 256, 256, 4), 1),
    (synth.MoeShape(1024, 1024, 16, 256, 256, 4), 1),
]


def test_decode_at_the_largest_shapes():
    dev = need_gpu()
    moe = _moe()
    stacks = {}
    refused, taken = [], None
    for shape, T in MAX_CANDIDATES:
        key = str(shape)
        if key not in stacks:
            stacks[key] = synth.make_stack(shape, 1, 4242, dev, zipf_s=None)
        st = stacks[key]
        x = synth.make_x(shape, T, 77, device=dev)
        if moe.moe_layer_path(shape, T, 8) == moe.MOE_PATH_DECODE:
            taken = (shape, T, st, x)
            break
        y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
        ws = moe.workspace(shape, T, moe.MOE_WS_DECODE, dev)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_layer_decode(shape, st.layer(0), x, T, y, workspace=ws)
        assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
        refused.append((shape, T, st, x))
    assert taken is not None, "the decode kernel takes none of the candidate shapes"
    shape, T, st, x = taken
    Lh = host_layer(st, 0)
    ref = oracle_layer(st, 0, bf16_bits(x))
    y, idx, w, lg = run_decode(shape, st.layer(0), x, T, dev)
    differ = check_routing_against_oracle(idx, w, lg, ref, bf16_bits(x), Lh, shape.top_k)
    keep = [t for t in range(T) if t not in differ]
    assert keep, "every token's routing is legitimately ambiguous; pick another seed"
    err = check_y(y[keep], ref["y"][keep])
    print(f"decode at {shape} T={T}: max|err|/RMS = {err:.2e}; refused: {[(str(s), t) for s, t, _, _ in refused]}")
    if refused:  # the largest refused shape, through the routing entry point (batched path)
        shape, T, st, x = refused[0]
        y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
        ws = moe.workspace(shape, T, moe.MOE_WS_FORWARD, dev)
        moe.moe_layer_forward(shape, st.layer(0), x, T, y, crossover=8, workspace=ws)
        ref = oracle_layer(st, 0, bf16_bits(x))
        err = check_y(y.cpu().numpy(), ref["y"])
        print(f"forward (batched) at {shape} T={T}: max|err|/RMS = {err:.2e}")
