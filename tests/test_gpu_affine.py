"""GPU parity of the general affine quantisation w = s*q + b (MLX-style group quantisation, xix.ai
Swiftlet article, paragraph on lineage) against the fp64 oracle, through the C ABI.

The workloads' recipe sets every bias to the zero point (b = -8 s or -128 s), which makes the
kernels' bias terms exactly zero. Here every bias is drawn independently of its scale
(synth affine_bias: bf16(U[-0.25, 0.25]), both signs, mostly far from -zp*s), so the decode
path's bias term (b + zp s) times the group sum of the activation limbs, and the batched path's
fp16 rounding of s*q + b with a real bias, are both exercised."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_common import bf16_bits, check_routing_against_oracle, check_y, host_layer, need_gpu, oracle_layer

pytestmark = pytest.mark.gpu


def _moe():
    import quantized_moe_decode_router_amd as moe
    return moe


def _routing_outs(shape, T, dev):
    return (torch.empty(T, shape.hidden, dtype=torch.float32, device=dev),
            torch.empty(T, shape.top_k, dtype=torch.int32, device=dev),
            torch.empty(T, shape.top_k, dtype=torch.float32, device=dev),
            torch.empty(T, shape.num_experts, dtype=torch.float32, device=dev))


def _check_layer(st, l, x, y, idx, w, lg, name):
    Lh = host_layer(st, l)
    ref = oracle_layer(st, l, bf16_bits(x))
    T = x.shape[0]
    differ = check_routing_against_oracle(idx, w, lg, ref, bf16_bits(x), Lh, st.shape.top_k)
    keep = [t for t in range(T) if t not in differ]
    assert keep, "every token's routing is legitimately ambiguous; pick another seed"
    # the biases dominate these outputs: make sure the bias term is really exercised
    assert np.sqrt(np.mean(ref["y"] ** 2)) > 0
    err = check_y(y[keep], ref["y"][keep])
    print(f"{name}: max|err|/RMS = {err:.2e} over {len(keep)}/{T} tokens")


DECODE = [
    ("35b_4bit_T1", synth.QWEN35B_4BIT.shape, 1, 11),
    ("35b_4bit_T8", synth.QWEN35B_4BIT.shape, 8, 12),
    ("35b_8bit_T1", synth.QWEN35B_8BIT.shape, 1, 13),
    ("35b_8bit_T8", synth.QWEN35B_8BIT.shape, 8, 14),
    ("80b_4bit_T1", synth.QWEN80B_4BIT.shape, 1, 15),
    ("tiny_T4", synth.TINY.shape, 4, 16),
]


@pytest.mark.parametrize("name,shape,T,seed", DECODE, ids=[c[0] for c in DECODE])
def test_decode_affine_bias(name, shape, T, seed):
    dev = need_gpu()
    moe = _moe()
    st = synth.make_stack(shape, 1, 5000 + seed, dev, affine_bias=True)
    x = synth.make_x(shape, T, seed, device=dev)
    y, idx, w, lg = _routing_outs(shape, T, dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_DECODE, dev)
    moe.moe_layer_decode(shape, st.layer(0), x, T, y, idx, w, lg, workspace=ws)
    assert moe.moe_read_status(ws) == 0
    _check_layer(st, 0, x, y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy(), name)


@pytest.mark.parametrize("bits,T", [(4, 2), (8, 1)])
def test_stack_affine_bias_every_layer(bits, T):
    """An unchained 3-layer stack in one launch: every layer against the oracle."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.QWEN35B_4BIT.shape if bits == 4 else synth.QWEN35B_8BIT.shape
    L = 3
    st = synth.make_stack(shape, L, 5100 + bits, dev, affine_bias=True)
    x = synth.make_x(shape, T, 21, device=dev)
    H, K, E = shape.hidden, shape.top_k, shape.num_experts
    y = torch.empty(T, H, dtype=torch.float32, device=dev)
    y_all = torch.empty(L, T, H, dtype=torch.float32, device=dev)
    idx_all = torch.empty(L, T, K, dtype=torch.int32, device=dev)
    w_all = torch.empty(L, T, K, dtype=torch.float32, device=dev)
    lg_all = torch.empty(L, T, E, dtype=torch.float32, device=dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=L)
    moe.moe_stack_decode(shape, st, L, x, T, y, None, y_all, idx_all, w_all, lg_all, workspace=ws,
                         flags=moe.MOE_STACK_INDEPENDENT)
    assert moe.moe_read_status(ws) == 0
    for l in range(L):
        _check_layer(st, l, x, y_all[l].cpu().numpy(), idx_all[l].cpu().numpy(), w_all[l].cpu().numpy(),
                     lg_all[l].cpu().numpy(), f"stack {bits}-bit layer {l}")


BATCHED = [
    ("35b_4bit_T33_zipf", synth.QWEN35B_4BIT.shape, 33, 21, 1.1),
    ("35b_8bit_T33", synth.QWEN35B_8BIT.shape, 33, 22, None),  # h reaches ~1e5 here: scaled h halves
    ("tiny_T9", synth.TINY.shape, 9, 23, None),
]


@pytest.mark.parametrize("name,shape,T,seed,zipf", BATCHED, ids=[c[0] for c in BATCHED])
def test_batched_affine_bias(name, shape, T, seed, zipf):
    dev = need_gpu()
    moe = _moe()
    st = synth.make_stack(shape, 1, 5200 + seed, dev, zipf_s=zipf, affine_bias=True)
    x = synth.make_x(shape, T, seed, device=dev)
    y, idx, w, lg = _routing_outs(shape, T, dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_BATCHED, dev)
    moe.moe_layer_batched(shape, st.layer(0), x, T, y, idx, w, lg, workspace=ws)
    assert moe.moe_read_status(ws) == 0
    _check_layer(st, 0, x, y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy(), name)


def test_batched_affine_bias_full_size():
    """T = 512 on the Zipf-skewed 35B-shaped 4-bit layer with affine biases: the routing of every
    token in given-logits mode (bit-exact indices, weights to 1e-6), and y on a sample that holds
    tokens of every 64-row tile of the most loaded expert plus a seeded random draw."""
    import oracle
    dev = need_gpu()
    moe = _moe()
    wl = synth.QWEN35B_BATCHED
    shape, T = wl.shape, wl.tokens
    st = synth.make_stack(shape, 1, 5300, dev, zipf_s=wl.zipf_s, affine_bias=True)
    x = synth.make_x(shape, T, 5300, device=dev)
    y, idx, w, lg = _routing_outs(shape, T, dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_BATCHED, dev)
    moe.moe_layer_batched(shape, st.layer(0), x, T, y, idx, w, lg, workspace=ws)
    assert moe.moe_read_status(ws) == 0
    y, idx, w, lg = y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()
    for t in range(T):
        want = oracle.topk(lg[t].astype(np.float64), shape.top_k)
        assert list(idx[t]) == list(want), t
        np.testing.assert_allclose(w[t], oracle.route_weights(lg[t].astype(np.float64), want), rtol=0, atol=1e-6)
    hot = int(np.bincount(idx.reshape(-1), minlength=shape.num_experts).argmax())
    rows = [t for t in range(T) if hot in idx[t]]  # the hot expert's rows, in pair (token) order
    sample = sorted(set(rows[::64]) | set(rows[63::64]) |
                    set(np.random.default_rng(5).choice(T, size=8, replace=False).tolist()))
    xb = bf16_bits(x)
    Lh = host_layer(st, 0)
    ref = oracle.layer_forward(Lh, xb[sample])
    differ = check_routing_against_oracle(idx[sample], w[sample], lg[sample], ref, xb[sample], Lh, shape.top_k)
    keep = [i for i in range(len(sample)) if i not in differ]
    err = check_y(y[sample][keep], ref["y"][keep])
    print(f"batched affine T={T}: max|err|/RMS = {err:.2e} over {len(keep)} sampled tokens "
          f"({len(rows)} rows of expert {hot})")


def test_table_decode_affine_bias():
    """Every layer of an unchained expert-table decode (pinned host container) against the oracle."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.QWEN35B_4BIT.shape
    L, T = 2, 2
    st = synth.make_stack(shape, L, 5400, dev, affine_bias=True)
    x = synth.make_x(shape, T, 31, device=dev)
    stride = moe.moe_expert_stride(shape)
    n = L * shape.num_experts * stride
    buf = torch.empty(n + 4096, dtype=torch.uint8, pin_memory=True)
    off = (-buf.data_ptr()) % 4096
    cont = buf[off:off + n]
    moe.moe_pack_experts(shape, st, L, cont)
    torch.cuda.synchronize()
    table = (cont.data_ptr() + torch.arange(L * shape.num_experts, dtype=torch.int64) * stride).to(dev)
    H, K, E = shape.hidden, shape.top_k, shape.num_experts
    y = torch.empty(T, H, dtype=torch.float32, device=dev)
    y_all = torch.empty(L, T, H, dtype=torch.float32, device=dev)
    idx_all = torch.empty(L, T, K, dtype=torch.int32, device=dev)
    w_all = torch.empty(L, T, K, dtype=torch.float32, device=dev)
    lg_all = torch.empty(L, T, E, dtype=torch.float32, device=dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=L)
    moe.moe_stack_decode_table(shape, st, L, table, x, T, y, None, y_all, idx_all, w_all, lg_all, workspace=ws,
                               flags=moe.MOE_STACK_INDEPENDENT)
    assert moe.moe_read_status(ws) == 0
    for l in range(L):
        _check_layer(st, l, x, y_all[l].cpu().numpy(), idx_all[l].cpu().numpy(), w_all[l].cpu().numpy(),
                     lg_all[l].cpu().numpy(), f"table layer {l}")
