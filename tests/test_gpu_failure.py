"""Failure handling on the GPU, forced from the host so that every kernel still exits normally:
the sticky status word (a decode call that finds it set writes nothing), a tiny bound on the decode
kernel's waits (the wait gives up, MOE_ERR_TIMEOUT is reported, the device stays usable), and the
batched path's fp16 operand range (inside it the output matches the oracle; beyond it the call
reports MOE_ERR_UNSUPPORTED, while the decode path computes the same layer correctly)."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_common import CANARY, bf16_bits, check_routing_against_oracle, check_y, host_layer, need_gpu, oracle_layer

pytestmark = pytest.mark.gpu


def _moe():
    import quantized_moe_decode_router_amd as moe
    return moe


def _canary_like(shape, dev):
    return torch.full(shape, CANARY, dtype=torch.int32, device=dev)


@pytest.mark.parametrize("word", [5, 2, 1])
def test_sticky_status_blocks_decode(word):
    """A non-zero status word makes the decode and stack calls write nothing; moe_read_status
    returns the word; zero-filling the workspace recovers."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.QWEN35B_4BIT.shape
    L, T = 3, 2
    st = synth.make_stack(shape, L, 61, dev)
    x = synth.make_x(shape, T, 1, device=dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=L)
    ws.view(torch.int32)[0] = word
    yc = _canary_like((T, shape.hidden), dev)
    idx = _canary_like((L, T, shape.top_k), dev)
    moe.moe_stack_decode(shape, st, L, x, T, yc.view(torch.float32), topk_idx_all=idx, workspace=ws)
    assert moe.moe_read_status(ws) == word
    assert torch.all(yc == CANARY) and torch.all(idx == CANARY)
    wsd = moe.workspace(shape, T, moe.MOE_WS_DECODE, dev)
    wsd.view(torch.int32)[0] = word
    yd = _canary_like((T, shape.hidden), dev)
    moe.moe_layer_decode(shape, st.layer(0), x, T, yd.view(torch.float32), workspace=wsd)
    assert moe.moe_read_status(wsd) == word
    assert torch.all(yd == CANARY)
    ws.zero_()
    y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    moe.moe_stack_decode(shape, st, L, x, T, y, workspace=ws)
    assert moe.moe_read_status(ws) == 0 and torch.all(torch.isfinite(y))


def test_wait_bound_gives_up_and_device_recovers():
    """With the wait bound set to one poll (workspace word 2) the 40-layer stack's exchanges give
    up: MOE_ERR_TIMEOUT, every workgroup ends. A fresh workspace then gives the normal result."""
    dev = need_gpu()
    moe = _moe()
    wl = synth.QWEN35B_4BIT
    shape, L, T = wl.shape, wl.n_layers, 1
    st = synth.make_workload(wl, dev)
    x = synth.make_x(shape, T, 2, device=dev)
    ref = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    ws0 = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=L)
    moe.moe_stack_decode(shape, st, L, x, T, ref, workspace=ws0)
    assert moe.moe_read_status(ws0) == 0
    ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=L)
    ws.view(torch.int32)[2] = 1
    y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    moe.moe_stack_decode(shape, st, L, x, T, y, workspace=ws)
    assert moe.moe_read_status(ws) == moe.MOE_ERR_TIMEOUT
    # later calls on the failed workspace do nothing (sticky) and return promptly
    moe.moe_stack_decode(shape, st, L, x, T, y, workspace=ws)
    assert moe.moe_read_status(ws) == moe.MOE_ERR_TIMEOUT
    ws.zero_()
    moe.moe_stack_decode(shape, st, L, x, T, y, workspace=ws)
    assert moe.moe_read_status(ws) == 0
    assert torch.equal(y, ref)
    moe.moe_stack_decode(shape, st, L, x, T, y, workspace=ws0)
    assert moe.moe_read_status(ws0) == 0 and torch.equal(y, ref)


def _scaled_layer(shape, seed, dev, scale_exp, x_exp, T):
    """The tiny-shaped recipe with every scale multiplied by 2^scale_exp (biases stay -8 s, so
    s*q + b = s (q - 8) reaches 7 * 2^scale_exp * 0.02) and x multiplied by 2^x_exp; both scalings
    are exact in bf16. The layer's output is the recipe's times 2^(scale_exp + x_exp)-ish, so the
    oracle comparison is as meaningful as at the recipe's own magnitudes."""
    st = synth.make_stack(shape, 1, seed, dev)
    f = 2.0 ** scale_exp
    for t in (st.w13_scales, st.w13_biases, st.w2_scales, st.w2_biases, st.s13_scales, st.s13_biases,
              st.s2_scales, st.s2_biases):
        t.copy_((t.float() * f).to(torch.bfloat16))
    x = (synth.make_x(shape, T, seed, device=dev).float() * 2.0 ** x_exp).to(torch.bfloat16)
    return st, x


def _batched(moe, shape, st, x, T, dev):
    y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    idx = torch.empty(T, shape.top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, shape.top_k, dtype=torch.float32, device=dev)
    lg = torch.empty(T, shape.num_experts, dtype=torch.float32, device=dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_BATCHED, dev)
    moe.moe_layer_batched(shape, st.layer(0), x, T, y, idx, w, lg, workspace=ws)
    return moe.moe_read_status(ws), y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


@pytest.mark.parametrize("scale_exp,x_exp", [(10, -10), (-6, 6), (0, 3), (-6, 15)])
def test_batched_fp16_range_inside(scale_exp, x_exp):
    """Scales times 2^10 (weights up to ~140, x ~ 1e-3) or 2^-6 (weights ~ 2e-3, x ~ 64); x ~ 8 at
    the recipe's weights (h ~ 64 times the recipe's); weights times 2^-6 with x ~ 3e4 (|x| up to
    ~1e5, beyond fp16's 65504: scaled per token; h ~ 1e6: scaled per tile and group): status 0, y
    within the layer tolerance of the oracle."""
    dev = need_gpu()
    moe = _moe()
    shape, T = synth.QWEN35B_4BIT.shape, 12
    st, x = _scaled_layer(shape, 6100 + scale_exp, dev, scale_exp, x_exp, T)
    status, y, idx, w, lg = _batched(moe, shape, st, x, T, dev)
    assert status == 0
    ref = oracle_layer(st, 0, bf16_bits(x))
    differ = check_routing_against_oracle(idx, w, lg, ref, bf16_bits(x), host_layer(st, 0), shape.top_k)
    keep = [t for t in range(T) if t not in differ]
    assert keep
    check_y(y[keep], ref["y"][keep])


def test_batched_fp16_range_beyond():
    """Scales times 2^19 (weights s*q + b up to ~7e4 and biases to ~-8e4, beyond fp16's 65504): the
    batched call reports MOE_ERR_UNSUPPORTED (through moe_layer_forward too), and the decode path,
    which has no fp16 operands, computes the layer within the tolerance."""
    dev = need_gpu()
    moe = _moe()
    shape, T = synth.TINY.shape, 4
    scale_exp, x_exp = 19, -19
    st, x = _scaled_layer(shape, 6200, dev, scale_exp, x_exp, T)
    status = _batched(moe, shape, st, x, T, dev)[0]
    assert status == moe.MOE_ERR_UNSUPPORTED
    wsf = moe.workspace(shape, T, moe.MOE_WS_FORWARD, dev)
    y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    moe.moe_layer_forward(shape, st.layer(0), x, T, y, workspace=wsf, crossover=1)
    assert moe.moe_read_status(wsf) == moe.MOE_ERR_UNSUPPORTED
    # the decode path on the same layer and input
    yd = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
    idx = torch.empty(T, shape.top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, shape.top_k, dtype=torch.float32, device=dev)
    lg = torch.empty(T, shape.num_experts, dtype=torch.float32, device=dev)
    ws = moe.workspace(shape, T, moe.MOE_WS_DECODE, dev)
    moe.moe_layer_decode(shape, st.layer(0), x, T, yd, idx, w, lg, workspace=ws)
    assert moe.moe_read_status(ws) == 0
    ref = oracle_layer(st, 0, bf16_bits(x))
    idx, w, lg = idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()
    differ = check_routing_against_oracle(idx, w, lg, ref, bf16_bits(x), host_layer(st, 0), shape.top_k)
    keep = [t for t in range(T) if t not in differ]
    assert keep
    assert np.all(np.isfinite(yd.cpu().numpy()))
    check_y(yd.cpu().numpy()[keep], ref["y"][keep])
