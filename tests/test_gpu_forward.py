"""GPU tests of moe_layer_forward, the entry point that picks the decode or the batched path by
token count (the route boundary of moe_layer_path), through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_common import bf16_bits, check_routing_against_oracle, check_y, host_layer, need_gpu, oracle_layer

pytestmark = pytest.mark.gpu


def _moe():
    import quantized_moe_decode_router_amd as moe
    return moe


def _outputs(shape, T, dev):
    return (torch.empty(T, shape.hidden, dtype=torch.float32, device=dev),
            torch.empty(T, shape.top_k, dtype=torch.int32, device=dev),
            torch.empty(T, shape.top_k, dtype=torch.float32, device=dev),
            torch.empty(T, shape.num_experts, dtype=torch.float32, device=dev))


def run_forward(shape, layer, x, T, dev, ws=None, crossover=0):
    moe = _moe()
    y, idx, w, lg = _outputs(shape, T, dev)
    if ws is None:
        ws = moe.workspace(shape, T, moe.MOE_WS_FORWARD, dev)
    moe.moe_layer_forward(shape, layer, x, T, y, idx, w, lg, workspace=ws, crossover=crossover)
    assert moe.moe_read_status(ws) == 0
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


def run_direct(shape, layer, x, T, dev, path):
    moe = _moe()
    y, idx, w, lg = _outputs(shape, T, dev)
    if path == moe.MOE_PATH_DECODE:
        ws = moe.workspace(shape, T, moe.MOE_WS_DECODE, dev)
        moe.moe_layer_decode(shape, layer, x, T, y, idx, w, lg, workspace=ws)
    else:
        ws = moe.workspace(shape, T, moe.MOE_WS_BATCHED, dev)
        moe.moe_layer_batched(shape, layer, x, T, y, idx, w, lg, workspace=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


@pytest.mark.parametrize("T,crossover", [(1, 0), (2, 0), (3, 0), (8, 0), (9, 0), (23, 0), (5, 4), (4, 4),
                                         (8, 8)])
def test_forward_is_the_chosen_path(T, crossover):
    """moe_layer_forward returns exactly (bit for bit) what the path moe_layer_path names returns,
    and that is within the layer tolerance of the fp64 oracle."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.TINY.shape
    st = synth.make_stack(shape, 1, 4100 + T, dev)
    x = synth.make_x(shape, T, 41 + T, device=dev)
    path = moe.moe_layer_path(shape, T, crossover)
    want = moe.MOE_PATH_DECODE if T <= min(crossover or moe.MOE_DEFAULT_CROSSOVER, 8) else moe.MOE_PATH_BATCHED
    assert path == want
    got = run_forward(shape, st.layer(0), x, T, dev, crossover=crossover)
    ref_path = run_direct(shape, st.layer(0), x, T, dev, path)
    for a, b in zip(got, ref_path):
        np.testing.assert_array_equal(a, b)
    y, idx, w, lg = got
    Lh = host_layer(st, 0)
    ref = oracle_layer(st, 0, bf16_bits(x))
    differ = check_routing_against_oracle(idx, w, lg, ref, bf16_bits(x), Lh, shape.top_k)
    keep = [t for t in range(T) if t not in differ]
    assert keep
    err = check_y(y[keep], ref["y"][keep])
    print(f"forward T={T} crossover={crossover} path={'decode' if path == 0 else 'batched'}: "
          f"max|err|/RMS = {err:.2e}")


def test_forward_workspace_shared_across_the_boundary():
    """One MOE_WS_FORWARD workspace sized for the largest T serves decode and batched calls in any
    order: batched calls do not disturb the decode exchange words, and every call equals a call
    on a fresh workspace."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.QWEN35B_4BIT.shape
    st = synth.make_stack(shape, 1, 4200, dev)
    big = moe.workspace(shape, 64, moe.MOE_WS_FORWARD, dev)
    for T in (1, 64, 3, 9, 8, 2):
        x = synth.make_x(shape, T, 400 + T, device=dev)
        a = run_forward(shape, st.layer(0), x, T, dev, ws=big)
        b = run_forward(shape, st.layer(0), x, T, dev)
        for u, v in zip(a, b):
            np.testing.assert_array_equal(u, v)
