"""The allocation-free decode entry point (moe_stack_decode_static) through the C ABI: bit for bit
the results of moe_stack_decode with a workspace, on two calls in a row (the second smaller), with
and without MOE_STATIC_RESET, and a request beyond its fixed scratch refused on the host."""
import pytest
import torch

import synth
from tests.gpu_common import need_gpu

pytestmark = pytest.mark.gpu


def _moe():
    import quantized_moe_decode_router_amd as moe
    return moe


def _outs(shape, L, T, dev):
    H, K, E = shape.hidden, shape.top_k, shape.num_experts
    return dict(y=torch.empty(T, H, dtype=torch.float32, device=dev),
                x_all=torch.empty(L, T, H, dtype=torch.bfloat16, device=dev),
                y_all=torch.empty(L, T, H, dtype=torch.float32, device=dev),
                idx_all=torch.empty(L, T, K, dtype=torch.int32, device=dev),
                w_all=torch.empty(L, T, K, dtype=torch.float32, device=dev),
                logits_all=torch.empty(L, T, E, dtype=torch.float32, device=dev))


def _args(o):
    return (o["y"], o["x_all"], o["y_all"], o["idx_all"], o["w_all"], o["logits_all"])


@pytest.mark.parametrize("bits", [4, 8])
def test_static_equals_workspace_decode_twice(bits):
    dev = need_gpu()
    moe = _moe()
    shape = synth.QWEN35B_4BIT.shape if bits == 4 else synth.QWEN35B_8BIT.shape
    st = synth.make_stack(shape, 6, 700 + bits, dev)
    for L, T, flags in ((6, 4, 0), (3, 1, 0), (2, 2, moe.MOE_STACK_INDEPENDENT),
                        (4, 1, moe.MOE_STATIC_RESET)):
        x = synth.make_x(shape, T, 10 * L + T, device=dev)
        ref = _outs(shape, L, T, dev)
        ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=L)
        moe.moe_stack_decode(shape, st, L, x, T, *_args(ref), workspace=ws, flags=flags & moe.MOE_STACK_INDEPENDENT)
        assert moe.moe_read_status(ws) == 0
        got = _outs(shape, L, T, dev)
        moe.moe_stack_decode_static(shape, st, L, x, T, *_args(got), flags=flags)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(got[k], ref[k]), (L, T, flags, k)


def test_static_refuses_beyond_its_scratch():
    dev = need_gpu()
    moe = _moe()
    shape = synth.QWEN35B_4BIT.shape
    st = synth.make_stack(shape, 1, 9, dev)
    x = synth.make_x(shape, 8, 1, device=dev)
    y = torch.empty(8, shape.hidden, dtype=torch.float32, device=dev)
    # 4096 layers at T = 8 need ~1.8 GB of exchange words, far beyond the 32 MiB scratch: refused
    # on the host before anything is launched or read
    with pytest.raises(moe.MoeError) as e:
        moe.moe_stack_decode_static(shape, st, 4096, x, 8, y)
    assert e.value.status == moe.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoeError) as e:
        moe.moe_stack_decode_static(shape, st, 1, x, 8, y, flags=4)
    assert e.value.status == moe.MOE_ERR_INVALID_ARG
    # and the scratch still serves a valid call afterwards
    moe.moe_stack_decode_static(shape, st, 1, x, 8, y)
    ref = torch.empty_like(y)
    ws = moe.workspace(shape, 8, moe.MOE_WS_STACK, dev, n_layers=1)
    moe.moe_stack_decode(shape, st, 1, x, 8, ref, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
