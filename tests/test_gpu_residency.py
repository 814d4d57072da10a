"""GPU parity of the expert-residency tier through the C ABI: the packed container against the
oracle's blocks, decode through an expert table (device container, pinned host container, a
mixed table) against the plain stack decode bit for bit and against the fp64 oracle, and a
multi-step decode loop whose cache decisions match the oracle's policy access by access while
every step's output stays identical to the all-resident decode."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import residency as R
from tests.gpu_common import bf16_bits, check_routing_against_oracle, check_y, host_layer, need_gpu, oracle_layer

pytestmark = pytest.mark.gpu


def _moe():
    import quantized_moe_decode_router_amd as moe
    return moe


def _container(moe, shape, st, n_layers, where):
    stride = moe.moe_expert_stride(shape)
    n = n_layers * shape.num_experts * stride
    if where == "host":
        buf = torch.empty(n + 4096, dtype=torch.uint8, pin_memory=True)
    else:
        buf = torch.empty(n + 4096, dtype=torch.uint8, device="cuda")
    off = (-buf.data_ptr()) % 4096
    c = buf[off:off + n]
    moe.moe_pack_experts(shape, st, n_layers, c)
    torch.cuda.synchronize()
    return buf, c, stride


def _no_routed(st):
    """The stack without its routed expert arrays: the table decode must not need them."""
    return dataclasses.replace(st, w13_codes=None, w13_scales=None, w13_biases=None, w2_codes=None,
                               w2_scales=None, w2_biases=None)


def _outs(shape, n_layers, T, dev):
    H, K, E = shape.hidden, shape.top_k, shape.num_experts
    return dict(y=torch.empty(T, H, dtype=torch.float32, device=dev),
                x_all=torch.empty(n_layers, T, H, dtype=torch.bfloat16, device=dev),
                y_all=torch.empty(n_layers, T, H, dtype=torch.float32, device=dev),
                idx_all=torch.empty(n_layers, T, K, dtype=torch.int32, device=dev),
                w_all=torch.empty(n_layers, T, K, dtype=torch.float32, device=dev),
                logits_all=torch.empty(n_layers, T, E, dtype=torch.float32, device=dev))


def _pieces(shape, stride):
    """Mask of the block bytes the layout defines (the padding between pieces is unspecified)."""
    lay = R.expert_block_layout(shape.hidden, shape.inter, shape.bits)
    m = np.zeros(stride, dtype=bool)
    for off, n in zip(lay["offsets"], lay["sizes"]):
        m[off:off + n] = True
    return m


def _landing(shape, n_layers, T, stride, dev):
    n = n_layers * T * shape.top_k * stride
    buf = torch.empty(n + 4096, dtype=torch.uint8, device=dev)
    off = (-buf.data_ptr()) % 4096
    return buf[off:off + n]


def _run(moe, shape, st, n_layers, x, T, dev, table=None, flags=0, ws=None, landing=None):
    o = _outs(shape, n_layers, T, dev)
    if ws is None:
        ws = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=n_layers)
    args = (x, T, o["y"], o["x_all"], o["y_all"], o["idx_all"], o["w_all"], o["logits_all"])
    if table is None:
        moe.moe_stack_decode(shape, st, n_layers, *args, workspace=ws, flags=flags)
    else:
        moe.moe_stack_decode_table(shape, _no_routed(st), n_layers, table, *args, workspace=ws, flags=flags,
                                   landing=landing)
    assert moe.moe_read_status(ws) == 0
    return {k: v.cpu() for k, v in o.items()}


def _same(a, b):
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("where", ["device", "host"])
def test_pack_experts_matches_oracle_blocks(where):
    dev = need_gpu()
    moe = _moe()
    shape = synth.TINY.shape
    Lyr = 3
    st = synth.make_stack(shape, Lyr, 41, dev)
    _, c, stride = _container(moe, shape, st, Lyr, where)
    assert stride == R.expert_block_layout(shape.hidden, shape.inter, shape.bits)["stride"]
    got = c.cpu().numpy().reshape(Lyr * shape.num_experts, stride)
    h = {k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy() for k, v in st.tensors().items()}
    lay = R.expert_block_layout(shape.hidden, shape.inter, shape.bits)
    piece = np.zeros(stride, dtype=bool)  # the bytes the layout defines (padding is unspecified)
    for off, n in zip(lay["offsets"], lay["sizes"]):
        piece[off:off + n] = True
    for l in range(Lyr):
        for e in range(shape.num_experts):
            want = R.pack_block(h["w13_codes"][l, e], h["w13_scales"][l, e].view(np.uint16),
                                h["w13_biases"][l, e].view(np.uint16), h["w2_codes"][l, e],
                                h["w2_scales"][l, e].view(np.uint16), h["w2_biases"][l, e].view(np.uint16),
                                shape.hidden, shape.inter, shape.bits)
            assert np.array_equal(got[l * shape.num_experts + e][piece], want[piece]), (l, e)


TABLE_CASES = [
    ("tiny_T4_device", synth.TINY.shape, 3, 4, "device"),
    ("tiny_T1_host", synth.TINY.shape, 3, 1, "host"),
    ("tiny_T8_mixed", synth.TINY.shape, 2, 8, "mixed"),
    ("q35b_T1_mixed", synth.QWEN35B_4BIT.shape, 3, 1, "mixed"),
    ("q35b_T3_host", synth.QWEN35B_4BIT.shape, 2, 3, "host"),
    ("q35b_8bit_T2_mixed", synth.QWEN35B_8BIT.shape, 2, 2, "mixed"),
    ("q35b_8bit_T1_host", synth.QWEN35B_8BIT.shape, 2, 1, "host"),
    ("q80b_T2_mixed", synth.QWEN80B_4BIT.shape, 2, 2, "mixed"),
    # an odd expert count stages the table row in 4-byte units
    ("odd_e15_T2_mixed", synth.MoeShape(256, 15, 3, 128, 128, 4), 3, 2, "mixed"),
]


@pytest.mark.parametrize("name,shape,n_layers,T,where", TABLE_CASES, ids=[c[0] for c in TABLE_CASES])
def test_table_decode_equals_stack_decode(name, shape, n_layers, T, where):
    """Routed experts read through the table, wherever their blocks are, give the plain stack
    decode's results bit for bit (y, every layer's x, y, routing and logits)."""
    dev = need_gpu()
    moe = _moe()
    st = synth.make_stack(shape, n_layers, 77 + T, dev, zipf_s=1.1)
    x = synth.make_x(shape, T, 5, device=dev)
    want = _run(moe, shape, st, n_layers, x, T, dev)
    keep = []
    if where == "mixed":
        _, cd, stride = _container(moe, shape, st, n_layers, "device")
        _, ch, _ = _container(moe, shape, st, n_layers, "host")
        keep += [cd, ch]
        n = n_layers * shape.num_experts
        base = torch.where(torch.arange(n) % 2 == 0, torch.tensor(cd.data_ptr()), torch.tensor(ch.data_ptr()))
        table = (base + torch.arange(n, dtype=torch.int64) * stride).to(dev)
    else:
        _, c, stride = _container(moe, shape, st, n_layers, where)
        keep.append(c)
        n = n_layers * shape.num_experts
        table = (c.data_ptr() + torch.arange(n, dtype=torch.int64) * stride).to(dev)
    got = _run(moe, shape, st, n_layers, x, T, dev, table=table)
    _same(want, got)
    print(f"{name}: identical to the stack decode over {n_layers} layers x {T} tokens")


@pytest.mark.parametrize("name,shape,n_layers,T", [("tiny_T4", synth.TINY.shape, 3, 4),
                                                   ("tiny_T8", synth.TINY.shape, 2, 8),
                                                   ("q35b_T3", synth.QWEN35B_4BIT.shape, 2, 3),
                                                   ("q35b_8bit_T1", synth.QWEN35B_8BIT.shape, 2, 1),
                                                   ("q80b_T2", synth.QWEN80B_4BIT.shape, 2, 2)])
def test_landing_blocks_hold_the_marked_experts(name, shape, n_layers, T):
    """With every table entry marked (bit 0) and a landing buffer, the call's results are unchanged
    and landing block [l][t][k] holds every piece of the expert that (layer, token, slot) selected;
    unmarked entries (here the odd experts, read from HBM) write nothing."""
    dev = need_gpu()
    moe = _moe()
    st = synth.make_stack(shape, n_layers, 55 + T, dev, zipf_s=0.5)
    x = synth.make_x(shape, T, 3, device=dev)
    want = _run(moe, shape, st, n_layers, x, T, dev)
    _, ch, stride = _container(moe, shape, st, n_layers, "host")
    _, cd, _ = _container(moe, shape, st, n_layers, "device")
    E, K = shape.num_experts, shape.top_k
    n = n_layers * E
    keys = torch.arange(n, dtype=torch.int64)
    odd = keys % 2 == 1
    table = torch.where(odd, cd.data_ptr() + keys * stride, (ch.data_ptr() + keys * stride) | 1).to(dev)
    land = _landing(shape, n_layers, T, stride, dev)
    land.fill_(0xA5)
    got = _run(moe, shape, st, n_layers, x, T, dev, table=table, landing=land)
    _same(want, got)
    idx = got["idx_all"].numpy()
    blocks = land.cpu().numpy().reshape(n_layers, T, K, stride)
    cont = ch.numpy().reshape(n, stride)
    m = _pieces(shape, stride)
    for l in range(n_layers):
        for t in range(T):
            for k in range(K):
                e = int(idx[l, t, k])
                if e % 2 == 0:
                    assert np.array_equal(blocks[l, t, k][m], cont[l * E + e][m]), (l, t, k)
                else:
                    assert np.all(blocks[l, t, k] == 0xA5), (l, t, k)


BATCHED_TABLE_CASES = [
    ("tiny_T33_mixed", synth.TINY.shape, 33, "mixed", None),
    ("q35b_T128_host_zipf", synth.QWEN35B_4BIT.shape, 128, "host", 1.1),
    ("q35b_8bit_T64_mixed", synth.QWEN35B_8BIT.shape, 64, "mixed", None),
    ("q80b_T40_mixed", synth.QWEN80B_4BIT.shape, 40, "mixed", 0.5),
]


@pytest.mark.parametrize("name,shape,T,where,zipf", BATCHED_TABLE_CASES, ids=[c[0] for c in BATCHED_TABLE_CASES])
def test_batched_table_equals_batched(name, shape, T, where, zipf):
    """The batched layer with its routed experts read through a table row (pinned host memory,
    or alternating host and device blocks) gives moe_layer_batched's outputs bit for bit."""
    dev = need_gpu()
    moe = _moe()
    st = synth.make_stack(shape, 1, 31 + T, dev, zipf_s=zipf)
    x = synth.make_x(shape, T, 13, device=dev)
    E, K = shape.num_experts, shape.top_k
    _, ch, stride = _container(moe, shape, st, 1, "host")
    keys = torch.arange(E, dtype=torch.int64)
    if where == "mixed":
        _, cd, _ = _container(moe, shape, st, 1, "device")
        table = torch.where(keys % 2 == 0, ch.data_ptr() + keys * stride, cd.data_ptr() + keys * stride).to(dev)
    else:
        table = (ch.data_ptr() + keys * stride).to(dev)
    outs = []
    for use_table in (False, True):
        y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
        idx = torch.empty(T, K, dtype=torch.int32, device=dev)
        w = torch.empty(T, K, dtype=torch.float32, device=dev)
        lg = torch.empty(T, E, dtype=torch.float32, device=dev)
        ws = moe.workspace(shape, T, moe.MOE_WS_BATCHED, dev)
        if use_table:
            moe.moe_layer_batched_table(shape, _no_routed(st).layer(0), table, x, T, y, idx, w, lg, workspace=ws)
        else:
            moe.moe_layer_batched(shape, st.layer(0), x, T, y, idx, w, lg, workspace=ws)
        torch.cuda.synchronize()
        outs.append([t.cpu() for t in (y, idx, w, lg)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    print(f"{name}: identical to moe_layer_batched")


def test_prefill_admits_the_routed_experts_first():
    """Prefill of one layer from a pinned container: route, admit the selected experts into the
    pool (moe_cache_admit), then the batched layer through the rewritten table: its outputs are
    moe_layer_batched's bit for bit, the pool holds the admitted blocks, and the policy's
    decisions match the oracle's on the same keys."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.QWEN35B_4BIT.shape
    T, E, K = 96, shape.num_experts, shape.top_k
    st = synth.make_stack(shape, 1, 4242, dev, zipf_s=1.1)
    x = synth.make_x(shape, T, 21, device=dev)
    _, c, stride = _container(moe, shape, st, 1, "host")
    slots = 48
    pool = torch.empty(slots * stride + 4096, dtype=torch.uint8, device=dev)
    off = (-pool.data_ptr()) % 4096
    pool_v = pool[off:off + slots * stride]
    table = torch.empty(E, dtype=torch.int64, device=dev)
    cache = moe.MoeCache(shape, 1, c, pool_v, slots, table)
    try:
        lg = torch.empty(T, E, dtype=torch.float32, device=dev)
        idx = torch.empty(T, K, dtype=torch.int32, device=dev)
        w = torch.empty(T, K, dtype=torch.float32, device=dev)
        moe.moe_route(shape, st.layer(0), x, T, lg, idx, w)
        keys = np.unique(idx.cpu().numpy())
        hits, misses = cache.admit(keys)
        want_hit, want_slot, _ = R.lfu_recency(slots, keys)
        assert (hits, misses) == (sum(want_hit), len(keys) - sum(want_hit))
        outs = []
        for use_table in (False, True):
            y = torch.empty(T, shape.hidden, dtype=torch.float32, device=dev)
            ws = moe.workspace(shape, T, moe.MOE_WS_BATCHED, dev)
            if use_table:
                moe.moe_layer_batched_table(shape, _no_routed(st).layer(0), table, x, T, y, workspace=ws)
            else:
                moe.moe_layer_batched(shape, st.layer(0), x, T, y, workspace=ws)
            torch.cuda.synchronize()
            outs.append(y.cpu())
        assert torch.equal(outs[0], outs[1])
        owners = cache.owners()
        m = _pieces(shape, stride)
        pool_np = pool_v.cpu().numpy().reshape(slots, stride)
        cont = c.numpy().reshape(E, stride)
        for s_, k in enumerate(owners.tolist()):
            if k >= 0:
                assert np.array_equal(pool_np[s_][m], cont[k][m]), (s_, k)
        print(f"admitted {misses} of {len(keys)} selected experts into {slots} slots")
    finally:
        cache.close()


def test_table_decode_against_oracle():
    """Every layer of an unchained table decode (host container) against the fp64 oracle."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.TINY.shape
    Lyr, T = 3, 4
    st = synth.make_stack(shape, Lyr, 303, dev)
    x = synth.make_x(shape, T, 8, device=dev)
    _, c, stride = _container(moe, shape, st, Lyr, "host")
    table = (c.data_ptr() + torch.arange(Lyr * shape.num_experts, dtype=torch.int64) * stride).to(dev)
    got = _run(moe, shape, st, Lyr, x, T, dev, table=table, flags=moe.MOE_STACK_INDEPENDENT)
    for l in range(Lyr):
        ref = oracle_layer(st, l, bf16_bits(x))
        idx, w, lg = got["idx_all"][l].numpy(), got["w_all"][l].numpy(), got["logits_all"][l].numpy()
        differ = check_routing_against_oracle(idx, w, lg, ref, bf16_bits(x), host_layer(st, l), shape.top_k)
        keep = [t for t in range(T) if t not in differ]
        assert keep
        check_y(got["y_all"][l].numpy()[keep], ref["y"][keep])


@pytest.mark.parametrize("slots_frac,T,landing", [(0.0, 1, False), (0.25, 1, False), (0.5, 2, False), (1.0, 1, False),
                                                  (0.25, 1, True), (0.5, 3, True), (0.1, 2, True), (1.0, 8, True)])
def test_cached_decode_loop(slots_frac, T, landing):
    """Several decode steps through a cache over a pinned host container: each step's output is
    the all-resident decode's bit for bit, the hits and misses are the oracle policy's on the
    same routing, and every pool slot holds its owner's block."""
    dev = need_gpu()
    moe = _moe()
    shape = synth.TINY.shape
    Lyr, steps = 4, 6
    E, K = shape.num_experts, shape.top_k
    st = synth.make_stack(shape, Lyr, 909, dev, zipf_s=1.1)
    _, c, stride = _container(moe, shape, st, Lyr, "host")
    slots = int(round(slots_frac * Lyr * E))
    pool = torch.empty(max(slots, 1) * stride + 4096, dtype=torch.uint8, device=dev)
    off = (-pool.data_ptr()) % 4096
    pool_v = pool[off:off + max(slots, 1) * stride]
    table = torch.empty(Lyr * E, dtype=torch.int64, device=dev)
    land = _landing(shape, Lyr, T, stride, dev) if landing else None
    cache = moe.MoeCache(shape, Lyr, c, pool_v if slots else None, slots, table, landing=land)
    ws_t = moe.workspace(shape, T, moe.MOE_WS_STACK, dev, n_layers=Lyr)
    keys_all = []
    try:
        for step in range(steps):
            x = synth.make_x(shape, T, 31, step=step, device=dev)
            want = _run(moe, shape, st, Lyr, x, T, dev)
            got = _run(moe, shape, st, Lyr, x, T, dev, table=table, ws=ws_t, landing=land)
            _same(want, got)
            idx = got["idx_all"].numpy()
            keys = R.routing_keys(idx, E)
            h_o, _, _ = R.lfu_recency(slots, np.concatenate(keys_all + [keys]))
            keys_all.append(keys)
            hits, misses = cache.update(idx, T, K)
            assert hits == sum(h_o[-len(keys):]) and hits + misses == len(keys), step
        torch.cuda.synchronize()
        h_o, slot_o, _ = R.lfu_recency(slots, np.concatenate(keys_all))
        owners = cache.owners()
        want_owner = [-1] * slots
        for k, s in zip(np.concatenate(keys_all).tolist(), slot_o):
            if s >= 0:
                want_owner[s] = k
        assert owners.tolist() == want_owner
        th = table.cpu().numpy().astype(np.uint64)
        pool_np = pool_v.cpu().numpy().reshape(-1, stride) if slots else None
        cont = c.numpy().reshape(-1, stride)
        m = _pieces(shape, stride)
        for s, k in enumerate(owners.tolist()):
            if k >= 0:
                assert np.array_equal(pool_np[s][m], cont[k][m]), (s, k)
                assert int(th[k]) == pool_v.data_ptr() + s * stride
        resident = set(k for k in owners.tolist() if k >= 0)
        for k in range(Lyr * E):
            if k not in resident:
                assert int(th[k]) == (c.data_ptr() + k * stride) | (1 if landing else 0)
        hits, misses, copied = cache.stats()
        assert hits == sum(h_o) and misses == len(h_o) - sum(h_o)
        print(f"slots {slots}: hit rate {hits / (hits + misses):.2f}, copied {copied} B")
    finally:
        cache.close()
