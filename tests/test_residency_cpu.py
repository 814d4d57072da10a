"""Expert residency on the host: the oracle's LFU + recency policy pinned by hand-worked and
closed-form cases, the library's policy (moe_cache_policy_run) against the oracle access by
access, the container layout, and the host-side argument checks of the residency entry points."""
import ctypes
import os

import numpy as np
import pytest

import quantized_moe_decode_router_amd as moe
from quantized_moe_decode_router_amd import binding
from oracle import residency as R

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from quantized_moe_decode_router_amd import build
        build.build()
    return moe.lib()


class Shape:
    def __init__(self, H=2048, E=256, K=8, I=512, Is=512, bits=4):
        self.hidden, self.num_experts, self.top_k, self.inter, self.shared_inter, self.bits = H, E, K, I, Is, bits


def zipf_keys(rng, n_keys, n, a=1.1):
    p = 1.0 / np.arange(1, n_keys + 1) ** a
    p /= p.sum()
    return rng.permutation(n_keys)[rng.choice(n_keys, size=n, p=p)].astype(np.int32)


# ---- oracle pins -----------------------------------------------------------------------------

def test_hand_worked_trace():
    rows = [list(map(int, l.split())) for l in open(os.path.join(HERE, "golden", "lfu_recency_trace.txt"))
            if l.strip() and not l.startswith("#")]
    keys = [r[0] for r in rows]
    hit, slot, ev = R.lfu_recency(3, keys)
    assert hit == [r[1] for r in rows]
    assert slot == [r[2] for r in rows]
    assert ev == [r[3] for r in rows]


def test_one_slot_hits_exactly_on_repeats():
    keys = np.random.default_rng(1).integers(0, 4, 300)
    hit, _, _ = R.lfu_recency(1, keys)
    assert hit == [0] + [int(keys[i] == keys[i - 1]) for i in range(1, len(keys))]


def test_pool_as_large_as_the_keys_misses_once_per_key():
    keys = zipf_keys(np.random.default_rng(2), 50, 2000)
    hit, slot, ev = R.lfu_recency(50, keys)
    first = list(dict.fromkeys(keys.tolist()))
    assert hit.count(0) == len(first)
    assert set(ev) == {-1}
    assert [slot[keys.tolist().index(k)] for k in first] == list(range(len(first)))


def test_cyclic_scan_never_hits():
    # every resident key has frequency 1, so the least recently used goes: a cyclic scan over one
    # more key than slots always misses (evicting the most recent instead would hit)
    keys = list(range(9)) * 20
    hit, _, ev = R.lfu_recency(8, keys)
    assert sum(hit) == 0
    assert ev[:8] == [-1] * 8 and ev[8:] == keys[:len(keys) - 8]


def test_frequent_key_survives_a_scan():
    keys = [0, 0, 0] + list(range(1, 60)) + [0]
    hit, _, ev = R.lfu_recency(2, keys)
    assert 0 not in ev and hit[-1] == 1
    assert sum(hit) == 3


def test_no_slots_never_hits():
    hit, slot, ev = R.lfu_recency(0, [3, 3, 3])
    assert hit == [0, 0, 0] and slot == [-1, -1, -1] and ev == [-1, -1, -1]


def test_policy_invariants_on_zipf_traces():
    rng = np.random.default_rng(3)
    for slots in (1, 5, 40):
        keys = zipf_keys(rng, 200, 3000)
        hit, slot, ev = R.lfu_recency(slots, keys)
        resident = {}
        for k, h, s, e in zip(keys.tolist(), hit, slot, ev):
            if h:
                assert resident[s] == k and e == -1
            else:
                assert k not in resident.values()
                assert (e == -1) == (s not in resident) and (e == -1 or resident[s] == e)
            resident[s] = k
            assert len(resident) <= slots


def test_routing_keys_order():
    idx = np.array([[[3, 1]], [[0, 2]]])  # [L=2][T=1][K=2], E = 4
    assert R.routing_keys(idx, 4).tolist() == [3, 1, 4, 6]


def test_block_layout_closed_form():
    lay = R.expert_block_layout(2048, 512, 4)
    # 4-bit gate|up codes 1 MiB, their scales and biases 64 KiB each, down codes 512 KiB, down
    # scales and biases 32 KiB each: all 256-aligned, the sum a multiple of 4 KiB
    assert lay["sizes"] == [1 << 20, 65536, 65536, 1 << 19, 32768, 32768]
    assert lay["stride"] == 1769472 == sum(lay["sizes"])
    # H 64, I 128, 8-bit: gate|up codes 16384 B, scales 512 B each, down codes 8192 B, scales 256 B each
    assert R.expert_block_layout(64, 128, 8)["offsets"] == [0, 16384, 16896, 17408, 25600, 25856]


def test_pack_block_round_trip():
    rng = np.random.default_rng(4)
    H, I, bits = 128, 128, 4
    parts = [rng.integers(0, 256, (2 * I, H // 2), dtype=np.uint8), rng.integers(0, 65536, (2 * I, H // 64), dtype=np.uint16),
             rng.integers(0, 65536, (2 * I, H // 64), dtype=np.uint16), rng.integers(0, 256, (H, I // 2), dtype=np.uint8),
             rng.integers(0, 65536, (H, I // 64), dtype=np.uint16), rng.integers(0, 65536, (H, I // 64), dtype=np.uint16)]
    blk = R.pack_block(*parts, H, I, bits)
    lay = R.expert_block_layout(H, I, bits)
    for off, n, a in zip(lay["offsets"], lay["sizes"], parts):
        assert np.array_equal(blk[off:off + n].view(a.dtype).reshape(a.shape), a)


# ---- the library's policy against the oracle ---------------------------------------------------

@pytest.mark.parametrize("slots", [0, 1, 3, 64, 400])
def test_library_policy_matches_oracle(L, slots):
    rng = np.random.default_rng(100 + slots)
    keys = zipf_keys(rng, 40 * 64, 4000, a=1.05)
    want = R.lfu_recency(slots, keys)
    got = moe.moe_cache_policy_run(slots, 40 * 64, keys)
    for w, g in zip(want, got):
        assert np.array_equal(np.asarray(w, dtype=np.int32), g)


def test_library_policy_hand_worked_trace(L):
    rows = [list(map(int, l.split())) for l in open(os.path.join(HERE, "golden", "lfu_recency_trace.txt"))
            if l.strip() and not l.startswith("#")]
    hit, slot, ev = moe.moe_cache_policy_run(3, 10, [r[0] for r in rows])
    assert hit.tolist() == [r[1] for r in rows] and slot.tolist() == [r[2] for r in rows]
    assert ev.tolist() == [r[3] for r in rows]


def test_library_policy_on_routing_order(L):
    # decode routing of several calls: distinct experts per (layer, token), keys in layer, token, slot order
    rng = np.random.default_rng(7)
    Lyr, T, K, E = 6, 2, 4, 32
    keys = np.concatenate([R.routing_keys(np.stack([[rng.choice(E, K, replace=False) for _ in range(T)]
                                                    for _ in range(Lyr)]), E) for _ in range(30)])
    want = R.lfu_recency(50, keys)
    got = moe.moe_cache_policy_run(50, Lyr * E, keys)
    assert all(np.array_equal(np.asarray(w, dtype=np.int32), g) for w, g in zip(want, got))


def test_library_stride_matches_oracle_layout(L):
    for H, I, bits in ((2048, 512, 4), (2048, 512, 8), (256, 128, 4), (1024, 256, 8)):
        assert moe.moe_expert_stride(Shape(H=H, I=I, Is=0, bits=bits, E=8, K=2)) == \
            R.expert_block_layout(H, I, bits)["stride"]
    assert moe.moe_expert_stride(Shape(bits=5)) == 0


# ---- host-side argument checks (nothing is enqueued) -------------------------------------------

def test_residency_host_checks(L):
    s = binding.shape_struct(Shape())
    inval = moe.MOE_ERR_INVALID_ARG
    out = ctypes.c_void_p()
    stride = moe.moe_expert_stride(Shape())
    n = 2 * 256
    big = n * stride
    # out missing, slots out of range, misaligned or short container, short pool or table
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10000, big, 0x20000, 4 * stride, 4, 0x30000, n * 8, None, 0, None, None) == inval
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10000, big, 0x20000, 4 * stride, -1, 0x30000, n * 8, None, 0, None, ctypes.byref(out)) == inval
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10000, big, 0x20000, 4 * stride, n + 1, 0x30000, n * 8, None, 0, None, ctypes.byref(out)) == inval
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10008, big, 0x20000, 4 * stride, 4, 0x30000, n * 8, None, 0, None, ctypes.byref(out)) == inval
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10000, big - 1, 0x20000, 4 * stride, 4, 0x30000, n * 8, None, 0, None, ctypes.byref(out)) == inval
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10000, big, 0x20000, 4 * stride - 1, 4, 0x30000, n * 8, None, 0, None, ctypes.byref(out)) == inval
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10000, big, 0x20000, 4 * stride, 4, 0x30000, n * 8 - 8, None, 0, None, ctypes.byref(out)) == inval
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10000, big, None, 0, 4, 0x30000, n * 8, None, 0, None, ctypes.byref(out)) == inval
    assert out.value is None
    assert L.moe_cache_update(None, None, 1, 8, None, None, None) == inval
    assert L.moe_cache_admit(None, None, 0, None, None, None) == inval
    assert L.moe_cache_stats(None, None, None, None) == inval
    assert L.moe_cache_owners(None, None) == inval
    L.moe_cache_destroy(None)
    keys = np.array([0, 5], dtype=np.int32)
    buf = np.zeros(2, dtype=np.int32)
    assert L.moe_cache_policy_run(2, 5, keys.ctypes.data, 2, buf.ctypes.data, buf.ctypes.data, buf.ctypes.data) == inval
    assert L.moe_cache_policy_run(-1, 5, keys.ctypes.data, 1, buf.ctypes.data, buf.ctypes.data, buf.ctypes.data) == inval
    # table decode without a table; packing into a misaligned or short container
    lay = binding.MoeLayer()
    assert L.moe_stack_decode_table(ctypes.byref(s), ctypes.byref(lay), 1, None, None, 0, 0, 0x1000, 1, 0x2000, None,
                                    None, None, None, None, 0x3000, 1 << 30, None) == inval
    assert L.moe_layer_batched_table(ctypes.byref(s), ctypes.byref(lay), None, 0x1000, 4, 0x2000, None, None, None,
                                     0x3000, 1 << 30, None) == inval
    # a landing buffer needs a table, 4096-byte alignment and L * T * K blocks
    tab = 0x40000
    for landing, lb in ((0x80000, 0), (0x80010, 1 << 40)):
        assert L.moe_stack_decode_table(ctypes.byref(s), ctypes.byref(lay), 1, tab, landing, lb, 0, 0x1000, 1, 0x2000,
                                        None, None, None, None, None, 0x3000, 1 << 30, None) == inval
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10000, big, 0x20000, 4 * stride, 4, 0x30000, n * 8, 0x80010,
                              1 << 40, None, ctypes.byref(out)) == inval
    assert L.moe_cache_create(ctypes.byref(s), 2, 0x10000, big, 0x20000, 4 * stride, 4, 0x30000, n * 8, 0x80000,
                              2 * 8 * stride - 1, None, ctypes.byref(out)) == inval
    q = binding.MoeQWeight(0x1000, 0x2000, 0x3000)
    lay = binding.MoeLayer(0x4000, None, 0x5000, q, q, q, q)
    assert L.moe_pack_experts(ctypes.byref(s), ctypes.byref(lay), 1, 0x10010, big, None) == inval
    assert L.moe_pack_experts(ctypes.byref(s), ctypes.byref(lay), 1, 0x10000, 256 * stride - 1, None) == inval
