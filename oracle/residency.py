"""Plain-Python oracle of the expert-residency tier: the fixed-stride expert container and the
bounded expert pool with LFU + recency eviction.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. It shares no code with the HIP library or its Python binding and imports
neither.

What the pages fix (Swiftlet as the AgentLens project page describes it under "How it works", the
xix.ai article in its scheduling and lineage paragraphs, and the Chinese summary's highlights):
routed experts are repacked into fixed-stride blocks so that one expert is one contiguous read;
popular experts are kept in a bounded pool; eviction is "LFU plus recency". Readings taken where
the pages say no more:
  * frequency is the number of uses since the expert entered the pool (admission counts as one);
  * the victim is the resident expert with the lowest frequency, and among equals the one used
    least recently ("recency" breaks the ties);
  * a free slot, when there is one, is the lowest-numbered one;
  * one decode call's routing is fed in the order layer, token, slot; a key is l * E + e.
The container layout (piece order, 256-byte piece alignment, 4 KiB block rounding) is this
framework's own choice; the pages fix only that the stride is fixed.
"""
from __future__ import annotations

import numpy as np


def lfu_recency(slots: int, keys) -> tuple[list[int], list[int], list[int]]:
    """Run the policy over a key sequence. Per access: hit (0/1), the slot the key occupies
    afterwards (-1 when there are no slots), the key evicted (-1 if none)."""
    owner = [-1] * slots      # key held by each slot
    freq = [0] * slots        # uses since admission
    last = [0] * slots        # time of the last use
    hits, where, evicted = [], [], []
    for now, key in enumerate(keys, start=1):
        key = int(key)
        if key in owner:
            s = owner.index(key)
            freq[s] += 1
            last[s] = now
            hits.append(1)
            where.append(s)
            evicted.append(-1)
            continue
        hits.append(0)
        if slots == 0:
            where.append(-1)
            evicted.append(-1)
            continue
        if -1 in owner:
            s = owner.index(-1)
            gone = -1
        else:
            # smallest frequency, then the oldest last use
            s = min(range(slots), key=lambda i: (freq[i], last[i]))
            gone = owner[s]
        owner[s], freq[s], last[s] = key, 1, now
        where.append(s)
        evicted.append(gone)
    return hits, where, evicted


def routing_keys(topk_idx_all: np.ndarray, num_experts: int) -> np.ndarray:
    """Keys of one decode call's routing [L][T][K], in the order layer, token, slot."""
    a = np.asarray(topk_idx_all, dtype=np.int64)
    L = a.shape[0]
    return (a + np.arange(L, dtype=np.int64).reshape(L, *([1] * (a.ndim - 1))) * num_experts).reshape(-1)


def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def expert_block_layout(hidden: int, inter: int, bits: int) -> dict:
    """Byte offsets and sizes of the six pieces of one expert's block, and the stride."""
    c13 = 2 * inter * hidden * bits // 8
    s13 = 2 * inter * (hidden // 64) * 2
    c2 = hidden * inter * bits // 8
    s2 = hidden * (inter // 64) * 2
    sizes = [c13, s13, s13, c2, s2, s2]
    offs, o = [], 0
    for n in sizes:
        offs.append(o)
        o += _round_up(n, 256)
    stride = _round_up(offs[-1] + sizes[-1], 4096)
    return {"offsets": offs, "sizes": sizes, "stride": stride}


def pack_block(w13_codes, w13_scales, w13_biases, w2_codes, w2_scales, w2_biases, hidden, inter, bits) -> np.ndarray:
    """One expert's block as bytes (pieces given as that expert's arrays, any integer dtype)."""
    lay = expert_block_layout(hidden, inter, bits)
    out = np.zeros(lay["stride"], dtype=np.uint8)
    for off, n, a in zip(lay["offsets"], lay["sizes"],
                         (w13_codes, w13_scales, w13_biases, w2_codes, w2_scales, w2_biases)):
        b = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
        assert b.size == n, (b.size, n)
        out[off:off + n] = b
    return out
