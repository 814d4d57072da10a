"""Expert-permutation invariance on the GPU: renumbering the experts of a layer (router rows, router
bias and the routed experts' weights moved together; the shared expert stays) renumbers the
selection and changes nothing else. Every expert's logit, gate|up and down projection is computed
by the same arithmetic wherever its index places it (which workgroup, which router row of that
workgroup, which slot of a grouped-GEMM tile), and the combine runs over the selection slots, so
logits, weights and y are expected bit for bit equal on both paths, with idx mapped through the
permutation. A kernel whose result depended on where an expert sits -- a row or slot mix-up, a
reduction order tied to the expert index -- would break this."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests.gpu_common import need_gpu
from tests.test_gpu_batched import run_batched
from tests.test_gpu_decode import run_decode

pytestmark = pytest.mark.gpu

EXPERT_FIELDS = ("router", "router_bias", "w13_codes", "w13_scales", "w13_biases",
                 "w2_codes", "w2_scales", "w2_biases")


def permuted(layer, perm, dev):
    """The one-layer stack whose expert e is expert perm[e] of `layer`."""
    p = torch.from_numpy(perm.astype(np.int64)).to(dev)
    kw = {}
    for f in EXPERT_FIELDS:
        t = getattr(layer, f)
        kw[f] = None if t is None else t.index_select(1, p).contiguous()
    return dataclasses.replace(layer, **kw)


CASES = [
    ("decode_35b_4bit_T1", "decode", synth.QWEN35B_4BIT.shape, 1, None),
    ("decode_35b_8bit_T8", "decode", synth.QWEN35B_8BIT.shape, 8, None),
    ("decode_80b_4bit_T3", "decode", synth.QWEN80B_4BIT.shape, 3, None),
    ("batched_35b_4bit_T70_zipf", "batched", synth.QWEN35B_4BIT.shape, 70, 1.1),
    ("batched_tiny_T33", "batched", synth.TINY.shape, 33, None),
]


@pytest.mark.parametrize("name,path,shape,T,zipf", CASES, ids=[c[0] for c in CASES])
def test_expert_permutation_invariance(name, path, shape, T, zipf):
    dev = need_gpu()
    E = shape.num_experts
    st = synth.make_stack(shape, 1, 4100 + T, dev, zipf_s=zipf)
    x = synth.make_x(shape, T, 41 + T, device=dev)
    layer = st.layer(0)
    run = run_decode if path == "decode" else run_batched
    y, idx, w, lg = run(shape, layer, x, T, dev)
    for perm in (np.random.default_rng(T).permutation(E), np.arange(E)[::-1].copy()):
        inv = np.argsort(perm)
        yp, idxp, wp, lgp = run(shape, permuted(layer, perm, dev), x, T, dev)
        np.testing.assert_array_equal(lgp, lg[:, perm])
        np.testing.assert_array_equal(idxp, inv[idx])
        np.testing.assert_array_equal(wp, w)
        np.testing.assert_array_equal(yp, y)
    print(f"{name}: logits, selection, weights and y unchanged under two renumberings of {E} experts")
