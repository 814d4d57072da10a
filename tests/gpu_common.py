"""Shared pieces of the GPU parity tests: device setup, oracle comparisons and bounds."""
import math

import numpy as np
import pytest
import torch

from tests.helpers import bf16_bits, bits_to_f32, host_layer, rel_max_err

# Layer-output tolerance: max |y_gpu - y_oracle| <= 2e-3 * RMS(y_oracle) over a layer's [T, H]
# output, with fp32 accumulation on the GPU.
Y_TOL = 2e-3
# Routing weights: |w_gpu - w_oracle| <= 1e-6 when both select the same experts.
W_TOL = 1e-6
U32 = 2.0 ** -24


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import quantized_moe_decode_router_amd as moe
    moe.lib()  # fails loudly if the HIP library is missing
    return torch.device("cuda:0")


def gamma_n(n: int) -> float:
    return n * U32 / (1.0 - n * U32)


def logit_bound(x_f64: np.ndarray, R: np.ndarray, bias=None) -> np.ndarray:
    """Worst-case fp32 dot-product error in any summation order (Higham, Accuracy and
    Stability of Numerical Algorithms, 2nd ed., eq. 3.5): gamma_{H+1} * sum_h |x_h R_eh|,
    plus the rounding of the bias add."""
    H = x_f64.shape[-1]
    s = np.abs(R.astype(np.float64)) @ np.abs(x_f64)
    if bias is not None:
        s = s + np.abs(bias.astype(np.float64))
    return gamma_n(H + 1) * s


def topk_margin(l: np.ndarray, K: int) -> float:
    """Gap between the K-th and (K+1)-th largest logits (inf if K == E)."""
    if K >= l.shape[0]:
        return math.inf
    s = np.sort(l)[::-1]
    return float(s[K - 1] - s[K])


def oracle_layer(stack, l, x_bits):
    import oracle
    return oracle.layer_forward(host_layer(stack, l), x_bits)


def check_selection(gpu_idx_t, gpu_w_t, ref_logits_t, ref_idx_t, ref_w_t, K, bnd):
    """One token's routing against the oracle's own (fp64-logit) routing. `bnd` bounds
    |l_gpu - l_oracle| for every expert. Returns "exact" (same experts in the same order),
    "same_set" (same experts; neighbours whose logits are within 2*bnd may be ordered either way),
    or "ambiguous" (a different but valid set, possible only when the K-th margin is within
    2*bnd). Anything else fails. With the same set, the weights may differ from the oracle's by
    what the logit error moves a softmax weight: |dw_k| <= w_k (exp(2 bnd) - 1), plus fp32
    rounding."""
    g = [int(v) for v in gpu_idx_t]
    r = [int(v) for v in ref_idx_t]
    assert len(set(g)) == K and all(0 <= e < ref_logits_t.shape[0] for e in g)
    lg = ref_logits_t
    # the GPU order must be non-increasing in the oracle's logits up to the bound
    for a, b in zip(g, g[1:]):
        assert lg[a] >= lg[b] - 2 * bnd, f"order {g} inconsistent with the logits"
    assert abs(float(np.sum(gpu_w_t, dtype=np.float64)) - 1.0) <= 1e-6
    if set(g) == set(r):
        wmap = {e: w for e, w in zip(r, ref_w_t)}
        want = np.array([wmap[e] for e in g])
        tol = want * math.expm1(2 * bnd) + W_TOL
        assert np.all(np.abs(np.asarray(gpu_w_t[:K], np.float64) - want) <= tol), "weights beyond the bound"
        return "exact" if g == r else "same_set"
    margin = topk_margin(lg, K)
    assert margin <= 2 * bnd, f"selection {g} differs from {r} with an unambiguous margin {margin:.3e}"
    kth = np.sort(lg)[::-1][K - 1]
    assert all(lg[e] >= kth - 2 * bnd for e in g)
    return "ambiguous"


def check_routing_against_oracle(gpu_idx, gpu_w, gpu_logits, ref, x_bits, Lh, K):
    """Logits within the worst-case bound. In given-logits mode (the oracle's selection and
    weights evaluated on the GPU's own fp32 logits) the GPU's indices must be identical and its
    weights within 1e-6; against the oracle's own fp64 logits every token's selection is checked
    by check_selection. Returns the list of tokens whose selection was legitimately different
    from the own-logits oracle (their outputs are not comparable)."""
    import oracle
    x = bits_to_f32(x_bits).astype(np.float64)
    R = Lh.arrays["router"]
    bias = Lh.arrays.get("router_bias")
    differ = []
    for t in range(x.shape[0]):
        bnd = logit_bound(x[t], R, bias)
        if gpu_logits is not None:
            gl = gpu_logits[t].astype(np.float64)
            err = np.abs(gl - ref["logits"][t])
            assert np.all(err <= bnd), f"token {t}: logit error {err.max()} > bound"
            want = oracle.topk(gl, K)
            assert [int(v) for v in gpu_idx[t]] == [int(v) for v in want], f"token {t}: selection != oracle(given logits)"
            np.testing.assert_allclose(gpu_w[t], oracle.route_weights(gl, want), rtol=0, atol=W_TOL)
        kind = check_selection(gpu_idx[t], gpu_w[t], ref["logits"][t], ref["idx"][t], ref["w"][t], K, bnd.max())
        if kind == "ambiguous":
            differ.append(t)
    return differ


def check_y(gpu_y, ref_y, tol=Y_TOL):
    err = rel_max_err(gpu_y, ref_y)
    assert err <= tol, f"max |err| / RMS = {err:.3e} > {tol}"
    return err


CANARY = 0x5A5A5A5A  # as fp32: a NaN-free pattern no kernel produces by accident (2.9e16)
GUARD = 256          # 4-byte words of guard band on each side (keeps 16-byte alignment)


class Guarded:
    """4-byte output tensors (fp32 or int32) carved from the middle of a larger buffer whose guard
    bands hold a canary pattern; check() fails if any guard word changed (an out-of-bounds store)."""

    def __init__(self, dev):
        self.dev = dev
        self.bufs = []

    def empty(self, *shape, dtype=torch.float32):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.int32, device=self.dev)
        self.bufs.append((buf, n))
        return buf[GUARD:GUARD + n].view(dtype).view(*shape)

    def check(self):
        for buf, n in self.bufs:
            h = buf.cpu().numpy()
            assert np.all(h[:GUARD] == CANARY) and np.all(h[GUARD + n:] == CANARY), "store outside an output"


def x_from_bits(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(device)


__all__ = ["Guarded", "need_gpu", "logit_bound", "topk_margin", "oracle_layer", "check_routing_against_oracle",
           "check_y", "x_from_bits", "bf16_bits", "host_layer", "Y_TOL", "W_TOL"]
