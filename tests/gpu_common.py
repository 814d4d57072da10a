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


def check_routing_against_oracle(gpu_idx, gpu_w, gpu_logits, ref, x_bits, Lh, K):
    """Logits within the worst-case bound; indices equal wherever the oracle's top-k margin exceeds
    twice that bound (else both selections are valid and only validity is checked); weights
    within W_TOL where the indices agree. Returns the number of ambiguous tokens."""
    x = bits_to_f32(x_bits).astype(np.float64)
    R = Lh.arrays["router"]
    bias = Lh.arrays.get("router_bias")
    ambiguous = 0
    for t in range(x.shape[0]):
        bnd = logit_bound(x[t], R, bias)
        if gpu_logits is not None:
            err = np.abs(gpu_logits[t].astype(np.float64) - ref["logits"][t])
            assert np.all(err <= bnd), f"token {t}: logit error {err.max()} > bound"
        margin = topk_margin(ref["logits"][t], K)
        if margin > 2 * bnd.max():
            assert list(gpu_idx[t]) == list(ref["idx"][t]), f"token {t}: {gpu_idx[t]} vs {ref['idx'][t]}"
            np.testing.assert_allclose(gpu_w[t], ref["w"][t], rtol=0, atol=W_TOL)
        else:
            ambiguous += 1
            # valid selection: every chosen logit is within the bound of the K-th largest
            kth = np.sort(ref["logits"][t])[::-1][K - 1]
            assert np.all(ref["logits"][t][gpu_idx[t]] >= kth - 2 * bnd.max())
            assert len(set(gpu_idx[t].tolist())) == K
        assert abs(float(np.sum(gpu_w[t], dtype=np.float64)) - 1.0) <= 1e-6
    return ambiguous


def check_y(gpu_y, ref_y, tol=Y_TOL):
    err = rel_max_err(gpu_y, ref_y)
    assert err <= tol, f"max |err| / RMS = {err:.3e} > {tol}"
    return err


def x_from_bits(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(device)


__all__ = ["need_gpu", "logit_bound", "topk_margin", "oracle_layer", "check_routing_against_oracle",
           "check_y", "x_from_bits", "bf16_bits", "host_layer", "Y_TOL", "W_TOL"]
