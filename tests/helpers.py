"""Small shared test utilities: moving synthetic torch tensors to the oracle's numpy form."""
import numpy as np
import torch


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (any device)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 values."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def host_layer(stack, l: int):
    """oracle.HostLayer of layer l of a synth.LayerStack (device tensors are copied to host)."""
    import oracle
    arrays = {}
    for name, t in stack.tensors().items():
        a = t[l]
        if a.dtype == torch.bfloat16:
            arrays[name] = bf16_bits(a)
        else:
            arrays[name] = a.detach().cpu().contiguous().numpy()
    for name in ("s13_codes", "s13_scales", "s13_biases", "s2_codes", "s2_scales", "s2_biases"):
        if arrays.get(name) is not None:
            arrays[name] = arrays[name][0]  # drop the E=1 expert dim for the shared expert
    return oracle.HostLayer(stack.shape, arrays)


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / RMS(ref) over the whole array."""
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / max(rms, 1e-300)
