"""Seeded synthetic MoE layer stacks shaped like the models the pages describe.

Shapes
  * The 35B-A3B family routes each token to 8 of 256 experts and keeps one
    always-on shared expert; the 80B-A3B (Qwen3-Next) routes to 10 of 512
    (xix.ai Swiftlet article, paragraph on scheduling; Runnel README, "Target").
  * The Runnel 35B-A3B stack has 40 layers (Runnel README, "Target").
  * Expert weights are MLX-style group-quantised at 4 or 8 bits (xix.ai
    Swiftlet article, paragraph on lineage); gate and up are stored packed
    as one matrix per expert (Runnel README, intro and "Streaming CLI").
  The pages give neither hidden nor intermediate sizes nor a group size:
  hidden 2048, intermediate 512 and groups of 64 are the public sizes of
  these model families.

Value recipe (all seeded, counter-based, per layer and per tensor):
  codes   : uniform random bytes, i.e. every 4-bit nibble uniform on 0..15 and
            every 8-bit code uniform on 0..255
  scales  : bf16(U[0.005, 0.02]) per row and group of 64 input columns
  biases  : -8 * scale (4-bit) or -128 * scale (8-bit), exact in bf16 (the workloads' recipe);
            with affine_bias=True (parity tests of the general affine form w = s*q + b) an
            independent bf16(U[-0.25, 0.25]) per row and group instead, both signs, mostly far
            from -zero_point * scale
  router  : fp32 N(0, 0.02^2), [E, H];  shared-expert gate vector: same, [H]
  x       : bf16 N(0, 1), [T, H]
  router logit bias (batched workload only): -s * ln(rank_e), rank a seeded
            permutation of 1..E, s = 1.1 (a Zipf law with exponent s, in logit
            space; its normalising constant cancels inside the softmax)

Nothing here computes any part of the MoE layer; the module only lays out and
fills input tensors.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import rng

# tensor identifiers folded into each tensor's key
T_ROUTER, T_ROUTER_BIAS, T_SHARED_GATE = 1, 2, 3
T_W13_CODES, T_W13_SCALES = 4, 5
T_W2_CODES, T_W2_SCALES = 6, 7
T_S13_CODES, T_S13_SCALES = 8, 9
T_S2_CODES, T_S2_SCALES = 10, 11
T_X = 12
T_AFFINE_BIAS = 13  # folded into a matrix family's scale key for its independent biases


@dataclasses.dataclass(frozen=True)
class MoeShape:
    hidden: int
    num_experts: int
    top_k: int
    inter: int
    shared_inter: int  # 0 = no shared expert
    bits: int  # 4 or 8
    group_size: int = 64

    def codes_per_byte(self) -> int:
        return 8 // self.bits

    def expert_bytes(self, inter: Optional[int] = None) -> int:
        """Bytes of one expert's packed gate|up and down matrices (codes + bf16 scale + bf16 bias)."""
        i = self.inter if inter is None else inter
        weights = 3 * i * self.hidden
        return weights * self.bits // 8 + 2 * 2 * (weights // self.group_size)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: MoeShape
    n_layers: int
    tokens: int
    zipf_s: Optional[float] = None
    seed: int = 20260101

    def describe(self) -> str:
        s = self.shape
        return (f"{self.name}: H={s.hidden} E={s.num_experts} top-{s.top_k} I={s.inter} "
                f"shared I={s.shared_inter} {s.bits}-bit g{s.group_size}, {self.n_layers} layers, "
                f"T={self.tokens}" + (f", Zipf(s={self.zipf_s}) logit bias" if self.zipf_s else ""))


TINY = Workload("tiny_h256_e16_top2_4bit", MoeShape(256, 16, 2, 128, 128, 4), n_layers=1, tokens=4)
QWEN35B_4BIT = Workload("qwen3.6-35b-a3b_moe_4bit_decode", MoeShape(2048, 256, 8, 512, 512, 4),
                        n_layers=40, tokens=1)
QWEN80B_4BIT = Workload("qwen3-next-80b-a3b_moe_4bit_decode", MoeShape(2048, 512, 10, 512, 512, 4),
                        n_layers=48, tokens=1)
QWEN35B_8BIT = Workload("qwen3.6-35b-a3b_moe_8bit_decode", MoeShape(2048, 256, 8, 512, 512, 8),
                        n_layers=40, tokens=1)
QWEN35B_BATCHED = Workload("qwen3.6-35b-a3b_moe_4bit_batched512_zipf1.1",
                           MoeShape(2048, 256, 8, 512, 512, 4), n_layers=40, tokens=512, zipf_s=1.1)

ALL = {w.name: w for w in (TINY, QWEN35B_4BIT, QWEN80B_4BIT, QWEN35B_8BIT, QWEN35B_BATCHED)}


@dataclasses.dataclass
class LayerStack:
    """Stacked tensors of L layers, leading dim L; each tensor contiguous.

    Layout (row-major):
      router        f32  [L, E, H]
      router_bias   f32  [L, E] or None
      shared_gate   f32  [L, H]
      w13_codes     u8   [L, E, 2I, H*bits/8]   rows 0..I-1 gate, I..2I-1 up
      w13_scales    bf16 [L, E, 2I, H/G]        (w13_biases same shape)
      w2_codes      u8   [L, E, H, I*bits/8]
      w2_scales     bf16 [L, E, H, I/G]         (w2_biases same shape)
      s13_* / s2_*  as w13_* / w2_* with E = 1 and I = shared intermediate
    4-bit codes: input column 2j is the low nibble of byte j, column 2j+1 the high nibble.
    """
    shape: MoeShape
    n_layers: int
    router: torch.Tensor
    router_bias: Optional[torch.Tensor]
    shared_gate: Optional[torch.Tensor]
    w13_codes: torch.Tensor
    w13_scales: torch.Tensor
    w13_biases: torch.Tensor
    w2_codes: torch.Tensor
    w2_scales: torch.Tensor
    w2_biases: torch.Tensor
    s13_codes: Optional[torch.Tensor]
    s13_scales: Optional[torch.Tensor]
    s13_biases: Optional[torch.Tensor]
    s2_codes: Optional[torch.Tensor]
    s2_scales: Optional[torch.Tensor]
    s2_biases: Optional[torch.Tensor]

    def tensors(self):
        return {f.name: getattr(self, f.name) for f in dataclasses.fields(self)
                if isinstance(getattr(self, f.name), torch.Tensor)}

    def layer(self, l: int) -> "LayerStack":
        """A one-layer view (no copy) of layer l."""
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            if isinstance(v, torch.Tensor):
                v = v[l:l + 1]
            kw[f.name] = v
        kw["n_layers"] = 1
        return LayerStack(**kw)

    def to(self, device) -> "LayerStack":
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            if isinstance(v, torch.Tensor):
                v = v.to(device)
            kw[f.name] = v
        return LayerStack(**kw)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors().values())


def _alloc(shape: MoeShape, n_layers: int, device, with_bias: bool) -> LayerStack:
    H, E, I, Is, G = shape.hidden, shape.num_experts, shape.inter, shape.shared_inter, shape.group_size
    cpb = shape.codes_per_byte()

    def q(e, rows, cols):
        return (torch.empty((n_layers, e, rows, cols // cpb), dtype=torch.uint8, device=device),
                torch.empty((n_layers, e, rows, cols // G), dtype=torch.bfloat16, device=device),
                torch.empty((n_layers, e, rows, cols // G), dtype=torch.bfloat16, device=device))

    w13 = q(E, 2 * I, H)
    w2 = q(E, H, I)
    s13 = q(1, 2 * Is, H) if Is else (None, None, None)
    s2 = q(1, H, Is) if Is else (None, None, None)
    return LayerStack(
        shape=shape, n_layers=n_layers,
        router=torch.empty((n_layers, E, H), dtype=torch.float32, device=device),
        router_bias=torch.empty((n_layers, E), dtype=torch.float32, device=device) if with_bias else None,
        shared_gate=torch.empty((n_layers, H), dtype=torch.float32, device=device) if Is else None,
        w13_codes=w13[0], w13_scales=w13[1], w13_biases=w13[2],
        w2_codes=w2[0], w2_scales=w2[1], w2_biases=w2[2],
        s13_codes=s13[0], s13_scales=s13[1], s13_biases=s13[2],
        s2_codes=s2[0], s2_scales=s2[1], s2_biases=s2[2])


def _fill_scales_biases(scales: torch.Tensor, biases: torch.Tensor, key: int, bits: int,
                        affine_bias: bool = False) -> None:
    n = scales.numel()
    u = rng.uniform01(key, n, scales.device)
    s = (0.005 + 0.015 * u).to(torch.float32).to(torch.bfloat16)
    scales.view(-1).copy_(s)
    if affine_bias:
        ub = rng.uniform01(rng.derive_key(key, T_AFFINE_BIAS), n, scales.device)
        biases.view(-1).copy_((0.5 * ub - 0.25).to(torch.float32).to(torch.bfloat16))
        return
    zero_point = 8.0 if bits == 4 else 128.0
    biases.view(-1).copy_(s * (-zero_point))  # exact: power-of-two multiple of a bf16 value


def zipf_bias(shape: MoeShape, l: int, seed: int, zipf_s: float, device="cpu") -> torch.Tensor:
    """fp32 [E] router bias of layer l: -s * ln(rank_e), ranks a seeded permutation of 1..E."""
    perm = rng.permutation(rng.derive_key(seed, l, T_ROUTER_BIAS), shape.num_experts, device)
    rank = torch.empty_like(perm)
    rank[perm] = torch.arange(1, shape.num_experts + 1, device=device)
    return (-zipf_s * torch.log(rank.to(torch.float64))).to(torch.float32)


def with_zipf_bias(stack: LayerStack, seed: int, zipf_s: float) -> LayerStack:
    """The same weights (no copy) with the Zipf router bias of every layer attached."""
    dev = stack.router.device
    bias = torch.stack([zipf_bias(stack.shape, l, seed, zipf_s, dev) for l in range(stack.n_layers)])
    return dataclasses.replace(stack, router_bias=bias.contiguous())


def fill_layer(stack: LayerStack, l: int, seed: int, zipf_s: Optional[float] = None,
               affine_bias: bool = False) -> None:
    """Fill layer l of `stack` in place from (seed, l); affine_bias draws every quantisation
    bias independently of its scale (see the module recipe)."""
    sh = stack.shape
    dev = stack.router.device
    k = lambda tid: rng.derive_key(seed, l, tid)
    stack.router[l].view(-1).copy_((0.02 * rng.normal(k(T_ROUTER), stack.router[l].numel(), dev))
                                   .to(torch.float32))
    if stack.router_bias is not None:
        if zipf_s is None:
            stack.router_bias[l].zero_()
        else:
            stack.router_bias[l].copy_(zipf_bias(sh, l, seed, zipf_s, dev))
    if stack.shared_gate is not None:
        stack.shared_gate[l].copy_((0.02 * rng.normal(k(T_SHARED_GATE), sh.hidden, dev)).to(torch.float32))
    rng.fill_bytes(stack.w13_codes[l], k(T_W13_CODES))
    ab = affine_bias
    _fill_scales_biases(stack.w13_scales[l], stack.w13_biases[l], k(T_W13_SCALES), sh.bits, ab)
    rng.fill_bytes(stack.w2_codes[l], k(T_W2_CODES))
    _fill_scales_biases(stack.w2_scales[l], stack.w2_biases[l], k(T_W2_SCALES), sh.bits, ab)
    if stack.s13_codes is not None:
        rng.fill_bytes(stack.s13_codes[l], k(T_S13_CODES))
        _fill_scales_biases(stack.s13_scales[l], stack.s13_biases[l], k(T_S13_SCALES), sh.bits, ab)
        rng.fill_bytes(stack.s2_codes[l], k(T_S2_CODES))
        _fill_scales_biases(stack.s2_scales[l], stack.s2_biases[l], k(T_S2_SCALES), sh.bits, ab)


def make_stack(shape: MoeShape, n_layers: int, seed: int, device="cpu",
               zipf_s: Optional[float] = None, with_bias: Optional[bool] = None,
               affine_bias: bool = False) -> LayerStack:
    """Allocate and fill an n_layers stack; layer l depends only on (seed, l)."""
    if with_bias is None:
        with_bias = zipf_s is not None
    st = _alloc(shape, n_layers, device, with_bias)
    for l in range(n_layers):
        fill_layer(st, l, seed, zipf_s, affine_bias)
    return st


def make_x(shape: MoeShape, tokens: int, seed: int, step: int = 0, device="cpu") -> torch.Tensor:
    """bf16 [tokens, H] activations drawn N(0, 1); `step` selects a fresh draw per decode step."""
    key = rng.derive_key(seed, 1 << 20, T_X, step)
    return rng.normal(key, tokens * shape.hidden, device).to(torch.float32).to(torch.bfloat16) \
        .view(tokens, shape.hidden)


def make_workload(w: Workload, device="cpu", n_layers: Optional[int] = None) -> LayerStack:
    return make_stack(w.shape, w.n_layers if n_layers is None else n_layers, w.seed, device, w.zipf_s)


def algorithmic_decode_bytes(shape: MoeShape) -> int:
    """Bytes one batch-1 decode token must move through one layer: the K routed experts and
    the shared expert (codes + scales + biases), the fp32 router and shared-gate vector,
    the bf16 input row and the fp32 output row. Intermediates (logits, h) are excluded."""
    b = shape.top_k * shape.expert_bytes()
    if shape.shared_inter:
        b += shape.expert_bytes(shape.shared_inter) + 4 * shape.hidden
    b += 4 * shape.num_experts * shape.hidden
    b += 2 * shape.hidden + 4 * shape.hidden
    return b
