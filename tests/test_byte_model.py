"""Pins the algorithmic byte model (used for every GB/s and roofline figure) against the model
sizes the pages print. The pages' sizes are whole checkpoints (experts plus the dense core),
so the routed-expert bytes alone must come out just under them."""
import synth


def test_expert_bytes():
    s4 = synth.QWEN35B_4BIT.shape
    assert s4.expert_bytes() == 3 * 512 * 2048 // 2 + 2 * 2 * 3 * 512 * 2048 // 64 == 1769472
    assert synth.QWEN35B_8BIT.shape.expert_bytes() == 3342336


def test_routed_bytes_against_page_sizes():
    # xix.ai Swiftlet article, paragraph on numbers: the 4-bit 35B takes 18 GB on disk and the
    # 4-bit 80B 42 GB; the dense core resident in memory is ~1.3 GB / ~2.5 GB (paragraph on
    # scheduling). Runnel README, "Reproducibility tools": the 8-bit 35B shards total 36.8 GB.
    def routed(w):
        return w.n_layers * w.shape.num_experts * w.shape.expert_bytes()
    assert abs(routed(synth.QWEN35B_4BIT) / 1e9 - (18.0 - 1.3)) / 18.0 < 0.10
    assert abs(routed(synth.QWEN80B_4BIT) / 1e9 - (42.0 - 2.5)) / 42.0 < 0.10
    assert 0.85 < routed(synth.QWEN35B_8BIT) / 1e9 / 36.8 < 1.0


def test_decode_bytes_per_token():
    assert synth.algorithmic_decode_bytes(synth.QWEN35B_4BIT.shape) == 18042880
    assert synth.algorithmic_decode_bytes(synth.QWEN80B_4BIT.shape) == 23678976
    assert synth.algorithmic_decode_bytes(synth.QWEN35B_8BIT.shape) == 32198656


def test_multi_token_step_bytes_count_shared_weights_once():
    """bench.py's bytes of a T-token decode step: at T = 1 the per-token model times the layers;
    for T > 1 the router, shared gate and shared expert once per layer, each distinct routed expert
    once per layer, x and y per token."""
    import os
    import sys

    import torch
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    s = synth.QWEN35B_4BIT.shape
    L = 40
    assert bench.decode_step_bytes(s, L, 1) == L * synth.algorithmic_decode_bytes(s)
    T, K, E, H = 4, s.top_k, s.num_experts, s.hidden
    same = torch.arange(K, dtype=torch.int32).repeat(2, L, T, 1)  # every token picks experts 0..K-1
    once = 4 * E * H + 4 * H + s.expert_bytes(s.shared_inter)
    assert bench.decode_step_bytes(s, L, T, same) == L * (once + T * 6 * H + K * s.expert_bytes())
    disjoint = torch.arange(T * K, dtype=torch.int32).view(T, K).repeat(3, L, 1, 1)
    assert bench.decode_step_bytes(s, L, T, disjoint) == L * (once + T * 6 * H + T * K * s.expert_bytes())
    # the old model (per-token bytes times T) overcounts a step
    assert bench.decode_step_bytes(s, L, T, same) < L * T * synth.algorithmic_decode_bytes(s)


def test_pct_interpolates():
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    assert bench._pct([1.0, 2.0, 3.0, 4.0, 5.0], 50) == 3.0
    assert abs(bench._pct([0.0, 10.0], 10) - 1.0) < 1e-12
    assert bench._pct([7.0], 90) == 7.0
