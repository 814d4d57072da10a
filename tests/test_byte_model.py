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
