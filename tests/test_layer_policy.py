"""Host policy around the kernels: dense warm-up and per-layer ratios
(SparseLoRA article §三 and §四)."""
import pytest

from contextual_sparsity_lora_svd_amd.layer import LayerRatios, SparsitySchedule


def test_dense_warmup_is_the_first_tenth():
    s = SparsitySchedule([LayerRatios(ffn=75)], total_steps=1000)
    assert s.dense_steps == 100
    assert s.is_dense(0) and s.is_dense(99) and not s.is_dense(100)
    assert s.k(0, 99, "ffn", 11008) == 11008
    assert s.k(0, 100, "ffn", 11008) == 2752
    # rounding up: 7 steps at 10 % -> one dense step; no warm-up at 0 %
    assert SparsitySchedule([LayerRatios()], 7).dense_steps == 1
    assert SparsitySchedule([LayerRatios(ffn=50)], 7, dense_fraction=0.0).k(0, 0, "ffn", 10) == 5


def test_ratios_from_layer_ranges():
    # a layer-range configuration of the kind the article's implementation section
    # describes: most FFNs at 99 %, some attention projections sparse, the rest dense
    s = SparsitySchedule.from_ranges(32, total_steps=100, ffn=[(2, 29, 99)], qk=[(13, 28, 75)],
                                     vo=[(13, 28, 50)])
    assert s.dense_steps == 10
    assert s.ratios[0] == LayerRatios(0, 0, 0) and s.ratios[31] == LayerRatios(0, 0, 0)
    assert s.ratios[2] == LayerRatios(99, 0, 0) and s.ratios[13] == LayerRatios(99, 75, 50)
    assert s.k(5, 50, "ffn", 14336) == 143        # round half up of 1 % of 14336
    assert s.k(5, 5, "ffn", 14336) == 14336       # still dense
    assert s.k(0, 50, "ffn", 14336) == 14336      # a dense layer
    assert s.k(20, 50, "qk", 1024) == 256 and s.k(20, 50, "vo", 1024) == 512
    # a later range overrides an earlier one
    t = SparsitySchedule.from_ranges(4, 10, ffn=[(0, 3, 50), (1, 2, 90)])
    assert [r.ffn for r in t.ratios] == [50, 90, 90, 50]


def test_schedule_rejects_bad_input():
    with pytest.raises(ValueError):
        SparsitySchedule([LayerRatios(ffn=100)], 10)
    with pytest.raises(ValueError):
        SparsitySchedule([LayerRatios()], 0)
    with pytest.raises(ValueError):
        SparsitySchedule.from_ranges(4, 10, ffn=[(2, 5, 50)])


def test_quantized_base_option_is_validated_on_the_host():
    import torch
    import contextual_sparsity_lora_svd_amd as sl
    from contextual_sparsity_lora_svd_amd.layer import _quantized_base
    frozen = {"Wg": torch.zeros(4, 64)}
    assert _quantized_base(frozen, 16, torch.float32) is frozen
    with pytest.raises(sl.SparseLoraError):
        _quantized_base(frozen, 8, torch.bfloat16)
    with pytest.raises(sl.SparseLoraError):
        _quantized_base(frozen, 4, torch.float32)
