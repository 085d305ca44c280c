"""Contextual-sparsity LoRA (SparseLoRA-style) hot path for MI355X / gfx950.

The computation lives in libsparselora.so (hand-written HIP kernels behind the
C ABI in include/sparselora.h); this package is its Python binding.
"""
from .api import (  # noqa: F401
    SL_BF16, SL_CRIT_L2, SL_CRIT_QK_NORM, SL_CRIT_SWIGLU_L2, SL_F32, SL_MAX_SEQS, LIB_PATH,
    SIGNATURES, SL_EST_MAXJOBS, EstimateBuffers, EstimateMultiBuffers, FFNWeights, FFNWorkspace, Layout, QKVOWeights, QKVOWorkspace, SparseLoraError,
    TIMER_SLOTS, build_estimator, estimate_select, estimate_select_multi, estimate_select_noalloc, gemm_config, quantize_q4, timer_enable, timer_read, timer_reset, timer_select, ffn_bwd, ffn_fwd, k_from_ratio, lib, qkvo_bwd, qkvo_fwd,
)
from .layer import LayerRatios, SparseLoRAFFN, SparseLoRAQKVO, SparsitySchedule  # noqa: F401,E402
