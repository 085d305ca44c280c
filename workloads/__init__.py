"""Seeded synthetic workloads for the contextual-sparsity LoRA hot path.

This module only draws random inputs and describes their shapes.  It holds
none of the method's arithmetic: no estimator, no scores, no selection, no
forward or backward.  Both the CPU oracle (``oracle/``) and the HIP path's
tests and benchmark take their inputs from here, so the two sides see the
same numbers.

Input recipe (the pages evaluate on public task suites with trained LLaMA
weights; neither is available, so seeded synthetic layers of the same shapes
stand in for them):

* activations ``X = (Z @ M + 0.1 * E) * s`` with ``Z ~ N(0,1)[T x R_in]``,
  ``M ~ N(0,1)[R_in x D]``, ``E ~ N(0,1)[T x D]`` and per-feature scales
  ``s ~ LogNormal(0, 1)[D]`` applied after the noise;
* frozen weights and both LoRA factors ``~ N(0, 0.02^2)``;
* upstream gradients ``~ N(0, 1)``;
* every sequence is a context prompt followed by a dense output span at its
  end (SparseLoRA article, section on layer- and token-level sensitivity).

Seeds: ``numpy.random.default_rng(1000 * cfg + slot [+ 100 * layer])``.  Slots:
0 Z, 1 M, 2 E, 3 feature scales, 4..7 the same four for the attention input
``a``, 10+ frozen weights in declaration order, 30+ LoRA factors, 50+
upstream gradients, 60 output-span lengths.

Values for bf16 workloads are drawn in fp32 and rounded once to the nearest
bf16 (ties to even); both sides then read exactly the same values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "FFNShape", "AttnShape", "Workload", "WORKLOADS", "round_to_bf16", "make_planted_weight",
    "make_activations", "make_ffn_tensors", "make_attn_tensors", "output_spans",
    "ctx_lengths",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even), kept as fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32)


@dataclass(frozen=True)
class FFNShape:
    d_model: int
    d_ff: int
    lora_rank: int
    sparsity_pct: int          # per-layer channel sparsity (percent of d_ff dropped)


@dataclass(frozen=True)
class AttnShape:
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    lora_rank: int
    sparsity_qk_pct: int
    sparsity_vo_pct: int


@dataclass
class Workload:
    """One of the synthetic workloads: shapes, token layout and precision."""
    cfg: int
    name: str
    dtype: str                   # "f32" or "bf16"
    batch: int
    seq_len: int
    rank_in: int                 # rank of the low-rank part of X
    est_rank: int                # estimator (truncated SVD) rank
    ffn: List[FFNShape] = field(default_factory=list)    # one per layer
    attn: List[AttnShape] = field(default_factory=list)  # one per layer
    out_len: Optional[int] = None   # fixed output span per sequence, or None = drawn
    out_range: Optional[tuple] = None  # (lo, hi) inclusive when drawn

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny-swiglu-ffn-fp32", "f32", batch=2, seq_len=64, rank_in=32,
                est_rank=8, ffn=[FFNShape(256, 688, 8, 50)], out_len=16),
    2: Workload(2, "llama2-7b-ffn", "bf16", batch=4, seq_len=512, rank_in=64,
                est_rank=8, ffn=[FFNShape(4096, 11008, 16, 75)], out_len=128),
    3: Workload(3, "llama2-7b-qkvo", "bf16", batch=2, seq_len=1024, rank_in=64,
                est_rank=8, attn=[AttnShape(4096, 32, 32, 128, 16, 50, 50)], out_len=256),
    4: Workload(4, "llama2-7b-4-layer-stack", "bf16", batch=4, seq_len=512, rank_in=64,
                est_rank=8,
                ffn=[FFNShape(4096, 11008, 16, p) for p in (0, 30, 60, 90)],
                attn=[AttnShape(4096, 32, 32, 128, 16, p, p) for p in (0, 30, 60, 90)],
                out_range=(32, 256)),
    5: Workload(5, "llama3-8b-long-context", "bf16", batch=1, seq_len=4096, rank_in=128,
                est_rank=16, ffn=[FFNShape(4096, 14336, 32, 90)],
                attn=[AttnShape(4096, 32, 8, 128, 32, 50, 0)], out_len=512),
    # extreme-sparsity regime at the LLaMA2-7B shapes: 99 % of d_ff dropped
    # (k = 110 of 11008) and 75 % of the q/k and v/o channels
    6: Workload(6, "llama2-7b-extreme-sparsity", "bf16", batch=4, seq_len=512, rank_in=64,
                est_rank=8, ffn=[FFNShape(4096, 11008, 16, 99)],
                attn=[AttnShape(4096, 32, 32, 128, 16, 75, 75)], out_len=128),
}


def _rng(cfg: int, slot: int, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng(1000 * cfg + slot + 100 * layer)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


def output_spans(w: Workload) -> np.ndarray:
    """Length of the dense output span at the end of each sequence."""
    if w.out_len is not None:
        return np.full(w.batch, w.out_len, dtype=np.int64)
    lo, hi = w.out_range
    return _rng(w.cfg, 60).integers(lo, hi + 1, size=w.batch).astype(np.int64)


def ctx_lengths(w: Workload) -> np.ndarray:
    """Number of context tokens at the start of each sequence."""
    return (w.seq_len - output_spans(w)).astype(np.int32)


def make_activations(cfg: int, tokens: int, d_model: int, rank_in: int, dtype: str,
                     layer: int = 0, slot0: int = 0) -> np.ndarray:
    """``(Z @ M + 0.1 E) * s`` with a low-rank part and log-normal feature scales."""
    z = _rng(cfg, slot0 + 0, layer).standard_normal((tokens, rank_in), dtype=np.float32)
    m = _rng(cfg, slot0 + 1, layer).standard_normal((rank_in, d_model), dtype=np.float32)
    e = _rng(cfg, slot0 + 2, layer).standard_normal((tokens, d_model), dtype=np.float32)
    s = _rng(cfg, slot0 + 3, layer).lognormal(0.0, 1.0, size=d_model).astype(np.float32)
    x = (z @ m + np.float32(0.1) * e) * s[None, :]
    return _finish(x, dtype)


def _normal(cfg: int, slot: int, layer: int, shape, std: float, dtype: str) -> np.ndarray:
    x = _rng(cfg, slot, layer).standard_normal(shape, dtype=np.float32) * np.float32(std)
    return _finish(x, dtype)


def make_planted_weight(seed: int, out_f: int, in_f: int, alpha: float, dtype: str) -> np.ndarray:
    """``U diag(sigma) V^T`` with Haar-like orthonormal ``U [out, m]``, ``V [in, m]``
    (QR of Gaussians), ``m = min(out, in)`` and a power-law spectrum
    ``sigma_i ~ i^-alpha``, scaled to the mean square of ``N(0, 0.02^2)`` entries."""
    rng = np.random.default_rng(seed)
    m = min(out_f, in_f)
    U, _ = np.linalg.qr(rng.standard_normal((out_f, m)).astype(np.float32))
    V, _ = np.linalg.qr(rng.standard_normal((in_f, m)).astype(np.float32))
    s = np.arange(1, m + 1, dtype=np.float64) ** -float(alpha)
    s *= np.sqrt(out_f * in_f * 4e-4 / (s * s).sum())
    return _finish((U * s.astype(np.float32)) @ V.T, dtype)


def make_ffn_tensors(w: Workload, layer: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of one SwiGLU FFN layer in the natural (PyTorch Linear) layouts.

    ``Wg, Wu`` are ``[d_ff, d_model]``, ``Wd`` is ``[d_model, d_ff]``; LoRA
    ``A*`` are ``[r, in]`` and ``B*`` are ``[out, r]``.
    """
    f = w.ffn[layer]
    D, F, r, T = f.d_model, f.d_ff, f.lora_rank, w.tokens
    c, dt = w.cfg, w.dtype
    return {
        "X": make_activations(c, T, D, w.rank_in, dt, layer),
        "Wg": _normal(c, 10, layer, (F, D), 0.02, dt),
        "Wu": _normal(c, 11, layer, (F, D), 0.02, dt),
        "Wd": _normal(c, 12, layer, (D, F), 0.02, dt),
        "Ag": _normal(c, 30, layer, (r, D), 0.02, dt),
        "Bg": _normal(c, 31, layer, (F, r), 0.02, dt),
        "Au": _normal(c, 32, layer, (r, D), 0.02, dt),
        "Bu": _normal(c, 33, layer, (F, r), 0.02, dt),
        "Ad": _normal(c, 34, layer, (r, F), 0.02, dt),
        "Bd": _normal(c, 35, layer, (D, r), 0.02, dt),
        "dY": _normal(c, 50, layer, (T, D), 1.0, dt),
    }


def make_attn_tensors(w: Workload, layer: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of one q/k/v/o projection block in the natural layouts.

    ``Wq [Hq*hd, D]``, ``Wk, Wv [Hkv*hd, D]``, ``Wo [D, Hq*hd]``; ``a`` is the
    attention output ``[T, Hq*hd]`` that feeds the o projection.
    """
    s = w.attn[layer]
    D, r, T = s.d_model, s.lora_rank, w.tokens
    nq, nkv = s.n_q_heads * s.head_dim, s.n_kv_heads * s.head_dim
    c, dt = w.cfg, w.dtype
    base = 20 if w.ffn else 10   # attention weights follow the FFN weights when both exist
    lbase = 40 if w.ffn else 30
    gbase = 54 if w.ffn else 50
    return {
        "X": make_activations(c, T, D, w.rank_in, dt, layer),
        "a": make_activations(c, T, nq, w.rank_in, dt, layer, slot0=4),
        "Wq": _normal(c, base + 0, layer, (nq, D), 0.02, dt),
        "Wk": _normal(c, base + 1, layer, (nkv, D), 0.02, dt),
        "Wv": _normal(c, base + 2, layer, (nkv, D), 0.02, dt),
        "Wo": _normal(c, base + 3, layer, (D, nq), 0.02, dt),
        "Aq": _normal(c, lbase + 0, layer, (r, D), 0.02, dt),
        "Bq": _normal(c, lbase + 1, layer, (nq, r), 0.02, dt),
        "Ak": _normal(c, lbase + 2, layer, (r, D), 0.02, dt),
        "Bk": _normal(c, lbase + 3, layer, (nkv, r), 0.02, dt),
        "Av": _normal(c, lbase + 4, layer, (r, D), 0.02, dt),
        "Bv": _normal(c, lbase + 5, layer, (nkv, r), 0.02, dt),
        "Ao": _normal(c, lbase + 6, layer, (r, nq), 0.02, dt),
        "Bo": _normal(c, lbase + 7, layer, (D, r), 0.02, dt),
        "dq": _normal(c, gbase + 0, layer, (T, nq), 1.0, dt),
        "dk": _normal(c, gbase + 1, layer, (T, nkv), 1.0, dt),
        "dv": _normal(c, gbase + 2, layer, (T, nkv), 1.0, dt),
        "d_out": _normal(c, gbase + 3, layer, (T, D), 1.0, dt),
    }
