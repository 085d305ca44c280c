"""Training-step policy around the sparse LoRA kernels, and torch autograd
modules that run them.

SparseLoRA article §三: layers differ in how much sparsity they tolerate
(shallow layers kept denser than deep ones), so the ratio is set per layer and
per projection group; context rows are computed sparsely and output rows
densely.  §四: training starts dense (about the first tenth of the steps) and
switches to sparse computation after that.  §七: a configuration names layer
ranges and a ratio per range (e.g. 99 % of the FFN channels in a range of
layers).

Everything here is host-side bookkeeping: which k each call uses, the channel
sets (all channels while dense, the estimator's per-sequence choice after), the
buffers, and the routing of gradients.  Every arithmetic step runs in
libsparselora.so; the attention core between the q/k/v and o projections is
the caller's.
"""
import math
from dataclasses import dataclass
from typing import Callable, Dict, Optional, Sequence, Tuple

import torch

from . import api as sl

__all__ = ["LayerRatios", "SparsitySchedule", "SparseLoRAFFN", "SparseLoRAQKVO"]


@dataclass(frozen=True)
class LayerRatios:
    """Percent of channels dropped in one layer: FFN (of d_ff), q/k and v/o
    (of the kv channels n_kv_heads * head_dim)."""
    ffn: int = 0
    qk: int = 0
    vo: int = 0


class SparsitySchedule:
    """Per-layer ratios plus the dense warm-up.

    Steps ``0 .. dense_steps - 1`` are dense (k = N, no estimator), with
    ``dense_steps = ceil(dense_fraction * total_steps)``; every later step uses
    ``k = k_from_ratio(N, ratio)`` of its layer (a ratio of 0 stays dense)."""

    def __init__(self, ratios: Sequence[LayerRatios], total_steps: int, dense_fraction: float = 0.1):
        if total_steps < 1:
            raise ValueError("total_steps must be >= 1")
        if not 0.0 <= dense_fraction <= 1.0:
            raise ValueError("dense_fraction must be in [0, 1]")
        for r in ratios:
            for p in (r.ffn, r.qk, r.vo):
                if not 0 <= p < 100:
                    raise ValueError(f"ratio {p} outside [0, 100)")
        self.ratios = tuple(ratios)
        self.total_steps = int(total_steps)
        self.dense_steps = int(math.ceil(dense_fraction * total_steps))

    @classmethod
    def from_ranges(cls, n_layers: int, total_steps: int, ffn: Sequence[Tuple[int, int, int]] = (),
                    qk: Sequence[Tuple[int, int, int]] = (), vo: Sequence[Tuple[int, int, int]] = (),
                    dense_fraction: float = 0.1) -> "SparsitySchedule":
        """Ratios given as ``(first_layer, last_layer, percent)`` ranges,
        inclusive; layers outside every range stay dense.  A later range
        overrides an earlier one where they overlap."""
        per = [[0, 0, 0] for _ in range(n_layers)]
        for slot, ranges in enumerate((ffn, qk, vo)):
            for first, last, pct in ranges:
                if not 0 <= first <= last < n_layers:
                    raise ValueError(f"layer range {first}..{last} outside 0..{n_layers - 1}")
                for layer in range(first, last + 1):
                    per[layer][slot] = int(pct)
        return cls([LayerRatios(*p) for p in per], total_steps, dense_fraction)

    def is_dense(self, step: int) -> bool:
        return step < self.dense_steps

    def k(self, layer: int, step: int, kind: str, n: int) -> int:
        """Channels kept by projection group ``kind`` ("ffn", "qk", "vo") of
        ``layer`` at ``step``, out of ``n``."""
        if self.is_dense(step):
            return n
        pct = getattr(self.ratios[layer], kind)
        return n if pct == 0 else sl.k_from_ratio(n, pct)


def _all_channels(batch: int, n: int, device) -> torch.Tensor:
    return torch.arange(n, dtype=torch.int32, device=device).repeat(batch, 1).contiguous()


class _FFNStep(torch.autograd.Function):
    """Y = FFN(X) on the channel sets idx; gradients of X and the six LoRA
    factors from the kernels' backward."""

    @staticmethod
    def forward(ctx, X, Ag, Bg, Au, Bu, Ad, Bd, mod, layout, k, idx):
        lora = {n: t.detach().to(mod.dtype).contiguous()
                for n, t in zip(("Ag", "Bg", "Au", "Bu", "Ad", "Bd"), (Ag, Bg, Au, Bu, Ad, Bd))}
        t = dict(mod.frozen)
        t.update(lora)
        w = sl.FFNWeights(t, mod.lora_scale)
        Xc = X.detach().contiguous()
        Y, buf = sl.ffn_fwd(w, Xc, layout, k, idx, sl.FFNWorkspace(w, layout, k, X.device))
        ctx.state = (w, Xc, layout, k, idx, buf)
        return Y

    @staticmethod
    def backward(ctx, dY):
        w, Xc, layout, k, idx, buf = ctx.state
        g = sl.ffn_bwd(w, Xc, layout, k, idx, buf, dY.contiguous())
        ctx.state = None
        return (g["dX"], g["dAg"], g["dBg"], g["dAu"], g["dBu"], g["dAd"], g["dBd"],
                None, None, None, None)


def _quantized_base(frozen, base_bits: int, dtype):
    """The frozen weights as given (16) or as 4-bit codes and block scales (4)."""
    if base_bits == 16:
        return frozen
    if base_bits != 4 or dtype != torch.bfloat16:
        raise sl.SparseLoraError("base_bits must be 16, or 4 with bf16 weights")
    out = {}
    for n, w in frozen.items():
        out[n + "_q"], out[n + "_s"] = sl.quantize_q4(w)
    return out


class SparseLoRAFFN(torch.nn.Module):
    """One SwiGLU FFN with LoRA on gate, up and down and contextual channel
    sparsity.  Frozen weights (``Wg, Wu [d_ff, d_model]``, ``Wd [d_model, d_ff]``)
    are held in the compute dtype, the LoRA factors as fp32 parameters (cast
    to the compute dtype for each call; their gradients arrive in fp32).  The
    rank-``est_rank`` estimator of gate and up is built once, at construction.
    ``base_bits=4`` keeps the frozen weights as 4-bit codes and block scales
    (bf16 only; the estimator is built from the weights before quantization)."""

    def __init__(self, Wg: torch.Tensor, Wu: torch.Tensor, Wd: torch.Tensor, lora_rank: int,
                 est_rank: int = 8, lora_scale: float = 1.0, layer: int = 0,
                 schedule: Optional[SparsitySchedule] = None, init_std: float = 0.02,
                 generator: Optional[torch.Generator] = None, base_bits: int = 16):
        super().__init__()
        dev, dt = Wg.device, Wg.dtype
        d_ff, d_model = Wg.shape
        self.dtype, self.lora_scale, self.layer, self.schedule = dt, float(lora_scale), layer, schedule
        self.d_model, self.d_ff, self.est_rank = d_model, d_ff, est_rank
        self.frozen = {"Wg": Wg.contiguous(), "Wu": Wu.contiguous(), "WdT": Wd.t().contiguous()}

        def p(*shape):
            x = torch.randn(*shape, generator=generator, dtype=torch.float32) * init_std
            return torch.nn.Parameter(x.to(dev))
        self.Ag, self.Bg = p(lora_rank, d_model), p(d_ff, lora_rank)
        self.Au, self.Bu = p(lora_rank, d_model), p(d_ff, lora_rank)
        self.Ad, self.Bd = p(lora_rank, d_ff), p(d_model, lora_rank)
        self.est = (sl.build_estimator(self.frozen["Wg"], est_rank)[:2],
                    sl.build_estimator(self.frozen["Wu"], est_rank)[:2])
        self.frozen = _quantized_base(self.frozen, base_bits, dt)
        self.last_k, self.last_idx = None, None

    def channel_sets(self, X: torch.Tensor, layout: sl.Layout, k: int) -> torch.Tensor:
        if k == self.d_ff:
            return _all_channels(layout.batch, self.d_ff, X.device)
        (Pg, Qg), (Pu, Qu) = self.est
        idx, _ = sl.estimate_select(sl.SL_CRIT_SWIGLU_L2, X, layout, self.est_rank, Pg, Qg, Pu, Qu,
                                    self.d_ff, k)
        return idx.clone()

    def forward(self, X: torch.Tensor, layout: sl.Layout, step: int = 0, k: Optional[int] = None):
        if k is None:
            k = self.schedule.k(self.layer, step, "ffn", self.d_ff) if self.schedule else self.d_ff
        idx = self.channel_sets(X, layout, k)
        self.last_k, self.last_idx = k, idx
        return _FFNStep.apply(X, self.Ag, self.Bg, self.Au, self.Bu, self.Ad, self.Bd, self, layout, k, idx)


class _QKVOState:
    """Buffers shared by the two halves of one q/k/v/o call (the saved LoRA
    activations of both live in one buffer)."""

    def __init__(self, w, layout, k_qk, idx_qk, k_vo, idx_vo, buf):
        self.w, self.layout, self.k_qk, self.idx_qk, self.k_vo, self.idx_vo, self.buf = (
            w, layout, k_qk, idx_qk, k_vo, idx_vo, buf)


class _QKVStep(torch.autograd.Function):
    @staticmethod
    def forward(ctx, X, Aq, Bq, Ak, Bk, Av, Bv, st):
        Xc = X.detach().contiguous()
        o, _ = sl.qkvo_fwd(st.w, Xc, None, st.layout, st.k_qk, st.idx_qk, st.k_vo, st.idx_vo, st.buf)
        ctx.state = (st, Xc)
        return o["q"], o["k"], o["v"]

    @staticmethod
    def backward(ctx, dq, dk, dv):
        st, Xc = ctx.state
        # an output the loss does not reach has no gradient: zeros stand in
        shapes = ((st.w.heads[0] * st.w.heads[2]), (st.w.heads[1] * st.w.heads[2]))
        T = Xc.shape[0]
        z = lambda g, n: g.contiguous() if g is not None else torch.zeros(T, n, dtype=Xc.dtype,
                                                                          device=Xc.device)
        g = sl.qkvo_bwd(st.w, Xc, None, st.layout, st.k_qk, st.idx_qk, st.k_vo, st.idx_vo, st.buf,
                        dq=z(dq, shapes[0]), dk=z(dk, shapes[1]), dv=z(dv, shapes[1]))
        ctx.state = None
        return g["dX"], g["dAq"], g["dBq"], g["dAk"], g["dBk"], g["dAv"], g["dBv"], None


class _OStep(torch.autograd.Function):
    @staticmethod
    def forward(ctx, a, Ao, Bo, st):
        ac = a.detach().contiguous()
        o, _ = sl.qkvo_fwd(st.w, None, ac, st.layout, st.k_qk, st.idx_qk, st.k_vo, st.idx_vo, st.buf)
        ctx.state = (st, ac)
        return o["o"]

    @staticmethod
    def backward(ctx, d_out):
        st, ac = ctx.state
        g = sl.qkvo_bwd(st.w, None, ac, st.layout, st.k_qk, st.idx_qk, st.k_vo, st.idx_vo, st.buf,
                        d_out=d_out.contiguous())
        ctx.state = None
        return g["da"], g["dAo"], g["dBo"], None


class SparseLoRAQKVO(torch.nn.Module):
    """q/k/v/o projections with LoRA and contextual channel sparsity (QK-norm
    selection for q/k, L2 of v for v/o), around the caller's attention core:

        out = module(X, layout, attention, step)

    with ``attention(q, k, v) -> a`` on token-major ``[T, H * head_dim]``
    tensors (differentiable with torch autograd).  Frozen weights ``Wq [Hq hd, D]``,
    ``Wk, Wv [Hkv hd, D]``, ``Wo [D, Hq hd]`` in the compute dtype; LoRA
    factors fp32 parameters.  ``base_bits=4``: the frozen weights as 4-bit
    codes and block scales (as in SparseLoRAFFN)."""

    def __init__(self, Wq, Wk, Wv, Wo, heads: Sequence[int], lora_rank: int, est_rank: int = 8,
                 lora_scale: float = 1.0, layer: int = 0, schedule: Optional[SparsitySchedule] = None,
                 init_std: float = 0.02, generator: Optional[torch.Generator] = None, base_bits: int = 16):
        super().__init__()
        dev, dt = Wq.device, Wq.dtype
        self.heads = tuple(int(h) for h in heads)
        hq, hkv, hd = self.heads
        D = Wq.shape[1]
        self.dtype, self.lora_scale, self.layer, self.schedule = dt, float(lora_scale), layer, schedule
        self.d_model, self.nq, self.nkv, self.est_rank = D, hq * hd, hkv * hd, est_rank
        self.frozen = {"Wq": Wq.contiguous(), "Wk": Wk.contiguous(), "Wv": Wv.contiguous(),
                       "WoT": Wo.t().contiguous()}

        def p(*shape):
            x = torch.randn(*shape, generator=generator, dtype=torch.float32) * init_std
            return torch.nn.Parameter(x.to(dev))
        self.Aq, self.Bq = p(lora_rank, D), p(self.nq, lora_rank)
        self.Ak, self.Bk = p(lora_rank, D), p(self.nkv, lora_rank)
        self.Av, self.Bv = p(lora_rank, D), p(self.nkv, lora_rank)
        self.Ao, self.Bo = p(lora_rank, self.nq), p(D, lora_rank)
        self.est = {n: sl.build_estimator(self.frozen[n], est_rank)[:2] for n in ("Wq", "Wk", "Wv")}
        self.frozen = _quantized_base(self.frozen, base_bits, Wq.dtype)
        self.last_k, self.last_idx = None, None

    def channel_sets(self, X, layout, k_qk, k_vo):
        B = layout.batch
        if k_qk < self.nkv and k_vo < self.nkv:
            # both sets estimated: one call projects X once for q, k and v
            (Pq, Qq), (Pk, Qk), (Pv, Qv) = self.est["Wq"], self.est["Wk"], self.est["Wv"]
            jobs = [dict(crit=sl.SL_CRIT_QK_NORM, Pt0=Pq, Q0=Qq, Pt1=Pk, Q1=Qk, N=self.nkv, k=k_qk,
                         heads=self.heads),
                    dict(crit=sl.SL_CRIT_L2, Pt0=Pv, Q0=Qv, N=self.nkv, k=k_vo)]
            (iqk, _), (ivo, _) = sl.estimate_select_multi(X, layout, self.est_rank, jobs)
            return iqk, ivo
        if k_qk == self.nkv:
            iqk = _all_channels(B, self.nkv, X.device)
        else:
            (Pq, Qq), (Pk, Qk) = self.est["Wq"], self.est["Wk"]
            iqk, _ = sl.estimate_select(sl.SL_CRIT_QK_NORM, X, layout, self.est_rank, Pq, Qq, Pk, Qk,
                                        self.nkv, k_qk, heads=self.heads)
            iqk = iqk.clone()
        if k_vo == self.nkv:
            ivo = _all_channels(B, self.nkv, X.device)
        else:
            Pv, Qv = self.est["Wv"]
            ivo, _ = sl.estimate_select(sl.SL_CRIT_L2, X, layout, self.est_rank, Pv, Qv, None, None,
                                        self.nkv, k_vo)
            ivo = ivo.clone()
        return iqk, ivo

    def forward(self, X: torch.Tensor, layout: sl.Layout, attention: Callable, step: int = 0,
                k_qk: Optional[int] = None, k_vo: Optional[int] = None):
        s = self.schedule
        if k_qk is None:
            k_qk = s.k(self.layer, step, "qk", self.nkv) if s else self.nkv
        if k_vo is None:
            k_vo = s.k(self.layer, step, "vo", self.nkv) if s else self.nkv
        iqk, ivo = self.channel_sets(X, layout, k_qk, k_vo)
        lora = {n: getattr(self, n).detach().to(self.dtype).contiguous()
                for n in ("Aq", "Bq", "Ak", "Bk", "Av", "Bv", "Ao", "Bo")}
        t = dict(self.frozen)
        t.update(lora)
        w = sl.QKVOWeights(t, self.heads, self.lora_scale)
        st = _QKVOState(w, layout, k_qk, iqk, k_vo, ivo, sl.QKVOWorkspace(w, layout, k_qk, k_vo, X.device))
        st.lora = lora   # keep the cast factors alive for the backward
        self.last_k, self.last_idx = (k_qk, k_vo), (iqk, ivo)
        q, k, v = _QKVStep.apply(X, self.Aq, self.Bq, self.Ak, self.Bk, self.Av, self.Bv, st)
        a = attention(q, k, v)
        return _OStep.apply(a.contiguous(), self.Ao, self.Bo, st)
