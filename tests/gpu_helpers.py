"""Shared helpers of the GPU parity tests (not a test module)."""
from __future__ import annotations

import contextlib

import numpy as np
import torch

import oracle as O
from workloads import round_to_bf16

TOL = {"bf16": 2e-2, "f32": 1e-5}
GAP = 1e-4


def tdtype(dt: str):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def to_dev(x: np.ndarray, dt: str) -> torch.Tensor:
    """Upload values that are already representable in dt."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(tdtype(dt)).contiguous()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / (den if den > 0 else 1.0))


def assert_close(got, ref, dt, name):
    e = rel_err(got, ref)
    assert e <= TOL[dt], f"{name}: max-abs-err/|ref|_inf = {e:.3e} > {TOL[dt]:.0e}"
    return e


def factors(W: np.ndarray, rank: int, dt: str):
    """Estimator factors from the oracle's SVD, rounded to the call dtype:
    Pt [rank, in] and Q [rank, out]."""
    P, Q, _ = O.build_estimator(W, rank)
    Pt = np.ascontiguousarray(P.T, dtype=np.float32)
    Q = np.ascontiguousarray(Q, dtype=np.float32)
    if dt == "bf16":
        Pt, Q = round_to_bf16(Pt), round_to_bf16(Q)
    return Pt, Q


def check_selection(gpu_idx: np.ndarray, ora_scores: np.ndarray, k: int):
    """Index sets must be bit-exact wherever the k-th and (k+1)-th oracle scores
    differ by more than GAP relative.  Otherwise the GPU set must be a top-k of
    the oracle scores up to GAP: it holds every channel whose oracle score
    exceeds s_k (1 + GAP), and every channel it holds scores at least
    s_k (1 - GAP) (s_k = the k-th largest oracle score).  Returns the number of
    sequences compared exactly."""
    B, N = ora_scores.shape
    exact = 0
    for b in range(B):
        g = np.asarray(gpu_idx[b])
        assert len(g) == k and len(np.unique(g)) == k, f"seq {b}: indices not k distinct"
        assert np.all(np.diff(g) > 0), f"seq {b}: indices not ascending"
        assert g.min() >= 0 and g.max() < N, f"seq {b}: index out of range"
        s = ora_scores[b].astype(np.float64)
        ref = O.select_topk(ora_scores[b], k)
        if k == N:
            assert np.array_equal(g, np.arange(N))
            exact += 1
            continue
        order = np.lexsort((np.arange(N), -s))
        sk, sk1 = s[order[k - 1]], s[order[k]]
        if sk > 0 and (sk - sk1) / sk > GAP:
            assert np.array_equal(g, ref), f"seq {b}: index set differs with gap {(sk - sk1) / sk:.2e}"
            exact += 1
        else:
            must = np.nonzero(s > sk * (1 + GAP))[0]
            missing = np.setdiff1d(must, g)
            assert missing.size == 0, f"seq {b}: channels {missing[:8].tolist()} above s_k (1 + GAP) not chosen"
            assert s[g].min() >= sk * (1 - GAP) - 1e-30, f"seq {b}: a chosen score is below s_k (1 - GAP)"
    return exact


def check_scores(gpu_scores: np.ndarray, ora_scores: np.ndarray, tol: float, what: str = "scores"):
    """Per sequence, max |gpu - oracle| / max(oracle) <= tol."""
    for b in range(ora_scores.shape[0]):
        den = max(float(np.abs(ora_scores[b]).max()), 1e-30)
        e = float(np.abs(np.asarray(gpu_scores[b], np.float64) - ora_scores[b]).max()) / den
        assert e <= tol, f"{what}: seq {b} relative error {e:.2e} > {tol:.0e}"


@contextlib.contextmanager
def gemm_variant(variants: int):
    """Run the block with the given GEMM tile variants allowed (bit mask: 1
    wide N-gather, 2 tall 256 x 256 (N- and K-gather), 4 tall whatever the
    grid; 0 = 128 x 256 only)."""
    import contextual_sparsity_lora_svd_amd as sl
    prev = sl.gemm_config(variants)
    try:
        yield
    finally:
        sl.gemm_config(prev)
