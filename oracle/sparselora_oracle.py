"""CPU oracle for contextual-sparsity LoRA (SparseLoRA-style): TEST INFRASTRUCTURE.

This module is the plain, slow, obviously correct statement of what the
hot path computes.  Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the product library never does.  It shares no code
with the HIP path.

Sources (the pages):
  * "SparseLoRA article" = the lsdiaocha.cn write-up of SparseLoRA
    (ICML 2025), sections 一 (dynamic sparsity), 二 (SVD sparsity
    estimator), 三 (layer and token sensitivity), 六 (compatibility) and
    七 (implementation details).
  * "SparseLoRA abstract" = the xinfinite.net page "SparseLoRA：利用上下文
    稀疏性高效微调大语言模型", translated abstract paragraph.
  * "SALR page" = the lshu.cn SALR article, section 2.1, for the LoRA
    notation (frozen W plus a trained low-rank product of two factors).

Precision: every forward/backward quantity is computed in float64 from the
(already rounded) input values.  The channel scores decide an integer (the
selected set), so ``scores_*`` take a ``dtype`` and are evaluated in float32
when they are compared with the GPU, which scores in float32.

Readings where the pages are silent (each is listed in the design notes):
  R1 FFN activity is the SwiGLU intermediate h = SiLU(g) * u, estimated
     from both the gate and up factors.
  R2 the criterion is the sum of squares over the sequence's context
     tokens (monotone in the L2 norm); output tokens do not vote.
  R3 LoRA form y = x W^T + s (x A^T) B^T with A [r, in], B [out, r].
  R4 a dropped channel drops its LoRA part too (masked-dense form).
  R5 k from a percentage: round half up of (100 - p) * N / 100 in integers.
  R6 ties in the score order go to the lower channel index; the selected
     indices are returned in ascending order.
  R7 QK criterion, grouped-query form: the score of kv channel (g, d) is
     ||k_(g,d)||^2 * sum over the G query heads of group g of ||q_(h,d)||^2,
     which for G = 1 is (||q_c|| ||k_c||)^2.
  R8 v and o share one set chosen by the L2 score of v; o's input columns
     use it expanded to the query heads.
  R9 the estimator factors the frozen weight only; it never sees LoRA.
  R10 the singular values are folded into P: P = V_r diag(sigma_r),
      Q = U_r^T, so x P Q approximates x W^T.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

F64 = np.float64

__all__ = [
    "k_from_ratio", "build_estimator", "estimator_bytes", "silu", "sigmoid",
    "context_rows", "scores_swiglu_l2", "scores_l2", "scores_qk_norm",
    "select_topk", "expand_kv_to_q", "ffn_masks", "ffn_forward", "ffn_backward",
    "attn_masks", "qkvo_forward", "qkvo_backward", "estimate_select_ffn",
]


# --------------------------------------------------------------------------
# configuration arithmetic
# --------------------------------------------------------------------------
def k_from_ratio(n: int, sparsity_pct: int) -> int:
    """Channels kept at a per-layer sparsity percentage (reading R5).

    The per-layer ratio is SparseLoRA article §三 (non-uniform layer-wise
    sparsity) and §七 (per-layer configuration); the rounding is ours.
    """
    if not (0 <= sparsity_pct < 100):
        raise ValueError("sparsity percentage must be in [0, 100)")
    k = (n * (100 - sparsity_pct) + 50) // 100
    return max(int(k), 1)


# --------------------------------------------------------------------------
# a0: offline estimator build
# --------------------------------------------------------------------------
def build_estimator(W: np.ndarray, rank: int):
    """Truncated SVD of a frozen projection weight W [out, in].

    SparseLoRA article §二: the pretrained weight is decomposed once before
    training and only the leading singular values and vectors are kept;
    §七: rank 8 is the chosen trade-off.  Returns P [in, rank],
    Q [rank, out] and sigma [rank] with x @ P @ Q ~= x @ W.T (reading R10).
    """
    U, S, Vt = np.linalg.svd(np.asarray(W, dtype=F64), full_matrices=False)
    P = Vt[:rank].T * S[:rank][None, :]
    Q = U[:, :rank].T.copy()
    return P, Q, S[:rank].copy()


def estimator_bytes(projections: Sequence[tuple], rank: int, n_layers: int,
                    bytes_per_value: int = 2) -> int:
    """Memory of the estimator factors: per projection (out, in) the factors
    hold rank * (out + in) values (SparseLoRA article §七 quotes about 30 MB
    at rank 8)."""
    per_layer = sum(rank * (o + i) for (o, i) in projections)
    return per_layer * n_layers * bytes_per_value


# --------------------------------------------------------------------------
# a1/a2: scores over context tokens
# --------------------------------------------------------------------------
def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def context_rows(ctx_len: Sequence[int], seq_len: int, b: int) -> np.ndarray:
    """Token rows of sequence b that are context (its first ctx_len[b] rows).

    SparseLoRA article §三: context tokens are computed sparsely, the output
    tokens at the end of each sequence stay dense.
    """
    return np.arange(b * seq_len, b * seq_len + int(ctx_len[b]))


def scores_swiglu_l2(Xc, Pg, Qg, Pu, Qu, dtype=np.float32):
    """L2 activity of each FFN channel over one sequence's context tokens.

    SparseLoRA article §一 (L2-norm criterion for the FFN) and §二 (activations
    approximated through the low-rank factors); readings R1, R2.
    """
    Xc = np.asarray(Xc, dtype=dtype)
    g = (Xc @ np.asarray(Pg, dtype)) @ np.asarray(Qg, dtype)
    u = (Xc @ np.asarray(Pu, dtype)) @ np.asarray(Qu, dtype)
    one = dtype(1.0)
    h = g / (one + np.exp(-g)) * u
    return (h * h).sum(axis=0, dtype=dtype)


def scores_l2(Xc, P, Q, dtype=np.float32):
    """L2 criterion of a plain projection (v, and o through v): reading R8."""
    Xc = np.asarray(Xc, dtype=dtype)
    v = (Xc @ np.asarray(P, dtype)) @ np.asarray(Q, dtype)
    return (v * v).sum(axis=0, dtype=dtype)


def scores_qk_norm(Xc, Pq, Qq, Pk, Qk, n_q_heads, n_kv_heads, head_dim,
                   dtype=np.float32):
    """QK-norm criterion in kv-channel space (SparseLoRA article §一; R7).

    Returns one score per kv channel (g, d), index g * head_dim + d.
    """
    Xc = np.asarray(Xc, dtype=dtype)
    q = (Xc @ np.asarray(Pq, dtype)) @ np.asarray(Qq, dtype)
    k = (Xc @ np.asarray(Pk, dtype)) @ np.asarray(Qk, dtype)
    sq = (q * q).sum(axis=0, dtype=dtype).reshape(n_q_heads, head_dim)
    sk = (k * k).sum(axis=0, dtype=dtype).reshape(n_kv_heads, head_dim)
    G = n_q_heads // n_kv_heads
    sq_group = sq.reshape(n_kv_heads, G, head_dim).sum(axis=1, dtype=dtype)
    return (sk * sq_group).reshape(-1)


# --------------------------------------------------------------------------
# a3: top-k per sequence
# --------------------------------------------------------------------------
def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """The k highest-scoring channels, ties to the lower index, ascending.

    SparseLoRA article §一: per input, the most important channels are kept
    and the rest skipped; readings R6.
    """
    scores = np.asarray(scores)
    n = scores.shape[0]
    if not (1 <= k <= n):
        raise ValueError("k must be in [1, N]")
    order = np.lexsort((np.arange(n), -scores.astype(F64)))
    return np.sort(order[:k]).astype(np.int32)


def expand_kv_to_q(idx_kv: np.ndarray, n_q_heads: int, n_kv_heads: int,
                   head_dim: int) -> np.ndarray:
    """Query channels (h, d) whose kv channel (h // G, d) is selected (R7, R8)."""
    G = n_q_heads // n_kv_heads
    sel = np.zeros(n_kv_heads * head_dim, dtype=bool)
    sel[np.asarray(idx_kv)] = True
    sel = sel.reshape(n_kv_heads, 1, head_dim).repeat(G, axis=1).reshape(-1)
    return np.nonzero(sel)[0].astype(np.int32)


def estimate_select_ffn(X, ctx_len, seq_len, Pg, Qg, Pu, Qu, k, dtype=np.float32):
    """Scores and index sets for every sequence of an FFN layer."""
    B = len(ctx_len)
    F = np.asarray(Qg).shape[1]
    sc = np.zeros((B, F), dtype=dtype)
    idx = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        rows = context_rows(ctx_len, seq_len, b)
        sc[b] = scores_swiglu_l2(np.asarray(X)[rows], Pg, Qg, Pu, Qu, dtype)
        idx[b] = select_topk(sc[b], k)
    return sc, idx


# --------------------------------------------------------------------------
# a4/a5: SwiGLU FFN with LoRA on gate, up and down, masked-dense form
# --------------------------------------------------------------------------
def ffn_masks(ctx_len, seq_len, idx, n_channels) -> np.ndarray:
    """m[t, j] = 1 if channel j is computed at token t.

    Context rows of sequence b keep only the selected channels; output rows
    keep all of them (SparseLoRA article §三; SparseLoRA abstract: loss and
    gradients on the selected subset).
    """
    B = len(ctx_len)
    m = np.ones((B * seq_len, n_channels), dtype=F64)
    for b in range(B):
        rows = context_rows(ctx_len, seq_len, b)
        if rows.size:
            m[rows, :] = 0.0
            m[np.ix_(rows, np.asarray(idx[b], dtype=np.int64))] = 1.0
    return m


def ffn_forward(p: Dict[str, np.ndarray], ctx_len, seq_len, idx, s: float = 1.0):
    """Forward of the LoRA-adapted SwiGLU FFN on the selected channels.

    p holds X [T, D], Wg, Wu [F, D], Wd [D, F], Ag, Au [r, D], Bg, Bu [F, r],
    Ad [r, F], Bd [D, r].  Returns y and the intermediates the backward needs.
    LoRA form: SALR page §2.1 notation with scale s (reading R3).
    """
    X = np.asarray(p["X"], F64)
    Wg, Wu, Wd = (np.asarray(p[n], F64) for n in ("Wg", "Wu", "Wd"))
    Ag, Bg, Au, Bu, Ad, Bd = (np.asarray(p[n], F64) for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"))
    m = ffn_masks(ctx_len, seq_len, idx, Wg.shape[0])
    zg = X @ Ag.T
    g = X @ Wg.T + s * (zg @ Bg.T)
    zu = X @ Au.T
    u = X @ Wu.T + s * (zu @ Bu.T)
    h = m * silu(g) * u
    zd = h @ Ad.T
    y = h @ Wd.T + s * (zd @ Bd.T)
    return y, {"m": m, "zg": zg, "zu": zu, "g": g, "u": u, "h": h, "zd": zd}


def ffn_backward(p: Dict[str, np.ndarray], cache, dY, s: float = 1.0):
    """Hand-derived chain rule of ffn_forward; frozen W get no gradient.

    Returns dX and the six LoRA factor gradients (SparseLoRA abstract:
    gradients only over the selected subset).
    """
    X = np.asarray(p["X"], F64)
    Wg, Wu, Wd = (np.asarray(p[n], F64) for n in ("Wg", "Wu", "Wd"))
    Ag, Bg, Au, Bu, Ad, Bd = (np.asarray(p[n], F64) for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"))
    dy = np.asarray(dY, F64)
    m, zg, zu, g, u, h, zd = (cache[n] for n in ("m", "zg", "zu", "g", "u", "h", "zd"))
    dzd = s * (dy @ Bd)
    dBd = s * (dy.T @ zd)
    dh = (dy @ Wd + dzd @ Ad) * m
    dAd = dzd.T @ h
    sg = sigmoid(g)
    dg = dh * u * sg * (1.0 + g * (1.0 - sg))
    du = dh * g * sg
    dBg = s * (dg.T @ zg)
    dzg = s * (dg @ Bg)
    dAg = dzg.T @ X
    dBu = s * (du.T @ zu)
    dzu = s * (du @ Bu)
    dAu = dzu.T @ X
    dx = dg @ Wg + du @ Wu + dzg @ Ag + dzu @ Au
    return {"dX": dx, "dAg": dAg, "dBg": dBg, "dAu": dAu, "dBu": dBu,
            "dAd": dAd, "dBd": dBd}


# --------------------------------------------------------------------------
# a6/a7: q/k/v/o projections with LoRA, masked-dense form
# --------------------------------------------------------------------------
def attn_masks(ctx_len, seq_len, idx_qk, idx_vo, n_q_heads, n_kv_heads, head_dim):
    """Masks of q, k, v outputs and of o's input columns (readings R7, R8)."""
    nq, nkv = n_q_heads * head_dim, n_kv_heads * head_dim
    iq = [expand_kv_to_q(i, n_q_heads, n_kv_heads, head_dim) for i in idx_qk]
    io = [expand_kv_to_q(i, n_q_heads, n_kv_heads, head_dim) for i in idx_vo]
    return (ffn_masks(ctx_len, seq_len, iq, nq), ffn_masks(ctx_len, seq_len, idx_qk, nkv),
            ffn_masks(ctx_len, seq_len, idx_vo, nkv), ffn_masks(ctx_len, seq_len, io, nq))


def qkvo_forward(p, ctx_len, seq_len, idx_qk, idx_vo, heads, s: float = 1.0):
    """q, k, v of the block input X and o of the attention output a.

    Unselected channels of context rows come out as exactly 0; output rows
    are dense.  heads = (n_q_heads, n_kv_heads, head_dim).
    """
    X, a = np.asarray(p["X"], F64), np.asarray(p["a"], F64)
    P = {n: np.asarray(p[n], F64) for n in ("Wq", "Wk", "Wv", "Wo", "Aq", "Bq", "Ak", "Bk",
                                            "Av", "Bv", "Ao", "Bo")}
    mq, mk, mv, mo = attn_masks(ctx_len, seq_len, idx_qk, idx_vo, *heads)
    zq, zk, zv = X @ P["Aq"].T, X @ P["Ak"].T, X @ P["Av"].T
    q = mq * (X @ P["Wq"].T + s * (zq @ P["Bq"].T))
    k = mk * (X @ P["Wk"].T + s * (zk @ P["Bk"].T))
    v = mv * (X @ P["Wv"].T + s * (zv @ P["Bv"].T))
    am = mo * a
    zo = am @ P["Ao"].T
    o = am @ P["Wo"].T + s * (zo @ P["Bo"].T)
    cache = {"mq": mq, "mk": mk, "mv": mv, "mo": mo, "zq": zq, "zk": zk, "zv": zv,
             "am": am, "zo": zo}
    return {"q": q, "k": k, "v": v, "o": o}, cache


def qkvo_backward(p, cache, grads, s: float = 1.0):
    """Chain rule of qkvo_forward given dq, dk, dv and d_out."""
    X = np.asarray(p["X"], F64)
    P = {n: np.asarray(p[n], F64) for n in ("Wq", "Wk", "Wv", "Wo", "Aq", "Bq", "Ak", "Bk",
                                            "Av", "Bv", "Ao", "Bo")}
    out = {}
    dX = np.zeros_like(X)
    for name, mname in (("q", "mq"), ("k", "mk"), ("v", "mv")):
        dpre = cache[mname] * np.asarray(grads["d" + name], F64)
        z = cache["z" + name]
        A, Bm, W = P["A" + name], P["B" + name], P["W" + name]
        dz = s * (dpre @ Bm)
        out["dB" + name] = s * (dpre.T @ z)
        out["dA" + name] = dz.T @ X
        dX += dpre @ W + dz @ A
    dout = np.asarray(grads["d_out"], F64)
    dzo = s * (dout @ P["Bo"])
    out["dBo"] = s * (dout.T @ cache["zo"])
    out["dAo"] = dzo.T @ cache["am"]
    out["da"] = cache["mo"] * (dout @ P["Wo"] + dzo @ P["Ao"])
    out["dX"] = dX
    return out
