"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here reaches the oracle through something other than its own
formulas: planted spectra, brute force over subsets, explicit outer
products, central finite differences, merged-weight identities and a
library SwiGLU (torch.nn.functional) for the LoRA-free special case.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _orth(rng, n, k):
    q, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return q


# ----------------------------------------------------------------- k rule
@pytest.mark.parametrize("n,p,k", [(14336, 90, 1434), (11008, 30, 7706), (11008, 75, 2752),
                                   (11008, 60, 4403), (11008, 90, 1101), (4096, 90, 410),
                                   (4096, 30, 2867), (4096, 60, 1638), (688, 50, 344),
                                   (1024, 50, 512), (11008, 0, 11008), (1, 99, 1)])
def test_k_from_ratio_half_up(n, p, k):
    # (100 - p) * n / 100 rounded half up, at least one channel
    assert O.k_from_ratio(n, p) == k
    exact = n * (100 - p) / 100.0
    assert abs(O.k_from_ratio(n, p) - exact) <= 0.5 or k == 1


# ----------------------------------------------------------- estimator
def _planted(rng, out_f, in_f, sig):
    U = _orth(rng, out_f, len(sig))
    V = _orth(rng, in_f, len(sig))
    return U @ np.diag(sig) @ V.T, U, V


def test_estimator_planted_spectrum_product():
    rng = _rng(1)
    sig = np.geomspace(10.0, 0.01, 24)
    W, U, V = _planted(rng, 40, 30, sig)   # rank 24 < min(40, 30)
    for r in (1, 4, 8, 16):
        P, Q, s = O.build_estimator(W, r)
        assert P.shape == (30, r) and Q.shape == (r, 40)
        np.testing.assert_allclose(s, sig[:r], rtol=1e-10)
        expect = V[:, :r] @ np.diag(sig[:r]) @ U[:, :r].T   # from the planted factors
        np.testing.assert_allclose(P @ Q, expect, atol=1e-10)


def test_estimator_eckart_young_residual():
    rng = _rng(2)
    sig = np.geomspace(5.0, 0.05, 20)
    W, _, _ = _planted(rng, 20, 36, sig)
    for r in (2, 8, 12):
        P, Q, _ = O.build_estimator(W, r)
        resid = np.linalg.norm(W - (P @ Q).T) ** 2
        assert resid == pytest.approx(float((sig[r:] ** 2).sum()), rel=1e-9)


def test_estimator_full_rank_reproduces_weight():
    rng = _rng(3)
    W = rng.standard_normal((12, 9))
    P, Q, _ = O.build_estimator(W, 9)
    np.testing.assert_allclose((P @ Q).T, W, atol=1e-12)


def test_estimator_memory_matches_page_figure():
    with open(os.path.join(GOLDEN, "estimator_memory.json")) as f:
        g = json.load(f)
    D, F = 4096, 11008
    proj = [(F, D), (F, D), (D, D), (D, D), (D, D)]       # gate, up, q, k, v
    mb = O.estimator_bytes(proj, g["rank"], 32) / 1e6
    assert mb == pytest.approx(28.05, abs=0.01)
    assert abs(mb - g["figure_mb"]) / g["figure_mb"] < g["tolerance_rel"]
    # down and o added would overshoot the page's figure by a third
    assert O.estimator_bytes(proj + [(D, F), (D, D)], 8, 32) / 1e6 > 1.3 * g["figure_mb"]


# ---------------------------------------------------------------- select
def _canonical_brute(scores, k):
    n = len(scores)
    best, best_sets = None, []
    for sub in itertools.combinations(range(n), k):
        tot = float(sum(scores[j] for j in sub))
        if best is None or tot > best + 1e-12:
            best, best_sets = tot, [sub]
        elif abs(tot - best) <= 1e-12:
            best_sets.append(sub)
    return best, sorted(best_sets)


@pytest.mark.parametrize("seed", range(6))
def test_select_is_max_mass_and_canonical_under_ties(seed):
    rng = _rng(100 + seed)
    # planted exact ties: only 5 distinct values over 12 channels
    vals = rng.choice([0.0, 0.25, 1.0, 2.5, 7.0], size=12)
    k = 5
    sel = O.select_topk(vals, k)
    best, sets = _canonical_brute(vals, k)
    assert tuple(sel) in sets
    assert tuple(sel) == sets[0]            # lowest indices among the maximisers
    assert list(sel) == sorted(sel)


def test_select_edge_cases():
    s = np.array([3.0, 1.0, 2.0])
    assert list(O.select_topk(s, 3)) == [0, 1, 2]       # k = N is the identity
    assert list(O.select_topk(np.zeros(6), 2)) == [0, 1]  # empty context: all-zero scores
    with pytest.raises(ValueError):
        O.select_topk(s, 0)
    with pytest.raises(ValueError):
        O.select_topk(s, 4)


# ---------------------------------------------------------------- scores
def _tiny_ffn(rng, D=10, F=12, r=2, T=8, lora=True):
    p = {"X": rng.standard_normal((T, D)),
         "Wg": rng.standard_normal((F, D)) * 0.5, "Wu": rng.standard_normal((F, D)) * 0.5,
         "Wd": rng.standard_normal((D, F)) * 0.5,
         "Ag": rng.standard_normal((r, D)) * 0.3, "Au": rng.standard_normal((r, D)) * 0.3,
         "Ad": rng.standard_normal((r, F)) * 0.3,
         "Bg": rng.standard_normal((F, r)) * 0.3, "Bu": rng.standard_normal((F, r)) * 0.3,
         "Bd": rng.standard_normal((D, r)) * 0.3}
    if not lora:
        for n in ("Bg", "Bu", "Bd"):
            p[n] = np.zeros_like(p[n])
    return p


def test_full_rank_estimator_scores_equal_exact_activation_scores():
    rng = _rng(7)
    p = _tiny_ffn(rng, lora=False)
    T, D = p["X"].shape
    F = p["Wg"].shape[0]
    Pg, Qg, _ = O.build_estimator(p["Wg"], D)
    Pu, Qu, _ = O.build_estimator(p["Wu"], D)
    ctx = [T]
    # exact activations from the (dense) forward itself
    _, cache = O.ffn_forward(p, ctx, T, [np.arange(F)])
    exact = (cache["h"] ** 2).sum(0)
    est = O.scores_swiglu_l2(p["X"], Pg, Qg, Pu, Qu, dtype=np.float64)
    np.testing.assert_allclose(est, exact, rtol=1e-9)


@pytest.mark.parametrize("seed", range(3))
def test_full_rank_selection_maximises_retained_mass(seed):
    """Top-k of the full-rank estimate keeps the most L2 mass of the exact h."""
    rng = _rng(20 + seed)
    p = _tiny_ffn(rng, lora=False)
    T, D = p["X"].shape
    F = p["Wg"].shape[0]
    k = 5
    Pg, Qg, _ = O.build_estimator(p["Wg"], D)
    Pu, Qu, _ = O.build_estimator(p["Wu"], D)
    sc = O.scores_swiglu_l2(p["X"], Pg, Qg, Pu, Qu, dtype=np.float64)
    sel = set(O.select_topk(sc, k).tolist())
    h_dense = O.ffn_forward(p, [T], T, [np.arange(F)])[1]["h"]
    best = max(((O.ffn_forward(p, [T], T, [np.array(sub)])[1]["h"]) ** 2).sum()
               for sub in itertools.combinations(range(F), k))
    kept = ((O.ffn_forward(p, [T], T, [np.array(sorted(sel))])[1]["h"]) ** 2).sum()
    assert kept == pytest.approx(best, rel=1e-12)
    assert kept <= (h_dense ** 2).sum() + 1e-12


def test_l2_full_rank_equals_exact():
    rng = _rng(8)
    X = rng.standard_normal((7, 6))
    W = rng.standard_normal((9, 6))
    P, Q, _ = O.build_estimator(W, 6)
    np.testing.assert_allclose(O.scores_l2(X, P, Q, dtype=np.float64),
                               ((X @ W.T) ** 2).sum(0), rtol=1e-10)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (6, 1)])
def test_qk_norm_is_frobenius_of_logit_contributions(hq, hkv):
    """Score of kv channel (g, d) = sum over the group's query heads of the
    squared Frobenius norm of channel d's rank-1 part of the logits."""
    rng = _rng(9)
    hd, D, T = 3, 5, 4
    X = rng.standard_normal((T, D))
    Wq = rng.standard_normal((hq * hd, D))
    Wk = rng.standard_normal((hkv * hd, D))
    Pq, Qq, _ = O.build_estimator(Wq, D)
    Pk, Qk, _ = O.build_estimator(Wk, D)
    sc = O.scores_qk_norm(X, Pq, Qq, Pk, Qk, hq, hkv, hd, dtype=np.float64)
    q, k = X @ Wq.T, X @ Wk.T
    G = hq // hkv
    for g in range(hkv):
        for d in range(hd):
            tot = 0.0
            for h in range(g * G, (g + 1) * G):
                logits = np.outer(q[:, h * hd + d], k[:, g * hd + d])   # [T, T]
                tot += (logits ** 2).sum()
            assert sc[g * hd + d] == pytest.approx(tot, rel=1e-10)
    if hq == hkv:  # multi-head form: (||q_c|| ||k_c||)^2
        np.testing.assert_allclose(sc, (np.linalg.norm(q, axis=0) * np.linalg.norm(k, axis=0)) ** 2,
                                   rtol=1e-10)


def test_expand_kv_to_q():
    idx = np.array([0, 4, 5])      # hkv=2, hd=3: channels (0,0), (1,1), (1,2)
    out = O.expand_kv_to_q(idx, 4, 2, 3)
    # q heads 0,1 -> group 0; heads 2,3 -> group 1
    assert list(out) == [0, 3, 7, 8, 10, 11]


# ------------------------------------------------------- forward / backward
def _fd_check(f_loss, params, names, grads, eps=1e-6, rtol=1e-6):
    for n in names:
        x = params[n]
        g_fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = f_loss()
            x[i] = old - eps
            lm = f_loss()
            x[i] = old
            g_fd[i] = (lp - lm) / (2 * eps)
        scale = max(np.abs(g_fd).max(), 1e-12)
        assert np.abs(grads[n] - g_fd).max() / scale < rtol, n


def _ffn_tiny_case(seed, ctx=(2, 1), L=3, D=8, F=12, r=2, k=5):
    rng = _rng(seed)
    B = len(ctx)
    p = _tiny_ffn(rng, D=D, F=F, r=r, T=B * L)
    idx = [np.sort(rng.choice(F, size=k, replace=False)).astype(np.int32) for _ in range(B)]
    dY = rng.standard_normal((B * L, D))
    return p, list(ctx), L, idx, dY


@pytest.mark.parametrize("s", [1.0, 0.5])
def test_ffn_backward_matches_finite_differences(s):
    p, ctx, L, idx, dY = _ffn_tiny_case(11)

    def loss():
        y, _ = O.ffn_forward(p, ctx, L, idx, s)
        return float((y * dY).sum())

    _, cache = O.ffn_forward(p, ctx, L, idx, s)
    g = O.ffn_backward(p, cache, dY, s)
    grads = {"X": g["dX"], "Ag": g["dAg"], "Bg": g["dBg"], "Au": g["dAu"], "Bu": g["dBu"],
             "Ad": g["dAd"], "Bd": g["dBd"]}
    _fd_check(loss, p, list(grads), grads)


def test_ffn_lora_equals_merged_weights():
    rng = _rng(12)
    p = _tiny_ffn(rng)
    T = p["X"].shape[0]
    F = p["Wg"].shape[0]
    s = 0.7
    y, _ = O.ffn_forward(p, [T], T, [np.arange(F)], s)
    m = dict(p)
    m["Wg"] = p["Wg"] + s * p["Bg"] @ p["Ag"]
    m["Wu"] = p["Wu"] + s * p["Bu"] @ p["Au"]
    m["Wd"] = p["Wd"] + s * p["Bd"] @ p["Ad"]
    for n in ("Bg", "Bu", "Bd"):
        m[n] = np.zeros_like(p[n])
    y2, _ = O.ffn_forward(m, [T], T, [np.arange(F)], s)
    np.testing.assert_allclose(y, y2, atol=1e-12)


def test_ffn_zero_b_is_library_swiglu():
    torch = pytest.importorskip("torch")
    rng = _rng(13)
    p = _tiny_ffn(rng, lora=False)
    T = p["X"].shape[0]
    F = p["Wg"].shape[0]
    y, _ = O.ffn_forward(p, [T], T, [np.arange(F)])
    t = {n: torch.from_numpy(v) for n, v in p.items()}
    ref = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(t["X"], t["Wg"]))
        * torch.nn.functional.linear(t["X"], t["Wu"]), t["Wd"])
    np.testing.assert_allclose(y, ref.numpy(), atol=1e-12)
    dY = rng.standard_normal(y.shape)
    _, cache = O.ffn_forward(p, [T], T, [np.arange(F)])
    g = O.ffn_backward(p, cache, dY)
    assert np.abs(g["dAg"]).max() == 0 and np.abs(g["dAu"]).max() == 0
    assert np.abs(g["dAd"]).max() == 0


def test_ffn_zero_sparsity_is_dense_bitwise():
    p, ctx, L, _, dY = _ffn_tiny_case(14)
    F = p["Wg"].shape[0]
    full = [np.arange(F, dtype=np.int32)] * len(ctx)
    y_s, c_s = O.ffn_forward(p, ctx, L, full)
    y_d, c_d = O.ffn_forward(p, [0] * len(ctx), L, full)   # all rows dense
    assert np.array_equal(y_s, y_d)
    gs, gd = O.ffn_backward(p, c_s, dY), O.ffn_backward(p, c_d, dY)
    for n in gs:
        assert np.array_equal(gs[n], gd[n]), n


def test_ffn_mask_equals_zeroed_rows_model():
    """All rows context, one sequence: the sparse layer is the dense layer with
    the dropped channels' gate/up rows (and LoRA-B rows), down columns and
    LoRA-A_d columns zeroed."""
    rng = _rng(15)
    p = _tiny_ffn(rng)
    T = p["X"].shape[0]
    F = p["Wg"].shape[0]
    idx = np.array([1, 4, 5, 9], dtype=np.int32)
    drop = np.setdiff1d(np.arange(F), idx)
    dY = rng.standard_normal((T, p["X"].shape[1]))
    y, c = O.ffn_forward(p, [T], T, [idx])
    g = O.ffn_backward(p, c, dY)
    z = {n: v.copy() for n, v in p.items()}
    z["Wg"][drop] = 0
    z["Bg"][drop] = 0
    z["Wu"][drop] = 0
    z["Bu"][drop] = 0
    z["Wd"][:, drop] = 0
    z["Ad"][:, drop] = 0
    yz, cz = O.ffn_forward(z, [T], T, [np.arange(F)])
    gz = O.ffn_backward(z, cz, dY)
    np.testing.assert_allclose(y, yz, atol=1e-12)
    for n in ("dX", "dAg", "dAu", "dAd", "dBd", "dBu"):
        np.testing.assert_allclose(g[n], gz[n], atol=1e-12, err_msg=n)
    np.testing.assert_allclose(g["dBg"][idx], gz["dBg"][idx], atol=1e-12)
    # invariant: rows outside the union of the sets get nothing without output rows
    assert np.abs(g["dBg"][drop]).max() == 0 and np.abs(g["dBu"][drop]).max() == 0
    assert np.abs(g["dAd"][:, drop]).max() == 0


def test_ffn_sequence_permutation():
    p, ctx, L, idx, dY = _ffn_tiny_case(16, ctx=(2, 1, 3), L=3)
    y, c = O.ffn_forward(p, ctx, L, idx)
    g = O.ffn_backward(p, c, dY)
    perm = [2, 0, 1]
    rows = np.concatenate([np.arange(b * L, (b + 1) * L) for b in perm])
    q = dict(p)
    q["X"] = p["X"][rows]
    y2, c2 = O.ffn_forward(q, [ctx[b] for b in perm], L, [idx[b] for b in perm])
    g2 = O.ffn_backward(q, c2, dY[rows])
    np.testing.assert_allclose(y2, y[rows], atol=1e-12)
    np.testing.assert_allclose(g2["dX"], g["dX"][rows], atol=1e-12)
    for n in ("dAg", "dBg", "dAu", "dBu", "dAd", "dBd"):
        np.testing.assert_allclose(g2[n], g[n], atol=1e-11)


# ----------------------------------------------------------------- q/k/v/o
def _tiny_attn(rng, D=6, hq=4, hkv=2, hd=2, r=2, T=6):
    nq, nkv = hq * hd, hkv * hd
    sd = 0.5
    return {"X": rng.standard_normal((T, D)), "a": rng.standard_normal((T, nq)),
            "Wq": rng.standard_normal((nq, D)) * sd, "Wk": rng.standard_normal((nkv, D)) * sd,
            "Wv": rng.standard_normal((nkv, D)) * sd, "Wo": rng.standard_normal((D, nq)) * sd,
            "Aq": rng.standard_normal((r, D)) * sd, "Bq": rng.standard_normal((nq, r)) * sd,
            "Ak": rng.standard_normal((r, D)) * sd, "Bk": rng.standard_normal((nkv, r)) * sd,
            "Av": rng.standard_normal((r, D)) * sd, "Bv": rng.standard_normal((nkv, r)) * sd,
            "Ao": rng.standard_normal((r, nq)) * sd, "Bo": rng.standard_normal((D, r)) * sd}


def test_qkvo_backward_matches_finite_differences():
    rng = _rng(30)
    heads = (4, 2, 2)
    L, ctx = 3, [2, 1]
    p = _tiny_attn(rng, T=len(ctx) * L)
    nkv = heads[1] * heads[2]
    idx_qk = [np.array([0, 3]), np.array([1, 2])]
    idx_vo = [np.array([2]), np.array([0, 1, 3])[:2]]
    grads_in = {n: rng.standard_normal(v.shape) for n, v in
                (("dq", np.zeros((6, 8))), ("dk", np.zeros((6, nkv))), ("dv", np.zeros((6, nkv))),
                 ("d_out", np.zeros((6, 6))))}

    def loss():
        out, _ = O.qkvo_forward(p, ctx, L, idx_qk, idx_vo, heads, 0.8)
        return float(sum((out[n] * grads_in["d" + n if n != "o" else "d_out"]).sum()
                         for n in ("q", "k", "v", "o")))

    _, cache = O.qkvo_forward(p, ctx, L, idx_qk, idx_vo, heads, 0.8)
    g = O.qkvo_backward(p, cache, grads_in, 0.8)
    grads = {"X": g["dX"], "a": g["da"]}
    for n in ("q", "k", "v", "o"):
        grads["A" + n] = g["dA" + n]
        grads["B" + n] = g["dB" + n]
    _fd_check(loss, p, list(grads), grads)


def test_qkvo_zero_b_is_library_linear_and_masks_zero_context():
    torch = pytest.importorskip("torch")
    rng = _rng(31)
    heads = (4, 2, 2)
    L, ctx = 3, [3, 1]
    p = _tiny_attn(rng, T=6)
    for n in ("Bq", "Bk", "Bv", "Bo"):
        p[n] = np.zeros_like(p[n])
    idx_qk = [np.array([1, 2]), np.array([0, 3])]
    idx_vo = [np.array([0]), np.array([2, 3])]
    out, _ = O.qkvo_forward(p, ctx, L, idx_qk, idx_vo, heads)
    t = {n: torch.from_numpy(v) for n, v in p.items()}
    q_ref = torch.nn.functional.linear(t["X"], t["Wq"]).numpy()
    # output rows (token 5 of seq 1, and none of seq 0) are dense
    np.testing.assert_allclose(out["q"][4:], q_ref[4:], atol=1e-12)
    # seq 0 (all context): kv channels {1,2} -> q channels of heads 0,1 dim 1 and heads 2,3 dim 0
    keep = O.expand_kv_to_q(idx_qk[0], *heads)
    assert list(keep) == [1, 3, 4, 6]
    np.testing.assert_allclose(out["q"][:3, keep], q_ref[:3, keep], atol=1e-12)
    drop = np.setdiff1d(np.arange(8), keep)
    assert np.abs(out["q"][:3, drop]).max() == 0


# ------------------------------------------- q/k/v/o: zeroed-weights model
# An independent statement of the masked q/k/v/o layer (SparseLoRA article
# §一: q/k channels by the QK-norm, the rest by the L2 norm; SparseLoRA
# abstract: loss and gradients on the selected subset).  For the context rows
# of sequence b the sparse layer is the dense layer whose weights are
# multiplied by 0/1 masks built here from the sets by explicit loops over
# heads: rows of Wk, Bk outside S_qk; rows of Wq, Bq whose kv channel
# (h // G, d) is outside S_qk; rows of Wv, Bv outside S_vo; columns of Wo, Ao
# whose kv channel is outside S_vo.  Output rows use the unmasked weights.
# Gradients come from torch autograd in float64 through the masked weights.
_QKVO_PARAMS = ("Wq", "Wk", "Wv", "Wo", "Aq", "Bq", "Ak", "Bk", "Av", "Bv", "Ao", "Bo")


def _qkvo_zeroed_model(p, ctx, L, idx_qk, idx_vo, heads, grads_in, s):
    torch = pytest.importorskip("torch")
    hq, hkv, hd = heads
    G = hq // hkv
    nq, nkv = hq * hd, hkv * hd
    t = {n: torch.tensor(p[n], dtype=torch.float64, requires_grad=True)
         for n in _QKVO_PARAMS + ("X", "a")}
    outs = {n: [] for n in ("q", "k", "v", "o")}
    loss = 0.0
    row_groups = []
    for b in range(len(ctx)):
        rows = list(range(b * L, b * L + ctx[b]))
        row_groups.append((rows, set(int(c) for c in idx_qk[b]), set(int(c) for c in idx_vo[b])))
    out_rows = [r for b in range(len(ctx)) for r in range(b * L + ctx[b], (b + 1) * L)]
    row_groups.append((out_rows, None, None))
    order = []
    for rows, sqk, svo in row_groups:
        if not rows:
            continue
        order += rows
        kq = torch.ones(nq, dtype=torch.float64)
        kk = torch.ones(nkv, dtype=torch.float64)
        kv = torch.ones(nkv, dtype=torch.float64)
        ko = torch.ones(nq, dtype=torch.float64)
        if sqk is not None:
            for c in range(nkv):
                kk[c] = 1.0 if c in sqk else 0.0
                kv[c] = 1.0 if c in svo else 0.0
            for h in range(hq):
                for d in range(hd):
                    kvch = (h // G) * hd + d
                    kq[h * hd + d] = 1.0 if kvch in sqk else 0.0
                    ko[h * hd + d] = 1.0 if kvch in svo else 0.0
        Xr, ar = t["X"][rows], t["a"][rows]
        q = Xr @ (t["Wq"] * kq[:, None]).T + s * (Xr @ t["Aq"].T) @ (t["Bq"] * kq[:, None]).T
        k = Xr @ (t["Wk"] * kk[:, None]).T + s * (Xr @ t["Ak"].T) @ (t["Bk"] * kk[:, None]).T
        v = Xr @ (t["Wv"] * kv[:, None]).T + s * (Xr @ t["Av"].T) @ (t["Bv"] * kv[:, None]).T
        o = ar @ (t["Wo"] * ko[None, :]).T + s * (ar @ (t["Ao"] * ko[None, :]).T) @ t["Bo"].T
        for n, val in (("q", q), ("k", k), ("v", v), ("o", o)):
            outs[n].append(val)
            gname = "d_out" if n == "o" else "d" + n
            loss = loss + (val * torch.tensor(grads_in[gname][rows], dtype=torch.float64)).sum()
    names = list(_QKVO_PARAMS) + ["X", "a"]
    gr = torch.autograd.grad(loss, [t[n] for n in names])
    inv = np.argsort(order)
    fwd = {n: torch.cat(v, 0).detach().numpy()[inv] for n, v in outs.items()}
    grad = {n: g.numpy() for n, g in zip(names, gr)}
    return fwd, grad


def _qkvo_pin_case():
    rng = _rng(40)
    heads = (4, 2, 3)                 # GQA: two query heads per kv head
    D, r, L = 5, 2, 4
    ctx = [4, 2]                      # one all-context sequence, one mixed
    p = _tiny_attn(rng, D=D, hq=4, hkv=2, hd=3, r=r, T=len(ctx) * L)
    nq, nkv = 12, 6
    # q/k and v/o sets differ in every sequence, and differ between sequences
    idx_qk = [np.array([0, 2, 4]), np.array([1, 3, 5])]
    idx_vo = [np.array([1, 4]), np.array([0, 5])]
    T = len(ctx) * L
    grads_in = {"dq": rng.standard_normal((T, nq)), "dk": rng.standard_normal((T, nkv)),
                "dv": rng.standard_normal((T, nkv)), "d_out": rng.standard_normal((T, D))}
    return p, ctx, L, idx_qk, idx_vo, heads, grads_in


def _qkvo_mismatch(p, ctx, L, idx_qk, idx_vo, heads, grads_in, s=0.7):
    """Largest relative difference over every output and gradient between the
    oracle and the zeroed-weights model."""
    out, cache = O.qkvo_forward(p, ctx, L, idx_qk, idx_vo, heads, s)
    g = O.qkvo_backward(p, cache, grads_in, s)
    fwd, grad = _qkvo_zeroed_model(p, ctx, L, idx_qk, idx_vo, heads, grads_in, s)
    pairs = [(out[n], fwd[n]) for n in ("q", "k", "v", "o")]
    pairs += [(g["dX"], grad["X"]), (g["da"], grad["a"])]
    for n in ("q", "k", "v", "o"):
        pairs += [(g["dA" + n], grad["A" + n]), (g["dB" + n], grad["B" + n])]
    worst = 0.0
    for got, ref in pairs:
        den = max(np.abs(ref).max(), 1e-300)
        worst = max(worst, float(np.abs(got - ref).max() / den))
    return worst


def test_qkvo_mask_equals_zeroed_weights_model():
    case = _qkvo_pin_case()
    assert _qkvo_mismatch(*case) < 1e-12
    # the frozen weights get no gradient: the model's gradients of W are not compared,
    # and the oracle's da is zero in dropped columns of context rows
    p, ctx, L, idx_qk, idx_vo, heads, gi = case
    out, cache = O.qkvo_forward(p, ctx, L, idx_qk, idx_vo, heads, 0.7)
    g = O.qkvo_backward(p, cache, gi, 0.7)
    # seq 0 keeps kv channels {1, 4} = (head 0, d 1), (head 1, d 1) for o: query heads 0, 1
    # read kv head 0 and heads 2, 3 kv head 1, so only query columns 1, 4, 7, 10 survive
    assert np.abs(g["da"][0:4][:, [0, 2, 3, 5, 6, 8, 9, 11]]).max() == 0
    assert np.abs(g["da"][0:4][:, [1, 4, 7, 10]]).min() > 0


def _mutated_masks(kind):
    real = O.attn_masks

    def masks(ctx_len, seq_len, idx_qk, idx_vo, hq, hkv, hd):
        mq, mk, mv, mo = real(ctx_len, seq_len, idx_qk, idx_vo, hq, hkv, hd)
        if kind == "v_by_qk":
            return mq, mk, mk, mo
        if kind == "o_by_qk":
            return mq, mk, mv, mq
        if kind == "k_by_vo":
            return mq, mv, mv, mo
        if kind == "q_head_modulo":
            # query head h mapped to kv head h % hkv instead of h // G
            G = hq // hkv
            perm = np.array([((h % hkv) * G + h // hkv) * hd + d for h in range(hq) for d in range(hd)])
            inv = np.argsort(perm)
            return mq[:, inv], mk, mv, mo
        raise ValueError(kind)
    return masks


@pytest.mark.parametrize("kind", ["v_by_qk", "o_by_qk", "k_by_vo", "q_head_modulo"])
def test_qkvo_zeroed_model_rejects_wrong_masks(monkeypatch, kind):
    """Plant a wrong set pairing in the oracle (on the CPU) and show the pin catches it."""
    import oracle.sparselora_oracle as core
    monkeypatch.setattr(core, "attn_masks", _mutated_masks(kind))
    assert _qkvo_mismatch(*_qkvo_pin_case()) > 1e-3
