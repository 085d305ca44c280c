"""GPU parity of the q/k/v/o projections (QK-norm and L2 selection, forward,
backward) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import assert_close, check_scores, check_selection, factors, to_dev, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _api():
    import contextual_sparsity_lora_svd_amd as sl
    return sl


def _case(D, heads, r, ctx, L, dt, seed):
    hq, hkv, hd = heads
    nq, nkv = hq * hd, hkv * hd
    rng = np.random.default_rng(seed)
    T = len(ctx) * L

    def rnd(shape, std):
        x = (rng.standard_normal(shape) * std).astype(np.float32)
        return W.round_to_bf16(x) if dt == "bf16" else x

    def act(n):
        z = rng.standard_normal((T, 8)).astype(np.float32)
        m = rng.standard_normal((8, n)).astype(np.float32)
        x = (z @ m + 0.1 * rng.standard_normal((T, n)).astype(np.float32)) * \
            rng.lognormal(0, 1, n).astype(np.float32)
        return W.round_to_bf16(x) if dt == "bf16" else x

    return {"X": act(D), "a": act(nq),
            "Wq": rnd((nq, D), 0.05), "Wk": rnd((nkv, D), 0.05), "Wv": rnd((nkv, D), 0.05),
            "Wo": rnd((D, nq), 0.05),
            "Aq": rnd((r, D), 0.05), "Bq": rnd((nq, r), 0.05), "Ak": rnd((r, D), 0.05),
            "Bk": rnd((nkv, r), 0.05), "Av": rnd((r, D), 0.05), "Bv": rnd((nkv, r), 0.05),
            "Ao": rnd((r, nq), 0.05), "Bo": rnd((D, r), 0.05),
            "dq": rnd((T, nq), 1.0), "dk": rnd((T, nkv), 1.0), "dv": rnd((T, nkv), 1.0),
            "d_out": rnd((T, D), 1.0)}


def _weights(p, heads, dt, s):
    sl = _api()
    t = {n: to_dev(p[n], dt) for n in ("Wq", "Wk", "Wv", "Aq", "Bq", "Ak", "Bk", "Av", "Bv", "Ao", "Bo")}
    t["WoT"] = to_dev(np.ascontiguousarray(p["Wo"].T), dt)
    return sl.QKVOWeights(t, heads, lora_scale=s)


def _compare(p, heads, ctx, L, idx_qk, idx_vo, dt, s=1.0, split_calls=False):
    sl = _api()
    w = _weights(p, heads, dt, s)
    lay = sl.Layout(ctx, L)
    X, a = to_dev(p["X"], dt), to_dev(p["a"], dt)
    kqk, kvo = idx_qk.shape[1], idx_vo.shape[1]
    iqk = torch.from_numpy(np.ascontiguousarray(idx_qk, np.int32)).cuda()
    ivo = torch.from_numpy(np.ascontiguousarray(idx_vo, np.int32)).cuda()
    if split_calls:
        outs, buf = sl.qkvo_fwd(w, X, None, lay, kqk, iqk, kvo, ivo)
        outs, buf = sl.qkvo_fwd(w, None, a, lay, kqk, iqk, kvo, ivo, buf=buf, outs=outs)
        g = sl.qkvo_bwd(w, X, a, lay, kqk, iqk, kvo, ivo, buf, d_out=to_dev(p["d_out"], dt))
        g = sl.qkvo_bwd(w, X, a, lay, kqk, iqk, kvo, ivo, buf, dq=to_dev(p["dq"], dt),
                        dk=to_dev(p["dk"], dt), dv=to_dev(p["dv"], dt), out=g)
    else:
        outs, buf = sl.qkvo_fwd(w, X, a, lay, kqk, iqk, kvo, ivo)
        g = sl.qkvo_bwd(w, X, a, lay, kqk, iqk, kvo, ivo, buf, dq=to_dev(p["dq"], dt),
                        dk=to_dev(p["dk"], dt), dv=to_dev(p["dv"], dt), d_out=to_dev(p["d_out"], dt))
    torch.cuda.synchronize()
    ref, cache = O.qkvo_forward(p, ctx, L, list(idx_qk), list(idx_vo), heads, s)
    gr = O.qkvo_backward(p, cache, {n: p[n] for n in ("dq", "dk", "dv", "d_out")}, s)
    errs = {}
    for n in ("q", "k", "v", "o"):
        errs[n] = assert_close(to_np(outs[n]), ref[n], dt, n)
    # unselected context channels are exactly zero
    mq = cache["mq"]
    assert np.all(to_np(outs["q"])[mq == 0] == 0)
    for n in ("dX", "da", "dAq", "dBq", "dAk", "dBk", "dAv", "dBv", "dAo", "dBo"):
        errs[n] = assert_close(to_np(g[n]), gr[n], dt, n)
    assert np.all(to_np(g["da"])[cache["mo"] == 0] == 0)
    print(f"\n[{dt}] heads={heads} ctx={list(ctx)} kqk={kqk} kvo={kvo} " +
          " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)


def _sets(rng, B, n, k):
    return np.stack([np.sort(rng.choice(n, k, replace=False)) for _ in range(B)]).astype(np.int32)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("heads", [(4, 4, 16), (8, 2, 16)])
def test_qkvo_ragged(dt, heads):
    D, r, L = 64, 4, 40
    ctx = [40, 0, 23]
    p = _case(D, heads, r, ctx, L, dt, seed=21)
    rng = np.random.default_rng(22)
    nkv = heads[1] * heads[2]
    _compare(p, heads, ctx, L, _sets(rng, 3, nkv, 13), _sets(rng, 3, nkv, 21), dt, s=0.7)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_qkvo_split_calls_and_extremes(dt):
    heads = (8, 4, 32)
    D, r, L = 128, 8, 100
    ctx = [80, 100]
    p = _case(D, heads, r, ctx, L, dt, seed=23)
    rng = np.random.default_rng(24)
    nkv = heads[1] * heads[2]
    _compare(p, heads, ctx, L, _sets(rng, 2, nkv, 40), _sets(rng, 2, nkv, 64), dt, split_calls=True)
    full = np.tile(np.arange(nkv, dtype=np.int32), (2, 1))
    _compare(p, heads, ctx, L, full, np.array([[0], [nkv - 1]], np.int32), dt)


@pytest.mark.parametrize("variants", [1, 0, 6])
def test_qkvo_multi_tile_bf16(variants):
    """Several tiles per group on each GEMM variant: 1 the wide N-gather tiles,
    0 the 128 x 256 tiles only, 6 the tall 256 x 256 tiles whatever their grid
    (every product: the q/k/v and attention-output-gradient N-gathers, the o
    and input-gradient K-gathers)."""
    from tests.gpu_helpers import gemm_variant
    with gemm_variant(variants):
        _qkvo_multi_tile()


def _qkvo_multi_tile():
    heads = (16, 4, 64)
    D, r, L = 512, 16, 300
    ctx = [260, 300, 150]
    p = _case(D, heads, r, ctx, L, "bf16", seed=25)
    rng = np.random.default_rng(26)
    nkv = heads[1] * heads[2]
    _compare(p, heads, ctx, L, _sets(rng, 3, nkv, 130), _sets(rng, 3, nkv, 190), "bf16")


def _qk_l2_oracle(p, ctx, L, heads, Pq, Qq, Pk, Qk, Pv, Qv):
    B = len(ctx)
    qk, vo = [], []
    for b in range(B):
        rows = O.context_rows(ctx, L, b)
        qk.append(O.scores_qk_norm(p["X"][rows], Pq.T, Qq, Pk.T, Qk, *heads, dtype=np.float32))
        vo.append(O.scores_l2(p["X"][rows], Pv.T, Qv, dtype=np.float32))
    return np.stack(qk), np.stack(vo)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("heads", [(4, 4, 16), (8, 2, 16)])
def test_qk_norm_and_l2_select(dt, heads):
    sl = _api()
    D, r, L = 64, 4, 90
    ctx = [90, 17, 64]
    p = _case(D, heads, r, ctx, L, dt, seed=27)
    Pq, Qq = factors(p["Wq"], 8, dt)
    Pk, Qk = factors(p["Wk"], 8, dt)
    Pv, Qv = factors(p["Wv"], 8, dt)
    nkv = heads[1] * heads[2]
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], dt)
    ref_qk, ref_vo = _qk_l2_oracle(p, ctx, L, heads, Pq, Qq, Pk, Qk, Pv, Qv)
    k = nkv // 2
    idx, sc = sl.estimate_select(sl.SL_CRIT_QK_NORM, X, lay, 8, to_dev(Pq, dt), to_dev(Qq, dt),
                                 to_dev(Pk, dt), to_dev(Qk, dt), nkv, k, heads=heads, want_scores=True)
    idx2, sc2 = sl.estimate_select(sl.SL_CRIT_L2, X, lay, 8, to_dev(Pv, dt), to_dev(Qv, dt), None, None,
                                   nkv, k, want_scores=True)
    torch.cuda.synchronize()
    for got, ref in ((sc.cpu().numpy(), ref_qk), (sc2.cpu().numpy(), ref_vo)):
        for b in range(len(ctx)):
            e = np.abs(got[b] - ref[b]).max() / max(ref[b].max(), 1e-30)
            assert e < 2e-4, f"score rel err {e:.2e}"
    check_selection(idx.cpu().numpy(), ref_qk, k)
    check_selection(idx2.cpu().numpy(), ref_vo, k)


@pytest.mark.parametrize("rank", [12, 32])
def test_qk_norm_and_l2_select_high_rank(rank):
    """Estimator ranks past 8: the criterion's Gram matrix as one 16 x 16 tile
    (rank 12) and as 2 x 2 tiles (rank 32), context lengths off the 4-token
    step, and an all-output sequence."""
    sl = _api()
    heads = (4, 2, 16)
    D, r, L = 64, 4, 151
    ctx = [151, 45, 0]
    p = _case(D, heads, r, ctx, L, "f32", seed=28)
    Pq, Qq = factors(p["Wq"], rank, "f32")
    Pk, Qk = factors(p["Wk"], rank, "f32")
    Pv, Qv = factors(p["Wv"], rank, "f32")
    nkv = heads[1] * heads[2]
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], "f32")
    ref_qk, ref_vo = _qk_l2_oracle(p, ctx, L, heads, Pq, Qq, Pk, Qk, Pv, Qv)
    k = nkv // 2
    idx, sc = sl.estimate_select(sl.SL_CRIT_QK_NORM, X, lay, rank, to_dev(Pq, "f32"), to_dev(Qq, "f32"),
                                 to_dev(Pk, "f32"), to_dev(Qk, "f32"), nkv, k, heads=heads, want_scores=True)
    idx2, sc2 = sl.estimate_select(sl.SL_CRIT_L2, X, lay, rank, to_dev(Pv, "f32"), to_dev(Qv, "f32"), None, None,
                                   nkv, k, want_scores=True)
    torch.cuda.synchronize()
    for got, ref in ((sc.cpu().numpy(), ref_qk), (sc2.cpu().numpy(), ref_vo)):
        for b in range(len(ctx)):
            e = np.abs(got[b] - ref[b]).max() / max(ref[b].max(), 1e-30)
            assert e < 2e-4, f"rank {rank} seq {b} score rel err {e:.2e}"
        assert np.all(got[2] == 0.0)
    check_selection(idx.cpu().numpy(), ref_qk, k)
    check_selection(idx2.cpu().numpy(), ref_vo, k)


@pytest.mark.parametrize("heads", [(4, 4, 16), (8, 2, 16)])
def test_estimate_select_multi(heads):
    """QK-norm on q/k and L2 on v in one call: the oracle's scores and sets, and
    bit-for-bit the results of the two single-criterion calls."""
    sl = _api()
    D, r, L = 64, 4, 90
    ctx = [90, 17, 64]
    p = _case(D, heads, r, ctx, L, "bf16", seed=31)
    Pq, Qq = factors(p["Wq"], 8, "bf16")
    Pk, Qk = factors(p["Wk"], 8, "bf16")
    Pv, Qv = factors(p["Wv"], 8, "bf16")
    nkv = heads[1] * heads[2]
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], "bf16")
    ref_qk, ref_vo = _qk_l2_oracle(p, ctx, L, heads, Pq, Qq, Pk, Qk, Pv, Qv)
    kqk, kvo = nkv // 2, nkv // 3
    d = {n: to_dev(v, "bf16") for n, v in (("Pq", Pq), ("Qq", Qq), ("Pk", Pk), ("Qk", Qk), ("Pv", Pv), ("Qv", Qv))}
    jobs = [dict(crit=sl.SL_CRIT_QK_NORM, Pt0=d["Pq"], Q0=d["Qq"], Pt1=d["Pk"], Q1=d["Qk"], N=nkv, k=kqk,
                 heads=heads, want_scores=True),
            dict(crit=sl.SL_CRIT_L2, Pt0=d["Pv"], Q0=d["Qv"], N=nkv, k=kvo, want_scores=True)]
    (iqk, sqk), (ivo, svo) = sl.estimate_select_multi(X, lay, 8, jobs)
    i1, s1 = sl.estimate_select(sl.SL_CRIT_QK_NORM, X, lay, 8, d["Pq"], d["Qq"], d["Pk"], d["Qk"], nkv, kqk,
                                heads=heads, want_scores=True)
    i2, s2 = sl.estimate_select(sl.SL_CRIT_L2, X, lay, 8, d["Pv"], d["Qv"], None, None, nkv, kvo,
                                want_scores=True)
    torch.cuda.synchronize()
    for got, ref in ((sqk.cpu().numpy(), ref_qk), (svo.cpu().numpy(), ref_vo)):
        for b in range(len(ctx)):
            e = np.abs(got[b] - ref[b]).max() / max(ref[b].max(), 1e-30)
            assert e < 2e-4, f"score rel err {e:.2e}"
    check_selection(iqk.cpu().numpy(), ref_qk, kqk)
    check_selection(ivo.cpu().numpy(), ref_vo, kvo)
    assert torch.equal(iqk, i1) and torch.equal(ivo, i2)
    assert torch.equal(sqk, s1) and torch.equal(svo, s2)


def test_estimate_select_multi_swiglu_offset():
    """A SwiGLU job after an L2 job (its projections in later estimate columns)
    and a third L2 job: every job matches its single call and the oracle."""
    sl = _api()
    from tests.test_gpu_ffn import _ffn_case, _oracle_scores
    D, F, L = 128, 200, 70
    ctx = [70, 25]
    p = _ffn_case(D, F, 4, ctx, L, "f32", seed=33)
    Pg, Qg = factors(p["Wg"], 8, "f32")
    Pu, Qu = factors(p["Wu"], 8, "f32")
    Pd, Qd = factors(np.ascontiguousarray(p["Wd"].T), 8, "f32")     # an L2 job: d_model -> d_ff factors
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], "f32")
    dv = {n: to_dev(v, "f32") for n, v in (("Pg", Pg), ("Qg", Qg), ("Pu", Pu), ("Qu", Qu), ("Pd", Pd), ("Qd", Qd))}
    k1, k2 = 60, 90
    jobs = [dict(crit=sl.SL_CRIT_L2, Pt0=dv["Pd"], Q0=dv["Qd"], N=F, k=k1, want_scores=True),
            dict(crit=sl.SL_CRIT_SWIGLU_L2, Pt0=dv["Pg"], Q0=dv["Qg"], Pt1=dv["Pu"], Q1=dv["Qu"], N=F, k=k2,
                 want_scores=True)]
    (ia, sa), (ib, sb) = sl.estimate_select_multi(X, lay, 8, jobs)
    ja, ta = sl.estimate_select(sl.SL_CRIT_L2, X, lay, 8, dv["Pd"], dv["Qd"], None, None, F, k1, want_scores=True)
    jb, tb = sl.estimate_select(sl.SL_CRIT_SWIGLU_L2, X, lay, 8, dv["Pg"], dv["Qg"], dv["Pu"], dv["Qu"], F, k2,
                                want_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(ia, ja) and torch.equal(sa, ta)
    assert torch.equal(ib, jb) and torch.equal(sb, tb)
    ref = _oracle_scores(p, ctx, L, Pg, Qg, Pu, Qu)
    for b in range(len(ctx)):
        e = np.abs(sb.cpu().numpy()[b] - ref[b]).max() / max(ref[b].max(), 1e-30)
        assert e < 1e-4, f"SwiGLU score rel err {e:.2e}"
    check_selection(ib.cpu().numpy(), ref, k2)
    ref_l2 = np.stack([O.scores_l2(p["X"][O.context_rows(ctx, L, b)], Pd.T, Qd, dtype=np.float32)
                       for b in range(len(ctx))])
    for b in range(len(ctx)):
        e = np.abs(sa.cpu().numpy()[b] - ref_l2[b]).max() / max(ref_l2[b].max(), 1e-30)
        assert e < 1e-4, f"L2 score rel err {e:.2e}"
    check_selection(ia.cpu().numpy(), ref_l2, k1)


@pytest.mark.parametrize("cfg", [3, 5])
def test_full_size_workloads(cfg):
    """LLaMA2-7B q/k/v/o (multi-head) and LLaMA3-8B (grouped-query) at their sizes."""
    sl = _api()
    wl = W.WORKLOADS[cfg]
    s = wl.attn[0]
    heads = (s.n_q_heads, s.n_kv_heads, s.head_dim)
    p = W.make_attn_tensors(wl)
    ctx = [int(c) for c in W.ctx_lengths(wl)]
    L = wl.seq_len
    nkv = heads[1] * heads[2]
    kqk = O.k_from_ratio(nkv, s.sparsity_qk_pct)
    kvo = O.k_from_ratio(nkv, s.sparsity_vo_pct)
    Pq, Qq = factors(p["Wq"], wl.est_rank, "bf16")
    Pk, Qk = factors(p["Wk"], wl.est_rank, "bf16")
    Pv, Qv = factors(p["Wv"], wl.est_rank, "bf16")
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], "bf16")
    idx, sc = sl.estimate_select(sl.SL_CRIT_QK_NORM, X, lay, wl.est_rank, to_dev(Pq, "bf16"),
                                 to_dev(Qq, "bf16"), to_dev(Pk, "bf16"), to_dev(Qk, "bf16"), nkv, kqk,
                                 heads=heads, want_scores=True)
    idx_vo, sc_vo = sl.estimate_select(sl.SL_CRIT_L2, X, lay, wl.est_rank, to_dev(Pv, "bf16"),
                                       to_dev(Qv, "bf16"), None, None, nkv, kvo, want_scores=True)
    torch.cuda.synchronize()
    ref_qk, ref_vo = _qk_l2_oracle(p, ctx, L, heads, Pq, Qq, Pk, Qk, Pv, Qv)
    check_scores(sc.cpu().numpy(), ref_qk, 2e-4, "QK-norm scores")
    check_scores(sc_vo.cpu().numpy(), ref_vo, 1e-4, "L2 scores")
    n_exact = check_selection(idx.cpu().numpy(), ref_qk, kqk)
    n_vo = check_selection(idx_vo.cpu().numpy(), ref_vo, kvo)
    iqk = np.stack([O.select_topk(ref_qk[b], kqk) for b in range(len(ctx))])
    ivo = np.stack([O.select_topk(ref_vo[b], kvo) for b in range(len(ctx))])
    _compare(p, heads, ctx, L, iqk, ivo, "bf16", s=1.0)
    print(f"exact qk sets {n_exact}/{len(ctx)}, vo sets {n_vo}/{len(ctx)}", flush=True)


def test_side_stream_ordering_and_graph_capture():
    """The q/k/v/o calls overlap work on a side stream (operand packing, row
    layout, gradient reductions).  On a stream of the caller's, copies enqueued
    right after the calls see the final values; captured into a graph (where
    the calls keep to one stream), three replays with eager work between them
    match.  Everything bit for bit against eager calls on the default stream."""
    sl = _api()
    heads = (8, 2, 16)
    D, r, L = 128, 8, 120
    ctx = [100, 120, 40]
    p = _case(D, heads, r, ctx, L, "bf16", seed=45)
    nkv = heads[1] * heads[2]
    rng = np.random.default_rng(46)
    iqk = torch.from_numpy(np.stack([np.sort(rng.choice(nkv, 11, replace=False)) for _ in ctx]).astype(np.int32)).cuda()
    ivo = torch.from_numpy(np.stack([np.sort(rng.choice(nkv, 19, replace=False)) for _ in ctx]).astype(np.int32)).cuda()
    w = _weights(p, heads, "bf16", 0.5)
    lay = sl.Layout(ctx, L)
    X, a = to_dev(p["X"], "bf16"), to_dev(p["a"], "bf16")
    d = {n: to_dev(p[n], "bf16") for n in ("dq", "dk", "dv", "d_out")}

    outs, buf = sl.qkvo_fwd(w, X, a, lay, 11, iqk, 19, ivo)
    grads = sl.qkvo_bwd(w, X, a, lay, 11, iqk, 19, ivo, buf, **d)
    torch.cuda.synchronize()
    ref = {**{n: v.clone() for n, v in outs.items()}, **{n: v.clone() for n, v in grads.items()}}

    def step():
        sl.qkvo_fwd(w, X, a, lay, 11, iqk, 19, ivo, buf=buf, outs=outs)
        sl.qkvo_bwd(w, X, a, lay, 11, iqk, 19, ivo, buf, out=grads, **d)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    copies = []
    with torch.cuda.stream(s):
        for _ in range(2):
            step()
            copies.append({**{n: v.clone() for n, v in outs.items()}, **{n: v.clone() for n, v in grads.items()}})
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for c in copies:
        for n, v in ref.items():
            assert torch.equal(c[n], v), f"{n} differs on the caller's stream"

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for v in list(outs.values()) + list(grads.values()):
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, v in ref.items():
            got = outs[n] if n in outs else grads[n]
            assert torch.equal(got, v), f"replay {rep}: {n}"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_reads_only_saved(dt):
    """Everything the backward takes from the forward is in `saved` (z_q, z_k,
    z_v, z_o and the packed Bo^T, Ao^T): a backward given a copy of the saved
    buffer and a fresh workspace filled with 0xFF bytes (NaN in bf16 and fp32)
    matches, bit for bit, the backward that shares the forward's workspace."""
    sl = _api()
    heads = (8, 2, 16)
    D, r, L = 128, 8, 120
    ctx = [100, 120, 40]
    p = _case(D, heads, r, ctx, L, dt, seed=47)
    nkv = heads[1] * heads[2]
    rng = np.random.default_rng(48)
    iqk = torch.from_numpy(np.stack([np.sort(rng.choice(nkv, 11, replace=False)) for _ in ctx]).astype(np.int32)).cuda()
    ivo = torch.from_numpy(np.stack([np.sort(rng.choice(nkv, 19, replace=False)) for _ in ctx]).astype(np.int32)).cuda()
    w = _weights(p, heads, dt, 0.5)
    lay = sl.Layout(ctx, L)
    X, a = to_dev(p["X"], dt), to_dev(p["a"], dt)
    d = {n: to_dev(p[n], dt) for n in ("dq", "dk", "dv", "d_out")}
    outs, buf = sl.qkvo_fwd(w, X, a, lay, 11, iqk, 19, ivo)
    g1 = sl.qkvo_bwd(w, X, a, lay, 11, iqk, 19, ivo, buf, **d)
    buf2 = sl.QKVOWorkspace(w, lay, 11, 19, X.device)
    buf2.saved.copy_(buf.saved)
    buf2.ws.fill_(255)
    g2 = sl.qkvo_bwd(w, X, a, lay, 11, iqk, 19, ivo, buf2, **d)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), f"{n} differs with a fresh workspace"


@pytest.mark.parametrize("N", [32768, 65536])
def test_l2_select_at_channel_limits(N):
    """L2 criterion and top-k over 32768 channels (32 keys per thread held in
    registers) and 65536 (keys re-read from the workspace in every radix
    pass), two sequences, one of them short."""
    sl = _api()
    rng = np.random.default_rng(41)
    D, L, rank = 64, 48, 8
    ctx = [48, 21]
    X = W.round_to_bf16((rng.standard_normal((2 * L, D)) * rng.lognormal(0, 1, D)).astype(np.float32))
    Pt = W.round_to_bf16(rng.standard_normal((rank, D)).astype(np.float32) * 0.1)
    Q = W.round_to_bf16(rng.standard_normal((rank, N)).astype(np.float32) * 0.1)
    k = N // 4 + 3
    lay = sl.Layout(ctx, L)
    idx, sc = sl.estimate_select(sl.SL_CRIT_L2, to_dev(X, "bf16"), lay, rank, to_dev(Pt, "bf16"),
                                 to_dev(Q, "bf16"), None, None, N, k, want_scores=True)
    torch.cuda.synchronize()
    ref = np.stack([O.scores_l2(X[O.context_rows(ctx, L, b)], Pt.T, Q, dtype=np.float32)
                    for b in range(len(ctx))])
    check_scores(sc.cpu().numpy(), ref, 1e-4, "L2 scores")
    n_exact = check_selection(idx.cpu().numpy(), ref, k)
    print(f"\nN={N} k={k} exact sets {n_exact}/2", flush=True)
