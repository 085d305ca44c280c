"""GPU parity of the FFN hot path (estimate, select, forward, backward) against
the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import (assert_close, check_scores, check_selection, factors, gemm_variant, rel_err, to_dev,
                               to_np)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _api():
    import contextual_sparsity_lora_svd_amd as sl
    return sl


def _ffn_case(D, F, r, ctx, L, dt, seed, R_in=8):
    rng = np.random.default_rng(seed)
    T = len(ctx) * L

    def rnd(shape, std):
        x = (rng.standard_normal(shape) * std).astype(np.float32)
        return W.round_to_bf16(x) if dt == "bf16" else x

    z = rng.standard_normal((T, R_in)).astype(np.float32)
    m = rng.standard_normal((R_in, D)).astype(np.float32)
    sc = rng.lognormal(0, 1, D).astype(np.float32)
    X = (z @ m + 0.1 * rng.standard_normal((T, D)).astype(np.float32)) * sc
    X = W.round_to_bf16(X) if dt == "bf16" else X
    p = {"X": X, "Wg": rnd((F, D), 0.05), "Wu": rnd((F, D), 0.05), "Wd": rnd((D, F), 0.05),
         "Ag": rnd((r, D), 0.05), "Bg": rnd((F, r), 0.05), "Au": rnd((r, D), 0.05),
         "Bu": rnd((F, r), 0.05), "Ad": rnd((r, F), 0.05), "Bd": rnd((D, r), 0.05),
         "dY": rnd((T, D), 1.0)}
    return p


def _dev_weights(p, dt, s):
    sl = _api()
    t = {n: to_dev(p[n], dt) for n in ("Wg", "Wu", "Ag", "Bg", "Au", "Bu", "Ad", "Bd")}
    t["WdT"] = to_dev(np.ascontiguousarray(p["Wd"].T), dt)
    return sl.FFNWeights(t, lora_scale=s)


def _run_fwd_bwd(p, ctx, L, idx, dt, s=1.0):
    sl = _api()
    w = _dev_weights(p, dt, s)
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], dt)
    k = idx.shape[1]
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    Y, buf = sl.ffn_fwd(w, X, lay, k, idx_d)
    g = sl.ffn_bwd(w, X, lay, k, idx_d, buf, to_dev(p["dY"], dt))
    torch.cuda.synchronize()
    return to_np(Y), {n: to_np(v) for n, v in g.items()}


def _compare(p, ctx, L, idx, dt, s=1.0):
    y, g = _run_fwd_bwd(p, ctx, L, idx, dt, s)
    yr, cache = O.ffn_forward(p, ctx, L, list(idx), s)
    gr = O.ffn_backward(p, cache, p["dY"], s)
    errs = {"Y": assert_close(y, yr, dt, "Y")}
    for n in ("dX", "dAg", "dBg", "dAu", "dBu", "dAd", "dBd"):
        errs[n] = assert_close(g[n], gr[n], dt, n)
    print(f"\n[{dt}] ctx={list(ctx)} k={idx.shape[1]} errs " +
          " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    return errs


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ffn_ragged_groups_and_tails(dt):
    """Three sequences (all context / all output / mixed), k and r off the
    tile and chunk sizes, d_ff not a multiple of the tile."""
    _ragged_case(dt)


def _ragged_case(dt):
    D, F, r, L = 64, 136, 4, 50
    ctx = [50, 0, 37]
    p = _ffn_case(D, F, r, ctx, L, dt, seed=5)
    rng = np.random.default_rng(6)
    k = 37
    idx = np.stack([np.sort(rng.choice(F, k, replace=False)) for _ in ctx]).astype(np.int32)
    _compare(p, ctx, L, idx, dt, s=0.5)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ffn_dense_and_single_channel(dt):
    D, F, r, L = 128, 264, 8, 80
    ctx = [60, 80]
    p = _ffn_case(D, F, r, ctx, L, dt, seed=7)
    _compare(p, ctx, L, np.tile(np.arange(F, dtype=np.int32), (2, 1)), dt)      # k = N
    _compare(p, ctx, L, np.array([[5], [263]], dtype=np.int32), dt)           # k = 1


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ffn_multi_tile(dt):
    """Several M, N and K tiles and the output-group K split."""
    _multi_case(dt)


@pytest.mark.parametrize("case", ["ragged", "multi", "dense_single"])
def test_ffn_bf16_tall_kgather_tiles(case):
    """The same cases with every bf16 product on the tall 256 x 256 LDS-DMA
    tiles wherever its operands allow them, whatever their grid: the down and
    dX K-gathers, and the gate/up and dH N-gathers when aligned (ragged
    groups, a K segment whose channel count is not a multiple of 8, partial
    row tiles, k = N, k = 1)."""
    with gemm_variant(1 | 2 | 4):
        if case == "dense_single":
            D, F, r, L = 128, 264, 8, 80
            ctx = [60, 80]
            p = _ffn_case(D, F, r, ctx, L, "bf16", seed=7)
            _compare(p, ctx, L, np.tile(np.arange(F, dtype=np.int32), (2, 1)), "bf16")
            _compare(p, ctx, L, np.array([[5], [263]], dtype=np.int32), "bf16")
        else:
            (_ragged_case if case == "ragged" else _multi_case)("bf16")


def test_ffn_bf16_tall_tiles_at_group_size():
    """Context groups of 384 rows (one full and one partial 256-row tile) and
    a 512-row output group split along K, several column tiles."""
    with gemm_variant(2):
        D, F, r, L = 512, 2000, 16, 512
        ctx = [384, 384]
        p = _ffn_case(D, F, r, ctx, L, "bf16", seed=21)
        rng = np.random.default_rng(22)
        k = 600
        idx = np.stack([np.sort(rng.choice(F, k, replace=False)) for _ in ctx]).astype(np.int32)
        _compare(p, ctx, L, idx, "bf16")


@pytest.mark.parametrize("case", ["ragged", "multi"])
def test_ffn_bf16_narrow_gather_tiles(case):
    """The same cases with the wide N-gather tiles forbidden: the 128 x 256
    tiles that take operands the wide ones cannot (unaligned, K off 8)."""
    with gemm_variant(0):
        (_ragged_case if case == "ragged" else _multi_case)("bf16")


def _multi_case(dt):
    D, F, r, L = 512, 1104, 16, 300
    ctx = [290, 200, 300]
    p = _ffn_case(D, F, r, ctx, L, dt, seed=9)
    rng = np.random.default_rng(10)
    k = 300
    idx = np.stack([np.sort(rng.choice(F, k, replace=False)) for _ in ctx]).astype(np.int32)
    _compare(p, ctx, L, idx, dt)


def _estimate(p, ctx, L, Pg, Qg, Pu, Qu, rank, k, dt):
    sl = _api()
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], dt)
    F = Qg.shape[1]
    idx, sc = sl.estimate_select(sl.SL_CRIT_SWIGLU_L2, X, lay, rank, to_dev(Pg, dt), to_dev(Qg, dt),
                                 to_dev(Pu, dt), to_dev(Qu, dt), F, k, want_scores=True)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def _oracle_scores(p, ctx, L, Pg, Qg, Pu, Qu):
    B = len(ctx)
    out = []
    for b in range(B):
        rows = O.context_rows(ctx, L, b)
        out.append(O.scores_swiglu_l2(p["X"][rows], Pg.T, Qg, Pu.T, Qu, dtype=np.float32))
    return np.stack(out)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_estimate_select_matches_oracle(dt):
    D, F, r, L = 256, 688, 8, 200
    ctx = [200, 37, 0, 130]
    p = _ffn_case(D, F, r, ctx, L, dt, seed=11)
    Pg, Qg = factors(p["Wg"], 8, dt)
    Pu, Qu = factors(p["Wu"], 8, dt)
    k = 344
    idx, sc = _estimate(p, ctx, L, Pg, Qg, Pu, Qu, 8, k, dt)
    ref = _oracle_scores(p, ctx, L, Pg, Qg, Pu, Qu)
    for b in range(len(ctx)):
        e = np.abs(sc[b] - ref[b]).max() / max(ref[b].max(), 1e-30)
        assert e < 1e-4, f"seq {b} score rel err {e:.2e}"
    n_exact = check_selection(idx, ref, k)
    assert list(idx[2]) == list(range(k))   # empty context: ties everywhere -> lowest indices
    print(f"\n[{dt}] exact sets {n_exact}/{len(ctx)}", flush=True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("rank", [12, 32])
def test_estimate_select_high_rank(rank, dt):
    """SwiGLU criterion at estimator ranks past 8 (16- and 32-wide factor
    tiles on the matrix cores; in bf16 the three-term split of each projection
    spans two and three 32-wide k steps), a ragged channel block and a ragged
    token chunk."""
    D, F, r, L = 128, 360, 8, 140
    ctx = [140, 33]
    p = _ffn_case(D, F, r, ctx, L, dt, seed=13, R_in=rank)
    Pg, Qg = factors(p["Wg"], rank, dt)
    Pu, Qu = factors(p["Wu"], rank, dt)
    k = 120
    idx, sc = _estimate(p, ctx, L, Pg, Qg, Pu, Qu, rank, k, dt)
    ref = _oracle_scores(p, ctx, L, Pg, Qg, Pu, Qu)
    for b in range(len(ctx)):
        e = np.abs(sc[b] - ref[b]).max() / max(ref[b].max(), 1e-30)
        assert e < 1e-4, f"rank {rank} seq {b} score rel err {e:.2e}"
    check_selection(idx, ref, k)


@pytest.mark.parametrize("rank", [6, 8, 12])
@pytest.mark.parametrize("ctx", [[300, 0, 17, 260], [520, 129, 0]])
def test_estimate_select_sliced_stage1(rank, ctx):
    """bf16 SwiGLU estimate with d_in = 1544: the stage-1 product runs as four
    K slices, the last one 8 wide, summed by its finish launch.  Contexts of
    at most 512 tokens take 256-token criterion chunks (up to two partials per
    channel, added by the select kernel); the 520-token context takes
    128-token chunks and a separate score-sum launch.  An empty context sits
    among the others; ranks 6, 8 and 12 take the 8- and 16-wide factor tiles."""
    dt = "bf16"
    D, F, r = 1544, 520, 8
    L = max(ctx)
    p = _ffn_case(D, F, r, ctx, L, dt, seed=31 + rank, R_in=rank)
    Pg, Qg = factors(p["Wg"], rank, dt)
    Pu, Qu = factors(p["Wu"], rank, dt)
    k = 130
    idx, sc = _estimate(p, ctx, L, Pg, Qg, Pu, Qu, rank, k, dt)
    ref = _oracle_scores(p, ctx, L, Pg, Qg, Pu, Qu)
    check_scores(sc, ref, 1e-4)
    check_selection(idx, ref, k)
    for b, c in enumerate(ctx):
        if c == 0:
            assert list(idx[b]) == list(range(k))   # no context: all scores 0, lowest indices


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_backward_reads_only_saved(dt):
    """Everything the backward takes from the forward is in `saved` (z, z_d,
    G, U, H and the packed LoRA operands): a backward given a copy of the
    saved buffer and a fresh workspace filled with 0xFF bytes (NaN in bf16 and
    fp32) matches, bit for bit, the backward that shares the forward's
    workspace."""
    sl = _api()
    D, F, r, L = 512, 1104, 16, 300
    ctx = [290, 200, 300]
    p = _ffn_case(D, F, r, ctx, L, dt, seed=29)
    rng = np.random.default_rng(30)
    k = 300
    idx = np.stack([np.sort(rng.choice(F, k, replace=False)) for _ in ctx]).astype(np.int32)
    w = _dev_weights(p, dt, 0.5)
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], dt)
    idx_d = torch.from_numpy(idx).cuda()
    dY = to_dev(p["dY"], dt)
    _, buf = sl.ffn_fwd(w, X, lay, k, idx_d)
    g1 = sl.ffn_bwd(w, X, lay, k, idx_d, buf, dY)
    buf2 = sl.FFNWorkspace(w, lay, k, X.device)
    buf2.saved.copy_(buf.saved)
    buf2.ws.fill_(255)
    g2 = sl.ffn_bwd(w, X, lay, k, idx_d, buf2, dY)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), f"{n} differs with a fresh workspace"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_select_ties_and_k_extremes(dt):
    """Planted exact ties in the scores (zero factors) and k = 1, k = N."""
    sl = _api()
    D, F, L = 64, 96, 20
    ctx = [20, 10]
    p = _ffn_case(D, F, 4, ctx, L, dt, seed=12)
    Pg, Qg = factors(p["Wg"], 4, dt)
    Pu, Qu = factors(p["Wu"], 4, dt)
    Qu[:, 40:] = 0.0          # channels 40.. score exactly 0 -> ties
    for k in (1, 50, 80, F):
        idx, sc = _estimate(p, ctx, L, Pg, Qg, Pu, Qu, 4, k, dt)
        ref = _oracle_scores(p, ctx, L, Pg, Qg, Pu, Qu)
        check_selection(idx, ref, k)
        if k >= 50:
            for b in range(2):
                assert list(idx[b][40:]) == list(range(40, 40 + k - 40)), "ties must go to low indices"


def test_cfg1_workload_end_to_end():
    """The tiny fp32 workload: estimate, select, forward and backward."""
    w = W.WORKLOADS[1]
    p = W.make_ffn_tensors(w)
    f = w.ffn[0]
    ctx = [int(c) for c in W.ctx_lengths(w)]
    k = O.k_from_ratio(f.d_ff, f.sparsity_pct)
    Pg, Qg = factors(p["Wg"], w.est_rank, "f32")
    Pu, Qu = factors(p["Wu"], w.est_rank, "f32")
    idx, sc = _estimate(p, ctx, w.seq_len, Pg, Qg, Pu, Qu, w.est_rank, k, "f32")
    ref = _oracle_scores(p, ctx, w.seq_len, Pg, Qg, Pu, Qu)
    check_scores(sc, ref, 1e-4, "SwiGLU scores")
    n_exact = check_selection(idx, ref, k)
    use = idx if n_exact == len(ctx) else np.stack([O.select_topk(ref[b], k) for b in range(len(ctx))])
    _compare(p, ctx, w.seq_len, use, "f32")


def test_cfg2_full_size_parity():
    """LLaMA2-7B FFN shape at the benchmark's launch configuration."""
    w = W.WORKLOADS[2]
    p = W.make_ffn_tensors(w)
    f = w.ffn[0]
    ctx = [int(c) for c in W.ctx_lengths(w)]
    k = O.k_from_ratio(f.d_ff, f.sparsity_pct)
    Pg, Qg = factors(p["Wg"], w.est_rank, "bf16")
    Pu, Qu = factors(p["Wu"], w.est_rank, "bf16")
    idx, sc = _estimate(p, ctx, w.seq_len, Pg, Qg, Pu, Qu, w.est_rank, k, "bf16")
    ref = _oracle_scores(p, ctx, w.seq_len, Pg, Qg, Pu, Qu)
    check_scores(sc, ref, 1e-4, "SwiGLU scores")
    n_exact = check_selection(idx, ref, k)
    use = np.stack([O.select_topk(ref[b], k) for b in range(len(ctx))])
    errs = _compare(p, ctx, w.seq_len, use, "bf16")
    print(f"exact sets {n_exact}/{len(ctx)}", flush=True)


def test_backward_ordered_on_caller_stream():
    """The backward forks its gradient reductions onto a side stream and joins
    them back: on a stream of the caller's, work enqueued right after the call
    (a copy of every gradient, with no synchronisation in between) sees the
    final values, and the results equal those of the default stream bit for
    bit.  Repeated calls on one buffer set keep the same values."""
    sl = _api()
    D, F, r, L = 512, 1104, 16, 300
    ctx = [290, 200, 300]
    p = _ffn_case(D, F, r, ctx, L, "bf16", seed=17)
    rng = np.random.default_rng(18)
    idx = np.stack([np.sort(rng.choice(F, 300, replace=False)) for _ in ctx]).astype(np.int32)
    w = _dev_weights(p, "bf16", 1.0)
    lay = sl.Layout(ctx, L)
    X, dY = to_dev(p["X"], "bf16"), to_dev(p["dY"], "bf16")
    idx_d = torch.from_numpy(idx).cuda()
    _, buf = sl.ffn_fwd(w, X, lay, 300, idx_d)
    ref = {n: v.clone() for n, v in sl.ffn_bwd(w, X, lay, 300, idx_d, buf, dY).items()}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    copies = []
    with torch.cuda.stream(s):
        for _ in range(3):
            sl.ffn_fwd(w, X, lay, 300, idx_d, buf)
            g = sl.ffn_bwd(w, X, lay, 300, idx_d, buf, dY)
            copies.append({n: v.clone() for n, v in g.items()})   # same stream, no sync
    s.synchronize()
    for c in copies:
        for n, v in ref.items():
            assert torch.equal(c[n], v), f"{n} differs on the caller's stream"


def test_graph_capture_replays_match_eager():
    """Forward and backward captured into one graph (the library's side stream
    stays out of a capture): three replays, with eager work between them, each
    equal bit for bit to the eager results."""
    sl = _api()
    D, F, r, L = 256, 688, 8, 200
    ctx = [200, 37, 130]
    p = _ffn_case(D, F, r, ctx, L, "bf16", seed=19)
    rng = np.random.default_rng(20)
    k = 344
    idx = np.stack([np.sort(rng.choice(F, k, replace=False)) for _ in ctx]).astype(np.int32)
    w = _dev_weights(p, "bf16", 0.5)
    lay = sl.Layout(ctx, L)
    X, dY = to_dev(p["X"], "bf16"), to_dev(p["dY"], "bf16")
    idx_d = torch.from_numpy(idx).cuda()
    buf = sl.FFNWorkspace(w, lay, k, X.device)
    Y = torch.empty_like(X)
    sl.ffn_fwd(w, X, lay, k, idx_d, buf, Y=Y)
    out = sl.ffn_bwd(w, X, lay, k, idx_d, buf, dY)
    torch.cuda.synchronize()
    ref_y, ref = Y.clone(), {n: v.clone() for n, v in out.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sl.ffn_fwd(w, X, lay, k, idx_d, buf, Y=Y)
        sl.ffn_bwd(w, X, lay, k, idx_d, buf, dY, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sl.ffn_fwd(w, X, lay, k, idx_d, buf, Y=Y)
        sl.ffn_bwd(w, X, lay, k, idx_d, buf, dY, out=out)
    for rep in range(3):
        Y.zero_()
        for v in out.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref_y), f"replay {rep}: Y"
        for n, v in ref.items():
            assert torch.equal(out[n], v), f"replay {rep}: {n}"
