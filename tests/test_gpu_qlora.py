"""GPU parity of the sparse LoRA FFN over a 4-bit quantized frozen base
(SparseLoRA article §六) against the CPU oracle: the oracle quantizes the frozen
weights (codes and per-64-block scales), the GPU computes from the codes and
scales, and the oracle runs the same masked-dense forward and backward on the
exact dequantized weights."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _case(D, F, r, ctx, L, seed):
    rng = np.random.default_rng(seed)
    T = len(ctx) * L
    bf = lambda x: W.round_to_bf16(np.asarray(x, np.float32))
    X = bf(W.make_activations(seed, T, D, 16, "bf16"))
    Wg, Wu, WdT = (rng.standard_normal((F, D)) * 0.05 for _ in range(3))
    q = {}
    p = {"X": X, "dY": bf(rng.standard_normal((T, D)))}
    for n, w in (("Wg", Wg), ("Wu", Wu), ("WdT", WdT)):
        codes, scales = O.quantize_int4_rows(w)
        q[n + "_q"], q[n + "_s"] = codes, scales
        deq = O.dequantize_int4_rows(codes, scales)
        if n == "WdT":
            p["Wd"] = np.ascontiguousarray(deq.T)
        else:
            p[n] = deq
    for n, shape in (("Ag", (r, D)), ("Bg", (F, r)), ("Au", (r, D)), ("Bu", (F, r)), ("Ad", (r, F)),
                     ("Bd", (D, r))):
        p[n] = bf(rng.standard_normal(shape) * 0.05)
    return p, q


def _run(p, q, ctx, L, idx, s):
    import contextual_sparsity_lora_svd_amd as sl
    t = {n: torch.from_numpy(np.ascontiguousarray(v)).cuda() for n, v in q.items()}
    for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"):
        t[n] = to_dev(p[n], "bf16")
    w = sl.FFNWeights(t, lora_scale=s)
    assert w.quantized
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], "bf16")
    k = idx.shape[1]
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    Y, buf = sl.ffn_fwd(w, X, lay, k, idx_d)
    g = sl.ffn_bwd(w, X, lay, k, idx_d, buf, to_dev(p["dY"], "bf16"))
    torch.cuda.synchronize()
    return to_np(Y), {n: to_np(v) for n, v in g.items()}


def _compare(p, q, ctx, L, idx, s=1.0):
    y, g = _run(p, q, ctx, L, idx, s)
    yr, cache = O.ffn_forward(p, ctx, L, list(idx), s)
    gr = O.ffn_backward(p, cache, p["dY"], s)
    errs = {"Y": assert_close(y, yr, "bf16", "Y")}
    for n in ("dX", "dAg", "dBg", "dAu", "dBu", "dAd", "dBd"):
        errs[n] = assert_close(g[n], gr[n], "bf16", n)
    print(f"\n[q4] ctx={list(ctx)} k={idx.shape[1]} errs " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()),
          flush=True)


def _sets(rng, B, F, k):
    return np.stack([np.sort(rng.choice(F, k, replace=False)) for _ in range(B)]).astype(np.int32)


def test_qlora_ffn_ragged_groups():
    """All-context, all-output and mixed sequences; k and d_ff off the tiles."""
    D, F, r, L = 64, 136, 4, 50
    ctx = [50, 0, 37]
    p, q = _case(D, F, r, ctx, L, seed=31)
    _compare(p, q, ctx, L, _sets(np.random.default_rng(32), 3, F, 37), s=0.5)


def test_qlora_ffn_multi_tile():
    """Several M, N and K tiles, the output-group K split, LoRA rank 16."""
    D, F, r, L = 512, 1104, 16, 300
    ctx = [290, 200, 300]
    p, q = _case(D, F, r, ctx, L, seed=33)
    _compare(p, q, ctx, L, _sets(np.random.default_rng(34), 3, F, 300))


def test_qlora_ffn_dense_and_single_channel():
    D, F, r, L = 128, 264, 8, 80
    ctx = [60, 80]
    p, q = _case(D, F, r, ctx, L, seed=35)
    _compare(p, q, ctx, L, np.tile(np.arange(F, dtype=np.int32), (2, 1)))       # k = N
    _compare(p, q, ctx, L, np.array([[5], [263]], dtype=np.int32))            # k = 1


def test_qlora_rejects_fp32_and_ragged_width():
    import contextual_sparsity_lora_svd_amd as sl
    D, F, r, L = 64, 72, 4, 8
    ctx = [4]
    p, q = _case(D, F, r, ctx, L, seed=36)
    t = {n: torch.from_numpy(np.ascontiguousarray(v)).cuda() for n, v in q.items()}
    for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"):
        t[n] = to_dev(p[n], "f32")
    w = sl.FFNWeights(t)
    idx = torch.zeros((1, 4), dtype=torch.int32).cuda()
    with pytest.raises(sl.SparseLoraError):
        sl.ffn_fwd(w, to_dev(p["X"], "f32"), sl.Layout(ctx, L), 4, idx)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gpu_quantizer_matches_oracle_bit_exactly(dt):
    """Codes and scales are integer / fp32 decisions taken in fp32 on both sides."""
    import contextual_sparsity_lora_svd_amd as sl
    rng = np.random.default_rng(37)
    Wt = rng.standard_normal((300, 640)).astype(np.float32) * rng.lognormal(0, 2, (300, 1)).astype(np.float32)
    Wt[3, :64] = 0.0                                   # all-zero block
    Wt[4, :64] = np.arange(64) % 15 - 7.0              # exact codes, scale 1
    Wt[5, :64] = 0.0
    Wt[5, 0], Wt[5, 1], Wt[5, 2] = 7.0, 2.5, -3.5      # ties: rint -> 2 and -4
    if dt == "bf16":
        Wt = W.round_to_bf16(Wt)
    codes_r, scales_r = O.quantize_int4_rows(Wt)
    codes, scales = sl.quantize_q4(to_dev(Wt, dt))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), codes_r)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), scales_r.view(np.uint32))
    assert O.int4_codes(codes_r)[5, :3].tolist() == [7, 2, -4]


def _qkvo_q4(D, heads, r, ctx, L, seed):
    """The q/k/v/o case of tests/test_gpu_qkvo.py with its frozen weights
    quantized: device codes and scales, the oracle on the dequantized weights."""
    from tests.test_gpu_qkvo import _case as qkvo_case
    p = qkvo_case(D, heads, r, ctx, L, "bf16", seed)
    q = {}
    for n in ("Wq", "Wk", "Wv"):
        q[n + "_q"], q[n + "_s"] = O.quantize_int4_rows(p[n])
        p[n] = O.dequantize_int4_rows(q[n + "_q"], q[n + "_s"])
    q["WoT_q"], q["WoT_s"] = O.quantize_int4_rows(np.ascontiguousarray(p["Wo"].T))
    p["Wo"] = np.ascontiguousarray(O.dequantize_int4_rows(q["WoT_q"], q["WoT_s"]).T)
    return p, q


def _qkvo_compare(p, q, heads, ctx, L, idx_qk, idx_vo, s=1.0):
    import contextual_sparsity_lora_svd_amd as sl
    t = {n: torch.from_numpy(np.ascontiguousarray(v)).cuda() for n, v in q.items()}
    for n in ("Aq", "Bq", "Ak", "Bk", "Av", "Bv", "Ao", "Bo"):
        t[n] = to_dev(p[n], "bf16")
    w = sl.QKVOWeights(t, heads, lora_scale=s)
    lay = sl.Layout(ctx, L)
    X, a = to_dev(p["X"], "bf16"), to_dev(p["a"], "bf16")
    kqk, kvo = idx_qk.shape[1], idx_vo.shape[1]
    iqk = torch.from_numpy(np.ascontiguousarray(idx_qk, np.int32)).cuda()
    ivo = torch.from_numpy(np.ascontiguousarray(idx_vo, np.int32)).cuda()
    outs, buf = sl.qkvo_fwd(w, X, a, lay, kqk, iqk, kvo, ivo)
    g = sl.qkvo_bwd(w, X, a, lay, kqk, iqk, kvo, ivo, buf, dq=to_dev(p["dq"], "bf16"),
                    dk=to_dev(p["dk"], "bf16"), dv=to_dev(p["dv"], "bf16"), d_out=to_dev(p["d_out"], "bf16"))
    torch.cuda.synchronize()
    ref, cache = O.qkvo_forward(p, ctx, L, list(idx_qk), list(idx_vo), heads, s)
    gr = O.qkvo_backward(p, cache, {n: p[n] for n in ("dq", "dk", "dv", "d_out")}, s)
    errs = {}
    for n in ("q", "k", "v", "o"):
        errs[n] = assert_close(to_np(outs[n]), ref[n], "bf16", n)
    assert np.all(to_np(outs["q"])[cache["mq"] == 0] == 0)
    for n in ("dX", "da", "dAq", "dBq", "dAk", "dBk", "dAv", "dBv", "dAo", "dBo"):
        errs[n] = assert_close(to_np(g[n]), gr[n], "bf16", n)
    print(f"\n[q4] heads={heads} ctx={list(ctx)} kqk={kqk} kvo={kvo} " +
          " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)


@pytest.mark.parametrize("heads", [(4, 4, 16), (8, 2, 16)])
def test_qlora_qkvo_ragged(heads):
    D, r, L = 128, 8, 60
    ctx = [40, 60, 0]
    p, q = _qkvo_q4(D, heads, r, ctx, L, seed=41)
    nkv = heads[1] * heads[2]
    rng = np.random.default_rng(42)
    _qkvo_compare(p, q, heads, ctx, L, _sets(rng, 3, nkv, nkv * 5 // 16), _sets(rng, 3, nkv, nkv * 9 // 16 + 1),
                  s=0.5)


def test_qlora_qkvo_multi_tile():
    heads = (16, 4, 64)
    D, r, L = 512, 16, 300
    ctx = [260, 300, 150]
    p, q = _qkvo_q4(D, heads, r, ctx, L, seed=43)
    nkv = heads[1] * heads[2]
    rng = np.random.default_rng(44)
    _qkvo_compare(p, q, heads, ctx, L, _sets(rng, 3, nkv, 130), _sets(rng, 3, nkv, 190))
