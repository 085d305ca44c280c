"""The autograd modules and the schedule around the kernels, end to end: a
dense warm-up step and a sparse step of the FFN and of the q/k/v/o projections
(with a small differentiable attention core of the caller's between them), the
outputs and every gradient torch autograd routes compared with the oracle on
the same channel sets."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import assert_close, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _bf(x):
    return W.round_to_bf16(np.asarray(x, dtype=np.float32))


def _np_params(mod, names):
    return {n: _bf(getattr(mod, n).detach().cpu().numpy()) for n in names}


@pytest.mark.parametrize("step", [0, 5])
def test_ffn_module_warmup_then_sparse(step):
    import contextual_sparsity_lora_svd_amd as sl
    D, F, r, L = 128, 344, 8, 64
    ctx = [48, 40]
    T = len(ctx) * L
    rng = np.random.default_rng(21)
    Wg, Wu, Wd = (_bf(rng.standard_normal(s) * 0.05) for s in ((F, D), (F, D), (D, F)))
    X = W.make_activations(9, T, D, 16, "bf16")
    dY = _bf(rng.standard_normal((T, D)))
    sched = sl.SparsitySchedule([sl.LayerRatios(ffn=75)], total_steps=20)   # 2 dense steps
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    g = torch.Generator().manual_seed(3)
    mod = sl.SparseLoRAFFN(dev(Wg), dev(Wu), dev(Wd), r, est_rank=8, lora_scale=0.5, schedule=sched,
                           generator=g)
    lay = sl.Layout(ctx, L)
    Xd = dev(X).requires_grad_(True)
    Y = mod(Xd, lay, step=step)
    Y.backward(dev(dY))
    torch.cuda.synchronize()
    k = mod.last_k
    assert k == (F if step < 2 else sl.k_from_ratio(F, 75))
    idx = mod.last_idx.cpu().numpy()
    if step < 2:
        assert np.array_equal(idx, np.tile(np.arange(F, dtype=np.int32), (len(ctx), 1)))
    p = {"X": X, "Wg": Wg, "Wu": Wu, "Wd": Wd, "dY": dY}
    p.update(_np_params(mod, ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")))
    yr, cache = O.ffn_forward(p, ctx, L, list(idx), 0.5)
    gr = O.ffn_backward(p, cache, dY, 0.5)
    assert_close(to_np(Y), yr, "bf16", "Y")
    assert_close(to_np(Xd.grad), gr["dX"], "bf16", "dX")
    for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"):
        gp = getattr(mod, n).grad
        assert gp.dtype == torch.float32
        assert_close(to_np(gp), gr["d" + n], "bf16", "d" + n)


@pytest.mark.parametrize("step", [0, 5])
def test_qkvo_module_with_caller_attention(step):
    import contextual_sparsity_lora_svd_amd as sl
    D, hq, hkv, hd, r, L = 128, 4, 2, 16, 8, 48
    heads = (hq, hkv, hd)
    nq, nkv, G = hq * hd, hkv * hd, hq // hkv
    ctx = [32, 40]
    T = len(ctx) * L
    rng = np.random.default_rng(22)
    Wq, Wk, Wv = (_bf(rng.standard_normal(s) * 0.05) for s in ((nq, D), (nkv, D), (nkv, D)))
    Wo = _bf(rng.standard_normal((D, nq)) * 0.05)
    X = W.make_activations(10, T, D, 16, "bf16")
    dO = _bf(rng.standard_normal((T, D)))
    sched = sl.SparsitySchedule([sl.LayerRatios(qk=50, vo=50)], total_steps=20)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    mod = sl.SparseLoRAQKVO(dev(Wq), dev(Wk), dev(Wv), dev(Wo), heads, r, est_rank=4, lora_scale=0.5,
                            schedule=sched, generator=torch.Generator().manual_seed(4))
    lay = sl.Layout(ctx, L)

    def rep(x):   # kv heads -> query heads
        return x.view(T, hkv, 1, hd).expand(T, hkv, G, hd).reshape(T, nq)

    def attention(q, k, v):   # the caller's core: a = q * v + k per query head
        return (q.float() * rep(v).float() + rep(k).float()).to(q.dtype)

    Xd = dev(X).requires_grad_(True)
    out = mod(Xd, lay, attention, step=step)
    out.backward(dev(dO))
    torch.cuda.synchronize()
    iqk, ivo = (t.cpu().numpy() for t in mod.last_idx)
    kqk, kvo = mod.last_k
    assert (kqk, kvo) == ((nkv, nkv) if step < 2 else (sl.k_from_ratio(nkv, 50),) * 2)

    # oracle: q, k, v; the same attention core in fp64; o; then the chain back
    p = {"X": X, "Wq": Wq, "Wk": Wk, "Wv": Wv, "Wo": Wo, "a": np.zeros((T, nq), np.float32)}
    p.update(_np_params(mod, ("Aq", "Bq", "Ak", "Bk", "Av", "Bv", "Ao", "Bo")))
    ref, _ = O.qkvo_forward(p, ctx, L, list(iqk), list(ivo), heads, 0.5)

    def rep_np(x):
        return np.repeat(x.reshape(T, hkv, 1, hd), G, axis=2).reshape(T, nq)

    a_ref = ref["q"] * rep_np(ref["v"]) + rep_np(ref["k"])
    p["a"] = a_ref
    ref, cache = O.qkvo_forward(p, ctx, L, list(iqk), list(ivo), heads, 0.5)
    zero = {"dq": np.zeros((T, nq)), "dk": np.zeros((T, nkv)), "dv": np.zeros((T, nkv)), "d_out": dO}
    da = O.qkvo_backward(p, cache, zero, 0.5)["da"]
    dq = da * rep_np(ref["v"])
    dv = (da * ref["q"]).reshape(T, hkv, G, hd).sum(axis=2).reshape(T, nkv)
    dk = da.reshape(T, hkv, G, hd).sum(axis=2).reshape(T, nkv)
    gr = O.qkvo_backward(p, cache, {"dq": dq, "dk": dk, "dv": dv, "d_out": dO}, 0.5)
    assert_close(to_np(out), ref["o"], "bf16", "o")
    assert_close(to_np(Xd.grad), gr["dX"], "bf16", "dX")
    for n in ("Aq", "Bq", "Ak", "Bk", "Av", "Bv", "Ao", "Bo"):
        assert_close(to_np(getattr(mod, n).grad), gr["d" + n], "bf16", "d" + n)


def _deq(mod, n):
    return O.dequantize_int4_rows(mod.frozen[n + "_q"].cpu().numpy(), mod.frozen[n + "_s"].cpu().numpy())


def test_ffn_module_over_4bit_base():
    """A sparse step of the FFN module holding its frozen weights as 4-bit
    codes; the oracle runs on the dequantized weights."""
    import contextual_sparsity_lora_svd_amd as sl
    D, F, r, L = 128, 344, 8, 64
    ctx = [48, 40]
    T = len(ctx) * L
    rng = np.random.default_rng(23)
    Wg, Wu, Wd = (_bf(rng.standard_normal(s) * 0.05) for s in ((F, D), (F, D), (D, F)))
    X = W.make_activations(11, T, D, 16, "bf16")
    dY = _bf(rng.standard_normal((T, D)))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
    mod = sl.SparseLoRAFFN(dev(Wg), dev(Wu), dev(Wd), r, est_rank=8, lora_scale=0.5,
                           generator=torch.Generator().manual_seed(5), base_bits=4)
    assert set(mod.frozen) == {"Wg_q", "Wg_s", "Wu_q", "Wu_s", "WdT_q", "WdT_s"}
    lay = sl.Layout(ctx, L)
    Xd = dev(X).requires_grad_(True)
    k = sl.k_from_ratio(F, 60)
    Y = mod(Xd, lay, k=k)
    Y.backward(dev(dY))
    torch.cuda.synchronize()
    idx = mod.last_idx.cpu().numpy()
    p = {"X": X, "Wg": _deq(mod, "Wg"), "Wu": _deq(mod, "Wu"), "Wd": _deq(mod, "WdT").T, "dY": dY}
    p.update(_np_params(mod, ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")))
    yr, cache = O.ffn_forward(p, ctx, L, list(idx), 0.5)
    gr = O.ffn_backward(p, cache, dY, 0.5)
    assert_close(to_np(Y), yr, "bf16", "Y")
    assert_close(to_np(Xd.grad), gr["dX"], "bf16", "dX")
    for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"):
        assert_close(to_np(getattr(mod, n).grad), gr["d" + n], "bf16", "d" + n)
