"""GPU parity at the full sizes of the 4-layer stack (non-uniform sparsity,
random output spans) and of the LLaMA3-8B FFN, through the C ABI.

Each case selects channels on the GPU and checks the sets against the oracle's
fp32 scores (bit-exact where the score gap allows), then runs forward and
backward on the oracle's sets and compares every output and gradient with the
oracle."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import check_scores, check_selection, factors, to_dev
from tests.test_gpu_ffn import _compare as ffn_compare
from tests.test_gpu_ffn import _estimate as ffn_estimate
from tests.test_gpu_ffn import _oracle_scores as ffn_scores
from tests.test_gpu_qkvo import _compare as qkvo_compare
from tests.test_gpu_qkvo import _qk_l2_oracle

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _api():
    import contextual_sparsity_lora_svd_amd as sl
    return sl


def _ffn_layer(wl, layer):
    f = wl.ffn[layer]
    p = W.make_ffn_tensors(wl, layer)
    ctx = [int(c) for c in W.ctx_lengths(wl)]
    L = wl.seq_len
    k = O.k_from_ratio(f.d_ff, f.sparsity_pct)
    print(f"\n[{wl.name} layer {layer}] ctx={ctx} k={k}", flush=True)
    if k == f.d_ff:
        # dense layer: any estimate selects every channel; factors are irrelevant
        rng = np.random.default_rng(7)
        Pt = W.round_to_bf16((rng.standard_normal((wl.est_rank, f.d_model)) * 0.1).astype(np.float32))
        Q = W.round_to_bf16((rng.standard_normal((wl.est_rank, f.d_ff)) * 0.1).astype(np.float32))
        idx, _ = ffn_estimate(p, ctx, L, Pt, Q, Pt, Q, wl.est_rank, k, "bf16")
        assert np.array_equal(idx, np.tile(np.arange(k, dtype=idx.dtype), (len(ctx), 1)))
        use = idx
    else:
        Pg, Qg = factors(p["Wg"], wl.est_rank, "bf16")
        Pu, Qu = factors(p["Wu"], wl.est_rank, "bf16")
        idx, sc = ffn_estimate(p, ctx, L, Pg, Qg, Pu, Qu, wl.est_rank, k, "bf16")
        ref = ffn_scores(p, ctx, L, Pg, Qg, Pu, Qu)
        check_scores(sc, ref, 1e-4, "SwiGLU scores")
        n_exact = check_selection(idx, ref, k)
        print(f"exact sets {n_exact}/{len(ctx)}", flush=True)
        use = np.stack([O.select_topk(ref[b], k) for b in range(len(ctx))])
    ffn_compare(p, ctx, L, use, "bf16")


@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_stack_ffn_layer(layer):
    """4-layer stack, FFN of one layer: sparsity 0/30/60/90 %, spans 32-256."""
    _ffn_layer(W.WORKLOADS[4], layer)


@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_stack_qkvo_layer(layer):
    """4-layer stack, q/k/v/o of one layer (QK-norm and L2 selection)."""
    _qkvo_layer(W.WORKLOADS[4], layer)


def _qkvo_layer(wl, layer):
    sl = _api()
    s = wl.attn[layer]
    heads = (s.n_q_heads, s.n_kv_heads, s.head_dim)
    p = W.make_attn_tensors(wl, layer)
    ctx = [int(c) for c in W.ctx_lengths(wl)]
    L = wl.seq_len
    nkv = heads[1] * heads[2]
    kqk = O.k_from_ratio(nkv, s.sparsity_qk_pct)
    kvo = O.k_from_ratio(nkv, s.sparsity_vo_pct)
    print(f"\n[{wl.name} layer {layer}] ctx={ctx} k_qk={kqk} k_vo={kvo}", flush=True)
    if kqk == nkv and kvo == nkv:
        full = np.tile(np.arange(nkv, dtype=np.int32), (len(ctx), 1))
        qkvo_compare(p, heads, ctx, L, full, full, "bf16")
        return
    Pq, Qq = factors(p["Wq"], wl.est_rank, "bf16")
    Pk, Qk = factors(p["Wk"], wl.est_rank, "bf16")
    Pv, Qv = factors(p["Wv"], wl.est_rank, "bf16")
    lay = sl.Layout(ctx, L)
    X = to_dev(p["X"], "bf16")
    idx_qk, sc_qk = sl.estimate_select(sl.SL_CRIT_QK_NORM, X, lay, wl.est_rank, to_dev(Pq, "bf16"),
                                       to_dev(Qq, "bf16"), to_dev(Pk, "bf16"), to_dev(Qk, "bf16"), nkv,
                                       kqk, heads=heads, want_scores=True)
    idx_vo, sc_vo = sl.estimate_select(sl.SL_CRIT_L2, X, lay, wl.est_rank, to_dev(Pv, "bf16"),
                                       to_dev(Qv, "bf16"), None, None, nkv, kvo, want_scores=True)
    torch.cuda.synchronize()
    ref_qk, ref_vo = _qk_l2_oracle(p, ctx, L, heads, Pq, Qq, Pk, Qk, Pv, Qv)
    check_scores(sc_qk.cpu().numpy(), ref_qk, 2e-4, "QK-norm scores")
    check_scores(sc_vo.cpu().numpy(), ref_vo, 1e-4, "L2 scores")
    n1 = check_selection(idx_qk.cpu().numpy(), ref_qk, kqk)
    n2 = check_selection(idx_vo.cpu().numpy(), ref_vo, kvo)
    print(f"exact sets qk {n1}/{len(ctx)} vo {n2}/{len(ctx)}", flush=True)
    iqk = np.stack([O.select_topk(ref_qk[b], kqk) for b in range(len(ctx))])
    ivo = np.stack([O.select_topk(ref_vo[b], kvo) for b in range(len(ctx))])
    qkvo_compare(p, heads, ctx, L, iqk, ivo, "bf16")


def test_llama3_ffn_full_size():
    """LLaMA3-8B FFN (d_ff 14336, LoRA rank 32, estimator rank 16, 90 %), 4096 tokens."""
    _ffn_layer(W.WORKLOADS[5], 0)


def test_extreme_sparsity_ffn():
    """99 % FFN sparsity (k = 110 of 11008) at the LLaMA2-7B shape, 4 x 512 tokens."""
    _ffn_layer(W.WORKLOADS[6], 0)


def test_extreme_sparsity_qkvo():
    """75 % q/k and v/o sparsity (1024 of 4096 kv channels) at the LLaMA2-7B shape."""
    _qkvo_layer(W.WORKLOADS[6], 0)
