"""The allocation-free estimate-and-select entry point (fixed per-device
scratch in the library's device memory) against sl_estimate_select with a
caller workspace, through the C ABI: two calls in a row, the second smaller,
each bit-for-bit equal to the workspace variant (same kernels, same order)."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_helpers import factors, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _api():
    import contextual_sparsity_lora_svd_amd as sl
    return sl


def _case(D, F, ctx, L, seed):
    rng = np.random.default_rng(seed)
    T = len(ctx) * L
    X = (rng.standard_normal((T, 16)) @ rng.standard_normal((16, D)) + 0.1 * rng.standard_normal((T, D)))
    X = W.round_to_bf16((X * rng.lognormal(0, 1, D)).astype(np.float32))
    Wg = W.round_to_bf16((rng.standard_normal((F, D)) * 0.02).astype(np.float32))
    Wu = W.round_to_bf16((rng.standard_normal((F, D)) * 0.02).astype(np.float32))
    return X, Wg, Wu


def _both(sl, X, Wg, Wu, ctx, L, rank, k):
    Pg, Qg = factors(Wg, rank, "bf16")
    Pu, Qu = factors(Wu, rank, "bf16")
    lay = sl.Layout(ctx, L)
    F = Wg.shape[0]
    Xd = to_dev(X, "bf16")
    args = (to_dev(Pg, "bf16"), to_dev(Qg, "bf16"), to_dev(Pu, "bf16"), to_dev(Qu, "bf16"))
    ref_idx, ref_sc = sl.estimate_select(sl.SL_CRIT_SWIGLU_L2, Xd, lay, rank, *args, F, k, want_scores=True)
    idx = torch.full((len(ctx), k), -1, dtype=torch.int32, device="cuda")
    sc = torch.full((len(ctx), F), float("nan"), dtype=torch.float32, device="cuda")
    sl.estimate_select_noalloc(sl.SL_CRIT_SWIGLU_L2, Xd, lay, rank, *args, F, k, idx, sc)
    torch.cuda.synchronize()
    return (ref_idx, ref_sc), (idx, sc)


def test_noalloc_matches_workspace_variant_twice_shrinking():
    sl = _api()
    # first call: 4 sequences at the LLaMA2-7B FFN width; second: 2 shorter sequences, narrower
    for (D, F, ctx, L, k, seed) in ((1024, 11008, [384, 384, 200, 384], 512, 2752, 3),
                                    (512, 2000, [100, 37], 128, 500, 4)):
        X, Wg, Wu = _case(D, F, ctx, L, seed)
        (ri, rs), (gi, gs) = _both(sl, X, Wg, Wu, ctx, L, 8, k)
        print(f"\nD={D} F={F} ctx={ctx} k={k}", flush=True)
        assert torch.equal(gi, ri), "index sets differ from the workspace variant"
        assert torch.equal(gs, rs), "scores differ from the workspace variant"


def test_noalloc_rejects_calls_beyond_the_scratch():
    sl = _api()
    lay = sl.Layout([4000] * 64, 4096)
    L = sl.lib()
    need = L.sl_estimate_select_workspace_bytes(0, lay.ref, None, 8192, 32, 14336)
    assert need > (32 << 20)
    X = torch.empty(8, 8, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(64, 8, dtype=torch.int32, device="cuda")
    st = L.sl_estimate_select_noalloc(0, 1, lay.ref, None, X.data_ptr(), 8192, 32, X.data_ptr(),
                                      X.data_ptr(), X.data_ptr(), X.data_ptr(), 14336, 8, idx.data_ptr(),
                                      None, None)
    assert st == 6 and b"scratch" in L.sl_last_error()
