"""GPU estimator build (truncated SVD) against planted spectra and the
oracle's LAPACK SVD, through the C ABI."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import to_dev, to_np

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _planted(rng, out_f, in_f, sig):
    U, _ = np.linalg.qr(rng.standard_normal((out_f, len(sig))))
    V, _ = np.linalg.qr(rng.standard_normal((in_f, len(sig))))
    return U @ np.diag(sig) @ V.T, U, V


@pytest.mark.parametrize("shape", [(300, 200), (200, 520)])
def test_planted_spectrum_fp32(shape):
    import contextual_sparsity_lora_svd_amd as sl
    rng = np.random.default_rng(31)
    sig = np.geomspace(10.0, 0.01, 60)
    Wm, U, V = _planted(rng, *shape, sig)
    Wm = Wm.astype(np.float32)
    for r in (1, 8, 16):
        Pt, Q, s = sl.build_estimator(to_dev(Wm, "f32"), r)
        torch.cuda.synchronize()
        PQ = to_np(Pt).T @ to_np(Q)
        expect = V[:, :r] @ np.diag(sig[:r]) @ U[:, :r].T
        err = np.abs(PQ - expect).max() / np.abs(expect).max()
        assert err < 1e-4, f"rank {r}: P.Q rel err {err:.2e}"
        np.testing.assert_allclose(to_np(s), sig[:r], rtol=1e-4)


def test_bf16_weight_matches_lapack():
    import contextual_sparsity_lora_svd_amd as sl
    rng = np.random.default_rng(32)
    sig = np.geomspace(4.0, 0.05, 40)
    Wm, _, _ = _planted(rng, 256, 384, sig)
    Wm = W.round_to_bf16(Wm.astype(np.float32)) + W.round_to_bf16(
        (rng.standard_normal((256, 384)) * 1e-3).astype(np.float32))
    Wm = W.round_to_bf16(Wm)
    P, Qr, S = O.build_estimator(Wm, 8)
    Pt, Q, s = sl.build_estimator(to_dev(Wm, "bf16"), 8)
    torch.cuda.synchronize()
    PQ = to_np(Pt).T @ to_np(Q)
    ref = P @ Qr
    err = np.abs(PQ - ref).max() / np.abs(ref).max()
    assert err < 2e-2, f"P.Q rel err {err:.2e} (bf16 factors)"
    np.testing.assert_allclose(to_np(s), S, rtol=1e-3)


def test_eckart_young_residual_flat_spectrum():
    """Gaussian weight (flat spectrum): the rank-r residual must be close to the
    optimal one, sum of the trailing squared singular values."""
    import contextual_sparsity_lora_svd_amd as sl
    rng = np.random.default_rng(33)
    Wm = (rng.standard_normal((640, 320)) * 0.02).astype(np.float32)
    S = np.linalg.svd(Wm.astype(np.float64), compute_uv=False)
    r = 8
    Pt, Q, s = sl.build_estimator(to_dev(Wm, "f32"), r, iters=20)
    torch.cuda.synchronize()
    resid = np.linalg.norm(Wm - (to_np(Pt).T @ to_np(Q)).T) ** 2
    opt = float((S[r:] ** 2).sum())
    assert resid <= opt * 1.01, f"residual {resid:.4e} vs optimal {opt:.4e}"
    assert resid >= opt * (1 - 1e-6)
