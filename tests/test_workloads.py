"""The seeded input generators: planted-spectrum weights."""
import numpy as np

import workloads as W


def test_planted_weight_spectrum():
    out_f, in_f, alpha = 48, 32, 1.0
    Wt = W.make_planted_weight(5, out_f, in_f, alpha, "f32")
    s = np.linalg.svd(Wt.astype(np.float64), compute_uv=False)
    want = np.arange(1, in_f + 1, dtype=np.float64) ** -alpha
    want *= np.sqrt(out_f * in_f * 4e-4 / (want * want).sum())
    assert np.allclose(s, want, rtol=1e-4), (s[:4], want[:4])
    # mean square of N(0, 0.02^2) entries
    assert abs((Wt.astype(np.float64) ** 2).mean() - 4e-4) < 1e-7
    # seeded: same seed, same weight; bf16 is the rounded f32
    assert np.array_equal(Wt, W.make_planted_weight(5, out_f, in_f, alpha, "f32"))
    assert np.array_equal(W.make_planted_weight(5, out_f, in_f, alpha, "bf16"), W.round_to_bf16(Wt))
