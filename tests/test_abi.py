"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects invalid arguments on the host before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparselora.h")


@pytest.fixture(scope="module")
def sl():
    import contextual_sparsity_lora_svd_amd as m
    if not os.path.exists(m.LIB_PATH):
        from contextual_sparsity_lora_svd_amd import build
        build.build(verbose=False)
    m.lib()
    return m


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sl_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(sl):
    names = _declared()
    assert len(names) >= 18
    L = sl.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # the binding declares exactly the header's entry points
    assert sorted(sl.SIGNATURES) == names


def test_status_strings(sl):
    L = sl.lib()
    assert L.sl_abi_version() == 3
    for code in range(9):
        assert L.sl_status_string(code)
    assert L.sl_status_string(99) == b"unknown status"


def _ffn_weights(sl, D=64, F=128, r=4, ptr=16):
    return sl.api.SlFfnWeights(D, F, r, 1.0, *([ptr] * 9))


def test_ffn_validation_errors(sl):
    L = sl.lib()
    lay = sl.Layout([3, 4], 4)
    w = _ffn_weights(sl)
    P = 4096  # any aligned, never-dereferenced address: validation fails first
    # null pointers
    st = L.sl_ffn_fwd(1, lay.ref, ctypes.byref(w), None, 10, P, P, P, 1 << 30, P, 1 << 30, None)
    assert st == 1
    # misaligned
    st = L.sl_ffn_fwd(1, lay.ref, ctypes.byref(w), P + 2, 10, P, P, P, 1 << 30, P, 1 << 30, None)
    assert st == 2
    # bad dtype
    st = L.sl_ffn_fwd(7, lay.ref, ctypes.byref(w), P, 10, P, P, P, 1 << 30, P, 1 << 30, None)
    assert st == 4
    # k out of range
    for k in (0, 129):
        st = L.sl_ffn_fwd(1, lay.ref, ctypes.byref(w), P, k, P, P, P, 1 << 30, P, 1 << 30, None)
        assert st == 5
    # ctx_len beyond seq_len / batch beyond the limit
    bad = sl.Layout([5, 1], 4)
    assert L.sl_ffn_fwd(1, bad.ref, ctypes.byref(w), P, 10, P, P, P, 1 << 30, P, 1 << 30, None) == 5
    big = sl.Layout([1] * 65, 4)
    assert L.sl_ffn_fwd(1, big.ref, ctypes.byref(w), P, 10, P, P, P, 1 << 30, P, 1 << 30, None) == 5
    # shapes not multiples of 8
    w2 = _ffn_weights(sl, D=60)
    assert L.sl_ffn_fwd(1, lay.ref, ctypes.byref(w2), P, 10, P, P, P, 1 << 30, P, 1 << 30, None) == 3
    # buffers too small
    st = L.sl_ffn_fwd(1, lay.ref, ctypes.byref(w), P, 10, P, P, P, 16, P, 1 << 30, None)
    assert st == 6
    assert b"saved" in L.sl_last_error()
    # everything valid: the host has no gfx950 device, so the call stops at the
    # device check (an error status, nothing launched)
    st = L.sl_ffn_fwd(1, lay.ref, ctypes.byref(w), P, 10, P, P, P, 1 << 30, P, 1 << 30, None)
    assert st in (7, 8)


def test_size_queries_follow_the_layout(sl):
    L = sl.lib()
    lay = sl.Layout([3, 4], 4)
    s_small = L.sl_ffn_saved_bytes(1, lay.ref, 64, 128, 4, 8)
    s_big = L.sl_ffn_saved_bytes(1, lay.ref, 64, 128, 4, 64)
    assert 0 < s_small < s_big
    # saved = z (fp32, T x 2rp) + z_d (T x rp) + G, U, H compact (bf16)
    #         + the backward's LoRA operands, bf16, packed by the forward: Bd^T (rp x d_model),
    #           Ad^T (d_ff x rp), [Ag; Au] (2rp x d_model), B_g[S]^T and B_u[S]^T (per sequence
    #           rp x ldk), B_g^T and B_u^T (rp x d_ff); and the index ramp (d_ff ints)
    T, rp, D, F, B, ldk = 8, 8, 64, 128, 2, 8
    comp = 3 * 8 + 1 * 128     # 3 context rows x ldk(8) + 1 output row x d_ff
    def up(x):
        return (x + 255) // 256 * 256
    expect = (up(T * 2 * rp * 4) + up(T * rp * 4) + 3 * up(comp * 2) + up(rp * D * 2) + up(F * rp * 2)
              + up(2 * rp * D * 2) + 2 * up(B * rp * ldk * 2) + 2 * up(rp * F * 2) + up(F * 4))
    assert s_small == expect
    assert L.sl_ffn_workspace_bytes(1, lay.ref, 64, 128, 4, 0) == 0   # invalid k
    assert L.sl_estimator_workspace_bytes(100, 50, 65) == 0
    assert L.sl_estimator_workspace_bytes(100, 50, 8) > 0


def test_estimate_select_validation(sl):
    L = sl.lib()
    lay = sl.Layout([10], 10)
    P = 4096
    heads = sl.api.SlHeads(4, 2, 8)
    # QK-norm selects over kv channels: N must be n_kv_heads * head_dim
    st = L.sl_estimate_select(2, 1, lay.ref, ctypes.byref(heads), P, 64, 8, P, P, P, P, 32, 4, P,
                              None, P, 1 << 30, None)
    assert st == 3
    st = L.sl_estimate_select(9, 1, lay.ref, None, P, 64, 8, P, P, P, P, 16, 4, P, None, P, 1 << 30,
                              None)
    assert st == 4
    st = L.sl_estimate_select(0, 1, lay.ref, None, P, 64, 40, P, P, P, P, 16, 4, P, None, P, 1 << 30,
                              None)
    assert st == 5          # rank above 32
    st = L.sl_estimate_select(0, 1, lay.ref, None, P, 64, 8, P, P, None, P, 16, 4, P, None, P,
                              1 << 30, None)
    assert st == 1          # SwiGLU needs both factor pairs


def test_estimate_select_multi_validation(sl):
    L = sl.lib()
    lay = sl.Layout([10], 10)
    P = 4096
    J = sl.api.SlEstJob
    jobs = (J * 3)()
    for j in range(3):
        jobs[j].crit, jobs[j].N, jobs[j].k = 2, 16, 4
        jobs[j].heads = sl.api.SlHeads(4, 2, 8)
        jobs[j].Pt0 = jobs[j].Q0 = jobs[j].Pt1 = jobs[j].Q1 = jobs[j].idx = P
    # three QK-norm jobs are six projections: more than one call takes
    assert L.sl_estimate_select_multi_workspace_bytes(lay.ref, 64, 8, 3, jobs) == 0
    st = L.sl_estimate_select_multi(1, lay.ref, P, 64, 8, 3, jobs, P, 1 << 30, None)
    assert st == 5
    assert L.sl_estimate_select_multi(1, lay.ref, P, 64, 8, 0, jobs, P, 1 << 30, None) == 5   # no jobs
    jobs[1].crit = 1                                                                            # QK + L2
    assert L.sl_estimate_select_multi_workspace_bytes(lay.ref, 64, 8, 2, jobs) > 0
    jobs[1].k = 17                                                                              # k > N
    assert L.sl_estimate_select_multi(1, lay.ref, P, 64, 8, 2, jobs, P, 1 << 30, None) == 5
    jobs[1].k = 4
    jobs[1].idx = None
    assert L.sl_estimate_select_multi(1, lay.ref, P, 64, 8, 2, jobs, P, 1 << 30, None) == 1


def test_qkvo_validation(sl):
    L = sl.lib()
    lay = sl.Layout([5, 2], 6)
    P = 4096
    w = sl.api.SlQkvoWeights(64, sl.api.SlHeads(4, 3, 8), 4, 1.0, *([P] * 12))
    st = L.sl_qkvo_fwd(1, lay.ref, ctypes.byref(w), P, P, 4, P, 4, P, P, P, P, P, P, 1 << 30, P,
                       1 << 30, None)
    assert st == 3          # 4 query heads do not divide into 3 kv heads
    w = sl.api.SlQkvoWeights(64, sl.api.SlHeads(4, 2, 8), 4, 1.0, *([P] * 12))
    st = L.sl_qkvo_fwd(1, lay.ref, ctypes.byref(w), None, None, 4, P, 4, P, P, P, P, P, P, 1 << 30, P,
                       1 << 30, None)
    assert st == 1          # nothing to compute
    st = L.sl_qkvo_fwd(1, lay.ref, ctypes.byref(w), P, None, 17, P, 4, P, P, P, P, P, P, 1 << 30, P,
                       1 << 30, None)
    assert st == 5          # k_qk above the 16 kv channels


def test_k_rule_matches_oracle(sl):
    import oracle as O
    for n in (1, 7, 688, 4096, 11008, 14336):
        for pct in (0, 1, 30, 50, 60, 75, 90, 99):
            assert sl.k_from_ratio(n, pct) == O.k_from_ratio(n, pct)


def test_gemm_config_round_trip(sl):
    """The GEMM variant switch is per-thread host state: set, read back, restore."""
    import threading
    prev = sl.gemm_config(-1)
    assert prev == 3                       # wide and tall tiles allowed by default
    assert sl.gemm_config(0) == prev
    assert sl.gemm_config(-1) == 0
    assert sl.gemm_config(15) == 0         # bits past the known variants are dropped
    assert sl.gemm_config(-1) == 7
    seen = []
    t = threading.Thread(target=lambda: seen.append(sl.gemm_config(-1)))
    t.start()
    t.join()
    assert seen == [3]                     # another thread keeps its own default
    sl.gemm_config(prev)


def test_operand_extent_limits_rejected_before_launch(sl):
    """Every matrix the gather-GEMMs address must hold fewer than 2^31 elements;
    calls past that return SL_ERR_RANGE from host validation (nothing launched:
    the host has no GPU, so reaching the device check would give 7 or 8)."""
    L = sl.lib()
    P = 4096
    # X / dY: 64 x 4096 tokens x d_model 8192 = 2^31 elements
    lay = sl.Layout([2048] * 64, 4096)
    w = _ffn_weights(sl, D=8192, F=128, r=4)
    assert L.sl_ffn_workspace_bytes(1, lay.ref, 8192, 128, 4, 8) == 0
    assert L.sl_ffn_fwd(1, lay.ref, ctypes.byref(w), P, 8, P, P, P, 1 << 40, P, 1 << 40, None) == 5
    assert b"2^31" in L.sl_last_error()
    # one fewer sequence fits
    lay2 = sl.Layout([2048] * 63, 4096)
    assert L.sl_ffn_workspace_bytes(1, lay2.ref, 8192, 128, 4, 8) > 0
    # a frozen weight of d_ff x d_model = 2^31 elements (d_model and d_ff within their own limits)
    small = sl.Layout([3, 4], 4)
    w = _ffn_weights(sl, D=1 << 16, F=1 << 15, r=4)
    assert L.sl_ffn_fwd(1, small.ref, ctypes.byref(w), P, 8, P, P, P, 1 << 40, P, 1 << 40, None) == 5
    # the compact G / U / H buffers of a dense warm-up step: 64 x 8192 output rows x d_ff 14336 > 2^31
    lay3 = sl.Layout([0] * 64, 8192)
    assert L.sl_ffn_saved_bytes(1, lay3.ref, 64, 14336, 4, 14336) == 0
    w = _ffn_weights(sl, D=64, F=14336, r=4)
    assert L.sl_ffn_bwd(1, lay3.ref, ctypes.byref(w), P, 14336, P, P, 1 << 40, P, P,
                        ctypes.byref(sl.api.SlFfnGrads(*([P] * 6))), P, 1 << 40, None) == 5
    # q/k/v/o: T x Hq*hd past the limit
    heads = sl.api.SlHeads(128, 8, 256)               # Hq*hd = 32768
    wq = sl.api.SlQkvoWeights(64, heads, 4, 1.0, *([P] * 12))
    lay4 = sl.Layout([4096] * 16, 4096)               # T = 65536: T x 32768 = 2^31
    st = L.sl_qkvo_fwd(1, lay4.ref, ctypes.byref(wq), P, P, 4, P, 4, P, P, P, P, P, P, 1 << 40, P,
                       1 << 40, None)
    assert st == 5


def test_select_channel_limit(sl):
    """Selection runs over up to 65536 channels; every sequence's keys take N
    words of workspace."""
    L = sl.lib()
    lay = sl.Layout([10, 4], 10)
    P = 4096
    ws_lds = L.sl_estimate_select_workspace_bytes(1, lay.ref, None, 64, 8, 32768)
    ws_big = L.sl_estimate_select_workspace_bytes(1, lay.ref, None, 64, 8, 32769)
    assert ws_lds >= 2 * 32768 * 4 and ws_big > ws_lds
    assert L.sl_estimate_select_workspace_bytes(1, lay.ref, None, 64, 8, 65536) > 0
    assert L.sl_estimate_select_workspace_bytes(1, lay.ref, None, 64, 8, 65537) == 0
    st = L.sl_estimate_select(1, 1, lay.ref, None, P, 64, 8, P, P, None, None, 65537, 4, P, None, P,
                              1 << 30, None)
    assert st == 5
    st = L.sl_estimate_select(1, 1, lay.ref, None, P, 64, 8, P, P, None, None, 65536, 65536, P, None, P,
                              1 << 40, None)
    assert st in (7, 8)     # valid: stops at the device check on a host without a GPU
