"""ctypes binding of libsparselora.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
allocates outputs and scratch with torch, passes raw device pointers and the
current HIP stream, and turns status codes into exceptions.  It never falls
back to any other implementation: if the library is missing it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparselora.so")

SL_F32, SL_BF16 = 0, 1
SL_CRIT_SWIGLU_L2, SL_CRIT_L2, SL_CRIT_QK_NORM = 0, 1, 2
SL_MAX_SEQS = 64
SL_EST_MAXJOBS = 3

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class SlLayout(ctypes.Structure):
    _fields_ = [("batch", _i32), ("seq_len", _i32), ("ctx_len", ctypes.POINTER(_i32))]


class SlHeads(ctypes.Structure):
    _fields_ = [("n_q_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32)]


class SlEstJob(ctypes.Structure):
    _fields_ = [("crit", ctypes.c_int), ("heads", SlHeads), ("Pt0", _vp), ("Q0", _vp), ("Pt1", _vp),
                ("Q1", _vp), ("N", _i64), ("k", _i32), ("idx", _vp), ("scores", _vp)]


class SlFfnWeights(ctypes.Structure):
    _fields_ = [("d_model", _i64), ("d_ff", _i64), ("lora_rank", _i32), ("lora_scale", ctypes.c_float),
                ("Wg", _vp), ("Wu", _vp), ("WdT", _vp), ("Ag", _vp), ("Bg", _vp), ("Au", _vp),
                ("Bu", _vp), ("Ad", _vp), ("Bd", _vp),
                ("Wg_q", _vp), ("Wu_q", _vp), ("WdT_q", _vp), ("Wg_s", _vp), ("Wu_s", _vp), ("WdT_s", _vp)]


class SlFfnGrads(ctypes.Structure):
    _fields_ = [("dAg", _vp), ("dBg", _vp), ("dAu", _vp), ("dBu", _vp), ("dAd", _vp), ("dBd", _vp)]


class SlQkvoWeights(ctypes.Structure):
    _fields_ = [("d_model", _i64), ("heads", SlHeads), ("lora_rank", _i32),
                ("lora_scale", ctypes.c_float),
                ("Wq", _vp), ("Wk", _vp), ("Wv", _vp), ("WoT", _vp),
                ("Aq", _vp), ("Bq", _vp), ("Ak", _vp), ("Bk", _vp), ("Av", _vp), ("Bv", _vp),
                ("Ao", _vp), ("Bo", _vp),
                ("Wq_q", _vp), ("Wk_q", _vp), ("Wv_q", _vp), ("WoT_q", _vp),
                ("Wq_s", _vp), ("Wk_s", _vp), ("Wv_s", _vp), ("WoT_s", _vp)]


class SlQkvoGrads(ctypes.Structure):
    _fields_ = [("dAq", _vp), ("dBq", _vp), ("dAk", _vp), ("dBk", _vp), ("dAv", _vp), ("dBv", _vp),
                ("dAo", _vp), ("dBo", _vp)]


# name -> (restype, argtypes)
SIGNATURES = {
    "sl_abi_version": (ctypes.c_int, []),
    "sl_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sl_last_error": (ctypes.c_char_p, []),
    "sl_estimator_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "sl_build_estimator": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp,
                                          _vp, _sz, _vp]),
    "sl_estimate_select_workspace_bytes": (_sz, [ctypes.c_int, ctypes.POINTER(SlLayout),
                                                 ctypes.POINTER(SlHeads), _i64, _i32, _i64]),
    "sl_estimate_select": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.POINTER(SlLayout),
                                          ctypes.POINTER(SlHeads), _vp, _i64, _i32, _vp, _vp, _vp,
                                          _vp, _i64, _i32, _vp, _vp, _vp, _sz, _vp]),
    "sl_estimate_select_noalloc": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.POINTER(SlLayout),
                                                  ctypes.POINTER(SlHeads), _vp, _i64, _i32, _vp, _vp, _vp,
                                                  _vp, _i64, _i32, _vp, _vp, _vp]),
    "sl_estimate_select_multi_workspace_bytes": (_sz, [ctypes.POINTER(SlLayout), _i64, _i32, _i32,
                                                       ctypes.POINTER(SlEstJob)]),
    "sl_estimate_select_multi": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(SlLayout), _vp, _i64, _i32,
                                                _i32, ctypes.POINTER(SlEstJob), _vp, _sz, _vp]),
    "sl_ffn_saved_bytes": (_sz, [ctypes.c_int, ctypes.POINTER(SlLayout), _i64, _i64, _i32, _i32]),
    "sl_ffn_workspace_bytes": (_sz, [ctypes.c_int, ctypes.POINTER(SlLayout), _i64, _i64, _i32,
                                     _i32]),
    "sl_ffn_fwd": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(SlLayout),
                                  ctypes.POINTER(SlFfnWeights), _vp, _i32, _vp, _vp, _vp, _sz, _vp,
                                  _sz, _vp]),
    "sl_ffn_bwd": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(SlLayout),
                                  ctypes.POINTER(SlFfnWeights), _vp, _i32, _vp, _vp, _sz, _vp, _vp,
                                  ctypes.POINTER(SlFfnGrads), _vp, _sz, _vp]),
    "sl_timer_enable": (ctypes.c_int, [ctypes.c_int]),
    "sl_gemm_config": (ctypes.c_int, [ctypes.c_int]),
    "sl_quantize_q4": (ctypes.c_int, [ctypes.c_int, _vp, _i64, _i64, _vp, _vp, _vp]),
    "sl_timer_select": (None, [ctypes.c_uint32]),
    "sl_timer_reset": (None, []),
    "sl_timer_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int)]),
    "sl_qkvo_saved_bytes": (_sz, [ctypes.c_int, ctypes.POINTER(SlLayout),
                                  ctypes.POINTER(SlQkvoWeights)]),
    "sl_qkvo_workspace_bytes": (_sz, [ctypes.c_int, ctypes.POINTER(SlLayout),
                                      ctypes.POINTER(SlQkvoWeights), _i32, _i32]),
    "sl_qkvo_fwd": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(SlLayout),
                                   ctypes.POINTER(SlQkvoWeights), _vp, _vp, _i32, _vp, _i32, _vp,
                                   _vp, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp]),
    "sl_qkvo_bwd": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(SlLayout),
                                   ctypes.POINTER(SlQkvoWeights), _vp, _vp, _i32, _vp, _i32, _vp,
                                   _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp,
                                   ctypes.POINTER(SlQkvoGrads), _vp, _sz, _vp]),
}

_lib = None


class SparseLoraError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load the HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SparseLoraError(
                f"{LIB_PATH} is missing: build it with contextual_sparsity_lora_svd_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        L = lib()
        raise SparseLoraError(f"{what}: {L.sl_status_string(status).decode()} "
                              f"(status {status}): {L.sl_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SL_BF16
    if t.dtype == torch.float32:
        return SL_F32
    raise SparseLoraError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise SparseLoraError("tensors must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class Layout:
    """Host-side sequence layout (batch, seq_len, ctx_len[b])."""

    def __init__(self, ctx_len: Sequence[int], seq_len: int):
        self.ctx = (_i32 * len(ctx_len))(*[int(c) for c in ctx_len])
        self.c = SlLayout(len(ctx_len), int(seq_len), self.ctx)
        self.batch = len(ctx_len)
        self.seq_len = int(seq_len)

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _bytes_tensor(n: int, device) -> torch.Tensor:
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


def k_from_ratio(n: int, sparsity_pct: int) -> int:
    """Channels kept at a per-layer sparsity percentage: round half up of
    (100 - p) * n / 100, at least 1."""
    return max((n * (100 - int(sparsity_pct)) + 50) // 100, 1)


TIMER_SLOTS = {"estimate": 0, "select": 1, "gu_fwd": 2, "down_fwd": 3, "dh_bwd": 4, "dx_bwd": 5,
               "qkv_fwd": 6, "o_fwd": 7, "da_bwd": 8, "dxqkv_bwd": 9}


def timer_enable(max_launches: int):
    _check(lib().sl_timer_enable(int(max_launches)), "sl_timer_enable")


def timer_select(slots):
    """Record only the named slots (None: all)."""
    mask = 0xFFFFFFFF if slots is None else sum(1 << TIMER_SLOTS[n] for n in slots)
    lib().sl_timer_select(mask)


def timer_reset():
    lib().sl_timer_reset()


def quantize_q4(W: torch.Tensor):
    """4-bit codes (uint8 [rows, cols / 2]) and block scales (fp32 [rows, cols / 64])
    of a frozen weight W [rows, cols], for FFNWeights' quantized base."""
    rows, cols = W.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=W.device)
    scales = torch.empty((rows, max(cols // 64, 1)), dtype=torch.float32, device=W.device)
    _check(lib().sl_quantize_q4(_dtype_code(W), _ptr(W), rows, cols, _ptr(codes), _ptr(scales), _stream()),
           "sl_quantize_q4")
    return codes, scales


GEMM_WIDE, GEMM_TALL, GEMM_TALL_ALWAYS = 1, 2, 4


def gemm_config(variants: int = -1) -> int:
    """GEMM tile variants the calling thread allows, a bit mask: GEMM_WIDE
    (128 x 512 N-gather), GEMM_TALL (256 x 256 K-gather), GEMM_TALL_ALWAYS
    (tall tiles whatever their grid); 0 = 128 x 256 only; -1 only reads.
    Returns the previous setting."""
    return int(lib().sl_gemm_config(int(variants)))


def timer_read(slot: str):
    """(total milliseconds, launches) recorded for a slot since the last reset."""
    t = ctypes.c_double(0)
    n = ctypes.c_int(0)
    _check(lib().sl_timer_read(TIMER_SLOTS[slot], ctypes.byref(t), ctypes.byref(n)), "sl_timer_read")
    return t.value, n.value


# ---------------------------------------------------------------------------
def build_estimator(W: torch.Tensor, rank: int, iters: int = 0):
    """Truncated-SVD factors of a frozen weight W [out, in]: Pt [rank, in],
    Q [rank, out], sigma [rank] (fp32)."""
    L = lib()
    out_f, in_f = W.shape
    Pt = torch.empty(rank, in_f, dtype=W.dtype, device=W.device)
    Q = torch.empty(rank, out_f, dtype=W.dtype, device=W.device)
    sig = torch.empty(rank, dtype=torch.float32, device=W.device)
    ws = _bytes_tensor(L.sl_estimator_workspace_bytes(out_f, in_f, rank), W.device)
    _check(L.sl_build_estimator(_dtype_code(W), _ptr(W), out_f, in_f, rank, iters, _ptr(Pt),
                                _ptr(Q), _ptr(sig), _ptr(ws), ws.numel(), _stream()),
           "sl_build_estimator")
    return Pt, Q, sig


class EstimateBuffers:
    """Reusable idx / scores / scratch buffers of estimate_select."""

    def __init__(self, crit: int, layout: Layout, d_in: int, rank: int, N: int, k: int, device,
                 heads: Optional[Sequence[int]] = None, want_scores: bool = False):
        L = lib()
        self.heads = SlHeads(*heads) if heads is not None else None
        href = ctypes.byref(self.heads) if self.heads is not None else None
        self.idx = torch.empty(layout.batch, k, dtype=torch.int32, device=device)
        self.scores = (torch.empty(layout.batch, N, dtype=torch.float32, device=device)
                       if want_scores else None)
        self.ws = _bytes_tensor(L.sl_estimate_select_workspace_bytes(crit, layout.ref, href, d_in,
                                                                     rank, N), device)


def estimate_select(crit: int, X: torch.Tensor, layout: Layout, rank: int, Pt0, Q0, Pt1, Q1,
                    N: int, k: int, heads: Optional[Sequence[int]] = None,
                    want_scores: bool = False, bufs: Optional[EstimateBuffers] = None):
    """Per-sequence channel sets idx [batch, k] (int32, ascending) and,
    optionally, the scores [batch, N] (fp32)."""
    L = lib()
    bufs = bufs or EstimateBuffers(crit, layout, X.shape[1], rank, N, k, X.device, heads,
                                   want_scores)
    href = ctypes.byref(bufs.heads) if bufs.heads is not None else None
    _check(L.sl_estimate_select(crit, _dtype_code(X), layout.ref, href, _ptr(X), X.shape[1], rank,
                                _ptr(Pt0), _ptr(Q0), _ptr(Pt1), _ptr(Q1), N, k, _ptr(bufs.idx),
                                _ptr(bufs.scores), _ptr(bufs.ws), bufs.ws.numel(), _stream()),
           "sl_estimate_select")
    return bufs.idx, bufs.scores


def estimate_select_noalloc(crit: int, X: torch.Tensor, layout: Layout, rank: int, Pt0, Q0, Pt1, Q1,
                            N: int, k: int, idx: torch.Tensor, scores: Optional[torch.Tensor] = None,
                            heads: Optional[Sequence[int]] = None):
    """estimate_select into caller-owned idx [batch, k] (int32) and optional
    scores [batch, N] (fp32), with the library's fixed per-device scratch in
    place of a workspace: the call allocates no device memory."""
    L = lib()
    h = SlHeads(*heads) if heads is not None else None
    _check(L.sl_estimate_select_noalloc(crit, _dtype_code(X), layout.ref, ctypes.byref(h) if h else None,
                                        _ptr(X), X.shape[1], rank, _ptr(Pt0), _ptr(Q0), _ptr(Pt1), _ptr(Q1),
                                        N, k, _ptr(idx), _ptr(scores), _stream()),
           "sl_estimate_select_noalloc")
    return idx, scores


class EstimateMultiBuffers:
    """Reusable idx / scores / scratch buffers of estimate_select_multi.  Each
    job is a dict with crit, N, k and optionally heads and want_scores."""

    def __init__(self, layout: Layout, d_in: int, rank: int, jobs: Sequence[dict], device):
        L = lib()
        if not 1 <= len(jobs) <= SL_EST_MAXJOBS:
            raise ValueError(f"1..{SL_EST_MAXJOBS} jobs")
        self.c = (SlEstJob * len(jobs))()
        self.idx, self.scores = [], []
        for j, job in enumerate(jobs):
            c = self.c[j]
            c.crit, c.N, c.k = job["crit"], job["N"], job["k"]
            if job.get("heads") is not None:
                c.heads = SlHeads(*job["heads"])
            self.idx.append(torch.empty(layout.batch, job["k"], dtype=torch.int32, device=device))
            self.scores.append(torch.empty(layout.batch, job["N"], dtype=torch.float32, device=device)
                               if job.get("want_scores") else None)
        self.ws = _bytes_tensor(L.sl_estimate_select_multi_workspace_bytes(layout.ref, d_in, rank, len(jobs),
                                                                           self.c), device)


def estimate_select_multi(X: torch.Tensor, layout: Layout, rank: int, jobs: Sequence[dict],
                          bufs: Optional[EstimateMultiBuffers] = None):
    """Several criteria over one input X in one call.  Each job is a dict with
    crit, Pt0, Q0 (and Pt1, Q1 unless L2), N, k and optionally heads (QK-norm)
    and want_scores.  Returns [(idx, scores)] in job order, as separate
    estimate_select calls would."""
    L = lib()
    bufs = bufs or EstimateMultiBuffers(layout, X.shape[1], rank, jobs, X.device)
    for j, job in enumerate(jobs):
        c = bufs.c[j]
        c.Pt0, c.Q0 = _ptr(job["Pt0"]), _ptr(job["Q0"])
        c.Pt1, c.Q1 = _ptr(job.get("Pt1")), _ptr(job.get("Q1"))
        c.idx, c.scores = _ptr(bufs.idx[j]), _ptr(bufs.scores[j])
    _check(L.sl_estimate_select_multi(_dtype_code(X), layout.ref, _ptr(X), X.shape[1], rank, len(jobs), bufs.c,
                                      _ptr(bufs.ws), bufs.ws.numel(), _stream()),
           "sl_estimate_select_multi")
    return list(zip(bufs.idx, bufs.scores))


class FFNWeights:
    """Device tensors of one FFN layer: Wg, Wu, WdT, Ag, Bg, Au, Bu, Ad, Bd.

    A 4-bit frozen base replaces Wg, Wu, WdT by Wg_q, Wu_q, WdT_q (uint8 codes
    [d_ff, d_model / 2]) and Wg_s, Wu_s, WdT_s (fp32 scales [d_ff, d_model / 64])."""

    NAMES = ("Wg", "Wu", "WdT", "Ag", "Bg", "Au", "Bu", "Ad", "Bd")
    QNAMES = ("Wg_q", "Wu_q", "WdT_q", "Wg_s", "Wu_s", "WdT_s")

    def __init__(self, t: Dict[str, torch.Tensor], lora_scale: float = 1.0):
        self.t = t
        self.quantized = "Wg_q" in t
        if self.quantized:
            d_ff, half = t["Wg_q"].shape
            d_model = 2 * half
        else:
            d_ff, d_model = t["Wg"].shape
        r = t["Ag"].shape[0]
        self.c = SlFfnWeights(d_model, d_ff, r, float(lora_scale),
                              *[_ptr(t[n]) if n in t else None for n in self.NAMES + self.QNAMES])
        self.d_model, self.d_ff, self.r = d_model, d_ff, r
        self.dtype = _dtype_code(t["Ag"])

    @property
    def ref(self):
        return ctypes.byref(self.c)


class FFNWorkspace:
    """Reusable saved + scratch buffers for one (layout, shape, k)."""

    def __init__(self, w: FFNWeights, layout: Layout, k: int, device):
        L = lib()
        self.saved = _bytes_tensor(L.sl_ffn_saved_bytes(w.dtype, layout.ref, w.d_model, w.d_ff, w.r, k),
                                   device)
        self.ws = _bytes_tensor(L.sl_ffn_workspace_bytes(w.dtype, layout.ref, w.d_model, w.d_ff, w.r, k),
                                device)


def ffn_fwd(w: FFNWeights, X: torch.Tensor, layout: Layout, k: int, idx: torch.Tensor,
            buf: Optional[FFNWorkspace] = None, Y: Optional[torch.Tensor] = None):
    L = lib()
    buf = buf or FFNWorkspace(w, layout, k, X.device)
    Y = Y if Y is not None else torch.empty_like(X)
    _check(L.sl_ffn_fwd(w.dtype, layout.ref, w.ref, _ptr(X), k, _ptr(idx), _ptr(Y),
                        _ptr(buf.saved), buf.saved.numel(), _ptr(buf.ws), buf.ws.numel(), _stream()),
           "sl_ffn_fwd")
    return Y, buf


def ffn_bwd(w: FFNWeights, X: torch.Tensor, layout: Layout, k: int, idx: torch.Tensor,
            buf: FFNWorkspace, dY: torch.Tensor, out: Optional[Dict[str, torch.Tensor]] = None):
    L = lib()
    dev = X.device
    if out is None:
        out = {"dX": torch.empty_like(X)}
        for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"):
            out["d" + n] = torch.empty(w.t[n].shape, dtype=torch.float32, device=dev)
    g = SlFfnGrads(*[_ptr(out[n]) for n in ("dAg", "dBg", "dAu", "dBu", "dAd", "dBd")])
    _check(L.sl_ffn_bwd(w.dtype, layout.ref, w.ref, _ptr(X), k, _ptr(idx), _ptr(buf.saved),
                        buf.saved.numel(), _ptr(dY), _ptr(out["dX"]), ctypes.byref(g), _ptr(buf.ws),
                        buf.ws.numel(), _stream()),
           "sl_ffn_bwd")
    return out


class QKVOWeights:
    """Device tensors of one attention block's projections.  A 4-bit frozen
    base replaces Wq, Wk, Wv by Wq_q, Wk_q, Wv_q with Wq_s, Wk_s, Wv_s, and WoT
    by WoT_q with WoT_s (the format of FFNWeights' quantized base)."""

    NAMES = ("Wq", "Wk", "Wv", "WoT", "Aq", "Bq", "Ak", "Bk", "Av", "Bv", "Ao", "Bo")
    QNAMES = ("Wq_q", "Wk_q", "Wv_q", "WoT_q", "Wq_s", "Wk_s", "Wv_s", "WoT_s")

    def __init__(self, t: Dict[str, torch.Tensor], heads: Sequence[int], lora_scale: float = 1.0):
        self.t = t
        self.heads = tuple(int(h) for h in heads)
        d_model = t["Aq"].shape[1]
        r = t["Aq"].shape[0]
        self.c = SlQkvoWeights(d_model, SlHeads(*self.heads), r, float(lora_scale),
                               *[_ptr(t[n]) if n in t else None for n in self.NAMES + self.QNAMES])
        self.d_model, self.r = d_model, r
        self.dtype = _dtype_code(t["Aq"])

    @property
    def ref(self):
        return ctypes.byref(self.c)


class QKVOWorkspace:
    def __init__(self, w: QKVOWeights, layout: Layout, k_qk: int, k_vo: int, device):
        L = lib()
        self.saved = _bytes_tensor(L.sl_qkvo_saved_bytes(w.dtype, layout.ref, w.ref), device)
        self.ws = _bytes_tensor(L.sl_qkvo_workspace_bytes(w.dtype, layout.ref, w.ref, k_qk, k_vo),
                                device)


def qkvo_fwd(w: QKVOWeights, X: Optional[torch.Tensor], a: Optional[torch.Tensor], layout: Layout,
             k_qk: int, idx_qk: torch.Tensor, k_vo: int, idx_vo: torch.Tensor,
             buf: Optional[QKVOWorkspace] = None, outs: Optional[Dict[str, torch.Tensor]] = None):
    L = lib()
    ref = X if X is not None else a
    dev = ref.device
    hq, hkv, hd = w.heads
    T = layout.batch * layout.seq_len
    buf = buf or QKVOWorkspace(w, layout, k_qk, k_vo, dev)
    outs = dict(outs or {})
    if X is not None:
        outs.setdefault("q", torch.empty(T, hq * hd, dtype=ref.dtype, device=dev))
        outs.setdefault("k", torch.empty(T, hkv * hd, dtype=ref.dtype, device=dev))
        outs.setdefault("v", torch.empty(T, hkv * hd, dtype=ref.dtype, device=dev))
    if a is not None:
        outs.setdefault("o", torch.empty(T, w.d_model, dtype=ref.dtype, device=dev))
    _check(L.sl_qkvo_fwd(w.dtype, layout.ref, w.ref, _ptr(X), _ptr(a), k_qk, _ptr(idx_qk), k_vo,
                         _ptr(idx_vo), _ptr(outs.get("q")), _ptr(outs.get("k")), _ptr(outs.get("v")),
                         _ptr(outs.get("o")), _ptr(buf.saved), buf.saved.numel(), _ptr(buf.ws),
                         buf.ws.numel(), _stream()),
           "sl_qkvo_fwd")
    return outs, buf


def qkvo_bwd(w: QKVOWeights, X: Optional[torch.Tensor], a: Optional[torch.Tensor], layout: Layout,
             k_qk: int, idx_qk: torch.Tensor, k_vo: int, idx_vo: torch.Tensor, buf: QKVOWorkspace,
             dq=None, dk=None, dv=None, d_out=None, out: Optional[Dict[str, torch.Tensor]] = None):
    L = lib()
    ref = X if X is not None else a
    dev = ref.device
    out = dict(out or {})
    if dq is not None:
        out.setdefault("dX", torch.empty_like(X))
        for n in ("Aq", "Bq", "Ak", "Bk", "Av", "Bv"):
            out.setdefault("d" + n, torch.empty(w.t[n].shape, dtype=torch.float32, device=dev))
    if d_out is not None:
        out.setdefault("da", torch.empty_like(a))
        for n in ("Ao", "Bo"):
            out.setdefault("d" + n, torch.empty(w.t[n].shape, dtype=torch.float32, device=dev))
    g = SlQkvoGrads(*[_ptr(out.get(n)) for n in ("dAq", "dBq", "dAk", "dBk", "dAv", "dBv", "dAo",
                                                  "dBo")])
    _check(L.sl_qkvo_bwd(w.dtype, layout.ref, w.ref, _ptr(X), _ptr(a), k_qk, _ptr(idx_qk), k_vo,
                         _ptr(idx_vo), _ptr(buf.saved), buf.saved.numel(), _ptr(dq), _ptr(dk),
                         _ptr(dv), _ptr(d_out), _ptr(out.get("dX")), _ptr(out.get("da")),
                         ctypes.byref(g), _ptr(buf.ws), buf.ws.numel(), _stream()),
           "sl_qkvo_bwd")
    return out
