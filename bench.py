#!/usr/bin/env python3
"""Sparse LoRA FFN forward + backward at the LLaMA2-7B FFN shape on one MI355X.

One step is the whole hot path of one FFN layer over one batch: estimate and
score channels over each sequence's context tokens, select the top-k per
sequence, then the sparse LoRA forward and backward (output tokens dense).
Prints one JSON line with tokens/s, the roofline of the dominant kernel
(timed live with HIP events on the library's stream), the speedup over the
same kernels run dense, and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0
METRIC = "sparse LoRA FFN fwd+bwd tokens/s @7B shape; MFMA util; speedup vs dense"


def kernel_work(D, F, r, r_e, ctx, L, k):
    """Algorithmic FLOPs (GEMM kernels) and bytes (estimator, select) per launch."""
    B = len(ctx)
    T = B * L
    T_c = int(sum(ctx))
    T_o = T - T_c
    R = T_c * k + T_o * F          # row-channel pairs computed
    fl = {
        "gu_fwd": 4 * D * R + 4 * r * R,              # gate+up base + LoRA-B products
        "down_fwd": 2 * D * R + 2 * r * T * D,
        "dh_bwd": 2 * D * R + 2 * r * R,
        "dx_bwd": 4 * D * R + 4 * r * T * D,
    }
    nchunk = -(-max(ctx) // 64)
    by = {
        # X context rows + both factor pairs + score partials written
        "estimate": T_c * D * 2 + 2 * r_e * (D + F) * 2 + B * nchunk * F * 4,
        # partials read + indices written
        "select": B * nchunk * F * 4 + B * k * 4,
    }
    return fl, by, R


def measured_traffic(kernel):
    """HBM bytes per launch of a gather-GEMM from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when the GEMM source has changed
    since the counters were taken."""
    import hashlib
    summ = os.path.join(ROOT, "profiles", "gather_gemm_llama2-7b-ffn_hbm_traffic.md")
    src = os.path.join(ROOT, "contextual_sparsity_lora_svd_amd", "csrc", "sl_gemm.hpp")
    if not (os.path.exists(summ) and os.path.exists(src)):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    vals, ok = {}, False
    for line in open(summ):
        line = line.strip()
        if line.startswith("gemm_source_sha256:"):
            ok = line.split(":", 1)[1].strip() == sha
        elif line.startswith("traffic_bytes "):
            name, v = line[len("traffic_bytes "):].split(":")
            vals[name.strip()] = float(v)
    return vals.get(kernel) if ok else None


def to_dev(x, torch, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype).contiguous()


def cpu_baseline(p, ctx, L, Pt_g, Q_g, Pt_u, Q_u, k, budget_s):
    """The oracle as it stands on the host cores, on the first sequences of
    the same batch (as many as fit the budget)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()

    def run(nseq):
        rows = nseq * L
        sub = {n: (v[:rows] if n in ("X", "dY") else v) for n, v in p.items()}
        t0 = time.perf_counter()
        _, idx = O.estimate_select_ffn(sub["X"], ctx[:nseq], L, Pt_g.T, Q_g, Pt_u.T, Q_u, k)
        y, cache = O.ffn_forward(sub, ctx[:nseq], L, list(idx))
        O.ffn_backward(sub, cache, sub["dY"])
        return time.perf_counter() - t0

    t1 = run(1)
    nseq = int(max(1, min(len(ctx), budget_s // max(t1, 1e-3))))
    t = run(nseq) if nseq > 1 else t1
    env = {n: os.environ.get(n) for n in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    return {"value": nseq * L / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "host_cpus": os.cpu_count(), "blas_threads": int(threads),
            "thread_env": {n: v for n, v in env.items() if v is not None},
            "precision": "scores fp32 (they decide the selected set); forward and backward fp64",
            "sample": f"{nseq} of {len(ctx)} sequences ({nseq * L} tokens), estimate+select+fwd+bwd "
                      f"in numpy (scores fp32, fwd/bwd fp64, so the rate is an fp64-BLAS rate), "
                      f"one run of {t:.2f} s; cores = the BLAS threads numpy used"}


def attn_flops(D, nq, nkv, G, r, ctx, L, kqk, kvo):
    """Algorithmic FLOPs of q/k/v/o forward + backward (base and LoRA)."""
    def R(kc, n):
        return sum(c * kc + (L - c) * n for c in ctx)
    T = len(ctx) * L
    Rq, Rk, Rv, Ro = R(kqk * G, nq), R(kqk, nkv), R(kvo, nkv), R(kvo * G, nq)
    Rs = Rq + Rk + Rv + Ro
    return 4 * D * Rs + 3 * (8 * T * D * r + 2 * r * Rs)


def ffn_flops(D, F, r, ctx, L, k):
    """Algorithmic FLOPs of FFN forward + backward (base and LoRA)."""
    R = sum(c * k + (L - c) * F for c in ctx)
    T = len(ctx) * L
    return 12 * D * R + 18 * r * (T * D + R)


def ffn_extreme_bench(args, torch, sl, cfg=6):
    """FFN rows of the path in the extreme-sparsity regime (99 % of d_ff
    dropped, LLaMA2-7B shape): estimate, select, forward and backward, against
    the same kernels run dense."""
    wl = W.WORKLOADS[cfg]
    f = wl.ffn[0]
    D, F, r, r_e, L = f.d_model, f.d_ff, f.lora_rank, wl.est_rank, wl.seq_len
    ctx = [int(c) for c in W.ctx_lengths(wl)]
    B, T = len(ctx), len(ctx) * L
    k = sl.k_from_ratio(F, f.sparsity_pct)
    print(f"[bench] {wl.name} FFN: D={D} F={F} r={r} B={B} L={L} ctx={ctx} k={k}", file=sys.stderr, flush=True)
    p = W.make_ffn_tensors(wl)
    bf = torch.bfloat16
    t = {n: to_dev(p[n], torch, bf) for n in ("Wg", "Wu", "Ag", "Bg", "Au", "Bu", "Ad", "Bd")}
    t["WdT"] = to_dev(np.ascontiguousarray(p["Wd"].T), torch, bf)
    X, dY = to_dev(p["X"], torch, bf), to_dev(p["dY"], torch, bf)
    del p
    w = sl.FFNWeights(t, lora_scale=1.0)
    lay = sl.Layout(ctx, L)
    Ptg, Qg, _ = sl.build_estimator(t["Wg"], r_e)
    Ptu, Qu, _ = sl.build_estimator(t["Wu"], r_e)
    est = sl.EstimateBuffers(sl.SL_CRIT_SWIGLU_L2, lay, D, r_e, F, k, X.device)
    Y = torch.empty_like(X)
    grads = {"dX": torch.empty_like(X)}
    for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"):
        grads["d" + n] = torch.empty(t[n].shape, dtype=torch.float32, device=X.device)

    def run(kk, buf, idx=None):
        if idx is None:
            idx, _ = sl.estimate_select(sl.SL_CRIT_SWIGLU_L2, X, lay, r_e, Ptg, Qg, Ptu, Qu, F, kk, bufs=est)
        sl.ffn_fwd(w, X, lay, kk, idx, buf, Y=Y)
        sl.ffn_bwd(w, X, lay, kk, idx, buf, dY, out=grads)

    buf = sl.FFNWorkspace(w, lay, k, X.device)
    ms = timed(torch, lambda: run(k, buf), args.steps, args.warmup)
    full = torch.arange(F, dtype=torch.int32, device=X.device).repeat(B, 1).contiguous()
    bufd = sl.FFNWorkspace(w, lay, F, X.device)
    dense_ms = timed(torch, lambda: run(F, bufd, full), max(3, args.steps // 2), 2) if not args.no_dense else None
    fl = ffn_flops(D, F, r, ctx, L, k)
    print(f"[bench] extreme FFN step {ms:.3f} ms" + (f", dense {dense_ms:.3f} ms" if dense_ms else ""),
          file=sys.stderr, flush=True)
    return {"workload": wl.name, "batch": B, "seq_len": L, "ctx_len": ctx, "sparsity_pct": f.sparsity_pct,
            "k": k, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "effective_tflops": fl / (ms * 1e-3) / 1e12, "algorithmic_gflop": fl / 1e9,
            "dense_ms_per_step": dense_ms, "speedup_vs_dense": (dense_ms / ms) if dense_ms else None}


def qlora_bench(args, torch, sl, cfg=2):
    """The FFN rows over a 4-bit quantized frozen base (SparseLoRA article §六:
    SparseLoRA combined with a QLoRA-style base): the frozen weights are
    quantized on the GPU (sl_quantize_q4), then estimate, select, forward and
    backward run from the codes, against the same kernels run dense over the
    same quantized base (k = d_ff, no estimator)."""
    wl = W.WORKLOADS[cfg]
    f = wl.ffn[0]
    D, F, r, r_e, L = f.d_model, f.d_ff, f.lora_rank, wl.est_rank, wl.seq_len
    ctx = [int(c) for c in W.ctx_lengths(wl)]
    B, T = len(ctx), len(ctx) * L
    k = sl.k_from_ratio(F, f.sparsity_pct)
    p = W.make_ffn_tensors(wl)
    bf = torch.bfloat16
    t = {n: to_dev(p[n], torch, bf) for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")}
    X, dY = to_dev(p["X"], torch, bf), to_dev(p["dY"], torch, bf)
    base = {"Wg": to_dev(p["Wg"], torch, bf), "Wu": to_dev(p["Wu"], torch, bf),
            "WdT": to_dev(np.ascontiguousarray(p["Wd"].T), torch, bf)}
    del p
    for n, w0 in base.items():
        t[n + "_q"], t[n + "_s"] = sl.quantize_q4(w0)
    # the estimator factors of the frozen base the layer computes with
    deq = lambda n: (sl_dequant(torch, t[n + "_q"], t[n + "_s"])).to(bf)
    Ptg, Qg, _ = sl.build_estimator(deq("Wg"), r_e)
    Ptu, Qu, _ = sl.build_estimator(deq("Wu"), r_e)
    del base
    torch.cuda.empty_cache()
    w = sl.FFNWeights(t, lora_scale=1.0)
    lay = sl.Layout(ctx, L)
    est = sl.EstimateBuffers(sl.SL_CRIT_SWIGLU_L2, lay, D, r_e, F, k, X.device)
    Y = torch.empty_like(X)
    grads = {"dX": torch.empty_like(X)}
    for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"):
        grads["d" + n] = torch.empty(t[n].shape, dtype=torch.float32, device=X.device)

    def run(kk, buf, idx=None):
        if idx is None:
            idx, _ = sl.estimate_select(sl.SL_CRIT_SWIGLU_L2, X, lay, r_e, Ptg, Qg, Ptu, Qu, F, kk, bufs=est)
        sl.ffn_fwd(w, X, lay, kk, idx, buf, Y=Y)
        sl.ffn_bwd(w, X, lay, kk, idx, buf, dY, out=grads)

    buf = sl.FFNWorkspace(w, lay, k, X.device)
    ms = timed(torch, lambda: run(k, buf), args.steps, args.warmup)
    full = torch.arange(F, dtype=torch.int32, device=X.device).repeat(B, 1).contiguous()
    bufd = sl.FFNWorkspace(w, lay, F, X.device)
    dense_ms = timed(torch, lambda: run(F, bufd, full), max(3, args.steps // 2), 2) if not args.no_dense else None
    fl = ffn_flops(D, F, r, ctx, L, k)
    weight_bytes = sum(t[n].numel() * t[n].element_size() for n in ("Wg_q", "Wu_q", "WdT_q", "Wg_s", "Wu_s", "WdT_s"))
    print(f"[bench] 4-bit base FFN step {ms:.3f} ms" + (f", dense {dense_ms:.3f} ms" if dense_ms else ""),
          file=sys.stderr, flush=True)
    del t, w, buf, bufd, est, X, dY, Y, grads
    torch.cuda.empty_cache()
    attn = None if args.no_attn else attn_bench(args, torch, sl, quant=True)
    return {"workload": wl.name, "base": "int4, one fp32 scale per 64-element row block",
            "frozen_weight_bytes": weight_bytes, "bf16_weight_bytes": 3 * F * D * 2,
            "batch": B, "seq_len": L, "ctx_len": ctx, "sparsity_pct": f.sparsity_pct, "k": k,
            "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "effective_tflops": fl / (ms * 1e-3) / 1e12, "algorithmic_gflop": fl / 1e9,
            "dense_ms_per_step": dense_ms, "speedup_vs_dense": (dense_ms / ms) if dense_ms else None,
            "attention": attn}


def sl_dequant(torch, codes, scales):
    """code * scale of packed 4-bit codes (torch ops; used only to build the
    estimator factors of the quantized base offline)."""
    lo = (codes & 0xF).to(torch.int16)
    hi = (codes >> 4).to(torch.int16)
    q = torch.stack((lo, hi), dim=2).reshape(codes.shape[0], -1)
    q = torch.where(q >= 8, q - 16, q).float()
    return q * scales.repeat_interleave(64, dim=1)


def attn_bench(args, torch, sl, cfg=3, quant=False):
    """q/k/v/o rows of the path on a LLaMA2-7B attention workload: QK-norm and
    L2 selection over context tokens, sparse q/k/v/o forward and backward
    (quant: over 4-bit frozen bases quantized on the GPU)."""
    wl = W.WORKLOADS[cfg]
    s = wl.attn[0]
    heads = (s.n_q_heads, s.n_kv_heads, s.head_dim)
    D, r, r_e, L = s.d_model, s.lora_rank, wl.est_rank, wl.seq_len
    nq, nkv = heads[0] * heads[2], heads[1] * heads[2]
    G = heads[0] // heads[1]
    ctx = [int(c) for c in W.ctx_lengths(wl)]
    B = len(ctx)
    T = B * L
    kqk, kvo = sl.k_from_ratio(nkv, s.sparsity_qk_pct), sl.k_from_ratio(nkv, s.sparsity_vo_pct)
    print(f"[bench] {wl.name}: D={D} heads={heads} r={r} B={B} L={L} ctx={ctx} k_qk={kqk} k_vo={kvo}",
          file=sys.stderr, flush=True)
    p = W.make_attn_tensors(wl)
    bf = torch.bfloat16
    t = {n: to_dev(p[n], torch, bf) for n in ("Wq", "Wk", "Wv", "Aq", "Bq", "Ak", "Bk", "Av", "Bv", "Ao", "Bo")}
    t["WoT"] = to_dev(np.ascontiguousarray(p["Wo"].T), torch, bf)
    X, a = to_dev(p["X"], torch, bf), to_dev(p["a"], torch, bf)
    dq, dk, dv, dout = (to_dev(p[n], torch, bf) for n in ("dq", "dk", "dv", "d_out"))
    del p
    if quant:
        for n in ("Wq", "Wk", "Wv", "WoT"):
            t[n + "_q"], t[n + "_s"] = sl.quantize_q4(t[n])
            # the estimator factors of the base the layer computes with
            t[n] = sl_dequant(torch, t[n + "_q"], t[n + "_s"]).to(bf)
    lay = sl.Layout(ctx, L)
    f = {n: sl.build_estimator(t[n], r_e) for n in ("Wq", "Wk", "Wv")}
    if quant:
        for n in ("Wq", "Wk", "Wv", "WoT"):
            del t[n]
        torch.cuda.empty_cache()
    w = sl.QKVOWeights(t, heads)
    torch.cuda.synchronize()
    # q/k by the QK-norm and v/o by the L2 criterion, one estimate call over X
    jobs = [dict(crit=sl.SL_CRIT_QK_NORM, Pt0=f["Wq"][0], Q0=f["Wq"][1], Pt1=f["Wk"][0], Q1=f["Wk"][1], N=nkv,
                 k=kqk, heads=heads),
            dict(crit=sl.SL_CRIT_L2, Pt0=f["Wv"][0], Q0=f["Wv"][1], N=nkv, k=kvo)]
    est = sl.EstimateMultiBuffers(lay, D, r_e, jobs, X.device)
    buf = sl.QKVOWorkspace(w, lay, kqk, kvo, X.device)
    outs, grads = {}, {}

    def step():
        (iqk, _), (ivo, _) = sl.estimate_select_multi(X, lay, r_e, jobs, bufs=est)
        o, _ = sl.qkvo_fwd(w, X, a, lay, kqk, iqk, kvo, ivo, buf=buf, outs=outs)
        outs.update(o)
        g = sl.qkvo_bwd(w, X, a, lay, kqk, iqk, kvo, ivo, buf, dq=dq, dk=dk, dv=dv, d_out=dout, out=grads)
        grads.update(g)

    ms = timed(torch, step, args.steps, args.warmup)
    full = torch.arange(nkv, dtype=torch.int32, device=X.device).repeat(B, 1).contiguous()
    bufd = sl.QKVOWorkspace(w, lay, nkv, nkv, X.device)
    outs_d, grads_d = {}, {}

    def step_dense():
        o, _ = sl.qkvo_fwd(w, X, a, lay, nkv, full, nkv, full, buf=bufd, outs=outs_d)
        outs_d.update(o)
        g = sl.qkvo_bwd(w, X, a, lay, nkv, full, nkv, full, bufd, dq=dq, dk=dk, dv=dv, d_out=dout, out=grads_d)
        grads_d.update(g)

    dense_ms = timed(torch, step_dense, max(3, args.steps // 2), 2) if not args.no_dense else None
    fl = attn_flops(D, nq, nkv, G, r, ctx, L, kqk, kvo)
    print(f"[bench] attention step {ms:.3f} ms" + (f", dense {dense_ms:.3f} ms" if dense_ms else ""),
          file=sys.stderr, flush=True)
    return {"workload": wl.name, "batch": B, "seq_len": L, "ctx_len": ctx, "heads": list(heads),
            "k_qk": kqk, "k_vo": kvo, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "effective_tflops": fl / (ms * 1e-3) / 1e12, "algorithmic_gflop": fl / 1e9,
            "dense_ms_per_step": dense_ms, "speedup_vs_dense": (dense_ms / ms) if dense_ms else None}


def workload_bench(args, torch, sl, cfg):
    """Every layer of a workload (FFN and q/k/v/o rows where the workload has
    them): estimate + select where a layer is sparse (a layer at 0 % keeps
    every channel and needs no estimate), forward and backward, against the
    same kernels run dense (k = N, no estimator).  Reports tokens/s, effective
    TFLOP/s, the per-kernel breakdown with the dominant kernel's roofline, and
    the estimator's share of time and FLOPs."""
    wl = W.WORKLOADS[cfg]
    fp32 = wl.dtype == "f32"
    tdt = torch.float32 if fp32 else torch.bfloat16
    peak = PEAK_F32_TFLOPS if fp32 else PEAK_BF16_TFLOPS
    L, r_e = wl.seq_len, wl.est_rank
    ctx = [int(c) for c in W.ctx_lengths(wl)]
    B, T = len(ctx), len(ctx) * L
    Tc = sum(ctx)
    nlay = max(len(wl.ffn), len(wl.attn))
    print(f"[bench] {wl.name}: {nlay} layer(s), B={B} L={L} ctx={ctx}", file=sys.stderr, flush=True)
    dev = torch.device("cuda")
    lay = sl.Layout(ctx, L)
    sparse_steps, dense_steps = [], []
    kfl = {}                       # timer slot -> algorithmic FLOPs over all layers of one step
    est_fl = 0.0
    total_fl = 0.0
    dense_fl = 0.0
    desc = []

    def add(slot, v):
        kfl[slot] = kfl.get(slot, 0.0) + v

    def rows(kc, n):
        return sum(c * kc + (L - c) * n for c in ctx)

    for li in range(nlay):
        if li < len(wl.ffn):
            f = wl.ffn[li]
            D, F, r = f.d_model, f.d_ff, f.lora_rank
            k = sl.k_from_ratio(F, f.sparsity_pct)
            p = W.make_ffn_tensors(wl, li)
            t = {n: to_dev(p[n], torch, tdt) for n in ("Wg", "Wu", "Ag", "Bg", "Au", "Bu", "Ad", "Bd")}
            t["WdT"] = to_dev(np.ascontiguousarray(p["Wd"].T), torch, tdt)
            X, dY = to_dev(p["X"], torch, tdt), to_dev(p["dY"], torch, tdt)
            del p
            w = sl.FFNWeights(t, lora_scale=1.0)
            full = torch.arange(F, dtype=torch.int32, device=dev).repeat(B, 1).contiguous()
            grads = {"dX": torch.empty_like(X)}
            for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"):
                grads["d" + n] = torch.empty(t[n].shape, dtype=torch.float32, device=dev)
            Y = torch.empty_like(X)
            buf = sl.FFNWorkspace(w, lay, k, dev)
            bufd = sl.FFNWorkspace(w, lay, F, dev) if k < F else buf
            if k < F:
                Ptg, Qg, _ = sl.build_estimator(t["Wg"], r_e)
                Ptu, Qu, _ = sl.build_estimator(t["Wu"], r_e)
                est = sl.EstimateBuffers(sl.SL_CRIT_SWIGLU_L2, lay, D, r_e, F, k, dev)
                est_fl += 2 * Tc * D * 2 * r_e + 2 * Tc * r_e * 2 * F

                def s_ffn(X=X, dY=dY, w=w, buf=buf, Y=Y, grads=grads, k=k, F=F, est=est,
                          fac=(Ptg, Qg, Ptu, Qu)):
                    idx, _ = sl.estimate_select(sl.SL_CRIT_SWIGLU_L2, X, lay, r_e, *fac, F, k, bufs=est)
                    sl.ffn_fwd(w, X, lay, k, idx, buf, Y=Y)
                    sl.ffn_bwd(w, X, lay, k, idx, buf, dY, out=grads)
            else:
                def s_ffn(X=X, dY=dY, w=w, buf=buf, Y=Y, grads=grads, F=F, full=full):
                    sl.ffn_fwd(w, X, lay, F, full, buf, Y=Y)
                    sl.ffn_bwd(w, X, lay, F, full, buf, dY, out=grads)

            def d_ffn(X=X, dY=dY, w=w, buf=bufd, Y=Y, grads=grads, F=F, full=full):
                sl.ffn_fwd(w, X, lay, F, full, buf, Y=Y)
                sl.ffn_bwd(w, X, lay, F, full, buf, dY, out=grads)
            sparse_steps.append(s_ffn)
            dense_steps.append(d_ffn)
            R = rows(k, F)
            add("gu_fwd", 4 * D * R + 4 * r * R)
            add("down_fwd", 2 * D * R + 2 * r * T * D)
            add("dh_bwd", 2 * D * R + 2 * r * R)
            add("dx_bwd", 4 * D * R + 4 * r * T * D)
            total_fl += ffn_flops(D, F, r, ctx, L, k)
            dense_fl += ffn_flops(D, F, r, ctx, L, F)
            desc.append(f"layer {li} FFN d_ff {F} k {k}")
        if li < len(wl.attn):
            a_ = wl.attn[li]
            heads = (a_.n_q_heads, a_.n_kv_heads, a_.head_dim)
            D, r = a_.d_model, a_.lora_rank
            nq, nkv = heads[0] * heads[2], heads[1] * heads[2]
            G = heads[0] // heads[1]
            kqk = sl.k_from_ratio(nkv, a_.sparsity_qk_pct)
            kvo = sl.k_from_ratio(nkv, a_.sparsity_vo_pct)
            p = W.make_attn_tensors(wl, li)
            t = {n: to_dev(p[n], torch, tdt) for n in ("Wq", "Wk", "Wv", "Aq", "Bq", "Ak", "Bk", "Av", "Bv",
                                                       "Ao", "Bo")}
            t["WoT"] = to_dev(np.ascontiguousarray(p["Wo"].T), torch, tdt)
            X, a = to_dev(p["X"], torch, tdt), to_dev(p["a"], torch, tdt)
            gin = {n: to_dev(p[n], torch, tdt) for n in ("dq", "dk", "dv", "d_out")}
            del p
            w = sl.QKVOWeights(t, heads)
            full = torch.arange(nkv, dtype=torch.int32, device=dev).repeat(B, 1).contiguous()
            jobs = []
            if kqk < nkv:
                fq, fk = sl.build_estimator(t["Wq"], r_e), sl.build_estimator(t["Wk"], r_e)
                jobs.append(dict(crit=sl.SL_CRIT_QK_NORM, Pt0=fq[0], Q0=fq[1], Pt1=fk[0], Q1=fk[1], N=nkv,
                                 k=kqk, heads=heads))
                est_fl += 2 * Tc * D * 2 * r_e + 2 * Tc * r_e * (nq + nkv)
            if kvo < nkv:
                fv = sl.build_estimator(t["Wv"], r_e)
                jobs.append(dict(crit=sl.SL_CRIT_L2, Pt0=fv[0], Q0=fv[1], N=nkv, k=kvo))
                est_fl += 2 * Tc * D * r_e + 2 * Tc * r_e * nkv
            est = sl.EstimateMultiBuffers(lay, D, r_e, jobs, dev) if jobs else None
            buf = sl.QKVOWorkspace(w, lay, kqk, kvo, dev)
            bufd = sl.QKVOWorkspace(w, lay, nkv, nkv, dev)
            outs, grads = {}, {}

            def s_att(X=X, a=a, w=w, buf=buf, gin=gin, jobs=jobs, est=est, kqk=kqk, kvo=kvo, full=full,
                      outs=outs, grads=grads, nkv=nkv):
                res = sl.estimate_select_multi(X, lay, r_e, jobs, bufs=est) if jobs else []
                it = iter(res)
                iqk = next(it)[0] if kqk < nkv else full
                ivo = next(it)[0] if kvo < nkv else full
                o, _ = sl.qkvo_fwd(w, X, a, lay, kqk, iqk, kvo, ivo, buf=buf, outs=outs)
                outs.update(o)
                g = sl.qkvo_bwd(w, X, a, lay, kqk, iqk, kvo, ivo, buf, out=grads, **gin)
                grads.update(g)

            def d_att(X=X, a=a, w=w, buf=bufd, gin=gin, full=full, outs=outs, grads=grads, nkv=nkv):
                o, _ = sl.qkvo_fwd(w, X, a, lay, nkv, full, nkv, full, buf=buf, outs=outs)
                outs.update(o)
                g = sl.qkvo_bwd(w, X, a, lay, nkv, full, nkv, full, buf, out=grads, **gin)
                grads.update(g)
            sparse_steps.append(s_att)
            dense_steps.append(d_att)
            Rq, Rk, Rv, Ro = rows(kqk * G, nq), rows(kqk, nkv), rows(kvo, nkv), rows(kvo * G, nq)
            add("qkv_fwd", 2 * D * (Rq + Rk + Rv) + 2 * r * (Rq + Rk + Rv))
            add("o_fwd", 2 * D * Ro + 2 * r * T * D)
            add("da_bwd", 2 * D * Ro + 2 * r * Ro)
            add("dxqkv_bwd", 2 * D * (Rq + Rk + Rv) + 6 * r * T * D)
            total_fl += attn_flops(D, nq, nkv, G, r, ctx, L, kqk, kvo)
            dense_fl += attn_flops(D, nq, nkv, G, r, ctx, L, nkv, nkv)
            desc.append(f"layer {li} q/k/v/o heads {list(heads)} k_qk {kqk} k_vo {kvo}")
    torch.cuda.synchronize()

    def step():
        for fn in sparse_steps:
            fn()

    def step_dense():
        for fn in dense_steps:
            fn()

    # per-kernel breakdown (events around every main kernel), then the timed region
    sl.timer_enable(64 * nlay * (args.steps + 1))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sl.timer_reset()
    timed(torch, step, args.steps, 0)
    kern = {}
    for name in TIMER_NAMES:
        tot, n = sl.timer_read(name)
        if n:
            kern[name] = {"ms_per_step": tot / args.steps, "launches_per_step": n / args.steps,
                          "avg_launch_ms": tot / n}
    sl.timer_enable(0)
    ms = timed(torch, step, args.steps, 0)
    dense_ms = timed(torch, step_dense, max(3, args.steps // 2), 2) if not args.no_dense else None
    for name, v in kern.items():
        if name in kfl:
            v["tflops"] = kfl[name] / (v["ms_per_step"] * 1e-3) / 1e12
            v["mfma_frac"] = v["tflops"] / peak
    gem = [n for n in kern if n in kfl]
    dom = max(gem, key=lambda n: kern[n]["ms_per_step"]) if gem else None
    est_ms = sum(kern.get(n, {}).get("ms_per_step", 0.0) for n in ("estimate", "select"))
    print(f"[bench] {wl.name} step {ms:.3f} ms" + (f", dense {dense_ms:.3f} ms" if dense_ms else ""),
          file=sys.stderr, flush=True)
    out = {"workload": wl.name, "dtype": "f32" if fp32 else "bf16", "layers": desc, "batch": B,
           "seq_len": L, "ctx_len": ctx, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
           "effective_tflops": total_fl / (ms * 1e-3) / 1e12, "algorithmic_gflop": total_fl / 1e9,
           "dense_algorithmic_gflop": dense_fl / 1e9,
           "dense_ms_per_step": dense_ms, "speedup_vs_dense": (dense_ms / ms) if dense_ms else None,
           "estimator_share": {"time": est_ms / ms, "flops": est_fl / total_fl},
           "kernels": kern}
    if dom:
        fl_launch = kfl[dom] / kern[dom]["launches_per_step"]
        ach = fl_launch / (kern[dom]["avg_launch_ms"] * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                           "frac": ach / peak, "avg_launch_ms": kern[dom]["avg_launch_ms"],
                           "flops_per_launch": fl_launch}
    del sparse_steps, dense_steps
    torch.cuda.empty_cache()
    return out


TIMER_NAMES = ("estimate", "select", "gu_fwd", "down_fwd", "dh_bwd", "dx_bwd", "qkv_fwd", "o_fwd", "da_bwd",
               "dxqkv_bwd")


def timed(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-dense", action="store_true", help="skip the dense comparison")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--no-attn", action="store_true", help="skip the q/k/v/o workload")
    ap.add_argument("--no-extreme", action="store_true",
                    help="skip the extreme-sparsity workload (99 %% FFN, 75 %% q/k/v/o)")
    ap.add_argument("--no-qlora", action="store_true",
                    help="skip the FFN over a 4-bit quantized frozen base")
    ap.add_argument("--gemm-variants", type=int, default=-1,
                    help="GEMM tile variants to allow (bit mask: 1 wide N-gather, 2 tall 256 x 256, 4 tall always; "
                         "default: the library's)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the tiny fp32 FFN, 4-layer stack and LLaMA3-8B long-context workloads")
    ap.add_argument("--workload", type=int, default=0,
                    help="run only workload N's whole-path measurement and print it as the JSON line "
                         "(for profiling)")
    ap.add_argument("--extreme-ffn-only", action="store_true",
                    help="run only the 99 %% sparsity FFN step and print its measurements as the JSON line "
                         "(for profiling that step alone)")
    ap.add_argument("--attn-only", action="store_true",
                    help="run only the q/k/v/o workload and print its measurements as the JSON line "
                         "(for profiling that step alone)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain bf16 -> fp32 copy of 64 Mi elements (128 MiB read, "
                         "256 MiB written) to calibrate HBM byte counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the benchmark measures one GPU; sharding by sequence across GPUs is a design "
              "note, not built. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import contextual_sparsity_lora_svd_amd as sl
    if args.gemm_variants >= 0:
        sl.gemm_config(args.gemm_variants)

    if args.extreme_ffn_only:
        print(json.dumps(ffn_extreme_bench(args, torch, sl)), flush=True)
        return
    if args.attn_only:
        print(json.dumps(attn_bench(args, torch, sl)), flush=True)
        return
    if args.workload:
        print(json.dumps(workload_bench(args, torch, sl, args.workload)), flush=True)
        return

    wl = W.WORKLOADS[2]
    f = wl.ffn[0]
    D, F, r, r_e, L = f.d_model, f.d_ff, f.lora_rank, wl.est_rank, wl.seq_len
    ctx = [int(c) for c in W.ctx_lengths(wl)]
    B = len(ctx)
    T = B * L
    k = sl.k_from_ratio(F, f.sparsity_pct)
    print(f"[bench] {wl.name}: D={D} F={F} r={r} B={B} L={L} ctx={ctx} k={k}", file=sys.stderr,
          flush=True)
    p = W.make_ffn_tensors(wl)
    bf = torch.bfloat16
    t = {n: to_dev(p[n], torch, bf) for n in ("Wg", "Wu", "Ag", "Bg", "Au", "Bu", "Ad", "Bd")}
    t["WdT"] = to_dev(np.ascontiguousarray(p["Wd"].T), torch, bf)
    X = to_dev(p["X"], torch, bf)
    dY = to_dev(p["dY"], torch, bf)
    w = sl.FFNWeights(t, lora_scale=1.0)
    lay = sl.Layout(ctx, L)

    # offline estimator (a0): outside the step; its one-time cost is reported
    torch.cuda.synchronize()
    t_b = time.perf_counter()
    Ptg, Qg, _ = sl.build_estimator(t["Wg"], r_e)
    Ptu, Qu, _ = sl.build_estimator(t["Wu"], r_e)
    torch.cuda.synchronize()
    build_ms = (time.perf_counter() - t_b) * 1e3 / 2

    buf = sl.FFNWorkspace(w, lay, k, X.device)
    est = sl.EstimateBuffers(sl.SL_CRIT_SWIGLU_L2, lay, D, r_e, F, k, X.device)
    Y = torch.empty_like(X)
    grads = {"dX": torch.empty_like(X)}
    for n in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd"):
        grads["d" + n] = torch.empty(t[n].shape, dtype=torch.float32, device=X.device)

    def step():
        idx, _ = sl.estimate_select(sl.SL_CRIT_SWIGLU_L2, X, lay, r_e, Ptg, Qg, Ptu, Qu, F, k, bufs=est)
        sl.ffn_fwd(w, X, lay, k, idx, buf, Y=Y)
        sl.ffn_bwd(w, X, lay, k, idx, buf, dY, out=grads)

    # Per-kernel breakdown (events around every main kernel; the events add
    # idle gaps, so this pass is not the headline time).
    names = ("estimate", "select", "gu_fwd", "down_fwd", "dh_bwd", "dx_bwd")
    sl.timer_enable(64 * (args.steps + 1))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sl.timer_reset()
    ms_all = timed(torch, step, args.steps, 0)
    kern = {}
    for name in names:
        tot, n = sl.timer_read(name)
        if n:
            kern[name] = {"avg_ms": tot / n, "launches": n, "share": tot / (ms_all * args.steps)}
    fl, by, R = kernel_work(D, F, r, r_e, ctx, L, k)
    dom = max((n for n in kern if n in fl), key=lambda n: kern[n]["avg_ms"] * kern[n]["launches"])

    # Timed region: the whole step, with HIP events on the library's stream
    # around the dominant kernel only.
    sl.timer_select([dom])
    sl.timer_reset()
    ms = timed(torch, step, args.steps, 0)
    tot, n = sl.timer_read(dom)
    dom_ms = tot / n
    sl.timer_enable(0)
    print(f"[bench] sparse step {ms:.3f} ms (breakdown pass {ms_all:.3f} ms)", file=sys.stderr, flush=True)

    dom_tflops = fl[dom] / (dom_ms * 1e-3) / 1e12
    for n, v in kern.items():
        if n in fl:
            v["tflops"] = fl[n] / (v["avg_ms"] * 1e-3) / 1e12
            v["mfma_frac"] = v["tflops"] / PEAK_BF16_TFLOPS
        else:
            v["gbs"] = by[n] / (v["avg_ms"] * 1e-3) / 1e9
    total_flops = sum(fl.values())

    dense = None
    if not args.no_dense:
        idx_full = torch.arange(F, dtype=torch.int32, device=X.device).repeat(B, 1).contiguous()
        bufd = sl.FFNWorkspace(w, lay, F, X.device)

        def step_dense():
            sl.ffn_fwd(w, X, lay, F, idx_full, bufd, Y=Y)
            sl.ffn_bwd(w, X, lay, F, idx_full, bufd, dY, out=grads)

        dense_ms = timed(torch, step_dense, max(3, args.steps // 2), 2)
        dense = {"ms_per_step": dense_ms, "speedup": dense_ms / ms}
        print(f"[bench] dense step {dense_ms:.3f} ms", file=sys.stderr, flush=True)
        del bufd

    attn = None
    if not args.no_attn:
        del buf, est
        torch.cuda.empty_cache()
        attn = attn_bench(args, torch, sl)
    extreme = None
    if not args.no_extreme:
        torch.cuda.empty_cache()
        extreme = {"ffn": ffn_extreme_bench(args, torch, sl)}
        if not args.no_attn:
            extreme["attention"] = attn_bench(args, torch, sl, cfg=6)

    qlora = None
    if not args.no_qlora:
        torch.cuda.empty_cache()
        qlora = qlora_bench(args, torch, sl)

    others = None
    if not args.no_workloads:
        others = {}
        for c in (1, 4, 5):
            torch.cuda.empty_cache()
            o = workload_bench(args, torch, sl, c)
            others[o["workload"]] = o

    if args.copy_calibration:
        n = 64 << 20
        src = torch.ones(n, dtype=torch.bfloat16, device=X.device)
        dst = torch.empty(n, dtype=torch.float32, device=X.device)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(p, ctx, L, Ptg.float().cpu().numpy(), Qg.float().cpu().numpy(),
                           Ptu.float().cpu().numpy(), Qu.float().cpu().numpy(), k, args.cpu_budget_s)

    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "d_model": D, "d_ff": F, "lora_rank": r, "est_rank": r_e,
                   "batch": B, "seq_len": L, "ctx_len": ctx, "sparsity_pct": f.sparsity_pct,
                   "k": k, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": dom_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": dom_tflops / PEAK_BF16_TFLOPS, "traffic": measured_traffic(dom),
                     "avg_launch_ms": dom_ms, "flops_per_launch": fl[dom]},
        "effective_tflops": total_flops / (ms * 1e-3) / 1e12,
        "speedup_vs_dense": dense["speedup"] if dense else None,
        "dense_ms_per_step": dense["ms_per_step"] if dense else None,
        "estimator_share": {"time": (kern.get("estimate", {}).get("share", 0) +
                                     kern.get("select", {}).get("share", 0))},
        "kernels": kern,
        "estimator_build_ms_per_weight": build_ms,
        "attention": attn,
        "extreme_sparsity": extreme,
        "quantized_base": qlora,
        "workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
