"""Benchmark of the fused top-K KD loss (forward + backward, LM head included)
on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--mode tail]

Workload (the metric's configuration): a Qwen3-1.7B-shaped student head,
d = 2048, V = 151,936, T = 4096 tokens, bf16 h ~ N(0,1) and W ~ N(0,1/d);
teacher top-K = 15 log-probs + tail mass from Zipf-like teacher logits
(exponent 1.2, noise 0.3), built by the library's own row pass; vocabulary
chunk 8192 rows.  One step = one kd_topk_loss_fwd_bwd call (all its
kernels: sort/prep, logits + logsumexp + gather, per-token loss, the chunked
recompute, dz, dh and dW).  Inputs are resident in HBM before timing.

Prints ONE JSON line.  value = tokens/s of the whole job (1 GPU); the
roofline object covers the dominant kernel, timed live with HIP events on
the library's stream; cpu_baseline times the fp64 CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # MI355X HBM3E, bytes/s
METRIC = "fused top-K KD loss fwd+bwd tokens/s incl. LM head; % bf16 MFMA peak"
CFG = dict(T=4096, d=2048, V=151936, K=15, chunk=8192)
CACHE_CFG = dict(T=16384, d=4096, V=151936, K=256, rho=(0.9, 0.95))
LLAMA_CFG = dict(T=8192, d=2048, V=128256, K=256, K_rev=16, chunk=8192)
GEMM_KERNELS = {"k_pass1": 2, "k_zdz": 2, "k_dhdw": 4, "k_cache_gemm": 2}  # x T*d*V FLOP per step


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Source files each kernel family is built from (a change elsewhere leaves
# its recorded HBM traffic valid).
KERNEL_SOURCES = {
    "loss": ["loss.hip", "gemm.h", "kd_common.h", "kd_internal.h"],
    "cache": ["cache.hip", "gemm.h", "kd_common.h", "kd_internal.h"],
}


def kernel_family(kernel: str) -> str:
    return "cache" if kernel in ("k_cache_gemm", "k_topk_rows") else "loss"


def kernel_sources_hash(family: str = "loss") -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_kd_loss_amd", "csrc")
    for f in KERNEL_SOURCES[family]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current sources of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources") != kernel_sources_hash(kernel_family(kernel)):
        return None
    return rec.get("bytes_per_launch")


def build_inputs(torch, kd, synth, dev, T, d, V, K, seed=0):
    h, W = synth.student_head(T, d, V, seed=seed)
    hd, Wd = h.to(dev), W.to(dev)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    tlp = torch.empty((T, K), dtype=torch.float32, device=dev)
    mq = torch.empty(T, dtype=torch.float32, device=dev)
    rows = 1024
    for r0 in range(0, T, rows):
        r1 = min(T, r0 + rows)
        b0, nb = r0 // synth.BLOCK, (r1 - r0 + synth.BLOCK - 1) // synth.BLOCK
        zt = torch.from_numpy(synth.zipf_teacher_logits(T, V, seed=seed, first_block=b0, n_blocks=nb)).to(dev)
        o = kd.topk_rows(zt, K)
        idx[r0:r1] = o.idx
        tlp[r0:r1] = o.val - o.lse[:, None]
        mq[r0:r1] = o.m_q
        del zt
    torch.cuda.synchronize()
    return h, W, hd, Wd, idx, tlp, mq


def time_steps(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(steps):
        fn()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def kernel_profile(kd, torch, fn, steps):
    torch.cuda.synchronize()
    kd.profile_begin()
    for _ in range(steps):
        fn()
    prof = kd.profile_end()
    return {k: (ms / steps, n / steps) for k, (ms, n) in prof.items()}


def cpu_baseline(h, W, T, V, K, mode, seed=0, budget_s=15.0):
    """The fp64 oracle, untuned, on the first n tokens of the same workload."""
    import numpy as np

    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(x.get("num_threads", 1)) for x in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    W64 = synth.as_f64(W)
    nmax = min(T, 2048)
    zt = synth.zipf_teacher_logits(T, V, seed=seed, first_block=0, n_blocks=(nmax + synth.BLOCK - 1) // synth.BLOCK)

    def run(n):
        i, val, lse, m_q, _ = oracle.cache_from_logits(zt[:n], K)
        tl = oracle.teacher_logp(val, lse)
        h64 = synth.as_f64(h[:n])
        t0 = time.perf_counter()
        oracle.loss_fwd_bwd(h64, W64, i, tl, m_q, mode)
        return time.perf_counter() - t0
    n = min(64, nmax)
    dt = run(n)
    while dt < 0.5 * budget_s and n < nmax:
        n = min(nmax, max(n + 16, int(n * min(4.0, budget_s / max(dt, 1e-3)))))
        n = max(16, (n // 16) * 16)
        dt = run(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n} of the {T} tokens of the same workload (same h, W, teacher rows), "
                      f"fp64 numpy oracle, one fwd+bwd call timed ({dt:.1f} s)",
            "seconds": dt, "tokens": n}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", default="tail", choices=["renorm", "tail", "full", "reverse"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other modes, the hidden-state KL, the T=8192 K=256 line and the cache build")
    ap.add_argument("--no-memscan", action="store_true",
                    help="skip the long-context line (peak memory and tokens/s vs T at d=2560, K=64, 4K..32K)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 4 device copies of 1 GiB (fp32) for HBM counter calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}); multi-GPU runs are not part of this build",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import top_kd_loss_amd as kd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 28  # 1 GiB of fp32 read and 1 GiB written per copy
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n, "copies": 4}), flush=True)
        return
    T, d, V, K, chunk = CFG["T"], CFG["d"], CFG["V"], CFG["K"], CFG["chunk"]
    mode = kd.MODE_BY_NAME[args.mode]
    t0 = time.time()
    h, W, hd, Wd, idx, tlp, mq = build_inputs(torch, kd, synth, dev, T, d, V, K)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")

    def make_step(md):
        ws = torch.empty(kd.loss_workspace_bytes(T, d, V, K, md, chunk), dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        out = kd.LossOut(torch.empty((), **f32), torch.empty((T, d), **f32), torch.empty((V, d), **f32),
                         torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32))
        return lambda: kd.loss_fwd_bwd(hd, Wd, idx, tlp, mq, mode=md, chunk=chunk, workspace=ws, out=out)

    torch.cuda.reset_peak_memory_stats()
    step = make_step(mode)
    ms = time_steps(torch, step, args.steps, args.warmup)
    peak_mem = torch.cuda.max_memory_allocated()
    log(f"[bench] {args.mode}: {ms:.3f} ms/step")
    prof = kernel_profile(kd, torch, step, max(3, min(args.steps, 10)))
    log("[bench] per-kernel ms/step: " + ", ".join(f"{k}={v[0]:.3f}x{v[1]:.0f}" for k, v in prof.items()))

    tdv = T * d * V
    credited = 6 * tdv if mode in (kd.TAIL, kd.FULL) else 2 * tdv + 4 * T * K * d
    dom = max(prof.items(), key=lambda kv: kv[1][0])
    name, (kms, nlaunch) = dom
    if name in GEMM_KERNELS:
        work = GEMM_KERNELS[name] * tdv / nlaunch
        achieved = work / (kms / nlaunch * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": name, "achieved": achieved, "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s", "frac": achieved * 1e12 / PEAK_BF16,
                "traffic": measured_traffic(name), "avg_launch_ms": kms / nlaunch,
                "algorithmic_flop_per_launch": work}
    else:
        roof = {"bound": "hbm", "kernel": name, "achieved": None, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": None, "traffic": measured_traffic(name), "avg_launch_ms": kms / nlaunch}

    res = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"Qwen3-1.7B-shaped student head, {args.mode} mode", "T": T, "d": d, "V": V, "K": K,
                   "chunk": chunk, "mode": args.mode, "teacher": "Zipf-like logits, exponent 1.2, noise 0.3"},
        "mfma_frac_step": credited / (ms * 1e-3) / PEAK_BF16,
        "credited_flop_per_step": credited,
        "peak_mem_bytes": peak_mem,
        "roofline": roof,
        "kernels_ms_per_step": {k: round(v[0], 4) for k, v in prof.items()},
    }

    if not args.no_extras:
        other = kd.RENORM if mode != kd.RENORM else kd.TAIL
        ms2 = time_steps(torch, make_step(other), max(3, args.steps // 2), 2)
        cr2 = 6 * tdv if other in (kd.TAIL, kd.FULL) else 2 * tdv + 4 * T * K * d
        res["other_mode"] = {"mode": {kd.RENORM: "renorm", kd.TAIL: "tail"}[other], "ms_per_step": ms2,
                             "tokens_per_s": T / (ms2 * 1e-3), "mfma_frac_step": cr2 / (ms2 * 1e-3) / PEAK_BF16}
        log(f"[bench] other mode: {ms2:.3f} ms/step")
        res["more_modes"] = bench_more_modes(torch, kd, synth, dev, hd, Wd, idx, tlp, mq, max(3, args.steps // 4))
        log(f"[bench] more modes: {res['more_modes']}")
        res["kl_hidden"] = bench_kl_hidden(torch, kd, synth, dev, hd, Wd, max(3, args.steps // 4))
        log(f"[bench] kl_hidden: {res['kl_hidden']}")
        del hd, Wd
        torch.cuda.empty_cache()
        res["llama_k256"] = bench_llama_k256(torch, kd, synth, dev, max(3, args.steps // 4))
        log(f"[bench] llama k256: {res['llama_k256']}")
        res["cache_build"] = bench_cache_build(torch, kd, synth, dev)
        log(f"[bench] cache build: {res['cache_build']}")
        res["topk_rows"] = bench_topk_rows(torch, kd, dev)
        log(f"[bench] standalone row pass: {res['topk_rows']}")

    if not args.no_memscan and not args.no_extras:
        res["memscan"] = memscan(torch, kd, dev)

    if not args.no_cpu_baseline:
        t1 = time.time()
        res["cpu_baseline"] = cpu_baseline(h, W, T, V, K, mode)
        log(f"[bench] cpu baseline in {time.time() - t1:.1f}s")
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_more_modes(torch, kd, synth, dev, hd, Wd, idx, tlp, mq, steps):
    """Step time of the other objectives on the same workload: the tail-token
    reverse KL, the tail-corrected reverse KL (synthetic sampled tokens and
    teacher log-probs at them), and the tail-aware loss plus a 0.1-weighted
    hard-label cross-entropy term (synthetic labels)."""
    T, d, V, K, chunk = CFG["T"], CFG["d"], CFG["V"], CFG["K"], CFG["chunk"]
    y = torch.from_numpy(synth.token_labels(T, V, seed=5)).to(dev)
    tly = torch.full((T,), -12.0, dtype=torch.float32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = kd.LossOut(torch.empty((), **f32), torch.empty((T, d), **f32), torch.empty((V, d), **f32),
                     torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32))
    cases = {
        "tail_reverse": (kd.TAIL_REVERSE, {}),
        "reverse_tt": (kd.REVERSE_TT, {"labels": y, "labels_teacher_logp": tly}),
        "tail+ce0.1": (kd.TAIL, {"labels": y, "ce_weight": 0.1}),
    }
    res = {}
    for name, (md, kw) in cases.items():
        ws = torch.empty(kd.loss_workspace_bytes(T, d, V, K, md, chunk, kw.get("ce_weight", 0.0)),
                         dtype=torch.uint8, device=dev)
        fn = lambda: kd.loss_fwd_bwd(hd, Wd, idx, tlp, mq, mode=md, chunk=chunk, workspace=ws, out=out, **kw)
        ms = time_steps(torch, fn, steps, 1)
        res[name] = {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3)}
        del ws
    return res


def bench_kl_hidden(torch, kd, synth, dev, hd, Wd, steps):
    """Exact full-vocabulary KL with the teacher rebuilt from a cached hidden
    state: Qwen3-8B-shaped teacher head (d_t = 4096) over the same student."""
    T, d, V = CFG["T"], CFG["d"], CFG["V"]
    dt = 4096
    g, U, b = synth.teacher_head(T, dt, V, seed=1)
    gd, Ud, bd = g.to(dev), U.to(dev), b.to(dev)
    del g, U
    ws = torch.empty(kd.lib().kd_kl_hidden_workspace(T, d, dt, V, CFG["chunk"]), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = kd.KlOut(torch.empty((), **f32), torch.empty((T, d), **f32), torch.empty((V, d), **f32),
                   torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32))
    fn = lambda: kd.kl_hidden_fwd_bwd(hd, Wd, gd, Ud, bd, chunk=CFG["chunk"], workspace=ws, out=out)
    ms = time_steps(torch, fn, steps, 2)
    prof = kernel_profile(kd, torch, fn, 2)
    credited = 2 * T * d * V + 2 * T * dt * V + 4 * T * d * V      # student forward, teacher head, dh + dW
    executed = 2 * (2 * T * d * V) + 2 * (2 * T * dt * V) + 4 * T * d * V
    # the teacher's logsumexp read from the cache (lse_t of the call above): one teacher-head pass
    lse_t = out.lse_t.clone()
    fn_c = lambda: kd.kl_hidden_fwd_bwd(hd, Wd, gd, Ud, bd, chunk=CFG["chunk"], workspace=ws, out=out,
                                        teacher_lse=lse_t)
    ms_c = time_steps(torch, fn_c, steps, 2)
    executed_c = executed - 2 * T * dt * V
    del gd, Ud, bd, ws, out, lse_t
    torch.cuda.empty_cache()
    return {"workload": "Qwen3-8B-shaped teacher head (hidden-state cache) over the Qwen3-1.7B-shaped student",
            "T": T, "d": d, "d_teacher": dt, "V": V, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "mfma_frac_credited": credited / (ms * 1e-3) / PEAK_BF16,
            "mfma_frac_executed": executed / (ms * 1e-3) / PEAK_BF16,
            "kernels_ms_per_step": {k: round(v[0], 4) for k, v in prof.items()},
            "cached_teacher_lse": {"ms_per_step": ms_c, "tokens_per_s": T / (ms_c * 1e-3),
                                   "mfma_frac_credited": credited / (ms_c * 1e-3) / PEAK_BF16,
                                   "mfma_frac_executed": executed_c / (ms_c * 1e-3) / PEAK_BF16}}


def bench_llama_k256(torch, kd, synth, dev, steps):
    """Llama-3.2-1B-shaped student head, T=8192, V=128,256: the teacher cache
    keeps K=256 (renorm, tail, full); reverse KL runs on the student's own
    top-16, selected by the cache build on (h, W), with the teacher's
    log-probs gathered from the same synthetic teacher rows."""
    c = LLAMA_CFG
    T, d, V, K, Kr, chunk = c["T"], c["d"], c["V"], c["K"], c["K_rev"], c["chunk"]
    h, W = synth.student_head(T, d, V, seed=2)
    hd, Wd = h.to(dev), W.to(dev)
    del h, W
    sel = kd.cache_build(hd, Wd, None, Kr)                 # student top-16 (the REVERSE support)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    tlp = torch.empty((T, K), dtype=torch.float32, device=dev)
    mq = torch.empty(T, dtype=torch.float32, device=dev)
    tlp_rev = torch.empty((T, Kr), dtype=torch.float32, device=dev)
    rows = 1024
    for r0 in range(0, T, rows):
        r1 = min(T, r0 + rows)
        b0, nb = r0 // synth.BLOCK, (r1 - r0 + synth.BLOCK - 1) // synth.BLOCK
        zt = torch.from_numpy(synth.zipf_teacher_logits(T, V, seed=2, first_block=b0, n_blocks=nb)).to(dev)
        o = kd.topk_rows(zt, K)
        idx[r0:r1], tlp[r0:r1], mq[r0:r1] = o.idx, o.val - o.lse[:, None], o.m_q
        tlp_rev[r0:r1] = torch.gather(zt, 1, sel.idx[r0:r1].long()) - o.lse[:, None]
        del zt
    torch.cuda.synchronize()
    f32 = dict(dtype=torch.float32, device=dev)
    out = kd.LossOut(torch.empty((), **f32), torch.empty((T, d), **f32), torch.empty((V, d), **f32),
                     torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32))
    tdv = T * d * V
    res = {"workload": "Llama-3.2-1B-shaped student head", "T": T, "d": d, "V": V, "K": K, "chunk": chunk}
    for name, md in (("renorm", kd.RENORM), ("tail", kd.TAIL), ("full", kd.FULL)):
        ws = torch.empty(kd.loss_workspace_bytes(T, d, V, K, md, chunk), dtype=torch.uint8, device=dev)
        ms = time_steps(torch, lambda: kd.loss_fwd_bwd(hd, Wd, idx, tlp, mq, mode=md, chunk=chunk, workspace=ws,
                                                       out=out), steps, 2)
        cr = 6 * tdv if md in (kd.TAIL, kd.FULL) else 2 * tdv + 4 * T * K * d
        res[name] = {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "mfma_frac_step": cr / (ms * 1e-3) / PEAK_BF16}
        del ws
    wsc = torch.empty(kd.lib().kd_topk_cache_build_workspace(T, d, V, Kr, 0), dtype=torch.uint8, device=dev)
    ms_sel = time_steps(torch, lambda: kd.cache_build(hd, Wd, None, Kr, workspace=wsc), steps, 1)
    del wsc
    ws = torch.empty(kd.loss_workspace_bytes(T, d, V, Kr, kd.REVERSE, chunk), dtype=torch.uint8, device=dev)
    ridx = sel.idx
    ms_rev = time_steps(torch, lambda: kd.loss_fwd_bwd(hd, Wd, ridx, tlp_rev, None, mode=kd.REVERSE, chunk=chunk,
                                                       workspace=ws, out=out), steps, 2)
    # the selection's lse and values stand in for the loss's forward pass
    slse, sval = sel.lse, sel.val
    ms_rev_g = time_steps(torch, lambda: kd.loss_fwd_bwd(hd, Wd, ridx, tlp_rev, None, mode=kd.REVERSE, chunk=chunk,
                                                         workspace=ws, out=out, student_lse=slse,
                                                         student_logits=sval), steps, 2)
    res["reverse_student_top16"] = {"selection_ms": ms_sel, "loss_ms": ms_rev,
                                    "tokens_per_s": T / ((ms_sel + ms_rev) * 1e-3),
                                    "loss_ms_given_selection": ms_rev_g,
                                    "tokens_per_s_given_selection": T / ((ms_sel + ms_rev_g) * 1e-3)}
    del hd, Wd, idx, tlp, mq, tlp_rev, sel, ws, out
    torch.cuda.empty_cache()
    return res


def bench_topk_rows(torch, kd, dev, steps=5):
    """The standalone row pass (kd_topk_rows) on 2048 fp32 rows shaped like the
    cache build's teacher logits (V = 151,936, N(0, 1.1)), K = 256, with and
    without the two k_rho targets: algorithmic bytes = the row read once plus
    the outputs."""
    T, V, K = 2048, CACHE_CFG["V"], CACHE_CFG["K"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    z = torch.randn((T, V), generator=gen, device=dev, dtype=torch.float32) * 1.1
    res = {"workload": "teacher-logit rows, N(0, 1.1)", "rows": T, "V": V, "K": K}
    for name, rho in (("no_rho", ()), ("rho", CACHE_CFG["rho"])):
        ws = torch.empty(max(1, kd.lib().kd_topk_rows_workspace(T, V, K, len(rho))), dtype=torch.uint8, device=dev)
        ms = time_steps(torch, lambda: kd.topk_rows(z, K, rho, workspace=ws), steps, 2)
        alg = T * (4 * V) + T * (8 * K + 8 + 4 * len(rho))
        gbps = alg / (ms * 1e-3) / 1e9
        res[name] = {"rho": list(rho), "ms_per_call": ms, "algorithmic_GBps": gbps, "hbm_frac": gbps * 1e9 / PEAK_HBM}
    del z
    torch.cuda.empty_cache()
    return res


def bench_cache_build(torch, kd, synth, dev, steps=3):
    c = CACHE_CFG
    T, d, V, K, rho = c["T"], c["d"], c["V"], c["K"], c["rho"]
    g, U, b = synth.teacher_head(T, d, V, seed=0)
    gd, Ud, bd = g.to(dev), U.to(dev), b.to(dev)
    ws = torch.empty(kd.lib().kd_topk_cache_build_workspace(T, d, V, K, len(rho)), dtype=torch.uint8, device=dev)
    fn = lambda: kd.cache_build(gd, Ud, bd, K, rho, workspace=ws)
    ms = time_steps(torch, fn, steps, 1)
    prof = kernel_profile(kd, torch, fn, 1)
    gemm_ms = prof.get("k_cache_gemm", (0.0, 0))[0]
    rows_ms = prof.get("k_topk_rows", (0.0, 0))[0]
    rows_bytes = T * (4 * V) + T * (8 * K + 8 + 4 * len(rho))
    rows_nrho0 = None
    return {"workload": "Qwen3-8B-shaped teacher head", "T": T, "d": d, "V": V, "K": K, "rho": list(rho),
            "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "gemm_ms": gemm_ms, "gemm_mfma_frac": 2 * T * d * V / (gemm_ms * 1e-3) / PEAK_BF16 if gemm_ms else None,
            "rows_ms": rows_ms, "rows_algorithmic_GBps": rows_bytes / (rows_ms * 1e-3) / 1e9 if rows_ms else None,
            "rows_hbm_frac": rows_bytes / (rows_ms * 1e-3) / PEAK_HBM if rows_ms else None}


def memscan(torch, kd, dev):
    """Long-context, Qwen3-4B-shaped head (d=2560, V=151,936, K=64, tail mode):
    peak allocated memory of one fused step and its tokens/s vs T."""
    d, V, K = 2560, 151936, 64
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    W = (torch.randn((V, d), device=dev, generator=gen) / d ** 0.5).to(torch.bfloat16)
    out = {}
    for T in (4096, 8192, 16384, 32768):
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        h = torch.randn((T, d), device=dev, generator=gen).to(torch.bfloat16)
        idx = ((torch.arange(T, device=dev)[:, None] * 7919 + torch.arange(K, device=dev)[None, :] * 2371) % V).int()
        tlp = torch.full((T, K), -6.0, device=dev)
        mq = torch.full((T,), 1.0 - K * float(torch.exp(torch.tensor(-6.0))), device=dev)
        t0 = time.time()
        kd.loss_fwd_bwd(h, W, idx, tlp, mq, mode=kd.TAIL, chunk=8192)
        torch.cuda.synchronize()
        first = time.time() - t0
        peak = torch.cuda.max_memory_allocated() - base
        ms = time_steps(torch, lambda: kd.loss_fwd_bwd(h, W, idx, tlp, mq, mode=kd.TAIL, chunk=8192), 2, 0)
        out[str(T)] = {"peak_bytes_above_W": peak, "first_call_s": first, "ms_per_step": ms,
                       "tokens_per_s": T / (ms * 1e-3),
                       "mfma_frac_step": 6 * T * d * V / (ms * 1e-3) / PEAK_BF16}
        log(f"[bench] memscan T={T}: {out[str(T)]}")
        del h, idx, tlp, mq
    return out


if __name__ == "__main__":
    main()
