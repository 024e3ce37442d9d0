"""Benchmark of the fused top-K KD loss (forward + backward, LM head included)
on one MI355X.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--mode tail]

Workload (the metric's configuration, the largest fused-loss one): the
long-context Qwen3-4B-shaped student head, d = 2560, V = 151,936,
T = 32,768 tokens, bf16 h ~ N(0,1) and W ~ N(0,1/d); teacher top-K = 64
log-probs + tail mass from Zipf-like teacher logits (exponent 1.2, noise
0.3), built by the library's own row pass; vocabulary chunk 8192 rows; the
tail-aware (K+1)-bin loss.  One step = one kd_topk_loss_fwd_bwd call (all
its kernels: sort/prep, logits + logsumexp + gather, per-token loss, the
chunked recompute, dz, dh and dW).  Inputs are resident in HBM before
timing.

Prints ONE JSON line.  value = tokens/s of the whole job (1 GPU); the
roofline object covers the dominant kernel, timed live with HIP events on
the library's stream; cpu_baseline times the fp64 CPU oracle on a bounded
sample of the same workload.  Extra keys: the full-vocabulary mode on the
same inputs, peak memory and tokens/s vs T (4K..32K), the Qwen3-1.7B head
(T=4096, K=15: tail, renorm and the other objectives), the hidden-state KL,
the Llama-3.2-1B head (T=8192, K=256, and reverse KL on the student's own
top-16), the teacher-cache build (T=16,384, d=4096) and the standalone row
pass.
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
HEAD_CFG = dict(T=32768, d=2560, V=151936, K=64, chunk=8192, seed=0)
QWEN17_CFG = dict(T=4096, d=2048, V=151936, K=15, chunk=8192, seed=1)
CACHE_CFG = dict(T=16384, d=4096, V=151936, K=256, rho=(0.9, 0.95))
LLAMA_CFG = dict(T=8192, d=2048, V=128256, K=256, K_rev=16, chunk=8192)
GEMM_KERNELS = {"k_pass1": 2, "k_zdz": 2, "k_dhdw": 4, "k_cache_gemm": 2,   # x T*d*V FLOP per step
                "k_pass1_store": 2}
TOKEN_BLOCK = 8192      # tokens per block of the token-block option
TEACHER = "Zipf-like logits, exponent 1.2, noise 0.3"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Source files each kernel family is built from (a change elsewhere leaves
# its recorded HBM traffic valid).
KERNEL_SOURCES = {
    "loss": ["loss.hip", "gemm.h", "kd_common.h", "kd_internal.h"],
    "cache": ["cache.hip", "gemm.h", "kd_common.h", "kd_internal.h"],
}


ROW_KERNELS = ("k_topk_rows", "k_rows_cross", "k_topk_rows_exact")   # the row pass, all its launches


def kernel_family(kernel: str) -> str:
    return "cache" if kernel == "k_cache_gemm" or kernel in ROW_KERNELS else "loss"


def kernel_sources_hash(family: str = "loss") -> str:
    """Hash of the code a kernel family is built from: comments (the sources
    use // only) and blank lines do not count."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_kd_loss_amd", "csrc")
    for f in KERNEL_SOURCES[family]:
        for line in open(os.path.join(csrc, f), encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def workload_key(cfg: dict, mode: str) -> str:
    return f"{mode} T={cfg['T']} d={cfg['d']} V={cfg['V']} K={cfg['K']} chunk={cfg['chunk']}"


def cache_workload_key() -> str:
    c = CACHE_CFG
    return f"cache_build T={c['T']} d={c['d']} V={c['V']} K={c['K']} rho={','.join(str(r) for r in c['rho'])}"


def rows_workload_key(n_rho: int) -> str:
    rho = ",".join(str(r) for r in CACHE_CFG["rho"][:n_rho]) or "none"
    return f"topk_rows rows=2048 V={CACHE_CFG['V']} K={CACHE_CFG['K']} N(0,1.1) rho={rho}"


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on this workload and on the current sources of that
    kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        recs = json.load(open(path)).get("records", [])
    except (OSError, ValueError):
        return None
    src = kernel_sources_hash(kernel_family(kernel))
    for rec in recs:
        if rec.get("kernel") == kernel and rec.get("workload") == workload and rec.get("sources") == src:
            return rec.get("bytes_per_launch")
    return None


def teacher_cache_device(torch, kd, synth, dev, T, V, K, seed, rows=2048):
    """Teacher cache of Zipf-like teacher rows (drawn on the GPU) by the
    library's row pass: (idx, teacher_logp, m_q) on the device."""
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    tlp = torch.empty((T, K), dtype=torch.float32, device=dev)
    mq = torch.empty(T, dtype=torch.float32, device=dev)
    for r0 in range(0, T, rows):
        r1 = min(T, r0 + rows)
        zt = synth.zipf_teacher_logits_device(r1 - r0, V, seed, dev, first_row=r0)
        o = kd.topk_rows(zt, K)
        idx[r0:r1], tlp[r0:r1], mq[r0:r1] = o.idx, o.teacher_logp, o.m_q
        del zt, o
    torch.cuda.synchronize()
    return idx, tlp, mq


def build_inputs(torch, kd, synth, dev, cfg):
    T, d, V, K, seed = cfg["T"], cfg["d"], cfg["V"], cfg["K"], cfg["seed"]
    h, W = synth.student_head(T, d, V, seed=seed)
    hd, Wd = h.to(dev), W.to(dev)
    idx, tlp, mq = teacher_cache_device(torch, kd, synth, dev, T, V, K, seed)
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
    """Per-kernel HIP-event times of `steps` further calls (a separate pass:
    the event pairs around each launch add a little time of their own)."""
    torch.cuda.synchronize()
    kd.profile_begin()
    for _ in range(steps):
        fn()
    prof = kd.profile_end()
    return {k: (ms / steps, n / steps) for k, (ms, n) in prof.items()}


def loss_out(torch, kd, dev, T, d, V):
    f32 = dict(dtype=torch.float32, device=dev)
    return kd.LossOut(torch.empty((), **f32), torch.empty((T, d), **f32), torch.empty((V, d), **f32),
                      torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32))


def credited_flop(kd, mode, T, d, V, K):
    return 6 * T * d * V if mode in (kd.TAIL, kd.FULL, kd.TAIL_REVERSE, kd.REVERSE_TT) else 2 * T * d * V + 4 * T * K * d


def blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            x = info[0]
            return {"library": f"{x.get('internal_api')} ({os.path.basename(x.get('filepath', ''))})",
                    "threads": int(x.get("num_threads", 1))}
    except Exception:  # pragma: no cover
        pass
    return {"library": "unknown", "threads": None}


def cpu_baseline(h, W, zt_rows, T, V, K, mode, budget_s=15.0):
    """The fp64 oracle, untuned, on the first n tokens of the same workload
    (same h, W and teacher rows; the oracle builds its own cache of them)."""
    import numpy as np

    import oracle
    import synth
    W64 = synth.as_f64(W)
    nmax = zt_rows.shape[0]
    caches = {}

    def run(n):
        if n not in caches:
            i, val, lse, m_q, _ = oracle.cache_from_logits(zt_rows[:n], K)
            caches.clear()
            caches[n] = (i, oracle.teacher_logp(val, lse), m_q)
        i, tl, m_q = caches[n]
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
    b = blas_info()
    # cores: the threads the oracle actually ran on (BLAS's pool; its
    # elementwise numpy code is single-threaded), beside the cores the
    # process may use
    return {"value": n / dt, "unit": "tokens/s", "cores": b["threads"] or 1, "kind": "oracle",
            "sample": f"first {n} of the {T} tokens of the same workload (same h, W and teacher rows; oracle-built "
                      f"top-{K} cache), fp64 numpy oracle, one fwd+bwd call timed ({dt:.1f} s)",
            "seconds": dt, "tokens": n, "blas_library": b["library"], "blas_threads": b["threads"],
            "affinity_cores": len(os.sched_getaffinity(0))}


def roofline_of(prof, tdv, workload):
    """The dominant kernel's algorithmic rate from its average launch time."""
    dom = max(prof.items(), key=lambda kv: kv[1][0])
    name, (kms, nlaunch) = dom
    if name in GEMM_KERNELS:
        work = GEMM_KERNELS[name] * tdv / nlaunch
        achieved = work / (kms / nlaunch * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": name, "achieved": achieved, "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s", "frac": achieved * 1e12 / PEAK_BF16,
                "traffic": measured_traffic(name, workload), "avg_launch_ms": kms / nlaunch,
                "algorithmic_flop_per_launch": work}
    return {"bound": "hbm", "kernel": name, "achieved": None, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": None, "traffic": measured_traffic(name, workload), "avg_launch_ms": kms / nlaunch}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--mode", default="tail", choices=["renorm", "tail", "full", "reverse"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the full mode, the T=4096 K=15 line, the hidden-state KL, the T=8192 K=256 line, "
                         "the cache build and the standalone row pass")
    ap.add_argument("--no-memscan", action="store_true",
                    help="skip peak memory and tokens/s vs T (4K..32K) on the headline workload")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event pass")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="also time the vendor GEMM (torch.mm: hipBLASLt) on the three LM-head GEMM shapes of the "
                         "headline workload, for context")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 4 device copies of 1 GiB (fp32) for HBM counter calibration")
    ap.add_argument("--token-block", type=int, default=0,
                    help="time the token-block option (kd_topk_loss_fwd_bwd_tokblock, this many tokens per block) "
                         "as the step instead of the vocabulary-chunked call")
    ap.add_argument("--only", choices=["cache_build", "topk_rows", "llama_k256"],
                    help="only run the teacher-cache build (T=16384, d=4096), the standalone row pass, or the "
                         "Llama-3.2-1B-shaped head at K=256 (sparse backward) and print its JSON (for profiling)")
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
    if args.only == "cache_build":
        print(json.dumps(bench_cache_build(torch, kd, synth, dev, steps=max(1, args.steps))), flush=True)
        return
    if args.only == "topk_rows":
        print(json.dumps(bench_topk_rows(torch, kd, dev, steps=max(1, args.steps))), flush=True)
        return
    if args.only == "llama_k256":
        print(json.dumps(bench_llama_k256(torch, kd, synth, dev, steps=max(1, args.steps))), flush=True)
        return
    cfg = HEAD_CFG
    T, d, V, K, chunk = cfg["T"], cfg["d"], cfg["V"], cfg["K"], cfg["chunk"]
    mode = kd.MODE_BY_NAME[args.mode]
    t0 = time.time()
    h, W, hd, Wd, idx, tlp, mq = build_inputs(torch, kd, synth, dev, cfg)
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")

    out = loss_out(torch, kd, dev, T, d, V)

    def make_step(md, TT=T, fresh_out=False, tb=0):
        ws = torch.empty(kd.loss_workspace_bytes(TT, d, V, K, md, chunk, token_block=tb), dtype=torch.uint8,
                         device=dev)
        o = loss_out(torch, kd, dev, TT, d, V) if fresh_out else out
        hh, ii, tt_, mm = hd[:TT], idx[:TT], tlp[:TT], mq[:TT]
        return lambda: kd.loss_fwd_bwd(hh, Wd, ii, tt_, mm, mode=md, chunk=chunk, workspace=ws, out=o,
                                       token_block=tb)

    torch.cuda.reset_peak_memory_stats()
    step = make_step(mode, tb=args.token_block)
    ms = time_steps(torch, step, args.steps, args.warmup)
    peak_mem = torch.cuda.max_memory_allocated()
    log(f"[bench] {args.mode}: {ms:.3f} ms/step")
    tdv = T * d * V
    credited = credited_flop(kd, mode, T, d, V, K)
    wl = workload_key(cfg, args.mode) + (f" token_block={args.token_block}" if args.token_block else "")
    res = {
        "metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"long-context Qwen3-4B-shaped student head, {args.mode} mode", "T": T, "d": d,
                   "V": V, "K": K, "chunk": chunk, "mode": args.mode, "teacher": TEACHER,
                   "path": f"token blocks of {args.token_block}" if args.token_block else "vocabulary-chunked"},
        "mfma_frac_step": credited / (ms * 1e-3) / PEAK_BF16,
        "credited_flop_per_step": credited,
        "peak_mem_bytes": peak_mem,
    }
    if not args.no_profile:
        prof = kernel_profile(kd, torch, step, max(3, min(args.steps, 5)))
        log("[bench] per-kernel ms/step: " + ", ".join(f"{k}={v[0]:.3f}x{v[1]:.0f}" for k, v in prof.items()))
        res["roofline"] = roofline_of(prof, tdv, wl)
        res["kernels_ms_per_step"] = {k: round(v[0], 4) for k, v in prof.items()}
        res["kernels_ms_sum_profiled"] = round(sum(v[0] for v in prof.values()), 4)
    else:
        res["roofline"] = None

    if not args.no_extras:
        other = kd.FULL if mode != kd.FULL else kd.TAIL
        ms2 = time_steps(torch, make_step(other), args.steps, 2)
        cr2 = credited_flop(kd, other, T, d, V, K)
        res["other_mode"] = {"mode": {kd.FULL: "full", kd.TAIL: "tail"}[other], "ms_per_step": ms2,
                             "tokens_per_s": T / (ms2 * 1e-3), "mfma_frac_step": cr2 / (ms2 * 1e-3) / PEAK_BF16}
        log(f"[bench] other mode: {ms2:.3f} ms/step")

    if not args.no_extras and mode in (kd.TAIL, kd.FULL):
        res["token_block"] = {"token_block": TOKEN_BLOCK, "note": "kd_topk_loss_fwd_bwd_tokblock: the block's logits "
                              "kept as bf16 instead of recomputed in the backward (6TdV executed)"}
        for md, name in ((kd.TAIL, "tail"), (kd.FULL, "full")):
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats()
            fn = make_step(md, tb=TOKEN_BLOCK)
            ms_tb = time_steps(torch, fn, args.steps, 2)
            res["token_block"][name] = {
                "ms_per_step": ms_tb, "tokens_per_s": T / (ms_tb * 1e-3),
                "mfma_frac_step": credited_flop(kd, md, T, d, V, K) / (ms_tb * 1e-3) / PEAK_BF16,
                "peak_mem_bytes": torch.cuda.max_memory_allocated()}
            if md == mode and not args.no_profile:
                prof_tb = kernel_profile(kd, torch, fn, 3)
                res["token_block"][name]["kernels_ms_per_step"] = {k: round(v[0], 4) for k, v in prof_tb.items()}
            del fn
        log(f"[bench] token block: {res['token_block']}")

    if not args.no_memscan:
        res["memscan"] = memscan(torch, kd, dev, make_step, mode, cfg, args.steps)

    if args.gemm_reference:
        res["gemm_reference"] = gemm_reference(torch, dev, cfg)
        log(f"[bench] vendor GEMM reference: {res['gemm_reference']}")

    zt_rows = None
    if not args.no_cpu_baseline:
        zt_rows = synth.zipf_teacher_logits_device(2048, V, cfg["seed"], dev).cpu().numpy()
    del hd, Wd, idx, tlp, mq, out, step
    torch.cuda.empty_cache()

    if not args.no_extras:
        res["qwen3_1p7b"] = bench_qwen17(torch, kd, synth, dev, max(5, args.steps))
        log(f"[bench] qwen3-1.7b head: {res['qwen3_1p7b']}")
        res["llama_k256"] = bench_llama_k256(torch, kd, synth, dev, max(3, args.steps // 2))
        log(f"[bench] llama k256: {res['llama_k256']}")
        res["cache_build"] = bench_cache_build(torch, kd, synth, dev)
        log(f"[bench] cache build: {res['cache_build']}")
        res["topk_rows"] = bench_topk_rows(torch, kd, dev)
        log(f"[bench] standalone row pass: {res['topk_rows']}")

    if not args.no_cpu_baseline:
        t1 = time.time()
        res["cpu_baseline"] = cpu_baseline(h, W, zt_rows, T, V, K, mode)
        log(f"[bench] cpu baseline in {time.time() - t1:.1f}s")
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def gemm_reference(torch, dev, cfg, steps=5):
    """The vendor bf16 GEMM (torch.mm, hipBLASLt on ROCm; fp32 accumulation,
    bf16 output) on the library's GEMM shapes with the library's operand
    layouts: the logits of all T tokens from h [T, d] and W [V, d] (both
    k-contiguous, as pass 1 and its recompute read them), dW = dz^T h and
    dh = dz W of one 8192-row vocabulary chunk, and the teacher-cache block
    U g (2048 tokens, d = 4096).  Context for the library's own kernels,
    which carry the loss epilogues as well."""
    T, d, V = cfg["T"], cfg["d"], cfg["V"]
    C = cfg["chunk"]
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    h = torch.randn((T, d), device=dev, generator=g).to(torch.bfloat16)
    W = (torch.randn((V, d), device=dev, generator=g) / d ** 0.5).to(torch.bfloat16)
    dz = (torch.randn((T, C), device=dev, generator=g) * 1e-5).to(torch.bfloat16)
    Wc = W[:C].contiguous()
    out = {}

    def timed(name, fn, M, N, K):
        ms = time_steps(torch, fn, steps, 2)
        fl = 2.0 * M * N * K
        out[name] = {"M": M, "N": N, "K": K, "ms": ms, "TFLOP_s": fl / (ms * 1e-3) / 1e12,
                     "frac_of_2.5PF": fl / (ms * 1e-3) / PEAK_BF16}

    timed("logits h W^T", lambda: torch.mm(h, W.t()), T, V, d)
    timed("dW = dz^T h (one chunk)", lambda: torch.mm(dz.t(), h), C, d, T)
    timed("dh = dz W (one chunk)", lambda: torch.mm(dz, Wc), T, d, C)
    del h, W, dz, Wc
    torch.cuda.empty_cache()
    c = CACHE_CFG
    gt = torch.randn((2048, c["d"]), device=dev, generator=g).to(torch.bfloat16)
    U = (torch.randn((c["V"], c["d"]), device=dev, generator=g) / c["d"] ** 0.5).to(torch.bfloat16)
    timed("teacher-cache block U g", lambda: torch.mm(gt, U.t()), 2048, c["V"], c["d"])
    del gt, U
    torch.cuda.empty_cache()
    return out


def memscan(torch, kd, dev, make_step, mode, cfg, steps):
    """Peak allocated memory of one fused step above its inputs (outputs dh,
    dW, the per-token outputs and the workspace), and its tokens/s, at
    T = 4K, 8K, 16K, 32K on the headline workload's first T tokens (same W,
    h rows and teacher cache)."""
    d, V = cfg["d"], cfg["V"]
    out = {}
    for T in (4096, 8192, 16384, 32768):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        fn = make_step(mode, T, fresh_out=True)  # allocates the workspace and the outputs
        t0 = time.time()
        fn()
        torch.cuda.synchronize()
        first = time.time() - t0
        peak = torch.cuda.max_memory_allocated() - base
        ms = time_steps(torch, fn, steps, 1)
        out[str(T)] = {"peak_bytes_above_inputs": peak, "first_call_s": first, "ms_per_step": ms,
                       "tokens_per_s": T / (ms * 1e-3), "mfma_frac_step": 6 * T * d * V / (ms * 1e-3) / PEAK_BF16}
        del fn
        if mode in (kd.TAIL, kd.FULL):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            fn = make_step(mode, T, fresh_out=True, tb=TOKEN_BLOCK)
            fn()
            torch.cuda.synchronize()
            peak_tb = torch.cuda.max_memory_allocated() - base
            ms_tb = time_steps(torch, fn, steps, 1)
            out[str(T)]["token_block"] = {"peak_bytes_above_inputs": peak_tb, "ms_per_step": ms_tb,
                                          "tokens_per_s": T / (ms_tb * 1e-3),
                                          "mfma_frac_step": 6 * T * d * V / (ms_tb * 1e-3) / PEAK_BF16}
            del fn
        log(f"[bench] memscan T={T}: {out[str(T)]}")
    return out


def bench_qwen17(torch, kd, synth, dev, steps):
    """Qwen3-1.7B-shaped student head (T=4096, d=2048, V=151,936, K=15):
    tail and renorm, then the other objectives on the same inputs (tail-token
    reverse KL, tail-corrected reverse KL with synthetic sampled tokens,
    tail + 0.1 cross-entropy) and the exact hidden-state KL."""
    c = QWEN17_CFG
    T, d, V, K, chunk = c["T"], c["d"], c["V"], c["K"], c["chunk"]
    h, W, hd, Wd, idx, tlp, mq = build_inputs(torch, kd, synth, dev, c)
    del h, W
    out = loss_out(torch, kd, dev, T, d, V)
    y = torch.from_numpy(synth.token_labels(T, V, seed=5)).to(dev)
    tly = torch.full((T,), -12.0, dtype=torch.float32, device=dev)
    res = {"workload": "Qwen3-1.7B-shaped student head", "T": T, "d": d, "V": V, "K": K, "chunk": chunk}
    cases = {
        "tail": (kd.TAIL, {}),
        "renorm": (kd.RENORM, {}),
        "tail_reverse": (kd.TAIL_REVERSE, {}),
        "reverse_tt": (kd.REVERSE_TT, {"labels": y, "labels_teacher_logp": tly}),
        "tail+ce0.1": (kd.TAIL, {"labels": y, "ce_weight": 0.1}),
        "tail_token_block": (kd.TAIL, {"token_block": TOKEN_BLOCK}),
        "full_token_block": (kd.FULL, {"token_block": TOKEN_BLOCK}),
    }
    for name, (md, kw) in cases.items():
        ws = torch.empty(kd.loss_workspace_bytes(T, d, V, K, md, chunk, kw.get("ce_weight", 0.0),
                                                 kw.get("token_block", 0)), dtype=torch.uint8, device=dev)
        fn = lambda: kd.loss_fwd_bwd(hd, Wd, idx, tlp, mq, mode=md, chunk=chunk, workspace=ws, out=out, **kw)
        ms = time_steps(torch, fn, steps, 2)
        cr = credited_flop(kd, md, T, d, V, K)
        res[name] = {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "mfma_frac_step": cr / (ms * 1e-3) / PEAK_BF16}
        if name == "tail":
            prof = kernel_profile(kd, torch, fn, 3)
            res[name]["kernels_ms_per_step"] = {k: round(v[0], 4) for k, v in prof.items()}
        del ws
    res["kl_hidden"] = bench_kl_hidden(torch, kd, synth, dev, hd, Wd, max(3, steps // 2))
    del hd, Wd, idx, tlp, mq, out
    torch.cuda.empty_cache()
    return res


def bench_kl_hidden(torch, kd, synth, dev, hd, Wd, steps):
    """Exact full-vocabulary KL with the teacher rebuilt from a cached hidden
    state: Qwen3-8B-shaped teacher head (d_t = 4096) over the same student."""
    T, d, V, chunk = QWEN17_CFG["T"], QWEN17_CFG["d"], QWEN17_CFG["V"], QWEN17_CFG["chunk"]
    dt = 4096
    g, U, b = synth.teacher_head(T, dt, V, seed=1)
    gd, Ud, bd = g.to(dev), U.to(dev), b.to(dev)
    del g, U
    ws = torch.empty(kd.lib().kd_kl_hidden_workspace(T, d, dt, V, chunk), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = kd.KlOut(torch.empty((), **f32), torch.empty((T, d), **f32), torch.empty((V, d), **f32),
                   torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32))
    fn = lambda: kd.kl_hidden_fwd_bwd(hd, Wd, gd, Ud, bd, chunk=chunk, workspace=ws, out=out)
    ms = time_steps(torch, fn, steps, 2)
    credited = 2 * T * d * V + 2 * T * dt * V + 4 * T * d * V      # student forward, teacher head, dh + dW
    executed = 2 * (2 * T * d * V) + 2 * (2 * T * dt * V) + 4 * T * d * V
    lse_t = out.lse_t.clone()
    fn_c = lambda: kd.kl_hidden_fwd_bwd(hd, Wd, gd, Ud, bd, chunk=chunk, workspace=ws, out=out,
                                        teacher_lse=lse_t)
    ms_c = time_steps(torch, fn_c, steps, 2)
    executed_c = executed - 2 * T * dt * V
    del gd, Ud, bd, ws, out, lse_t
    torch.cuda.empty_cache()
    return {"workload": "Qwen3-8B-shaped teacher head (hidden-state cache) over the Qwen3-1.7B-shaped student",
            "T": T, "d": d, "d_teacher": dt, "V": V, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "mfma_frac_credited": credited / (ms * 1e-3) / PEAK_BF16,
            "mfma_frac_executed": executed / (ms * 1e-3) / PEAK_BF16,
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
    rows = 2048
    for r0 in range(0, T, rows):
        r1 = min(T, r0 + rows)
        zt = synth.zipf_teacher_logits_device(r1 - r0, V, 2, dev, first_row=r0)
        o = kd.topk_rows(zt, K)
        idx[r0:r1], tlp[r0:r1], mq[r0:r1] = o.idx, o.teacher_logp, o.m_q
        tlp_rev[r0:r1] = torch.gather(zt, 1, sel.idx[r0:r1].long()) - o.lse[:, None]
        del zt, o
    torch.cuda.synchronize()
    out = loss_out(torch, kd, dev, T, d, V)
    res = {"workload": "Llama-3.2-1B-shaped student head", "T": T, "d": d, "V": V, "K": K, "chunk": chunk}
    for name, md in (("renorm", kd.RENORM), ("tail", kd.TAIL), ("full", kd.FULL)):
        ws = torch.empty(kd.loss_workspace_bytes(T, d, V, K, md, chunk), dtype=torch.uint8, device=dev)
        ms = time_steps(torch, lambda: kd.loss_fwd_bwd(hd, Wd, idx, tlp, mq, mode=md, chunk=chunk, workspace=ws,
                                                       out=out), steps, 2)
        cr = credited_flop(kd, md, T, d, V, K)
        res[name] = {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "mfma_frac_step": cr / (ms * 1e-3) / PEAK_BF16}
        if md == kd.RENORM:
            # the sparse backward against its gathered bytes (2 T K d of W rows, as many of h, plus dW written)
            prof = kernel_profile(kd, torch, lambda: kd.loss_fwd_bwd(hd, Wd, idx, tlp, mq, mode=md, chunk=chunk,
                                                                       workspace=ws, out=out), 2)
            gath = 2 * T * K * d
            sdh, sdw = prof.get("k_sparse_dh", (0.0, 0))[0], prof.get("k_sparse_dw", (0.0, 0))[0]
            res[name]["kernels_ms_per_step"] = {k: round(v[0], 4) for k, v in prof.items()}
            res[name]["sparse_dh_gathered_GBps"] = gath / (sdh * 1e-3) / 1e9 if sdh else None
            res[name]["sparse_dw_GBps"] = (gath + 4 * V * d) / (sdw * 1e-3) / 1e9 if sdw else None
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
    the outputs (idx, val, teacher_logp, lse, m_q, k_rho)."""
    T, V, K = 2048, CACHE_CFG["V"], CACHE_CFG["K"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    z = torch.randn((T, V), generator=gen, device=dev, dtype=torch.float32) * 1.1 ** 0.5
    res = {"workload": "teacher-logit rows, N(0, 1.1)", "rows": T, "V": V, "K": K}
    for name, rho in (("no_rho", ()), ("rho", CACHE_CFG["rho"])):
        ws = torch.empty(max(1, kd.lib().kd_topk_rows_workspace(T, V, K, len(rho))), dtype=torch.uint8, device=dev)
        ms = time_steps(torch, lambda: kd.topk_rows(z, K, rho, workspace=ws), steps, 2)
        alg = T * (4 * V) + T * (12 * K + 8 + 4 * len(rho))
        gbps = alg / (ms * 1e-3) / 1e9
        res[name] = {"rho": list(rho), "ms_per_call": ms, "algorithmic_GBps": gbps, "hbm_frac": gbps * 1e9 / PEAK_HBM,
                     "algorithmic_bytes": alg, "traffic": measured_traffic("k_topk_rows", rows_workload_key(len(rho)))}
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
    rows_ms = sum(prof.get(k, (0.0, 0))[0] for k in ROW_KERNELS)
    rows_bytes = T * (4 * V) + T * (12 * K + 8 + 4 * len(rho))
    del gd, Ud, bd, ws
    torch.cuda.empty_cache()
    return {"workload": "Qwen3-8B-shaped teacher head", "T": T, "d": d, "V": V, "K": K, "rho": list(rho),
            "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "gemm_ms": gemm_ms, "gemm_mfma_frac": 2 * T * d * V / (gemm_ms * 1e-3) / PEAK_BF16 if gemm_ms else None,
            "rows_ms": rows_ms, "rows_algorithmic_GBps": rows_bytes / (rows_ms * 1e-3) / 1e9 if rows_ms else None,
            "rows_hbm_frac": rows_bytes / (rows_ms * 1e-3) / PEAK_HBM if rows_ms else None,
            "rows_algorithmic_bytes_per_launch": rows_bytes // (T // 2048),
            "rows_traffic": measured_traffic("k_topk_rows", cache_workload_key()),
            "gemm_traffic": measured_traffic("k_cache_gemm", cache_workload_key()),
            "kernels_ms_per_call": {k: round(v[0], 4) for k, v in prof.items()}}


if __name__ == "__main__":
    main()
