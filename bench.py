"""Benchmark of the hot path on one MI355X.

One step = one pass over the whole path on resident synthetic inputs:
  * HGEMM M = N = K = 8192, fp16 A (row-major) and B (column-major), fp32
    accumulation, fp32 C, alpha = 1, beta = 0;
  * TRMM Out = Aᵀ·B, n = m = 8192, A lower triangular fp16, B fp16, Out fp32,
    recursion split at n/2 down to 256-leaves.

Prints one JSON line.  `value` is the HGEMM throughput in TFLOP/s (2·M·N·K per
call over the average HGEMM kernel time, measured with HIP events on the
stream the kernels run on); the TRMM time per call is reported next to it.
`roofline` prices the HGEMM kernel and `trmm_roofline` the one-launch TRMM
against the dense fp16 MFMA peak; `cpu_baseline` times the fp64 oracle on a
bounded row block of the same HGEMM on this host's cores, and `check` holds
the oracle's verdict on 1024 sampled entries of each timed output;
`inputs_sha256` identifies the inputs.

    python bench.py [--gpus 1] [--steps 50] [--warmup 100] [--no-cpu-baseline]

The default warm-up (about 0.15 s of back-to-back steps) lets the shader
clock settle: under the board power cap it takes a few tens of milliseconds
of sustained MFMA load to reach its steady level, and the first calls after
an idle period run slower.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2516.6   # 256 CU × 4096 flop/clk/CU × 2.4 GHz, dense fp16 MFMA
PEAK_HBM_GBS = 8000.0


def kernel_source_hash():
    """Hash of the HGEMM kernels' code: the sources with // comments and
    blank lines removed, so that a comment edit keeps the profiles valid."""
    import re
    h = hashlib.sha256()
    for f in ("hg_fast.hip", "hg_ring.hip", "hg_kernels.hip", "hg_api.cpp", "hg_internal.h"):
        with open(os.path.join(ROOT, "half_precision_gemm_amd", "csrc", f), encoding="utf-8") as fh:
            code = [re.sub(r"//.*$", "", line).rstrip() for line in fh]
        h.update("\n".join(line for line in code if line).encode())
    return h.hexdigest()[:16]


def profile_record(name, src_hash):
    """A committed counter summary (profiles/<name>.json: HBM bytes per launch,
    shader clock), if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != src_hash:
        return None
    return d


def trmm_phase_bound_us(n, m, leaf, peak_tflops=PEAK_FP16_TFLOPS, hbm_gbs=PEAK_HBM_GBS):
    """Roofline of the recursion scheduled level by level: all leaves, then
    one batched GEMM (beta = 1, fp32 Out read and written) per level.  Each
    phase costs max(flops / MFMA peak, bytes / HBM bandwidth); returns the
    sum over phases in microseconds and the per-phase list."""
    phases = []
    leaves, levels = [], {}

    def rec(o, s_, depth):
        if s_ <= leaf:
            leaves.append(s_)
            return
        h = s_ // 2
        rec(o, h, depth + 1)
        levels.setdefault(depth, []).append((h, s_ - h))
        rec(o + h, s_ - h, depth + 1)
    rec(0, n, 0)
    # leaves: the triangle times B, B read (fp16), Out written (fp32), A's
    # diagonal blocks read (fp16)
    f = sum(L * (L + 1) * m for L in leaves)
    b = 2 * n * m + 4 * n * m + sum(2 * L * L for L in leaves)
    phases.append(("leaves", f, b))
    for d in sorted(levels, reverse=True):
        f = sum(2.0 * m * h * k for h, k in levels[d])
        # A21 (k×h fp16), B2 (k×m fp16), Out1 (h×m fp32) read and written
        b = sum(2 * h * k + 2 * k * m + 8 * h * m for h, k in levels[d])
        phases.append((f"level {d}", f, b))
    out = []
    for name, f, b in phases:
        t = max(f / (peak_tflops * 1e12), b / (hbm_gbs * 1e9)) * 1e6
        out.append({"phase": name, "flops": f, "bytes": b, "bound_us": round(t, 2)})
    return sum(p["bound_us"] for p in out), out


PROBE_SRC = os.path.join(ROOT, "mfma_ceiling.cpp")
PROBE_BIN = os.path.join(ROOT, "mfma_ceiling")


def build_probe(verbose=False):
    """Compile the MFMA-only ceiling probe (mfma_ceiling.cpp, a measurement
    tool of this benchmark, not part of the library) for gfx950."""
    import subprocess
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = PROBE_BIN + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", tmp, PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building mfma_ceiling")
    os.replace(tmp, PROBE_BIN)
    return PROBE_BIN


def mfma_ceiling():
    """Run the MFMA-only ceiling probe (register-resident fp16 operands drawn
    like the benchmark's); None if it is not built or fails."""
    import subprocess
    exe = PROBE_BIN
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        d = json.loads(r.stdout.strip().splitlines()[-1])
        d["frac_of_published_peak"] = round(d["mfma_ceiling_tflops"] / PEAK_FP16_TFLOPS, 4)
        return d
    except Exception as e:  # reported, never fatal for the benchmark
        return {"error": str(e)[:200]}


def cpu_baseline(A, Bt, target_s=15.0):
    """The oracle as it stands on a row block of the 8192³ HGEMM, sized for
    about target_s seconds; reported as TFLOP/s of that block."""
    import numpy as np
    import oracle
    K = A.shape[1]
    r = 96
    t0 = time.perf_counter()
    oracle.hgemm(np.ascontiguousarray(A[:r]), Bt)
    dt = time.perf_counter() - t0
    rows = int(max(8, min(A.shape[0], r * target_s / max(dt, 1e-6))))
    t0 = time.perf_counter()
    oracle.hgemm(np.ascontiguousarray(A[:rows]), Bt)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * Bt.shape[0] * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"fp64 oracle on rows 0..{rows - 1} of the 8192^3 HGEMM "
                      f"({rows}x{Bt.shape[0]} outputs, K={K}), {dt:.1f} s"}


WARM_S = 0.05


def _last_half_avg(ts):
    h = ts[len(ts) // 2:]
    return sum(h) / len(h)


def _time_calls(fn, warmup, reps, stream, warm_s=WARM_S):
    """Per-call HIP-event times (ms) of `reps` calls after `warmup` untimed
    ones (and at least `warm_s` seconds of them: from an idle GPU the shader
    clock takes some milliseconds to settle, longer than 20 calls of a short
    kernel), plus the mean over the same number of back-to-back calls (which
    includes launch cost)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < warm_s:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return ts[len(ts) // 2], ts[0], a.elapsed_time(b) / reps


def config_sweep(hg, stream, main_gemm_ms=None, main_trmm_ms=None, only=None):
    """Every configuration of the workload list: GPU median / min per call
    (HIP events on the kernels' stream), TFLOP/s, % of the fp16 MFMA peak and
    GB/s of compulsory traffic, next to the fp64 oracle on this host (in full
    for the three smaller HGEMMs, on the 1024 sampled entries for 8192³ and
    for the TRMM, with the time per entry).  The 8192³ HGEMM and the TRMM
    reuse the GPU times of the benchmark's timed steps."""
    import numpy as np
    import torch
    import oracle
    import workloads
    dev = torch.device("cuda:0")
    res = {}

    def want(name):
        return only is None or name in only
    reps = {"hgemm_256": 200, "hgemm_1000_ragged": 200, "hgemm_4096": 50}
    for name, w in workloads.WORKLOADS.items():
        if not want(name):
            continue
        print(f"[bench] config {name} ...", file=sys.stderr, flush=True)
        r = {}
        if isinstance(w, workloads.GemmWorkload):
            A, Bt, C = workloads.gemm_inputs(w)
            esz = 2 if w.out_dtype == "f16" else 4
            cbytes = w.M * w.N * esz * (2 if w.beta != 0.0 else 1)
            nbytes = 2 * (w.M * w.K + w.N * w.K) + cbytes
            if name in reps:
                Ad, Btd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
                Cd = torch.from_numpy(C).to(dev)
                fn = lambda: hg.hgemm(Ad, Btd, Cd, w.alpha, w.beta)
                med, mn, b2b = _time_calls(fn, 20, reps[name], stream)
                r.update({"gpu_ms_median": round(med, 5), "gpu_ms_min": round(mn, 5),
                          "gpu_ms_back_to_back_mean": round(b2b, 5), "reps": reps[name]})
                del Ad, Btd, Cd
            elif main_gemm_ms is not None:
                med = main_gemm_ms
                r.update({"gpu_ms_avg": round(med, 5), "from": "the benchmark's timed steps"})
            else:
                med = None
            if med:
                tf = w.flops / (med * 1e-3) / 1e12
                r.update({"tflops": round(tf, 2), "pct_of_fp16_mfma_peak": round(100 * tf / PEAK_FP16_TFLOPS, 3),
                          "compulsory_bytes": nbytes, "gbs": round(nbytes / (med * 1e-3) / 1e9, 1)})
            t0 = time.perf_counter()
            if w.M * w.N <= 4096 * 4096:
                oracle.hgemm(A, Bt, w.alpha, w.beta, C)
                dt = time.perf_counter() - t0
                r["oracle"] = {"seconds": round(dt, 4), "entries": w.M * w.N, "mode": "full",
                               "cores": oracle.num_threads()}
                if w.M * w.N <= 256 * 256:
                    # the same on one thread
                    nt = oracle.num_threads()
                    oracle.set_num_threads(1)
                    t0 = time.perf_counter()
                    oracle.hgemm(A, Bt, w.alpha, w.beta, C)
                    r["oracle"]["seconds_one_thread"] = round(time.perf_counter() - t0, 4)
                    oracle.set_num_threads(nt)
            else:
                ri, cj = workloads.sample_indices(w.seed, w.M, w.N)
                oracle.hgemm_sampled(A, Bt, ri, cj, w.alpha, w.beta, C)
                dt = time.perf_counter() - t0
                r["oracle"] = {"seconds": round(dt, 4), "entries": int(ri.size), "mode": "sampled",
                               "us_per_entry": round(dt / ri.size * 1e6, 2), "cores": oracle.num_threads()}
        else:
            if main_trmm_ms is not None:
                tf = w.flops / (main_trmm_ms * 1e-3) / 1e12
                r.update({"gpu_ms_avg": round(main_trmm_ms, 5), "from": "the benchmark's timed steps",
                          "schedule": "one launch (updates accumulated in registers)",
                          "effective_tflops": round(tf, 2),
                          "pct_of_fp16_mfma_peak": round(100 * tf / PEAK_FP16_TFLOPS, 2),
                          "mfma_bound_us": round(w.flops / (PEAK_FP16_TFLOPS * 1e12) * 1e6, 1)})
            TA, TB = workloads.trmm_inputs(w)
            ri, cj = workloads.sample_indices(w.seed, w.n, w.m)
            t0 = time.perf_counter()
            oracle.trmm_lower_trans_sampled(TA, TB, ri, cj, w.alpha)
            dt = time.perf_counter() - t0
            r["oracle"] = {"seconds": round(dt, 4), "entries": int(ri.size), "mode": "sampled",
                           "us_per_entry": round(dt / ri.size * 1e6, 2), "cores": oracle.num_threads()}
            del TA, TB
        res[name] = r
    if want("hgemm_bias_relu_8192"):
        # Fused bias + ReLU epilogue (next row), on the 8192³ inputs with fp16 out:
        # one launch, against the plain GEMM and the unfused sequence (GEMM, then
        # a bias-add pass and a ReLU pass over C).
        print("[bench] config hgemm_bias_relu_8192 ...", file=sys.stderr, flush=True)
        w = workloads.WORKLOADS["hgemm_8192"]
        A, Bt, _ = workloads.gemm_inputs(w)
        Ad, Btd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
        biasd = torch.from_numpy(np.random.default_rng(w.seed + 7).uniform(-1, 1, w.N)
                                 .astype(np.float32)).to(dev)
        Cd = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
        fused = lambda: hg.hgemm_bias_act(Ad, Btd, Cd, biasd, True)
        plain = lambda: hg.hgemm(Ad, Btd, Cd)

        def unfused():
            hg.hgemm(Ad, Btd, Cd)
            Cd.add_(biasd)
            Cd.relu_()
        tf_ms = _time_calls(fused, 20, 30, stream)
        tp_ms = _time_calls(plain, 20, 30, stream)
        tu_ms = _time_calls(unfused, 5, 30, stream)
        res["hgemm_bias_relu_8192"] = {
            "gpu_ms_median": round(tf_ms[0], 5), "gpu_ms_min": round(tf_ms[1], 5),
            "tflops": round(w.flops / (tf_ms[0] * 1e-3) / 1e12, 2),
            "plain_hgemm_fp16_out_ms_median": round(tp_ms[0], 5),
            "unfused_gemm_then_bias_then_relu_ms_median": round(tu_ms[0], 5),
            "note": "C = relu(A*B + bias), 8192^3, fp16 out, one launch; the unfused sequence adds "
                    "two passes over C (torch elementwise ops)"}
        del Ad, Btd, Cd, biasd
    if only is not None and "torch_matmul_8192" in only:
        # Same-box reference, only when asked for by name: the vendor GEMM
        # behind torch.matmul (fp16 C) on the 8192³ inputs, alternated with
        # this library's fp16-C GEMM, three rounds of 30 timed calls each.
        print("[bench] config torch_matmul_8192 ...", file=sys.stderr, flush=True)
        w = workloads.WORKLOADS["hgemm_8192"]
        A, Bt, _ = workloads.gemm_inputs(w)
        Ad, Btd = torch.from_numpy(A).to(dev), torch.from_numpy(Bt).to(dev)
        Bcm = Btd.t()                      # K×N column-major view: B of C = A·B
        Cv = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
        Co = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
        vendor = lambda: torch.matmul(Ad, Bcm, out=Cv)
        ours = lambda: hg.hgemm(Ad, Btd, Co)
        tv, to = [], []
        for _ in range(3):
            tv.append(_time_calls(vendor, 20, 30, stream)[0])
            to.append(_time_calls(ours, 20, 30, stream)[0])
        torch.cuda.synchronize()
        diff = (Cv.float() - Co.float()).abs().max().item()
        res["torch_matmul_8192"] = {
            "torch_matmul_fp16_out_ms_median": [round(x, 5) for x in tv],
            "hgemm_fp16_out_ms_median": [round(x, 5) for x in to],
            "max_abs_diff_fp16_outputs": diff,
            "note": "same-box reference: torch.matmul (fp16 in, fp16 out) against hgemm with fp16 C "
                    "on the same inputs, alternated, one median per round"}
        del Ad, Btd, Cv, Co
    if want("hgemm_bf16_8192"):
        # bf16 operands (next row): the 8192³ shape, values drawn as the HGEMM
        # workload's and rounded to bf16, fp32 C.
        print("[bench] config hgemm_bf16_8192 ...", file=sys.stderr, flush=True)
        w = workloads.WORKLOADS["hgemm_8192"]
        rng = np.random.default_rng(w.seed)
        Ab = workloads.uniform_bf16(rng, (w.M, w.K))
        Bb = workloads.uniform_bf16(rng, (w.N, w.K))
        Ad = torch.from_numpy(Ab.view(np.int16)).to(dev).view(torch.bfloat16)
        Btd = torch.from_numpy(Bb.view(np.int16)).to(dev).view(torch.bfloat16)
        Cd = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
        tb = _time_calls(lambda: hg.hgemm_bf16(Ad, Btd, Cd), 20, 30, stream)
        tfb = w.flops / (tb[0] * 1e-3) / 1e12
        # the same with the fused bias + ReLU and a bf16 C
        biasd = torch.from_numpy(np.random.default_rng(w.seed + 7).uniform(-1, 1, w.N)
                                 .astype(np.float32)).to(dev)
        Cb = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        tbe = _time_calls(lambda: hg.hgemm_bias_act(Ad, Btd, Cb, biasd, True), 20, 30, stream)
        res["hgemm_bf16_8192"] = {
            "gpu_ms_median": round(tb[0], 5), "gpu_ms_min": round(tb[1], 5), "tflops": round(tfb, 2),
            "pct_of_bf16_mfma_peak": round(100 * tfb / PEAK_FP16_TFLOPS, 3),
            "bias_relu_bf16_out_ms_median": round(tbe[0], 5),
            "bias_relu_bf16_out_tflops": round(w.flops / (tbe[0] * 1e-3) / 1e12, 2),
            "note": "bf16 A, B (v_mfma_f32_16x16x32_bf16), fp32 accumulation and C; dense bf16 peak "
                    "equals the fp16 one"}
        del Ad, Btd, Cd, Ab, Bb
    if want("hgemm_rowmajor_b_8192"):
        # Row-major B (next row; the GPU architecture page's matmul layout):
        # 8192³, fp32 C, B transposed into a workspace, then the GEMM.
        print("[bench] config hgemm_rowmajor_b_8192 ...", file=sys.stderr, flush=True)
        w = workloads.WORKLOADS["hgemm_8192"]
        A, Bt, _ = workloads.gemm_inputs(w)
        Ad = torch.from_numpy(A).to(dev)
        Brd = torch.from_numpy(np.ascontiguousarray(Bt.T)).to(dev)
        Cd = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
        work = torch.empty(hg.lib.hg_hgemm_layout_workspace_size(0, 0, w.M, w.N, w.K), dtype=torch.uint8,
                           device=dev)
        tl = _time_calls(lambda: hg.hgemm_layout(Ad, Brd, Cd, False, True, work=work), 20, 30, stream)
        res["hgemm_rowmajor_b_8192"] = {
            "gpu_ms_median": round(tl[0], 5), "gpu_ms_min": round(tl[1], 5),
            "tflops": round(w.flops / (tl[0] * 1e-3) / 1e12, 2),
            "note": "B given K x N row-major: one tiled transpose (128 MiB read + written) into the "
                    "workspace, then the K-contiguous GEMM"}
        del Ad, Brd, Cd, work, A, Bt
    if want("trmm_8192_by_level"):
        # The recursion scheduled as the page describes it: one batched launch
        # for the 32 leaves, then one batched beta = 1 GEMM launch per level,
        # deepest first (Out read and written in fp32 at every level); priced
        # against that schedule's per-phase roofline.
        print("[bench] config trmm_8192_by_level ...", file=sys.stderr, flush=True)
        w = workloads.WORKLOADS["trmm_8192"]
        TA, TB = workloads.trmm_inputs(w)
        Ad, Bd = torch.from_numpy(TA).to(dev), torch.from_numpy(TB).to(dev)
        Od = torch.empty((w.m, w.n), dtype=torch.float32, device=dev)
        ts = _time_calls(lambda: hg.trmm_lower_trans_by_level(Ad, Bd, Od, w.alpha, w.leaf), 5, 20, stream)
        bound_us, phases = trmm_phase_bound_us(w.n, w.m, w.leaf)
        res["trmm_8192_by_level"] = {
            "gpu_ms_median": round(ts[0], 5), "gpu_ms_min": round(ts[1], 5),
            "effective_tflops": round(w.flops / (ts[0] * 1e-3) / 1e12, 2),
            "phase_bound_us": round(bound_us, 1),
            "pct_of_phase_bound": round(100 * bound_us * 1e-3 / ts[0], 1),
            "phases": phases,
            "note": "leaves in one launch, then one beta = 1 GEMM launch per recursion level; "
                    "each phase bounded by max(flops / 2516.6 TFLOP/s, bytes / 8 TB/s)"}
        del Ad, Bd, Od, TA, TB
    if want("trmm_4096x256"):
        # Skinny right-hand side (next row): the TRMM page's usage example,
        # n = 4096, m = 256, one launch of 64x64 tiles; next to it the per-level
        # schedule on 4 streams.
        print("[bench] config trmm_4096x256 ...", file=sys.stderr, flush=True)
        w = workloads.TrmmWorkload("trmm_4096x256", 4096, 256, 1.0, 256, 6)
        TA, TB = workloads.trmm_inputs(w)
        Ad, Bd = torch.from_numpy(TA).to(dev), torch.from_numpy(TB).to(dev)
        Od = torch.empty((w.m, w.n), dtype=torch.float32, device=dev)
        ts = _time_calls(lambda: hg.trmm_lower_trans(Ad, Bd, Od, w.alpha, w.leaf), 20, 50, stream)
        # the same recursion with each phase's launches on 4 streams (the page's
        # usage notes) instead of one batched launch per phase
        streams4 = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(3)]
        t4 = _time_calls(lambda: hg.trmm_lower_trans_streams(Ad, Bd, Od, streams4, w.alpha, w.leaf), 20, 50,
                         stream)
        # compulsory traffic: A's lower triangle and B read once, Out written once (fp32)
        nb = w.n * (w.n + 1) + 2 * w.n * w.m + 4 * w.n * w.m
        res["trmm_4096x256"] = {"gpu_ms_median": round(ts[0], 5), "gpu_ms_min": round(ts[1], 5),
                                "gpu_ms_back_to_back_mean": round(ts[2], 5),
                                "effective_tflops": round(w.flops / (ts[0] * 1e-3) / 1e12, 2),
                                "compulsory_bytes": nb, "gbs": round(nb / (ts[0] * 1e-3) / 1e9, 1),
                                "four_streams_ms_median": round(t4[0], 5),
                                "note": "B 4096x256 (the TRMM page's usage example): the recursion in one launch "
                                        "of 64x64 tiles (too few 256x256 tiles for the big one-launch kernel)"}
        del Ad, Bd, Od, TA, TB
    if want("trmm_8192_lower_notrans"):
        # The page's usage call is the lower, non-transposed product (next row):
        # n = m = 8192 through hg_trmm (index map of A, B and Out row-reversed).
        print("[bench] config trmm_8192_lower_notrans ...", file=sys.stderr, flush=True)
        w = workloads.WORKLOADS["trmm_8192"]
        TA, TB = workloads.trmm_inputs(w)
        Ad, Bd = torch.from_numpy(TA).to(dev), torch.from_numpy(TB).to(dev)
        Od = torch.empty((w.m, w.n), dtype=torch.float32, device=dev)
        work = torch.empty(hg.trmm_workspace_size(w.n, w.m, "L", False), dtype=torch.uint8, device=dev)
        ts = _time_calls(lambda: hg.trmm(Ad, Bd, Od, w.alpha, "L", False, w.leaf, work), 5, 20, stream)
        res["trmm_8192_lower_notrans"] = {
            "gpu_ms_median": round(ts[0], 5), "gpu_ms_min": round(ts[1], 5),
            "effective_tflops": round(w.flops / (ts[0] * 1e-3) / 1e12, 2),
            "note": "Out = A*B, A lower (the TRMM page's usage call): transpose-and-reverse copy of A, "
                    "B and Out row-reversed around the lower-transposed recursion"}
        del Ad, Bd, Od, TA, TB, work
    if want("hgemm_splitk_512x512x65536"):
        # Split-K (next row): a 512×512 C has 16 tiles of 128×128 for 256 CUs
        # while K = 65536 is long; hgemm_splitk (slices chosen from the shape)
        # against the plain call.
        print("[bench] config hgemm_splitk_512x512x65536 ...", file=sys.stderr, flush=True)
        M = N = 512
        K = 65536
        rng = np.random.default_rng(8)
        Ad = torch.from_numpy(workloads.uniform_f16(rng, (M, K))).to(dev)
        Btd = torch.from_numpy(workloads.uniform_f16(rng, (N, K))).to(dev)
        Cd = torch.empty((M, N), dtype=torch.float32, device=dev)
        work = torch.empty(hg.splitk_workspace_size(M, N, K, 0), dtype=torch.uint8, device=dev)
        plain = _time_calls(lambda: hg.hgemm(Ad, Btd, Cd), 5, 20, stream)
        split = _time_calls(lambda: hg.hgemm_splitk(Ad, Btd, Cd, 1.0, 0.0, 0, work), 5, 20, stream)
        flops = 2.0 * M * N * K
        res["hgemm_splitk_512x512x65536"] = {
            "gpu_ms_median": round(split[0], 5), "gpu_ms_min": round(split[1], 5),
            "tflops": round(flops / (split[0] * 1e-3) / 1e12, 2),
            "plain_hgemm_ms_median": round(plain[0], 5),
            "plain_hgemm_tflops": round(flops / (plain[0] * 1e-3) / 1e12, 2),
            "note": "fp32 C; K cut into slices run side by side, partials summed in order in fp32"}
        del Ad, Btd, Cd, work
    if want("trmm_8192_inplace"):
        # In-place form B <- A*B (fp16 B overwritten), lower and not transposed.
        # B is restored from a copy before each timed call, outside the events.
        print("[bench] config trmm_8192_inplace ...", file=sys.stderr, flush=True)
        w = workloads.WORKLOADS["trmm_8192"]
        TA, TB = workloads.trmm_inputs(w)
        Ad, B0 = torch.from_numpy(TA).to(dev), torch.from_numpy(TB).to(dev)
        Bd = torch.empty_like(B0)
        work = torch.empty(hg.lib.hg_trmm_inplace_workspace_size(0, 0, w.n, w.m), dtype=torch.uint8,
                           device=dev)
        ts = []
        for i in range(25):
            Bd.copy_(B0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            hg.trmm_inplace(Ad, Bd, w.alpha, "L", False, w.leaf, work)
            b.record(stream)
            torch.cuda.synchronize()
            if i >= 5:
                ts.append(a.elapsed_time(b))
        ts.sort()
        res["trmm_8192_inplace"] = {
            "gpu_ms_median": round(ts[len(ts) // 2], 5), "gpu_ms_min": round(ts[0], 5),
            "effective_tflops": round(w.flops / (ts[len(ts) // 2] * 1e-3) / 1e12, 2),
            "note": "B <- A*B in fp16, A lower: the lower, non-transposed product in one launch "
                    "whose tiles round alpha*acc (fp32) to fp16 into the workspace, then one "
                    "device-to-device copy into B"}
        del Ad, B0, Bd, TA, TB, work
    for name, w in workloads.TRSM_WORKLOADS.items():
        if not want(name):
            continue
        print(f"[bench] config {name} ...", file=sys.stderr, flush=True)
        A_cm, B_cm = workloads.trsm_inputs(w)
        Ad, Bd = torch.from_numpy(A_cm).to(dev), torch.from_numpy(B_cm).to(dev)
        Od = torch.empty((w.m, w.n), dtype=torch.float32, device=dev)
        work = torch.empty(hg.trsm_workspace_size(w.n, w.m, w.leaf), dtype=torch.uint8, device=dev)
        fn = lambda: hg.trsm_lower_trans(Ad, Bd, Od, w.alpha, w.leaf, work)
        med, mn, b2b = _time_calls(fn, 5, 20, stream)
        tf = w.flops / (med * 1e-3) / 1e12
        # compulsory traffic: A's lower triangle and B read once, X written once (fp32)
        nbytes = w.n * (w.n + 1) + 2 * w.n * w.m + 4 * w.n * w.m
        r = {"gpu_ms_median": round(med, 5), "gpu_ms_min": round(mn, 5),
             "gpu_ms_back_to_back_mean": round(b2b, 5), "reps": 20,
             "tflops": round(tf, 2), "pct_of_fp16_mfma_peak": round(100 * tf / PEAK_FP16_TFLOPS, 3),
             "flops": "n^2*m", "compulsory_bytes": nbytes,
             "note": "triangular solve X = alpha*A^-T*B (next row after the hot path); "
                     "not part of the timed step"}
        del Ad, Bd, Od, work
        cols = np.array([0, w.m // 3, 2 * w.m // 3, w.m - 1], dtype=np.int64)
        t0 = time.perf_counter()
        oracle.trsm_lower_trans_cols(A_cm, B_cm, cols, w.alpha)
        dt = time.perf_counter() - t0
        r["oracle"] = {"seconds": round(dt, 4), "entries": int(cols.size * w.n),
                       "mode": f"{cols.size} full columns",
                       "us_per_column": round(dt / cols.size * 1e6, 1), "cores": oracle.num_threads()}
        res[name] = r
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trmm", action="store_true", help="time the HGEMM alone")
    ap.add_argument("--config", action="append", default=None, metavar="NAME",
                    help="run only this entry of the per-configuration sweep (repeatable)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration sweep (GPU and oracle times of every workload)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the MFMA-only throughput ceiling probe")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run one plain device-to-device copy of BYTES bytes, the "
                         "reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path is a single-GPU kernel; multi-GPU sharding is a design note only)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import half_precision_gemm_amd as hg
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wg = workloads.WORKLOADS["hgemm_8192"]
    wt = workloads.WORKLOADS["trmm_8192"]
    A, Bt, _ = workloads.gemm_inputs(wg)
    inputs = {"hgemm_8192": {"A": workloads.sha256(A), "Bt": workloads.sha256(Bt)}}
    Ad = torch.from_numpy(A).to(dev)
    Btd = torch.from_numpy(Bt).to(dev)
    Cd = torch.empty((wg.M, wg.N), dtype=torch.float32, device=dev)
    do_trmm = not args.no_trmm
    if do_trmm:
        TA, TB = workloads.trmm_inputs(wt)
        inputs["trmm_8192"] = {"A_cm": workloads.sha256(TA), "B_cm": workloads.sha256(TB)}
        TAd = torch.from_numpy(TA).to(dev)
        TBd = torch.from_numpy(TB).to(dev)
        del TA, TB
        TOut = torch.empty((wt.m, wt.n), dtype=torch.float32, device=dev)

    stream = torch.cuda.current_stream(dev)

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        hg.hgemm(Ad, Btd, Cd, wg.alpha, wg.beta)
        if evs is not None:
            evs[1].record(stream)
        if do_trmm:
            hg.trmm_lower_trans(TAd, TBd, TOut, wt.alpha, wt.leaf)
            if evs is not None:
                evs[2].record(stream)

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for k in range(args.steps):
        step(evs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    gemm_ms = [e[0].elapsed_time(e[1]) for e in evs]
    trmm_ms = [e[1].elapsed_time(e[2]) for e in evs] if do_trmm else []
    gemm_avg = sum(gemm_ms) / len(gemm_ms)
    tflops = wg.flops / (gemm_avg * 1e-3) / 1e12
    print(f"[bench] timed {args.steps} steps: hgemm avg {gemm_avg:.4f} ms "
          f"(min {min(gemm_ms):.4f}), {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)

    # The timed outputs at the 1024 sampled entries of each workload (the
    # oracle checks them after the sweep, in the CPU-baseline leg).
    ri_g, cj_g = workloads.sample_indices(wg.seed, wg.M, wg.N)
    gemm_samples = Cd[torch.from_numpy(ri_g).to(dev), torch.from_numpy(cj_g).to(dev)].cpu().numpy()
    if do_trmm:
        ri_t, cj_t = workloads.sample_indices(wt.seed, wt.n, wt.m)
        # Out(i, j) of the column-major n×m output sits at TOut[j, i]
        trmm_samples = TOut[torch.from_numpy(cj_t).to(dev), torch.from_numpy(ri_t).to(dev)].cpu().numpy()

    src_hash = kernel_source_hash()
    prof_g = profile_record("hgemm_8192_traffic", src_hash) or {}
    prof_t = profile_record("trmm_8192_traffic", src_hash) or {}

    def clock_fields(prof, achieved):
        # shader clock from SQ_BUSY_CYCLES over the kernel's duration in the
        # counter run, and the peak at that clock (256 CU × 4096 flop/clk)
        ghz = prof.get("shader_clock_ghz")
        if not ghz:
            return {"shader_clock_ghz": None, "frac_of_peak_at_that_clock": None}
        return {"shader_clock_ghz": ghz,
                "frac_of_peak_at_that_clock": round(achieved / (256 * 4096 * ghz * 1e-3), 4)}

    out = {
        "metric": "HGEMM TFLOP/s + % of MI355X FP16 MFMA peak at 8192^3; TRMM ms at n=8192",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 in, f32 accumulate",
        "data": "synthetic: numpy PCG64 uniform[-1,1] rounded to fp16, seeds 3 (HGEMM) and 4 (TRMM)",
        "config": {"workload": "hgemm_8192 + trmm_8192",
                   "hgemm": {"M": wg.M, "N": wg.N, "K": wg.K, "A": "row-major fp16",
                             "B": "col-major fp16", "C": "fp32", "alpha": 1.0, "beta": 0.0},
                   "trmm": ({"n": wt.n, "m": wt.m, "leaf": wt.leaf, "out": "fp32",
                             "A": "lower, col-major fp16", "B": "col-major fp16"}
                            if do_trmm else None)},
        "pct_of_fp16_mfma_peak": round(100.0 * tflops / PEAK_FP16_TFLOPS, 2),
        # Per step, in order: from an idle GPU the board's power control lets
        # the first launches run fast, then cuts the clock and takes about
        # twenty launches of this size to settle, so the average over few
        # warm-up steps sits above the later steps.
        "hgemm_ms": {"avg": round(gemm_avg, 4), "min": round(min(gemm_ms), 4),
                     "max": round(max(gemm_ms), 4),
                     "last_half_avg": round(_last_half_avg(gemm_ms), 4),
                     "per_step": [round(t, 4) for t in gemm_ms]},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP16_TFLOPS, 4),
                     "traffic": prof_g.get("hbm_bytes_per_launch"),
                     "kernel": "hgemm_fast_kernel (256x256 tile, 4 waves, v_mfma_f32_16x16x32_f16, 64-wide K stages) at M=N=K=8192, fp32 out",
                     "algorithmic_flops_per_launch": wg.flops,
                     "algorithmic_bytes_per_launch": 2 * (wg.M * wg.K + wg.N * wg.K) + 4 * wg.M * wg.N,
                     **clock_fields(prof_g, tflops)},
        "kernel_source_sha256_16": src_hash,
    }
    if do_trmm:
        tavg = sum(trmm_ms) / len(trmm_ms)
        ttf = wt.flops / (tavg * 1e-3) / 1e12
        out["trmm_ms"] = {"avg": round(tavg, 4), "min": round(min(trmm_ms), 4),
                          "max": round(max(trmm_ms), 4),
                          "last_half_avg": round(_last_half_avg(trmm_ms), 4),
                          "per_step": [round(t, 4) for t in trmm_ms]}
        out["trmm_effective_tflops"] = round(ttf, 2)
        # The one-launch TRMM is MFMA-bound: n(n+1)m useful flops against
        # 0.47 GB compulsory traffic (A's lower triangle, B, Out in fp32).
        out["trmm_roofline"] = {
            "bound": "mfma", "achieved": round(ttf, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ttf / PEAK_FP16_TFLOPS, 4),
            "bound_ms": round(wt.flops / (PEAK_FP16_TFLOPS * 1e12) * 1e3, 4),
            "traffic": prof_t.get("hbm_bytes_per_launch"),
            "kernel": "hgemm_fast_kernel, one-launch recursive TRMM (each 256x256 output tile walks its "
                      "leaf and its updates in its fp32 accumulators), n = m = 8192, leaf 256, fp32 out",
            "algorithmic_flops_per_launch": wt.flops,
            "algorithmic_bytes_per_launch": wt.n * (wt.n + 1) + 2 * wt.n * wt.m + 4 * wt.n * wt.m,
            **clock_fields(prof_t, ttf)}
    if not args.no_configs:
        out["configs"] = config_sweep(hg, stream, gemm_avg, only=args.config, main_trmm_ms=
                                      (sum(trmm_ms) / len(trmm_ms)) if do_trmm else None)
    if not args.no_ceiling:
        out["mfma_ceiling"] = mfma_ceiling()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(A, Bt)
        # The oracle on the sampled entries of what the timed steps computed.
        import oracle
        from tests.tolerance import bound
        chk = {}
        ref = oracle.hgemm_sampled(A, Bt, ri_g, cj_g, wg.alpha, wg.beta)
        err = np.abs(gemm_samples.astype(np.float64) - ref)
        chk["hgemm_8192"] = {"entries": int(ri_g.size), "max_abs_err": float(np.nanmax(err)),
                             "max_err_over_tolerance": float(np.nanmax(err / bound(wg.K, ref))),
                             "pass": bool((err <= bound(wg.K, ref)).all())}
        if do_trmm:
            TA, TB = workloads.trmm_inputs(wt)
            ref = oracle.trmm_lower_trans_sampled(TA, TB, ri_t, cj_t, wt.alpha)
            err = np.abs(trmm_samples.astype(np.float64) - ref)
            chk["trmm_8192"] = {"entries": int(ri_t.size), "max_abs_err": float(np.nanmax(err)),
                                "max_err_over_tolerance": float(np.nanmax(err / bound(wt.n, ref))),
                                "pass": bool((err <= bound(wt.n, ref)).all())}
            del TA, TB
        chk["rule"] = "|gpu - oracle| <= 1e-3*sqrt(K) + 2^-10*|oracle| (K = n for the TRMM)"
        out["check"] = chk
    golden = os.path.join(ROOT, "tests", "golden", "input_sha256.json")
    if os.path.exists(golden):
        with open(golden) as f:
            g = json.load(f)
        inputs["match_pinned_hashes"] = all(g.get(k, {}).get(a) == h for k, v in inputs.items()
                                            if isinstance(v, dict) for a, h in v.items())
    out["inputs_sha256"] = inputs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
