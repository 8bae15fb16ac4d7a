"""Benchmark: the full synthetic FP4 exploration rollout on one MI355X.

One step = one Stage-1 pass over 96 candidates x 4096 tokens x 3072 dims:
re-quantize the 8 weights (MXFP4), 6 Euler steps of a 4-block residual MLP
velocity (RMSNorm->MXFP4 -> FP4 GEMM 3072->12288 -> GELU->MXFP4 -> FP4 GEMM
12288->3072 + residual), proxy reward, top-12 / bottom-12 selection. All
inputs are resident in HBM before timing starts.

Prints one JSON line: candidates/s, the FP4 GEMM's achieved TFLOP/s against
the MXFP4 peak (HIP events around every GEMM launch of the timed steps), the
CPU oracle timed on bounded samples, rank agreement against the same rollout
with bf16 linears, and the Stage-2 block -- the BF16 regeneration of the
selected seeds and the FP4 step-count ablation -- all outside the timed
region.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--chunk C] [--no-cpu-baseline] [--no-rank-agreement]
                    [--no-stage2] [--ablation]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4 GEMM TFLOP/s (% of MI355X MXFP4 peak); FP4 rollout candidates/sec"
PEAK_FP4 = 10.1e15      # MI355X dense MXFP4 MFMA, FLOP/s
PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # bytes/s

# Bytes each GEMM launch moves between L2 and the memory fabric (Infinity
# Cache or HBM). By default they are measured in every run (measure_counters:
# rocprofv3 counter passes over one rollout step, in child processes, before
# this process touches the GPU). Where that cannot run, the figure of
# the committed profile is reported instead, from FETCH_SIZE (x2: every read
# request is 128 bytes, which the counter's formula weighs as 64) and
# WRITE_SIZE (x1) runs of this workload averaged over a step's GEMM launches;
# it holds only for the kernel sources it was taken with (null once those
# change). See profiles/rollout_96x4096x3072_kernels.md.
GEMM_TRAFFIC = {"sources": {"gemm_mx.hip": "ca85b2592cd118d5", "gemm_common.h": "d8952e405ad1a5b1",
                            "mx_common.h": "b3986ff8b932e392", "common.h": "ddd8489d61c6db40"},
                "hidden": "f32", "bytes_per_launch": 19.50e9}
COPY_BYTES = 1 << 30    # the known-size copy that calibrates the byte counters


def gemm_traffic(hidden):
    import hashlib
    if hidden != GEMM_TRAFFIC["hidden"]:
        return None
    csrc = os.path.join(ROOT, "fp4_quantized_diffusion_amd", "csrc")
    for name, digest in GEMM_TRAFFIC["sources"].items():
        with open(os.path.join(csrc, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != digest:
                return None
    return GEMM_TRAFFIC["bytes_per_launch"]


def gemm_variants(cfg):
    """The rollout step's GEMM launches by epilogue: (kernel template, launches
    per step). The first linear of every block quantizes GELU in its epilogue
    (of the fp32 sums, or with cfg["hidden_act"] == "bf16" of their bf16
    rounding); the second adds the residual, except in the last block, where
    it also takes the Euler step, and in the last step also the reward
    partial sums."""
    b, s = cfg["blocks"], cfg["steps"]
    gelu = "gemm_fp4_kernel<0, 3, 2>" if cfg.get("hidden_act") == "bf16" else "gemm_fp4_kernel<0, 5, 2>"
    return {"gelu_mxfp4": (gelu, b * s), "residual": ("gemm_fp4_kernel<0, 1, 2>", (b - 1) * s),
            "euler": ("gemm_fp4_kernel<0, 2, 2>", s - 1), "euler_reward": ("gemm_fp4_kernel<0, 4, 2>", 1)}


CLASS_NAMES = ("flux", "sana", "sd35")
CLASS_TMPL = "gemm_fp4_kernel<1, 0, 2>"   # bf16 C, panel operands: the class GEMMs (the rollout never uses it)
PROBE_CLASS_LAUNCHES = 2


def class_key(name, which, m, k, n):
    from fp4_quantized_diffusion_amd import inputs
    return f"{name}_{inputs.class_gemm(name, which)[0]}_{m}x{k}x{n}"


def class_shapes():
    """[(key, m, k, n)] of the class GEMMs, in the order the probe launches them."""
    from fp4_quantized_diffusion_amd import inputs
    out = []
    for name in CLASS_NAMES:
        for which in (1, 2):
            _, k, n = inputs.class_gemm(name, which)
            m = inputs.CLASS_SHAPES[name]["m"]
            out.append((class_key(name, which, m, k, n), m, k, n))
    return out


def traffic_probe(cfg):
    """The program measure_counters runs under rocprofv3: one device copy of
    COPY_BYTES, one step of the benchmark's rollout (the same inputs, buffers
    and launches as the timed steps), then PROBE_CLASS_LAUNCHES launches of
    each class GEMM (MXFP4, bf16 C) in class_shapes() order."""
    import torch
    import fp4_quantized_diffusion_amd as fq
    from fp4_quantized_diffusion_amd import inputs
    from fp4_quantized_diffusion_amd.rollout import Fp4Rollout
    fq.load_library()
    dev = "cuda:0"
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    noise, w1, w2, u = make_inputs(cfg, dev)
    work = torch.empty_like(noise)
    ro = Fp4Rollout(w1, w2, u, steps=cfg["steps"], k_top=cfg["k_top"], k_bottom=cfg["k_bottom"], chunk=cfg["n_cand"],
                    hidden=cfg["hidden_act"])
    ro.run(noise, work)
    torch.cuda.synchronize()
    print("counter probe: rollout step done", flush=True)
    del ro, noise, work, w1, w2
    torch.cuda.empty_cache()
    for name in CLASS_NAMES:
        for which in (1, 2):
            a, w = inputs.class_linear_device(name, which, dev)
            qa, qb = fq.quantize(a, "mx", layout="panel"), fq.quantize(w, "mx", layout="panel")
            c = torch.empty((a.shape[0], w.shape[0]), dtype=torch.bfloat16, device=dev)
            for _ in range(PROBE_CLASS_LAUNCHES):
                fq.gemm(qa, qb, "bf16", out=c)
            torch.cuda.synchronize()
            del a, w, qa, qb, c
    print("counter probe: done", flush=True)


def _under_profiler(env=None):
    env = os.environ if env is None else env
    return any(k.startswith(("ROCPROF", "ROCP_")) for k in env) or "rocprof" in env.get("LD_PRELOAD", "")


# The counter passes, one rocprofv3 run each (each within one pass's limits per
# counter block): bytes read and written past L2, then MFMA busy cycles and
# GPU-active cycles (the shader clock over each dispatch's duration).
COUNTER_PASSES = (("FETCH_SIZE",), ("WRITE_SIZE",), ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"))
N_XCD, N_SIMD = 8, 1024   # GRBM_GUI_ACTIVE sums the 8 XCDs; MFMA busy cycles sum 256 CUs x 4 SIMDs


def counter_dispatches(db, counters, variants):
    """The dispatches of a rocprofv3 results database, grouped into the
    calibration copy ("copy": device copies dispatched before the rollout's
    first GEMM), the rollout's GEMM variants and the class GEMMs ("class", in
    dispatch order): lists of (duration ns, {counter: value}). None when the
    copy or a variant has no dispatch."""
    import sqlite3
    con = sqlite3.connect(db)
    try:
        rows = con.execute("select dispatch_id, kernel_name, counter_name, value, start, end "
                           "from counters_collection").fetchall()
    finally:
        con.close()
    disp = {}
    for did, kname, cname, v, t0, t1 in rows:
        if cname in counters:
            d = disp.setdefault(did, [kname, (t1 - t0) if t0 is not None and t1 is not None else None, {}])
            d[2][cname] = float(v)
    def is_(kname, tmpl):
        return tmpl + "(" in kname or kname.endswith(tmpl)
    groups = {name: [] for name in variants}
    copies, cls, first_gemm = [], [], None
    for did in sorted(disp):
        kname, dur, vals = disp[did]
        if len(vals) != len(counters):
            continue
        if "__amd_rocclr_copyBuffer" in kname:
            copies.append((did, dur, vals))
        for name, (tmpl, _) in variants.items():
            if is_(kname, tmpl):
                groups[name].append((dur, vals))
                first_gemm = did if first_gemm is None else first_gemm
        if is_(kname, CLASS_TMPL):
            cls.append((dur, vals))
    # the calibration copy runs before anything else copies on the device;
    # later copies (input generation) are not it
    groups["copy"] = [(dur, vals) for did, dur, vals in copies if first_gemm is None or did < first_gemm]
    if not all(groups.values()):
        return None
    groups["class"] = cls
    return groups


def weighted_traffic(per, variants):
    """Mean read + write bytes per launch over a step's GEMM launches."""
    total = sum(n for _, n in variants.values())
    return sum((per[k]["read_GB"] + per[k]["write_GB"]) * 1e9 * variants[k][1] for k in variants) / total


def clock_stats(disps):
    """Shader clock (GHz) and MFMA busy fraction over dispatches of the clock
    pass: GPU-active cycles of one XCD over the dispatches' time, and MFMA busy
    cycles per SIMD over those cycles."""
    cyc = sum(v["GRBM_GUI_ACTIVE"] for _, v in disps) / N_XCD
    ns = sum(d for d, _ in disps)
    busy = sum(v["SQ_VALU_MFMA_BUSY_CYCLES"] for _, v in disps) / (cyc * N_SIMD)
    return cyc / ns, busy


def class_groups(disps, shapes, per_shape=PROBE_CLASS_LAUNCHES):
    """Pairs (key, dispatches) of the class GEMMs from their dispatches in
    launch order; none unless every shape has its launches."""
    if len(disps) != per_shape * len(shapes):
        return []
    return [(key, disps[i * per_shape:(i + 1) * per_shape]) for i, (key, _, _, _) in enumerate(shapes)]


def measure_counters(cfg, timeout_s=420):
    """Counters of the rollout's GEMMs, taken now: child processes run
    traffic_probe under `rocprofv3 --pmc <counters>`, one run per entry of
    COUNTER_PASSES. Gives the bytes per launch between L2 and the memory
    fabric (each byte counter scaled by what it reads for the COPY_BYTES copy
    in the same run), and each variant's shader clock and MFMA busy fraction.
    Returns (dict, None) or (None, reason). Must run before this process
    initializes the GPU, so the children start from a process with no GPU
    state."""
    import shutil
    import signal
    import subprocess
    import tempfile
    prof = shutil.which("rocprofv3")
    if prof is None:
        return None, "rocprofv3 not on PATH"
    tmp = tempfile.mkdtemp(prefix="fp4r_counters_")
    env = dict(os.environ)
    env.setdefault("TMPDIR", "/tmp")
    variants = gemm_variants(cfg)
    shapes = class_shapes()
    per = {name: {} for name in variants}
    per_class = {}
    factors = {}
    all_disp = []
    try:
        for i, counters in enumerate(COUNTER_PASSES):
            t0 = time.time()
            tag = "+".join(counters)
            out_name = f"pass{i}"
            cmd = [prof, "--pmc", *counters, "-d", tmp, "-o", out_name, "--", sys.executable,
                   os.path.join(ROOT, "bench.py"), "--traffic-probe", "--tokens", str(cfg["tokens"]),
                   "--hidden", cfg["hidden_act"]]
            logf = os.path.join(tmp, out_name + ".log")
            with open(logf, "w") as lf:
                p = subprocess.Popen(cmd, stdout=lf, stderr=subprocess.STDOUT, cwd=tmp, env=env,
                                     start_new_session=True)
                try:
                    rc = p.wait(timeout=timeout_s)
                except subprocess.TimeoutExpired:
                    os.killpg(p.pid, signal.SIGKILL)
                    p.wait()
                    return None, f"{tag} pass exceeded {timeout_s} s"
            with open(logf, errors="replace") as lf:
                text = lf.read()
            db = os.path.join(tmp, out_name + "_results.db")
            # rocprofv3 may end with a non-zero status after the program's own
            # end; the results count when the probe finished and the file is there
            if "counter probe: rollout step done" not in text or not os.path.exists(db):
                return None, f"{tag} pass failed (status {rc}): {text.strip().splitlines()[-1:]}"
            g = counter_dispatches(db, counters, variants)
            if g is None or any(len(g[n]) != variants[n][1] for n in variants):
                return None, f"{tag} pass: the GEMM launches counted differ from one step's"
            if counters[0] in ("FETCH_SIZE", "WRITE_SIZE"):
                c = counters[0]
                key = "read" if c == "FETCH_SIZE" else "write"
                f = COPY_BYTES / (sum(v[c] for _, v in g["copy"]) * 1024.0)
                # the copy reads and writes COPY_BYTES: FETCH_SIZE counts 128-byte reads as 64 (x2), WRITE_SIZE x1
                if not (1.6 < f < 2.4 if key == "read" else 0.8 < f < 1.2):
                    return None, f"{c} copy calibration factor {f:.3f} is outside its expected range"
                factors[key] = round(f, 4)
                for name in variants:
                    gb = [v[c] * 1024.0 * f / 1e9 for _, v in g[name]]
                    per[name][key + "_GB"] = round(sum(gb) / len(gb), 3)
                    per[name][key + "_GB_range"] = [round(min(gb), 3), round(max(gb), 3)]
                for ck, ds in class_groups(g["class"], shapes):
                    per_class.setdefault(ck, {})[key + "_GB"] = round(
                        sum(v[c] for _, v in ds) / len(ds) * 1024.0 * f / 1e9, 3)
            else:
                if any(d is None or d <= 0 for name in variants for d, _ in g[name]):
                    return None, "clock pass: dispatches without timestamps"
                for name in variants:
                    clk, busy = clock_stats(g[name])
                    per[name]["sclk_GHz"] = round(clk, 3)
                    per[name]["mfma_busy"] = round(busy, 4)
                    all_disp += g[name]
                for ck, ds in class_groups(g["class"], shapes):
                    if all(d is not None and d > 0 for d, _ in ds):
                        clk, busy = clock_stats(ds)
                        per_class.setdefault(ck, {}).update(sclk_GHz=round(clk, 3), mfma_busy=round(busy, 4))
            log(f"counter pass {tag}: {time.time() - t0:.1f}s")
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    for n in variants:
        per[n]["launches_per_step"] = variants[n][1]
    clk, busy = clock_stats(all_disp)
    return {"bytes_per_launch": weighted_traffic(per, variants), "by_variant": per, "counter_factors": factors,
            "sclk_GHz": round(clk, 3), "mfma_busy": round(busy, 4), "class_gemms": per_class}, None


class PowerSampler:
    """Socket power during a region, sampled by `amd-smi metric -p` in a
    background thread (a child process per sample, 2 s timeout each); empty
    where amd-smi is missing or reports nothing.

    amd-smi is a Python script: it is started with this interpreter directly,
    so no launcher process replaces itself with another program. Under a
    profiler nothing is sampled: the profiler's preloaded library would
    initialise the GPU in every child process."""

    def __init__(self, period_s=0.1):
        import os
        import shutil
        path = shutil.which("amd-smi")
        self.cmd = None
        if path and not _under_profiler():
            path = os.path.realpath(path)
            with open(path, "rb") as f:
                first = f.readline()
            self.cmd = [sys.executable, path] if first.startswith(b"#!") and b"python" in first else [path]
        self.period = period_s
        self.samples = []

    def _loop(self):
        import re
        import subprocess
        while not self.stop.is_set():
            try:
                r = subprocess.run([*self.cmd, "metric", "-p", "--json"], capture_output=True, text=True, timeout=2)
                m = re.search(r'"socket_power":\s*\{\s*"value":\s*([0-9.]+)', r.stdout)
                if m:
                    self.samples.append(float(m.group(1)))
            except (subprocess.SubprocessError, OSError):
                return
            self.stop.wait(self.period)

    def __enter__(self):
        import threading
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._loop, daemon=True) if self.cmd else None
        if self.thread:
            self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        if self.thread:
            self.thread.join(timeout=5)

    def summary(self):
        if not self.samples:
            return None
        return {"socket_W_mean": round(sum(self.samples) / len(self.samples), 1), "socket_W_max": max(self.samples),
                "samples": len(self.samples), "source": "amd-smi metric -p, every 0.1 s over the timed steps"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class EventTimer:
    """Records a HIP event pair around each launch on the current stream."""

    def __init__(self):
        self.events = {}
        self.enabled = True

    def __call__(self, name, fn):
        if not self.enabled:
            return fn()
        import torch
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.events.setdefault(name, []).append((s, e))
        return out

    def summary(self):
        return {k: (len(v), sum(s.elapsed_time(e) for s, e in v) / len(v)) for k, v in self.events.items()}


def make_inputs(cfg, device):
    import torch
    from fp4_quantized_diffusion_amd import inputs
    t0 = time.time()
    noise = inputs.rollout_noise_all(cfg["seed"], cfg["n_cand"], cfg["tokens"], cfg["dim"])
    noise_d = torch.from_numpy(noise).to(device)
    del noise
    w1, w2 = [], []
    for b in range(cfg["blocks"]):
        a, bb = inputs.rollout_weights(cfg["seed"], b, cfg["dim"], cfg["hidden"])
        w1.append(torch.from_numpy(a).to(device).bfloat16())
        w2.append(torch.from_numpy(bb).to(device).bfloat16())
    u = torch.from_numpy(inputs.reward_vector(cfg["seed"], cfg["dim"])).to(device)
    log(f"inputs ready in {time.time() - t0:.1f}s")
    return noise_d, w1, w2, u


def bf16_rewards(noise, w1, w2, u, steps, chunk):
    """Proxy rewards of every candidate under the same rollout with BF16
    linears (stage2.Bf16Regenerator), for the rank agreement."""
    from fp4_quantized_diffusion_amd import stage2
    return stage2.Bf16Regenerator(w1, w2, u, chunk=chunk).run(noise, steps)[1]


def ablation_extras(noise, w1, w2, u, cfg, chunk, r_fp4, sel):
    """--ablation only: the DiffusionNFT loss forward on the BF16-regenerated
    selected seeds and the extreme-value diagnostic."""
    from fp4_quantized_diffusion_amd import stage2
    regen = stage2.Bf16Regenerator(w1, w2, u, chunk=min(chunk, 8))
    x_regen, r_regen = regen.regenerate(noise, sel, 20)
    return {"nft_loss_forward": nft_forward(x_regen, r_regen, w1, w2, cfg["tokens"], min(chunk, 8)),
            "evt_diagnostic": evt_diagnostic(r_fp4, noise, w1, w2, u, cfg, min(chunk, 8))}


def nft_forward(x0, r_raw, w1, w2, tokens, chunk, beta=0.1, seed=3):
    """DiffusionNFT loss forward on the regenerated samples (VeRL-Omni
    DiffusionNFT docs, "Algorithm"): r = the normalized rewards
    (select_topk_bottomk's r_norm), x_t = (1 - t) x0 + t eps at a random t
    per sample (fp4_nft_noise), v_old from the network, v_theta from the
    network with a small weight perturbation standing in for the trained
    adapter, then fp4_nft_loss; the two kernels are timed against HBM."""
    import torch
    import fp4_quantized_diffusion_amd as fq
    from fp4_quantized_diffusion_amd import stage2
    n, _, dim = x0.shape
    g = torch.Generator(device=x0.device).manual_seed(seed)
    eps = torch.randn(x0.shape, generator=g, device=x0.device)
    t = torch.rand(n, generator=g, device=x0.device)
    _, _, rn = fq.select(r_raw.float().contiguous(), 1, 1)
    xt = fq.nft_noise(x0.contiguous(), eps, t)
    w1p = [w + (0.01 * w.float().std() * torch.randn(w.shape, generator=g, device=w.device)).bfloat16() for w in w1]
    v_old = torch.empty_like(xt)
    v_theta = torch.empty_like(xt)
    flat = xt.view(-1, dim)
    for c0 in range(0, n, chunk):
        rows = slice(c0 * tokens, (c0 + chunk) * tokens)
        v_old.view(-1, dim)[rows] = stage2.bf16_velocity(flat[rows], w1, w2)
        v_theta.view(-1, dim)[rows] = stage2.bf16_velocity(flat[rows], w1p, w2)
    loss, terms = fq.nft_loss(v_old, v_theta, x0.contiguous(), eps, rn, beta)
    x0c = x0.contiguous()
    t_noise = time_launches([lambda: fq.nft_noise(x0c, eps, t, out=xt)], reps=20)
    t_loss = time_launches([lambda: fq.nft_loss(v_old, v_theta, x0c, eps, rn, beta)], reps=20)
    elems = x0.numel()
    return {"samples": n, "beta": beta, "loss": round(float(loss.item()), 6),
            "noise_us": round(t_noise[0], 1), "noise_tbps": round(elems * 12 / t_noise[0] / 1e6, 3),
            "loss_us": round(t_loss[0], 1), "loss_tbps": round(elems * 16 / t_loss[0] / 1e6, 3)}


def evt_diagnostic(r_fp4, noise, w1, w2, u, cfg, bchunk):
    """The extreme-value statement of the aitrends summary: the expected
    reward range of the FP4-selected extremes is at least
    2 sigma sqrt(2 log N) - 4 Delta, with sigma the reward spread and Delta
    the largest FP4-vs-BF16 reward perturbation. One draw of N candidates:
    W = BF16 reward of the FP4 top-1 seed minus that of the FP4 bottom-1
    seed, both rollouts with the same step count."""
    import math
    s = cfg["steps"]
    r4 = np.asarray(r_fp4, dtype=np.float64)
    rb = bf16_rewards(noise, w1, w2, u, s, bchunk).cpu().numpy().astype(np.float64)
    n = len(r4)
    sigma = float(rb.std())
    delta = float(np.abs(r4 - rb).max())
    w = float(rb[int(np.argmax(r4))] - rb[int(np.argmin(r4))])
    bound = 2 * sigma * math.sqrt(2 * math.log(n)) - 4 * delta
    return {"n": n, "steps": s, "sigma_bf16": round(sigma, 6), "delta_max": round(delta, 6),
            "range_of_fp4_extremes_in_bf16": round(w, 6), "bound": round(bound, 6), "holds": bool(w >= bound)}


def blas_env():
    """BLAS library, its thread count and the thread variables, for the CPU figures."""
    env = {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS") if k in os.environ}
    try:
        from threadpoolctl import threadpool_info
        pools = [{"api": p.get("internal_api"), "threads": p.get("num_threads"), "version": p.get("version")}
                 for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception as e:  # reported, never fatal
        pools = [{"error": repr(e)}]
    return {"blas": pools, "env": env, "os_cpu_count": os.cpu_count()}


def cpu_baseline(cfg, tokens_sample=512, w_rows_sample=1024, gemm_rows=512):
    """The CPU oracle on bounded samples of the workload (numpy float64,
    the host's BLAS threads), scaled to candidates/s:
    (a) the tiny configuration in full (128 x 256 x 512: quantize both
        operands, GEMM, 8 rewards, top-2 / bottom-2), reported as is;
    (b) the oracle's MXFP4 quantization of a w_rows_sample-row slice of one
        W1, scaled by element count to all 8 weights (once per rollout);
    (c) the oracle rollout of 1 candidate x tokens_sample tokens through the
        6 steps of the 4-block network (weights in quantized form), scaled by
        4096 / tokens_sample tokens per candidate and by the 96 candidates;
    (d) a gemm_rows-row slice of the FLUX.1-class up projection (36864 x 3072
        x 12288): the oracle's activation quantization and exact GEMM,
        reported in TFLOP/s and scaled to the whole GEMM.
    value = 96 / ((b) + 96 (c))."""
    from fp4_quantized_diffusion_amd import inputs
    from oracle import gemm as ogemm, mxfp4, reward as oreward, rollout as orollout
    dim, hidden, blocks = cfg["dim"], cfg["hidden"], cfg["blocks"]
    rng = np.random.default_rng(0)
    # (a) tiny configuration
    t0 = time.perf_counter()
    x, b = inputs.tiny(0)
    ca, sa = mxfp4.quantize(x)
    cb, sb = mxfp4.quantize(b)
    c, _ = ogemm.gemm_mx(ca, sa, cb, sb)
    oreward.select(oreward.proxy_reward(c, 16), 2, 2)
    t_tiny = time.perf_counter() - t0
    # (b) weight re-quantization
    w_slice = inputs.weights(rng, w_rows_sample, dim)
    t0 = time.perf_counter()
    mxfp4.quantize(w_slice)
    t_wq = (time.perf_counter() - t0) * (2 * blocks * hidden * dim) / w_slice.size
    # (c) rollout slice; quantized weights for the timing sample: random codes / scales of the right shapes
    q1 = [orollout.QuantLinear.from_quantized("mx", rng.integers(0, 256, (hidden, dim // 2), dtype=np.uint8),
                                              rng.integers(118, 124, (hidden, dim // 32), dtype=np.uint8))
          for _ in range(blocks)]
    q2 = [orollout.QuantLinear.from_quantized("mx", rng.integers(0, 256, (dim, hidden // 2), dtype=np.uint8),
                                              rng.integers(118, 124, (dim, hidden // 32), dtype=np.uint8))
          for _ in range(blocks)]
    noise = inputs.rollout_noise(cfg["seed"], 0, tokens_sample, dim)[None]
    u = inputs.reward_vector(cfg["seed"], dim)
    t0 = time.perf_counter()
    orollout.rollout(noise, q1, q2, u, n_steps=cfg["steps"], k_top=1, k_bottom=0)
    t_cand = (time.perf_counter() - t0) * cfg["tokens"] / tokens_sample
    # (d) FLUX-class GEMM slice (the weight quantization is outside the timing: once per iteration)
    m_full, k, n = 36864, 3072, 12288
    act = inputs.activations(rng, gemm_rows, k)
    wq = q1[0].w_hat if (k, n) == (dim, hidden) else None
    t0 = time.perf_counter()
    a_hat = mxfp4.dequant(*mxfp4.quantize(act))
    ogemm.gemm_dense(a_hat, wq)
    t_gemm = time.perf_counter() - t0
    flop = 2.0 * gemm_rows * k * n
    total = t_wq + cfg["n_cand"] * t_cand
    env = blas_env()
    threads = env["blas"][0].get("threads") if env["blas"] and "threads" in env["blas"][0] else None
    return {"value": round(cfg["n_cand"] / total, 6), "unit": "candidates/s",
            "cores": int(threads or os.environ.get("OMP_NUM_THREADS") or os.cpu_count()),
            "kind": "oracle",
            "sample": (f"oracle MXFP4 quantization of a {w_rows_sample}x{dim} weight slice (scaled by elements to "
                       f"all {2 * blocks} weights: {t_wq:.1f}s) + oracle rollout of 1 candidate x {tokens_sample} "
                       f"tokens, {cfg['steps']} steps x {blocks} blocks (scaled x{cfg['tokens'] // tokens_sample} "
                       f"tokens, x{cfg['n_cand']} candidates: {cfg['n_cand'] * t_cand:.1f}s); numpy float64"),
            "tiny_config_seconds": round(t_tiny, 4),
            "flux_up_gemm_slice": {"rows": gemm_rows, "of": [m_full, k, n], "seconds": round(t_gemm, 3),
                                   "tflops": round(flop / t_gemm / 1e12, 4),
                                   "full_gemm_seconds_scaled": round(t_gemm * m_full / gemm_rows, 1)},
            "host": env}


def cpu_quantizers_full(chunk_rows=4096):
    """--cpu-full: the oracle's MXFP4 quantization of every class activation
    in full (the rows in chunks, each chunk quantized by the oracle as it
    stands; only the quantization is timed, not the draws)."""
    from fp4_quantized_diffusion_amd import inputs
    from oracle import mxfp4
    out = {}
    for name in ("flux", "sana", "sd35"):
        cfg = inputs.CLASS_SHAPES[name]
        for which in (1, 2):
            _, k, _ = inputs.class_gemm(name, which)
            m = cfg["m"]
            rng = np.random.default_rng([cfg["seed"], which, 0])
            t = 0.0
            for r0 in range(0, m, chunk_rows):
                a = inputs.activations(rng, min(chunk_rows, m - r0), k, cfg["act"])
                t0 = time.perf_counter()
                mxfp4.quantize(a)
                t += time.perf_counter() - t0
            key = f"mx_quantize_act_{name}_{m}x{k}"
            out[key] = {"seconds": round(t, 2), "gb_per_s": round(m * k * 2.53125 / t / 1e9, 4)}
            log(f"cpu oracle {key}: {t:.1f}s")
    return out


def time_launches(fns, reps=50, warm_ms=100.0):
    """Median / p10 / p90 (microseconds) of one launch, from a HIP event pair
    around each call on the current stream. fns: one callable per rotating
    input set (called round-robin). Warm-up runs for about warm_ms first, so
    the timed launches see the clock the card settles at under this load."""
    import torch
    fns[0]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < warm_ms or i < 2 * len(fns):
        fns[i % len(fns)]()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = []
    for i in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fns[i % len(fns)]()
        e.record()
        ev.append((s, e))
    torch.cuda.synchronize()
    us = np.sort(np.array([s.elapsed_time(e) * 1e3 for s, e in ev]))
    return float(np.median(us)), float(np.percentile(us, 10)), float(np.percentile(us, 90))


def class_benchmarks(dev, n_sets=4):
    """The FLUX.1-, SANA- and SD3.5-L-class linears at full size: MXFP4 GEMM
    (panel operands, bf16 C, operands pre-quantized) against torch's bf16
    GEMM (F.linear) on the same shapes, plus the quantizers' bandwidth and
    the NVFP4-style GEMM on the FLUX shapes. n_sets input sets rotate so that
    the Infinity Cache cannot hold the operands between launches."""
    import torch
    import torch.nn.functional as F
    import fp4_quantized_diffusion_amd as fq
    from fp4_quantized_diffusion_amd import inputs

    def rate(flop, us, peak):
        return {"tflops": round(flop / us / 1e6, 1), "frac_of_peak": round(flop / us / 1e-6 / peak, 4)}

    gemms, mem = {}, {}
    for name in CLASS_NAMES:
        for which in (1, 2):
            t0 = time.time()
            draws = [inputs.class_linear_device(name, which, dev, draw=d) for d in range(n_sets)]
            m, k = draws[0][0].shape
            n = draws[0][1].shape[0]
            qa = [fq.quantize(a, "mx", layout="panel") for a, _ in draws]
            qb = [fq.quantize(w, "mx", layout="panel") for _, w in draws]
            c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            flop = 2.0 * m * n * k
            key = class_key(name, which, m, k, n)
            f_us = time_launches([lambda i=i: fq.gemm(qa[i], qb[i], "bf16", out=c) for i in range(n_sets)])
            b_us = time_launches([lambda i=i: F.linear(draws[i][0], draws[i][1]) for i in range(n_sets)])
            g = {"m": m, "k": k, "n": n,
                 "mxfp4_us": [round(v, 1) for v in f_us], **{"mxfp4_" + a: b for a, b in
                                                            rate(flop, f_us[0], PEAK_FP4).items()},
                 "bf16_us": [round(v, 1) for v in b_us], **{"bf16_" + a: b for a, b in
                                                           rate(flop, b_us[0], PEAK_BF16).items()},
                 "mxfp4_speedup_vs_bf16": round(b_us[0] / f_us[0], 3)}
            # activation re-quantization (panel layout, bf16 in): 2 + 0.5 + 1/32 bytes per element
            q_us = time_launches([lambda i=i: fq.quantize(draws[i][0], "mx", out=qa[i]) for i in range(n_sets)])
            mem[f"mx_quantize_act_{name}_{m}x{k}"] = {"us": [round(v, 1) for v in q_us],
                                                      "tbps": round(m * k * 2.53125 / q_us[0] / 1e6, 3),
                                                      "frac_of_hbm": round(m * k * 2.53125 / q_us[0] / 1e-6 / PEAK_HBM, 4)}
            if name == "flux":
                qn_a = [fq.quantize(a, "nv") for a, _ in draws]
                qn_b = [fq.quantize(w, "nv") for _, w in draws]
                nv_us = time_launches([lambda i=i: fq.gemm(qn_a[i], qn_b[i], "bf16", out=c) for i in range(n_sets)])
                g.update({"nvfp4_us": [round(v, 1) for v in nv_us],
                          **{"nvfp4_" + a + "_bf16_peak": b for a, b in rate(flop, nv_us[0], PEAK_BF16).items()}})
                # two passes: tensor amax (2 B/elem), then codes + E4M3 scales (2 + 0.5 + 1/16)
                nq_us = time_launches([lambda i=i: fq.quantize(draws[i][0], "nv", out=qn_a[i]) for i in range(n_sets)])
                mem[f"nv_quantize_act_{name}_{m}x{k}"] = {"us": [round(v, 1) for v in nq_us],
                                                          "tbps": round(m * k * 4.5625 / nq_us[0] / 1e6, 3),
                                                          "frac_of_hbm": round(m * k * 4.5625 / nq_us[0] / 1e-6 / PEAK_HBM, 4)}
                wq_us = time_launches([lambda i=i: fq.quantize(draws[i][1], "mx", out=qb[i]) for i in range(n_sets)])
                mem[f"mx_quantize_weight_{name}_{n}x{k}"] = {"us": [round(v, 1) for v in wq_us],
                                                             "tbps": round(n * k * 2.53125 / wq_us[0] / 1e6, 3)}
                # LoRA (rank 32, fp32 adapters) merged and re-quantized in one pass: the
                # weight's 2.53 B/elem plus the adapters, and 2 r + 2 fp32 FLOP per element
                r = 32
                lb = [torch.randn(n, r, device=dev) * 0.01 for _ in range(n_sets)]
                la = [torch.randn(r, k, device=dev) * 0.05 for _ in range(n_sets)]
                lq_us = time_launches([lambda i=i: fq.quantize_lora(draws[i][1], lb[i], la[i], 2.0, out=qb[i])
                                       for i in range(n_sets)])
                lbytes = n * k * 2.53125 + (n + k) * r * 4
                mem[f"mx_quantize_lora_r{r}_weight_{name}_{n}x{k}"] = {
                    "us": [round(v, 1) for v in lq_us], "tbps": round(lbytes / lq_us[0] / 1e6, 3),
                    "fp32_tflops": round((2 * r + 2) * n * k / lq_us[0] / 1e6, 2),
                    "vs_plain_requantize": round(lq_us[0] / wq_us[0], 2)}
                # NVFP4-style: a tensor-amax pass over the merged weight, then the
                # merge again and the codes (2 + 0.5 + 1/16 B/elem written and read)
                qn_w = [fq.quantize(draws[i][1], "nv") for i in range(n_sets)]
                ln_us = time_launches([lambda i=i: fq.quantize_lora(draws[i][1], lb[i], la[i], 2.0, fmt="nv",
                                                                    out=qn_w[i]) for i in range(n_sets)])
                nbytes = 2 * (n * k * 2 + (n + k) * r * 4) + n * k * (0.5 + 1 / 16)
                mem[f"nv_quantize_lora_r{r}_weight_{name}_{n}x{k}"] = {
                    "us": [round(v, 1) for v in ln_us], "tbps": round(nbytes / ln_us[0] / 1e6, 3),
                    "fp32_tflops": round(2 * (2 * r + 2) * n * k / ln_us[0] / 1e6, 2), "passes": 2}
                del qn_w
                del qn_a, qn_b, lb, la
            gemms[key] = g
            log(f"class {key}: mxfp4 {f_us[0]:.0f} us ({g['mxfp4_tflops']} TF/s), bf16 {b_us[0]:.0f} us "
                f"({g['bf16_tflops']} TF/s) [{time.time() - t0:.1f}s]")
            del draws, qa, qb, c
            torch.cuda.empty_cache()
    return gemms, mem


def rollout_step_kernels(x, v, u, cfg):
    """The unfused Euler update (a7), proxy reward (a8) and selection (a9) at
    the rollout's size, each timed on its own (the rollout fuses the first
    two into its last GEMMs). x and v are [n_cand * tokens, dim] fp32 of
    4.83 GB each, far beyond the Infinity Cache, so no rotation is needed;
    the Euler update runs in place on x."""
    import torch
    import fp4_quantized_diffusion_amd as fq
    from fp4_quantized_diffusion_amd import binding as fb

    n, tokens, dim = cfg["n_cand"], cfg["tokens"], cfg["dim"]
    numel = x.numel()
    out = {}
    e_us = time_launches([lambda: fq.euler(x, v, 1.0, 5.0 / 6.0, out=x)])
    out[f"euler_step_{n}x{tokens}x{dim}_f32"] = {
        "us": [round(a, 1) for a in e_us], "tbps": round(12.0 * numel / e_us[0] / 1e6, 3),
        "frac_of_hbm": round(12.0 * numel / e_us[0] / 1e-6 / PEAK_HBM, 4)}
    r = torch.empty(n, dtype=torch.float32, device=x.device)
    r_us = time_launches([lambda: fq.proxy_reward(x, n, tokens, u, out=r)])
    out[f"proxy_reward_{n}x{tokens}x{dim}"] = {
        "us": [round(a, 1) for a in r_us], "tbps": round(4.0 * numel / r_us[0] / 1e6, 3),
        "frac_of_hbm": round(4.0 * numel / r_us[0] / 1e-6 / PEAK_HBM, 4)}
    kt, kb = cfg["k_top"], cfg["k_bottom"]
    top = torch.empty(kt, dtype=torch.int32, device=x.device)
    bottom = torch.empty(kb, dtype=torch.int32, device=x.device)
    rn = torch.empty(n, dtype=torch.float32, device=x.device)
    stream = torch.cuda.current_stream().cuda_stream

    def sel():
        st = fb.select_topk_bottomk(r.data_ptr(), n, kt, kb, top.data_ptr(), bottom.data_ptr(), rn.data_ptr(),
                                    stream)
        assert st == 0, fb.status_str(st)
    s_us = time_launches([sel])
    # latency-bound: one workgroup, event pair around the two kernels of the call
    out[f"select_{n}_top{kt}_bottom{kb}"] = {"us": [round(a, 1) for a in s_us]}
    return out


def gelu_epilogue_variants(x, w1, cfg):
    """The first linear's fused GELU + MXFP4 epilogue at the rollout's size,
    two ways: GELU of the fp32 sums (fp4_gemm_panel_gelu_f32, the default and
    the oracle's reading) and GELU of bf16(C) from the LDS table
    (fp4_gemm_panel_gelu), each timed alone. x: fp32 [rows, dim]; w1: the
    first block's bf16 weight."""
    import fp4_quantized_diffusion_amd as fq
    a1 = fq.quantize(x, "mx", prologue="rmsnorm", layout="panel")
    wq = fq.quantize(w1, "mx", layout="panel")
    out = fq.gemm_gelu(a1, wq)
    t_tab = time_launches([lambda: fq.gemm_gelu(a1, wq, out=out)], reps=10)
    t_f32 = time_launches([lambda: fq.gemm_gelu(a1, wq, out=out, exact=True)], reps=10)
    flop = 2.0 * x.shape[0] * cfg["dim"] * cfg["hidden"]
    return {"shape": [x.shape[0], cfg["dim"], cfg["hidden"]],
            "f32_us": [round(a, 1) for a in t_f32], "bf16_table_us": [round(a, 1) for a in t_tab],
            "f32_tflops": round(flop / t_f32[0] / 1e6, 1), "bf16_table_tflops": round(flop / t_tab[0] / 1e6, 1)}


def other_hidden_rollout(noise, work, w1, w2, u, cfg, chunk, layout, steps=3):
    """The same rollout with the other reading of the hidden activation
    (bf16 when the run's is fp32), timed the same way, outside the main timed
    region: its rate, and how its rewards rank against the main run's."""
    import torch
    from fp4_quantized_diffusion_amd.rollout import Fp4Rollout
    other = "bf16" if cfg["hidden_act"] == "f32" else "f32"
    ro = Fp4Rollout(w1, w2, u, steps=cfg["steps"], k_top=cfg["k_top"], k_bottom=cfg["k_bottom"], chunk=chunk,
                    layout=layout, hidden=other)
    ro.run(noise, work)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r, top, bottom, _ = ro.run(noise, work)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    return other, sec, r


def run_config(args):
    """(cfg, candidates per chunk, whether this is the default workload) for
    the parsed arguments: the rollout's sizes, with the token count and the
    hidden activation's precision (cfg["hidden_act"]; cfg["hidden"] is the
    hidden width) from the arguments."""
    from fp4_quantized_diffusion_amd.inputs import ROLLOUT
    cfg = dict(ROLLOUT)
    cfg["tokens"] = args.tokens
    cfg["hidden_act"] = args.hidden or ("bf16" if args.overlap else "f32")
    chunk = args.chunk or cfg["n_cand"]
    default = (args.layout == "panel" and not args.overlap and args.tokens == 4096 and chunk == cfg["n_cand"]
               and cfg["hidden_act"] == "f32")
    return cfg, chunk, default


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--chunk", type=int, default=0, help="candidates per network pass (0 = all 96)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rank-agreement", action="store_true")
    ap.add_argument("--no-class-gemms", action="store_true",
                    help="skip the FLUX/SANA/SD3.5-class GEMM, bf16 baseline and quantizer timings")
    ap.add_argument("--no-step-kernels", action="store_true",
                    help="skip the standalone Euler / proxy reward / selection timings at the rollout's size")
    ap.add_argument("--tokens", type=int, default=4096, help="tokens per candidate (4096 is the workload)")
    ap.add_argument("--layout", choices=("panel", "row"), default="panel", help="FP4 operand layout of the GEMMs")
    ap.add_argument("--overlap", action="store_true",
                    help="two-stream schedule (GEMMs beside quantizers; stores the hidden activation as bf16)")
    ap.add_argument("--hidden", choices=("f32", "bf16"), default=None,
                    help="the first linear's output into GELU: f32 (default; the oracle's arithmetic) or bf16 "
                         "(rounded first: a faster epilogue, but a different network)")
    ap.add_argument("--cpu-full", action="store_true",
                    help="also time the oracle's quantization of every class activation in full (minutes of CPU)")
    ap.add_argument("--no-stage2", action="store_true",
                    help="skip the Stage-2 block (BF16 regeneration of the selected seeds, FP4 step-count ablation)")
    ap.add_argument("--ablation", action="store_true",
                    help="a finer step-count ablation (2, 3, 4, 6, 8, 10 FP4 steps), plus the DiffusionNFT loss "
                         "forward on the regenerated seeds and the extreme-value diagnostic")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before warmup, run one device copy of MIB MiB (a known-size kernel for scaling "
                         "profiler byte counters); not part of any step")
    ap.add_argument("--no-other-hidden", action="store_true",
                    help="skip the comparison rollout with the other reading of the hidden activation")
    ap.add_argument("--no-traffic", action="store_true",
                    help="skip the live GEMM byte-counter passes (roofline.traffic then comes from the profile)")
    ap.add_argument("--traffic-probe", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.traffic_probe:
        from fp4_quantized_diffusion_amd.inputs import ROLLOUT
        traffic_probe(dict(ROLLOUT, tokens=args.tokens, hidden_act=args.hidden or "f32"))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the rollout shards over candidates "
              "with no cross-GPU traffic besides a 384-byte reward exchange, which this build does not run.",
              file=sys.stderr)
        sys.exit(2)

    cfg, chunk, default_workload = run_config(args)
    # the counters first, while this process has no GPU state
    traffic, counters, traffic_src = None, None, None
    if default_workload:
        if args.no_traffic or _under_profiler():
            why = "--no-traffic" if args.no_traffic else "this run is itself profiled"
        else:
            t0 = time.time()
            counters, why = measure_counters(cfg)
            log(f"GEMM counters: {time.time() - t0:.1f}s" + (f" (not measured: {why})" if why else ""))
        if counters is not None:
            traffic = counters["bytes_per_launch"]
            traffic_src = {"source": "measured in this run: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, "
                                     "then --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE, each in a child "
                                     "process over one step of this rollout (all its GEMM launches) and two "
                                     "launches of each class GEMM; byte factors from a 1 GiB device copy in "
                                     "the same runs",
                           "by_variant": counters["by_variant"], "counter_factors": counters["counter_factors"]}
        else:
            traffic = gemm_traffic(cfg["hidden_act"])
            traffic_src = {"source": "profile (profiles/rollout_96x4096x3072_kernels.md)" if traffic is not None
                           else "none: the profile's counters were taken with other GEMM sources or "
                                "another hidden activation",
                           "not_measured": why}

    import torch
    import fp4_quantized_diffusion_amd as fq
    from fp4_quantized_diffusion_amd.rollout import Fp4Rollout

    fq.load_library()
    dev = "cuda:0"
    noise, w1, w2, u = make_inputs(cfg, dev)
    work = torch.empty_like(noise)
    timer = EventTimer()
    ro = Fp4Rollout(w1, w2, u, steps=cfg["steps"], k_top=cfg["k_top"], k_bottom=cfg["k_bottom"], chunk=chunk,
                    timer=timer, layout=args.layout, overlap=args.overlap, hidden=cfg["hidden_act"])

    if args.copy_calibration:
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: {args.copy_calibration} MiB read + {args.copy_calibration} MiB written")
    timer.enabled = False
    for i in range(args.warmup):
        ro.run(noise, work)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    timer.enabled = True
    torch.cuda.synchronize()
    with PowerSampler() as power:
        t0 = time.perf_counter()
        for i in range(args.steps):
            rewards, top, bottom, rn = ro.run(noise, work)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    sec = (t1 - t0) / args.steps
    top_l, bottom_l = top.tolist(), bottom.tolist()
    log(f"timed {args.steps} steps: {sec * 1e3:.1f} ms/step; top {top_l[:4]}... bottom {bottom_l[:4]}...")

    ks = timer.summary()
    n_gemm, gemm_ms = ks["gemm"]
    # each step runs 2 GEMMs per block over all candidates; a launch covers
    # the rows of one chunk, so price it by the step's FLOPs over its launches
    step_flop = 2.0 * 2 * cfg["blocks"] * cfg["steps"] * cfg["n_cand"] * cfg["tokens"] * cfg["dim"] * cfg["hidden"]
    gemm_flop = step_flop / (n_gemm / args.steps)
    m_rows = int(round(gemm_flop / (2.0 * cfg["dim"] * cfg["hidden"])))
    achieved = gemm_flop / (gemm_ms * 1e-3)
    kernels = {k: {"launches_per_step": n // args.steps, "avg_us": round(ms * 1e3, 2)} for k, (n, ms) in ks.items()}

    out = {
        "metric": METRIC,
        "value": round(cfg["n_cand"] / sec, 4),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": f"fp4_rollout_{cfg['n_cand']}x{cfg['tokens']}x{cfg['dim']}_mlp{cfg['hidden']}"
                               f"x{cfg['blocks']}blk_{cfg['steps']}step_top{cfg['k_top']}_bottom{cfg['k_bottom']}",
                   "n_cand": cfg["n_cand"], "tokens": cfg["tokens"], "dim": cfg["dim"], "hidden": cfg["hidden"],
                   "blocks": cfg["blocks"], "euler_steps": cfg["steps"], "chunk_candidates": chunk,
                   "operand_layout": args.layout, "two_stream_overlap": args.overlap,
                   "hidden_activation": cfg["hidden_act"],
                   "gemm_shapes": [[m_rows, cfg["dim"], cfg["hidden"]], [m_rows, cfg["hidden"], cfg["dim"]]]},
        # the recorded traffic is that of the default workload (panel layout, one stream, all candidates)
        "roofline": {"bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": PEAK_FP4 / 1e12,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP4, 4),
                     "traffic": None if traffic is None else round(traffic / 1e9, 2),
                     "traffic_unit": "GB per launch (L2 <-> fabric reads + writes, rocprofv3 counters)",
                     "traffic_detail": traffic_src,
                     "kernel": f"gemm_fp4_kernel, {args.layout} layout (MXFP4 x MXFP4, fp32 accumulate; "
                               + (f"the first linear's launches quantize "
                                  f"{'GELU(C)' if cfg['hidden_act'] == 'f32' else 'GELU(bf16(C))'} to MXFP4 in their "
                                  "epilogue, the second's add the residual, the last block's also apply the Euler step)"
                                  if args.layout == "panel" else "the second linear's launches add the residual)"),
                     "flop_per_launch": gemm_flop, "avg_launch_us": round(gemm_ms * 1e3, 2)},
        "gemm_tflops": round(achieved / 1e12, 2),
        "gemm_frac_of_mxfp4_peak": round(achieved / PEAK_FP4, 4),
        "kernels": kernels,
        "power": power.summary(),
    }
    if counters is not None:
        # the spec peak scaled to the shader clock the GEMMs ran at (counter pass of this run)
        out["roofline"]["sclk_GHz"] = counters["sclk_GHz"]
        out["roofline"]["mfma_busy"] = counters["mfma_busy"]
        out["roofline"]["frac_of_clock_adjusted_peak"] = round(achieved / (PEAK_FP4 * counters["sclk_GHz"] / 2.4), 4)
    if not args.no_class_gemms:
        t0 = time.time()
        out["class_gemms"], out["memory_kernels"] = class_benchmarks(dev)
        if counters is not None:
            for key, m, k, n in class_shapes():
                g, cs = out["class_gemms"].get(key), counters["class_gemms"].get(key, {})
                if g is None or "sclk_GHz" not in cs:
                    continue
                # operands' codes and scales read once, bf16 C written once
                alg = (m + n) * k * (0.5 + 1 / 32) + 2.0 * m * n
                g.update({"sclk_GHz": cs["sclk_GHz"], "mfma_busy": cs["mfma_busy"],
                          "mxfp4_frac_of_clock_adjusted_peak": round(
                              g["mxfp4_tflops"] * 1e12 / (PEAK_FP4 * cs["sclk_GHz"] / 2.4), 4),
                          "read_GB": cs.get("read_GB"), "write_GB": cs.get("write_GB"),
                          "algorithmic_GB": round(alg / 1e9, 3)})
        log(f"class benchmarks: {time.time() - t0:.1f}s")
    if not args.no_step_kernels:
        # after the rollout's outputs are read: the Euler timing overwrites `work`
        t0 = time.time()
        out["rollout_step_kernels"] = rollout_step_kernels(work.view(-1, cfg["dim"]), noise.view(-1, cfg["dim"]),
                                                           u, cfg)
        out["rollout_step_kernels"]["gelu_epilogue"] = gelu_epilogue_variants(noise.view(-1, cfg["dim"]), w1[0], cfg)
        log(f"standalone step kernels: {time.time() - t0:.1f}s")
    if not args.no_other_hidden and not args.overlap:
        # the other reading of the hidden activation, for comparison (not the headline: a different network)
        from fp4_quantized_diffusion_amd import stage2
        t0 = time.time()
        other, osec, r_other = other_hidden_rollout(noise, work, w1, w2, u, cfg, chunk, args.layout)
        out["other_hidden_rollout"] = {
            "hidden_activation": other, "ms_per_step": round(osec * 1e3, 3),
            "candidates_per_s": round(cfg["n_cand"] / osec, 4),
            "rank_agreement_with_headline": stage2.rank_stats(r_other.cpu().numpy(), rewards.cpu().numpy(),
                                                             cfg["k_top"])}
        log(f"rollout with the {other} hidden activation: {osec * 1e3:.1f} ms/step [{time.time() - t0:.1f}s]")
    if not args.no_rank_agreement:
        from fp4_quantized_diffusion_amd import stage2
        try:
            t0 = time.time()
            r_bf16 = bf16_rewards(noise, w1, w2, u, cfg["steps"], min(chunk, 8))
            out["rank_agreement_vs_bf16"] = stage2.rank_stats(rewards.cpu().numpy(), r_bf16.cpu().numpy(),
                                                              cfg["k_top"])
            log(f"bf16 rollout for rank agreement: {time.time() - t0:.1f}s")
        except Exception as e:  # reported, never fatal
            out["rank_agreement_vs_bf16"] = {"error": repr(e)}
    if not args.no_stage2:
        # Stage 2 and the step-count ablation, outside the timed region: FP4
        # explorations with 2..10 steps ranked against a 20-step BF16 rollout of
        # every candidate, and the BF16 regeneration of the 24 seeds the 6-step
        # exploration keeps
        from fp4_quantized_diffusion_amd import stage2
        t0 = time.time()
        steps_list = (2, 3, 4, 6, 8, 10) if args.ablation else (2, 4, 6, 10)
        out["stage2"] = stage2.step_ablation(noise, w1, w2, u, cfg["k_top"], cfg["k_bottom"], fp4_steps=steps_list,
                                             ref_steps=20, explore_steps=cfg["steps"], chunk=chunk,
                                             bf16_chunk=min(chunk, 8))
        log(f"stage 2 and step ablation: {time.time() - t0:.1f}s")
        if args.ablation:
            sel = torch.cat([top, bottom])
            out["stage2"].update(ablation_extras(noise, w1, w2, u, cfg, chunk, rewards.cpu().numpy(), sel))
    if not args.no_cpu_baseline:
        t0 = time.time()
        out["cpu_baseline"] = cpu_baseline(cfg)
        if args.cpu_full:
            out["cpu_baseline"]["class_quantizers_full"] = cpu_quantizers_full()
        log(f"cpu baseline: {time.time() - t0:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
