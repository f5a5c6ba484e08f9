"""Throughput of the Muon hot path on one MI355X, as one JSON line.

A step is one fused Muon step (momentum -> Frobenius norm -> Newton-Schulz -> update scale ->
decoupled weight decay) over the whole synthetic batch, through the C ABI. The default
workload is the Kimi-K2-shaped expert batch: 648 bf16 matrices of 2048 x 7168 (216 experts x
up/gate/down), Gaussian entries plus a rank-32 spike, with stabilized Gram Newton-Schulz
(fp16 iterates, restart after step 2, K = 5). The standard iteration is timed beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--variant gram|standard]
                    [--batch B] [--no-cpu-baseline] [--skip-standard]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "newton_schulz_matrix_muon_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kind_work(kind: str, groups):
    """Algorithmic work of one launch of a kernel kind over the groups [(batch, n, m), ...]
    (a launch covers every group): (amount, unit, bound)."""
    from newton_schulz_matrix_muon_amd import flops
    per = {"gemm_symprod": (lambda n, m: flops.sym_flops(n, n), "flop", "mfma"),
           "gemm_square": (lambda n, m: 2 * n ** 3, "flop", "mfma"),
           "gemm_syrk": (lambda n, m: flops.sym_flops(n, m), "flop", "mfma"),
           "gemm_rect": (lambda n, m: flops.rect_flops(n, m), "flop", "mfma"),
           # read G (bf16) and M (fp32), write M (fp32) and the bf16 copy of N
           "prep_norm": (lambda n, m: n * m * (2 + 4 + 4 + 2), "byte", "hbm")}
    if kind not in per:
        return None
    f, unit, bound = per[kind]
    return sum(B * f(n, m) for B, n, m in groups), unit, bound


ADAMW_KW = dict(lr=2e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def adamw_params(torch, dev):
    """The Kimi-K2 parameters that stay on AdamW (guide, hybrid strategy): the 163840 x 7168
    token embedding, 60 router projections 384 x 7168, and 122 RMSNorm scales of 7168 (bf16
    parameters and gradients, fp32 moments)."""
    sizes = [163840 * 7168] + [384 * 7168] * 60 + [7168] * 122
    gen = torch.Generator(device=dev).manual_seed(4242)
    out = []
    for n in sizes:
        p = (0.02 * torch.randn(n, generator=gen, device=dev)).to(torch.bfloat16)
        g = (1e-3 * torch.randn(n, generator=gen, device=dev)).to(torch.bfloat16)
        out.append((p, g, torch.zeros(n, device=dev), torch.zeros(n, device=dev)))
    return out


def bench_adamw(args):
    """AdamW on the Kimi-K2 1-D / embedding parameters alone: parameter updates per second and
    the kernel's HBM roofline (22 bytes per bf16 parameter: read p, g, m, v; write p, m, v)."""
    import torch
    from newton_schulz_matrix_muon_amd import ops
    dev = torch.device("cuda:0")
    vec = adamw_params(torch, dev)
    ps, gs, ms, vs = (list(x) for x in zip(*vec))
    numel = sum(p.numel() for p in ps)
    for _ in range(args.warmup):
        ops.adamw_step(ps, gs, ms, vs, **ADAMW_KW)
    torch.cuda.synchronize()
    ops.timing_reset()
    ops.timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ops.adamw_step(ps, gs, ms, vs, **ADAMW_KW)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    ops.timing_enable(False)
    ms_tot, launches = ops.timing_query()["adamw"]
    per_launch = launches // args.steps
    # the embedding is the first launch's dominant tensor; per launch bytes = its tensors' bytes
    step_bytes = 22 * numel
    avg_s = ms_tot / launches / 1e3
    achieved = step_bytes / per_launch / avg_s / 1e9
    out = {"metric": "AdamW parameter updates/sec (hybrid optimizer, 1-D and embedding side)",
           "value": numel / sec, "unit": "parameters/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": sec * 1e3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "kimi_k2_adamw_embedding_163840x7168+60x384x7168+122x7168_bf16",
                      "parameters": numel, **ADAMW_KW},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": achieved / PEAK_HBM_GBS, "traffic": None, "kernel": "adamw",
                        "avg_launch_ms": avg_s * 1e3, "launches": launches,
                        "note": "bytes per launch averaged over the step's launches"},
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)


class ClockSampler:
    """Samples the GPU's reported graphics clock (sysfs pp_dpm_sclk, the line marked '*') and
    board power (hwmon power1_average or power1_input, with the power1_cap limit) every
    `period` seconds on a host thread, to put the MFMA peak in terms of the clock the run
    actually had and to show whether the run sat at the power limit."""

    def __init__(self, period: float = 0.02):
        import glob
        import threading
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.power_path, self.cap_w = None, None
        if self.path:
            dev = os.path.dirname(self.path)
            for name in ("power1_average", "power1_input"):
                cand = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", name)))
                if cand:
                    self.power_path = cand[0]
                    cap = os.path.join(os.path.dirname(cand[0]), "power1_cap")
                    try:
                        self.cap_w = int(open(cap).read()) / 1e6
                    except (OSError, ValueError):
                        pass
                    break
        self.samples = []
        self.power = []
        self.period = period
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            for line in open(self.path):
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            if self.power_path:
                try:
                    self.power.append(int(open(self.power_path).read()) / 1e6)
                except (OSError, ValueError):
                    pass
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._t.join()

    def summary(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        out = {"median_mhz": xs[len(xs) // 2], "min_mhz": xs[0], "max_mhz": xs[-1],
               "samples": len(xs), "source": "sysfs pp_dpm_sclk"}
        if self.power:
            ps = sorted(self.power)
            out["power_w"] = {"median": ps[len(ps) // 2], "min": ps[0], "max": ps[-1],
                              "cap": self.cap_w, "source": os.path.basename(self.power_path)}
        return out


def kernel_source_digest() -> str:
    """sha256 over the HIP sources (name + bytes, sorted): ties recorded counters to a build."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def recorded_traffic(kind: str, workload: str):
    """HBM bytes per launch of `kind` from the committed FETCH_SIZE / WRITE_SIZE summary of this
    workload, or None when there is none or the kernels changed since it was taken."""
    import glob
    for path in glob.glob(os.path.join(PROFILES, "hbm_traffic_*.md")):
        for line in open(path):
            if not line.startswith("traffic-json: "):
                continue
            rec = json.loads(line[len("traffic-json: "):])
            if rec.get("workload") != workload or rec.get("source_sha256") != kernel_source_digest():
                continue
            k = rec.get("kinds", {}).get(kind)
            if k:
                return k["bytes_per_launch"], os.path.basename(path)
    return None, None


def copy_probe(mib: int):
    """A plain device copy of `mib` MiB (calibrates the HBM byte counters)."""
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline(G_host, W_host, budget_s: float, variant: str, kw: dict):
    """The fp64 oracle's Muon step on a bounded sample of the same workload (host cores)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    ns = (lambda x: oracle.ns_gram(x, restarts=(2,))) if variant == "gram" else oracle.ns_standard
    done, t0 = 0, time.perf_counter()
    while done < len(G_host):
        oracle.muon_step(W_host[done], G_host[done], np.zeros_like(G_host[done]), kw["lr"],
                         kw["momentum"], kw["weight_decay"], nesterov=kw["nesterov"],
                         scale_coeff=kw["scale_coeff"], ns=ns)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    from newton_schulz_matrix_muon_amd import flops
    r, c = G_host[0].shape
    per = flops.gram_flops(r, c) if variant == "gram" else flops.standard_flops(r, c)
    return {"value": done / dt, "unit": "matrices/s", "cores": int(cores), "kind": "oracle",
            "fp64_gflops": done * per / dt / 1e9,
            "sample": f"{done} of the batch's matrices, fused Muon step with "
                      f"{'stabilized Gram' if variant == 'gram' else 'standard'} Newton-Schulz, "
                      f"numpy fp64, {dt:.1f} s"}


def vendor_gemm(args):
    """Context for the roofline: the vendor library's plain batched products (torch.bmm, fp16,
    contiguous operands, no epilogue) on the shapes of the step's products. Not part of the
    library; prints one JSON line of its own."""
    import torch
    B, n, m = args.batch, min(args.rows, args.cols), max(args.rows, args.cols)
    dt = torch.float16
    gen = torch.Generator(device="cuda").manual_seed(7)
    A = torch.randn(B, n, n, device="cuda", dtype=dt, generator=gen)

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    C = torch.randn(B, n, n, device="cuda", dtype=dt, generator=gen)
    D = torch.empty(B, n, n, device="cuda", dtype=dt)
    ms = timed(lambda: torch.bmm(A, C, out=D))
    out["square_nxnxn"] = {"ms": ms, "tflops": 2 * B * n ** 3 / ms / 1e9}
    del C, D
    X = torch.randn(B, n, m, device="cuda", dtype=dt, generator=gen)
    Y = torch.empty(B, n, m, device="cuda", dtype=dt)
    ms = timed(lambda: torch.bmm(A, X, out=Y))
    out["rect_nxnxm"] = {"ms": ms, "tflops": 2 * B * n * n * m / ms / 1e9}
    del Y
    Xt = X.transpose(1, 2).contiguous()
    R = torch.empty(B, n, n, device="cuda", dtype=dt)
    ms = timed(lambda: torch.bmm(X, Xt, out=R))
    out["gram_nxmxn_full"] = {"ms": ms, "tflops": 2 * B * n * n * m / ms / 1e9}
    print(json.dumps({"comparison": "torch.bmm fp16 (vendor GEMM), plain batched products",
                      "batch": B, "n": n, "m": m, "products": out}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--variant", choices=["gram", "standard"], default="gram")
    ap.add_argument("--workload", choices=["experts", "experts_1408", "dense_ffn", "k2_full", "k2_hybrid",
                                           "adamw"], default="experts",
                    help="experts: the Kimi-K2 expert batch, --batch x --rows x --cols (default 648 x "
                         "2048 x 7168) Gaussian plus a rank-32 spike; experts_1408: 64 x 1408 x 2048 "
                         "low-rank (s_i = i^-0.7) plus 0.05 noise, lr 2e-4, wd 0.1; dense_ffn: 3 x 7168 x "
                         "18432 low-rank (s_i = i^-0.5) plus 0.05 noise; k2_full: the whole Kimi-K2 Muon "
                         "step in one grouped call (432 x 2048 x 7168 up/gate, 216 x 7168 x 2048 down, "
                         "3 x 7168 x 18432 dense); k2_hybrid: k2_full plus AdamW on the 1-D / embedding "
                         "parameters; adamw: the AdamW side alone")
    ap.add_argument("--batch", type=int, default=648)
    ap.add_argument("--rows", type=int, default=2048)
    ap.add_argument("--cols", type=int, default=7168)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-standard", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="comparison only: time torch.bmm (the vendor GEMM library) on the plain "
                         "products of the step's shapes and print that instead of the bench line")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "--gpus > 1 is not supported: this library runs on one GPU (the "
                          "batch of matrices would shard across GPUs with no exchange inside "
                          "Newton-Schulz)"}))
        sys.exit(2)

    import torch
    import synth
    from newton_schulz_matrix_muon_amd import flops, ops

    dev = torch.device("cuda:0")
    if args.copy_probe_mib > 0:
        log(f"copy probe: {args.copy_probe_mib} MiB")
        copy_probe(args.copy_probe_mib)
    if args.workload == "adamw":
        return bench_adamw(args)
    if args.vendor_gemm:
        return vendor_gemm(args)
    # inputs: (generator name, workload index of the seeds) per preset
    gen_kind, widx = "spike", 2
    steps_kw = dict(lr=0.02, momentum=0.95, weight_decay=0.01, scale_coeff=0.2, nesterov=True)
    if args.workload == "experts":
        shapes = [(args.batch, args.rows, args.cols)]
        workload = f"kimi_k2_experts_{args.batch}x{args.rows}x{args.cols}_bf16_gaussian_plus_rank32_spike"
    elif args.workload == "experts_1408":
        shapes = [(64, 1408, 2048)]
        gen_kind, widx = ("lowrank", 0.7), 1
        steps_kw.update(lr=2e-4, weight_decay=0.1)
        workload = "experts_64x1408x2048_bf16_powerlaw0.7_plus_noise0.05"
    elif args.workload == "dense_ffn":
        shapes = [(3, 7168, 18432)]
        gen_kind, widx = ("lowrank", 0.5), 3
        workload = "kimi_k2_dense_ffn_3x7168x18432_bf16_powerlaw0.5_plus_noise0.05"
    else:
        shapes = [(432, 2048, 7168), (216, 7168, 2048), (3, 7168, 18432)]
        workload = "kimi_k2_full_step_432x2048x7168+216x7168x2048+3x7168x18432_bf16_gaussian_plus_rank32_spike"
        if args.workload == "k2_hybrid":
            workload = "kimi_k2_hybrid_step_muon_" + workload[len("kimi_k2_full_step_"):] + "+adamw_1d_embedding"
    vectors = adamw_params(torch, dev) if args.workload == "k2_hybrid" else None
    groups = [(B, min(r, c), max(r, c)) for B, r, c in shapes]
    total = sum(B for B, _, _ in shapes)
    Gs, Ws, Ms = [], [], []
    for i, (B, r, c) in enumerate(shapes):
        if gen_kind == "spike":
            log(f"generating {B} x {r} x {c} bf16 gradients (Gaussian + rank-32 spike)")
            Gs.append(synth.torch_gaussian_plus_spike(B, r, c, workload_index=widx, device=dev))
        else:
            log(f"generating {B} x {r} x {c} bf16 gradients (power law i^-{gen_kind[1]} + 0.05 noise)")
            Gs.append(synth.torch_lowrank_plus_noise(B, r, c, power=gen_kind[1], noise=0.05,
                                                     workload_index=widx, device=dev, chunk=1 if r * c > 1 << 26 else 8))
        Ws.append(synth.torch_weights(B, r, c, workload_index=widx, device=dev, seed_offset=500_000 + i))
        Ms.append(torch.zeros(B, r, c, dtype=torch.float32, device=dev))

    p_g = ops.ns_params(io_dtype=ops.BF16, restart_mask=1 << 2)
    p_s = ops.ns_params(io_dtype=ops.BF16, restart_mask=0)
    if len(shapes) == 1:
        ws_bytes = max(ops.workspace_bytes(ops.GRAM, Gs[0], p_g), ops.workspace_bytes(ops.STANDARD, Gs[0], p_s))
    else:
        ws_bytes = max(ops.workspace_bytes_grouped(ops.GRAM, Gs, p_g),
                       ops.workspace_bytes_grouped(ops.STANDARD, Gs, p_s))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    log(f"workspace {ws_bytes / 1e9:.1f} GB")

    cpu = None
    if not args.no_cpu_baseline:
        # bounded sample: the oracle stops after --cpu-budget seconds (one matrix at least, which
        # for the 7168 x 18432 dense matrices is already ~30 s of host work)
        k = 1 if shapes[0][1] * shapes[0][2] > 1 << 26 else min(shapes[0][0], 24)
        Gh = Gs[0][:k].double().cpu().numpy()
        Wh = Ws[0][:k].double().cpu().numpy()

    def step(variant_code):
        if len(shapes) == 1:
            ops.muon_step(Ws[0], Gs[0], Ms[0], variant=variant_code, workspace=ws, **steps_kw)
        elif vectors is None:
            ops.muon_step_grouped(Ws, Gs, Ms, variant=variant_code, workspace=ws, **steps_kw)
        else:
            ops.hybrid_step(list(zip(Ws, Gs, Ms)), vectors,
                            muon=dict(variant=variant_code, workspace=ws, **steps_kw), adamw=ADAMW_KW)

    per_step_ms = []

    def timed(variant_code, steps, warmup, with_kernel_timing):
        for _ in range(warmup):
            step(variant_code)
        torch.cuda.synchronize()
        if with_kernel_timing:
            ops.timing_reset()
            ops.timing_enable(True)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        evs[0].record()
        for i in range(steps):
            step(variant_code)
            evs[i + 1].record()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        kt = None
        if with_kernel_timing:
            ops.timing_enable(False)
            kt = ops.timing_query()
            per_step_ms[:] = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        return dt / steps, kt

    main_code = ops.GRAM if args.variant == "gram" else ops.STANDARD
    log(f"timing {args.variant}: warmup {args.warmup}, steps {args.steps}")
    with ClockSampler() as clk:
        sec, kt = timed(main_code, args.steps, args.warmup, True)
    # event timing adds a few microseconds per launch; report the untimed run too
    sec_plain, _ = timed(main_code, max(1, args.steps // 2), 0, False)
    log(f"{args.variant}: {sec * 1e3:.2f} ms/step (with events), {sec_plain * 1e3:.2f} ms/step plain")

    def work(fn):
        return sum(B * fn(r, c) for B, r, c in shapes)

    def algo(variant):
        return work(flops.gram_flops if variant == "gram" else flops.standard_flops)

    def executed(variant):
        return work(flops.gram_executed_flops if variant == "gram" else flops.standard_flops)

    variants = {}
    def summarize(name, s):
        f = algo(name)
        variants[name] = {"ms_per_step": s * 1e3, "matrices_per_s": total / s,
                          "algorithmic_tflops": f / s / 1e12,
                          "executed_tflops": executed(name) / s / 1e12,
                          "frac_bf16_peak": f / s / 1e12 / PEAK_MFMA_TFLOPS,
                          "std_equivalent_tflops": work(flops.standard_dense_flops) / s / 1e12}
    summarize(args.variant, sec)
    if not args.skip_standard:
        other = "standard" if args.variant == "gram" else "gram"
        oc = ops.STANDARD if other == "standard" else ops.GRAM
        log(f"timing {other}")
        s2, _ = timed(oc, max(1, args.steps // 2), 1, False)
        summarize(other, s2)
        log(f"{other}: {s2 * 1e3:.2f} ms/step")

    # dominant kernel and its roofline
    kinds = {k: v for k, v in kt.items() if v[1] > 0}
    dom = max(kinds, key=lambda k: kinds[k][0])
    tot_ms, launches = kinds[dom]
    avg_s = tot_ms / launches / 1e3
    amount, unit, bound = kind_work(dom, groups)
    if dom in ("prep_norm", "finalize_norm"):   # one launch per group: average group's work
        amount /= len(groups)
    if unit == "flop":
        achieved = amount / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_MFMA_TFLOPS, "traffic": None}
    else:
        achieved = amount / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None}
    traffic, tsrc = recorded_traffic(dom, workload)
    roof["traffic"] = traffic
    if traffic is not None:
        roof["traffic_unit"] = "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
        roof["traffic_source"] = f"profiles/{tsrc}"
    clock = clk.summary()
    if clock and unit == "flop":
        # the dense peak scales with the graphics clock (2.4 GHz at the published figure)
        roof["frac_at_run_clock"] = achieved / (PEAK_MFMA_TFLOPS * clock["median_mhz"] / 2400.0)
    roof["kernel"] = dom
    roof["avg_launch_ms"] = avg_s * 1e3
    roof["launches"] = launches
    per_kind = {}
    for k, (ms, cnt) in kinds.items():
        w = kind_work(k, groups)
        e = {"total_ms_per_step": ms / args.steps, "launches_per_step": cnt / args.steps,
             "avg_launch_ms": ms / cnt}
        if w:
            amt, u, _ = w
            # a GEMM launch covers every group; the norm kernels run once per group
            rounds = cnt / args.steps / (len(groups) if k in ("prep_norm", "finalize_norm") else 1)
            e["achieved"] = amt * rounds / (ms / args.steps / 1e3) / (1e12 if u == "flop" else 1e9)
            e["unit"] = "TFLOP/s" if u == "flop" else "GB/s"
        per_kind[k] = e

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(Gh, Wh, args.cpu_budget, args.variant, steps_kw)

    config = {"workload": workload,
              "groups": [{"batch": B, "rows": r, "cols": c} for B, r, c in shapes],
              "step": f"fused Muon step, {args.variant} Newton-Schulz K=5"
                      + (" (fp16 iterates, restart after step 2)" if args.variant == "gram" else ""),
              "lr": steps_kw["lr"], "momentum": steps_kw["momentum"], "nesterov": steps_kw["nesterov"],
              "weight_decay": steps_kw["weight_decay"], "scale": "0.2*sqrt(max(rows, cols))"}
    if len(shapes) == 1:
        config.update(batch=shapes[0][0], rows=shapes[0][1], cols=shapes[0][2])
    out = {
        "metric": "NS-orthogonalized matrices/sec and effective TFLOP/s (% bf16 MFMA peak)",
        "value": total / sec,
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 io, fp16 iterates",
        "data": "synthetic",
        "config": config,
        "effective_tflops": variants[args.variant]["algorithmic_tflops"],
        "frac_bf16_peak": variants[args.variant]["frac_bf16_peak"],
        "ms_per_step_plain": sec_plain * 1e3,
        "step_ms": {"median": sorted(per_step_ms)[len(per_step_ms) // 2], "min": min(per_step_ms),
                    "max": max(per_step_ms)},
        "sclk": clk.summary(),
        "variants": variants,
        "kernels": per_kind,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
