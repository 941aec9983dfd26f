"""Benchmark: one GPU's share of a headwise-chunked causal GQA attention layer,
forward + backward, through the C ABI.

Workload (default): Llama3-8B attention shape at long context -- S = 131072,
d_model 4096, 32 query heads, 8 KV heads, d_head 128, U = 4 (one KV group per
stage), causal, bf16; seed-0 Gaussian inputs drawn on the GPU (X ~ N(0,1),
W ~ N(0, 1/d_model), dO ~ N(0,1)).  A step is one forward and one backward of
the whole layer (every stage); inputs are resident in HBM before timing.

Prints one JSON line.  `value` is causal attention fwd+bwd TFLOP/s on the
step's wall clock (algorithmic flops 7*d*S*(S+1) per query head: 2 matmuls
forward, 5 backward, causal pairs only), so projection and gradient GEMM time
is counted against it.  Per-kernel times come from HIP events recorded around
every launch on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attn fwd+bwd TFLOP/s & % bf16 MFMA peak at S=128K; peak bytes vs U"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="llama8b_s128k")
    ap.add_argument("--U", type=int, default=None)
    ap.add_argument("--pipeline", action="store_true",
                    help="stage pipelining: the GEMMs of neighbouring stages on a second stream")
    ap.add_argument("--rope-theta", type=float, default=0.0,
                    help="rotary embedding of queries and keys with this base (0: none)")
    ap.add_argument("--out-proj", action="store_true",
                    help="the layer with its output projection (upipe_fwd_out / upipe_bwd_out)")
    ap.add_argument("--qk-norm", action="store_true",
                    help="QK-norm of queries and keys (eps 1e-6), through upipe_fwd_ex / upipe_bwd_ex")
    ap.add_argument("--skip-cpu-baseline", action="store_true",
                    help="omit the oracle timing (profiling runs only)")
    ap.add_argument("--cpu-baseline-S", type=int, default=16384)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (HBM counter calibration)")
    return ap.parse_args()


def attn_flops(S, H, d, causal=True):
    pairs = S * (S + 1) / 2 if causal else float(S) * S
    return 14.0 * d * pairs * H  # 2 fwd + 5 bwd matmuls, 2*d flops each per pair


H_ALL = 32  # query heads of the layer (set from the workload in main)


def kernel_work(kind, S, D, d, U, r, causal=True):
    """Algorithmic work of one launch of `kind` in a stage of U query heads
    (U >= r: whole groups).  Returns (amount, unit)."""
    pairs = S * (S + 1) / 2 if causal else float(S) * S
    nkv = max(1, U // r)
    if kind == "attn_fwd":
        return 4.0 * d * pairs * U, "flop"        # S = QK^T, O = PV
    if kind == "attn_dkv":
        return 8.0 * d * pairs * U, "flop"        # QK^T, dO V^T, P^T dO, dS^T Q
    if kind == "attn_dq":
        return 2.0 * d * pairs * U, "flop"        # dS K
    if kind == "proj":
        return 2.0 * S * D * d * (U + 2 * nkv), "flop"
    if kind == "dw":
        return 2.0 * S * D * d * (U + 2 * nkv), "flop"
    if kind == "dx":
        return 2.0 * S * D * d * (U + 2 * nkv), "flop"
    if kind == "bwd_pre":
        return (2.0 * 2 * S * d + 12.0 * S) * U, "byte"  # read O, dO (bf16), LSE; write D, LSE*log2e (fp32)
    if kind == "fill":
        return 4.0 * S * D, "byte"
    if kind == "dout":  # output projection's dO = dY Wo for a stage's heads
        return 2.0 * S * D * d * U, "flop"
    if kind in ("oproj", "dwo"):  # Y = O Wo^T and dWo = dY^T O, one launch for all heads (H <= 64)
        return 2.0 * S * D * d * H_ALL, "flop"
    return 0.0, "flop"


KERNEL_SOURCES = ("bf16_common.h", "kernels_bf16.hip", "kernels_dkv.hip", "rope_device.h")


def _code_only(text):
    """C++ source without its comments and blank-line / trailing-space
    differences, so that editing a comment keeps the hash."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = []
    for line in text.splitlines():
        code = re.sub(r"//.*$", "", line).rstrip()
        if code:
            out.append(code)
    return "\n".join(out)


def source_sha():
    """First 16 hex digits of the sha256 over the code (comments stripped) of
    the bf16 kernel sources."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "headwise_chunked_context_stage_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic_llama8b_s128k_U4.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except ValueError:
        return None
    if t.get("source_sha") != source_sha():
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def gpu_sclk_sample(out: dict, delay_s: float = 0.5):
    """The shader clock the driver reports while the timed steps execute: the
    current level ('*') of each card's pp_dpm_sclk in sysfs (what
    rocm-smi --showclocks prints), read from this process after delay_s."""
    import glob

    time.sleep(delay_s)
    found = []
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            cur = [ln.strip() for ln in open(f) if ln.strip().endswith("*")]
        except OSError:
            continue
        if cur:
            found.append("%s: %s" % (f.split("/")[4], cur[0]))
    out["sclk"] = found or None


def cpu_baseline(S_sample, D, d, S_full=None, H_full=None, G_full=None):
    """The fp64 oracle on a bounded sample of the workload: one query head and
    its KV head at S_sample tokens, full d_model, causal, forward + backward.
    With the full layer's shape, also an extrapolated full-layer time, scaling
    the measured time by the ratio of total work (causal attention plus
    projections) -- an estimate, labelled as such."""
    import numpy as np

    import oracle
    from headwise_chunked_context_stage_amd.synth import LayerShape, make_inputs, to_numpy_exact

    oracle.build(force=False)
    shape = LayerShape(S=S_sample, D=D, H=1, G=1, d=d)
    inp = make_inputs(shape, "bf16", seed=0, device="cpu")
    arrs = [to_numpy_exact(inp[k]) for k in ("X", "Wq", "Wk", "Wv", "dO")]
    nthreads = oracle.default_threads()
    t0 = time.perf_counter()
    out = oracle.backward(*arrs, 1, 1, d, causal=True, nthreads=nthreads)
    dt = time.perf_counter() - t0
    assert np.isfinite(out["dX"]).all()
    flops = attn_flops(S_sample, 1, d)
    extra = {}
    if S_full and H_full and G_full:
        work = lambda S, H, G: attn_flops(S, H, d) + 8.0 * S * D * (H + 2 * G) * d
        extra["extrapolated_full_layer_s"] = dt * work(S_full, H_full, G_full) / work(S_sample, 1, 1)
        extra["extrapolation"] = ("sample time x (full-layer / sample) work, work = 7 d S(S+1) H "
                                  "+ 8 S D (H + 2G) d; an estimate, not a measurement")
    return {
        **extra,
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": nthreads,
        "cpu_model": host_cpu_model(),
        "kind": "oracle",
        "sample": ("1 query head + its KV head, S=%d, d_model=%d, d_head=%d, causal, fwd+bwd "
                   "incl. projections and weight/input gradients; %.1f s; TFLOP/s counts causal "
                   "attention flops only, as for the GPU value" % (S_sample, D, d, dt)),
        "seconds": dt,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU's share of the layer; the multi-GPU layer (head shards "
              "with all-to-all exchanges between devices) is not implemented (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from headwise_chunked_context_stage_amd import upipe
    from headwise_chunked_context_stage_amd.layer import alloc_outputs, backward, forward
    from headwise_chunked_context_stage_amd.synth import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    upipe.lib()
    cfg = CONFIGS[args.config]
    shape = cfg["shape"]
    U = args.U or cfg["U"][0]
    S, D, H, G, d = shape.S, shape.D, shape.H, shape.G, shape.d
    r = H // G
    global H_ALL
    H_ALL = min(H, 64)
    dev = torch.device("cuda:0")
    print("bench: %s S=%d D=%d H=%d G=%d d=%d U=%d%s" % (args.config, S, D, H, G, d, U,
                                                       " pipelined" if args.pipeline else ""),
          file=sys.stderr, flush=True)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("bench: calibration copy of %d bytes" % n, file=sys.stderr, flush=True)
        del src, dst
    inp = make_inputs(shape, cfg["dtype"], seed=0, device="cuda", out_proj=args.out_proj,
                      qk_norm=args.qk_norm)
    plan = upipe.Plan(S, D, H, G, d, U, causal=True, dtype=cfg["dtype"], pipeline=args.pipeline,
                      rope_theta=args.rope_theta, out_proj=args.out_proj, qk_norm=args.qk_norm)
    out = alloc_outputs(plan, dev)
    if args.out_proj:
        out["Y"] = torch.empty((S, D), dtype=torch.float32, device=dev)
        out["dWo"] = torch.empty((D, H * d), dtype=torch.float32, device=dev)
    fio = bio = None
    if args.qk_norm:  # every option through the io-struct entry points
        out["dq_norm"] = torch.empty((d,), dtype=torch.float32, device=dev)
        out["dk_norm"] = torch.empty((d,), dtype=torch.float32, device=dev)
        fio = dict(X=inp["X"], Wq=inp["Wq"], Wk=inp["Wk"], Wv=inp["Wv"], q_norm=inp["q_norm"],
                   k_norm=inp["k_norm"], O=out["O"], LSE=out["LSE"])
        bio = dict(fio, dX=out["dX"], dWq=out["dWq"], dWk=out["dWk"], dWv=out["dWv"],
                   dq_norm=out["dq_norm"], dk_norm=out["dk_norm"])
        if args.out_proj:
            fio.update(Wo=inp["Wo"], Y=out["Y"])
            bio.update(Wo=inp["Wo"], dY=inp["dY"], dWo=out["dWo"])
        else:
            bio["dO"] = inp["dO"]
    torch.cuda.synchronize()
    mem_before = torch.cuda.memory_allocated()

    def step():
        if args.qk_norm:
            plan.fwd_ex(fio, out["ws"])
            plan.bwd_ex(bio, out["ws"])
        elif args.out_proj:
            plan.fwd_out(inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"], out["O"],
                         out["LSE"], out["Y"], out["ws"])
            plan.bwd_out(inp["dY"], inp["X"], inp["Wq"], inp["Wk"], inp["Wv"], inp["Wo"],
                         out["O"], out["LSE"], out["dX"], out["dWq"], out["dWk"], out["dWv"],
                         out["dWo"], out["ws"])
        else:
            forward(plan, inp, out)
            backward(plan, inp, out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    upipe.upipe_timing_enable(True)
    upipe.upipe_timing_read()  # drop anything pending
    torch.cuda.synchronize()
    # step boundaries as events on the stream every call is enqueued on (the
    # current stream: the library runs there unless pipelined, and a
    # pipelined call joins its helper stream back before returning)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    import threading

    clock = {}
    sampler = threading.Thread(target=gpu_sclk_sample, args=(clock,), daemon=True)
    t0 = time.perf_counter()
    marks[0].record()
    sampler.start()
    for i in range(args.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    sampler.join(timeout=60)
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    upipe.upipe_timing_enable(False)
    ktimes = upipe.upipe_timing_read()
    high_water_delta = torch.cuda.max_memory_allocated() - mem_before
    for k in ("O", "LSE", "dX", "dWq", "dWk", "dWv"):
        assert torch.isfinite(out[k]).all(), k

    ms_per_step = 1e3 * elapsed / args.steps
    aflops = attn_flops(S, H, d)
    value = aflops / (ms_per_step * 1e-3) / 1e12
    proj_flops = 8.0 * S * D * (H + 2 * G) * d + (6.0 * S * D * H * d if args.out_proj else 0.0)

    kernels = {}
    for kind, rec in ktimes.items():
        if rec["launches"] == 0:
            continue
        n_per_step = rec["launches"] / args.steps
        avg_ms = rec["ms"] / rec["launches"]
        work, unit = kernel_work(kind, S, D, d, min(U, H), r)
        ent = {"ms_per_step": rec["ms"] / args.steps, "launches_per_step": n_per_step,
               "avg_launch_ms": avg_ms}
        if kind in ("attn_fwd", "attn_dkv", "attn_dq", "proj", "dw", "dx", "oproj", "dout",
                    "dwo") and (U >= r or kind in ("attn_fwd", "attn_dkv", "attn_dq")):
            ent["tflops"] = work / (avg_ms * 1e-3) / 1e12
        elif kind in ("bwd_pre", "fill"):
            ent["gbps"] = work / (avg_ms * 1e-3) / 1e9
        kernels[kind] = ent
    attn_ms = sum(kernels.get(k, {}).get("ms_per_step", 0.0)
                  for k in ("attn_fwd", "bwd_pre", "attn_dkv", "attn_dq"))
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dwork, dunit = kernel_work(dominant, S, D, d, min(U, H), r)
    dk = kernels[dominant]
    if dunit == "flop":
        achieved = dwork / (dk["avg_launch_ms"] * 1e-3) / 1e12
        roof = {"kernel": dominant, "bound": "mfma", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": traffic_for(dominant),
                "work_per_launch": dwork, "avg_launch_ms": dk["avg_launch_ms"]}
    else:
        achieved = dwork / (dk["avg_launch_ms"] * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic_for(dominant),
                "work_per_launch": dwork, "avg_launch_ms": dk["avg_launch_ms"]}

    # measured dense-MFMA ceiling of this chip (every CU, 2 waves per SIMD,
    # random bf16 operands, ~0.1 s per run so the clock has settled; best of
    # two): context for frac, which stays against the published peak
    ceiling = max(upipe.upipe_mfma_ceiling(2, 1 << 16) for _ in range(2))
    roof["measured_mfma_ceiling"] = ceiling
    if dunit == "flop":
        roof["frac_of_measured_ceiling"] = roof["achieved"] / ceiling
    for k, ent in kernels.items():
        if "tflops" in ent:
            ent["frac_of_peak"] = ent["tflops"] / PEAK_BF16_TFLOPS
        if k == "dx":  # fp32 dX read-modify-write per stage launch, against HBM
            ent["dX_rmw_gbps"] = 8.0 * S * D / (ent["avg_launch_ms"] * 1e-3) / 1e9

    peak_by_u = {}
    for u in cfg["U"] + (1, H):
        if H % u == 0 and (r % u == 0 or u % r == 0):
            p = upipe.Plan(S, D, H, G, d, u, causal=True, dtype=cfg["dtype"])
            peak_by_u[str(u)] = {"fwd": p.peak_bytes_phase(0), "bwd": p.peak_bytes_phase(1),
                                 "pages_projection_form_6SUd": 6 * S * u * d}

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_ms_median": step_ms[len(step_ms) // 2],
        "step_ms_min": step_ms[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == "bf16" else "f32",
        "data": "synthetic (seed-0 Gaussian X, W, dO drawn on the GPU; no dataset or weights)",
        "config": {"workload": "causal GQA attention layer fwd+bwd, one GPU, Llama3-8B attention "
                               "shape" if args.config.startswith("llama") else args.config,
                   "name": args.config, "S": S, "d_model": D, "H": H, "G": G, "d_head": d,
                   "U": U, "pipeline": args.pipeline, "rope_theta": args.rope_theta,
                   "out_proj": args.out_proj, "qk_norm": args.qk_norm, "causal": True,
                   "seed": 0},
        "host": {"cpu_model": host_cpu_model(), "gpu_sclk_during_steps": clock.get("sclk")},
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "attn_kernels_tflops": aflops / (attn_ms * 1e-3) / 1e12 if attn_ms > 0 else None,
        "attn_kernels_pct_peak": (100.0 * aflops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
                                  if attn_ms > 0 else None),
        "layer_tflops_incl_projections": (aflops + proj_flops) / (ms_per_step * 1e-3) / 1e12,
        "tokens_per_s_layer_fwd_bwd": S / (ms_per_step * 1e-3),
        "peak_bytes": {"U": U, "ws_fwd": plan.peak_bytes_phase(0),
                       "ws_bwd": plan.peak_bytes_phase(1),
                       "device_high_water_delta_during_steps": high_water_delta,
                       "by_U": peak_by_u},
        "kernels": kernels,
        "roofline": roof,
        "kernel_source_sha": source_sha(),
        "torch": torch.__version__,
    }
    if not args.skip_cpu_baseline:
        print("bench: timing the oracle on the host (bounded sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_baseline_S, D, d, S, H, G)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
