#!/usr/bin/env python3
"""Throughput of one GPU's tensor-parallel GPT layer shard, forward + backward.

A step is one mt_layer_fwd + mt_layer_bwd of the shard over one micro-batch of seeded
synthetic inputs already resident in HBM. Default workload: the GPT-175B layer shape,
shard 0 of tp=8 (h=12288, 12 of 96 heads of 128, seq 2048, micro-batch 1, bf16).

Reported (one JSON line): model TFLOP/s = 3 x (forward GEMM + causal attention FLOPs)
per step / step time, its fraction of the MI355X dense bf16 MFMA peak, the roofline
of the dominant kernel (the step's largest launch, the FC2 backward pair; timed live
with HIP events that the library records on its stream around that launch, in a pass of
further steps after the headline ones), the graphics clock sampled while steps run, the
fp64 oracle timed on the host, and (outside the timed steps) the fused AdamW step over
the shard's parameters against HBM bandwidth.

Headline timing: W warmup steps, then K steps with library timing off, each between its
own pair of HIP events on the library's stream, each preceded (outside its events) by a
512 MiB write that evicts the previous step's data from the 256 MB MALL; ms_per_step is
the median of the K step times.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "model TFLOP/s per GPU, GPT layer-shard fwd+bwd; % of bf16 MFMA peak"
# HBM traffic of the reported kernel launch, measured with rocprofv3 counters and committed
# as a summary per launch label; it is reported only while the GEMM sources hash to the
# value recorded there.
def traffic_file(label: str, workload: str = "gpt175b_tp8") -> str:
    return os.path.join(ROOT, "profiles", f"{label}_{workload}_traffic.txt")


GEMM_SOURCES = ["tensor_layer_gemms_amd/csrc/gemm_dma.hpp", "tensor_layer_gemms_amd/csrc/gemm_kernels.hpp",
                "tensor_layer_gemms_amd/csrc/gemm_bf16.hip", "tensor_layer_gemms_amd/csrc/gemm.hpp",
                "tensor_layer_gemms_amd/csrc/device_common.hpp"]


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str = "gpt175b_tp8"):
    """Bytes per launch of `kernel` from the committed counter summary of `workload`, or
    None when the summary is missing, is for another kernel, or predates the current GEMM
    sources."""
    try:
        kv = {}
        with open(traffic_file(kernel, workload)) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("label") != kernel or kv.get("gemm_source_hash") != gemm_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


SCRUB_BYTES = 512 << 20  # written before every timed step: twice the 256 MB MALL

# Precision modes each workload has a green oracle parity test in (tests/test_gpu_parity.py);
# the first is the default. The 1T shard and the h=8192 stage need the compensated logits
# (MT_BF16_QK): with bf16 Q and K their normwise error is ~2.3-3%, over the 2e-2 bar.
PARITY_MODES = {"tiny_fp32": ("fp32",), "gpt_h1024": ("bf16", "bf16qk"), "gpt175b_tp8": ("bf16", "bf16qk"),
                "gpt1t_tp8": ("bf16qk",)}
PARITY_MODES.update({f"gpt_h8192_stage_mb{b}": ("bf16qk",) for b in (1, 2, 4, 8)})


def workload_mode(workload: str, requested=None) -> str:
    """The mode bench.py runs `workload` in: the requested one if its parity is green,
    else the workload's default; exits on a mode without a green parity test."""
    modes = PARITY_MODES.get(workload)
    if modes is None:
        sys.exit(f"bench.py: unknown workload {workload!r} (one of {sorted(PARITY_MODES)})")
    if requested is None:
        return modes[0]
    if requested not in modes:
        sys.exit(f"bench.py: {workload} has no green oracle parity test in mode {requested} (modes: {modes})")
    return requested


def dominant_pass(mt, torch, step, scrub, stream, label: str, steps: int, workload: str):
    """Roofline of the launch labelled `label`: its algorithmic FLOPs over its average
    duration, from HIP events the library records around that launch on its stream
    during `steps` further steps (scrubbed like the headline steps)."""
    mt.timing_reset()
    mt.timing_enable(True, label)
    for i in range(steps):
        scrub.fill_(i & 0xFF)
        step()
    torch.cuda.synchronize()
    mt.timing_enable(False)
    recs = [r for r in mt.timing_records() if r[0] == label]
    mt.timing_reset()
    if not recs:
        return None
    durs = sorted(r[1] for r in recs)
    avg_ms = sum(durs) / len(durs)
    kflops = recs[0][2]
    achieved = kflops / (avg_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": committed_traffic(label, workload), "kernel": label,
            "avg_ms": round(avg_ms, 4), "median_ms": round(statistics.median(durs), 4), "launches": len(recs),
            "gflop_per_launch": round(kflops / 1e9, 2)}


def clock_pass(torch, step, stream, seconds: float = 3.0, settle: float = 1.0):
    """Graphics clock while the steps run: amd-smi's GPU metrics (the mean of the eight
    XCDs' current clocks, MHz), sampled from a host thread every ~20 ms while untimed
    steps run for `seconds`; the metrics table refreshes about once a second, so samples
    from the first `settle` seconds (still showing the idle clock) are dropped. Median and
    range of the kept samples; None when the amd-smi library is not usable here."""
    import threading
    try:
        sys.path.insert(0, "/opt/rocm/share/amd_smi")
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # noqa: BLE001 - the clock is reported as unavailable
        return {"mhz": None, "reason": f"amd-smi unavailable: {type(e).__name__}"}

    def read():
        m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
        v = m.get("current_gfxclks")
        if isinstance(v, (list, tuple)):
            v = [x for x in v if isinstance(x, (int, float)) and 0 < x < 10000]
            if v:
                return sum(v) / len(v)
        v = m.get("current_gfxclk")
        return float(v) if isinstance(v, (int, float)) and 0 < v < 10000 else None

    samples, stop = [], threading.Event()
    t_start = [0.0]

    def sampler():
        while not stop.is_set():
            try:
                v = read()
            except Exception:  # noqa: BLE001
                v = None
            if v is not None and time.perf_counter() - t_start[0] >= settle:
                samples.append(v)
            time.sleep(0.02)

    th = threading.Thread(target=sampler, daemon=True)
    torch.cuda.synchronize()
    t_start[0] = time.perf_counter()
    th.start()
    while time.perf_counter() - t_start[0] < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    if not samples:
        return {"mhz": None, "reason": "no gpu-metrics clock field"}
    samples.sort()
    return {"mhz": round(statistics.median(samples), 1), "min": round(samples[0], 1), "max": round(samples[-1], 1),
            "samples": len(samples), "source": "amd-smi gpu_metrics current_gfxclks (mean of the XCDs), "
                                              f"{seconds - settle:.0f} s of steps after {settle:.0f} s settling"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt175b_tp8")
    ap.add_argument("--dominant", default="fc2_dgrad_wgrad",
                    help="label of the kernel launch whose roofline is reported (default: the step's largest "
                         "launch, the FC2 backward dgrad + wgrad pair)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-optimizer", action="store_true", help="skip the fused AdamW step measurement")
    ap.add_argument("--no-sp", action="store_true", help="skip the sequence-parallel share measurement")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the graphics-clock samples (3 s of untimed steps; for profiled runs)")
    ap.add_argument("--mode", choices=["bf16", "bf16qk", "fp32"], default=None,
                    help="precision mode (default: the workload's, see PARITY_MODES); bf16qk = MT_BF16_QK, the "
                         "attention logits from hi + lo pairs of Q and K")
    ap.add_argument("--breakdown", action="store_true", help="also print a per-launch time breakdown (stderr)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes three times (counter calibration)")
    return ap.parse_args()


def copy_probe(nbytes: int) -> None:
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}), flush=True)


def recompute_report(shape, ms_per_step: float, saved_bytes: int):
    """Hardware vs model FLOPs of the fused-attention path, and the activation bytes it
    does not store. The backward recomputes the attention probabilities P = exp(S - L)
    from Q, K and the saved row log-sum-exp instead of keeping P (selective
    recomputation of the attention core). In the MT_BF16_QK mode the logits are formed
    in three segments (Q_hi K_hi + Q_hi K_lo + Q_lo K_hi) and the QKV forward adds
    U_lo W_qk^T. Counted per head product over the s (s + 1) / 2 causal (query, key)
    pairs, as the model FLOPs are: forward n logit segments + P V; backward, key-block
    part n logit segments + dP + dV + dK, row-block part n logit segments + dP + dQ,
    with n = 3 (MT_BF16_QK) or 1."""
    if shape.dtype != "bf16" or shape.head_dim not in (64, 128, 160):
        return None
    B, s, at, d = shape.micro_batch, shape.seq, shape.heads_per_shard, shape.head_dim
    M, h, t = shape.tokens, shape.h, shape.tp
    nseg = 3 if shape.qk_pairs else 1
    unit = 2.0 * B * at * d * s * (s + 1) / 2  # one causal head product
    model = si_model_flops(shape)
    attn_model = 6 * unit
    attn_hw = (nseg + 1) * unit + (nseg + 3) * unit + (nseg + 2) * unit
    qkv_comp = 2.0 * M * (2 * h // t) * h if shape.qk_pairs else 0.0
    hw = model - attn_model + attn_hw + qkv_comp
    p_bytes = B * at * s * s * 2  # bf16 probabilities a materialised backward would keep
    return {"model_gflop": round(model / 1e9, 1), "hardware_gflop": round(hw / 1e9, 1),
            "hardware_tflops": round(hw / (ms_per_step * 1e-3) / 1e12, 1),
            # the backward's logits recomputed in both parts (every segment)
            "bwd_logit_recompute_gflop": round(2 * nseg * unit / 1e9, 1),
            # dP formed in both backward parts (one extra head product)
            "bwd_dp_duplicate_gflop": round(unit / 1e9, 1),
            # forward (MT_BF16_QK): the two extra logit segments and U_lo W_qk^T
            "fwd_compensation_gflop": round(((nseg - 1) * unit + qkv_comp) / 1e9, 1),
            "p_bytes_not_stored": int(p_bytes), "saved_store_bytes": int(saved_bytes)}


def si_model_flops(shape) -> float:
    import seeded_inputs as si
    return si.model_flops(shape, causal=True)


def optimizer_step(mt, si, torch, shape, stream, warmup: int = 2, iters: int = 10):
    """Fused AdamW step over the shard's parameters in one flat fp32 buffer (with the
    bf16 copy): average launch time from HIP events on the library's stream, against
    HBM bandwidth (30 bytes per parameter: read p, g, m, v; write p, m, v, bf16 p)."""
    n = si.shard_param_count(shape)
    print(f"[bench] AdamW step over {n} parameters", file=sys.stderr, flush=True)
    bufs = [torch.from_numpy(a).cuda() for a in si.adam_case(n, seed=0)]
    q = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    hp = si.ADAM_HPARAMS
    for _ in range(warmup):
        mt.adamw_step(*bufs, q, stream=stream, **hp)
    torch.cuda.synchronize()
    mt.timing_reset()
    mt.timing_enable(True, "adamw")
    for _ in range(iters):
        mt.adamw_step(*bufs, q, stream=stream, **hp)
    torch.cuda.synchronize()
    mt.timing_enable(False)
    recs = [r for r in mt.timing_records() if r[0] == "adamw"]
    mt.timing_reset()
    avg_ms = sum(r[1] for r in recs) / len(recs)
    nbytes = recs[0][3]
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    return {"kernel": "adamw", "params": n, "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "avg_ms": round(avg_ms, 4),
            "launches": len(recs), "bytes_per_launch": int(nbytes)}


def sp_share(mt, si, torch, shape, w, x, dout, stream, warmup: int = 3, iters: int = 10):
    """One rank's sequence-parallel share of the same layer step (shard 0 of the group):
    LayerNorm, bias + residual on the rank's seq/tp rows, the attention and MLP blocks on
    the gathered rows. The collectives are not part of one GPU's work: each gathered
    buffer holds this rank's rows (written by its own calls) and synthetic rows standing
    for the other ranks; the rank's reduce-scattered rows are its own partial's rows (the
    one-GPU stand-in, as the identity is for the all-reduce). Micro-batch 1, so the
    rank's rows are the first seq/tp rows and every slot is a pointer offset."""
    if shape.micro_batch != 1 or shape.seq % shape.tp or shape.dtype != "bf16" or shape.qk_pairs:
        return None
    print("[bench] sequence-parallel share of the step (rank 0)", file=sys.stderr, flush=True)
    sh = mt.make_shape(shape.h, shape.heads, shape.seq, shape.micro_batch, shape.tp, shape.shard, "bf16")
    M, h = shape.tokens, shape.h
    n = M // shape.tp
    act = torch.bfloat16
    f32 = dict(dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)  # seeded synthetic rows standing for the other ranks
    U, V2, dOut, dX2 = (torch.randn(M, h, device="cuda", generator=gen).to(act) for _ in range(4))
    O, Y, dV2, dU = (torch.empty(M, h, dtype=act, device="cuda") for _ in range(4))
    xi, douti = x[:n], dout[:n]
    x2, dx2f = torch.empty(n, h, **f32), torch.empty(n, h, **f32)
    out_i, dx_i = torch.empty(n, h, dtype=act, device="cuda"), torch.empty(n, h, dtype=act, device="cuda")
    st = [torch.empty(n, **f32) for _ in range(4)]
    g = {k: torch.empty(v.shape, **f32) for k, v in w.items()}
    asv = torch.empty(mt.attn_saved_bytes(sh), dtype=torch.uint8, device="cuda")
    msv = torch.empty(mt.mlp_saved_bytes(sh), dtype=torch.uint8, device="cuda")
    aws = torch.empty(mt.attn_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    mws = torch.empty(mt.mlp_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    lws = torch.empty(mt.sp_ln_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    dOut[:n] = douti

    def step():
        mt.sp_ln_fwd(sh, xi, w["ln1_g"], w["ln1_b"], U[:n], st[0], st[1], stream=stream)
        mt.attn_fwd(sh, U, w["w_qkv"], w["b_qkv"], w["w_o"], O, asv, aws, stream)
        mt.sp_ln_fwd(sh, xi, w["ln2_g"], w["ln2_b"], V2[:n], st[2], st[3], resid=O[:n], bias=w["b_o"], x2=x2,
                     stream=stream)
        mt.mlp_fwd(sh, V2, w["w_fc1"], w["b_fc1"], w["w_fc2"], Y, msv, mws, stream)
        mt.sp_add_fwd(sh, x2, Y[:n], w["b_fc2"], out_i, stream=stream)
        mt.mlp_bwd(sh, V2, w["w_fc1"], w["w_fc2"], msv, dOut, dV2, g["w_fc1"], g["b_fc1"], g["w_fc2"], mws, stream)
        mt.sp_ln_bwd(sh, dV2[:n], x2, w["ln2_g"], st[2], st[3], douti, dX2[:n], g["ln2_g"], g["ln2_b"], lws,
                     xin_f32=True, dres_f32=False, dx_f32=dx2f, dsum=g["b_o"], dres_sum=g["b_fc2"], stream=stream)
        mt.attn_bwd(sh, U, w["w_qkv"], w["w_o"], asv, dX2, dU, g["w_qkv"], g["b_qkv"], g["w_o"], aws, stream)
        mt.sp_ln_bwd(sh, dU[:n], xi, w["ln1_g"], st[0], st[1], dx2f, dx_i, g["ln1_g"], g["ln1_b"], lws,
                     xin_f32=False, dres_f32=True, stream=stream)

    for _ in range(warmup):
        step()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(iters):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / iters
    mt.timing_reset()
    mt.timing_enable(True, "sp_")
    step()
    torch.cuda.synchronize()
    mt.timing_enable(False)
    row_ms = sum(r[1] for r in mt.timing_records())
    mt.timing_reset()
    flops = si.model_flops(shape, causal=True)
    # activations a rank keeps between its forward and backward for the row-local parts:
    # x2 (fp32) and four fp32 row statistics over n rows, against M rows without SP
    return {"rank": 0, "rows": n, "ms_per_step": round(ms, 4), "model_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "row_local_ms": round(row_ms, 4), "steps": iters,
            "row_local_saved_bytes": int(n * h * 4 + 4 * n * 4), "tp_row_local_saved_bytes": int(M * h * 4 + 4 * M * 4)}


def cpu_baseline(case, shape, min_seconds: float = 10.0, max_steps: int = 5):
    """The fp64 oracle, as it stands, on whole steps of the same workload: repeated until
    at least min_seconds of CPU work (at most max_steps steps)."""
    import numpy as np
    import oracle
    import seeded_inputs as si
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in pools] or [1])
        if pools:
            blas = f"{pools[0].get('internal_api', '?')} {pools[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    steps = 0
    while steps < max_steps and (steps == 0 or time.perf_counter() - t0 < min_seconds):
        out, c = oracle.layer_fwd(case.x, case.layers[:1], shape.micro_batch, shape.seq, shape.head_dim)
        dx, g = oracle.layer_bwd(case.dout, c, case.layers[:1])
        del out, c, dx, g
        steps += 1
    dt = time.perf_counter() - t0
    flops = steps * si.model_flops(shape)
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} full fwd+bwd step(s) of the same shard (h={case.shape.h}, M={shape.tokens}) in "
                      f"NumPy fp64, {dt:.1f} s", "seconds": round(dt, 2), "cpu": cpu_model(), "blas": blas,
            "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU's tensor-parallel shard only (asked for --gpus {args.gpus}); the "
              "tensor-parallel all-reduce is not part of it. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import seeded_inputs as si
    import tensor_layer_gemms_amd as mt

    if not os.path.exists(mt.LIB_PATH):
        from tensor_layer_gemms_amd.build import build
        build()
    mt.lib()
    mode = workload_mode(args.workload, args.mode)
    w = si.WORKLOADS[args.workload]
    shape = w.shape.replace(qk_pairs=mode == "bf16qk")
    print(f"[bench] generating seeded inputs for {args.workload}", file=sys.stderr, flush=True)
    case = si.workload_case(args.workload)
    dev = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16 if shape.dtype == "bf16" else torch.float32)  # noqa
    sh = mt.make_shape(shape.h, shape.heads, shape.seq, shape.micro_batch, shape.tp, shape.shard, mode)
    L = w.layers
    weights = [{k: dev(v) for k, v in p.items()} for p in case.layers]
    grads = [{k: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in p.items()} for p in case.layers]
    acts = [dev(case.x)] + [torch.empty_like(dev(case.x)) for _ in range(L)]
    dout = dev(case.dout)
    dxs = [torch.empty_like(dout) for _ in range(L)]
    saved = [torch.empty(mt.layer_saved_bytes(sh), dtype=torch.uint8, device="cuda") for _ in range(L)]
    ws = torch.empty(mt.layer_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    for l in range(L):
        mt.check_layer_tensors(sh, weights[l], grads[l], x=acts[l], out=acts[l + 1], dx=dxs[l])
    stream = torch.cuda.current_stream()

    def step():
        for l in range(L):
            mt.layer_fwd(sh, weights[l], acts[l], acts[l + 1], saved[l], ws, stream)
        g = dout
        for l in reversed(range(L)):
            mt.layer_bwd(sh, weights[l], acts[l], saved[l], g, dxs[l], grads[l], ws, stream)
            g = dxs[l]

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-launch breakdown (untimed pass, every launch bracketed by events)
    breakdown = None
    if args.breakdown:
        mt.timing_reset()
        mt.timing_enable(True, None)
        step()
        torch.cuda.synchronize()
        mt.timing_enable(False)
        breakdown = mt.timing_records()
        mt.timing_reset()

    # Headline: K steps with library timing off. Each step is bracketed by its own pair of
    # events on the library's stream; before each step (outside its events) a 512 MiB
    # write evicts the previous step's weights and activations from the 256 MB MALL.
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        scrub.fill_(i & 0xFF)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = sorted(a.elapsed_time(b) for a, b in ev)
    ms_per_step = statistics.median(step_ms)
    flops_step = L * si.model_flops(shape, causal=True)
    dense_step = L * si.model_flops(shape, causal=False)
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    # The dominant launch, timed in a separate pass of the same steps: the library records
    # HIP events around that launch only.
    roofline = dominant_pass(mt, torch, step, scrub, stream, args.dominant, args.steps, args.workload)
    sclk = None if args.no_clock else clock_pass(torch, step, stream)

    optim = None if args.no_optimizer else optimizer_step(mt, si, torch, shape, stream)
    sp = sp_share(mt, si, torch, shape, weights[0], acts[0], dout, stream) if L == 1 and not args.no_sp else None

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host (whole steps, at least 10 s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case, shape)

    if breakdown:
        tot = sum(r[1] for r in breakdown)
        print(f"[bench] breakdown of one step ({tot:.3f} ms in launches):", file=sys.stderr)
        for lab, ms, fl, by in breakdown:
            rate = f"{fl / ms / 1e9:8.1f} TFLOP/s" if fl else f"{by / ms / 1e6:8.1f} GB/s   "
            print(f"  {lab:18s} {ms:8.4f} ms {100 * ms / tot:5.1f}%  {rate}", file=sys.stderr)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if shape.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": args.workload, "h": shape.h, "heads": shape.heads, "heads_per_shard":
                   shape.heads_per_shard, "head_dim": shape.head_dim, "seq": shape.seq,
                   "micro_batch": shape.micro_batch, "tp": shape.tp, "shard": shape.shard, "layers": L,
                   "mode": mode,
                   "gflop_per_step_causal": round(flops_step / 1e9, 1),
                   "gflop_per_step_dense": round(dense_step / 1e9, 1)},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "dense_count_tflops": round(dense_step / (ms_per_step * 1e-3) / 1e12, 2),
        "wall_s_timed": round(wall, 3),
        "step_ms": {"median": round(ms_per_step, 4), "mean": round(sum(step_ms) / len(step_ms), 4),
                    "min": round(step_ms[0], 4), "max": round(step_ms[-1], 4),
                    "mall_scrub_bytes": SCRUB_BYTES},
        "sclk": sclk,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "optimizer_step": optim,
        "sp_share": sp,
        "recompute": recompute_report(shape, ms_per_step, mt.layer_saved_bytes(sh)) if L == 1 else None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
