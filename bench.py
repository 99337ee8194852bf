"""Benchmark of one MuonClip optimizer step on one MI355X.

A step is the whole hot path over one batch of synthetic input: the per-head
max logit of every attention layer (max_logits_per_head) followed by
muonclip_step (momentum, Newton-Schulz, RMS-matched decoupled update, QK-Clip)
over every 2-D parameter of the workload. Inputs are resident in HBM before
the timed region starts.

Default workload: one full K2-shaped layer (MLA attention with 64 heads of
192/128, S_max over one causal sequence of 32768 tokens; the five MLA
projections, the dense 7168 x 18432 FFN and 385 experts of 7168 x 2048 /
2048 x 7168, 1163 bf16 matrices with fp32 momentum). --config 2 is the MHA
layer, 3 the MLA layer, 4 the experts alone, 1 the tiny fp32 case.

Prints one JSON line. `value` is the median step time in ms over the timed
steps (lower is better); the same line carries the Newton-Schulz TFLOP/s,
S_max Glogits/s and its fraction of the MFMA peak, elementwise GB/s, the
roofline of the dominant kernel (the NS GEMM) measured with HIP events around
every launch of the library in a second pass that runs one lane, and the fp64
oracle timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MuonClip step ms & NS TFLOP/s (% MFMA peak); S_max Glogits/s; elementwise GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def smax_peak_glogits(d_q: int) -> float:
    """Logits per second at the bf16 MFMA peak: 2 d_q FLOPs per logit."""
    return PEAK_BF16_TFLOPS * 1e12 / (2.0 * d_q) / 1e9


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5, help="workload 1..5 (default: 5, the full K2-shaped layer)")
    ap.add_argument("--experts", type=int, default=385, help="expert count for workloads 4/5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--overlap-smax", action="store_true",
                    help="run the S_max pass on a second stream beside momentum and Newton-Schulz "
                         "(muonclip_step_overlapped) instead of before the step")
    ap.add_argument("--cpu-sample-s", type=float, default=15.0)
    ap.add_argument("--adamw", action="store_true",
                    help="time the AdamW entry point (the parameters Muon does not cover) on a "
                         "synthetic set: one 512M-element vector plus 64 norm-sized vectors of 7168")
    ap.add_argument("--attention", action="store_true",
                    help="time attention_forward (softmax attention with S_max taken from its own row "
                         "maxima) on the attention shape of --config (2: MHA layer, 3: MLA layer), against "
                         "the same forward without S_max and the separate max_logits_per_head pass")
    ap.add_argument("--clip", action="store_true",
                    help="time qk_clip_apply alone on the MLA layer's q_b (12288 x 1536) and kv_b (16384 x 512) "
                         "with every head above tau (4 bytes per clipped bf16 element)")
    ap.add_argument("--reference", action="store_true",
                    help="time the vendor baselines on this GPU: torch's streaming kernels (read, copy, add of "
                         "4 GiB fp32 tensors) and hipBLASLt (torch.bmm / mm) on the Newton-Schulz product shapes of "
                         "64 expert matrices and an 8192^3 bf16 GEMM")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain streaming copy of MIB MiB (read + write) five times, "
                         "to calibrate the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


GEMM_SOURCE = os.path.join(ROOT, "muonclip_step_amd", "csrc", "ns_gemm.hip")


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"ns_gemm_traffic_{workload}.txt")


def gemm_source_hash() -> str:
    import hashlib
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """Memory bytes per ns_gemm launch from the committed rocprofv3 counter
    runs of this workload (profiles/ns_gemm_traffic_<workload>.txt), or None
    when there are none or they were taken on another kernel source."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("ns_gemm_source_sha256_16") != gemm_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib: int):
    """A plain streaming kernel of known size: reads and writes mib MiB."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}), flush=True)


def ns_flops(rows, cols, steps):
    m, n = min(rows, cols), max(rows, cols)
    return steps * 2.0 * (2.0 * n * m * m + m ** 3)


def build_workload(cfg, dev):
    """Device buffers for every matrix plus Q/K of every attention layer."""
    import numpy as np
    import torch

    import muonclip_step_amd as mc
    import workloads as wl

    mats, keep = [], []
    host_w = {}
    for i, s in enumerate(cfg.matrices):
        if s.device_drawn:
            w, g, m = wl.draw_device_tensors(cfg, i, dev)
        else:
            wh = wl.draw_weight(cfg, i)
            host_w[s.name] = wh
            w = torch.from_numpy(wh).to(torch.bfloat16 if s.w_dtype == "bf16" else torch.float32).to(dev)
            g = torch.from_numpy(wl.draw_grad(cfg, i)).to(dev)
            m = torch.from_numpy(wl.draw_momentum(cfg, i)).to(dev)
        keep += [w, g, m]
        mats.append(mc.matrix(w, g, m, clip_slot=s.clip_slot, period=s.period, segments=s.segments))
    attn = None
    if cfg.attn is not None:
        q, k, ks = wl.draw_attention_inputs(cfg, host_w)
        dt = torch.bfloat16 if cfg.attn.dtype == "bf16" else torch.float32
        qd = torch.from_numpy(np.ascontiguousarray(q)).to(dt).to(dev)
        kd = torch.from_numpy(np.ascontiguousarray(k)).to(dt).to(dev)
        ksd = torch.from_numpy(np.ascontiguousarray(ks)).to(dt).to(dev) if ks is not None else None
        attn = (qd, kd, ksd)
        del q, k, ks
    return mats, keep, attn


def cpu_baseline(cfg, budget_s, dev=None):
    """The fp64 oracle on a bounded sample of the same workload, scaled to a
    full step: whole matrices (momentum -> NS -> update -> clip) until the
    budget is spent (the smallest device-drawn matrix first, copied to the
    host, then the host-drawn ones, smallest first), and S_max of a few
    (sample, head) slices."""
    import numpy as np

    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    hp = cfg.hparams
    t_mat, done_mats, flops_done = 0.0, 0, 0.0
    total_flops = sum(ns_flops(s.rows, s.cols, hp["ns_steps"]) for s in cfg.matrices)
    order = sorted((i for i, s in enumerate(cfg.matrices) if not s.device_drawn),
                   key=lambda i: ns_flops(cfg.matrices[i].rows, cfg.matrices[i].cols, hp["ns_steps"]))
    dev_ids = [i for i, s in enumerate(cfg.matrices) if s.device_drawn]
    first_dev = min(dev_ids, key=lambda i: ns_flops(cfg.matrices[i].rows, cfg.matrices[i].cols, hp["ns_steps"]),
                    default=None)
    if first_dev is not None and dev is not None:
        order = [first_dev] + order
    for i in order:
        s = cfg.matrices[i]
        if s.device_drawn:
            wd, gd, md = wl.draw_device_tensors(cfg, i, dev)
            w, g, m = wd.float().cpu().numpy(), gd.cpu().numpy(), md.cpu().numpy()
            del wd, gd, md
        else:
            w, g, m = wl.draw_weight(cfg, i), wl.draw_grad(cfg, i), wl.draw_momentum(cfg, i)
        t0 = time.perf_counter()
        oracle.muonclip_step_matrix(w.astype(np.float64), g.astype(np.float64), m.astype(np.float64),
                                    lr=hp["lr"], mu=hp["mu"], weight_decay=hp["weight_decay"],
                                    w_dtype=s.w_dtype)
        t_mat += time.perf_counter() - t0
        done_mats += 1
        flops_done += ns_flops(s.rows, s.cols, hp["ns_steps"])
        if t_mat > budget_s * 0.7:
            break
    ms_muon = t_mat / flops_done * total_flops * 1e3 if flops_done else float("nan")
    ms_smax, sl = 0.0, 0
    a = cfg.attn
    if a is not None:
        q = wl.quantize_bf16(wl.normal(99, 0, (1, a.T, 1, a.d_q), 1.0))
        k = wl.quantize_bf16(wl.normal(99, 1, (1, a.T, 1, a.d_k), 1.0))
        ks = wl.quantize_bf16(wl.normal(99, 2, (1, a.T, a.d_shared), 1.0)) if a.d_shared else None
        t0 = time.perf_counter()
        while True:
            oracle.max_logits(q, k, ks, a.causal, 1.0 / math.sqrt(a.d_q))
            sl += 1
            if time.perf_counter() - t0 > budget_s * 0.3:
                break
        per = (time.perf_counter() - t0) / sl
        ms_smax = per * a.B * a.H * 1e3
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu_model)
    except OSError:
        pass
    return {"value": ms_muon + ms_smax, "unit": "ms per step (extrapolated)", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model,
            "sample": f"{done_mats} of {len(cfg.matrices)} matrices through the full fp64 step, scaled by NS "
                      f"FLOPs to all matrices; S_max on {sl} single (sample, head) slices of T={a.T if a else 0},"
                      f" scaled by B*H" if a else f"{done_mats} matrices, scaled by NS FLOPs"}


def adamw_bench(args):
    """AdamW over bf16 parameters with fp32 gradients and moments: 24 bytes
    per element (read p, g, m, v; write p, m, v). Prints its own JSON line."""
    import torch

    import muonclip_step_amd as mc
    mc.load()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    sizes = [512 * 1024 * 1024] + [7168] * 64
    keep, vecs = [], []
    for n in sizes:
        p = (torch.randn(n, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        g = torch.randn(n, generator=gen, device=dev) * 1e-3
        m = torch.zeros(n, device=dev)
        v = torch.zeros(n, device=dev)
        keep += [p, g, m, v]
        vecs.append(mc.vector(p, g, m, v))
    elems = sum(sizes)
    torch.cuda.synchronize()
    for t in range(1, args.warmup + 1):
        mc.adamw_step(vecs, mc.adamw_hparams(step=t))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(args.warmup + 1, args.warmup + 1 + args.steps):
        mc.adamw_step(vecs, mc.adamw_hparams(step=t))
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = elems * 24.0 / (ms * 1e-3) / 1e9
    # context: a plain device copy of 4 GiB (read + write) on the same GPU
    src = torch.empty(1 << 30, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    print(json.dumps({"metric": "AdamW GB/s (non-matrix parameters)", "value": round(gbs, 1), "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
                      "higher_is_better": True, "dtype": "f32", "data": "synthetic",
                      "config": {"workload": "adamw", "elements": elems, "vectors": len(sizes),
                                 "bytes_per_element": 24},
                      "copy_gbs": round(copy_gbs, 1),
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}}), flush=True)


def attention_bench(args):
    """attention_forward on one attention layer's seeded Q, K, V (resident on
    the device): with S_max and lse (the fused path), without them (the plain
    forward), and max_logits_per_head alone (the pass the fused path makes
    unnecessary). Prints its own JSON line; value = the fused forward in ms."""
    import numpy as np
    import torch

    import muonclip_step_amd as mc
    import workloads as wl
    mc.load()
    if args.config not in (2, 3):
        raise SystemExit("--attention covers --config 2 (MHA layer) and 3 (MLA layer)")
    cfg = wl.config(args.config)
    a = cfg.attn
    print(f"[bench] drawing Q, K, V of {cfg.name}", file=sys.stderr, flush=True)
    wts = {s.name: wl.draw_weight(cfg, i) for i, s in enumerate(cfg.matrices) if not s.device_drawn}
    q, k, ks = wl.draw_attention_inputs(cfg, wts)
    v = wl.draw_attention_values(cfg, wts)
    dev = torch.device("cuda:0")
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(dev)
    qd, kd, vd = up(q), up(k), up(v)
    ksd = up(ks) if ks is not None else None
    del q, k, ks, v, wts
    o = torch.empty(a.B, a.T, a.H, a.d_v, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(a.B, a.H, a.T, dtype=torch.float32, device=dev)
    smax = torch.empty(a.H, dtype=torch.float32, device=dev)
    fused = lambda: mc.attention_forward(qd, kd, ksd, vd, causal=True, out=o, lse=lse, s_max=smax)
    plain = lambda: mc.attention_forward(qd, kd, ksd, vd, causal=True, out=o)
    separate = lambda: mc.max_logits_per_head(qd, kd, ksd, causal=True, out=smax)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_fused, ms_plain, ms_sep = timed(fused), timed(plain), timed(separate)
    mc.profile_enable(True)
    for _ in range(args.steps):
        fused()
    torch.cuda.synchronize()
    prof = mc.profile_read()
    mc.profile_enable(False)
    at = prof["attention"]
    tflops = at["flops"] / (at["ms"] * 1e-3) / 1e12
    pairs = a.B * a.H * a.T * (a.T + 1) / 2
    print(json.dumps({
        "metric": "attention forward with S_max ms (fused S_max source)", "value": round(ms_fused, 4), "unit": "ms",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_fused, 4),
        "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name + "_attention", "attention": f"B{a.B} T{a.T} H{a.H} d{a.d_q}/{a.d_v} causal"},
        "forward_without_smax_ms": round(ms_plain, 4),
        "smax_overhead_ms": round(ms_fused - ms_plain, 4),
        "separate_max_logits_pass_ms": round(ms_sep, 4),
        "logits": int(pairs),
        "roofline": {"bound": "mfma", "kernel": "attn_fwd", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "avg_launch_us": round(at["ms"] / max(1, at["launches"]) * 1e3, 2)},
    }), flush=True)


def reference_bench(args):
    """Vendor baselines on this GPU, as context for the roofline fractions:
    the HBM rates torch's own streaming kernels reach, and the bf16 rates of
    hipBLASLt (through torch.bmm / torch.mm, every operand contiguous) on the
    three Newton-Schulz products of a 64-matrix wave of 2048 x 7168 expert
    matrices (full products: the library computes only the upper tiles of
    the two symmetric ones) and on an 8192^3 GEMM. Prints one JSON line."""
    import torch
    dev = torch.device("cuda:0")

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
    n = 1 << 29                                    # 2 GiB fp32 per tensor (one launch per op)
    a = torch.ones(n, device=dev)
    b = torch.ones(n, device=dev)
    c = torch.empty(n, device=dev)
    out["hbm_read_sum_gbs"] = round(4 * n / (timed(lambda: a.sum()) * 1e-3) / 1e9, 1)
    out["hbm_copy_gbs"] = round(8 * n / (timed(lambda: c.copy_(a)) * 1e-3) / 1e9, 1)
    out["hbm_add_2r1w_gbs"] = round(12 * n / (timed(lambda: torch.add(a, b, out=c)) * 1e-3) / 1e9, 1)
    del a, b, c
    B, m, k = 64, 2048, 7168
    P = torch.randn(B, m, m, device=dev).to(torch.bfloat16)
    X = torch.randn(B, m, k, device=dev).to(torch.bfloat16)
    XT = X.transpose(1, 2).contiguous()
    Y = torch.empty(B, m, k, device=dev, dtype=torch.bfloat16)
    G = torch.empty(B, m, m, device=dev, dtype=torch.bfloat16)
    f_mmk, f_mmm = 2.0 * B * m * m * k, 2.0 * B * m ** 3
    out["hipblaslt_apply_tflops"] = round(f_mmk / (timed(lambda: torch.bmm(P, X, out=Y)) * 1e-3) / 1e12, 1)
    out["hipblaslt_gram_full_tflops"] = round(f_mmk / (timed(lambda: torch.bmm(X, XT, out=G)) * 1e-3) / 1e12, 1)
    out["hipblaslt_aa_full_tflops"] = round(f_mmm / (timed(lambda: torch.bmm(P, P, out=G)) * 1e-3) / 1e12, 1)
    del P, X, XT, Y, G
    s8 = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    t8 = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    out["hipblaslt_mm8192_tflops"] = round(2.0 * 8192 ** 3 / (timed(lambda: torch.mm(s8, t8)) * 1e-3) / 1e12, 1)
    print(json.dumps({"metric": "vendor baselines on this GPU", "unit": "GB/s and TFLOP/s", "n_gpus": 1,
                      "config": {"workload": "reference", "expert_wave": "64 x (2048 x 7168)"}, **out}), flush=True)


def clip_bench(args):
    """qk_clip_apply on the MLA projections that carry head rows (q_b: q^C
    rows by sqrt(gamma), q^R rows by gamma; kv_b: k^C rows by sqrt(gamma))
    with an S_max above tau on every head, so every head's segments are read
    and written: 4 bytes per clipped bf16 element. Prints its own JSON line."""
    import numpy as np
    import torch

    import muonclip_step_amd as mc
    import workloads as wl
    mc.load()
    dev = torch.device("cuda:0")
    cfg = wl.config(3)
    names = [s.name for s in cfg.matrices]
    mats, keep, clipped = [], [], 0
    for nm in ("q_b", "kv_b"):
        i = names.index(nm)
        s = cfg.matrices[i]
        w = torch.from_numpy(wl.draw_weight(cfg, i)).to(torch.bfloat16).to(dev)
        d = torch.zeros(w.shape, dtype=torch.float32, device=dev)   # g, m: unused by the clip
        keep += [w, d]
        mats.append(mc.matrix(w, d, d, clip_slot=0, period=s.period, segments=s.segments))
        clipped += (s.rows // s.period) * sum(seg[1] for seg in s.segments) * s.cols
    H = cfg.attn.H
    s_max = torch.from_numpy(np.full(H, 2.0 * cfg.tau, np.float32)).to(dev)   # gamma = 0.5 on every head
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        mc.qk_clip_apply(mats, s_max, 1, H, cfg.tau)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        mc.qk_clip_apply(mats, s_max, 1, H, cfg.tau)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    ms = per[len(per) // 2]
    mc.profile_enable(True)
    for _ in range(args.steps):
        mc.qk_clip_apply(mats, s_max, 1, H, cfg.tau)
    torch.cuda.synchronize()
    prof = mc.profile_read()
    mc.profile_enable(False)
    k = prof["clip_apply"]
    kern_gbs = clipped * 4.0 * args.steps / (k["ms"] * 1e-3) / 1e9
    gbs = clipped * 4.0 / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "QK-Clip apply GB/s (standalone, every head clipped)", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "mla_clip", "matrices": "q_b 12288x1536, kv_b 16384x512", "clipped_elements": clipped,
                   "bytes_per_element": 4},
        "roofline": {"bound": "hbm", "kernel": "clip_apply", "achieved": round(kern_gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(kern_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "avg_launch_us": round(k["ms"] / max(1, k["launches"]) * 1e3, 2),
                     "launches_per_call": k["launches"] // args.steps},
    }), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported by this build "
              "(the step shards by whole matrices; no multi-GPU path exists here).", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.adamw:
        adamw_bench(args)
        return
    if args.attention:
        attention_bench(args)
        return
    if args.clip:
        clip_bench(args)
        return
    if args.reference:
        reference_bench(args)
        return

    import muonclip_step_amd as mc
    import workloads as wl

    mc.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kw = {"n_experts": args.experts} if args.config in (4, 5) else {}
    cfg = wl.config(args.config, **kw)
    print(f"[bench] building workload {cfg.name}", file=sys.stderr, flush=True)
    mats, keep, attn = build_workload(cfg, dev)
    hp = mc.hparams(**{**cfg.hparams, "tau": cfg.tau})
    H = cfg.attn.H if cfg.attn else 1
    s_max = torch.empty(H, dtype=torch.float32, device=dev)
    gamma = torch.empty(H, dtype=torch.float32, device=dev)
    ws = torch.empty(mc.workspace_size(mats, hp), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    ready = torch.cuda.Event()

    def step(overlap=args.overlap_smax):
        if attn is not None:
            q, k, ks = attn
            if overlap:
                # S_max on a second stream beside momentum and Newton-Schulz;
                # only the launches that read it wait for it
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    mc.max_logits_per_head(q, k, ks, causal=cfg.attn.causal, out=s_max)
                    ready.record(side)
                mc.muonclip_step(mats, hp, s_max=s_max, slots=1, heads=H, gamma_out=gamma, workspace=ws,
                                 s_max_ready=ready)
                torch.cuda.current_stream().wait_stream(side)
            else:
                mc.max_logits_per_head(q, k, ks, causal=cfg.attn.causal, out=s_max)
                mc.muonclip_step(mats, hp, s_max=s_max, slots=1, heads=H, gamma_out=gamma, workspace=ws)
        else:
            mc.muonclip_step(mats, hp, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    # one event between consecutive steps: every step's time, back to back
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] +
                                                                     step_ms[len(step_ms) // 2])
    ms_mean = ev[0].elapsed_time(ev[-1]) / args.steps
    print(f"[bench] median step {ms:.3f} ms; profiling one more pass per kernel", file=sys.stderr, flush=True)

    # per-kernel HIP events around every launch of the library, with the S_max
    # pass serialised and the step on one lane (the library does that while
    # profiling), so that no kernel's time includes another's
    prof_steps = min(args.steps, 5) if args.config in (4, 5) else args.steps
    mc.profile_enable(True)
    for _ in range(prof_steps):
        step(overlap=False)
    torch.cuda.synchronize()
    prof = mc.profile_read()
    mc.profile_enable(False)
    per_step = {k: {"ms": v["ms"] / prof_steps, "launches": v["launches"] // prof_steps} for k, v in prof.items()}
    g = prof.get("ns_gemm", {"ms": float("nan"), "flops": 0.0, "launches": 1})
    gemm_tflops = g["flops"] / (g["ms"] * 1e-3) / 1e12 if g["ms"] else float("nan")
    ml = prof.get("max_logits")
    n_logits = 0
    if cfg.attn is not None:
        a = cfg.attn
        n_logits = a.B * a.H * (a.T * (a.T + 1) // 2 if a.causal else a.T * a.T)
    smax_glogits = (n_logits * prof_steps / (ml["ms"] * 1e-3) / 1e9) if ml and ml["ms"] else None
    ew_bytes = sum(prof[k]["bytes"] for k in ("momentum_norm", "update_clip") if k in prof)
    ew_ms = sum(prof[k]["ms"] for k in ("momentum_norm", "update_clip") if k in prof)
    ew_gbs = ew_bytes / (ew_ms * 1e-3) / 1e9 if ew_ms else None
    ns_total = sum(ns_flops(s.rows, s.cols, hp.ns_steps) for s in cfg.matrices)
    ns_ms = sum(prof[k]["ms"] for k in ("ns_gemm", "splitk_reduce", "norm_finalize") if k in prof) / prof_steps
    # the NS GEMM and its split-K finishes, which together do the algorithmic work
    gemm_ms = sum(prof[k]["ms"] for k in ("ns_gemm", "splitk_reduce") if k in prof) / prof_steps
    gemm_alg_tflops = ns_total / (gemm_ms * 1e-3) / 1e12 if gemm_ms else float("nan")
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a host sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, args.cpu_sample_s, dev)
    out = {
        "metric": METRIC,
        "value": round(ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_mean": round(ms_mean, 4),
        "ms_per_step_min_max": [round(step_ms[0], 4), round(step_ms[-1], 4)],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "config": args.config, "matrices": len(cfg.matrices),
                   "elements": wl.elements(cfg),
                   "attention": None if cfg.attn is None else
                   f"B{cfg.attn.B} T{cfg.attn.T} H{cfg.attn.H} d{cfg.attn.d_q} "
                   f"{'causal' if cfg.attn.causal else 'full'} {cfg.attn.kind}",
                   "smax_pass": "second stream" if args.overlap_smax and cfg.attn else "serial",
                   "parallelism": "single GPU"},
        "ns_tflops_algorithmic": round(ns_total / (ns_ms * 1e-3) / 1e12, 2) if ns_ms else None,
        "ns_gemm_tflops": round(gemm_tflops, 2),
        "ns_mfma_frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
        "smax_glogits_s": round(smax_glogits, 1) if smax_glogits else None,
        "smax_mfma_frac": round(smax_glogits / smax_peak_glogits(cfg.attn.d_q), 4) if smax_glogits else None,
        "elementwise_gbs": round(ew_gbs, 1) if ew_gbs else None,
        "kernels_ms_per_step": {k: round(v["ms"], 4) for k, v in per_step.items()},
        # achieved: the method's algorithmic FLOPs (10 (2 n m^2 + m^3) per
        # matrix and step) over the NS GEMM kernel time; the launches run
        # fewer dense FLOPs (the Gram-space head), reported beside it
        "roofline": {"bound": "mfma", "kernel": "ns_gemm", "achieved": round(gemm_alg_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(gemm_alg_tflops / PEAK_BF16_TFLOPS, 4),
                     "flops": "algorithmic, 10 (2 n m^2 + m^3) per matrix and step",
                     "algorithmic_flops_per_step": ns_total,
                     "launched_dense_flops_per_step": g["flops"] / prof_steps,
                     "launched_dense_tflops": round(gemm_tflops, 2),
                     "launched_dense_frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(cfg.name),
                     "algorithmic_bytes_per_launch": round(g.get("bytes", 0.0) / max(1, g["launches"])),
                     "launches_per_step": per_step.get("ns_gemm", {}).get("launches"),
                     "ms_per_step": round(per_step.get("ns_gemm", {}).get("ms", float("nan")), 3),
                     "timing": "HIP events around each launch, one lane, %d steps" % prof_steps,
                     "avg_launch_us": round(g["ms"] / max(1, g["launches"]) * 1e3, 2)},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)
    del keep


if __name__ == "__main__":
    main()
