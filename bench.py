#!/usr/bin/env python3
"""Benchmark of one GLM-5.2-shaped MoE-layer forward on one MI355X.

A step is one full layer forward (router, top-k, dispatch, Q8_0 of x, gate-up +
SwiGLU, down, combine) over one batch of synthetic tokens, inputs already in HBM.
Workloads (GLM shape: H=6144, 256 routed experts in 8 groups, top-4 groups,
top-8, I=2048, one shared expert, rsf 2.5; int4 weights from N(0,0.02) with
per-row scales; Zipf(1.1) correction bias; hidden states N(0,1)):
  decode32  T=32 decode batch (default; the metric's headline workload)
  decode1   T=1
  mtp192    64 sequences x 3 positions, correlated (rho 0.8)
  prefill   T=2048
  stack40   40 layers at decode T=32: layers 0-19 resident in HBM, layers 20-39 with
            routed experts in pinned host memory behind a 64-slot LRU cache each
            (prints its own line: tokens/s, hit rate, PCIe bytes/s)
Weights rotate over --copies layer copies (different seeds) and every step
uses fresh tokens, so the 256 MB last-level cache cannot serve weights from a
previous step.

Prints one JSON line (rank 0). Multi-GPU runs are not supported: the library
runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

DEFAULT_GEMM_MIN = 5  # the library default of moe_config.gemm_min_tokens

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
# VALU lane-operations per second (non-packed): 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_OPS = 256 * 4 * 16 * 2.4e9
METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / int8 MFMA % (prefill)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 50; stack40: 12)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 5; stack40: 4)")
    ap.add_argument("--workload", default="decode32", choices=["decode32", "decode1", "mtp192", "prefill", "stack40"],
                    help="the headline workload of the JSON line")
    ap.add_argument("--configs", default=None,
                    help="comma-separated further workloads measured in the same run and reported under 'configs' "
                         "(default with the decode32 headline: decode1,mtp192,prefill,stack40; '' for none)")
    ap.add_argument("--config-steps", type=int, default=20, help="timed steps of each further workload")
    ap.add_argument("--graph", action="store_true",
                    help="also time the steps replayed as HIP graphs (one captured graph per step, same inputs)")
    ap.add_argument("--stack-layers", type=int, default=40, help="stack40: layers in the stack")
    ap.add_argument("--streamed", type=int, default=20, help="stack40: last layers whose experts stream from host")
    ap.add_argument("--slots", type=int, default=64, help="stack40: HBM expert slots per streamed layer")
    ap.add_argument("--pin", type=int, default=None,
                    help="stack40: after the warm-up steps (which record usage) pin this many of the most used "
                         "experts per streamed layer (learning cache); default %(default)s = 3/4 of the slots")
    ap.add_argument("--host-copies", type=int, default=12,
                    help="stack40: distinct host copies of routed experts; streamed layer j reads copy j mod this "
                         "(pinned host memory is capped below 20 layers' 97 GB on the measured box)")
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--gemm-min", type=int, default=0)
    ap.add_argument("--weight-bits", type=int, default=4, choices=[4, 8],
                    help="expert weight codes: 4 (row-tiled int4, the default) or 8 (row-tiled int8)")
    ap.add_argument("--topp", type=float, default=0.0,
                    help="adaptive expert top-p in (0, 1): keep the heaviest slots up to this weight (0: off)")
    ap.add_argument("--group-size", type=int, default=0,
                    help="int4 only: one weight scale per this many elements along K (0: one per row)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="run the plain read and copy kernels over 1 GiB (for hardware byte-counter calibration)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="summarise rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of a benchmark run and of "
                         "a --calibrate run into per-launch HBM bytes of the dominant kernel")
    a = ap.parse_args()
    if a.steps is None:
        a.steps = 12 if a.workload == "stack40" else 50
    if a.warmup is None:
        a.warmup = 4 if a.workload == "stack40" else 5
    if a.configs is None:
        a.configs = "decode1,mtp192,prefill,stack40" if a.workload == "decode32" else ""
    a.configs = [w for w in a.configs.split(",") if w and w != a.workload]
    bad = [w for w in a.configs if w not in ("decode32", "decode1", "mtp192", "prefill", "stack40")]
    if bad:
        ap.error(f"unknown workloads in --configs: {bad}")
    return a


def tokens_of(workload):
    return {"decode32": 32, "decode1": 1, "mtp192": 192, "prefill": 2048}[workload]


def make_inputs(shape, workload, n, seed):
    from synth import synth
    T = tokens_of(workload)
    xs = []
    for s in range(n):
        if workload == "mtp192":
            xs.append(synth.mtp_hidden_states(shape, 64, 3, 0.8, seed=seed, step=s))
        else:
            xs.append(synth.hidden_states(shape, T, seed=seed, step=s))
    return xs


def routing_stats(moe, cfg, layer, x_dev, ws, gemm_min):
    """Unique experts and bucket sizes of one batch (router + dispatch, outside the timed region)."""
    import torch
    T = x_dev.shape[0]
    E, K = cfg.n_experts, cfg.top_k
    dev = x_dev.device
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    moe.moe_router(cfg, x_dev, layer.router_w, layer.bias, ids, w, None, ws)
    outs = [torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
            torch.empty(T * K, dtype=torch.int32, device=dev), torch.empty(T * K, dtype=torch.int32, device=dev),
            torch.empty(E, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev)]
    moe.moe_dispatch(cfg, ids, *outs, ws)
    counts = outs[0].cpu().numpy()
    gm = gemm_min if gemm_min > 0 else DEFAULT_GEMM_MIN
    nz = counts[counts > 0]
    NS = cfg.n_shared  # each shared expert is one bucket of all T tokens
    return dict(U=int(nz.size), gemv_experts=int((nz < gm).sum()) + (NS if T < gm else 0),
                mfma_experts=int((nz >= gm).sum()) + (NS if T >= gm else 0),
                gemv_tokens=int(nz[nz < gm].sum()) + (NS * T if T < gm else 0),
                mfma_tokens=int(nz[nz >= gm].sum()) + (NS * T if T >= gm else 0), counts=counts)


SAMPLE_TOKENS = 8  # tokens of the CPU sample (each distinct expert they route to is generated once)


def cpu_baseline(shape, x, seconds, seed, weight_bits=4, group_size=0, topp=0.0):
    """The oracle as it stands, single-threaded, over the first SAMPLE_TOKENS tokens of the first batch: they are
    routed once and each distinct expert they need is generated once (outside the timing); then passes over
    them are timed until `seconds` of oracle time have been spent."""
    from oracle import oracle as O
    from synth import synth
    cfg = O.Cfg.of(shape, topp=topp)
    Wr = synth.router_weights(shape, seed)
    bias = synth.router_bias(shape, seed)
    x = x[:SAMPLE_TOKENS]
    T = x.shape[0]
    ids_all, _, _ = O.route(cfg, O.router_logits(x, Wr), bias)

    def gen(e, shared):
        if shared:
            w13, w2 = synth.shared_w13(shape, e, seed, 0), synth.shared_w2(shape, e, seed, 0)
        else:
            w13, w2 = synth.expert_w13(shape, e, seed, 0), synth.expert_w2(shape, e, seed, 0)
        if group_size:
            return O.quant_int4_grouped(w13, group_size) + O.quant_int4_grouped(w2, group_size)
        quant = O.quant_int8_rows if weight_bits == 8 else O.quant_int4_rows
        return quant(w13) + quant(w2)

    experts = {int(e): gen(int(e), False) for e in np.unique(ids_all) if e >= 0}
    shared = gen(0, True)
    done, t_oracle, passes = 0, 0.0, 0
    while t_oracle < seconds and passes < 20:
        for t in range(T):
            xt = x[t:t + 1]
            t0 = time.perf_counter()
            z = O.router_logits(xt, Wr)
            ids, w, _ = O.route(cfg, z, bias)
            qx, dx = O.q8_0(xt[0])
            rows = [O.expert_token(*experts[int(e)], qx, dx)["out"] if e >= 0 else np.zeros(shape.hidden, np.float32)
                    for e in ids[0]]
            rows.append(O.expert_token(*shared, qx, dx)["out"])
            O.combine(np.stack(rows[:-1])[None], np.stack(rows[-1:])[:, None], w, ids)
            t_oracle += time.perf_counter() - t0
            done += 1
            if t_oracle >= seconds:
                break
        passes += 1
    return dict(value=done / t_oracle, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{done} tokens ({passes} pass(es) over the first {T} tokens of the first batch), each: "
                       f"fp64 router over "
                       f"{shape.n_experts} experts, {shape.top_k} routed + 1 shared int{weight_bits}xint8 expert FFNs"
                       f"{f' (scales per {group_size})' if group_size else ''}, combine; "
                       f"{t_oracle:.1f} s of single-threaded oracle time (weight generation excluded)")


# sources the expert kernels are compiled from (their HBM counters go stale when either changes)
KERNEL_SRC = [os.path.join(ROOT, "int4_quantized_expert_amd", "csrc", f) for f in ("k_expert.hip", "moe_internal.h")]
CAL_BYTES = 1 << 30


def source_sha256():
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def calibrate():
    """Plain streaming kernels of known size: 1 GiB read, 1 GiB copied (read + written)."""
    import torch

    import int4_quantized_expert_amd as moe
    src = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty(CAL_BYTES, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        moe.moe_membench_read(src, 2048, 1, sink)
        moe.moe_membench_copy(src, dst, 4096)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate": "k_read 1 GiB x3, k_copy 1 GiB x3"}), flush=True)


def _pmc_rows(path):
    """(kernel name, counter value) per dispatch from a rocprofv3 counter_collection CSV."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            name = row["Kernel_Name"]
            out.setdefault(key, [name, 0.0])
            out[key][1] += float(row["Counter_Value"])
    return list(out.values())


def _mean_kib(rows, needle):
    v = [val for name, val in rows if needle in name]
    return (sum(v) / len(v), len(v)) if v else (float("nan"), 0)


def pmc_summary(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    """Per-launch HBM bytes of the dominant kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled
    by what the same counter reads for plain kernels of known traffic."""
    cal_read_kib, _ = _mean_kib(_pmc_rows(cal_fetch_csv), "k_read")
    cal_copy_kib, _ = _mean_kib(_pmc_rows(cal_write_csv), "k_copy")
    f_fetch = CAL_BYTES / (cal_read_kib * 1024.0)
    f_write = CAL_BYTES / (cal_copy_kib * 1024.0)
    lines = [f"calibration: k_read of {CAL_BYTES} B reads FETCH_SIZE {cal_read_kib:.1f} KiB -> factor {f_fetch:.4f}; "
             f"k_copy of {CAL_BYTES} B reads WRITE_SIZE {cal_copy_kib:.1f} KiB -> factor {f_write:.4f}", ""]
    lines.append("| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read B | HBM write B |")
    lines.append("|---|---|---|---|---|---|")
    fr, wr = _pmc_rows(fetch_csv), _pmc_rows(write_csv)
    names = sorted({n for n, _ in fr})
    res = {}
    for n in names:
        fk, cnt = _mean_kib(fr, n)
        wk, _ = _mean_kib(wr, n)
        rb, wb = fk * 1024.0 * f_fetch, wk * 1024.0 * f_write
        short = n.split("(")[0][:60]
        lines.append(f"| `{short}` | {cnt} | {fk:.1f} | {wk:.1f} | {rb:.4g} | {wb:.4g} |")
        res[n] = rb + wb
    print("\n".join(lines))
    for n, t in res.items():
        for k in ("k_gateup_gemv", "k_gateup_mfma"):
            if k in n:
                print(f"\ntraffic {k} bytes_per_launch {t:.6g}")
    print(f"source_sha256 {source_sha256()}")


def traffic_of(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None once the kernel source has changed."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    val, sha = None, None
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 4 and parts[0] == "traffic" and parts[1] == kernel:
                val = float(parts[3])
            if len(parts) == 2 and parts[0] == "source_sha256":
                sha = parts[1]
    return val if (val is not None and sha == source_sha256()) else None


def run_stack(args):
    """Stacked decode: every step runs all layers in order at T=32 on one residual stream (h = fresh tokens; layer
    input = weightless RMSNorm(h), eps 1e-6; h += the layer's output; the glue runs in torch on the compute stream);
    streamed layers go through their caches."""
    import torch

    import int4_quantized_expert_amd as moe
    from synth import synth
    from tests.harness import GpuLayer, config_of, host_experts

    sh = synth.GLM
    T, NL, NSTR = 32, args.stack_layers, args.streamed
    cfg = config_of(sh, args.gemm_min)
    dev = torch.device("cuda:0")
    layers, caches, hosts = [], [], []
    t_setup = time.perf_counter()
    for l in range(NL):
        g = GpuLayer(sh, seed=args.seed, layer=l)
        if l >= NL - NSTR:
            j = l - (NL - NSTR)
            if j < args.host_copies:
                hosts.append(host_experts(g))
            else:
                hosts.append(hosts[j % args.host_copies])
            for name in ("w13", "s13", "w2", "s2"):  # routed experts now live on the host only
                setattr(g, name, torch.empty(1, dtype=getattr(g, name).dtype, device=dev))
            caches.append(moe.ExpertCache(cfg, args.slots, T))
        layers.append(g)
        if (l + 1) % 10 == 0:
            print(f"stack setup: {l + 1}/{NL} layers", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_setup = time.perf_counter() - t_setup
    n_steps = args.warmup + args.steps
    xs = [torch.from_numpy(synth.hidden_states(sh, T, seed=args.seed, step=s * 64)).to(dev) for s in range(n_steps)]
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=dev)
    y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    wts = [g.weights() for g in layers]

    h = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
    inp = torch.empty_like(h)

    def step(s):
        with torch.cuda.stream(compute):
            h.copy_(xs[s])
            for l in range(NL):
                torch.mul(h, torch.rsqrt(torch.mean(h * h, dim=1, keepdim=True) + 1e-6), out=inp)
                if l >= NL - NSTR:
                    c = caches[l - (NL - NSTR)]
                    c.forward(wts[l], hosts[l - (NL - NSTR)][0], inp, y, ws, compute, copy)
                else:
                    moe.moe_layer_forward(cfg, wts[l], inp, y, ws, stream=compute)
                h.add_(y)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    n_pin = args.slots * 3 // 4 if args.pin is None else args.pin
    if n_pin > 0:  # learning cache: the warm-up steps recorded each layer's usage
        for j, c in enumerate(caches):
            c.pin_hottest(n_pin, hosts[j][0], copy)
    st0 = [c.stats() for c in caches]
    t0 = time.perf_counter()
    for s in range(args.warmup, n_steps):
        step(s)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st1 = [c.stats() for c in caches]
    hits = sum(b["hits"] - a["hits"] for a, b in zip(st0, st1))
    misses = sum(b["misses"] - a["misses"] for a, b in zip(st0, st1))
    h2d = sum(b["bytes_h2d"] - a["bytes_h2d"] for a, b in zip(st0, st1))
    h2d_ms = sum(b["h2d_ms"] - a["h2d_ms"] for a, b in zip(st0, st1))
    # pinned host -> device peak of this machine, one 1 GiB copy
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    peak = (1 << 30) / (e0.elapsed_time(e1) / 1e3) / 1e9
    ms = dt * 1e3 / args.steps
    out = {"metric": "stacked decode tokens/s (GLM-5.2 MoE layers, T=32)", "value": round(T / (ms / 1e3), 2),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
           "higher_is_better": True, "dtype": "i8", "data": "synthetic",
           "config": {"workload": f"glm5.2-moe stack{NL}: {NL - NSTR} resident + {NSTR} streamed layers, "
                                  f"{args.slots} HBM slots per streamed layer, {n_pin} pinned by usage", "tokens": T,
                      "host_copies": min(NSTR, args.host_copies), "pinned_per_layer": n_pin,
                      "learning_steps": args.warmup, "residual": "h += layer(rmsnorm(h)) between layers"},
           "hit_rate": round(hits / max(1, hits + misses), 4), "hits": hits, "misses": misses,
           "h2d_bytes_per_step": round(h2d / args.steps), "h2d_gbs_over_step": round(h2d / dt / 1e9, 2),
           "pinned_h2d_peak_gbs": round(peak, 2),
           # time the copy stream spent moving experts, summed over layers, per step; the rest of the step is
           # compute that did not overlap a copy
           "h2d_busy_ms_per_step": round(h2d_ms / args.steps, 2),
           "h2d_busy_frac": round(h2d_ms / args.steps / ms, 4), "setup_s": round(t_setup, 1)}
    print(json.dumps(out), flush=True)
    for c in caches:
        c.destroy()


def heat_summary(stats):
    """Expert heat of the timed steps: how many routed positions the unique experts get (bucket sizes), the
    hottest experts' counts and the share of positions the hottest 8 experts take."""
    edges = [(1, 1), (2, 2), (3, 4), (5, 8), (9, 16), (17, 32), (33, 64), (65, 128), (129, 1 << 30)]
    hist = {f"{lo}" if lo == hi else (f"{lo}-{hi}" if hi < 1 << 30 else f"{lo}+"): 0.0 for lo, hi in edges}
    hot, share = [], []
    for st in stats:
        c = st["counts"][st["counts"] > 0]
        for (lo, hi), k in zip(edges, hist):
            hist[k] += float(((c >= lo) & (c <= hi)).sum()) / len(stats)
        srt = np.sort(c)[::-1]
        hot.append(srt[:5].astype(np.float64))
        share.append(float(srt[:8].sum()) / max(1.0, float(c.sum())))
    return dict(bucket_sizes={k: round(v, 2) for k, v in hist.items()},
                hottest5_mean=[round(float(v), 1) for v in np.mean(hot, axis=0)],
                top8_share=round(float(np.mean(share)), 4))


def measured_hbm_peak(moe, torch):
    """Best streaming read rate of plain grid-stride read kernels over 4 GiB (GB/s), a few launch shapes."""
    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = 0.0
    for blocks in (2048, 4096, 8192):
        for unroll in (2, 4, 8):
            moe.moe_membench_read(buf, blocks, unroll, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                moe.moe_membench_read(buf, blocks, unroll, sink)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, 3 * n / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del buf
    return round(best, 1)


def measured_compute_peaks(moe, torch):
    """Best rates of plain compute kernels of known operation count: int8 MFMA (TOP/s; 4 chains of
    v_mfma_i32_32x32x32_i8 per wavefront, 65,536 ops each) and fp32 VALU fused multiply-adds (lane-ops/s; 8 chains
    per lane), each over a few launch shapes. The kernels' outputs are checked against their closed forms."""
    best_mfma, best_valu = 0.0, 0.0
    for blocks in (512, 1024, 2048):
        it = 4000
        out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
        moe.moe_peakbench_mfma_i8(blocks, it, 1, out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.moe_peakbench_mfma_i8(blocks, it, 1, out)
        e1.record()
        torch.cuda.synchronize()
        if not bool((out == 2048 * it).all()):
            raise RuntimeError("int8 MFMA rate kernel: wrong result")
        best_mfma = max(best_mfma, blocks * 4 * 4 * it * 65536.0 / (e0.elapsed_time(e1) / 1e3) / 1e12)
        it = 20000
        outf = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        moe.moe_peakbench_valu_fma(blocks, it, 1.0, 0.0, outf)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        moe.moe_peakbench_valu_fma(blocks, it, 1.0, 0.0, outf)
        e1.record()
        torch.cuda.synchronize()
        lane = torch.arange(blocks * 256, device="cuda") % 64
        if not bool((outf == (8 * lane + 28).float()).all()):
            raise RuntimeError("fp32 VALU rate kernel: wrong result")
        best_valu = max(best_valu, blocks * 256 * 8.0 * it / (e0.elapsed_time(e1) / 1e3))
    return round(best_mfma, 1), best_valu


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return dict(cpu_model=model, nproc=os.cpu_count(), nproc_available=avail)


def measure(args, workload, steps, moe, torch, shape, cfg, layers, wts, hbm_measured, peaks=(None, None)):
    """One workload's timed pass and its roofline figures (the JSON fields of a bench line, without the CPU
    baseline)."""
    T = tokens_of(workload)
    dev = torch.device("cuda:0")
    WB, GSZ = args.weight_bits, args.group_size
    n_in = args.warmup + steps
    xs_host = make_inputs(shape, workload, min(n_in, 64), args.seed)
    xs = [torch.from_numpy(x).to(dev) for x in xs_host]
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device=dev)
    y = torch.empty((T, shape.hidden), dtype=torch.float32, device=dev)
    ncopy = len(layers)

    # routing statistics of every timed step (outside the timed region)
    stats = []
    for s in range(steps):
        i = args.warmup + s
        stats.append(routing_stats(moe, cfg, layers[i % ncopy], xs[i % len(xs)], ws, args.gemm_min))

    stream = torch.cuda.current_stream()
    for s in range(args.warmup):
        moe.moe_layer_forward(cfg, wts[s % ncopy], xs[s % len(xs)], y, ws)
    torch.cuda.synchronize()
    # dominant kernel: the gate-up launch of the path that moves most bytes (the path
    # with more experts on average); the timed region records HIP events around it
    # only (on the stream it runs on)
    mfma_major = np.mean([s["mfma_experts"] for s in stats]) > np.mean([s["gemv_experts"] for s in stats])
    kname = "gateup_mfma" if mfma_major else "gateup_gemv"
    # counter summaries are per kernel, workload and weight width
    pmc_workload = workload + ("_int8w" if WB == 8 else "") + (f"_g{GSZ}" if GSZ else "") + \
        (f"_topp{args.topp:g}" if 0 < args.topp < 1 else "")
    kidx = moe.STAGES.index(kname)

    def timed(stages):
        moe.moe_prof_enable(steps, stages)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for s in range(steps):
            i = args.warmup + s
            moe.moe_layer_forward(cfg, wts[i % ncopy], xs[i % len(xs)], y, ws)
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        p = moe.moe_prof_read(steps)
        moe.moe_prof_disable()
        return ms, p

    def clean():
        """The timed value: the same steps with no stage events at all."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for s in range(steps):
            i = args.warmup + s
            moe.moe_layer_forward(cfg, wts[i % ncopy], xs[i % len(xs)], y, ws)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    ms_step = clean()
    # the dominant kernel's launch durations: events around that launch only
    ms_kernel_pass, prof = timed([kname])
    # per-stage breakdown: a third pass over the same steps with every stage's
    # events (their own cost inflates it; not part of the timed value)
    ms_staged, prof_all = timed(None)
    ms_graph = None
    if args.graph:
        # each step captured once as a HIP graph (the library's launches, helper-stream fork and join included),
        # then the same steps replayed back to back
        cap = torch.cuda.Stream()
        with torch.cuda.stream(cap):
            moe.moe_layer_forward(cfg, wts[0], xs[0], y, ws)  # helper stream and events of this stream exist now
        torch.cuda.synchronize()
        graphs = []
        for s in range(steps):
            i = args.warmup + s
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                moe.moe_layer_forward(cfg, wts[i % ncopy], xs[i % len(xs)], y, ws)
            graphs.append(g)
        for g in graphs[:3]:
            g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for g in graphs:
            g.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms_graph = t0.elapsed_time(t1) / steps
        del graphs

    H, I, E = shape.hidden, shape.inter, shape.n_experts
    # gate+up codes + fp32 scales (one per row, or one per group of GSZ along K)
    w13_bytes = 2 * I * H * WB // 8 + (2 * I * (H // GSZ) if GSZ else 2 * I) * 4
    w2_bytes = H * I * WB // 8 + (H * (I // GSZ) if GSZ else H) * 4
    U = np.array([s["U"] for s in stats], np.float64)
    layer_bytes = (E * H * 4 + E * 4) + (U + 1) * (w13_bytes + w2_bytes) + 2 * T * H * 4
    stage_ms = prof_all.mean(0)
    if workload == "prefill":
        # the timed launch is the MFMA gate/up of every bucket from the threshold up, the shared experts' included
        ops = np.array([2.0 * s["mfma_tokens"] * 2 * I * H for s in stats])
        kt = prof[:, kidx] / 1e3
        achieved = float(np.mean(ops / kt) / 1e12)
        # the exact block epilogue: one int->fp32 conversion and one fused multiply-add per (row, token, block)
        valu = np.array([2.0 * s["mfma_tokens"] * 2 * I * (H // 32) for s in stats])
        valu_frac = float(np.mean(valu / kt) / VALU_PEAK_OPS)
        mfma_meas, valu_meas = peaks
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=INT8_PEAK_TOPS, unit="TOP/s",
                    frac=round(achieved / INT8_PEAK_TOPS, 4), traffic=traffic_of("k_" + kname, pmc_workload),
                    kernel="k_" + kname,
                    kernel_ms=round(float(kt.mean() * 1e3), 4),
                    frac_of_measured_peak=round(achieved / mfma_meas, 4) if mfma_meas else None,
                    per_unit="2*2I*H int8 ops per (token, expert) in the MFMA gate/up launch",
                    valu_epilogue=dict(ops_per_launch=float(valu.mean()), peak=VALU_PEAK_OPS, frac=round(valu_frac, 4),
                                       frac_of_measured_peak=round(float(np.mean(valu / kt)) / valu_meas, 4)
                                       if valu_meas else None,
                                       per_unit="2 VALU lane-ops (convert + FMA) per (row, token, 32-block)"))
    else:
        # HBM-bound (decode on the GEMV path, MTP verify on the MFMA path): the path's experts' gate/up weights
        # and scales, Q8_0 activations in and Q8_0 h out per token
        ne, nt = ("mfma_experts", "mfma_tokens") if kname == "gateup_mfma" else ("gemv_experts", "gemv_tokens")
        gb = np.array([s[ne] * w13_bytes + s[nt] * (H + H // 32 * 4 + I + I // 32 * 4) for s in stats], np.float64)
        kt = prof[:, kidx] / 1e3
        achieved = float(np.mean(gb / kt) / 1e9)
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic_of("k_" + kname, pmc_workload),
                    kernel="k_" + kname, algorithmic_bytes=round(float(gb.mean()), 1),
                    kernel_ms=round(float(kt.mean() * 1e3), 4),
                    frac_of_measured_peak=round(achieved / hbm_measured, 4) if hbm_measured else None,
                    per_unit=f"{w13_bytes} B of gate/up weights+scales per {'MFMA' if kname == 'gateup_mfma' else 'GEMV'}"
                             f"-path expert, plus Q8_0 activations in and Q8_0 h out per token")
    layer_gbs = float(np.mean(layer_bytes / (ms_step / 1e3)) / 1e9)
    out = {
        "value": round(T / (ms_step / 1e3), 1),
        "unit": "tokens/s",
        "steps": steps,
        "ms_per_step": round(ms_step, 5),
        "config": {"workload": f"glm5.2-moe-layer {workload}", "tokens": T, "hidden": H, "experts": E,
                   "groups": shape.n_group, "topk_group": shape.topk_group, "top_k": shape.top_k, "inter": I,
                   "shared": shape.n_shared, "rsf": shape.rsf, "gemm_min_tokens": args.gemm_min or DEFAULT_GEMM_MIN,
                   "layer_copies": ncopy, "weight_bits": WB, "group_size": GSZ, "topp": args.topp},
        "layer_hbm_gbs": round(layer_gbs, 1),
        "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
        "layer_hbm_frac_of_measured_peak": round(layer_gbs / hbm_measured, 4) if hbm_measured else None,
        "unique_experts_mean": round(float(U.mean()), 2),
        "routed_slots_mean": round(float(np.mean([st["counts"].sum() for st in stats])), 2),
        "heat": heat_summary(stats),
        "stage_ms": {n: round(float(v), 5) for n, v in zip(moe.STAGES, stage_ms)},
        "ms_per_step_kernel_events": round(ms_kernel_pass, 5),
        "ms_per_step_all_stage_events": round(ms_staged, 5),
        "ms_per_step_graph_replay": round(ms_graph, 5) if ms_graph else None,
        "roofline": roof,
    }
    # layer-level view: every expert's int8 ops (MFMA and v_dot4 paths) against the dense int8 MFMA peak, and the
    # larger of the HBM and MFMA lower bounds against the measured step
    routed = float(np.mean([st["counts"].sum() for st in stats]))  # T*K, or fewer with adaptive top-p
    ops_layer = 2.0 * (routed + shape.n_shared * T) * (2 * I * H + H * I)
    t_mem = layer_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = ops_layer / (INT8_PEAK_TOPS * 1e12)
    out["layer_int8_ops"] = ops_layer
    out["layer_int8_mfma_frac"] = round(ops_layer / (ms_step / 1e3) / (INT8_PEAK_TOPS * 1e12), 4)
    out["combined_roofline_frac"] = round(float(np.mean(np.maximum(t_mem, t_mfma))) / (ms_step / 1e3), 4)
    del ws, xs
    return out, xs_host


def stack_child(args):
    """The 40-layer stack in a child process of its own (its pinned host copies and 120 GB of device memory are
    released with it, and a failure there cannot take the main line down). Returns its JSON or an error."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", "stack40", "--steps", "8", "--warmup", "4",
           "--seed", str(args.seed)]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=420)
    except subprocess.TimeoutExpired:
        return {"error": "stack40 child exceeded 420 s"}
    for line in reversed(r.stdout.strip().splitlines()):
        if line.startswith("{"):
            try:
                return json.loads(line)
            except ValueError:
                break
    return {"error": f"stack40 child exited {r.returncode}: {r.stderr.strip()[-300:]}"}


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate:
        calibrate()
        return
    if args.workload == "stack40":
        if args.weight_bits != 4 or args.group_size or args.topp:
            print("stack40 streams int4 experts with row scales only.", file=sys.stderr)
            sys.exit(2)
        run_stack(args)
        return
    import torch

    import int4_quantized_expert_amd as moe
    from synth import synth
    from tests.harness import GpuLayer, config_of

    shape = synth.GLM
    WB, GSZ = args.weight_bits, args.group_size
    cfg = config_of(shape, args.gemm_min, WB, GSZ, args.topp)
    hbm_measured = measured_hbm_peak(moe, torch)
    peaks = measured_compute_peaks(moe, torch)
    layers = [GpuLayer(shape, seed=args.seed + c, weight_bits=WB, group_size=GSZ) for c in range(args.copies)]
    wts = [l.weights() for l in layers]
    head, xs_host = measure(args, args.workload, args.steps, moe, torch, shape, cfg, layers, wts, hbm_measured, peaks)
    out = {"metric": METRIC, "value": head.pop("value"), "unit": head.pop("unit"), "n_gpus": 1,
           "steps": head.pop("steps"), "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic"}
    out.update(head)
    out["hbm_measured_peak_gbs"] = hbm_measured
    out["hbm_measured_peak_how"] = "best of plain grid-stride read kernels over 4 GiB (2048-8192 workgroups x 256 " \
                                   "lanes, 2-8 16-byte loads in flight per lane)"
    out["mfma_i8_measured_peak_tops"] = peaks[0]
    out["valu_measured_peak_lane_ops"] = peaks[1]
    out["compute_measured_peaks_how"] = "best of plain kernels over 512-2048 workgroups of 4 wavefronts: 4 " \
                                        "independent v_mfma_i32_32x32x32_i8 chains per wavefront; 8 independent " \
                                        "fp32 FMA chains per lane"
    configs = {}
    for w in args.configs:
        if w == "stack40":
            continue
        print(f"bench: measuring {w}", file=sys.stderr, flush=True)
        configs[w], _ = measure(args, w, args.config_steps, moe, torch, shape, cfg, layers, wts, hbm_measured, peaks)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(shape, xs_host[0], args.cpu_baseline_seconds, args.seed, WB, GSZ, args.topp)
        cb.update(host_cpu())
        out["cpu_baseline"] = cb
    if "stack40" in args.configs:
        del wts, layers
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        print("bench: measuring stack40 in a child process", file=sys.stderr, flush=True)
        configs["stack40"] = stack_child(args)
    if configs:
        out["configs"] = configs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
