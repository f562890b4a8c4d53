#!/usr/bin/env python3
"""Benchmark of the StreamBP hot path on one MI355X.

Default workload: the weighted-token chunked LM head + cross-entropy
forward/backward, the largest single-GPU configuration: T=131072 tokens
packed as 8 sequences of 16384, d=3584, V=152064, D=32 in bf16 (fp32
accumulation); synthetic N(0,1) hidden states, N(0, 0.02^2) weights and
uniform targets, the first 25% of every sequence loss-masked, one N(0,1)
weight per sequence, loss normalised by the unmasked count.  A "step" is
one full call of the path on that batch (logits GEMM, softmax-CE row
kernels, dH and dW GEMMs for every chunk that holds a target, loss
reduction), inputs resident in HBM.

Prints ONE JSON line: tokens/s, ms per step, peak HBM bytes of the call,
the fraction of bf16 MFMA peak over the whole step, the roofline of the
dominant kernel (timed live with hipEvents on the launch stream through the
library's kernel timer), and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload I] [--no-cpu-baseline]

Workloads (--workload): 0..4 the LM-head, attention and layer configurations
(4 is the default; 1 the unweighted LM head at T=32768, d=4096, V=128256,
D=16), 5 the forward-only per-token log-probability on the
weighted LM-head shapes, 6 and 7 the attention and layer workloads over 8
packed sequences of random lengths, 8 the whole-model backward (4 layers
with rotary embedding under the LM head; the layer inputs come from an
untimed chunked forward).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "backward tokens/sec + peak HBM bytes vs seq len T; % of bf16 MFMA peak"
METRIC_LOGPROB = "forward per-token log-prob tokens/sec; % of bf16 MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter record of
    this workload (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated), or
    None when there is no record or the kernel sources changed since."""
    import glob
    import hashlib
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")):
        with open(path) as f:
            rec = json.load(f)
        if rec.get("workload") != workload or kernel not in rec.get("kernels", {}):
            continue
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest()[:16] != rec["source_sha"]:
            return None
        k = rec["kernels"][kernel]
        return int(k["read_bytes"] + k["write_bytes"])
    return None


# rocprofv3 kernel symbol of each library timer name (traffic records)
KERNEL_SYMBOLS = {
    "gemm_logits": "gemm_nt_bf16_ring_kernel<5, false, false>",
    "gemm_dH": "gemm_nt_bf16_ring_kernel<4, false, false>",
    "gemm_dW": "gemm_nt_bf16_ring_kernel<1, true, true>",
    "gemm_layer_dW": "gemm_nt_bf16_ring_kernel<1, true, true>",
    "gemm_logits_lp": "gemm_nt_bf16_ring_kernel<6, false, false>",
    "ce_grad": "ce_grad_kernel<unsigned short, false, true>",
    "attn_dkdv": "attn_dkdv_kernel<128>",
    "attn_dq": "attn_dq_kernel<128>",
    "attn_fwd": "attn_fwd_kernel<128>",
}
# sources whose kernels a record covers (their hash invalidates it)
TRAFFIC_SOURCES = {
    "gemm": ["memory_efficient_exact_amd/csrc/gemm.hip", "memory_efficient_exact_amd/csrc/ce.hip",
             "memory_efficient_exact_amd/csrc/common.h", "memory_efficient_exact_amd/csrc/kernels.h"],
    "attn": ["memory_efficient_exact_amd/csrc/attn.hip", "memory_efficient_exact_amd/csrc/attn.h",
             "memory_efficient_exact_amd/csrc/common.h"],
}


def _pmc_per_dispatch(csv_path, counter):
    """Mean of `counter` per dispatch, by kernel symbol, from a rocprofv3
    --pmc counter_collection CSV (the counter summed over its instances)."""
    import csv
    per = {}
    with open(csv_path) as f:
        rows = list(csv.DictReader(f))
    key = {k.lower(): k for k in rows[0]} if rows else {}
    kn, cn, cv = key.get("kernel_name"), key.get("counter_name"), key.get("counter_value")
    did = key.get("dispatch_id") or key.get("correlation_id")
    tot = {}
    for r in rows:
        if r[cn] != counter:
            continue
        name = r[kn].replace("void ", "").replace("sbp::", "").split("(")[0].strip()
        d = tot.setdefault(name, {})
        d[r[did]] = d.get(r[did], 0.0) + float(r[cv])
    for name, d in tot.items():
        per[name] = (sum(d.values()) / len(d), len(d))
    return per


def traffic_record(args):
    """Write profiles/<workload>_traffic.json from four rocprofv3 --pmc runs
    (FETCH_SIZE and WRITE_SIZE of the workload and of the 1 GiB copy)."""
    import hashlib
    import synthetic
    fetch = _pmc_per_dispatch(args.fetch_csv, "FETCH_SIZE")
    write = _pmc_per_dispatch(args.write_csv, "WRITE_SIZE")
    cfetch = _pmc_per_dispatch(args.copy_fetch_csv, "FETCH_SIZE")
    cwrite = _pmc_per_dispatch(args.copy_write_csv, "WRITE_SIZE")
    copy = [k for k in cfetch if "copyBuffer" in k][0]
    gib_kib = float(1 << 20)
    fscale = gib_kib / cfetch[copy][0]
    wscale = gib_kib / cwrite[copy][0]
    cfg = synthetic.WORKLOADS[args.workload]
    srcs = TRAFFIC_SOURCES[args.traffic_sources]
    h = hashlib.sha256()
    for src in srcs:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    kernels = {}
    for lib_name in args.traffic_kernels.split(","):
        sym = KERNEL_SYMBOLS[lib_name]
        if sym in fetch and sym in write:
            kernels[lib_name] = {"read_bytes": fetch[sym][0] * 1024 * fscale,
                                 "write_bytes": write[sym][0] * 1024 * wscale}
    rec = {"workload": cfg["name"], "source_sha": h.hexdigest()[:16], "sources": srcs,
           "fetch_scale": fscale, "write_scale": wscale, "kernels": kernels}
    out = os.path.join(ROOT, "profiles", f"{cfg['name']}_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"wrote {out}")
    print(f"copy: FETCH_SIZE {cfetch[copy][0]:.0f} KiB, WRITE_SIZE {cwrite[copy][0]:.0f} KiB per 1 GiB copy")
    print("| kernel | dispatches | FETCH_SIZE KiB/disp | WRITE_SIZE KiB/disp | scaled read GiB | scaled write GiB |")
    print("|---|---|---|---|---|---|")
    for name in fetch:
        if name not in write:
            continue
        fk, n = fetch[name]
        wk, _ = write[name]
        print(f"| `{name}` | {n} | {fk:.0f} | {wk:.0f} | {fk * fscale / gib_kib:.3f} | {wk * wscale / gib_kib:.3f} |")


def peak_bytes(idx, T, D, D_lm=None, dw_group=None):
    """Peak device bytes of one call of workload `idx` at sequence length T
    and chunk count D: its inputs, outputs, weights, gradients and the
    workspace the library asks for (the library allocates nothing else).
    LM head: weight-gradient groups of `dw_group` chunks (None: the largest
    the call uses, about 4096 tokens)."""
    import torch
    import synthetic
    import memory_efficient_exact_amd as sbp
    c = synthetic.WORKLOADS[idx]
    bf = torch.bfloat16
    if c["kind"] == "lmhead":
        d, V = c["d"], c["V"]
        g = sbp.lmhead_ce_max_group(T, D) if dw_group is None else dw_group
        ws = sbp.lmhead_ce_workspace_size(T, d, V, D, bf, g)
        return 2 * (2 * T * d) + 2 * V * d + 4 * V * d + 4 * T + ws + (4 * T if c.get("weighted") else 0)
    if c["kind"] == "layer":
        d, F, kd, qd = c["d"], c["F"], c["Hkv"] * c["dh"], c["Hq"] * c["dh"]
        P = qd * d + 2 * kd * d + d * qd + 3 * F * d
        ws = sbp.layer_bwd_workspace_size(T, d, c["Hq"], c["Hkv"], c["dh"], F, D, bf)
        return 3 * (2 * T * d) + 2 * P + 4 * P + 2 * 4 * d + 2 * 2 * d + ws
    if c["kind"] == "model":
        d, F, V, L = c["d"], c["F"], c["V"], c["n_layers"]
        kd, qd = c["Hkv"] * c["dh"], c["Hq"] * c["dh"]
        P = qd * d + 2 * kd * d + d * qd + 3 * F * d + 2 * d
        ws = sbp.model_bwd_workspace_size(T, d, c["Hq"], c["Hkv"], c["dh"], F, L, V, D_lm or D, D,
                                          False, bf, 1e-6, c["rope_theta"])
        return (L + 2) * (2 * T * d) + L * 6 * P + 6 * V * d + 6 * d + 4 * T + ws
    raise ValueError(c["kind"])


def max_t_report(budget=288e9, margin=2e9):
    """Largest T whose call fits `budget` bytes of HBM (less a margin for the
    runtime), chunked at the workload's chunk length and unchunked (D = 1)."""
    import synthetic
    out = []
    for idx, tc in ((1, 2048), (3, 4096), (8, 4096)):
        c = synthetic.WORKLOADS[idx]
        tc_lm = 2048

        def fits(T, chunked):
            if chunked:
                D = max(1, T // tc)
                Dl = max(1, T // tc_lm) if c["kind"] == "model" else None
            else:
                D, Dl = 1, (1 if c["kind"] == "model" else None)
            return peak_bytes(idx, T, D, Dl) <= budget - margin

        row = {"workload": c["name"]}
        for chunked in (True, False):
            lo, hi = tc, tc
            while fits(hi * 2, chunked):
                hi *= 2
            hi *= 2
            while hi - lo > tc:  # bisection on multiples of the chunk length
                mid = (lo + hi) // 2 // tc * tc
                if mid <= lo:
                    break
                lo, hi = (mid, hi) if fits(mid, chunked) else (lo, mid)
            row["max_T_chunked" if chunked else "max_T_D1"] = lo
        row["ratio"] = round(row["max_T_chunked"] / row["max_T_D1"], 2)
        out.append(row)
    print(json.dumps({"budget_bytes": budget, "margin_bytes": margin, "rows": out}), flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", type=int, default=4)
    p.add_argument("--D", type=int, default=None, help="override the chunk count")
    p.add_argument("--D-lm", type=int, default=None,
                   help="override the LM head's chunk count (whole-model workload)")
    p.add_argument("--T", type=int, default=None, help="override the sequence length")
    p.add_argument("--dw-group", type=int, default=None,
                   help="LM head: chunks per weight-gradient GEMM (default: about 4096 tokens)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=None)
    p.add_argument("--copy-calibration", action="store_true",
                   help="run a plain 1 GiB device copy (reference for HBM byte counters)")
    p.add_argument("--library-gemm", action="store_true",
                   help="time torch's library bf16 GEMMs on the LM head's three products")
    p.add_argument("--max-t", action="store_true",
                   help="(no GPU) largest T whose call fits 288 GB, chunked and unchunked")
    p.add_argument("--traffic-record", action="store_true",
                   help="(no GPU) write the workload's HBM traffic record from four --pmc CSVs")
    p.add_argument("--fetch-csv")
    p.add_argument("--write-csv")
    p.add_argument("--copy-fetch-csv")
    p.add_argument("--copy-write-csv")
    p.add_argument("--traffic-kernels", default="gemm_logits,ce_grad,gemm_dH,gemm_dW")
    p.add_argument("--traffic-sources", default="gemm")
    p.add_argument("--sweep-D", default=None,
                   help="LM-head workloads: comma-separated chunk counts; one JSON line per "
                        "(D, weight-gradient group) with tokens/s and peak HBM bytes")
    return p.parse_args()


def sweep_d(args, dev):
    """Peak HBM bytes and tokens/s of an LM-head workload over D, for the
    smallest workspace (one chunk per weight-gradient GEMM) and the largest
    group the call uses (about 4096 tokens); inputs drawn once."""
    import torch
    import synthetic
    import memory_efficient_exact_amd as sbp
    cfg = dict(synthetic.WORKLOADS[args.workload])
    if cfg["kind"] != "lmhead":
        raise SystemExit("--sweep-D is for the LM-head workloads")
    T = args.T or cfg["T"]
    d, V = cfg["d"], cfg["V"]
    inp = synthetic.workload_inputs(args.workload, T=T)
    H, W, tg = inp.H.to(dev), inp.W.to(dev), inp.targets.to(dev)
    w = None if inp.weights is None else inp.weights.to(dev)
    dW = torch.empty(V, d, dtype=torch.float32, device=dev)
    y = inp.targets
    for D in [int(x) for x in args.sweep_D.split(",")]:
        rows = sum(e - s for s, e in sbp.chunk_table(T, D) if (y[s:e] >= 0).any())
        for G in sorted({1, sbp.lmhead_ce_max_group(T, D)}):
            ws = torch.empty(sbp.lmhead_ce_workspace_size(T, d, V, D, H.dtype, G),
                             dtype=torch.uint8, device=dev)

            def step():
                return sbp.lmhead_ce(H, W, tg, w, D=D, dW=dW, workspace=ws)

            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats(dev)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                step()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            print(json.dumps({"workload": cfg["name"], "T": T, "D": D, "T_c": T // D,
                              "dw_group": G, "workspace_bytes": ws.numel(),
                              "peak_hbm_bytes": torch.cuda.max_memory_allocated(dev),
                              "ms_per_step": round(ms, 3), "tokens_per_s": round(T / (ms / 1e3), 1),
                              "mfma_frac_step": round(6.0 * rows * V * d / (ms / 1e3) / 1e12 / 2500.0, 4)}),
                  flush=True)
            del ws


def copy_calibration(dev):
    """A plain device-to-device copy of known size: 1 GiB read + 1 GiB
    written per launch, the reference the FETCH_SIZE / WRITE_SIZE counters of
    the path's kernels are scaled by."""
    import torch
    n = 1 << 28  # fp32 elements = 1 GiB
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                      "launches": 3}), flush=True)


def library_gemm(dev, reps=10):
    """torch's library bf16 GEMMs (hipBLASLt on ROCm) on the LM head's three
    products at T_c = 2048, a weight-gradient group of K = 4096 tokens, d =
    4096, V = 128256, timed with events on torch's stream: a same-box context
    for the path's own GEMM kernels, not part of the path.  Operands are
    contiguous; the fp32 weight-gradient case reads the fp32 C and writes a
    fresh fp32 result (the same HBM traffic as the path's read-modify-write)."""
    import torch
    Tc, Kg, d, V = 2048, 4096, 4096, 128256
    g = torch.Generator(device=dev).manual_seed(0)
    bf = torch.bfloat16

    def rnd(*shape):
        return (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * 0.1).to(bf)

    H = rnd(Tc, d)
    Wt = rnd(d, V)
    W = rnd(V, d)
    dZ = rnd(Tc, V)
    dZt = rnd(V, Kg)
    Hg = rnd(Kg, d)
    dW = torch.zeros(V, d, dtype=torch.float32, device=dev)
    cases = [
        ("logits Z = H W^T, bf16 out", lambda: torch.mm(H, Wt), 2.0 * Tc * V * d),
        ("input grad dH = dZ W, bf16 out", lambda: torch.mm(dZ, W), 2.0 * Tc * V * d),
        ("input grad dH = dZ W, fp32 out", lambda: torch.mm(dZ, W, out_dtype=torch.float32),
         2.0 * Tc * V * d),
        ("weight grad dW += dZ^T H, fp32 accumulate",
         lambda: torch.addmm(dW, dZt, Hg, out_dtype=torch.float32),
         2.0 * V * d * Kg),
        ("weight grad dZ^T H, bf16 out", lambda: torch.mm(dZt, Hg), 2.0 * V * d * Kg),
    ]
    rows = []
    for name, fn, flops in cases:
        try:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            rows.append({"product": name, "ms": round(ms, 4),
                         "tflops": round(flops / ms / 1e9, 1)})
        except RuntimeError as e:
            rows.append({"product": name, "error": str(e).splitlines()[0][:200]})
        print(json.dumps(rows[-1]), flush=True)
    print(json.dumps({"library_gemm": rows, "T_c": Tc, "K_g": Kg, "d": d, "V": V,
                      "torch": torch.__version__}), flush=True)


def lmhead_setup(cfg, dev):
    import torch
    import synthetic
    import memory_efficient_exact_amd as sbp
    inp = synthetic.workload_inputs(cfg["index"], T=cfg["T"])
    H, W, tg = inp.H.to(dev), inp.W.to(dev), inp.targets.to(dev)
    w = None if inp.weights is None else inp.weights.to(dev)
    T, d, V, D = cfg["T"], cfg["d"], cfg["V"], cfg["D"]
    dW = torch.empty(V, d, dtype=torch.float32, device=dev)
    # weight-gradient group: the largest the call uses (about 4096 tokens)
    # unless --dw-group asks for another
    G = sbp.lmhead_ce_max_group(T, D) if cfg.get("dw_group") is None else cfg["dw_group"]
    cfg["dw_group"] = G
    ws = torch.empty(sbp.lmhead_ce_workspace_size(T, d, V, D, H.dtype, G), dtype=torch.uint8,
                     device=dev)
    red = "mean_valid"

    def step():
        return sbp.lmhead_ce(H, W, tg, w, D=D, reduction=red, dW=dW, workspace=ws)

    y = inp.targets
    n_valid = int((y >= 0).sum())
    # algorithmic flops: 3 GEMMs of 2*N*V*d over the rows of chunks that hold a
    # valid token (fully masked chunks are skipped)
    rows = 0
    for s, e in sbp.chunk_table(T, D):
        if (y[s:e] >= 0).any():
            rows += e - s
    flops = 6.0 * rows * V * d
    return step, flops, inp, n_valid


def logprob_setup(cfg, dev):
    import torch
    import synthetic
    import memory_efficient_exact_amd as sbp
    inp = synthetic.workload_inputs(cfg["index"], T=cfg["T"])
    H, W, tg = inp.H.to(dev), inp.W.to(dev), inp.targets.to(dev)
    T, d, V, D = cfg["T"], cfg["d"], cfg["V"], cfg["D"]
    ws = torch.empty(sbp.lmhead_logprob_workspace_size(T, d, V, D, H.dtype), dtype=torch.uint8,
                     device=dev)

    def step():
        return sbp.lmhead_logprob(H, W, tg, D=D, lse=True, workspace=ws)

    y = inp.targets
    n_valid = int((y >= 0).sum())
    # algorithmic flops: the logits GEMM, 2 N V d over the rows of chunks that
    # hold a valid token (fully masked chunks are skipped)
    rows = sum(e - s for s, e in sbp.chunk_table(T, D) if (y[s:e] >= 0).any())
    return step, 2.0 * rows * V * d, inp, n_valid


def attn_setup(cfg, dev):
    import torch
    import synthetic
    import memory_efficient_exact_amd as sbp
    inp = synthetic.workload_inputs(cfg["index"], T=cfg["T"])
    Q, K, V, dO = (x.to(dev) for x in (inp.Q, inp.K, inp.V, inp.dO))
    B, T, Hq, Hkv, dh, D = cfg["B"], cfg["T"], cfg["Hq"], cfg["Hkv"], cfg["dh"], cfg["D"]
    dK = torch.empty(B, T, Hkv, dh, dtype=torch.float32, device=dev)
    dV = torch.empty_like(dK)
    cu = synthetic.workload_cu(cfg["index"], T)
    if cu is None:
        nb = sbp.attn_bwd_workspace_size(B, T, Hq, Hkv, dh, D, Q.dtype)
        cut = None
    else:
        nb = sbp.attn_bwd_packed_workspace_size(T, Hq, Hkv, dh, D, Q.dtype)
        cut = torch.tensor(cu, dtype=torch.int32, device=dev)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def step():
        return sbp.attn_bwd(Q, K, V, dO, D=D, dK=dK, dV=dV, workspace=ws, cu_seqlens=cut)

    # algorithmic work: 7 causal units of 2*Hq*dh*T(T+1)/2*B (forward
    # recompute 2, backward 5); packed: the pairs of each sequence only
    return step, 7.0 * attn_unit(Hq, dh, T, B, cu), inp


def attn_unit(Hq, dh, T, B=1, cu=None):
    """One attention unit: 2 Hq dh flops per visible (query, key) pair."""
    if cu is None:
        return 2.0 * Hq * dh * T * (T + 1) / 2 * B
    return sum(2.0 * Hq * dh * (b - a) * (b - a + 1) / 2 for a, b in zip(cu, cu[1:]))


def layer_setup(cfg, dev):
    import torch
    import synthetic
    import memory_efficient_exact_amd as sbp
    L = synthetic.workload_inputs(cfg["index"], T=cfg["T"])
    x, dy = L.x.to(dev), L.dy.to(dev)
    w = {k: v.to(dev) for k, v in L.w.items()}
    T, d, Hq, Hkv, dh, F, D = (cfg[k] for k in ("T", "d", "Hq", "Hkv", "dh", "F", "D"))
    grads = {k: torch.empty(v.shape, dtype=torch.float32, device=dev) for k, v in w.items()}
    cu = synthetic.workload_cu(cfg["index"], T)
    if cu is None:
        nb = sbp.layer_bwd_workspace_size(T, d, Hq, Hkv, dh, F, D, x.dtype, L.eps)
        cut = None
    else:
        nb = sbp.layer_bwd_packed_workspace_size(T, d, Hq, Hkv, dh, F, D, x.dtype, L.eps)
        cut = torch.tensor(cu, dtype=torch.int32, device=dev)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def step():
        return sbp.layer_bwd(x, dy, w, Hq, Hkv, dh, L.eps, D=D, grads=grads, workspace=ws,
                             cu_seqlens=cut)

    # algorithmic work: 6 P T for the linear maps (forward recompute 2, backward
    # 4; P = number of projection weights) plus 7 attention units
    P = (Hq * dh) * d + 2 * (Hkv * dh) * d + d * (Hq * dh) + 3 * F * d
    return step, 6.0 * P * T + 7.0 * attn_unit(Hq, dh, T, 1, cu), L


def model_setup(cfg, dev):
    """Whole-model backward: the layer inputs come from the chunked forward
    (untimed); the step is one sbp_model_bwd call."""
    import torch
    import synthetic
    import memory_efficient_exact_amd as sbp
    M = synthetic.workload_inputs(cfg["index"], T=cfg["T"])
    T, d, Hq, Hkv, dh, F, V = (cfg[k] for k in ("T", "d", "Hq", "Hkv", "dh", "F", "V"))
    layers = [{k: v.to(dev) for k, v in w.items()} for w in M.layers]
    xs = sbp.model_fwd(M.x0.to(dev), layers, Hq, Hkv, dh, M.eps, cfg["D"], None, M.rope_theta)
    g_f, W, y = M.g_final.to(dev), M.W.to(dev), M.targets.to(dev)
    grads = [{k: torch.empty(v.shape, dtype=torch.float32, device=dev) for k, v in w.items()}
             for w in layers]
    dg_f = torch.empty(d, dtype=torch.float32, device=dev)
    dW = torch.empty(V, d, dtype=torch.float32, device=dev)
    nb = sbp.model_bwd_workspace_size(T, d, Hq, Hkv, dh, F, len(layers), V, cfg["D_lm"], cfg["D"],
                                      False, xs[0].dtype, M.eps, M.rope_theta)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def step():
        return sbp.model_bwd(xs, layers, g_f, W, y, None, Hq=Hq, Hkv=Hkv, dh=dh, eps=M.eps,
                             D_lm=cfg["D_lm"], D_layer=cfg["D"], rope_theta=M.rope_theta,
                             grads=grads, dg_final=dg_f, dW_lm=dW, workspace=ws)

    # algorithmic work: the LM head's 6 T V d plus, per layer, 6 P T for the
    # linear maps and 7 attention units
    P = (Hq * dh) * d + 2 * (Hkv * dh) * d + d * (Hq * dh) + 3 * F * d
    flops = 6.0 * T * V * d + len(layers) * (6.0 * P * T + 7.0 * attn_unit(Hq, dh, T))
    return step, flops, M


def cpu_baseline_model(M, cfg, sample):
    """The oracle, untouched, on the first `sample` tokens of the same input."""
    import oracle
    import synthetic
    f = synthetic.to_f64
    layers = [{k: f(v) for k, v in w.items()} for w in M.layers]
    x0, g_f, W = f(M.x0[:sample]), f(M.g_final), f(M.W)
    y = M.targets[:sample].numpy()
    t0 = time.perf_counter()
    oracle.model_bwd(x0, layers, g_f, W, y, Hq=M.Hq, Hkv=M.Hkv, dh=M.dh, eps=M.eps,
                     rope_theta=M.rope_theta)
    dt = time.perf_counter() - t0
    return {"value": sample / dt, "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"first {sample} of {cfg['T']} tokens through all {len(layers)} layers and "
                      f"the full LM head (fp64 NumPy, unchunked, forward included); {dt:.1f} s"}


def cpu_baseline_layer(L, cfg, sample):
    """The oracle, untouched, on the first `sample` tokens of the same input."""
    import oracle
    import synthetic
    w = {k: synthetic.to_f64(v) for k, v in L.w.items()}
    x = synthetic.to_f64(L.x[:sample])
    dy = synthetic.to_f64(L.dy[:sample])
    cu = synthetic.workload_cu(cfg["index"], cfg["T"])
    if cu is not None:  # the sequences that fall inside the sample
        cu = [c for c in cu if c < sample] + [sample]
    t0 = time.perf_counter()
    oracle.layer_bwd(x, dy, w, L.Hq, L.Hkv, L.dh, L.eps, cu_seqlens=cu)
    dt = time.perf_counter() - t0
    return {"value": sample / dt, "unit": "tokens/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"first {sample} of {cfg['T']} tokens with the full weights (fp64 NumPy, "
                      f"unchunked); {dt:.1f} s; attention cost per token grows with T, so this "
                      f"overstates the oracle's rate at full T"}


def cpu_baseline_attn(inp, cfg, sample_heads=1):
    """The oracle, untouched, on one q head's share of the same input."""
    import math
    import oracle
    import synthetic
    G = cfg["Hq"] // cfg["Hkv"]
    Q = synthetic.to_f64(inp.Q[:, :, :sample_heads])
    K = synthetic.to_f64(inp.K[:, :, :1])
    V = synthetic.to_f64(inp.V[:, :, :1])
    dO = synthetic.to_f64(inp.dO[:, :, :sample_heads])
    cu = synthetic.workload_cu(cfg["index"], cfg["T"])
    t0 = time.perf_counter()
    if cu is None:
        oracle.attn_bwd(Q, K, V, dO, 1.0 / math.sqrt(cfg["dh"]))
    else:
        oracle.attn_bwd_packed(Q, K, V, dO, 1.0 / math.sqrt(cfg["dh"]), cu)
    dt = time.perf_counter() - t0
    scale = cfg["Hq"] / sample_heads
    tokens = cfg["B"] * cfg["T"]
    return {"value": tokens / (dt * scale), "unit": "tokens/s", "cores": _blas_threads(),
            "kind": "oracle",
            "sample": f"{sample_heads} of {cfg['Hq']} q heads (1 kv head), full T={cfg['T']}; "
                      f"{dt:.1f} s, scaled by {scale:g} to all heads"}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count()


def cpu_baseline_lmhead(inp, cfg, sample):
    """The oracle, untouched, on `sample` tokens of the same input: the
    first ones that hold a target (masked prompt tokens cost the oracle
    nothing, so they would overstate its rate)."""
    import numpy as np
    import torch
    import oracle
    import synthetic
    threads = _blas_threads()
    y_all = inp.targets.numpy()
    rows = np.nonzero(y_all >= 0)[0][:sample]
    idx = torch.from_numpy(rows)
    H = synthetic.to_f64(inp.H[idx])
    W = synthetic.to_f64(inp.W)
    y = y_all[rows]
    wts = None if inp.weights is None else synthetic.to_f64(inp.weights[idx])
    t0 = time.perf_counter()
    oracle.lmhead_ce(H, W, y, wts)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {len(rows)} tokens with a target, of {cfg['T']}; full V={cfg['V']} "
                      f"and d={cfg['d']} (fp64 NumPy, unchunked); {dt:.1f} s"}


def cpu_baseline_logprob(inp, cfg, sample):
    """The log-prob oracle, untouched, on `sample` tokens of the same input,
    taken from the sequences' unmasked parts (the device skips only chunks
    with no valid token)."""
    import numpy as np
    import torch
    import oracle
    import synthetic
    threads = _blas_threads()
    y = inp.targets.numpy()
    rows = np.nonzero(y >= 0)[0][:sample]
    H = synthetic.to_f64(inp.H[torch.from_numpy(rows)])
    W = synthetic.to_f64(inp.W)
    t0 = time.perf_counter()
    oracle.lmhead_logprob(H, W, y[rows], row_block=1024)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {len(rows)} valid of {cfg['T']} tokens, full V={cfg['V']} and "
                      f"d={cfg['d']} (fp64 NumPy, unchunked); {dt:.1f} s"}


def main():
    args = parse()
    if args.traffic_record:
        traffic_record(args)
        return
    if args.max_t:
        max_t_report()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; multi-GPU data parallelism is not built)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synthetic
    import memory_efficient_exact_amd as sbp
    sbp.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return
    if args.library_gemm:
        library_gemm(dev)
        return
    if args.sweep_D:
        sweep_d(args, dev)
        return

    idx = args.workload
    cfg = dict(synthetic.WORKLOADS[idx])
    cfg["index"] = idx
    if args.D:
        cfg["D"] = args.D
    if args.D_lm:
        cfg["D_lm"] = args.D_lm
    if args.T:
        cfg["T"] = args.T
    if args.dw_group:
        cfg["dw_group"] = args.dw_group
    # a counter record describes the workload's own shapes only
    own_shapes = not (args.D or args.D_lm or args.T or args.dw_group)
    n_valid = None
    if cfg["kind"] == "lmhead":
        step, flops, inp, n_valid = lmhead_setup(cfg, dev)
    elif cfg["kind"] == "logprob":
        step, flops, inp, n_valid = logprob_setup(cfg, dev)
    elif cfg["kind"] == "attn":
        step, flops, inp = attn_setup(cfg, dev)
    elif cfg["kind"] == "model":
        step, flops, inp = model_setup(cfg, dev)
    else:
        step, flops, inp = layer_setup(cfg, dev)
    dtype = cfg["dtype"]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base_mem = torch.cuda.memory_allocated(dev)

    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with sbp.profile() as prof:
        e0.record(stream)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_gpu = e0.elapsed_time(e1) / args.steps
    ms_wall = (t1 - t0) * 1e3 / args.steps
    ms = max(ms_gpu, ms_wall)
    peak = torch.cuda.max_memory_allocated(dev)
    T = cfg["T"]
    tokens = T * cfg.get("B", 1)
    value = tokens / (ms / 1e3)

    # The library's timer counts each launch's flops as issued; the LM head's
    # GEMMs of fully masked chunks (groups) are launched but return at once,
    # so there each GEMM kind is credited a third of the step's algorithmic
    # flops (the three chunk GEMMs have the same 2 N V d each).
    if cfg["kind"] == "lmhead":
        for kname in ("gemm_logits", "gemm_dH", "gemm_dW"):
            if kname in prof:
                prof[kname] = dict(prof[kname], flops=flops * args.steps / 3.0)
    elif cfg["kind"] == "logprob" and "gemm_logits_lp" in prof:
        prof["gemm_logits_lp"] = dict(prof["gemm_logits_lp"], flops=flops * args.steps)
    # The attention kernels count the pairs of one causal row of T tokens; over
    # a whole step (every chunk) that is T(T+1)/2 pairs, against the sum over
    # packed sequences of L(L+1)/2 that is really visible.
    cu_step = synthetic.workload_cu(idx, T)
    if cu_step is not None and cfg["kind"] in ("attn", "layer"):
        ratio = attn_unit(cfg["Hq"], cfg["dh"], T, 1, cu_step) / attn_unit(cfg["Hq"], cfg["dh"], T)
        for kname in ("attn_fwd", "attn_dkdv", "attn_dq"):
            if kname in prof:
                prof[kname] = dict(prof[kname], flops=prof[kname]["flops"] * ratio)
    # dominant kernel and its roofline (live hipEvent timing inside the call)
    dom = max(prof.items(), key=lambda kv: kv[1]["ms"])
    name, k = dom
    if k["flops"] > 0:
        ach = k["flops"] / (k["ms"] / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_TFLOPS[dtype],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS[dtype], 4),
                "traffic": measured_traffic(cfg["name"], name) if own_shapes else None,
                "kernel": name, "avg_launch_ms": round(k["ms"] / k["launches"], 4),
                "flops_per_launch": k["flops"] / k["launches"]}
    else:
        ach = k["bytes"] / (k["ms"] / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(cfg["name"], name) if own_shapes else None,
                "kernel": name,
                "avg_launch_ms": round(k["ms"] / k["launches"], 4),
                "bytes_per_launch": k["bytes"] / k["launches"]}
    kernels = {n: {"launches": v["launches"] // args.steps,
                   "ms_per_step": round(v["ms"] / args.steps, 3),
                   "tflops": round(v["flops"] / (v["ms"] / 1e3) / 1e12, 1) if v["flops"] else None,
                   "gbs": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1) if v["bytes"] and not v["flops"] else None}
               for n, v in sorted(prof.items(), key=lambda kv: -kv[1]["ms"])}

    out = {
        "metric": METRIC if cfg["kind"] != "logprob" else METRIC_LOGPROB,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {k: v for k, v in cfg.items() if k not in ("kind", "name", "index", "dtype")}
                  | {"workload": cfg["name"]} | ({"valid_tokens": n_valid} if n_valid else {})
                  | ({"cu_seqlens": cu} if (cu := synthetic.workload_cu(idx, T)) else {}),
        "peak_hbm_bytes": int(peak),
        "peak_hbm_bytes_call": int(peak - base_mem),
        "mfma_frac_step": round(flops / (ms / 1e3) / 1e12 / PEAK_TFLOPS[dtype], 4),
        "roofline": roof,
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        if cfg["kind"] == "logprob":
            out["cpu_baseline"] = cpu_baseline_logprob(inp, cfg, args.cpu_sample or 12288)
        elif cfg["kind"] == "lmhead":
            sample = args.cpu_sample or (4096 if cfg["V"] * cfg["d"] > 1e8 else min(T, 4096))
            out["cpu_baseline"] = cpu_baseline_lmhead(inp, cfg, sample)
        elif cfg["kind"] == "attn":
            out["cpu_baseline"] = cpu_baseline_attn(inp, cfg)
        elif cfg["kind"] == "model":
            out["cpu_baseline"] = cpu_baseline_model(inp, cfg, args.cpu_sample or 1024)
        else:
            out["cpu_baseline"] = cpu_baseline_layer(inp, cfg, args.cpu_sample or 1024)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
