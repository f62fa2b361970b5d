#!/usr/bin/env python3
"""Benchmark of the selective-scan forward pass on one MI355X.

A step is one call of ``ssm_selective_scan_fwd`` over the Mamba-1.4B-layer workload
(batch 8, d_inner 4096, N 16, L 4096, bf16 I/O, fp32 arithmetic, silu(z) gate, softplus on):
every stage of the scan runs inside it. Inputs are generated once, copied to HBM and stay
resident; the timed region covers exactly ``--steps`` calls between two device
synchronisations, timed with HIP events on the stream the kernels are launched on.

Prints one JSON line: throughput in Gtoken*channel/s, the roofline of the dominant kernel
(algorithmic bytes per launch / average launch time, against the 8 TB/s HBM peak), and the fp64
CPU oracle timed on a bounded sample of the same workload on the host cores.

``--copy-calibration`` runs only a plain device copy of a known size (for scaling the
FETCH_SIZE / WRITE_SIZE counters of a profiler run).
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
WORKLOAD = 2           # Mamba-1.4B layer scan


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_24_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(cfg_key: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the current
    kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{cfg_key}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def device_inputs(cfg, torch):
    import numpy as np
    import ssmgen
    dev = {}
    for name in cfg.shapes():
        arr = ssmgen.make_tensor(cfg, name)
        if arr.dtype == np.uint16:
            t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(arr)
        dev[name] = t.to("cuda")
        del arr
    return dev


def cpu_baseline(cfg, budget_s: float):
    """The fp64 oracle, as it stands, on a sample of whole channels of the workload (batch 0,
    channels 0..S-1, all L steps), S grown until the run takes about ``budget_s`` seconds."""
    import numpy as np
    import oracle
    import ssmgen
    threads = oracle.cpu_threads()
    L = cfg.L

    def run(nch):
        sub = ssmgen.with_shape(cfg, batch=1, dim=nch)
        inputs = {}
        for name in sub.shapes():
            # channels 0..nch-1 of batch 0 are the first rows of every per-channel tensor
            full_shape = sub.shapes()[name]
            d = sub.dist_of(name)
            count = int(np.prod(full_shape))
            inputs[name] = ssmgen.fill(cfg.seed, ssmgen.TENSOR_IDS[name], d.kind, d.p0, d.p1,
                                       count, sub.dtype_of(name)).reshape(full_shape)
        t0 = time.perf_counter()
        oracle.scan_inputs(inputs, sub, nthreads=threads)
        return time.perf_counter() - t0

    nch = max(threads, 16)
    dt = run(nch)
    while dt < budget_s / 4 and nch < cfg.dim:
        nch = min(cfg.dim, nch * 4)
        dt = run(nch)
    if dt < budget_s / 2 and nch < cfg.dim:
        nch = min(cfg.dim, int(nch * budget_s / max(dt, 1e-3)))
        dt = run(nch)
    return {
        "value": round(nch * L / dt / 1e9, 6),
        "unit": "Gtoken\u00b7channel/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{nch} of {cfg.batch * cfg.dim} channels (batch 0, channels 0..{nch - 1}, "
                  f"all {L} steps): {nch * L * cfg.N / 1e9:.3f} G fp64 state updates in "
                  f"{dt:.2f} s",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 skips it)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--check", action="store_true", help="compare sampled channels with the oracle")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / args.steps
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                          "ms": round(ms, 4), "GBs_read_plus_write": round(2 * nbytes / ms / 1e6, 1)}))
        return

    import ssmgen
    import selective_state_space_24_amd as ssm

    cfg = ssmgen.CONFIGS[WORKLOAD]
    dev = device_inputs(cfg, torch)
    y = torch.empty_like(dev["x"])
    stream = torch.cuda.current_stream()
    desc = ssm.describe(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["z"], y)
    ws_bytes = ssm.workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        rc = ssm.fwd_raw(desc, dev["x"].data_ptr(), dev["delta"].data_ptr(), dev["A"].data_ptr(),
                         dev["B"].data_ptr(), dev["C"].data_ptr(), dev["D"].data_ptr(),
                         dev["z"].data_ptr(), dev["delta_bias"].data_ptr(), True, y.data_ptr(),
                         ws.data_ptr() if ws_bytes else None, ws_bytes, stream.cuda_stream)
        if rc != 0:
            raise ssm.ScanError(rc, "ssm_selective_scan_fwd")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    check = None
    if args.check:
        import numpy as np
        import oracle
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from scan_cases import channel_oracle, sample_channels
        worst = 0.0
        for b, d in sample_channels(cfg, 8):
            yg = y[b, d].float().cpu().numpy().astype(np.float64)
            worst = max(worst, oracle.rel_err(yg, channel_oracle(cfg, b, d)))
        check = worst

    tokch = cfg.tokch
    alg_bytes = cfg.algorithmic_bytes()
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    traffic = traffic_from_profile("mamba14b_layer")
    out = {
        "metric": "selective-scan Gtoken\u00b7channel/s and achieved HBM GB/s vs peak, 1 MI355X",
        "value": round(tokch / (ms * 1e-3) / 1e9, 3),
        "unit": "Gtoken\u00b7channel/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Mamba-1.4B layer selective scan (S6 forward)",
            "batch": cfg.batch, "d_inner": cfg.dim, "seq_len": cfg.L, "d_state": cfg.N,
            "io_dtype": cfg.io, "gate": "silu(z)", "delta_softplus": cfg.softplus,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "algorithmic_bytes_per_step": alg_bytes,
        "kernel_source": kernel_source_hash(),
    }
    if check is not None:
        out["sampled_max_rel_err"] = check
    if args.cpu_budget > 0:
        del dev, y
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
