#!/usr/bin/env python3
"""Benchmark of the selective-scan forward pass on one MI355X.

A step is one call of ``ssm_selective_scan_fwd`` over the Mamba-1.4B-layer workload
(batch 8, d_inner 4096, N 16, L 4096, bf16 I/O, fp32 arithmetic, silu(z) gate, softplus on):
every stage of the scan runs inside it. Inputs are generated once, copied to HBM and stay
resident; the timed region covers exactly ``--steps`` calls between two device
synchronisations, timed with HIP events on the stream the kernels are launched on.

Prints one JSON line: throughput in Gtoken*channel/s; the HBM roofline of the scan kernel
(algorithmic bytes per launch / average launch time against the 8 TB/s peak, with the bytes
counted by a committed profile of the current kernel source beside them, and the fraction of a
device copy's bandwidth measured in the same run); the ALU roofline that actually bounds it
(algorithmic flops per launch / launch time against the peak of the same fp32 instruction mix at
full issue, see ``alu_model``); and the fp64 CPU oracle timed on the host cores over whole batch
entries of the same workload.

``--workload bwd`` measures the backward pass (all input gradients) of the same workload, and
``--workload bwd-heads`` that of the scalar-decay heads config (recurrent form).
``--workload heads`` measures the scalar-decay heads scan (batch 4, 64 heads x 64 channels,
N 128, L 8192, bf16 I/O) in its chunked matrix form on the matrix cores (``--algorithm
recurrent`` for the step-by-step recurrence instead); its roofline is HBM bandwidth, with the
algorithmic matrix flops reported beside it against the bf16 MFMA peak.
``--workload complex`` measures the scan with a complex diagonal A (complex A, B and C; batch 8,
d_inner 1536, N 16, L 2048, bf16 I/O): its roofline is the fp32 VALU issue of its instruction mix
(exp2, sin and cos per state update), with the HBM figures beside it.
``--workload decode`` measures instead one recurrent decoding step (``ssm_selective_state_update``)
on the Mamba-1.4B layer at batch 1024: a step reads and writes the fp32 state once, so its
roofline is HBM bandwidth. ``--workload lsweep`` times the scan at a fixed batch x channels
(1 x 2048, the million-token config's) over L = 2^12 .. 2^20 and fits the slope of log time
against log L (1 for a linear-time scan). ``--copy-calibration`` runs only a plain device copy of
a known size (for scaling the FETCH_SIZE / WRITE_SIZE counters of a profiler run).
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure
WORKLOAD = 2           # Mamba-1.4B layer scan
HEADS_WORKLOAD = 4     # scalar-decay heads scan


def kernel_source_hash(names=None) -> str:
    """Hash of the library's kernel sources: all of csrc/, or the named files of it (those that
    define one kernel and its launch)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_24_amd", "csrc")
    for name in sorted(names if names is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(cfg_key: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the current
    source of that kernel (the files the record lists, else all of csrc/); None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{cfg_key}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec.get("source_hash") != kernel_source_hash(rec.get("sources")):
            return None
    except (OSError, ValueError):
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


VALU_CYCLES = 4   # SIMD cycles per wavefront-wide unpacked fp32 instruction
TRANS_CYCLES = 8  # per wavefront-wide exp2 / log2 / rcp


def alu_model(cfg):
    """Minimal fp32 instruction stream of the method per token*channel: (flops, SIMD cycles).

    Issue costs of a wavefront-wide (64-lane) instruction on one SIMD: an unpacked fp32
    add/mul/fma/max takes 4 cycles (16 lanes per cycle, the rate of the 78.6 TFLOP/s vector
    figure: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz; the 157.3 TFLOP/s fp32 figure
    needs the packed two-wide fp32 instructions, which this library's build switches off);
    exp2, log2 and rcp take 8 cycles. The profiler's VALU-busy counter charges exactly these
    costs (1 and 2 four-cycle units per instruction). Flops count an fma as 2 and every other
    operation, transcendentals included, as 1.
      per state update (t, channel, n): delta*a, exp2, u*B, h fma, readout fma -> 7 flops, 24 cyc
        (head mode: delta*a and exp2 once per (t, head) instead; complex A: 13 fp32 ops and
        exp2, sin, cos -> 22 flops, 76 cyc)
      per (t, channel): bias add (1, 4), softplus (10, 44: |v|*log2e, exp2, 1+e, log2, two
        subtractions of the log1p correction, fma, max, add), u = delta*x (1, 4), D skip fma
        (2, 4), silu gate (6, 32: z*log2e, exp2, 1+e, rcp, z*r, y*g)
    Unpacking and packing of bf16 are not counted (they are not arithmetic of the method).
    """
    valu, trans = VALU_CYCLES, TRANS_CYCLES
    head = cfg.a_mode == "head"
    rows_per_ch = 1.0 / cfg.headdim if head else 1.0
    fl = cy = 0.0
    if cfg.a_mode == "complex":
        # delta*Re(A), exp2, delta*Im(A), whole turns dropped, sin, cos, |Abar| cos, |Abar| sin,
        # delta*x*B (two parts), the complex update (4 fma), Re(C h) (2 fma)
        fl += cfg.N * 22
        cy += cfg.N * (13 * valu + 3 * trans)
    elif head:
        fl += cfg.N * 5 + 2 * rows_per_ch
        cy += cfg.N * 3 * valu + (valu + trans) * rows_per_ch
    else:
        fl += cfg.N * 7
        cy += cfg.N * (4 * valu + trans)
    if cfg.has_bias:
        fl += 1 * rows_per_ch
        cy += valu * rows_per_ch
    if cfg.softplus:
        fl += 10 * rows_per_ch
        cy += (7 * valu + 2 * trans) * rows_per_ch
    fl += 1
    cy += valu
    if cfg.has_D:
        fl += 2
        cy += valu
    if cfg.gate:
        fl += 6
        cy += 4 * valu + 2 * trans
    return fl, cy


SIMDS = 256 * 4
CLOCK_HZ = 2.4e9


def alu_peak_tflops(cfg) -> float:
    fl, cy = alu_model(cfg)
    return fl * 64 / cy * SIMDS * CLOCK_HZ / 1e12


def cpu_baseline(cfg, budget_s: float, scan=None):
    """The fp64 oracle, as it stands, over whole batch entries of the workload (inputs of one
    entry generated untimed, then the oracle timed on them), until every entry is done or the
    time budget is spent."""
    import oracle
    import ssmgen
    threads = oracle.cpu_threads()
    spent, done = 0.0, 0
    for b in range(cfg.batch):
        inputs = ssmgen.make_batch_entry(cfg, b)
        one = ssmgen.with_shape(cfg, batch=1)
        t0 = time.perf_counter()
        (scan or oracle.scan_inputs)(inputs, one, nthreads=threads)
        spent += time.perf_counter() - t0
        done += 1
        del inputs
        if spent >= budget_s:
            break
    tokch = done * cfg.dim * cfg.L
    return {
        "value": round(tokch / spent / 1e9, 6),
        "unit": "Gtoken\u00b7channel/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"batch entries 0..{done - 1} of {cfg.batch} ({done * cfg.dim} channels x "
                   f"{cfg.L} steps, {tokch * cfg.N / 1e9:.2f} G fp64 state updates) in "
                   f"{spent:.2f} s; input generation untimed"),
    }


def alu_model_bwd(cfg):
    """Minimal fp32 instruction stream of the gradient per token*channel: (flops, SIMD cycles),
    costs as in ``alu_model`` (diagonal A, delta * B rule).
      per state update: the states recomputed once (delta*a, exp2, u*B, fma: 5 flops, 20 cyc),
        with a gate their readout C h for dz (fma: 2 flops, 4 cyc), and the reverse step (gh += gy C; gy h for dC; exp2 of delta*a; g = gh (h_prev dA);
        ddelta part += g a; da += g delta; gh u for dB; sb += gh B; gh *= dA: 15 flops,
        10 plain ops + 1 transcendental = 48 cyc)
      per (t, channel): softplus and its derivative sigmoid (14 flops, 64 cyc), u = delta*x,
        the gate silu and silu' (12 flops, 52 cyc), y = readout + D x and dz (3 flops, 8 cyc),
        dx += gy D, dD += gy x, dbias += (4 fma/add: 7 flops, 16 cyc), and the two state sums
        ddelta part += x sb, dx part = delta sb (3 flops, 8 cyc)
    The sums over lanes for dB and dC and over the batch are not counted.
    With one A per head (``cfg.a_mode == "head"``) the decay and its exp2 are per (t, head): per
    state update the recompute is u*B and the h fma (3 flops, 8 cyc), the reverse step gh += gy C,
    gy h, gh h_prev sum, gh u, gh B sum, gh *= dA (9 flops, 24 cyc), and per (t, channel) two
    exp2 of delta*a (recompute and reverse) with the sums a dA s1 and delta dA s1 (4 flops)."""
    valu, trans = VALU_CYCLES, TRANS_CYCLES
    if cfg.a_mode == "head":
        fl = cfg.N * (3 + 9) + 2 + 4
        cy = cfg.N * (2 * valu + 6 * valu) + 2 * (valu + trans) + 3 * valu
        if cfg.gate:
            fl += cfg.N * 2
            cy += cfg.N * valu
        if cfg.softplus:
            fl += 14
            cy += 10 * valu + 3 * trans
        fl += 1
        cy += valu
        if cfg.gate:
            fl += 12
            cy += 9 * valu + 2 * trans
        fl += 3 + 7
        cy += 2 * valu + 4 * valu
        return fl, cy
    fl = cfg.N * (5 + 15) + 3
    cy = cfg.N * ((3 * valu + trans) + (10 * valu + trans)) + 2 * valu
    if cfg.gate:
        fl += cfg.N * 2
        cy += cfg.N * valu
    if cfg.softplus:
        fl += 14
        cy += 10 * valu + 3 * trans
    fl += 1
    cy += valu
    if cfg.gate:
        fl += 12
        cy += 9 * valu + 2 * trans
    fl += 3 + 7
    cy += 2 * valu + 4 * valu
    return fl, cy


def bwd_bytes(cfg) -> int:
    """Algorithmic bytes of the backward pass: the forward's inputs and dy read once; dx, ddelta,
    dz written in the io dtype; dB, dC (fp32), dA, dD, dbias written once."""
    io = 4 if cfg.io == "f32" else 2
    tok = cfg.batch * cfg.dim * cfg.L
    reads = cfg.algorithmic_bytes() - tok * io  # forward inputs (without y)
    reads += tok * io                           # dy
    writes = tok * io * (3 if cfg.gate else 2)  # dx, ddelta, dz
    writes += 2 * cfg.batch * cfg.ngroups * cfg.N * cfg.L * 4 + cfg.dim * cfg.N * 4 + 2 * cfg.dim * 4
    return reads + writes


def run_bwd(args, torch, heads=False):
    import numpy as np
    import ssmgen
    import selective_state_space_24_amd as ssm
    cfg = ssmgen.CONFIGS[HEADS_WORKLOAD if heads else WORKLOAD]
    dev = device_inputs(cfg, torch)
    dy = torch.randn(cfg.batch, cfg.dim, cfg.L, device="cuda").to(dev["x"].dtype)
    stream = torch.cuda.current_stream()
    desc = ssm.describe(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["z"], dy)
    g = {"dx": torch.empty_like(dev["x"]), "ddelta": torch.empty_like(dev["delta"]),
         "dz": torch.empty_like(dev["z"]), "dA": torch.empty_like(dev["A"]),
         "dB": torch.empty(dev["B"].shape, device="cuda"),
         "dC": torch.empty(dev["C"].shape, device="cuda"),
         "dD": torch.empty_like(dev["D"]), "ddelta_bias": torch.empty_like(dev["delta_bias"])}
    ws_bytes = ssm.bwd_workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        rc = ssm.bwd_raw(desc, dev["x"].data_ptr(), dev["delta"].data_ptr(), dev["A"].data_ptr(),
                         dev["B"].data_ptr(), dev["C"].data_ptr(), dev["D"].data_ptr(),
                         dev["z"].data_ptr(), dev["delta_bias"].data_ptr(), True, None,
                         dy.data_ptr(), g["dx"].data_ptr(), g["ddelta"].data_ptr(),
                         g["dA"].data_ptr(), g["dB"].data_ptr(), g["dC"].data_ptr(),
                         g["dD"].data_ptr(), g["dz"].data_ptr(), g["ddelta_bias"].data_ptr(),
                         None, ws.data_ptr(), ws_bytes, stream.cuda_stream)
        if rc != 0:
            raise ssm.ScanError(rc, "ssm_selective_scan_bwd")

    ms, pct = timed_steps(step, args, torch, stream)
    fl, cy = alu_model_bwd(cfg)
    peak = fl * 64 / cy * SIMDS * CLOCK_HZ / 1e12
    achieved = fl * cfg.tokch / (ms * 1e-3) / 1e12
    nbytes = bwd_bytes(cfg)
    out = {
        "metric": "selective-scan backward Gtoken\u00b7channel/s, 1 MI355X",
        "value": round(cfg.tokch / (ms * 1e-3) / 1e9, 3),
        "unit": "Gtoken\u00b7channel/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": f"f32 arithmetic and state, {cfg.io} io", "data": "synthetic",
        "config": {"workload": ("scalar-decay heads selective scan backward (all input "
                                "gradients; one A per head, 64 heads x 64)" if heads else
                                "Mamba-1.4B layer selective scan backward (all input gradients)"),
                   "batch": cfg.batch, "d_inner": cfg.dim, "seq_len": cfg.L, "d_state": cfg.N,
                   "io_dtype": cfg.io, "gate": "silu(z)", "delta_softplus": cfg.softplus},
        "roofline": {"bound": "alu", "achieved": round(achieved, 2), "peak": round(peak, 2),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None},
        "hbm": {"algorithmic_bytes": nbytes,
                "algorithmic_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "step_ms": {"p10": round(pct(0.1), 5), "median": round(pct(0.5), 5),
                    "p90": round(pct(0.9), 5)},
        "launches_per_step": 5 if heads else 4,
        "kernel_source": kernel_source_hash(),
    }
    if args.cpu_budget > 0:
        import oracle
        del dev, dy, g, ws
        torch.cuda.empty_cache()
        threads = min(oracle.cpu_threads(), cfg.batch)  # the oracle's backward splits the batch
        if heads:
            # one batch entry (the oracle's backward runs one thread per entry) is about 40 s of
            # work: a sample of 8 heads of entry 0 instead, 8 threads at once
            from concurrent.futures import ThreadPoolExecutor
            nh = 8
            dyh = np.random.default_rng(0).standard_normal((cfg.headdim * nh, cfg.L))

            def one(h):
                d0 = h * cfg.headdim
                sub = ssmgen.block_config(cfg, d0, d0 + cfg.headdim)
                inp = ssmgen.make_channel_block(cfg, 0, d0, d0 + cfg.headdim, nthreads=1)
                return inp, sub
            blocks = [one(h) for h in range(nh)]
            t0 = time.perf_counter()
            with ThreadPoolExecutor(max_workers=nh) as ex:
                list(ex.map(lambda i: oracle.scan_inputs_bwd(
                    blocks[i][0], dyh[None, i * cfg.headdim:(i + 1) * cfg.headdim], blocks[i][1],
                    nthreads=1), range(nh)))
            spent = time.perf_counter() - t0
            tok = nh * cfg.headdim * cfg.L
            out["cpu_baseline"] = {
                "value": round(tok / spent / 1e9, 6), "unit": out["unit"], "cores": nh,
                "kind": "oracle",
                "sample": f"{nh} heads of batch entry 0 ({nh * cfg.headdim} channels x {cfg.L} "
                          f"steps), one thread per head, in {spent:.2f} s; input generation "
                          f"untimed"}
        else:
            inputs = ssmgen.make_inputs(cfg)
            dyh = np.random.default_rng(0).standard_normal((cfg.batch, cfg.dim, cfg.L))
            t0 = time.perf_counter()
            oracle.scan_inputs_bwd(inputs, dyh, cfg, nthreads=threads)
            spent = time.perf_counter() - t0
            out["cpu_baseline"] = {
                "value": round(cfg.tokch / spent / 1e9, 6), "unit": out["unit"], "cores": threads,
                "kind": "oracle",
                "sample": f"the whole workload once ({cfg.batch} batch entries, one thread each) "
                          f"in {spent:.2f} s; input generation untimed"}
    print(json.dumps(out), flush=True)


def chunked_flops(cfg, Q: int = 64) -> int:
    """Algorithmic matrix flops of the chunked form per launch, per (batch, head, chunk of Q):
    the causal C.B tile (Q(Q+1)/2 entries of N multiply-adds), the causal intra-chunk product
    (Q(Q+1)/2 x headdim), the inter-chunk product C^T H and the state update B x (Q N headdim
    each); a multiply-add counts 2. The bf16 hi + lo operand pairs, which double some of the
    executed products, are not counted."""
    P, N = cfg.headdim, cfg.N
    tri = Q * (Q + 1) // 2
    per_chunk = 2 * (tri * N + tri * P + 2 * Q * N * P)
    nchunks = (cfg.L + Q - 1) // Q
    return per_chunk * nchunks * cfg.batch * (cfg.dim // P)


def run_heads(args, torch):
    import ssmgen
    import selective_state_space_24_amd as ssm
    cfg = ssmgen.CONFIGS[HEADS_WORKLOAD]
    dev = device_inputs(cfg, torch)
    y = torch.empty_like(dev["x"])
    stream = torch.cuda.current_stream()
    desc = ssm.describe(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["z"], y)
    algo = ssm.ALGORITHMS[args.algorithm]
    ext = ssm.ScanExt(ssm.SSM_DISC_DELTA_B, algo, None, None)
    ws_bytes = ssm.workspace_size(desc) if algo == ssm.SSM_ALGO_RECURRENT else 0
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        rc = ssm.fwd_ext_raw(desc, dev["x"].data_ptr(), dev["delta"].data_ptr(),
                             dev["A"].data_ptr(), dev["B"].data_ptr(), dev["C"].data_ptr(),
                             dev["D"].data_ptr(), dev["z"].data_ptr(),
                             dev["delta_bias"].data_ptr(), True, y.data_ptr(), ext,
                             ws.data_ptr() if ws_bytes else None, ws_bytes, stream.cuda_stream)
        if rc != 0:
            raise ssm.ScanError(rc, "ssm_selective_scan_fwd_ext")

    ms, pct = timed_steps(step, args, torch, stream)
    nbytes = cfg.algorithmic_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    flops = chunked_flops(cfg)
    tflops = flops / (ms * 1e-3) / 1e12
    chunked = algo != ssm.SSM_ALGO_RECURRENT
    out = {
        "metric": "selective-scan Gtoken\u00b7channel/s and achieved HBM GB/s vs peak, 1 MI355X",
        "value": round(cfg.tokch / (ms * 1e-3) / 1e9, 3),
        "unit": "Gtoken\u00b7channel/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16 matrix products, fp32 accumulation and state, bf16 io" if chunked
                  else f"f32 arithmetic and state, {cfg.io} io"),
        "data": "synthetic",
        "config": {"workload": "scalar-decay heads selective scan (one A per head, B/C shared "
                               "by all heads)" + (", chunked matrix form" if chunked else
                                                  ", recurrent form"),
                   "batch": cfg.batch, "d_inner": cfg.dim, "heads": cfg.dim // cfg.headdim,
                   "headdim": cfg.headdim, "seq_len": cfg.L, "d_state": cfg.N,
                   "io_dtype": cfg.io, "gate": "silu(z)", "delta_softplus": cfg.softplus,
                   "algorithm": args.algorithm},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile("heads_chunked") if chunked else None},
        "mfma": {"algorithmic_flops": flops, "achieved_TFLOPs": round(tflops, 1),
                 "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                 "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)} if chunked else None,
        "step_ms": {"p10": round(pct(0.1), 5), "median": round(pct(0.5), 5),
                    "p90": round(pct(0.9), 5)},
        "launches_per_step": 1 if (chunked or ws_bytes == 0) else 2,
        "kernel_source": kernel_source_hash(),
    }
    if args.cpu_budget > 0:
        del dev, y
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(out), flush=True)


def decode_bytes(cfg) -> int:
    """Algorithmic bytes of one decoding step: the fp32 state read and written, every other
    input read once and y written once."""
    return cfg.algorithmic_bytes() + 2 * cfg.batch * cfg.dim * cfg.N * 4


def run_decode(args, torch):
    import numpy as np
    import ssmgen
    import selective_state_space_24_amd as ssm
    cfg = ssmgen.DECODE_CONFIGS["mamba14b_decode"]
    dev = device_inputs(cfg, torch)
    rng = np.random.default_rng(0)
    state0 = rng.standard_normal((cfg.batch, cfg.dim, cfg.N)).astype(np.float32)
    state = torch.from_numpy(state0).cuda()
    sq = {k: (v[..., 0].contiguous() if k in ("x", "delta", "z", "B", "C") else v)
          for k, v in dev.items()}
    y = torch.empty_like(sq["x"])
    stream = torch.cuda.current_stream()
    desc = ssm.describe_step(state, sq["x"], sq["delta"], sq["A"], sq["B"], sq["C"], sq["z"], y)

    def step():
        rc = ssm.state_update_raw(desc, state.data_ptr(), sq["x"].data_ptr(), sq["delta"].data_ptr(),
                                  sq["A"].data_ptr(), sq["B"].data_ptr(), sq["C"].data_ptr(),
                                  sq["D"].data_ptr(), sq["z"].data_ptr(), sq["delta_bias"].data_ptr(),
                                  True, y.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise ssm.ScanError(rc, "ssm_selective_state_update")

    ms, pct = timed_steps(step, args, torch, stream)
    nbytes = decode_bytes(cfg)
    achieved = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "selective-SSM decode step: tokens/s and achieved HBM GB/s vs peak, 1 MI355X",
        "value": round(cfg.batch / (ms * 1e-3), 1),
        "unit": "tokens/s (one token per sequence per step, one layer)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"f32 arithmetic and state, {cfg.io} io", "data": "synthetic",
        "config": {"workload": "Mamba-1.4B layer decode step", "batch": cfg.batch,
                   "d_inner": cfg.dim, "d_state": cfg.N, "io_dtype": cfg.io,
                   "state": "fp32, updated in place", "gate": "silu(z)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile("mamba14b_decode")},
        "algorithmic_bytes_per_step": nbytes,
        "step_ms": {"p10": round(pct(0.1), 5), "median": round(pct(0.5), 5),
                    "p90": round(pct(0.9), 5)},
        "launches_per_step": 1,
        "kernel_source": kernel_source_hash(),
    }
    if args.cpu_budget > 0:
        import oracle
        threads = oracle.cpu_threads()
        inputs = ssmgen.make_inputs(cfg)
        spent, steps = 0.0, 0
        h = state0.astype(np.float64)
        while spent < args.cpu_budget and steps < 50:
            t0 = time.perf_counter()
            _, h = oracle.scan_inputs(inputs, cfg, h0=h, return_final_state=True,
                                      nthreads=threads)
            spent += time.perf_counter() - t0
            steps += 1
        out["cpu_baseline"] = {
            "value": round(steps * cfg.batch / spent, 1), "unit": out["unit"], "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} whole decoding steps of the workload (batch {cfg.batch}) in "
                      f"{spent:.2f} s; input generation untimed"}
    print(json.dumps(out), flush=True)


def timed_steps(step, args, torch, stream):
    """W untimed steps, then K steps between two synchronisations, timed with events on the
    launch stream (each step also timed alone for percentiles)."""
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s_ev, e_ev in ev:
        s_ev.record(stream)
        step()
        e_ev.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    per = sorted(s_ev.elapsed_time(e_ev) for s_ev, e_ev in ev)
    pct = lambda q: per[min(len(per) - 1, int(q * (len(per) - 1) + 0.5))]
    return ms, pct


def measure_copy_GBs(torch, nbytes: int = 1 << 30, reps: int = 20) -> float:
    """Read + write bandwidth of a plain device-to-device copy of ``nbytes`` (event-timed on the
    current stream after a short warm-up): the practical ceiling of a streaming kernel."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def run_lsweep(args, torch):
    """Time per call of the scan over L = 2^12 .. 2^20 at batch 1 x 2048 channels (bf16, N 16,
    gate and softplus on). Inputs are drawn on the GPU with the workload's distributions from a
    seeded generator (timing only: the parity tests cover these shapes)."""
    import math
    import selective_state_space_24_amd as ssm
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    batch, dim, N = 1, 2048, 16
    A = -torch.arange(1, N + 1, dtype=torch.float32, device="cuda").repeat(dim, 1).contiguous()
    D = torch.randn(dim, generator=g, device="cuda")
    u = torch.rand(dim, generator=g, device="cuda") * 0.099 + 0.001
    bias = torch.log(torch.expm1(u))
    points = []
    stream = torch.cuda.current_stream()
    for e in range(12, 21):
        L = 1 << e
        bf = torch.bfloat16
        x = torch.randn(batch, dim, L, generator=g, device="cuda").to(bf)
        dl = (0.5 * torch.randn(batch, dim, L, generator=g, device="cuda")).to(bf)
        z = torch.randn(batch, dim, L, generator=g, device="cuda").to(bf)
        B = torch.randn(batch, 1, N, L, generator=g, device="cuda").to(bf)
        C = torch.randn(batch, 1, N, L, generator=g, device="cuda").to(bf)
        y = torch.empty_like(x)
        desc = ssm.describe(x, dl, A, B, C, z, y)
        ws_bytes = ssm.workspace_size(desc)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

        def step():
            rc = ssm.fwd_raw(desc, x.data_ptr(), dl.data_ptr(), A.data_ptr(), B.data_ptr(),
                             C.data_ptr(), D.data_ptr(), z.data_ptr(), bias.data_ptr(), True,
                             y.data_ptr(), ws.data_ptr() if ws_bytes else None, ws_bytes,
                             stream.cuda_stream)
            if rc != 0:
                raise ssm.ScanError(rc, "ssm_selective_scan_fwd")

        sub = argparse.Namespace(warmup=max(3, min(args.warmup, 20)), steps=max(5, min(args.steps, 20)))
        ms, pct = timed_steps(step, sub, torch, stream)
        tokch = batch * dim * L
        points.append({"L": L, "ms": round(ms, 5), "median_ms": round(pct(0.5), 5),
                       "Gtokch_s": round(tokch / (ms * 1e-3) / 1e9, 2),
                       "launches": 1 if ws_bytes == 0 else 2})
        print(f"[lsweep] L={L}: {ms:.4f} ms", file=sys.stderr, flush=True)
        del x, dl, z, B, C, y, ws
        torch.cuda.empty_cache()
    xs = [math.log(pt["L"]) for pt in points]
    ys = [math.log(pt["ms"]) for pt in points]
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    slope = sum((a - mx) * (b - my) for a, b in zip(xs, ys)) / sum((a - mx) ** 2 for a in xs)
    # the same fit over the points whose segment plan fills the chip (L >= 2^15)
    big = [(a, b) for a, b, pt in zip(xs, ys, points) if pt["L"] >= 1 << 15]
    mbx, mby = sum(a for a, _ in big) / len(big), sum(b for _, b in big) / len(big)
    slope_big = (sum((a - mbx) * (b - mby) for a, b in big) /
                 sum((a - mbx) ** 2 for a, _ in big))
    last = points[-1]
    out = {
        "metric": "selective-scan time vs sequence length at fixed batch x channels, 1 MI355X",
        "value": round(slope, 4), "unit": "d log(time) / d log(L)", "n_gpus": 1,
        "steps": sub.steps, "warmup": sub.warmup, "ms_per_step": last["ms"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 arithmetic and state, bf16 io", "data": "synthetic (seeded, on the GPU)",
        "config": {"workload": "S6 forward scan, batch 1 x d_inner 2048, N 16, L 2^12..2^20",
                   "gate": "silu(z)", "delta_softplus": True},
        "slope_L_ge_32768": round(slope_big, 4),
        "points": points,
        "kernel_source": kernel_source_hash(),
    }
    print(json.dumps(out), flush=True)


def run_complex(args, torch):
    import oracle
    import ssmgen
    import selective_state_space_24_amd as ssm
    cfg = ssmgen.COMPLEX_CONFIG
    dev = device_inputs(cfg, torch)
    y = torch.empty_like(dev["x"])
    stream = torch.cuda.current_stream()
    desc = ssm.describe(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["z"], y)

    def step():
        rc = ssm.fwd_raw(desc, dev["x"].data_ptr(), dev["delta"].data_ptr(), dev["A"].data_ptr(),
                         dev["B"].data_ptr(), dev["C"].data_ptr(), dev["D"].data_ptr(),
                         dev["z"].data_ptr(), dev["delta_bias"].data_ptr(), True, y.data_ptr(),
                         None, 0, stream.cuda_stream)
        if rc != 0:
            raise ssm.ScanError(rc, "ssm_selective_scan_fwd")

    ms, pct = timed_steps(step, args, torch, stream)
    fl, cy = alu_model(cfg)
    achieved = fl * cfg.tokch / (ms * 1e-3) / 1e12
    peak = alu_peak_tflops(cfg)
    nbytes = cfg.algorithmic_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "selective-scan Gtoken\u00b7channel/s and achieved HBM GB/s vs peak, 1 MI355X",
        "value": round(cfg.tokch / (ms * 1e-3) / 1e9, 3),
        "unit": "Gtoken\u00b7channel/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": f"f32 arithmetic and complex state, {cfg.io} io", "data": "synthetic",
        "config": {"workload": "selective scan with a complex diagonal A (complex A, B, C; "
                               "real delta, x, z)",
                   "batch": cfg.batch, "d_inner": cfg.dim, "seq_len": cfg.L, "d_state": cfg.N,
                   "io_dtype": cfg.io, "gate": "silu(z)", "delta_softplus": cfg.softplus},
        # the kernel is bound by VALU issue: the peak is that of its own instruction mix at full
        # issue on 1024 SIMDs at 2.4 GHz (alu_model)
        "roofline": {"bound": "alu", "achieved": round(achieved, 2), "peak": round(peak, 2),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_from_profile("complex_layer"),
                     "derivation": (f"per 64 token*channels: {cfg.N} complex state updates x "
                                    f"(13 fp32 ops x {VALU_CYCLES} cycles + exp2, sin, cos x "
                                    f"{TRANS_CYCLES} cycles) + bias, softplus, delta*x, D skip "
                                    f"and silu gate = {cy:.0f} SIMD cycles for {fl:.0f} flops; "
                                    f"1024 SIMDs at 2.4 GHz")},
        "hbm": {"algorithmic_bytes": nbytes, "achieved_GBs": round(gbs, 1),
                "peak_GBs": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4)},
        "step_ms": {"p10": round(pct(0.1), 5), "median": round(pct(0.5), 5),
                    "p90": round(pct(0.9), 5)},
        "launches_per_step": 1,
        "kernel_source": kernel_source_hash(),
    }
    if args.cpu_budget > 0:
        del dev, y
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget, scan=oracle.scan_inputs_complex)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # Under sustained load the clock settles over the first ~20 launches (a launch right after
    # a short warm-up runs up to 20% slower than in steady state), so the default warm-up runs
    # past that transient; the timed steps then measure the steady state.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 skips it)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--workload", choices=("scan", "decode", "bwd", "bwd-heads", "heads",
                                           "lsweep", "complex"), default="scan")
    ap.add_argument("--algorithm", choices=("chunked", "recurrent"), default="chunked",
                    help="--workload heads: the form of the scan")
    ap.add_argument("--config", type=int, choices=(0, 1, 2, 3, 4), default=WORKLOAD,
                    help="--workload scan: the config timed (default: the Mamba-1.4B layer)")
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

    if args.workload == "decode":
        run_decode(args, torch)
        return
    if args.workload in ("bwd", "bwd-heads"):
        run_bwd(args, torch, heads=args.workload == "bwd-heads")
        return
    if args.workload == "heads":
        run_heads(args, torch)
        return
    if args.workload == "lsweep":
        run_lsweep(args, torch)
        return
    if args.workload == "complex":
        run_complex(args, torch)
        return

    import ssmgen
    import selective_state_space_24_amd as ssm

    cfg = ssmgen.CONFIGS[args.config]
    dev = device_inputs(cfg, torch)
    y = torch.empty_like(dev["x"])
    stream = torch.cuda.current_stream()
    desc = ssm.describe(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], dev.get("z"), y)
    ws_bytes = ssm.workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def ptr(name):
        t = dev.get(name)
        return t.data_ptr() if t is not None else None

    def step():
        rc = ssm.fwd_raw(desc, ptr("x"), ptr("delta"), ptr("A"), ptr("B"), ptr("C"), ptr("D"),
                         ptr("z"), ptr("delta_bias"), cfg.softplus, y.data_ptr(),
                         ws.data_ptr() if ws_bytes else None, ws_bytes, stream.cuda_stream)
        if rc != 0:
            raise ssm.ScanError(rc, "ssm_selective_scan_fwd")

    # the device-copy reference runs first: it is part of the line, and it also brings the GPU
    # out of idle (the clock ramps up over the first ~10 ms of load) before the warm-up steps
    copy_gbs = measure_copy_GBs(torch)
    ms, pct = timed_steps(step, args, torch, stream)

    # one launch per step when the sequence is not split along L (no workspace needed)
    launches = 1 if ws_bytes == 0 else 2
    tokch = cfg.tokch
    alg_bytes = cfg.algorithmic_bytes()
    fl, _ = alu_model(cfg)
    alg_flops = fl * tokch
    peak = alu_peak_tflops(cfg)
    launch_ms = ms if launches == 1 else None
    achieved = alg_flops / (launch_ms * 1e-3) / 1e12 if launch_ms else None
    traffic = traffic_from_profile("mamba14b_layer") if args.config == WORKLOAD else None
    hbm_gbs = alg_bytes / (launch_ms * 1e-3) / 1e9 if launch_ms else None
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
        "dtype": f"f32 arithmetic and state, {cfg.io} io",
        "data": "synthetic",
        "config": {
            "workload": ("Mamba-1.4B layer selective scan (S6 forward)" if args.config == WORKLOAD
                         else f"selective scan (S6 forward), {cfg.name}"),
            "batch": cfg.batch, "d_inner": cfg.dim, "seq_len": cfg.L, "d_state": cfg.N,
            "io_dtype": cfg.io, "gate": "silu(z)" if cfg.gate else None,
            "delta_softplus": cfg.softplus, "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(hbm_gbs, 1) if hbm_gbs else None,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(hbm_gbs / HBM_PEAK_GBS, 4) if hbm_gbs else None,
            "traffic": traffic,
            "algorithmic_bytes": alg_bytes,
            "copy_GBs": round(copy_gbs, 1),
            "frac_of_copy": round(hbm_gbs / copy_gbs, 4) if hbm_gbs else None,
            "counter_GBs": round(traffic / (launch_ms * 1e-3) / 1e9, 1)
            if (traffic and launch_ms) else None,
        },
        # what actually bounds this kernel: fp32 VALU and transcendental issue. The peak is that
        # of the method's own instruction mix at full issue on 1024 SIMDs at 2.4 GHz (alu_model)
        "alu": {
            "achieved": round(achieved, 2) if achieved else None,
            "peak": round(peak, 2),
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4) if achieved else None,
            "frac_of_fp32_vector_peak": round(achieved / 78.6, 4) if achieved else None,
            "derivation": (f"per 64 token*channels: {cfg.N} state updates x (4 fp32 ops x "
                           f"{VALU_CYCLES} cycles + 1 exp2 x {TRANS_CYCLES} cycles) + bias, "
                           f"softplus, delta*x, D skip and silu gate = {alu_model(cfg)[1]:.0f} "
                           f"SIMD cycles for {fl:.0f} flops; 1024 SIMDs at 2.4 GHz"),
        },
        "step_ms": {"p10": round(pct(0.1), 5), "median": round(pct(0.5), 5),
                    "p90": round(pct(0.9), 5)},
        "launches_per_step": launches,
        "kernel_source": kernel_source_hash(),
    }
    if args.cpu_budget > 0:
        del dev, y
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
