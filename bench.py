#!/usr/bin/env python3
"""Throughput of volumetric delay-and-sum on one MI355X.

One step is one pass of the whole hot path over one volume of the workload:
das_permute (B x Q x M x K -> the kernel's permuted layout) followed by
das_beamform, inputs already resident in HBM.

Prints ONE JSON line.  `value` is accumulations (voxels x receivers x
transmit events x frames) per second of whole steps (permute + beamform);
`kernel_value` is the same count per second of beamform kernel time alone.
The roofline object describes the beamform kernel, timed with HIP events on
the stream it runs on, against its arithmetic roofline, with the on-chip
delivery ceiling beside it; cpu_baseline times the fp64 oracle on bounded
slabs of the same volume on the host, single-threaded and on P threads.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3        # MI355X vector fp32 (published)
PEAK_FP64_TFLOPS = 78.6         # MI355X vector fp64 (published)
PEAK_F16_MFMA_TFLOPS = 2500.0   # MI355X dense fp16 matrix (published)
REPACK_MAX_LISTED = 4096        # receivers up to which the repack kernel lists each tile's live ones
PEAK_HBM_GBS = 8000.0
CUS, SCLK_HZ = 256, 2.4e9

# LDS bytes per clock per CU that gfx950 serves for the read pattern of each
# staged kernel instance, measured on the box with a microbenchmark (one
# 1024-thread workgroup per CU on all CUs, random rows, wall-clock time)
LDS_BCLK = {
    "two ds_read_b64 (8-byte lanes)": 160.0,
    "two ds_read_b128 (16-byte lanes, split rows)": 219.0,
    "16 ds_read_b128 per lane, two whole 128-B rows, bank-group order": 238.0,
    # the same instructions and bank groups over 128-byte slots, half the rows' bytes
    "8 ds_read_b128 per lane, two 64-B binary16 rows in 128-B slots, bank-group order": 238.0,
}


_COMMENT = re.compile(r"/\*.*?\*/|//[^\n]*", re.S)


# the source file of each kernel; a stored reading depends on it, on the
# shared device headers and on the host code that picks and launches it
KERNEL_SOURCES = {
    "das_bi_rows_kernel": "das_bi_rows.hip",
    "das_bi_staged_kernel": "das_batch_inner_staged.hip",
    "das_batch_inner_kernel": "das_batch_inner.hip",
    "das_baseline_kernel": "das_baseline.hip",
    "das_baseline_f64_kernel": "das_baseline_f64.hip",
    "das_repack_kernel": "das_repack.hip",
    "permute_f32_kernel": "das_permute.hip",
    "tx_tables_kernel": "das_tx.hip",
}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code (comments and whitespace dropped) of a kernel's source
    file, the shared headers and the host API; a stored counter reading is
    valid only for the same hash."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "volumetric_delay_sum_amd", "csrc")
    for name in sorted({KERNEL_SOURCES[kernel], "das_device.h", "das_internal.h", "das_api.cpp"}):
        with open(os.path.join(csrc, name), encoding="utf-8", errors="replace") as fh:
            code = " ".join(_COMMENT.sub(" ", fh.read()).split())
        h.update(name.encode())
        h.update(code.encode())
    return h.hexdigest()[:16]


def stored_counter(kernel: str, workload: str, field: str):
    """A reading of the committed counter summary (profiles/traffic.json) for
    a kernel and workload, if it was taken on these sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}:{workload}")
        if rec and rec.get("source_hash") == kernel_source_hash(kernel):
            return rec.get(field)
    except Exception:
        return None
    return None


def pick_bound(t_hbm: float, t_alu: float, hbm_frac, valu_busy) -> str:
    """Which roof binds a launch: HBM if its algorithmic bytes at 8 TB/s take
    longer than its flops at the vector peak, or if the HBM bytes the
    counters saw keep HBM busier (fraction of 8 TB/s) than the VALU is busy
    (VALUBusy read on the same sources); else the ALU."""
    if t_hbm > t_alu:
        return "hbm"
    if hbm_frac is not None and valu_busy is not None and hbm_frac > valu_busy:
        return "hbm"
    return "alu"


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it matches these sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
        rec = data.get(f"{kernel}:{workload}")
        if rec and rec.get("source_hash") == kernel_source_hash(kernel):
            return rec.get("hbm_bytes_per_launch")
    except Exception:
        return None
    return None


def listed_slots(cfg, tile, block):
    """Receiver slots a kernel that lists each voxel tile's receivers sweeps.
    Each tile of tile = (tx, ty, tz) voxels lists the receivers with a
    non-zero receive weight for one of its voxels (the f-number cone) and
    sweeps the list in steps of `block` entries; the rest are exact zeros it
    skips.  Per tile and receiver the cone test is taken at the tile's voxel
    nearest to the receiver laterally on its deepest plane (where the cone is
    widest), which is where the kernel's per-voxel test first passes.  Returns
    the sum over tiles of (steps x block) times the tile's voxel count."""
    import numpy as np
    import das_synth
    px, py, pz = tile
    rx = das_synth.array_positions(cfg).astype(np.float64)
    (ox, oy, oz), (sx, sy, sz), (nx, ny, nz) = das_synth.voxel_grid(cfg)
    ct = np.cos(np.arctan(1.0 / (2.0 * cfg.f_number)))
    a_, b_ = (1.0 - ct * ct) * 1.001, ct * ct
    txs, tys, tzs = np.arange(0, nx, px), np.arange(0, ny, py), np.arange(0, nz, pz)
    def nearest(p, o, s, lo, span, n):                 # nearest voxel centre of [lo, lo + span) to p
        i = np.clip(np.rint((p[None, :] - o) / s), lo[:, None], np.minimum(lo + span, n)[:, None] - 1)
        return o + i * s - p[None, :]
    dx2 = nearest(rx[:, 0], ox, sx, txs, px, nx) ** 2  # tiles_x x M
    dy2 = nearest(rx[:, 1], oy, sy, tys, py, ny) ** 2  # tiles_y x M
    dz = oz + (np.minimum(tzs + pz, nz) - 1) * sz      # deepest plane of each tile depth (array at z = 0)
    slots = 0
    for z in dz:
        rho2 = dy2[:, None, :] + dx2[None, :, :]       # tiles_y x tiles_x x M
        live = (z - rx[:, 2][None, None, :] > 0) & (b_ * rho2 < a_ * (z - rx[:, 2][None, None, :]) ** 2)
        slots += (np.ceil(live.sum(-1) / block) * block).sum()
    return float(slots * px * py * pz)


def executed_fraction(cfg, info):
    """Share of the sum's terms the whole-row kernel executes: 8 x 8 x 2 voxel
    tiles, each sweeping its receiver list in blocks of 8, NIT blocks a step.
    Returns executed term slots (steps x NIT x 8 receivers x 128 voxels x
    events x frames) over N M Q B."""
    if not info["whole_rows"] or cfg.f_number <= 0:
        return 1.0
    return listed_slots(cfg, (8, 8, 2), info["receivers_per_step"]) / (cfg.N * cfg.M)


def executed_fraction_repack(cfg, receivers_per_step):
    """Share of the sum's terms the repack kernel executes: 16 x 16 x 1 voxel
    tiles, each sweeping its receiver list a step of 8 (one 32-frame tile
    a wave) or 4 (two) receivers at a time."""
    if cfg.f_number <= 0 or cfg.M > REPACK_MAX_LISTED:
        return 1.0
    return listed_slots(cfg, (16, 16, 1), receivers_per_step) / (cfg.N * cfg.M)


def executed_fraction_baseline(cfg):
    """Share of the sum's terms the baseline kernels (fp32 / complex64 and
    float64 / complex128) execute.  A wave holds an 8 x 8 lateral patch of voxels on one plane and
    skips a receiver (all its events and frames) when the receiver's cone
    contains none of the patch's voxels; per patch and receiver the test is
    taken at the patch's voxel nearest to the receiver laterally.  Returns
    executed (wave, receiver) slots x 64 voxels over N M (padding voxels of
    ragged patches included, as the kernel runs them)."""
    import numpy as np
    import das_synth
    if cfg.f_number <= 0:
        return 1.0
    rx = das_synth.array_positions(cfg).astype(np.float64)
    (ox, oy, oz), (sx, sy, sz), (nx, ny, nz) = das_synth.voxel_grid(cfg)
    t2 = (1.0 / (2.0 * cfg.f_number)) ** 2
    pxs, pys = np.arange(0, nx, 8), np.arange(0, ny, 8)
    def nearest(p, o, s, lo, n):
        i = np.clip(np.rint((p[None, :] - o) / s), lo[:, None], np.minimum(lo + 8, n)[:, None] - 1)
        return o + i * s - p[None, :]
    dx2 = nearest(rx[:, 0], ox, sx, pxs, nx) ** 2
    dy2 = nearest(rx[:, 1], oy, sy, pys, ny) ** 2
    live = 0
    for iz in range(nz):
        dz = oz + iz * sz - rx[:, 2]
        rho2 = dy2[:, None, :] + dx2[None, :, :]
        live += ((dz[None, None, :] > 0) & (rho2 < t2 * dz[None, None, :] ** 2)).sum()
    return float(live * 64 / (cfg.N * cfg.M))


def repack_mfma(cfg, plan, h16: bool, launch_ms: float, launches: int, q_launch: int, executed: float):
    """Matrix-core side of the repack variant: each (32-voxel group, event,
    swept receiver slot, 32-frame tile) issues at least one 16-position
    block of products, each a 32 x 32 x 16 fp16 matrix product (2 x 16,384
    flops), three per block with float32 samples (hi and lo parts), two with
    binary16 samples; windows wider than 16 positions add blocks, so these
    are lower bounds of the flops the matrix cores run, against their dense
    fp16 peak.  `executed`: the share of (voxel, receiver) slots the tiles'
    receiver lists sweep (1: every receiver)."""
    groups = -(-cfg.grid[0] // 16) * -(-cfg.grid[1] // 16) * cfg.grid[2] * 8   # 8 x 4 groups of 16 x 16 tiles
    group_rx = groups * cfg.M if executed >= 1.0 else executed * cfg.N * cfg.M / 32
    ftiles = -(-cfg.B // 32)
    products = 2 if h16 else 3
    flops = group_rx * q_launch * ftiles * products * 2 * 32 * 32 * 16
    tf = flops / (launch_ms * 1e-3) / 1e12
    return {"peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s", "issued_flops_per_launch_min": flops,
            "achieved_min": tf, "frac_min": tf / PEAK_F16_MFMA_TFLOPS, "products_per_block": products,
            "note": "lower bounds: one 16-position block per (group, event, listed receiver, frame tile); the useful "
                    "flops are in achieved / frac above"}


def delivery_ceiling(plan, iq: bool, h16: bool):
    """On-chip delivery roofline of the LDS-staged batch-inner kernels: every
    accumulation (voxel, receiver, event, frame) needs its two samples in
    registers, so the LDS's bytes per clock bound the accumulation rate at
    CUS * sclk * (B/clk/CU) / (bytes per accumulation)."""
    if not plan.batch_inner or not plan.info["staged"]:
        return None
    sample = (8 if iq else 4) // (2 if h16 else 1)        # bytes of one stored sample
    lane = sample * plan.info["frames_per_lane"]           # bytes of one lane's tap
    if plan.info["whole_rows"]:
        pattern = ("8 ds_read_b128 per lane, two 64-B binary16 rows in 128-B slots, bank-group order" if h16
                   else "16 ds_read_b128 per lane, two whole 128-B rows, bank-group order")
    else:
        pattern = ("two ds_read_b128 (16-byte lanes, split rows)" if lane == 16
                   else "two ds_read_b64 (8-byte lanes)" if lane == 8 else None)
    if pattern is None:
        return {"bytes_per_accumulation": 2 * sample, "lane_tap_bytes": lane, "lds_B_per_clk_per_cu": None,
                "ceiling_gacc_s": None}
    bclk = LDS_BCLK[pattern]
    return {"bytes_per_accumulation": 2 * sample, "lane_tap_bytes": lane, "read_pattern": pattern,
            "lds_B_per_clk_per_cu": bclk, "ceiling_gacc_s": CUS * SCLK_HZ * bclk / (2 * sample) / 1e9}


def oracle_rates(oracle, fields, cfg, rf_host, rx, tau, w, cap: int, threads: int):
    """The unmodified single-threaded oracle timed on the host: one depth slab
    prefix (1 thread), then `threads` threads on disjoint slabs of the same
    volume at once (the oracle releases the interpreter while it runs).
    Returns (voxels of the one-thread sample, its result, seconds, P-thread
    accumulations, P-thread seconds)."""
    import concurrent.futures as cf
    import numpy as np
    nx, ny, nz = cfg.grid
    per_vox = cfg.M * cfg.Q * cfg.B
    iz = nz // 2
    vox = np.arange(iz * nx * ny, (iz + 1) * nx * ny, dtype=np.int64)[:cap]
    t1 = time.perf_counter()
    ref = oracle.das_sum(fields, rf_host, rx, tau, w, voxels=vox)
    one_s = time.perf_counter() - t1
    # P threads, each a sample half as large, on other depth slabs
    share = max(1, cap // 2)
    slabs = [(iz + 1 + t) % nz for t in range(threads)]
    chunks = [np.arange(z * nx * ny, (z + 1) * nx * ny, dtype=np.int64)[:share] for z in slabs]
    t1 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda v: oracle.das_sum(fields, rf_host, rx, tau, w, voxels=v), chunks))
    multi_s = time.perf_counter() - t1
    return vox, ref, one_s, sum(c.size for c in chunks) * per_vox, multi_s


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="main", help="workload: tiny, mid, main, main-c64, large")
    ap.add_argument("--layout", default="qmkb", choices=["kqmb", "qmkb"],
                    help="permuted layout (QMKB: whole volumes in one chunk; KQMB: chunks under 4 GiB)")
    ap.add_argument("--algorithm", default="batch_inner", choices=["batch_inner", "baseline", "repack"])
    ap.add_argument("--q-chunk", type=int, default=0,
                    help="transmit events per permute/beamform pair (0: as many as the plan allows)")
    ap.add_argument("--streamed", action="store_true",
                    help="time das_beamform_streamed: each chunk's permute overlapped with the previous "
                         "chunk's beamform on a second stream (the kernel times still come from the "
                         "event-timed chunked pass)")
    ap.add_argument("--wide", action="store_true",
                    help="float64 samples (complex128 for IQ workloads): the baseline's fp64 path")
    ap.add_argument("--storage", default="native", choices=["native", "f16"],
                    help="samples in the permuted buffer: as given, or rounded to binary16 by the permute "
                         "(batch-inner; the arithmetic stays fp32)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-f16-compare", action="store_true",
                    help="skip the side line that times the same step with binary16 storage (native-storage "
                         "batch-inner runs only)")
    ap.add_argument("--cpu-voxels", type=int, default=0, help="oracle sample size (0: one depth slab)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the multi-core oracle rate (0: the host's cores available to this process, "
                         "at most 16)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of 1 GiB, three times (a kernel of known HBM bytes for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings), and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        a = torch.randn(1 << 28, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"copy calibration: 3 copies of {a.numel() * 4} bytes", file=sys.stderr)
        return

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the q-sharded multi-GPU design is described but not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import das_synth
    import volumetric_delay_sum_amd as das

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    das.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = das_synth.get_config(args.config)
    fields = das_synth.problem_fields(cfg)
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    rx = das_synth.array_positions(cfg)
    tau, w = das_synth.tx_tables(cfg)
    rf = das_synth.rf(cfg, device=dev)
    if args.wide:
        if args.algorithm != "baseline":
            print("bench.py: --wide runs the baseline algorithm (--algorithm baseline)", file=sys.stderr)
            sys.exit(2)
        rf = rf.double()                      # the same samples, held as float64
    rx_d = torch.from_numpy(rx).to(dev)
    tau_d = torch.from_numpy(tau).to(dev)
    w_d = torch.from_numpy(w).to(dev)

    h16 = args.storage == "f16"
    if h16 and (args.wide or args.algorithm == "baseline"):
        print("bench.py: --storage f16 is a batch-inner / repack option for fp32 / complex64 samples",
              file=sys.stderr)
        sys.exit(2)
    plan = das.plan_from_fields(fields, algorithm=args.algorithm, layout=args.layout, wide=args.wide,
                                storage=args.storage)
    out = torch.empty(plan.output_shape(), dtype=torch.float64 if args.wide else torch.float32, device=dev)
    bi = plan.permuted_input
    # events per das_permute / das_beamform pair (all Q unless the layout's
    # 32-bit offsets need chunks); chunks after the first accumulate into out
    qc = plan.max_q_chunk() if bi else cfg.Q
    if args.q_chunk > 0:
        qc = min(qc, args.q_chunk)
    chunks = [(q0, min(qc, cfg.Q - q0)) for q0 in range(0, cfg.Q, qc)]
    perm = torch.empty(plan.permuted_shape(qc), dtype=plan.permuted_dtype(), device=dev) if bi else None
    per_event = perm.numel() // qc if bi else 0
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        """ev: list of (start, mid, end) event triples, one per chunk."""
        for i, (q0, n) in enumerate(chunks):
            e = ev[i] if ev is not None else None
            if e is not None:
                e[0].record(stream)
            if bi:
                view = perm.view(-1)[: per_event * n]
                plan.permute(rf, view, q0, n, stream=stream)
            if e is not None:
                e[1].record(stream)
            plan.beamform(view if bi else rf, rx_d, tau_d, w_d, out, q0, n, accumulate=(i > 0), stream=stream)
            if e is not None:
                e[2].record(stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in chunks] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    perm_ms = [sum(e[0].elapsed_time(e[1]) for e in ev) for ev in events]
    kern_ms = [sum(e[1].elapsed_time(e[2]) for e in ev) for ev in events]
    launch_ms = [e[1].elapsed_time(e[2]) for ev in events for e in ev]
    print(f"[bench] timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    streamed_desc = ""
    if args.streamed:
        if not bi:
            print("bench.py: --streamed needs the batch-inner algorithm", file=sys.stderr)
            sys.exit(2)
        perm_b = torch.empty_like(perm)
        s_perm, s_beam = torch.cuda.Stream(dev), torch.cuda.Stream(dev)

        def streamed_step():
            plan.beamform_streamed(rf, rx_d, tau_d, w_d, out, perm, perm_b, qc,
                                   stream_permute=s_perm, stream_beamform=s_beam)

        for _ in range(max(1, args.warmup)):
            streamed_step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            streamed_step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        streamed_desc = ", streamed: permute of chunk c+1 on a second stream overlaps beamform of chunk c"
        print(f"[bench] streamed: {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    # The same step with binary16 storage, for comparison (not the metric: its
    # samples are rounded): permute into half the bytes, same kernels widening
    # the halves.  Timed like the steps above, after them.
    f16_compare = None
    if bi and not h16 and not plan.repack and not args.no_f16_compare and not args.streamed:
        plan16 = das.plan_from_fields(fields, algorithm=args.algorithm, layout=args.layout, storage="f16")
        perm16 = torch.empty(plan16.permuted_shape(qc), dtype=plan16.permuted_dtype(), device=dev)
        pe16 = perm16.numel() // qc
        out16 = torch.empty_like(out)

        def step16(e=None):
            for i, (q0, n) in enumerate(chunks):
                if e is not None:
                    e[i][0].record(stream)
                view16 = perm16.view(-1)[: pe16 * n]
                plan16.permute(rf, view16, q0, n, stream=stream)
                if e is not None:
                    e[i][1].record(stream)
                plan16.beamform(view16, rx_d, tau_d, w_d, out16, q0, n, accumulate=(i > 0), stream=stream)
                if e is not None:
                    e[i][2].record(stream)

        for _ in range(args.warmup):
            step16()
        torch.cuda.synchronize()
        ev16 = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in chunks] for _ in range(args.steps)]
        t16 = time.perf_counter()
        for i in range(args.steps):
            step16(ev16[i])
        torch.cuda.synchronize()
        wall16 = time.perf_counter() - t16
        k16 = float(np.mean([sum(e[1].elapsed_time(e[2]) for e in ev) for ev in ev16]))
        p16 = float(np.mean([sum(e[0].elapsed_time(e[1]) for e in ev) for ev in ev16]))
        ms16 = wall16 * 1e3 / args.steps
        f16_compare = {"ms_per_step": ms16, "kernel_ms_per_step": k16, "permute_ms": p16,
                       "value": das_synth.accumulations(cfg) / (ms16 * 1e-3) / 1e9,
                       "kernel_gacc_s": das_synth.accumulations(cfg) / (k16 * 1e-3) / 1e9,
                       "note": "the same step with binary16 samples in the permuted buffer (rounded by the "
                               "permute, widened to fp32 in the kernel), timed after the steps above; a "
                               "comparison, not the metric"}
        del perm16, out16
        print(f"[bench] binary16 storage: {args.steps} steps in {wall16:.3f} s", file=sys.stderr, flush=True)

    # the transmit-table generator on this workload's events (not part of a
    # step: the tables are inputs); HBM-write bound, 8 bytes per (event, voxel)
    if cfg.tx == "plane":
        tx_events = [(das.TX_PLANE, (0.0, 0.0, 1.0), 1.0)] * cfg.Q
    else:
        tx_events = [(das.TX_DIVERGING, (vx, vy, -cfg.src_depth), 1.0) for vx, vy in cfg.sources]
    tau_g, w_g = torch.empty_like(tau_d), torch.empty_like(w_d)
    plan.tx_tables(tx_events, tau_g, w_g, stream=stream)
    tx_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a, b in tx_ev:
        a.record(stream)
        plan.tx_tables(tx_events, tau_g, w_g, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    tx_ms = float(np.median([a.elapsed_time(b) for a, b in tx_ev]))
    tx_bytes = 8 * cfg.Q * cfg.N
    tx_tables = {"ms": tx_ms, "bytes": tx_bytes, "GB_s": tx_bytes / (tx_ms * 1e-3) / 1e9,
                 "hbm_frac": tx_bytes / (tx_ms * 1e-3) / 1e9 / 8000.0,
                 "launches": (cfg.Q + 15) // 16,
                 "matches_host_tables": bool(torch.equal(w_g, w_d)) and
                 int((tau_g.view(torch.int32) - tau_d.view(torch.int32)).abs().max().item()) <= 1}
    del tau_g, w_g

    accs = das_synth.accumulations(cfg)
    ms_step = wall * 1e3 / args.steps
    value = accs / (ms_step * 1e-3) / 1e9
    kern_avg = float(np.mean(kern_ms))              # beamform time per step (all chunks)
    launch_avg = float(np.mean(launch_ms))          # per beamform launch
    perm_avg = float(np.mean(perm_ms))
    flops_per_acc = 16 if cfg.iq else 4         # 2 FMA (real) or 8 FMA (complex) per accumulation
    achieved = accs * flops_per_acc / (kern_avg * 1e-3) / 1e12
    if plan.repack:
        kernel_name = "das_repack_kernel"
    elif bi:
        kernel_name = ("das_bi_rows_kernel" if plan.info["whole_rows"] else "das_bi_staged_kernel") \
            if plan.info["staged"] else "das_batch_inner_kernel"
    else:
        kernel_name = "das_baseline_f64_kernel" if args.wide else "das_baseline_kernel"
    peak = PEAK_FP64_TFLOPS if args.wide else PEAK_FP32_TFLOPS
    traffic = stored_traffic(kernel_name, cfg.name + ("-f16" if h16 else ""))
    # which roof binds: the algorithmic bytes of one launch (its samples, its
    # events' tables, the output read and written) at 8 TB/s against its flops
    # at the vector peak; then the same with the HBM bytes the counters saw
    q_l = chunks[0][1]
    in_bytes = (perm.numel() * perm.element_size() * q_l // qc) if bi else rf.numel() * rf.element_size() * q_l // cfg.Q
    out_bytes = out.numel() * out.element_size()
    alg_bytes = in_bytes + 8 * q_l * cfg.N + 2 * out_bytes
    launch_flops = accs * flops_per_acc * q_l / cfg.Q
    t_hbm, t_alu = alg_bytes / (PEAK_HBM_GBS * 1e9), launch_flops / (peak * 1e12)
    hbm_frac_measured = traffic / (launch_avg * 1e-3) / (PEAK_HBM_GBS * 1e9) if traffic else None
    valu_busy = stored_counter(kernel_name, cfg.name + ("-f16" if h16 else ""), "valu_busy")
    bound = pick_bound(t_hbm, t_alu, hbm_frac_measured, valu_busy)
    bound_basis = {"algorithmic_bytes_per_launch": alg_bytes, "hbm_time_ms_at_peak": t_hbm * 1e3,
                   "alu_time_ms_at_peak": t_alu * 1e3,
                   "hbm_frac_from_counters": hbm_frac_measured,
                   "valu_busy_from_counters": valu_busy,
                   "rule": "hbm if the launch's algorithmic bytes at 8 TB/s take longer than its flops at the "
                           "vector peak, or if the counted HBM bytes per launch time, as a fraction of 8 TB/s, "
                           "exceed the VALU busy fraction (VALUBusy) the counters read on the same sources; "
                           "else alu"}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        nx, ny, nz = cfg.grid
        # bounded samples: about 8e8 accumulations single-threaded (some 17 s on the host), then half
        # that on each of P threads, unless asked otherwise
        cap = args.cpu_voxels or max(1, int(8e8 // (cfg.M * cfg.Q * cfg.B)))
        threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
        print(f"[bench] cpu baseline: oracle on {min(cap, nx * ny)} voxels, then {threads} threads",
              file=sys.stderr, flush=True)
        rf_host = rf.cpu().numpy()
        if h16:
            rf_host = oracle.to_binary16(rf_host)      # the samples the kernel reads
        vox, ref, cpu_s, multi_acc, multi_s = oracle_rates(oracle, fields, cfg, rf_host, rx, tau, w, cap, threads)
        cpu_acc = vox.size * cfg.M * cfg.Q * cfg.B
        y = out.cpu().numpy().astype(np.float64)
        y = (y[..., 0] + 1j * y[..., 1]) if cfg.iq else y
        y = y[:, vox]
        comps = [(y.real, ref.real), (y.imag, ref.imag)] if cfg.iq else [(y, ref)]
        parity = [(float(np.abs(g - r).max() / np.abs(r).max()), float(np.linalg.norm(g - r) / np.linalg.norm(r)))
                  for g, r in comps]
        iz = nz // 2
        cpu = {"value": multi_acc / multi_s / 1e9, "unit": "G acc/s", "cores": threads, "kind": "oracle",
               "sample": f"{cfg.name}: {threads} threads, each the single-threaded fp64 C oracle on its own depth "
                         f"slab ({max(1, cap // 2)} voxels x all {cfg.Q} events x {cfg.M} receivers x {cfg.B} "
                         f"frames), {multi_acc:.3e} accumulations in {multi_s:.1f} s"
                         + (" of the binary16-rounded samples" if h16 else ""),
               "one_core": {"value": cpu_acc / cpu_s / 1e9, "cores": 1,
                            "sample": f"depth slab iz={iz} ({vox.size} voxels), {cpu_acc:.3e} accumulations "
                                      f"in {cpu_s:.1f} s"},
               "gpu_parity_on_sample": {"max_rel": max(p[0] for p in parity), "l2_rel": max(p[1] for p in parity)}}

    info = plan.info
    if bi and not plan.repack:
        executed = executed_fraction(cfg, info)
    elif not bi:
        executed = executed_fraction_baseline(cfg)
    else:
        executed = executed_fraction_repack(cfg, 4 if cfg.B % 64 == 0 else 8)
    delivery = delivery_ceiling(plan, cfg.iq, h16) if not args.wide else None
    if delivery and delivery.get("ceiling_gacc_s"):
        kg = accs / (kern_avg * 1e-3) / 1e9
        delivery["achieved_gacc_s"] = kg
        delivery["frac"] = kg / delivery["ceiling_gacc_s"]
        delivery["alu_ceiling_gacc_s"] = peak * 1e12 / flops_per_acc / 1e9
        delivery["executed_frac"] = kg * executed / delivery["ceiling_gacc_s"]
    rec = {
        "metric": "G voxel·receiver·transmit·frame accumulations/s (fp32), % of bounding roofline",
        "value": value,
        "unit": "G acc/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("c128" if cfg.iq else "f64") if args.wide else ("c64" if cfg.iq else "f32"),
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: {cfg.grid[0]}x{cfg.grid[1]}x{cfg.grid[2]} voxels, "
                         f"{cfg.array[0]}x{cfg.array[1]} array (M={cfg.M}), Q={cfg.Q} "
                         f"{'plane' if cfg.tx == 'plane' else 'diverging'} waves, K={cfg.K}, B={cfg.B}, "
                         + ((f"{'complex128 IQ' if cfg.iq else 'fp64 RF'}") if args.wide else
                            (f"{'complex64 IQ' if cfg.iq else 'fp32 RF'}"))),
            "step": ((f"das_permute + das_beamform (batch-inner, layout {args.layout.upper()}"
                      f", {len(chunks)} chunk(s) of <= {qc} events{streamed_desc})") if bi
                     else "das_beamform (baseline)"),
            "accumulations_per_step": accs,
            "frames_per_lane": info["frames_per_lane"],
            "storage": ("binary16 samples in the permuted buffer (rounded by the permute, widened to fp32 "
                        "in the kernel)") if h16 else "samples as given",
        },
        "value_basis": "whole steps (permute + beamform) per second of wall time, inputs resident in HBM",
        "kernel_value": accs / (kern_avg * 1e-3) / 1e9,
        "roofline": {
            "bound": bound,
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": traffic,
            "kernel": kernel_name,
            "kernel_ms_per_step": kern_avg,
            "kernel_basis": ("HIP events around each das_beamform call on the bench stream: for whole-row "
                             "plans the tile-order pass (rows_cost_kernel, rows_order_kernel) and the beamform "
                             "kernel"),
            "kernel_ms_per_launch": launch_avg,
            "launches_per_step": len(chunks),
            "kernel_gacc_s": accs / (kern_avg * 1e-3) / 1e9,
            "flops_per_accumulation": flops_per_acc,
            "bound_basis": bound_basis,
            "delivery": delivery,
            "mfma": repack_mfma(cfg, plan, h16, launch_avg, len(chunks), q_l, executed) if plan.repack else None,
            "executed": {"fraction_of_terms": executed, "tflops": achieved * executed,
                         "frac": achieved * executed / peak,
                         "note": ("achieved and frac count every term of the sum; the kernel skips the "
                                  + ("receivers outside all the apertures of a wave's 8 x 8 voxels"
                                     if not bi else "receivers outside each tile's receive aperture")
                                  + " (exact zeros), so it executes this fraction of them, at this rate")
                                 if executed < 1.0 else "the kernel executes every term"},
        },
        "permute_ms": perm_avg if bi else None,
        "binary16_storage": f16_compare,
        "tx_tables": tx_tables,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
