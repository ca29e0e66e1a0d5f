"""Benchmark of the block-scaled small-M decode GEMV on one MI355X.

One step = one qgemv_run_ws call (dispatch + kernel) over one batch of synthetic
input: Y[M, N] = A[M, K] . dequant(W)^T, with a workspace allocated and zeroed once
before the timed region (plans that split K across workgroups use it, others ignore
it; --no-workspace times qgemv_run instead). The weights are cold: the timed loop rotates
through enough copies of the weight (>= 1 GiB together, several times the 256 MB
last-level cache) that every call streams its weight from HBM. Inputs are resident in
HBM before the timed region starts.

Prints one JSON line. `value` is achieved GB/s = weight bytes (codes + block scales +
zero points) per call / average time per call. The roofline object reports the same
bytes against the 8 TB/s HBM peak; its `traffic` is the HBM bytes per launch that two
rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE) measured for this workload, read from
the summaries under profiles/ and only while the built kernels still hash to what
was profiled (null otherwise). `cpu_baseline` times the CPU oracle on a bounded sample
of the same workload on this host.

Profiling helpers (no GPU needed):
  --calib-copy-mib X      also run one plain copy kernel of X MiB (torch.neg on fp32)
                          before the warmup, so a counter run can scale its readings
  --trace-summary DIR     per-kernel durations from a rocprofv3 --kernel-trace database
  --traffic-record F W    FETCH_SIZE run dir F and WRITE_SIZE run dir W -> traffic record
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sqlite3
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "u8_m1_k4096_n4096"
HBM_PEAK_GBS = 8000.0
COLD_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--shape", default=None, metavar="FMT:ACT:N:K:BS",
                   help="time an arbitrary shape instead of a named workload (e.g. fp8:f16:8192:4096:128), "
                        "drawn by synth.make_problem with its default value distributions")
    p.add_argument("--seed", type=int, default=7, help="seed for --shape")
    p.add_argument("--m", type=int, default=None, help="rows of A (default: the workload's first M; 1 for --shape)")
    p.add_argument("--flags", type=int, default=0, help="qgemv_desc.flags (force a family, K split)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time for the oracle sample")
    p.add_argument("--warm", action="store_true", help="reuse one weight copy (cache-warm; not the metric)")
    p.add_argument("--bias", action="store_true", help="add the optional per-column bias (fused epilogue)")
    p.add_argument("--no-workspace", action="store_true",
                   help="time qgemv_run (no workspace: K is never split across workgroups)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="run one plain copy kernel of this many MiB before the warmup (counter calibration)")
    p.add_argument("--trace-summary", metavar="DIR", default=None)
    p.add_argument("--traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None)
    return p.parse_args()


# ----------------------------------------------------------------------------------
# rocprofv3 databases (rocpd SQLite) -> short text summaries


def _elf_section(path, name):
    """Bytes of section `name` of a 64-bit little-endian ELF file (plain header walk)."""
    import struct

    with open(path, "rb") as fh:
        data = fh.read()
    if data[:4] != b"\x7fELF" or data[4] != 2 or data[5] != 1:
        raise ValueError(f"{path}: not a 64-bit little-endian ELF file")
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)

    def sh(i):
        name_off, _, _, _, off, size = struct.unpack_from("<IIQQQQ", data, shoff + i * shentsize)
        return name_off, off, size

    _, str_off, _ = sh(shstrndx)
    for i in range(shnum):
        name_off, off, size = sh(i)
        end = data.index(b"\0", str_off + name_off)
        if data[str_off + name_off:end].decode() == name:
            return data[off:off + size]
    raise ValueError(f"{path}: no section {name}")


def kernel_source_hash() -> str:
    """Hash of the built library's device code (its `.hip_fatbin` section: every
    gfx950 kernel, nothing of the host side): a traffic figure is valid only for the
    kernels it was measured on, and stays valid across host-only changes."""
    lib = os.path.join(ROOT, "block_quantized_weight_amd", "libqgemv.so")
    return hashlib.sha256(_elf_section(lib, ".hip_fatbin")).hexdigest()[:16]


def _dbs(d):
    out = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not out:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return out


def trace_durations(d):
    """{kernel name: [durations in ns]} from --kernel-trace databases under d."""
    res = {}
    for db in _dbs(d):
        con = sqlite3.connect(db)
        for name, start, end in con.execute("select name, start, end from kernels"):
            res.setdefault(name, []).append(end - start)
        con.close()
    return res


def counter_means(d):
    """{kernel name: {counter: (mean per dispatch, dispatches)}} from --pmc databases."""
    acc = {}
    for db in _dbs(d):
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, counter_name, value from counters_collection").fetchall()
        con.close()
        for name, ctr, v in rows:
            acc.setdefault(name, {}).setdefault(ctr, []).append(float(v))
    return {k: {c: (sum(v) / len(v), len(v)) for c, v in cs.items()} for k, cs in acc.items()}


def print_trace_summary(d):
    rows = sorted(trace_durations(d).items(), key=lambda kv: -sum(kv[1]))
    tot = sum(sum(v) for _, v in rows) or 1
    print(f"{'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9} {'time %':>7}  kernel")
    for name, v in rows:
        print(f"{len(v):6d} {sum(v) / len(v) / 1e3:9.3f} {min(v) / 1e3:9.3f} {max(v) / 1e3:9.3f} "
              f"{100.0 * sum(v) / tot:7.2f}  {name}")


def _is_qgemv(name):
    return "qgemv::" in name


def _is_calib(name):
    return "neg" in name.lower()


def traffic_record(fetch_dir, write_dir, args):
    """Scale the qgemv kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch, as the
    counters report them) by what the same counters read for the calibration copy
    kernel, whose true traffic is known (it reads and writes X MiB)."""
    if args.calib_copy_mib <= 0:
        raise SystemExit("--traffic-record needs --calib-copy-mib (the size the runs used)")
    from block_quantized_weight_amd import synth

    true_bytes = args.calib_copy_mib * (1 << 20)
    M = args.m if args.m is not None else synth.WORKLOADS[args.workload]["ms"][0]
    rec = {"workload": args.workload, "M": M, "flags": args.flags, "ws": not args.no_workspace,
           "src_hash": kernel_source_hash(), "calib_bytes": true_bytes}
    for key, d, ctr in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        cm = counter_means(d)
        q = [(k, v[ctr]) for k, v in cm.items() if _is_qgemv(k) and ctr in v]
        c = [(k, v[ctr]) for k, v in cm.items() if _is_calib(k) and ctr in v]
        if len(q) != 1 or len(c) != 1:
            raise SystemExit(f"{ctr}: expected one qgemv kernel and one calibration kernel, got {q} / {c}")
        (qk, (qv, qn)), (ck, (cv, cn)) = q[0], c[0]
        factor = true_bytes / cv  # bytes per counter unit
        rec[key] = {"kernel": qk, "counter_kib": round(qv, 3), "dispatches": qn,
                    "calib_counter_kib": round(cv, 3), "bytes_per_unit": round(factor, 4),
                    "bytes": round(qv * factor)}
        rec["calib_kernel"] = ck.split("(")[0][:60] + " (torch.neg, fp32)"
    rec["traffic_bytes"] = rec["fetch"]["bytes"] + rec["write"]["bytes"]
    print("traffic_record: " + json.dumps(rec, sort_keys=True))


def lookup_traffic(workload, M, flags, ws=True):
    """HBM bytes per launch from a committed counter summary, or None when there is
    none for this workload and entry point or the built kernels changed since it was
    taken."""
    want = kernel_source_hash()
    for f in sorted(glob.glob(os.path.join(PROFILES, "*.md")) + glob.glob(os.path.join(PROFILES, "*.txt"))):
        with open(f) as fh:
            for line in fh:
                if not line.startswith("traffic_record: "):
                    continue
                try:
                    rec = json.loads(line[len("traffic_record: "):])
                except ValueError:
                    continue
                if (rec.get("workload"), rec.get("M"), rec.get("flags"), rec.get("ws", False), rec.get("src_hash")) == \
                        (workload, M, flags, ws, want):
                    return rec["traffic_bytes"]
    return None


def cpu_baseline(prob, M, target_s):
    """Time the CPU oracle (as it stands) on a bounded column sample of the workload."""
    import numpy as np

    import oracle
    from block_quantized_weight_amd import synth

    # pick a column count that takes roughly target_s, after a short calibration
    ncal = min(prob.N, 256)
    sub = synth.Problem(**{**prob.__dict__, "N": ncal, "W": prob.W[:ncal], "scales": prob.scales[:ncal],
                           "zp": None if prob.zp is None else prob.zp[:ncal]})
    t0 = time.perf_counter()
    oracle.gemv(sub, M=M)
    dt = max(time.perf_counter() - t0, 1e-4)
    ncols = int(min(prob.N, max(ncal, ncal * target_s / dt)))
    reps = max(1, int(math.ceil(ncal * target_s / dt / max(ncols, 1))))
    sub = synth.Problem(**{**prob.__dict__, "N": ncols, "W": prob.W[:ncols], "scales": prob.scales[:ncols],
                           "zp": None if prob.zp is None else prob.zp[:ncols]})
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.gemv(sub, M=M)
    el = (time.perf_counter() - t0) / reps
    bytes_per_col = prob.weight_bytes() / prob.N
    return {"value": round(bytes_per_col * ncols / el / 1e9, 6), "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{ncols} of {prob.N} columns x {reps} repetition(s), M={M}, fp64 plain loops, "
                      f"{el * 1e3:.1f} ms per sample pass"}


def main():
    args = parse()
    if args.trace_summary:
        print_trace_summary(args.trace_summary)
        return
    if args.traffic_record:
        traffic_record(*args.traffic_record, args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the weight would be split by "
              "output columns, one shard per GPU, with no communication in the product). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_quantized_weight_amd as bqw
    from block_quantized_weight_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.shape:
        fmt, act, n_s, k_s, bs_s = args.shape.split(":")
        M = args.m if args.m is not None else 1
        prob = synth.make_problem(fmt, act, int(n_s), int(k_s), int(bs_s), M, args.seed, name="shape",
                                  ms=(M,), with_bias=args.bias)
        workload = f"shape_{fmt}_{act}_n{n_s}_k{k_s}_bs{bs_s}"
        seed = args.seed
    else:
        prob = synth.workload(args.workload, with_bias=args.bias)
        M = args.m if args.m is not None else prob.ms[0]
        workload = args.workload
        seed = synth.WORKLOADS[args.workload]["seed"]
    wbytes = prob.weight_bytes()
    copies = 1 if args.warm else max(2, int(math.ceil(COLD_BYTES / wbytes)))

    # device buffers: one copy of each input per rotation slot
    def dev_t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    W0 = dev_t(prob.W)
    S0 = dev_t(prob.scales if prob.scales.dtype == np.float32 else prob.scales.view(np.uint8))
    Z0 = None if prob.zp is None else dev_t(prob.zp)
    tdt = torch.float16 if prob.act == "f16" else torch.bfloat16
    A = dev_t(prob.A[:M].view(np.int16)).view(tdt).contiguous()
    bias = None if prob.bias is None else dev_t(prob.bias.view(np.int16)).view(tdt)
    Y = torch.empty((M, prob.N), dtype=tdt, device=dev)
    slots = []
    for i in range(copies):
        W = W0 if i == 0 else W0.clone()
        S = S0 if i == 0 else S0.clone()
        Z = Z0 if (i == 0 or Z0 is None) else Z0.clone()
        q = bqw.QGemv(prob.fmt, prob.act, prob.N, prob.K, prob.bs, W, S, Z, prob.tensor_scale, args.flags,
                      bias=bias)
        slots.append((q, W, S, Z))
    use_ws = not args.no_workspace
    plan = slots[0][0].plan(M, with_workspace=use_ws)
    # one workspace for every rotation slot (their plans are the same), zeroed once
    ws = torch.zeros(max(256, plan["workspace_bytes"]), dtype=torch.uint8, device=dev) if use_ws else None
    stream = torch.cuda.current_stream()
    if args.calib_copy_mib > 0:
        # one plain copy kernel of known size, for scaling counter readings
        csrc = torch.ones(args.calib_copy_mib * (1 << 18), dtype=torch.float32, device=dev)
        cdst = torch.empty_like(csrc)
        torch.cuda.synchronize()
        torch.neg(csrc, out=cdst)
        torch.cuda.synchronize()
        del csrc, cdst
    torch.cuda.synchronize()

    for i in range(args.warmup):
        slots[i % copies][0].run(A, Y, M, stream, workspace=ws)
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        slots[i % copies][0].run(A, Y, M, stream, workspace=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    ms_per = ms_total / args.steps
    gbs = wbytes / (ms_per * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(prob, M, args.cpu_seconds)

    out = {
        "metric": "achieved HBM GB/s (weight bytes / kernel time), cold weights",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per, 6),
        "us_per_call": round(ms_per * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{prob.fmt} x {prob.act} -> f32 acc",
        "data": "synthetic",
        "config": {"workload": workload, "format": prob.fmt, "act": prob.act, "M": M, "N": prob.N,
                   "K": prob.K, "block_size": prob.bs, "weight_bytes": wbytes, "cold_copies": copies,
                   "plan": plan, "flags": args.flags, "seed": seed, "bias": bool(args.bias),
                   "entry": "qgemv_run_ws" if use_ws else "qgemv_run"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if args.shape else lookup_traffic(args.workload, M, args.flags, use_ws)},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 4),
    }
    for q, *_ in slots:
        q.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
