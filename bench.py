"""Benchmark of the block-scaled small-M decode GEMV on one MI355X.

One step = one qgemv_run_ws call (dispatch + kernel) over one batch of synthetic
input: Y[M, N] = A[M, K] . dequant(W)^T, with a workspace allocated and zeroed once
before the timed region (plans that split K across workgroups use it, others ignore
it; --no-workspace times qgemv_run instead). The weights are cold: the timed loop
rotates through R copies of the weight (R * weight bytes >= 1 GiB, four times the
256 MB last-level cache; R <= 4096, copies held in one device buffer per array), and
the rotation continues from the warmup, so every call streams a weight last touched
at least 1 GiB of traffic earlier (310 MB for the 75 KB tiny case, still past the
cache). Inputs are resident in HBM before the timed region starts. Before the W warmup
calls of every timed loop, untimed calls run in synchronized chunks until --settle-ms
(default 100) of wall time have passed, the rotation continuing through them: from
idle the GPU needs some 30 ms of load (about 500 calls of the 4-bit lm_head) before a
call settles at its steady time, and the first hundred run some 15% slower, so a
short warmup alone would time the clocks' ramp, not the kernel.

The default workload is the 4-bit lm_head (K = 4096, N = 151936, bf16): `value` is its
achieved GB/s at M = 1 = weight bytes (codes + block scales + zero points) per call /
average time per call; the same line carries the M sweep 1, 2, 4, 8, 16 of that weight
(us/call, GB/s, t(M)/t(1), plan), then every other named workload timed the same way
(`extra_workloads`: the FP8 5120 x 6144 projection at M = 1, 4, 8, the 8-bit 4096 x 4096
weight at M = 1, the NVFP4 lm_head at M = 1 and 4, NVFP4 2048 x 2048 at M = 4, the 4-bit
1024 x 2048 split-K case at M = 8 and the tiny 4-bit case at M = 1), each with the plain
read control of its own weight bytes unless --no-read-control.
`roofline` reports the M = 1 figure against the 8 TB/s HBM peak and against a plain
streaming read of the same bytes (the control kernel in libreadctl.so, timed with the
same cold rotation); its `traffic` is the HBM bytes per launch that two rocprofv3
counter runs (FETCH_SIZE, WRITE_SIZE) measured for this workload, read from the
summaries under profiles/ and only while the built kernels still hash to what was
profiled (null otherwise). `cpu_baseline` times the CPU oracle on a bounded sample of
the same workload on this host, on all threads and on one.

Profiling helpers (no GPU needed):
  --calib-copy-mib X      also run one plain copy kernel of X MiB (torch.neg on fp32)
                          before the warmup, so a counter run can scale its readings
  --trace-summary DIR     per-kernel durations from a rocprofv3 --kernel-trace database
                          (with --steps K, also each kernel's mean over its last K
                          launches: the timed calls of a profiled bench run)
  --counter-summary DIR   per-kernel counter means per dispatch from a rocprofv3 --pmc database
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

DEFAULT_WORKLOAD = "u4_k4096_n151936"
# second workload of the default line: the FP8 projection at the metric's M = 1, 4, 8
# the other named workloads, each at its own row counts (the NVFP4 lm_head also at M = 1)
EXTRA_WORKLOADS = (("fp8_k6144_n5120", (1, 4, 8)), ("u8_m1_k4096_n4096", (1,)), ("nvfp4_m4_k2048_n248320", (1, 4)),
                   ("nvfp4_m4_k2048_n2048", (4,)), ("u4_m8_k2048_n1024", (8,)), ("u4_m1_k512_n256", (1,)))
METRIC = "achieved HBM GB/s (weight bytes/kernel time) and us/call at M=1,4,8"
HBM_PEAK_GBS = 8000.0
COLD_BYTES = 1 << 30
MAX_COPIES = 4096
PROFILES = os.path.join(ROOT, "profiles")
READ_CONTROL_LIB = os.path.join(ROOT, "block_quantized_weight_amd", "libreadctl.so")


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--settle-ms", type=float, default=100.0,
                   help="untimed calls before each timed loop's warmup, in synchronized chunks, until this "
                        "much wall time has passed (the GPU clocks' ramp from idle; 0 = none)")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--shape", default=None, metavar="FMT:ACT:N:K:BS",
                   help="time an arbitrary shape instead of a named workload (e.g. fp8:f16:8192:4096:128), "
                        "drawn by synth.make_problem with its default value distributions")
    p.add_argument("--seed", type=int, default=7, help="seed for --shape")
    p.add_argument("--m", type=int, default=None,
                   help="rows of A (default: the workload's M sweep, the first M as the headline; 1 for --shape)")
    p.add_argument("--no-extra", action="store_true", help="skip the other named workloads' lines")
    p.add_argument("--no-read-control", action="store_true", help="skip the plain streaming read control")
    p.add_argument("--no-tune", dest="tune", action="store_false",
                   help="skip qgemv_tune (by default each M is also tuned and the kept launch timed cold)")
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
    p.add_argument("--counter-summary", metavar="DIR", default=None)
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
    """{kernel name: [durations in ns], in launch order} from --kernel-trace databases
    under d."""
    rows = []
    for db in _dbs(d):
        con = sqlite3.connect(db)
        rows += con.execute("select name, start, end from kernels").fetchall()
        con.close()
    res = {}
    for name, start, end in sorted(rows, key=lambda r: r[1]):
        res.setdefault(name, []).append(end - start)
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


def print_counter_summary(d):
    """One line per qgemv kernel: each counter's mean per dispatch."""
    for name, cs in sorted(counter_means(d).items()):
        if _is_qgemv(name):
            n = max(x[1] for x in cs.values())
            vals = ", ".join(f"{c} {v[0]:.1f}" for c, v in sorted(cs.items()))
            print(f"{name}: {vals} ({n} dispatches)")


def print_trace_summary(d, last=0):
    """One line per kernel: launches, mean / min / max duration, share of the time;
    with last > 0 also the mean over the kernel's last `last` launches."""
    rows = sorted(trace_durations(d).items(), key=lambda kv: -sum(kv[1]))
    tot = sum(sum(v) for _, v in rows) or 1
    tail = f" {'last ' + str(last):>9}" if last else ""
    print(f"{'calls':>6} {'avg us':>9} {'min us':>9} {'max us':>9}{tail} {'time %':>7}  kernel")
    for name, v in rows:
        t = f" {sum(v[-last:]) / len(v[-last:]) / 1e3:9.3f}" if last else ""
        print(f"{len(v):6d} {sum(v) / len(v) / 1e3:9.3f} {min(v) / 1e3:9.3f} {max(v) / 1e3:9.3f}{t} "
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _sub_problem(prob, ncols):
    from block_quantized_weight_amd import synth

    return synth.Problem(**{**prob.__dict__, "N": ncols, "W": prob.W[:ncols], "scales": prob.scales[:ncols],
                            "zp": None if prob.zp is None else prob.zp[:ncols],
                            "bias": None if prob.bias is None else prob.bias[:ncols]})


def _time_oracle(prob, M, target_s, nthreads):
    """(GB/s of weight, columns, repetitions, seconds per pass) of the oracle on a column
    sample sized to take about target_s."""
    import oracle

    ncal = min(prob.N, 256 if nthreads != 1 else 32)
    t0 = time.perf_counter()
    oracle.gemv(_sub_problem(prob, ncal), M=M, nthreads=nthreads)
    dt = max(time.perf_counter() - t0, 1e-4)
    ncols = int(min(prob.N, max(ncal, ncal * target_s / dt)))
    reps = max(1, int(math.ceil(ncal * target_s / dt / max(ncols, 1))))
    sub = _sub_problem(prob, ncols)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.gemv(sub, M=M, nthreads=nthreads)
    el = (time.perf_counter() - t0) / reps
    return prob.weight_bytes() / prob.N * ncols / el / 1e9, ncols, reps, el


def cpu_baseline(prob, M, target_s):
    """Time the CPU oracle (as it stands) on a bounded column sample of the workload: on
    all host threads (the reported value) and on one thread."""
    import oracle

    nt = oracle.max_threads()
    gbs, ncols, reps, el = _time_oracle(prob, M, target_s, nt)
    gbs1, ncols1, reps1, el1 = _time_oracle(prob, M, max(target_s / 2, 0.05), 1)
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": nt, "kind": "oracle",
            "sample": f"{ncols} of {prob.N} columns x {reps} repetition(s), M={M}, fp64 plain loops, "
                      f"{el * 1e3:.1f} ms per sample pass",
            "single_thread": {"value": round(gbs1, 6), "unit": "GB/s", "cores": 1,
                              "sample": f"{ncols1} columns x {reps1} repetition(s), {el1 * 1e3:.1f} ms per pass"},
            "cpu_model": cpu_model(), "host_threads": os.cpu_count()}


class Rotation:
    """R cold copies of a problem's weight arrays, each array's copies in one device
    buffer, and one handle per copy (R * weight bytes >= COLD_BYTES, R <= MAX_COPIES)."""

    def __init__(self, prob, flags, dev, warm=False):
        import numpy as np
        import torch

        import block_quantized_weight_amd as bqw

        wbytes = prob.weight_bytes()
        self.copies = 1 if warm else int(min(MAX_COPIES, max(2, math.ceil(COLD_BYTES / wbytes))))
        R = self.copies

        def rep(a):
            t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            buf = torch.empty((R,) + tuple(t.shape), dtype=t.dtype, device=dev)
            buf[0].copy_(t)
            if R > 1:
                buf[1:].copy_(t.unsqueeze(0).expand((R - 1,) + tuple(t.shape)))
            return buf

        self.W = rep(prob.W)
        self.S = rep(prob.scales if prob.scales.dtype == np.float32 else prob.scales.view(np.uint8))
        self.Z = None if prob.zp is None else rep(prob.zp)
        tdt = torch.float16 if prob.act == "f16" else torch.bfloat16
        self.bias = None if prob.bias is None else \
            torch.from_numpy(prob.bias.view(np.int16)).to(dev).view(tdt)
        self.tensor_scale = prob.tensor_scale
        self.handles = [bqw.QGemv(prob.fmt, prob.act, prob.N, prob.K, prob.bs, self.W[i], self.S[i],
                                  None if self.Z is None else self.Z[i], prob.tensor_scale, flags, bias=self.bias)
                        for i in range(R)]

    def handle_with(self, flags, i=0):
        """A handle on weight copy i with other descriptor flags."""
        import block_quantized_weight_amd as bqw

        h0 = self.handles[0]
        return bqw.QGemv(h0.fmt, h0.act, h0.N, h0.K, h0.block_size, self.W[i], self.S[i],
                         None if self.Z is None else self.Z[i], self.tensor_scale, flags, bias=self.bias)

    def close(self):
        for q in self.handles:
            q.close()


def settle(call, settle_ms, chunk=32):
    """Untimed call(i), i = 0, 1, ..., in chunks of `chunk` each followed by a device
    synchronize, until settle_ms of wall time have passed (so the host never runs far
    ahead of the GPU). Returns the number of calls made."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(chunk):
            call(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_calls(hs, A, Y, M, stream, ws, warmup, steps, settle_ms=0.0):
    """(ms per call from HIP events on the launch stream, wall seconds of the timed
    loop), the calls rotating over the handles hs (one per weight copy). Settle calls
    (settle_ms), then the warmup, then the timed loop: the rotation runs on through
    all three."""
    import torch

    R = len(hs)

    def call(i):
        hs[i % R].run(A, Y, M, stream, workspace=ws)

    i0 = settle(call, settle_ms)
    for i in range(i0, i0 + warmup):
        call(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(i0 + warmup, i0 + warmup + steps):
        call(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0


READ_CONTROL_SHAPES = ((2048, 4), (4096, 4), (4096, 8), (8192, 4), (8192, 8), (16384, 4), (32768, 4), (65536, 4), (131072, 4),
                       (2048, 16))


def time_read_control(nbytes, dev, stream, warmup, steps, settle_ms=0.0):
    """The plain streaming read of nbytes, cold like the GEMV (settle calls and warmup
    as for the GEMV, the rotation continuing into the timed loop), for each (workgroups, loads in flight per
    lane) of READ_CONTROL_SHAPES: the fastest, as the control is a ceiling. Returns
    (ms per read, GB/s, shape, {shape: GB/s})."""
    import ctypes

    import torch

    if not os.path.exists(READ_CONTROL_LIB):
        raise SystemExit(f"{READ_CONTROL_LIB} is missing: build with block_quantized_weight_amd.build.build()")
    L = ctypes.CDLL(READ_CONTROL_LIB)
    L.read_control.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                               ctypes.c_void_p, ctypes.c_void_p]
    L.read_control.restype = ctypes.c_int
    nb = (nbytes + 15) // 16 * 16
    R = int(min(MAX_COPIES, max(2, math.ceil(COLD_BYTES / nb))))
    buf = torch.randint(0, 255, (R, nb), dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    never = 0x9E3779B9  # the xor fold of random bytes lands here with probability 2^-32
    best, table = None, {}
    for blocks, unroll in READ_CONTROL_SHAPES:
        def go(i):
            rc = L.read_control(buf[i % R].data_ptr(), nb, blocks, unroll, never, sink.data_ptr(), stream.cuda_stream)
            if rc:
                raise RuntimeError(f"read control launch failed ({rc})")

        i0 = settle(go, settle_ms)
        for i in range(i0, i0 + warmup):
            go(i)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(i0 + warmup, i0 + warmup + steps):
            go(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        gbs = nb / (ms * 1e-3) / 1e9
        table[f"{blocks}x256 threads, {unroll} loads"] = round(gbs, 1)
        if best is None or ms < best[0]:
            best = (ms, gbs, (blocks, unroll))
    del buf
    return best[0], best[1], best[2], table


def tuned_calls(rot, A, Y, M, stream, ws, args, wbytes, auto_ms):
    """qgemv_tune on the first copy's handle (it times every call cold, after a cache
    sweep), then the kept flags timed like the automatic plan, over the same copies."""
    q = rot.handle_with(args.flags)
    info = q.tune(A, Y, M=M, with_workspace=ws is not None, workspace=ws)
    f = info["chosen_flags"]
    res = {"flags": hex(f), "candidates": info["candidates"], "probe_auto_us": round(info["auto_us"], 3),
           "probe_chosen_us": round(info["chosen_us"], 3), "plan": q.plan(M, with_workspace=ws is not None)}
    if f == 0:
        msc = auto_ms  # the automatic launch was kept: its cold time stands
    else:
        hs = [rot.handle_with(args.flags | f, i) for i in range(rot.copies)]
        msc, _ = time_calls(hs, A, Y, M, stream, ws, args.warmup, args.steps, args.settle_ms)
        for h in hs:
            h.close()
    q.close()
    res["us_per_call"] = round(msc * 1e3, 3)
    res["gbs"] = round(wbytes / (msc * 1e-3) / 1e9, 2)
    return res


def measure(prob, ms, args, dev, stream):
    """Time the problem at every M in ms: {M: {...}} plus the rotation size."""
    import torch

    rot = Rotation(prob, args.flags, dev, warm=args.warm)
    tdt = torch.float16 if prob.act == "f16" else torch.bfloat16
    import numpy as np

    A_all = torch.from_numpy(prob.A.view(np.int16)).to(dev).view(tdt)
    use_ws = not args.no_workspace
    wbytes = prob.weight_bytes()
    out = {}
    ws = None
    for M in ms:
        plan = rot.handles[0].plan(M, with_workspace=use_ws)
        if use_ws and (ws is None or ws.numel() < plan["workspace_bytes"]):
            ws = torch.zeros(max(256, plan["workspace_bytes"]), dtype=torch.uint8, device=dev)
        A = A_all[:M].contiguous()
        Y = torch.empty((M, prob.N), dtype=tdt, device=dev)
        msc, wall = time_calls(rot.handles, A, Y, M, stream, ws if use_ws else None, args.warmup, args.steps,
                               args.settle_ms)
        out[M] = {"us_per_call": round(msc * 1e3, 3), "gbs": round(wbytes / (msc * 1e-3) / 1e9, 2),
                  "ms_per_step": msc, "wall_s": round(wall, 4), "plan": plan}
        if args.tune:
            out[M]["tuned"] = tuned_calls(rot, A, Y, M, stream, ws if use_ws else None, args, wbytes, msc)
    t1 = out[ms[0]]["us_per_call"]
    for M in ms:
        out[M]["t_over_t_first"] = round(out[M]["us_per_call"] / t1, 3)
    copies = rot.copies
    rot.close()
    return out, copies


def main():
    args = parse()
    if args.counter_summary:
        print_counter_summary(args.counter_summary)
        return
    if args.trace_summary:
        print_trace_summary(args.trace_summary, args.steps)
        return
    if args.traffic_record:
        traffic_record(*args.traffic_record, args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the weight would be split by "
              "output columns, one shard per GPU, with no communication in the product). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from block_quantized_weight_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    if args.shape:
        fmt, act, n_s, k_s, bs_s = args.shape.split(":")
        M = args.m if args.m is not None else 1
        prob = synth.make_problem(fmt, act, int(n_s), int(k_s), int(bs_s), M, args.seed, name="shape",
                                  ms=(M,), with_bias=args.bias)
        workload = f"shape_{fmt}_{act}_n{n_s}_k{k_s}_bs{bs_s}"
        seed = args.seed
        ms = (M,)
    else:
        prob = synth.workload(args.workload, with_bias=args.bias)
        ms = (args.m,) if args.m is not None else tuple(prob.ms)
        workload = args.workload
        seed = synth.WORKLOADS[args.workload]["seed"]
    if args.calib_copy_mib > 0:
        # one plain copy kernel of known size, for scaling counter readings
        csrc = torch.ones(args.calib_copy_mib * (1 << 18), dtype=torch.float32, device=dev)
        cdst = torch.empty_like(csrc)
        torch.cuda.synchronize()
        torch.neg(csrc, out=cdst)
        torch.cuda.synchronize()
        del csrc, cdst
    wbytes = prob.weight_bytes()
    sweep, copies = measure(prob, ms, args, dev, stream)
    M = ms[0]
    head = sweep[M]
    gbs = head["gbs"]
    ms_per = head["ms_per_step"]

    extra = {}
    if not args.no_extra and not args.shape and args.workload == DEFAULT_WORKLOAD and args.m is None:
        for name, ems in EXTRA_WORKLOADS:
            p2 = synth.workload(name)
            res, c2 = measure(p2, ems, args, dev, stream)
            e = {"weight_bytes": p2.weight_bytes(), "cold_copies": c2,
                 "by_m": {str(m): {k: v for k, v in r.items() if k != "ms_per_step"} for m, r in res.items()}}
            if not args.no_read_control:
                rms2, rgbs2, _, _ = time_read_control(p2.weight_bytes(), dev, stream, args.warmup, args.steps,
                                                      args.settle_ms)
                e["read_control"] = {"us_per_read": round(rms2 * 1e3, 3), "gbs": round(rgbs2, 2)}
                for r in e["by_m"].values():
                    r["frac_of_read_control"] = round(r["gbs"] / rgbs2, 4)
            extra[name] = e
            del p2

    read = None
    if not args.no_read_control:
        rms, rgbs, shape, table = time_read_control(wbytes, dev, stream, args.warmup, args.steps, args.settle_ms)
        read = {"bytes": wbytes, "us_per_read": round(rms * 1e3, 3), "gbs": round(rgbs, 2),
                "kernel": f"k_read_control (libreadctl.so): 16-byte nontemporal loads, {shape[1]} in flight per "
                          f"lane, {shape[0]} workgroups of 256 threads (fastest of the shapes tried)",
                "shapes_gbs": table}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(prob, M, args.cpu_seconds)

    use_ws = not args.no_workspace
    out = {
        "metric": METRIC,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_per, 6),
        "us_per_call": head["us_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{prob.fmt} x {prob.act} -> f32 acc",
        "data": "synthetic",
        "config": {"workload": workload, "format": prob.fmt, "act": prob.act, "M": M, "N": prob.N,
                   "K": prob.K, "block_size": prob.bs, "weight_bytes": wbytes, "cold_copies": copies,
                   "plan": head["plan"], "flags": args.flags, "seed": seed, "bias": bool(args.bias),
                   "entry": "qgemv_run_ws" if use_ws else "qgemv_run"},
        "m_sweep": {str(m): {k: v for k, v in r.items() if k != "ms_per_step"} for m, r in sweep.items()},
        "extra_workloads": extra or None,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if args.shape else lookup_traffic(args.workload, M, args.flags, use_ws),
                     "read_control_gbs": None if read is None else read["gbs"],
                     "frac_of_read_control": None if read is None else round(gbs / read["gbs"], 4)},
        "read_control": read,
        "cpu_baseline": cpu,
        "wall_s": head["wall_s"],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
