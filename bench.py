#!/usr/bin/env python3
"""Throughput of the gfx950 selective scan on one GPU.

Headline workload: the Mamba-mini block forward at batch 8, L=2048,
D_inner=1536, N=16, float32 -- fused 4-tap causal conv + SiLU, softplus step
size, the dt*B recurrence, readout and SiLU(z) gate, one ssm_scan_fwd call
per step on inputs already resident in HBM.  Two input replicas alternate so
that no step finds the previous step's data in the 256 MB last-level cache.

Printed: one JSON line with the headline value (scan elements/s =
B*L*D*N / time), the dominant kernel's roofline figures (algorithmic bytes
over its average HIP-event duration), the oracle's CPU baseline and, under
"extra", the other workloads: backward, the L=256 block, the 65,536-token
bf16 two-level scan and the six-block streaming decode.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COPY_PROBE_ELEMS = 1 << 26          # 256 MiB read + 256 MiB written
PREWARM_MS = 200                    # untimed headline launches before the warmup steps (clock ramp)
CPU_SAMPLE_S = 10.0                 # host seconds the oracle is timed for on the headline workload
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_fwd_B8_L2048_traffic.md")
FWD_SOURCE = os.path.join(ROOT, "selective_state_space_ssm_amd", "csrc", "scan_fwd.hip")


def measured_traffic():
    """HBM bytes per launch of the forward kernel from the committed counter
    summary, if it was taken on the current kernel source (else None)."""
    import hashlib
    try:
        txt = open(TRAFFIC_FILE).read()
        sha = hashlib.sha256(open(FWD_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    vals = {}
    for line in txt.splitlines():
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != sha:
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_bytes(B, L, D, N, W, es, gate=True, conv=True, dt=True):
    """x, dt_raw (not with a constant decay), y (+ z) once each; B, C; parameters."""
    per_tok = B * L * D * es * ((3 if dt else 2) + (1 if gate else 0))
    bc = 2 * B * L * N * es
    params = 4 * ((D if dt else 0) + D * N + D + (D * W + D if conv else 0))
    return per_tok + bc + params


def bwd_bytes(B, L, D, N, es, gate=True, W=0):
    reads = B * L * D * es * (3 + (1 if gate else 0)) + 2 * B * L * N * es   # x, dt, dy (+z), B, C
    writes = B * L * D * es * (2 + (1 if gate else 0)) + 2 * B * L * N * es  # dx, ddt (+dz), dB, dC
    params = 4 * (3 * D + D * N) + 4 * (3 * D + D * N)                        # read + grads written
    if W:
        params += 2 * 4 * (D * W + D)                                          # conv taps, bias and grads
    return reads + writes + params


PROBE_LIB = os.path.join(ROOT, "selective_state_space_ssm_amd", "libssm_probe.so")
PROBE_KINDS = {"v_fma_f32": (0, 1), "v_mul_f32": (1, 1), "v_exp_f32": (2, 1),
               "v_exp_f32 + 4 v_fma_f32": (3, 5), "v_add_f32 row_ror:8 (DPP)": (4, 1),
               "v_permlane16_swap_b32": (5, 1)}
NUM_SIMDS = 256 * 4          # MI355X: 256 CUs of 4 SIMDs
SIMD_LANES_PER_CYCLE = 16    # a wave64 fp32 VALU instruction issues over 4 cycles


def probe_lib():
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise ImportError("libssm_probe.so is not built (run selective_state_space_ssm_amd/build.py)")
    lib = ctypes.CDLL(PROBE_LIB)
    p, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.probe_rate.argtypes = [i32, i32, i32, f32, f32, p, p, p]
    lib.probe_rate.restype = i32
    lib.probe_copy.argtypes = [p, p, i64, i32, p]
    lib.probe_copy.restype = i32
    return lib


def isa_rates(torch):
    """Issue rates of single VALU instructions on every SIMD (8 wavefronts per
    SIMD, 8 independent chains per lane), the shader clock they ran at, and
    the wave64 cycles per instruction that follow.  Kernels from
    libssm_probe.so, built with the scan library's flags."""
    import ctypes
    lib = probe_lib()
    blocks, chains = 256 * 8, 8
    out = torch.empty(blocks * 256, device="cuda")
    clk = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for name, (kind, ops) in PROBE_KINDS.items():
        iters = 4096 if ops == 1 else 1024

        def launch():
            rc = lib.probe_rate(kind, blocks, iters, ctypes.c_float(0.9999), ctypes.c_float(1e-4),
                                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(clk.data_ptr()), stream)
            if rc != 0:
                raise RuntimeError("probe_rate(%s) failed: %d" % (name, rc))

        for _ in range(3):
            launch()
        tm = EventTimer(torch)
        for _ in range(5):
            tm.run(launch)
        ms = tm.mean_ms()
        lane_ops = blocks * 256 * iters * chains * ops
        rate = lane_ops / (ms * 1e-3)
        c = clk.view(blocks, 4).cpu().double()
        ratio = float(((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2])).median())
        res[name] = {"lane_ops_per_s": rate, "us": round(ms * 1e3, 2), "memtime_per_realtime_tick": round(ratio, 3)}
    # clock from the FMA rate: one wave64 instruction per SIMD every 4 cycles
    fma = res["v_fma_f32"]["lane_ops_per_s"]
    clock = fma / (NUM_SIMDS * SIMD_LANES_PER_CYCLE)
    for name, r in res.items():
        r["wave64_cycles_per_instr"] = round(NUM_SIMDS * 64 * clock / r["lane_ops_per_s"], 3)
    return {"rates": res, "clock_GHz_if_fma_is_4_cycles": round(clock / 1e9, 4),
            "note": "lane_ops_per_s counts every instruction (the mix counts 5 per exp); "
                    "memtime_per_realtime_tick is s_memtime over the 100 MHz s_memrealtime counter"}


def copy_ceiling(torch, nbytes=1 << 30, reps=10):
    """A plain streaming copy of `nbytes` (read + write, far beyond the 256 MB
    last-level cache) timed with the headline's event protocol: the practical
    HBM ceiling next to the specification.  Returns GB/s counted as bytes
    read + bytes written."""
    import ctypes
    lib = probe_lib()
    a = torch.ones(nbytes // 4, device="cuda")
    b = torch.empty_like(a)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch():
        rc = lib.probe_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), nbytes // 16, 4096, stream)
        if rc != 0:
            raise RuntimeError("probe_copy failed: %d" % rc)

    for _ in range(3):
        launch()
    tm = EventTimer(torch)
    for _ in range(reps):
        tm.run(launch)
    ms = tm.mean_ms()
    ok = bool(torch.equal(a[:1024], b[:1024])) and bool(torch.equal(a[-1024:], b[-1024:]))
    del a, b
    torch.cuda.empty_cache()
    if not ok:
        raise RuntimeError("copy probe produced wrong data")
    return 2 * nbytes / (ms * 1e-3) / 1e9, ms


class EventTimer:
    """HIP-event durations of individual launches on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def run(self, fn):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self):
        self.torch.cuda.synchronize()
        return sum(s.elapsed_time(e) for s, e in self.pairs) / max(1, len(self.pairs))


SETTLE_MS = 60


def settle(torch, fn, ms=SETTLE_MS):
    """Untimed calls of fn for about ms of wall time (at least two), so that a
    workload is timed at the loaded clocks and with its first-call effects
    (fresh output pages, cold instruction caches) behind it."""
    t0 = time.perf_counter()
    n = 0
    while n < 2 or time.perf_counter() - t0 < ms * 1e-3:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed launches first; the GPU needs ~10 ms of work to reach steady clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle's CPU timing")
    ap.add_argument("--no-extra", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-model-decode", action="store_true",
                    help="skip the whole-model decode extras (their many small launches make counter passes slow)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--probe", action="store_true",
                    help="only measure instruction rates, clock and the copy ceiling, print them as JSON")
    ap.add_argument("--decode-eager", type=int, default=0, metavar="S",
                    help="only run 12 whole-model decode steps of S streams, eagerly (no graph), for counter "
                         "passes under rocprofv3; print a JSON line")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import seeded_inputs as si
    import selective_state_space_ssm_amd as ssm

    ssm.lib()
    torch.cuda.set_device(0)
    if args.probe:
        gbs, ms = copy_ceiling(torch)
        print(json.dumps({"copy_GBps": round(gbs, 1), "copy_us": round(ms * 1e3, 1), "isa": isa_rates(torch)}),
              flush=True)
        return
    dev = lambda a, dt=torch.float32: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda", dt)
    if args.decode_eager > 0:
        decode_eager(torch, si, ssm, dev, args.decode_eager)
        return

    # ------------------------------------------------------------ headline
    B, L, D, N, W = 8, 2048, 1536, 16, 4
    log("generating inputs B=%d L=%d D=%d N=%d" % (B, L, D, N))
    reps = []
    for r in range(2):
        p = si.mamba_block(B, L, D, N, W, workload=si.WL_FWDBWD, seed=r)
        reps.append({k: dev(v) for k, v in p.items()})
        reps[-1]["y"] = torch.empty(B, L, D, device="cuda")

    def fwd(rp):
        ssm.ssm_scan_fwd(rp["x"], rp["dt_raw"], rp["A_log"], rp["B"], rp["C"], dt_bias=rp["dt_bias"],
                         Dskip=rp["Dskip"], z=rp["z"], conv_w=rp["conv_w"], conv_b=rp["conv_b"], y=rp["y"])

    # the plain-copy ceiling first: measured with the same event protocol, and
    # its ~5 ms of streaming also brings the clocks to their loaded state
    # before the warmup steps (a cold GPU runs the first launches slower)
    copy_gbs = None
    try:
        copy_gbs, _ = copy_ceiling(torch)
        log("plain copy: %.1f GB/s" % copy_gbs)
    except Exception as e:
        log("copy probe failed: %r" % (e,))
    # The GPU raises its clocks over the first ~100 ms of sustained work
    # (measured: 186 us per launch after 5 warmup launches, 170 after 40, 156
    # after 400): untimed launches of the same step for PREWARM_MS of wall
    # time come before the W warmup steps, so that W only has to cover what
    # the caller asks of it and the timed steps see the loaded clocks.
    t_pre = time.perf_counter()
    pre = 0
    while time.perf_counter() - t_pre < PREWARM_MS * 1e-3:
        for _ in range(16):
            fwd(reps[pre % 2])
            pre += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        fwd(reps[i % 2])
    torch.cuda.synchronize()
    timer = EventTimer(torch)
    t0 = time.perf_counter()
    for i in range(args.steps):
        timer.run(lambda: fwd(reps[i % 2]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = timer.mean_ms()
    elems = B * L * D * N
    nbytes = fwd_bytes(B, L, D, N, W, 4)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    log("forward: %.2f us/launch, %.1f GB/s (%.1f%% of %.0f)" % (kern_ms * 1e3, achieved,
                                                                  100 * achieved / HBM_PEAK_GBS, HBM_PEAK_GBS))
    out = {
        "metric": "scan elements/s (B*L*D*N), forward, Mamba-mini block",
        "value": elems * args.steps / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm": {"ms": PREWARM_MS, "launches": pre},
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded normal inputs of the Mamba-mini shapes)",
        "config": {"workload": "mamba-mini block forward scan, fused conv4+SiLU, dt*B, SiLU(z) gate",
                   "batch": B, "seq_len": L, "d_inner": D, "d_state": N, "conv_width": W,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "kernel": "scan_fwd_kernel", "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(kern_ms * 1e3, 3)},
    }
    del reps
    torch.cuda.empty_cache()
    # the practical ceiling: a plain copy timed the same way
    if copy_gbs:
        out["roofline"]["copy_GBps"] = round(copy_gbs, 1)
        out["roofline"]["frac_of_copy"] = round(achieved / copy_gbs, 4)

    # ------------------------------------------------------------ extras
    extra = {}
    if not args.no_extra:
        try:
            extra["isa_rates"] = isa_rates(torch)
        except Exception as e:
            log("instruction-rate probe failed: %r" % (e,))
        try:
            extra.update(bench_extras(torch, np, si, ssm, dev, args))
        except Exception as e:  # report, keep the headline line
            log("extra workloads failed: %r" % (e,))
            extra["error"] = repr(e)
    if args.copy_probe:
        # a plain elementwise kernel of known size (reads 4n bytes, writes 4n
        # bytes): the reference that FETCH_SIZE / WRITE_SIZE are scaled by
        n = COPY_PROBE_ELEMS
        a = torch.ones(n, device="cuda")
        bb = torch.empty(n, device="cuda")
        for _ in range(3):
            torch.neg(a, out=bb)
        torch.cuda.synchronize()
        extra["copy_probe_bytes_each_way"] = n * 4
    out["extra"] = extra

    # ------------------------------------------------------------ CPU baseline
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(np, si)
            if not args.no_extra:
                out["cpu_baseline"]["extras"] = cpu_baseline_extras(np, si)
        except Exception as e:
            log("cpu baseline failed: %r" % (e,))
            out["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(out), flush=True)


def bench_extras(torch, np, si, ssm, dev, args):
    ex = {}
    reps = max(5, args.steps // 2)

    # backward at the headline shape
    B, L, D, N = 8, 2048, 1536, 16
    p = si.mamba_block(B, L, D, N, 4, workload=si.WL_FWDBWD, with_dy=True)
    P = {k: dev(v) for k, v in p.items()}
    u = ssm.conv1d_causal(P["x"], P["conv_w"], P["conv_b"])
    out = {}
    ws = torch.empty(ssm.ssm_scan_bwd_workspace_size(ssm.ssm_scan_desc(B, L, D, N, 0, 0, 0, 0)),
                     dtype=torch.uint8, device="cuda")

    def bwd():
        ssm.ssm_scan_bwd(u, P["dt_raw"], P["A_log"], P["B"], P["C"], P["dy"], dt_bias=P["dt_bias"],
                         Dskip=P["Dskip"], z=P["z"], out=out, workspace=ws)

    settle(torch, bwd)
    tm = EventTimer(torch)
    for _ in range(reps):
        tm.run(bwd)
    ms = tm.mean_ms()
    nb = bwd_bytes(B, L, D, N, 4)
    ex["backward_B8_L2048"] = {"us_per_call": round(ms * 1e3, 2), "elements_per_s": B * L * D * N / (ms * 1e-3),
                               "algorithmic_GBps": round(nb / (ms * 1e-3) / 1e9, 1), "algorithmic_bytes": nb}
    log("backward: %.1f us" % (ms * 1e3))

    # the same backward with the conv prologue (x in; dx, dconv_w, dconv_b out: the library runs the
    # conv, the scan backward from its output and the conv backward)
    outc = {}
    wsc = torch.empty(ssm.ssm_scan_bwd_workspace_size(ssm.ssm_scan_desc(B, L, D, N, 4, 0, 0, 0)),
                      dtype=torch.uint8, device="cuda")

    def bwd_conv():
        ssm.ssm_scan_bwd(P["x"], P["dt_raw"], P["A_log"], P["B"], P["C"], P["dy"], dt_bias=P["dt_bias"],
                         Dskip=P["Dskip"], z=P["z"], conv_w=P["conv_w"], conv_b=P["conv_b"], out=outc,
                         workspace=wsc)

    settle(torch, bwd_conv)
    tm = EventTimer(torch)
    for _ in range(reps):
        tm.run(bwd_conv)
    ms = tm.mean_ms()
    nb = bwd_bytes(B, L, D, N, 4, W=4)
    ex["backward_conv_B8_L2048"] = {"us_per_call": round(ms * 1e3, 2),
                                    "elements_per_s": B * L * D * N / (ms * 1e-3),
                                    "algorithmic_GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                                    "algorithmic_bytes": nb}
    log("backward with the conv prologue: %.1f us" % (ms * 1e3))
    del wsc

    # conv alone and the L=256 block
    tm = EventTimer(torch)
    for _ in range(reps):
        tm.run(lambda: ssm.conv1d_causal(P["x"], P["conv_w"], P["conv_b"], y=u))
    ms = tm.mean_ms()
    nb = 2 * B * L * D * 4 + 4 * D * 5
    ex["conv1d_B8_L2048"] = {"us_per_call": round(ms * 1e3, 2), "algorithmic_GBps": round(nb / (ms * 1e-3) / 1e9, 1)}
    del P, u, out, outc, ws
    torch.cuda.empty_cache()

    B2, L2 = 8, 256
    q = si.mamba_block(B2, L2, D, N, 4, workload=si.WL_BLOCK)
    Q = {k: dev(v) for k, v in q.items()}
    y2 = torch.empty(B2, L2, D, device="cuda")
    f2 = lambda: ssm.ssm_scan_fwd(Q["x"], Q["dt_raw"], Q["A_log"], Q["B"], Q["C"], dt_bias=Q["dt_bias"],
                                  Dskip=Q["Dskip"], z=Q["z"], conv_w=Q["conv_w"], conv_b=Q["conv_b"], y=y2)
    settle(torch, f2)
    tm = EventTimer(torch)
    for _ in range(reps):
        tm.run(f2)
    ms = tm.mean_ms()
    nb = fwd_bytes(B2, L2, D, N, 4, 4)
    ex["forward_B8_L256"] = {"us_per_call": round(ms * 1e3, 2), "elements_per_s": B2 * L2 * D * N / (ms * 1e-3),
                             "algorithmic_GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                             "note": "working set fits the 256 MB last-level cache"}
    del Q, y2
    torch.cuda.empty_cache()

    # the constant decay source (decay fixed per channel and state, no step
    # size): the headline shape with state width 16, and width 1
    for Nc in (16, 1):
        c = si.mamba_block(B, L, D, Nc, 4, workload=si.WL_FWDBWD, const_decay=True)
        Cc = {k: dev(c[k]) for k in ("x", "A_log", "B", "C", "z", "Dskip", "conv_w", "conv_b")}
        del c
        yc = torch.empty(B, L, D, device="cuda")
        fc = lambda: ssm.ssm_scan_fwd(Cc["x"], None, Cc["A_log"], Cc["B"], Cc["C"], Dskip=Cc["Dskip"], z=Cc["z"],
                                      conv_w=Cc["conv_w"], conv_b=Cc["conv_b"], y=yc, disc=ssm.SSM_DECAY_CONST)
        settle(torch, fc)
        tm = EventTimer(torch)
        for _ in range(reps):
            tm.run(fc)
        ms = tm.mean_ms()
        nb = fwd_bytes(B, L, D, Nc, 4, 4, dt=False)
        ex["forward_const_decay_B8_L2048_N%d" % Nc] = {
            "us_per_call": round(ms * 1e3, 2), "elements_per_s": B * L * D * Nc / (ms * 1e-3),
            "algorithmic_GBps": round(nb / (ms * 1e-3) / 1e9, 1), "algorithmic_bytes": nb}
        log("constant-decay forward, N=%d: %.1f us" % (Nc, ms * 1e3))
        del Cc, yc
        torch.cuda.empty_cache()

    # long sequence, bf16, two-level scan
    L4 = 65536
    r = si.mamba_block(1, L4, D, N, 4, workload=si.WL_LONG, bf16=True, with_dy=True)
    bf = torch.bfloat16
    R = {k: dev(r[k], bf) for k in ("x", "dt_raw", "B", "C", "z")}
    R.update({k: dev(r[k]) for k in ("dt_bias", "A_log", "Dskip")})
    y4 = torch.empty(1, L4, D, device="cuda", dtype=bf)
    desc = ssm.ssm_scan_desc(1, L4, D, N, 0, 1, 0, 0)
    ws4 = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_size(desc)), dtype=torch.uint8, device="cuda")
    f4 = lambda: ssm.ssm_scan_fwd(R["x"], R["dt_raw"], R["A_log"], R["B"], R["C"], dt_bias=R["dt_bias"],
                                  Dskip=R["Dskip"], z=R["z"], y=y4, workspace=ws4)
    settle(torch, f4)
    tm = EventTimer(torch)
    for _ in range(reps):
        tm.run(f4)
    ms = tm.mean_ms()
    nb = fwd_bytes(1, L4, D, N, 4, 2, conv=False)
    ex["forward_bf16_B1_L65536_chunked"] = {"us_per_call": round(ms * 1e3, 2),
                                            "elements_per_s": L4 * D * N / (ms * 1e-3),
                                            "algorithmic_GBps": round(nb / (ms * 1e-3) / 1e9, 1)}
    # the same long sequence with the 4-tap conv fused (x in instead of u; the
    # conv-fused forward splits time with the headline kernel's layout)
    cw4, cb4 = dev(r["conv_w"]), dev(r["conv_b"])
    descc = ssm.ssm_scan_desc(1, L4, D, N, 4, 1, 0, 0)
    ws4c = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_size(descc)), dtype=torch.uint8, device="cuda")
    f4c = lambda: ssm.ssm_scan_fwd(R["x"], R["dt_raw"], R["A_log"], R["B"], R["C"], dt_bias=R["dt_bias"],
                                   Dskip=R["Dskip"], z=R["z"], conv_w=cw4, conv_b=cb4, y=y4, workspace=ws4c)
    settle(torch, f4c)
    tm = EventTimer(torch)
    for _ in range(reps):
        tm.run(f4c)
    ms = tm.mean_ms()
    nb = fwd_bytes(1, L4, D, N, 4, 2, conv=True)
    ex["forward_bf16_B1_L65536_chunked_conv_fused"] = {"us_per_call": round(ms * 1e3, 2),
                                                       "elements_per_s": L4 * D * N / (ms * 1e-3),
                                                       "algorithmic_GBps": round(nb / (ms * 1e-3) / 1e9, 1)}
    log("long bf16 forward, conv fused: %.1f us" % (ms * 1e3))
    del y4, ws4, ws4c
    torch.cuda.empty_cache()

    # backward of the same workload, split in time by the library
    R["dy"] = dev(r["dy"], bf)
    del r
    wsb = torch.empty(ssm.ssm_scan_bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
    outb = {}
    b4 = lambda: ssm.ssm_scan_bwd(R["x"], R["dt_raw"], R["A_log"], R["B"], R["C"], R["dy"], dt_bias=R["dt_bias"],
                                  Dskip=R["Dskip"], z=R["z"], out=outb, workspace=wsb)
    settle(torch, b4)
    tm = EventTimer(torch)
    for _ in range(max(3, reps // 2)):
        tm.run(b4)
    ms = tm.mean_ms()
    nb = bwd_bytes(1, L4, D, N, 2)
    ex["backward_bf16_B1_L65536_chunked"] = {"us_per_call": round(ms * 1e3, 2),
                                             "elements_per_s": L4 * D * N / (ms * 1e-3),
                                             "algorithmic_GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                                             "algorithmic_bytes": nb}
    log("long bf16 backward (time split): %.1f us" % (ms * 1e3))
    del R, wsb, outb
    torch.cuda.empty_cache()

    # streaming decode: 6 blocks x 256 streams x 1536 channels x 16 states,
    # 1,024 token steps; inputs for a pool of 32 steps are resident and
    # cycled.  Token steps are captured in a HIP graph (32 steps per graph)
    # so that host launch overhead stays out of the device timeline.
    nblk, S, steps, pool = 6, 256, 1024, 32
    prm = {k: dev(v) for k, v in si.stream_params(nblk, D, N, 4).items()}
    h = torch.zeros(nblk, S, D, N, device="cuda")
    cs = torch.zeros(nblk, S, 3, D, device="cuda")
    toks = []
    for t in range(pool):
        per = [si.stream_token_torch(k, t, S, D, N, "cuda") for k in range(nblk)]
        toks.append({kk: torch.stack([pp[kk] for pp in per]).contiguous() for kk in per[0]})
    ys = torch.empty(nblk, S, D, device="cuda")

    def per_block(t):
        i = toks[t]
        for k in range(nblk):
            ssm.ssm_step(h[k:k + 1], i["x"][k:k + 1], i["dt_raw"][k:k + 1], prm["A_log"][k:k + 1],
                         i["B"][k:k + 1], i["C"][k:k + 1], conv_state=cs[k:k + 1], z=i["z"][k:k + 1],
                         conv_w=prm["conv_w"][k:k + 1], conv_b=prm["conv_b"][k:k + 1],
                         dt_bias=prm["dt_bias"][k:k + 1], Dskip=prm["Dskip"][k:k + 1], y=ys[k:k + 1])

    def stacked(t):
        i = toks[t]
        ssm.ssm_step(h, i["x"], i["dt_raw"], prm["A_log"], i["B"], i["C"], conv_state=cs, z=i["z"],
                     conv_w=prm["conv_w"], conv_b=prm["conv_b"], dt_bias=prm["dt_bias"], Dskip=prm["Dskip"], y=ys)

    # the same stacked step with the state stored in bf16 (an option of
    # ssm_step: updated in float32, rounded when stored)
    h16 = torch.zeros(nblk, S, D, N, device="cuda", dtype=torch.bfloat16)

    def stacked_bf16_state(t):
        i = toks[t]
        ssm.ssm_step(h16, i["x"], i["dt_raw"], prm["A_log"], i["B"], i["C"], conv_state=cs, z=i["z"],
                     conv_w=prm["conv_w"], conv_b=prm["conv_b"], dt_bias=prm["dt_bias"], Dskip=prm["Dskip"], y=ys)

    per_block_bytes = (2 * S * D * N * 4 + 2 * S * 3 * D * 4 + S * D * 4 * 4 + 2 * S * N * 4
                       + 4 * (D * N + 3 * D + 4 * D))
    bytes16 = per_block_bytes - 2 * S * D * N * 2
    for name, fn, nb in (("per_block_launches", per_block, per_block_bytes),
                         ("stacked_one_launch", stacked, per_block_bytes),
                         ("stacked_one_launch_bf16_state", stacked_bf16_state, bytes16)):
        for t in range(4):
            fn(t)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for t in range(pool):
                fn(t)
        gr.replay()
        torch.cuda.synchronize()
        tm = EventTimer(torch)
        t0 = time.perf_counter()
        for _ in range(steps // pool):
            tm.run(gr.replay)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = tm.mean_ms() / pool       # per token step
        ex["streaming_6blk_256streams_" + name] = {
            "tokens_per_s": S / (ms * 1e-3), "tokens_per_s_wall": S * steps / wall,
            "us_per_token_step": round(ms * 1e3, 2),
            "algorithmic_GBps": round(nblk * nb / (ms * 1e-3) / 1e9, 1),
            "note": "state + history of the 6 blocks (%d MB) fit the 256 MB last-level cache"
                    % round(nblk * S * (D * N * (2 if nb == bytes16 else 4) + 3 * D * 4) / 1e6)}
        log("streaming %s: %.1f us per token step" % (name, ms * 1e3))
    # The stacked step again, with the last-level cache emptied before every
    # step (an untimed read and write of an unrelated 1 GiB buffer), so that
    # the state streams from HBM: the gap to the resident loop above shows
    # how much of that loop's state stayed in the 256 MB cache.
    flush = torch.empty(1 << 28, device="cuda")
    stacked(0)
    tm = EventTimer(torch)
    for t in range(64):
        flush.add_(1.0)
        tm.run(lambda: stacked(t % pool))
    ms = tm.mean_ms()
    ex["streaming_6blk_256streams_stacked_one_launch_cache_flushed"] = {
        "tokens_per_s": S / (ms * 1e-3), "us_per_token_step": round(ms * 1e3, 2),
        "algorithmic_GBps": round(nblk * per_block_bytes / (ms * 1e-3) / 1e9, 1),
        "note": "each step timed alone after a 1 GiB pass over another buffer: the state comes from HBM"}
    log("streaming stacked_one_launch, cache flushed before each step: %.1f us per token step" % (ms * 1e3))
    del flush
    del h, cs, toks, ys, prm
    torch.cuda.empty_cache()

    if args.no_model_decode:
        return ex
    # the whole Mamba-mini model (random-init weights), one token per stream
    # per step: embedding, 6 blocks (LayerNorm, in_proj + conv, x_proj,
    # dt_proj, the selective step, out_proj + residual), final LayerNorm and
    # the tied 4096-token head.  Steps captured in HIP graphs of 32 tokens.
    cfg = si.MAMBA_MINI
    mp = si.model_params(cfg)
    emb = dev(mp["emb"])
    nfw, nfb = dev(mp["norm_f_w"]), dev(mp["norm_f_b"])
    layers = ssm.ModelLayers([{k: dev(v) for k, v in lay.items()} for lay in mp["layers"]])
    wbytes = 4 * (sum(v.size for lay in mp["layers"] for v in lay.values()) + mp["emb"].size)
    for Sm in (1, 256):
        desc = ssm.model_desc(cfg, Sm)
        ws = torch.empty(ssm.ssm_model_decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
        hm = torch.zeros(cfg["n_layers"], Sm, cfg["d_inner"], cfg["d_state"], device="cuda")
        cm = torch.zeros(cfg["n_layers"], Sm, cfg["conv_width"] - 1, cfg["d_inner"], device="cuda")
        tk = torch.from_numpy(si.model_tokens(cfg, Sm, pool).T.copy()).cuda()   # [pool, S]
        lg = torch.empty(Sm, cfg["vocab"], device="cuda")

        def dstep(t):
            ssm.ssm_model_decode_step(desc, emb, layers, tk[t], hm, cm, logits=lg, norm_f_w=nfw, norm_f_b=nfb,
                                      workspace=ws)

        for t in range(4):
            dstep(t)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for t in range(pool):
                dstep(t)
        gr.replay()
        torch.cuda.synchronize()
        tm = EventTimer(torch)
        nrep = max(4, 256 // pool)
        t0 = time.perf_counter()
        for _ in range(nrep):
            tm.run(gr.replay)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = tm.mean_ms() / pool
        ex["decode_mamba_mini_%dstream%s" % (Sm, "" if Sm == 1 else "s")] = {
            "tokens_per_s": Sm / (ms * 1e-3), "tokens_per_s_wall": Sm * nrep * pool / wall,
            "us_per_token_step": round(ms * 1e3, 2), "weights_MB": round(wbytes / 1e6, 1),
            "note": "6 blocks + tied head, random-init weights (no quality claim); the pages' browser "
                    "figure is 535 tokens/s for one stream on an unspecified machine"}
        log("model decode, %d stream(s): %.1f us per token step" % (Sm, ms * 1e3))
        del ws, hm, cm, tk, lg
    return ex


def decode_eager(torch, si, ssm, dev, S, steps=12):
    """Mamba-mini decode steps of S streams launched one by one (no graph),
    so that a profiler sees every dispatch of every step."""
    cfg = si.MAMBA_MINI
    mp = si.model_params(cfg)
    emb = dev(mp["emb"])
    nfw, nfb = dev(mp["norm_f_w"]), dev(mp["norm_f_b"])
    layers = ssm.ModelLayers([{k: dev(v) for k, v in lay.items()} for lay in mp["layers"]])
    desc = ssm.model_desc(cfg, S)
    ws = torch.empty(ssm.ssm_model_decode_workspace_size(desc), dtype=torch.uint8, device="cuda")
    hm = torch.zeros(cfg["n_layers"], S, cfg["d_inner"], cfg["d_state"], device="cuda")
    cm = torch.zeros(cfg["n_layers"], S, cfg["conv_width"] - 1, cfg["d_inner"], device="cuda")
    tk = torch.from_numpy(si.model_tokens(cfg, S, steps).T.copy()).cuda()   # [steps, S]
    lg = torch.empty(S, cfg["vocab"], device="cuda")
    for t in range(steps):
        ssm.ssm_model_decode_step(desc, emb, layers, tk[t], hm, cm, logits=lg, norm_f_w=nfw, norm_f_b=nfb,
                                  workspace=ws)
        torch.cuda.synchronize()
        log("decode step %d of %d streams done" % (t, S))
    print(json.dumps({"decode_eager": {"streams": S, "steps": steps,
                                       "logits_finite": bool(torch.isfinite(lg).all())}}), flush=True)


def cpu_baseline(np, si):
    """The float64 oracle, as it stands, on the host cores: the whole
    headline forward (conv, then the scan with the gate) over all 8 batch
    rows with every host thread, repeated for about CPU_SAMPLE_S seconds (the
    mean per run is reported), and batch row 0 alone on one thread."""
    import oracle
    oracle.build(force=False)
    Bs, L, D, N, W = 8, 2048, 1536, 16, 4
    p = si.mamba_block(Bs, L, D, N, W, workload=si.WL_FWDBWD)
    f = lambda k: np.ascontiguousarray(p[k], np.float64)
    args = {k: f(k) for k in ("x", "dt_raw", "B", "C", "z", "dt_bias", "A_log", "Dskip", "conv_w", "conv_b")}
    del p

    def run(rows):
        sl = lambda k: args[k][rows] if args[k].ndim == 3 else args[k]
        u, _ = oracle.conv1d_causal(sl("x"), args["conv_w"], args["conv_b"], want_state=False)
        oracle.scan_fwd(u, sl("dt_raw"), args["A_log"], sl("B"), sl("C"), dt_bias=args["dt_bias"],
                        Dskip=args["Dskip"], z=sl("z"))

    cores = oracle.num_threads()
    # whole-workload runs repeated until about CPU_SAMPLE_S seconds of host
    # time are spent (at least two runs, at most 500)
    times, t_start = [], time.perf_counter()
    while len(times) < 2 or (time.perf_counter() - t_start < CPU_SAMPLE_S and len(times) < 500):
        t0 = time.perf_counter()
        run(slice(0, Bs))
        times.append(time.perf_counter() - t0)
    reps = len(times)
    dt = sum(times) / reps
    oracle.set_num_threads(1)
    t0 = time.perf_counter()
    run(slice(0, 1))
    dt1 = time.perf_counter() - t0
    oracle.set_num_threads(cores)
    return {"value": Bs * L * D * N / dt, "unit": "elements/s", "cores": cores, "kind": "oracle",
            "sample": "the whole forward workload (conv + scan + gate, B=8, L=2048, D=1536, N=16, float64), "
                      "%d runs in %.1f s, mean %.3f s per run" % (reps, sum(times), dt),
            "single_thread": {"value": L * D * N / dt1, "unit": "elements/s", "cores": 1,
                              "sample": "batch row 0 of the same workload, %.2f s" % dt1}}

def cpu_baseline_extras(np, si):
    """The oracle on bounded samples of the extra workloads, all host
    threads, each a few seconds at most: the backward (batch row 0 of the
    B=8, L=2048 workload), the constant-decay forward (whole workload), the
    streaming step (one block-step of 256 streams) and the whole-model decode
    (one stream, 8 tokens; 256 streams, 2 tokens)."""
    import oracle
    from oracle import mamba_model as mm
    ex = {}
    cores = oracle.num_threads()
    B, L, D, N = 8, 2048, 1536, 16

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    p = si.mamba_block(1, L, D, N, 4, workload=si.WL_FWDBWD, with_dy=True)
    u, _ = oracle.conv1d_causal(p["x"], p["conv_w"], p["conv_b"])
    dt = timed(lambda: oracle.scan_bwd(u, p["dt_raw"], p["A_log"], p["B"], p["C"], p["dy"], dt_bias=p["dt_bias"],
                                       Dskip=p["Dskip"], z=p["z"]))
    ex["backward_B8_L2048"] = {"value": L * D * N / dt, "unit": "elements/s", "cores": cores,
                               "sample": "batch row 0 (1/8 of the workload), %.2f s" % dt}
    c = si.mamba_block(B, L, D, N, 4, workload=si.WL_FWDBWD, const_decay=True)

    def const_fwd():
        uc, _ = oracle.conv1d_causal(c["x"], c["conv_w"], c["conv_b"], want_state=False)
        oracle.scan_fwd(uc, None, c["A_log"], c["B"], c["C"], Dskip=c["Dskip"], z=c["z"], disc=oracle.DECAY_CONST)

    dt = timed(const_fwd)
    ex["forward_const_decay_B8_L2048_N16"] = {"value": B * L * D * N / dt, "unit": "elements/s", "cores": cores,
                                              "sample": "the whole workload, %.2f s" % dt}
    del c, p, u
    r = np.random.default_rng(0)
    S = 256
    h = np.zeros((S, D, N))
    cs = np.zeros((S, 3, D))
    prm = si.stream_params(1, D, N, 4)
    x, dtr, z = (r.standard_normal((S, D)) for _ in range(3))
    Bm, Cm = (r.standard_normal((S, N)) for _ in range(2))
    dt = timed(lambda: oracle.step(h, cs, x, dtr, Bm, Cm, prm["A_log"][0], z=z, conv_w=prm["conv_w"][0],
                                   conv_b=prm["conv_b"][0], dt_bias=prm["dt_bias"][0], Dskip=prm["Dskip"][0]))
    ex["streaming_step_one_block_256streams"] = {"value": S / dt, "unit": "stream-steps/s (one block)",
                                                 "cores": cores, "sample": "one block-step, %.3f s" % dt}
    mp = si.model_params(si.MAMBA_MINI)
    for Sm, T in ((1, 8), (256, 2)):
        hm, cm = mm.new_state(si.MAMBA_MINI, Sm)
        tok = si.model_tokens(si.MAMBA_MINI, Sm, T)
        dt = timed(lambda: [mm.decode_step(mp, tok[:, t], hm, cm) for t in range(T)])
        ex["decode_mamba_mini_%dstream%s" % (Sm, "" if Sm == 1 else "s")] = {
            "value": Sm * T / dt, "unit": "tokens/s", "cores": cores,
            "sample": "%d token step(s), %.2f s" % (T, dt)}
    return ex


if __name__ == "__main__":
    main()
