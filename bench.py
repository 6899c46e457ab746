"""Throughput of the SSD scan forward on one MI355X.

One step = one ssd_scan_fwd call (the whole hot path: dt/cumsum, chunk state,
state passing, chunk scan with the D/z epilogue) over the long bf16 workload:
batch 1 x seqlen 65536, 128 heads of 64, dstate 128, 8 B/C groups, chunk
256, D on, z off (65536 tokens per step).  Inputs are seeded, synthetic and
resident in HBM before timing starts (one call touches 2.4 GB, ten times the
256 MB Infinity Cache).

Prints one JSON line: tokens/s over exactly `--steps` back-to-back calls, the
per-call median and minimum from HIP events (a second pass), the roofline of
the dominant kernel (its algorithmic bytes per launch over its mean launch
time, from events the library records around each stage on the launch
stream -- a third pass), its HBM traffic from committed rocprofv3 counter
summaries, the machine's measured peaks next to the datasheet ones, the CPU
oracle on a bounded sample of the same workload, and (unless --no-others) a
line per further workload: the other four scan configurations (fp32 1 x 256;
fp32 2 x 2048 at ngroups 1, 2, 4; bf16 8 x 4096; fp32 4 x 8192 as four
chained 2048-step segments), packed sequences, one-token decode, the block
around the scan and the backward.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from ssd_workloads import WORKLOADS, make_inputs, make_seq_idx  # noqa: E402

PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak (datasheet)
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (datasheet)
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E (datasheet)

HEADLINE = "bf16_b1_L65536_H128_P64_N128_G8_Q256"
TRAFFIC_DIR = os.path.join(ROOT, "profiles", "traffic")
CSRC = os.path.join(ROOT, "selective_state_space_ssd_amd", "csrc")
MIN_CALLS = 30


# --------------------------------------------------------------------------
# algorithmic work
# --------------------------------------------------------------------------

def alg_flops(w):
    """Algorithmic flops of one call, by stage (chunked SSD, causal, C.B^T once
    per group): chunk state 2QPN per (chunk, head); state passing 2PN per
    (chunk, head); chunk scan 2QPN + PQ(Q+1) per (chunk, head); C.B^T NQ(Q+1)
    per (chunk, group), in the stage that forms it: the state-passing launch
    when the fp32 four-heads chunk scan runs with two or more of its
    workgroups per group (it reads the tiles from there), else the chunk
    scan."""
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size
    if w.segments > 1:
        L //= w.segments
    nc = math.ceil(L / Q)
    gram = b * nc * G * N * Q * (Q + 1)
    group_scan = (Q in (64, 128) and N in (64, 128) and (H // G) % 4 == 0 and H // G >= 8
                  and w.dtype == "f32")
    return {
        "prep": b * L * H * 2.0,
        "chunk_state": b * nc * H * 2.0 * Q * P * N,
        "state_passing": b * nc * H * 2.0 * P * N + (gram if group_scan else 0),
        "chunk_scan": b * nc * H * (2.0 * Q * P * N + P * Q * (Q + 1)) + (0 if group_scan else gram),
    }


def alg_bytes(w):
    """Bytes one call must move: read x, dt, B, C, (z), (init), A, D, dt_bias;
    write out, (final).  Intermediates are not counted.  For a continuation
    workload, one segment call."""
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    if w.segments > 1:
        L //= w.segments
    es = 2 if w.dtype == "bf16" else 4
    n = b * L * H * P * es * (2 + (1 if w.gate else 0))     # x, out, z
    n += b * L * H * es + 2 * b * L * G * N * es              # dt, B, C
    n += 3 * H * 4
    st = b * H * P * N * 4
    n += st * ((1 if (w.init or w.segments > 1) else 0) + (1 if w.final else 0))
    return n


# --------------------------------------------------------------------------
# measured peaks and counter summaries
# --------------------------------------------------------------------------

def measured_peaks(dev):
    """Streaming-copy HBM rate and matrix-core rates, from libssd_peaks.so
    (selective_state_space_ssd_amd/csrc/ssd_peaks.hip), timed with events."""
    import torch
    from selective_state_space_ssd_amd import _build
    lib = ctypes.CDLL(_build.PEAKS_LIB_PATH)
    p = ctypes.c_void_p
    lib.ssd_peak_copy.argtypes = [p, p, ctypes.c_size_t, p]
    lib.ssd_peak_copy.restype = ctypes.c_int
    lib.ssd_peak_mfma.argtypes = [p, ctypes.c_int, ctypes.c_int, ctypes.c_int, p]
    lib.ssd_peak_mfma.restype = ctypes.c_int
    lib.ssd_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.ssd_peak_mfma_flops.restype = ctypes.c_double
    s = torch.cuda.current_stream(dev)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        best = math.inf
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            fn()
            b.record(s)
            b.synchronize()
            best = min(best, a.elapsed_time(b) / 1e3)
        return best

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def copy():
        if lib.ssd_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, s.cuda_stream) != 0:
            raise RuntimeError("ssd_peak_copy failed")

    t = timed(copy, 5)
    assert torch.equal(dst[:1024], src[:1024])
    del src, dst
    res = {"hbm_copy_GBs": 2 * nbytes / t / 1e9,
           "hbm_copy_note": "1 GiB read + 1 GiB written per launch, best of 5"}
    wgs, iters = 256 * 8, 2000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    for kind, name in ((0, "fp32_32x32x2"), (3, "fp32_16x16x4"), (1, "bf16_32x32x16"),
                       (2, "bf16_16x16x32")):
        def run():
            if lib.ssd_peak_mfma(sink.data_ptr(), kind, wgs, iters, s.cuda_stream) != 0:
                raise RuntimeError("ssd_peak_mfma failed")
        t = timed(run, 3)
        res[f"mfma_{name}_TFLOPs"] = lib.ssd_peak_mfma_flops(kind, wgs, iters) / t / 1e12
    return res


def measured_traffic(workload, stage):
    """HBM bytes per launch of the kernel of `stage` on `workload`, from the
    committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary
    (profiles/traffic/<workload>.<stage>.json, written by rocprof_summary.py
    --traffic), or None when there is none or the kernel's sources have
    changed since the counters were taken."""
    path = os.path.join(TRAFFIC_DIR, f"{workload}.{stage}.json")
    if not os.path.exists(path):
        return None
    from rocprof_summary import sources_hash
    t = json.load(open(path))
    if sources_hash([os.path.join(CSRC, n) for n in t["sources"]]) != t["sources_sha256_16"]:
        return None
    return {"bytes_per_launch": t["bytes_per_dispatch"], "kernel": t["kernel"],
            "fetch_factor": t["fetch_factor"], "write_factor": t["write_factor"]}


# --------------------------------------------------------------------------
# timing
# --------------------------------------------------------------------------

WARMUP_SECONDS = 0.3


def time_calls(call, n, warmup, dev, n_events=None):
    """`warmup` untimed calls, continued until at least WARMUP_SECONDS have
    passed (the GPU's clocks take tens of milliseconds to settle after an
    idle stretch: measured right after five calls, the batch 8 x 4096 bf16
    call read 483 us per call against 409 us once settled), then exactly `n`
    back-to-back calls timed by the host clock between two synchronizations,
    then `n_events` (default: `n`, at least 30) more calls each bracketed by
    HIP events on the launch stream.  Returns wall seconds per call and the
    events' median, min and mean in ms."""
    import torch
    s = torch.cuda.current_stream(dev)
    t_w = time.perf_counter()
    k = 0
    while k < warmup or time.perf_counter() - t_w < WARMUP_SECONDS:
        call(k)
        k += 1
        if k >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(n):
        call(k)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / n
    ne = max(n if n_events is None else n_events, MIN_CALLS)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(ne)]
    for k in range(ne):
        evs[k][0].record(s)
        call(k)
        evs[k][1].record(s)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    return {"wall_s_per_call": wall, "median_ms": float(np.median(ms)),
            "min_ms": float(ms.min()), "mean_ms": float(ms.mean()), "calls": n,
            "event_calls": ne}


# --------------------------------------------------------------------------
# the scan workloads
# --------------------------------------------------------------------------

class ScanWorkload:
    """Device copies of a workload's inputs (`copies` of them, rotated call by
    call) and the calls of the scan on the automatic path."""

    def __init__(self, w, dev, copies=1, inp=None):
        import torch
        import selective_state_space_ssd_amd as ssd
        self.w, self.dev = w, dev
        self.code = ssd.SSD_BF16 if w.dtype == "bf16" else ssd.SSD_F32
        L = w.seqlen // w.segments
        self.seg_len = L
        self.path = ssd.taken_path(w.batch, L, w.nheads, w.headdim, w.dstate, w.ngroups,
                                   w.chunk_size, self.code)
        self.ws_bytes = ssd.workspace_size(w.batch, L, w.nheads, w.headdim, w.dstate,
                                           w.ngroups, w.chunk_size, self.code)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.sets = []
        for c in range(copies):
            src = inp if (inp is not None and c == 0) else make_inputs(w)
            t = {}
            for k in ("x", "z", "B", "C", "dt"):
                if src.get(k) is None:
                    t[k] = None
                elif w.dtype == "bf16":
                    t[k] = torch.from_numpy(src["bits"][k].view(np.int16)).to(dev).view(
                        torch.bfloat16)
                else:
                    t[k] = torch.from_numpy(src[k]).to(dev)
            for k in ("A", "D", "dt_bias", "initial_states"):
                t[k] = None if src.get(k) is None else torch.from_numpy(src[k]).to(dev)
            t["out"] = torch.empty_like(t["x"])
            st_shape = (w.batch, w.nheads, w.headdim, w.dstate)
            t["state"] = (torch.zeros(st_shape, dtype=torch.float32, device=dev)
                          if (w.final or w.segments > 1) else None)
            self.sets.append(t)

    def _args(self, t, seg):
        w, ptr = self.w, (lambda v: None if v is None else v.data_ptr())
        L = self.seg_len
        lo = seg * L

        def sl(v):
            return None if v is None else v[:, lo:lo + L] if w.segments > 1 else v

        x, dt, B, C, z, out = (sl(t[k]) for k in ("x", "dt", "B", "C", "z", "out"))
        if w.segments > 1:  # a segment's slice of [b, L, ...] is not contiguous: use copies
            x, dt, B, C, out = (t.setdefault(f"seg{seg}_{k}", v.contiguous())
                                for k, v in (("x", x), ("dt", dt), ("B", B), ("C", C),
                                             ("out", out)))
            z = None if z is None else t.setdefault(f"seg{seg}_z", z.contiguous())
        init = t["state"] if (w.segments > 1 and seg > 0) else t["initial_states"]
        return (ptr(x), ptr(dt), ptr(t["A"]), ptr(B), ptr(C), ptr(t["D"]), ptr(z),
                ptr(t["dt_bias"]), 0.0, math.inf, w.chunk_size, w.ngroups, ptr(init), ptr(out),
                ptr(t["state"]), w.batch, L, w.nheads, w.headdim, w.dstate, self.code,
                self.ws.data_ptr(), self.ws_bytes)

    def prepare(self):
        """Argument tuples per (copy, segment)."""
        self.argv = [[self._args(t, s) for s in range(self.w.segments)] for t in self.sets]

    def call(self, k, timing=None):
        import torch
        import selective_state_space_ssd_amd as ssd
        s = torch.cuda.current_stream(self.dev).cuda_stream
        for seg, a in enumerate(self.argv[k % len(self.argv)]):
            st = ssd.scan_fwd_raw(*a, s, timing=None if timing is None else timing[seg])
            if st != 0:
                raise ssd.SsdError(st, ssd.status_string(st))


def describe(w):
    opts = []
    opts.append("z gate on" if w.gate else "z off")
    opts.append("D on" if w.skip else "D off")
    if w.final:
        opts.append("final states returned")
    seg = (f" as {w.segments} chained segments of {w.seqlen // w.segments} (initial state = "
           "the previous segment's final state, in place)" if w.segments > 1 else "")
    return (f"ssd_scan_fwd {w.dtype} batch {w.batch} x seqlen {w.seqlen}{seg}, {w.nheads} heads "
            f"x headdim {w.headdim}, dstate {w.dstate}, ngroups {w.ngroups}, chunk "
            f"{w.chunk_size}, {', '.join(opts)}")


STAGE_KERNELS = {
    "staged": {"prep": "dt_cumsum_kernel", "chunk_state": "chunk_state kernel",
               "state_passing": "state_passing_kernel", "chunk_scan": "chunk scan kernel"},
    "staged_scan": {"chunk_state": "state_scan_kernel (stages 1-3)",
                    "chunk_scan": "chunk scan kernel"},
    "chain": {"chunk_scan": "chain_scan_bf16_kernel"},
    "chain_segmented": {"chunk_state": "unit_state_bf16_kernel",
                        "chunk_scan": "chain_scan_bf16_kernel (segments)"},
    "fused_head": {"prep": "fused set-up kernel", "chunk_scan": "fused_scan_bf16_kernel"},
    "fused_group": {"prep": "fused set-up kernel", "chunk_scan": "fused_group_bf16_kernel"},
}


def scan_line(names, dev, steps, warmup, peaks, copies=1, inp=None):
    """One line for a step made of the scan calls of `names` (one workload,
    or several run back to back as one step): tokens/s, per-step median and
    min, the dominant kernel's roofline and the whole call's fractions of
    both rooflines."""
    import selective_state_space_ssd_amd as ssd
    works = [ScanWorkload(WORKLOADS[n], dev, copies, inp if i == 0 else None)
             for i, n in enumerate(names)]
    for sw in works:
        sw.prepare()
    import torch
    step = lambda k: [sw.call(k) for sw in works]
    tm = time_calls(step, steps, warmup, dev)
    n = tm["event_calls"]
    # per-stage launch times: a third pass with events the library records
    # around each stage on the launch stream
    launches_per_step = sum(sw.w.segments for sw in works)
    stage_ms = np.zeros(len(ssd.STAGES))
    for k in range(n):
        tms = [[ssd.Timing() for _ in range(sw.w.segments)] for sw in works]
        for sw, t in zip(works, tms):
            sw.call(k, t)
        torch.cuda.synchronize()
        stage_ms += np.sum([t.read() for row in tms for t in row], axis=0) / n
    dom = int(np.argmax(stage_ms))
    stage = ssd.STAGES[dom]
    w0 = works[0].w
    bf16 = w0.dtype == "bf16"
    tokens = sum(sw.w.tokens for sw in works)
    step_s = tm["wall_s_per_call"]
    fl = [alg_flops(sw.w) for sw in works]
    segs = [sw.w.segments for sw in works]
    dom_flops = sum(f[stage] * s for f, s in zip(fl, segs))
    path_flops = sum(sum(f.values()) * s for f, s in zip(fl, segs))
    path_bytes = sum(alg_bytes(sw.w) * sw.w.segments for sw in works)
    dom_s = stage_ms[dom] / 1e3
    mean_launch_s = dom_s / launches_per_step
    if bf16:  # HBM-bound (flop per byte below the bf16 ridge): the call's bytes
        ach = path_bytes / dom_s / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS,
                "frac_of_measured_peak": ach / peaks["hbm_copy_GBs"] if peaks else None,
                "alg_bytes_per_launch": path_bytes / launches_per_step}
    else:     # fp32 matrix-bound: the stage's flops
        ach = dom_flops / dom_s / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_FP32_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_FP32_MFMA_TFLOPS,
                "frac_of_measured_peak": (ach / peaks["mfma_fp32_32x32x2_TFLOPs"]
                                          if peaks else None),
                "alg_flops_per_launch": dom_flops / launches_per_step}
    traffic = measured_traffic(names[0], stage) if len(names) == 1 else None
    roof.update({"kernel": STAGE_KERNELS.get(works[0].path, {}).get(stage, stage),
                 "stage": stage, "path": works[0].path,
                 "traffic": traffic["bytes_per_launch"] if traffic else None,
                 "traffic_source": (f"profiles/traffic/{names[0]}.{stage}.json" if traffic
                                    else None),
                 "launches_timed": n * launches_per_step,
                 "mean_launch_us": mean_launch_s * 1e6})
    peak_fl = (PEAK_BF16_MFMA_TFLOPS if bf16 else PEAK_FP32_MFMA_TFLOPS) * 1e12
    t_hbm, t_mfma = path_bytes / (PEAK_HBM_GBS * 1e9), path_flops / peak_fl
    return {
        "workload": " + ".join(describe(sw.w) for sw in works),
        "names": list(names),
        "path": works[0].path,
        "tokens_per_step": tokens,
        "tokens_per_s": tokens / step_s,
        "ms_per_step": step_s * 1e3,
        "ms_per_step_events": {k: tm[k] for k in ("median_ms", "min_ms", "mean_ms")},
        "steps_timed": tm["calls"],
        "steps_timed_events": n,
        "roofline": roof,
        "call": {"alg_bytes": path_bytes, "alg_flops": path_flops,
                 "hbm_frac": t_hbm / step_s, "mfma_frac": t_mfma / step_s,
                 "binding": "hbm" if t_hbm >= t_mfma else "mfma",
                 "binding_frac": max(t_hbm, t_mfma) / step_s,
                 "stage_us_per_step": {s: float(stage_ms[i] * 1e3)
                                       for i, s in enumerate(ssd.STAGES)}},
    }


# --------------------------------------------------------------------------
# further workloads (packed sequences, decode, block, backward)
# --------------------------------------------------------------------------

def _line_timing(tm):
    return {"us_per_call": tm["wall_s_per_call"] * 1e6,
            "us_per_call_events": {k.replace("_ms", "_us"): tm[k] * 1e3
                                   for k in ("median_ms", "min_ms", "mean_ms")},
            "calls": tm["calls"]}


def decode_workload(dev, warmup, batch=128, nheads=64, dstate=128, ngroups=8):
    """One-token decode steps (bf16 inputs, fp32 state updated in place, z and D
    on): the short-sequence kernel.  Bound by reading and writing the state, so
    the roofline is HBM on the state bytes plus the token's inputs."""
    import torch
    import selective_state_space_ssd_amd as ssd
    P = 64
    g = torch.Generator(device="cpu").manual_seed(11)

    def bf(*shape):
        return torch.randn(*shape, generator=g).to(torch.bfloat16).to(dev)

    x, z = bf(batch, 1, nheads, P), bf(batch, 1, nheads, P)
    dt = bf(batch, 1, nheads)
    B, C = bf(batch, 1, ngroups, dstate), bf(batch, 1, ngroups, dstate)
    A = (-torch.exp(torch.rand(nheads, generator=g) * math.log(16.0))).to(dev)
    D = torch.randn(nheads, generator=g).to(dev)
    dt_bias = torch.full((nheads,), -2.0).to(dev)
    state = torch.randn(batch, nheads, P, dstate, generator=g).to(dev)
    out = torch.empty_like(x)
    a = (x.data_ptr(), dt.data_ptr(), A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(),
         z.data_ptr(), dt_bias.data_ptr(), 0.0, math.inf, 128, ngroups, state.data_ptr(),
         out.data_ptr(), state.data_ptr(), batch, 1, nheads, P, dstate, ssd.SSD_BF16, None, 0)
    s = torch.cuda.current_stream(dev).cuda_stream

    def call(k):
        st = ssd.scan_fwd_raw(*a, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    tm = time_calls(call, 100, warmup, dev)
    el = tm["median_ms"] / 1e3
    nbytes = 2 * batch * nheads * P * dstate * 4 + batch * (
        3 * nheads * P * 2 + nheads * 2 + 2 * ngroups * dstate * 2)
    return {
        "workload": f"one-token decode, bf16 inputs, batch {batch}, {nheads} heads x headdim 64, "
                    f"dstate {dstate}, ngroups {ngroups}, z and D on, fp32 state in place",
        "path": "step", "tokens_per_s": batch / tm["wall_s_per_call"], **_line_timing(tm),
        "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": nbytes / el / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": nbytes / el / 1e9 / PEAK_HBM_GBS,
                     "alg_bytes": nbytes, "time": "median of the per-call events"},
    }


def varlen_workload(dev, warmup, name="f32_b2_L2048_H32_P64_N128_G1_Q128", mean_len=256):
    """Packed sequences (seq_idx) on a workload's shape: each row holds
    sequences of mean length `mean_len` (uniform lengths 1 .. 2*mean-1).  The
    same calls without seq_idx are timed alongside."""
    import torch
    import selective_state_space_ssd_amd as ssd
    w = WORKLOADS[name]
    sw = ScanWorkload(w, dev, copies=2 if w.dtype == "f32" else 1)
    sw.prepare()
    ws_bytes = max(ssd.varlen_workspace_size(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                                             w.ngroups, w.chunk_size, sw.code), sw.ws_bytes)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    seq = torch.from_numpy(make_seq_idx(w.batch, w.seqlen, mean_len, 77)).to(dev)
    s = torch.cuda.current_stream(dev).cuda_stream

    def run(k, packed):
        a = list(sw.argv[k % len(sw.argv)][0])
        a[-2], a[-1] = ws.data_ptr(), ws_bytes
        st = (ssd.scan_fwd_varlen_raw(*a[:15], seq.data_ptr(), *a[15:], s) if packed
              else ssd.scan_fwd_raw(*a, s))
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    tp = time_calls(lambda k: run(k, True), MIN_CALLS, warmup, dev)
    tu = time_calls(lambda k: run(k, False), MIN_CALLS, warmup, dev)
    el = tp["median_ms"] / 1e3
    nseq = int((seq[:, 1:] != seq[:, :-1]).sum().item()) + w.batch
    line = {
        "workload": f"ssd_scan_fwd_varlen {w.dtype} batch {w.batch} x seqlen {w.seqlen} holding "
                    f"{nseq} packed sequences (mean length {mean_len}), {w.nheads} heads x "
                    f"headdim 64, dstate {w.dstate}, chunk {w.chunk_size}, ngroups {w.ngroups}",
        "path": ssd.taken_path(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                               w.chunk_size, sw.code, varlen=True),
        "tokens_per_s": w.tokens / tp["wall_s_per_call"], **_line_timing(tp),
        "plain_us_per_call_events": {"median_us": tu["median_ms"] * 1e3,
                                     "min_us": tu["min_ms"] * 1e3},
    }
    if w.dtype == "f32":
        fl = sum(alg_flops(w).values())
        line["roofline"] = {"bound": "mfma", "achieved": fl / el / 1e12,
                            "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                            "frac": fl / el / 1e12 / PEAK_FP32_MFMA_TFLOPS, "alg_flops": fl,
                            "kernels": "whole call", "time": "median of the per-call events"}
    else:
        nbytes = alg_bytes(w) + w.batch * w.seqlen * 4
        line["roofline"] = {"bound": "hbm", "achieved": nbytes / el / 1e9, "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": nbytes / el / 1e9 / PEAK_HBM_GBS,
                            "alg_bytes": nbytes, "kernels": "whole call",
                            "time": "median of the per-call events"}
    return line


def block_workload(dev, warmup, ngroups=1, norm_groups=1):
    """The block around the scan (split + conv1d + SiLU prologue, scan, gated
    RMSNorm epilogue) at mamba issue #647's repro size: fp32, batch 2 x seqlen
    2048, dim 2048 (32 heads of 64), dstate 128, conv width 4, chunk 128, with
    seeded random inputs.  Calls alternate two input copies.  The scan alone on
    same-shaped inputs (no gate) is timed alongside; the difference is the
    prologue and epilogue, whose algorithmic bytes over that time give the
    HBM roofline line."""
    import torch
    import selective_state_space_ssd_amd as ssd
    b, L, H, P, N, W, Q = 2, 2048, 32, 64, 128, 4, 128
    G = ngroups
    dim, gn = H * P, G * N
    width = 2 * dim + 2 * gn + H
    rng = np.random.default_rng(21)
    f = lambda *shape: torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dev)
    zx = [f(b, L, width) for _ in range(2)]
    cw, cb = 0.5 * f(dim + 2 * gn, W), 0.1 * f(dim + 2 * gn)
    dt_bias = torch.full((H,), -2.0, device=dev)
    A = -torch.exp(torch.from_numpy(rng.uniform(0, math.log(16.0), H).astype(np.float32)).to(dev))
    D, nw = f(H), 1.0 + 0.1 * f(dim)
    out = torch.empty((b, L, dim), device=dev)
    wsz = ssd.block_workspace_size(b, L, H, P, N, G, Q, ssd.SSD_F32, W, norm_groups)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    xs = [f(b, L, H, P) for _ in range(2)]
    Bs, Cs, dts = f(b, L, G, N), f(b, L, G, N), f(b, L, H)
    y = torch.empty_like(xs[0])
    swsz = ssd.workspace_size(b, L, H, P, N, G, Q, ssd.SSD_F32)
    sws = torch.empty(swsz, dtype=torch.uint8, device=dev)

    def block_call(k):
        st = ssd.split_conv1d_scan_fwd_raw(
            zx[k % 2].data_ptr(), cw.data_ptr(), cb.data_ptr(), dt_bias.data_ptr(), A.data_ptr(),
            D.data_ptr(), Q, None, 0.0, math.inf, nw.data_ptr(), 1e-5, P, G, norm_groups,
            out.data_ptr(), None, b, L, H, N, W, ssd.SSD_F32, ws.data_ptr(), wsz, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    def scan_call(k):
        st = ssd.scan_fwd_raw(xs[k % 2].data_ptr(), dts.data_ptr(), A.data_ptr(), Bs.data_ptr(),
                              Cs.data_ptr(), D.data_ptr(), None, dt_bias.data_ptr(), 0.0,
                              math.inf, Q, G, None, y.data_ptr(), None, b, L, H, P, N,
                              ssd.SSD_F32, sws.data_ptr(), swsz, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    tb = time_calls(block_call, MIN_CALLS, warmup, dev)
    ts = time_calls(scan_call, MIN_CALLS, warmup, dev)
    extra = (tb["median_ms"] - ts["median_ms"]) / 1e3
    halo = 1.0 + (W - 1) / 32.0
    nbytes = b * L * 4 * ((dim + 2 * gn + H) * (1.0 + halo) + 3 * dim)
    return {
        "workload": f"ssd_split_conv1d_scan_fwd f32 batch 2 x seqlen 2048, dim 2048 (32 heads x "
                    f"headdim 64), dstate 128, ngroups {G}, conv width 4, chunk 128, gated "
                    f"RMSNorm over {'the whole width' if norm_groups == 1 else 'each group'}",
        "tokens_per_s": b * L / tb["wall_s_per_call"], **_line_timing(tb),
        "scan_alone_us_per_call_events": {"median_us": ts["median_ms"] * 1e3,
                                          "min_us": ts["min_ms"] * 1e3},
        "roofline": {"kernels": "prologue + epilogue (block median minus scan median)",
                     "bound": "hbm", "achieved": nbytes / extra / 1e9 if extra > 0 else None,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": nbytes / extra / 1e9 / PEAK_HBM_GBS if extra > 0 else None,
                     "alg_bytes": nbytes},
    }


def bwd_alg_flops(w, T=64):
    """Algorithmic flops of one backward call: the forward re-run in T-step
    blocks plus, per (block, head), the causal in-block products (C.B^T once
    per group, dY.x^T, the masked products with dY, C and B: T(T+1)/2 pairs
    each) and the five T x P x N products with the block's states (P_c, G.B,
    X.G, dY.H_in and the state part of dC)."""
    from dataclasses import replace
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    nb = math.ceil(L / T)
    fwd = sum(alg_flops(replace(w, chunk_size=T)).values())
    pairs = T * (T + 1) / 2
    per = 2.0 * (pairs * (P + P + 2 * N) + 5 * T * P * N)
    return fwd + b * nb * (H * per + G * 2.0 * pairs * N)


def bwd_workload(dev, warmup, name="f32_b2_L2048_H32_P64_N128_G1_Q128", dtype="f32"):
    """The backward (every gradient, dfinal zero, z, D and dt_bias on) of the
    batch 2 x seqlen 2048 workload at ngroups 1, alternating two input copies;
    the forward on the same inputs is timed alongside.  dtype "bf16": x, dt,
    B, C, z, dout and their gradients in bf16 (the inputs rounded)."""
    import torch
    import selective_state_space_ssd_amd as ssd
    w = WORKLOADS[name]
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    io = torch.bfloat16 if dtype == "bf16" else torch.float32
    code = ssd.SSD_BF16 if dtype == "bf16" else ssd.SSD_F32
    rng = np.random.default_rng(31)
    copies = []
    for _ in range(2):
        t = {k: torch.from_numpy(v).to(dev) for k, v in make_inputs(w).items()
             if isinstance(v, np.ndarray)}
        t["dout"] = torch.from_numpy(rng.standard_normal((b, L, H, P)).astype(np.float32)).to(dev)
        for k in ("x", "dt", "B", "C", "z", "dout"):
            t[k] = t[k].to(io)
        copies.append(t)
    e = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    eio = lambda *shape: torch.empty(shape, dtype=io, device=dev)
    gr = dict(dx=eio(b, L, H, P), ddt=eio(b, L, H), dA=e(H), dB=eio(b, L, G, N),
              dC=eio(b, L, G, N), dD=e(H), dz=eio(b, L, H, P), ddt_bias=e(H))
    wsz = ssd.bwd_workspace_size(b, L, H, P, N, G, w.chunk_size, code)
    ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
    fsz = ssd.workspace_size(b, L, H, P, N, G, w.chunk_size, code)
    fws = torch.empty(max(fsz, 1), dtype=torch.uint8, device=dev)
    out = torch.empty((b, L, H, P), dtype=io, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream

    def bwd_call(k):
        t = copies[k % 2]
        st = ssd.scan_bwd_raw(
            t["x"].data_ptr(), t["dt"].data_ptr(), t["A"].data_ptr(), t["B"].data_ptr(),
            t["C"].data_ptr(), t["D"].data_ptr(), t["z"].data_ptr(), t["dt_bias"].data_ptr(),
            0.0, math.inf, w.chunk_size, G, None, t["dout"].data_ptr(), None,
            gr["dx"].data_ptr(), gr["ddt"].data_ptr(), gr["dA"].data_ptr(), gr["dB"].data_ptr(),
            gr["dC"].data_ptr(), gr["dD"].data_ptr(), gr["dz"].data_ptr(),
            gr["ddt_bias"].data_ptr(), None, b, L, H, P, N, code, ws.data_ptr(), wsz, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    def fwd_call(k):
        t = copies[k % 2]
        st = ssd.scan_fwd_raw(t["x"].data_ptr(), t["dt"].data_ptr(), t["A"].data_ptr(),
                              t["B"].data_ptr(), t["C"].data_ptr(), t["D"].data_ptr(),
                              t["z"].data_ptr(), t["dt_bias"].data_ptr(), 0.0, math.inf,
                              w.chunk_size, G, None, out.data_ptr(), None, b, L, H, P, N,
                              code, fws.data_ptr(), fsz, s)
        if st != 0:
            raise ssd.SsdError(st, ssd.status_string(st))

    tb = time_calls(bwd_call, MIN_CALLS, warmup, dev)
    tf = time_calls(fwd_call, MIN_CALLS, warmup, dev)
    fl = bwd_alg_flops(w)
    el = tb["median_ms"] / 1e3
    return {
        "workload": f"ssd_scan_bwd {dtype} batch 2 x seqlen 2048, 32 heads x headdim 64, "
                    "dstate 128, ngroups 1, z gate, D and dt_bias on: every gradient (forward "
                    "re-run inside" + (", inputs widened to fp32 and bf16 gradients rounded)"
                                       if dtype == "bf16" else ")"),
        "tokens_per_s": w.tokens / tb["wall_s_per_call"], **_line_timing(tb),
        "forward_us_per_call_events": {"median_us": tf["median_ms"] * 1e3,
                                       "min_us": tf["min_ms"] * 1e3},
        "roofline": {"kernels": "whole call", "bound": "mfma", "achieved": fl / el / 1e12,
                     "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": fl / el / 1e12 / PEAK_FP32_MFMA_TFLOPS, "alg_flops": fl,
                     "time": "median of the per-call events"},
    }


# --------------------------------------------------------------------------
# CPU baseline
# --------------------------------------------------------------------------

def _cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family, model and
    stepping numbers (a virtualised host may give only the vendor's name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v
            if not line.strip() and fields:
                break
    except OSError:
        pass
    if not fields:
        return "unknown"
    extra = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return fields.get("model name", "unknown") + (f" ({extra})" if extra else "")


def cpu_baseline(w, inp, min_seconds=10.0, heads_per_pass=16):
    """The oracle (untuned fp64 recurrence, OpenMP over batch x heads) on a
    bounded sample of workload `w`: passes of `heads_per_pass` whole heads
    (every timestep, cycling through the heads) until `min_seconds` have
    passed, scaled to tokens/s of the whole workload (tokens x heads done /
    heads)."""
    import oracle
    threads = oracle.max_threads()
    H = w.nheads
    done, elapsed, h0 = 0, 0.0, 0
    while elapsed < min_seconds:
        mask = np.zeros((w.batch, H), bool)
        hs = [(h0 + j) % H for j in range(min(heads_per_pass, H))]
        mask[:, hs] = True
        t0 = time.perf_counter()
        oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                       dt_bias=inp["dt_bias"], head_mask=mask)
        elapsed += time.perf_counter() - t0
        done += int(mask.sum())
        h0 += len(hs)
    frac = done / (w.batch * H)
    return {"value": w.tokens * frac / elapsed, "unit": "tokens/s",
            "cores": min(threads, heads_per_pass * w.batch), "kind": "oracle",
            "sample": f"{done} (batch, head) pair-scans of the {w.batch * H} of the {w.name} "
                      f"workload (heads cycled), every timestep ({elapsed:.1f} s of fp64 "
                      f"recurrence, OpenMP over the pairs of a pass, {heads_per_pass} per pass); "
                      f"value = tokens x {frac:.4f} / time",
            "cpu": _cpu_model(), "threads_available": threads}


def cpu_baseline_single_thread(name="f32_b1_L256_H4_P64_N16_G1_Q64", min_seconds=2.0):
    """The oracle with one thread on the small fp32 workload."""
    import oracle
    w = WORKLOADS[name]
    inp = make_inputs(w)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < min_seconds:
        oracle.ssd_fwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                       dt_bias=inp["dt_bias"], nthreads=1)
        n += 1
    el = time.perf_counter() - t0
    return {"value": w.tokens * n / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole calls of {w.name} in {el:.1f} s, one thread"}


# --------------------------------------------------------------------------

OTHER_SCAN_LINES = (
    ("f32_b1_L256_H4_P64_N16_G1_Q64",),
    ("f32_b2_L2048_H32_P64_N128_G1_Q128",),
    ("f32_b2_L2048_H32_P64_N128_G2_Q128",),
    ("f32_b2_L2048_H32_P64_N128_G4_Q128",),
    ("bf16_b8_L4096_H64_P64_N128_G8_Q256",),
    ("f32_b4_L8192x4seg_H32_P64_N128_G1_Q128",),
)


# the further lines by name (bench.py --only NAME runs one of them alone)
EXTRA_LINES = {
    "varlen_f32": lambda dev, warmup: varlen_workload(dev, warmup),
    "varlen_bf16": lambda dev, warmup: varlen_workload(
        dev, warmup, "bf16_b8_L4096_H64_P64_N128_G8_Q256", 512),
    "decode": lambda dev, warmup: decode_workload(dev, warmup),
    "block": lambda dev, warmup: block_workload(dev, warmup),
    "bwd_f32": lambda dev, warmup: bwd_workload(dev, warmup),
    "bwd_bf16": lambda dev, warmup: bwd_workload(dev, warmup, dtype="bf16"),
}


def main():
    global MIN_CALLS, WARMUP_SECONDS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=WARMUP_SECONDS,
                    help="least time each line's warm-up lasts (counter runs use 0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="measure the headline workload only")
    ap.add_argument("--only", default=None,
                    help="measure only this workload (a name of ssd_workloads.WORKLOADS, or one "
                         "of " + ", ".join(EXTRA_LINES) + ") and print its line (for counter "
                         "runs)")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--min-calls", type=int, default=MIN_CALLS,
                    help="least number of event-timed calls per line (counter runs use fewer)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="before the measurements, run 3 streaming device copies of this many "
                         "MiB (the reference kernel for calibrating HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the scan is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_ssd_amd as ssd  # noqa: F401

    MIN_CALLS = max(1, args.min_calls)
    WARMUP_SECONDS = max(0.0, args.warmup_seconds)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_mb > 0:
        from selective_state_space_ssd_amd import _build
        lib = ctypes.CDLL(_build.PEAKS_LIB_PATH)
        lib.ssd_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]
        nb = args.copy_mb << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            assert lib.ssd_peak_copy(src.data_ptr(), dst.data_ptr(), nb,
                                     torch.cuda.current_stream(dev).cuda_stream) == 0
        torch.cuda.synchronize()
        del src, dst

    peaks = None if args.no_peaks else measured_peaks(dev)
    if args.only in EXTRA_LINES:
        line = EXTRA_LINES[args.only](dev, args.warmup)
        line["peaks_measured"] = peaks
        print(json.dumps(line), flush=True)
        return
    if args.only:
        w1 = WORKLOADS[args.only]
        line = scan_line((args.only,), dev, args.steps, args.warmup, peaks,
                         copies=2 if (w1.dtype == "f32" and w1.segments == 1) else 1)
        line["peaks_measured"] = peaks
        print(json.dumps(line), flush=True)
        return

    w = WORKLOADS[HEADLINE]
    inp = make_inputs(w)
    head = scan_line((HEADLINE,), dev, args.steps, args.warmup, peaks, inp=inp)
    torch.cuda.empty_cache()
    line = {
        "metric": "SSD scan fwd tokens/sec at 1 MI355X; % of MFMA/HBM roofline",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps_timed"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_events": head["ms_per_step_events"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": describe(w) + " (one ssd_scan_fwd call per step)",
            "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads, "headdim": w.headdim,
            "dstate": w.dstate, "ngroups": w.ngroups, "chunk_size": w.chunk_size,
            "tokens_per_step": w.tokens, "path": head["path"], "launch": "eager",
        },
        "roofline": head["roofline"],
        "call": head["call"],
        "peaks": {"datasheet": {"hbm_GBs": PEAK_HBM_GBS, "mfma_fp32_TFLOPs": PEAK_FP32_MFMA_TFLOPS,
                                "mfma_bf16_TFLOPs": PEAK_BF16_MFMA_TFLOPS},
                  "measured": peaks},
        "cpu_baseline": None,
    }
    if not args.no_others:
        others = []
        for names in OTHER_SCAN_LINES:
            w2 = WORKLOADS[names[0]]
            others.append(scan_line(names, dev, args.steps, args.warmup, peaks,
                                    copies=2 if (w2.dtype == "f32" and w2.segments == 1) else 1))
            torch.cuda.empty_cache()
        for fn in EXTRA_LINES.values():
            others.append(fn(dev, args.warmup))
            torch.cuda.empty_cache()
        line["other_workloads"] = others
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp)
        line["cpu_baseline_single_thread"] = cpu_baseline_single_thread()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
